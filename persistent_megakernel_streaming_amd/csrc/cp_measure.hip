// Measurement kernels of the depth-loop library.
//
// The mstar pull request "Qwen3-TTS: Run the 1.7B Depth Loop as One
// Persistent Kernel on Hopper" (#1183), section "Where the depth loop's time
// goes", prices a frame against two floors: the weight-read floor (bullet
// "The floor": every position re-reads all layer weights) and the fixed
// latency each of the frame's dependent phases costs (bullet "Phases").  These
// two kernels measure both on this device:
//   stream_read_kernel  reads a buffer once with 16-byte loads, nothing else:
//                       bytes / its time is the best streaming-read rate for a
//                       working set of that size (Infinity Cache or HBM);
//   chain_kernel        a chain of phases with no work in them: in each phase
//                       every workgroup stores one tagged word and waits until
//                       the words of the phase's other workgroups carry the
//                       phase's tag (the hand-off the persistent executor uses,
//                       with the data reduced to the tags);
//   chain_counter_kernel the same chain handed off the way the pages' kernel
//                       does ("How it works": counters in global memory):
//                       store the word, release fence, add one to a counter;
//                       the readers poll the counter, take an acquire fence
//                       and then read the words.
#include <hip/hip_runtime.h>

#include "cp_device.h"

namespace cpms {

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t v4u;

__device__ __forceinline__ uint32_t fold(const v4u& a) { return a[0] ^ a[1] ^ a[2] ^ a[3]; }

// Units i, i + S, i + 2S, ... of n, S the grid's thread count; four loads in
// flight per thread.  The xor of everything read is stored only if it equals
// a value no real buffer is expected to give, which keeps the loads alive.
__global__ __launch_bounds__(256) void stream_read_kernel(const v4u* __restrict__ src, uint64_t n, uint32_t* sink) {
  const uint64_t S = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * S < n; i += 4 * S) {
    const v4u a = src[i], b = src[i + S], c = src[i + 2 * S], d = src[i + 3 * S];
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n; i += S) acc ^= fold(src[i]);
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// One wave per workgroup.  Phase k (tag = base + k + 1): lane 0 stores the tag
// into slot [k & 1][w] (16 bytes, cache policy SP); then the wave reloads (cache
// policy LP) the slots of the workgroups it waits for -- all of them, or with
// `local` the ones whose index is congruent to w modulo 8, the workgroups the
// persistent executor deals to w's XCD -- until each carries the tag.  A slot of
// parity k & 1 is written again only in phase k + 2, which no workgroup enters
// before every workgroup it waits for has finished waiting in phase k + 1,
// hence in phase k.  A wait that runs past spin_limit reloads sets *err and
// ends the workgroup's chain; the others then run out of polls too.
template <int SP, int LP>
__global__ __launch_bounds__(64) void chain_kernel(uint32_t* slots, uint32_t n_wg, uint32_t n_phases, uint32_t base,
                                                   uint32_t local, uint32_t spin_limit, uint32_t* err) {
  const uint32_t w = blockIdx.x, lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(slots, (short)0, (int)(2 * n_wg * 16), 0x00020000);
  // slots this lane checks: up to four workgroups
  uint32_t who[4];
  int nw = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = local ? (lane + 64 * i) * 8 + (w & 7) : lane + 64 * i;
    who[i] = v < n_wg ? v : w;  // past the grid: its own slot (written before the wait)
    if (v < n_wg) nw = i + 1;
  }
  for (uint32_t k = 0; k < n_phases; ++k) {
    const uint32_t tag = base + k + 1, par = k & 1;
    if (lane == 0) __builtin_amdgcn_raw_buffer_store_b128(v4u{tag, tag, tag, tag}, r, (par * n_wg + w) * 16, 0, SP);
    uint32_t n = 0;
    while (true) {
      uint32_t bad = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (par * n_wg + who[i]) * 16, 0, LP);
        bad |= (i < nw) ? (v[0] ^ tag) : 0u;
      }
      if (__builtin_amdgcn_ballot_w64(bad != 0) == 0) break;
      if (++n > spin_limit) {
        if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      // every 1024 polls: has another workgroup given up already?
      if ((n & 1023u) == 0 &&
          __builtin_amdgcn_readfirstlane(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)))
        return;
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// The counter form of the all-to-all chain.  Phase k (tag = base + k + 1):
// lane 0 stores the tag into slot [k & 1][w] (agent-coherent), orders that
// store before the next with a release fence at agent scope and adds one to
// the counter that follows the slots.  The wave polls the counter until every
// workgroup has added its one for this phase (it then holds tag * n_wg: the
// counter starts at zero and the tags run on from launch to launch without a
// gap, from base 0), takes an acquire fence and reads every workgroup's word
// once; a word without the phase's tag would be a failure of the protocol and
// sets *err.  A slot of parity k & 1 is written again only in phase k + 2,
// which no workgroup enters before every workgroup has added its one for
// phase k + 1, after its reads of phase k.
__global__ __launch_bounds__(64) void chain_counter_kernel(uint32_t* slots, uint32_t n_wg, uint32_t n_phases,
                                                           uint32_t base, uint32_t spin_limit, uint32_t* err) {
  const uint32_t w = blockIdx.x, lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(slots, (short)0, (int)(2 * n_wg * 16), 0x00020000);
  uint32_t* counter = slots + 2 * n_wg * 4;
  uint32_t who[4];
  int nw = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = lane + 64 * i;
    who[i] = v < n_wg ? v : w;
    if (v < n_wg) nw = i + 1;
  }
  for (uint32_t k = 0; k < n_phases; ++k) {
    const uint32_t tag = base + k + 1, par = k & 1;
    if (lane == 0) {
      __builtin_amdgcn_raw_buffer_store_b128(v4u{tag, tag, tag, tag}, r, (par * n_wg + w) * 16, 0, 16);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t target = tag * n_wg;
    uint32_t n = 0;
    while (true) {
      const uint32_t c = __builtin_amdgcn_readfirstlane(__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if ((int32_t)(c - target) >= 0) break;
      if (++n > spin_limit) {
        if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      if ((n & 1023u) == 0 &&
          __builtin_amdgcn_readfirstlane(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)))
        return;
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    uint32_t bad = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (par * n_wg + who[i]) * 16, 0, 16);
      bad |= (i < nw) ? (v[0] ^ tag) : 0u;
    }
    if (__builtin_amdgcn_ballot_w64(bad != 0) != 0) {
      if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(4096), dim3(256), 0, s, (const v4u*)buf, bytes / 16, sink);
  return hipGetLastError();
}

// Cache-policy bits of buffer instructions (gfx950): sc0 = 1, sc1 = 16.
hipError_t launch_chain(uint32_t* slots, int n_wg, int n_phases, uint32_t base, int local, int variant, uint32_t* err,
                        hipStream_t s) {
  // at most ~65 ms of polling per wait: a variant whose stores the readers
  // cannot see ends with *err set instead of running for seconds
  constexpr uint32_t kChainSpin = 1u << 16;
  const dim3 g(n_wg), t(64);
  const uint32_t nw = (uint32_t)n_wg, np = (uint32_t)n_phases, lo = local != 0;
  switch (variant) {
    case 0: hipLaunchKernelGGL((chain_kernel<16, 16>), g, t, 0, s, slots, nw, np, base, lo, kChainSpin, err); break;
    case 1: hipLaunchKernelGGL((chain_kernel<0, 16>), g, t, 0, s, slots, nw, np, base, lo, kChainSpin, err); break;
    case 2: hipLaunchKernelGGL((chain_kernel<0, 1>), g, t, 0, s, slots, nw, np, base, lo, kChainSpin, err); break;
    case 3: hipLaunchKernelGGL((chain_kernel<0, 17>), g, t, 0, s, slots, nw, np, base, lo, kChainSpin, err); break;
    case 4: hipLaunchKernelGGL((chain_kernel<17, 17>), g, t, 0, s, slots, nw, np, base, lo, kChainSpin, err); break;
    case 5: hipLaunchKernelGGL(chain_counter_kernel, g, t, 0, s, slots, nw, np, base, kChainSpin, err); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpms
