// Device code of the depth-loop library: the task bodies, the persistent
// executor and the one-launch-per-phase executor.
//
// The frame and its phases follow mstar pull request #1183 ("Qwen3-TTS: Run
// the 1.7B Depth Loop as One Persistent Kernel on Hopper"), section "How it
// works": one resident workgroup per compute unit walks a static task list and
// runs one tile per task; attention waits only on the qkv tiles of its own kv
// head; o and down may split their K loop and add the partial sums in a fixed
// order, with no atomics on data, so a frame is bit-identical from run to run.
// The megakernel pattern itself (resident blocks, dependencies that only point
// to earlier work, weights fetched before the wait) is the one of the handbook
// chapter "The gaps between kernels: PDL and megakernels", section
// "Megakernels: the whole forward pass in one kernel".
//
// Hand-off between workgroups.  MI355X has eight XCDs, each with its own L2,
// and a 256-workgroup counter barrier with agent-scope acquire/release costs
// several microseconds there.  Instead the data is its own ready signal, in
// one of two forms:
//   * the activations a projection streams (position inputs, residuals,
//     attention and SwiGLU outputs) are plain values in buffers where every
//     element is written at most once per frame and holds a sentinel (all
//     bits set, a NaN no producer stores) until then; a reader reloads a unit
//     until none of its elements is the sentinel, and the region is refilled
//     with the sentinel at the end of every frame;
//   * everything else (q, K/V, split-K partials, norm partials, logits) is
//     stored as 64-bit words {payload, tag}: the payload is two bf16 (or one
//     fp32) and the tag is epoch * 1024 + the writer's phase index, and a
//     reader reloads until every word carries the tag it expects.
// Values are written with agent-coherent (sc1) stores and read with
// agent-coherent loads; there are no counters, no store-completion waits and
// no cache write-back or invalidate on the path.  Weights, norms and
// embedding tables never change during a frame and use ordinary loads and
// direct-to-LDS copies.
#include <hip/hip_runtime.h>

#include <vector>

#include "cp_device.h"

namespace cpms {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kSC1 = 16;  // buffer cache policy bit: coherent at agent scope

// LDS layout of the misc region (after the two weight-tile slots).
constexpr int kRedAccLds = 1024;  // cross-wave MFMA accumulators (8 KiB)
constexpr int kRedSsLds = 9216;   // cross-wave sums of squares (1 KiB)

// ------------------------------------------------------------------ memory helpers

// A raw buffer resource over [p, p + bytes): loads past the end return zero,
// stores past the end are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16c(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1); }
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ __forceinline__ u32x2 ld8(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0); }
__device__ __forceinline__ void st16c(rsrc_t r, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSC1); }
__device__ __forceinline__ void st8c(rsrc_t r, uint32_t off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kSC1); }
__device__ __forceinline__ void st4c(rsrc_t r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kSC1); }
__device__ __forceinline__ u32x2 ld8c(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSC1); }
__device__ __forceinline__ void st16(rsrc_t r, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
__device__ __forceinline__ void st4(rsrc_t r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0); }

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Returns once the load that wrote x has completed, and with it (a wave's
// vector-memory operations complete in issue order) every vector-memory
// operation the wave issued before it: the compiler must make x valid for the
// asm, and the asm keeps later memory operations after it.
__device__ __forceinline__ void wait_for(const u32x4& x) { asm volatile("" ::"v"(x) : "memory"); }

// Trace stamp k of the current task (100 MHz constant clock), thread 0 only.
// tr is null when the plan does not trace.
__device__ __forceinline__ void stamp(uint64_t* tr, int k) {
  if (tr && threadIdx.x == 0) tr[k] = __builtin_amdgcn_s_memrealtime();
}

// Index of the XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xfu;
}


// Tagged-word stores that stay in this XCD's L2 (`local`: every reader runs
// on this XCD and loads agent-coherently) or write through to memory.
__device__ __forceinline__ void st8x(rsrc_t r, uint32_t off, u32x2 v, bool local) {
  if (local) __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
  else st8c(r, off, v);
}
__device__ __forceinline__ void st16x(rsrc_t r, uint32_t off, u32x4 v, bool local) {
  if (local) st16(r, off, v);
  else st16c(r, off, v);
}

// ------------------------------------------------------------------ numerics

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f2bf(float f) {
  const bf16x2 v = {(__bf16)f, (__bf16)0.0f};
  return __builtin_bit_cast(uint32_t, v) & 0xffffu;
}
// Two floats -> packed bf16 pair (lo in bits 0..15), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// The same, kept as one instruction: the compiler otherwise splits a pack
// whose halves are used separately into two conversions.
__device__ __forceinline__ uint32_t pack_bf16_1(float lo, float hi) {
  uint32_t r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

// Element e of a 16-byte payload chunk as float.
template <int BF>
__device__ __forceinline__ float chunk_elem(const u32x4& v, int e) {
  if constexpr (BF) return bf2f((v[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
  else return __uint_as_float(v[e]);
}

// Rounds to the activation type (returns the rounded value as float).
template <int BF>
__device__ __forceinline__ float act_val(float f) {
  if constexpr (BF) return bf2f(f2bf(f));
  else return f;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
// v from lane (lane ^ M) for M = 16, 32: the gfx950 row swaps (rows of 16
// lanes trade places with their neighbours, or halves of the wave).
template <int M>
__device__ __forceinline__ uint32_t swap_xor_u(uint32_t v) {
  static_assert(M == 16 || M == 32, "row swap distance");
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
// v from another lane by a DPP pattern CTRL that pairs lanes within rows:
// quad permutations 0xB1 (lane ^ 1) and 0x4E (lane ^ 2), half-row mirror
// 0x141 (lanes i and 7 - i of each 8), row mirror 0x140 (i and 15 - i).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// Applies f(value from a partner lane) over a tree that reaches all 64
// lanes: quads, half rows, rows by DPP, then the two row swaps.  With an
// exchange that is commutative and associative every lane ends with the same
// result.
template <typename F>
__device__ __forceinline__ void wave_tree(F&& f) {
  f([](uint32_t v) { return dpp_u<0xB1>(v); });
  f([](uint32_t v) { return dpp_u<0x4E>(v); });
  f([](uint32_t v) { return dpp_u<0x141>(v); });
  f([](uint32_t v) { return dpp_u<0x140>(v); });
  f([](uint32_t v) { return swap_xor_u<16>(v); });
  f([](uint32_t v) { return swap_xor_u<32>(v); });
}

// Value of v in lane `src` (a constant), for every lane: a scalar read, not
// an LDS round trip.
__device__ __forceinline__ float lane_f(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
// v from the lane whose index differs in bit 0 (1) or bit 1 (2), by DPP quad
// permutation.
template <int M>
__device__ __forceinline__ float quad_xor_f(float v) {
  static_assert(M == 1 || M == 2, "quad permutation");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), M == 1 ? 0xB1 : 0x4E, 0xF, 0xF, false));
}

// (value, index) that wins an argmax: larger value, then lower index.
__device__ __forceinline__ bool beats(float v, uint32_t i, float bv, uint32_t bi) {
  return v > bv || (v == bv && i < bi);
}

// ------------------------------------------------------------------ tagged words

__device__ __forceinline__ uint32_t tag_of(uint32_t epoch, uint32_t phase) { return (epoch << 10) | phase; }

// A 16-byte load holds two tagged words: [payload, tag, payload, tag].
__device__ __forceinline__ bool ll_ok(const u32x4& v, uint32_t tag) { return v[1] == tag && v[3] == tag; }

// Tagged pair of payload words for a 16-byte store.
__device__ __forceinline__ u32x4 ll_pair(uint32_t p0, uint32_t p1, uint32_t tag) { return u32x4{p0, tag, p1, tag}; }

// The payloads of a 16-byte pair of tagged words times s, in the activation
// type (bf16: each value rounded to nearest even); tags kept.
template <int BF>
__device__ __forceinline__ u32x4 scale_pair(const u32x4& v, float s) {
  if constexpr (BF)
    return u32x4{pack_bf16(bf2f(v[0] & 0xffffu) * s, bf2f(v[0] >> 16) * s), v[1],
                 pack_bf16(bf2f(v[2] & 0xffffu) * s, bf2f(v[2] >> 16) * s), v[3]};
  else
    return u32x4{__float_as_uint(__uint_as_float(v[0]) * s), v[1], __float_as_uint(__uint_as_float(v[2]) * s), v[3]};
}

// ------------------------------------------------------------------ sentinel operands

// Operand buffers hold plain values; an element not yet written this frame
// holds the sentinel, all bits set.  As an unsigned 16-bit (bf16) or 32-bit
// (fp32) number the sentinel is the largest there is, so the maximum over a
// unit's elements tells whether one is still missing (v_pk_max_u16 takes two
// bf16 at a time).  Producers never store it: a value whose bits are all set
// (a NaN) is stored with its sign bit cleared (still a NaN).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int BF>
__device__ __forceinline__ uint32_t sop_max(uint32_t m, uint32_t w) {
  if constexpr (BF)
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m), __builtin_bit_cast(u16x2, w)));
  else
    return m > w ? m : w;
}
// No sentinel among the elements whose maximum is m.
template <int BF>
__device__ __forceinline__ bool sop_clear(uint32_t m) {
  if constexpr (BF) return (m & 0xffffu) != 0xffffu && (m >> 16) != 0xffffu;
  else return m != 0xffffffffu;
}
// The stored form of a packed bf16 pair or an fp32 value: never the sentinel.
template <int BF>
__device__ __forceinline__ uint32_t sop_canon(uint32_t w) {
  if constexpr (BF) return w ^ (((w & 0xffffu) == 0xffffu) ? 0x8000u : 0u) ^ (((w >> 16) == 0xffffu) ? 0x80000000u : 0u);
  else return w == 0xffffffffu ? 0x7fffffffu : w;
}

// Operand order of a buffer of K columns: for 16-row tile rt, MFMA chunk c
// (4 E columns) and lane (q, rl) of the MFMA B operand, the 16-byte unit of
// row rt * 16 + rl, columns c * 4E + q * E ... + E - 1 lies at
// (rt * NC + c) * 1024 + (q * 16 + rl) * 16, NC = K / (4E): one wave load
// instruction reads 1 KiB in one piece, one MFMA operand per lane.  Returns
// the byte offset of element (row, n).
template <int BF>
__device__ __forceinline__ uint32_t sop_off(int row, int n, int K) {
  constexpr int ESZ = BF ? 2 : 4, E = 16 / ESZ, KS = 4 * E;
  return (uint32_t)((row >> 4) * (K / KS) + n / KS) * 1024 + (uint32_t)(((n % KS) / E) * 16 + (row & 15)) * 16 +
         (uint32_t)(n % E) * ESZ;
}
// Bytes of one plane of `rows` rows (rounded up to 16) and K columns.
template <int BF>
__device__ __forceinline__ uint32_t sop_bytes(int rows, int K) {
  return (uint32_t)((rows + 15) & ~15) * K * (BF ? 2 : 4);
}
// Stores four consecutive columns n .. n+3 (n a multiple of 4) of one row:
// 8 bytes (bf16) or one 16-byte unit (fp32), contiguous in operand order.
template <int BF>
__device__ __forceinline__ void st_sop4(rsrc_t r, int row, int n, int K, const float (&v)[4]) {
  if constexpr (BF) {
    st8c(r, sop_off<1>(row, n, K), u32x2{sop_canon<1>(pack_bf16(v[0], v[1])), sop_canon<1>(pack_bf16(v[2], v[3]))});
  } else {
    st16c(r, sop_off<0>(row, n, K),
          u32x4{sop_canon<0>(__float_as_uint(v[0])), sop_canon<0>(__float_as_uint(v[1])),
                sop_canon<0>(__float_as_uint(v[2])), sop_canon<0>(__float_as_uint(v[3]))});
  }
}

// Gives up a wait after spin_limit polls and raises the error word, so a
// broken schedule ends the kernel instead of hanging it.
struct Spin {
  uint32_t n = 0;
  __device__ __forceinline__ bool next(const DevPlan& pl) {
    if (++n > pl.spin_limit) {
      __hip_atomic_store(pl.state + 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    if ((n & 4095u) == 0 && __hip_atomic_load(pl.state + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    __builtin_amdgcn_s_sleep(1);
    return true;
  }
};

// ------------------------------------------------------------------ weights -> LDS

// Direct-to-LDS copy of a task's packed weight tile: 1 KiB chunks (64 lanes
// x 16 B) with global_load_lds_dwordx4, dealt round-robin to the four waves.
__device__ __forceinline__ void issue_tile(const DevPlan& pl, const DevTask& tk, uint8_t* slot) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint32_t nch = tk.w_bytes >> 10;
  const uint8_t* src = pl.wblob + tk.w_off;
  // (unrolled: 1516 -> 1510 us per one-row frame; a buffer-resource form
  // of the same copy measured 20-30 us slower)
#pragma unroll 4
  for (uint32_t c = wave; c < nch; c += 4) {
    __builtin_amdgcn_global_load_lds((const void*)(src + c * 1024 + lane * 16),
                                     (void __attribute__((address_space(3)))*)(slot + c * 1024), 16, 0, 0);
  }
}

// Where the next task's tile goes, and whether there is one.
struct Next {
  DevTask tk;  // loaded when the current task starts
  bool valid;
  uint8_t* slot;
  __device__ __forceinline__ void issue(const DevPlan& pl) const {
    if (valid) issue_tile(pl, tk, slot);
  }
};

// ------------------------------------------------------------------ projections

enum Epi { EPI_QKV, EPI_GU, EPI_HEAD, EPI_PART };

// The MFMA step for one 16-byte chunk of K per lane.
template <int BF>
__device__ __forceinline__ f32x4 mma(const u32x4& w, const u32x4& x, f32x4 acc) {
  if constexpr (BF) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, x), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w[e]), __uint_as_float(x[e]), acc, 0, 0, 0);
    return acc;
  }
}

// Tag check of the first n of N tagged 16-byte units: true when every word
// carries `tag`.
template <int N>
__device__ __forceinline__ bool units_ok(const u32x4 (&v)[N], uint32_t tag, int n = N) {
  uint32_t d = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n) d |= (v[i][1] ^ tag) | (v[i][3] ^ tag);
  return d == 0;
}
// The same for single tagged words (8-byte loads).
template <int N>
__device__ __forceinline__ bool units_ok(const u32x2 (&v)[N], uint32_t tag, int n = N) {
  uint32_t d = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n) d |= v[i][1] ^ tag;
  return d == 0;
}
__device__ __forceinline__ u32x4 ld_coherent(rsrc_t r, uint32_t off, u32x4*) { return ld16c(r, off); }
__device__ __forceinline__ u32x2 ld_coherent(rsrc_t r, uint32_t off, u32x2*) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSC1);
}

// Reloads of tagged units while polling, as one asm block: all loads, then a
// wait for them.  Hidden from the compiler's own wait bookkeeping, they do
// not make it treat the polled registers as the newest loads in flight (it
// would then drain every load issued after them wherever they are read).
// The block starts with five wait states: the compiler does not guard inline
// asm against the hazard of a vector-memory instruction reading SGPRs (here
// the buffer resource) that a VALU instruction (v_readlane) has just written.
__device__ __forceinline__ void asm_reload(u32x4 (&v)[1], rsrc_t r, const uint32_t (&o)[1]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx4 %0, %1, %2, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0])
               : "v"(o[0]), "s"(r)
               : "memory");
}

__device__ __forceinline__ void asm_reload(u32x4 (&v)[2], rsrc_t r, const uint32_t (&o)[2]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx4 %0, %2, %4, 0 offen sc1\n"
               "buffer_load_dwordx4 %1, %3, %4, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0]), "+v"(v[1])
               : "v"(o[0]), "v"(o[1]), "s"(r)
               : "memory");
}

__device__ __forceinline__ void asm_reload(u32x4 (&v)[4], rsrc_t r, const uint32_t (&o)[4]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx4 %0, %4, %8, 0 offen sc1\n"
               "buffer_load_dwordx4 %1, %5, %8, 0 offen sc1\n"
               "buffer_load_dwordx4 %2, %6, %8, 0 offen sc1\n"
               "buffer_load_dwordx4 %3, %7, %8, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])
               : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "s"(r)
               : "memory");
}

__device__ __forceinline__ void asm_reload(u32x4 (&v)[6], rsrc_t r, const uint32_t (&o)[6]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx4 %0, %6, %12, 0 offen sc1\n"
               "buffer_load_dwordx4 %1, %7, %12, 0 offen sc1\n"
               "buffer_load_dwordx4 %2, %8, %12, 0 offen sc1\n"
               "buffer_load_dwordx4 %3, %9, %12, 0 offen sc1\n"
               "buffer_load_dwordx4 %4, %10, %12, 0 offen sc1\n"
               "buffer_load_dwordx4 %5, %11, %12, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5])
               : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "v"(o[5]), "s"(r)
               : "memory");
}

__device__ __forceinline__ void asm_reload(u32x4 (&v)[8], rsrc_t r, const uint32_t (&o)[8]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx4 %0, %8, %16, 0 offen sc1\n"
               "buffer_load_dwordx4 %1, %9, %16, 0 offen sc1\n"
               "buffer_load_dwordx4 %2, %10, %16, 0 offen sc1\n"
               "buffer_load_dwordx4 %3, %11, %16, 0 offen sc1\n"
               "buffer_load_dwordx4 %4, %12, %16, 0 offen sc1\n"
               "buffer_load_dwordx4 %5, %13, %16, 0 offen sc1\n"
               "buffer_load_dwordx4 %6, %14, %16, 0 offen sc1\n"
               "buffer_load_dwordx4 %7, %15, %16, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
               : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "v"(o[5]), "v"(o[6]), "v"(o[7]), "s"(r)
               : "memory");
}

__device__ __forceinline__ void asm_reload(u32x4 (&v)[16], rsrc_t r, const uint32_t (&o)[16]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx4 %0, %16, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %1, %17, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %2, %18, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %3, %19, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %4, %20, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %5, %21, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %6, %22, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %7, %23, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %8, %24, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %9, %25, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %10, %26, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %11, %27, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %12, %28, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %13, %29, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %14, %30, %32, 0 offen sc1\n"
               "buffer_load_dwordx4 %15, %31, %32, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
               : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "v"(o[5]), "v"(o[6]), "v"(o[7]), "v"(o[8]), "v"(o[9]), "v"(o[10]), "v"(o[11]), "v"(o[12]), "v"(o[13]), "v"(o[14]), "v"(o[15]), "s"(r)
               : "memory");
}

__device__ __forceinline__ void asm_reload(u32x2 (&v)[1], rsrc_t r, const uint32_t (&o)[1]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx2 %0, %1, %2, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0])
               : "v"(o[0]), "s"(r)
               : "memory");
}

__device__ __forceinline__ void asm_reload(u32x2 (&v)[16], rsrc_t r, const uint32_t (&o)[16]) {
  asm volatile("s_nop 4\n"
               "buffer_load_dwordx2 %0, %16, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %1, %17, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %2, %18, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %3, %19, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %4, %20, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %5, %21, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %6, %22, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %7, %23, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %8, %24, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %9, %25, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %10, %26, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %11, %27, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %12, %28, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %13, %29, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %14, %30, %32, 0 offen sc1\n"
               "buffer_load_dwordx2 %15, %31, %32, 0 offen sc1\n"
               "s_waitcnt vmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
               : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "v"(o[5]), "v"(o[6]), "v"(o[7]), "v"(o[8]), "v"(o[9]), "v"(o[10]), "v"(o[11]), "v"(o[12]), "v"(o[13]), "v"(o[14]), "v"(o[15]), "s"(r)
               : "memory");
}

// Sentinel check of the first n of N operand units (16 or 8 bytes each).
template <int BF, int N>
__device__ __forceinline__ bool sop_units_ok(const u32x4 (&v)[N], int n = N) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t mi = sop_max<BF>(sop_max<BF>(v[i][0], v[i][1]), sop_max<BF>(v[i][2], v[i][3]));
    m = (i < n) ? sop_max<BF>(m, mi) : m;
  }
  return sop_clear<BF>(m);
}
template <int BF, int N>
__device__ __forceinline__ bool sop_units_ok(const u32x2 (&v)[N], int n = N) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) m = (i < n) ? sop_max<BF>(m, sop_max<BF>(v[i][0], v[i][1])) : m;
  return sop_clear<BF>(m);
}

// A set of units a lane is waiting for: N loads already issued into v, their
// offsets in r, and what makes them current -- CK = 0: the tag they must
// carry; CK = 1 (bf16) or 2 (fp32): no sentinel left among their elements.
// Units from `nload` on are neither checked nor reloaded (they may hold
// anything).  ASM: reloads through asm_reload (every unit, those past nload
// being rereads nobody checks).
template <typename T, int N, typename Off, bool ASM, int CK = 0>
struct Pend {
  T (&v)[N];
  rsrc_t r;
  Off off;
  uint32_t tag;
  bool active;
  int nload;
  __device__ __forceinline__ bool current() const {
    if constexpr (CK == 0) return units_ok(v, tag, nload);
    else return sop_units_ok<CK == 1>(v, nload);
  }
  // (both sides always evaluated: the check then reads every unit on every
  // path, so the compiler knows the loads are complete after a wait)
  __device__ __forceinline__ bool ok() const { return !active | current(); }
  __device__ __forceinline__ void reload() {
    if (active && !current()) {
      if constexpr (ASM) {
        uint32_t o[N];
#pragma unroll
        for (int i = 0; i < N; ++i) o[i] = off(i);
        asm_reload(v, r, o);
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
          if (i < nload) v[i] = ld_coherent(r, off(i), (T*)nullptr);
      }
    }
  }
};
template <bool ASM = false, typename T, int N, typename Off>
__device__ __forceinline__ Pend<T, N, Off, ASM> pend(T (&v)[N], rsrc_t r, Off off, uint32_t tag, bool active,
                                                     int nload = N) {
  return Pend<T, N, Off, ASM>{v, r, off, tag, active, nload};
}
// A set of operand units (sentinel check, activation type BF).
template <int BF, bool ASM = false, typename T, int N, typename Off>
__device__ __forceinline__ Pend<T, N, Off, ASM, BF ? 1 : 2> spend(T (&v)[N], rsrc_t r, Off off, bool active,
                                                                 int nload = N) {
  return Pend<T, N, Off, ASM, BF ? 1 : 2>{v, r, off, 0u, active, nload};
}

// Waits until every set of every lane carries its tag.  When the data is
// there this is one check per set; otherwise each stale set is reloaded with
// agent-coherent loads, all sets in the same round trip, and checked again.
// The loop itself is wave-uniform.
template <typename... Ps>
__device__ __forceinline__ void await_all(const DevPlan& pl, Ps&&... ps) {
  Spin sp;
  while (__builtin_amdgcn_ballot_w64(!(ps.ok() && ...)) != 0) {
    if (!sp.next(pl)) break;
    (ps.reload(), ...);
  }
}

// Projection tile: out[row][16 columns] = W_tile . a[row] over the task's K
// range, for every live row, with MFMA 16x16 tiles (A = the weight tile from
// LDS, B = 16 rows of activations).  KIND fixes the operand, its RMSNorm and
// the epilogue at compile time:
//   T_QKV  : RMSNorm(layer input) -> q (RoPE), k (RoPE), v
//   T_O    : attention output -> + residual (split-K partials in fixed order)
//   T_GU   : RMSNorm(residual) -> silu(gate) * up
//   T_DOWN : SwiGLU output -> + residual (split-K partials in fixed order)
//   T_HEAD : RMSNorm(last residual) -> logits, per-tile argmax candidate
//   T_INPROJ: frame input (plain rows) -> position-0 input (split-K partials)
// RMSNorm: the gain g is folded into the packed weight tile at plan creation
// (W . (g x / rms(x)) = (W g) . x / rms(x)), so the MFMAs take the residual
// rows as they are and the fp32 result is scaled by 1 / rms(x) of its row.
// NOQK: the QK-norm variant is not compiled in (the plain many-row form of
// plans without it: 2392 -> 2369 us per 64-row frame).
template <int BF, int KIND, bool ONE = false, bool ASM = !ONE, bool NOQK = false>
__device__ __forceinline__ void proj_task(const DevPlan& pl, const DevFrame& fr, const DevTask& tk, uint32_t epoch,
                                          uint8_t* slot, uint32_t* misc, uint64_t* tr, bool lcl,
                                          int r0, int gr) {
  constexpr int ESZ = BF ? 2 : 4;     // bytes per activation element
  constexpr int E = 16 / ESZ;         // elements per 16-byte payload chunk
  constexpr int KS = 4 * E;           // K elements one chunk step covers across the 4 lane groups
  constexpr bool XLL = KIND != T_INPROJ;  // operand rows are tagged words
  constexpr bool NORM = KIND == T_QKV || KIND == T_GU || KIND == T_HEAD;
  constexpr int NB = KIND == T_GU ? 2 : 1;  // weight tiles per chunk (gate and up)
  constexpr bool PART = KIND == T_O || KIND == T_DOWN || KIND == T_INPROJ;
  constexpr bool RESID = KIND == T_O || KIND == T_DOWN;
  // Operand groups: NU chunks (one 16-byte load per lane each) per group,
  // DEPTH groups in flight per wave.  Groups of 8 have half the waits and
  // checks of groups of 4 (four of 4 in flight: 2646 us per 64-row frame;
  // three of 8: 2516; three of 8 for the normed projections and two for the
  // split-K ones, whose K slices are two or three groups at 64 rows: 2504;
  // two of 8 everywhere 2531, four of 8 2900, eight of 2 2977, two of 16
  // spill).  A wave's K range is whole groups (wpr below; the plan keeps
  // split-K slices in whole groups), which at 32 rows or fewer can leave
  // waves of a split-K task idle: measured no slower than groups of 4 there.
  constexpr int NU = 8;
  constexpr int DEPTH = NORM ? 3 : 2;
  constexpr uint32_t CST = 64;              // frame-input bytes per chunk step
  // ONE: a frame of one row.  Only row 0 of the operand tile is loaded, its
  // 16-byte units packed densely over the lanes (one load instruction per 16
  // chunks instead of one per chunk), and handed to the MFMA lanes with
  // ds_bpermute; the row's sum of squares is taken from those units.
  static_assert(!ONE || XLL, "one-row operands are tagged");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 4, rl = lane & 15;
  const int rows = fr.rows;
  const int H = pl.H, Rmax = pl.Rmax, P = pl.P;
  const int l = tk.layer, p = tk.pos;
  const uint32_t my_tag = tag_of(epoch, tk.phase);

  // Operand buffers have a plane per layer and position; the tagged split-K
  // partials that positions 0 and 1 (in flight together) would share are
  // doubled and picked by position parity.
  const int par = p & 1;
  const uint32_t hbytes = sop_bytes<BF>(Rmax, H);
  auto plane = [&](int ll, int pp) -> size_t { return (size_t)(ll * P + pp); };
  uint8_t* const xin = (uint8_t*)pl.xin;
  uint8_t* const hres = (uint8_t*)pl.hres;
  uint8_t* const hmid = (uint8_t*)pl.hmid;
  const uint8_t* xsrc;
  uint32_t ld;                     // operand row length (elements)
  int kt = H, k0 = 0;
  if constexpr (KIND == T_QKV) {
    xsrc = (l == 0) ? xin + (size_t)p * hbytes : hres + plane(l - 1, p) * hbytes;
    ld = H;
  } else if constexpr (KIND == T_GU) {
    xsrc = hmid + plane(l, p) * hbytes; ld = H;
  } else if constexpr (KIND == T_HEAD) {
    xsrc = hres + plane(pl.L - 1, p) * hbytes; ld = H;
  } else if constexpr (KIND == T_O) {
    // (the many-row executor runs down tasks through this instantiation too:
    // one body for both split-K kinds keeps the kernel's code smaller,
    // 2375 -> 2351 us per 64-row frame; the one-row kernel keeps two)
    if (ONE || tk.type == T_O) {
      ld = pl.nq * pl.d; xsrc = (const uint8_t*)pl.abuf + plane(l, p) * sop_bytes<BF>(Rmax, ld);
    } else {
      ld = pl.I; xsrc = (const uint8_t*)pl.mbuf + plane(l, p) * sop_bytes<BF>(Rmax, ld);
    }
  } else if constexpr (KIND == T_DOWN) {
    ld = pl.I; xsrc = (const uint8_t*)pl.mbuf + plane(l, p) * sop_bytes<BF>(Rmax, ld);
  } else {
    ld = pl.Din; xsrc = (const uint8_t*)fr.hidden_in;
  }
  if constexpr (PART) {
    kt = (int)ld / tk.nsplit;
    k0 = tk.split * kt;
  }
  const int nck = kt * ESZ / 64;  // 16-byte payload chunks per lane over the task's K range

  // Waves and row tiles: a wave owns 16 rows of a group of gr <= 64 rows
  // starting at row r0; with few rows the waves of a row tile split K and add
  // their results through LDS in a fixed order.  A frame of more than 64 rows
  // runs the task once per group of 64, the weight tile staying in LDS; with
  // row groups each task is one group of 32.
  const int rows_h = min(rows - r0, gr);
  const int nrt = (rows_h + 15) >> 4;                 // row tiles of this group holding live rows (1..4)
  int wpr = nrt == 1 ? 4 : (nrt == 2 ? 2 : 1);        // waves per row tile
  // each wave takes whole groups of NU chunks (one-row frames: blocks of 4)
  while (wpr > 1 && nck % ((ONE ? 4 : NU) * wpr)) wpr >>= 1;
  const int rt = wave / wpr, ks = wave % wpr;
  const int rta = (r0 >> 4) + rt;                     // the row tile in the frame
  const int ncw = nck / wpr;                          // chunks this wave handles (a multiple of NU)
  const int ng = ncw / NU;
  const int c0 = ks * ncw;
  const int row = rta * 16 + rl;
  const bool wave_live = rt < nrt;
  const bool live = wave_live && row < rows;

  // Operand rows.  Operand buffers are in operand order: the unit of chunk
  // c of this lane is at xoff + c * 1024.  A lane whose row is past the
  // frame's rows reads values of no use (left out of every wait; they only
  // reach that row's MFMA column, which is never stored).  The frame input is
  // plain row-major; its resource ends at the last row, so rows past it read
  // zeros.  Every load of an operand unit is agent-coherent; a unit that still
  // holds a sentinel is loaded again.
  const uint32_t xrow = (uint32_t)ld * ESZ;  // frame input only
  const rsrc_t rx = XLL ? make_rsrc(xsrc, sop_bytes<BF>(Rmax, ld)) : make_rsrc(xsrc, (uint32_t)rows * xrow);
  const uint32_t xoff = XLL ? (uint32_t)(rta * (ld / KS) + k0 / KS + c0) * 1024 + (uint32_t)lane * 16
                            : (uint32_t)row * xrow + (uint32_t)(k0 + q * E) * ESZ + c0 * CST;
  auto uoff = [=](int g) {
    return [=](int u) -> uint32_t { return xoff + (uint32_t)(g * NU + u) * (XLL ? 1024u : CST); };
  };
  // DEPTH groups in flight: set xs[s] holds groups g = s (mod DEPTH).
  u32x4 xs[DEPTH][NU];
  auto load = [&](u32x4 (&x)[NU], int g) {
    if (g < ng) {
#pragma unroll
      for (int u = 0; u < NU; ++u) x[u] = XLL ? ld16c(rx, uoff(g)(u)) : ld16(rx, uoff(g)(u));
    }
  };
  // ONE: piece P = c * 4 + q' (chunk c of this wave, lane group q') is
  // loaded by lane P % 64 of instruction P / 64; lanes past the last piece
  // load a duplicate.
  constexpr int NJ1 = 2;  // at most 32 chunks per wave
  u32x4 xo[NJ1];
  const int npc = 4 * ncw, nj1 = (npc + 63) / 64;
  const uint32_t xbase1 = (uint32_t)(k0 / KS + c0) * 1024;
  auto oo = [=](int j) -> uint32_t {
    const int P = (j * 64 + lane) % npc;
    return xbase1 + (uint32_t)((P >> 2) * 1024 + (P & 3) * 256);
  };
  if (wave_live) {
    if constexpr (ONE) {
#pragma unroll
      for (int j = 0; j < NJ1; ++j) xo[j] = ld16c(rx, oo(j < nj1 ? j : nj1 - 1));  // (past nj1: not waited for)
    } else {
      // (the first four groups without branches; past the last group,
      // the last one is read again and never waited for)
      auto load0 = [&](u32x4 (&x)[NU], int g) {
        const int gg = g < ng ? g : ng - 1;
#pragma unroll
        for (int u = 0; u < NU; ++u) x[u] = XLL ? ld16c(rx, uoff(gg)(u)) : ld16(rx, uoff(gg)(u));
      };
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) load0(xs[s], s);
    }
  }
  // RoPE angles of a qkv tile's two rotary pairs per lane.
  float rope_cs[2] = {1.f, 1.f}, rope_sn[2] = {0.f, 0.f};
  if constexpr (KIND == T_QKV) {
    const int d = pl.d, th = d / 16, tpg = (pl.gq + 2) * th, lt = tk.tile % tpg;
    // (loaded for v tiles too, which do not use them: no branch between loads)
    const int i0 = 8 * (lt % th) + 2 * q;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      rope_cs[pr] = pl.rope[(p * (d / 2) + i0 + pr) * 2];
      rope_sn[pr] = pl.rope[(p * (d / 2) + i0 + pr) * 2 + 1];
    }
  }
  // The data is its own signal: wait for the first group, then for this
  // task's weight tile (issued during the previous task) to be in LDS.  With tagged operands the tile's copy is older than
  // every load of group 0 (the executor issues it before it dispatches the
  // task, and a task's loads are its own code, behind that dispatch), so
  // group 0 having arrived covers this wave's part of it and the later groups
  // stay in flight.  A wave with no live rows issued no operand loads but
  // still copied its share of the tile, and waits for every load; so do
  // one-row frames and untagged operands.  (wave_live is wave-uniform.)
  if constexpr (ONE)
    await_all(pl, spend<BF>(xo, rx, oo, wave_live, nj1));
  else
    await_all(pl, spend<BF, ASM>(xs[0], rx, uoff(0), XLL && live));
  if (XLL && !ONE && wave_live) wait_for(xs[0][0]);
  else wait_vm();
  __syncthreads();
  stamp(tr, 2);

  // RMSNorm needs the sum of squares of each row over all of K.  The
  // projection streams the whole row anyway, so it takes the sum from its
  // own operand units instead of waiting for partial sums from the tiles
  // that produced the row (which would be a wait on every producer tile
  // before the first MFMA).  Many rows: one more MFMA per chunk, x x^T, whose
  // diagonal holds the rows' sums (2349 -> 2217 us per 64-row frame, and
  // 2166 with the producers no longer writing partials; squares taken with
  // vector ALU instructions in the K loop instead: 2422).  ONE: each wave
  // holds its pieces of row 0 whole after the first load and adds their
  // squares there (1575 -> 1547 us per one-row frame).  Waves that split K
  // add their sums after the K loop, in wave order.
  float ssl = 0.f;
  if constexpr (NORM && ONE) {
#pragma unroll
    for (int j = 0; j < NJ1; ++j)
      if (j < nj1 && j * 64 + lane < npc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (BF) {
            const float lo = __uint_as_float(xo[j][e] << 16), hi = __uint_as_float(xo[j][e] & 0xffff0000u);
            ssl = fmaf(lo, lo, ssl);
            ssl = fmaf(hi, hi, ssl);
          } else {
            const float v = __uint_as_float(xo[j][e]);
            ssl = fmaf(v, v, ssl);
          }
        }
      }
    wave_tree([&](auto other) { ssl += __uint_as_float(other(__float_as_uint(ssl))); });
  }

  const uint8_t* wt = slot + lane * 16 + (size_t)c0 * NB * 1024;
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0}, accs = {0, 0, 0, 0};
  auto step = [&](u32x4 (&xr)[NU], int g) {
    if constexpr (XLL) await_all(pl, spend<BF, ASM>(xr, rx, uoff(g), live));
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int c = g * NU + i;
      const u32x4 x = xr[i];
      if constexpr (NORM && !ONE) accs = mma<BF>(x, x, accs);
      const u32x4 w0 = *(const u32x4*)(wt + c * NB * 1024);
      if constexpr (NB == 2) {
        const u32x4 w1 = *(const u32x4*)(wt + (c * 2 + 1) * 1024);
        acc0 = mma<BF>(w0, x, acc0);
        acc1 = mma<BF>(w1, x, acc1);
      } else {
        if (i & 1) acc1 = mma<BF>(w0, x, acc1);
        else acc0 = mma<BF>(w0, x, acc0);
      }
    }
  };
  if (wave_live && ONE) {
    // chunk c of instruction j = c / 16: the unit of lane group q sits in
    // lane (c % 16) * 4 + q (every MFMA column gets row 0)
#pragma unroll
    for (int j = 0; j < NJ1; ++j) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (j * 16 + h * 4 >= ncw) break;  // ncw is a multiple of 4: whole blocks of 4 chunks
#pragma unroll
        for (int cj = 0; cj < 4; ++cj) {
          const int ci = h * 4 + cj, c = j * 16 + ci;
          const int a = (ci * 4 + q) * 4;
          const u32x4 x = {(uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)xo[j][0]),
                           (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)xo[j][1]),
                           (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)xo[j][2]),
                           (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)xo[j][3])};
          const u32x4 w0 = *(const u32x4*)(wt + c * NB * 1024);
          if constexpr (NB == 2) {
            const u32x4 w1 = *(const u32x4*)(wt + (c * 2 + 1) * 1024);
            acc0 = mma<BF>(w0, x, acc0);
            acc1 = mma<BF>(w1, x, acc1);
          } else {
            if (c & 1) acc1 = mma<BF>(w0, x, acc1);
            else acc0 = mma<BF>(w0, x, acc0);
          }
        }
      }
      if (j == 0) stamp(tr, 3);
    }
    if constexpr (NB == 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc0[v] = acc0[v] + acc1[v];
    }
  } else if (wave_live) {
    // Each set is refilled with the group DEPTH ahead right after its use,
    // so DEPTH - 1 or DEPTH groups are always on their way.  The compiler's
    // waits are in issue order: a set's wait then covers only the loads
    // issued before it (its polling reloads are in asm; compiler-issued
    // reloads made every set look like the newest loads and drained all of
    // them at each group).
    for (int g = 0; g < ng; g += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        if (s == 0 || g + s < ng) {
          step(xs[s], g + s);
          if (s == 0 && g == 0) stamp(tr, 3);
          load(xs[s], g + s + DEPTH);
        }
      }
    }
    if constexpr (NB == 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc0[v] = acc0[v] + acc1[v];
    }
  }
  stamp(tr, 4);
  if constexpr (NORM && !ONE) {
    // the row's sum of squares: the diagonal of the Gram block x x^T, entry
    // (rl, rl) in lane (rl / 4) * 16 + rl, element rl % 4
    const int v = rl & 3;
    const float mine = v == 0 ? accs[0] : (v == 1 ? accs[1] : (v == 2 ? accs[2] : accs[3]));
    ssl = __shfl(mine, (rl >> 2) * 16 + rl, 64);
  }
  if (wpr > 1) {
    // K parts of a row tile: (((k0 + k1) + k2) + k3), in the wave of part 0
    f32x4* red_acc = (f32x4*)((uint8_t*)misc + kRedAccLds);  // [4 waves][2][64 lanes]
    float* red_ss = (float*)((uint8_t*)misc + kRedSsLds);  // [4 waves][64 lanes]
    if (wave_live) {
      if constexpr (NORM) red_ss[wave * 64 + lane] = ssl;
      red_acc[(wave * 2 + 0) * 64 + lane] = acc0;
      if constexpr (NB == 2) red_acc[(wave * 2 + 1) * 64 + lane] = acc1;
    }
    __syncthreads();
    if (wave_live && ks == 0) {
      for (int k = 1; k < wpr; ++k) {
        if constexpr (NORM) ssl = ssl + red_ss[(rt * wpr + k) * 64 + lane];
        const f32x4 a = red_acc[((rt * wpr + k) * 2 + 0) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc0[v] = acc0[v] + a[v];
        if constexpr (NB == 2) {
          const f32x4 b = red_acc[((rt * wpr + k) * 2 + 1) * 64 + lane];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc1[v] = acc1[v] + b[v];
        }
      }
    }
  }
  if constexpr (NORM) {  // W (g . x / rms(x)) = (W g) x / rms(x): the gain is in the packed tile
    const float rinv = 1.0f / sqrtf(ssl / (float)H + pl.eps);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc0[v] = acc0[v] * rinv;
      if constexpr (NB == 2) acc1[v] = acc1[v] * rinv;
    }
  }
  const bool epi_wave = wave_live && ks == 0;
  const uint32_t slots = (uint32_t)(16 * tk.tile + 4 * q);  // this lane's 4 output slots

  if constexpr (PART) {
    // Split-K: the owner (split 0) collects its partners' partials (tagged
    // with this phase, in split order) and the residual.
    const bool owner = tk.split == 0;
    uint64_t part_off;
    void* out;
    const void* resid = nullptr;
    if constexpr (KIND == T_O) {
      if (ONE || tk.type == T_O) {
        part_off = pl.part_o_off + (uint64_t)par * pl.part_stride; out = hmid + plane(l, p) * hbytes;
        resid = (l == 0) ? xin + (size_t)p * hbytes : hres + plane(l - 1, p) * hbytes;
      } else {  // a down task (many-row executor)
        part_off = pl.part_d_off + (uint64_t)par * pl.part_stride; out = hres + plane(l, p) * hbytes;
        resid = hmid + plane(l, p) * hbytes;
      }
    } else if constexpr (KIND == T_DOWN) {
      part_off = pl.part_d_off + (uint64_t)par * pl.part_stride; out = hres + plane(l, p) * hbytes;
      resid = hmid + plane(l, p) * hbytes;
    } else {
      part_off = pl.part_in_off; out = xin;
    }
    const rsrc_t rp = make_rsrc(pl.part + part_off, (uint32_t)pl.part_stride * 8);
    const uint32_t pbase = (uint32_t)((tk.tile * tk.nsplit * Rmax + row) * 16 + 4 * q) * 8;
    const uint32_t pstep = (uint32_t)Rmax * 16 * 8;  // bytes between splits of a tile
    auto po = [=](int u) -> uint32_t { return pbase + (1 + (u >> 1)) * pstep + (u & 1) * 16; };
    const rsrc_t rr = make_rsrc(resid, hbytes);
    auto ro = [=](int) -> uint32_t { return sop_off<BF>(row, (int)slots, H); };
    // the residual's four slots: 8 bytes (bf16) or one 16-byte unit (fp32)
    u32x4 pv[6];
    u32x2 rw[1];
    u32x4 rq[1];
    const int npart = tk.nsplit - 1;
    if (epi_wave && !owner) {
      if (live) {
        // With the owner on this XCD the partials stay in its L2 (plain
        // stores; the owner's agent-coherent loads read the L2); a workgroup
        // not on the XCD the placement assumed writes through to memory.
        const uint32_t o = pbase + tk.split * pstep;
        const u32x4 p0 = ll_pair(__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), my_tag);
        const u32x4 p1 = ll_pair(__float_as_uint(acc0[2]), __float_as_uint(acc0[3]), my_tag);
        if ((tk.flags & kTaskLocalPartials) && lcl) {
          st16(rp, o, p0);
          st16(rp, o + 16, p1);
        } else {
          st16c(rp, o, p0);
          st16c(rp, o + 16, p1);
        }
      }
    } else if (epi_wave) {
      // (splits past the last partner reread the last one, or read beyond the
      // tile's partials when there is no partner; never waited for)
#pragma unroll
      for (int u = 0; u < 6; ++u) pv[u] = ld16c(rp, po((u >> 1) < npart ? u : 2 * npart - 2 + (u & 1)));
      if constexpr (RESID) {
        if constexpr (BF) rw[0] = ld8c(rr, ro(0));
        else rq[0] = ld16c(rr, ro(0));
      }
    }
    if (epi_wave && owner) {
      if constexpr (BF)
        await_all(pl, pend<ASM>(pv, rp, po, my_tag, live && npart > 0, 2 * npart),
                  spend<BF, ASM>(rw, rr, ro, RESID && live));
      else
        await_all(pl, pend<ASM>(pv, rp, po, my_tag, live && npart > 0, 2 * npart),
                  spend<BF, ASM>(rq, rr, ro, RESID && live));
      f32x4 s = acc0;
#pragma unroll
      for (int sp = 1; sp < 4; ++sp)
        if (sp <= npart) {
          const u32x4 a = pv[2 * sp - 2], b = pv[2 * sp - 1];
          s[0] = s[0] + __uint_as_float(a[0]); s[1] = s[1] + __uint_as_float(a[2]);
          s[2] = s[2] + __uint_as_float(b[0]); s[3] = s[3] + __uint_as_float(b[2]);
        }
      float h[4];
      if constexpr (RESID) {
        const u32x4 r4 = BF ? u32x4{rw[0][0], rw[0][1], 0, 0} : rq[0];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = act_val<BF>(s[e] + chunk_elem<BF>(r4, e));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = act_val<BF>(s[e]);
      }
      if (live) st_sop4<BF>(make_rsrc(out, hbytes), row, (int)slots, H, h);
    }
  } else {
    if (epi_wave && live) {
      if constexpr (KIND == T_QKV) {
        const int d = pl.d, th = d / 16, gq = pl.gq, nkv = pl.nkv;
        const int tpg = (gq + 2) * th;
        const int g = tk.tile / tpg, lt = tk.tile % tpg;
        const uint32_t kvoff = (uint32_t)(((l * Rmax + row) * nkv + g) * P + p) * d;
        const uint32_t kvbytes = (uint32_t)pl.L * Rmax * nkv * P * d * ESZ * 2;
        const uint32_t kv_tag = tag_of(epoch, kKvPhase);
        // q, k and v stay in this XCD's L2 when the attention of kv group g runs here
        const bool lqkv = (tk.flags & kTaskLocalQkv) && lcl;
        if (lt < (gq + 1) * th) {
          // q or k head: slots (4q + v) hold rotary pairs 8 tih + 2q + (v >> 1), half v & 1
          const int tih = lt % th;
          const bool isq = lt < gq * th;
          const int hq = g * gq + lt / th;
          const int i0 = 8 * tih + 2 * q;
          // QK-norm: the head's RMSNorm scales it by one number, 1 / rms of
          // the whole head, which RoPE (a rotation of pairs) commutes with.
          // The tile applies the gains and RoPE and stores the head unscaled
          // (K in a staging buffer), with its 16 dims' sum of squares; the
          // attention task adds the head's partials and scales.
          const bool qkn = !NOQK && pl.qk_norm;
          float xg[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) xg[v] = acc0[v];
          if (qkn) {
            float ss = ((acc0[0] * acc0[0] + acc0[1] * acc0[1]) + acc0[2] * acc0[2]) + acc0[3] * acc0[3];
            ss += shfl_xor_f(ss, 16);
            ss += shfl_xor_f(ss, 32);
            const float* gn = pl.qk_gain + ((size_t)l * 2 + (isq ? 0 : 1)) * d;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
              xg[2 * pr] = acc0[2 * pr] * gn[i0 + pr];
              xg[2 * pr + 1] = acc0[2 * pr + 1] * gn[i0 + pr + d / 2];
            }
            const int nh = pl.nq + nkv;
            const uint32_t nbytes = (uint32_t)2 * Rmax * nh * th * 8;
            if (q == 0)
              st8x(make_rsrc(pl.qkn, nbytes), (uint32_t)((((par * Rmax + row) * nh + (isq ? hq : pl.nq + g)) * th + tih) * 8),
                   u32x2{__float_as_uint(ss), my_tag}, lqkv);
          }
          float y[4];
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const float x1 = xg[2 * pr], x2 = xg[2 * pr + 1];
            y[2 * pr] = x1 * rope_cs[pr] - x2 * rope_sn[pr];
            y[2 * pr + 1] = x2 * rope_cs[pr] + x1 * rope_sn[pr];
          }
          // dims i0, i0 + 1 (first halves) and i0 + d/2, i0 + d/2 + 1 (second halves)
          const uint32_t qdbytes = (uint32_t)Rmax * pl.nq * d * ESZ * 2;
          const uint32_t kvelems = (uint32_t)pl.L * Rmax * nkv * P * d;
          const uint32_t krbytes = qkn ? (uint32_t)2 * Rmax * nkv * d * ESZ * 2 : 0u;
          const rsrc_t r = isq ? make_rsrc((uint8_t*)pl.qbuf + (size_t)par * qdbytes, qdbytes)
                               : make_rsrc(pl.kc, kvbytes + krbytes);
          // (QK-norm: K before its scale goes to the staging buffer behind the cache)
          const uint32_t base = isq ? (uint32_t)(row * pl.nq * d + hq * d)
                                    : (qkn ? kvelems + (uint32_t)(((par * Rmax + row) * nkv + g) * d) : kvoff);
          const uint32_t tg = (isq || qkn) ? my_tag : kv_tag;
          if constexpr (BF) {
            st8x(r, (base + i0) * 4, u32x2{pack_bf16(y[0], y[2]), tg}, lqkv);
            st8x(r, (base + i0 + d / 2) * 4, u32x2{pack_bf16(y[1], y[3]), tg}, lqkv);
          } else {
            st16x(r, (base + i0) * 8, ll_pair(__float_as_uint(y[0]), __float_as_uint(y[2]), tg), lqkv);
            st16x(r, (base + i0 + d / 2) * 8, ll_pair(__float_as_uint(y[1]), __float_as_uint(y[3]), tg), lqkv);
          }
        } else {
          const int tih = lt - (gq + 1) * th;
          const rsrc_t rvc = make_rsrc(pl.vc, kvbytes);
          const uint32_t vo = (kvoff + 16 * tih + 4 * q) * ESZ * 2;
          if constexpr (BF) {
            st16x(rvc, vo, ll_pair(pack_bf16(acc0[0], acc0[1]), pack_bf16(acc0[2], acc0[3]), kv_tag), lqkv);
          } else {
            st16x(rvc, vo, ll_pair(__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), kv_tag), lqkv);
            st16x(rvc, vo + 16, ll_pair(__float_as_uint(acc0[2]), __float_as_uint(acc0[3]), kv_tag), lqkv);
          }
        }
      } else if constexpr (KIND == T_GU) {
        float m[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = acc0[v], uv = acc1[v];
          m[v] = (gv / (1.0f + expf(-gv))) * uv;
        }
        const uint32_t mbytes = sop_bytes<BF>(Rmax, pl.I);
        st_sop4<BF>(make_rsrc((uint8_t*)pl.mbuf + plane(l, p) * mbytes, mbytes), row, 16 * tk.tile + 4 * q, pl.I, m);
      }
    }
    if constexpr (KIND == T_HEAD) {
      if (epi_wave) {
        const int V = pl.V;
        const uint32_t n0 = slots;
        if (live) {
          const rsrc_t rz = make_rsrc(pl.zbuf, (uint32_t)Rmax * V * 8);
          st16c(rz, (uint32_t)(row * V + n0) * 8, ll_pair(__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), my_tag));
          st16c(rz, (uint32_t)(row * V + n0) * 8 + 16, ll_pair(__float_as_uint(acc0[2]), __float_as_uint(acc0[3]), my_tag));
          if (fr.logits)
            st16(make_rsrc(fr.logits, (uint32_t)rows * (P - 1) * V * 4), (uint32_t)((row * (P - 1) + (p - 1)) * V + n0) * 4,
                 u32x4{__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), __float_as_uint(acc0[2]), __float_as_uint(acc0[3])});
        }
        // best (value, index) of the tile for this row
        float bv = acc0[0];
        uint32_t bi = n0;
#pragma unroll
        for (int v = 1; v < 4; ++v)
          if (beats(acc0[v], n0 + v, bv, bi)) { bv = acc0[v]; bi = n0 + v; }
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
          const float ov = shfl_xor_f(bv, m);
          const uint32_t oi = (uint32_t)__shfl_xor((int)bi, m, 64);
          if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (live && q == 0)
          st16c(make_rsrc(pl.cand, (uint32_t)Rmax * pl.n_head_tiles * 16), (uint32_t)(row * pl.n_head_tiles + tk.tile) * 16,
                ll_pair(__float_as_uint(bv), bi, my_tag));
      }
    }
  }

  stamp(tr, 5);
}

// ------------------------------------------------------------------ attention

// One kv head g for a group of rows: every (row, q head of g) pair is one
// wave's work.  Scores: lane (t, c) takes position t and a quarter c of the
// head dimension; softmax over t <= p in float; output: lane owns d/64 dims.
template <int BF, int D, bool ASM, bool NOQK = false>
__device__ __forceinline__ void attn_task(const DevPlan& pl, const DevFrame& fr, const DevTask& tk, uint32_t epoch,
                                          uint64_t* tr) {
  constexpr int ESZ = BF ? 2 : 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int d = D;  // head dim (64 or 128; the plan refuses others)
  const int gq = pl.gq, nkv = pl.nkv, P = pl.P, Rmax = pl.Rmax;
  const int l = tk.layer, p = tk.pos;
  const int ngroups = Rmax / pl.attn_rows;
  const int g = tk.tile / ngroups, rg = tk.tile % ngroups;
  const int npairs = pl.attn_rows * gq;
  const uint32_t qdbytes = (uint32_t)Rmax * pl.nq * d * ESZ * 2;
  const rsrc_t rq = make_rsrc((uint8_t*)pl.qbuf + (size_t)(p & 1) * qdbytes, qdbytes);
  const uint32_t kvbytes = (uint32_t)pl.L * Rmax * nkv * P * d * ESZ * 2;
  // QK-norm: this position's K comes unscaled from the staging buffer behind
  // the cache, with the per-tile sums of squares of the q and k heads
  const bool qkn = !NOQK && pl.qk_norm;
  const uint32_t krbytes = qkn ? (uint32_t)2 * Rmax * nkv * d * ESZ * 2 : 0u;
  const rsrc_t rk = make_rsrc(pl.kc, kvbytes + krbytes), rv = make_rsrc(pl.vc, kvbytes);
  const int th = d / 16, nh = pl.nq + nkv;
  const rsrc_t rn = make_rsrc(pl.qkn, qkn ? (uint32_t)2 * Rmax * nh * th * 8 : 0u);
  const uint32_t abytes = sop_bytes<BF>(Rmax, pl.nq * d);  // attention output, operand order for o
  const rsrc_t ra = make_rsrc((uint8_t*)pl.abuf + (size_t)(l * P + p) * abytes, abytes);
  const uint32_t q_tag = tag_of(epoch, tk.ph_in0), kv_tag = tag_of(epoch, kKvPhase);
  const uint32_t my_tag = tag_of(epoch, tk.phase);
  const int t = lane >> 2, c = lane & 3;
  constexpr int dq = d / 4;              // dims per score lane
  constexpr int nld = dq * ESZ * 2 / 16; // 16-byte tagged loads per score lane (4, 8 or 16)
  constexpr int dpl = d / 64;            // output dims per lane (1 or 2)
  for (int pi = wave; pi < npairs; pi += 4) {
    const int row = rg * pl.attn_rows + pi / gq;
    const int hq = g * gq + pi % gq;
    if (row >= fr.rows) continue;  // wave-uniform
    const uint32_t kvrow = (uint32_t)((l * Rmax + row) * nkv + g) * P;
    // Q and K of this lane's quarter of the head dims
    constexpr int NQ = BF ? 8 : 16;  // 16-byte tagged loads per score lane at most
    u32x4 qv[NQ], kv[NQ];
    // (chunk i of lane quarter c is the head's 16-byte unit 4 i + c: one
    // load instruction reads 64 contiguous bytes of each position's K row,
    // not 16 bytes of 64 different cache lines)
    const uint32_t q0 = ((uint32_t)(row * pl.nq * d + hq * d)) * ESZ * 2 + c * 16;
    const uint32_t k0 = ((uint32_t)((kvrow + t) * d)) * ESZ * 2 + c * 16;
    auto qo = [=](int i) { return q0 + i * 64; };
    // (loads without branches: units past nld repeat the last one and
    // positions past p read position p; neither is part of the wait)
    const uint32_t kclamp = (uint32_t)(min(t, p) - t) * (uint32_t)(d * ESZ * 2);
    // QK-norm: position p (and the clamped lanes past it) read the staging
    // buffer, written by the qkv phase with its tag
    const bool rawk = qkn && t >= p;
    const uint32_t kr0 = kvbytes + ((uint32_t)((((p & 1) * Rmax + row) * nkv + g) * d)) * ESZ * 2 + c * 16;
    auto ko = [=](int i) { return rawk ? kr0 + i * 64 : k0 + kclamp + i * 64; };
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int iu = i < nld ? i : nld - 1;
      qv[i] = ld16c(rq, qo(iu));
      kv[i] = ld16c(rk, ko(iu));
    }
    // QK-norm: the head's per-tile sums of squares, q head hq and kv head g
    // (every lane the same words)
    u32x4 qs[4] = {}, ks[4] = {};
    const uint32_t qn0 = (uint32_t)((((p & 1) * Rmax + row) * nh + hq) * th) * 8;
    const uint32_t kn0 = (uint32_t)((((p & 1) * Rmax + row) * nh + pl.nq + g) * th) * 8;
    auto qso = [=](int i) { return qn0 + i * 16; };
    auto kso = [=](int i) { return kn0 + i * 16; };
    if (qkn) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int iu = i < th / 2 ? i : th / 2 - 1;
        qs[i] = ld16c(rn, qso(iu));
        ks[i] = ld16c(rn, kso(iu));
      }
    }
    // V of this lane's dims for every t <= p: the word holding them (bf16),
    // or the aligned pair of words (fp32)
    const uint32_t vrow = (uint32_t)(d * ESZ * 2);
    const uint32_t v0 = ((uint32_t)(kvrow * d + lane * dpl) * ESZ * 2) & (BF ? ~7u : ~15u);
    auto vo = [=](int tt) { return v0 + tt * vrow; };
    u32x2 vw[16];
    u32x4 vv[BF ? 1 : 16];
    // (every position is loaded, so the loads issue without branches; those
    // past p stay out of the wait and are masked below)
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const uint32_t o = vo(min(tt, P - 1));
      if constexpr (BF) vw[tt] = __builtin_amdgcn_raw_buffer_load_b64(rv, o, 0, kSC1);
      else vv[tt] = ld16c(rv, o);
    }
    // Q and K (this position's from the qkv phase just before, earlier ones
    // long ready) and V, all in one wait.  Every set reloads in asm, the
    // QK-norm partials too: a compiler-issued reload in the wait loop, even
    // one that never runs, measured 30 us slower per 64-row frame.
    const uint32_t k_tag = rawk ? q_tag : kv_tag;
    if constexpr (BF)
      await_all(pl, pend<ASM>(qv, rq, qo, q_tag, true, nld), pend<ASM>(kv, rk, ko, k_tag, t <= p, nld),
                pend<ASM>(vw, rv, vo, kv_tag, true, p + 1), pend<ASM>(qs, rn, qso, q_tag, qkn, th / 2),
                pend<ASM>(ks, rn, kso, q_tag, qkn, th / 2));
    else
      await_all(pl, pend<ASM>(qv, rq, qo, q_tag, true, nld), pend<ASM>(kv, rk, ko, k_tag, t <= p, nld),
                pend<ASM>(vv, rv, vo, kv_tag, true, p + 1), pend<ASM>(qs, rn, qso, q_tag, qkn, th / 2),
                pend<ASM>(ks, rn, kso, q_tag, qkn, th / 2));
    if (qkn) {
      // 1 / rms of the q head and of the k head (partials in tile order),
      // then Q and this position's K scaled and rounded as stored; the
      // row's first q head writes that K into the cache for later positions
      float ssq = 0.f, ssk = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < th / 2) {
          ssq = (ssq + __uint_as_float(qs[i][0])) + __uint_as_float(qs[i][2]);
          ssk = (ssk + __uint_as_float(ks[i][0])) + __uint_as_float(ks[i][2]);
        }
      const float rnq = 1.0f / sqrtf(ssq / (float)d + pl.eps), rnk = 1.0f / sqrtf(ssk / (float)d + pl.eps);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        qv[i] = scale_pair<BF>(qv[i], rnq);
        if (t == p) kv[i] = scale_pair<BF>(kv[i], rnk);
      }
      if (t == p && pi % gq == 0) {
#pragma unroll
        for (int i = 0; i < NQ; ++i)
          if (i < nld) st16c(rk, k0 + i * 64, ll_pair(kv[i][0], kv[i][2], kv_tag));
      }
    }
    if (pi < 4) stamp(tr, 2);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      if (i < nld) {
        const u32x4 qp = {qv[i][0], qv[i][2], 0, 0}, kp = {kv[i][0], kv[i][2], 0, 0};
#pragma unroll
        for (int e = 0; e < 8 / ESZ; ++e) dot += chunk_elem<BF>(qp, e) * chunk_elem<BF>(kp, e);
      }
    dot += quad_xor_f<1>(dot);
    dot += quad_xor_f<2>(dot);
    const float s = (t <= p) ? dot * pl.attn_scale : -INFINITY;
    // max and sum over the 16 positions (lanes 4t hold position t's values)
    float m = lane_f(s, 0);
#pragma unroll
    for (int tt = 1; tt < 16; ++tt) m = fmaxf(m, lane_f(s, tt * 4));
    const float e = (t <= p) ? expf(s - m) : 0.f;
    float sum = lane_f(e, 0);
#pragma unroll
    for (int tt = 1; tt < 16; ++tt) sum += lane_f(e, tt * 4);
    const float w = e / sum;
    // output: sum over t in ascending order
    // (positions past p add an exact 0: weight and value both selected to 0)
    float o0 = 0.f, o1 = 0.f;
    const int wsel = (lane * dpl) & 1;  // fp32, one dim per lane: which word of the pair
    float wv[16];
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) wv[tt] = lane_f(w, tt * 4);
    if (dpl == 2) {
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const bool on = tt <= p;
        const float wt = on ? wv[tt] : 0.f;
        float v0, v1;
        if constexpr (BF) {
          v0 = bf2f(vw[tt][0] & 0xffffu);
          v1 = bf2f(vw[tt][0] >> 16);
        } else {
          v0 = __uint_as_float(vv[tt][0]);
          v1 = __uint_as_float(vv[tt][2]);
        }
        o0 += wt * (on ? v0 : 0.f);
        o1 += wt * (on ? v1 : 0.f);
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const bool on = tt <= p;
        const float wt = on ? wv[tt] : 0.f;
        float v0;
        if constexpr (BF) v0 = bf2f((lane & 1) ? (vw[tt][0] >> 16) : (vw[tt][0] & 0xffffu));
        else v0 = __uint_as_float(vv[tt][wsel * 2]);
        o0 += wt * (on ? v0 : 0.f);
      }
    }
    const int an = hq * d + lane * dpl;  // first output column of this lane
    const uint32_t ao = sop_off<BF>(row, an, pl.nq * d);
    if constexpr (BF) {
      if (dpl == 2) {
        st4c(ra, ao, sop_canon<1>(pack_bf16(o0, o1)));
      } else {
        // two lanes share a dword: the even lane writes both dims
        const float o_nb = __shfl_xor(o0, 1, 64);
        if ((lane & 1) == 0) st4c(ra, ao, sop_canon<1>(pack_bf16(o0, o_nb)));
      }
    } else {
      if (dpl == 2) st8c(ra, ao, u32x2{sop_canon<0>(__float_as_uint(o0)), sop_canon<0>(__float_as_uint(o1))});
      else st4c(ra, ao, sop_canon<0>(__float_as_uint(o0)));
    }
  }
  stamp(tr, 5);
}

// ------------------------------------------------------------------ draw + embed

// Writes embedding row `code` of table j as the input of position j + 1 (when
// there is one, in operand order) and adds it to the row's fp32 embedding sum.  All draws of a row run in one workgroup, so the
// sum is carried in program order with ordinary loads and stores.
template <int BF>
__device__ __forceinline__ void embed_row(const DevPlan& pl, const DevFrame& fr, int j, int row, int code,
                                          bool first) {
  constexpr int ESZ = BF ? 2 : 4;
  const int H = pl.H, V = pl.V;
  const rsrc_t re = make_rsrc(pl.embed, (uint32_t)pl.P * V * H * ESZ);
  const rsrc_t rs = make_rsrc(fr.embsum, (uint32_t)fr.rows * H * 4);
  const uint32_t hbytes = sop_bytes<BF>(pl.Rmax, H);
  const rsrc_t rx = make_rsrc((uint8_t*)pl.xin + (size_t)(j + 1) * hbytes, hbytes);
  const uint32_t ebase = (uint32_t)((j * V + code) * H);
  const bool feeds = j + 1 < pl.P;  // the row is the input of position j + 1
  // thread t covers elements 4t .. 4t+3: four threads per 16-column tile
  for (int k = threadIdx.x * 4; k < ((H + 1023) / 1024) * 1024; k += kThreads * 4) {
    const bool in = k < H;
    // (both loads without branches, so they go out together; past H the
    // last four elements are read again and not used)
    const int kc = in ? k : H - 4;
    float ev[4];
    if constexpr (BF) {
      const u32x2 e = ld8(re, (ebase + kc) * 2);
      ev[0] = bf2f(e[0] & 0xffffu); ev[1] = bf2f(e[0] >> 16); ev[2] = bf2f(e[1] & 0xffffu); ev[3] = bf2f(e[1] >> 16);
    } else {
      const u32x4 e = ld16(re, (ebase + kc) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) ev[i] = __uint_as_float(e[i]);
    }
    u32x4 sv = ld16(rs, (uint32_t)(row * H + kc) * 4);  // (not used by the first embedding)
    if (!in) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ev[i] = 0.f;
    }
    if (in && feeds) st_sop4<BF>(rx, row, k, H, ev);
    if (in) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = __float_as_uint(first ? ev[i] : __uint_as_float(sv[i]) + ev[i]);
      st16(rs, (uint32_t)(row * H + k) * 4, sv);
    }
  }
}

template <int BF>
__device__ __forceinline__ void embed0_task(const DevPlan& pl, const DevFrame& fr, const DevTask& tk, uint32_t epoch,
                                            uint64_t* tr) {
  const int row = (int)tk.tile;
  if (row < fr.rows) {
    int code = fr.code0[row];
    code = code < 0 ? 0 : (code >= pl.V ? pl.V - 1 : code);
    embed_row<BF>(pl, fr, 0, row, code, true);
  }
  stamp(tr, 5);
}

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds, each two 64 x 64 -> 128-bit products
// whose halves are mixed with the other two words and the key, then a Weyl
// step of the key.  Returns word 0 of the output block.
__device__ __forceinline__ uint64_t philox4x64_w0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                  uint64_t k1) {
  constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull, kMul1 = 0xCA5A826395121157ull;
  constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull, kWeyl1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kMul0, c0), lo0 = kMul0 * c0;
    const uint64_t hi1 = __umul64hi(kMul1, c2), lo1 = kMul1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += kWeyl0; k1 += kWeyl1;
  }
  return c0;
}

// Sort key of a scaled logit: larger value first, then lower index.  -0 is
// taken as +0 so that equal values tie on the index alone.
__device__ __forceinline__ uint64_t rank_key(float y, uint32_t i) {
  uint32_t u = __float_as_uint(y == 0.0f ? 0.0f : y);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(~i);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t u = (uint32_t)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~(uint32_t)k; }

// Bitonic compare-exchange helpers for the sampler's sort (descending keys).
// `keep_max`: this side of the pair keeps the larger key.
__device__ __forceinline__ uint64_t cx_pick(uint64_t mine, uint64_t other, bool keep_max) {
  return keep_max ? (mine > other ? mine : other) : (mine < other ? mine : other);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Sorts the block's Vp = 256 * NE keys descending; thread t holds elements
// t * NE .. t * NE + NE - 1 in k[], and ends holding ranks in the same places.
// Strides below NE stay in registers, strides below 64 * NE use wave
// shuffles, larger strides go through LDS (xch: Vp keys).
template <int NE>
__device__ __forceinline__ void block_sort_desc(uint64_t (&k)[NE], int Vp, uint64_t* xch) {
  const int tid = threadIdx.x;
  for (int kb = 2; kb <= Vp; kb <<= 1) {
    for (int h = kb >> 1; h > 0; h >>= 1) {
      if (h < NE) {
        // in registers: one compile-time stride per branch, so k[] stays in VGPRs
#pragma unroll
        for (int hh = NE / 2; hh >= 1; hh >>= 1) {
          if (hh == h) {
#pragma unroll
            for (int e = 0; e < NE; ++e) {
              if ((e & hh) == 0) {
                const bool desc = ((tid * NE + e) & kb) == 0;
                const uint64_t a = k[e], b = k[e + hh];
                const bool swap = desc ? (a < b) : (a > b);
                k[e] = swap ? b : a;
                k[e + hh] = swap ? a : b;
              }
            }
          }
        }
      } else if (h < 64 * NE) {
        const int lm = h / NE;  // lane distance
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int i = tid * NE + e;
          const bool desc = (i & kb) == 0, low = (tid & lm) == 0;
          k[e] = cx_pick(k[e], shfl_xor_u64(k[e], lm), desc == low);
        }
      } else {
        const int tm = h / NE;  // thread distance
        __syncthreads();
#pragma unroll
        for (int e = 0; e < NE; ++e) xch[tid * NE + e] = k[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int i = tid * NE + e;
          const bool desc = (i & kb) == 0, low = (tid & tm) == 0;
          k[e] = cx_pick(k[e], xch[(tid ^ tm) * NE + e], desc == low);
        }
      }
    }
  }
}

// Exclusive prefix sum over the block (thread order) and the block total.
// red: 8 doubles of LDS.
__device__ __forceinline__ double block_exscan(double v, double* red, double& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const double t = red[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// The kk largest of the block's keys (kk < 256 NE), sorted descending into
// xch[0 .. kk) and into ranks tid * NE + e < kk of k.  The kk-th largest key
// is found a byte at a time from the top, with exact counts per byte value
// (it stops as soon as a whole byte class is kept); the kept keys are then
// ranked by counting the larger ones (keys are distinct: they carry the
// index).  tmp: kk keys, hist: 260 words, red: as block_exscan.
template <int NE>
__device__ __forceinline__ void block_topk_desc(uint64_t (&k)[NE], int kk, uint64_t* xch, uint64_t* tmp,
                                                uint32_t* hist, double* red) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)kk;
  for (int b = 7; b >= 0; --b) {
    hist[tid] = 0;  // one bin per thread
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if ((k[e] & pmask) == prefix) atomicAdd(&hist[(uint32_t)(k[e] >> (8 * b)) & 255u], 1u);
    __syncthreads();
    // thread t takes bin 255 - t: thread order is descending key order
    const uint32_t c = hist[255 - tid];
    double total;
    const uint32_t before = (uint32_t)block_exscan((double)c, red, total);
    if (before < remaining && remaining <= before + c) {
      hist[256] = 255u - (uint32_t)tid;
      hist[257] = before;
      hist[258] = c;
    }
    __syncthreads();
    const uint32_t bin = hist[256], nbefore = hist[257], nclass = hist[258];
    __syncthreads();
    prefix |= (uint64_t)bin << (8 * b);
    pmask |= 0xFFull << (8 * b);
    remaining -= nbefore;
    if (remaining == nclass) break;  // the whole class is kept
  }
  // exactly kk keys are >= prefix
  if (tid == 0) hist[259] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < NE; ++e)
    if (k[e] >= prefix) tmp[atomicAdd(&hist[259], 1u)] = k[e];
  __syncthreads();
  if (tid < kk) {
    const uint64_t key = tmp[tid];
    int r = 0;
    for (int j = 0; j < kk; ++j) r += tmp[j] > key ? 1 : 0;
    xch[r] = key;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < NE; ++e) k[e] = tid * NE + e < kk ? xch[tid * NE + e] : 0ull;
}

// Block minimum of an int.  red: 4 words of LDS.
__device__ __forceinline__ int block_min_int(int v, uint32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = min(v, __shfl_xor(v, m, 64));
  if (lane == 0) red[wave] = (uint32_t)v;
  __syncthreads();
  int r = (int)red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = min(r, (int)red[w]);
  __syncthreads();
  return r;
}

// Block maximum of (score, index): larger score, then lower index.
__device__ __forceinline__ uint32_t block_argmax(double sc, uint32_t idx, double* red, uint32_t* redi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const double os = __shfl_xor(sc, m, 64);
    const uint32_t oi = (uint32_t)__shfl_xor((int)idx, m, 64);
    if (os > sc || (os == sc && oi < idx)) { sc = os; idx = oi; }
  }
  if (lane == 0) { red[wave] = sc; redi[wave] = idx; }
  __syncthreads();
  double bs = red[0];
  uint32_t bi = redi[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w)
    if (red[w] > bs || (red[w] == bs && redi[w] < bi)) { bs = red[w]; bi = redi[w]; }
  __syncthreads();
  return bi;
}

// Sampled draw of one row (the row's whole workgroup), in the order the
// sampler is defined: y = z / T; the top-k largest y (ties to the lower
// index; k <= 0 or k >= V keeps all); softmax over them; top-p keeps the
// shortest rank-order prefix whose mass reaches p (the crossing token
// included; p >= 1 keeps all, p <= 0 the first); then Gumbel-max: the code is
// the kept i with the largest y_i - log(-log u_i), u_i from Philox4x64-10 with
// key (seed, 0) and counter (offset + j - 1, i, 0, 0): the top 23 bits m of
// word 0 give u = (2m + 1) / 2^24.  T <= 0 is a greedy draw on z.
// z: this thread's NE logits, element index threadIdx.x * NE + e (V = 256 NE).
// lds_scratch: the LDS scratch (at most V * 8 + 128 + 12 KiB is used).
// Kept out of line: it runs once per draw and would otherwise add to the
// register pressure of every task body.
template <int NE>
struct ZRow {
  float v[NE];
};
struct DrawArgs {
  float T, top_p;
  int top_k;
  uint64_t seed, ctr;  // Philox key word 0 and counter word 0 of this draw
};
// A byte in LDS.  The sampler's out-of-line functions take their scratch as
// this type: through a generic pointer argument every access would be a FLAT
// access, which waits on both memory counters.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
// 64-bit v from lane ^ 1 (CTRL 0xB1) or lane ^ 2 (0x4E), by DPP.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u<CTRL>((uint32_t)v);
}

// The Gumbel-max code of one row for top-k cuts of at most 64 keys, or -1
// (the same in every thread) when the candidates below are too many and the
// caller has to select in full.  k[]: the row's sort keys, as in
// block_sort_desc.  The kk-th largest of the 64 quad maxima (the largest key
// of each four threads) is a floor for the kk-th largest key, since kk
// distinct keys reach it; only keys at or above it can be kept.  For logits
// in no particular order they are about twice kk; up to 256 of them are
// ranked by counting.  Then one wave computes the top-p prefix while another
// computes the Gumbel noise of the kept ranks, one rank per lane.  The result
// is the one the full selection gives.  (Out of line: inlined into the
// sampler it changed the register allocation of the executors' task bodies,
// which then ran slower.)
template <int NE>
__device__ __noinline__ int small_k_code(const uint64_t (&k)[NE], int kk, const DrawArgs& da, lds_u8* lds_scratch) {
  uint8_t* scratch = (uint8_t*)lds_scratch;
  constexpr int kCand = kThreads;  // candidate list size
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t* xch = (uint64_t*)scratch;               // ranks 0 .. kk-1
  double* noise = (double*)(scratch + 512);         // their Gumbel noise
  uint64_t* qmx = (uint64_t*)(scratch + 1024);      // the 64 quad maxima
  uint64_t* floor_key = (uint64_t*)(scratch + 1536);
  uint32_t* cnt = (uint32_t*)(scratch + 1544);      // [0] candidates, [1] the code
  uint64_t* cand = (uint64_t*)(scratch + 2048);     // kCand + 16 keys, zero-padded
  uint64_t mx = k[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) mx = k[e] > mx ? k[e] : mx;
  uint64_t o = dpp_u64<0xB1>(mx);
  mx = o > mx ? o : mx;
  o = dpp_u64<0x4E>(mx);
  mx = o > mx ? o : mx;
  if ((lane & 3) == 0) qmx[tid >> 2] = mx;
  cand[tid] = 0;  // zero keys count as smaller than every key
  if (tid < 16) cand[kCand + tid] = 0;
  if (tid == 0) cnt[0] = 0;
  __syncthreads();
  if (wave == 0) {  // the kk-th largest quad maximum (they are distinct)
    const uint64_t x = qmx[lane];
    const u32x4* mv = (const u32x4*)qmx;
    int above = 0;
#pragma unroll
    for (int j0 = 0; j0 < 32; j0 += 16) {
      u32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = mv[j0 + u];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint64_t a = ((uint64_t)v[u][1] << 32) | v[u][0], c = ((uint64_t)v[u][3] << 32) | v[u][2];
        above += (a > x ? 1 : 0) + (c > x ? 1 : 0);
      }
    }
    if (above == kk - 1) floor_key[0] = x;
  }
  __syncthreads();
  const uint64_t fl = floor_key[0];
#pragma unroll
  for (int e = 0; e < NE; ++e)
    if (k[e] >= fl) {
      const uint32_t at = atomicAdd(cnt, 1u);
      if (at < (uint32_t)kCand) cand[at] = k[e];
    }
  __syncthreads();
  const int C = (int)cnt[0];
  if (C > kCand) return -1;
  if (tid < C) {
    // rank among the candidates, 16 keys a step (the zero padding past C
    // counts for nothing)
    const uint64_t key = cand[tid];
    const u32x4* cv = (const u32x4*)cand;
    int r = 0;
    for (int j0 = 0; j0 < C; j0 += 16) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = cv[j0 / 2 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint64_t a = ((uint64_t)v[u][1] << 32) | v[u][0], c = ((uint64_t)v[u][3] << 32) | v[u][2];
        r += (a > key ? 1 : 0) + (c > key ? 1 : 0);
      }
    }
    if (r < kk) xch[r] = key;
  }
  __syncthreads();
  const float pp = da.top_p;
  int n_keep = kk;
  uint64_t key = 0;
  if (wave == 0) {
    key = lane < kk ? xch[lane] : 0ull;
    if (pp <= 0.0f) {
      n_keep = 1;
    } else if (pp < 1.0f) {  // softmax weights relative to the largest y, fp64, rank order
      const double ymax = (double)key_value(xch[0]);
      const double w = lane < kk ? exp((double)key_value(key) - ymax) : 0.0;
      double cum = w;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const double y = __shfl_up(cum, d, 64);
        if (lane >= d) cum += y;
      }
      const double Z = __shfl(cum, 63, 64);
      const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < kk && cum / Z >= (double)pp);
      if (hit) n_keep = __ffsll((unsigned long long)hit);  // the first crossing rank, included
    }
  } else if (wave == 1 && lane < kk) {
    // -log(-log u) of rank `lane`, u from word 0 of the token's Philox block
    const uint64_t m = philox4x64_w0(da.ctr, (uint64_t)key_index(xch[lane]), 0, 0, da.seed, 0) >> 41;
    const double u = (double)(2 * m + 1) * (1.0 / 16777216.0);
    noise[lane] = -log(-log(u));
  }
  __syncthreads();
  if (wave == 0) {
    double sc = -INFINITY;
    uint32_t bi = 0xffffffffu;
    if (lane < n_keep) {
      bi = key_index(key);
      sc = (double)key_value(key) + noise[lane];
    }
    wave_tree([&](auto other) {
      const uint64_t sb = (uint64_t)__double_as_longlong(sc);
      const double os = __longlong_as_double(
          (long long)(((uint64_t)other((uint32_t)(sb >> 32)) << 32) | other((uint32_t)sb)));
      const uint32_t oi = other(bi);
      if (os > sc || (os == sc && oi < bi)) { sc = os; bi = oi; }
    });
    if (lane == 0) cnt[1] = bi;
  }
  __syncthreads();
  return (int)cnt[1];
}

template <int NE>
__device__ __noinline__ int sampled_code(ZRow<NE> zr, DrawArgs da, lds_u8* lds_scratch) {
  uint8_t* scratch = (uint8_t*)lds_scratch;
  const int V = kThreads * NE;
  uint64_t* xch = (uint64_t*)scratch;
  double* red = (double*)(scratch + (size_t)V * 8);
  uint32_t* redi = (uint32_t*)(red + 8);
  const float* z = zr.v;
  const float T = da.T;
  const int tid = threadIdx.x;
  if (!(T > 0.0f)) {  // greedy on z: the largest value, lowest index
    double bs = -INFINITY;
    uint32_t bi = 0xffffffffu;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if ((double)z[e] > bs) { bs = (double)z[e]; bi = (uint32_t)(tid * NE + e); }
    return (int)block_argmax(bs, bi, red, redi);
  }
  // keys of y = z / T (IEEE division), sorted descending: rank tid * NE + e
  uint64_t k[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) k[e] = rank_key(z[e] / T, (uint32_t)(tid * NE + e));
  const int tk = da.top_k;
  const int kk = (tk <= 0 || tk >= V) ? V : tk;
  if (kk <= 64) {
    const int code = small_k_code<NE>(k, kk, da, (lds_u8*)scratch);
    if (code >= 0) return code;
  }
  if (kk < kThreads) {
    // only the top kk ranks matter: select them instead of sorting all V
    uint64_t* tmp = (uint64_t*)(scratch + (size_t)V * 8 + 128);
    uint32_t* hist = (uint32_t*)(scratch + (size_t)V * 8 + 128 + kThreads * 8);
    block_topk_desc<NE>(k, kk, xch, tmp, hist, red);
  } else {
    block_sort_desc<NE>(k, V, xch);
  }
  const float pp = da.top_p;
  // ranks to LDS: the Gumbel step deals them round-robin over the block (the
  // kept ranks are the first few, which one thread would otherwise hold)
  __syncthreads();
#pragma unroll
  for (int e = 0; e < NE; ++e) xch[tid * NE + e] = k[e];
  __syncthreads();
  int n_keep = kk;
  if (pp <= 0.0f) {
    n_keep = 1;
  } else if (pp < 1.0f) {  // softmax weights relative to the largest y, fp64
    const double ymax = (double)key_value(xch[0]);
    double w[NE], wsum = 0.0;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      w[e] = (tid * NE + e < kk) ? exp((double)key_value(k[e]) - ymax) : 0.0;
      wsum += w[e];
    }
    double Z;
    double cum = block_exscan(wsum, red, Z);
    int first = 0x7fffffff;  // first rank whose cumulative mass reaches p
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      cum += w[e];
      if (first == 0x7fffffff && tid * NE + e < kk && cum / Z >= (double)pp) first = tid * NE + e;
    }
    const int fmin = block_min_int(first, redi);
    if (fmin < kk) n_keep = fmin + 1;
  }
  // Gumbel-max over the kept ranks
  const uint64_t seed = da.seed, ctr = da.ctr;
  double best_s = -INFINITY;
  uint32_t best_i = 0xffffffffu;
  for (int r = tid; r < n_keep; r += kThreads) {
    const uint64_t key = xch[r];
    const uint32_t i = key_index(key);
    const uint64_t m = philox4x64_w0(ctr, (uint64_t)i, 0, 0, seed, 0) >> 41;
    const double u = (double)(2 * m + 1) * (1.0 / 16777216.0);
    const double sc = (double)key_value(key) - log(-log(u));
    if (sc > best_s || (sc == best_s && i < best_i)) { best_s = sc; best_i = i; }
  }
  return (int)block_argmax(best_s, best_i, red, redi);
}

// The row's V = 256 NE logits (tagged words from the head tiles; thread t
// takes elements t NE .. t NE + NE - 1) and its sampled code.
template <int NE>
__device__ __forceinline__ int sampled_row(const DevPlan& pl, const DevFrame& fr, int row, int j, uint32_t in_tag,
                                           uint8_t* scratch, uint64_t* tr) {
  const rsrc_t rz = make_rsrc(pl.zbuf, (uint32_t)pl.Rmax * pl.V * 8);
  const uint32_t zb = (uint32_t)(row * pl.V + threadIdx.x * NE) * 8;
  float z[NE];
  if constexpr (NE == 1) {
    u32x2 zw[1];
    auto zo = [=](int) -> uint32_t { return zb; };
    zw[0] = __builtin_amdgcn_raw_buffer_load_b64(rz, zb, 0, kSC1);
    await_all(pl, pend(zw, rz, zo, in_tag, true));
    stamp(tr, 2);
    z[0] = __uint_as_float(zw[0][0]);
  } else {
    u32x4 zw[NE / 2];
    auto zo = [=](int u) -> uint32_t { return zb + u * 16; };
#pragma unroll
    for (int u = 0; u < NE / 2; ++u) zw[u] = ld16c(rz, zo(u));
    await_all(pl, pend(zw, rz, zo, in_tag, true));
    stamp(tr, 2);
#pragma unroll
    for (int e = 0; e < NE; ++e) z[e] = __uint_as_float(zw[e >> 1][(e & 1) * 2]);
  }
  ZRow<NE> zr;
#pragma unroll
  for (int e = 0; e < NE; ++e) zr.v[e] = z[e];
  const DrawArgs da = {fr.temperature[row], fr.top_p[row], fr.top_k[row], fr.seed[row],
                       fr.offset[row] + (uint64_t)(j - 1)};
  return sampled_code<NE>(zr, da, (lds_u8*)scratch);
}

template <int BF, bool ASM>
__device__ __forceinline__ void draw_task(const DevPlan& pl, const DevFrame& fr, const DevTask& tk, uint32_t epoch,
                                          uint8_t* slot, uint32_t* misc, uint64_t* tr) {
  const int row = (int)tk.tile, p = tk.pos;
  const uint32_t in_tag = tag_of(epoch, tk.ph_in0);
  if (row < fr.rows && fr.sampled) {
    int code;
    switch (pl.V) {
      case 256: code = sampled_row<1>(pl, fr, row, p, in_tag, slot, tr); break;
      case 512: code = sampled_row<2>(pl, fr, row, p, in_tag, slot, tr); break;
      case 1024: code = sampled_row<4>(pl, fr, row, p, in_tag, slot, tr); break;
      case 2048: code = sampled_row<8>(pl, fr, row, p, in_tag, slot, tr); break;
      default: code = sampled_row<16>(pl, fr, row, p, in_tag, slot, tr); break;
    }
    code = (code < 0 || code >= pl.V) ? 0 : code;
    if (threadIdx.x == 0) {
      st4(make_rsrc(fr.codes, (uint32_t)fr.rows * (pl.P - 1) * 4), (uint32_t)(row * (pl.P - 1) + p - 1) * 4,
          (uint32_t)code);
      if (p == pl.P - 1) {  // the frame's draws of this row are done: advance its offset
        const uint64_t o = fr.offset[row] + (uint64_t)(pl.P - 1);
        st8c(make_rsrc(fr.offset, (uint32_t)fr.rows * 8), (uint32_t)row * 8, u32x2{(uint32_t)o, (uint32_t)(o >> 32)});
      }
    }
    embed_row<BF>(pl, fr, p, row, code, false);
  } else if (row < fr.rows) {
    if (threadIdx.x < 64) {
      // the head tiles' (value, index) candidates of this row, tile order
      const int lane = threadIdx.x;
      const rsrc_t rc = make_rsrc(pl.cand, (uint32_t)pl.Rmax * pl.n_head_tiles * 16);
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      for (int i0 = 0; i0 < pl.n_head_tiles; i0 += 64 * 4) {
        u32x4 cv[4];
        const uint32_t cbase = (uint32_t)(row * pl.n_head_tiles + i0 + lane) * 16;
        auto co = [=](int k) { return cbase + k * 64 * 16; };
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = i0 + k * 64 + lane;
          cv[k] = i < pl.n_head_tiles ? ld16c(rc, co(k)) : u32x4{0, in_tag, 0xffffffffu, in_tag};
        }
        await_all(pl, pend<ASM>(cv, rc, co, in_tag, true, (pl.n_head_tiles - i0 - lane + 63) / 64));
        if (i0 == 0) stamp(tr, 2);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = i0 + k * 64 + lane;
          if (i < pl.n_head_tiles && beats(__uint_as_float(cv[k][0]), cv[k][2], bv, bi)) {
            bv = __uint_as_float(cv[k][0]);
            bi = cv[k][2];
          }
        }
      }
      wave_tree([&](auto other) {
        const float ov = __uint_as_float(other(__float_as_uint(bv)));
        const uint32_t oi = other(bi);
        if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      });
      if (lane == 0) {
        misc[1] = bi < (uint32_t)pl.V ? bi : 0u;
        st4(make_rsrc(fr.codes, (uint32_t)fr.rows * (pl.P - 1) * 4), (uint32_t)(row * (pl.P - 1) + p - 1) * 4, misc[1]);
      }
    }
    __syncthreads();
    embed_row<BF>(pl, fr, p, row, (int)misc[1], false);
  }
  stamp(tr, 5);
}

// ------------------------------------------------------------------ executors

// ONE: the executor was launched for a one-row frame (the densely loaded
// operand path; a separate kernel, so the many-row code is left as it is).
// PLAIN: the executor's plain form (head_dim 128 only: attention for head_dim
// 64 is not compiled into it, which keeps the kernel's code smaller).
template <int BF, bool ONE, bool PLAIN = false, bool NOQK = false>
// lcl: XCD-local hand-offs allowed in this frame.
__device__ __forceinline__ void run_task(const DevPlan& pl, const DevFrame& fr, const DevTask& tk, uint32_t epoch,
                                         uint8_t* slot, uint32_t* misc, uint64_t* tr, bool lcl) {
  switch (tk.type) {
    case T_ATTN:
      if (PLAIN || pl.d == 128) attn_task<BF, 128, !ONE, NOQK>(pl, fr, tk, epoch, tr);
      else attn_task<BF, 64, !ONE, NOQK>(pl, fr, tk, epoch, tr);
      break;
    case T_EMBED0: embed0_task<BF>(pl, fr, tk, epoch, tr); break;
    case T_DRAW: draw_task<BF, !ONE>(pl, fr, tk, epoch, slot, misc, tr); break;
// (one-row frames: only a task of row group 0 has the row)
#define CP_PROJ(K)                                                                                  \
  if constexpr (ONE) {                                                                              \
    if ((tk.flags >> kTaskGroupShift) == 0) proj_task<BF, K, ONE, !ONE, NOQK>(pl, fr, tk, epoch, slot, misc, tr, lcl, 0, 64); \
  } else if (pl.grp_rows) {                                                                         \
    const int r0 = (tk.flags >> kTaskGroupShift) * pl.grp_rows;                                     \
    if (r0 < fr.rows) proj_task<BF, K, ONE, !ONE, NOQK>(pl, fr, tk, epoch, slot, misc, tr, lcl, r0, pl.grp_rows); \
  } else {                                                                                          \
    for (int rh = 0; rh * 64 < fr.rows; ++rh)                                                       \
      proj_task<BF, K, ONE, !ONE, NOQK>(pl, fr, tk, epoch, slot, misc, tr, lcl, rh * 64, 64);  \
  }
    case T_QKV: CP_PROJ(T_QKV) break;
    case T_O: CP_PROJ(T_O) break;
    case T_GU: CP_PROJ(T_GU) break;
    case T_DOWN:
      if constexpr (ONE) {
        CP_PROJ(T_DOWN)
      } else {
        CP_PROJ(T_O)
      }
      break;
    case T_HEAD: CP_PROJ(T_HEAD) break;
#undef CP_PROJ
    default:
      if constexpr (ONE) {
        if ((tk.flags >> kTaskGroupShift) == 0) proj_task<BF, T_INPROJ, false, !ONE>(pl, fr, tk, epoch, slot, misc, tr, lcl, 0, 64);
      } else if (pl.grp_rows) {
        const int r0 = (tk.flags >> kTaskGroupShift) * pl.grp_rows;
        if (r0 < fr.rows) proj_task<BF, T_INPROJ, false, !ONE>(pl, fr, tk, epoch, slot, misc, tr, lcl, r0, pl.grp_rows);
      } else {
        for (int rh = 0; rh * 64 < fr.rows; ++rh)
          proj_task<BF, T_INPROJ, false, !ONE>(pl, fr, tk, epoch, slot, misc, tr, lcl, rh * 64, 64);
      }
      break;
  }
}

// Clears every tagged buffer; one whole workgroup.
__device__ __forceinline__ void clear_tagged(const DevPlan& pl) {
#pragma unroll
  for (int b = 0; b < kMaxClear; ++b) {
    if (b >= pl.n_clear) break;
    const uint64_t words = pl.clear[b].bytes / 8;
    uint64_t* w = (uint64_t*)pl.clear[b].p;
    for (uint64_t i = threadIdx.x; i < words; i += kThreads)
      __hip_atomic_store(w + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_vm();
  __syncthreads();
}

// Refills this workgroup's share (workgroup w of n) of the operand region
// with the sentinel, with agent-coherent 16-byte stores.
__device__ __forceinline__ void refill_operands(const DevPlan& pl, uint32_t w, uint32_t n) {
  const uint64_t units = pl.opbuf_bytes / 16;
  const uint64_t per = (units + n - 1) / n, u0 = (uint64_t)w * per;
  const uint64_t u1 = u0 + per < units ? u0 + per : units;
  uint8_t* base = (uint8_t*)pl.opbuf;
  for (uint64_t u = u0 + threadIdx.x; u < u1; u += kThreads) {
    // (one resource per 2 GiB window: buffer offsets are 32-bit)
    const uint64_t byte = u * 16, win = byte >> 31;
    const rsrc_t r = make_rsrc(base + (win << 31), 0x80000000u);
    st16c(r, (uint32_t)(byte - (win << 31)), u32x4{~0u, ~0u, ~0u, ~0u});
  }
}

// Moves the plan to the next frame's epoch.  Run by one whole workgroup once
// every task of the frame has finished.  When the next epoch would leave the
// tag space, every tagged buffer is cleared (a few milliseconds, once every
// four million frames) and the count restarts at 1, so no stale word can carry
// a tag a later frame expects.  With `defer` the clear is left to
// clear_pending_kernel, which runs after the frame's K/V have been copied out.
__device__ __forceinline__ void advance_epoch(const DevPlan& pl, uint32_t epoch, bool defer) {
  if (epoch + 1 < kEpochWrap) {
    if (threadIdx.x == 0) __hip_atomic_store(pl.state, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (!defer) clear_tagged(pl);
  if (threadIdx.x == 0) {
    if (defer) __hip_atomic_store(pl.state + 96, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(pl.state, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// PLAIN: no trace stamps, XCD-local hand-offs allowed and head_dim 128; those choices are then constants in
// the task bodies (as runtime checks, 64-row frames measured 76 us slower,
// the local-hand-off check alone cost one-row frames 44 us, and the unused
// head_dim-64 attention 19 us per 64-row frame: the kernel's code is larger
// than the instruction cache, so code that never runs still costs).
template <int BF, bool TL, bool ONE, bool PLAIN, bool NOQK>
__global__ __launch_bounds__(kThreads, 1) void persistent_kernel(DevPlan pl, DevFrame fr) {
  extern __shared__ __align__(1024) uint8_t lds[];
  uint32_t* misc = (uint32_t*)(lds + 2 * kSlotBytes);
  const uint32_t epoch = __hip_atomic_load(pl.state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // XCD-local hand-offs need the workgroups that share one (the split-K
  // partners and owner of a tile; the qkv tiles and attention tasks of a kv
  // group) on one XCD.  The schedule puts them on workgroups of one residue
  // mod 8, and the hardware deals workgroup i to XCD (i + r) mod 8, with a
  // rotation r that changes from launch to launch (a graph replay or the
  // next launch on a stream can start at another XCD) but is the same for
  // every workgroup of a launch: residues stay together whatever r is.  The
  // plan checks at creation that the dealing is such a rotation.
  const bool lcl = PLAIN || __builtin_amdgcn_readfirstlane(pl.local_ok) != 0;
  const uint32_t b = pl.wg_begin[blockIdx.x], e = pl.wg_begin[blockIdx.x + 1];
  // With TL the workgroup's task records are copied to LDS once: reading a
  // record from memory between tasks would make the wave wait for every
  // memory operation still in flight, the previous task's stores and the
  // next tile's copy included.  (TL needs every list to fit kTaskLds.)
  constexpr uint32_t kWords = sizeof(DevTask) / 4;
  uint32_t* tw = (uint32_t*)(lds + 2 * kSlotBytes + kMiscLds);
  if constexpr (TL) {
    const rsrc_t rt = make_rsrc((void*)pl.tasks, (uint32_t)pl.n_tasks * (uint32_t)sizeof(DevTask));
    for (uint32_t w = threadIdx.x; w < (e - b) * kWords; w += kThreads)
      tw[w] = __builtin_amdgcn_raw_buffer_load_b32(rt, (b * kWords + w) * 4, 0, 0);
    wait_vm();
    __syncthreads();
  }
  auto task_at = [&](uint32_t i) -> DevTask {
    if constexpr (TL) {
      DevTask t;
      __builtin_memcpy(&t, tw + (i - b) * kWords, sizeof(DevTask));
      return t;
    } else {
      return pl.tasks[i];
    }
  };
  DevTask cur = {};
  if (b < e) {
    cur = task_at(b);
    issue_tile(pl, cur, lds);
  }
  for (uint32_t i = b; i < e; ++i) {
    uint64_t* tr = (!PLAIN && pl.trace_on) ? pl.trace + (size_t)i * kTraceStamps : nullptr;
    stamp(tr, 0);
    const int s = (i - b) & 1;
    const bool more = i + 1 < e;
    const DevTask nxt = more ? task_at(i + 1) : DevTask{};
    const Next nx = {nxt, more, lds + (s ^ 1) * kSlotBytes};
    stamp(tr, 1);
    run_task<BF, ONE, PLAIN, NOQK>(pl, fr, cur, epoch, lds + s * kSlotBytes, misc, tr, lcl);
    __syncthreads();  // LDS (tile slot, reductions) of this task is free again
    stamp(tr, 6);
    // The next task's tile copy goes out once every wave has issued this
    // task's outputs: the CU's waves share one memory instruction queue and
    // each wave's operations retire in order, so a copy issued earlier would
    // hold up this task's operand and partial-sum waits and delay its stores
    // on their way to the consumers.
    nx.issue(pl);
    stamp(tr, 7);
    cur = nxt;
  }
  // Frame end.  Every workgroup waits (bounded) until all have finished their
  // tasks -- each has waited for its own loads, so no operand is read any
  // more -- then refills its share of the operand region with the sentinel;
  // the kernel's end makes those stores visible to the next frame.  Arrivals
  // count on one of two counters by epoch parity; the last arriver zeroes
  // the other one, which the next frame uses, and moves the plan to the next
  // epoch.  Before a wrapping frame's clear, partials held in an XCD's L2
  // (plain stores) are written back, so that none lands in memory after the
  // clear.
  if (epoch + 1 >= kEpochWrap) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* arrive = pl.state + 128 + 32 * (epoch & 1);
    const uint32_t old = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t n = (uint32_t)pl.n_wg;
    misc[0] = old == n - 1;
    if (old == n - 1) __hip_atomic_store(pl.state + 128 + 32 * ((epoch + 1) & 1), 0u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    Spin sp;
    while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n)
      if (!sp.next(pl)) break;
  }
  __syncthreads();
  refill_operands(pl, blockIdx.x, (uint32_t)pl.n_wg);
  if (misc[0]) advance_epoch(pl, epoch, fr.defer_clear);
}

template <int BF, bool ONE>
__global__ __launch_bounds__(kThreads, 1) void phase_kernel(DevPlan pl, DevFrame fr, const DevTask* tasks) {
  extern __shared__ __align__(1024) uint8_t lds[];
  uint32_t* misc = (uint32_t*)(lds + 2 * kSlotBytes);
  const uint32_t epoch = __hip_atomic_load(pl.state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const DevTask tk = tasks[blockIdx.x];
  issue_tile(pl, tk, lds);
  run_task<BF, ONE>(pl, fr, tk, epoch, lds, misc, nullptr, false);  // (per-phase tasks carry no local flags)
}

// The per-phase executor's last launches of a frame: the sentinel refill of
// the operand region (a grid of its own), then the epoch.
__global__ __launch_bounds__(kThreads, 1) void refill_operands_kernel(DevPlan pl) {
  refill_operands(pl, blockIdx.x, gridDim.x);
}
__global__ __launch_bounds__(kThreads, 1) void bump_epoch_kernel(DevPlan pl, int defer) {
  // (a plan may run its next frame on the persistent executor, whose
  // arrival counters must then be zero whatever the epoch's parity)
  if (threadIdx.x == 0) {
    __hip_atomic_store(pl.state + 128, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(pl.state + 160, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  advance_epoch(pl, __hip_atomic_load(pl.state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), defer != 0);
}

// The clear a wrapping frame deferred (state[96] set), after its K/V copy.
__global__ __launch_bounds__(kThreads, 1) void clear_pending_kernel(DevPlan pl) {
  if (__hip_atomic_load(pl.state + 96, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;
  clear_tagged(pl);
  if (threadIdx.x == 0) __hip_atomic_store(pl.state + 96, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copies the payload of tagged K/V words (bf16 pairs or fp32) out of the
// plan's cache into the caller's untagged layout: rows [0, rows) of every layer.
__global__ void unpack_kv_kernel(const uint64_t* src, uint32_t* dst, uint32_t words_per_row, uint32_t rows,
                                 uint32_t rmax, uint32_t layers) {
  const uint64_t per_layer = (uint64_t)rows * words_per_row;
  const uint64_t n = (uint64_t)layers * per_layer;
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t l = i / per_layer, rem = i % per_layer;
    dst[i] = (uint32_t)src[l * rmax * words_per_row + rem];
  }
}

}  // namespace cpms

// ------------------------------------------------------------------ host-side launchers

namespace cpms {

// Executor variants: activation type, task list in LDS (persistent), and a
// one-row frame (its own code path; task lists that do not fit LDS keep the
// general path).
// (the plain form only with task lists in LDS; lists too long for LDS take
// the general form with its runtime checks)
#define CP_PERSISTENT_VARIANTS(X)                                                                         \
  X(1, true, true, true, false) X(1, true, true, false, false) X(1, true, false, true, true)                 \
  X(1, true, false, true, false) X(1, true, false, false, false) X(1, false, false, false, false)            \
  X(0, true, true, true, false) X(0, true, true, false, false) X(0, true, false, true, true)                 \
  X(0, true, false, true, false) X(0, true, false, false, false) X(0, false, false, false, false)
#define CP_PHASE_VARIANTS(X) X(1, true) X(1, false) X(0, true) X(0, false)

hipError_t launch_persistent(const DevPlan& pl, const DevFrame& fr, hipStream_t s) {
  const dim3 g(pl.n_wg), t(kThreads);
  const bool one = fr.rows == 1 && pl.tasks_in_lds;
  const bool plain = pl.tasks_in_lds && !pl.trace_on && pl.local_ok && pl.d == 128;
  const bool nq = plain && !one && !pl.qk_norm;
#define X(B, T, O, PL, NQK)                                                                        \
  if (pl.bf16 == B && (pl.tasks_in_lds != 0) == T && one == O && plain == PL && nq == NQK) {       \
    hipLaunchKernelGGL((persistent_kernel<B, T, O, PL, NQK>), g, t, kLdsBytes, s, pl, fr);         \
    return hipGetLastError();                                                                    \
  }
  CP_PERSISTENT_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_phase(const DevPlan& pl, const DevFrame& fr, const DevTask* tasks, int n, hipStream_t s) {
  const bool one = fr.rows == 1;
#define X(B, O)                                                                            \
  if (pl.bf16 == B && one == O) {                                                          \
    hipLaunchKernelGGL((phase_kernel<B, O>), dim3(n), dim3(kThreads), kLdsBytes, s, pl, fr, tasks); \
    return hipGetLastError();                                                             \
  }
  CP_PHASE_VARIANTS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_bump_epoch(const DevPlan& pl, int defer_clear, hipStream_t s) {
  hipLaunchKernelGGL(refill_operands_kernel, dim3(pl.n_wg), dim3(kThreads), 0, s, pl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bump_epoch_kernel, dim3(1), dim3(kThreads), 0, s, pl, defer_clear);
  return hipGetLastError();
}

hipError_t launch_clear_pending(const DevPlan& pl, hipStream_t s) {
  hipLaunchKernelGGL(clear_pending_kernel, dim3(1), dim3(kThreads), 0, s, pl);
  return hipGetLastError();
}

hipError_t launch_unpack_kv(const void* src, void* dst, uint32_t words_per_row, uint32_t rows, uint32_t rmax,
                            uint32_t layers, hipStream_t s) {
  hipLaunchKernelGGL(unpack_kv_kernel, dim3(256), dim3(256), 0, s, (const uint64_t*)src, (uint32_t*)dst,
                     words_per_row, rows, rmax, layers);
  return hipGetLastError();
}

hipError_t set_kernel_attributes() {
  hipError_t e;
#define X(B, T, O, PL, NQK)                                                                                  \
  if ((e = hipFuncSetAttribute((const void*)persistent_kernel<B, T, O, PL, NQK>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                               kLdsBytes)))                                                                   \
    return e;
  CP_PERSISTENT_VARIANTS(X)
#undef X
#define X(B, O)                                                                                                \
  if ((e = hipFuncSetAttribute((const void*)phase_kernel<B, O>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes))) \
    return e;
  CP_PHASE_VARIANTS(X)
#undef X
  return hipSuccess;
}

// Records the XCD of every workgroup of a grid shaped like the persistent
// one (n_wg workgroups of kThreads threads, kLdsBytes of LDS each).
__global__ __launch_bounds__(kThreads, 1) void xcd_map_kernel(uint32_t* out) {
  extern __shared__ __align__(1024) uint8_t lds[];
  if (threadIdx.x == 0) {
    lds[0] = 1;
    out[blockIdx.x] = xcc_id();
  }
}

// Whether workgroup i of the persistent grid runs on XCD i % 8, the dealing
// the split-K placement assumes.  buf: n_wg words of device memory to record
// into, or null to allocate (and free) them here.
hipError_t check_xcd_dealing(int n_wg, bool& dealt, uint32_t* buf) {
  dealt = false;
  if (n_wg % 8) return hipSuccess;
  uint32_t* d = buf;
  hipError_t e = hipFuncSetAttribute((const void*)xcd_map_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e == hipSuccess && !buf) e = hipMalloc(&d, (size_t)n_wg * 4);
  if (e != hipSuccess) return e;
  std::vector<uint32_t> h(n_wg, 0xffffffffu);
  hipLaunchKernelGGL(xcd_map_kernel, dim3(n_wg), dim3(kThreads), kLdsBytes, 0, d);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpy(h.data(), d, (size_t)n_wg * 4, hipMemcpyDeviceToHost);
  const hipError_t f = buf ? hipSuccess : hipFree(d);
  if (e != hipSuccess) return e;
  if (f != hipSuccess) return f;
  // workgroup i on XCD (i + r) mod 8 for one rotation r
  dealt = true;
  for (int i = 0; i < n_wg; ++i) dealt = dealt && h[i] == ((uint32_t)i + h[0]) % 8;
  return hipSuccess;
}

int occupancy_per_cu(int bf16) {
  // the smallest over the executor's forms for this activation type
  int best = INT32_MAX;
#define X(B, T, O, PL, NQK)                                                                                 \
  if (bf16 == B) {                                                                                         \
    int n = 0;                                                                                             \
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, persistent_kernel<B, T, O, PL, NQK>, kThreads, kLdsBytes) != \
        hipSuccess)                                                                                        \
      return -1;                                                                                           \
    best = n < best ? n : best;                                                                            \
  }
  CP_PERSISTENT_VARIANTS(X)
#undef X
  return best == INT32_MAX ? -1 : best;
}

}  // namespace cpms
