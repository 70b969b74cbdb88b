// Device code of the depth-loop library: the task bodies, the persistent
// executor and the one-launch-per-phase executor.
//
// The frame and its phases follow mstar pull request #1183 ("Qwen3-TTS: Run
// the 1.7B Depth Loop as One Persistent Kernel on Hopper"), section "How it
// works": one resident workgroup per compute unit walks a static task list; a
// task waits on counters in device memory, runs one tile and signals a
// counter; attention waits only on the qkv tiles of its own kv head; o and
// down split their K loop and add the partial sums in a fixed order, with no
// atomics on data, so a frame is bit-identical from run to run.  The megakernel
// pattern itself (resident blocks, counter dependencies that only point to
// earlier work, prefetching weights before waiting) is the one of the handbook
// chapter "The gaps between kernels: PDL and megakernels", section
// "Megakernels: the whole forward pass in one kernel".
//
// Hand-off between workgroups (MI355X has eight XCDs, each with its own L2):
// every value one workgroup writes and another reads is stored and loaded with
// the agent-coherent cache policy (sc1), the writer waits for its stores to
// complete before it adds to a counter, and the reader polls the counter with
// agent-scope atomic loads.  No L2 write-back or invalidate is needed, because
// no cross-workgroup value is ever held in a non-coherent cache line.
// Weights and inputs never change during a frame and use the ordinary path.
#include <hip/hip_runtime.h>

#include "cp_device.h"

namespace cpms {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kSC1 = 16;  // buffer cache policy bit: coherent at agent scope

// ------------------------------------------------------------------ memory helpers

// A raw buffer resource over [p, p + bytes): loads past the end return zero,
// stores past the end are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16c(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1); }
__device__ __forceinline__ u32x2 ld8c(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSC1); }
__device__ __forceinline__ uint32_t ld4c(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSC1); }
__device__ __forceinline__ uint32_t ld2c(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kSC1); }
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ __forceinline__ uint32_t ld4(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ __forceinline__ uint32_t ld2(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0); }
__device__ __forceinline__ void st16c(rsrc_t r, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSC1); }
__device__ __forceinline__ void st8c(rsrc_t r, uint32_t off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kSC1); }
__device__ __forceinline__ void st4c(rsrc_t r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kSC1); }
__device__ __forceinline__ void st2c(rsrc_t r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, kSC1); }

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Trace stamp k of the current task (100 MHz constant clock), thread 0 only.
// tr is null when the plan does not trace.
__device__ __forceinline__ void stamp(uint64_t* tr, int k) {
  if (tr && threadIdx.x == 0) tr[k] = __builtin_amdgcn_s_memrealtime();
}

// ------------------------------------------------------------------ numerics

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

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

// Element e of a 16-byte chunk as float.
template <int BF>
__device__ __forceinline__ float chunk_elem(const u32x4& v, int e) {
  if constexpr (BF) return bf2f((v[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
  else return __uint_as_float(v[e]);
}

// Rounds to the activation type and returns the stored bits.
template <int BF>
__device__ __forceinline__ uint32_t to_act(float f) {
  if constexpr (BF) return f2bf(f);
  else return __float_as_uint(f);
}
template <int BF>
__device__ __forceinline__ float act_val(float f) {
  if constexpr (BF) return bf2f(f2bf(f));
  else return f;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// (value, index) that wins an argmax: larger value, then lower index.
__device__ __forceinline__ bool beats(float v, uint32_t i, float bv, uint32_t bi) {
  return v > bv || (v == bv && i < bi);
}

// ------------------------------------------------------------------ sync

__device__ __forceinline__ uint32_t ld_ctr(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 waits until every sub-counter of the task's groups has reached its
// share of this frame's target; the rest of the workgroup waits at the barrier.
// A wait gives up after spin_limit polls and raises the error word, so a
// broken schedule ends the kernel instead of hanging it.
__device__ __forceinline__ void wait_deps(const DevPlan& pl, const Task& tk, uint32_t epoch) {
  if (threadIdx.x < 64 && tk.nwait) {
    const int lane = threadIdx.x;
#pragma unroll
    for (int k = 0; k < kMaxWaits; ++k) {
      if (k >= tk.nwait) break;
      const CtrGroup gp = pl.groups[tk.wait[k]];
      const uint32_t target = (uint32_t)gp.per_sub * epoch;
      if (lane < gp.nsub) {
        const uint32_t* c = pl.ctr + (size_t)(gp.base + lane) * kCtrStride;
        uint32_t spins = 0;
        while (ld_ctr(c) < target) {
          if (++spins > pl.spin_limit) {
            __hip_atomic_store(pl.state + 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          if ((spins & 1023u) == 0 && ld_ctr(pl.state + 64)) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
  }
  __syncthreads();
}

// Every wave waits for its own stores, then one thread adds to the group.
__device__ __forceinline__ void signal_group(const DevPlan& pl, uint32_t grp, uint32_t slot, bool persistent,
                                             uint64_t* tr) {
  stamp(tr, 5);
  wait_vm();
  __syncthreads();
  stamp(tr, 6);
  if (persistent && threadIdx.x == 0 && grp != kNone) {
    const CtrGroup gp = pl.groups[grp];
    __hip_atomic_fetch_add(pl.ctr + (size_t)(gp.base + slot % gp.nsub) * kCtrStride, 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  stamp(tr, 7);
}

// ------------------------------------------------------------------ weights -> LDS

// Byte offset of the gain row staged in the misc LDS region.
constexpr int kGainLds = 1024;    // RMSNorm gain row (<= 2 KiB)
constexpr int kRedSsLds = 4096;   // cross-wave sums of squares (256 B)
constexpr int kRedAccLds = 8192;  // cross-wave MFMA accumulators (8 KiB)

// Gain row (of the [2L + 1][H] table) a projection task normalises with, or -1.
__device__ __forceinline__ int gain_row_of(const DevPlan& pl, const Task& tk) {
  switch (tk.type) {
    case T_QKV: return 2 * tk.layer;
    case T_GU: return 2 * tk.layer + 1;
    case T_HEAD: return 2 * pl.L;
    default: return -1;
  }
}

// Direct-to-LDS copies of the task's packed weight tile and, for normalising
// tasks, its RMSNorm gain row: 1 KiB chunks (64 lanes x 16 B) with
// global_load_lds_dwordx4, dealt round-robin to the four waves.
__device__ __forceinline__ void issue_tile(const DevPlan& pl, const Task& tk, uint8_t* slot, uint8_t* misc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t nch = tk.w_bytes >> 10;
  const uint8_t* src = pl.wblob + tk.w_off;
  for (uint32_t c = wave; c < nch; c += 4) {
    __builtin_amdgcn_global_load_lds((const void*)(src + c * 1024 + lane * 16),
                                     (void __attribute__((address_space(3)))*)(slot + c * 1024), 16, 0, 0);
  }
  const int gr = gain_row_of(pl, tk);
  if (gr >= 0) {
    const uint32_t gbytes = (uint32_t)pl.H * (pl.bf16 ? 2 : 4);  // <= 2 KiB
    const uint8_t* gsrc = (const uint8_t*)pl.gains + (size_t)gr * gbytes;
    for (uint32_t c = 3 - wave; c < (gbytes + 1023) / 1024; c += 4) {
      __builtin_amdgcn_global_load_lds((const void*)(gsrc + c * 1024 + lane * 16),
                                       (void __attribute__((address_space(3)))*)(misc + kGainLds + c * 1024), 16, 0, 0);
    }
  }
}

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

// Sum of squares of a residual row comes from its producers as H/16 partials
// (one per 16-column tile, in tile order); ssq slot ids: position inputs
// 0 .. P-1, residual after down P + 2*parity + layer parity, residual after o
// P + 4 + parity.
__device__ __forceinline__ float* ssq_slot(const DevPlan& pl, int slot) {
  return pl.ssq + (size_t)slot * pl.Rmax * (pl.H / 16);
}

// Sum of squares of the four values a lane stores, added over the `span`
// lanes (xor distances `first`, `2 first`, ...) that share one 16-column tile.
__device__ __forceinline__ float tile_ssq(const float (&v)[4], int first, int span) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = fmaf(v[e], v[e], s);
  for (int m = first; m < first * span; m <<= 1) s += shfl_xor_f(s, m);
  return s;
}

template <int BF>
__device__ __forceinline__ void proj_task(const DevPlan& pl, const DevFrame& fr, const Task& tk, uint32_t epoch,
                                          uint8_t* slot, uint32_t* misc, bool persistent, uint64_t* tr) {
  constexpr int ESZ = BF ? 2 : 4;     // bytes per activation element
  constexpr int E = 16 / ESZ;         // elements per 16-byte chunk
  constexpr int KS = 4 * E;           // K elements one chunk step covers across the 4 lane groups
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 4, rl = lane & 15;
  const int rows = fr.rows;
  const int H = pl.H, Rmax = pl.Rmax, P = pl.P;
  const int l = tk.layer, p = tk.pos;

  // Operand source, K range, norm and epilogue of this task kind.
  const void* xsrc;
  uint32_t xbytes, ld;  // buffer bytes and row stride (elements)
  int k0 = 0, kt;
  int in_ssq = -1;      // ssq slot of a normalised input (-1: no norm)
  int out_ssq = -1;     // ssq slot of a residual output (EPI_PART)
  int nb = 1;
  Epi epi;
  const void* resid = nullptr;  // residual (EPI_PART)
  void* out = nullptr;          // output (EPI_PART)
  uint64_t part_off = 0;
  // Buffers that two positions in flight at once (0 and 1) would share are
  // doubled and picked by position parity.
  const int par = p & 1;
  const uint32_t hbytes = (uint32_t)Rmax * H * ESZ;
  const uint32_t qdbytes = (uint32_t)Rmax * pl.nq * pl.d * ESZ;
  uint8_t* hres = (uint8_t*)pl.hres + (size_t)par * 2 * hbytes;   // [layer parity]
  uint8_t* hmid = (uint8_t*)pl.hmid + (size_t)par * hbytes;
  const uint8_t* layer_in = (l == 0) ? (const uint8_t*)pl.xin + (size_t)p * hbytes : hres + (size_t)((l - 1) & 1) * hbytes;
  const int layer_in_ssq = (l == 0) ? p : P + 2 * par + ((l - 1) & 1);
  switch (tk.type) {
    case T_QKV:
      xsrc = layer_in; xbytes = hbytes; ld = H; kt = H; in_ssq = layer_in_ssq; epi = EPI_QKV; break;
    case T_GU:
      xsrc = hmid; xbytes = hbytes; ld = H; kt = H; in_ssq = P + 4 + par; nb = 2; epi = EPI_GU; break;
    case T_HEAD:
      xsrc = hres + (size_t)((pl.L - 1) & 1) * hbytes; xbytes = hbytes; ld = H; kt = H;
      in_ssq = P + 2 * par + ((pl.L - 1) & 1); epi = EPI_HEAD; break;
    case T_O:
      xsrc = (const uint8_t*)pl.abuf + (size_t)par * qdbytes; ld = pl.nq * pl.d; xbytes = qdbytes;
      kt = (int)ld / tk.nsplit; k0 = tk.split * kt; epi = EPI_PART; resid = layer_in; out = hmid;
      out_ssq = P + 4 + par; part_off = pl.part_o_off + (uint64_t)par * pl.part_stride; break;
    case T_DOWN:
      xsrc = (const uint8_t*)pl.mbuf + (size_t)par * Rmax * pl.I * ESZ; ld = pl.I; xbytes = (uint32_t)Rmax * ld * ESZ;
      kt = pl.I / tk.nsplit; k0 = tk.split * kt; epi = EPI_PART; resid = hmid;
      out = hres + (size_t)(l & 1) * hbytes; out_ssq = P + 2 * par + (l & 1);
      part_off = pl.part_d_off + (uint64_t)par * pl.part_stride; break;
    default:  // T_INPROJ
      xsrc = fr.hidden_in; ld = pl.Din; xbytes = (uint32_t)fr.rows * ld * ESZ; kt = pl.Din / tk.nsplit;
      k0 = tk.split * kt; epi = EPI_PART; out = pl.xin; out_ssq = 0; part_off = pl.part_in_off; break;
  }
  const int nck = kt * ESZ / 64;  // 16-byte chunks per lane over the task's K range

  // Waves and row tiles: a wave owns 16 rows; with few rows the waves of a
  // row tile split K and add their results through LDS in a fixed order.
  const int nrt = (rows + 15) >> 4;                   // row tiles holding live rows (1..4)
  int wpr = nrt == 1 ? 4 : (nrt == 2 ? 2 : 1);        // waves per row tile
  while (wpr > 1 && nck % (4 * wpr)) wpr >>= 1;        // each wave takes whole groups of 4 chunks
  const int rt = wave / wpr, ks = wave % wpr;
  const int ncw = nck / wpr;                          // chunks this wave handles (a multiple of 4)
  const int c0 = ks * ncw;
  const int row = rt * 16 + rl;
  const bool wave_live = rt < nrt;
  const bool live = wave_live && row < rows;
  f32x4* red_acc = (f32x4*)((uint8_t*)misc + kRedAccLds);    // [4 waves][2][64 lanes]
  const uint32_t ssq_bytes = (uint32_t)Rmax * (H / 16) * 4;

  // Loads that do not depend on the K loop go out first: the sum-of-squares
  // partials of a normalised input, the residual of an unsplit o / down tile
  // and the RoPE angles of a qkv tile.
  const rsrc_t rx = make_rsrc(xsrc, xbytes);
  const uint32_t xoff = ((uint32_t)row * ld + k0 + q * E) * ESZ + c0 * 64;
  u32x4 ssv[4];
  const int nsq = H / 64;  // partials per lane (H/16 partials over 4 lanes), <= 4
  if (in_ssq >= 0) {
    const rsrc_t rs = make_rsrc(ssq_slot(pl, in_ssq), ssq_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i * 4 < nsq) ssv[i] = live ? ld16c(rs, (uint32_t)(row * (H / 16) + q * nsq + 4 * i) * 4) : u32x4{0, 0, 0, 0};
  }
  const uint32_t eo = (uint32_t)(row * H + 16 * tk.tile + 4 * q) * ESZ;  // this lane's 4 output slots
  u32x4 rv = {0, 0, 0, 0};
  if (epi == EPI_PART && tk.nsplit == 1 && resid && live && ks == 0) {
    const rsrc_t rr = make_rsrc(resid, hbytes);
    if constexpr (BF) {
      const u32x2 h = ld8c(rr, eo);
      rv[0] = h[0]; rv[1] = h[1];
    } else {
      rv = ld16c(rr, eo);
    }
  }
  float rope_cs[2] = {1.f, 1.f}, rope_sn[2] = {0.f, 0.f};
  if (tk.type == T_QKV) {
    const int d = pl.d, th = d / 16, tpg = (pl.gq + 2) * th, lt = tk.tile % tpg;
    if (lt < (pl.gq + 1) * th) {
      const int i0 = 8 * (lt % th) + 2 * q;
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        rope_cs[pr] = pl.rope[(p * (d / 2) + i0 + pr) * 2];
        rope_sn[pr] = pl.rope[(p * (d / 2) + i0 + pr) * 2 + 1];
      }
    }
  }

  // K loop over groups of four chunks: the next group's loads are in flight
  // while the current one is scaled and multiplied.
  u32x4 xa[4], xb[4];
  auto load_group = [&](u32x4 (&x)[4], int g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = live ? ld16c(rx, xoff + (g * 4 + i) * 64) : u32x4{0, 0, 0, 0};
  };
  const int ng = ncw / 4;
  if (wave_live) load_group(xa, 0);
  wait_vm();        // this wave's share of the weight tile (and the first group) have landed
  __syncthreads();  // every wave's share of the tile is in LDS
  stamp(tr, 2);

  float rinv = 1.f;
  if (in_ssq >= 0 && wave_live) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i * 4 < nsq)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += __uint_as_float(ssv[i][e]);
    ss += shfl_xor_f(ss, 16);
    ss += shfl_xor_f(ss, 32);
    rinv = 1.0f / sqrtf(ss / (float)H + pl.eps);
  }
  stamp(tr, 3);

  const bool norm = in_ssq >= 0;
  const bool unit = pl.unit_gains != 0;
  const uint8_t* gl = (const uint8_t*)misc + kGainLds + c0 * 64;  // gain row staged with the tile
  const uint8_t* wt = slot + lane * 16 + (size_t)c0 * nb * 1024;
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  // a = round(round(x * r) * g) in the activation type, then the MFMAs
  auto process = [&](u32x4 (&x)[4], int g) {
    u32x4 w[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = *(const u32x4*)(wt + ((g * 4 + i) * nb) * 1024);
      if (nb == 2) w[2 * i + 1] = *(const u32x4*)(wt + ((g * 4 + i) * nb + 1) * 1024);
    }
    if (norm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 gv = *(const u32x4*)(gl + ((g * 4 + i) * KS + q * E) * ESZ);
        u32x4 o;
        if constexpr (BF) {
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            const uint32_t xw = x[i][w2];
            const float t0 = __uint_as_float(xw << 16) * rinv, t1 = __uint_as_float(xw & 0xffff0000u) * rinv;
            if (unit) {
              o[w2] = pack_bf16(t0, t1);
            } else {
              const uint32_t gw = gv[w2];
              o[w2] = pack_bf16(t0 * __uint_as_float(gw << 16), t1 * __uint_as_float(gw & 0xffff0000u));
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = __uint_as_float(x[i][e]) * rinv;
            o[e] = __float_as_uint(unit ? t : t * __uint_as_float(gv[e]));
          }
        }
        x[i] = live ? o : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (nb == 1) {
        if (i & 1) acc1 = mma<BF>(w[2 * i], x[i], acc1);
        else acc0 = mma<BF>(w[2 * i], x[i], acc0);
      } else {
        acc0 = mma<BF>(w[2 * i], x[i], acc0);
        acc1 = mma<BF>(w[2 * i + 1], x[i], acc1);
      }
    }
  };
  if (wave_live) {
    for (int g = 0; g < ng; g += 2) {
      if (g + 1 < ng) load_group(xb, g + 1);
      process(xa, g);
      if (g + 1 >= ng) break;
      if (g + 2 < ng) load_group(xa, g + 2);
      process(xb, g + 1);
    }
    if (nb == 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc0[v] = acc0[v] + acc1[v];
    }
  }
  stamp(tr, 4);
  if (wpr > 1) {
    // K parts of a row tile: (((k0 + k1) + k2) + k3), in the wave of part 0
    if (wave_live) {
      red_acc[(wave * 2 + 0) * 64 + lane] = acc0;
      if (nb == 2) red_acc[(wave * 2 + 1) * 64 + lane] = acc1;
    }
    __syncthreads();
    if (wave_live && ks == 0) {
      acc0 = red_acc[(rt * wpr * 2 + 0) * 64 + lane];
      if (nb == 2) acc1 = red_acc[(rt * wpr * 2 + 1) * 64 + lane];
      for (int k = 1; k < wpr; ++k) {
        const f32x4 a = red_acc[((rt * wpr + k) * 2 + 0) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc0[v] = acc0[v] + a[v];
        if (nb == 2) {
          const f32x4 b = red_acc[((rt * wpr + k) * 2 + 1) * 64 + lane];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc1[v] = acc1[v] + b[v];
        }
      }
    }
  }
  const bool epi_wave = wave_live && ks == 0;

  // Lane (q, rl) of an epilogue wave holds output slots 4q .. 4q+3 of row `row`.
  if (epi_wave) {
    if (epi == EPI_QKV) {
      const int d = pl.d, th = d / 16, gq = pl.gq, nkv = pl.nkv;
      const int tpg = (gq + 2) * th;
      const int g = tk.tile / tpg, lt = tk.tile % tpg;
      const uint32_t kvoff = (uint32_t)(((l * Rmax + row) * nkv + g) * P + p) * d;
      const uint32_t kvbytes = (uint32_t)pl.L * Rmax * nkv * P * d * ESZ;
      if (live) {
        if (lt < (gq + 1) * th) {
          // q or k head: slots (4q + v) hold rotary pairs 8 tih + 2q + (v >> 1), half v & 1
          const int tih = lt % th;
          const bool isq = lt < gq * th;
          const int hq = g * gq + lt / th;
          const int i0 = 8 * tih + 2 * q;
          float y[4];
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const float x1 = acc0[2 * pr], x2 = acc0[2 * pr + 1];
            const float cs = rope_cs[pr], sn = rope_sn[pr];
            y[2 * pr] = x1 * cs - x2 * sn;
            y[2 * pr + 1] = x2 * cs + x1 * sn;
          }
          // dims i0, i0 + 1 (first halves) and i0 + d/2, i0 + d/2 + 1 (second halves)
          rsrc_t r;
          uint32_t base;
          if (isq) {
            r = make_rsrc((uint8_t*)pl.qbuf + (size_t)par * qdbytes, qdbytes);
            base = (uint32_t)(row * pl.nq * d + hq * d);
          } else {
            r = make_rsrc(pl.kc, kvbytes);
            base = kvoff;
          }
          if constexpr (BF) {
            st4c(r, (base + i0) * 2, pack_bf16(y[0], y[2]));
            st4c(r, (base + i0 + d / 2) * 2, pack_bf16(y[1], y[3]));
          } else {
            st8c(r, (base + i0) * 4, u32x2{__float_as_uint(y[0]), __float_as_uint(y[2])});
            st8c(r, (base + i0 + d / 2) * 4, u32x2{__float_as_uint(y[1]), __float_as_uint(y[3])});
          }
        } else {
          const int tih = lt - (gq + 1) * th;
          const rsrc_t r = make_rsrc(pl.vc, kvbytes);
          const uint32_t o = (kvoff + 16 * tih + 4 * q) * ESZ;
          if constexpr (BF) st8c(r, o, u32x2{pack_bf16(acc0[0], acc0[1]), pack_bf16(acc0[2], acc0[3])});
          else st16c(r, o, u32x4{__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), __float_as_uint(acc0[2]), __float_as_uint(acc0[3])});
        }
      }
    } else if (epi == EPI_GU) {
      if (live) {
        float m[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = acc0[v], uv = acc1[v];
          m[v] = (gv / (1.0f + expf(-gv))) * uv;
        }
        const rsrc_t r = make_rsrc((uint8_t*)pl.mbuf + (size_t)par * Rmax * pl.I * ESZ, (uint32_t)Rmax * pl.I * ESZ);
        const uint32_t o = (uint32_t)(row * pl.I + 16 * tk.tile + 4 * q) * ESZ;
        if constexpr (BF) st8c(r, o, u32x2{pack_bf16(m[0], m[1]), pack_bf16(m[2], m[3])});
        else st16c(r, o, u32x4{__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]), __float_as_uint(m[3])});
      }
    } else if (epi == EPI_HEAD) {
      const int V = pl.V;
      const uint32_t n0 = 16 * tk.tile + 4 * q;
      if (live) {
        const u32x4 z = {__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), __float_as_uint(acc0[2]), __float_as_uint(acc0[3])};
        st16c(make_rsrc(pl.zbuf, (uint32_t)Rmax * V * 4), (uint32_t)(row * V + n0) * 4, z);
        if (fr.logits)
          st16c(make_rsrc(fr.logits, (uint32_t)rows * (P - 1) * V * 4), (uint32_t)((row * (P - 1) + (p - 1)) * V + n0) * 4, z);
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
        st8c(make_rsrc(pl.cand, (uint32_t)Rmax * pl.n_head_tiles * 8), (uint32_t)(row * pl.n_head_tiles + tk.tile) * 8,
             u32x2{__float_as_uint(bv), bi});
    } else if (tk.nsplit == 1) {  // EPI_PART, unsplit: residual add, store, sum of squares
      float h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = act_val<BF>(resid ? acc0[e] + chunk_elem<BF>(rv, e) : acc0[e]);
      const float sq = tile_ssq(h, 16, 4);
      if (live) {
        const rsrc_t ro = make_rsrc(out, hbytes);
        if constexpr (BF) st8c(ro, eo, u32x2{pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3])});
        else st16c(ro, eo, u32x4{__float_as_uint(h[0]), __float_as_uint(h[1]), __float_as_uint(h[2]), __float_as_uint(h[3])});
        if (q == 0) st4c(make_rsrc(ssq_slot(pl, out_ssq), ssq_bytes), (uint32_t)(row * (H / 16) + tk.tile) * 4, __float_as_uint(sq));
      }
    } else {  // EPI_PART, split: fp32 partial of this split
      if (live) {
        const uint32_t o = (uint32_t)(((tk.tile * tk.nsplit + tk.split) * Rmax + row) * 16 + 4 * q) * 4;
        st16c(make_rsrc(pl.part + part_off, (uint32_t)pl.part_stride * 4), o,
              u32x4{__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), __float_as_uint(acc0[2]), __float_as_uint(acc0[3])});
      }
    }
  }

  if (epi != EPI_PART || tk.nsplit == 1) {
    signal_group(pl, tk.sig, tk.sig_slot, persistent, tr);
    return;
  }

  // Split-K: the last of the nsplit tasks of this tile to arrive adds the
  // partials in split order (then the residual) and stores the tile.
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(pl.ctr + (size_t)tk.tctr * kCtrStride, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    misc[0] = (old == (uint32_t)tk.nsplit * epoch - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (misc[0] == 0) return;  // uniform across the workgroup

  {
    const int t = threadIdx.x;  // 64 rows x 4 column quads
    const int r = t >> 2, c4 = (t & 3) * 4;
    const rsrc_t rp = make_rsrc(pl.part + part_off, (uint32_t)pl.part_stride * 4);
    // issue every load (partials and residual) before using any
    const uint32_t ro_off = (uint32_t)(r * H + 16 * tk.tile + c4) * ESZ;
    u32x4 pv[4];
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
      if (sp < tk.nsplit)
        pv[sp] = r < rows ? ld16c(rp, (uint32_t)(((tk.tile * tk.nsplit + sp) * Rmax + r) * 16 + c4) * 4) : u32x4{0, 0, 0, 0};
    u32x4 hv = {0, 0, 0, 0};
    if (resid && r < rows) {
      const rsrc_t rr = make_rsrc(resid, hbytes);
      if constexpr (BF) {
        const u32x2 h = ld8c(rr, ro_off);
        hv[0] = h[0]; hv[1] = h[1];
      } else {
        hv = ld16c(rr, ro_off);
      }
    }
    f32x4 s = {0, 0, 0, 0};
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
      if (sp < tk.nsplit)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = s[e] + __uint_as_float(pv[sp][e]);
    float h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = act_val<BF>(resid ? s[e] + chunk_elem<BF>(hv, e) : s[e]);
    const float sq = tile_ssq(h, 1, 4);
    if (r < rows) {
      const rsrc_t ro = make_rsrc(out, hbytes);
      if constexpr (BF) st8c(ro, ro_off, u32x2{pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3])});
      else st16c(ro, ro_off, u32x4{__float_as_uint(h[0]), __float_as_uint(h[1]), __float_as_uint(h[2]), __float_as_uint(h[3])});
      if ((t & 3) == 0)
        st4c(make_rsrc(ssq_slot(pl, out_ssq), ssq_bytes), (uint32_t)(r * (H / 16) + tk.tile) * 4, __float_as_uint(sq));
    }
  }
  signal_group(pl, tk.sig, tk.sig_slot, persistent, tr);
}

// ------------------------------------------------------------------ attention

// One kv head g for a group of rows: every (row, q head of g) pair is one
// wave's work.  Scores: lane (t, c) takes position t and a quarter c of the
// head dimension; softmax over t <= p in float; output: lane owns d/64 dims.
template <int BF>
__device__ __forceinline__ void attn_task(const DevPlan& pl, const DevFrame& fr, const Task& tk, bool persistent,
                                          uint64_t* tr) {
  constexpr int ESZ = BF ? 2 : 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d = pl.d, gq = pl.gq, nkv = pl.nkv, P = pl.P, Rmax = pl.Rmax;
  const int l = tk.layer, p = tk.pos;
  const int ngroups = Rmax / pl.attn_rows;
  const int g = tk.tile / ngroups, rg = tk.tile % ngroups;
  const int npairs = pl.attn_rows * gq;
  const uint32_t qdbytes = (uint32_t)Rmax * pl.nq * d * ESZ;
  const rsrc_t rq = make_rsrc((uint8_t*)pl.qbuf + (size_t)(p & 1) * qdbytes, qdbytes);
  const uint32_t kvbytes = (uint32_t)pl.L * Rmax * nkv * P * d * ESZ;
  const rsrc_t rk = make_rsrc(pl.kc, kvbytes), rv = make_rsrc(pl.vc, kvbytes);
  const rsrc_t ra = make_rsrc((uint8_t*)pl.abuf + (size_t)(p & 1) * qdbytes, qdbytes);
  const int t = lane >> 2, c = lane & 3;
  const int dq = d / 4;                  // dims per score lane
  const int nchunk = dq * ESZ / 16;      // 16-byte chunks per score lane (2, 4 or 8)
  const int dpl = d / 64;                // output dims per lane (1 or 2)
  for (int pi = wave; pi < npairs; pi += 4) {
    const int row = rg * pl.attn_rows + pi / gq;
    const int hq = g * gq + pi % gq;
    if (row >= fr.rows) continue;  // wave-uniform
    const uint32_t kvrow = (uint32_t)((l * Rmax + row) * nkv + g) * P;
    // every load of the pair (Q, K and V for t <= p) is issued before any is used
    const uint32_t dbase = (uint32_t)(lane * dpl);
    u32x4 qv[8], kv[8];
    const uint32_t qo = (uint32_t)(row * pl.nq * d + hq * d + c * dq) * ESZ;
    const uint32_t ko = (uint32_t)((kvrow + t) * d + c * dq) * ESZ;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nchunk) {
        qv[i] = ld16c(rq, qo + i * 16);
        kv[i] = (t <= p) ? ld16c(rk, ko + i * 16) : u32x4{0, 0, 0, 0};
      }
    u32x2 vv[16];  // V[t][dbase .. dbase + dpl) for t = 0 .. 15
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      if (tt <= p) {
        const uint32_t vo = (uint32_t)((kvrow + tt) * d + dbase) * ESZ;
        if (ESZ * dpl == 8) vv[tt] = ld8c(rv, vo);
        else if (ESZ * dpl == 4) vv[tt] = u32x2{ld4c(rv, vo), 0u};
        else vv[tt] = u32x2{ld2c(rv, vo), 0u};
      }
    }
    // scores
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nchunk)
#pragma unroll
        for (int e = 0; e < 16 / ESZ; ++e) dot += chunk_elem<BF>(qv[i], e) * chunk_elem<BF>(kv[i], e);
    dot += shfl_xor_f(dot, 1);
    dot += shfl_xor_f(dot, 2);
    const float s = (t <= p) ? dot * pl.attn_scale : -INFINITY;
    float m = s;
#pragma unroll
    for (int k = 4; k <= 32; k <<= 1) m = fmaxf(m, shfl_xor_f(m, k));
    const float e = (t <= p) ? expf(s - m) : 0.f;
    float sum = e;
#pragma unroll
    for (int k = 4; k <= 32; k <<= 1) sum += shfl_xor_f(sum, k);
    const float w = e / sum;
    // output: sum over t in ascending order
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const float wt = __shfl(w, tt * 4, 64);
      if (tt <= p) {
        if constexpr (BF) {
          if (dpl == 2) {
            o0 += wt * bf2f(vv[tt][0] & 0xffffu);
            o1 += wt * bf2f(vv[tt][0] >> 16);
          } else {
            o0 += wt * bf2f(vv[tt][0] & 0xffffu);
          }
        } else {
          o0 += wt * __uint_as_float(vv[tt][0]);
          if (dpl == 2) o1 += wt * __uint_as_float(vv[tt][1]);
        }
      }
    }
    const uint32_t ao = (uint32_t)(row * pl.nq * d + hq * d + dbase) * ESZ;
    if constexpr (BF) {
      if (dpl == 2) st4c(ra, ao, pack_bf16(o0, o1));
      else st2c(ra, ao, f2bf(o0));
    } else {
      if (dpl == 2) st8c(ra, ao, u32x2{__float_as_uint(o0), __float_as_uint(o1)});
      else st4c(ra, ao, __float_as_uint(o0));
    }
  }
  signal_group(pl, tk.sig, tk.sig_slot, persistent, tr);
}

// ------------------------------------------------------------------ draw + embed

// Writes embedding row `code` of table j as the input of position j + 1 (when
// there is one) and adds it to the row's fp32 embedding sum.
template <int BF>
__device__ __forceinline__ void embed_row(const DevPlan& pl, const DevFrame& fr, int j, int row, int code, bool first) {
  constexpr int ESZ = BF ? 2 : 4;
  const int H = pl.H, V = pl.V;
  const rsrc_t re = make_rsrc(pl.embed, (uint32_t)pl.P * V * H * ESZ);
  const rsrc_t rs = make_rsrc(fr.embsum, (uint32_t)fr.rows * H * 4);
  const rsrc_t rx = make_rsrc(pl.xin, (uint32_t)pl.P * pl.Rmax * H * ESZ);
  const uint32_t ebase = (uint32_t)((j * V + code) * H);
  const uint32_t xbase = (uint32_t)(((j + 1) * pl.Rmax + row) * H);
  const bool feeds = j + 1 < pl.P;  // the row is the input of position j + 1
  // thread t covers elements 4t .. 4t+3: four threads per 16-column tile
  for (int k = threadIdx.x * 4; k < ((H + 1023) / 1024) * 1024; k += kThreads * 4) {
    const bool in = k < H;
    float ev[4] = {0.f, 0.f, 0.f, 0.f};
    u32x4 sv = {0, 0, 0, 0};
    if (in) {
      if constexpr (BF) {
        const u32x2 e = __builtin_amdgcn_raw_buffer_load_b64(re, (ebase + k) * 2, 0, 0);
        ev[0] = bf2f(e[0] & 0xffffu); ev[1] = bf2f(e[0] >> 16); ev[2] = bf2f(e[1] & 0xffffu); ev[3] = bf2f(e[1] >> 16);
        if (feeds) st8c(rx, (xbase + k) * 2, e);
      } else {
        const u32x4 e = ld16(re, (ebase + k) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) ev[i] = __uint_as_float(e[i]);
        if (feeds) st16c(rx, (xbase + k) * 4, e);
      }
      if (!first) sv = ld16c(rs, (uint32_t)(row * H + k) * 4);
    }
    const float sq = tile_ssq(ev, 1, 4);
    if (in) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = __float_as_uint(first ? ev[i] : __uint_as_float(sv[i]) + ev[i]);
      st16c(rs, (uint32_t)(row * H + k) * 4, sv);
      if (feeds && (threadIdx.x & 3) == 0)
        st4c(make_rsrc(ssq_slot(pl, j + 1), (uint32_t)pl.Rmax * (H / 16) * 4), (uint32_t)(row * (H / 16) + k / 16) * 4,
             __float_as_uint(sq));
    }
  }
}

template <int BF>
__device__ __forceinline__ void embed0_task(const DevPlan& pl, const DevFrame& fr, const Task& tk, bool persistent,
                                            uint64_t* tr) {
  const int row = (int)tk.tile;
  if (row < fr.rows) {
    int code = fr.code0[row];
    code = code < 0 ? 0 : (code >= pl.V ? pl.V - 1 : code);
    embed_row<BF>(pl, fr, 0, row, code, true);
  }
  signal_group(pl, tk.sig, tk.sig_slot, persistent, tr);
}

template <int BF>
__device__ __forceinline__ void draw_task(const DevPlan& pl, const DevFrame& fr, const Task& tk, uint32_t* misc,
                                          bool persistent, uint64_t* tr) {
  const int row = (int)tk.tile, p = tk.pos;
  if (row < fr.rows) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const rsrc_t rc = make_rsrc(pl.cand, (uint32_t)pl.Rmax * pl.n_head_tiles * 8);
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      for (int i = lane; i < pl.n_head_tiles; i += 64) {
        const u32x2 cv = ld8c(rc, (uint32_t)(row * pl.n_head_tiles + i) * 8);
        const float v = __uint_as_float(cv[0]);
        if (beats(v, cv[1], bv, bi)) { bv = v; bi = cv[1]; }
      }
#pragma unroll
      for (int m = 1; m <= 32; m <<= 1) {
        const float ov = shfl_xor_f(bv, m);
        const uint32_t oi = (uint32_t)__shfl_xor((int)bi, m, 64);
        if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (lane == 0) {
        misc[1] = bi < (uint32_t)pl.V ? bi : 0u;
        st4c(make_rsrc(fr.codes, (uint32_t)fr.rows * (pl.P - 1) * 4), (uint32_t)(row * (pl.P - 1) + p - 1) * 4, misc[1]);
      }
    }
    __syncthreads();
    embed_row<BF>(pl, fr, p, row, (int)misc[1], false);
  }
  signal_group(pl, tk.sig, tk.sig_slot, persistent, tr);
}

// ------------------------------------------------------------------ executors

template <int BF>
__device__ __forceinline__ void run_task(const DevPlan& pl, const DevFrame& fr, const Task& tk, uint32_t epoch,
                                         uint8_t* slot, uint32_t* misc, bool persistent, uint64_t* tr) {
  switch (tk.type) {
    case T_ATTN: attn_task<BF>(pl, fr, tk, persistent, tr); break;
    case T_EMBED0: embed0_task<BF>(pl, fr, tk, persistent, tr); break;
    case T_DRAW: draw_task<BF>(pl, fr, tk, misc, persistent, tr); break;
    default: proj_task<BF>(pl, fr, tk, epoch, slot, misc, persistent, tr); break;
  }
}

template <int BF>
__global__ __launch_bounds__(kThreads, 1) void persistent_kernel(DevPlan pl, DevFrame fr) {
  extern __shared__ __align__(1024) uint8_t lds[];
  uint32_t* misc = (uint32_t*)(lds + 2 * kSlotBytes);
  const uint32_t epoch = ld_ctr(pl.state);
  const uint32_t b = pl.wg_begin[blockIdx.x], e = pl.wg_begin[blockIdx.x + 1];
  for (uint32_t i = b; i < e; ++i) {
    const Task tk = pl.tasks[i];
    uint64_t* tr = pl.trace_on ? pl.trace + (size_t)i * kTraceStamps : nullptr;
    stamp(tr, 0);
    uint8_t* slot = lds + ((i - b) & 1) * kSlotBytes;
    issue_tile(pl, tk, slot, (uint8_t*)misc);  // lands while the workgroup waits
    wait_deps(pl, tk, epoch);
    stamp(tr, 1);
    run_task<BF>(pl, fr, tk, epoch, slot, misc, true, tr);
  }
  // The last workgroup to finish moves the plan to the next frame.
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(pl.state + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)pl.n_wg * epoch - 1)
      __hip_atomic_store(pl.state, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int BF>
__global__ __launch_bounds__(kThreads, 1) void phase_kernel(DevPlan pl, DevFrame fr, const Task* tasks) {
  extern __shared__ __align__(1024) uint8_t lds[];
  uint32_t* misc = (uint32_t*)(lds + 2 * kSlotBytes);
  const uint32_t epoch = ld_ctr(pl.state);
  const Task tk = tasks[blockIdx.x];
  issue_tile(pl, tk, lds, (uint8_t*)misc);
  run_task<BF>(pl, fr, tk, epoch, lds, misc, false, nullptr);
}

__global__ void bump_epoch_kernel(uint32_t* state) {
  const uint32_t e = ld_ctr(state);
  __hip_atomic_store(state, e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace cpms

// ------------------------------------------------------------------ host-side launchers

namespace cpms {

const void* persistent_kernel_ptr(int bf16) {
  return bf16 ? (const void*)persistent_kernel<1> : (const void*)persistent_kernel<0>;
}

hipError_t launch_persistent(const DevPlan& pl, const DevFrame& fr, hipStream_t s) {
  if (pl.bf16)
    hipLaunchKernelGGL(persistent_kernel<1>, dim3(pl.n_wg), dim3(kThreads), kLdsBytes, s, pl, fr);
  else
    hipLaunchKernelGGL(persistent_kernel<0>, dim3(pl.n_wg), dim3(kThreads), kLdsBytes, s, pl, fr);
  return hipGetLastError();
}

hipError_t launch_phase(const DevPlan& pl, const DevFrame& fr, const Task* tasks, int n, hipStream_t s) {
  if (pl.bf16)
    hipLaunchKernelGGL(phase_kernel<1>, dim3(n), dim3(kThreads), kLdsBytes, s, pl, fr, tasks);
  else
    hipLaunchKernelGGL(phase_kernel<0>, dim3(n), dim3(kThreads), kLdsBytes, s, pl, fr, tasks);
  return hipGetLastError();
}

hipError_t launch_bump_epoch(uint32_t* state, hipStream_t s) {
  hipLaunchKernelGGL(bump_epoch_kernel, dim3(1), dim3(1), 0, s, state);
  return hipGetLastError();
}

hipError_t set_kernel_attributes() {
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)persistent_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)persistent_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes))) return e;
  if ((e = hipFuncSetAttribute((const void*)phase_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes))) return e;
  return hipFuncSetAttribute((const void*)phase_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

int occupancy_per_cu(int bf16) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bf16 ? persistent_kernel<1> : persistent_kernel<0>, kThreads,
                                                   kLdsBytes) != hipSuccess)
    return -1;
  return n;
}

}  // namespace cpms
