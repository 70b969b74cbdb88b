// Internal layout shared by the host planner (cp_plan.cpp) and the device code
// (cp_kernels.hip).  Nothing here crosses the C ABI.
#pragma once
#include <stdint.h>

namespace cpms {

// Task kinds, one per phase type of the frame.
enum TaskType : uint8_t {
  T_INPROJ = 1,  // input projection tile (split-K partial, last arriver reduces)
  T_EMBED0 = 2,  // embedding of code 0 for one row
  T_QKV = 3,     // RMSNorm + qkv projection tile + RoPE
  T_ATTN = 4,    // attention for one kv head and a group of rows
  T_O = 5,       // o projection split-K partial (+ residual by the last arriver)
  T_GU = 6,      // RMSNorm + stacked gate/up tile + SwiGLU
  T_DOWN = 7,    // down projection split-K partial (+ residual by the last arriver)
  T_HEAD = 8,    // final RMSNorm + code head tile + per-tile argmax candidates
  T_DRAW = 9,    // draw + embedding for one row
};

constexpr int kMaxWaits = 4;
constexpr uint32_t kNone = 0xffffffffu;
constexpr int kTileN = 16;          // output slots per projection tile
constexpr int kMaxRows = 128;
constexpr int kThreads = 256;       // 4 waves per workgroup
constexpr int kSlotBytes = 64 * 1024;  // one weight-tile slot in LDS (two slots)
constexpr int kMiscLds = 12288;  // flags, cross-wave reductions
constexpr int kTaskLds = 19968;  // the persistent workgroup's task records (832 of them)
constexpr int kLdsBytes = 2 * kSlotBytes + kMiscLds + kTaskLds;  // 162816 of the CU's 163840
constexpr int kCtrStride = 32;      // uint32 words between sub-counters (128 B)
constexpr int kTraceStamps = 8;     // timestamps per task in a traced frame

// A group of sub-counters: a phase (or part of one) signals it, a later task
// waits on it.  Producer i adds to sub-counter i % nsub; each sub-counter
// receives per_sub adds per frame, so a frame's epoch e is complete at
// per_sub * e.
struct CtrGroup {
  uint32_t base;     // index of the first sub-counter (in units of kCtrStride words)
  uint16_t nsub;
  uint16_t per_sub;
};

constexpr uint32_t kKvPhase = 1023;  // tag phase of K/V cache words (each written once per frame)
constexpr int kMaxPhases = 1023;     // phase ids must stay below kKvPhase
// A tag is epoch * 1024 + phase in 32 bits, so epochs live in [1, kEpochWrap).
// Before the epoch would reach kEpochWrap every tagged buffer is cleared and
// the count restarts at 1 (epoch 0 is the tag of cleared memory).
constexpr uint32_t kEpochWrap = (1u << 22) - 1;
constexpr int kMaxClear = 16;
// Reloads of stale data a device-side wait makes before it gives up.
constexpr uint32_t kDefaultSpinLimit = 1u << 22;
// Device bytes the library holds on each device for the scratch of a plan
// made by cp_plan_create_static.
constexpr size_t kStaticScratchBytes = (size_t)160 << 20;

// Task flag: the split-K partners of this task's tile and their owner run on
// workgroups of one XCD, so partials go through that XCD's L2 (plain stores,
// agent-coherent loads) instead of out to memory and back.
constexpr uint8_t kTaskLocalPartials = 1;
// Task flag (qkv): the attention tasks that read this tile's q, k and v run on
// this workgroup's XCD, so the stores stay in its L2.
constexpr uint8_t kTaskLocalQkv = 2;
// Task flags, bits 4-7: the row group of a projection task when the plan
// runs row groups (DevPlan::grp_rows rows each).
constexpr int kTaskGroupShift = 4;

struct Span {
  void* p;
  uint64_t bytes;  // a multiple of 8
};

struct Task {
  uint8_t type;
  uint8_t split;     // split-K index
  uint8_t nsplit;    // split-K ways (1: not split)
  uint8_t flags;     // kTaskLocalPartials, kTaskLocalQkv
  uint16_t layer;
  uint16_t pos;
  uint32_t tile;     // projection n-tile, attention (kv head, row group), row
  uint16_t phase;    // global phase index (tags this task's outputs)
  uint16_t ph_in0;   // phase whose outputs are this task's main input
  uint16_t ph_in1;   // phase of the residual input (o / down), else unused
  uint16_t pad1;
  uint32_t w_off;    // byte offset of the packed weight tile
  uint32_t w_bytes;  // its size (multiple of 1 KiB), 0 for tasks without weights
  // Dependency description used only by the host validator: counter groups
  // the task reads from and the group it completes.
  uint32_t wait[kMaxWaits];
  uint32_t nwait;
  uint32_t sig;
  uint32_t sig_slot;
};

// What a workgroup needs to run one task (24 bytes, six scalar registers):
// the host's Task without the dependency bookkeeping its validator uses.
struct DevTask {
  uint8_t type, split, nsplit, flags;
  uint16_t layer, pos;
  uint16_t tile, phase;
  uint16_t ph_in0, ph_in1;
  uint32_t w_off, w_bytes;
};
static_assert(sizeof(DevTask) == 24, "DevTask layout");

struct DevPlan {
  // shapes
  int L, H, Din, nq, nkv, d, I, P, V, Rmax;
  int gq;             // q heads per kv head
  int attn_rows;      // rows per attention task
  int n_head_tiles;   // vocab / 16
  int bf16;           // activation type
  float eps;
  float attn_scale;   // 1 / sqrt(head_dim)
  uint32_t spin_limit;
  int n_wg;
  int n_tasks;
  int tasks_in_lds;             // every workgroup's list fits kTaskLds: the executor copies it to LDS
  int layout_pad0;              // unused (see layout_pad1)
  int local_ok;                 // XCD-local hand-offs allowed (not CP_FLAG_NO_LOCAL)
  int grp_rows;                 // CP_FLAG_ROW_GROUPS: rows per projection task (0: all, in passes of 64)
  // task lists
  const DevTask* tasks;         // all tasks, grouped by workgroup
  const uint32_t* wg_begin;     // [n_wg + 1]
  uint32_t* state;              // [0] epoch, [64] error word, [96] clear pending,
                                // [128 + 32 (epoch & 1)] frame-end arrivals of the persistent executor
  // weights (plan-owned copies)
  const uint8_t* wblob;         // packed projection tiles
  const void* embed;            // [P][V][H]
  const float* rope;            // [P][d/2][2]: cos, sin
  const float* qk_gain;         // QK-norm: [L][q, k][d] head-norm gains (else null)
  int qk_norm;                  // the QK-norm variant
  // activations and scratch (act = dtype)
  // The buffers a projection reads (position inputs, residuals, attention
  // and SwiGLU outputs) hold plain activations in the kernels' operand order
  // (sop_off in the kernel source), one plane per layer and position, so
  // that no element is written twice in a frame; an element not yet written
  // holds the sentinel (all bits set), and the whole region is refilled with
  // it at the end of every frame.  Rp = Rmax rounded up to 16.  The other
  // cross-workgroup buffers hold tagged 64-bit words (2 * dtype size bytes
  // per element); those marked [2] are doubled by position parity:
  // positions 0 and 1 can be in flight at the same time.
  void* xin;                    // [P][Rp][H] position inputs
  void* hres;                   // [L][P][Rp][H] residual after down
  void* hmid;                   // [L][P][Rp][H] residual after o
  void* abuf;                   // [L][P][Rp][nq d] attention output
  void* mbuf;                   // [L][P][Rp][I] SwiGLU output
  void* opbuf;                  // the region holding the five above
  uint64_t opbuf_bytes;
  void* qbuf;                   // [2][Rmax][nq d] rotated q, row-major, tagged
  void* kc;                     // [L][Rmax][nkv][P][d]
  void* kraw;                   // QK-norm: [2][Rmax][nkv][d] K before its head norm, right after kc
  uint64_t* qkn;                // QK-norm: [2][Rmax][nq + nkv][d/16] per-tile sums of squares of q, k heads
  void* vc;
  uint64_t* part;               // split-K partials, each buffer [H/16 tiles][nsplit][Rmax][16] words
  // Unused.  With this word and layout_pad0 left out of the kernel argument,
  // the executor's code came out 23 us per 64-row frame slower (measured
  // A/B, same sources otherwise).
  uint32_t* layout_pad1;
  uint64_t* zbuf;               // [Rmax][V] words: logits of the current head
  uint64_t* cand;               // [Rmax][n_head_tiles][2] words: (value, index) of each head tile
  uint64_t* trace;              // plan-owned trace staging (unused if no trace)
  int trace_on;
  int n_o_split, n_d_split, n_in_split;
  uint64_t part_o_off, part_d_off, part_in_off;  // word offsets into part
  uint64_t part_stride;                          // words of one split-K buffer
  Span clear[kMaxClear];                         // every buffer that holds tagged words
  int n_clear;
};

struct DevFrame {
  int rows;
  int sampled;
  int defer_clear;  // K/V are copied out after the kernel: leave a wrap's clear to clear_pending_kernel
  const void* hidden_in;
  const int32_t* code0;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const uint64_t* seed;
  uint64_t* offset;
  int32_t* codes;
  float* embsum;
  float* logits;
  uint64_t* trace;
};

}  // namespace cpms
