// Host side of the depth-loop library: configuration checks, the co-residency
// check, weight repacking, the static per-workgroup task lists and the C ABI
// declared in include/cp.h.
//
// The schedule follows mstar pull request #1183 ("Qwen3-TTS: Run the 1.7B
// Depth Loop as One Persistent Kernel on Hopper"), section "How it works":
// the host builds a static task list per workgroup; a frame is the input
// projection, qkv / attention / o / gate-up / down per layer and position,
// a head per position after the first, and 16 embedding steps (15 after a
// draw); attention waits per kv head; o and down split K across workgroups
// and add the partials in a fixed order.  Deadlock freedom follows the rules
// of the handbook chapter "The gaps between kernels: PDL and megakernels",
// section "Megakernels": the grid is no larger than what is resident at once,
// and every wait points to work that comes earlier in the global phase order,
// which is also the order of every workgroup's own list.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/cp.h"
#include "cp_device.h"

namespace cpms {
hipError_t launch_persistent(const DevPlan& pl, const DevFrame& fr, hipStream_t s);
hipError_t launch_phase(const DevPlan& pl, const DevFrame& fr, const DevTask* tasks, int n, hipStream_t s);
hipError_t launch_bump_epoch(const DevPlan& pl, int defer_clear, hipStream_t s);
hipError_t launch_clear_pending(const DevPlan& pl, hipStream_t s);
hipError_t launch_unpack_kv(const void* src, void* dst, uint32_t words_per_row, uint32_t rows, uint32_t rmax,
                            uint32_t layers, hipStream_t s);
hipError_t set_kernel_attributes();
int occupancy_per_cu(int bf16);
hipError_t check_xcd_dealing(int n_wg, bool& dealt, uint32_t* buf);
hipError_t static_scratch(int device, void** ptr, size_t* bytes);
hipError_t launch_fill(void* p, size_t bytes, uint32_t pattern);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_chain(uint32_t* slots, int n_wg, int n_phases, uint32_t base, int local, int variant, uint32_t* err,
                        hipStream_t s);
}  // namespace cpms

using namespace cpms;

struct cp_plan {
  cp_config cfg{};
  int device = 0;
  int cu_count = 0;
  DevPlan dp{};
  std::vector<Task> tasks;              // grouped by workgroup
  std::vector<uint32_t> wg_begin;
  std::vector<Task> phase_tasks;        // grouped by phase (per-phase executor)
  std::vector<uint32_t> phase_begin;
  std::vector<CtrGroup> groups;
  uint32_t n_ctr = 0;
  int n_phases = 0;
  int crossover = 0;  // frames with fewer rows run the per-phase executor
  int max_tasks_wg = 0;
  bool xcd_dealing = false;             // persistent workgroup i runs on XCD (i + r) % 8, one r per launch (checked)
  DevTask* d_phase_tasks = nullptr;
  std::vector<void*> allocs;
  int64_t packed_bytes = 0, scratch_bytes = 0, weight_bytes_frame = 0;
  std::string err;
  // A plan made by cp_plan_create_static allocates nothing: its scratch is
  // carved from the library's static array on its device, its constants
  // (repacked weights, tables) from the caller's arena.  While `measuring`,
  // alloc() only adds up sizes.
  bool is_static = false, measuring = false;
  uint8_t* st_base = nullptr;
  size_t st_cap = 0, st_used = 0;
  uint8_t* arena = nullptr;
  size_t arena_cap = 0, arena_used = 0;
};

// The live static plan of each device (at most one: they share the array).
static std::mutex g_static_mu;
static const cp_plan* g_static_owner[64];

static thread_local std::string g_create_err;

namespace {

#define HIPCHK(plan, call)                                                                   \
  do {                                                                                       \
    hipError_t e_ = (call);                                                                  \
    if (e_ != hipSuccess) {                                                                  \
      (plan)->err = std::string(#call) + ": " + hipGetErrorString(e_);                       \
      return CP_ERR_HIP;                                                                     \
    }                                                                                        \
  } while (0)

#define TRY(x)                  \
  do {                          \
    cp_status s_ = (x);         \
    if (s_ != CP_OK) return s_; \
  } while (0)

cp_status fail(cp_plan* p, cp_status s, const std::string& msg) {
  p->err = msg;
  return s;
}

// ---------------------------------------------------------------- planning

struct Builder {
  cp_plan* P;
  int n_wg;
  std::vector<std::vector<Task>> per_wg;
  std::vector<std::vector<Task>> per_phase;
  uint32_t next_ctr = 0;

  uint32_t group(int count, int max_sub = 16) {
    // a group of nsub sub-counters, each receiving count / nsub adds per frame
    int nsub = std::min(max_sub, count);
    while (count % nsub) --nsub;
    CtrGroup g{next_ctr, (uint16_t)nsub, (uint16_t)(count / nsub)};
    next_ctr += nsub;
    P->groups.push_back(g);
    return (uint32_t)P->groups.size() - 1;
  }
  uint32_t counter() { return next_ctr++; }

  // Appends one phase; wg_of maps a task's index in the phase to a workgroup.
  int next_phase() const { return (int)per_phase.size(); }
  void phase(std::vector<Task> ts, const std::vector<int>& wg_of) {
    const uint32_t ph = (uint32_t)per_phase.size();
    for (size_t i = 0; i < ts.size(); ++i) {
      ts[i].phase = (uint16_t)ph;
      per_wg[wg_of[i] % n_wg].push_back(ts[i]);
    }
    per_phase.push_back(std::move(ts));
  }
};

Task make_task(uint8_t type, int l, int p, uint32_t tile) {
  Task t{};
  t.type = type;
  t.layer = (uint16_t)l;
  t.pos = (uint16_t)p;
  t.tile = tile;
  t.nsplit = 1;
  t.sig = kNone;
  for (auto& w : t.wait) w = kNone;
  return t;
}

void add_wait(Task& t, uint32_t g) {
  if (t.nwait < (uint32_t)kMaxWaits) t.wait[t.nwait++] = g;
}

// Spreads n tasks over the workgroups starting at a rotating offset.
std::vector<int> spread(int n, int n_wg, int& rot) {
  std::vector<int> m(n);
  for (int i = 0; i < n; ++i) m[i] = (rot + i) % n_wg;
  rot = (rot + n) % n_wg;
  return m;
}

// Spreads n tasks over the workgroups in rotation order like spread, but
// (when n <= n_wg) puts the workgroups marked late -- the owners of the last
// split-K phase, which add their partners' partial sums after their own K
// part -- after all the others.
std::vector<int> spread_late_last(int n, int n_wg, int& rot, const std::vector<char>& late) {
  if (n > n_wg) return spread(n, n_wg, rot);
  std::vector<int> m;
  for (int pass = 0; pass < 2; ++pass)
    for (int i = 0; i < n_wg && (int)m.size() < n; ++i) {
      const int w = (rot + i) % n_wg;
      if ((late[w] != 0) == (pass == 1)) m.push_back(w);
    }
  rot = (rot + n) % n_wg;
  return m;
}

// Split-K tasks (tile t, split s): the nsplit partners of a tile share an XCD
// (workgroups are dealt to XCDs round-robin by id) when the phase fills the
// grid; `local` tells whether they do.
std::vector<int> split_map(int tiles, int nsplit, int n_wg, int& rot, bool& local) {
  std::vector<int> m(tiles * nsplit);
  local = tiles * nsplit <= n_wg && n_wg % 8 == 0 && tiles % 8 == 0;
  if (local) {
    // a rotating start in whole groups of 8 keeps tile t on XCD t % 8
    const int base = (rot / 8) * 8;
    for (int t = 0; t < tiles; ++t)
      for (int s = 0; s < nsplit; ++s) m[t * nsplit + s] = (base + ((t / 8) * nsplit + s) * 8 + (t % 8)) % n_wg;
    rot = (rot + tiles * nsplit) % n_wg;
    return m;
  }
  return spread(tiles * nsplit, n_wg, rot);
}

void mark_local(std::vector<Task>& ts, bool local, uint8_t flag = kTaskLocalPartials) {
  if (local)
    for (Task& t : ts) t.flags |= flag;
}

// Tasks dealt to the workgroups of given XCDs (workgroup i runs on XCD i % 8):
// task k goes to XCD xcd[k], to that XCD's workgroups in turn from a rotating
// start.  Needs n_wg % 8 == 0.
std::vector<int> xcd_deal(const std::vector<int>& xcd, int n_wg, int& rot) {
  std::vector<int> m(xcd.size());
  int rank[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int per = n_wg / 8, start = (rot / 8) % per;
  for (size_t k = 0; k < xcd.size(); ++k) {
    const int x = xcd[k] % 8;
    m[k] = ((start + rank[x]++) % per) * 8 + x;
  }
  rot = (rot + (int)xcd.size()) % n_wg;
  return m;
}

}  // namespace

// fp32 -> bf16 bits, round to nearest even (finite inputs: products of
// finite weights and gains).
static uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Appends rows[*][k0, k0 + kt) in MFMA fragment order: for each K chunk c
// (4 * E elements), each 16-row block b, each lane (row lane % 16, elements
// (lane / 16) * E ... + E - 1 of the chunk): 16 bytes.  With `gain`, every
// element is first multiplied by gain[k] in fp32 and rounded back to the
// storage type: the RMSNorm gain that precedes the projection, folded in.
static void pack_tile(std::vector<uint8_t>& blob, const std::vector<const uint8_t*>& rows, int k0, int kt, int esz,
                      const float* gain = nullptr) {
  const int E = 16 / esz, KS = 4 * E, nb = (int)rows.size() / 16;
  for (int c = 0; c < kt / KS; ++c)
    for (int b = 0; b < nb; ++b)
      for (int lane = 0; lane < 64; ++lane) {
        const int k = k0 + c * KS + (lane / 16) * E;
        const uint8_t* src = rows[16 * b + lane % 16] + (size_t)k * esz;
        if (!gain) {
          blob.insert(blob.end(), src, src + 16);
          continue;
        }
        uint8_t out[16];
        for (int e = 0; e < E; ++e) {
          float f;
          if (esz == 2) {
            const uint32_t bits = (uint32_t)((const uint16_t*)src)[e] << 16;
            std::memcpy(&f, &bits, 4);
            const uint16_t r = to_bf16(f * gain[k + e]);
            std::memcpy(out + 2 * e, &r, 2);
          } else {
            std::memcpy(&f, src + 4 * e, 4);
            f *= gain[k + e];
            std::memcpy(out + 4 * e, &f, 4);
          }
        }
        blob.insert(blob.end(), out, out + 16);
      }
}

static cp_status validate(const cp_config* c, std::string& msg) {
  if (c->abi_version != CP_ABI_VERSION) { msg = "abi_version mismatch"; return CP_ERR_UNSUPPORTED; }
  if (c->n_layers < 1 || c->hidden < 1 || c->input_dim < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 1 || c->intermediate < 1 || c->n_positions < 1 || c->vocab < 1 || c->max_rows < 1) {
    msg = "non-positive size";
    return CP_ERR_INVALID_ARGUMENT;
  }
  if (c->dtype != CP_DTYPE_F32 && c->dtype != CP_DTYPE_BF16) { msg = "dtype"; return CP_ERR_UNSUPPORTED; }
  if (c->exec != CP_EXEC_PERSISTENT && c->exec != CP_EXEC_PER_PHASE) { msg = "exec"; return CP_ERR_UNSUPPORTED; }
  const int esz = c->dtype == CP_DTYPE_BF16 ? 2 : 4;
  if (c->head_dim != 64 && c->head_dim != 128) { msg = "head_dim must be 64 or 128"; return CP_ERR_UNSUPPORTED; }
  if (c->n_q_heads % c->n_kv_heads) { msg = "n_q_heads must be a multiple of n_kv_heads"; return CP_ERR_UNSUPPORTED; }
  if (c->n_positions < 2 || c->n_positions > 16) { msg = "n_positions must be in 2..16"; return CP_ERR_UNSUPPORTED; }
  if (c->max_rows > kMaxRows) { msg = "max_rows must be <= 128"; return CP_ERR_UNSUPPORTED; }
  if (c->vocab != 256 && c->vocab != 512 && c->vocab != 1024 && c->vocab != 2048 && c->vocab != 4096) {
    msg = "vocab must be 256, 512, 1024, 2048 or 4096";
    return CP_ERR_UNSUPPORTED;
  }
  if (c->hidden % 64 || c->input_dim % 256 || c->intermediate % 256 || c->vocab % 64) {
    msg = "input_dim and intermediate must be multiples of 256, hidden and vocab of 64";
    return CP_ERR_UNSUPPORTED;
  }
  if (c->hidden % 256 || c->hidden > 1024) { msg = "hidden must be a multiple of 256, at most 1024"; return CP_ERR_UNSUPPORTED; }
  if ((c->n_q_heads * c->head_dim / 4) * esz > 2048 || (c->intermediate / 4) * esz > 2048 ||
      (c->input_dim / 4) * esz > 2048) {
    msg = "split-K slice too large";
    return CP_ERR_UNSUPPORTED;
  }
  if (c->n_q_heads % 4) { msg = "n_q_heads must be a multiple of 4"; return CP_ERR_UNSUPPORTED; }
  // an o split (n_q_heads / 4 heads) must read at most kMaxWaits kv heads
  const int gq = c->n_q_heads / c->n_kv_heads, hps = c->n_q_heads / 4;
  if ((hps - 1) / gq + 2 > kMaxWaits && hps / gq > kMaxWaits) { msg = "kv grouping not supported"; return CP_ERR_UNSUPPORTED; }
  if (c->flags & ~(CP_FLAG_TRACE | CP_FLAG_NO_LOCAL | CP_FLAG_ROW_GROUPS)) {
    msg = "unknown flag";
    return CP_ERR_UNSUPPORTED;
  }
  if ((c->flags & CP_FLAG_ROW_GROUPS) && c->exec != CP_EXEC_PERSISTENT) {
    msg = "CP_FLAG_ROW_GROUPS needs the persistent executor";
    return CP_ERR_UNSUPPORTED;
  }
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) { msg = "rms_eps / rope_theta"; return CP_ERR_INVALID_ARGUMENT; }
  return CP_OK;
}

// Split-K ways for o, down and the input projection: four where the shapes
// allow.  The partners of a tile share the owner's XCD and hand over their
// partials through its L2 (about 0.5 us), so splitting pays at every row
// count: it cuts the activation bytes each workgroup streams by four (at 1
// row, 2.75 -> 2.41 ms per frame against unsplit o and halved down).  A
// choice must keep the weight tile within one LDS slot, each wave's K share
// within 32 chunks and in whole operand groups of 8 chunks, and every o split
// on whole kv heads.
static cp_status choose_splits(cp_plan* P) {
  const cp_config& c = P->cfg;
  const int esz = c.dtype == CP_DTYPE_BF16 ? 2 : 4;
  const int R = c.max_rows;
  const int nrt = (R + 15) / 16, wpr_min = nrt == 1 ? 4 : (nrt == 2 ? 2 : 1);
  const int gq = c.n_q_heads / c.n_kv_heads;
  auto ok = [&](int K, int ns) {
    if (K % (16 * ns)) return false;
    const int kt = K / ns;
    const int nck = kt * esz / 64;
    return kt * esz * 64 % 64 == 0 && nck % 8 == 0 && 16 * kt * esz <= kSlotBytes && nck / wpr_min <= 32;
  };
  const int order[3] = {4, 2, 1};
  int ns_o = 0, ns_d = 0, ns_in = 0;
  for (int i = 0; i < 3 && !ns_o; ++i) {
    const int ns = order[i];
    if (c.n_q_heads % ns == 0 && (c.n_q_heads / ns) % gq == 0 && c.n_kv_heads % ns == 0 &&
        ok(c.n_q_heads * c.head_dim, ns))
      ns_o = ns;
  }
  for (int i = 0; i < 3 && !ns_d; ++i)
    if ((c.intermediate / 16) % order[i] == 0 && ok(c.intermediate, order[i])) ns_d = order[i];
  for (int i = 0; i < 3 && !ns_in; ++i)
    if (ok(c.input_dim, order[i])) ns_in = order[i];
  if (!ns_o || !ns_d || !ns_in) return fail(P, CP_ERR_UNSUPPORTED, "no split-K choice fits these shapes");
  P->dp.n_o_split = ns_o;
  P->dp.n_d_split = ns_d;
  P->dp.n_in_split = ns_in;
  return CP_OK;
}

static cp_status build_schedule(cp_plan* P) {
  TRY(choose_splits(P));
  const cp_config& c = P->cfg;
  const int L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, d = c.head_dim;
  const int I = c.intermediate, Pn = c.n_positions, V = c.vocab, R = c.max_rows;
  const int gq = nq / nkv;
  const int n_wg = P->cu_count;
  Builder B{P, n_wg, std::vector<std::vector<Task>>(n_wg), {}, 0};
  const int ht = H / 16, qkv_tiles = (nq + 2 * nkv) * d / 16, tpg = (gq + 2) * d / 16;
  const int gu_tiles = I / 16, head_tiles = V / 16;
  const int ns_o = P->dp.n_o_split, ns_d = P->dp.n_d_split, ns_in = P->dp.n_in_split;
  // Row groups: projection tasks of 32 rows, G per tile, run back to back by
  // one workgroup (their signals count G times).
  const int G = (P->cfg.flags & CP_FLAG_ROW_GROUPS) && R > 32 ? (R + 31) / 32 : 1;
  P->dp.grp_rows = G > 1 ? 32 : 0;
  auto grouped = [&](std::vector<Task>& ts, std::vector<int>& m) {
    if (G == 1) return;
    std::vector<Task> t2;
    std::vector<int> m2;
    for (size_t i = 0; i < ts.size(); ++i)
      for (int g = 0; g < G; ++g) {
        Task k = ts[i];
        k.flags |= (uint8_t)(g << kTaskGroupShift);
        t2.push_back(k);
        m2.push_back(m[i]);
      }
    ts.swap(t2);
    m.swap(m2);
  };
  int ar = std::max(1, 4 / gq);
  while (R % ar) --ar;
  const int agroups = R / ar;
  P->dp.attn_rows = ar;
  const int gu_per_split = gu_tiles / ns_d;
  const int kv_per_osplit = nkv / ns_o;  // kv heads whose attention output one o split reads
  int rot = 0;
  std::vector<char> late(n_wg, 0);  // owners of the last split-K phase

  // Every task records the phases whose outputs it reads (ph_in0, ph_in1):
  // its input words must carry those phases' tags.  The counter groups below
  // describe the same dependencies for the host validator.
  // Draws (and the code-0 embedding) of a row always run in one workgroup,
  // which carries the row's embedding sum in program order.
  std::vector<int> row_wg(R);
  for (int r = 0; r < R; ++r) row_wg[r] = r % n_wg;

  // input projection (split-K) and code-0 embedding: no inputs from the frame
  const uint32_t g_inp = B.group(ht * G);
  const int ph_inp = B.next_phase();
  {
    std::vector<Task> ts;
    for (int t = 0; t < ht; ++t)
      for (int s = 0; s < ns_in; ++s) {
        Task k = make_task(T_INPROJ, 0, 0, t);
        k.split = (uint8_t)s; k.nsplit = (uint8_t)ns_in; k.sig = g_inp; k.sig_slot = t;
        ts.push_back(k);
      }
    bool local = false;
    std::vector<int> m = split_map(ht, ns_in, n_wg, rot, local);
    mark_local(ts, local);
    grouped(ts, m);
    B.phase(ts, m);
  }
  const uint32_t g_emb0 = B.group(R);
  const int ph_emb0 = B.next_phase();
  {
    std::vector<Task> ts;
    for (int r = 0; r < R; ++r) {
      Task k = make_task(T_EMBED0, 0, 0, r);
      k.sig = g_emb0; k.sig_slot = r;
      ts.push_back(k);
    }
    B.phase(ts, row_wg);
  }

  std::vector<std::vector<uint32_t>> g_qkv(Pn * L);  // [p * L + l][g]
  std::vector<std::vector<uint32_t>> g_attn(Pn * L);  // [p * L + l][o split]
  const bool qkn = P->cfg.qk_norm != 0;
  uint32_t g_prev_draw = kNone;
  int ph_prev_draw = -1;
  for (int p = 0; p < Pn; ++p) {
    uint32_t g_layer_in = (p == 0) ? g_inp : (p == 1 ? g_emb0 : g_prev_draw);
    int ph_layer_in = (p == 0) ? ph_inp : (p == 1 ? ph_emb0 : ph_prev_draw);
    for (int l = 0; l < L; ++l) {
      // qkv
      std::vector<uint32_t>& gq_groups = g_qkv[p * L + l];
      for (int g = 0; g < nkv; ++g) gq_groups.push_back(B.group(tpg * G, 4));
      const int ph_qkv = B.next_phase();
      {
        std::vector<Task> ts;
        for (int t = 0; t < qkv_tiles; ++t) {
          Task k = make_task(T_QKV, l, p, t);
          add_wait(k, g_layer_in);
          k.ph_in0 = (uint16_t)ph_layer_in;
          k.sig = gq_groups[t / tpg]; k.sig_slot = t % tpg;
          ts.push_back(k);
        }
        // kv group g's tiles on XCD g % 8, where its attention tasks run
        if (n_wg % 8 == 0) {
          std::vector<int> x(qkv_tiles);
          for (int t = 0; t < qkv_tiles; ++t) x[t] = t / tpg;
          mark_local(ts, true, kTaskLocalQkv);
          std::vector<int> m = xcd_deal(x, n_wg, rot);
          grouped(ts, m);
          B.phase(ts, m);
        } else {
          std::vector<int> m = spread(qkv_tiles, n_wg, rot);
          grouped(ts, m);
          B.phase(ts, m);
        }
      }
      // Position 0 has no head: the residual after its last layer feeds
      // nothing, so only the last layer's qkv (its K/V) is computed there --
      // and, with QK-norm, its attention, which writes the normed K.
      if (p == 0 && l == L - 1 && !qkn) break;
      // attention, per kv head; it completes the group of the o split that reads it
      std::vector<uint32_t> g_att(ns_o);
      for (int s = 0; s < ns_o; ++s) g_att[s] = B.group(kv_per_osplit * agroups);
      const int ph_att = B.next_phase();
      {
        std::vector<Task> ts;
        for (int g = 0; g < nkv; ++g)
          for (int rg = 0; rg < agroups; ++rg) {
            Task k = make_task(T_ATTN, l, p, g * agroups + rg);
            add_wait(k, gq_groups[g]);
            if (p == 1) add_wait(k, g_qkv[0 * L + l][g]);  // position 0's K/V of this layer
            // QK-norm: earlier positions' K, normed and stored by their attention
            if (qkn && p >= 1) add_wait(k, g_attn[(p - 1) * L + l][g / kv_per_osplit]);
            k.ph_in0 = (uint16_t)ph_qkv;
            k.sig = g_att[g / kv_per_osplit]; k.sig_slot = (g % kv_per_osplit) * agroups + rg;
            ts.push_back(k);
          }
        if (n_wg % 8 == 0) {
          std::vector<int> x(nkv * agroups);
          for (int i = 0; i < nkv * agroups; ++i) x[i] = i / agroups;
          B.phase(ts, xcd_deal(x, n_wg, rot));
        } else {
          B.phase(ts, spread(nkv * agroups, n_wg, rot));
        }
      }
      g_attn[p * L + l] = g_att;
      if (p == 0 && l == L - 1) break;
      // o (split-K over q heads; a split reads only the kv heads of its slice)
      const uint32_t g_o = B.group(ht * G);
      const int ph_o = B.next_phase();
      {
        std::vector<Task> ts;
        for (int t = 0; t < ht; ++t)
          for (int s = 0; s < ns_o; ++s) {
            Task k = make_task(T_O, l, p, t);
            k.split = (uint8_t)s; k.nsplit = (uint8_t)ns_o; k.sig = g_o; k.sig_slot = t;
            k.ph_in0 = (uint16_t)ph_att;
            k.ph_in1 = (uint16_t)ph_layer_in;
            add_wait(k, g_att[s]);
            add_wait(k, g_layer_in);  // the residual
            ts.push_back(k);
          }
        bool local = false;
        std::vector<int> m = split_map(ht, ns_o, n_wg, rot, local);
        mark_local(ts, local);
        late.assign(n_wg, 0);
        for (int t = 0; t < ht; ++t) late[m[t * ns_o] % n_wg] = 1;
        grouped(ts, m);
        B.phase(ts, m);
      }
      // gate/up
      std::vector<uint32_t> g_gu(ns_d);
      for (int s = 0; s < ns_d; ++s) g_gu[s] = B.group(gu_per_split * G, 4);
      const int ph_gu = B.next_phase();
      {
        std::vector<Task> ts;
        for (int t = 0; t < gu_tiles; ++t) {
          Task k = make_task(T_GU, l, p, t);
          add_wait(k, g_o);
          k.ph_in0 = (uint16_t)ph_o;
          k.sig = g_gu[t / gu_per_split]; k.sig_slot = t % gu_per_split;
          ts.push_back(k);
        }
        // One-row frames: off the o owners, whose sums come last (about 30 us
        // per frame; slower by 20 us at 64 rows, where it is not used).
        std::vector<int> m = R == 1 ? spread_late_last(gu_tiles, n_wg, rot, late) : spread(gu_tiles, n_wg, rot);
        grouped(ts, m);
        B.phase(ts, m);
      }
      // down (split-K over the intermediate; a split reads the gate/up tiles of its slice)
      const uint32_t g_down = B.group(ht * G);
      const int ph_down = B.next_phase();
      {
        std::vector<Task> ts;
        for (int t = 0; t < ht; ++t)
          for (int s = 0; s < ns_d; ++s) {
            Task k = make_task(T_DOWN, l, p, t);
            k.split = (uint8_t)s; k.nsplit = (uint8_t)ns_d; k.sig = g_down; k.sig_slot = t;
            k.ph_in0 = (uint16_t)ph_gu;
            k.ph_in1 = (uint16_t)ph_o;
            add_wait(k, g_gu[s]);
            add_wait(k, g_o);  // the residual
            ts.push_back(k);
          }
        bool local = false;
        std::vector<int> m = split_map(ht, ns_d, n_wg, rot, local);
        mark_local(ts, local);
        late.assign(n_wg, 0);
        for (int t = 0; t < ht; ++t) late[m[t * ns_d] % n_wg] = 1;
        grouped(ts, m);
        B.phase(ts, m);
      }
      g_layer_in = g_down;
      ph_layer_in = ph_down;
    }
    if (p == 0) continue;
    // head p and draw p
    const uint32_t g_head = B.group(head_tiles * G);
    const int ph_head = B.next_phase();
    {
      std::vector<Task> ts;
      for (int t = 0; t < head_tiles; ++t) {
        Task k = make_task(T_HEAD, L - 1, p, t);
        add_wait(k, g_layer_in);
        k.ph_in0 = (uint16_t)ph_layer_in;
        k.sig = g_head; k.sig_slot = t;
        ts.push_back(k);
      }
      std::vector<int> m = spread_late_last(head_tiles, n_wg, rot, late);  // off the down owners
      grouped(ts, m);
      B.phase(ts, m);
    }
    const uint32_t g_draw = B.group(R);
    const int ph_draw = B.next_phase();
    {
      std::vector<Task> ts;
      for (int r = 0; r < R; ++r) {
        Task k = make_task(T_DRAW, L - 1, p, r);
        add_wait(k, g_head);
        k.ph_in0 = (uint16_t)ph_head;
        k.sig = g_draw; k.sig_slot = r;
        ts.push_back(k);
      }
      B.phase(ts, row_wg);
    }
    g_prev_draw = g_draw;
    ph_prev_draw = ph_draw;
  }
  if (B.next_phase() > kMaxPhases) return fail(P, CP_ERR_UNSUPPORTED, "too many phases for the tag space");

  P->n_ctr = B.next_ctr;  // counters of the validator's dependency model (not allocated)
  P->n_phases = (int)B.per_phase.size();
  P->tasks.clear();
  P->wg_begin.assign(1, 0);
  P->max_tasks_wg = 0;
  for (auto& v : B.per_wg) {
    P->tasks.insert(P->tasks.end(), v.begin(), v.end());
    P->wg_begin.push_back((uint32_t)P->tasks.size());
    P->max_tasks_wg = std::max(P->max_tasks_wg, (int)v.size());
  }
  P->phase_tasks.clear();
  P->phase_begin.assign(1, 0);
  for (auto& v : B.per_phase) {
    P->phase_tasks.insert(P->phase_tasks.end(), v.begin(), v.end());
    P->phase_begin.push_back((uint32_t)P->phase_tasks.size());
  }
  return CP_OK;
}

// Checks the schedule invariants that deadlock freedom and correctness rest
// on: waits only point to groups signalled by earlier phases; every group
// receives exactly its per-frame count; each workgroup's list is in phase
// order; weight tiles fit an LDS slot and the packed blob.
static cp_status check_schedule(cp_plan* P) {
  const size_t ng = P->groups.size();
  std::vector<int> first_sig(ng, INT32_MAX), last_sig(ng, -1);
  std::vector<int64_t> count(ng, 0);
  std::vector<std::vector<int>> slot_count(ng);
  for (size_t g = 0; g < ng; ++g) slot_count[g].assign(P->groups[g].nsub, 0);
  std::vector<int> split_seen;
  for (const Task& t : P->phase_tasks) {
    if (t.sig != kNone) {
      if (t.sig >= ng) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: bad signal group");
      first_sig[t.sig] = std::min(first_sig[t.sig], (int)t.phase);
      last_sig[t.sig] = std::max(last_sig[t.sig], (int)t.phase);
      // split-K tasks signal once per tile (by the last arriver)
      if (t.nsplit == 1 || t.split == 0) {
        count[t.sig] += 1;
        slot_count[t.sig][t.sig_slot % P->groups[t.sig].nsub] += 1;
      }
    }
    if (t.w_bytes > (uint32_t)kSlotBytes || t.w_bytes % 1024) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: weight tile too large");
    if ((int64_t)t.w_off + t.w_bytes > P->packed_bytes) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: tile outside blob");
    if (t.type != T_INPROJ && t.type != T_EMBED0 && t.ph_in0 >= t.phase)
      return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: input from a later phase");
    if ((t.type == T_O || t.type == T_DOWN) && t.ph_in1 >= t.phase)
      return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: residual from a later phase");
  }
  for (size_t g = 0; g < ng; ++g) {
    const CtrGroup& G = P->groups[g];
    if (count[g] != (int64_t)G.nsub * G.per_sub) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: group count mismatch");
    for (int s = 0; s < G.nsub; ++s)
      if (slot_count[g][s] != G.per_sub) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: sub-counter count mismatch");
  }
  for (const Task& t : P->phase_tasks)
    for (uint32_t k = 0; k < t.nwait; ++k) {
      if (t.wait[k] >= ng) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: bad wait group");
      if (last_sig[t.wait[k]] >= (int)t.phase) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: wait on a later phase");
    }
  for (size_t w = 0; w + 1 < P->wg_begin.size(); ++w)
    for (uint32_t i = P->wg_begin[w] + 1; i < P->wg_begin[w + 1]; ++i)
      if (P->tasks[i].phase < P->tasks[i - 1].phase) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: list out of order");
  // A split-K owner waits for its partners in the same phase: no partner may
  // sit later in the owner's own list, and a phase with partners must fit the
  // grid (the per-phase executor runs it as one co-resident launch).
  for (size_t w = 0; w + 1 < P->wg_begin.size(); ++w)
    for (uint32_t i = P->wg_begin[w]; i < P->wg_begin[w + 1]; ++i) {
      const Task& a = P->tasks[i];
      if (a.nsplit > 1 && a.split == 0)
        for (uint32_t j = i + 1; j < P->wg_begin[w + 1] && P->tasks[j].phase == a.phase; ++j)
          if (P->tasks[j].tile == a.tile && P->tasks[j].split != 0 &&
              (P->tasks[j].flags >> kTaskGroupShift) == (a.flags >> kTaskGroupShift))
            return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: split partner after its owner");
    }
  for (size_t ph = 0; ph + 1 < P->phase_begin.size() && P->cfg.exec == CP_EXEC_PER_PHASE; ++ph) {
    const Task& f = P->phase_tasks[P->phase_begin[ph]];
    if (f.nsplit > 1 && (int)(P->phase_begin[ph + 1] - P->phase_begin[ph]) > P->cu_count)
      return fail(P, CP_ERR_UNSUPPORTED, "schedule: split phase larger than the grid");
  }
  // XCD-local hand-offs (workgroup w runs on XCD w % 8): the partners of a
  // kTaskLocalPartials tile share its owner's XCD, and the qkv tiles marked
  // kTaskLocalQkv share the XCD of every attention task reading them (same
  // layer, position, kv group).  A broken placement would make a reader spin
  // on words that never leave another XCD's L2.
  {
    const int nkv = P->cfg.n_kv_heads, tpg = (P->cfg.n_q_heads / nkv + 2) * P->cfg.head_dim / 16;
    const int agroups = P->cfg.max_rows / std::max(1, P->dp.attn_rows);
    std::vector<int> owner_xcd(P->n_phases * 4096, -1), qkv_xcd(P->n_phases * 64, -1);
    for (size_t w = 0; w + 1 < P->wg_begin.size(); ++w)
      for (uint32_t i = P->wg_begin[w]; i < P->wg_begin[w + 1]; ++i) {
        const Task& t = P->tasks[i];
        const int x = (int)(w % 8);
        if ((t.flags & kTaskLocalPartials) && t.split == 0 && t.tile < 4096) owner_xcd[t.phase * 4096 + t.tile] = x;
        if ((t.flags & kTaskLocalQkv) && (int)(t.tile / tpg) < 64) {
          int& q = qkv_xcd[t.phase * 64 + t.tile / tpg];
          if (q >= 0 && q != x) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: a kv group's qkv tiles span XCDs");
          q = x;
        }
      }
    for (size_t w = 0; w + 1 < P->wg_begin.size(); ++w)
      for (uint32_t i = P->wg_begin[w]; i < P->wg_begin[w + 1]; ++i) {
        const Task& t = P->tasks[i];
        const int x = (int)(w % 8);
        if ((t.flags & kTaskLocalPartials) && t.split != 0 && t.tile < 4096 && owner_xcd[t.phase * 4096 + t.tile] != x)
          return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: split partner off its owner's XCD");
        if (t.type == T_ATTN) {
          const int g = (int)t.tile / agroups;
          const int q = g < 64 ? qkv_xcd[t.ph_in0 * 64 + g] : -1;
          if (q >= 0 && q != x) return fail(P, CP_ERR_INVALID_ARGUMENT, "schedule: attention off its kv group's XCD");
        }
      }
  }
  return CP_OK;
}

// ---------------------------------------------------------------- weights

static cp_status fetch(cp_plan* P, const void* dptr, size_t bytes, std::vector<uint8_t>& out) {
  if (!dptr) return fail(P, CP_ERR_INVALID_ARGUMENT, "NULL weight pointer");
  out.resize(bytes);
  HIPCHK(P, hipMemcpy(out.data(), dptr, bytes, hipMemcpyDeviceToHost));
  return CP_OK;
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Device allocation, zero-filled (or filled with `fill`, a byte repeated):
// memory a previous plan freed may still hold tagged words that a frame of
// this plan would otherwise accept.  Tagged buffers are also recorded for the
// clear at the epoch wrap.  A static plan carves it from the library's array
// and fills it with a kernel.
static cp_status alloc(cp_plan* P, void** p, size_t bytes, bool tagged = false, uint8_t fill = 0) {
  if (bytes == 0) bytes = 256;
  bytes = (bytes + 15) & ~(size_t)15;
  if (P->is_static) {
    const size_t off = round256(P->st_used);
    P->st_used = off + bytes;
    *p = P->st_base + off;  // (while measuring: a placeholder, never dereferenced)
    if (!P->measuring) {
      if (P->st_used > P->st_cap) return fail(P, CP_ERR_OUT_OF_MEMORY, "static scratch overflow");
      HIPCHK(P, launch_fill(*p, bytes, 0x01010101u * fill));
    }
  } else {
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
      P->err = std::string("hipMalloc: ") + hipGetErrorString(e);
      return CP_ERR_OUT_OF_MEMORY;
    }
    P->allocs.push_back(*p);
    HIPCHK(P, hipMemset(*p, fill, bytes));
  }
  P->scratch_bytes += (int64_t)bytes;
  if (tagged) {
    if (P->dp.n_clear >= kMaxClear) return fail(P, CP_ERR_INVALID_ARGUMENT, "too many tagged buffers");
    P->dp.clear[P->dp.n_clear++] = Span{*p, (uint64_t)bytes};
  }
  return CP_OK;
}

// Copies host data into plan memory (skipped while a static plan measures).
static cp_status upload(cp_plan* P, void* dst, const void* src, size_t bytes) {
  if (P->measuring) return CP_OK;
  HIPCHK(P, hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice));
  return CP_OK;
}

// Device memory for the plan's constants (repacked weights, embedding
// tables, RoPE table): the caller's arena for a static plan, else alloc().
static cp_status alloc_const(cp_plan* P, void** p, size_t bytes) {
  if (!P->is_static) return alloc(P, p, bytes);
  const size_t off = round256(P->arena_used);
  if (off + bytes > P->arena_cap)
    return fail(P, CP_ERR_INVALID_ARGUMENT, "weight arena too small: needs cp_plan_info.const_bytes (cp_schedule_check)");
  *p = P->arena + off;
  P->arena_used = off + bytes;
  return CP_OK;
}

// Device bytes of a plan's constants, each of the three rounded up to 256.
static int64_t const_bytes(const cp_config& c) {
  const int64_t esz = c.dtype == CP_DTYPE_BF16 ? 2 : 4;
  const int64_t L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, d = c.head_dim;
  const int64_t I = c.intermediate, Pn = c.n_positions, V = c.vocab, Din = c.input_dim;
  const int64_t blob = esz * (L * ((nq + 2 * nkv) * d * H + H * nq * d + 3 * I * H) + (Pn - 1) * V * H + H * Din);
  return (int64_t)(round256((size_t)blob) + round256((size_t)(Pn * V * H * esz)) + round256((size_t)(Pn * d * 4)) +
                   (c.qk_norm ? round256((size_t)(L * 2 * d * 4)) : 0));
}


static cp_status pack_weights(cp_plan* P, const cp_weights* w) {
  const cp_config& c = P->cfg;
  const int L = c.n_layers, H = c.hidden, Din = c.input_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int d = c.head_dim, I = c.intermediate, Pn = c.n_positions, V = c.vocab;
  const int esz = c.dtype == CP_DTYPE_BF16 ? 2 : 4;
  const int gq = nq / nkv, th = d / 16, tpg = (gq + 2) * th, qkv_tiles = nkv * tpg, ht = H / 16;
  const int ns_o = P->dp.n_o_split, ns_d = P->dp.n_d_split, ns_in = P->dp.n_in_split;
  const int qd = nq * d;
  std::vector<uint8_t> blob;
  blob.reserve((size_t)esz * ((size_t)L * ((nq + 2 * nkv) * d * H + H * qd + 3 * I * H) + (size_t)(Pn - 1) * V * H + (size_t)H * Din));
  // offsets [l][kind][tile][split]
  std::vector<uint32_t> off_qkv(L * qkv_tiles), off_o(L * ht * ns_o), off_gu(L * (I / 16)), off_d(L * ht * ns_d);
  std::vector<uint32_t> off_head((Pn - 1) * (V / 16)), off_in(ht * ns_in);
  std::vector<uint8_t> m, m2;
  auto rowp = [&](const std::vector<uint8_t>& mat, int cols, int r) { return mat.data() + (size_t)r * cols * esz; };
  auto check_size = [&]() { return blob.size() < 0xffffffffull; };
  if (!w->w_qkv || !w->w_o || !w->w_gate || !w->w_up || !w->w_down || !w->attn_norm || !w->mlp_norm || !w->embed ||
      !w->w_head)
    return fail(P, CP_ERR_INVALID_ARGUMENT, "NULL weight list");
  // RMSNorm gains, widened to fp32 (exact for bf16): folded into the packed
  // tiles of the projection each norm feeds (qkv, gate/up, heads).
  if (!w->final_norm) return fail(P, CP_ERR_INVALID_ARGUMENT, "NULL final_norm");
  auto gain_f32 = [&](const void* src, std::vector<float>& out) -> cp_status {
    TRY(fetch(P, src, (size_t)H * esz, m));
    out.resize(H);
    for (int i = 0; i < H; ++i) {
      if (esz == 2) {
        const uint32_t bits = (uint32_t)((const uint16_t*)m.data())[i] << 16;
        std::memcpy(&out[i], &bits, 4);
      } else {
        std::memcpy(&out[i], m.data() + (size_t)i * 4, 4);
      }
    }
    return CP_OK;
  };
  std::vector<std::vector<float>> g_attn(L), g_mlp(L);
  std::vector<float> g_final;
  for (int l = 0; l < L; ++l) {
    TRY(gain_f32(w->attn_norm[l], g_attn[l]));
    TRY(gain_f32(w->mlp_norm[l], g_mlp[l]));
  }
  TRY(gain_f32(w->final_norm, g_final));
  for (int l = 0; l < L; ++l) {
    TRY(fetch(P, w->w_qkv[l], (size_t)(nq + 2 * nkv) * d * H * esz, m));
    for (int t = 0; t < qkv_tiles; ++t) {
      const int g = t / tpg, lt = t % tpg;
      std::vector<const uint8_t*> rows(16);
      for (int j = 0; j < 16; ++j) {
        const int qq = j / 4, v = j % 4;
        int r;
        if (lt < (gq + 1) * th) {
          const int tih = lt % th;
          const int dim = 8 * tih + 2 * qq + (v >> 1) + (v & 1) * (d / 2);  // rotary pair layout
          r = (lt < gq * th) ? (g * gq + lt / th) * d + dim : qd + g * d + dim;
        } else {
          r = qd + nkv * d + g * d + 16 * (lt - (gq + 1) * th) + j;
        }
        rows[j] = rowp(m, H, r);
      }
      off_qkv[l * qkv_tiles + t] = (uint32_t)blob.size();
      pack_tile(blob, rows, 0, H, esz, g_attn[l].data());
    }
    TRY(fetch(P, w->w_o[l], (size_t)H * qd * esz, m));
    for (int t = 0; t < ht; ++t)
      for (int s = 0; s < ns_o; ++s) {
        std::vector<const uint8_t*> rows(16);
        for (int j = 0; j < 16; ++j) rows[j] = rowp(m, qd, 16 * t + j);
        off_o[(l * ht + t) * ns_o + s] = (uint32_t)blob.size();
        pack_tile(blob, rows, s * (qd / ns_o), qd / ns_o, esz);
      }
    TRY(fetch(P, w->w_gate[l], (size_t)I * H * esz, m));
    TRY(fetch(P, w->w_up[l], (size_t)I * H * esz, m2));
    for (int t = 0; t < I / 16; ++t) {
      std::vector<const uint8_t*> rows(32);
      for (int j = 0; j < 16; ++j) {
        rows[j] = rowp(m, H, 16 * t + j);
        rows[16 + j] = rowp(m2, H, 16 * t + j);
      }
      off_gu[l * (I / 16) + t] = (uint32_t)blob.size();
      pack_tile(blob, rows, 0, H, esz, g_mlp[l].data());
    }
    TRY(fetch(P, w->w_down[l], (size_t)H * I * esz, m));
    for (int t = 0; t < ht; ++t)
      for (int s = 0; s < ns_d; ++s) {
        std::vector<const uint8_t*> rows(16);
        for (int j = 0; j < 16; ++j) rows[j] = rowp(m, I, 16 * t + j);
        off_d[(l * ht + t) * ns_d + s] = (uint32_t)blob.size();
        pack_tile(blob, rows, s * (I / ns_d), I / ns_d, esz);
      }
    if (!check_size()) return fail(P, CP_ERR_UNSUPPORTED, "packed weights exceed 4 GiB");
  }
  for (int j = 1; j < Pn; ++j) {
    TRY(fetch(P, w->w_head[j - 1], (size_t)V * H * esz, m));
    for (int t = 0; t < V / 16; ++t) {
      std::vector<const uint8_t*> rows(16);
      for (int i = 0; i < 16; ++i) rows[i] = rowp(m, H, 16 * t + i);
      off_head[(j - 1) * (V / 16) + t] = (uint32_t)blob.size();
      pack_tile(blob, rows, 0, H, esz, g_final.data());
    }
  }
  TRY(fetch(P, w->w_in, (size_t)H * Din * esz, m));
  for (int t = 0; t < ht; ++t)
    for (int s = 0; s < ns_in; ++s) {
      std::vector<const uint8_t*> rows(16);
      for (int j = 0; j < 16; ++j) rows[j] = rowp(m, Din, 16 * t + j);
      off_in[t * ns_in + s] = (uint32_t)blob.size();
      pack_tile(blob, rows, s * (Din / ns_in), Din / ns_in, esz);
    }
  if (!check_size()) return fail(P, CP_ERR_UNSUPPORTED, "packed weights exceed 4 GiB");

  // attach tiles to tasks
  auto attach = [&](Task& t) {
    switch (t.type) {
      case T_QKV: t.w_off = off_qkv[t.layer * qkv_tiles + t.tile]; t.w_bytes = 16 * H * esz; break;
      case T_O: t.w_off = off_o[(t.layer * ht + t.tile) * ns_o + t.split]; t.w_bytes = 16 * (qd / ns_o) * esz; break;
      case T_GU: t.w_off = off_gu[t.layer * (I / 16) + t.tile]; t.w_bytes = 32 * H * esz; break;
      case T_DOWN: t.w_off = off_d[(t.layer * ht + t.tile) * ns_d + t.split]; t.w_bytes = 16 * (I / ns_d) * esz; break;
      case T_HEAD: t.w_off = off_head[(t.pos - 1) * (V / 16) + t.tile]; t.w_bytes = 16 * H * esz; break;
      case T_INPROJ: t.w_off = off_in[t.tile * ns_in + t.split]; t.w_bytes = 16 * (Din / ns_in) * esz; break;
      default: t.w_off = 0; t.w_bytes = 0; break;
    }
  };
  for (Task& t : P->tasks) attach(t);
  for (Task& t : P->phase_tasks) attach(t);

  void* dblob;
  if (blob.size() != (size_t)esz * ((size_t)L * ((nq + 2 * nkv) * d * H + H * qd + 3 * I * H) + (size_t)(Pn - 1) * V * H +
                                    (size_t)H * Din))
    return fail(P, CP_ERR_INVALID_ARGUMENT, "internal: packed weight size");
  TRY(alloc_const(P, &dblob, blob.size()));
  HIPCHK(P, hipMemcpy(dblob, blob.data(), blob.size(), hipMemcpyHostToDevice));
  P->dp.wblob = (const uint8_t*)dblob;
  P->packed_bytes = (int64_t)blob.size();

  // embedding tables [P][V][H], RoPE table [P][d/2][2]
  void* de;
  TRY(alloc_const(P, &de, (size_t)Pn * V * H * esz));
  for (int j = 0; j < Pn; ++j) {
    if (!w->embed[j]) return fail(P, CP_ERR_INVALID_ARGUMENT, "NULL embedding table");
    HIPCHK(P, hipMemcpy((uint8_t*)de + (size_t)j * V * H * esz, w->embed[j], (size_t)V * H * esz, hipMemcpyDeviceToDevice));
  }
  P->dp.embed = de;
  std::vector<float> rope((size_t)Pn * (d / 2) * 2);
  for (int p = 0; p < Pn; ++p)
    for (int i = 0; i < d / 2; ++i) {
      const double ang = (double)p * std::pow((double)c.rope_theta, -2.0 * i / (double)d);
      rope[((size_t)p * (d / 2) + i) * 2] = (float)std::cos(ang);
      rope[((size_t)p * (d / 2) + i) * 2 + 1] = (float)std::sin(ang);
    }
  void* dr;
  TRY(alloc_const(P, &dr, rope.size() * 4));
  HIPCHK(P, hipMemcpy(dr, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));
  P->dp.rope = (const float*)dr;
  if (c.qk_norm) {
    // head-norm gains [L][q, k][d], fp32 (exact for bf16)
    if (!w->q_norm || !w->k_norm) return fail(P, CP_ERR_INVALID_ARGUMENT, "NULL q_norm / k_norm list");
    std::vector<float> qk((size_t)L * 2 * d);
    for (int l = 0; l < L; ++l)
      for (int k = 0; k < 2; ++k) {
        const void* src = (k ? w->k_norm : w->q_norm)[l];
        if (!src) return fail(P, CP_ERR_INVALID_ARGUMENT, "NULL q_norm / k_norm");
        TRY(fetch(P, src, (size_t)d * esz, m));
        for (int i = 0; i < d; ++i) {
          float v;
          if (esz == 2) {
            const uint32_t bits = (uint32_t)((const uint16_t*)m.data())[i] << 16;
            std::memcpy(&v, &bits, 4);
          } else {
            std::memcpy(&v, m.data() + (size_t)i * 4, 4);
          }
          if (!std::isfinite(v)) return fail(P, CP_ERR_INVALID_ARGUMENT, "non-finite q_norm / k_norm gain");
          qk[((size_t)l * 2 + k) * d + i] = v;
        }
      }
    void* dq;
    TRY(alloc_const(P, &dq, qk.size() * 4));
    HIPCHK(P, hipMemcpy(dq, qk.data(), qk.size() * 4, hipMemcpyHostToDevice));
    P->dp.qk_gain = (const float*)dq;
  }
  int64_t wb = (int64_t)esz * ((int64_t)Pn * L * ((nq + 2 * nkv) * d * H + (int64_t)H * qd + 3LL * I * H) +
                               (int64_t)(Pn - 1) * V * H + (int64_t)H * Din);
  P->weight_bytes_frame = wb;
  return CP_OK;
}

// Device records of host tasks (fields the kernels read; every value fits).
// Device task records; `local` keeps the XCD-local flags (persistent grid on
// a device whose workgroup-to-XCD dealing was checked), else they are cleared.
static std::vector<DevTask> to_dev(const std::vector<Task>& ts, bool local) {
  std::vector<DevTask> out(ts.size());
  for (size_t i = 0; i < ts.size(); ++i) {
    const Task& t = ts[i];
    DevTask& d = out[i];
    d.type = t.type; d.split = t.split; d.nsplit = t.nsplit;
    d.flags = local ? t.flags : (uint8_t)(t.flags & ~(kTaskLocalPartials | kTaskLocalQkv));
    d.layer = t.layer; d.pos = t.pos; d.tile = (uint16_t)t.tile; d.phase = t.phase;
    d.ph_in0 = t.ph_in0; d.ph_in1 = t.ph_in1; d.w_off = t.w_off; d.w_bytes = t.w_bytes;
  }
  return out;
}

static cp_status alloc_scratch(cp_plan* P) {
  const cp_config& c = P->cfg;
  const int L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, d = c.head_dim;
  const int I = c.intermediate, Pn = c.n_positions, V = c.vocab, R = c.max_rows;
  const int esz = c.dtype == CP_DTYPE_BF16 ? 2 : 4;
  DevPlan& dp = P->dp;
  void* p;
  const size_t e2 = (size_t)esz * 2;  // tagged words: payload + tag per element pair (bf16) or element (fp32)
  // Projection operands (position inputs, residuals, attention and SwiGLU
  // outputs): plain values in the kernels' operand order, whole 16-row tiles,
  // a plane per layer and position, in one region that starts (and every
  // frame ends) filled with the sentinel, all bits set.
  const size_t Rp = (size_t)((R + 15) / 16) * 16;
  const size_t hb = Rp * H * esz, ab = Rp * nq * d * esz, mb = Rp * I * esz, planes = (size_t)L * Pn;
  const size_t opb = Pn * hb + 2 * planes * hb + planes * ab + planes * mb;
  TRY(alloc(P, &p, opb, false, 0xff));
  dp.opbuf = p;
  dp.opbuf_bytes = opb;  // a multiple of 16: Rp is
  dp.xin = p;
  dp.hres = (uint8_t*)dp.xin + Pn * hb;
  dp.hmid = (uint8_t*)dp.hres + planes * hb;
  dp.abuf = (uint8_t*)dp.hmid + planes * hb;
  dp.mbuf = (uint8_t*)dp.abuf + planes * ab;
  TRY(alloc(P, &p, (size_t)2 * R * nq * d * e2, true)); dp.qbuf = p;     // row-major (attention input)
  // QK-norm: behind the K cache (one buffer resource covers both), the raw
  // normed-to-be K of the position in flight, [2 parity][Rmax][nkv][d]
  const size_t kcb = (size_t)L * R * nkv * Pn * d * e2, krb = c.qk_norm ? (size_t)2 * R * nkv * d * e2 : 0;
  TRY(alloc(P, &p, kcb + krb, true)); dp.kc = p;
  dp.kraw = c.qk_norm ? (uint8_t*)p + kcb : nullptr;
  if (c.qk_norm) {
    // per-tile sums of squares of every q and k head, [2 parity][Rmax][nq + nkv][d / 16] words
    TRY(alloc(P, &p, (size_t)2 * R * (nq + nkv) * (d / 16) * 8, true)); dp.qkn = (uint64_t*)p;
  }
  dp.qk_norm = c.qk_norm ? 1 : 0;
  TRY(alloc(P, &p, (size_t)L * R * nkv * Pn * d * e2, true)); dp.vc = p;
  const size_t part_one = (size_t)(H / 16) * 4 * R * 16;  // words per split-K phase buffer
  TRY(alloc(P, &p, part_one * 5 * 8, true)); dp.part = (uint64_t*)p;       // o[2], down[2], in
  dp.part_stride = part_one;
  dp.part_o_off = 0;
  dp.part_d_off = 2 * part_one;
  dp.part_in_off = 4 * part_one;
  TRY(alloc(P, &p, (size_t)R * V * 8, true)); dp.zbuf = (uint64_t*)p;
  TRY(alloc(P, &p, (size_t)R * (V / 16) * 16, true)); dp.cand = (uint64_t*)p;
  TRY(alloc(P, &p, 256 * 4)); dp.state = (uint32_t*)p;
  std::vector<uint32_t> st(256, 0);
  st[0] = 1;  // first frame is epoch 1; zeroed buffers carry tag 0, which no frame expects
  TRY(upload(P, dp.state, st.data(), st.size() * 4));
  const std::vector<DevTask> dev_tasks = to_dev(P->tasks, P->xcd_dealing), dev_phase = to_dev(P->phase_tasks, false);
  TRY(alloc(P, &p, dev_tasks.size() * sizeof(DevTask))); dp.tasks = (const DevTask*)p;
  TRY(upload(P, p, dev_tasks.data(), dev_tasks.size() * sizeof(DevTask)));
  TRY(alloc(P, &p, P->wg_begin.size() * 4)); dp.wg_begin = (const uint32_t*)p;
  TRY(upload(P, p, P->wg_begin.data(), P->wg_begin.size() * 4));
  TRY(alloc(P, &p, dev_phase.size() * sizeof(DevTask))); P->d_phase_tasks = (DevTask*)p;
  TRY(upload(P, p, dev_phase.data(), dev_phase.size() * sizeof(DevTask)));
  if (c.flags & CP_FLAG_TRACE) {
    TRY(alloc(P, &p, P->tasks.size() * kTraceStamps * 8)); dp.trace = (uint64_t*)p;  // zeroed by alloc
    dp.trace_on = 1;
  }
  return CP_OK;
}

// ---------------------------------------------------------------- C ABI

extern "C" {

const char* cp_status_string(cp_status s) {
  switch (s) {
    case CP_OK: return "ok";
    case CP_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CP_ERR_UNSUPPORTED: return "unsupported";
    case CP_ERR_NOT_CORESIDENT: return "persistent grid cannot be co-resident";
    case CP_ERR_OUT_OF_MEMORY: return "out of device memory";
    case CP_ERR_HIP: return "HIP runtime error";
    case CP_ERR_DEVICE_TIMEOUT: return "device-side wait timed out";
  }
  return "unknown status";
}

const char* cp_plan_last_error(const cp_plan* plan) { return plan ? plan->err.c_str() : ""; }
const char* cp_last_create_error(void) { return g_create_err.c_str(); }

cp_status cp_plan_destroy(cp_plan* plan) {
  if (!plan) return CP_OK;
  if (plan->is_static) {
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (plan->device >= 0 && plan->device < 64 && g_static_owner[plan->device] == plan)
      g_static_owner[plan->device] = nullptr;
  }
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(plan->device);
  for (void* p : plan->allocs) (void)hipFree(p);
  (void)hipSetDevice(prev);
  delete plan;
  return CP_OK;
}

static cp_status create_impl(cp_plan* P, const cp_config* cfg, const cp_weights* w, int dev) {
  // (a static plan arrives with is_static and its arena set)
  std::string msg;
  cp_status s = validate(cfg, msg);
  if (s != CP_OK) return fail(P, s, msg);
  P->cfg = *cfg;
  P->device = dev;
  int ndev = 0;
  HIPCHK(P, hipGetDeviceCount(&ndev));
  if (dev < 0 || dev >= ndev) return fail(P, CP_ERR_INVALID_ARGUMENT, "no such device");
  HIPCHK(P, hipSetDevice(dev));
  hipDeviceProp_t prop;
  HIPCHK(P, hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(P, CP_ERR_UNSUPPORTED, std::string("needs gfx950, found ") + prop.gcnArchName);
  P->cu_count = prop.multiProcessorCount;
  if ((size_t)prop.sharedMemPerBlock < (size_t)kLdsBytes)
    return fail(P, CP_ERR_NOT_CORESIDENT, "not enough LDS per workgroup");
  HIPCHK(P, set_kernel_attributes());
  const int bf = cfg->dtype == CP_DTYPE_BF16;
  if (occupancy_per_cu(bf) < 1) return fail(P, CP_ERR_NOT_CORESIDENT, "persistent kernel does not fit one CU");

  DevPlan& dp = P->dp;
  dp.L = cfg->n_layers; dp.H = cfg->hidden; dp.Din = cfg->input_dim; dp.nq = cfg->n_q_heads;
  dp.nkv = cfg->n_kv_heads; dp.d = cfg->head_dim; dp.I = cfg->intermediate; dp.P = cfg->n_positions;
  dp.V = cfg->vocab; dp.Rmax = cfg->max_rows; dp.gq = dp.nq / dp.nkv; dp.n_head_tiles = dp.V / 16;
  dp.bf16 = bf; dp.eps = cfg->rms_eps; dp.attn_scale = (float)(1.0 / std::sqrt((double)cfg->head_dim));
  dp.spin_limit = kDefaultSpinLimit;
  dp.n_wg = P->cu_count;
  if (P->is_static) {
    void* base = nullptr;
    HIPCHK(P, static_scratch(dev, &base, &P->st_cap));
    P->st_base = (uint8_t*)base;
    if ((size_t)dp.n_wg * 4 > P->st_cap) return fail(P, CP_ERR_OUT_OF_MEMORY, "static scratch too small");
  }
  // (a static plan records the dealing into its scratch array, which is
  // zeroed again when its buffers are carved)
  HIPCHK(P, check_xcd_dealing(dp.n_wg, P->xcd_dealing, P->is_static ? (uint32_t*)P->st_base : nullptr));
  TRY(build_schedule(P));
  dp.n_tasks = (int)P->tasks.size();
  if (P->is_static) {
    // the scratch this plan needs, before anything is written
    if ((int64_t)P->arena_cap < const_bytes(*cfg))
      return fail(P, CP_ERR_INVALID_ARGUMENT,
                  "weight arena of " + std::to_string(P->arena_cap) + " bytes; the plan's constants need " +
                      std::to_string(const_bytes(*cfg)) + " (cp_plan_info.const_bytes)");
    P->measuring = true;
    TRY(alloc_scratch(P));
    P->measuring = false;
    if (P->st_used > P->st_cap)
      return fail(P, CP_ERR_OUT_OF_MEMORY,
                  "the plan's scratch needs " + std::to_string(P->st_used) + " bytes, more than the " +
                      std::to_string(P->st_cap) + " bytes the library holds per device for static plans; "
                      "use cp_plan_create, or fewer rows or layers");
    P->st_used = 0;
    P->scratch_bytes = 0;
    dp.n_clear = 0;
  }
  TRY(pack_weights(P, w));
  TRY(check_schedule(P));
  dp.tasks_in_lds = (int64_t)P->max_tasks_wg * (int64_t)sizeof(DevTask) <= kTaskLds;
  dp.local_ok = (cfg->flags & CP_FLAG_NO_LOCAL) ? 0 : 1;
  TRY(alloc_scratch(P));
  HIPCHK(P, hipDeviceSynchronize());
  return CP_OK;
}

cp_status cp_plan_create(const cp_config* cfg, const cp_weights* w, int hip_device, cp_plan** out) {
  if (!out) return CP_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  g_create_err.clear();
  if (!cfg || !w) {
    g_create_err = "NULL config or weights";
    return CP_ERR_INVALID_ARGUMENT;
  }
  cp_plan* P = new cp_plan();
  int prev = 0;
  (void)hipGetDevice(&prev);
  cp_status s = create_impl(P, cfg, w, hip_device);
  (void)hipSetDevice(prev);
  if (s != CP_OK) {
    g_create_err = P->err;
    cp_plan_destroy(P);
    return s;
  }
  *out = P;
  return CP_OK;
}

cp_status cp_plan_create_static(const cp_config* cfg, const cp_weights* w, int hip_device, void* weight_arena,
                                uint64_t arena_bytes, cp_plan** out) {
  if (!out) return CP_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  g_create_err.clear();
  if (!cfg || !w || !weight_arena) {
    g_create_err = "NULL config, weights or weight arena";
    return CP_ERR_INVALID_ARGUMENT;
  }
  if (hip_device < 0 || hip_device >= 64) {
    g_create_err = "no such device";
    return CP_ERR_INVALID_ARGUMENT;
  }
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (g_static_owner[hip_device]) {
    g_create_err = "a static plan already lives on this device (they share its scratch array): destroy it first";
    return CP_ERR_INVALID_ARGUMENT;
  }
  cp_plan* P = new cp_plan();
  P->is_static = true;
  P->arena = (uint8_t*)weight_arena;
  P->arena_cap = (size_t)arena_bytes;
  int prev = 0;
  (void)hipGetDevice(&prev);
  cp_status s = create_impl(P, cfg, w, hip_device);
  (void)hipSetDevice(prev);
  if (s != CP_OK) {
    g_create_err = P->err;
    P->is_static = false;  // not the owner: destroy must not touch the slot
    cp_plan_destroy(P);
    return s;
  }
  g_static_owner[hip_device] = P;
  *out = P;
  return CP_OK;
}

cp_status cp_schedule_check(const cp_config* cfg, int cu_count, cp_plan_info* info) {
  g_create_err.clear();
  if (!cfg || !info || cu_count < 1) {
    g_create_err = "NULL argument or cu_count < 1";
    return CP_ERR_INVALID_ARGUMENT;
  }
  cp_plan P;
  std::string msg;
  cp_status s = validate(cfg, msg);
  if (s == CP_OK) {
    P.cfg = *cfg;
    P.cu_count = cu_count;
    P.packed_bytes = INT64_MAX;  // no weights: tile bounds are not checked here
    s = build_schedule(&P);
    if (s == CP_OK) s = check_schedule(&P);
    msg = P.err;
  }
  if (s != CP_OK) {
    g_create_err = msg;
    return s;
  }
  std::memset(info, 0, sizeof *info);
  info->n_phases = P.n_phases;
  info->n_tasks = (int32_t)P.tasks.size();
  info->n_workgroups = cu_count;
  info->max_tasks_per_workgroup = P.max_tasks_wg;
  info->const_bytes = const_bytes(*cfg);
  return CP_OK;
}

cp_status cp_plan_query(const cp_plan* P, cp_plan_info* info) {
  if (!P || !info) return CP_ERR_INVALID_ARGUMENT;
  info->n_phases = P->n_phases;
  info->n_tasks = (int32_t)P->tasks.size();
  info->n_workgroups = P->cu_count;
  info->lds_bytes = kLdsBytes;
  info->weight_bytes_per_frame = P->weight_bytes_frame;
  info->packed_weight_bytes = P->packed_bytes;
  info->scratch_bytes = P->scratch_bytes;
  info->trace_words = (P->cfg.flags & CP_FLAG_TRACE) ? (int64_t)P->tasks.size() * kTraceStamps : 0;
  info->cu_count = P->cu_count;
  info->max_tasks_per_workgroup = P->max_tasks_wg;
  info->const_bytes = const_bytes(P->cfg);
  return CP_OK;
}

cp_status cp_frame_run(cp_plan* P, const cp_frame_io* io, void* stream) {
  if (!P || !io) return CP_ERR_INVALID_ARGUMENT;
  const cp_config& c = P->cfg;
  if (io->rows < 1 || io->rows > c.max_rows) return fail(P, CP_ERR_INVALID_ARGUMENT, "rows out of range");
  if (!io->hidden_in || !io->code0 || !io->codes || !io->embsum)
    return fail(P, CP_ERR_INVALID_ARGUMENT, "hidden_in, code0, codes and embsum are required");
  const int nsamp = (io->temperature != nullptr) + (io->top_k != nullptr) + (io->top_p != nullptr) +
                    (io->seed != nullptr) + (io->offset != nullptr);
  if (nsamp != 0 && nsamp != 5) return fail(P, CP_ERR_INVALID_ARGUMENT, "sampling arrays must be all set or all NULL");
  if (io->trace && !(c.flags & CP_FLAG_TRACE)) return fail(P, CP_ERR_INVALID_ARGUMENT, "trace needs CP_FLAG_TRACE");
  // rows below the crossover run the per-phase executor (same buffers, same task bodies)
  const bool persistent = c.exec == CP_EXEC_PERSISTENT && io->rows >= P->crossover;
  if (io->trace && !persistent) return fail(P, CP_ERR_UNSUPPORTED, "trace needs the persistent executor");
  DevFrame fr{};
  fr.rows = io->rows;
  fr.sampled = nsamp == 5;
  fr.defer_clear = (io->k_cache || io->v_cache) ? 1 : 0;
  fr.hidden_in = io->hidden_in;
  fr.code0 = io->code0;
  fr.temperature = io->temperature;
  fr.top_k = io->top_k;
  fr.top_p = io->top_p;
  fr.seed = io->seed;
  fr.offset = io->offset;
  fr.codes = io->codes;
  fr.embsum = io->embsum;
  fr.logits = io->logits;
  fr.trace = io->trace;
  hipStream_t s = (hipStream_t)stream;
  int prev = 0;
  (void)hipGetDevice(&prev);
  if (prev != P->device) HIPCHK(P, hipSetDevice(P->device));
  hipError_t e = hipSuccess;
  if (persistent) {
    e = launch_persistent(P->dp, fr, s);
  } else {
    for (int ph = 0; ph < P->n_phases && e == hipSuccess; ++ph) {
      const uint32_t b = P->phase_begin[ph], n = P->phase_begin[ph + 1] - b;
      e = launch_phase(P->dp, fr, P->d_phase_tasks + b, (int)n, s);
    }
    if (e == hipSuccess) e = launch_bump_epoch(P->dp, fr.defer_clear, s);
  }
  if (e == hipSuccess && (io->k_cache || io->v_cache)) {
    const int esz = c.dtype == CP_DTYPE_BF16 ? 2 : 4;
    const uint32_t wpr = (uint32_t)((size_t)c.n_kv_heads * c.n_positions * c.head_dim * esz / 4);
    if (io->k_cache) e = launch_unpack_kv(P->dp.kc, io->k_cache, wpr, io->rows, c.max_rows, c.n_layers, s);
    if (e == hipSuccess && io->v_cache) e = launch_unpack_kv(P->dp.vc, io->v_cache, wpr, io->rows, c.max_rows, c.n_layers, s);
    if (e == hipSuccess) e = launch_clear_pending(P->dp, s);
  }
  if (e == hipSuccess && io->trace)
    e = hipMemcpyAsync(io->trace, P->dp.trace, P->tasks.size() * kTraceStamps * 8, hipMemcpyDeviceToDevice, s);
  if (prev != P->device) (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail(P, CP_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return CP_OK;
}

static void fill_task_table(const cp_plan* P, int32_t* out) {
  for (size_t w = 0; w + 1 < P->wg_begin.size(); ++w)
    for (uint32_t i = P->wg_begin[w]; i < P->wg_begin[w + 1]; ++i) {
      const Task& t = P->tasks[i];
      int32_t* o = out + (size_t)i * 8;
      o[0] = (int32_t)t.phase; o[1] = t.type; o[2] = t.layer; o[3] = t.pos;
      o[4] = (int32_t)t.tile; o[5] = t.split; o[6] = (int32_t)w; o[7] = (int32_t)(i - P->wg_begin[w]);
    }
}

cp_status cp_plan_task_table(const cp_plan* P, int32_t* out, int64_t n_tasks) {
  if (!P || !out || n_tasks != (int64_t)P->tasks.size()) return CP_ERR_INVALID_ARGUMENT;
  fill_task_table(P, out);
  return CP_OK;
}

cp_status cp_schedule_task_table(const cp_config* cfg, int cu_count, int32_t* out, int64_t n_tasks) {
  g_create_err.clear();
  if (!cfg || !out || cu_count < 1) {
    g_create_err = "NULL argument or cu_count < 1";
    return CP_ERR_INVALID_ARGUMENT;
  }
  cp_plan P;
  std::string msg;
  cp_status s = validate(cfg, msg);
  if (s == CP_OK) {
    P.cfg = *cfg;
    P.cu_count = cu_count;
    P.packed_bytes = INT64_MAX;
    s = build_schedule(&P);
    if (s == CP_OK) s = check_schedule(&P);
    msg = P.err;
  }
  if (s != CP_OK) {
    g_create_err = msg;
    return s;
  }
  if (n_tasks != (int64_t)P.tasks.size()) {
    g_create_err = "n_tasks does not match the schedule";
    return CP_ERR_INVALID_ARGUMENT;
  }
  fill_task_table(&P, out);
  return CP_OK;
}

cp_status cp_plan_set_epoch(cp_plan* P, uint32_t epoch) {
  if (!P) return CP_ERR_INVALID_ARGUMENT;
  if (epoch < 1 || epoch >= kEpochWrap) return fail(P, CP_ERR_INVALID_ARGUMENT, "epoch out of range");
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(P->device);
  // [0] epoch; [128], [160] the persistent executor's frame-end arrival
  // counters, both zero before a frame whatever its epoch's parity
  const uint32_t st[2] = {epoch, 0u};
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(P->dp.state, &st[0], 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(P->dp.state + 128, &st[1], 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(P->dp.state + 160, &st[1], 4, hipMemcpyHostToDevice);
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail(P, CP_ERR_HIP, std::string("set epoch: ") + hipGetErrorString(e));
  return CP_OK;
}

cp_status cp_plan_set_crossover(cp_plan* P, int rows) {
  if (!P) return CP_ERR_INVALID_ARGUMENT;
  if (rows < 0 || rows > P->cfg.max_rows + 1) return fail(P, CP_ERR_INVALID_ARGUMENT, "crossover rows out of range");
  if (rows > 0 && P->cfg.exec != CP_EXEC_PERSISTENT) return fail(P, CP_ERR_UNSUPPORTED, "crossover needs a persistent plan");
  // per-phase launches hold a phase's split-K partners and owner at once
  for (size_t ph = 0; rows > 0 && ph + 1 < P->phase_begin.size(); ++ph) {
    const Task& f = P->phase_tasks[P->phase_begin[ph]];
    if (f.nsplit > 1 && (int)(P->phase_begin[ph + 1] - P->phase_begin[ph]) > P->cu_count)
      return fail(P, CP_ERR_UNSUPPORTED, "schedule: split phase larger than the grid");
  }
  P->crossover = rows;
  return CP_OK;
}

cp_status cp_plan_set_spin_limit(cp_plan* P, uint32_t polls) {
  if (!P) return CP_ERR_INVALID_ARGUMENT;
  P->dp.spin_limit = polls ? polls : kDefaultSpinLimit;
  return CP_OK;
}

cp_status cp_plan_device_status(cp_plan* P) {
  if (!P) return CP_ERR_INVALID_ARGUMENT;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(P->device);
  uint32_t st[128];
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(st, P->dp.state, sizeof st, hipMemcpyDeviceToHost);
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail(P, CP_ERR_HIP, std::string("device status: ") + hipGetErrorString(e));
  if (st[64]) return fail(P, CP_ERR_DEVICE_TIMEOUT, "a device-side wait gave up");
  return CP_OK;
}

cp_status cp_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return CP_ERR_INVALID_ARGUMENT;
  return launch_stream_read(buf, bytes, sink, (hipStream_t)stream) == hipSuccess ? CP_OK : CP_ERR_HIP;
}

cp_status cp_chain_run(uint32_t* slots, int n_workgroups, int n_phases, uint32_t tag_base, int xcd_local, int variant,
                       uint32_t* error_word, void* stream) {
  if (!slots || !error_word || n_workgroups < 1 || n_workgroups > 256 || n_phases < 1 ||
      (xcd_local && n_workgroups % 8) || (uint64_t)tag_base + (uint64_t)n_phases > 0xffffffffull || variant < 0 ||
      variant > 5 || (variant >= 1 && variant <= 3 && !xcd_local) ||
      (variant == 5 && (xcd_local || ((uint64_t)tag_base + (uint64_t)n_phases) * (uint64_t)n_workgroups > 0xffffffffull)))
    return CP_ERR_INVALID_ARGUMENT;
  return launch_chain(slots, n_workgroups, n_phases, tag_base, xcd_local, variant, error_word, (hipStream_t)stream) ==
                 hipSuccess
             ? CP_OK
             : CP_ERR_HIP;
}

}  // extern "C"
