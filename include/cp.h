/*
 * cp.h -- C ABI of the MI355X depth-loop library (libcpms.so).
 *
 * The library runs the depth loop of a codec-TTS code predictor: per frame an
 * input projection, then n_positions depth positions, each walked through every
 * decoder layer (qkv, attention, o, gate/up, down), a code head and a draw at
 * every position after the first, and n_positions code embeddings whose sum is
 * returned with the codes.  This is the frame of the mstar pull request
 * "Qwen3-TTS: Run the 1.7B Depth Loop as One Persistent Kernel on Hopper"
 * (#1183), section "How it works" (first bullet: the phases of a frame); the
 * outputs are the ones its section "Testing" compares (codes, embedding sums,
 * KV cache, logits).
 *
 * Two executors compute bitwise-identical frames from the same task bodies:
 *   CP_EXEC_PERSISTENT  one launch of one workgroup per compute unit that walks
 *                       a static per-workgroup task list (section "How it
 *                       works", first and second bullets).  Workgroups hand
 *                       data to each other through device memory, where the
 *                       data is its own ready signal.  The activations a
 *                       projection streams (position inputs, residuals,
 *                       attention and SwiGLU outputs) live in buffers with a
 *                       plane per layer and position, written once per
 *                       frame; until then an element holds a sentinel (all
 *                       bits set, a NaN no producer stores), and the reader
 *                       reloads until none is left.  After the frame every
 *                       workgroup meets at one counter and refills its share
 *                       of those buffers with the sentinel.  Every other value
 *                       (q, K/V, split-K partials, logits) is stored
 *                       next to a 32-bit tag (epoch * 1024 + the writer's
 *                       phase), and the reader reloads the words until every
 *                       tag is the one it expects.  No fence is on the path.
 *   CP_EXEC_PER_PHASE   one launch per phase (the unfused comparison, the
 *                       "loop" of section "Where the depth loop's time goes").
 *
 * Conventions for every call:
 *   - every call returns a cp_status; no exception or abort crosses the ABI;
 *   - "device" pointers are HIP device allocations on the plan's device;
 *     "host" pointers are ordinary process memory;
 *   - sizes are element counts unless a name says bytes;
 *   - matrices are row-major [out][in], the layout of nn.Linear;
 *   - the activation type of a plan (dtype) is also the storage type of its
 *     weights, input hidden and KV outputs: IEEE fp32, or bf16 as 16-bit words;
 *   - a call refused on the host (CP_ERR_INVALID_ARGUMENT, CP_ERR_UNSUPPORTED)
 *     enqueues nothing, so the caller can run its own per-launch loop instead
 *     (section "How it works", opening paragraphs: a step the kernel cannot
 *     take runs the loop, and startup logs why).
 */
#ifndef CP_H
#define CP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CP_ABI_VERSION 3

typedef enum {
  CP_OK = 0,
  CP_ERR_INVALID_ARGUMENT = 1, /* NULL where a pointer is required, rows out of range, ... */
  CP_ERR_UNSUPPORTED = 2,      /* shape, dtype or setting the library does not run */
  CP_ERR_NOT_CORESIDENT = 3,   /* the persistent grid cannot be resident all at once */
  CP_ERR_OUT_OF_MEMORY = 4,
  CP_ERR_HIP = 5,              /* a HIP runtime call failed; see cp_plan_last_error */
  CP_ERR_DEVICE_TIMEOUT = 6    /* a device-side wait gave up (reported by cp_plan_device_status) */
} cp_status;

typedef enum { CP_DTYPE_F32 = 0, CP_DTYPE_BF16 = 1 } cp_dtype;
typedef enum { CP_EXEC_PERSISTENT = 0, CP_EXEC_PER_PHASE = 1 } cp_exec;

/* Plan flags. */
#define CP_FLAG_TRACE 0x1u /* record eight timestamps per task (persistent executor; see cp_frame_io.trace) */
/* Every hand-off writes through to memory: no split-K partials or q/k/v kept
 * in one XCD's L2 for readers on that XCD.  A plan also runs this way when,
 * at its creation, the device did not deal workgroup i to XCD (i + r) mod 8
 * for one rotation r (the readers of an XCD-local hand-off must share the
 * writer's XCD).  For measurement, and for a device whose dealing could
 * change after that check. */
#define CP_FLAG_NO_LOCAL 0x4u
/* Two (or more) row groups in flight, the second item of section "What's
 * left in the frame, open": every projection task of a frame of more than 32
 * rows is split into tasks of 32 rows that one workgroup runs back to back
 * on the same weight tile, so that while one group's operands are in flight
 * the workgroup computes the other's.  Not bit for bit the default plan's
 * results: the waves of a 32-row task split K and add their parts in another
 * order (within the same tolerances against the reference).  Measured slower
 * than the default on MI355X (the groups never drift apart, and every phase
 * pays two task overheads).  Persistent executor only (CP_ERR_UNSUPPORTED
 * with CP_EXEC_PER_PHASE). */
#define CP_FLAG_ROW_GROUPS 0x8u

/* Shapes and settings of a plan.  Supported (else CP_ERR_UNSUPPORTED):
 * head_dim 64 or 128; n_q_heads a multiple of 4 and of n_kv_heads; hidden a
 * multiple of 256 up to 1024; input_dim and intermediate multiples of 256;
 * vocab 256, 512, 1024, 2048 or 4096; 2 <= n_positions <= 16;
 * 1 <= max_rows <= 128 (the pages' frame stops at 64 rows, section "How it
 * works", opening paragraphs, and lists the 128-row frame under "What's left
 * in the frame, open"; here a projection task of a frame over 64 rows runs
 * its two groups of 64 rows one after the other on the weight tile it holds
 * in LDS). */
typedef struct {
  int32_t abi_version;  /* CP_ABI_VERSION */
  int32_t n_layers;
  int32_t hidden;
  int32_t input_dim;    /* width of the input hidden that the input projection maps to hidden */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate; /* SwiGLU width */
  int32_t n_positions;  /* depth positions per frame; n_positions - 1 heads and draws */
  int32_t vocab;        /* codes per codebook */
  int32_t max_rows;     /* rows (independent requests) a frame may carry */
  int32_t dtype;        /* cp_dtype */
  float rms_eps;        /* RMSNorm epsilon, e.g. 1e-6 */
  float rope_theta;     /* RoPE base, e.g. 1e4 */
  int32_t exec;         /* cp_exec */
  uint32_t flags;       /* CP_FLAG_* */
  int32_t qk_norm;      /* nonzero: the Qwen3-style variant, an RMSNorm of every q and k head (over
                           head_dim, gains cp_weights.q_norm / k_norm, the same epsilon) between
                           the qkv projection and RoPE; the handbook page "The gaps between kernels:
                           PDL and megakernels" lists it fused with RoPE (section on fusing kernels) */
} cp_config;

/* Weights of the code predictor (section "Cost": hidden 1024, 16 q and 8 kv
 * heads of 128, intermediate 3072, 5 layers for the 1.7B model; other shapes
 * within the limits above are accepted).  Read only inside cp_plan_create:
 * the plan copies and repacks them, so the caller may free them afterwards.  Single matrices are device
 * pointers; per-layer, per-table and per-head lists are HOST arrays of device
 * pointers. */
typedef struct {
  const void* w_in;               /* [hidden][input_dim] input projection */
  const void* const* embed;       /* n_positions x [vocab][hidden]; table j embeds code j */
  const void* const* attn_norm;   /* n_layers x [hidden] */
  const void* const* w_qkv;       /* n_layers x [(nq + 2 nkv) head_dim][hidden]; rows q heads | k heads | v heads */
  const void* const* w_o;         /* n_layers x [hidden][nq head_dim] */
  const void* const* mlp_norm;    /* n_layers x [hidden] */
  const void* const* w_gate;      /* n_layers x [intermediate][hidden] */
  const void* const* w_up;        /* n_layers x [intermediate][hidden] */
  const void* const* w_down;      /* n_layers x [hidden][intermediate] */
  const void* final_norm;         /* [hidden] */
  const void* const* w_head;      /* (n_positions - 1) x [vocab][hidden]; entry j-1 is head j */
  const void* const* q_norm;      /* n_layers x [head_dim] (qk_norm only, else ignored) */
  const void* const* k_norm;      /* n_layers x [head_dim] (qk_norm only, else ignored) */
} cp_weights;

/* One frame's inputs and outputs (section "Testing": codes and embedding
 * sums, the KV cache and logits are what a frame is checked on): all device
 * pointers, borrowed until the frame's stream work completes. */
typedef struct {
  int32_t rows;              /* 1 .. max_rows */
  const void* hidden_in;     /* [rows][input_dim], dtype */
  const int32_t* code0;      /* [rows] code 0 (from outside the loop), each in [0, vocab) */
  /* Sampling, [rows] each (section "How it works", sampler bullet: a kernel
   * that draws in place reads each row's temperature, top-k, top-p, seed and
   * offset, and moves the offsets as that many single draws would).  All
   * five NULL: greedy for every row (the lowest index of the largest logit).  Some but not all NULL:
   * CP_ERR_INVALID_ARGUMENT.  Draw j of a row (j = 1 .. n_positions-1), as
   * the sampler is defined: y = logits / temperature; keep the top_k largest
   * y (ties to the lower index); softmax over them; keep the shortest prefix
   * in rank order whose probability mass reaches top_p (the crossing token
   * included); the code is the kept i with the largest y_i - log(-log u_i),
   * u_i = (2m + 1) / 2^24 with m the top 23 bits of word 0 of
   * Philox4x64-10(counter = (offset + j - 1, i, 0, 0), key = (seed, 0)).
   * Per-row values never fail on the device: temperature <= 0 is greedy;
   * top_k <= 0 or >= vocab is no top-k cut; top_p >= 1 is no top-p cut,
   * top_p <= 0 keeps the best token only. */
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const uint64_t* seed;
  uint64_t* offset;          /* in/out: advanced by n_positions - 1 in place */
  int32_t* codes;            /* out [rows][n_positions - 1], codes 1 .. n_positions-1 */
  float* embsum;             /* out [rows][hidden]: fp32 sum of the n_positions code embeddings */
  float* logits;             /* optional out [rows][n_positions - 1][vocab] (fp32) */
  void* k_cache;             /* optional out [n_layers][rows][n_kv_heads][n_positions][head_dim], dtype, post-RoPE */
  void* v_cache;             /* optional out, same layout */
  uint64_t* trace;           /* optional out, cp_plan_info.trace_words words (needs CP_FLAG_TRACE and the
                                persistent executor): per task, in the order of cp_plan_task_table, eight
                                timestamps of the device's 100 MHz constant clock, written by the task's
                                workgroup:
                                  0 task start, 1 dispatched (next task's record read),
                                  2 dependencies met (projections: first operand group and
                                    weight tile in place; attention: Q, K, V of its first pair; draw: the
                                    head's logits or candidates),
                                  3 first operand group consumed, 4 K loop done (projections),
                                  5 outputs issued, 6 end-of-task barrier passed, 7 next tile copy issued.
                                Stamps a task kind does not pass through (2-4 for the code-0 embedding,
                                3-4 for attention and draws) hold no value of the frame.  The timestamps
                                follow the eight-per-task split of section "Where the depth loop's time
                                goes" ("Inside a task"). */
} cp_frame_io;

typedef struct {
  int32_t n_phases;          /* dependent phases of one frame */
  int32_t n_tasks;           /* tasks over all workgroups */
  int32_t n_workgroups;      /* persistent grid size (one per compute unit) */
  int32_t lds_bytes;         /* dynamic LDS per workgroup */
  int64_t weight_bytes_per_frame; /* algorithmic weight bytes one frame reads */
  int64_t packed_weight_bytes;    /* device bytes of the repacked weights */
  int64_t scratch_bytes;          /* device bytes of plan-owned scratch */
  int64_t trace_words;            /* uint64 words a traced frame writes */
  int32_t cu_count;
  int32_t max_tasks_per_workgroup;
  int64_t const_bytes;            /* device bytes of the plan's constants (repacked weights, embedding tables,
                                     RoPE table, each rounded up to 256): the weight arena cp_plan_create_static
                                     needs; cp_schedule_check reports it too */
} cp_plan_info;

typedef struct cp_plan cp_plan; /* opaque, owned by the library */

/* Validates cfg, checks that the persistent grid is co-resident on
 * hip_device (CP_ERR_NOT_CORESIDENT otherwise: the workgroups wait on each
 * other, so all of them must be resident at once -- section "How it works",
 * last bullet), repacks the weights, builds the static per-workgroup task
 * lists (section "How it works", first bullet) and allocates all scratch.
 * On success *out owns the plan; on failure *out is NULL and
 * cp_last_create_error() says why.  Allocates device memory (hipMalloc);
 * synchronises the device. */
cp_status cp_plan_create(const cp_config* cfg, const cp_weights* w, int hip_device, cp_plan** out);

/* For callers that cannot allocate device memory (code that forbids
 * hipMalloc: serving loops or harnesses that own the device's memory).  The
 * same plan as cp_plan_create, with no device allocation: the repacked
 * weights and tables are written into weight_arena (caller-owned device
 * memory on hip_device of at least cp_plan_info.const_bytes bytes, as
 * cp_schedule_check reports for cfg, else CP_ERR_INVALID_ARGUMENT; it must
 * outlive the plan), and every scratch buffer of the plan is carved from an
 * array of 160 MiB the library holds on each device it runs on until the
 * process ends (a plan that needs more -- the 5-layer bf16 loop at 64 rows
 * needs about 130 MiB, the 10-layer one at 64 rows more -- is refused with
 * CP_ERR_OUT_OF_MEMORY and a message giving both sizes).  The plan's part of
 * the array is initialised with a kernel at creation.  All static plans of a device share that
 * one array, so only one may live per device at a time: a second
 * cp_plan_create_static on a device whose static plan has not been destroyed
 * is refused (CP_ERR_INVALID_ARGUMENT).  Its frames behave as those of
 * cp_plan_create's plans (same kernels, same results); cp_plan_destroy frees
 * only the host object.  Synchronises the device. */
cp_status cp_plan_create_static(const cp_config* cfg, const cp_weights* w, int hip_device, void* weight_arena,
                                uint64_t arena_bytes, cp_plan** out);

/* Enqueues one frame on hip_stream (a hipStream_t; NULL = default stream) and
 * returns without waiting.  Checks io on the host first and enqueues nothing
 * on an error (CP_ERR_INVALID_ARGUMENT: rows outside 1..max_rows, a required
 * pointer NULL, some but not all sampling arrays, a trace buffer without
 * CP_FLAG_TRACE).  The call allocates nothing and never synchronises, so it
 * may be captured into a HIP graph and replayed (section "Testing": a
 * captured frame replays what it ran).  Frames of one plan must be
 * stream-ordered: the persistent executor holds every compute unit while it
 * runs (section "Cost": the frame holds every SM), and two of its frames in
 * flight at once on one device could wait on each other; a device-side wait
 * that gives up is reported by cp_plan_device_status. */
cp_status cp_frame_run(cp_plan* plan, const cp_frame_io* io, void* hip_stream);

/* The static task list as a table (host memory `out`, 8 int32 per task), for
 * decoding traces and for tests of the schedule.  Writes, in trace order: phase index, task type (1 input
 * projection, 2 code-0 embedding, 3 qkv, 4 attention, 5 o, 6 gate/up, 7 down,
 * 8 head, 9 draw), layer, position, tile, split-K index, workgroup, index in
 * the workgroup's list.  n_tasks must equal cp_plan_info.n_tasks. */
cp_status cp_plan_task_table(const cp_plan* plan, int32_t* out, int64_t n_tasks);

/* Frees everything the plan owns (device memory and the host object).  NULL
 * is accepted.  The plan's frames must have completed. */
cp_status cp_plan_destroy(cp_plan* plan);

/* Fills *info (host memory) with the plan's sizes; touches no device. */
cp_status cp_plan_query(const cp_plan* plan, cp_plan_info* info);

/* Synchronises the plan's device and reports CP_ERR_DEVICE_TIMEOUT if a
 * device-side wait gave up since the plan was created, else CP_OK.  Every
 * wait is bounded (a poll count, see cp_plan_set_spin_limit), so a broken
 * schedule or two frames waiting on each other end the kernel with this
 * error instead of hanging the device (handbook chapter "The gaps between
 * kernels: PDL and megakernels", section "Megakernels": deadlock is the
 * price of cross-block waits).  The error stays set for the plan's life. */
cp_status cp_plan_device_status(cp_plan* plan);

/* Frame epochs.  Every tagged word one workgroup hands to another carries
 * the epoch of the frame that wrote it, so a reader can tell this frame's
 * data from anything older.  Epochs count 1, 2, ... per frame (cp_frame_run) and wrap
 * after 4194302 frames: the frame that reaches the limit also clears every
 * tagged buffer, and the next frame is epoch 1 again.  cp_plan_set_epoch makes
 * the plan's next frame run as `epoch` (1 <= epoch <= 4194302), so that the
 * wrap can be exercised; it synchronises the device and returns
 * CP_ERR_INVALID_ARGUMENT for an epoch outside that range. */
cp_status cp_plan_set_epoch(cp_plan* plan, uint32_t epoch);

/* Bounds every device-side wait of the plan's later frames to `polls`
 * reloads of stale data (0 restores the default of 4194304, several seconds
 * of polling).  A wait that runs out raises the plan's error word; every
 * later wait of that frame then gives up at once and the kernel ends
 * normally, with CP_ERR_DEVICE_TIMEOUT from cp_plan_device_status and the
 * frame's outputs undefined.  For tests of the time-out path: a small bound
 * forces it without any wait having to hang.  Touches no device. */
cp_status cp_plan_set_spin_limit(cp_plan* plan, uint32_t polls);

/* Row-count crossover dispatch (mstar pull request #1183, section "Cost": the
 * frame costs about the same at any row count and lost to the unfused loop
 * at 1 row on H200, so small steps should run the loop once the crossover is
 * measured).  Frames of a persistent plan with fewer than `rows` rows then
 * run the per-phase executor on the same buffers and task bodies (results
 * bit for bit as the persistent executor's); 0 (the default) keeps every
 * frame persistent.  On MI355X the persistent frame is measured faster at
 * every row count from 1 to 64, so the default stays 0.  CP_ERR_INVALID_ARGUMENT
 * for rows outside 0 .. max_rows + 1; CP_ERR_UNSUPPORTED for a per-phase
 * plan or a schedule whose split-K phases need more workgroups than the
 * device holds at once.  A traced frame (cp_frame_io.trace) below the
 * crossover is refused.  Touches no device. */
cp_status cp_plan_set_crossover(cp_plan* plan, int rows);

const char* cp_status_string(cp_status s);

/* Text of the last error recorded on the plan ("" if none). */
const char* cp_plan_last_error(const cp_plan* plan);

/* Text of the last error of a cp_plan_create or cp_schedule_check call that
 * failed (per calling thread). */
const char* cp_last_create_error(void);

/* Builds the per-workgroup task lists cfg would get on a device of cu_count
 * compute units and checks their invariants, touching no device (section
 * "Testing": the task lists are checked on the host): every task waits only
 * on dependency groups (the outputs of one phase, or of one kv head's tiles)
 * that earlier phases complete; every group is completed exactly once per
 * frame by the tasks that make it; every workgroup's list is in phase
 * order.  On success fills n_phases, n_tasks, n_workgroups and
 * max_tasks_per_workgroup of info (other fields zero).  For tests and
 * planning tools; cp_plan_create runs the same checks. */
cp_status cp_schedule_check(const cp_config* cfg, int cu_count, cp_plan_info* info);

/* The task table of the schedule cp_schedule_check builds for cfg and
 * cu_count, in cp_plan_task_table's layout ([n_tasks][8] int32: phase, type,
 * layer, pos, tile, split, workgroup, index in the workgroup's list), touching
 * no device (section "Testing": task lists are inspected on the host).
 * n_tasks must equal the count cp_schedule_check reports, else
 * CP_ERR_INVALID_ARGUMENT; other errors as cp_schedule_check.  For tests of
 * the placement and for planning tools. */
cp_status cp_schedule_task_table(const cp_config* cfg, int cu_count, int32_t* out, int64_t n_tasks);

/* ---------------------------------------------------------------- measurement
 * Two floors the pull request prices a frame against (section "Where the
 * depth loop's time goes"): the weight-read floor (bullet "The floor") and the
 * fixed latency of each dependent phase (bullet "Phases"). */

/* Enqueues one read of the device buffer [buf, buf + bytes) with 16-byte
 * loads and nothing else (bytes a positive multiple of 16, else
 * CP_ERR_INVALID_ARGUMENT).  bytes divided by the launch's time is the
 * streaming-read rate of a working set of that size.  sink: one device uint32
 * the kernel may write (to keep its loads).  Allocates nothing; does not
 * synchronise. */
cp_status cp_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* hip_stream);

/* Enqueues a chain of n_phases phases with no work in them on n_workgroups
 * one-wave workgroups (1..256): in phase k every workgroup stores the tag
 * tag_base + k + 1 into its slot and waits until the slots of the workgroups
 * it depends on carry it -- all of them, or with xcd_local the ones whose
 * index is congruent to its own modulo 8 (the workgroups the persistent
 * executor places on one XCD; n_workgroups then a multiple of 8).  The time
 * of the launch divided by n_phases is the per-phase cost of a tagged-word
 * hand-off.  variant picks the stores' and loads' cache policy:
 *   0  agent-coherent stores and loads (the executor's cross-XCD hand-off);
 *   1  plain stores, agent-coherent loads (its XCD-local hand-off);
 *   2  plain stores, workgroup-coherent loads;
 *   3  plain stores, system-coherent loads;
 *   4  system-coherent stores and loads;
 *   5  the hand-off through counters in global memory of [PR] "How it works"
 *      for comparison: each workgroup stores its word, takes a release fence
 *      and adds one to a counter; the others poll the counter, take an
 *      acquire fence and read the words (all-to-all only).
 * variants 1-3 need xcd_local (plain stores stay in the writer's XCD);
 * variant 5 refuses it.
 * slots: device memory of 2 * n_workgroups * 16 bytes (variant 5: 16 more,
 * the counter), zero before the first launch; tags must grow from launch to
 * launch (tag_base of the next launch >= this tag_base + n_phases, at most
 * 2^32 - 1 in all; variant 5: exactly this tag_base + n_phases, the first
 * launch's 0, and tag_base + n_phases at most 2^32 / n_workgroups).  error_word: a
 * device uint32 set to 1 if a wait gave up (every wait is bounded, about
 * 65536 polls).  Allocates nothing; does not synchronise. */
cp_status cp_chain_run(uint32_t* slots, int n_workgroups, int n_phases, uint32_t tag_base, int xcd_local, int variant,
                       uint32_t* error_word, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
