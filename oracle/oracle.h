/*
 * CPU oracle of the codec-TTS depth loop -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package's smoke check and the CPU-baseline leg of
 * the benchmark may load this library.  The product path never calls it.
 *
 * What it computes is the depth loop of the mstar pull request "Qwen3-TTS:
 * Run the 1.7B Depth Loop as One Persistent Kernel on Hopper" (#1183), section
 * "How it works": per frame, an input projection, then 16 depth positions
 * each walked through every decoder layer (qkv, attention, o, gate/up, down),
 * a code head and a draw at every position after the first, and 16 code
 * embeddings (the first from a given code, the other 15 from the draws), whose
 * sum is returned with the codes.  Section "Testing" names the outputs that
 * are compared: codes, embedding sums, KV cache and logits.
 *
 * Arithmetic: dot products and softmax are taken in double precision and
 * rounded once to float where the device keeps a float; when cfg->bf16 is set
 * the value is then rounded to bfloat16 (round to nearest even) at exactly the
 * points where the device stores a bf16 activation.  Work is split across
 * threads over rows and output elements only, never over a reduction, so the
 * result does not depend on the thread count.
 *
 * Parity of the whole frame against an outside implementation is pinned by
 * the test suite through the pieces it is made of (see oracle.c).
 */
#ifndef DEPTH_LOOP_ORACLE_H
#define DEPTH_LOOP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_layers, hidden, input_dim, n_q_heads, n_kv_heads, head_dim;
  int32_t intermediate, n_positions, vocab;
  int32_t bf16;          /* nonzero: round activations to bf16 at the storage points */
  double rms_eps;        /* RMSNorm epsilon */
  double rope_theta;     /* RoPE base */
  int32_t qk_norm;       /* nonzero: RMSNorm of every q and k head (gains q_norm, k_norm) before RoPE */
} orc_cfg;

/* Weights as float values (bf16 weights widened exactly), row-major [out][in]. */
typedef struct {
  const float *w_in;       /* [hidden][input_dim] */
  const float *embed;      /* [P][vocab][hidden]; table j embeds code j */
  const float *attn_norm;  /* [L][hidden] */
  const float *w_qkv;      /* [L][(nq + 2 nkv) d][hidden]; rows q heads | k heads | v heads */
  const float *w_o;        /* [L][hidden][nq d] */
  const float *mlp_norm;   /* [L][hidden] */
  const float *w_gate;     /* [L][inter][hidden] */
  const float *w_up;       /* [L][inter][hidden] */
  const float *w_down;     /* [L][hidden][inter] */
  const float *final_norm; /* [hidden] */
  const float *w_head;     /* [P-1][vocab][hidden]; head j (position j) at index j-1 */
  const float *q_norm;     /* [L][head_dim] (qk_norm only) */
  const float *k_norm;     /* [L][head_dim] (qk_norm only) */
} orc_weights;

typedef struct {
  int32_t rows;
  const float *hidden_in;       /* [rows][input_dim] */
  const int32_t *code0;         /* [rows] code 0, from outside the loop */
  /* Sampling parameters, [rows] each; all NULL selects greedy for every row. */
  const float *temperature;
  const int32_t *top_k;
  const float *top_p;
  const uint64_t *seed;
  const uint64_t *offset_in;
  /* Optional teacher forcing [rows][P-1]: these codes, not the oracle's own
     draws, feed the next position and the embedding sum. */
  const int32_t *forced_codes;
  /* Outputs. */
  int32_t *codes;               /* [rows][P-1] the oracle's own draw at each position */
  float *embsum;                /* [rows][hidden] */
  float *logits;                /* NULL or [rows][P-1][vocab] */
  float *k_cache, *v_cache;     /* NULL or [L][rows][P][nkv][d] (post-RoPE K) */
  float *pos_hidden;            /* NULL or [rows][P][hidden] residual stream after the last layer */
  uint64_t *offset_out;         /* NULL or [rows] */
  double *margins;              /* NULL or [rows][P-1][4], see orc_draw */
  int32_t n_threads;            /* <= 0: library default */
  /* NULL or [rows][P][L][ORC_STAGES][orc_stage_width(cfg)]: every stage's
     values for each row, position and layer, as stored (for the tests that
     pin where rounding happens).  Stage s holds ORC_STAGE_LEN(s) leading
     values of its slot. */
  float *stages;
  float *final_normed;          /* NULL or [rows][P-1][hidden]: the final-norm output before head j */
} orc_frame;

/* Stages recorded per (row, position, layer). */
enum {
  ORC_ST_H_IN = 0,   /* the layer's input residual row [hidden] */
  ORC_ST_A,          /* attention RMSNorm output [hidden] */
  ORC_ST_QKV_RAW,    /* W_qkv . a as float, before the head norms and RoPE [(nq + 2 nkv) d] */
  ORC_ST_QKV,        /* q, k, v after RoPE, as stored [(nq + 2 nkv) d] */
  ORC_ST_ATT,        /* attention output as stored [nq d] */
  ORC_ST_H_MID,      /* residual after o, as stored [hidden] */
  ORC_ST_A2,         /* MLP RMSNorm output [hidden] */
  ORC_ST_GATE,       /* W_gate . a2 as float [inter] */
  ORC_ST_UP,         /* W_up . a2 as float [inter] */
  ORC_ST_M,          /* SwiGLU output as stored [inter] */
  ORC_ST_H_OUT,      /* residual after down, as stored [hidden] */
  ORC_STAGES
};

/* Floats per stage slot: the largest of hidden, (nq + 2 nkv) d and inter. */
int32_t orc_stage_width(const orc_cfg *cfg);

/* Runs one frame.  Returns 0 on success, a negative value for invalid input. */
int orc_frame_run(const orc_cfg *cfg, const orc_weights *w, orc_frame *fr);

/* Philox4x64-10 block function: out = philox(ctr, key). */
void orc_philox4x64(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);

/* One draw from logits z[vocab] (see oracle.c for the rule).  temperature <= 0
   means greedy.  margins[4] (may be NULL) receives: the gap between the best and
   second-best deciding score; the gap at the top-k boundary; p minus the mass
   before the top-p crossing token; the mass including it minus p.  Margins that
   do not apply are +inf. */
int32_t orc_draw(const float *z, int32_t vocab, float temperature, int32_t top_k, float top_p,
                 uint64_t seed, uint64_t counter, double *margins);

/* The kept set of a sampled draw, in rank order; returns its size. */
int32_t orc_kept_set(const float *z, int32_t vocab, float temperature, int32_t top_k, float top_p,
                     int32_t *kept);

/* bf16 round-to-nearest-even of a float (returned as a float). */
float orc_round_bf16(float x);

#ifdef __cplusplus
}
#endif
#endif
