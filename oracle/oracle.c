/*
 * CPU oracle of the codec-TTS depth loop -- TEST INFRASTRUCTURE ONLY.
 * Used by the tests, the smoke check and the benchmark's CPU baseline; the
 * product path never loads it.  It shares no code with the HIP library.
 *
 * Source of the method: mstar pull request #1183, "Qwen3-TTS: Run the 1.7B
 * Depth Loop as One Persistent Kernel on Hopper".
 *   - "How it works": the frame's phases (input projection; qkv, attention,
 *     o, gate/up, down per layer and position; 15 heads; 16 embedding steps,
 *     15 of which draw a code first); the draw uses per-row temperature,
 *     top-k, top-p, seed and offset, and offsets advance as that many single
 *     draws would.
 *   - "Testing": codes, embedding sums, KV cache and logits are the outputs.
 * Readings where the pages leave a step open (the decoder layer is the usual
 * pre-norm Llama-style block with RMSNorm, rotate-half RoPE, grouped-query
 * attention and SwiGLU; position 0 holds the projected input hidden, position
 * 1 the embedding of code 0, position j+1 the embedding of code j; head j runs
 * at position j; the draw is temperature -> top-k -> top-p -> Gumbel-max with
 * Philox4x64-10 noise) are listed with the design notes of this repository.
 *
 * Pins (in the test suite): the transformer stack against an fp64 Llama
 * forward from the transformers library; Philox against numpy's Philox;
 * the draw against brute force and the Gumbel-max sampling law; the
 * embedding sum, the offsets and the causal structure against their
 * definitions; the bf16 rounding points stage by stage (every recorded stage
 * recomputed from the one before it with numpy and torch's bf16 rounding, a
 * planted frame worked out by hand, and mutants with one rounding removed,
 * moved or added, each of which must fail).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ---------------------------------------------------------------- rounding */

float orc_round_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return x; /* inf / nan unchanged */
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  memcpy(&x, &u, 4);
  return x;
}

/* Rounds a double to the stored activation type: float, then bf16 if asked. */
static inline float store_act(const orc_cfg *c, double v) {
  float f = (float)v;
  return c->bf16 ? orc_round_bf16(f) : f;
}

/* Dot product in double precision, K in ascending order. */
static inline double dot(const float *a, const float *b, int n) {
  double s = 0.0;
  for (int k = 0; k < n; ++k) s += (double)a[k] * (double)b[k];
  return s;
}

/* ---------------------------------------------------------------- philox */

/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
   as 1, 2, 3", SC'11): ten rounds of two 64x64->128 multiplies with a Weyl
   key schedule. */
void orc_philox4x64(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    unsigned __int128 p0 = (unsigned __int128)M0 * x0;
    unsigned __int128 p1 = (unsigned __int128)M1 * x2;
    uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    uint64_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    k0 += W0; k1 += W1;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Uniform in (0, 1) for vocabulary entry i of one draw: word 0 of
   philox(counter = (draw counter, i, 0, 0), key = (seed, 0)); its top 23 bits
   m give u = (2m + 1) / 2^24, exact in float and never 0 or 1. */
static double draw_uniform(uint64_t seed, uint64_t counter, int32_t i) {
  uint64_t ctr[4] = {counter, (uint64_t)(uint32_t)i, 0, 0}, key[2] = {seed, 0}, o[4];
  orc_philox4x64(ctr, key, o);
  uint64_t m = o[0] >> 41;
  return (double)(2 * m + 1) * (1.0 / 16777216.0);
}

/* ---------------------------------------------------------------- draw */

typedef struct { float v; int32_t i; } ranked;

/* Larger value first; equal values by lower index. */
static int rank_cmp(const void *pa, const void *pb) {
  const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

/* Sampled draw, steps in order:
     y = z / T (float division);
     top-k: the k largest y, ties to the lower index (k <= 0 or k >= V: all);
     softmax over them (double);
     top-p: in rank order keep the shortest prefix whose mass reaches p (the
       crossing token is kept; p >= 1 keeps all, p <= 0 only the first);
     Gumbel-max: code = argmax over kept i of y_i - log(-log u_i), ties to the
       lower index.
   This draws exactly from the renormalised kept distribution. */
static int32_t sampled_draw(const float *z, int32_t V, float T, int32_t top_k, float top_p,
                            uint64_t seed, uint64_t counter, int32_t *kept_out,
                            int32_t *n_kept_out, double *margins) {
  ranked *r = (ranked *)malloc(sizeof(ranked) * (size_t)V);
  float *y = (float *)malloc(sizeof(float) * (size_t)V);
  for (int32_t i = 0; i < V; ++i) {
    y[i] = z[i] / T;
    r[i].v = y[i];
    r[i].i = i;
  }
  qsort(r, (size_t)V, sizeof(ranked), rank_cmp);
  int32_t kk = (top_k <= 0 || top_k >= V) ? V : top_k;
  double m_k = (kk < V) ? (double)r[kk - 1].v - (double)r[kk].v : INFINITY;

  double *w = (double *)malloc(sizeof(double) * (size_t)kk);
  double Z = 0.0;
  for (int32_t t = 0; t < kk; ++t) {
    w[t] = exp((double)r[t].v - (double)r[0].v);
    Z += w[t];
  }
  int32_t n_keep;
  double m_before = INFINITY, m_at = INFINITY;
  if (top_p >= 1.0f) {
    n_keep = kk;
  } else if (top_p <= 0.0f) {
    n_keep = 1;
  } else {
    double cum = 0.0;
    n_keep = kk;
    for (int32_t t = 0; t < kk; ++t) {
      double before = cum;
      cum += w[t] / Z;
      if (cum >= (double)top_p) {
        n_keep = t + 1;
        m_before = (double)top_p - before;
        m_at = cum - (double)top_p;
        break;
      }
    }
  }
  int32_t best = -1;
  double best_s = -INFINITY, second_s = -INFINITY;
  for (int32_t t = 0; t < n_keep; ++t) {
    int32_t i = r[t].i;
    double u = draw_uniform(seed, counter, i);
    double s = (double)y[i] - log(-log(u));
    if (s > best_s || (s == best_s && i < best)) {
      second_s = best_s;
      best_s = s;
      best = i;
    } else if (s > second_s) {
      second_s = s;
    }
  }
  if (kept_out)
    for (int32_t t = 0; t < n_keep; ++t) kept_out[t] = r[t].i;
  if (n_kept_out) *n_kept_out = n_keep;
  if (margins) {
    margins[0] = (n_keep > 1) ? best_s - second_s : INFINITY;
    margins[1] = m_k;
    margins[2] = m_before;
    margins[3] = m_at;
  }
  free(w);
  free(y);
  free(r);
  return best;
}

/* Greedy draw: the lowest index holding the largest logit. */
static int32_t greedy_draw(const float *z, int32_t V, double *margins) {
  int32_t best = 0;
  for (int32_t i = 1; i < V; ++i)
    if (z[i] > z[best]) best = i;
  double second = -INFINITY;
  for (int32_t i = 0; i < V; ++i)
    if (i != best && (double)z[i] > second) second = (double)z[i];
  if (margins) {
    margins[0] = (V > 1) ? (double)z[best] - second : INFINITY;
    margins[1] = margins[2] = margins[3] = INFINITY;
  }
  return best;
}

int32_t orc_draw(const float *z, int32_t vocab, float temperature, int32_t top_k, float top_p,
                 uint64_t seed, uint64_t counter, double *margins) {
  if (vocab <= 0) return -1;
  if (!(temperature > 0.0f)) return greedy_draw(z, vocab, margins);
  return sampled_draw(z, vocab, temperature, top_k, top_p, seed, counter, NULL, NULL, margins);
}

int32_t orc_kept_set(const float *z, int32_t vocab, float temperature, int32_t top_k, float top_p,
                     int32_t *kept) {
  int32_t n = 0;
  if (vocab <= 0) return 0;
  if (!(temperature > 0.0f)) {
    kept[0] = greedy_draw(z, vocab, NULL);
    return 1;
  }
  sampled_draw(z, vocab, temperature, top_k, top_p, 0, 0, kept, &n, NULL);
  return n;
}

/* ---------------------------------------------------------------- layer parts */

/* RMSNorm: out_i = store(float(float(h_i * r) * g_i)), r = 1 / sqrt(mean(h^2) + eps)
   rounded to float.  The products are float products, in that order. */
static void rmsnorm(const orc_cfg *c, const float *h, const float *g, float *out) {
  int H = c->hidden;
  double ss = 0.0;
  for (int i = 0; i < H; ++i) ss += (double)h[i] * (double)h[i];
  float r = (float)(1.0 / sqrt(ss / (double)H + c->rms_eps));
  for (int i = 0; i < H; ++i) {
    float t = h[i] * r;
    float v = t * g[i];
    out[i] = c->bf16 ? orc_round_bf16(v) : v;
  }
}

/* Head norm of the QK-norm variant (the per-head RMSNorm of q and k that
   Qwen3-style attention applies before RoPE; the handbook page "The gaps
   between kernels: PDL and megakernels" lists it fused with RoPE in one
   kernel): over one head's d values, the same float products as rmsnorm, in
   float, with no bf16 rounding (the head is rounded once, after RoPE). */
static void headnorm(const orc_cfg *c, float *x, const float *g) {
  const int d = c->head_dim;
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += (double)x[i] * (double)x[i];
  float r = (float)(1.0 / sqrt(ss / (double)d + c->rms_eps));
  for (int i = 0; i < d; ++i) {
    float t = x[i] * r;
    x[i] = t * g[i];
  }
}

int32_t orc_stage_width(const orc_cfg *c) {
  int32_t wd = c->hidden;
  const int32_t qkv = (c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
  if (qkv > wd) wd = qkv;
  if (c->intermediate > wd) wd = c->intermediate;
  return wd;
}

/* Copies n values of each row's stage s at (p, l) into fr->stages. */
static void record(const orc_cfg *c, orc_frame *fr, int p, int l, int s, const float *src, int stride, int n) {
  if (!fr->stages) return;
  const size_t W = (size_t)orc_stage_width(c);
  for (int r = 0; r < fr->rows; ++r) {
    float *dst = fr->stages + ((((size_t)r * c->n_positions + p) * c->n_layers + l) * ORC_STAGES + s) * W;
    memcpy(dst, src + (size_t)r * stride, sizeof(float) * n);
  }
}

int orc_frame_run(const orc_cfg *c, const orc_weights *w, orc_frame *fr) {
  if (!c || !w || !fr) return -1;
  const int L = c->n_layers, H = c->hidden, Din = c->input_dim, nq = c->n_q_heads,
            nkv = c->n_kv_heads, d = c->head_dim, I = c->intermediate, P = c->n_positions,
            V = c->vocab, R = fr->rows;
  if (L < 1 || H < 1 || Din < 1 || nq < 1 || nkv < 1 || nq % nkv || d < 2 || d % 2 || I < 1 ||
      P < 2 || V < 1 || R < 0)
    return -2;
  if (R == 0) return 0;
  if (!fr->hidden_in || !fr->code0 || !fr->codes || !fr->embsum) return -3;
  if (c->qk_norm && (!w->q_norm || !w->k_norm)) return -3;
  const int sampled = fr->temperature != NULL;
  if (sampled && !(fr->top_k && fr->top_p && fr->seed && fr->offset_in)) return -4;
  for (int r = 0; r < R; ++r)
    if (fr->code0[r] < 0 || fr->code0[r] >= V) return -5;
  if (fr->forced_codes)
    for (int i = 0; i < R * (P - 1); ++i)
      if (fr->forced_codes[i] < 0 || fr->forced_codes[i] >= V) return -5;

  const int nt = fr->n_threads > 0 ? fr->n_threads : omp_get_max_threads();
  const int qd = nq * d, QKV = (nq + 2 * nkv) * d, half = d / 2;
  const size_t kv_stride_l = (size_t)R * P * nkv * d;

  float *h = (float *)calloc((size_t)R * H, sizeof(float));      /* residual stream */
  float *a = (float *)calloc((size_t)R * H, sizeof(float));      /* normed activation */
  float *qkv = (float *)calloc((size_t)R * QKV, sizeof(float));  /* projection, float */
  float *att = (float *)calloc((size_t)R * qd, sizeof(float));   /* attention output */
  float *gt = (float *)calloc((size_t)R * I, sizeof(float));
  float *up = (float *)calloc((size_t)R * I, sizeof(float));
  float *mm = (float *)calloc((size_t)R * I, sizeof(float));
  float *z = (float *)calloc((size_t)R * V, sizeof(float));
  float *kc = (float *)calloc((size_t)L * kv_stride_l, sizeof(float));
  float *vc = (float *)calloc((size_t)L * kv_stride_l, sizeof(float));
  float *nxt = (float *)calloc((size_t)R * H, sizeof(float));     /* next position's input */
  float *cs = (float *)calloc((size_t)P * half, sizeof(float));
  float *sn = (float *)calloc((size_t)P * half, sizeof(float));
  if (!h || !a || !qkv || !att || !gt || !up || !mm || !z || !kc || !vc || !nxt || !cs || !sn) {
    free(h); free(a); free(qkv); free(att); free(gt); free(up); free(mm); free(z);
    free(kc); free(vc); free(nxt); free(cs); free(sn);
    return -6;
  }

  /* RoPE angles: position p, pair i rotates by p * theta^(-2i/d); cos and sin
     are taken in double and rounded to float. */
  for (int p = 0; p < P; ++p)
    for (int i = 0; i < half; ++i) {
      double ang = (double)p * pow(c->rope_theta, -2.0 * (double)i / (double)d);
      cs[p * half + i] = (float)cos(ang);
      sn[p * half + i] = (float)sin(ang);
    }

  /* Input projection (position 0's input): u0 = store(W_in . x). */
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
  for (int r = 0; r < R; ++r)
    for (int n = 0; n < H; ++n) {
      h[(size_t)r * H + n] = store_act(c, dot(w->w_in + (size_t)n * Din, fr->hidden_in + (size_t)r * Din, Din));
    }

  /* Embedding of code 0: position 1's input and the first term of the sum. */
  for (int r = 0; r < R; ++r) {
    const float *e = w->embed + ((size_t)0 * V + fr->code0[r]) * H;
    memcpy(nxt + (size_t)r * H, e, sizeof(float) * H);
    memcpy(fr->embsum + (size_t)r * H, e, sizeof(float) * H);
  }

  for (int p = 0; p < P; ++p) {
    if (p > 0) memcpy(h, nxt, sizeof(float) * (size_t)R * H);
    for (int l = 0; l < L; ++l) {
      const float *wqkv = w->w_qkv + (size_t)l * QKV * H;
      const float *wo = w->w_o + (size_t)l * H * qd;
      const float *wg = w->w_gate + (size_t)l * I * H;
      const float *wu = w->w_up + (size_t)l * I * H;
      const float *wd = w->w_down + (size_t)l * H * I;
      float *kl = kc + (size_t)l * kv_stride_l, *vl = vc + (size_t)l * kv_stride_l;
      record(c, fr, p, l, ORC_ST_H_IN, h, H, H);

      /* qkv: a = RMSNorm(h) * g_attn; [q|k|v] = W_qkv . a (float). */
      for (int r = 0; r < R; ++r) rmsnorm(c, h + (size_t)r * H, w->attn_norm + (size_t)l * H, a + (size_t)r * H);
      record(c, fr, p, l, ORC_ST_A, a, H, H);
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
      for (int r = 0; r < R; ++r)
        for (int n = 0; n < QKV; ++n)
          qkv[(size_t)r * QKV + n] = (float)dot(wqkv + (size_t)n * H, a + (size_t)r * H, H);
      record(c, fr, p, l, ORC_ST_QKV_RAW, qkv, QKV, QKV);

      /* QK-norm variant: each q head and k head normed on its own; then RoPE
         at position p on every q and k head (pairs i, i + d/2), then the
         stored Q, K, V. */
#pragma omp parallel for schedule(static) num_threads(nt)
      for (int r = 0; r < R; ++r) {
        float *row = qkv + (size_t)r * QKV;
        for (int hd = 0; hd < nq + nkv; ++hd) {
          float *x = row + (size_t)hd * d;
          if (c->qk_norm) headnorm(c, x, (hd < nq ? w->q_norm : w->k_norm) + (size_t)l * d);
          for (int i = 0; i < half; ++i) {
            double x1 = x[i], x2 = x[i + half], co = cs[p * half + i], si = sn[p * half + i];
            double y1 = x1 * co - x2 * si, y2 = x2 * co + x1 * si;
            x[i] = (float)y1;
            x[i + half] = (float)y2;
          }
        }
        for (int n = 0; n < QKV; ++n) row[n] = store_act(c, row[n]);
        for (int g = 0; g < nkv; ++g) {
          size_t o = (((size_t)r * P + p) * nkv + g) * d;
          memcpy(kl + o, row + qd + (size_t)g * d, sizeof(float) * d);
          memcpy(vl + o, row + qd + (size_t)(nkv + g) * d, sizeof(float) * d);
        }
      }
      record(c, fr, p, l, ORC_ST_QKV, qkv, QKV, QKV);

      /* Attention: q head hq reads kv head hq / (nq / nkv); causal over t <= p;
         scale 1 / sqrt(d); softmax in double; output stored. */
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
      for (int r = 0; r < R; ++r)
        for (int hq = 0; hq < nq; ++hq) {
          const int g = hq / (nq / nkv);
          const float *q = qkv + (size_t)r * QKV + (size_t)hq * d;
          double s[64], e[64];
          double mx = -INFINITY, zs = 0.0;
          double *sp = (p + 1 <= 64) ? s : (double *)malloc(sizeof(double) * (p + 1));
          double *ep = (p + 1 <= 64) ? e : (double *)malloc(sizeof(double) * (p + 1));
          for (int t = 0; t <= p; ++t) {
            const float *k = kl + (((size_t)r * P + t) * nkv + g) * d;
            sp[t] = dot(q, k, d) / sqrt((double)d);
            if (sp[t] > mx) mx = sp[t];
          }
          for (int t = 0; t <= p; ++t) {
            ep[t] = exp(sp[t] - mx);
            zs += ep[t];
          }
          for (int i = 0; i < d; ++i) {
            double o = 0.0;
            for (int t = 0; t <= p; ++t)
              o += (ep[t] / zs) * (double)vl[(((size_t)r * P + t) * nkv + g) * d + i];
            att[(size_t)r * qd + (size_t)hq * d + i] = store_act(c, o);
          }
          if (sp != s) free(sp);
          if (ep != e) free(ep);
        }
      record(c, fr, p, l, ORC_ST_ATT, att, qd, qd);

      /* o projection and residual: h = store(h + W_o . attn). */
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
      for (int r = 0; r < R; ++r)
        for (int n = 0; n < H; ++n) {
          double v = (double)h[(size_t)r * H + n] + dot(wo + (size_t)n * qd, att + (size_t)r * qd, qd);
          a[(size_t)r * H + n] = store_act(c, v); /* a used as scratch for the new h */
        }
      memcpy(h, a, sizeof(float) * (size_t)R * H);
      record(c, fr, p, l, ORC_ST_H_MID, h, H, H);

      /* gate/up: a2 = RMSNorm(h) * g_mlp; m = store(silu(W_gate . a2) * (W_up . a2)),
         silu(x) = x / (1 + exp(-x)). */
      for (int r = 0; r < R; ++r) rmsnorm(c, h + (size_t)r * H, w->mlp_norm + (size_t)l * H, a + (size_t)r * H);
      record(c, fr, p, l, ORC_ST_A2, a, H, H);
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
      for (int r = 0; r < R; ++r)
        for (int n = 0; n < I; ++n) {
          float gv = (float)dot(wg + (size_t)n * H, a + (size_t)r * H, H);
          float uv = (float)dot(wu + (size_t)n * H, a + (size_t)r * H, H);
          double sl = (double)gv / (1.0 + exp(-(double)gv));
          gt[(size_t)r * I + n] = gv;
          up[(size_t)r * I + n] = uv;
          mm[(size_t)r * I + n] = store_act(c, sl * (double)uv);
        }
      record(c, fr, p, l, ORC_ST_GATE, gt, I, I);
      record(c, fr, p, l, ORC_ST_UP, up, I, I);
      record(c, fr, p, l, ORC_ST_M, mm, I, I);

      /* down projection and residual: h = store(h + W_down . m). */
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
      for (int r = 0; r < R; ++r)
        for (int n = 0; n < H; ++n) {
          double v = (double)h[(size_t)r * H + n] + dot(wd + (size_t)n * I, mm + (size_t)r * I, I);
          a[(size_t)r * H + n] = store_act(c, v);
        }
      memcpy(h, a, sizeof(float) * (size_t)R * H);
      record(c, fr, p, l, ORC_ST_H_OUT, h, H, H);
    }

    if (fr->pos_hidden)
      for (int r = 0; r < R; ++r)
        memcpy(fr->pos_hidden + ((size_t)r * P + p) * H, h + (size_t)r * H, sizeof(float) * H);
    if (p == 0) continue; /* no head at position 0 */

    /* Head p: f = RMSNorm(h) * g_final; z = W_head_p . f (float, not rounded). */
    const int j = p;
    const float *wh = w->w_head + (size_t)(j - 1) * V * H;
    for (int r = 0; r < R; ++r) rmsnorm(c, h + (size_t)r * H, w->final_norm, a + (size_t)r * H);
    if (fr->final_normed)
      for (int r = 0; r < R; ++r)
        memcpy(fr->final_normed + ((size_t)r * (P - 1) + (j - 1)) * H, a + (size_t)r * H, sizeof(float) * H);
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
    for (int r = 0; r < R; ++r)
      for (int n = 0; n < V; ++n) z[(size_t)r * V + n] = (float)dot(wh + (size_t)n * H, a + (size_t)r * H, H);

    /* Draw j, then embed the code with table j (sum in float, in order j). */
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int r = 0; r < R; ++r) {
      const float *zr = z + (size_t)r * V;
      double *mg = fr->margins ? fr->margins + ((size_t)r * (P - 1) + (j - 1)) * 4 : NULL;
      int32_t code;
      if (sampled)
        code = orc_draw(zr, V, fr->temperature[r], fr->top_k[r], fr->top_p[r], fr->seed[r],
                        fr->offset_in[r] + (uint64_t)(j - 1), mg);
      else
        code = orc_draw(zr, V, 0.0f, 0, 1.0f, 0, 0, mg);
      fr->codes[(size_t)r * (P - 1) + (j - 1)] = code;
      if (fr->logits) memcpy(fr->logits + ((size_t)r * (P - 1) + (j - 1)) * V, zr, sizeof(float) * V);
      int32_t use = fr->forced_codes ? fr->forced_codes[(size_t)r * (P - 1) + (j - 1)] : code;
      const float *e = w->embed + ((size_t)j * V + use) * H;
      float *sr = fr->embsum + (size_t)r * H;
      for (int i = 0; i < H; ++i) sr[i] = sr[i] + e[i];
      if (p < P - 1) memcpy(nxt + (size_t)r * H, e, sizeof(float) * H);
    }
  }

  if (fr->k_cache) memcpy(fr->k_cache, kc, sizeof(float) * (size_t)L * kv_stride_l);
  if (fr->v_cache) memcpy(fr->v_cache, vc, sizeof(float) * (size_t)L * kv_stride_l);
  if (fr->offset_out)
    for (int r = 0; r < R; ++r)
      fr->offset_out[r] = sampled ? fr->offset_in[r] + (uint64_t)(P - 1) : 0;

  free(h); free(a); free(qkv); free(att); free(gt); free(up); free(mm); free(z);
  free(kc); free(vc); free(nxt); free(cs); free(sn);
  return 0;
}
