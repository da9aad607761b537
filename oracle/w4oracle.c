/*
 * CPU oracle for the batched-concurrent int4 (W4A16, group-wise) MoE decode
 * step.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the product library never does,
 * and this file shares no code, header or table with it.
 *
 * What it computes is the plain per-stream transformer decode step with
 * dequantised weights.  In the batched design ("Batched-concurrent 4-bit
 * serving on Apple Silicon", section 3) no row of a batched product depends
 * on another row, and the per-stream steps each work on their own stream's
 * data, so a batch of B streams gives exactly what B separate single-stream
 * steps give; the oracle therefore takes the streams one at a time and never
 * batches.
 *
 * Precision (workload definition): int4 group dequant w = q * s, exact in
 * fp32; every dot product accumulates in fp32, sequentially over k; values are
 * stored as IEEE binary16 (round to nearest even) at the points marked "=>h".
 * Built with -ffp-contract=off so each * and + rounds on its own.  Threads
 * (OpenMP) only split independent outputs, never one dot product.
 *
 * Readings of points the pages leave open are listed where they are used.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* Threads the oracle's parallel loops use (1 without OpenMP). */
EXPORT int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the threads of the parallel loops (n >= 1; no effect without OpenMP). */
EXPORT void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, round to nearest, ties to even.           */
/* ------------------------------------------------------------------------ */
EXPORT float orc_h2f(uint16_t h) {
  unsigned sign = (h >> 15) & 1u, ex = (h >> 10) & 0x1fu, man = h & 0x3ffu;
  float v;
  if (ex == 0)
    v = ldexpf((float)man, -24); /* zero and subnormals: man * 2^-24 */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexpf((float)(man | 0x400u), (int)ex - 25); /* 1.man * 2^(ex-15) */
  return sign ? -v : v;
}

EXPORT uint16_t orc_f2h(float f) {
  uint16_t sign = signbit(f) ? 0x8000u : 0u;
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  float a = fabsf(f);
  if (a >= 65520.0f) return (uint16_t)(sign | 0x7c00u); /* past the max finite's halfway point */
  if (a == 0.0f) return sign;
  int e2;
  frexpf(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
  int e = e2 - 1;          /* a in [2^e, 2^(e+1)) */
  if (e < -14) e = -14;    /* subnormal range shares the quantum of the smallest binade */
  float quantum = ldexpf(1.0f, e - 10);
  float n = rintf(a / quantum); /* exact division by a power of two; rint = ties to even */
  float v = n * quantum;        /* the rounded magnitude, exact */
  if (v == 0.0f) return sign;
  if (v >= 65536.0f) return (uint16_t)(sign | 0x7c00u);
  if (v < ldexpf(1.0f, -14)) return (uint16_t)(sign | (uint16_t)(v / ldexpf(1.0f, -24)));
  frexpf(v, &e2);
  int ev = e2 - 1;
  unsigned man = (unsigned)(v / ldexpf(1.0f, ev - 10)) - 1024u;
  return (uint16_t)(sign | ((unsigned)(ev + 15) << 10) | man);
}

static float H2F[65536];
static int h2f_ready = 0;
static void h2f_init(void) {
  if (h2f_ready) return;
  for (unsigned i = 0; i < 65536u; i++) H2F[i] = orc_h2f((uint16_t)i);
  h2f_ready = 1;
}
#define HF(x) (H2F[(x)])

EXPORT void orc_init(void) { h2f_init(); }

EXPORT void orc_h2f_array(const uint16_t* h, float* f, int64_t n) {
  for (int64_t i = 0; i < n; i++) f[i] = orc_h2f(h[i]);
}
EXPORT void orc_f2h_array(const float* f, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; i++) h[i] = orc_f2h(f[i]);
}

/* ------------------------------------------------------------------------ */
/* int4 code of element k of a packed row.  Reading: 4-bit two's complement, */
/* element 2j in the low nibble of byte j, element 2j+1 in the high nibble   */
/* ("packed-int4", section 1 of the batched-serving page; values in [-8,7],  */
/* two per byte, per the workload definition).                               */
/* ------------------------------------------------------------------------ */
static inline int code_at(const uint8_t* row, int k) {
  unsigned b = row[k >> 1];
  unsigned nib = (k & 1) ? (b >> 4) : (b & 15u);
  return nib >= 8 ? (int)nib - 16 : (int)nib;
}

EXPORT int orc_code_at(const uint8_t* row, int k) { return code_at(row, k); }

/* One output of y = x . dequant(W)^T: sum over k of x_k * (q[n][k] * s[n][k/g]),
 * fp32, k ascending.  x is given as floats (exact images of fp16 values). */
static float w4_dot(const float* xf, const uint8_t* prow, const uint16_t* srow, int K, int g) {
  float acc = 0.0f;
  for (int k = 0; k < K; k++) {
    float w = (float)code_at(prow, k) * HF(srow[k / g]); /* exact: 4 bits x 11 bits */
    acc = acc + xf[k] * w;
  }
  return acc;
}

/* Dense W4A16 projection ("Batched-concurrent 4-bit serving", section 1: each
 * packed-int4 dense weight applied to the B rows).  x fp16 [B][K], P [N][K/2],
 * S [N][K/g] fp16.  Writes y16 = fp16 [B][N] (=>h) and/or y32 = fp32 [B][N]. */
EXPORT void orc_w4_gemm(int B, int N, int K, int g, const uint16_t* x, const uint8_t* P,
                        const uint16_t* S, uint16_t* y16, float* y32) {
  h2f_init();
  float* xf = (float*)malloc(sizeof(float) * (size_t)B * K);
  for (int64_t i = 0; i < (int64_t)B * K; i++) xf[i] = HF(x[i]);
  for (int b = 0; b < B; b++) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
      float acc = w4_dot(xf + (size_t)b * K, P + (size_t)n * (K / 2), S + (size_t)n * (K / g), K, g);
      if (y32) y32[(size_t)b * N + n] = acc;
      if (y16) y16[(size_t)b * N + n] = orc_f2h(acc);
    }
  }
  free(xf);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm: out_i = x_i * (1/sqrt(mean(x^2) + eps)) * gamma_i  =>h.           */
/* ------------------------------------------------------------------------ */
EXPORT void orc_rmsnorm(int H, const uint16_t* x, const uint16_t* gamma, float eps, uint16_t* out) {
  h2f_init();
  float ss = 0.0f;
  for (int i = 0; i < H; i++) {
    float v = HF(x[i]);
    ss = ss + v * v;
  }
  float r = 1.0f / sqrtf(ss / (float)H + eps);
  for (int i = 0; i < H; i++) out[i] = orc_f2h((HF(x[i]) * r) * HF(gamma[i]));
}

/* ------------------------------------------------------------------------ */
/* Rotary embedding at position p, rotate-half pairs (i, i + D/2):           */
/*   theta_i = p * base^(-2i/D) (fp64), (a, b) -> (a cos - b sin, a sin + b cos) =>h. */
/* x, out: [nh][D] fp16 (may alias).                                         */
/* ------------------------------------------------------------------------ */
EXPORT void orc_rope(int nh, int D, int pos, double base, const uint16_t* x, uint16_t* out) {
  h2f_init();
  int half = D / 2;
  for (int i = 0; i < half; i++) {
    double ang = (double)pos * pow(base, -2.0 * (double)i / (double)D);
    float c = (float)cos(ang), s = (float)sin(ang);
    for (int h = 0; h < nh; h++) {
      float a = HF(x[h * D + i]), b = HF(x[h * D + i + half]);
      uint16_t o0 = orc_f2h(a * c - b * s);
      uint16_t o1 = orc_f2h(a * s + b * c);
      out[h * D + i] = o0;
      out[h * D + i + half] = o1;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* GQA decode attention for one stream over positions 0..npos-1 of its own   */
/* KV ("Per-stream KV-slot isolation", section 1: a stream's K/V lives in its */
/* own slot).  q head h reads kv head floor(h * Hkv / Hq).                    */
/*   z_j = (q_h . K_j) * (1/sqrt(D)); P_j = exp(z_j - max z) / sum; o = sum P_j V_j  =>h */
/* K and V rows: pointer to position 0 of kv head 0, row stride kv_stride    */
/* elements between positions (kv heads are D apart inside a position).      */
/* ------------------------------------------------------------------------ */
EXPORT void orc_attention(int Hq, int Hkv, int D, int npos, const uint16_t* q, const uint16_t* Kc,
                          const uint16_t* Vc, int64_t kv_stride, uint16_t* o) {
  h2f_init();
  float scale = (float)(1.0 / sqrt((double)D));
#pragma omp parallel for schedule(static)
  for (int h = 0; h < Hq; h++) {
    int g = (int)(((int64_t)h * Hkv) / Hq);
    float* z = (float*)malloc(sizeof(float) * (size_t)npos);
    float m = -INFINITY;
    for (int j = 0; j < npos; j++) {
      const uint16_t* kr = Kc + (size_t)j * kv_stride + (size_t)g * D;
      float dot = 0.0f;
      for (int i = 0; i < D; i++) dot = dot + HF(q[h * D + i]) * HF(kr[i]);
      z[j] = dot * scale;
      if (z[j] > m) m = z[j];
    }
    float sum = 0.0f;
    for (int j = 0; j < npos; j++) {
      z[j] = expf(z[j] - m);
      sum = sum + z[j];
    }
    for (int j = 0; j < npos; j++) z[j] = z[j] / sum;
    for (int i = 0; i < D; i++) {
      float acc = 0.0f;
      for (int j = 0; j < npos; j++) acc = acc + z[j] * HF(Vc[(size_t)j * kv_stride + (size_t)g * D + i]);
      o[h * D + i] = orc_f2h(acc);
    }
    free(z);
  }
}

/* ------------------------------------------------------------------------ */
/* Top-k softmax routing (one stream).  Reading: experts ranked by logit,    */
/* descending, ties to the lower expert id; the first k are selected (rank   */
/* r = 0..k-1) and weighted by the softmax over the k selected logits:       */
/*   w_r = exp(l_r - l_0) / sum_r' exp(l_r' - l_0).                          */
/* ------------------------------------------------------------------------ */
/* Weights of a ranked selection ids[0..k-1]: the softmax over the selected
 * logits, w_r = exp(l_{ids r} - l_{ids 0}) / sum_r' exp(l_{ids r'} - l_{ids 0}),
 * summed in rank order. */
EXPORT void orc_route_weights(int k, const float* logits, const int32_t* ids, float* w) {
  float sum = 0.0f;
  for (int r = 0; r < k; r++) {
    w[r] = expf(logits[ids[r]] - logits[ids[0]]);
    sum = sum + w[r];
  }
  for (int r = 0; r < k; r++) w[r] = w[r] / sum;
}

EXPORT void orc_topk_softmax(int E, int k, const float* logits, int32_t* ids, float* w) {
  unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
  for (int r = 0; r < k; r++) {
    int best = -1;
    for (int e = 0; e < E; e++) {
      if (taken[e]) continue;
      if (best < 0 || logits[e] > logits[best]) best = e; /* strict: keeps the lower id on ties */
    }
    taken[best] = 1;
    ids[r] = best;
  }
  orc_route_weights(k, logits, ids, w);
  free(taken);
}

/* Routing of one stream: the top-k of its logits, or, when force is not
 * NULL, the ranked expert ids given there (weighted by the softmax over those
 * experts' logits, as above).  The forced form replays a routing decision
 * taken elsewhere at a near-tie of the k-th and (k+1)-th logits, where either
 * choice is a correct top-k within the tolerance; with force equal to this
 * function's own top-k it changes nothing. */
static void route_one(int E, int k, const float* logits, const int32_t* force, int32_t* ids, float* w) {
  if (force) {
    memcpy(ids, force, sizeof(int32_t) * (size_t)k);
    orc_route_weights(k, logits, ids, w);
  } else {
    orc_topk_softmax(E, k, logits, ids, w);
  }
}

/* (stream, expert) bucketing: the B*k (stream, rank) pairs ordered by expert,
 * then by stream ("one grouped sparse-expert operation" over all B streams'
 * selected experts, section 1 of the batched-serving page).  counts[E],
 * offsets[E+1] (exclusive prefix sums), pair_stream / pair_rank [B*k]. */
EXPORT void orc_bucket(int B, int k, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                       int32_t* pair_stream, int32_t* pair_rank) {
  int pos = 0;
  for (int e = 0; e < E; e++) {
    offsets[e] = pos;
    counts[e] = 0;
    for (int b = 0; b < B; b++)
      for (int r = 0; r < k; r++)
        if (ids[b * k + r] == e) {
          pair_stream[pos] = b;
          pair_rank[pos] = r;
          pos++;
          counts[e]++;
        }
  }
  offsets[E] = pos;
}

/* ------------------------------------------------------------------------ */
/* Weight tables.  Canonical layouts; pointer arrays indexed by layer.       */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_layers, hidden, n_q, n_kv, head_dim, n_experts, top_k, inter, vocab, group;
  float rms_eps;
  double rope_theta;
  /* per layer, canonical packed [N][K/2] and scales [N][K/g]; experts stacked on the lead axis */
  const uint16_t** attn_norm;
  const uint8_t** qkv_p;
  const uint16_t** qkv_s;
  const uint8_t** o_p;
  const uint16_t** o_s;
  const uint16_t** moe_norm;
  const uint8_t** r_p;
  const uint16_t** r_s;
  const uint8_t** gate_p;
  const uint16_t** gate_s;
  const uint8_t** up_p;
  const uint16_t** up_s;
  const uint8_t** down_p;
  const uint16_t** down_s;
  const uint8_t* emb_p;
  const uint16_t* emb_s;
  const uint16_t* final_norm;
  const uint8_t* lm_p;
  const uint16_t* lm_s;
} orc_model;

/* Grouped-expert SwiGLU MLP for one stream (section 1 of the batched-serving
 * page: the selected experts of each stream).  Reading of SwiGLU:
 *   gate = x.Wg^T =>h, up = x.Wu^T =>h, a = silu(gate) * up =>h with
 *   silu(t) = t / (1 + exp(-t)); y_r = a.Wd^T =>h;
 *   out = sum_r w_r * y_r (fp32, rank order) =>h.                           */
static void moe_one(const orc_model* m, int l, const uint16_t* xn, const int32_t* ids, const float* w,
                    uint16_t* out) {
  int H = m->hidden, I = m->inter, g = m->group, k = m->top_k;
  float* xf = (float*)malloc(sizeof(float) * (size_t)H);
  float* af = (float*)malloc(sizeof(float) * (size_t)I);
  uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)k * H);
  for (int i = 0; i < H; i++) xf[i] = HF(xn[i]);
  for (int r = 0; r < k; r++) {
    int e = ids[r];
    const uint8_t* gp = m->gate_p[l] + (size_t)e * I * (H / 2);
    const uint16_t* gs = m->gate_s[l] + (size_t)e * I * (H / g);
    const uint8_t* upp = m->up_p[l] + (size_t)e * I * (H / 2);
    const uint16_t* ups = m->up_s[l] + (size_t)e * I * (H / g);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < I; n++) {
      uint16_t gt = orc_f2h(w4_dot(xf, gp + (size_t)n * (H / 2), gs + (size_t)n * (H / g), H, g));
      uint16_t ut = orc_f2h(w4_dot(xf, upp + (size_t)n * (H / 2), ups + (size_t)n * (H / g), H, g));
      float t = HF(gt);
      float silu = t / (1.0f + expf(-t));
      af[n] = HF(orc_f2h(silu * HF(ut)));
    }
    const uint8_t* dp = m->down_p[l] + (size_t)e * H * (I / 2);
    const uint16_t* ds = m->down_s[l] + (size_t)e * H * (I / g);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < H; n++)
      y[(size_t)r * H + n] = orc_f2h(w4_dot(af, dp + (size_t)n * (I / 2), ds + (size_t)n * (I / g), I, g));
  }
  for (int n = 0; n < H; n++) {
    float acc = 0.0f;
    for (int r = 0; r < k; r++) acc = acc + w[r] * HF(y[(size_t)r * H + n]);
    out[n] = orc_f2h(acc);
  }
  free(xf);
  free(af);
  free(y);
}

/* MoE block for B streams given router logits (config of the grouped-expert
 * layer): per stream, top-k softmax then the SwiGLU experts; no residual.
 * x fp16 [B][H] (the post-norm input), logits f32 [B][E] -> y fp16 [B][H].
 * force [B][k]: ranked expert ids to use instead of the top-k, or NULL.      */
EXPORT void orc_moe(const orc_model* m, int l, int B, const uint16_t* x, const float* logits,
                    const int32_t* force, uint16_t* y, int32_t* ids_out, float* w_out) {
  h2f_init();
  int k = m->top_k, E = m->n_experts, H = m->hidden;
  for (int b = 0; b < B; b++) {
    int32_t ids[256];
    float w[256];
    route_one(E, k, logits + (size_t)b * E, force ? force + (size_t)b * k : NULL, ids, w);
    if (ids_out) memcpy(ids_out + (size_t)b * k, ids, sizeof(int32_t) * k);
    if (w_out) memcpy(w_out + (size_t)b * k, w, sizeof(float) * k);
    moe_one(m, l, x + (size_t)b * H, ids, w, y + (size_t)b * H);
  }
}

/* KV arena of the oracle: K and V each [L][slots][cap][Hkv][D] fp16, indexed
 * by a stable per-stream slot ("Per-stream KV-slot isolation", section 1). */
typedef struct {
  int32_t n_slots, cap;
  uint16_t* k;
  uint16_t* v;
} orc_arena;

static size_t arena_off(const orc_model* m, const orc_arena* a, int l, int slot, int pos) {
  return ((((size_t)l * a->n_slots + slot) * a->cap + pos) * m->n_kv) * (size_t)m->head_dim;
}

/* One decoder layer for one stream at position p (p keys already cached in
 * its slot; the new key is written at p, attention covers 0..p).
 * h: fp16 [H] residual stream, updated in place.  force: ranked expert ids
 * [k] replacing the top-k (see route_one), or NULL. */
static void layer_one(const orc_model* m, orc_arena* a, int l, int slot, int p, uint16_t* h,
                      const int32_t* force, int32_t* ids_out, float* logits_out) {
  int H = m->hidden, Hq = m->n_q, Hkv = m->n_kv, D = m->head_dim, g = m->group;
  int nq = Hq * D, nkv = Hkv * D, nqkv = nq + 2 * nkv, E = m->n_experts, k = m->top_k;
  uint16_t* xn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* qkv = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nqkv);
  uint16_t* att = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nq);
  uint16_t* proj = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  float* lg = (float*)malloc(sizeof(float) * (size_t)E);
  /* attention block */
  orc_rmsnorm(H, h, m->attn_norm[l], m->rms_eps, xn);
  orc_w4_gemm(1, nqkv, H, g, xn, m->qkv_p[l], m->qkv_s[l], qkv, NULL);
  orc_rope(Hq, D, p, m->rope_theta, qkv, qkv);             /* q heads */
  orc_rope(Hkv, D, p, m->rope_theta, qkv + nq, qkv + nq);  /* k heads */
  size_t off = arena_off(m, a, l, slot, p);
  memcpy(a->k + off, qkv + nq, sizeof(uint16_t) * (size_t)nkv);
  memcpy(a->v + off, qkv + nq + nkv, sizeof(uint16_t) * (size_t)nkv);
  size_t base = arena_off(m, a, l, slot, 0);
  orc_attention(Hq, Hkv, D, p + 1, qkv, a->k + base, a->v + base, (int64_t)nkv, att);
  orc_w4_gemm(1, H, nq, g, att, m->o_p[l], m->o_s[l], proj, NULL);
  for (int i = 0; i < H; i++) h[i] = orc_f2h(HF(h[i]) + HF(proj[i]));
  /* MoE block */
  orc_rmsnorm(H, h, m->moe_norm[l], m->rms_eps, xn);
  orc_w4_gemm(1, E, H, g, xn, m->r_p[l], m->r_s[l], NULL, lg);   /* router logits stay fp32 */
  int32_t ids[256];
  float w[256];
  route_one(E, k, lg, force, ids, w);
  if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * k);
  if (logits_out) memcpy(logits_out, lg, sizeof(float) * E);
  moe_one(m, l, xn, ids, w, proj);
  for (int i = 0; i < H; i++) h[i] = orc_f2h(HF(h[i]) + HF(proj[i]));
  free(xn);
  free(qkv);
  free(att);
  free(proj);
  free(lg);
}

/* One layer for B streams (slots[b], positions[b]); h fp16 [B][H] in/out.
 * force [B][k] ranked expert ids replacing the top-k, or NULL; ids_out [B][k]
 * and logits_out [B][E] (router) optional. */
EXPORT void orc_layer_step(const orc_model* m, orc_arena* a, int l, int B, const int32_t* slots,
                           const int32_t* positions, uint16_t* h, const int32_t* force, int32_t* ids_out,
                           float* logits_out) {
  h2f_init();
  for (int b = 0; b < B; b++)
    layer_one(m, a, l, slots[b], positions[b], h + (size_t)b * m->hidden,
              force ? force + (size_t)b * m->top_k : NULL, ids_out ? ids_out + (size_t)b * m->top_k : NULL,
              logits_out ? logits_out + (size_t)b * m->n_experts : NULL);
}

/* Embedding row of a token, dequantised and stored =>h (step O1). */
static void embed_row(const orc_model* m, int token, uint16_t* h) {
  const int H = m->hidden, g = m->group;
  const uint8_t* er = m->emb_p + (size_t)token * (H / 2);
  const uint16_t* es = m->emb_s + (size_t)token * (H / g);
  for (int i = 0; i < H; i++) h[i] = orc_f2h((float)code_at(er, i) * HF(es[i / g]));
}

/* h [B][hidden] = the embedding rows of tokens[b]. */
EXPORT void orc_embed(const orc_model* m, int B, const int32_t* tokens, uint16_t* h) {
  h2f_init();
  for (int b = 0; b < B; b++) embed_row(m, tokens[b], h + (size_t)b * m->hidden);
}

/* Whole decode step for B streams: embedding row of the token (dequantised
 * =>h), every layer, final RMSNorm, output projection =>h, greedy argmax
 * (ties to the lower id).  Greedy decoding per the batched-serving page,
 * section 3.  logits fp16 [B][V] (optional), next [B], ids_out [L][B][k];
 * force [L][B][k]: ranked expert ids replacing every layer's top-k, or NULL. */
EXPORT void orc_decode_step(const orc_model* m, orc_arena* a, int B, const int32_t* slots,
                            const int32_t* positions, const int32_t* tokens, const int32_t* force,
                            uint16_t* logits, int32_t* next, int32_t* ids_out, float* router_out) {
  h2f_init();
  int H = m->hidden, V = m->vocab, g = m->group, k = m->top_k, E = m->n_experts;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* hn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* lg = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)V);
  for (int b = 0; b < B; b++) {
    embed_row(m, tokens[b], h);
    for (int l = 0; l < m->n_layers; l++)
      layer_one(m, a, l, slots[b], positions[b], h, force ? force + ((size_t)l * B + b) * k : NULL,
                ids_out ? ids_out + ((size_t)l * B + b) * k : NULL,
                router_out ? router_out + ((size_t)l * B + b) * E : NULL);
    orc_rmsnorm(H, h, m->final_norm, m->rms_eps, hn);
    orc_w4_gemm(1, V, H, g, hn, m->lm_p, m->lm_s, lg, NULL);
    int best = 0;
    for (int v = 1; v < V; v++)
      if (HF(lg[v]) > HF(lg[best])) best = v;
    next[b] = best;
    if (logits) memcpy(logits + (size_t)b * V, lg, sizeof(uint16_t) * (size_t)V);
  }
  free(h);
  free(hn);
  free(lg);
}

/* Prefill of one joining stream ("Per-stream KV-slot isolation ...", section
 * 1: a stream is seeded once, at join): its prompt tokens[0..P-1] go through
 * the model at positions 0..P-1 of its slot, in order, each exactly as one
 * decode step of that stream alone (the causal definition: token t attends
 * to the K/V of tokens 0..t).  The slot then holds the prompt's K/V; the
 * output is the last token's logits fp16 [V] (next-token distribution) and
 * its greedy id.  force [L][P][k]: ranked expert ids replacing every top-k,
 * or NULL; ids_out [L][P][k] and router_out [L][P][E] (fp32 router logits)
 * optional. */
EXPORT void orc_prefill(const orc_model* m, orc_arena* a, int slot, int P, const int32_t* tokens,
                        const int32_t* force, uint16_t* logits, int32_t* next, int32_t* ids_out,
                        float* router_out) {
  h2f_init();
  int H = m->hidden, V = m->vocab, g = m->group, k = m->top_k, L = m->n_layers;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* hn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  for (int t = 0; t < P; t++) {
    embed_row(m, tokens[t], h);
    for (int l = 0; l < L; l++)
      layer_one(m, a, l, slot, t, h, force ? force + ((size_t)l * P + t) * k : NULL,
                ids_out ? ids_out + ((size_t)l * P + t) * k : NULL,
                router_out ? router_out + ((size_t)l * P + t) * m->n_experts : NULL);
  }
  orc_rmsnorm(H, h, m->final_norm, m->rms_eps, hn);
  orc_w4_gemm(1, V, H, g, hn, m->lm_p, m->lm_s, logits, NULL);
  int best = 0;
  for (int v = 1; v < V; v++)
    if (HF(logits[v]) > HF(logits[best])) best = v;
  *next = best;
  free(h);
  free(hn);
}

/* ------------------------------------------------------------------------ */
/* Non-greedy sampling of the next token (beyond the pages' greedy decoding,  */
/* which "Batched-concurrent 4-bit serving on Apple Silicon", section 5,      */
/* names as not validated).  Readings: the usual temperature / top-k / top-p  */
/* (nucleus) sampling, taken in this order:                                   */
/*  1. rank every id by (logit descending, id ascending), NaN ranking as      */
/*     -inf; keep the first top_k;                                            */
/*  2. temperature 0, or top_k 1: the first id (greedy);                      */
/*  3. weights e_r = exp((l_r - l_0) * (1/T)) over the kept ranks, running     */
/*     sums c_r = e_0 + ... + e_r in rank order (fp32);                       */
/*  4. nucleus: the shortest prefix 0..m with c_m >= top_p * c_{k-1};          */
/*  5. the draw u in [0, 1): the first rank r <= m with u * c_m < c_r, else m. */
/* The draw is counter-based, so a stream's samples depend only on its own    */
/* seed and positions: u = (z >> 40) * 2^-24, z the output number pos of the  */
/* SplitMix64 generator started at seed (Steele, Lea and Flood 2014; Vigna's  */
/* splitmix64.c): z = seed + (pos + 1) * 0x9E3779B97F4A7C15, then            */
/* z ^= z >> 30, z *= 0xBF58476D1CE4E5B9, z ^= z >> 27,                       */
/* z *= 0x94D049BB133111EB, z ^= z >> 31.                                     */
/* ------------------------------------------------------------------------ */
EXPORT uint64_t orc_splitmix(uint64_t seed, uint64_t pos) {
  uint64_t z = seed + (pos + 1u) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

EXPORT float orc_draw(uint64_t seed, uint64_t pos) {
  return (float)(orc_splitmix(seed, pos) >> 40) * 0x1p-24f;
}

static float rank_value(uint16_t h) {
  float v = HF(h);
  return v != v ? -INFINITY : v;
}

EXPORT int32_t orc_sample(int V, const uint16_t* logits, float temperature, int top_k, float top_p,
                          uint64_t seed, uint64_t pos) {
  h2f_init();
  int k = top_k < V ? top_k : V;
  if (k < 1) k = 1; /* V >= 1 and top_k >= 1 by contract */
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  unsigned char* taken = (unsigned char*)calloc((size_t)V, 1);
  for (int r = 0; r < k; r++) { /* selection in rank order: larger value, then lower id */
    int best = -1;
    for (int i = 0; i < V; i++) {
      if (taken[i]) continue;
      if (best < 0 || rank_value(logits[i]) > rank_value(logits[best])) best = i;
    }
    taken[best] = 1;
    ids[r] = best;
  }
  int32_t out = ids[0];
  if (temperature > 0.0f && k > 1) {
    float inv_t = 1.0f / temperature;
    float* c = (float*)malloc(sizeof(float) * (size_t)k);
    float l0 = rank_value(logits[ids[0]]);
    float run = 0.0f;
    for (int r = 0; r < k; r++) {
      float e = expf((rank_value(logits[ids[r]]) - l0) * inv_t);
      run = run + e;
      c[r] = run;
    }
    int m = 0;
    float need = top_p * c[k - 1];
    while (m < k - 1 && c[m] < need) m++;
    float t = orc_draw(seed, pos) * c[m];
    int r = 0;
    while (r < m && !(t < c[r])) r++;
    out = ids[r];
    free(c);
  }
  free(ids);
  free(taken);
  return out;
}

/* Attention-only step (slot-indexed GQA decode with a KV append), B streams:
 * q [B][Hq][D], k_new/v_new [B][Hkv][D] are written at positions[b] of
 * slots[b] in layer l, then attention over 0..positions[b] (positions[b] + 1
 * keys) -> o [B][Hq][D].  The slot is the stream's stable KV home ("Per-stream
 * KV-slot isolation for parallel low-bit decode on Apple Silicon", section 1):
 * nothing outside (layer l, slots[b], positions[b]) is written. */
EXPORT void orc_attn_step(const orc_model* m, orc_arena* a, int l, int B, const int32_t* slots,
                          const int32_t* positions, const uint16_t* q, const uint16_t* k_new,
                          const uint16_t* v_new, uint16_t* o) {
  h2f_init();
  int Hq = m->n_q, Hkv = m->n_kv, D = m->head_dim, nkv = Hkv * D;
  for (int b = 0; b < B; b++) {
    size_t off = arena_off(m, a, l, slots[b], positions[b]);
    memcpy(a->k + off, k_new + (size_t)b * nkv, sizeof(uint16_t) * (size_t)nkv);
    memcpy(a->v + off, v_new + (size_t)b * nkv, sizeof(uint16_t) * (size_t)nkv);
    size_t base = arena_off(m, a, l, slots[b], 0);
    orc_attention(Hq, Hkv, D, positions[b] + 1, q + (size_t)b * Hq * D, a->k + base, a->v + base,
                  (int64_t)nkv, o + (size_t)b * Hq * D);
  }
}
