/*
 * qsa_oracle.c -- plain, slow CPU oracle for the Qwen Sparse Attention (QSA)
 * hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no source,
 * header, table or helper with the HIP library, and never calls it.
 *
 * Sources (cited by site and section; all five pages describe the report
 * "On the Design of Qwen3.8-Next Architecture: Evaluation, Efficiency, and
 * Training Stability"):
 *   [hub]   gunjandhanuka.github.io research-hub note, "Key ideas", the
 *           "QSA compressed indexer" bullet: keys average-pooled into blocks
 *           of r, partial RoPE (64 of 128 dims) after compression,
 *           I_ib = sum_h ReLU(<q_i^h, kbar_b>), top-k_B = ceil(K/r) blocks plus
 *           the current-block tail, K = 2048, r = 4.
 *   [glide] paperglide.net reader, section "Qwen Sparse Attention": the toy
 *           walk-through (pool, block-causal scoring, top-K_B, expansion,
 *           incomplete-block tail) and Figure 3 (indexer -> top-k indices ->
 *           micro-block sparse attention mask -> sparse core attention).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - RoPE pairing is rotate-half inside the rotated dims: pair (j, j + R/2),
 *     angle pos * theta^(-2j/R), R = rope_dims, on dims [0, R).
 *   - A pooled key of block b sits at the block's last position (b+1)r-1;
 *     a query sits at its own token position.
 *   - Block b is visible to query i iff (b+1)r-1 <= i, i.e. b < floor((i+1)/r).
 *   - Tail of query i: tokens floor((i+1)/r)*r .. i, always attended.
 *   - Selection: min(k_B, visible) blocks under the total order
 *     (score descending, block id ascending); ids written ascending, -1 pad.
 *   - No scaling and no head weights in the block score; no RMSNorm on the
 *     pooled keys.
 *   - Attention: logits <q, k> * scale, query head h reads KV head
 *     floor(h * hkv / hq); one block selection per token for all heads.
 *
 * Arithmetic: every input element is read as its exact stored value and all
 * arithmetic is in double.  Pooled keys are rounded once, round-to-nearest-
 * even, to the storage type.  Queries are rotated in double and NOT rounded.
 * No blocking, fusion or reordering beyond the definitions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Read element i of an array stored as float32 (dt=0) or bfloat16 (dt=1). */
static double orc_ld(const void* p, int dt, int64_t i) {
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* Round a double to a binary format with `prec` significant bits and minimum
 * normal exponent `emin` (bf16: 8, -126; fp32: 24, -126), round-half-even. */
static double orc_round(double v, int prec, int emin, double maxval) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e); /* |v| = m * 2^e, m in [0.5, 1): leading bit weight 2^(e-1) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  double ulp = ldexp(1.0, lead - (prec - 1));
  double q = nearbyint(v / ulp) * ulp; /* v/ulp is exact: power-of-two scale */
  if (fabs(q) > maxval) q = copysign(INFINITY, v);
  return q;
}

/* Store double v into element i of a float32 or bfloat16 array. */
static void orc_st(void* p, int dt, int64_t i, double v) {
  if (dt == ORC_F32) {
    ((float*)p)[i] = (float)orc_round(v, 24, -126, 3.4028234663852886e38);
    return;
  }
  float f = (float)orc_round(v, 8, -126, 3.3895313892515355e38);
  uint32_t bits;
  memcpy(&bits, &f, 4);
  ((uint16_t*)p)[i] = (uint16_t)(bits >> 16); /* exact: low 16 bits are zero */
}

/* Rotate dims [0, R) of x in place by position pos: pair (j, j + R/2) turns
 * by angle pos * theta^(-2j/R) ([hub]: partial RoPE on 64 of 128 dims). */
static void orc_rope(double* x, int R, double theta, double pos) {
  int half = R / 2;
  for (int j = 0; j < half; ++j) {
    double ang = pos * pow(theta, -2.0 * (double)j / (double)R);
    double c = cos(ang), s = sin(ang);
    double a = x[j], b = x[j + half];
    x[j] = a * c - b * s;
    x[j + half] = a * s + b * c;
  }
}

/* Exposed for the RoPE pins: rotate n rows of d values (double, in place),
 * row t at position pos[t]. */
void orc_rope_rows(double* x, int64_t n, int d, int R, double theta, const int64_t* pos) {
  for (int64_t t = 0; t < n; ++t) orc_rope(x + t * d, R, theta, (double)pos[t]);
}

/* Number of complete blocks visible to the query at position i. */
static int64_t orc_nvis(int64_t i, int r) { return (i + 1) / r; }

/*
 * Pool keys of blocks [b0, b1) ([hub] avg-pool into blocks of r, then partial
 * RoPE after compression; [glide] "block 0 gets (k0+k1)/2").
 *   k_idx: [n_tok][d] in dtype dt_in; kbar_out: [(b1-b0)][d] in dtype dt_out.
 */
void orc_pool(const void* k_idx, int dt_in, int d, int r, int R, double theta,
              int64_t b0, int64_t b1, void* kbar_out, int dt_out) {
  double* m = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t b = b0; b < b1; ++b) {
    for (int c = 0; c < d; ++c) {
      double s = 0.0;
      for (int t = 0; t < r; ++t) s += orc_ld(k_idx, dt_in, (b * r + t) * (int64_t)d + c);
      m[c] = s / (double)r;
    }
    orc_rope(m, R, theta, (double)((b + 1) * r - 1));
    for (int c = 0; c < d; ++c) orc_st(kbar_out, dt_out, (b - b0) * (int64_t)d + c, m[c]);
  }
  free(m);
}

/*
 * Pool keys of blocks [b0, b1) with the block mean RMS-normalised before the
 * rotation ([glide] "Qwen Sparse Attention": the toy average-pools the keys
 * and applies RMSNorm to obtain the compressed keys; [hub]: partial RoPE
 * after the compression):  y_c = m_c * gamma_c / sqrt((1/d) sum_c m_c^2 + eps).
 *   gamma: [d] gain (double); kbar_out: [(b1-b0)][d] in dtype dt_out.
 */
void orc_pool_rmsnorm(const void* k_idx, int dt_in, int d, int r, int R, double theta,
                      int64_t b0, int64_t b1, const double* gamma, double eps, void* kbar_out,
                      int dt_out) {
  double* m = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t b = b0; b < b1; ++b) {
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
      double s = 0.0;
      for (int t = 0; t < r; ++t) s += orc_ld(k_idx, dt_in, (b * r + t) * (int64_t)d + c);
      m[c] = s / (double)r;
      ss += m[c] * m[c];
    }
    double inv = 1.0 / sqrt(ss / (double)d + eps);
    for (int c = 0; c < d; ++c) m[c] = m[c] * gamma[c] * inv;
    orc_rope(m, R, theta, (double)((b + 1) * r - 1));
    for (int c = 0; c < d; ++c) orc_st(kbar_out, dt_out, (b - b0) * (int64_t)d + c, m[c]);
  }
  free(m);
}

/*
 * Block scores of one query ([hub] I_ib = sum_h ReLU(<q_i^h, kbar_b>), MQA:
 * h_idx query heads against one shared key head; [glide] the compressed
 * causal mask: token i scores only the blocks complete by i).
 *   q_row: [h][d] (not rotated), kbar: [>= nvis][d].  scores: [nvis(pos)].
 * Returns the number of visible blocks.
 */
int64_t orc_scores(const void* q_row, const void* kbar, int dt, int h, int d, int r,
                   int R, double theta, int64_t pos, double* scores) {
  double* q = (double*)malloc(sizeof(double) * (size_t)(h * d));
  for (int t = 0; t < h * d; ++t) q[t] = orc_ld(q_row, dt, t);
  for (int hh = 0; hh < h; ++hh) orc_rope(q + hh * d, R, theta, (double)pos);
  int64_t nb = orc_nvis(pos, r);
  for (int64_t b = 0; b < nb; ++b) {
    double s = 0.0;
    for (int hh = 0; hh < h; ++hh) {
      double dot = 0.0;
      for (int c = 0; c < d; ++c) dot += q[hh * d + c] * orc_ld(kbar, dt, b * (int64_t)d + c);
      s += dot > 0.0 ? dot : 0.0;
    }
    scores[b] = s;
  }
  free(q);
  return nb;
}

typedef struct {
  double s;
  int64_t id;
} orc_pair;

/* score descending, then block id ascending */
static int orc_cmp_pair(const void* a, const void* b) {
  const orc_pair* x = (const orc_pair*)a;
  const orc_pair* y = (const orc_pair*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int orc_cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Top-k_B selection ([hub] top-k_B = ceil(K/r) blocks; [glide] "select the
 * top K_B blocks per query").  Full sort, then the first min(kB, nb) ids,
 * written ascending and padded with -1.  Returns the count.
 */
int orc_select(const double* scores, int64_t nb, int kB, int32_t* idx_row) {
  int cnt = (int)(nb < kB ? nb : kB);
  if (nb <= kB) {
    for (int t = 0; t < cnt; ++t) idx_row[t] = t;
  } else {
    orc_pair* p = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)nb);
    for (int64_t b = 0; b < nb; ++b) {
      p[b].s = scores[b];
      p[b].id = b;
    }
    qsort(p, (size_t)nb, sizeof(orc_pair), orc_cmp_pair);
    for (int t = 0; t < cnt; ++t) idx_row[t] = (int32_t)p[t].id;
    free(p);
    qsort(idx_row, (size_t)cnt, sizeof(int32_t), orc_cmp_i32);
  }
  for (int t = cnt; t < kB; ++t) idx_row[t] = -1;
  return cnt;
}

/*
 * Softmax attention of one query over an explicit token list ([glide]
 * Figure 3: sparse core attention over the selected tokens).
 *   q_row: [hq][D]; k, v: [hkv][n_cap][D]; tok: nT token rows.
 *   out: [hq][D] in double.
 */
static void orc_attend_list(const void* q_row, const void* k, const void* v, int dt,
                            int64_t n_cap, const int64_t* tok, int64_t nT, int hq, int hkv, int D,
                            double scale, double* out) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(nT > 0 ? nT : 1));
  for (int h = 0; h < hq; ++h) {
    int g = (int)(((int64_t)h * hkv) / hq);
    const int64_t kv0 = (int64_t)g * n_cap * D;
    double mx = -INFINITY;
    for (int64_t j = 0; j < nT; ++j) {
      double dot = 0.0;
      for (int c = 0; c < D; ++c)
        dot += orc_ld(q_row, dt, (int64_t)h * D + c) * orc_ld(k, dt, kv0 + tok[j] * D + c);
      w[j] = dot * scale;
      if (w[j] > mx) mx = w[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < nT; ++j) {
      w[j] = exp(w[j] - mx);
      z += w[j];
    }
    for (int c = 0; c < D; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < nT; ++j) acc += w[j] * orc_ld(v, dt, kv0 + tok[j] * D + c);
      out[(int64_t)h * D + c] = acc / z;
    }
  }
  free(w);
}

/*
 * Sparse core attention of one query ([glide] Figure 3: selected blocks are
 * expanded to token indices and joined with the incomplete-block tail; each
 * query attends only to that set).
 *   q_row: [hq][D]; k, v: [hkv][n_cap][D]; idx_row: cnt block ids.
 *   out: [hq][D] in double.  Returns |T_i|.
 */
int64_t orc_attend(const void* q_row, const void* k, const void* v, int dt, int64_t n_cap,
                   int64_t pos, const int32_t* idx_row, int cnt, int r, int hq, int hkv,
                   int D, double scale, double* out) {
  int64_t nb = orc_nvis(pos, r);
  int64_t ntail = pos + 1 - nb * r;
  int64_t nT = (int64_t)cnt * r + ntail;
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nT > 0 ? nT : 1));
  int64_t u = 0;
  for (int s = 0; s < cnt; ++s)
    for (int t = 0; t < r; ++t) tok[u++] = (int64_t)idx_row[s] * r + t;
  for (int64_t t = nb * r; t <= pos; ++t) tok[u++] = t;
  orc_attend_list(q_row, k, v, dt, n_cap, tok, nT, hq, hkv, D, scale, out);
  free(tok);
  return nT;
}

/*
 * Attention of one new token of a decode step whose new tokens share one
 * block selection ([glide] "QSA Ablations and Efficiency": the top-k indices
 * are reused across speculative decoding steps).  The selection (idx_row,
 * cnt) was made at position f, the step's first new token; the token at
 * position pos >= f attends to the selected blocks' tokens and to every
 * token from floor((f+1)/r)*r to pos (its incomplete block and the blocks
 * completed after f, which the selection could not score).  Returns |T|.
 */
int64_t orc_attend_shared(const void* q_row, const void* k, const void* v, int dt,
                          int64_t n_cap, int64_t f, int64_t pos, const int32_t* idx_row, int cnt,
                          int r, int hq, int hkv, int D, double scale, double* out) {
  int64_t start = orc_nvis(f, r) * r;
  int64_t nT = (int64_t)cnt * r + (pos + 1 - start);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nT > 0 ? nT : 1));
  int64_t u = 0;
  for (int s = 0; s < cnt; ++s)
    for (int t = 0; t < r; ++t) tok[u++] = (int64_t)idx_row[s] * r + t;
  for (int64_t t = start; t <= pos; ++t) tok[u++] = t;
  orc_attend_list(q_row, k, v, dt, n_cap, tok, nT, hq, hkv, D, scale, out);
  free(tok);
  return nT;
}

/*
 * Indexer for a list of query rows of one sequence: scores + selection.
 *   q_idx: [n_q][h][d] raw, row t at position pos0 + t; kbar: [nb_cap][d].
 *   rows: which t to compute.  idx: [nrows][kB], cnt: [nrows].
 * OpenMP over rows.
 */
void orc_index_rows(const void* q_idx, const void* kbar, int dt, int h, int d, int r, int R,
                    double theta, int kB, int64_t pos0, const int64_t* rows, int64_t nrows,
                    int32_t* idx, int32_t* cnt) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < nrows; ++u) {
    int64_t t = rows[u];
    int64_t pos = pos0 + t;
    int64_t nb = orc_nvis(pos, r);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    const char* qrow = (const char*)q_idx + (size_t)t * h * d * (dt == ORC_F32 ? 4 : 2);
    orc_scores(qrow, kbar, dt, h, d, r, R, theta, pos, sc);
    cnt[u] = orc_select(sc, nb, kB, idx + u * kB);
    free(sc);
  }
}

/* Scores of listed rows (for near-tie analysis in the tests): scores row u is
 * written at out + u * stride, nb(pos0 + rows[u]) values. */
void orc_score_rows(const void* q_idx, const void* kbar, int dt, int h, int d, int r, int R,
                    double theta, int64_t pos0, const int64_t* rows, int64_t nrows,
                    double* out, int64_t stride) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < nrows; ++u) {
    int64_t t = rows[u];
    const char* qrow = (const char*)q_idx + (size_t)t * h * d * (dt == ORC_F32 ? 4 : 2);
    orc_scores(qrow, kbar, dt, h, d, r, R, theta, pos0 + t, out + u * stride);
  }
}

/*
 * Attention for a list of query rows of one sequence, given their block
 * selections.  q: [n_q][hq][D], row t at position pos0 + t; k, v:
 * [hkv][n_cap][D]; idx: [nrows][kB]; cnt: [nrows]; out: [nrows][hq][D].
 */
void orc_attend_rows(const void* q, const void* k, const void* v, int dt, int64_t n_cap,
                     int64_t pos0, const int64_t* rows, int64_t nrows, const int32_t* idx,
                     const int32_t* cnt, int kB, int r, int hq, int hkv, int D, double scale,
                     double* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < nrows; ++u) {
    int64_t t = rows[u];
    const char* qrow = (const char*)q + (size_t)t * hq * D * (dt == ORC_F32 ? 4 : 2);
    orc_attend(qrow, k, v, dt, n_cap, pos0 + t, idx + u * kB, cnt[u], r, hq, hkv, D, scale,
               out + u * (int64_t)hq * D);
  }
}

/*
 * The same three steps for query rows given with explicit positions: row u
 * of q_rows (h x d indexer values, or hq x D attention values) sits at token
 * position pos[u].  Used where only a sample of a long sequence's rows is
 * checked.  OpenMP over rows.
 */
void orc_index_at(const void* q_rows, const void* kbar, int dt, int h, int d, int r, int R,
                  double theta, int kB, const int64_t* pos, int64_t nrows, int32_t* idx,
                  int32_t* cnt) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < nrows; ++u) {
    int64_t nb = orc_nvis(pos[u], r);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    const char* qrow = (const char*)q_rows + (size_t)u * h * d * (dt == ORC_F32 ? 4 : 2);
    orc_scores(qrow, kbar, dt, h, d, r, R, theta, pos[u], sc);
    cnt[u] = orc_select(sc, nb, kB, idx + u * kB);
    free(sc);
  }
}

void orc_score_at(const void* q_rows, const void* kbar, int dt, int h, int d, int r, int R,
                  double theta, const int64_t* pos, int64_t nrows, double* out, int64_t stride) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < nrows; ++u) {
    const char* qrow = (const char*)q_rows + (size_t)u * h * d * (dt == ORC_F32 ? 4 : 2);
    orc_scores(qrow, kbar, dt, h, d, r, R, theta, pos[u], out + u * stride);
  }
}

void orc_attend_at(const void* q_rows, const void* k, const void* v, int dt, int64_t n_cap,
                   const int64_t* pos, int64_t nrows, const int32_t* idx, const int32_t* cnt,
                   int kB, int r, int hq, int hkv, int D, double scale, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < nrows; ++u) {
    const char* qrow = (const char*)q_rows + (size_t)u * hq * D * (dt == ORC_F32 ? 4 : 2);
    orc_attend(qrow, k, v, dt, n_cap, pos[u], idx + u * kB, cnt[u], r, hq, hkv, D, scale,
               out + u * (int64_t)hq * D);
  }
}

/* ------------------------------------------------------------------------
 * Training path ([hub] "Key ideas", native-trainability bullet: stage 1
 * distils the indexer -- KL divergence of its block scores to the teacher's
 * block-max-pooled dense attention, the indexer trained alone -- and stage 2
 * trains it jointly with the sparse attention).
 * ------------------------------------------------------------------------ */

/*
 * Backward of the sparse core attention of one query row: given the upstream
 * gradient dout_row [hq][D] of out_row, accumulate dq_row [hq][D] (written)
 * and dk_acc, dv_acc [hkv][n_cap][D] (added to) in double.  The selection is
 * not differentiated (a discrete choice).  With P the softmax weights over
 * T_i, dP_j = <dout, v_j>, Dsum = sum_j P_j dP_j, dS_j = P_j (dP_j - Dsum):
 * dq = scale sum_j dS_j k_j, dk_j += scale dS_j q, dv_j += P_j dout.
 */
void orc_attend_backward(const void* q_row, const void* k, const void* v, int dt, int64_t n_cap,
                         int64_t pos, const int32_t* idx_row, int cnt, int r, int hq, int hkv,
                         int D, double scale, const double* dout_row, double* dq_row,
                         double* dk_acc, double* dv_acc) {
  int64_t nb = orc_nvis(pos, r);
  int64_t nT = (int64_t)cnt * r + (pos + 1 - nb * r);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nT > 0 ? nT : 1));
  double* w = (double*)malloc(sizeof(double) * (size_t)(nT > 0 ? nT : 1));
  double* dp = (double*)malloc(sizeof(double) * (size_t)(nT > 0 ? nT : 1));
  int64_t u = 0;
  for (int s = 0; s < cnt; ++s)
    for (int t = 0; t < r; ++t) tok[u++] = (int64_t)idx_row[s] * r + t;
  for (int64_t t = nb * r; t <= pos; ++t) tok[u++] = t;
  for (int h = 0; h < hq; ++h) {
    int g = (int)(((int64_t)h * hkv) / hq);
    const int64_t kv0 = (int64_t)g * n_cap * D;
    double mx = -INFINITY;
    for (int64_t j = 0; j < nT; ++j) {
      double dot = 0.0;
      for (int c = 0; c < D; ++c)
        dot += orc_ld(q_row, dt, (int64_t)h * D + c) * orc_ld(k, dt, kv0 + tok[j] * D + c);
      w[j] = dot * scale;
      if (w[j] > mx) mx = w[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < nT; ++j) {
      w[j] = exp(w[j] - mx);
      z += w[j];
    }
    double dsum = 0.0;
    for (int64_t j = 0; j < nT; ++j) {
      w[j] /= z;
      double d = 0.0;
      for (int c = 0; c < D; ++c) d += dout_row[(int64_t)h * D + c] * orc_ld(v, dt, kv0 + tok[j] * D + c);
      dp[j] = d;
      dsum += w[j] * d;
    }
    for (int c = 0; c < D; ++c) dq_row[(int64_t)h * D + c] = 0.0;
    for (int64_t j = 0; j < nT; ++j) {
      double ds = w[j] * (dp[j] - dsum);
      for (int c = 0; c < D; ++c) {
        dq_row[(int64_t)h * D + c] += scale * ds * orc_ld(k, dt, kv0 + tok[j] * D + c);
        dk_acc[kv0 + tok[j] * D + c] += scale * ds * orc_ld(q_row, dt, (int64_t)h * D + c);
        dv_acc[kv0 + tok[j] * D + c] += w[j] * dout_row[(int64_t)h * D + c];
      }
    }
  }
  free(tok);
  free(w);
  free(dp);
}

/*
 * Indexer distillation of one query row at position pos (stage 1).
 *   teacher: dense causal attention of the row, p_j^h = softmax over j <= pos
 *            of scale <q^h, k_j^{g(h)}>; block b's weight is the largest
 *            head-summed probability among its r tokens,
 *            a_b = max_{t<r} sum_h p_{br+t}^h, for the visible blocks
 *            b < nb(pos); teacher distribution t_b = a_b / sum_b a_b;
 *   student: s_b = softmax over the visible b of I_b = sum_h ReLU(<q~^h, kbar_b>)
 *            (q~ = q_idx rotated at pos, kbar as stored);
 *   loss:    KL(t || s) = sum_b t_b (ln t_b - ln s_b)  (0 when nb(pos) = 0).
 * Gradients (teacher held fixed): with g_b = s_b - t_b,
 *   dq~^h = sum_b g_b [<q~^h, kbar_b> > 0] kbar_b -> dq_idx_row = its rotation
 *   back (angle -pos), written; dkbar_acc[b] += g_b sum_h [...] q~^h.
 * Returns the row's loss.
 */
double orc_distill_row(const void* q_row, const void* k, int dt, int64_t n_cap, int hq,
                       int hkv, int D, double scale, const void* q_idx_row, const void* kbar,
                       int h, int d, int r, int R, double theta, int64_t pos,
                       double* dq_idx_row, double* dkbar_acc, double* g_out) {
  int64_t nb = orc_nvis(pos, r);
  for (int c = 0; c < h * d; ++c) dq_idx_row[c] = 0.0;
  if (nb == 0) return 0.0;
  int64_t n = pos + 1;
  /* teacher: head-summed probabilities of tokens 0..pos */
  double* ps = (double*)calloc((size_t)n, sizeof(double));
  double* w = (double*)malloc(sizeof(double) * (size_t)n);
  for (int hh = 0; hh < hq; ++hh) {
    int g = (int)(((int64_t)hh * hkv) / hq);
    const int64_t kv0 = (int64_t)g * n_cap * D;
    double mx = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int c = 0; c < D; ++c)
        dot += orc_ld(q_row, dt, (int64_t)hh * D + c) * orc_ld(k, dt, kv0 + j * D + c);
      w[j] = dot * scale;
      if (w[j] > mx) mx = w[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      w[j] = exp(w[j] - mx);
      z += w[j];
    }
    for (int64_t j = 0; j < n; ++j) ps[j] += w[j] / z;
  }
  double* a = (double*)malloc(sizeof(double) * (size_t)nb);
  double asum = 0.0;
  for (int64_t b = 0; b < nb; ++b) {
    double m = ps[b * r];
    for (int t = 1; t < r; ++t)
      if (ps[b * r + t] > m) m = ps[b * r + t];
    a[b] = m;
    asum += m;
  }
  /* student */
  double* q = (double*)malloc(sizeof(double) * (size_t)(h * d));
  for (int c = 0; c < h * d; ++c) q[c] = orc_ld(q_idx_row, dt, c);
  for (int hh = 0; hh < h; ++hh) orc_rope(q + hh * d, R, theta, (double)pos);
  double* I = (double*)malloc(sizeof(double) * (size_t)nb);
  unsigned char* pos_dot = (unsigned char*)malloc((size_t)(nb * h));
  double imax = -INFINITY;
  for (int64_t b = 0; b < nb; ++b) {
    double s = 0.0;
    for (int hh = 0; hh < h; ++hh) {
      double dot = 0.0;
      for (int c = 0; c < d; ++c) dot += q[hh * d + c] * orc_ld(kbar, dt, b * (int64_t)d + c);
      pos_dot[b * h + hh] = dot > 0.0;
      s += dot > 0.0 ? dot : 0.0;
    }
    I[b] = s;
    if (s > imax) imax = s;
  }
  double zs = 0.0;
  for (int64_t b = 0; b < nb; ++b) zs += exp(I[b] - imax);
  double lz = imax + log(zs); /* ln sum_b exp(I_b) */
  double loss = 0.0;
  double* dq = (double*)calloc((size_t)(h * d), sizeof(double));
  for (int64_t b = 0; b < nb; ++b) {
    double t = a[b] / asum;
    double ls = I[b] - lz;
    if (t > 0.0) loss += t * (log(t) - ls);
    double gb = exp(ls) - t;
    if (g_out) g_out[b] = gb; /* d loss / d I_b, for callers that need it */
    for (int hh = 0; hh < h; ++hh) {
      if (!pos_dot[b * h + hh]) continue;
      for (int c = 0; c < d; ++c) {
        dq[hh * d + c] += gb * orc_ld(kbar, dt, b * (int64_t)d + c);
        dkbar_acc[b * (int64_t)d + c] += gb * q[hh * d + c];
      }
    }
  }
  /* back through the rotation: rotate by -pos */
  for (int hh = 0; hh < h; ++hh) orc_rope(dq + hh * d, R, theta, -(double)pos);
  for (int c = 0; c < h * d; ++c) dq_idx_row[c] = dq[c];
  free(ps);
  free(w);
  free(a);
  free(q);
  free(I);
  free(pos_dot);
  free(dq);
  return loss;
}

/*
 * Backward of the pooling (orc_pool): the gradient of the raw indexer keys
 * of blocks [b0, b1) given the gradient dkbar [(b1-b0)][d] of the pooled
 * keys: each of the block's r keys receives (1/r) times dkbar rotated back
 * (angle -(b+1)r+1).  dk_out: [(b1-b0) r][d], written.
 */
void orc_pool_backward(const double* dkbar, int d, int r, int R, double theta, int64_t b0,
                       int64_t b1, double* dk_out) {
  double* m = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t b = b0; b < b1; ++b) {
    for (int c = 0; c < d; ++c) m[c] = dkbar[(b - b0) * (int64_t)d + c];
    orc_rope(m, R, theta, -(double)((b + 1) * r - 1));
    for (int t = 0; t < r; ++t)
      for (int c = 0; c < d; ++c) dk_out[((b - b0) * r + t) * (int64_t)d + c] = m[c] / (double)r;
  }
  free(m);
}
