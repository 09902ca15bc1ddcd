/*
 * CPU oracle for Speed3R's dual-branch sparse global attention (forward pass).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls this file: only
 * the test suite, the smoke check and the CPU-baseline leg of the benchmark do. It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it computes, step by step, in float64 from float32 copies of the bf16 inputs:
 *
 *  Method (Speed3R paper summary on gist.science, "Technische samenvatting / Methodologie":
 *  section 1 "Dual-Branch Attention Mechanisme", section 2 "Gated Aggregation"; project README
 *  "Overview"):
 *   1. Compression branch: the key and value tokens are cut into contiguous blocks of B tokens
 *      (the last block may be shorter) and each block is average-pooled into one coarse token.
 *   2. Every query attends with softmax to all coarse tokens; that attention gives the
 *      compression output and, summed over the queries of a query block, a score for each
 *      (query block, key block) pair.
 *   3. Selection branch: per query block the k key blocks with the highest score are chosen, and
 *      each query of the block runs exact softmax attention over the tokens of those blocks.
 *   4. Gated aggregation: per head, out = g_cmp * O_cmp + g_sel * O_sel.
 *
 *  Readings where the pages are silent (each also listed in the design notes):
 *   - blocks are contiguous over the flattened token order, query blocks = key blocks = B;
 *   - a short last block is pooled over its real tokens only;
 *   - softmax scale is 1/sqrt(D) in both branches unless given;
 *   - the block score is the sum over the block's queries of the normalised compressed
 *     attention probabilities;
 *   - top-k is taken per head, ties go to the smaller block index, indices are returned in
 *     ascending order, k is clamped to the number of blocks;
 *   - optional forced blocks (the VGGT variant keeps the reference frame's tokens dense,
 *     summary "Methodologie" 3): the first F key blocks are always selected and top-k is taken
 *     over the remaining blocks, so a row holds min(F, Nb) + min(k, Nb - min(F, Nb)) blocks;
 *     optionally each query block's own key block is always selected as well (top-k then runs
 *     over the blocks that are neither forced nor its own);
 *   - the top-k decision is made on the scores rounded to float32 (the precision the GPU
 *     kernel decides in);
 *   - no masking (bidirectional attention).
 *
 *  Backward pass (trainable sparse attention: the arXiv abstract and the README call the model
 *  end-to-end trainable): s3r_oracle_backward differentiates the forward above with the
 *  selection held fixed (top-k is piecewise constant, so no gradient flows through the block
 *  scores), by the chain rule through each step: gated sum, both softmax attentions, and the
 *  block means.
 *
 * Layout conventions: a token tensor x is addressed as x[t*st + h*sh + d] (float32), pooled
 * tensors as p[(h*Nb + j)*D + d] (float64). All outputs are caller-allocated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int64_t n_blocks(int64_t T, int32_t B) { return (T + B - 1) / B; }

static int64_t block_len(int64_t T, int32_t B, int64_t j) {
  int64_t end = (j + 1) * (int64_t)B;
  if (end > T) end = T;
  return end - j * (int64_t)B;
}

/* Step 1: mean over each contiguous block of B tokens (short last block: mean over its own
 * tokens). Sum in float64, then divide. out is [H][Nb][D]. */
void s3r_oracle_pool(int64_t T, int32_t H, int32_t D, int32_t B, const float* x, int64_t st,
                     int64_t sh, double* out) {
  const int64_t Nb = n_blocks(T, B);
#pragma omp parallel for collapse(2) schedule(static)
  for (int32_t h = 0; h < H; ++h) {
    for (int64_t j = 0; j < Nb; ++j) {
      const int64_t n = block_len(T, B, j);
      for (int32_t d = 0; d < D; ++d) {
        double s = 0.0;
        for (int64_t t = j * B; t < j * B + n; ++t) s += (double)x[t * st + h * sh + d];
        out[((int64_t)h * Nb + j) * D + d] = s / (double)n;
      }
    }
  }
}

/* Step 2 for one head h and one query block i: logits c_tj = scale * q_t . Kc_j over all
 * coarse tokens j, log-sum-exp L_t, probabilities P_tj = exp(c_tj - L_t), compressed output
 * O_cmp_t = sum_j P_tj Vc_j and block scores S_j = sum_{t in block i} P_tj.
 * lse: [n_i], ocmp: [n_i][D], score: [Nb]. */
void s3r_oracle_cmp_row(int64_t T, int32_t H, int32_t D, int32_t B, double scale,
                        const float* q, int64_t qst, int64_t qsh, const double* kc,
                        const double* vc, int32_t h, int64_t i, double* lse, double* ocmp,
                        double* score) {
  const int64_t Nb = n_blocks(T, B);
  if (h < 0 || h >= H || i < 0 || i >= Nb) return;
  const int64_t n_i = block_len(T, B, i);
  double* c = (double*)malloc(sizeof(double) * (size_t)Nb);
  for (int64_t j = 0; j < Nb; ++j) score[j] = 0.0;
  for (int64_t a = 0; a < n_i; ++a) {
    const int64_t t = i * B + a;
    const float* qt = q + t * qst + h * qsh;
    double m = -INFINITY;
    for (int64_t j = 0; j < Nb; ++j) {
      const double* kj = kc + ((int64_t)h * Nb + j) * D;
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += (double)qt[d] * kj[d];
      c[j] = scale * dot;
      if (c[j] > m) m = c[j];
    }
    double s = 0.0;
    for (int64_t j = 0; j < Nb; ++j) s += exp(c[j] - m);
    const double L = m + log(s);
    lse[a] = L;
    double* o = ocmp + a * D;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < Nb; ++j) {
      const double p = exp(c[j] - L);
      score[j] += p;
      const double* vj = vc + ((int64_t)h * Nb + j) * D;
      for (int32_t d = 0; d < D; ++d) o[d] += p * vj[d];
    }
  }
  free(c);
}

typedef struct {
  float v;
  int64_t j;
} scored;

static int by_score_desc_index_asc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j) ? 1 : 0;
}

static int int32_asc(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x < y) ? -1 : (x > y) ? 1 : 0;
}

/* Step 3a: the k largest of score[0..n) by (score descending, index ascending), written in
 * ascending index order. k is clamped to n. Returns the number written. */
int32_t s3r_oracle_topk(const float* score, int64_t n, int32_t k, int32_t* sel) {
  const int64_t k_eff = (k < n) ? k : n;
  scored* all = (scored*)malloc(sizeof(scored) * (size_t)n);
  for (int64_t j = 0; j < n; ++j) {
    all[j].v = score[j];
    all[j].j = j;
  }
  qsort(all, (size_t)n, sizeof(scored), by_score_desc_index_asc);
  for (int64_t a = 0; a < k_eff; ++a) sel[a] = (int32_t)all[a].j;
  qsort(sel, (size_t)k_eff, sizeof(int32_t), int32_asc);
  free(all);
  return (int32_t)k_eff;
}

/* Step 3b for one head h and one query block i: every query of the block attends with
 * softmax to the tokens of the union of the listed key blocks (a block listed twice counts
 * once). osel: [n_i][D]. */
void s3r_oracle_sel_row(int64_t T, int32_t H, int32_t D, int32_t B, double scale, const float* q,
                        int64_t qst, int64_t qsh, const float* k, int64_t kst, int64_t ksh,
                        const float* v, int64_t vst, int64_t vsh, int32_t h, int64_t i,
                        const int32_t* sel, int32_t nsel, double* osel) {
  const int64_t Nb = n_blocks(T, B);
  if (h < 0 || h >= H || i < 0 || i >= Nb) return;
  const int64_t n_i = block_len(T, B, i);
  char* chosen = (char*)calloc((size_t)Nb, 1);
  int64_t n_u = 0;
  for (int32_t a = 0; a < nsel; ++a) {
    const int64_t j = sel[a];
    if (j >= 0 && j < Nb && !chosen[j]) {
      chosen[j] = 1;
      n_u += block_len(T, B, j);
    }
  }
  int64_t* u_tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_u > 0 ? n_u : 1));
  int64_t w = 0;
  for (int64_t j = 0; j < Nb; ++j)
    if (chosen[j])
      for (int64_t t = j * B; t < j * B + block_len(T, B, j); ++t) u_tok[w++] = t;
  double* c = (double*)malloc(sizeof(double) * (size_t)(n_u > 0 ? n_u : 1));
  for (int64_t a = 0; a < n_i; ++a) {
    const float* qt = q + (i * B + a) * qst + h * qsh;
    double m = -INFINITY;
    for (int64_t u = 0; u < n_u; ++u) {
      const float* ku = k + u_tok[u] * kst + h * ksh;
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += (double)qt[d] * (double)ku[d];
      c[u] = scale * dot;
      if (c[u] > m) m = c[u];
    }
    double s = 0.0;
    for (int64_t u = 0; u < n_u; ++u) s += exp(c[u] - m);
    double* o = osel + a * D;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t u = 0; u < n_u; ++u) {
      const double p = exp(c[u] - m) / s;
      const float* vu = v + u_tok[u] * vst + h * vsh;
      for (int32_t d = 0; d < D; ++d) o[d] += p * (double)vu[d];
    }
  }
  free(c);
  free(u_tok);
  free(chosen);
}

/* Plain softmax attention of queries t0..t0+nt-1 (head h) over all T keys. out: [nt][D]. */
void s3r_oracle_dense_rows(int64_t T, int32_t H, int32_t D, double scale, const float* q,
                           int64_t qst, int64_t qsh, const float* k, int64_t kst, int64_t ksh,
                           const float* v, int64_t vst, int64_t vsh, int32_t h, int64_t t0,
                           int64_t nt, double* out) {
  if (h < 0 || h >= H || t0 < 0 || t0 + nt > T) return;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t a = 0; a < nt; ++a) {
    double* c = (double*)malloc(sizeof(double) * (size_t)T);
    const float* qt = q + (t0 + a) * qst + h * qsh;
    double m = -INFINITY;
    for (int64_t u = 0; u < T; ++u) {
      const float* ku = k + u * kst + h * ksh;
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += (double)qt[d] * (double)ku[d];
      c[u] = scale * dot;
      if (c[u] > m) m = c[u];
    }
    double s = 0.0;
    for (int64_t u = 0; u < T; ++u) s += exp(c[u] - m);
    double* o = out + a * D;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t u = 0; u < T; ++u) {
      const double p = exp(c[u] - m) / s;
      const float* vu = v + u * vst + h * vsh;
      for (int32_t d = 0; d < D; ++d) o[d] += p * (double)vu[d];
    }
    free(c);
  }
}

/* Length of a selection row: the forced prefix, the query block's own block when `own` asks
 * for it (and it is not forced already), plus top-k of the rest. Rows whose own block lies in
 * the prefix hold one block fewer and end with -1. */
int32_t s3r_oracle_num_selected(int64_t T, int32_t B, int32_t topk, int32_t forced,
                                int32_t own) {
  const int64_t Nb = n_blocks(T, B);
  const int64_t f = (forced < Nb) ? forced : Nb;
  const int64_t o = (own && f < Nb) ? 1 : 0;
  const int64_t rest = Nb - f - o;
  return (int32_t)(f + o + ((topk < rest) ? topk : rest));
}

static int int32_asc_sel(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Selection row of query block i: blocks 0..f-1, then (own) block i, then the top-k of the
 * remaining blocks by f32 score, all in ascending order, padded with -1 to n_sel. */
static void select_row(const float* score, int64_t Nb, int64_t i, int32_t f, int32_t own,
                       int32_t topk, int32_t n_sel, int32_t* out) {
  int32_t n = 0;
  for (int32_t a = 0; a < f; ++a) out[n++] = a;
  const int own_here = own && i >= f;
  if (own_here) out[n++] = (int32_t)i;
  /* candidates: blocks f..Nb-1 except i */
  float* cs = (float*)malloc(sizeof(float) * (size_t)(Nb > 0 ? Nb : 1));
  int32_t* cj = (int32_t*)malloc(sizeof(int32_t) * (size_t)(Nb > 0 ? Nb : 1));
  int32_t* pick = (int32_t*)malloc(sizeof(int32_t) * (size_t)(Nb > 0 ? Nb : 1));
  int64_t nc = 0;
  for (int64_t j = f; j < Nb; ++j) {
    if (own_here && j == i) continue;
    cs[nc] = score[j];
    cj[nc] = (int32_t)j;
    ++nc;
  }
  if (nc > 0) {
    const int32_t got = s3r_oracle_topk(cs, nc, topk, pick);
    for (int32_t a = 0; a < got; ++a) out[n++] = cj[pick[a]];
  }
  qsort(out, (size_t)n, sizeof(int32_t), int32_asc_sel);
  while (n < n_sel) out[n++] = -1;
  free(cs);
  free(cj);
  free(pick);
}

/* The whole forward pass for a list of (head, query block) rows, given the pooled tensors.
 * Per row r (B_ = B, n_i <= B rows of each per-query output are written):
 *   lse[r][B][1], ocmp[r][B][D], score[r][Nb] (float32, the values top-k decides on),
 *   sel[r][n_sel], osel[r][B][D], out[r][B][D], n_sel = s3r_oracle_num_selected().
 * If sel_in is not NULL it supplies the selected blocks ([r][n_sel]) instead of top-k.
 * Gate of (t, h, branch b) is gates[t*gate_st + h*2 + b] (gate_st = 0: per-head gates). */
void s3r_oracle_forward_rows(int64_t T, int32_t H, int32_t D, int32_t B, int32_t topk,
                             int32_t forced, int32_t own, double scale, const float* q, int64_t qst, int64_t qsh,
                             const float* k, int64_t kst, int64_t ksh, const float* v,
                             int64_t vst, int64_t vsh, const double* kc, const double* vc,
                             const float* gates, int64_t gate_st, int64_t n_rows,
                             const int32_t* row_h, const int64_t* row_i, const int32_t* sel_in,
                             double* lse, double* ocmp, float* score, int32_t* sel,
                             double* osel, double* out) {
  const int64_t Nb = n_blocks(T, B);
  const int32_t k_eff = s3r_oracle_num_selected(T, B, topk, forced, own);
  const int32_t f = (int32_t)((forced < Nb) ? forced : Nb);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int32_t h = row_h[r];
    const int64_t i = row_i[r];
    const int64_t n_i = block_len(T, B, i);
    double* s64 = (double*)malloc(sizeof(double) * (size_t)Nb);
    double* my_lse = lse + r * B;
    double* my_ocmp = ocmp + r * B * D;
    s3r_oracle_cmp_row(T, H, D, B, scale, q, qst, qsh, kc, vc, h, i, my_lse, my_ocmp, s64);
    float* my_score = score + r * Nb;
    for (int64_t j = 0; j < Nb; ++j) my_score[j] = (float)s64[j];
    int32_t* my_sel = sel + r * k_eff;
    if (sel_in) {
      memcpy(my_sel, sel_in + r * k_eff, sizeof(int32_t) * (size_t)k_eff);
    } else {
      select_row(my_score, Nb, i, f, own, topk, k_eff, my_sel);
    }
    double* my_osel = osel + r * B * D;
    s3r_oracle_sel_row(T, H, D, B, scale, q, qst, qsh, k, kst, ksh, v, vst, vsh, h, i, my_sel,
                       k_eff, my_osel);
    double* my_out = out + r * B * D;
    for (int64_t a = 0; a < n_i; ++a) {
      const int64_t t = i * B + a;
      const double g_cmp = gates[t * gate_st + h * 2 + 0];
      const double g_sel = gates[t * gate_st + h * 2 + 1];
      for (int32_t d = 0; d < D; ++d)
        my_out[a * D + d] = g_cmp * my_ocmp[a * D + d] + g_sel * my_osel[a * D + d];
    }
    free(s64);
  }
}

int s3r_oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the OpenMP loops over independent rows use from now on (timing at one thread and at
 * every core); the results do not depend on it. */
void s3r_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}

/* Gradient of the forward pass for one head h, with the selection sel ([Nb][nsel]) fixed.
 * dout is the gradient of out ([T][H][D] addressed like the inputs, dst/dsh); dq, dk, dv are
 * [T][H][D] (contiguous, only head h written, zero them first); dgate is [T][2] for per-token
 * gates (gate_st != 0) or [2] for per-head gates, accumulated.
 *   out_t      = g0 O_cmp_t + g1 O_sel_t
 *   compression: c_tj = scale q_t.Kc_j, P = softmax_j, O_cmp_t = sum_j P_tj Vc_j
 *     dO = g0 dout_t;  dg0 += dout_t.O_cmp_t;  dVc_j += P_tj dO;  dP_tj = dO.Vc_j
 *     dc_tj = P_tj (dP_tj - sum_j' P_tj' dP_tj');  dq_t += scale sum_j dc_tj Kc_j;
 *     dKc_j += scale dc_tj q_t;  then every token of block j gets dKc_j / n_j, dVc_j / n_j.
 *   selection (tokens u of the union of the selected blocks): the same with k_u, v_u, g1. */
void s3r_oracle_backward_head(int64_t T, int32_t H, int32_t D, int32_t B, double scale,
                              const float* q, int64_t qst, int64_t qsh, const float* k,
                              int64_t kst, int64_t ksh, const float* v, int64_t vst, int64_t vsh,
                              const float* gates, int64_t gate_st, const float* dout,
                              int64_t dst, int64_t dsh, const int32_t* sel, int32_t nsel,
                              int32_t h, double* dq, double* dk, double* dv, double* dgate) {
  const int64_t Nb = n_blocks(T, B);
  double* kc = (double*)calloc((size_t)(Nb * D), sizeof(double));
  double* vc = (double*)calloc((size_t)(Nb * D), sizeof(double));
  double* dkc = (double*)calloc((size_t)(Nb * D), sizeof(double));
  double* dvc = (double*)calloc((size_t)(Nb * D), sizeof(double));
  double* c = (double*)malloc(sizeof(double) * (size_t)(T > Nb ? T : Nb));
  double* dp = (double*)malloc(sizeof(double) * (size_t)(T > Nb ? T : Nb));
  int64_t* u_tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)T);
  char* chosen = (char*)malloc((size_t)Nb);
  /* block means of this head */
  for (int64_t j = 0; j < Nb; ++j) {
    const int64_t n = block_len(T, B, j);
    for (int32_t d = 0; d < D; ++d) {
      double sk = 0.0, sv = 0.0;
      for (int64_t t = j * B; t < j * B + n; ++t) {
        sk += (double)k[t * kst + h * ksh + d];
        sv += (double)v[t * vst + h * vsh + d];
      }
      kc[j * D + d] = sk / (double)n;
      vc[j * D + d] = sv / (double)n;
    }
  }
  for (int64_t t = 0; t < T; ++t) {
    const float* qt = q + t * qst + h * qsh;
    const float* gt = dout + t * dst + h * dsh;
    const double g0 = gates[t * gate_st + h * 2 + 0];
    const double g1 = gates[t * gate_st + h * 2 + 1];
    double* dqt = dq + (t * H + h) * D;
    double* dg = dgate + (gate_st ? t * 2 : 0);
    /* ---- compression branch ---- */
    double m = -INFINITY;
    for (int64_t j = 0; j < Nb; ++j) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += (double)qt[d] * kc[j * D + d];
      c[j] = scale * dot;
      if (c[j] > m) m = c[j];
    }
    double ssum = 0.0;
    for (int64_t j = 0; j < Nb; ++j) ssum += exp(c[j] - m);
    double delta = 0.0, go = 0.0;
    for (int64_t j = 0; j < Nb; ++j) {
      const double p = exp(c[j] - m) / ssum;
      c[j] = p;
      double dpj = 0.0, oj = 0.0;
      for (int32_t d = 0; d < D; ++d) {
        dpj += g0 * (double)gt[d] * vc[j * D + d];
        oj += (double)gt[d] * vc[j * D + d];
      }
      dp[j] = dpj;
      delta += p * dpj;
      go += p * oj; /* dout_t . O_cmp_t */
      for (int32_t d = 0; d < D; ++d) dvc[j * D + d] += p * g0 * (double)gt[d];
    }
    dg[0] += go;
    for (int64_t j = 0; j < Nb; ++j) {
      const double dcj = c[j] * (dp[j] - delta);
      for (int32_t d = 0; d < D; ++d) {
        dqt[d] += scale * dcj * kc[j * D + d];
        dkc[j * D + d] += scale * dcj * (double)qt[d];
      }
    }
    /* ---- selection branch over the union of the selected blocks of t's query block ---- */
    const int64_t i = t / B;
    memset(chosen, 0, (size_t)Nb);
    for (int32_t a = 0; a < nsel; ++a) {
      const int64_t j = sel[i * nsel + a];
      if (j >= 0 && j < Nb) chosen[j] = 1;
    }
    int64_t n_u = 0;
    for (int64_t j = 0; j < Nb; ++j)
      if (chosen[j])
        for (int64_t u = j * B; u < j * B + block_len(T, B, j); ++u) u_tok[n_u++] = u;
    m = -INFINITY;
    for (int64_t a = 0; a < n_u; ++a) {
      const float* ku = k + u_tok[a] * kst + h * ksh;
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += (double)qt[d] * (double)ku[d];
      c[a] = scale * dot;
      if (c[a] > m) m = c[a];
    }
    ssum = 0.0;
    for (int64_t a = 0; a < n_u; ++a) ssum += exp(c[a] - m);
    delta = 0.0;
    go = 0.0;
    for (int64_t a = 0; a < n_u; ++a) {
      const double p = exp(c[a] - m) / ssum;
      c[a] = p;
      const float* vu = v + u_tok[a] * vst + h * vsh;
      double dpa = 0.0, oa = 0.0;
      for (int32_t d = 0; d < D; ++d) {
        dpa += g1 * (double)gt[d] * (double)vu[d];
        oa += (double)gt[d] * (double)vu[d];
      }
      dp[a] = dpa;
      delta += p * dpa;
      go += p * oa; /* dout_t . O_sel_t */
      double* dvu = dv + (u_tok[a] * H + h) * D;
      for (int32_t d = 0; d < D; ++d) dvu[d] += p * g1 * (double)gt[d];
    }
    dg[1] += go;
    for (int64_t a = 0; a < n_u; ++a) {
      const double dsa = c[a] * (dp[a] - delta);
      const float* ku = k + u_tok[a] * kst + h * ksh;
      double* dku = dk + (u_tok[a] * H + h) * D;
      for (int32_t d = 0; d < D; ++d) {
        dqt[d] += scale * dsa * (double)ku[d];
        dku[d] += scale * dsa * (double)qt[d];
      }
    }
  }
  /* block means: each token of block j receives 1/n_j of the pooled gradients */
  for (int64_t j = 0; j < Nb; ++j) {
    const int64_t n = block_len(T, B, j);
    for (int64_t t = j * B; t < j * B + n; ++t)
      for (int32_t d = 0; d < D; ++d) {
        dk[(t * H + h) * D + d] += dkc[j * D + d] / (double)n;
        dv[(t * H + h) * D + d] += dvc[j * D + d] / (double)n;
      }
  }
  free(kc);
  free(vc);
  free(dkc);
  free(dvc);
  free(c);
  free(dp);
  free(u_tok);
  free(chosen);
}

/* All heads (in parallel; each head writes only its own slices). dgates: [T][H][2] for
 * per-token gates, [H][2] otherwise; every output is overwritten. */
void s3r_oracle_backward(int64_t T, int32_t H, int32_t D, int32_t B, double scale,
                         const float* q, int64_t qst, int64_t qsh, const float* k, int64_t kst,
                         int64_t ksh, const float* v, int64_t vst, int64_t vsh,
                         const float* gates, int64_t gate_st, const float* dout, int64_t dst,
                         int64_t dsh, const int32_t* sel, int32_t nsel, double* dq, double* dk,
                         double* dv, double* dgates) {
  const int64_t Nb = n_blocks(T, B);
  memset(dq, 0, sizeof(double) * (size_t)(T * H * D));
  memset(dk, 0, sizeof(double) * (size_t)(T * H * D));
  memset(dv, 0, sizeof(double) * (size_t)(T * H * D));
  const int64_t n_dg = gate_st ? T * H * 2 : (int64_t)H * 2;
  memset(dgates, 0, sizeof(double) * (size_t)n_dg);
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t h = 0; h < H; ++h) {
    double* dg = (double*)calloc((size_t)(gate_st ? T * 2 : 2), sizeof(double));
    s3r_oracle_backward_head(T, H, D, B, scale, q, qst, qsh, k, kst, ksh, v, vst, vsh, gates,
                             gate_st, dout, dst, dsh, sel + (int64_t)h * Nb * nsel, nsel, h, dq,
                             dk, dv, dg);
    if (gate_st) {
      for (int64_t t = 0; t < T; ++t) {
        dgates[(t * H + h) * 2 + 0] = dg[t * 2 + 0];
        dgates[(t * H + h) * 2 + 1] = dg[t * 2 + 1];
      }
    } else {
      dgates[h * 2 + 0] = dg[0];
      dgates[h * 2 + 1] = dg[1];
    }
    free(dg);
  }
}

