/*
 * hs_oracle.c - plain, slow CPU oracle of query-guided block-sparse decode
 * attention. TEST INFRASTRUCTURE ONLY: used by the tests, by the smoke check
 * and by the benchmark's CPU-baseline leg. No product code path calls it.
 *
 * It shares no source, header or helper with the GPU library. Every function
 * is a direct, unblocked loop over the definition it cites, in double
 * precision. Stored inputs (float32, or bfloat16 bit patterns) are widened to
 * double exactly.
 *
 * Pages cited (title, section):
 *   [QSA]    "8x256K long-context sparse attention: porting HiSparse to QSA"
 *   [HiSp]   untitled HiSparse project write-up (trdm.cn)
 *   [SGL]    "SGLang hierarchical sparse attention: analysis and practice"
 *   [SparDA] SparDA article (2kiu.com)
 *
 * Readings where the pages leave a step open (each one is also listed with
 * its justification in the design notes of the repository):
 *   - Quest's "most likely relevance" of q with a key box is taken as the
 *     largest q.k over the box: sum_i max(q_i * min_i, q_i * max_i).
 *   - A KV group's block score is the sum of its query heads' scores.
 *   - Scores are unscaled dot products; ranking uses the score rounded to
 *     float32 ([QSA 5.1]: fp32 block scores, compared at full fp32
 *     precision), ties broken by lower block index.
 *   - Window: every block holding any of the last W tokens.
 *   - Two-level: top-k is global over the fine blocks inside the selected
 *     coarse blocks.
 *   - Attention is the exact softmax over the selected tokens only, scale
 *     1/sqrt(d) unless given.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HSO_F32 0
#define HSO_BF16 1

static double widen_one(const void* base, int dtype, size_t i) {
  if (dtype == HSO_F32) return (double)((const float*)base)[i];
  uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Logical -> physical addressing of a paged cache ([SGL 2.2]: the page table
 * maps a logical block to its physical page; [HiSp 3.2]: a page holds its
 * tokens contiguously). Row t of unit (b, g) is
 *   pool[page_table[b][t / P]][g][t % P][0 .. d).
 * Writes rows[t][i] for t < T. Returns 0, or -1 if a page id is out of range. */
int hso_gather_unit(const void* pool, int dtype, const int32_t* page_table,
                    int max_pages, int num_phys_pages, int num_kv_heads,
                    int page_size, int head_dim, int b, int g, int T,
                    double* rows) {
  for (int t = 0; t < T; ++t) {
    int32_t page = page_table[(size_t)b * max_pages + t / page_size];
    if (page < 0 || page >= num_phys_pages) return -1;
    size_t off = (((size_t)page * num_kv_heads + g) * page_size + t % page_size) *
                 (size_t)head_dim;
    for (int i = 0; i < head_dim; ++i)
      rows[(size_t)t * head_dim + i] = widen_one(pool, dtype, off + i);
  }
  return 0;
}

/* Mean-pooled keys of each S-token block over its valid tokens
 * ([SparDA 3.1]: block representative = mean pooling; [QSA 2.2]: a summary
 * vector per block). mu[beta][i] = (1/n_beta) sum_{t in beta, t < T} k_t,i. */
void hso_summary_mean(const double* rows, int T, int d, int S, double* mu) {
  int nb = (T + S - 1) / S;
  for (int beta = 0; beta < nb; ++beta) {
    int t0 = beta * S, t1 = t0 + S < T ? t0 + S : T;
    for (int i = 0; i < d; ++i) {
      double sum = 0.0;
      for (int t = t0; t < t1; ++t) sum += rows[(size_t)t * d + i];
      mu[(size_t)beta * d + i] = sum / (double)(t1 - t0);
    }
  }
}

/* Per-dimension key bounding box of each block ([SGL 3.1.2]: Quest keeps the
 * minimum and maximum of every key dimension per block). */
void hso_summary_minmax(const double* rows, int T, int d, int S, double* mn,
                        double* mx) {
  int nb = (T + S - 1) / S;
  for (int beta = 0; beta < nb; ++beta) {
    int t0 = beta * S, t1 = t0 + S < T ? t0 + S : T;
    for (int i = 0; i < d; ++i) {
      double lo = rows[(size_t)t0 * d + i], hi = lo;
      for (int t = t0 + 1; t < t1; ++t) {
        double v = rows[(size_t)t * d + i];
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      mn[(size_t)beta * d + i] = lo;
      mx[(size_t)beta * d + i] = hi;
    }
  }
}

/* Block score against mean summaries ([QSA 2.2]: a light dot product of the
 * query with each block's summary), summed over the G query heads that share
 * the KV head: s_beta = sum_j sum_i q_j,i mu_beta,i. Rows listed in `rows_of`
 * (or 0..n-1 when NULL). */
void hso_scores_mean(const double* q, int G, int d, const double* mu,
                     const int32_t* rows_of, int n, double* s) {
  for (int c = 0; c < n; ++c) {
    int beta = rows_of ? rows_of[c] : c;
    double acc = 0.0;
    for (int j = 0; j < G; ++j)
      for (int i = 0; i < d; ++i)
        acc += q[(size_t)j * d + i] * mu[(size_t)beta * d + i];
    s[c] = acc;
  }
}

/* Quest relevance bound ([SGL 3.1.2]): for each head the largest value q.k
 * can take for a k inside the block's box, sum_i max(q_i m_i, q_i M_i),
 * summed over the G heads of the group. */
void hso_scores_minmax(const double* q, int G, int d, const double* mn,
                       const double* mx, const int32_t* rows_of, int n,
                       double* s) {
  for (int c = 0; c < n; ++c) {
    int beta = rows_of ? rows_of[c] : c;
    double acc = 0.0;
    for (int j = 0; j < G; ++j)
      for (int i = 0; i < d; ++i) {
        double a = q[(size_t)j * d + i] * mn[(size_t)beta * d + i];
        double b = q[(size_t)j * d + i] * mx[(size_t)beta * d + i];
        acc += a > b ? a : b;
      }
    s[c] = acc;
  }
}

typedef struct {
  float key;   /* the score at the pages' precision: float32 */
  int32_t id;  /* block index */
} hso_cand;

static int by_score_desc_then_id(const void* pa, const void* pb) {
  const hso_cand* a = (const hso_cand*)pa;
  const hso_cand* b = (const hso_cand*)pb;
  if (a->key > b->key) return -1;
  if (a->key < b->key) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

/* Top-k blocks ([QSA 2.2] top-k candidate blocks; [HiSp 3.3] Top-K of the
 * table in descending order): order the n candidates by (score rounded to
 * float32, descending; block id, ascending) and keep the first min(k, n).
 * ids[c] is the block id of candidate c (or c when NULL). Writes the kept ids
 * in rank order to out and returns their number. */
int hso_topk(const double* s, const int32_t* ids, int n, int k, int32_t* out) {
  if (k <= 0 || n <= 0) return 0;
  hso_cand* c = (hso_cand*)malloc(sizeof(hso_cand) * (size_t)n);
  for (int i = 0; i < n; ++i) {
    c[i].key = (float)s[i];
    c[i].id = ids ? ids[i] : i;
  }
  qsort(c, (size_t)n, sizeof(hso_cand), by_score_desc_then_id);
  int m = k < n ? k : n;
  for (int i = 0; i < m; ++i) out[i] = c[i].id;
  free(c);
  return m;
}

/* Blocks of the local window ([QSA 2.2] window level: the latest W tokens
 * are always attended; [HiSp 3.3] the window's blocks are forced): block
 * beta is in the window when it holds any token of [T - W, T), i.e. when
 * (beta + 1) * S > T - W. Sets mark[beta] = 1 for those. */
void hso_window(int T, int S, int W, uint8_t* mark) {
  int nb = (T + S - 1) / S;
  if (W <= 0) return;
  for (int beta = 0; beta < nb; ++beta)
    if ((int64_t)(beta + 1) * S > (int64_t)T - W) mark[beta] = 1;
}

/* Whole selection of one unit ([QSA 2.2] coarse level -> fine level ->
 * window, merged; [HiSp 3.3] window forced, then top-K).
 *   q          [G][d]
 *   fine_a/b   fine summaries: mean rows (fine_b NULL) or min / max rows
 *   coarse_a/b coarse summaries (coarse level used when top_k_coarse > 0)
 * Output: ascending block ids (no duplicates) and their count; `fine_scores`
 * (optional, [ceil(T/S)]) receives the fine score of every block that was a
 * candidate and NAN for the others; `coarse_ids` (optional, [top_k_coarse])
 * the kept coarse blocks in rank order. Returns the count. */
int hso_select_unit(const double* q, int G, int d, int T, int S,
                    const double* fine_a, const double* fine_b, int top_k,
                    int W, int C, const double* coarse_a,
                    const double* coarse_b, int top_k_coarse, int32_t* ids_out,
                    double* fine_scores, int32_t* coarse_ids, int* n_coarse) {
  int nb = (T + S - 1) / S;
  if (T <= 0) {
    if (n_coarse) *n_coarse = 0;
    return 0;
  }
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)nb);
  int ncand = 0;
  if (top_k_coarse > 0) {
    int nc = (T + C - 1) / C;
    double* sc = (double*)malloc(sizeof(double) * (size_t)nc);
    if (coarse_b) hso_scores_minmax(q, G, d, coarse_a, coarse_b, NULL, nc, sc);
    else hso_scores_mean(q, G, d, coarse_a, NULL, nc, sc);
    int32_t* gam = (int32_t*)malloc(sizeof(int32_t) * (size_t)nc);
    int ng = hso_topk(sc, NULL, nc, top_k_coarse, gam);
    uint8_t* in_gamma = (uint8_t*)calloc((size_t)nc, 1);
    for (int i = 0; i < ng; ++i) in_gamma[gam[i]] = 1;
    /* fine candidates: the S-blocks lying inside a kept C-block */
    for (int beta = 0; beta < nb; ++beta)
      if (in_gamma[(int64_t)beta * S / C]) cand[ncand++] = beta;
    if (coarse_ids)
      for (int i = 0; i < ng; ++i) coarse_ids[i] = gam[i];
    if (n_coarse) *n_coarse = ng;
    free(in_gamma);
    free(gam);
    free(sc);
  } else {
    for (int beta = 0; beta < nb; ++beta) cand[ncand++] = beta;
    if (n_coarse) *n_coarse = 0;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)(ncand > 0 ? ncand : 1));
  if (fine_b) hso_scores_minmax(q, G, d, fine_a, fine_b, cand, ncand, s);
  else hso_scores_mean(q, G, d, fine_a, cand, ncand, s);
  if (fine_scores) {
    for (int beta = 0; beta < nb; ++beta) fine_scores[beta] = NAN;
    for (int c = 0; c < ncand; ++c) fine_scores[cand[c]] = s[c];
  }
  int32_t* top = (int32_t*)malloc(sizeof(int32_t) * (size_t)(ncand > 0 ? ncand : 1));
  int ntop = hso_topk(s, cand, ncand, top_k, top);
  uint8_t* mark = (uint8_t*)calloc((size_t)nb, 1);
  for (int i = 0; i < ntop; ++i) mark[top[i]] = 1;
  hso_window(T, S, W, mark);
  int count = 0;
  for (int beta = 0; beta < nb; ++beta)
    if (mark[beta]) ids_out[count++] = beta;
  free(mark);
  free(top);
  free(s);
  free(cand);
  return count;
}

/* Exact softmax attention of G query heads over the tokens of the listed
 * blocks ([QSA 3.3]: attention visits only the selected blocks; the softmax
 * is normalised over exactly the visited set):
 *   A = { t < T : t in block ids[c] for some c },
 *   l_t = scale * q_j . k_t,  m = max_{t in A} l_t,
 *   out_j = sum_{t in A} exp(l_t - m) v_t / sum_{t in A} exp(l_t - m).
 * Two passes over A, in double. Block ids outside [0, ceil(T/S)) are
 * ignored; an id listed twice counts once. Empty A gives out_j = 0. */
void hso_attend_unit(const double* q, int G, int d, const double* K,
                     const double* V, int T, const int32_t* ids, int count,
                     int S, double scale, double* out) {
  int nb = (T + S - 1) / S;
  uint8_t* inA = (uint8_t*)calloc((size_t)(nb > 0 ? nb : 1), 1);
  for (int c = 0; c < count; ++c)
    if (ids[c] >= 0 && ids[c] < nb) inA[ids[c]] = 1;
  double* logit = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  for (int j = 0; j < G; ++j) {
    const double* qj = q + (size_t)j * d;
    double m = -INFINITY;
    int any = 0;
    for (int t = 0; t < T; ++t) {
      if (!inA[t / S]) continue;
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += qj[i] * K[(size_t)t * d + i];
      logit[t] = scale * dot;
      if (logit[t] > m) m = logit[t];
      any = 1;
    }
    double* oj = out + (size_t)j * d;
    for (int i = 0; i < d; ++i) oj[i] = 0.0;
    if (!any) continue;
    double denom = 0.0;
    for (int t = 0; t < T; ++t) {
      if (!inA[t / S]) continue;
      double p = exp(logit[t] - m);
      denom += p;
      for (int i = 0; i < d; ++i) oj[i] += p * V[(size_t)t * d + i];
    }
    for (int i = 0; i < d; ++i) oj[i] /= denom;
  }
  free(logit);
  free(inA);
}
