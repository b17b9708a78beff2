/*
 * sanitize_main.c - drives every function of the CPU oracle (oracle/hs_oracle.c)
 * and of the input generator (synth/synth.c) on small and edge-case shapes,
 * for a host-only AddressSanitizer / UndefinedBehaviorSanitizer build made by
 * tests/test_sanitize.py. Buffers are sized exactly as the Python wrappers
 * size them, so an out-of-bounds access in either file is reported.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle */
int hso_gather_unit(const void* pool, int dtype, const int32_t* page_table, int max_pages,
                    int num_phys_pages, int num_kv_heads, int page_size, int head_dim, int b,
                    int g, int T, double* rows);
void hso_summary_mean(const double* rows, int T, int d, int S, double* mu);
void hso_summary_minmax(const double* rows, int T, int d, int S, double* mn, double* mx);
void hso_scores_mean(const double* q, int G, int d, const double* mu, const int32_t* rows_of,
                     int n, double* s);
void hso_scores_minmax(const double* q, int G, int d, const double* mn, const double* mx,
                       const int32_t* rows_of, int n, double* s);
int hso_topk(const double* s, const int32_t* ids, int n, int k, int32_t* out);
void hso_window(int T, int S, int W, uint8_t* mark);
int hso_select_unit(const double* q, int G, int d, int T, int S, const double* fine_a,
                    const double* fine_b, int top_k, int W, int C, const double* coarse_a,
                    const double* coarse_b, int top_k_coarse, int32_t* ids_out,
                    double* fine_scores, int32_t* coarse_ids, int* n_coarse);
void hso_attend_unit(const double* q, int G, int d, const double* K, const double* V, int T,
                     const int32_t* ids, int count, int S, double scale, double* out);
/* generator */
uint64_t synth_mix64(uint64_t z);
void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double* out);
void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double* out);
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, float* out);
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                       uint16_t* out);
double synth_normal_one(uint64_t seed, uint64_t stream, uint64_t index);
void synth_round_bf16(const double* x, int64_t n, uint16_t* out);
void synth_round_f32(const double* x, int64_t n, float* out);

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) exit(2);
  return p;
}

static int cdiv(int a, int b) { return (a + b - 1) / b; }

/* One selection + attention of a unit with T tokens through both levels. */
static void unit_case(int T, int d, int G, int S, int C, int k, int kc, int W, int minmax) {
  double* q = xmalloc(sizeof(double) * G * d);
  double* K = xmalloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * d);
  double* V = xmalloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * d);
  synth_normal_f64(11, 1, 0, (int64_t)G * d, q);
  synth_normal_f64(11, 2, 0, (int64_t)T * d, K);
  synth_normal_f64(11, 3, 0, (int64_t)T * d, V);
  const int nb = cdiv(T, S), nc = C > 0 ? cdiv(T, C) : 0;
  double* fa = xmalloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1) * d);
  double* fb = minmax ? xmalloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1) * d) : NULL;
  double* ca = nc ? xmalloc(sizeof(double) * (size_t)nc * d) : NULL;
  if (minmax) hso_summary_minmax(K, T, d, S, fa, fb);
  else hso_summary_mean(K, T, d, S, fa);
  if (nc) hso_summary_mean(K, T, d, C, ca);
  int32_t* ids = xmalloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
  double* fs = xmalloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
  int32_t* cids = xmalloc(sizeof(int32_t) * (size_t)(kc > 0 ? kc : 1));
  int ncs = 0;
  const int cnt = hso_select_unit(q, G, d, T, S, fa, fb, k, W, C > 0 ? C : 1, ca, NULL,
                                  nc ? kc : 0, ids, fs, cids, &ncs);
  for (int i = 1; i < cnt; ++i)
    if (ids[i] <= ids[i - 1]) {
      fprintf(stderr, "ids not ascending\n");
      exit(3);
    }
  double* out = xmalloc(sizeof(double) * G * d);
  hso_attend_unit(q, G, d, K, V, T, ids, cnt, S, 1.0 / sqrt((double)d), out);
  /* block size 1: a token list with out-of-range entries */
  int32_t toks[6] = {0, T - 1, T, -1, 1 << 30, T / 2};
  hso_attend_unit(q, G, d, K, V, T, toks, 6, 1, 0.125, out);
  free(out);
  free(cids);
  free(fs);
  free(ids);
  free(ca);
  free(fb);
  free(fa);
  free(V);
  free(K);
  free(q);
}

int main(void) {
  /* generator */
  double u[257], x[257];
  float f[257];
  uint16_t h[257];
  synth_uniform_f64(1, 2, 3, 257, u);
  synth_normal_f64(1, 2, 0, 257, x);
  synth_normal_f64(1, 2, 1, 0, x);
  synth_normal_f32(1, 2, 5, 257, f);
  synth_normal_bf16(1, 2, 7, 257, h);
  (void)synth_normal_one(1, 2, 3);
  (void)synth_mix64(0x1234);
  x[0] = INFINITY;
  x[1] = -INFINITY;
  x[2] = NAN;
  x[3] = 3.4e38;
  x[4] = -0.0;
  x[5] = 1e-45;
  synth_round_bf16(x, 257, h);
  synth_round_f32(x, 257, f);

  /* top-k on empty, tiny and tied inputs */
  double s[9] = {1, 2, 2, -0.0, 0.0, 5, 5, 5, -1};
  int32_t id9[9] = {8, 7, 6, 5, 4, 3, 2, 1, 0}, out9[9];
  int32_t dummy;
  hso_topk(s, NULL, 0, 3, &dummy);
  hso_topk(s, NULL, 9, 0, out9);
  hso_topk(s, NULL, 9, 4, out9);
  hso_topk(s, id9, 9, 100, out9);
  uint8_t mark[8] = {0};
  hso_window(0, 64, 10, mark);
  hso_window(100, 16, 1000, mark);
  hso_window(100, 16, 0, mark);

  /* selection + attention: partial blocks, k = 0, k >= n, windows longer than
   * the context, one token, empty context, two levels with ragged tails */
  unit_case(0, 64, 1, 16, 0, 4, 0, 32, 0);
  unit_case(1, 64, 2, 16, 0, 4, 0, 0, 1);
  unit_case(999, 64, 4, 16, 0, 0, 0, 40, 1);
  unit_case(999, 64, 4, 16, 0, 1000, 0, 0, 0);
  unit_case(1000, 128, 8, 32, 0, 7, 0, 100000, 1);
  unit_case(4133, 64, 2, 64, 1024, 16, 3, 512, 0);
  unit_case(4133, 64, 2, 64, 1024, 16, 100, 0, 0);
  unit_case(3000, 64, 1, 8, 64, 40, 0, 16, 1);

  /* gather through a page table with an invalid entry (returns -1) */
  const int P = 16, hkv = 2, d = 64, npg = 4, nphys = 8;
  float* pool = xmalloc(sizeof(float) * nphys * hkv * P * d);
  uint16_t* poolb = xmalloc(sizeof(uint16_t) * nphys * hkv * P * d);
  synth_normal_f32(3, 4, 0, (int64_t)nphys * hkv * P * d, pool);
  synth_normal_bf16(3, 4, 0, (int64_t)nphys * hkv * P * d, poolb);
  int32_t pt[2 * 4] = {0, 1, 2, 3, 7, 6, 5, 4};
  double* rows = xmalloc(sizeof(double) * npg * P * d);
  if (hso_gather_unit(pool, 0, pt, npg, nphys, hkv, P, d, 1, 1, npg * P, rows) != 0) return 4;
  if (hso_gather_unit(poolb, 1, pt, npg, nphys, hkv, P, d, 0, 0, npg * P - 5, rows) != 0)
    return 5;
  pt[2] = nphys;
  if (hso_gather_unit(pool, 0, pt, npg, nphys, hkv, P, d, 0, 1, npg * P, rows) != -1) return 6;
  pt[2] = -1;
  if (hso_gather_unit(pool, 0, pt, npg, nphys, hkv, P, d, 0, 1, npg * P, rows) != -1) return 7;
  free(rows);
  free(poolb);
  free(pool);
  printf("sanitized oracle and generator: ok\n");
  return 0;
}
