/*
 * Host-only exercise of the CPU oracle (oracle/oracle.c) and of the host twin
 * of the input generator (synth/csrc/synth_host.c), built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/test_sanitizers.py. It calls every
 * exported function on small shapes, edge values included (zeros, subnormals,
 * huge and negative inputs, an all-zero MXFP4 block, ragged K), and checks a
 * few results, so that an out-of-bounds access, an overflow or another
 * undefined operation in either file stops the run with a report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle.c */
void orc_init_constants(void);
void orc_widen_bf16(const uint16_t* in, int64_t n, float* out);
void orc_dequant_mxfp4(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K, float* out);
float orc_sigmoid(float l);
void orc_router(const float* x, const float* Wr, const float* b, int64_t T, int64_t d, int64_t E,
                float* s_out, float* key_out);
double orc_round_bf16(double v);
double orc_store(double v, int storage);
void orc_store_array(double* v, int64_t n, int storage);
void orc_linear(const double* A, int64_t n, int64_t K, const float* W, int64_t N, double* out);
double orc_situ_glu(double g, double v, double c);
void orc_glu(const double* G, const double* V, int64_t n, double c, int storage, double* H);
void orc_rmsnorm(const double* u, int64_t rows, int64_t D, double eps, const float* gain, int storage,
                 double* out);
/* synth_host.c */
uint64_t synth_key(uint64_t seed, uint64_t tensor_id);
void synth_normal_f32(uint64_t key, uint64_t start, int64_t n, float sigma, const float* table, float* out);
void synth_normal_bf16(uint64_t key, uint64_t start, int64_t n, float sigma, const float* table,
                       uint16_t* out);
void synth_uniform_f32(uint64_t key, uint64_t start, int64_t n, float halfwidth, float* out);
void synth_mxfp4(uint64_t key, uint64_t row0, int64_t rows, int64_t K, float sigma, const float* table,
                 uint8_t* packed, uint8_t* scales);

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

int main(void) {
  orc_init_constants();

  /* generator: a table with the full 16-bit index range, every entry point */
  float* table = xmalloc(65536 * sizeof(float));
  for (int i = 0; i < 65536; ++i) table[i] = (float)((i - 32768) / 8192.0);
  const uint64_t key = synth_key(7, 3);
  const int64_t n = 1000;
  float* f = xmalloc(n * sizeof(float));
  uint16_t* h = xmalloc(n * sizeof(uint16_t));
  synth_normal_f32(key, (uint64_t)1 << 40, n, 0.5f, table, f);
  synth_normal_bf16(key, 17, n, 1e-38f, table, h);            /* subnormal masters */
  synth_uniform_f32(key, 0, n, 0.1f, f);
  for (int64_t i = 0; i < n; ++i) CHECK(fabsf(f[i]) <= 0.1f);
  const int64_t rows = 5, K = 96;
  uint8_t* packed = xmalloc(rows * K / 2);
  uint8_t* scales = xmalloc(rows * K / 32);
  synth_mxfp4(key, 3, rows, K, 0.25f, table, packed, scales);
  synth_mxfp4(key, 0, rows, K, 0.0f, table, packed, scales);  /* all-zero blocks */
  for (int64_t i = 0; i < rows * K / 32; ++i) CHECK(scales[i] == 0);
  synth_mxfp4(key, 11, rows, K, 1e-39f, table, packed, scales);   /* subnormal block maxima */

  /* decoding */
  float* wide = xmalloc(rows * K * sizeof(float));
  synth_mxfp4(key, 3, rows, K, 0.25f, table, packed, scales);
  orc_dequant_mxfp4(packed, scales, rows, K, wide);
  uint16_t bits[6] = {0x0000, 0x8000, 0x0001, 0x7F7F, 0xFF7F, 0x3F80};
  float wb[6];
  orc_widen_bf16(bits, 6, wb);
  CHECK(wb[5] == 1.0f && wb[0] == 0.0f);

  /* router on a tiny layer, with extreme logits */
  const int64_t T = 4, d = 40, E = 9;
  float* x = xmalloc(T * d * sizeof(float));
  float* Wr = xmalloc(E * d * sizeof(float));
  float* b = xmalloc(E * sizeof(float));
  for (int64_t i = 0; i < T * d; ++i) x[i] = (float)((i * 37) % 11) - 5.0f;
  for (int64_t i = 0; i < E * d; ++i) Wr[i] = (float)((i * 13) % 7) * 0.5f - 1.5f;
  for (int64_t e = 0; e < E; ++e) b[e] = 0.01f * (float)e;
  float* s = xmalloc(T * E * sizeof(float));
  float* kk = xmalloc(T * E * sizeof(float));
  orc_router(x, Wr, b, T, d, E, s, kk);
  for (int64_t i = 0; i < T * E; ++i) CHECK(s[i] >= 0.0f && s[i] <= 1.0f);
  const float ls[7] = {-1e30f, -100.0f, -87.5f, 0.0f, 1e-40f, 87.5f, 1e30f};
  for (int i = 0; i < 7; ++i) {
    float v = orc_sigmoid(ls[i]);
    CHECK(v >= 0.0f && v <= 1.0f);
  }

  /* fp64 pieces */
  const double rv[6] = {0.0, -0.0, 1e-300, -3.0e38, 1.0 + 1.0 / 512, INFINITY};
  for (int i = 0; i < 6; ++i) {
    (void)orc_round_bf16(rv[i]);
    (void)orc_store(rv[i], 0);
    (void)orc_store(rv[i], 1);
  }
  const int64_t NA = 3, KA = 40, NW = 6;
  double* A = xmalloc(NA * KA * sizeof(double));
  for (int64_t i = 0; i < NA * KA; ++i) A[i] = sin((double)i);
  double* out = xmalloc(NA * NW * sizeof(double));
  orc_linear(A, NA, KA, Wr, NW, out);
  orc_store_array(out, NA * NW, 1);
  double* G = xmalloc(NA * NW * sizeof(double));
  orc_glu(out, out, NA * NW, 8.0, 1, G);
  (void)orc_situ_glu(-800.0, 1e300, 8.0);
  double* nrm = xmalloc(NA * NW * sizeof(double));
  float gain[6] = {1, 2, 3, 4, 5, 6};
  orc_rmsnorm(G, NA, NW, 1e-6, gain, 1, nrm);
  memset(G, 0, NA * NW * sizeof(double));
  orc_rmsnorm(G, NA, NW, 1e-6, NULL, 0, nrm);                   /* u = 0 gives n = 0 */
  for (int64_t i = 0; i < NA * NW; ++i) CHECK(nrm[i] == 0.0);

  free(table); free(f); free(h); free(packed); free(scales); free(wide); free(x); free(Wr); free(b);
  free(s); free(kk); free(A); free(out); free(G); free(nrm);
  printf("sanitized oracle and generator: ok\n");
  return 0;
}
