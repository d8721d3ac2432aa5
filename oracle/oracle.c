/*
 * CPU oracle of the Stable LatentMoE layer forward: arithmetic core.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously correct
 * definition that the GPU path is checked against. Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never does, and shares no code with it.
 *
 * Sources (the pages are cited by title and section):
 *  - "Kimi K3の896エキスパートを「896人の専門家」と呼ぶと何がズレるか" (lilting.ch):
 *      section "ルーターは計算の割当器": router s = Sigmoid(W_r x); a per-expert
 *      balancing bias is added for choosing the top 16; the mixing weights are
 *      the original (unbiased) scores, normalised.
 *      section "K3のエキスパートは896個の小型LLMではない": z = W_down x;
 *      u = sum over the top 16 of p_i E_i(z); y = E1_shared(x) + E2_shared(x)
 *      + W_up RMSNorm(u).
 *  - "Kimi K3 テクニカルレポート" (jiwasawa.github.io), section "幅のスケーリング:
 *      Stable LatentMoE": SiTU-GLU keeps SwiGLU's local shape and puts a smooth
 *      cap on both branches (closed form fixed by the workload specification:
 *      act(g, v) = c*tanh(SiLU(g)/c) * c*tanh(v/c)).
 *  - "Kimi K3 ... Open Frontier Intelligence" (ai-tech-express.jp), section
 *      "MXFP4 Quantization-Aware Training": 4-bit MXFP4 weights; element and
 *      scale encodings follow the OCP Microscaling Formats v1.0 specification.
 *
 * Precision: everything is fp64 except the router (below), whose fp32
 * arithmetic is fixed exactly because the top-k choice and the gates must be
 * reproduced bit for bit. Storage points (z, h, o, n and the shared-expert
 * activations) are rounded to the activation dtype, as a kernel that stores
 * them in that dtype would; y itself is returned unrounded.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp (no FMA contraction,
 * so every operation below is exactly the one written).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* ------------------------------------------------------------------------- */
/* Storage decoding (exact).                                                  */
/* ------------------------------------------------------------------------- */

/* bf16 bit pattern -> fp32: the bf16 bits are the high half of the fp32. */
void orc_widen_bf16(const uint16_t* in, int64_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)in[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        out[i] = f;
    }
}

/* OCP MX e2m1 element: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
   Magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static double e2m1_value(unsigned code) {
    unsigned e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * m                       /* subnormal: m * 2^(1-1) * 0.5 */
                          : ldexp(1.0 + 0.5 * m, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

/* MXFP4 [rows, K] -> fp32: value = e2m1(nibble) * 2^(scale_byte - 127); element
   2i of a row is the low nibble of byte i; one scale byte per 32 elements. */
void orc_dequant_mxfp4(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K,
                       float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = packed[r * (K / 2) + k / 2];
            unsigned code = (k % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
            int sc = (int)scales[r * (K / 32) + k / 32] - 127;
            out[r * K + k] = (float)ldexp(e2m1_value(code), sc);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Router: logits, sigmoid, biased keys (fp32, order fixed).                  */
/* ------------------------------------------------------------------------- */

/* exp(-a) ... the sigmoid 1 / (1 + e^(-l)) built from IEEE-754 operations only:
   Cody & Waite range reduction (a = n ln2 + r, ln2 split in two fp32 parts so
   n*LN2_HI is exact) and the Taylor polynomial of e^r to degree 7 in Horner
   form; every step is one correctly rounded fp32 operation (fmaf, rintf with
   ties-to-even, exact scaling by 2^n, one division). The constants are derived
   here from their definitions. */
static float LN2_HI, LN2_LO, LOG2E_F, INV_FACT[8];

void orc_init_constants(void) {
    const double ln2 = 0.693147180559945309417232121458176568;
    LN2_HI = (float)ln2;
    LN2_LO = (float)(ln2 - (double)LN2_HI);
    LOG2E_F = (float)(1.0 / ln2);
    double f = 1.0;
    for (int j = 0; j < 8; ++j) {
        if (j > 0) f *= (double)j;
        INV_FACT[j] = (float)(1.0 / f);
    }
}

float orc_sigmoid(float l) {
    float a = -l;                       /* e^(-l) = e^a */
    if (a > 87.0f) a = 87.0f;
    if (a < -87.0f) a = -87.0f;
    float n = rintf(a * LOG2E_F);
    float r = fmaf(-n, LN2_HI, a);
    r = fmaf(-n, LN2_LO, r);
    float p = INV_FACT[7];
    for (int j = 6; j >= 0; --j) p = fmaf(p, r, INV_FACT[j]);
    float e = ldexpf(p, (int)n);
    return 1.0f / (1.0f + e);
}

/* l[t][e] = sum_k x[t][k] * W_r[e][k], accumulated as acc = fmaf(x, w, acc)
   from acc = +0 with k ascending; s = sigmoid(l); key = s + b[e]. */
void orc_router(const float* x, const float* Wr, const float* b, int64_t T, int64_t d,
                int64_t E, float* s_out, float* key_out) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        const float* xt = x + t * d;
        for (int64_t e = 0; e < E; ++e) {
            const float* we = Wr + e * d;
            float acc = 0.0f;
            for (int64_t k = 0; k < d; ++k) acc = fmaf(xt[k], we[k], acc);
            float s = orc_sigmoid(acc);
            s_out[t * E + e] = s;
            key_out[t * E + e] = s + b[e];
        }
    }
}

/* ------------------------------------------------------------------------- */
/* fp64 pieces of the expert / shared / latent paths.                         */
/* ------------------------------------------------------------------------- */

/* Round to bf16 (8 significant bits, nearest, ties to even; subnormal bf16
   spacing 2^-133 below 2^-126). */
double orc_round_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int ex;
    frexp(v, &ex);                      /* v = m * 2^ex, 0.5 <= |m| < 1 */
    int q = ex - 8;                     /* quantum of an 8-bit significand */
    if (q < -133) q = -133;
    double r = nearbyint(ldexp(v, -q));  /* default rounding mode: ties to even */
    return ldexp(r, q);
}

/* storage: 0 = fp32, 1 = bf16 */
double orc_store(double v, int storage) {
    return storage == 1 ? orc_round_bf16(v) : (double)(float)v;
}

void orc_store_array(double* v, int64_t n, int storage) {
    for (int64_t i = 0; i < n; ++i) v[i] = orc_store(v[i], storage);
}

/* out[i][o] = sum_k A[i][k] * W[o][k] (fp64, k ascending); W is [N, K]. */
void orc_linear(const double* A, int64_t n, int64_t K, const float* W, int64_t N, double* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < N; ++o) {
        const float* w = W + o * K;
        for (int64_t i = 0; i < n; ++i) {
            const double* a = A + i * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += a[k] * (double)w[k];
            out[i * N + o] = acc;
        }
    }
}

/* SiTU-GLU: c*tanh(SiLU(g)/c) * c*tanh(v/c), SiLU(g) = g / (1 + e^-g). */
double orc_situ_glu(double g, double v, double c) {
    double silu = g / (1.0 + exp(-g));
    return (c * tanh(silu / c)) * (c * tanh(v / c));
}

/* h[i][f] = store(act(G[i][f], V[i][f])) */
void orc_glu(const double* G, const double* V, int64_t n, double c, int storage, double* H) {
    for (int64_t i = 0; i < n; ++i) H[i] = orc_store(orc_situ_glu(G[i], V[i], c), storage);
}

/* n = store(u / sqrt(mean(u^2) + eps) * gain), one row of width D. */
void orc_rmsnorm(const double* u, int64_t rows, int64_t D, double eps, const float* gain,
                 int storage, double* out) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* ur = u + r * D;
        double ss = 0.0;
        for (int64_t i = 0; i < D; ++i) ss += ur[i] * ur[i];
        double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (int64_t i = 0; i < D; ++i)
            out[r * D + i] = orc_store(ur[i] * inv * (gain ? (double)gain[i] : 1.0), storage);
    }
}
