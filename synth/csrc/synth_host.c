/*
 * Seeded synthetic inputs for the Stable LatentMoE layer: host twin.
 *
 * This file holds none of the layer's arithmetic. It only turns
 * (seed, tensor id, element index) into a value, so that any slice of any
 * tensor can be regenerated on its own (the CPU checker regenerates one
 * expert's weights at a time; the device twin in synth_dev.hip fills GPU
 * memory with the same bits).
 *
 * Generator (counter-based):
 *   key        = mix64(seed * G + tensor_id * H + C)
 *   word(c)    = mix64(key + (c + 1) * G)          -- the (c+1)-th SplitMix64
 *                                                      output from state `key`
 *   mix64      = the SplitMix64 output function (Steele, Lea & Flood,
 *                "Fast splittable pseudorandom number generators", OOPSLA 2014)
 *   element i of a "normal" tensor uses bits [16*(i%4), 16*(i%4)+15] of
 *   word(i/4) as an index j into a 65536-entry table of standard-normal
 *   quantiles at the bin midpoints (j + 0.5) / 65536; value = table[j] * sigma
 *   in fp32, then stored as fp32 or rounded to bf16 (round to nearest even).
 *   element i of a "uniform" tensor uses the top 24 bits m of word(i):
 *   value = fp32((2m - 2^24) * 2^-24) * halfwidth  (one rounding, in fp32).
 *
 * MXFP4 weights (OCP Microscaling Formats v1.0, e2m1 elements, e8m0 scales,
 * 32-element blocks along K): the bf16 master of element (row, k) is the
 * normal value at counter row*K + k; per block X = floor(log2(amax)) - 2 is
 * stored as the biased byte X + 127 (0 for an all-zero block), and each
 * element is v / 2^X rounded to the nearest e2m1 value (ties to the even
 * code), saturating at +-6. Element 2i of a row goes to the low nibble of
 * byte i.
 *
 * Built with gcc -O2 -ffp-contract=off (no contraction of the fp32 multiply).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define GOLD 0x9E3779B97F4A7C15ULL
#define HKEY 0xD1B54A32D192ED03ULL
#define CKEY 0x632BE59BD9B4E019ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tensor_id) {
    return mix64(seed * GOLD + tensor_id * HKEY + CKEY);
}

static inline uint64_t word_at(uint64_t key, uint64_t c) {
    return mix64(key + (c + 1) * GOLD);
}

static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* fp32 -> bf16, round to nearest even (inputs here are finite). */
static inline uint16_t bf16_rne(float f) {
    uint32_t u = f2u(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float normal_at(uint64_t key, uint64_t i, float sigma, const float* table) {
    uint64_t w = word_at(key, i >> 2);
    uint32_t j = (uint32_t)((w >> (16 * (i & 3))) & 0xFFFFu);
    return table[j] * sigma;
}

void synth_normal_f32(uint64_t key, uint64_t start, int64_t n, float sigma,
                      const float* table, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = normal_at(key, start + (uint64_t)i, sigma, table);
}

void synth_normal_bf16(uint64_t key, uint64_t start, int64_t n, float sigma,
                       const float* table, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_rne(normal_at(key, start + (uint64_t)i, sigma, table));
}

void synth_uniform_f32(uint64_t key, uint64_t start, int64_t n, float halfwidth, float* out) {
    for (int64_t i = 0; i < n; ++i) {
        uint64_t m = word_at(key, start + (uint64_t)i) >> 40;           /* 24 bits */
        float v = (float)((int64_t)(2 * m) - (int64_t)(1u << 24)) * (1.0f / 16777216.0f);
        out[i] = v * halfwidth;
    }
}

/* e2m1 code (magnitude 0..7) of |q| by round-to-nearest, ties to even code. */
static inline uint32_t e2m1_code(float a) {
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
           (uint32_t)(a > 5.0f);
}

/* Quantise one 32-element block of bf16 masters (given as bf16 bits). */
static void quant_block(const uint16_t* m, uint8_t* packed16, uint8_t* scale) {
    uint32_t amax_bits = 0;
    for (int i = 0; i < 32; ++i) {
        uint32_t a = m[i] & 0x7FFFu;
        if (a > amax_bits) amax_bits = a;        /* |bf16| orders like its bits */
    }
    if (amax_bits == 0) {
        *scale = 0;
        memset(packed16, 0, 16);
        return;
    }
    /* floor(log2(amax)) for a bf16 value: its unbiased exponent (normal) or
       the position of its leading mantissa bit (subnormal). */
    int e;
    uint32_t ef = (amax_bits >> 7) & 0xFFu;
    if (ef != 0) {
        e = (int)ef - 127;
    } else {
        uint32_t mant = amax_bits & 0x7Fu;
        int p = 6;
        while (!(mant & (1u << p))) --p;
        e = -133 + p;
    }
    int x = e - 2;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    *scale = (uint8_t)(x + 127);
    double inv = ldexp(1.0, -x);
    for (int i = 0; i < 16; ++i) {
        uint8_t byte = 0;
        for (int h = 0; h < 2; ++h) {
            float v = u2f((uint32_t)m[2 * i + h] << 16);
            float q = (float)((double)v * inv);        /* exact power-of-two scaling */
            uint32_t code = e2m1_code(fabsf(q));
            if (q < 0.0f || (v == 0.0f && signbit(v))) code |= 8u;
            byte |= (uint8_t)(code << (4 * h));
        }
        packed16[i] = byte;
    }
}

/* rows x K matrix; K a multiple of 32. packed: rows*K/2 bytes, scales: rows*K/32. */
void synth_mxfp4(uint64_t key, uint64_t row0, int64_t rows, int64_t K, float sigma,
                 const float* table, uint8_t* packed, uint8_t* scales) {
    int64_t nblk = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < rows * nblk; ++b) {
        int64_t r = b / nblk, kb = b % nblk;
        uint16_t m[32];
        uint64_t base = (row0 + (uint64_t)r) * (uint64_t)K + (uint64_t)(kb * 32);
        for (int i = 0; i < 32; ++i)
            m[i] = bf16_rne(normal_at(key, base + (uint64_t)i, sigma, table));
        quant_block(m, packed + r * (K / 2) + kb * 16, scales + r * nblk + kb);
    }
}
