/*
 * Seeded synthetic inputs for the sparse-MoE expert-FFN layer.
 *
 * This module is shared by the oracle side and the GPU side as an INPUT
 * source only: it draws activations, router weights, router biases and
 * block-quantised expert weights from a counter-based generator, and writes
 * them in the canonical byte format both sides read.  It contains none of the
 * layer's arithmetic (no routing, no dequantisation, no FFN).
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Draw i of a stream with key K is
 * mix(K + (i+1)*0x9E3779B97F4A7C15), where mix is the SplitMix64 output
 * function; the key of a stream is derived by chaining mix over
 * (seed, tag, a, b).  A normal deviate is the Irwin-Hall sum of the four
 * 16-bit fields of one draw, centred and scaled to unit variance.
 *
 * Shapes and distributions follow the two model families the pages describe
 * (Qwen3.8-Flash-Next: 48 layers x 512 experts, top-10, hidden 2560, expert
 * FF 640 -- teardown page "Strata 引擎深度拆解", section 二; DeepSeek-V4-Flash:
 * 43 layers, 256 routed + 1 shared, top-6, hidden 4096, FF 2048 -- page
 * "Strata 改源码去跑 DeepSeek V4 Flash？", section 二 GGUF table).
 *
 * Canonical expert format (blocks of BW consecutive weights along the input
 * dimension of one output row; BW = 32 for q4b32 and q2b32, 64 for q2b64):
 *   expert = G rows [F x H], then U rows [F x H], then D rows [H x F];
 *   each row is K/BW blocks (K = H for G and U, K = F for D);
 *   block  = fp16 scale d (little-endian) followed by the codes;
 *   q4b32: weight j in byte j>>1, low nibble first   (18 bytes per block),
 *          w = d*(q-8);
 *   q2b32: weight j in byte j>>2 at bit 2*(j&3)       (10 bytes per block),
 *          w = d*(q-2);
 *   q2b64: as q2b32 with 64 weights per block          (18 bytes per block,
 *          2.25 bits per weight: the size of the pages' 2-bit expert blob).
 * Quantiser used to make the codes from N(0, 0.02) draws:
 *   d = fp16_rne(fp32_rne(absmax / qmax)) with qmax = 7 (q4) or 1 (q2);
 *   q = clamp(rne(w/d) + o, 0, 2^bits - 1); if d == 0 every q = o.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define TAG_X 1u
#define TAG_ROUTER 2u
#define TAG_BIAS 3u
#define TAG_PERM 4u
#define TAG_EXPERT 5u
#define TAG_RAW 6u

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint32_t tag, uint32_t a, uint32_t b) {
    uint64_t k = sm_mix(seed + GOLDEN);
    k = sm_mix(k ^ (((uint64_t)tag << 32) | (uint64_t)a));
    k = sm_mix(k + GOLDEN * (uint64_t)(b + 1u));
    return k;
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return sm_mix(key + (i + 1u) * GOLDEN); }

static inline double normal_of(uint64_t r) {
    /* sum_j (f_j + 0.5)/65536 over the four 16-bit fields f_j, computed exactly */
    uint64_t s = (r & 0xFFFFu) + ((r >> 16) & 0xFFFFu) + ((r >> 32) & 0xFFFFu) + (r >> 48);
    double u = (double)(int64_t)(s + 2u) * (1.0 / 65536.0);
    return (u - 2.0) * 1.7320508075688772; /* sqrt(3): Irwin-Hall(4) has variance 1/3 */
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* IEEE binary16 from binary32, round to nearest even. */
static inline uint16_t f32_to_f16_rne(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u, ax = x & 0x7FFFFFFFu;
    if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds to infinity */
    if (ax < 0x38800000u) {                                     /* below 2^-14: binary16 subnormal */
        float v;
        memcpy(&v, &ax, 4);
        return (uint16_t)(sign | (uint16_t)nearbyintf(v * 0x1p24f));
    }
    uint32_t r = ax - 0x38000000u; /* rebias the exponent from 127 to 15 */
    r += 0xFFFu + ((r >> 13) & 1u);
    return (uint16_t)(sign | (r >> 13));
}

/* binary16 of a double: rounded to binary32 first, then to binary16 (both RNE). */
static inline uint16_t f64_to_f16_rne(double v) { return f32_to_f16_rne((float)v); }

static double f16_bits_value(uint16_t h) {
    int e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double v = (e == 0) ? ldexp((double)f, -24)
             : (e == 31) ? (f ? NAN : INFINITY)
                         : ldexp((double)(f + 1024), e - 25);
    return (h & 0x8000u) ? -v : v;
}

int64_t moe_gen_block_bytes(int32_t fmt) { return fmt == 1 ? 18 : fmt == 2 ? 10 : fmt == 3 ? 18 : -1; }

/* Weights per block. */
int32_t moe_gen_block_weights(int32_t fmt) { return fmt == 3 ? 64 : 32; }

int64_t moe_gen_expert_bytes(int32_t H, int32_t F, int32_t fmt) {
    int64_t bb = moe_gen_block_bytes(fmt);
    const int32_t bw = moe_gen_block_weights(fmt);
    if (bb < 0 || H <= 0 || F <= 0 || H % bw || F % bw) return -1;
    return 3 * (int64_t)H * F / bw * bb;
}

/* Quantise one block of weights (32, or 64 for fmt 3) into canonical bytes
 * (fmt 1 = q4b32, 2 = q2b32, 3 = q2b64). */
void moe_gen_quantize_block(const double* w, int32_t fmt, uint8_t* out) {
    const int bits = fmt == 1 ? 4 : 2;
    const double qmax = fmt == 1 ? 7.0 : 1.0;
    const int o = 1 << (bits - 1), nmax = (1 << bits) - 1;
    const int bw = moe_gen_block_weights(fmt);
    double amax = 0.0;
    for (int j = 0; j < bw; ++j) {
        double a = fabs(w[j]);
        amax = a > amax ? a : amax;
    }
    uint16_t d16 = f64_to_f16_rne(amax / qmax);
    double d = f16_bits_value(d16);
    out[0] = (uint8_t)(d16 & 0xFF);
    out[1] = (uint8_t)(d16 >> 8);
    int q[64];
    if (d != 0.0) {
        for (int j = 0; j < bw; ++j) {
            double r = nearbyint(w[j] / d) + (double)o;
            q[j] = (int)(r < 0.0 ? 0.0 : r > (double)nmax ? (double)nmax : r);
        }
    } else {
        for (int j = 0; j < bw; ++j) q[j] = o;
    }
    if (bits == 4)
        for (int j = 0; j < 16; ++j) out[2 + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
    else
        for (int j = 0; j < bw / 4; ++j)
            out[2 + j] = (uint8_t)(q[4 * j] | (q[4 * j + 1] << 2) | (q[4 * j + 2] << 4) | (q[4 * j + 3] << 6));
}

/* n normal deviates of stream (seed, tag, a, b), draws [start, start+n). */
void moe_gen_normals(uint64_t seed, uint32_t tag, uint32_t a, uint32_t b, uint64_t start, uint64_t n,
                     double* out) {
    uint64_t key = stream_key(seed, tag, a, b);
    for (uint64_t i = 0; i < n; ++i) out[i] = normal_of(draw(key, start + i));
}

/* n bf16 values scale*N(0,1) of stream (seed, tag, a, b). */
void moe_gen_bf16_normal(uint64_t seed, uint32_t tag, uint32_t a, uint32_t b, double scale, uint64_t n,
                         uint16_t* out) {
    uint64_t key = stream_key(seed, tag, a, b);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = f32_to_bf16_rne((float)(scale * normal_of(draw(key, (uint64_t)i))));
}

/* Activations: window w of shape [T x H] bf16, N(0,1). */
void moe_gen_x(uint64_t seed, uint32_t window, int32_t T, int32_t H, uint16_t* out) {
    moe_gen_bf16_normal(seed, TAG_X, window, 0u, 1.0, (uint64_t)T * (uint64_t)H, out);
}

/* Router weights of one layer: [E x H] bf16, N(0, 0.02). */
void moe_gen_router(uint64_t seed, uint32_t layer, int32_t E, int32_t H, uint16_t* out) {
    moe_gen_bf16_normal(seed, TAG_ROUTER, layer, 0u, 0.02, (uint64_t)E * (uint64_t)H, out);
}

/* Router bias of one layer, fp32 [E].
 * kind 0: none (zeros).
 * kind 1: Zipf, b_e = -s*ln(rank_e), rank a seeded permutation of 1..E (Fisher-Yates).
 * kind 2: normal, b_e = sigma*N(0,1). */
void moe_gen_bias(uint64_t seed, uint32_t layer, int32_t E, int32_t kind, double param, float* out) {
    if (kind == 1) {
        int32_t rank[4096];
        if (E > 4096) return;
        for (int32_t i = 0; i < E; ++i) rank[i] = i + 1;
        uint64_t key = stream_key(seed, TAG_PERM, layer, 0u);
        for (int32_t i = E - 1; i > 0; --i) {
            int32_t j = (int32_t)(draw(key, (uint64_t)i) % (uint64_t)(i + 1));
            int32_t t = rank[i]; rank[i] = rank[j]; rank[j] = t;
        }
        for (int32_t e = 0; e < E; ++e) out[e] = (float)(-param * log((double)rank[e]));
    } else if (kind == 2) {
        uint64_t key = stream_key(seed, TAG_BIAS, layer, 0u);
        for (int32_t e = 0; e < E; ++e) out[e] = (float)(param * normal_of(draw(key, (uint64_t)e)));
    } else {
        for (int32_t e = 0; e < E; ++e) out[e] = 0.0f;
    }
}

/* Canonical bytes of experts [e_begin, e_begin+count) of one layer.
 * raw == 0: quantised N(0, 0.02) draws.
 * raw == 1: every code uniform over its full range and d = fp16(0.002*N(0,1)),
 *           so that every code value (including 0) occurs. */
void moe_gen_experts(uint64_t seed, uint32_t layer, int32_t e_begin, int32_t count, int32_t H, int32_t F,
                     int32_t fmt, int32_t raw, uint8_t* out) {
    const int64_t bb = moe_gen_block_bytes(fmt);
    const int64_t per_expert = moe_gen_expert_bytes(H, F, fmt);
    if (per_expert < 0) return;
    const int64_t rows_total = 2 * (int64_t)F + H; /* G rows, U rows, D rows */
    const int bits = fmt == 1 ? 4 : 2;
    const int64_t bw = moe_gen_block_weights(fmt);
#pragma omp parallel for schedule(dynamic, 16) collapse(2)
    for (int32_t ei = 0; ei < count; ++ei) {
        for (int64_t row = 0; row < rows_total; ++row) {
            const uint32_t e = (uint32_t)(e_begin + ei);
            const uint64_t key = stream_key(seed, raw ? TAG_RAW : TAG_EXPERT, layer, e);
            const int64_t K = row < 2 * (int64_t)F ? H : F;
            /* element offset of this row inside the expert: G and U rows have H
             * elements, D rows have F; all three matrices hold F*H elements. */
            const int64_t elem0 = row < 2 * (int64_t)F ? row * H : 2 * (int64_t)F * H + (row - 2 * (int64_t)F) * F;
            const int64_t byte0 = row < 2 * (int64_t)F ? row * (H / bw) * bb
                                                      : 2 * (int64_t)F * (H / bw) * bb + (row - 2 * (int64_t)F) * (F / bw) * bb;
            uint8_t* dst = out + (int64_t)ei * per_expert + byte0;
            if (!raw) {
                double w[4096];
                for (int64_t c0 = 0; c0 < K; c0 += 4096) {
                    const int64_t n = K - c0 < 4096 ? K - c0 : 4096;
                    for (int64_t j = 0; j < n; ++j) w[j] = 0.02 * normal_of(draw(key, (uint64_t)(elem0 + c0 + j)));
                    for (int64_t blk = 0; blk < n / bw; ++blk)
                        moe_gen_quantize_block(w + blk * bw, fmt, dst + (c0 / bw + blk) * bb);
                }
            } else {
                for (int64_t blk = 0; blk < K / bw; ++blk) {
                    uint8_t* o = dst + blk * bb;
                    uint64_t r0 = draw(key, (uint64_t)(elem0 + blk * bw));
                    uint16_t d16 = f64_to_f16_rne(0.002 * normal_of(r0));
                    o[0] = (uint8_t)(d16 & 0xFF);
                    o[1] = (uint8_t)(d16 >> 8);
                    for (int j = 0; j < bits * bw / 8; ++j)
                        o[2 + j] = (uint8_t)(draw(key, (uint64_t)(elem0 + blk * bw + 1 + j)) >> 24);
                }
            }
        }
    }
}
