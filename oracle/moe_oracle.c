/*
 * fp64 CPU oracle for one sparse mixture-of-experts layer over block-quantised
 * expert weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the GPU library.
 *
 * It is the plain definition of what the layer computes, written with naive
 * loops in double precision:
 *
 *   logits  l[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]           (sum in h order)
 *   select  the first k experts of the list sorted by (l descending, e ascending)
 *   weights p = softmax over all E of l[t];  w_tj = p[id_tj] / sum_j' p[id_tj']
 *   expert  g = G x, u = U x, a_f = silu(g_f) * u_f, o = D a      (silu(z) = z/(1+e^-z))
 *   combine y_t = sum_j w_tj * o_{t,id_tj}  (+ o_shared with weight 1)
 *   permute a stable counting sort of the pair indices i = t*k + j by expert id
 *   (hash-routed layers take their experts from a token-id table instead of
 *   the top-k, see oracle_route_hash)
 *
 * Where the definition comes from:
 *  - Sparse top-k routing over hundreds of experts with a shared expert, and
 *    the fused gate/up/down expert tensors: page "Strata 改源码去跑 DeepSeek V4
 *    Flash？", section 二 (GGUF table: 256 routed + 1 shared, 6 active,
 *    ffn_{gate,up,down}_exps 256x2048x4096, router bias in layers 3-42), and
 *    the teardown page "Strata 引擎深度拆解", section 二 (48 layers x 512
 *    experts, 10 active per token).
 *  - E and k are runtime values (section 三 of the first page: expert_count and
 *    expert_used_count are the only geometry read from the file).
 *  - The pages never print the routing function, the activation or the
 *    combine rule.  The readings taken here: softmax over all experts, top-k
 *    on the logits with the lower expert id first among equal logits, the
 *    k weights renormalised to sum to 1, the router bias added to the logits
 *    before both selection and softmax, SwiGLU = silu(gate) * up, and the
 *    shared expert added with weight 1 outside the renormalisation.
 *
 * Inputs are decoded exactly: bf16 and IEEE binary16 bit patterns become
 * doubles, and a block weight is d*(q-o) with o = 8 (q4b32) or 2 (q2b32,
 * q2b64).
 * Canonical block layout: fp16 scale d (little-endian), then the codes;
 * q4b32 weight j in byte j>>1 (low nibble first), q2b32 and q2b64 weight j in
 * byte j>>2 at bit 2*(j&3).  An expert is its G rows [F x H], then U rows
 * [F x H], then D rows [H x F], each row K/BW blocks along its input dimension
 * (BW = 32, or 64 for q2b64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_Q4B32 1
#define ORACLE_Q2B32 2
#define ORACLE_Q2B64 3

/* bf16 bit pattern -> double (exact). */
double oracle_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE 754 binary16 bit pattern -> double (exact), from the format definition:
 * exponent field 0 is subnormal f * 2^-24, 31 is inf/NaN, else (1024+f)*2^(e-25). */
double oracle_fp16(uint16_t h) {
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return (h & 0x8000) ? -v : v;
}

int64_t oracle_block_bytes(int fmt) {
    return fmt == ORACLE_Q4B32 ? 18 : fmt == ORACLE_Q2B32 ? 10 : fmt == ORACLE_Q2B64 ? 18 : -1;
}

/* Weights per block: 32, or 64 for q2b64 (one fp16 scale per 64 two-bit
 * codes, 2.25 bits per weight: the size of the 2-bit expert blob on the page
 * "Strata 改源码去跑 DeepSeek V4 Flash？", section 三 item 4 (1,382,400 bytes
 * per 2560 x 640 expert), and of the Q2_0 tier's 34 GB expert total, section
 * 一 of the same page). */
int oracle_block_weights(int fmt) { return fmt == ORACLE_Q2B64 ? 64 : 32; }

/* Weight j (0..31, or 0..63 for q2b64) of one canonical block. */
double oracle_block_weight(const uint8_t* blk, int fmt, int j) {
    double d = oracle_fp16((uint16_t)(blk[0] | (blk[1] << 8)));
    int q, o;
    if (fmt == ORACLE_Q4B32) {
        q = (blk[2 + (j >> 1)] >> (4 * (j & 1))) & 0xF;
        o = 8;
    } else {
        q = (blk[2 + (j >> 2)] >> (2 * (j & 3))) & 0x3;
        o = 2;
    }
    return d * (double)(q - o);
}

/* Dequantise a [rows x K] matrix stored as canonical blocks. */
void oracle_dequant_rows(const uint8_t* blocks, int rows, int K, int fmt, double* out) {
    const int64_t bb = oracle_block_bytes(fmt);
    const int bw = oracle_block_weights(fmt);
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < K; ++c)
            out[(int64_t)r * K + c] = oracle_block_weight(blocks + ((int64_t)r * (K / bw) + c / bw) * bb, fmt, c % bw);
}

/* Byte offsets of the three matrices inside one expert. */
static void expert_parts(int H, int F, int fmt, int64_t* g, int64_t* u, int64_t* d) {
    const int64_t bb = oracle_block_bytes(fmt);
    const int bw = oracle_block_weights(fmt);
    *g = 0;
    *u = (int64_t)F * (H / bw) * bb;
    *d = 2 * (int64_t)F * (H / bw) * bb;
}

/* y = M v for M [rows x K] in canonical blocks; sum in column order. */
static void matvec(const uint8_t* blocks, int rows, int K, int fmt, const double* v, double* y) {
    const int64_t bb = oracle_block_bytes(fmt);
    const int bw = oracle_block_weights(fmt);
    for (int r = 0; r < rows; ++r) {
        double s = 0.0;
        for (int c = 0; c < K; ++c)
            s += oracle_block_weight(blocks + ((int64_t)r * (K / bw) + c / bw) * bb, fmt, c % bw) * v[c];
        y[r] = s;
    }
}

/* One expert FFN on one token: out[H] = D (silu(G x) * (U x)); optionally h[F]. */
void oracle_expert_ffn(const uint8_t* expert, int H, int F, int fmt, const double* x, double* out, double* h_out) {
    int64_t og, ou, od;
    expert_parts(H, F, fmt, &og, &ou, &od);
    double* g = (double*)malloc(sizeof(double) * (size_t)F);
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* a = (double*)malloc(sizeof(double) * (size_t)F);
    matvec(expert + og, F, H, fmt, x, g);
    matvec(expert + ou, F, H, fmt, x, u);
    for (int f = 0; f < F; ++f) a[f] = g[f] / (1.0 + exp(-g[f])) * u[f];
    matvec(expert + od, H, F, fmt, a, out);
    if (h_out) memcpy(h_out, a, sizeof(double) * (size_t)F);
    free(g);
    free(u);
    free(a);
}

/* Router logits [T x E] in double; bias may be NULL. */
void oracle_router_logits(const uint16_t* x, int T, int H, const uint16_t* W, int E, const float* bias,
                          double* logits) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int h = 0; h < H; ++h) s += oracle_bf16(x[(int64_t)t * H + h]) * oracle_bf16(W[(int64_t)e * H + h]);
            logits[(int64_t)t * E + e] = s + (bias ? (double)bias[e] : 0.0);
        }
}

typedef struct { double l; int e; } cand;

static int cand_cmp(const void* pa, const void* pb) {
    const cand* a = (const cand*)pa;
    const cand* b = (const cand*)pb;
    if (a->l > b->l) return -1;
    if (a->l < b->l) return 1;
    return (a->e > b->e) - (a->e < b->e);
}

/* Top-k selection and renormalised softmax weights for T tokens.
 * ids[T x k] in selection order (logit descending, lower id first on ties). */
void oracle_select_topk(const double* logits, int T, int E, int k, int32_t* ids, double* w) {
    cand* c = (cand*)malloc(sizeof(cand) * (size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    for (int t = 0; t < T; ++t) {
        const double* l = logits + (int64_t)t * E;
        for (int e = 0; e < E; ++e) { c[e].l = l[e]; c[e].e = e; }
        qsort(c, (size_t)E, sizeof(cand), cand_cmp);
        /* softmax over all E */
        double m = l[0];
        for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
        double z = 0.0;
        for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - m); z += p[e]; }
        for (int e = 0; e < E; ++e) p[e] /= z;
        /* renormalise over the selected k */
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += p[c[j].e];
        for (int j = 0; j < k; ++j) {
            ids[(int64_t)t * k + j] = c[j].e;
            w[(int64_t)t * k + j] = p[c[j].e] / s;
        }
    }
    free(c);
    free(p);
}

/* Hash routing, the reading taken for DeepSeek V4 Flash's tid2eid layers
 * (page "Strata 改源码去跑 DeepSeek V4 Flash？", section 二: layers 0-2 route
 * by a token-id -> experts table, the other layers by score with a router
 * bias).  The page gives the table's name and layers only; read here: the
 * experts of token t are row tok[t] of the [vocab x k] table, in table order,
 * and their weights are the softmax over all E logits renormalised over those
 * k experts, the same weight rule as score routing.  The caller guarantees
 * 0 <= tok[t] < vocab and distinct ids in [0, E) per row. */
void oracle_route_hash(const double* logits, int T, int E, int k, const int32_t* table, const int32_t* tok,
                       int32_t* ids, double* w) {
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    for (int t = 0; t < T; ++t) {
        const double* l = logits + (int64_t)t * E;
        const int32_t* row = table + (int64_t)tok[t] * k;
        double m = l[0];
        for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
        double z = 0.0;
        for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - m); z += p[e]; }
        for (int e = 0; e < E; ++e) p[e] /= z;
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += p[row[j]];
        for (int j = 0; j < k; ++j) {
            ids[(int64_t)t * k + j] = row[j];
            w[(int64_t)t * k + j] = p[row[j]] / s;
        }
    }
    free(p);
}

/* Stable counting sort of the pair indices i = t*k + j by expert id.
 * offsets[E+1] (exclusive prefix of the counts, offsets[E] = P),
 * perm[P] (pair indices grouped by expert, ascending i inside a group),
 * inv_perm[P] (position of pair i in perm), active[U] (experts with a
 * non-empty group, ascending), *n_active = U.  Any output may be NULL. */
void oracle_permutation(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, int32_t* active, int32_t* n_active) {
    const int P = T * k;
    int32_t* cnt = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
    int32_t* off = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
    for (int i = 0; i < P; ++i) cnt[ids[i]] += 1;
    for (int e = 0; e < E; ++e) off[e + 1] = off[e] + cnt[e];
    if (offsets) memcpy(offsets, off, sizeof(int32_t) * ((size_t)E + 1));
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * ((size_t)E + 1));
    memcpy(next, off, sizeof(int32_t) * ((size_t)E + 1));
    for (int i = 0; i < P; ++i) {
        int pos = next[ids[i]]++;
        if (perm) perm[pos] = i;
        if (inv_perm) inv_perm[i] = pos;
    }
    int u = 0;
    for (int e = 0; e < E; ++e)
        if (cnt[e] > 0) {
            if (active) active[u] = e;
            ++u;
        }
    if (n_active) *n_active = u;
    free(cnt);
    free(off);
    free(next);
}

/* Combine step for a list of tokens.  x rows are bf16 [H]; experts holds the
 * canonical bytes of experts 0..E-1 (+ the shared expert at index E when S=1),
 * each expert_bytes long.  ids/w are the routing of those tokens [n x k].
 * y[n x H] = sum_j w_tj * FFN_{id_tj}(x_t) (+ FFN_shared(x_t)).
 * Pairs are evaluated in parallel and summed per token in slot order. */
void oracle_combine(const uint16_t* x_rows, int n, int H, int F, int E, int S, int k, int fmt, const int32_t* ids,
                    const double* w, const uint8_t* experts, int64_t expert_bytes, double* y) {
    const int per = k + S;
    double* o = (double*)malloc(sizeof(double) * (size_t)n * per * H);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < (int64_t)n * per; ++q) {
        const int t = (int)(q / per), j = (int)(q % per);
        const int e = j < k ? ids[(int64_t)t * k + j] : E;
        double* xd = (double*)malloc(sizeof(double) * (size_t)H);
        for (int h = 0; h < H; ++h) xd[h] = oracle_bf16(x_rows[(int64_t)t * H + h]);
        oracle_expert_ffn(experts + (int64_t)e * expert_bytes, H, F, fmt, xd, o + q * H, NULL);
        free(xd);
    }
    for (int t = 0; t < n; ++t)
        for (int h = 0; h < H; ++h) {
            double s = 0.0;
            for (int j = 0; j < k; ++j) s += w[(int64_t)t * k + j] * o[((int64_t)t * per + j) * H + h];
            if (S) s += o[((int64_t)t * per + k) * H + h];
            y[(int64_t)t * H + h] = s;
        }
    free(o);
}

/* Whole layer on T tokens: logits, selection, weights, combine.  ids/w/logits may be NULL. */
void oracle_moe_layer(const uint16_t* x, int T, int H, int F, int E, int S, int k, int fmt, const uint16_t* Wr,
                      const float* bias, const uint8_t* experts, int64_t expert_bytes, double* y, int32_t* ids_out,
                      double* w_out, double* logits_out) {
    double* l = (double*)malloc(sizeof(double) * (size_t)T * E);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * k);
    double* w = (double*)malloc(sizeof(double) * (size_t)T * k);
    oracle_router_logits(x, T, H, Wr, E, bias, l);
    oracle_select_topk(l, T, E, k, ids, w);
    oracle_combine(x, T, H, F, E, S, k, fmt, ids, w, experts, expert_bytes, y);
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * k);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)T * k);
    if (logits_out) memcpy(logits_out, l, sizeof(double) * (size_t)T * E);
    free(l);
    free(ids);
    free(w);
}

/* bf16 round-to-nearest-even of a double, going through binary32 as the
 * residual add of a layer chain does: x_{l+1} = bf16(fp32(x_l) + fp32(y_l)). */
uint16_t oracle_residual_bf16(uint16_t x, double y) {
    float s = (float)oracle_bf16(x) + (float)y;
    uint32_t u;
    memcpy(&u, &s, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Pre-norm of a layer chain: unit-gain RMS normalisation of one token's
 * hidden state, h_i = bf16_rne(x_i / sqrt(mean_j x_j^2 + eps)), in fp64 with a
 * single rounding to bf16.  The MoE-only chains keep each layer's input at
 * the unit scale the activations are drawn at (the pages' models normalise
 * the input of every block; without it the residual stream of random experts
 * grows without bound and overflows bf16 within a few tens of layers). */
void oracle_rmsnorm_bf16(const uint16_t* x, int n, double eps, uint16_t* h) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) {
        const double v = oracle_bf16(x[i]);
        ss += v * v;
    }
    const double r = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i) {
        const double v = oracle_bf16(x[i]) * r;
        /* round the double to bf16, nearest-even, from its exact binary64 bits */
        uint64_t u;
        memcpy(&u, &v, 8);
        const uint64_t sign = u >> 63;
        const int e = (int)((u >> 52) & 0x7FF);
        uint16_t out;
        if (e == 0x7FF) {
            out = (uint16_t)((sign << 15) | 0x7F80u | ((u & 0xFFFFFFFFFFFFFull) ? 0x40u : 0u));
        } else {
            /* value = m * 2^(e - 1075) with m = 2^52 | mantissa; bf16 keeps 8 significant bits */
            const double a = fabs(v);
            int ex;
            const double fr = frexp(a, &ex);             /* a = fr * 2^ex, fr in [0.5, 1) */
            double q = ldexp(fr, 8);                      /* 8 significant bits in the integer part */
            if (ex - 8 < -133) q = ldexp(a, 133);         /* subnormal bf16: fixed quantum 2^-133 */
            const double fl = floor(q);
            const double rem = q - fl;
            double rq = fl;
            if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) rq = fl + 1.0;
            const double rv = ex - 8 < -133 ? ldexp(rq, -133) : ldexp(rq, ex - 8);
            const float f = (float)rv;                    /* exact: rv has at most 8 significant bits */
            uint32_t fu;
            memcpy(&fu, &f, 4);
            out = (uint16_t)((fu >> 16) | (sign << 15));
            (void)e;
        }
        h[i] = out;
    }
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/* Threads for the oracle's later parallel loops (a timing knob, no arithmetic). */
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
