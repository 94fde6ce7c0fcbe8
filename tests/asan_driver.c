/*
 * AddressSanitizer / UndefinedBehaviorSanitizer driver for the CPU-side test
 * infrastructure: the fp64 oracle and the seeded input generator, built with
 * -fsanitize=address,undefined and run on small layers of every expert format
 * (with and without a shared expert), hash routing, the permutation, the
 * pre-norm and the residual rounding.  Exit status 0 and "asan ok" on success;
 * the sanitizers abort on the first invalid access.  Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t moe_gen_expert_bytes(int32_t H, int32_t F, int32_t fmt);
void moe_gen_x(uint64_t seed, uint32_t window, int32_t T, int32_t H, uint16_t* out);
void moe_gen_router(uint64_t seed, uint32_t layer, int32_t E, int32_t H, uint16_t* out);
void moe_gen_bias(uint64_t seed, uint32_t layer, int32_t E, int32_t kind, double param, float* out);
void moe_gen_experts(uint64_t seed, uint32_t layer, int32_t e_begin, int32_t count, int32_t H, int32_t F,
                     int32_t fmt, int32_t raw, uint8_t* out);
void oracle_router_logits(const uint16_t* x, int T, int H, const uint16_t* W, int E, const float* bias,
                          double* logits);
void oracle_route_hash(const double* logits, int T, int E, int k, const int32_t* table, const int32_t* tok,
                       int32_t* ids, double* w);
void oracle_permutation(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, int32_t* active, int32_t* n_active);
void oracle_moe_layer(const uint16_t* x, int T, int H, int F, int E, int S, int k, int fmt, const uint16_t* Wr,
                      const float* bias, const uint8_t* experts, int64_t expert_bytes, double* y, int32_t* ids_out,
                      double* w_out, double* logits_out);
void oracle_rmsnorm_bf16(const uint16_t* x, int n, double eps, uint16_t* h);
uint16_t oracle_residual_bf16(uint16_t x, double y);

static void* xalloc(size_t n) {
    void* p = malloc(n);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static int run_layer(int fmt, int S, int raw) {
    const int T = 5, H = 256, F = 128, E = 12, k = 3;
    const int64_t eb = moe_gen_expert_bytes(H, F, fmt);
    if (eb <= 0) return 1;
    uint16_t* x = xalloc(sizeof(uint16_t) * T * H);
    uint16_t* W = xalloc(sizeof(uint16_t) * E * H);
    float* b = xalloc(sizeof(float) * E);
    uint8_t* ex = xalloc((size_t)eb * (E + S));
    double* y = xalloc(sizeof(double) * T * H);
    int32_t* ids = xalloc(sizeof(int32_t) * T * k);
    double* w = xalloc(sizeof(double) * T * k);
    double* lg = xalloc(sizeof(double) * T * E);
    moe_gen_x(3, 1, T, H, x);
    moe_gen_router(3, 0, E, H, W);
    moe_gen_bias(3, 0, E, 1, 1.1, b);
    moe_gen_experts(3, 0, 0, E + S, H, F, fmt, raw, ex);
    oracle_moe_layer(x, T, H, F, E, S, k, fmt, W, b, ex, eb, y, ids, w, lg);
    /* permutation of the routing, and hash routing through a table */
    int32_t* off = xalloc(sizeof(int32_t) * (E + 1));
    int32_t* perm = xalloc(sizeof(int32_t) * T * k);
    int32_t* inv = xalloc(sizeof(int32_t) * T * k);
    int32_t* act = xalloc(sizeof(int32_t) * E);
    int32_t nact = 0;
    oracle_permutation(ids, T, k, E, off, perm, inv, act, &nact);
    const int vocab = 7;
    int32_t* table = xalloc(sizeof(int32_t) * vocab * k);
    for (int v = 0; v < vocab; ++v)
        for (int j = 0; j < k; ++j) table[v * k + j] = (v + 5 * j) % E;
    int32_t tok[5] = {0, 6, 3, 3, 1};
    oracle_route_hash(lg, T, E, k, table, tok, ids, w);
    /* pre-norm and residual rounding of the stream */
    uint16_t* h = xalloc(sizeof(uint16_t) * T * H);
    for (int t = 0; t < T; ++t) oracle_rmsnorm_bf16(x + t * H, H, 1e-6, h + t * H);
    uint32_t acc = 0;
    for (int i = 0; i < T * H; ++i) acc += oracle_residual_bf16(h[i], y[i]);
    free(x); free(W); free(b); free(ex); free(y); free(ids); free(w); free(lg);
    free(off); free(perm); free(inv); free(act); free(table); free(h);
    return nact > 0 && acc != 0xFFFFFFFFu ? 0 : 1;
}

int main(void) {
    for (int fmt = 1; fmt <= 3; ++fmt)
        for (int S = 0; S <= 1; ++S)
            for (int raw = 0; raw <= 1; ++raw)
                if (run_layer(fmt, S, raw)) {
                    fprintf(stderr, "layer fmt %d S %d raw %d failed\n", fmt, S, raw);
                    return 1;
                }
    printf("asan ok\n");
    return 0;
}
