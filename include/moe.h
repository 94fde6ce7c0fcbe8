/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts layer.
 *
 * One layer computes, for T tokens of hidden state x [T x H]:
 *   1. router logits l = x Wr^T + b                     (Wr [E x H] bf16, b [E] fp32)
 *   2. per token, the top-k experts by (logit descending, lower id first on
 *      equal logits), with weights w_j = softmax over the k selected logits
 *      (the renormalised softmax over all E experts)
 *   3. the (token, expert) pairs grouped by expert with a stable counting sort
 *   4. per pair, the expert FFN  D (silu(G x) * (U x))  over block-quantised
 *      weights (G, U [F x H], D [H x F])
 *   5. y_t = sum_j w_tj * FFN_{e_tj}(x_t)  (+ the shared expert with weight 1)
 *
 * What the pages fix and what they leave open:
 *  - Sparse top-k routing over hundreds of experts, a shared expert and fused
 *    gate/up/down expert tensors: page "Strata 改源码去跑 DeepSeek V4 Flash？",
 *    section 二 (GGUF table: 256 routed + 1 shared, 6 active, FF 2048,
 *    hidden 4096, router bias); the teardown page "Strata 引擎深度拆解",
 *    section 二 (48 layers x 512 experts, 10 active per token).
 *  - E and k are runtime values and a wrong expert width is rejected, not
 *    reinterpreted: the first page, section 三 (items 2 and 4).
 *  - The layer as a function of fixed weights (a hidden state in, the
 *    weighted sum of its routed experts' FFN outputs out): the first page,
 *    section 六.
 *  - The routing function, the activation and the combine rule are not on
 *    the pages.  Readings used: softmax top-k with renormalisation, bias added
 *    to the logits before selection and softmax, SwiGLU, shared expert added
 *    with weight 1.
 *
 * Expert byte format accepted by moe_load_experts ("canonical blocks"): an
 * expert is G rows, then U rows, then D rows; every row is a sequence of
 * blocks of BW consecutive weights along its input dimension; a block is an
 * fp16 scale d (little-endian) followed by the codes:
 *   MOE_Q4B32  BW 32, 18 bytes/block, weight j in byte j>>1 (low nibble first), w = d*(q-8)
 *   MOE_Q2B32  BW 32, 10 bytes/block, weight j in byte j>>2 at bit 2*(j&3),     w = d*(q-2)
 *   MOE_Q2B64  BW 64, 18 bytes/block, weight j in byte j>>2 at bit 2*(j&3),     w = d*(q-2)
 * so one expert is 3*H*F/BW blocks (q4b32 at H=4096, F=2048: 14,155,776 bytes).
 * MOE_Q2B64 spends 2.25 bits per weight: 1,382,400 bytes per 2560 x 640
 * expert, the size of the 2-bit expert blob on the page "Strata 改源码去跑
 * DeepSeek V4 Flash？", section 三 item 4, and 34 GB for all experts of the
 * Q2_0 tier in section 一 (the page does not print the layout; one fp16 scale
 * per 64 codes is the reading taken).
 *
 * Conventions for every call:
 *  - Device pointers are plain device addresses on the context's device,
 *    16-byte aligned, contiguous, owned by the caller and alive until the
 *    work queued on the passed stream has completed.  Host pointers are
 *    read before the call returns.
 *  - Calls are ordered on the HIP stream passed in (NULL = the null stream)
 *    and never synchronise the device implicitly, except moe_load_experts
 *    and moe_destroy, which are synchronous.
 *  - Validation runs before any launch: a call that returns an error has
 *    queued no work and changed no state.  A HIP runtime failure returns
 *    MOE_EHIP and poisons the context (every later call returns MOE_ESTATE).
 *  - No C++ exception crosses this interface.  moe_last_error() returns a
 *    thread-local description of the last non-OK status of this thread.
 *  - A context must not be used from two host threads at once.  Calls on one
 *    context share its scratch memory: queue them on one stream.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1, /* bad argument: shape, format, size, alignment, NULL pointer */
    MOE_ENOMEM = -2, /* device or pinned host allocation failed */
    MOE_EHIP = -3,   /* a HIP runtime call failed; the context is poisoned */
    MOE_ESTATE = -4, /* layer used before it was loaded, or poisoned context */
    MOE_ERANGE = -5  /* T larger than the context's max_tokens */
} moe_status;

typedef enum { MOE_Q4B32 = 1, MOE_Q2B32 = 2, MOE_Q2B64 = 3 } moe_quant;

/* Layer geometry, fixed for the lifetime of a context (E and k are runtime
 * values, as the pages' engine reads them from the model file).
 *   hidden, ffn : H and F, positive multiples of 32 (of 64 for MOE_Q2B64),
 *                 H <= 4096, F <= 2048
 *   n_experts   : E routed experts, 1..1024
 *   n_shared    : 0 or 1 always-on shared expert (expert index E)
 *   top_k       : k in [1, min(E, 16)]
 *   n_layers    : L >= 1; every layer has its own router and experts
 *   quant       : MOE_Q4B32, MOE_Q2B32 or MOE_Q2B64
 *   max_tokens  : largest T accepted by moe_route/moe_forward (1..65536);
 *                 scratch memory is sized for it
 *   device      : HIP device ordinal */
typedef struct {
    int32_t abi_version; /* MOE_ABI_VERSION */
    int32_t hidden, ffn, n_experts, n_shared, top_k, n_layers, quant, max_tokens, device;
} moe_config;

/* One upload of weights for one layer (host memory, read synchronously).
 *   router_w    : [E x H] bf16 bit patterns, or NULL to leave the router as is
 *   router_bias : [E] fp32, or NULL (a router upload with NULL bias sets b = 0)
 *   experts     : expert_count experts in canonical blocks, experts
 *                 [expert_begin, expert_begin + expert_count); index E is the
 *                 shared expert.  NULL with expert_count = 0 uploads none.
 *   experts_bytes must equal expert_count * moe_expert_bytes(H, F, quant)
 *                 (3*H*F/32 * 18, 3*H*F/32 * 10 or 3*H*F/64 * 18).
 *   tid2eid     : NULL to leave the layer's routing as is, or a [vocab x k]
 *                 int32 table (vocab >= 1, ids in [0, E), distinct within a
 *                 row) that makes the layer hash-routed from this upload on:
 *                 token t's experts are row token_ids[t] of the table, in
 *                 table order, and their weights are the softmax of the
 *                 layer's router logits renormalised over them.  The page
 *                 "Strata 改源码去跑 DeepSeek V4 Flash？", section 二, lists
 *                 this routing (tensor tid2eid) for layers 0-2 of DeepSeek
 *                 V4 Flash and score routing with a router bias for layers
 *                 3-42; the weight rule is a reading (the page gives none).
 *                 A hash-routed layer still needs its router uploaded.
 *   vocab       : rows of tid2eid (ignored when tid2eid is NULL) */
typedef struct {
    int32_t layer, expert_begin, expert_count;
    const uint16_t* router_w;
    const float* router_bias;
    const uint8_t* experts;
    size_t experts_bytes;
    const int32_t* tid2eid;
    int32_t vocab;
} moe_layer_weights;

#define MOE_FWD_RESIDUAL 1 /* x_{l+1} = bf16(fp32(x_l) + y_l); else x_{l+1} = bf16(y_l) */
#define MOE_FWD_PROFILE 2  /* time every kernel with a HIP event pair bound to its dispatch (moe_profile_read) */
#define MOE_FWD_PRENORM 4  /* each layer's MoE input is h_l = bf16(x_l / sqrt(mean(x_l^2) + 1e-6)) per token,
                              fp32 arithmetic, unit gain; the residual still adds to x_l.  The pages' models
                              normalise every block input; an MoE-only chain of random experts without it
                              grows without bound and overflows bf16 within a few tens of layers. */

/* One forward pass through layers [layer_begin, layer_begin + layer_count).
 *   x      : [T x H] bf16, device, input of the first layer
 *   y      : [T x H] bf16, device, output of the last layer (the residual
 *            sum when MOE_FWD_RESIDUAL is set); may not alias x
 *   trace_x  : NULL or [layer_count x T x H] bf16, each layer's MoE input (x_l,
 *              or h_l when MOE_FWD_PRENORM is set)
 *   trace_ids: NULL or [layer_count x T x k] int32, each layer's routing
 *   trace_w  : NULL or [layer_count x T x k] fp32, each layer's weights
 *   token_ids: NULL or [T] int32, device, 4-byte aligned; required when a
 *              layer of the range is hash-routed (ids are clamped into
 *              [0, vocab) on the device) */
typedef struct {
    int32_t layer_begin, layer_count, T, flags;
    const void* x;
    void* y;
    void* trace_x;
    int32_t* trace_ids;
    float* trace_w;
    const int32_t* token_ids;
} moe_fwd_args;

typedef struct moe_ctx moe_ctx;

/* Allocate the context on cfg->device: one device arena holding every
 * expert of every layer (L x (E+S) slots), the routers, and scratch sized by
 * max_tokens.  Returns MOE_EINVAL for a bad geometry, MOE_ENOMEM when the
 * arena does not fit (nothing stays allocated).  *out is set only on MOE_OK. */
moe_status moe_create(const moe_config* cfg, moe_ctx** out);

/* Upload router weights and/or experts of one layer.  The canonical blocks are
 * copied through a bounded pinned staging buffer and re-laid-out on the
 * device into the context's slot format.  Returns when the host memory is no
 * longer read; the device work is ordered before any later call on the
 * context.  MOE_EINVAL on a wrong byte count, range or layer. */
moe_status moe_load_experts(moe_ctx* ctx, const moe_layer_weights* w);

/* Routing of one layer (steps 1-3 above) for T tokens of x [T x H] bf16.
 *   token_ids : NULL, or [T] int32, device: the tokens' ids, required when the
 *             layer is hash-routed (see moe_layer_weights.tid2eid)
 *   ids     : [T x k] int32, device; expert ids per token in selection order
 *             (table order for a hash-routed layer)
 *   w       : [T x k] fp32, device; renormalised weights, same order, sum 1
 *   offsets : NULL or [E+1] int32, device; exclusive prefix sum of the number
 *             of pairs per expert (offsets[E] = T*k)
 *   perm    : NULL or [T*k] int32, device; pair indices i = t*k + j grouped by
 *             expert id, ascending i inside a group (stable)
 * MOE_ESTATE if the layer's router is not loaded; MOE_EINVAL if the layer is
 * hash-routed and token_ids is NULL; T = 0 is a no-op. */
moe_status moe_route(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const int32_t* token_ids, int32_t* ids,
                     float* w, int32_t* offsets, int32_t* perm, void* hip_stream);

/* Whole layers (steps 1-5) for T tokens; see moe_fwd_args.  MOE_ESTATE if a
 * layer's router or any of its experts is not loaded, MOE_ERANGE if
 * T > max_tokens, MOE_OK and no work for T = 0.
 * T <= 8 (a decode or verify window) runs the GEMV-shaped decode kernels,
 * whose expert arithmetic is exact up to fp32 accumulation.  T > 8 (prefill,
 * "Qwen3.8-Flash-Next UD-Q4_K_XL 引擎对比", section 四: compute-bound) groups
 * the tokens by expert and runs grouped GEMMs on bf16 MFMA; there the
 * dequantised weights and the SwiGLU activations are rounded to bf16 before
 * the contractions.  Routing (ids, weights, offsets, perm) is exact on both
 * paths. */
moe_status moe_forward(moe_ctx* ctx, const moe_fwd_args* args, void* hip_stream);

/* Wait for the context's work, free everything it owns.  NULL is a no-op. */
moe_status moe_destroy(moe_ctx* ctx);

/* Thread-local text of the last non-OK status returned to this thread. */
const char* moe_last_error(void);

/* Kernel kinds reported by moe_profile_read. */
typedef enum {
    MOE_K_ROUTER = 0,       /* router GEMV, decode path */
    MOE_K_TOPK_SORT = 1,    /* top-k, weights, counting sort, decode path */
    MOE_K_GATEUP = 2,       /* dequant + gate/up GEMV + SwiGLU, decode path */
    MOE_K_DOWN = 3,         /* dequant + down GEMV per expert, decode path */
    MOE_K_COMBINE = 4,      /* ordered weighted combine (+ residual), decode path */
    MOE_K_PF_ROUTER = 5,    /* prefill router */
    MOE_K_PF_TOPK = 6,      /* prefill top-k + weights (hash-routed layer: table lookup + exact logits of the k ids) */
    MOE_K_PF_SORT = 7,      /* prefill counting sort (three launches: histogram, scan, scatter) */
    MOE_K_PF_GEMM1 = 8,     /* prefill grouped GEMM gate/up + SwiGLU */
    MOE_K_PF_GEMM2 = 9,     /* prefill grouped GEMM down */
    MOE_K_PF_COMBINE = 10,  /* prefill weighted combine */
    MOE_K_NORM = 11         /* per-token RMS pre-norm (MOE_FWD_PRENORM; prefill only: decode windows normalise
                               inside the router kernel) */
} moe_kernel_kind;

typedef struct {
    int32_t kernel; /* moe_kernel_kind */
    int32_t layer;
    float ms;       /* hipEventElapsedTime of the start/stop events bound to the kernel's dispatch */
} moe_kernel_time;

/* Durations of the kernels launched by moe_forward calls made with
 * MOE_FWD_PROFILE since the previous read, in launch order.  Waits for those
 * events, writes at most cap records, sets *n_out to the number written and
 * forgets all recorded launches.  Profiling keeps at most 65536 launches. */
moe_status moe_profile_read(moe_ctx* ctx, moe_kernel_time* out, int32_t cap, int32_t* n_out);

/* moe_route_static: routing of one decode window (steps 1-3 above, score
 * routing, no shared expert) on caller-owned router weights, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It needs no context and calls no
 * allocating routine; its scratch (fp64 logits, per-block sums of x, inverse
 * permutation, active list) is one file-scope device array of 96 KiB per GPU,
 * held until the process ends, whose address is looked up once per device on
 * the first call made with that device current.  The same kernels as
 * moe_route for T <= 8 run on the stream passed in, so the results are those
 * of moe_route on a context holding the same router.
 *   x        : [T x H] bf16, device, 16-byte aligned
 *   T        : 0..8 (MOE_ERANGE above; 0 is a no-op)
 *   hidden   : H, positive multiple of 32, at most 4096
 *   n_experts: E, 1..1024;  top_k: k in [1, min(E, 16)]
 *   router_w : [E x H] bf16, device, 16-byte aligned;  router_bias: [E] fp32, device, or NULL
 *   ids, w   : [T x k], device (as moe_route);  offsets [E+1], perm [T*k]: device or NULL
 * MOE_ERANGE when the scratch for (E, k, H) would exceed the array (it never
 * does within the limits above).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (two streams, two host threads) race;
 * order them on one stream. */
moe_status moe_route_static(const void* x, int32_t T, int32_t hidden, int32_t n_experts, int32_t top_k,
                            const void* router_w, const float* router_bias, int32_t* ids, float* w, int32_t* offsets,
                            int32_t* perm, void* hip_stream);

/* Canonical bytes of one expert (3*H*F/BW blocks of the quant's block size BW),
 * or -1 for a bad shape or quant. */
int64_t moe_expert_bytes(int32_t hidden, int32_t ffn, int32_t quant);

/* Device bytes the context holds: expert arena, routers and scratch. */
moe_status moe_memory_bytes(const moe_ctx* ctx, uint64_t* arena_bytes, uint64_t* scratch_bytes);

#ifdef __cplusplus
}
#endif
#endif
