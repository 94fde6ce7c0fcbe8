// Prefill path of the MI355X sparse-MoE layer (T > 8 tokens per call).
//
// Prefill is the compute-bound side of the engine ("Qwen3.8-Flash-Next
// UD-Q4_K_XL 引擎对比", section 四: prefill is limited by compute, decode by
// bandwidth, and the engine's prefill path rather than memory was what held
// it back).  Tokens are grouped by expert and run through grouped GEMMs on
// bf16 MFMA, one group per expert plus one for the shared expert
// ("Strata 改源码去跑 DeepSeek V4 Flash？", section 二: routed top-k experts
// plus an always-on shared expert).
//
//   k_pf_router   x Wr^T on v_mfma_f32_32x32x16_bf16 (fp32), 128 x 256 tiles
//                 staged in LDS by DMA, K split into up to 8 partial sums
//                 (added in order, with the bias, by the top-k kernel)
//   k_pf_topk     one wave per token: candidates = every expert whose fp32
//                 logit lies within twice the fp32 error bound of the k-th
//                 largest; candidates re-scored exactly (fp64 sum of the exact
//                 bf16 products); exact top-k (logit descending, lower id
//                 first); softmax over the selected logits
//   k_pf_hist     per 256-token block: per-expert token bitmasks -> pair
//                 counts and stable in-block ranks
//   k_pf_scan     offsets, block bases and the grouped-GEMM tile list
//                 (128-row M-blocks of every expert, then of the shared one)
//   k_pf_scatter  perm / inv / row -> token map
//   k_pf_gemm<1>  grouped GEMM gate|up + SwiGLU -> h (bf16, sorted rows)
//   k_pf_gemm<2>  grouped GEMM down -> o (fp32, sorted rows)
//   k_pf_combine  y_t = sum_j w_tj o[inv(t, j)] (+ o[shared row of t]) (+ x_t)
//
// GEMM workgroup: 4 waves, an M-block of up to 128 sorted rows (32-row
// slices; only slices holding rows run MFMAs) by 256 output columns; wave w
// owns 64 columns as two 32-column groups.  The activation tile of each
// 128-wide K chunk is gathered by buffer DMA into double-buffered LDS (256-byte
// rows, segments XOR-swizzled by row: conflict-free b128 reads); the weights
// never touch LDS: every wave
// loads the codes of its own columns in the slot layout and dequantises them
// in registers straight into MFMA B operands, w = d*(q - o) computed exactly
// in fp32 and rounded once to bf16.  Work items are mapped XCD-aware: the
// N-tiles of one M-block run on one XCD, so its activation tile is fetched
// into that XCD's L2 once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- router statistics (load time)
// rstat[0] = max_e ||W_r[e]||_2 (rounded up), rstat[1] = max_e |b[e]|; both
// non-negative, so their fp32 bit patterns order like the values.
__global__ __launch_bounds__(256) void k_router_stats(const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
                                                      int E, int H, float* __restrict__ rstat) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    double s = 0.0;
    for (int h = lane * 8; h < H; h += 512) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Wr + (int64_t)e * H + h);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double a = bf2f(v[q] & 0xFFFFu), b = bf2f(v[q] >> 16);
            s += a * a + b * b;
        }
    }
    s = wave_sum_f64(s);
    if (lane == 0) {
        const float n = (float)sqrt(s) * 1.000001f;
        atomicMax(reinterpret_cast<unsigned int*>(rstat), __float_as_uint(n));
        if (bias) atomicMax(reinterpret_cast<unsigned int*>(rstat + 1), __float_as_uint(fabsf(bias[e])));
    }
}

// ---------------------------------------------------------------- router (MFMA, fp32)
// Grid (ceil(E/256), ceil(T/128), KS), 256 threads: workgroup (n, m, s)
// computes the 128 x 256 tile (tokens 128 m.., experts 256 n..) of the
// partial sums over K = [s H/KS, (s+1) H/KS) and stores them unrounded to
// part[s][t][e]; the top-k kernel adds the KS partials in order and the bias.
// Wave (wm, wn) owns rows 64 wm.. and columns 128 wn.. (2 x 4 MFMA tiles of
// 32 x 32).  K advances in chunks of 32: the A tile (128 rows of x) and the B
// tile (256 router rows) of a chunk, 4 16-byte segments per row, are copied to
// LDS by buffer-load DMA (each instruction fills 64 consecutive slots), three
// chunks ahead; segment p of row r sits in slot 4 r + (p ^ ((r / 4) % 4)), so
// the MFMA operand reads (32 rows, one segment) hit 32 distinct banks groups.
// A wave issues exactly 6 DMA instructions per chunk and no other vector
// loads in the loop, so "at most 6 c loads outstanding" means every chunk
// older than the c newest has landed.
constexpr int kPrRows = 128, kPrCols = 256, kPrBuf = 4;
constexpr int kPrBufBytes = (kPrRows + kPrCols) * 4 * 16;  // 24 KB per chunk
constexpr int kPrLds = kPrBuf * kPrBufBytes;

__device__ __forceinline__ void pr_wait(int chunks_after) {
    // s_waitcnt vmcnt(6 c): immediates for c = 0..2
    if (chunks_after >= 2) __builtin_amdgcn_s_waitcnt(0x0F7C);       // vmcnt(12)
    else if (chunks_after == 1) __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                         // vmcnt(0)
}

__global__ __launch_bounds__(256) void k_pf_router(const uint16_t* __restrict__ x, int T,
                                                   const uint16_t* __restrict__ Wr, int E, int H, int klen,
                                                   float* __restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int e0 = blockIdx.x * kPrCols, t0 = blockIdx.y * kPrRows, ks = blockIdx.z;
    const int nk = klen / 32;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, T * H * 2,
                                                                        0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Wr), 0, E * H * 2,
                                                                        0x00020000);
    // this wave's 6 instructions per chunk: q = wave + 4 j; q < 8 fills A slots
    // 64 q.., else B slots 64 (q - 8)..; the lane's source segment (byte offset
    // in x or Wr; the chunk adds its K offset as the scalar offset)
    uint32_t voff[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
        const int q = wave + 4 * j;
        const int slot = 64 * (q < 8 ? q : q - 8) + lane;
        const int r = slot >> 2, p = (slot & 3) ^ ((r >> 2) & 3);
        const int row = q < 8 ? min(t0 + r, T - 1) : min(e0 + r, E - 1);
        voff[j] = (uint32_t)((row * H + 8 * p) * 2);
    }
    auto issue = [&](int kc) {
        uint8_t* buf = smem + (kc % kPrBuf) * kPrBufBytes;
        const uint32_t soff = (uint32_t)((ks * klen + kc * 32) * 2);
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            const int q = wave + 4 * j;
            uint8_t* dst = buf + (q < 8 ? 0 : kPrRows * 64) + 1024 * (q < 8 ? q : q - 8);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 8 ? xr : wr, (__attribute__((address_space(3))) void*)dst,
                                                     16, voff[j], soff, 0, 0);
        }
    };
    const int wm = wave & 1, wn = wave >> 1;
    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    for (int c = 0; c < kPrBuf - 1 && c < nk; ++c) issue(c);
    for (int kc = 0; kc < nk; ++kc) {
        // this wave's DMA of chunk kc has landed; the barrier makes it so for
        // every wave (a bare barrier: a release fence would wait for the DMA
        // of the newer chunks too), and the acquire keeps the LDS reads after it
        pr_wait(min(kPrBuf - 2, nk - 1 - kc));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // the buffer of chunk kc - 1 is free: every wave has passed this barrier
        if (kc + kPrBuf - 1 < nk) issue(kc + kPrBuf - 1);
        const u32x4_t* sa = reinterpret_cast<const u32x4_t*>(smem + (kc % kPrBuf) * kPrBufBytes);
        const u32x4_t* sb = sa + kPrRows * 4;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int p = 2 * st + (lane >> 5);
            u32x4_t a[2], b[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 64 * wm + 32 * i + (lane & 31);
                a[i] = sa[4 * r + (p ^ ((r >> 2) & 3))];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 128 * wn + 32 * j + (lane & 31);
                b[j] = sb[4 * r + (p ^ ((r >> 2) & 3))];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
        }
    }
    // lane holds C[m = 8(v/4) + 4(lane/32) + v%4][n = lane%32] of each tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + 128 * wn + 32 * j + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (t < T && e < E) part[((int64_t)ks * T + t) * E + e] = acc[i][j][v];
            }
        }
}

// ---------------------------------------------------------------- top-k (exact)
// Grid ceil(T/4), 256 threads: wave w routes token 4b + w.  J = ceil(E/64)
// logits per lane.
//
// Error bound of an fp32 logit: the MFMA sum of H exact products has error at
// most H*2^-21 * sum_h |x_h w_eh| (four units of fp32 rounding per term, a
// deliberately loose constant), and sum_h |x_h w_eh| <= ||x|| ||w_e|| by
// Cauchy-Schwarz; the bias add adds one rounding of |l| <= ||x|| Wmax + Bmax.
// So every fp32 logit is within tol = H*2^-21 * (||x|| Wmax + Bmax) of the
// exact one, and any expert whose fp32 logit is below L_k - 2 tol (L_k the
// k-th largest fp32 logit) is beaten exactly by each of the k fp32 leaders:
// the exact top-k lies inside the candidate set.
// Exact logits of experts ea and eb for the token whose x row the wave holds
// in xv (lane l: elements 8 l + 512 i .. +7, zero past H): the fp64 sum of the
// exact bf16 x bf16 products in a fixed order (per lane, then the wave tree),
// plus the bias.  The result is wave-uniform.
__device__ __forceinline__ void exact_logit2(const u32x4_t (&xv)[8], const uint16_t* __restrict__ Wr,
                                             const float* __restrict__ bias, int H, int lane, int ea, int eb,
                                             double& sa, double& sb) {
    const uint16_t* wa = Wr + (int64_t)ea * H;
    const uint16_t* wb = Wr + (int64_t)eb * H;
    sa = 0.0;
    sb = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (512 * i < H) {
            const int h0 = min(lane * 8 + 512 * i, H - 8);  // lanes past H hold x = 0
            const u32x4_t va = *reinterpret_cast<const u32x4_t*>(wa + h0);
            const u32x4_t vb = *reinterpret_cast<const u32x4_t*>(wb + h0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x0 = bf2f(xv[i][q] & 0xFFFFu), x1 = bf2f(xv[i][q] >> 16);
                sa += (double)(x0 * bf2f(va[q] & 0xFFFFu));
                sa += (double)(x1 * bf2f(va[q] >> 16));
                sb += (double)(x0 * bf2f(vb[q] & 0xFFFFu));
                sb += (double)(x1 * bf2f(vb[q] >> 16));
            }
        }
    }
    sa = wave_sum_f64(sa) + (bias ? (double)bias[ea] : 0.0);
    sb = wave_sum_f64(sb) + (bias ? (double)bias[eb] : 0.0);
}

template <int J>
__global__ __launch_bounds__(256) void k_pf_topk(const uint16_t* __restrict__ x, int T,
                                                 const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
                                                 const float* __restrict__ rstat, int E, int H, int k, PrefillBufs pb,
                                                 int32_t* __restrict__ trace_ids, float* __restrict__ trace_w) {
    __shared__ int s_e[4][64 * J];
    __shared__ double s_l[4][64 * J];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // no workgroup barrier below
    // the fp32 logits' K-split partials (at most 8) are requested first, all at
    // once (clamped split index, unconditional loads), then the x row
    float pl[8][J];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int j = 0; j < J; ++j)
            pl[q][j] = pb.logits[((int64_t)min(q, pb.ksplit - 1) * T + t) * E + min(lane + 64 * j, E - 1)];
    // x row in registers (H <= 4096: 8 x 16 bytes per lane; zero past H)
    const uint16_t* xr = x + (int64_t)t * H;
    u32x4_t xv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int h0 = lane * 8 + 512 * i;
        xv[i] = *reinterpret_cast<const u32x4_t*>(xr + min(h0, H - 8));
    }
    // the bias values in one branch (its loads are waited for at the join, after the ones above)
    float bv[J];
#pragma unroll
    for (int j = 0; j < J; ++j) bv[j] = 0.f;
    if (bias) {
#pragma unroll
        for (int j = 0; j < J; ++j) bv[j] = bias[min(lane + 64 * j, E - 1)];
    }
    float lf[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        // fp32 logit: the partials added in split order (a skipped partial keeps the sum), then the bias
        float sl = pl[0][j];
#pragma unroll
        for (int q = 1; q < 8; ++q) sl = q < pb.ksplit ? sl + pl[q][j] : sl;
        lf[j] = sl + bv[j];
    }
    double xx = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (lane * 8 + 512 * i >= H) xv[i] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double a = bf2f(xv[i][q] & 0xFFFFu), b = bf2f(xv[i][q] >> 16);
            xx += a * a + b * b;
        }
    }
    const double xnorm = sqrt(wave_sum_f64(xx));
    // k-th largest fp32 logit, on 32-bit keys: the order-preserving image of
    // the logit with its low 10 bits replaced by 1023 - e (unique keys; each
    // lane's J keys sorted once, then k rounds of the wave maximum of the
    // lanes' heads).  Clearing 10 low bits never raises a key, so the value
    // read back is at most the k-th largest logit: the threshold below can
    // only admit more candidates.
    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        const uint32_t u = __float_as_uint(lf[j] + 0.0f);
        const uint32_t kf = (u >> 31) ? ~u : (u | 0x80000000u);
        key[j] = e < E ? (kf & ~0x3FFu) | (uint32_t)(1023 - e) : 0u;
    }
#pragma unroll
    for (int i = 1; i < J; ++i)
#pragma unroll
        for (int j = i; j > 0; --j) {
            const uint32_t a = key[j - 1], b = key[j];
            key[j - 1] = a > b ? a : b;
            key[j] = a > b ? b : a;
        }
    uint32_t kth = 0;
    for (int r = 0; r < k; ++r) {
        kth = wave_max_u32(key[0]);
        const uint32_t m = key[0] == kth ? ~0u : 0u;  // the owner drops its head
#pragma unroll
        for (int j = 0; j + 1 < J; ++j) key[j] = (key[j + 1] & m) | (key[j] & ~m);
        key[J - 1] &= ~m;
    }
    const uint32_t kb = kth & ~0x3FFu;
    const float kth_v = __uint_as_float((kb >> 31) ? (kb & 0x7FFFFFFFu) : ~kb);
    const double tol = ldexp((double)H, -21) * (xnorm * (double)rstat[0] + (double)rstat[1]);
    const double thr = (double)kth_v - 2.0 * tol;
    // candidate list, ascending expert id
    int nc = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const bool c = lane + 64 * j < E && (double)lf[j] >= thr;
        const uint64_t m = __ballot(c);
        if (c) s_e[wave][nc + __popcll(m & ((1ull << lane) - 1ull))] = lane + 64 * j;
        nc += __popcll(m);
    }
    if (nc < k) {  // only with non-finite inputs: take every expert, so the ids stay in range
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (lane + 64 * j < E) s_e[wave][lane + 64 * j] = lane + 64 * j;
        nc = E;
    }
    wave_lds_sync();
    // exact logits of the candidates, two per pass
    for (int r = 0; r < nc; r += 2) {
        const int ea = s_e[wave][r], eb = s_e[wave][min(r + 1, nc - 1)];
        double sa, sb;
        exact_logit2(xv, Wr, bias, H, lane, ea, eb, sa, sb);
        if (lane == 0) {
            s_l[wave][r] = sa;
            if (r + 1 < nc) s_l[wave][r + 1] = sb;
        }
    }
    wave_lds_sync();
    // exact selection among the candidates
    uint64_t ck[J];
    int cid[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int q = lane + 64 * j;
        ck[j] = q < nc ? order_key(s_l[wave][q]) : 0ull;
        cid[j] = q < nc ? s_e[wave][q] : 0x7FFFFFFF;
    }
    uint32_t used = 0;
    double my_l = 0.0;
    int my_e = 0;
    for (int r = 0; r < k; ++r) {
        uint64_t bk = 0;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (!((used >> j) & 1u) && cid[j] != 0x7FFFFFFF && ahead(ck[j], cid[j], bk, be)) { bk = ck[j]; be = cid[j]; }
        wave_argmax(bk, be);
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (cid[j] == be) used |= 1u << j;
        if (lane == r) {
            my_l = key_value(bk);
            my_e = be;
        }
    }
    // weights: softmax over the k selected exact logits (lane r holds rank r)
    const double lmax = __shfl(my_l, 0);
    const double ex = lane < k ? exp(my_l - lmax) : 0.0;
    const double z = wave_sum_f64(ex);
    if (lane < k) {
        const float wv = (float)(ex / z);
        pb.ids[(int64_t)t * k + lane] = my_e;
        pb.w[(int64_t)t * k + lane] = wv;
        if (trace_ids) trace_ids[(int64_t)t * k + lane] = my_e;
        if (trace_w) trace_w[(int64_t)t * k + lane] = wv;
    }
}

// Hash-routed layer, one wave per token: the experts of token t are row
// tok[t] (clamped into [0, vocab)) of the [vocab x k] table, in table order;
// their exact logits give the weights (softmax over the k logits, which is
// the softmax over all E renormalised over them).  No other logit is needed,
// so the layer's router GEMM does not run.
__global__ __launch_bounds__(256) void k_pf_hash(const uint16_t* __restrict__ x, int T,
                                                 const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
                                                 const int32_t* __restrict__ tab, const int32_t* __restrict__ tok,
                                                 int vocab, int H, int k, PrefillBufs pb,
                                                 int32_t* __restrict__ trace_ids, float* __restrict__ trace_w) {
    __shared__ double s_l[4][kMaxTopK];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // no workgroup barrier below
    const uint16_t* xr = x + (int64_t)t * H;
    u32x4_t xv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int h0 = lane * 8 + 512 * i;
        xv[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (h0 < H) xv[i] = *reinterpret_cast<const u32x4_t*>(xr + h0);
    }
    const int32_t* ids = tab + (int64_t)min(max(tok[t], 0), vocab - 1) * k;
    for (int r = 0; r < k; r += 2) {
        double sa, sb;
        exact_logit2(xv, Wr, bias, H, lane, ids[r], ids[min(r + 1, k - 1)], sa, sb);
        if (lane == 0) {
            s_l[wave][r] = sa;
            if (r + 1 < k) s_l[wave][r + 1] = sb;
        }
    }
    wave_lds_sync();
    const double my_l = lane < k ? s_l[wave][lane] : -HUGE_VAL;
    const int my_e = lane < k ? ids[lane] : 0;
    double lmax = my_l;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) lmax = fmax(lmax, __shfl_xor(lmax, o));
    const double ex = lane < k ? exp(my_l - lmax) : 0.0;
    const double z = wave_sum_f64(ex);
    if (lane < k) {
        const float wv = (float)(ex / z);
        pb.ids[(int64_t)t * k + lane] = my_e;
        pb.w[(int64_t)t * k + lane] = wv;
        if (trace_ids) trace_ids[(int64_t)t * k + lane] = my_e;
        if (trace_w) trace_w[(int64_t)t * k + lane] = wv;
    }
}

// ---------------------------------------------------------------- counting sort
// Grid nblk = ceil(T/256), 256 threads: thread i is token 256b + i.  A
// token's experts are distinct, so the rank of pair (t, j) inside its
// (block, expert) group is the number of earlier tokens of the block that
// chose the same expert: a popcount over that expert's token bitmask.
__global__ __launch_bounds__(256) void k_pf_hist(int T, int E, int k, PrefillBufs pb) {
    __shared__ uint32_t s_bits[kMaxExperts][kPfBlockTokens / 32];
    const int b = blockIdx.x;
    for (int i = threadIdx.x; i < E * (kPfBlockTokens / 32); i += blockDim.x) (&s_bits[0][0])[i] = 0u;
    __syncthreads();
    const int tl = threadIdx.x;
    const int t = b * kPfBlockTokens + tl;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicOr(&s_bits[pb.ids[(int64_t)t * k + j]][tl >> 5], 1u << (tl & 31));
    __syncthreads();
    if (t < T)
        for (int j = 0; j < k; ++j) {
            const int e = pb.ids[(int64_t)t * k + j];
            int r = __popc(s_bits[e][tl >> 5] & ((1u << (tl & 31)) - 1u));
            for (int w = 0; w < (tl >> 5); ++w) r += __popc(s_bits[e][w]);
            pb.rank[(int64_t)t * k + j] = r;
        }
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kPfBlockTokens / 32; ++w) c += __popc(s_bits[e][w]);
        pb.blkcnt[(int64_t)b * E + e] = (uint32_t)c;
    }
}

// Exclusive scan over the threads of the workgroup; *total = sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = 0, all = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        const int s = s_wave[w];
        base += w < wave ? s : 0;
        all += s;
    }
    __syncthreads();
    *total = all;
    return base + incl - v;
}

// One workgroup of 1024 threads; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void k_pf_scan(int T, int E, int k, int S, int nblk, PrefillBufs pb) {
    __shared__ int s_wave[16];
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E)
        for (int b = 0; b < nblk; ++b) tot += (int)pb.blkcnt[(int64_t)b * E + e];
    int all = 0;
    const int off = block_exclusive_scan(e < E ? tot : 0, s_wave, &all);
    if (e < E) {
        pb.offsets[e] = off;
        int run = off;
        for (int b = 0; b < nblk; ++b) {
            pb.blkbase[(int64_t)b * E + e] = run;
            run += (int)pb.blkcnt[(int64_t)b * E + e];
        }
    }
    // M-blocks: routed experts in ascending id, then the shared group (rows [P, P + T))
    const int nt = e < E ? (tot + kPfTileRows - 1) / kPfTileRows : 0;
    int nt_all = 0;
    const int t0 = block_exclusive_scan(nt, s_wave, &nt_all);
    for (int i = 0; i < nt; ++i) {
        int* tl = pb.tiles + 4 * (t0 + i);
        tl[0] = off + i * kPfTileRows;
        tl[1] = min(kPfTileRows, tot - i * kPfTileRows);
        tl[2] = e;
        tl[3] = 0;
    }
    const int P = T * k;
    const int nts = S ? (T + kPfTileRows - 1) / kPfTileRows : 0;
    for (int i = threadIdx.x; i < nts; i += blockDim.x) {
        int* tl = pb.tiles + 4 * (nt_all + i);
        tl[0] = P + i * kPfTileRows;
        tl[1] = min(kPfTileRows, T - i * kPfTileRows);
        tl[2] = E;
        tl[3] = 0;
    }
    if (threadIdx.x == 0) {
        pb.offsets[E] = P;
        pb.ntiles[0] = nt_all + nts;
    }
}

__global__ __launch_bounds__(256) void k_pf_scatter(int T, int E, int k, int S, PrefillBufs pb) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int P = T * k;
    if (i < P) {
        const int t = i / k;
        const int e = pb.ids[i];
        const int pos = pb.blkbase[(int64_t)(t / kPfBlockTokens) * E + e] + pb.rank[i];
        pb.perm[pos] = i;
        pb.inv[i] = pos;
        pb.rowtok[pos] = t;
    } else if (S && i < P + T) {
        pb.rowtok[i] = i - P;
    }
}

// ---------------------------------------------------------------- grouped GEMMs
// Activation tile of one 128-wide K chunk: 128 rows of 256 bytes, written by
// direct global->LDS loads.  Slot p of row r holds the row's 16-byte segment
// p ^ (r % 16), so the b128 fragment reads of 16 consecutive rows at one
// segment hit 16 distinct bank groups.
constexpr int kATileBytes = 128 * 256;
constexpr int kGemmLds = 2 * kATileBytes;  // double buffer
// VALU instructions of one K step's dequantisation (two B operands), spread
// over the step's MFMAs by the scheduling groups
constexpr int kDeqValu = 40;

// Work item of block b.  Workgroups are dealt to the 8 XCDs round-robin, so
// block b runs on XCD x = b % 8 as its slot s = b / 8 there.  M-blocks are
// dealt to the XCDs round-robin too (the i-th M-block of XCD x is list entry
// x + 8 i, counted from the end of the list), and slot s holds N-tile s % ntn
// of that XCD's M-block s / ntn: the N-tiles of an M-block run one after the
// other on one XCD (its activation tile is fetched into that L2 once), and
// large and small groups spread evenly over the XCDs.  The list ends with
// the shared expert's full blocks, so walking it backwards starts each XCD
// on the longest items.  The grid holds 8 ceil(ntiles / 8) ntn blocks.
__device__ __forceinline__ bool pf_item(int ntn, int ntiles, int& m, int& n) {
    const int b = blockIdx.x, x = b & 7, s = b >> 3;
    const int i = s / ntn;
    const int mi = x + 8 * i;
    if (mi >= ntiles) return false;
    m = ntiles - 1 - mi;
    n = s - i * ntn;
    return true;
}

// Raw codes of one chunk for one 32-column group, as the lane needs them for
// v_mfma_f32_32x32x16_bf16: lane l (column n = l%32, half = l/32) holds the
// slot-lanes (n%16, g = half) and (n%16, g = half + 2) of its row tile, i.e.
// elements 8 half..+7 and 16 + 8 half..+7 of each block, plus the row's four
// block scales.
template <int FMT> struct BCodes;
template <> struct BCodes<1> { u32x4_t c0, c1; u32x2_t sc; };
template <> struct BCodes<2> { u32x2_t c0, c1; u32x2_t sc; };
template <> struct BCodes<3> { u32x2_t c0, c1; u32x2_t sc; };  // q2 codes; sc.x = the two 64-block scales

// Weight codes and activations are read through buffer resources: the
// wave-uniform base and the chunk's offset live in scalar registers, the
// lane's offset is a loop-invariant 32-bit register, so advancing a chunk
// costs no vector instruction.  dword3 0x00020000: raw 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Codes of one chunk: soff = the chunk's byte offset in the expert slot;
// offc / offs = the lane's byte offsets of its first code word and of its
// scales in a chunk; lstr = the byte stride of the slot's code lanes (16 for
// q4, and for the interleaved G|U units of q2 / q2b64; 8 for their D).  A row
// tile past the matrix (N not a multiple of the tile) reads the last one
// again: the columns it feeds are never stored.
template <int FMT>
__device__ __forceinline__ void load_bcodes(BCodes<FMT>& b, __amdgpu_buffer_rsrc_t r, uint32_t soff, uint32_t offc,
                                            uint32_t offs, uint32_t lstr) {
    if constexpr (FMT == 1) {
        b.c0 = __builtin_amdgcn_raw_buffer_load_b128(r, offc, soff, 0);
        b.c1 = __builtin_amdgcn_raw_buffer_load_b128(r, offc + 32 * 16, soff, 0);
    } else {
        b.c0 = __builtin_amdgcn_raw_buffer_load_b64(r, offc, soff, 0);
        b.c1 = __builtin_amdgcn_raw_buffer_load_b64(r, offc + 32 * lstr, soff, 0);
    }
    if constexpr (FMT == 3)
        b.sc = u32x2_t{__builtin_amdgcn_raw_buffer_load_b32(r, offs, soff, 0), 0u};
    else
        b.sc = __builtin_amdgcn_raw_buffer_load_b64(r, offs, soff, 0);
}

__device__ __forceinline__ float h16lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)); }
__device__ __forceinline__ float h16hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// 8 consecutive weights d*(q - o) as a bf16 B operand.  One and-or puts two
// codes into an fp16 pair as 0x6400 | q = 1024 + q (exact), and one fma per
// weight, d (1024 + q) + c with c = -(1024 + o) d, gives the exact weight:
// c is exact in fp32 (d's 11 significant bits times 129 or 513), the product
// is formed exactly inside the fma, and d (q - o) has at most 15 significant
// bits.  The pack rounds it once to bf16.  v_fma_mix_f32 takes d and the
// codes as fp16 operands (either half of a register), c as fp32.
// kb: 0x64006400 held in a VGPR, so that the mask-and-or is one v_and_or_b32
// (VOP3 takes at most one scalar or constant operand, which the mask uses).
__device__ __forceinline__ uint32_t fp16_bias_bits() {
    uint32_t k;
    asm("v_mov_b32 %0, 0x64006400" : "=v"(k));
    return k;
}
// q4 word: nibble p (bits 4p) = element 2p, nibble p+4 (bits 16+4p) = element 2p+1.
__device__ __forceinline__ u32x4_t deq_q4(uint32_t w, float d, float c, uint32_t kb) {
    u32x4_t r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t v = ((w >> (4 * p)) & 0x000F000Fu) | kb;
        r[p] = pack_bf16(fmaf(d, h16lo(v), c), fmaf(d, h16hi(v), c));
    }
    return r;
}
// q2 (block bits already at 0..7 and 16..23): bits 2p = element 2p, bits 16+2p = element 2p+1.
__device__ __forceinline__ u32x4_t deq_q2(uint32_t w, float d, float c, uint32_t kb) {
    u32x4_t r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t v = ((w >> (2 * p)) & 0x00030003u) | kb;
        r[p] = pack_bf16(fmaf(d, h16lo(v), c), fmaf(d, h16hi(v), c));
    }
    return r;
}
// B operand of K step ks (block ks / 2: lo half for even ks, hi half for odd);
// a dead chunk (live false) gets zero scales.
// sc: the row's four fp16 block scales (zeroed for a dead chunk).
// (Written with scalar halves: the same product over bit-cast f16x2 words
// has been compiled to reuse the first word's products for the second.)
// (q2b64: block j of 32 weights takes the scale of 64-block j / 2, in sc.x.)
template <int FMT> __device__ __forceinline__ _Float16 scale_h(u32x2_t s, int j) {
    if constexpr (FMT == 3) return __builtin_bit_cast(_Float16, (uint16_t)((j & 2) ? (s.x >> 16) : (s.x & 0xFFFFu)));
    const uint32_t w = (j & 2) ? s.y : s.x;
    return __builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFFu)));
}
template <int FMT>
__device__ __forceinline__ u32x4_t deq_half(const BCodes<FMT>& b, int ks, u32x2_t sc, uint32_t kb) {
    const int j = ks >> 1;
    const float d = (float)scale_h<FMT>(sc, j);
    const float c = d * (FMT == 1 ? -1032.f : -1026.f);
    if constexpr (FMT == 1) {
        return deq_q4((ks & 1) ? b.c1[j] : b.c0[j], d, c, kb);
    } else {
        return deq_q2(((ks & 1) ? b.c1[j >> 1] : b.c0[j >> 1]) >> (8 * (j & 1)), d, c, kb);
    }
}

// Per-thread state of one GEMM work item, shared by the slice-count
// specialisations of the main loop.
// Every load address is a wave-uniform base plus a 32-bit lane offset, so the
// loads take the scalar-base form and the per-chunk address math is scalar.
struct GemmItem {
    __amdgpu_buffer_rsrc_t ar;  // activation rows (x, or the M-block's rows of h)
    __amdgpu_buffer_rsrc_t br;  // the group's expert slot
    uint32_t aoff[8];           // byte offsets of this lane's 8 A segments in chunk 0 (rows past nrows repeat the last)
    uint32_t boffc[2];          // per 32-column group: byte offset of this lane's code words in chunk 0
    uint32_t boffs[2];          // ... and of its row's scales
    int row0, nrows, nt, wave, nk, K;
    uint32_t chunk_bytes;       // byte stride of consecutive chunks of a row tile
    uint32_t lstr;              // byte stride of the code lanes of a chunk
};

// Main loop and epilogue for NS 32-row slices.  Every slice of the item holds
// at least one row, so the loop body is branch-free: per 32-wide K block the
// wave dequantises the four B operands it needs, reads the 2 NS activation
// fragments, and issues 4 NS MFMAs.  Chunk kc + 1 (activations by DMA into the
// other LDS buffer, weight codes into registers) is requested before chunk kc
// is computed.
template <int FMT, int MODE, int NS>
__device__ __forceinline__ void gemm_item(GemmItem& it, uint8_t* As, const Geom& g, const PrefillBufs& pb) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = lane & 31, half = lane >> 5;
    // wave w loads the rows of slice w: instruction q covers rows 32w + 4q .. +3,
    // lane l writes slot l % 16 of row 32w + 4q + l / 16.  A segment past K
    // is replaced by the row's last one (its weights are zero).  The loads are
    // issued without branches (the waits of a load under a branch are placed
    // at the join), so waves past the last slice load rows no one reads.
    auto load_a = [&](int kc, int buf) {
        uint8_t* dst = As + buf * kATileBytes + it.wave * 8192;
        const uint32_t soff = (uint32_t)kc * 256;
        if (kc * 128 + 128 <= it.K) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(it.ar, (__attribute__((address_space(3))) void*)(dst + q * 1024),
                                                         16, it.aoff[q], soff, 0, 0);
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int e = kc * 128 + 8 * ((lane & 15) ^ ((4 * q + (lane >> 4)) & 15));
                const uint32_t over = (uint32_t)max(e - (it.K - 8), 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(it.ar, (__attribute__((address_space(3))) void*)(dst + q * 1024),
                                                         16, it.aoff[q] - 2 * over, soff, 0, 0);
            }
        }
    };
    f32x16_t acc[NS][2];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[s][gi][i] = 0.f;

    // weight codes of even chunks in bc0, odd chunks in bc1 (no copies between chunks)
    BCodes<FMT> bc0[2], bc1[2];
    load_a(0, 0);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) load_bcodes<FMT>(bc0[gi], it.br, 0u, it.boffc[gi], it.boffs[gi], it.lstr);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
    __syncthreads();
    // LDS byte offset of this lane's fragment row (slice 0) and its segment swizzle
    const uint8_t* al0 = As + (lane & 31) * 256;
    const int swz = lane & 15;
    const uint32_t kb = fp16_bias_bits();
    // chunk kc >= nk (the partner of the last chunk when nk is odd) repeats the
    // last chunk's data with zero scales: it adds exact zeros
    auto chunk = [&](int kc, int buf, const BCodes<FMT>(&cb)[2], BCodes<FMT>(&nb)[2]) {
        const bool live = kc < it.nk;
        const int kn = min(kc + 1, it.nk - 1);  // past the end: the last chunk again
        load_a(kn, buf ^ 1);
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
            load_bcodes<FMT>(nb[gi], it.br, (uint32_t)kn * it.chunk_bytes, it.boffc[gi], it.boffs[gi], it.lstr);
        // the next chunk is requested before this chunk's work (the scheduler
        // would otherwise sink the loads to their use)
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* al = al0 + buf * kATileBytes;
        // 16-wide K steps (block ks / 2, half ks % 2), software-pipelined: the
        // activation fragments and the dequantised weights of step ks + 1 are
        // prepared while the MFMAs of step ks run
        auto read_a = [&](int ks, u32x4_t (&af)[NS]) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                af[s] = *reinterpret_cast<const u32x4_t*>(al + s * 8192 + (((2 * ks + half) ^ swz) << 4));
        };
        u32x2_t sc[2];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) sc[gi] = live ? cb[gi].sc : u32x2_t{0u, 0u};
        u32x4_t afc[NS], b0c, b1c;
        read_a(0, afc);
        b0c = deq_half<FMT>(cb[0], 0, sc[0], kb);
        b1c = deq_half<FMT>(cb[1], 0, sc[1], kb);
        // issue order of this region: step 0's reads and dequantisation, then
        // per step the next step's reads followed by its MFMAs, each MFMA
        // followed by a share of the next step's dequantisation
        __builtin_amdgcn_sched_group_barrier(0x100, NS, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kDeqValu, 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4_t afn[NS], b0n, b1n;
            if (ks < 7) {
                read_a(ks + 1, afn);
                b0n = deq_half<FMT>(cb[0], ks + 1, sc[0], kb);
                b1n = deq_half<FMT>(cb[1], ks + 1, sc[1], kb);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                acc[s][0] = mfma32(afc[s], b0c, acc[s][0]);
                acc[s][1] = mfma32(afc[s], b1c, acc[s][1]);
            }
            if (ks < 7) {
#pragma unroll
                for (int s = 0; s < NS; ++s) afc[s] = afn[s];
                b0c = b0n;
                b1c = b1n;
                __builtin_amdgcn_sched_group_barrier(0x100, NS, 0);
            }
#pragma unroll
            for (int i = 0; i < 2 * NS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, (kDeqValu + 2 * NS - 1) / (2 * NS), 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): chunk kc + 1 has landed
        __syncthreads();
    };
    // pairs of chunks without a branch between them: a load whose only use
    // sits under a branch is moved there by the compiler, past the barrier
    for (int kc = 0; kc < it.nk; kc += 2) {
        chunk(kc, 0, bc0, bc1);
        chunk(kc + 1, 1, bc1, bc0);
    }
    // epilogue: lane holds C[m = 32 s + 8(i/4) + 4 half + i%4][column n] of both groups
    if constexpr (MODE == 1) {
        // SwiGLU -> bf16 tile [row][128 features] in LDS (the activation
        // buffers are idle after the last barrier), then 16-byte row stores
        uint16_t* hl = reinterpret_cast<uint16_t*>(As);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = s * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                const float gv = acc[s][0][i], uv = acc[s][1][i];
                hl[m * 128 + 32 * it.wave + n] = (uint16_t)f2bf(gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv);
            }
        __syncthreads();
        const int nfe = min(128, g.F - it.nt * 128);  // features of this tile (a multiple of 32)
#pragma unroll
        for (int q = 0; q < 2 * NS; ++q) {
            const int idx = tid + 256 * q, r = idx >> 4, c8 = (idx & 15) * 8;
            if (r < it.nrows && c8 < nfe)
                *reinterpret_cast<u32x4_t*>(pb.h + (int64_t)(it.row0 + r) * g.F + it.nt * 128 + c8) =
                    *reinterpret_cast<const u32x4_t*>(hl + r * 128 + c8);
        }
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = s * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                if (m < it.nrows) {
#pragma unroll
                    for (int gi = 0; gi < 2; ++gi) {
                        const int col = it.nt * 256 + 64 * it.wave + 32 * gi + n;
                        if (col < g.H) pb.o[(int64_t)(it.row0 + m) * g.H + col] = acc[s][gi][i];
                    }
                }
            }
        }
    }
}

// MODE 1: A = gathered x rows, K = H; group 0 = G rows, group 1 = the same U
// rows; epilogue SwiGLU -> h.  MODE 2: A = h rows, K = F; groups = two
// consecutive 32-row stripes of D; epilogue -> o.
template <int FMT, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_pf_gemm(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ slots, Geom g, PrefillBufs pb, int ntn) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int mt, nt;
    if (!pf_item(ntn, pb.ntiles[0], mt, nt)) return;
    const int* tl = pb.tiles + 4 * mt;
    GemmItem it;
    it.row0 = tl[0];
    it.nrows = tl[1];
    const int grp = tl[2];
    it.nt = nt;
    const int tid = threadIdx.x, lane = tid & 63;
    it.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nslice = (it.nrows + 31) >> 5;
    it.K = MODE == 1 ? g.H : g.F;
    const MatGeom& mg = MODE == 1 ? g.gu : g.dn;
    it.nk = mg.nch;
    // q2 / q2b64 store G and U, and D's row tiles 2 rp, 2 rp + 1, in interleaved units of two chunks' size
    constexpr bool il = FMT != 1;
    it.chunk_bytes = (uint32_t)mg.chunk_bytes * (il ? 2u : 1u);
    it.lstr = il ? 16u : (uint32_t)QF<FMT>::kCW;
    it.br = make_rsrc(slots + (int64_t)grp * g.slot_bytes, (uint32_t)g.slot_bytes);
    const int n = lane & 31, half = lane >> 5;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
        int rt;
        uint32_t base;
        if constexpr (MODE == 1) {
            rt = nt * 8 + 2 * it.wave + (n >> 4);
            base = (uint32_t)(gi ? g.u_off : g.g_off);
        } else {
            rt = nt * 16 + 4 * it.wave + 2 * gi + (n >> 4);
            base = (uint32_t)g.d_off;
        }
        // lane l takes the slot-lanes (n % 16, half) and (n % 16, half + 2) of its row tile;
        // interleaved units: G's (D: the even tile's) bytes first in every lane entry and
        // scale row, then U's (the odd tile's)
        constexpr uint32_t sb = FMT == 3 ? 4 : 8;
        const uint32_t rtc = (uint32_t)min(rt, mg.rows / 16 - 1);
        const uint32_t urow = il && MODE == 2 ? rtc >> 1 : rtc;  // unit row of the tile
        const uint32_t tile = base + urow * (uint32_t)mg.nch * it.chunk_bytes;
        const uint32_t part = !il ? 0u : MODE == 1 ? (uint32_t)gi : (rtc & 1u);
        it.boffc[gi] = tile + (uint32_t)((n & 15) + 16 * half) * it.lstr + part * QF<FMT>::kCW;
        it.boffs[gi] = tile + 64 * it.lstr + (uint32_t)(n & 15) * sb * (il ? 2u : 1u) + part * sb;
    }
    // A: lane l of instruction q of wave w fetches segment (l % 16) ^ (r % 16)
    // of tile row r = 32 w + 4 q + l / 16
    // (MODE 2: the M-block's rows are contiguous in h; its first row goes into
    // the base, so the lane offsets stay below 128 F 2 bytes)
    if constexpr (MODE == 1)
        it.ar = make_rsrc(x, (uint32_t)(pb.T * g.H * 2));
    else
        it.ar = make_rsrc(pb.h + (int64_t)it.row0 * g.F, (uint32_t)(it.nrows * g.F * 2));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int r = 32 * it.wave + 4 * q + (lane >> 4);
        const int rr = min(r, it.nrows - 1);
        const uint32_t seg = (uint32_t)((lane & 15) ^ (r & 15));
        if constexpr (MODE == 1)
            it.aoff[q] = 2 * ((uint32_t)pb.rowtok[it.row0 + rr] * (uint32_t)g.H + 8 * seg);
        else
            it.aoff[q] = 2 * ((uint32_t)rr * (uint32_t)g.F + 8 * seg);
    }
    uint8_t* As = smem;
    switch (nslice) {
        case 1: gemm_item<FMT, MODE, 1>(it, As, g, pb); break;
        case 2: gemm_item<FMT, MODE, 2>(it, As, g, pb); break;
        case 3: gemm_item<FMT, MODE, 3>(it, As, g, pb); break;
        default: gemm_item<FMT, MODE, 4>(it, As, g, pb); break;
    }
}

// ---------------------------------------------------------------- combine
// Thread per (token, 4 consecutive columns): the k routed rows in slot order,
// then the shared row, then the residual.
template <int KM>
__global__ __launch_bounds__(256) void k_pf_combine(const uint16_t* __restrict__ x, int T, int H, int k, int S,
                                                    PrefillBufs pb, uint16_t* __restrict__ y, int residual) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int h4 = H / 4;
    if (i >= T * h4) return;
    const int t = i / h4, c = (i - t * h4) * 4;
    // every row index and weight first, then every row (read once: non-temporal),
    // so the k + 1 rows cost one memory round trip after the indices; k <= KM
    int64_t row[KM];
    float w[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        const int jj = min(j, k - 1);
        row[j] = pb.inv[(int64_t)t * k + jj];
        w[j] = pb.w[(int64_t)t * k + jj];
    }
    u32x2_t xv = {0u, 0u};
    if (residual) xv = *reinterpret_cast<const u32x2_t*>(x + (int64_t)t * H + c);
    f32x4_t o[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
        o[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pb.o + row[j] * H + c));
    // the shared row exists only with S; without it the load repeats row 0's and is unused
    const int64_t srow = S ? (int64_t)T * k + t : row[0];
    const f32x4_t os = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pb.o + srow * H + c));
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KM; ++j)
        if (j < k) {
#pragma unroll
            for (int q = 0; q < 4; ++q) s[q] += w[j] * o[j][q];
        }
    if (S) {
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] += os[q];
    }
    uint32_t out[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        float a = s[2 * q], b = s[2 * q + 1];
        if (residual) {
            a += bf2f(xv[q] & 0xFFFFu);
            b += bf2f(xv[q] >> 16);
        }
        out[q] = f2bf(a) | (f2bf(b) << 16);
    }
    *reinterpret_cast<u32x2_t*>(y + (int64_t)t * H + c) = u32x2_t{out[0], out[1]};
}

// ---------------------------------------------------------------- launchers
hipError_t launch_router_stats(const uint16_t* Wr, const float* bias, int E, int H, float* rstat, hipStream_t st) {
    hipError_t e = hipMemsetAsync(rstat, 0, 2 * sizeof(float), st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_router_stats, dim3((E + 3) / 4), dim3(256), 0, st, Wr, bias, E, H, rstat);
    return hipGetLastError();
}

hipError_t launch_pf_router(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const Geom& g,
                            PrefillBufs pb, const Launch& lc) {
    (void)bias;  // added by the top-k kernel
    static LdsGrant granted;
    hipError_t e = ensure_lds(k_pf_router, kPrLds, granted);
    if (e != hipSuccess) return e;
    const int ks = pf_router_splits(T, g.E, g.H);
    launch(k_pf_router, dim3((g.E + kPrCols - 1) / kPrCols, (T + kPrRows - 1) / kPrRows, ks), dim3(256), kPrLds, lc,
           x, T, Wr, g.E, g.H, g.H / ks, pb.logits);
    return hipGetLastError();
}

hipError_t launch_pf_topk(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const float* rstat,
                          const Geom& g, PrefillBufs pb, int32_t* trace_ids, float* trace_w, const Launch& lc) {
    pb.ksplit = pf_router_splits(T, g.E, g.H);
    const dim3 grid((T + 3) / 4);
    if (g.E <= 64)
        launch(k_pf_topk<1>, grid, dim3(256), 0, lc, x, T, Wr, bias, rstat, g.E, g.H, g.k, pb, trace_ids, trace_w);
    else if (g.E <= 256)
        launch(k_pf_topk<4>, grid, dim3(256), 0, lc, x, T, Wr, bias, rstat, g.E, g.H, g.k, pb, trace_ids, trace_w);
    else if (g.E <= 512)
        launch(k_pf_topk<8>, grid, dim3(256), 0, lc, x, T, Wr, bias, rstat, g.E, g.H, g.k, pb, trace_ids, trace_w);
    else
        launch(k_pf_topk<16>, grid, dim3(256), 0, lc, x, T, Wr, bias, rstat, g.E, g.H, g.k, pb, trace_ids, trace_w);
    return hipGetLastError();
}

hipError_t launch_pf_hash(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const int32_t* tab,
                          const int32_t* tok, int vocab, const Geom& g, PrefillBufs pb, int32_t* trace_ids,
                          float* trace_w, const Launch& lc) {
    launch(k_pf_hash, dim3((T + 3) / 4), dim3(256), 0, lc, x, T, Wr, bias, tab, tok, vocab, g.H, g.k, pb, trace_ids,
           trace_w);
    return hipGetLastError();
}

hipError_t launch_pf_hist(int T, const Geom& g, PrefillBufs pb, const Launch& lc) {
    launch(k_pf_hist, dim3((T + kPfBlockTokens - 1) / kPfBlockTokens), dim3(256), 0, lc, T, g.E, g.k, pb);
    return hipGetLastError();
}

hipError_t launch_pf_scan(int T, const Geom& g, PrefillBufs pb, const Launch& lc) {
    const int nblk = (T + kPfBlockTokens - 1) / kPfBlockTokens;
    launch(k_pf_scan, dim3(1), dim3(1024), 0, lc, T, g.E, g.k, g.S, nblk, pb);
    return hipGetLastError();
}

hipError_t launch_pf_scatter(int T, const Geom& g, PrefillBufs pb, const Launch& lc) {
    launch(k_pf_scatter, dim3((T * g.k + T + 255) / 256), dim3(256), 0, lc, T, g.E, g.k, g.S, pb);
    return hipGetLastError();
}

template <int FMT, int MODE>
static hipError_t launch_gemm(const uint16_t* x, const uint8_t* slots, const Geom& g, PrefillBufs pb,
                              const Launch& lc) {
    static LdsGrant granted;
    hipError_t e = ensure_lds(k_pf_gemm<FMT, MODE>, kGemmLds, granted);
    if (e != hipSuccess) return e;
    const int ntn = MODE == 1 ? (g.F + 127) / 128 : (g.H + 255) / 256;
    launch(k_pf_gemm<FMT, MODE>, dim3(((pb.max_tiles + 7) & ~7) * ntn), dim3(256), kGemmLds, lc, x, slots, g, pb, ntn);
    return hipGetLastError();
}

hipError_t launch_pf_gemm1(const uint16_t* x, int T, const uint8_t* layer_slots, const Geom& g, PrefillBufs pb,
                           const Launch& lc) {
    pb.T = T;
    switch (g.fmt) {
        case 1: return launch_gemm<1, 1>(x, layer_slots, g, pb, lc);
        case 2: return launch_gemm<2, 1>(x, layer_slots, g, pb, lc);
        default: return launch_gemm<3, 1>(x, layer_slots, g, pb, lc);
    }
}

hipError_t launch_pf_gemm2(const uint8_t* layer_slots, const Geom& g, PrefillBufs pb, const Launch& lc) {
    switch (g.fmt) {
        case 1: return launch_gemm<1, 2>(nullptr, layer_slots, g, pb, lc);
        case 2: return launch_gemm<2, 2>(nullptr, layer_slots, g, pb, lc);
        default: return launch_gemm<3, 2>(nullptr, layer_slots, g, pb, lc);
    }
}

hipError_t launch_pf_combine(const uint16_t* x, int T, const Geom& g, PrefillBufs pb, uint16_t* y, int residual,
                             const Launch& lc) {
    const dim3 grid((T * (g.H / 4) + 255) / 256);
    if (g.k <= 8)
        launch(k_pf_combine<8>, grid, dim3(256), 0, lc, x, T, g.H, g.k, g.S, pb, y, residual);
    else
        launch(k_pf_combine<kMaxTopK>, grid, dim3(256), 0, lc, x, T, g.H, g.k, g.S, pb, y, residual);
    return hipGetLastError();
}

}  // namespace moe
