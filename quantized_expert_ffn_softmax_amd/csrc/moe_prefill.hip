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
//   k_pf_router   logits = x Wr^T + b on v_mfma_f32_32x32x16_bf16 (fp32)
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
// 128-wide K chunk is gathered into double-buffered LDS (rows padded to 272
// bytes, conflict-free b128 reads); the weights never touch LDS: every wave
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
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}
// (lo, hi) -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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
// Grid (ceil(E/64), ceil(T/64)), 256 threads: wave (wm, wn) computes a 32x32
// tile of logits, A = x rows (tokens), B = router rows (experts), straight
// from global memory (rows clamped, results masked).  Lane l holds row l%32,
// k = 8(l/32)..+7 of each 16-wide K step.
__global__ __launch_bounds__(256) void k_pf_router(const uint16_t* __restrict__ x, int T,
                                                   const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
                                                   int E, int H, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.y * 64 + (wave >> 1) * 32, e0 = blockIdx.x * 64 + (wave & 1) * 32;
    const int tr = min(t0 + (lane & 31), T - 1), er = min(e0 + (lane & 31), E - 1);
    const uint16_t* xa = x + (int64_t)tr * H + 8 * (lane >> 5);
    const uint16_t* wb = Wr + (int64_t)er * H + 8 * (lane >> 5);
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    int k0 = 0;
    for (; k0 + 64 <= H; k0 += 64) {
        u32x4_t a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = *reinterpret_cast<const u32x4_t*>(xa + k0 + 16 * j);
            b[j] = *reinterpret_cast<const u32x4_t*>(wb + k0 + 16 * j);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma32(a[j], b[j], acc);
    }
    for (; k0 < H; k0 += 16)
        acc = mfma32(*reinterpret_cast<const u32x4_t*>(xa + k0), *reinterpret_cast<const u32x4_t*>(wb + k0), acc);
    // lane holds C[m = 8(i/4) + 4(lane/32) + i%4][n = lane%32]
    const int e = e0 + (lane & 31);
    const float be = (bias && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = t0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (t < T && e < E) logits[(int64_t)t * E + e] = acc[i] + be;
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
    // x row in registers (H <= 4096: 8 x 16 bytes per lane; zero past H)
    const uint16_t* xr = x + (int64_t)t * H;
    u32x4_t xv[8];
    double xx = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int h0 = lane * 8 + 512 * i;
        xv[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (h0 < H) xv[i] = *reinterpret_cast<const u32x4_t*>(xr + h0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double a = bf2f(xv[i][q] & 0xFFFFu), b = bf2f(xv[i][q] >> 16);
            xx += a * a + b * b;
        }
    }
    const double xnorm = sqrt(wave_sum_f64(xx));
    // k-th largest fp32 logit
    float lf[J];
    uint64_t key[J];
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        lf[j] = pb.logits[(int64_t)t * E + min(e, E - 1)];
        key[j] = order_key((double)lf[j]);
        if (e >= E) taken |= 1u << j;
    }
    uint64_t kth = 0;
    for (int r = 0; r < k; ++r) {
        uint64_t bk = 0;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (!((taken >> j) & 1u) && ahead(key[j], lane + 64 * j, bk, be)) { bk = key[j]; be = lane + 64 * j; }
        wave_argmax(bk, be);
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        kth = bk;
    }
    const double tol = ldexp((double)H, -21) * (xnorm * (double)rstat[0] + (double)rstat[1]);
    const double thr = key_value(kth) - 2.0 * tol;
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
        const uint16_t* wa = Wr + (int64_t)ea * H;
        const uint16_t* wb = Wr + (int64_t)eb * H;
        double sa = 0.0, sb = 0.0;
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
constexpr int kLdsRow = 136;                // bf16 per LDS row: 128 + 8 (rows 272 bytes apart: b128 reads conflict-free)
constexpr int kLdsTile = 128 * kLdsRow;     // one activation tile (elements)
constexpr int kGemmLds = 2 * kLdsTile * 2;  // double buffer, bytes

// Work item of block b: V = ntiles * ntn items, item i = (M-block i / ntn,
// N-tile i % ntn).  Workgroups are dealt to the 8 XCDs round-robin (b % 8), so
// XCD x is given the contiguous item range [x V/8, (x+1) V/8) (remainder to
// the first XCDs): all N-tiles of an M-block share one XCD's L2.
__device__ __forceinline__ bool pf_item(int ntn, int ntiles, int& m, int& n) {
    const int V = ntiles * ntn;
    const int b = blockIdx.x;
    if (b >= V) return false;
    const int xcd = b & 7, s = b >> 3;
    const int q = V >> 3, r = V & 7;
    const int L = xcd * q + min(xcd, r) + s;
    m = L / ntn;
    n = L - m * ntn;
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

template <int FMT>
__device__ __forceinline__ void load_bcodes(BCodes<FMT>& b, const uint8_t* chunk, int n16, int half, bool valid) {
    if constexpr (FMT == 1) {
        b.c0 = *reinterpret_cast<const u32x4_t*>(chunk + (n16 + 16 * half) * 16);
        b.c1 = *reinterpret_cast<const u32x4_t*>(chunk + (n16 + 16 * (half + 2)) * 16);
    } else {
        b.c0 = *reinterpret_cast<const u32x2_t*>(chunk + (n16 + 16 * half) * 8);
        b.c1 = *reinterpret_cast<const u32x2_t*>(chunk + (n16 + 16 * (half + 2)) * 8);
    }
    b.sc = *reinterpret_cast<const u32x2_t*>(chunk + 64 * QF<FMT>::kCW + n16 * 8);
    if (!valid) b.sc = u32x2_t{0u, 0u};  // row tile past the matrix: zero weights
}

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

// 8 consecutive weights d*(q - o) as a bf16 B operand.  d*q is exact in fp32
// (11 + 4 significant bits) and -o*d is exact (o a power of two), so the fma
// is the exact weight; the pack rounds it once to bf16.
// q4 word: nibble p (bits 4p) = element 2p, nibble p+4 (bits 16+4p) = element 2p+1.
__device__ __forceinline__ u32x4_t deq_q4(uint32_t w, float d) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // bytes: e0 e4 e1 e5
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // bytes: e2 e6 e3 e7
    const float c = -8.f * d;
    return u32x4_t{pack_bf16(fmaf(d, ub0(lo), c), fmaf(d, ub2(lo), c)),
                   pack_bf16(fmaf(d, ub0(hi), c), fmaf(d, ub2(hi), c)),
                   pack_bf16(fmaf(d, ub1(lo), c), fmaf(d, ub3(lo), c)),
                   pack_bf16(fmaf(d, ub1(hi), c), fmaf(d, ub3(hi), c))};
}
// q2 (block bits already at 0..7 and 16..23): bits 2p = element 2p, bits 16+2p = element 2p+1.
__device__ __forceinline__ u32x4_t deq_q2(uint32_t w, float d) {
    const float c = -2.f * d;
    u32x4_t r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t v = (w >> (2 * p)) & 0x00030003u;
        r[p] = pack_bf16(fmaf(d, ub0(v), c), fmaf(d, ub2(v), c));
    }
    return r;
}
// B operands of block j: K steps 2j (lo) and 2j+1 (hi).
template <int FMT>
__device__ __forceinline__ void deq_block(const BCodes<FMT>& b, int j, u32x4_t& lo, u32x4_t& hi) {
    const float d = scale_of(b.sc, j);
    if constexpr (FMT == 1) {
        lo = deq_q4(b.c0[j], d);
        hi = deq_q4(b.c1[j], d);
    } else {
        lo = deq_q2(b.c0[j >> 1] >> (8 * (j & 1)), d);
        hi = deq_q2(b.c1[j >> 1] >> (8 * (j & 1)), d);
    }
}

// MODE 1: A = gathered x rows, K = H; group 0 = G rows, group 1 = the same U
// rows; epilogue SwiGLU -> h.  MODE 2: A = h rows, K = F; groups = two
// consecutive 32-row stripes of D; epilogue -> o.
template <int FMT, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_pf_gemm(const uint16_t* __restrict__ x, const uint8_t* __restrict__ slots,
                                                 Geom g, PrefillBufs pb, int ntn) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int mt, nt;
    if (!pf_item(ntn, pb.ntiles[0], mt, nt)) return;
    const int* tl = pb.tiles + 4 * mt;
    const int row0 = tl[0], nrows = tl[1], grp = tl[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nslice = (nrows + 31) >> 5;
    uint16_t* As = reinterpret_cast<uint16_t*>(smem);
    const int K = MODE == 1 ? g.H : g.F;
    const MatGeom& mg = MODE == 1 ? g.gu : g.dn;
    const int nk = mg.nch;
    const uint8_t* slot = slots + (int64_t)grp * g.slot_bytes;
    // B: this lane's row tiles of the two groups
    const int n = lane & 31, half = lane >> 5;
    const uint8_t* bt[2];
    bool bvalid[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
        int rt;
        const uint8_t* base;
        if constexpr (MODE == 1) {
            rt = nt * 8 + 2 * wave + (n >> 4);
            base = slot + (gi ? g.u_off : g.g_off);
        } else {
            rt = nt * 16 + 4 * wave + 2 * gi + (n >> 4);
            base = slot + g.d_off;
        }
        bvalid[gi] = rt < mg.rows / 16;
        bt[gi] = base + (int64_t)min(rt, mg.rows / 16 - 1) * mg.tile_bytes;
    }
    // A: 128 rows x 16 segments of 16 bytes per chunk, 8 per thread (rows past nrows repeat the last)
    const uint16_t* abase = MODE == 1 ? x : pb.h;
    uint32_t aoff[8];  // element offsets (< 2^32: T*H and (T*k + T)*F are bounded by the context limits)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int i = tid + 256 * q;
        const int r = min(i >> 4, nrows - 1);
        if constexpr (MODE == 1)
            aoff[q] = (uint32_t)pb.rowtok[row0 + r] * (uint32_t)g.H + 8 * (i & 15);
        else
            aoff[q] = (uint32_t)(row0 + r) * (uint32_t)g.F + 8 * (i & 15);
    }
    u32x4_t av[8];
    auto load_a = [&](int kc) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int kk = kc * 128 + 8 * ((tid + 256 * q) & 15);
            av[q] = u32x4_t{0u, 0u, 0u, 0u};
            if (kk < K) av[q] = *reinterpret_cast<const u32x4_t*>(abase + (aoff[q] + kc * 128));
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = tid + 256 * q;
            *reinterpret_cast<u32x4_t*>(As + buf * kLdsTile + (i >> 4) * kLdsRow + 8 * (i & 15)) = av[q];
        }
    };
    BCodes<FMT> cb[2], nb[2];
    f32x16_t acc[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[s][gi][i] = 0.f;

    load_a(0);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) load_bcodes<FMT>(cb[gi], bt[gi], n & 15, half, bvalid[gi]);
    store_a(0);
    if (nk > 1) load_a(1);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        const int kn = min(kc + 1, nk - 1);
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
            load_bcodes<FMT>(nb[gi], bt[gi] + (int64_t)kn * mg.chunk_bytes, n & 15, half, bvalid[gi]);
        const uint16_t* al = As + buf * kLdsTile + (lane & 31) * kLdsRow + 8 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4_t b0[2], b1[2];
            deq_block<FMT>(cb[0], j, b0[0], b0[1]);
            deq_block<FMT>(cb[1], j, b1[0], b1[1]);
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
                const int ks = 2 * j + ss;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s < nslice) {
                        const u32x4_t af = *reinterpret_cast<const u32x4_t*>(al + s * 32 * kLdsRow + 16 * ks);
                        acc[s][0] = mfma32(af, b0[ss], acc[s][0]);
                        acc[s][1] = mfma32(af, b1[ss], acc[s][1]);
                    }
                }
            }
        }
        if (kc + 1 < nk) store_a(buf ^ 1);
        if (kc + 2 < nk) load_a(kc + 2);
        __syncthreads();
        cb[0] = nb[0];
        cb[1] = nb[1];
    }
    // epilogue: lane holds C[m = 32 s + 8(i/4) + 4 half + i%4][column n] of both groups
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (s < nslice) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = s * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                if (m < nrows) {
                    if constexpr (MODE == 1) {
                        const int f = nt * 128 + 32 * wave + n;
                        if (f < g.F) {
                            const float gv = acc[s][0][i], uv = acc[s][1][i];
                            const float hv = gv / (1.0f + __expf(-gv)) * uv;
                            pb.h[(int64_t)(row0 + m) * g.F + f] = (uint16_t)f2bf(hv);
                        }
                    } else {
#pragma unroll
                        for (int gi = 0; gi < 2; ++gi) {
                            const int col = nt * 256 + 64 * wave + 32 * gi + n;
                            if (col < g.H) pb.o[(int64_t)(row0 + m) * g.H + col] = acc[s][gi][i];
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- combine
// Thread per (token, 4 consecutive columns): the k routed rows in slot order,
// then the shared row, then the residual.
__global__ __launch_bounds__(256) void k_pf_combine(const uint16_t* __restrict__ x, int T, int H, int k, int S,
                                                    PrefillBufs pb, uint16_t* __restrict__ y, int residual) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int h4 = H / 4;
    if (i >= T * h4) return;
    const int t = i / h4, c = (i - t * h4) * 4;
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const float w = pb.w[(int64_t)t * k + j];
        const f32x4_t o = *reinterpret_cast<const f32x4_t*>(pb.o + (int64_t)pb.inv[(int64_t)t * k + j] * H + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] += w * o[q];
    }
    if (S) {
        const f32x4_t o = *reinterpret_cast<const f32x4_t*>(pb.o + ((int64_t)T * k + t) * H + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] += o[q];
    }
    uint32_t out[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        float a = s[2 * q], b = s[2 * q + 1];
        if (residual) {
            const uint32_t xv = *reinterpret_cast<const uint32_t*>(x + (int64_t)t * H + c + 2 * q);
            a += bf2f(xv & 0xFFFFu);
            b += bf2f(xv >> 16);
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
    launch(k_pf_router, dim3((g.E + 63) / 64, (T + 63) / 64), dim3(256), 0, lc, x, T, Wr, bias, g.E, g.H, pb.logits);
    return hipGetLastError();
}

hipError_t launch_pf_topk(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const float* rstat,
                          const Geom& g, PrefillBufs pb, int32_t* trace_ids, float* trace_w, const Launch& lc) {
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
    static int granted = 64 * 1024;
    hipError_t e = ensure_lds(k_pf_gemm<FMT, MODE>, kGemmLds, granted);
    if (e != hipSuccess) return e;
    const int ntn = MODE == 1 ? (g.F + 127) / 128 : (g.H + 255) / 256;
    launch(k_pf_gemm<FMT, MODE>, dim3(pb.max_tiles * ntn), dim3(256), kGemmLds, lc, x, slots, g, pb, ntn);
    return hipGetLastError();
}

hipError_t launch_pf_gemm1(const uint16_t* x, const uint8_t* layer_slots, const Geom& g, PrefillBufs pb,
                           const Launch& lc) {
    return g.fmt == 1 ? launch_gemm<1, 1>(x, layer_slots, g, pb, lc) : launch_gemm<2, 1>(x, layer_slots, g, pb, lc);
}

hipError_t launch_pf_gemm2(const uint8_t* layer_slots, const Geom& g, PrefillBufs pb, const Launch& lc) {
    return g.fmt == 1 ? launch_gemm<1, 2>(nullptr, layer_slots, g, pb, lc)
                      : launch_gemm<2, 2>(nullptr, layer_slots, g, pb, lc);
}

hipError_t launch_pf_combine(const uint16_t* x, int T, const Geom& g, PrefillBufs pb, uint16_t* y, int residual,
                             const Launch& lc) {
    launch(k_pf_combine, dim3((T * (g.H / 4) + 255) / 256), dim3(256), 0, lc, x, T, g.H, g.k, g.S, pb, y, residual);
    return hipGetLastError();
}

}  // namespace moe
