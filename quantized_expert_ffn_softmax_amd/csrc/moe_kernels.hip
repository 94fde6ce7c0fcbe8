// Decode-path kernels of the MI355X sparse-MoE layer (gfx950, wave64).
//
// Per layer and call (T <= 8 tokens):
//   k_router_decode   router GEMV (+bias) with fp64 accumulation of the exact
//                     bf16 x bf16 products; also the per-block sums of x
//   k_topk_sort       one workgroup: wave top-k per token (logit descending,
//                     lower id on ties), renormalised softmax weights, stable
//                     counting sort of the (token, expert) pairs, the list of
//                     active experts and the per-(expert, token) weight table
//   k_gateup_decode   per (active expert, 16-row tile of F): fused dequant +
//                     gate/up GEMV on bf16 MFMA + SwiGLU; writes w*h split
//                     into bf16 hi/lo halves as the down projection's operand
//   k_down_decode     per 16-row tile of H: down GEMV over all active experts
//                     in ascending order, atomic-free weighted combine,
//                     optional residual, bf16 output
//
// Method references (pages): sparse top-k routing with a shared expert and
// gate/up/down expert tensors -- "Strata 改源码去跑 DeepSeek V4 Flash？",
// section 二; 512 experts, 10 active -- teardown "Strata 引擎深度拆解",
// section 二; decode is bandwidth-bound -- "Qwen3.8-Flash-Next UD-Q4_K_XL 引擎
// 对比", section 四; grouping the verify window's tokens by expert so one read
// of an expert serves several tokens -- teardown section 一 (multi-token CPU
// expert kernel) and section 二.1 (verify window).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float h2f(uint32_t h16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h16); }
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Offset constant of the bias trick: an operand value is 128 + q, the weight
// is d*(q - o), so the contraction over a block is d*(R - (128+o)*S).
template <int FMT> struct QF;
template <> struct QF<1> { static constexpr float kBias = 136.0f; static constexpr int kCW = 16; };
template <> struct QF<2> { static constexpr float kBias = 130.0f; static constexpr int kCW = 8; };

// Block j (0..3) of a chunk as the MFMA B operand: four bf16 pairs (128+q).
template <int FMT> __device__ __forceinline__ u32x4_t unpack(const uint32_t* cw, int j);
template <> __device__ __forceinline__ u32x4_t unpack<1>(const uint32_t* cw, int j) {
    const uint32_t w = cw[j];
    u32x4_t r;
    r.x = (w & 0x000F000Fu) | 0x43004300u;
    r.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    r.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    r.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return r;
}
template <> __device__ __forceinline__ u32x4_t unpack<2>(const uint32_t* cw, int j) {
    const uint32_t w = cw[j >> 1] >> (8 * (j & 1));
    u32x4_t r;
    r.x = (w & 0x00030003u) | 0x43004300u;
    r.y = ((w >> 2) & 0x00030003u) | 0x43004300u;
    r.z = ((w >> 4) & 0x00030003u) | 0x43004300u;
    r.w = ((w >> 6) & 0x00030003u) | 0x43004300u;
    return r;
}

template <int FMT> __device__ __forceinline__ void load_codes(const uint8_t* chunk, int lane, uint32_t* cw) {
    if constexpr (FMT == 1) {
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(chunk + lane * 16);
        cw[0] = v.x; cw[1] = v.y; cw[2] = v.z; cw[3] = v.w;
    } else {
        u32x2_t v = *reinterpret_cast<const u32x2_t*>(chunk + lane * 8);
        cw[0] = v.x; cw[1] = v.y;
    }
}
__device__ __forceinline__ u32x2_t load_scales(const uint8_t* chunk, int cw_bytes, int n) {
    return *reinterpret_cast<const u32x2_t*>(chunk + 64 * cw_bytes + n * 8);
}
__device__ __forceinline__ float scale_of(u32x2_t s, int j) {
    const uint32_t w = (j & 2) ? s.y : s.x;
    return h2f((j & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// One chunk (4 blocks) of a 16-row tile against A operands A[0..3]:
//   acc[i] += sum_j d[n][j] * sum_k A[m][k] (128 + q[n][k])
//   corr   += S[m][4c+g] * d[n][4c+g]     (v_mfma_f32_16x16x4f32, K = the 4 blocks)
template <int FMT>
__device__ __forceinline__ void chunk_mac(const uint32_t* cw, u32x2_t sc, const u32x4_t* A, float s_corr, int g,
                                         f32x4_t& acc, f32x4_t& corr) {
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4_t R = mfma_bf16(A[j], unpack<FMT>(cw, j), zero);
        const float d = scale_of(sc, j);
        acc[0] += d * R[0];
        acc[1] += d * R[1];
        acc[2] += d * R[2];
        acc[3] += d * R[3];
    }
    corr = mfma_f32(s_corr, scale_of(sc, g), corr);
}

// ---------------------------------------------------------------- repack
// Canonical blocks (host format) -> slot layout described in moe_internal.h.
// Grid: (ceil(max_nch/4), F/16*2 + H/16, count), block 256 = 4 chunks x 64 lanes.
__global__ __launch_bounds__(256) void k_repack(const uint8_t* __restrict__ canon, uint8_t* __restrict__ slots,
                                                Geom g) {
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int rt_all = blockIdx.y;
    const int ex = blockIdx.z;
    const int rtF = g.F / 16;
    int mat = rt_all < rtF ? 0 : rt_all < 2 * rtF ? 1 : 2;
    const int rt = mat == 0 ? rt_all : mat == 1 ? rt_all - rtF : rt_all - 2 * rtF;
    const MatGeom& m = mat == 2 ? g.dn : g.gu;
    if (c >= m.nch) return;
    const int bb = g.fmt == 1 ? 18 : 10;
    const uint8_t* src = canon + (int64_t)ex * g.canon_expert_bytes +
                         (mat == 0 ? 0 : mat == 1 ? (int64_t)g.F * (g.H / 32) * bb : 2LL * g.F * (g.H / 32) * bb);
    uint8_t* dst = slots + (int64_t)ex * g.slot_bytes + (mat == 0 ? g.g_off : mat == 1 ? g.u_off : g.d_off) +
                   (int64_t)rt * m.tile_bytes + (int64_t)c * m.chunk_bytes;
    const int n = lane & 15, gs = lane >> 4;
    const int row = rt * 16 + n;
    const int o = g.fmt == 1 ? 8 : 2;
    auto code = [&](int b, int e) -> uint32_t {  // element e of block b of this row
        if (b >= m.nb) return (uint32_t)o;
        const uint8_t* blk = src + ((int64_t)row * m.nb + b) * bb + 2;
        return g.fmt == 1 ? (blk[e >> 1] >> (4 * (e & 1))) & 0xFu : (blk[e >> 2] >> (2 * (e & 3))) & 0x3u;
    };
    if (g.fmt == 1) {
        uint32_t w[4];
        for (int j = 0; j < 4; ++j) {
            const int b = c * 4 + j;
            uint32_t v = 0;
            for (int p = 0; p < 4; ++p)
                v |= (code(b, 8 * gs + 2 * p) << (4 * p)) | (code(b, 8 * gs + 2 * p + 1) << (16 + 4 * p));
            w[j] = v;
        }
        *reinterpret_cast<u32x4_t*>(dst + lane * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
    } else {
        uint32_t w[2];
        for (int jj = 0; jj < 2; ++jj) {
            uint32_t v = 0;
            for (int hb = 0; hb < 2; ++hb) {
                const int b = c * 4 + 2 * jj + hb;
                for (int p = 0; p < 4; ++p)
                    v |= (code(b, 8 * gs + 2 * p) << (8 * hb + 2 * p)) | (code(b, 8 * gs + 2 * p + 1) << (16 + 8 * hb + 2 * p));
            }
            w[jj] = v;
        }
        *reinterpret_cast<u32x2_t*>(dst + lane * 8) = u32x2_t{w[0], w[1]};
    }
    if (gs == 0) {
        uint16_t s[4];
        for (int j = 0; j < 4; ++j) {
            const int b = c * 4 + j;
            if (b < m.nb) {
                const uint8_t* blk = src + ((int64_t)row * m.nb + b) * bb;
                s[j] = (uint16_t)(blk[0] | (blk[1] << 8));
            } else {
                s[j] = 0;
            }
        }
        *reinterpret_cast<u32x2_t*>(dst + 64 * (g.fmt == 1 ? 16 : 8) + n * 8) =
            u32x2_t{(uint32_t)s[0] | ((uint32_t)s[1] << 16), (uint32_t)s[2] | ((uint32_t)s[3] << 16)};
    }
}

hipError_t launch_repack(const uint8_t* canon, uint8_t* slots, int count, const Geom& g, hipStream_t st) {
    const int max_nch = g.gu.nch > g.dn.nch ? g.gu.nch : g.dn.nch;
    dim3 grid((max_nch + 3) / 4, 2 * (g.F / 16) + g.H / 16, count);
    hipLaunchKernelGGL(k_repack, grid, dim3(256), 0, st, canon, slots, g);
    return hipGetLastError();
}

// ---------------------------------------------------------------- router
// logits[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]: every bf16 x bf16 product is
// exact in fp32 and is accumulated in fp64 (fixed reduction tree), so the
// selection agrees with an fp64 evaluation except at logit gaps near 1e-15.
// Grid: ceil(E/2) workgroups of 4 waves; waves (0,1) -> expert 2b, (2,3) ->
// expert 2b+1; the two waves of an expert split H in halves.
// Workgroup 0 also writes sx[b][m] = sum of x[m][32b..32b+31] (fp32, m < T,
// zero elsewhere), the per-block sums used to remove the operand offset.
__global__ __launch_bounds__(256) void k_router_decode(const uint16_t* __restrict__ x, int T,
                                                       const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
                                                       int E, int H, int nbp, double* __restrict__ logits,
                                                       float* __restrict__ sx) {
    __shared__ double part[4][kMaxDecodeT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 2 + (wave >> 1);
    const int half = wave & 1;
    const int Hh = H / 2;
    double acc[kMaxDecodeT];
#pragma unroll
    for (int t = 0; t < kMaxDecodeT; ++t) acc[t] = 0.0;
    if (e < E) {
        const uint16_t* wrow = Wr + (int64_t)e * H + half * Hh;
        for (int h0 = lane * 8; h0 < Hh; h0 += 512) {
            const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(wrow + h0);
            float wf[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wf[2 * q] = __uint_as_float(wv[q] << 16);
                wf[2 * q + 1] = __uint_as_float(wv[q] & 0xFFFF0000u);
            }
#pragma unroll
            for (int t = 0; t < kMaxDecodeT; ++t) {
                if (t < T) {
                    const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(x + (int64_t)t * H + half * Hh + h0);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[t] += (double)(__uint_as_float(xv[q] << 16) * wf[2 * q]);
                        acc[t] += (double)(__uint_as_float(xv[q] & 0xFFFF0000u) * wf[2 * q + 1]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kMaxDecodeT; ++t) {
        double v = acc[t];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) part[wave][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < 2 * kMaxDecodeT) {
        const int pair = threadIdx.x / kMaxDecodeT, t = threadIdx.x % kMaxDecodeT;
        const int ee = blockIdx.x * 2 + pair;
        if (ee < E && t < T)
            logits[(int64_t)t * E + ee] = (part[2 * pair][t] + part[2 * pair + 1][t]) + (bias ? (double)bias[ee] : 0.0);
    }
    if (blockIdx.x == 0) {
        const int nb = H / 32;
        for (int i = threadIdx.x; i < nbp * 16; i += blockDim.x) {
            const int b = i >> 4, m = i & 15;
            float s = 0.f;
            if (m < T && b < nb) {
                const uint16_t* xr = x + (int64_t)m * H + b * 32;
                for (int q = 0; q < 32; ++q) s += bf2f(xr[q]);
            }
            sx[i] = s;
        }
    }
}

hipError_t launch_router_decode(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const Geom& g,
                                RouteBufs rb, hipStream_t st) {
    hipLaunchKernelGGL(k_router_decode, dim3((g.E + 1) / 2), dim3(256), 0, st, x, T, Wr, bias, g.E, g.H,
                       g.gu.nch * 4, rb.logits, rb.sx);
    return hipGetLastError();
}

// ---------------------------------------------------------------- top-k + sort
// One workgroup of 512 threads; wave t handles token t (T <= 8).
__global__ __launch_bounds__(512) void k_topk_sort(int T, int E, int k, int S, const double* __restrict__ logits,
                                                   int32_t* __restrict__ ids, float* __restrict__ wout,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                   int32_t* __restrict__ inv, int32_t* __restrict__ nact,
                                                   int32_t* __restrict__ act, float* __restrict__ wtab,
                                                   int32_t* __restrict__ trace_ids, float* __restrict__ trace_w) {
    __shared__ int32_t s_ids[kMaxDecodeT * kMaxTopK];
    __shared__ float s_w[kMaxDecodeT * kMaxTopK];
    __shared__ uint32_t s_cnt[kMaxExperts];
    __shared__ uint32_t s_wavesum[8];
    __shared__ int32_t s_aidx[kMaxExperts];
    __shared__ int32_t s_off[kMaxExperts];
    __shared__ float s_wtab[(kMaxDecodeT * kMaxTopK + 1) * kMaxDecodeT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int P = T * k;

    if (wave < T) {
        const int t = wave;
        constexpr int J = kMaxExperts / 64;
        double v[J];
        bool taken[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane + 64 * j;
            v[j] = e < E ? logits[(int64_t)t * E + e] : -__builtin_huge_val();
            taken[j] = e >= E;
        }
        double sel_v0 = 0.0, my_v = 0.0;
        int my_e = 0;
        for (int r = 0; r < k; ++r) {
            double bv = -__builtin_huge_val();
            int be = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int e = lane + 64 * j;
                if (!taken[j] && (v[j] > bv || (v[j] == bv && e < be))) { bv = v[j]; be = e; }
            }
            for (int off = 32; off > 0; off >>= 1) {
                const double ov = __shfl_xor(bv, off);
                const int oe = __shfl_xor(be, off);
                if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
            }
            if ((be & 63) == lane) {
#pragma unroll
                for (int j = 0; j < J; ++j)
                    if (lane + 64 * j == be) taken[j] = true;
            }
            if (r == 0) sel_v0 = bv;
            if (lane == r) { my_v = bv; my_e = be; }
        }
        // renormalised softmax over the k selected logits (fp64)
        const double ex = lane < k ? exp(my_v - sel_v0) : 0.0;
        double z = ex;
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
        if (lane < k) {
            const float wv = (float)(ex / z);
            s_ids[t * k + lane] = my_e;
            s_w[t * k + lane] = wv;
            ids[t * k + lane] = my_e;
            wout[t * k + lane] = wv;
            if (trace_ids) trace_ids[t * k + lane] = my_e;
            if (trace_w) trace_w[t * k + lane] = wv;
        }
    }
    for (int e = threadIdx.x; e < kMaxExperts; e += blockDim.x) s_cnt[e] = 0;
    __syncthreads();
    if (threadIdx.x < P) atomicAdd(&s_cnt[s_ids[threadIdx.x]], 1u);
    __syncthreads();
    // exclusive scan of packed (count << 16 | nonempty) over E <= 1024 entries, 2 per thread
    const int e0 = 2 * threadIdx.x;
    const uint32_t c0 = e0 < E ? s_cnt[e0] : 0u, c1 = e0 + 1 < E ? s_cnt[e0 + 1] : 0u;
    const uint32_t p0 = (c0 << 16) | (c0 ? 1u : 0u), p1 = (c1 << 16) | (c1 ? 1u : 0u);
    uint32_t incl = p0 + p1;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_wavesum[wave] = incl;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += s_wavesum[w];
    const uint32_t ex0 = base + incl - (p0 + p1);
    const uint32_t ex1 = ex0 + p0;
    if (e0 < E) {
        offsets[e0] = s_off[e0] = (int32_t)(ex0 >> 16);
        s_aidx[e0] = (int32_t)(ex0 & 0xFFFFu);
        if (c0) act[ex0 & 0xFFFFu] = e0;
    }
    if (e0 + 1 < E) {
        offsets[e0 + 1] = s_off[e0 + 1] = (int32_t)(ex1 >> 16);
        s_aidx[e0 + 1] = (int32_t)(ex1 & 0xFFFFu);
        if (c1) act[ex1 & 0xFFFFu] = e0 + 1;
    }
    uint32_t total = 0;
    for (int w = 0; w < 8; ++w) total += s_wavesum[w];
    const int U = (int)(total & 0xFFFFu);
    const int nA = U + S;
    if (threadIdx.x == 0) {
        offsets[E] = P;
        nact[0] = nA;
        if (S) act[U] = E;
    }
    for (int i = threadIdx.x; i < nA * kMaxDecodeT; i += blockDim.x) s_wtab[i] = 0.f;
    __syncthreads();
    if (threadIdx.x < P) {
        const int i = threadIdx.x, e = s_ids[i];
        int rank = 0;
        for (int q = 0; q < i; ++q) rank += s_ids[q] == e;
        const int pos = s_off[e] + rank;
        perm[pos] = i;
        inv[i] = pos;
        s_wtab[s_aidx[e] * kMaxDecodeT + i / k] = s_w[i];
    }
    if (S && threadIdx.x < T) s_wtab[U * kMaxDecodeT + threadIdx.x] = 1.0f;
    __syncthreads();
    for (int i = threadIdx.x; i < nA * kMaxDecodeT; i += blockDim.x) wtab[i] = s_wtab[i];
}

hipError_t launch_topk_sort_decode(int T, const Geom& g, RouteBufs rb, int32_t* trace_ids, float* trace_w,
                                   hipStream_t st) {
    hipLaunchKernelGGL(k_topk_sort, dim3(1), dim3(512), 0, st, T, g.E, g.k, g.S, rb.logits, rb.ids, rb.w, rb.offsets,
                       rb.perm, rb.inv, rb.nact, rb.act, rb.wtab, trace_ids, trace_w);
    return hipGetLastError();
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// Grid (F/16, maxA), 256 threads.  Workgroup (rt, a): rows 16rt..16rt+15 of G
// and U of active expert a; the 4 waves split K = H by chunks.  The MFMA
// computes C[m = token][n = row] with A = x (rows m >= T are zero).
template <int FMT>
__global__ __launch_bounds__(256) void k_gateup_decode(const uint16_t* __restrict__ x, int T,
                                                       const uint8_t* __restrict__ slots, Geom g,
                                                       const float* __restrict__ sx, const int32_t* __restrict__ nact,
                                                       const int32_t* __restrict__ act, const float* __restrict__ wtab,
                                                       uint32_t* __restrict__ afrag, float* __restrict__ spart) {
    __shared__ f32x4_t red[4][4][64];
    const int a = blockIdx.y;
    if (a >= nact[0]) return;
    const int rt = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, gs = lane >> 4, m = lane & 15;
    const int e = act[a];
    const MatGeom& mg = g.gu;
    const uint8_t* Gt = slots + (int64_t)e * g.slot_bytes + g.g_off + (int64_t)rt * mg.tile_bytes;
    const uint8_t* Ut = slots + (int64_t)e * g.slot_bytes + g.u_off + (int64_t)rt * mg.tile_bytes;
    const int c0 = wave * mg.nch / 4, c1 = (wave + 1) * mg.nch / 4;
    const bool xrow = m < T;
    const uint16_t* xr = x + (int64_t)m * g.H + 8 * gs;
    f32x4_t accG = {0.f, 0.f, 0.f, 0.f}, accU = accG, corG = accG, corU = accG;
    for (int c = c0; c < c1; ++c) {
        uint32_t cg[4], cu[4];
        load_codes<FMT>(Gt + (int64_t)c * mg.chunk_bytes, lane, cg);
        load_codes<FMT>(Ut + (int64_t)c * mg.chunk_bytes, lane, cu);
        const u32x2_t sg = load_scales(Gt + (int64_t)c * mg.chunk_bytes, QF<FMT>::kCW, n);
        const u32x2_t su = load_scales(Ut + (int64_t)c * mg.chunk_bytes, QF<FMT>::kCW, n);
        u32x4_t A[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = c * 4 + j;
            A[j] = (xrow && b < mg.nb) ? *reinterpret_cast<const u32x4_t*>(xr + b * 32) : u32x4_t{0u, 0u, 0u, 0u};
        }
        const float s = sx[(c * 4 + gs) * 16 + m];
        chunk_mac<FMT>(cg, sg, A, s, gs, accG, corG);
        chunk_mac<FMT>(cu, su, A, s, gs, accU, corU);
    }
    red[wave][0][lane] = accG;
    red[wave][1][lane] = accU;
    red[wave][2][lane] = corG;
    red[wave][3][lane] = corU;
    __syncthreads();
    if (wave != 0) return;
    f32x4_t sG = red[0][0][lane], sU = red[0][1][lane], qG = red[0][2][lane], qU = red[0][3][lane];
    for (int w = 1; w < 4; ++w) {
        sG += red[w][0][lane];
        sU += red[w][1][lane];
        qG += red[w][2][lane];
        qU += red[w][3][lane];
    }
    // lane holds (token t = 4*gs + i, row f = 16*rt + n); tokens < 8 live in gs 0..1
    const int nbFp = g.dn.nch * 4;
    const int bF = rt >> 1, kf0 = 16 * (rt & 1);
    const int kf = kf0 + n;
    uint16_t* af16 = reinterpret_cast<uint16_t*>(afrag) + ((int64_t)a * nbFp + bF) * 64 * 8;
    float shi[4], slo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * gs + i;
        const float gv = sG[i] - QF<FMT>::kBias * qG[i];
        const float uv = sU[i] - QF<FMT>::kBias * qU[i];
        const float h = gv / (1.0f + expf(-gv)) * uv;
        const float wt = t < kMaxDecodeT ? wtab[a * kMaxDecodeT + t] : 0.f;
        const float v = wt * h;
        const uint32_t hi = f2bf(v);
        const uint32_t lo = f2bf(v - bf2f(hi));
        shi[i] = bf2f(hi);
        slo[i] = bf2f(lo);
        if (t < T) {
            af16[(t + 16 * (kf >> 3)) * 8 + (kf & 7)] = (uint16_t)hi;
            af16[(8 + t + 16 * (kf >> 3)) * 8 + (kf & 7)] = (uint16_t)lo;
        }
    }
    // per-half-block row sums of the operand halves, reduced over the 16 rows n of this lane group
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        for (int off = 1; off < 16; off <<= 1) {
            shi[i] += __shfl_xor(shi[i], off);
            slo[i] += __shfl_xor(slo[i], off);
        }
    }
    if (n == 0 && gs < 2) {
        float* sp = spart + (((int64_t)a * nbFp + bF) * 2 + (rt & 1)) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * gs + i;
            if (t < T) {
                sp[t] = shi[i];
                sp[8 + t] = slo[i];
            }
        }
    }
}

hipError_t launch_gateup_decode(const uint16_t* x, int T, const uint8_t* layer_slots, const Geom& g, RouteBufs rb,
                                DecodeBufs db, hipStream_t st) {
    const int maxA = (g.E < T * g.k ? g.E : T * g.k) + g.S;
    dim3 grid(g.F / 16, maxA);
    if (g.fmt == 1)
        hipLaunchKernelGGL(k_gateup_decode<1>, grid, dim3(256), 0, st, x, T, layer_slots, g, rb.sx, rb.nact, rb.act,
                           rb.wtab, db.afrag, db.spart);
    else
        hipLaunchKernelGGL(k_gateup_decode<2>, grid, dim3(256), 0, st, x, T, layer_slots, g, rb.sx, rb.nact, rb.act,
                           rb.wtab, db.afrag, db.spart);
    return hipGetLastError();
}

// ---------------------------------------------------------------- down + combine
// Grid H/16, 512 threads.  Workgroup rt owns rows 16rt..16rt+15 of y; wave w
// takes active experts a = w, w+8, ...; partial sums are added in wave order,
// so the result does not depend on timing.  A = [w*h hi rows 0..7 | lo rows 8..15].
template <int FMT>
__global__ __launch_bounds__(512) void k_down_decode(const uint16_t* __restrict__ x, int T,
                                                     const uint8_t* __restrict__ slots, Geom g,
                                                     const int32_t* __restrict__ nact, const int32_t* __restrict__ act,
                                                     const uint32_t* __restrict__ afrag,
                                                     const float* __restrict__ spart, uint16_t* __restrict__ y,
                                                     int residual) {
    __shared__ f32x4_t red[8][32];
    const int rt = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, gs = lane >> 4, m = lane & 15;
    const int nA = nact[0];
    const MatGeom& md = g.dn;
    const int nbFp = md.nch * 4;
    const bool mrow = (m & 7) < T;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, corr = acc;
    for (int a = wave; a < nA; a += 8) {
        const int e = act[a];
        const uint8_t* Dt = slots + (int64_t)e * g.slot_bytes + g.d_off + (int64_t)rt * md.tile_bytes;
        const u32x4_t* af = reinterpret_cast<const u32x4_t*>(afrag) + (int64_t)a * nbFp * 64;
        const float* sp = spart + (int64_t)a * nbFp * 32;
        for (int c = 0; c < md.nch; ++c) {
            uint32_t cw[4];
            load_codes<FMT>(Dt + (int64_t)c * md.chunk_bytes, lane, cw);
            const u32x2_t sc = load_scales(Dt + (int64_t)c * md.chunk_bytes, QF<FMT>::kCW, n);
            u32x4_t A[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int b = c * 4 + j;
                A[j] = (mrow && b < md.nb) ? af[(int64_t)b * 64 + lane] : u32x4_t{0u, 0u, 0u, 0u};
            }
            const int bq = c * 4 + gs;
            const float s = (mrow && bq < md.nb) ? sp[bq * 32 + m] + sp[bq * 32 + 16 + m] : 0.f;
            chunk_mac<FMT>(cw, sc, A, s, gs, acc, corr);
        }
    }
    f32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[i] - QF<FMT>::kBias * corr[i];
    f32x4_t other;
#pragma unroll
    for (int i = 0; i < 4; ++i) other[i] = __shfl_xor(v[i], 32);
    if (lane < 32) red[wave][lane] = v + other;
    __syncthreads();
    if (wave != 0 || lane >= 32) return;
    f32x4_t s = red[0][lane];
    for (int w = 1; w < 8; ++w) s += red[w][lane];
    const int hrow = rt * 16 + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * gs + i;
        if (t < T) {
            float out = s[i];
            if (residual) out += bf2f(x[(int64_t)t * g.H + hrow]);
            y[(int64_t)t * g.H + hrow] = (uint16_t)f2bf(out);
        }
    }
}

hipError_t launch_down_decode(const uint16_t* x, int T, const uint8_t* layer_slots, const Geom& g, RouteBufs rb,
                              DecodeBufs db, uint16_t* y, int residual, hipStream_t st) {
    dim3 grid(g.H / 16);
    if (g.fmt == 1)
        hipLaunchKernelGGL(k_down_decode<1>, grid, dim3(512), 0, st, x, T, layer_slots, g, rb.nact, rb.act, db.afrag,
                           db.spart, y, residual);
    else
        hipLaunchKernelGGL(k_down_decode<2>, grid, dim3(512), 0, st, x, T, layer_slots, g, rb.nact, rb.act, db.afrag,
                           db.spart, y, residual);
    return hipGetLastError();
}

}  // namespace moe
