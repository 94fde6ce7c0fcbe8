// Decode-path kernels of the MI355X sparse-MoE layer (gfx950, wave64).
//
// Per layer and call (T <= 8 tokens), five launches:
//   k_router_decode   one workgroup per expert: router GEMV (+bias) with fp64
//                     accumulation of the exact bf16 x bf16 products; also
//                     the per-block sums of x (and, for chain layers, the
//                     per-token RMS pre-norm of x)
//   k_topk_sort       one workgroup: top-k per token (logit descending, lower
//                     id on ties; DPP wave maxima over pre-sorted per-lane
//                     lists of 32-bit keys), renormalised softmax
//                     weights, stable counting sort of the (token, expert)
//                     pairs from per-expert token bitmasks, active-expert list
//                     and weight table
//   k_gateup_decode   one workgroup per (active expert, 16-row tile of F):
//                     fused dequant + gate/up GEMV on bf16 MFMA + SwiGLU; all
//                     weight loads issued on entry (non-temporal); writes
//                     v = w * SwiGLU as bf16 hi/lo halves in MFMA-operand
//                     order
//   k_down_decode     per (active expert, 128-row group of H): down GEMV with
//                     the expert's operand staged once in LDS; stores one
//                     partial row block per expert
//   k_combine_decode  one-wave workgroups, a thread per output element: sums
//                     the experts in ascending active order (no atomics,
//                     deterministic), adds the residual, writes bf16
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

#include "moe_device.h"

namespace moe {

// One chunk (4 blocks) of a 16-row tile against A operands A[0..3]:
//   acc[i] += sum_j d[n][j] * sum_k A[m][k] (128 + q[n][k])
//   corr   += S[m][4c+g] * d[n][4c+g]     (v_mfma_f32_16x16x4f32, K = the 4 blocks)
// Only the first NV result registers are scaled and accumulated (a lane's
// register i holds output row 4 (lane / 16) + i; callers that leave rows
// 4 g + i, i >= NV, zero need only NV of them).
// q2b64: the two 32-weight halves of a 64-block share one scale, so their
// products are summed by the MFMA and scaled once.
template <int FMT, int NV = 4>
__device__ __forceinline__ void chunk_mac(const uint32_t* cw, u32x2_t sc, const u32x4_t* A, float s_corr, int g,
                                         f32x4_t& acc, f32x4_t& corr) {
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == 3) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4_t R = mfma_bf16(A[2 * h], unpack<FMT>(cw, 2 * h, bf16_bias_bits()), zero);
            R = mfma_bf16(A[2 * h + 1], unpack<FMT>(cw, 2 * h + 1, bf16_bias_bits()), R);
            const float d = scale_of<FMT>(sc, 2 * h);
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[i] += d * R[i];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4_t R = mfma_bf16(A[j], unpack<FMT>(cw, j, bf16_bias_bits()), zero);
            const float d = scale_of<FMT>(sc, j);
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[i] += d * R[i];
        }
    }
    corr = mfma_f32(s_corr, scale_of<FMT>(sc, g), corr);
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
    const int bb = g.fmt == 2 ? 10 : 18;              // canonical block bytes
    const int bsh = g.fmt == 3 ? 1 : 0;               // log2(canonical block weights / 32)
    const int64_t gu_bytes = (int64_t)g.F * (g.H / 32 >> bsh) * bb;
    const uint8_t* src = canon + (int64_t)ex * g.canon_expert_bytes + (mat == 0 ? 0 : mat == 1 ? gu_bytes : 2 * gu_bytes);
    // lane stride of the codes, scale-row stride, and this matrix's byte inside both
    // (q2 / q2b64 store G and U, and D's row tiles 2 rp, 2 rp + 1, in interleaved units of two chunks' size)
    const bool il = g.fmt != 1;
    const int cwb = g.fmt == 1 ? 16 : 8, sb = g.fmt == 3 ? 4 : 8;
    const int part = mat < 2 ? mat : rt & 1;  // which half of the unit
    uint8_t* dst = slots + (int64_t)ex * g.slot_bytes;
    if (il)
        dst += (mat < 2 ? 0 : g.d_off) + ((int64_t)(mat < 2 ? rt : rt >> 1) * m.nch + c) * 2 * m.chunk_bytes;
    else
        dst += (mat == 0 ? g.g_off : mat == 1 ? g.u_off : g.d_off) + (int64_t)rt * m.tile_bytes +
               (int64_t)c * m.chunk_bytes;
    const int lstride = il ? 2 * cwb : cwb, sstride = il ? 2 * sb : sb;
    const int lpos = il ? part * cwb : 0, spos = il ? part * sb : 0;
    const int n = lane & 15, gs = lane >> 4;
    const int row = rt * 16 + n;
    const int o = g.fmt == 1 ? 8 : 2;
    auto code = [&](int b, int e) -> uint32_t {  // element e of 32-block b of this row
        if (b >= m.nb) return (uint32_t)o;
        const int ec = e + ((b & bsh) << 5);      // element inside the canonical block
        const uint8_t* blk = src + ((int64_t)row * (m.nb >> bsh) + (b >> bsh)) * bb + 2;
        return g.fmt == 1 ? (blk[ec >> 1] >> (4 * (ec & 1))) & 0xFu : (blk[ec >> 2] >> (2 * (ec & 3))) & 0x3u;
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
        *reinterpret_cast<u32x4_t*>(dst + lane * lstride + lpos) = u32x4_t{w[0], w[1], w[2], w[3]};
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
        *reinterpret_cast<u32x2_t*>(dst + lane * lstride + lpos) = u32x2_t{w[0], w[1]};
    }
    if (gs == 0) {
        // scales of the chunk's canonical blocks (4, or 2 for q2b64); padding blocks get 0
        const int nsc = 4 >> bsh;
        uint16_t s[4];
        for (int j = 0; j < nsc; ++j) {
            const int b = c * nsc + j;
            if (b < (m.nb >> bsh)) {
                const uint8_t* blk = src + ((int64_t)row * (m.nb >> bsh) + b) * bb;
                s[j] = (uint16_t)(blk[0] | (blk[1] << 8));
            } else {
                s[j] = 0;
            }
        }
        uint8_t* sdst = dst + 64 * lstride + n * sstride + spos;
        if (g.fmt == 3)
            *reinterpret_cast<uint32_t*>(sdst) = (uint32_t)s[0] | ((uint32_t)s[1] << 16);
        else
            *reinterpret_cast<u32x2_t*>(sdst) =
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
// Grid E workgroups of 4 waves; workgroup e computes the logits of expert e
// for every token.  Wave w sums the quarter h in [w H/4, (w+1) H/4): every
// bf16 x bf16 product is exact in fp32 and is accumulated in fp64; the four
// quarter sums are added in a fixed order, so the selection agrees with an
// fp64 evaluation except at logit gaps near 1e-15.  A lane owns NJ 16-byte
// segments of its quarter (NJ = ceil(H / 2048)) and requests the router
// row's segments and the TT token rows' segments (TT = T rounded up to a power
// of two; rows past T repeat the last) all at once, before any math.
// PRE: the layer's input is the per-token unit-gain RMS pre-norm of x,
// h = bf16(x / sqrt(mean(x^2) + eps)) (fp32; sum of squares per lane, wave
// tree, the four quarters in a fixed order): every workgroup computes the same
// scales from the rows it holds, normalises them in registers, and workgroup 0
// writes h to hm for the expert kernels (so the separate pre-norm launch of a
// chain layer is not needed).
// All threads of the grid also share the per-block sums
// sx[b][m] = sum_{q<32} in[m][32b+q] of the layer input (x, or h with PRE;
// fp32, in q order; zero for m >= T).
template <int NJ, int TT, bool PRE>
__global__ __launch_bounds__(256) void k_router_decode(const uint16_t* __restrict__ x, int T,
                                                       const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
                                                       int E, int H, int nbp, double* __restrict__ logits,
                                                       float* __restrict__ sx, uint16_t* __restrict__ hm) {
    __shared__ double s_part[4][TT];
    __shared__ float s_ss[4][TT];
    __shared__ float s_r[kMaxDecodeT];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int e = blockIdx.x;
    const int ns = H / 32;  // 16-byte segments per quarter
    const int h0 = wave * (H / 4);
    u32x4_t wv[NJ], xv[NJ][TT];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int seg = min(lane + 64 * j, ns - 1);
        wv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Wr + (int64_t)e * H + h0 + 8 * seg));
#pragma unroll
        for (int t = 0; t < TT; ++t)
            xv[j][t] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)min(t, T - 1) * H + h0 + 8 * seg);
    }
    // lane l ends the wave reductions below with token l >> TSH's sum
    constexpr int TSH = TT == 1 ? 6 : TT == 2 ? 5 : TT == 4 ? 4 : 3;
    const bool tlead = (lane & ((1 << TSH) - 1)) == 0;
    if constexpr (PRE) {
        float ssv[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (lane + 64 * j < ns) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float lo = __uint_as_float(xv[j][t][q] << 16);
                        const float hi = __uint_as_float(xv[j][t][q] & 0xFFFF0000u);
                        ss = fmaf(lo, lo, ss);
                        ss = fmaf(hi, hi, ss);
                    }
                }
            }
            ssv[t] = ss;
        }
        const float ssw = wave_sum_scatter<TT>(ssv, lane);
        if (tlead) s_ss[wave][lane >> TSH] = ssw;
        __syncthreads();
        if ((int)threadIdx.x < TT) {
            const int t = threadIdx.x;
            const float tot = (s_ss[0][t] + s_ss[1][t]) + (s_ss[2][t] + s_ss[3][t]);
            s_r[t] = 1.0f / sqrtf(tot / (float)H + kNormEps);
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float r = s_r[t];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xv[j][t][q] = pack_bf16(__uint_as_float(xv[j][t][q] << 16) * r,
                                            __uint_as_float(xv[j][t][q] & 0xFFFF0000u) * r);
                if (blockIdx.x == 0 && t < T && lane + 64 * j < ns)
                    *reinterpret_cast<u32x4_t*>(hm + (int64_t)t * H + h0 + 8 * (lane + 64 * j)) = xv[j][t];
            }
        }
    }
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (lane + 64 * j < ns) {
            float wf[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wf[2 * q] = __uint_as_float(wv[j][q] << 16);
                wf[2 * q + 1] = __uint_as_float(wv[j][q] & 0xFFFF0000u);
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[t] += (double)(__uint_as_float(xv[j][t][q] << 16) * wf[2 * q]);
                    acc[t] += (double)(__uint_as_float(xv[j][t][q] & 0xFFFF0000u) * wf[2 * q + 1]);
                }
            }
        }
    }
    const double accw = wave_sum_scatter<TT>(acc, lane);
    if (tlead) s_part[wave][lane >> TSH] = accw;
    __syncthreads();
    if ((int)threadIdx.x < T) {
        const int t = threadIdx.x;
        const double be = bias ? (double)bias[e] : 0.0;
        logits[(int64_t)t * E + e] = ((s_part[0][t] + s_part[1][t]) + (s_part[2][t] + s_part[3][t])) + be;
    }
    const int nb = H / 32;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nbp * 16; i += gridDim.x * blockDim.x) {
        const int b = i >> 4, m = i & 15;
        float s = 0.f;
        if (m < T && b < nb) {
            const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (int64_t)m * H + b * 32);
            const float r = PRE ? s_r[m] : 1.0f;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const u32x4_t v = xr[q4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (PRE) {
                        const uint32_t hv = pack_bf16(__uint_as_float(v[q] << 16) * r,
                                                      __uint_as_float(v[q] & 0xFFFF0000u) * r);
                        s += __uint_as_float(hv << 16);
                        s += __uint_as_float(hv & 0xFFFF0000u);
                    } else {
                        s += __uint_as_float(v[q] << 16);
                        s += __uint_as_float(v[q] & 0xFFFF0000u);
                    }
                }
            }
        }
        sx[i] = s;
    }
}

hipError_t launch_router_decode(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const Geom& g,
                                RouteBufs rb, uint16_t* hm, const Launch& lc) {
    const dim3 grid(g.E);
    const int nj = (g.H / 32 + 63) / 64;  // 1 or 2 (H <= 4096)
#define MOE_ROUTER_CASE(NJ, TT)                                                                                     \
    if (nj == NJ && T <= TT) {                                                                                      \
        if (hm)                                                                                                     \
            launch(k_router_decode<NJ, TT, true>, grid, dim3(256), 0, lc, x, T, Wr, bias, g.E, g.H, g.gu.nch * 4,   \
                   rb.logits, rb.sx, hm);                                                                           \
        else                                                                                                        \
            launch(k_router_decode<NJ, TT, false>, grid, dim3(256), 0, lc, x, T, Wr, bias, g.E, g.H, g.gu.nch * 4,  \
                   rb.logits, rb.sx, hm);                                                                           \
        return hipGetLastError();                                                                                   \
    }
    MOE_ROUTER_CASE(1, 1) MOE_ROUTER_CASE(1, 2) MOE_ROUTER_CASE(1, 4) MOE_ROUTER_CASE(1, 8)
    MOE_ROUTER_CASE(2, 1) MOE_ROUTER_CASE(2, 2) MOE_ROUTER_CASE(2, 4) MOE_ROUTER_CASE(2, 8)
#undef MOE_ROUTER_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- top-k + sort
// One workgroup of 4 waves; wave w routes token w, and token w+4 when R2 = 2
// (windows of 5 to 8 tokens; R2 = 1 skips that round's logit loads) (selection on
// 32-bit keys of the fp32-rounded logit and the id, with an exact fp64
// fallback when two of the k+1 best keys agree above the id bits, see
// wave_topk_fast; weights from the fp64 logits).  The counting
// sort uses one bitmask of tokens per expert: the pairs of a token have
// distinct experts, so the rank of pair (t, j) inside the group of expert e is
// the number of tokens t' < t that chose e, and the group size is popc(mask).
template <int J, int R2>
__global__ __launch_bounds__(256) void k_topk_sort(int T, int E, int k, int S, RouteBufs rb,
                                                   const int32_t* __restrict__ tab, const int32_t* __restrict__ tok,
                                                   int vocab, int32_t* __restrict__ trace_ids,
                                                   float* __restrict__ trace_w) {
    __shared__ uint32_t s_mask[kMaxExperts];
    __shared__ int32_t s_off[kMaxExperts];
    __shared__ int32_t s_aidx[kMaxExperts];
    __shared__ int32_t s_ids[kMaxDecodeT * kMaxTopK];
    __shared__ float s_w[kMaxDecodeT * kMaxTopK];
    __shared__ float s_wtab[(kMaxDecodeT * kMaxTopK + 1) * kMaxDecodeT];
    __shared__ uint32_t s_wsum[4];
    __shared__ int s_U;
    __shared__ double s_lg[4][64 * J];  // a wave's logits of its current token
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = T * k;
    // logits of this wave's tokens (t = wave, and wave + 4 when R2 = 2, i.e. T > 4) are
    // requested first (unconditional loads with clamped indices: all of them are in flight together)
    double raw[R2][J];
#pragma unroll
    for (int r = 0; r < R2; ++r) {
        const int t = min(wave + 4 * r, T - 1);
#pragma unroll
        for (int j = 0; j < J; ++j) raw[r][j] = rb.logits[(int64_t)t * E + min(lane + 64 * j, E - 1)];
    }
    for (int e = tid; e < E; e += blockDim.x) s_mask[e] = 0u;
    for (int i = tid; i < (P + S) * kMaxDecodeT; i += blockDim.x) s_wtab[i] = 0.f;
    __syncthreads();

#pragma unroll
    for (int r2 = 0; r2 < R2; ++r2) {
        const int t = wave + 4 * r2;
        if (t >= T) break;
        int my_e = 0;
        double my_l = 0.0;
        double l0;
        if (tab) {
            // hash-routed layer: the experts are row tok[t] of the table, in table order
            my_e = lane < k ? tab[(int64_t)min(max(tok[t], 0), vocab - 1) * k + lane] : 0;
            my_l = lane < k ? rb.logits[(int64_t)t * E + my_e] : -HUGE_VAL;
            l0 = my_l;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) l0 = fmax(l0, __shfl_xor(l0, o));
        } else if (wave_topk_fast<J>(raw[r2], E, k, lane, my_e)) {
            // the exact fp64 logits of the selected experts, from this wave's copy in LDS
#pragma unroll
            for (int j = 0; j < J; ++j) s_lg[wave][lane + 64 * j] = raw[r2][j];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            my_l = s_lg[wave][my_e];
        } else {
            // fp32 ties among the k+1 best: select on the fp64 logits, (logit, id) order
            uint64_t key[J];
            uint32_t taken = 0;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                key[j] = lane + 64 * j < E ? order_key(raw[r2][j]) : 0ull;
                if (lane + 64 * j >= E) taken |= 1u << j;
            }
            for (int r = 0; r < k; ++r) {
                uint64_t bk = 0;
                int be = 0x7FFFFFFF;
#pragma unroll
                for (int j = 0; j < J; ++j)
                    if (!((taken >> j) & 1u) && ahead(key[j], lane + 64 * j, bk, be)) { bk = key[j]; be = lane + 64 * j; }
                wave_argmax(bk, be);
                if ((be & 63) == lane) taken |= 1u << (be >> 6);
                if (lane == r) { my_l = key_value(bk); my_e = be; }
            }
        }
        if (!tab) l0 = __shfl(my_l, 0);  // rank 0 holds the largest selected logit
        // renormalised softmax over the selected logits (fp64)
        const double ex = lane < k ? exp(my_l - l0) : 0.0;
        const double z = wave_sum_f64(ex);
        if (lane < k) {
            const float wv = (float)(ex / z);
            s_ids[t * k + lane] = my_e;
            s_w[t * k + lane] = wv;
            atomicOr(&s_mask[my_e], 1u << t);
            rb.ids[t * k + lane] = my_e;
            rb.w[t * k + lane] = wv;
            if (trace_ids) trace_ids[t * k + lane] = my_e;
            if (trace_w) trace_w[t * k + lane] = wv;
        }
    }
    __syncthreads();
    // exclusive scan over experts of (pairs << 16 | non-empty), 4 experts per thread
    uint32_t p[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * 4 + j;
        const uint32_t mk = e < E ? s_mask[e] : 0u;
        p[j] = ((uint32_t)__popc(mk) << 16) | (mk ? 1u : 0u);
        tot += p[j];
    }
    const uint32_t incl = wave_incl_scan_u32(tot);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    uint32_t ex = incl - tot;
    for (int w = 0; w < wave; ++w) ex += s_wsum[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * 4 + j;
        if (e < E) {
            rb.offsets[e] = s_off[e] = (int32_t)(ex >> 16);
            s_aidx[e] = (int32_t)(ex & 0xFFFFu);
        }
        ex += p[j];
    }
    if (tid == (int)blockDim.x - 1) {  // entries past E add nothing: ex is the grand total
        rb.offsets[E] = (int32_t)(ex >> 16);
        s_U = (int32_t)(ex & 0xFFFFu);
    }
    __syncthreads();
    const int U = s_U;
    if (tid < P) {
        const int t = tid / k, e = s_ids[tid];
        const int rank = __popc(s_mask[e] & ((1u << t) - 1u));
        const int pos = s_off[e] + rank;
        rb.perm[pos] = tid;
        rb.inv[tid] = pos;
        const int a = s_aidx[e];
        if (rank == 0) rb.act[a] = e;
        s_wtab[a * kMaxDecodeT + t] = s_w[tid];
    }
    if (tid == 0) {
        rb.nact[0] = U + S;
        if (S) rb.act[U] = E;
    }
    if (S && tid < T) s_wtab[U * kMaxDecodeT + tid] = 1.0f;
    __syncthreads();
    for (int i = tid; i < (U + S) * kMaxDecodeT; i += blockDim.x) rb.wtab[i] = s_wtab[i];
}

hipError_t launch_topk_sort_decode(int T, const Geom& g, RouteBufs rb, const int32_t* tab, const int32_t* tok, int vocab,
                                   int32_t* trace_ids, float* trace_w, const Launch& lc) {
    // R2 = 1 for windows of up to 4 tokens: one token per wave, no second round of logit loads
#define MOE_TOPK_CASE(J, R2) \
    launch(k_topk_sort<J, R2>, dim3(1), dim3(256), 0, lc, T, g.E, g.k, g.S, rb, tab, tok, vocab, trace_ids, trace_w)
    if (g.E <= 256) {
        if (T <= 4) MOE_TOPK_CASE(4, 1); else MOE_TOPK_CASE(4, 2);
    } else if (g.E <= 512) {
        if (T <= 4) MOE_TOPK_CASE(8, 1); else MOE_TOPK_CASE(8, 2);
    } else {
        if (T <= 4) MOE_TOPK_CASE(16, 1); else MOE_TOPK_CASE(16, 2);
    }
#undef MOE_TOPK_CASE
    return hipGetLastError();
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// One workgroup per work item (active expert a, 16-row tile rt of F): rows
// 16rt..16rt+15 of G and U.  The grid covers every item the call can have
// (min(E, T k) + S experts), workgroups past the active count exit at once,
// and the footprint is small enough that all items are resident together, so
// every weight byte of the call is requested within the first microseconds.
// The 4 waves split K = H into contiguous ranges of at most NC chunks and
// issue all their loads on entry (unconditional, indices clamped, so the
// compiler counts them) right after the workgroup's share of x, which is
// written to LDS as soon as it arrives, with the weights still in flight.
// The MFMA computes C[m][n = row] with A = x: row m = 4 g + i carries token
// R g + i for i < R (R = 1 for T <= 4, else 2), so a lane's results for its
// tokens sit in its first R result registers and only those are scaled and
// used; the other rows read some token's row and their results are ignored
// (the MFMA rows are independent), so LDS holds just the T rows of x.
// Output: v = w_t,a * silu(g) * u as the bf16 hi/lo A fragments of the down
// projection, and their per-half-block sums.
// (slots and sx are deliberately not __restrict__: with it the compiler may
// treat their loads as invariant and sink them past the barrier into the
// branch that uses them, which serialises the weight stream behind staging.)
template <int FMT, int NC, int XPER, int R>
__global__ __launch_bounds__(256) void k_gateup_decode(const uint16_t* __restrict__ x, int T,
                                                       const uint8_t* slots, Geom g,
                                                       const float* sx, const int32_t* __restrict__ nact,
                                                       const int32_t* __restrict__ act, const float* __restrict__ wtab,
                                                       int maxA, uint32_t* __restrict__ afrag,
                                                       float* __restrict__ spart) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int rtn = g.F / 16;
    const int a = blockIdx.x / rtn, rt = blockIdx.x - a * rtn;
    const int na = nact[0];
    const int e = act[min(a, maxA - 1)];  // requested together with nact
    if (a >= na) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, gs = lane >> 4, m = lane & 15;
    const int mt = (m & 3) < R ? R * (m >> 2) + (m & 3) : 15;  // token of A row m (T <= 8: 15 is no token)
    const MatGeom& mg = g.gu;
    const int c0 = wave * mg.nch / 4, c1 = (wave + 1) * mg.nch / 4;
    constexpr int CWN = FMT == 1 ? 4 : 2;
    // q4: row tile rt of G and of U; q2 / q2b64: the interleaved G|U units of row tile rt
    const int64_t base = (int64_t)e * g.slot_bytes + (int64_t)rt * mg.tile_bytes * (FMT == 1 ? 1 : 2);
    const uint8_t* Gt = slots + base + g.g_off;
    const uint8_t* Ut = slots + base + g.u_off;
    const int h8 = g.H / 8, xs8 = h8 + 1;
    // [T][H + 8]: rows padded against bank conflicts
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    const float inv_h8 = 1.0f / (float)h8;  // q < 4096, h8 <= 512: (q + 0.5) / h8 is never within 1e-3 of an integer
    // element q of row t lands at q + t (rows are h8 + 1 elements apart in LDS)
    const auto xslot = [=](int q) { return q + (int)(((float)q + 0.5f) * inv_h8); };
    StageRegs<XPER> xst;
    xst.issue(reinterpret_cast<const u32x4_t*>(x), T * h8);
    uint32_t cg[NC][CWN], cu[NC][CWN];
    u32x2_t sg[NC], su[NC];
    float sxv[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) sxv[j] = sx[(min(c0 + j, mg.nch - 1) * 4 + gs) * 16 + mt];
    __builtin_amdgcn_sched_barrier(0);
    // chunk by chunk (scheduling barriers keep the order), so the math on
    // chunk j can start as soon as chunk j has arrived
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = min(c0 + j, mg.nch - 1);
        if constexpr (FMT == 1) {
            const int64_t off = (int64_t)c * mg.chunk_bytes;
            load_codes<FMT>(Gt + off, lane, cg[j]);
            sg[j] = load_scales<FMT>(Gt + off, n);
            load_codes<FMT>(Ut + off, lane, cu[j]);
            su[j] = load_scales<FMT>(Ut + off, n);
        } else {
            load_pair_unit<FMT>(Gt + (int64_t)c * 2 * mg.chunk_bytes, lane, n, cg[j], cu[j], sg[j], su[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // routing weights of this lane's tokens R gs + i (used by wave 0 in the epilogue)
    float wt[R];
#pragma unroll
    for (int i = 0; i < R; ++i) wt[i] = wtab[a * kMaxDecodeT + R * gs + i];
    const int xstride = g.H + 8;
    xst.commit(reinterpret_cast<u32x4_t*>(xs), T * h8, xslot, T * xs8);
    __syncthreads();
    const uint16_t* xl = xs + (mt < T ? mt : 0) * xstride + 8 * gs;
    f32x4_t accG = {0.f, 0.f, 0.f, 0.f}, accU = accG, corG = accG, corU = accG;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = c0 + j;
        if (c < c1) {
            // blocks past nb (K padding) have zero scales and zero block sums:
            // any finite operand works, so the block index is clamped
            u32x4_t A[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                A[q] = *reinterpret_cast<const u32x4_t*>(xl + min(c * 4 + q, mg.nb - 1) * 32);
            chunk_mac<FMT, R>(cg[j], sg[j], A, sxv[j], gs, accG, corG);
            chunk_mac<FMT, R>(cu[j], su[j], A, sxv[j], gs, accU, corU);
        }
    }
    // waves 1..3 hand their partial sums to wave 0 through the LDS area x occupied
    __syncthreads();
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);  // [3][4][64]
    if (wave > 0) {
        red[((wave - 1) * 4 + 0) * 64 + lane] = accG;
        red[((wave - 1) * 4 + 1) * 64 + lane] = accU;
        red[((wave - 1) * 4 + 2) * 64 + lane] = corG;
        red[((wave - 1) * 4 + 3) * 64 + lane] = corU;
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        accG += red[(w * 4 + 0) * 64 + lane];
        accU += red[(w * 4 + 1) * 64 + lane];
        corG += red[(w * 4 + 2) * 64 + lane];
        corU += red[(w * 4 + 3) * 64 + lane];
    }
    // lane holds (token t = R gs + i, row f = 16 rt + n) in result register i < R.
    // v = w * silu(g) * u becomes the down projection's A operand, k = f, in
    // the layout of one MFMA fragment per 32-wide block of F: token t's bf16 hi
    // part in row 4 (t % 4) + 2 (t / 4) and its bf16 lo part in the row after,
    // plus the per-half-block row sums of both parts (all 16 rows; zeros for
    // t >= T).  R = 2: the fragment is stored whole (lane = row + 16 k-slice,
    // 64 lanes).  R = 1 (T <= 4): rows 4 gs + 2, 4 gs + 3 are zero, and only
    // the 32 lanes of rows 4t, 4t + 1 are stored, lane 8 k-slice + 2 t + (0 hi,
    // 1 lo): half the fragment traffic and LDS of the down projection.
    const int nbFp = g.dn.nch * 4;
    const int bF = rt >> 1, kf = 16 * (rt & 1) + n;
    constexpr int FL = R == 1 ? 32 : 64;
    uint16_t* af16 = reinterpret_cast<uint16_t*>(afrag) + ((int64_t)a * nbFp + bF) * FL * 8 + (kf & 7);
    const int ksl = kf >> 3;  // k-slice of f inside the block
    float shi[R], slo[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int t = R * gs + i;
        const float gv = accG[i] - QF<FMT>::kBias * corG[i];
        const float uv = accU[i] - QF<FMT>::kBias * corU[i];
        const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        const float v = t < T ? wt[i] * h : 0.f;  // rows t >= T are written as zeros
        const uint32_t hi = f2bf(v);
        const uint32_t lo = f2bf(v - bf2f(hi));
        shi[i] = row_sum_f32(bf2f(hi));
        slo[i] = row_sum_f32(bf2f(lo));
        const int fl = R == 1 ? 8 * ksl + 2 * t : 4 * (t & 3) + 2 * (t >> 2) + 16 * ksl;
        af16[fl * 8] = (uint16_t)hi;
        af16[(fl + 1) * 8] = (uint16_t)lo;
    }
    if (n == 0) {
        float* sp = spart + (((int64_t)a * nbFp + bF) * 2 + (rt & 1)) * 16;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int t = R * gs + i, rh = 4 * (t & 3) + 2 * (t >> 2);
            sp[rh] = shi[i];
            sp[rh + 1] = slo[i];
        }
        if constexpr (R == 1) {
            sp[4 * gs + 2] = 0.f;
            sp[4 * gs + 3] = 0.f;
        }
    }
}

template <int FMT, int NC, int XPER, int R>
hipError_t launch_gateup_r(const uint16_t* x, int T, const uint8_t* slots, const Geom& g, RouteBufs rb,
                           DecodeBufs db, int maxA_T, int maxA, const Launch& lc) {
    static LdsGrant granted;
    const int xbytes = T * (g.H + 8) * 2 + 16;  // + the dummy slot of the staging stores
    const int lds = xbytes > 3 * 4 * 64 * 16 ? xbytes : 3 * 4 * 64 * 16;
    hipError_t e = ensure_lds(k_gateup_decode<FMT, NC, XPER, R>, lds, granted);
    if (e != hipSuccess) return e;
    launch(k_gateup_decode<FMT, NC, XPER, R>, dim3(maxA_T * (g.F / 16)), dim3(256), lds, lc, x, T, slots, g,
           rb.sx, rb.nact, rb.act, rb.wtab, maxA, db.afrag, db.spart);
    return hipGetLastError();
}

template <int FMT, int NC, int XPER>
hipError_t launch_gateup_x(const uint16_t* x, int T, const uint8_t* slots, const Geom& g, RouteBufs rb,
                           DecodeBufs db, int maxA_T, int maxA, const Launch& lc) {
    if (T <= 4) return launch_gateup_r<FMT, NC, XPER, 1>(x, T, slots, g, rb, db, maxA_T, maxA, lc);
    return launch_gateup_r<FMT, NC, XPER, 2>(x, T, slots, g, rb, db, maxA_T, maxA, lc);
}

template <int FMT, int NC>
hipError_t launch_gateup_nc(const uint16_t* x, int T, const uint8_t* slots, const Geom& g, RouteBufs rb,
                            DecodeBufs db, int maxA_T, int maxA, const Launch& lc) {
    const int per = (T * (g.H / 8) + 255) / 256;  // <= 16
    if (per <= 2) return launch_gateup_x<FMT, NC, 2>(x, T, slots, g, rb, db, maxA_T, maxA, lc);
    if (per <= 4) return launch_gateup_x<FMT, NC, 4>(x, T, slots, g, rb, db, maxA_T, maxA, lc);
    if (per <= 5) return launch_gateup_x<FMT, NC, 5>(x, T, slots, g, rb, db, maxA_T, maxA, lc);
    if (per <= 8) return launch_gateup_x<FMT, NC, 8>(x, T, slots, g, rb, db, maxA_T, maxA, lc);
    return launch_gateup_x<FMT, NC, 16>(x, T, slots, g, rb, db, maxA_T, maxA, lc);
}

hipError_t launch_gateup_decode(const uint16_t* x, int T, const uint8_t* layer_slots, const Geom& g, RouteBufs rb,
                                DecodeBufs db, int maxA, const Launch& lc) {
    const int maxA_T = (g.E < T * g.k ? g.E : T * g.k) + g.S;
    const int per_wave = (g.gu.nch + 3) / 4;
#define MOE_GATEUP_CASE(F, N) \
    if (per_wave <= N) return launch_gateup_nc<F, N>(x, T, layer_slots, g, rb, db, maxA_T, maxA, lc);
    if (g.fmt == 1) {
        MOE_GATEUP_CASE(1, 2) MOE_GATEUP_CASE(1, 3) MOE_GATEUP_CASE(1, 4) MOE_GATEUP_CASE(1, 5)
        MOE_GATEUP_CASE(1, 6) return launch_gateup_nc<1, 8>(x, T, layer_slots, g, rb, db, maxA_T, maxA, lc);
    }
    if (g.fmt == 3) {
        MOE_GATEUP_CASE(3, 2) MOE_GATEUP_CASE(3, 3) MOE_GATEUP_CASE(3, 4) MOE_GATEUP_CASE(3, 5)
        MOE_GATEUP_CASE(3, 6) return launch_gateup_nc<3, 8>(x, T, layer_slots, g, rb, db, maxA_T, maxA, lc);
    }
    MOE_GATEUP_CASE(2, 2) MOE_GATEUP_CASE(2, 3) MOE_GATEUP_CASE(2, 4) MOE_GATEUP_CASE(2, 5)
    MOE_GATEUP_CASE(2, 6) return launch_gateup_nc<2, 8>(x, T, layer_slots, g, rb, db, maxA_T, maxA, lc);
#undef MOE_GATEUP_CASE
}

// ---------------------------------------------------------------- down projection
constexpr int kRing = 8;  // chunks in flight per wave beyond the one being multiplied

// Grid (ceil(H/128), min(E, T k) + S), 8 / RP waves.  Workgroup (rg, a)
// computes the down projection of active expert a for rows 128rg..128rg+127
// (wave w: row tiles 8rg + RP w .. + RP - 1; RP = 2 for q2 / q2b64, whose D
// stores row tiles in pairs, so one 16-byte load per lane brings the codes of
// both and each operand fragment read from LDS feeds both).  The workgroup
// first requests the expert's A fragments (token t: v hi in row 4 (t % 4) +
// 2 (t / 4), v lo in the row after, so a lane's result registers 0, 1 hold
// token lane / 16 and 2, 3 token lane / 16 + 4; NV = 2 for T <= 4 skips the
// latter and stages the compact 32-lane fragments: the lanes of the zero rows
// take a zero operand), then each wave requests the first RING chunks of its
// row tiles; the fragments go to LDS as soon as they arrive and every further
// chunk is requested as one is consumed.  K = F fits one pass (nch <= NC).
// Output: part[a][t][row].
template <int FMT, int NC, int FPER, int NV, int RP, int RING>
__global__ __launch_bounds__(512 / RP) void k_down_decode(int T, const uint8_t* slots, Geom g,
                                                          const int32_t* __restrict__ nact,
                                                          const int32_t* __restrict__ act, int maxA,
                                                          const uint32_t* __restrict__ afrag, const float* spart,
                                                          float* __restrict__ part) {
    static_assert(RP == 1 || FMT != 1, "row-tile pairs exist for q2 / q2b64 only");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int a = blockIdx.y;
    const int na = nact[0];
    const int e = act[min(a, maxA - 1)];  // requested together with nact
    if (a >= na) return;
    const int rg = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, gs = lane >> 4, m = lane & 15;
    const MatGeom& md = g.dn;
    const int nbp = md.nch * 4;
    const int rt = rg * 8 + wave * RP;  // first row tile of this wave
    const bool live = rt < g.H / 16;
    // RP = 1: row tile rt; RP = 2: the unit row of tiles rt, rt + 1 (units of two chunks' size)
    const uint8_t* Dt = slots + (int64_t)e * g.slot_bytes + g.d_off + (int64_t)(live ? rt : 0) * md.tile_bytes;
    constexpr int CWN = FMT == 1 ? 4 : 2;
    constexpr int FL = NV == 2 ? 32 : 64;  // fragment lanes stored per block
    // this lane's fragment entry; the lanes of zero rows (compact form) read
    // their neighbour's (the same address: a broadcast) and use zero
    const int fl = NV == 2 ? 8 * (lane >> 4) + 2 * ((lane & 15) >> 2) + (lane & 1) : lane;
    const bool fzero = NV == 2 && (lane & 2);
    u32x4_t* frag = reinterpret_cast<u32x4_t*>(smem);
    StageRegs<FPER> fst;
    fst.issue(reinterpret_cast<const u32x4_t*>(afrag) + (int64_t)a * nbp * FL, nbp * FL);
    const float* sp = spart + (int64_t)a * nbp * 32;
    f32x4_t acc[RP], corr[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) acc[r] = corr[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // ring depth RING (chosen by the launcher): all chunks for K of up to 8
    // chunks; for the 16-chunk case (F = 2048) the deepest ring that keeps the
    // whole grid resident at once: 2 (58 VGPRs, 8 waves per SIMD) for a
    // DeepSeek-shaped window of 4 tokens, 8 when the grid fills at most two
    // waves per SIMD (a window of 1)
    constexpr int R = RING;
    uint32_t cw[R][RP][CWN];
    u32x2_t sc[R][RP];
    float s0[R], s1[R];
    // ring of R chunks (codes, scales and the block sums of the fragment rows)
    // with unconditional (clamped) loads, fully unrolled over NC
    auto load = [&](int c, int i) {
        const int cc = min(c, md.nch - 1);
        const int bq = cc * 4 + gs;
        s0[i] = sp[bq * 32 + m];
        s1[i] = sp[bq * 32 + 16 + m];
        if constexpr (RP == 1) {
            const int64_t off = (int64_t)cc * md.chunk_bytes;
            load_codes<FMT>(Dt + off, lane, cw[i][0]);
            sc[i][0] = load_scales<FMT>(Dt + off, n);
        } else {
            load_pair_unit<FMT>(Dt + (int64_t)cc * 2 * md.chunk_bytes, lane, n, cw[i][0], cw[i][1], sc[i][0],
                                sc[i][1]);
        }
    };
    // The fragments of all token rows are written (zeros for t >= T); chunks
    // past nch (NC > nch) carry zero scales and add nothing.
    auto compute = [&](int c, int i) {
        u32x4_t A[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // padding blocks (K past F) take a zero operand too: their staged
            // entries may hold fragments of a call with the other layout
            const u32x4_t f = frag[min(c * 4 + j, nbp - 1) * FL + fl];
            A[j] = fzero || c * 4 + j >= md.nb ? u32x4_t{0u, 0u, 0u, 0u} : f;
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const u32x2_t scc = c < md.nch ? sc[i][r] : u32x2_t{0u, 0u};  // padding chunk (NC > nch): zero scales
            chunk_mac<FMT, NV>(cw[i][r], scc, A, s0[i] + s1[i], gs, acc[r], corr[r]);
        }
    };
#pragma unroll
    for (int i = 0; i < R; ++i) {
        load(i, i);
        __builtin_amdgcn_sched_barrier(0);  // chunk order kept: the math on chunk i waits for chunk i only
    }
    fst.commit(frag, nbp * FL, [](int q) { return q; }, nbp * FL);
    __syncthreads();
    // waves past the last row tile compute on tile 0 and discard the result:
    // no branch around the refill loads
    if constexpr (NC <= 8) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            compute(i, i % R);
            if (i + R < NC) load(i + R, i % R);
        }
    } else {
        // long K (16 chunks): guarded steps keep the register footprint of one chunk
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            if (i < md.nch) compute(i, i % R);
            if (i + R < NC && i + R < md.nch) load(i + R, i % R);
        }
    }
    if (!live) return;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        float v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = acc[r][i] - QF<FMT>::kBias * corr[r][i];
#pragma unroll
        for (int h = 0; h < NV / 2; ++h) {
            const int t = gs + 4 * h;  // hi + lo
            if (t < T) part[((int64_t)a * kMaxDecodeT + t) * g.H + (rt + r) * 16 + n] = v[2 * h] + v[2 * h + 1];
        }
    }
}

template <int FMT, int NC, int FPER, int NV, int RING>
hipError_t launch_down_r(int T, const uint8_t* slots, const Geom& g, RouteBufs rb, DecodeBufs db, dim3 grid, int lds,
                         int maxA, const Launch& lc) {
    constexpr int RP = FMT == 1 ? 1 : 2;  // row tiles per wave
    static LdsGrant granted;
    hipError_t e = ensure_lds(k_down_decode<FMT, NC, FPER, NV, RP, RING>, lds, granted);
    if (e != hipSuccess) return e;
    launch(k_down_decode<FMT, NC, FPER, NV, RP, RING>, grid, dim3(512 / RP), lds, lc, T, slots, g, rb.nact, rb.act,
           maxA, db.afrag, db.spart, db.part);
    return hipGetLastError();
}

template <int FMT, int NC, int FPER, int NV>
hipError_t launch_down_v(int T, const uint8_t* slots, const Geom& g, RouteBufs rb, DecodeBufs db, dim3 grid, int lds,
                         int maxA, const Launch& lc) {
    if constexpr (NC <= 8) {
        return launch_down_r<FMT, NC, FPER, NV, NC < kRing ? NC : kRing>(T, slots, g, rb, db, grid, lds, maxA, lc);
    } else {
        // the grid's waves against the chip's 1024 SIMDs: a ring of 8 while every
        // wave fits at two per SIMD, of 4 at four per SIMD, else 2
        const int64_t waves = (int64_t)grid.x * grid.y * (FMT == 1 ? 8 : 4);
        if (waves <= 2 * 1024) return launch_down_r<FMT, NC, FPER, NV, 8>(T, slots, g, rb, db, grid, lds, maxA, lc);
        if (waves <= 4 * 1024) return launch_down_r<FMT, NC, FPER, NV, 4>(T, slots, g, rb, db, grid, lds, maxA, lc);
        return launch_down_r<FMT, NC, FPER, NV, 2>(T, slots, g, rb, db, grid, lds, maxA, lc);
    }
}

template <int FMT, int NC, int FPER>
hipError_t launch_down_f(int T, const uint8_t* slots, const Geom& g, RouteBufs rb, DecodeBufs db, dim3 grid, int lds,
                         int maxA, const Launch& lc) {
    if (T <= 4) return launch_down_v<FMT, NC, FPER, 2>(T, slots, g, rb, db, grid, lds, maxA, lc);
    return launch_down_v<FMT, NC, FPER, 4>(T, slots, g, rb, db, grid, lds, maxA, lc);
}

template <int FMT, int NC>
hipError_t launch_down_nc(int T, const uint8_t* slots, const Geom& g, RouteBufs rb, DecodeBufs db, dim3 grid, int lds,
                          int maxA, const Launch& lc) {
    const int threads = FMT == 1 ? 512 : 256;  // 8 / RP waves
    const int per = (g.dn.nch * 4 * (T <= 4 ? 32 : 64) + threads - 1) / threads;  // <= 16 (F <= 2048)
    if (per <= 2) return launch_down_f<FMT, NC, 2>(T, slots, g, rb, db, grid, lds, maxA, lc);
    if (per <= 4) return launch_down_f<FMT, NC, 4>(T, slots, g, rb, db, grid, lds, maxA, lc);
    if constexpr (FMT != 1) {  // 256 threads stage up to 16 fragments each
        if (per > 8) return launch_down_f<FMT, NC, 16>(T, slots, g, rb, db, grid, lds, maxA, lc);
    }
    return launch_down_f<FMT, NC, 8>(T, slots, g, rb, db, grid, lds, maxA, lc);
}

hipError_t launch_down_decode(int T, const uint8_t* layer_slots, const Geom& g, RouteBufs rb, DecodeBufs db, int maxA,
                              const Launch& lc) {
    const int maxA_T = (g.E < T * g.k ? g.E : T * g.k) + g.S;
    const int lds = g.dn.nch * 4 * (T <= 4 ? 32 : 64) * 16 + 16;  // fragments + the dummy slot of the staging stores
    dim3 grid((g.H + kDownRowsPerWG - 1) / kDownRowsPerWG, maxA_T);
    const int nch = g.dn.nch;  // <= 16 (F <= 2048)
#define MOE_DOWN_CASE(F, N) \
    if (nch <= N) return launch_down_nc<F, N>(T, layer_slots, g, rb, db, grid, lds, maxA, lc);
    if (g.fmt == 1) {
        MOE_DOWN_CASE(1, 2) MOE_DOWN_CASE(1, 4) MOE_DOWN_CASE(1, 5) MOE_DOWN_CASE(1, 8)
        return launch_down_nc<1, 16>(T, layer_slots, g, rb, db, grid, lds, maxA, lc);
    }
    if (g.fmt == 3) {
        MOE_DOWN_CASE(3, 2) MOE_DOWN_CASE(3, 4) MOE_DOWN_CASE(3, 5) MOE_DOWN_CASE(3, 8)
        return launch_down_nc<3, 16>(T, layer_slots, g, rb, db, grid, lds, maxA, lc);
    }
    MOE_DOWN_CASE(2, 2) MOE_DOWN_CASE(2, 4) MOE_DOWN_CASE(2, 5) MOE_DOWN_CASE(2, 8)
    return launch_down_nc<2, 16>(T, layer_slots, g, rb, db, grid, lds, maxA, lc);
#undef MOE_DOWN_CASE
}

// ---------------------------------------------------------------- pre-norm
// One workgroup per token: sum of squares in fp32 (each thread strides over
// 16-byte groups, then a fixed wave/LDS tree), then h = bf16(x * 1/sqrt(ms + eps)).
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ x, int H, uint16_t* __restrict__ h) {
    __shared__ float s_part[4];
    const int t = blockIdx.x;
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (int64_t)t * H);
    u32x4_t* hr = reinterpret_cast<u32x4_t*>(h + (int64_t)t * H);
    const int n16 = H / 8;
    float ss = 0.f;
    for (int i = threadIdx.x; i < n16; i += blockDim.x) {
        const u32x4_t v = xr[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = bf2f(v[q] & 0xFFFFu), b = bf2f(v[q] >> 16);
            ss = fmaf(a, a, ss);
            ss = fmaf(b, b, ss);
        }
    }
    ss = row_sum_f32(ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
    const float r = 1.0f / sqrtf(tot / (float)H + kNormEps);
    for (int i = threadIdx.x; i < n16; i += blockDim.x) {
        const u32x4_t v = xr[i];
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16(bf2f(v[q] & 0xFFFFu) * r, bf2f(v[q] >> 16) * r);
        hr[i] = o;
    }
}

hipError_t launch_rmsnorm(const uint16_t* x, int T, int H, uint16_t* h, const Launch& lc) {
    launch(k_rmsnorm, dim3(T), dim3(256), 0, lc, x, H, h);
    return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// y[t][h] = bf16( sum_{a < nact} part[a][t][h]  (+ x[t][h]) ), experts added in
// ascending active order (routed experts by id, then the shared expert).  The
// partials are requested 32 at a time (unconditional loads, clamped index;
// entries past nact are added as zeros), so the sum costs ceil(nact / 32)
// memory round trips (one for the decode shapes' 20-30 active experts); the
// residual is requested with the first batch.
constexpr int kCombineBatch = 32;
__global__ __launch_bounds__(256) void k_combine_decode(const uint16_t* __restrict__ x, int T, int H,
                                                        const int32_t* __restrict__ nact,
                                                        const float* __restrict__ part, uint16_t* __restrict__ y,
                                                        int residual) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * H) return;
    const int nA = nact[0];
    const float xr = bf2f(x[i]);
    const float* p = part + i;  // part[a][t][h] with t*H + h = i
    const int64_t stride = (int64_t)kMaxDecodeT * H;
    float s = 0.f;
    for (int a0 = 0; a0 < nA; a0 += kCombineBatch) {
        float v[kCombineBatch];
#pragma unroll
        for (int q = 0; q < kCombineBatch; ++q) v[q] = p[min(a0 + q, nA - 1) * stride];
#pragma unroll
        for (int q = 0; q < kCombineBatch; ++q) s += a0 + q < nA ? v[q] : 0.f;
    }
    if (residual) s += xr;
    y[i] = (uint16_t)f2bf(s);
}

hipError_t launch_combine_decode(const uint16_t* x, int T, const Geom& g, RouteBufs rb, DecodeBufs db, uint16_t* y,
                                 int residual, const Launch& lc) {
    // one-wave workgroups: the partial rows' requests spread over four times as many CUs
    launch(k_combine_decode, dim3((T * g.H + 63) / 64), dim3(64), 0, lc, x, T, g.H, rb.nact, db.part, y,
                       residual);
    return hipGetLastError();
}

}  // namespace moe
