// Device helpers shared by the decode and prefill kernels of libmoe (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {

// Launch on lc.st; with profiling events, the start/stop events are bound to the
// dispatch itself (hipExtLaunchKernelGGL), so they time the kernel alone.
template <class K, class... Args>
inline void launch(K kernel, dim3 grid, dim3 block, uint32_t lds, const Launch& lc, Args... args) {
    if (lc.start)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, lc.st, lc.start, lc.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, lc.st, args...);
}

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
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// (lo, hi) -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---------------------------------------------------------------- slot format
// Offset constant of the bias trick: an operand value is 128 + q, the weight
// is d*(q - o), so the contraction over a block is d*(R - (128+o)*S).
template <int FMT> struct QF;
template <> struct QF<1> { static constexpr float kBias = 136.0f; static constexpr int kCW = 16; };
template <> struct QF<2> { static constexpr float kBias = 130.0f; static constexpr int kCW = 8; };
// q2b64: q2 codes, one scale per 64 weights (two consecutive 32-blocks share it)
template <> struct QF<3> { static constexpr float kBias = 130.0f; static constexpr int kCW = 8; };

// The exponent bits 0x4300 of both bf16 halves, held in a VGPR.  The asm
// only materialises the constant: as an opaque register value it lets each
// (w & mask) | bits below become one v_and_or_b32 (VOP3 takes at most one
// scalar or constant operand, which the mask uses).
__device__ __forceinline__ uint32_t bf16_bias_bits() {
    uint32_t k;
    asm("v_mov_b32 %0, 0x43004300" : "=v"(k));
    return k;
}
// Block j (0..3) of a chunk as the MFMA B operand: four bf16 pairs (128+q).
template <int FMT> __device__ __forceinline__ u32x4_t unpack(const uint32_t* cw, int j, uint32_t k);
template <> __device__ __forceinline__ u32x4_t unpack<1>(const uint32_t* cw, int j, uint32_t k) {
    const uint32_t w = cw[j];
    u32x4_t r;
    r.x = (w & 0x000F000Fu) | k;
    r.y = ((w >> 4) & 0x000F000Fu) | k;
    r.z = ((w >> 8) & 0x000F000Fu) | k;
    r.w = ((w >> 12) & 0x000F000Fu) | k;
    return r;
}
template <> __device__ __forceinline__ u32x4_t unpack<2>(const uint32_t* cw, int j, uint32_t k) {
    const uint32_t w = cw[j >> 1] >> (8 * (j & 1));
    u32x4_t r;
    r.x = (w & 0x00030003u) | k;
    r.y = ((w >> 2) & 0x00030003u) | k;
    r.z = ((w >> 4) & 0x00030003u) | k;
    r.w = ((w >> 6) & 0x00030003u) | k;
    return r;
}
template <> __device__ __forceinline__ u32x4_t unpack<3>(const uint32_t* cw, int j, uint32_t k) {
    return unpack<2>(cw, j, k);
}

// Expert weights are read once per call: non-temporal loads keep them from
// displacing the activations and operand fragments in the caches.
template <int FMT> __device__ __forceinline__ void load_codes(const uint8_t* chunk, int lane, uint32_t* cw) {
    if constexpr (FMT == 1) {
        u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(chunk + lane * 16));
        cw[0] = v.x; cw[1] = v.y; cw[2] = v.z; cw[3] = v.w;
    } else {
        u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(chunk + lane * 8));
        cw[0] = v.x; cw[1] = v.y;
    }
}
// Row n's chunk scales: four fp16 (blocks 0..3), or for q2b64 two fp16 in .x
// (block j of 32 weights takes the scale of 64-block j / 2).
template <int FMT> __device__ __forceinline__ u32x2_t load_scales(const uint8_t* chunk, int n) {
    if constexpr (FMT == 3)
        return u32x2_t{__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(chunk + 64 * QF<FMT>::kCW + n * 4)),
                       0u};
    else
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(chunk + 64 * QF<FMT>::kCW + n * 8));
}
// One interleaved unit of q2 / q2b64 (chunk c of two row tiles stored
// together: of G and U, or of D's row tiles 2 rp and 2 rp + 1): the lane's
// codes of both in one 16-byte load, row n's scales of both in one load (16
// bytes for q2, 8 for q2b64).
template <int FMT>
__device__ __forceinline__ void load_pair_unit(const uint8_t* unit, int lane, int n, uint32_t* cg, uint32_t* cu,
                                               u32x2_t& sg, u32x2_t& su) {
    static_assert(FMT != 1, "q4 slots are not interleaved");
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(unit + lane * 16));
    cg[0] = v.x; cg[1] = v.y; cu[0] = v.z; cu[1] = v.w;
    if constexpr (FMT == 3) {
        const u32x2_t sv = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(unit + 64 * 16 + n * 8));
        sg = u32x2_t{sv.x, 0u};
        su = u32x2_t{sv.y, 0u};
    } else {
        const u32x4_t sv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(unit + 64 * 16 + n * 16));
        sg = u32x2_t{sv.x, sv.y};
        su = u32x2_t{sv.z, sv.w};
    }
}
template <int FMT> __device__ __forceinline__ float scale_of(u32x2_t s, int j) {
    if constexpr (FMT == 3) return h2f((j & 2) ? (s.x >> 16) : (s.x & 0xFFFFu));
    const uint32_t w = (j & 2) ? s.y : s.x;
    return h2f((j & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// ---------------------------------------------------------------- wave helpers
// DPP lane permutations (GFX9 encodings): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.  Applied in this order, followed by xor 16 and
// xor 32, every lane ends up combined with every other lane of the wave.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL> __device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ double dpp_f64(double v) {
    const int lo = dpp<CTRL>(__double2loint(v)), hi = dpp<CTRL>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}
// Sum over the 16 lanes of each DPP row (every lane of the row gets it).
__device__ __forceinline__ float row_sum_f32(float v) {
    v += __int_as_float(dpp<kDppXor1>(__float_as_int(v)));
    v += __int_as_float(dpp<kDppXor2>(__float_as_int(v)));
    v += __int_as_float(dpp<kDppHalfMirror>(__float_as_int(v)));
    v += __int_as_float(dpp<kDppMirror>(__float_as_int(v)));
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<kDppXor1>(v);
    v += dpp_f64<kDppXor2>(v);
    v += dpp_f64<kDppHalfMirror>(v);
    v += dpp_f64<kDppMirror>(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Wave sums of N values per lane at once (N = 1, 2, 4, 8), reduce-scatter
// style: for each lane bit 5, 4, 3 (as many as log2 N) a lane keeps half of
// its remaining values and adds the partner lane's copy of them, so the
// exchanges shrink by half each time; the lanes left per value are then summed
// with DPP (and the cross-row exchanges N < 4 still needs).  Lane l returns
// the sum of value l >> (6 - log2 N) over all 64 lanes (every lane of that
// group of 64 / N lanes holds it).  Fixed order: deterministic.
constexpr int kDppRowRor8 = 0x128;  // row_ror:8 (lane l <-> l ^ 8 inside a row of 16)
template <class V> __device__ __forceinline__ V xchg_lane(V v, int bit) {
    if constexpr (sizeof(V) == 8) {
        if (bit == 8) return dpp_f64<kDppRowRor8>(v);
        return __shfl_xor(v, bit);
    } else {
        if (bit == 8) return __int_as_float(dpp<kDppRowRor8>(__float_as_int(v)));
        return __shfl_xor(v, bit);
    }
}
template <int N, class V> __device__ __forceinline__ V wave_sum_scatter(V (&a)[N], int lane) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "1, 2, 4 or 8 values");
    int cnt = N;
#pragma unroll
    for (int bit = 32; bit >= 8 && bit * N > 32; bit >>= 1) {
        const int half = cnt / 2;
        const bool up = (lane & bit) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            if (i < half) {
                const V keep = up ? a[i + half] : a[i], send = up ? a[i] : a[i + half];
                a[i] = keep + xchg_lane(send, bit);
            }
        }
        cnt = half;
    }
    V v = a[0];
    if constexpr (sizeof(V) == 8) {
        v += dpp_f64<kDppXor1>(v);
        v += dpp_f64<kDppXor2>(v);
        v += dpp_f64<kDppHalfMirror>(v);
        if constexpr (N <= 4) v += dpp_f64<kDppMirror>(v);
    } else {
        v += __int_as_float(dpp<kDppXor1>(__float_as_int(v)));
        v += __int_as_float(dpp<kDppXor2>(__float_as_int(v)));
        v += __int_as_float(dpp<kDppHalfMirror>(__float_as_int(v)));
        if constexpr (N <= 4) v += __int_as_float(dpp<kDppMirror>(__float_as_int(v)));
    }
    if constexpr (N <= 2) v += __shfl_xor(v, 16);
    if constexpr (N == 1) v += __shfl_xor(v, 32);
    return v;
}

// Total order of doubles as unsigned keys (-0 folded into +0).
__device__ __forceinline__ uint64_t order_key(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v + 0.0);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double key_value(uint64_t k) {
    const uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __longlong_as_double((long long)u);
}
// (key, id) ordering of the selection: larger logit first, lower id on equal logits
__device__ __forceinline__ bool ahead(uint64_t k1, int e1, uint64_t k2, int e2) {
    return k1 > k2 || (k1 == k2 && e1 < e2);
}
template <int CTRL> __device__ __forceinline__ void argmax_step(uint64_t& k, int& e) {
    const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)k);
    const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(k >> 32));
    const int oe = dpp<CTRL>(e);
    const uint64_t ok = ((uint64_t)hi << 32) | lo;
    if (ahead(ok, oe, k, e)) { k = ok; e = oe; }
}
template <int CTRL, int ROWS> __device__ __forceinline__ void argmax_bcast(uint64_t& k, int& e) {
    // lanes outside ROWS keep their own value (old = own), so the compare is a no-op there
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)k, (int)(uint32_t)k, CTRL, ROWS, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(k >> 32), (int)(uint32_t)(k >> 32), CTRL,
                                                              ROWS, 0xF, false);
    const int oe = __builtin_amdgcn_update_dpp(e, e, CTRL, ROWS, 0xF, false);
    const uint64_t ok = ((uint64_t)hi << 32) | lo;
    if (ahead(ok, oe, k, e)) { k = ok; e = oe; }
}
// Wave-wide best (key, id): row-level DPP butterflies, then row_bcast:15 and
// row_bcast:31 carry the row winners into lane 63, which is read back as a
// wave-uniform value.  Only VALU/DPP operations, no LDS round trips.
__device__ __forceinline__ void wave_argmax(uint64_t& k, int& e) {
    argmax_step<kDppXor1>(k, e);
    argmax_step<kDppXor2>(k, e);
    argmax_step<kDppHalfMirror>(k, e);
    argmax_step<kDppMirror>(k, e);
    argmax_bcast<0x142, 0xA>(k, e);  // row_bcast:15 into rows 1 and 3
    argmax_bcast<0x143, 0xC>(k, e);  // row_bcast:31 into rows 2 and 3
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
    e = __builtin_amdgcn_readlane(e, 63);
    k = ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum of a 32-bit key (DPP butterflies within rows, row
// broadcasts into lane 63, read back as a wave-uniform value).
template <int CTRL> __device__ __forceinline__ void max_step_u32(uint32_t& k) {
    const uint32_t o = (uint32_t)dpp<CTRL>((int)k);
    k = o > k ? o : k;
}
template <int CTRL, int ROWS> __device__ __forceinline__ void max_bcast_u32(uint32_t& k) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)k, (int)k, CTRL, ROWS, 0xF, false);
    k = o > k ? o : k;
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// row of 16 (lanes shifted in from outside the row add 0), then row 15's total
// into rows 1 and 3 and row 31's into rows 2 and 3 (DPP row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
    max_step_u32<kDppXor1>(k);
    max_step_u32<kDppXor2>(k);
    max_step_u32<kDppHalfMirror>(k);
    max_step_u32<kDppMirror>(k);
    max_bcast_u32<0x142, 0xA>(k);
    max_bcast_u32<0x143, 0xC>(k);
    return (uint32_t)__builtin_amdgcn_readlane((int)k, 63);
}

// Top-k of the logits a wave holds (lane l, slot j: expert l + 64 j, valid
// below E <= 1024), selected on one 32-bit key per expert: the order-preserving
// image of the fp32-rounded logit with its low 10 bits replaced by 1023 - e
// (value descending, then id ascending), so every comparison is one unsigned
// compare.  Each lane sorts its J keys once; a round takes the wave maximum of
// the lanes' heads and the winning lane drops its head.  Rounding to fp32 and
// dropping 10 low bits are both monotone: if the k+1 best keys differ above
// bit 10, their order is the fp64 order; otherwise (near or exact ties) the
// function returns false and the caller selects on the fp64 values.  On
// success lane r < k holds the id of rank r in my_e.
template <int J>
__device__ __forceinline__ bool wave_topk_fast(const double* raw, int E, int k, int lane, int& my_e) {
    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        const uint32_t u = __float_as_uint((float)raw[j] + 0.0f);
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
    uint32_t mine = 0;
    for (int r = 0; r <= k; ++r) {
        const uint32_t best = wave_max_u32(key[0]);
        // the winning lane drops its head: a bitwise select (v_bfi_b32), not an indexed move
        const uint32_t m = key[0] == best ? ~0u : 0u;
#pragma unroll
        for (int j = 0; j + 1 < J; ++j) key[j] = (key[j + 1] & m) | (key[j] & ~m);
        key[J - 1] &= ~m;
        mine = lane == r ? best : mine;
    }
    const uint32_t hv = mine >> 10;
    const uint32_t hn = (uint32_t)__shfl_down((int)hv, 1);
    if (__ballot(lane < k && (mine == 0u || hv == hn))) return false;
    my_e = lane < k ? 1023 - (int)(mine & 0x3FFu) : 0;
    return true;
}

// Raise a kernel's dynamic LDS limit when a launch needs more than the
// default 64 KiB.  The limit belongs to the kernel on each device, so what has
// been granted is kept per device ordinal (ordinals from kLdsDevices on set the
// attribute on every launch that needs it), and a mutex orders the updates of
// host threads that launch at the same time.  One LdsGrant per kernel.
constexpr int kLdsDefault = 64 * 1024;
constexpr int kLdsDevices = 64;
struct LdsGrant {
    std::mutex mu;
    int bytes[kLdsDevices];
    LdsGrant() {
        for (int& b : bytes) b = kLdsDefault;
    }
};
template <class K> hipError_t ensure_lds(K kernel, int bytes, LdsGrant& granted) {
    if (bytes <= kLdsDefault) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool tracked = dev >= 0 && dev < kLdsDevices;
    std::lock_guard<std::mutex> lk(granted.mu);
    if (tracked && bytes <= granted.bytes[dev]) return hipSuccess;
    e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && tracked) granted.bytes[dev] = bytes;
    return e;
}

// Two-step copy of n16 <= PER * blockDim.x 16-byte elements from global
// memory to LDS: issue() requests every element into registers, commit()
// stores them.  Loads and stores are unconditional (indices clamped; a slot
// past the end, `dummy`, takes the stores of out-of-range lanes), so the code
// is branch-free: loads the caller issues between the two steps (the
// weights) keep exact wait counts and the stores wait for the staged elements
// only.  A scheduling barrier after issue() keeps the staged loads first in
// the memory queue.  n16 >= 1.
template <int PER> struct StageRegs {
    u32x4_t v[PER];
    __device__ __forceinline__ void issue(const u32x4_t* __restrict__ src, int n16) {
#pragma unroll
        for (int j = 0; j < PER; ++j) v[j] = src[min((int)threadIdx.x + j * (int)blockDim.x, n16 - 1)];
        __builtin_amdgcn_sched_barrier(0);
    }
    template <class Map>
    __device__ __forceinline__ void commit(u32x4_t* dst, int n16, Map dst_index, int dummy) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = (int)threadIdx.x + j * (int)blockDim.x;
            dst[i < n16 ? dst_index(i) : dummy] = v[j];
        }
    }
};

}  // namespace moe
