// Internal declarations shared by the host runtime and the kernels of libmoe.
//
// Device layout of one expert slot (gfx950 decode/prefill format)
// ----------------------------------------------------------------
// A quantised matrix [R x K] (R output rows, K input dim, blocks of 32 along K)
// is stored as R/16 "row tiles" of 16 rows.  A row tile is a sequence of
// chunks of 4 blocks (K padded up to a multiple of 128 with zero-scale
// blocks).  One chunk is laid out for a 64-lane wave that feeds the bf16
// MFMA v_mfma_f32_16x16x32_bf16 with the weights as its B operand:
//
//   codes : 64 lanes x CW bytes, lane l = n + 16*g holds row n (0..15) of the
//           tile and k-slice g (elements 8g..8g+7 of each block)
//           q4 (CW = 16): word j = block j of the chunk; nibble p (bits 4p)
//                          holds element 8g+2p, nibble p+4 (bits 16+4p) holds
//                          element 8g+2p+1, p = 0..3
//           q2 (CW = 8):  word j = blocks 2j (bits 0..7, 16..23) and 2j+1
//                          (bits 8..15, 24..31); inside a block half, bits 2p
//                          hold element 8g+2p and bits 16+2p element 8g+2p+1
//           q2b64 codes: as q2 (a 64-weight block is two 32-weight halves)
//   scales: 16 rows x 4 fp16, row n's scales of blocks 0..3 (8 bytes);
//           q2b64: 16 rows x 2 fp16, row n's scales of its two 64-blocks
//           (4 bytes), so a q2b64 chunk is 576 bytes against q2's 640
//
// With that bit order, (word >> s) & mask | 0x4300 0x4300 is the bf16 pair
// (128 + q_k, 128 + q_k+1) for consecutive k, so a code is turned into an
// exact MFMA operand with one shift and one and-or; the offset 128 + o is
// removed after the contraction with the per-block sums of the other operand.
//
// An expert slot holds G and U (F/16 row tiles each, K = H), then D (H/16 row
// tiles, K = F), and is padded to a multiple of 256 bytes.  q4: G, then U, as
// two matrices.  q2 and q2b64: G and U interleaved chunk by chunk, so that a
// lane of the decode gate/up kernel reads both with one 16-byte load: unit
// (rt, c) at (rt nch + c) 2 chunk_bytes holds 64 lanes x 16 bytes (the lane's
// G code bytes, then its U code bytes), then 16 rows x 2 s bytes (row n's G
// scales, then its U scales; s = 8 for q2, 4 for q2b64).  Their D pairs its
// row tiles the same way: unit (rp, c) at d_off + (rp nch + c) 2 chunk_bytes
// holds row tiles 2 rp (first half of every lane entry and scale row) and
// 2 rp + 1 (second half); H is a multiple of 32, so every tile has its pair.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

constexpr int kChunkBlocks = 4;
constexpr int kMaxDecodeT = 8;   // decode path: tokens share one 16-row MFMA tile (hi/lo halves)
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;

struct MatGeom {
    int rows;        // R
    int K;           // input dim
    int nb;          // K / 32
    int nch;         // chunks per row tile (nb padded to a multiple of 4, / 4)
    int chunk_bytes; // q4: 1152, q2: 640, q2b64: 576
    int64_t tile_bytes;
    int64_t bytes;   // rows/16 * tile_bytes
};

struct Geom {
    int H, F, E, S, k, fmt, L;
    MatGeom gu;      // G and U: [F x H]
    MatGeom dn;      // D: [H x F]
    int64_t g_off, u_off, d_off;  // g_off = u_off = 0 when G and U are interleaved (q2, q2b64)
    int64_t slot_bytes;
    int64_t canon_expert_bytes;
};

inline int code_bytes_per_lane(int fmt) { return fmt == 1 ? 16 : 8; }
inline int scale_bytes_per_row(int fmt) { return fmt == 3 ? 4 : 8; }  // per chunk
inline int canon_block_weights(int fmt) { return fmt == 3 ? 64 : 32; }
inline int canon_block_bytes(int fmt) { return fmt == 2 ? 10 : 18; }
inline bool gu_interleaved(int fmt) { return fmt != 1; }

inline MatGeom make_mat(int rows, int K, int fmt) {
    MatGeom m;
    m.rows = rows;
    m.K = K;
    m.nb = K / 32;
    m.nch = (m.nb + kChunkBlocks - 1) / kChunkBlocks;
    m.chunk_bytes = 64 * code_bytes_per_lane(fmt) + 16 * scale_bytes_per_row(fmt);
    m.tile_bytes = (int64_t)m.nch * m.chunk_bytes;
    m.bytes = (int64_t)(rows / 16) * m.tile_bytes;
    return m;
}

inline Geom make_geom(int H, int F, int E, int S, int k, int fmt, int L) {
    Geom g;
    g.H = H; g.F = F; g.E = E; g.S = S; g.k = k; g.fmt = fmt; g.L = L;
    g.gu = make_mat(F, H, fmt);
    g.dn = make_mat(H, F, fmt);
    g.g_off = 0;
    g.u_off = gu_interleaved(fmt) ? 0 : g.gu.bytes;
    g.d_off = 2 * g.gu.bytes;
    g.slot_bytes = (2 * g.gu.bytes + g.dn.bytes + 255) / 256 * 256;
    g.canon_expert_bytes = 3LL * H * F / canon_block_weights(fmt) * canon_block_bytes(fmt);
    return g;
}

// Per-call routing scratch (device), sized for max_tokens by the runtime.
struct RouteBufs {
    double* logits;   // [T x E]
    float* sx;        // [nbH_pad x 16] per-block sums of the x rows (rows >= T zero)
    int32_t* ids;     // [T x k]
    float* w;         // [T x k]
    int32_t* offsets; // [E + 1]
    int32_t* perm;    // [T*k]
    int32_t* inv;     // [T*k]
    int32_t* nact;    // [1]   number of active experts incl. the shared one
    int32_t* act;     // [maxA] expert id of active slot a (ascending; shared last)
    float* wtab;      // [maxA x 8] routing weight of token t for active slot a (decode)
};

// Decode FFN scratch.
struct DecodeBufs {
    uint32_t* afrag;  // [maxA x nbF_pad x 64 x 4] v = w*SwiGLU as bf16 hi/lo MFMA A fragments (T <= 4: 32 lanes per block)
    float* spart;     // [maxA x nbF_pad x 2 x 16] per-half-block sums of the fragment rows
    float* part;      // [maxA x 8 x H] per-expert down projections
};

constexpr int kDownRowsPerWG = 128;  // 8 waves x 16 rows

// Prefill scratch (T > kMaxDecodeT), sized for max_tokens.
constexpr int kPfBlockTokens = 256;  // tokens per counting-sort block
constexpr int kPfTileRows = 128;     // rows of one grouped-GEMM M-block
struct PrefillBufs {
    float* logits;     // [ksplit x T x E] fp32 MFMA partial logits (K split; no bias)
    int32_t* ids;      // [T x k]
    float* w;          // [T x k]
    uint32_t* blkcnt;  // [nblk x E] pairs per (token block, expert)
    int32_t* rank;     // [T x k]   rank of the pair inside its (block, expert) group
    int32_t* offsets;  // [E + 1]
    int32_t* perm;     // [T*k]
    int32_t* inv;      // [T*k]
    int32_t* rowtok;   // [T*k + S*T] token of each sorted row (routed rows by expert, then shared rows)
    int32_t* blkbase;  // [nblk x E] first sorted position of the (block, expert) group
    int32_t* tiles;    // [max_tiles x 4] (row0, nrows, group, 0)
    int32_t* ntiles;   // [1]
    uint16_t* h;       // [(T*k + S*T) x F] bf16 SwiGLU output in sorted row order
    float* o;          // [(T*k + S*T) x H] fp32 per-row expert outputs
    int max_tiles;
    int T;             // tokens of the current call (set by the GEMM launchers on their copy)
    int ksplit;        // K split of the router logits (set by the top-k launcher on its copy)
};
// K split of the prefill router GEMM: doubled (up to 8, keeping H / 32 a
// multiple) while the 128 x 256 tiles times the split fill at most 256
// workgroups, so a chunk of a few thousand tokens still covers the CUs.
inline int pf_router_splits(int T, int E, int H) {
    const int tiles = ((T + 127) / 128) * ((E + 255) / 256);
    int ks = 1;
    while (ks < 8 && tiles * ks * 2 <= 256 && (H / 32) % (ks * 2) == 0) ks *= 2;
    return ks;
}
// floats of the partial-logit buffer for chunks of up to Tm tokens: with a
// split, the tiles times the split are at most 256 (so ks T E <= 256 x 128 x 256)
inline int64_t pf_router_partial_floats(int Tm, int E) {
    const int64_t one = (int64_t)Tm * E;
    return std::max<int64_t>(one, std::min<int64_t>(8 * one, 256LL * 128 * 256));
}
inline int prefill_max_tiles(int T, int k, int E, int S) {
    const int64_t P = (int64_t)T * k;
    return (int)((P + kPfTileRows - 1) / kPfTileRows + std::min<int64_t>(E, P) +
                 (S ? (T + kPfTileRows - 1) / kPfTileRows : 0));
}

// Stream and optional profiling events of one launch.
struct Launch {
    hipStream_t st;
    hipEvent_t start = nullptr, stop = nullptr;
};

// Launchers (return hipGetLastError()).
hipError_t launch_repack(const uint8_t* canon, uint8_t* slots, int count, const Geom& g, hipStream_t st);
// hm: NULL, or [T x H] bf16 that receives the per-token RMS pre-norm of x, which
// the router then routes on (fused pre-norm of a decode chain layer)
hipError_t launch_router_decode(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const Geom& g,
                                RouteBufs rb, uint16_t* hm, const Launch& lc);
// tab: NULL (score routing) or the layer's [vocab x k] hash table; tok: the tokens' ids
hipError_t launch_topk_sort_decode(int T, const Geom& g, RouteBufs rb, const int32_t* tab, const int32_t* tok, int vocab,
                                   int32_t* trace_ids, float* trace_w, const Launch& lc);
hipError_t launch_gateup_decode(const uint16_t* x, int T, const uint8_t* layer_slots, const Geom& g, RouteBufs rb,
                                DecodeBufs db, int maxA, const Launch& lc);
hipError_t launch_down_decode(int T, const uint8_t* layer_slots, const Geom& g, RouteBufs rb, DecodeBufs db, int maxA,
                              const Launch& lc);
hipError_t launch_combine_decode(const uint16_t* x, int T, const Geom& g, RouteBufs rb, DecodeBufs db, uint16_t* y,
                                 int residual, const Launch& lc);

// Per-token unit-gain RMS normalisation h = bf16(x / sqrt(mean(x^2) + eps)), fp32.
constexpr float kNormEps = 1e-6f;
hipError_t launch_rmsnorm(const uint16_t* x, int T, int H, uint16_t* h, const Launch& lc);

// Prefill launchers; rstat = {max_e ||W_r[e]||_2, max_e |b[e]|} of the layer's router.
hipError_t launch_router_stats(const uint16_t* Wr, const float* bias, int E, int H, float* rstat, hipStream_t st);
hipError_t launch_pf_router(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const Geom& g,
                            PrefillBufs pb, const Launch& lc);
hipError_t launch_pf_topk(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const float* rstat,
                          const Geom& g, PrefillBufs pb, int32_t* trace_ids, float* trace_w, const Launch& lc);
// Hash-routed prefill layer: ids from the table, exact logits of those ids, weights.
hipError_t launch_pf_hash(const uint16_t* x, int T, const uint16_t* Wr, const float* bias, const int32_t* tab,
                          const int32_t* tok, int vocab, const Geom& g, PrefillBufs pb, int32_t* trace_ids,
                          float* trace_w, const Launch& lc);
hipError_t launch_pf_hist(int T, const Geom& g, PrefillBufs pb, const Launch& lc);
hipError_t launch_pf_scan(int T, const Geom& g, PrefillBufs pb, const Launch& lc);
hipError_t launch_pf_scatter(int T, const Geom& g, PrefillBufs pb, const Launch& lc);
hipError_t launch_pf_gemm1(const uint16_t* x, int T, const uint8_t* layer_slots, const Geom& g, PrefillBufs pb,
                           const Launch& lc);
hipError_t launch_pf_gemm2(const uint8_t* layer_slots, const Geom& g, PrefillBufs pb, const Launch& lc);
hipError_t launch_pf_combine(const uint16_t* x, int T, const Geom& g, PrefillBufs pb, uint16_t* y, int residual,
                             const Launch& lc);

}  // namespace moe
