"""GPU parity of the prefill path (T > 8: grouped GEMMs on MFMA) against the
fp64 oracle, through the C ABI.

Routing (ids, weights, offsets, perm) is compared for every token; y is
compared over the whole [T x H] output at sizes the oracle finishes in
seconds, and for the 4096-token chunk over the whole rows of the tokens at the
first and last row of every M-block of the grouped GEMMs (a token's output
depends only on its own row, so the oracle evaluates those rows alone).
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from moe_inputs.configs import C1, C2, C5, MoEConfig, Q2B32, Q4B32

from parity import (W_TOL, assert_y_close, bf16_dev_to_bits, bf16_dev_to_f64, load_layer, min_routing_gap,
                    to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _check_routing(ctx, cfg, layer, xd, x, W, b, what):
    ids, w, offsets, perm = ctx.route(layer, xd)
    lg = oracle.router_logits(x, W, b)
    ids_ref, w_ref = oracle.select_topk(lg, cfg.k)
    off_ref, perm_ref, _, _ = oracle.permutation(ids_ref, cfg.E)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref, err_msg=f"{what}: ids")
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_ref, err_msg=f"{what}: offsets")
    np.testing.assert_array_equal(perm.cpu().numpy(), perm_ref, err_msg=f"{what}: perm")
    dw = float(np.abs(w.cpu().numpy().astype(np.float64) - w_ref).max())
    assert dw <= W_TOL, f"{what}: weights differ by {dw:.2e}"
    return lg, ids_ref, off_ref


def _check_full(ctx, cfg, seed, layer, window, T, W, b, ex, what):
    import torch
    x = mi.gen_x(seed, window, T, cfg.H)
    xd = to_dev_bf16(x)
    print(f"[prefill] {what} seed={seed} layer={layer} T={T}", flush=True)
    lg, _, off = _check_routing(ctx, cfg, layer, xd, x, W, b, what)
    y = ctx.forward(xd, layer_begin=layer, layer_count=1)
    torch.cuda.synchronize()
    y_ref, _, _, _ = oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex, cfg.expert_bytes)
    r, mx = assert_y_close(bf16_dev_to_f64(y), y_ref, what)
    print(f"[prefill] {what}: rel-L2 {r:.2e} max-abs {mx:.2e} min-gap {min_routing_gap(lg, cfg.k):.2e} "
          f"max rows/expert {int(np.diff(off).max())}", flush=True)
    return y


# Small shapes that still span several 128-row M-blocks, ragged N-tiles
# (F = 160: 1.25 gate/up tiles; H = 640: 2.5 down tiles) and padded K chunks
# (K/32 = 3 and 7 blocks).
PF_Q4_SHARED = MoEConfig("pf_q4_shared", (1000,), 512, 256, 24, 1, 4, 2, Q4B32, mi.BIAS_NORMAL, 0.5)
PF_Q2 = MoEConfig("pf_q2", (600,), 640, 160, 40, 0, 6, 1, Q2B32, mi.BIAS_ZIPF, 1.1)
PF_ODD = MoEConfig("pf_odd", (300,), 96, 224, 7, 1, 3, 1, Q2B32, mi.BIAS_NONE, 0.0)
PF_WIDE = MoEConfig("pf_wide", (200,), 256, 64, 1000, 0, 16, 1, Q4B32, mi.BIAS_ZIPF, 1.1)  # 16 logits per lane
# Padded K with whole N-tiles: gate/up at H = 544 (17 blocks, F = 256: two
# full 128-feature tiles), down at F = 352 (11 blocks, H = 512: two full tiles).
PF_W8_K1 = MoEConfig("pf_w8_k1", (300,), 544, 256, 12, 1, 3, 1, Q4B32, mi.BIAS_NORMAL, 0.5)
PF_W8_K2 = MoEConfig("pf_w8_k2", (300,), 512, 352, 10, 0, 2, 1, Q2B32, mi.BIAS_NONE, 0.0)


@pytest.mark.parametrize("cfg", [PF_Q4_SHARED, PF_Q2, PF_ODD, PF_WIDE, PF_W8_K1, PF_W8_K2], ids=lambda c: c.name)
def test_small_prefill_full_output(torch_cuda, cfg):
    from quantized_expert_ffn_softmax_amd import MoEContext
    T = cfg.T[0]
    with MoEContext.from_config(cfg, max_tokens=T) as ctx:
        for layer in range(cfg.L):
            W, b, ex = load_layer(ctx, cfg, 7, layer)
            _check_full(ctx, cfg, 7, layer, layer, T, W, b, ex, f"{cfg.name}/T{T}")


@pytest.mark.parametrize("T", [9, 37, 128, 129, 257])
def test_ragged_token_counts(torch_cuda, T):
    """Prefill sizes just past the decode limit and around the 128-row M-block and 256-token sort block."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = PF_Q4_SHARED
    with MoEContext.from_config(cfg, max_tokens=300, n_layers=1) as ctx:
        W, b, ex = load_layer(ctx, cfg, 11, 0)
        _check_full(ctx, cfg, 11, 0, T, T, W, b, ex, f"ragged/T{T}")


def test_c1_shape_prefill(torch_cuda):
    """The tiny shape (16 experts: one logit per lane) with a 64-token chunk."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(C1, max_tokens=64) as ctx:
        W, b, ex = load_layer(ctx, C1, 1, 0)
        _check_full(ctx, C1, 1, 0, 3, 64, W, b, ex, "C1/T64")


def test_c2_shape_prefill(torch_cuda):
    """The Qwen-shaped layer (512 experts, q2b32, Zipf bias) with a 96-token chunk."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(C2, max_tokens=96) as ctx:
        W, b, ex = load_layer(ctx, C2, 1, 0)
        _check_full(ctx, C2, 1, 0, 5, 96, W, b, ex, "C2/T96")


def tile_edge_tokens(off, perm, k, T, S, rows_per_tile=128):
    """Tokens of the first and last sorted row of every M-block of the grouped
    GEMMs: expert e's rows off[e]..off[e+1] cut into blocks of 128 rows (the
    last one ragged), then the shared expert's T rows cut the same way.  A
    token's output row depends on every N-tile of both GEMMs, so checking these
    tokens' whole rows compares an output of every (expert, M-block) tile."""
    toks = set()
    E = len(off) - 1
    for e in range(E):
        for r0 in range(int(off[e]), int(off[e + 1]), rows_per_tile):
            r1 = min(r0 + rows_per_tile, int(off[e + 1])) - 1
            toks.add(int(perm[r0]) // k)
            toks.add(int(perm[r1]) // k)
    if S:
        for t0 in range(0, T, rows_per_tile):
            toks.add(t0)
            toks.add(min(t0 + rows_per_tile, T) - 1)
    return np.array(sorted(toks), dtype=np.int64)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_c5_prefill_chunk(torch_cuda, seed):
    """4096 tokens x hidden 4096, 256+1 experts, top-6, q4b32: routing for every
    token; y over the whole rows of the tokens that sit at the first and last
    row of every M-block of the grouped GEMMs (every (expert, 128-row block)
    tile has two of its rows' outputs compared, ragged tails included), with
    rel-L2 and max-abs taken over all those rows together."""
    import torch
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = C5
    T = 4096
    with MoEContext.from_config(cfg) as ctx:
        W, b, ex = load_layer(ctx, cfg, seed, 0)
        x = mi.gen_x(seed, 0, T, cfg.H)
        xd = to_dev_bf16(x)
        print(f"[prefill] C5 seed={seed}", flush=True)
        lg, ids_ref, off = _check_routing(ctx, cfg, 0, xd, x, W, b, f"C5/seed{seed}")
        _, perm_ref, _, _ = oracle.permutation(ids_ref, cfg.E)
        counts = np.diff(off)
        y = ctx.forward(xd)
        torch.cuda.synchronize()
        yg = bf16_dev_to_f64(y)
        sample = tile_edge_tokens(off, perm_ref, cfg.k, T, cfg.S)
        n_tiles = int(sum((c + 127) // 128 for c in counts)) + (T + 127) // 128
        print(f"[prefill] C5 seed={seed}: rows/expert max {counts.max()} mean {counts.mean():.1f}; {n_tiles} M-blocks,"
              f" {len(sample)} tokens checked", flush=True)
        y_ref, ids_s, _, _ = oracle.moe_layer(np.ascontiguousarray(x[sample]), cfg.H, cfg.F, cfg.E, cfg.S, cfg.k,
                                              cfg.fmt, W, b, ex, cfg.expert_bytes)
        np.testing.assert_array_equal(ids_s, ids_ref[sample])
        r, mx = assert_y_close(yg[sample], y_ref, f"C5/seed{seed} tile-edge rows")
        print(f"[prefill] C5 seed={seed}: tile-edge rows rel-L2 {r:.2e} max-abs {mx:.2e}", flush=True)
        # property at any size: y is finite and its rows are not all zero
        assert np.isfinite(yg).all()
        assert (np.abs(yg).max(axis=1) > 0).all()


def test_prefill_chain_teacher_forced(torch_cuda):
    """Two layers with the residual: each layer's traced input reproduces its
    own single-layer output, and the chain's output is the residual sum."""
    import torch
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = PF_Q4_SHARED
    T = 150
    with MoEContext.from_config(cfg, max_tokens=T) as ctx:
        inputs = [load_layer(ctx, cfg, 13, layer) for layer in range(2)]
        x = mi.gen_x(13, 0, T, cfg.H)
        xd = to_dev_bf16(x)
        y, tx, tids, tw = ctx.forward(xd, 0, 2, residual=True, trace=True)
        torch.cuda.synchronize()
        txb = bf16_dev_to_bits(tx)
        np.testing.assert_array_equal(txb[0], x)
        for layer, (W, b, ex) in enumerate(inputs):
            y_ref, ids_ref, w_ref, _ = oracle.moe_layer(txb[layer], cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b,
                                                        ex, cfg.expert_bytes)
            np.testing.assert_array_equal(tids[layer].cpu().numpy(), ids_ref)
            assert np.abs(tw[layer].cpu().numpy() - w_ref).max() <= W_TOL
            if layer == 0:
                # layer 1's input is the residual stream bf16(x0 + y0), rounded once from fp32
                assert_y_close(oracle.bf16_to_f64(txb[1]), oracle.bf16_to_f64(txb[0]) + y_ref, "residual stream")
        y_last = oracle.moe_layer(txb[1], cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, *inputs[1], cfg.expert_bytes)[0]
        y_ref = oracle.bf16_to_f64(txb[1]) + y_last
        assert_y_close(bf16_dev_to_f64(y), y_ref, "prefill chain output")


@pytest.mark.parametrize("cfg,T", [(PF_Q4_SHARED, 300), (PF_Q2, 600), (PF_ODD, 300)], ids=lambda v: getattr(v, "name", str(v)))
def test_prefill_raw_codes_cover_every_code_value(torch_cuda, cfg, T):
    """Uniform codes over the full range (0 and the maximum included) and
    random-sign scales through the grouped GEMMs' in-register dequantisation."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(cfg, max_tokens=T, n_layers=1) as ctx:
        W, b, ex = load_layer(ctx, cfg, 9, 0, raw=True)
        _check_full(ctx, cfg, 9, 0, 2, T, W, b, ex, f"{cfg.name}/raw/T{T}")


def test_prefill_determinism_bitwise(torch_cuda):
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = PF_Q2
    with MoEContext.from_config(cfg, max_tokens=600) as ctx:
        load_layer(ctx, cfg, 3, 0)
        x = to_dev_bf16(mi.gen_x(3, 0, 600, cfg.H))
        outs = [bf16_dev_to_bits(ctx.forward(x)) for _ in range(3)]
        assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_prefill_tie_break(torch_cuda):
    """Experts 3 and 11 with identical router rows and bias tie exactly for every token; the lower id wins."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = MoEConfig("tie_pf", (40,), 256, 64, 16, 0, 1, 1, Q4B32, mi.BIAS_NONE, 0.0)
    W = mi.gen_router(5, 0, cfg.E, cfg.H)
    W[11] = W[3]
    bias = np.zeros(cfg.E, dtype=np.float32)
    bias[3] = bias[11] = 50.0
    ex = mi.gen_experts(5, 0, 0, cfg.E, cfg.H, cfg.F, cfg.fmt)
    with MoEContext.from_config(cfg, max_tokens=40) as ctx:
        ctx.load(0, router_w=W, router_bias=bias, experts=ex)
        x = mi.gen_x(5, 0, 40, cfg.H)
        ids, w, _, _ = ctx.route(0, to_dev_bf16(x))
        assert ids.cpu().numpy().ravel().tolist() == [3] * 40
        assert np.all(w.cpu().numpy() == 1.0)


def test_decode_and_prefill_agree_on_routing(torch_cuda):
    """T = 8 (decode kernels) and the same 8 rows inside a T = 16 call (prefill kernels) route identically."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = PF_Q2
    with MoEContext.from_config(cfg, max_tokens=16) as ctx:
        load_layer(ctx, cfg, 4, 0)
        x = mi.gen_x(4, 0, 16, cfg.H)
        ids8, w8, _, _ = ctx.route(0, to_dev_bf16(np.ascontiguousarray(x[:8])))
        ids16, w16, _, _ = ctx.route(0, to_dev_bf16(x))
        np.testing.assert_array_equal(ids8.cpu().numpy(), ids16.cpu().numpy()[:8])
        assert np.abs(w8.cpu().numpy() - w16.cpu().numpy()[:8]).max() <= 1e-7


def test_long_chunk_many_sort_blocks(torch_cuda):
    """A 12,000-token chunk: 47 256-token sort blocks, several 128-row M-blocks
    per expert, a shared expert over every token."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = MoEConfig("pf_long", (12000,), 256, 128, 64, 1, 8, 1, Q4B32, mi.BIAS_ZIPF, 0.5)
    with MoEContext.from_config(cfg, max_tokens=12000) as ctx:
        W, b, ex = load_layer(ctx, cfg, 13, 0)
        _check_full(ctx, cfg, 13, 0, 0, 12000, W, b, ex, "long/T12000")


def test_max_sizes_chunk(torch_cuda):
    """The largest call the boundary accepts in every dimension at once: a
    65,536-token chunk (max_tokens), hidden 4096, FF 2048, top-16, a shared
    expert (1.1M sorted rows; o alone is 18 GB), so every 64-bit offset and the
    tile list run at their limits.  Routing and y on sampled tokens (the
    first, the last and 24 seeded ones); y finite and non-zero everywhere."""
    import torch
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = MoEConfig("pf_max", (65536,), 4096, 2048, 64, 1, 16, 1, Q4B32, mi.BIAS_NORMAL, 0.5)
    T = 65536
    with MoEContext.from_config(cfg, max_tokens=T) as ctx:
        W, b, ex = load_layer(ctx, cfg, 21, 0)
        x = mi.gen_x(21, 0, T, cfg.H)
        xd = to_dev_bf16(x)
        print(f"[prefill] max sizes: T={T} H={cfg.H} F={cfg.F} E={cfg.E}+{cfg.S} k={cfg.k}", flush=True)
        ids, w, offsets, perm = ctx.route(0, xd)
        y = ctx.forward(xd)
        torch.cuda.synchronize()
        off = offsets.cpu().numpy()
        assert off[0] == 0 and off[-1] == T * cfg.k and (np.diff(off) >= 0).all()
        pm = perm.cpu().numpy()
        assert np.array_equal(np.sort(pm), np.arange(T * cfg.k))
        rng = np.random.default_rng(21)
        sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 24, replace=False)]))
        y_ref, ids_s, w_s, _ = oracle.moe_layer(np.ascontiguousarray(x[sample]), cfg.H, cfg.F, cfg.E, cfg.S, cfg.k,
                                                cfg.fmt, W, b, ex, cfg.expert_bytes)
        np.testing.assert_array_equal(ids.cpu().numpy()[sample], ids_s)
        assert np.abs(w.cpu().numpy()[sample].astype(np.float64) - w_s).max() <= W_TOL
        yg = bf16_dev_to_f64(y)
        r, mx = assert_y_close(yg[sample], y_ref, "max sizes sampled")
        print(f"[prefill] max sizes: sampled rel-L2 {r:.2e} max-abs {mx:.2e}", flush=True)
        assert np.isfinite(yg).all()
        assert (np.abs(yg).max(axis=1) > 0).all()
