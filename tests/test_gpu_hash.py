"""GPU parity of hash-routed layers (a [vocab x k] token-id -> experts table
instead of the top-k; DeepSeek V4 Flash's layers 0-2) against the oracle,
through the C ABI: decode windows, prefill chunks, a chain mixing hash-routed
and score-routed layers, token ids outside the table, and the argument checks.

The oracle's hash routing (oracle.route_hash) is pinned by the CPU tests; the
experts and the combine are the same oracle functions as for score routing.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from moe_inputs.configs import MoEConfig, Q2B32, Q4B32

from parity import W_TOL, assert_y_close, bf16_dev_to_bits, bf16_dev_to_f64, to_dev_bf16

pytestmark = pytest.mark.gpu

SEED = 9
VOCAB = 97
HASH_DS = MoEConfig("hash_ds", (4,), 512, 128, 24, 1, 6, 2, Q4B32, mi.BIAS_NORMAL, 0.5)
HASH_QW = MoEConfig("hash_qw", (4,), 640, 160, 40, 0, 10, 2, Q2B32, mi.BIAS_ZIPF, 1.1)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _ctx(cfg, max_tokens, hash_layers):
    from quantized_expert_ffn_softmax_amd import MoEContext
    ctx = MoEContext.from_config(cfg, max_tokens=max_tokens)
    tables = {}
    for layer in range(cfg.L):
        W, b, ex = mi.layer_inputs(cfg, SEED, layer)
        tab = mi.gen_tid2eid(SEED, layer, VOCAB, cfg.E, cfg.k) if layer in hash_layers else None
        ctx.load(layer, router_w=W, router_bias=b, experts=ex, tid2eid=tab)
        tables[layer] = (W, b, ex, tab)
    return ctx, tables


def _ref_layer(cfg, x_bits, W, b, ex, tab, tok):
    lg = oracle.router_logits(x_bits, W, b)
    if tab is None:
        ids, w = oracle.select_topk(lg, cfg.k)
    else:
        ids, w = oracle.route_hash(lg, tab, tok)
    y = oracle.combine(x_bits, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, ids, w, ex, cfg.expert_bytes)
    return y, ids, w


def _dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("cfg", [HASH_DS, HASH_QW], ids=lambda c: c.name)
@pytest.mark.parametrize("T", [1, 4, 8, 37, 300])
def test_hash_layer_matches_oracle(torch_cuda, cfg, T):
    """Layer 0 hash-routed: ids are the table rows of the tokens (bit-exact, in
    table order), weights within 1e-6, offsets/perm exact, y within the bar;
    decode windows (T <= 8) and prefill chunks (T > 8)."""
    import torch
    ctx, tables = _ctx(cfg, max(T, 8), hash_layers={0})
    with ctx:
        W, b, ex, tab = tables[0]
        x = mi.gen_x(SEED, T, T, cfg.H)
        tok = mi.gen_token_ids(SEED, T, T, VOCAB)
        xd, tokd = to_dev_bf16(x), _dev_i32(tok)
        print(f"[hash] {cfg.name} T={T}", flush=True)
        ids, w, offsets, perm = ctx.route(0, xd, token_ids=tokd)
        y = ctx.forward(xd, 0, 1, token_ids=tokd)
        torch.cuda.synchronize()
        y_ref, ids_ref, w_ref = _ref_layer(cfg, x, W, b, ex, tab, tok)
        np.testing.assert_array_equal(ids.cpu().numpy(), tab[tok])
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        assert np.abs(w.cpu().numpy().astype(np.float64) - w_ref).max() <= W_TOL
        off_ref, perm_ref, _, _ = oracle.permutation(ids_ref, cfg.E)
        np.testing.assert_array_equal(offsets.cpu().numpy(), off_ref)
        np.testing.assert_array_equal(perm.cpu().numpy(), perm_ref)
        r, mx = assert_y_close(bf16_dev_to_f64(y), y_ref, f"{cfg.name} T={T}")
        print(f"[hash] {cfg.name} T={T}: rel-L2 {r:.2e} max-abs {mx:.2e}", flush=True)


@pytest.mark.parametrize("T", [4, 64])
def test_chain_mixing_hash_and_score_layers(torch_cuda, T):
    """Two layers with the residual, layer 0 hash-routed and layer 1 by score
    (the pages' DeepSeek layout: hash layers first): per-layer routing on the
    GPU's own layer input (trace_x) equals the oracle's, and layer 1's output
    matches the oracle within the bar."""
    import torch
    cfg = HASH_DS
    ctx, tables = _ctx(cfg, max(T, 8), hash_layers={0})
    with ctx:
        x = mi.gen_x(SEED, 50 + T, T, cfg.H)
        tok = mi.gen_token_ids(SEED, 50 + T, T, VOCAB)
        y, tx, tids, tw = ctx.forward(to_dev_bf16(x), 0, 2, residual=True, trace=True, token_ids=_dev_i32(tok))
        torch.cuda.synchronize()
        txb = bf16_dev_to_bits(tx)
        for layer in range(2):
            W, b, ex, tab = tables[layer]
            y_ref, ids_ref, w_ref = _ref_layer(cfg, txb[layer], W, b, ex, tab, tok)
            np.testing.assert_array_equal(tids.cpu().numpy()[layer], ids_ref, err_msg=f"layer {layer}")
            assert np.abs(tw.cpu().numpy()[layer].astype(np.float64) - w_ref).max() <= W_TOL
        # layer 1 output: y = x_1 + MoE_1(x_1), x_1 the GPU's own layer input
        W, b, ex, tab = tables[1]
        y1_ref, _, _ = _ref_layer(cfg, txb[1], W, b, ex, tab, tok)
        assert_y_close(bf16_dev_to_f64(y), oracle.bf16_to_f64(txb[1]) + y1_ref, f"chain T={T}")


def test_token_ids_outside_the_table_are_clamped(torch_cuda):
    """Ids below 0 use row 0, ids at or above vocab use row vocab-1 (both paths)."""
    import torch
    cfg = HASH_DS
    ctx, tables = _ctx(cfg, 64, hash_layers={0})
    with ctx:
        tab = tables[0][3]
        for T in (4, 20):
            tok = np.array(([-5, VOCAB, 3, 10 ** 6] * 5)[:T], dtype=np.int32)
            x = mi.gen_x(SEED, 77, T, cfg.H)
            ids, _, _, _ = ctx.route(0, to_dev_bf16(x), token_ids=_dev_i32(tok))
            torch.cuda.synchronize()
            np.testing.assert_array_equal(ids.cpu().numpy(), tab[np.clip(tok, 0, VOCAB - 1)])


def test_hash_argument_checks(torch_cuda):
    """A hash-routed layer without token ids, and bad tables, are rejected
    before any work; a new table (other vocab) replaces the old one."""
    import torch
    from quantized_expert_ffn_softmax_amd import MOE_EINVAL, MoEContext, MoEError
    cfg = HASH_DS
    with MoEContext.from_config(cfg, max_tokens=16) as ctx:
        W, b, ex = mi.layer_inputs(cfg, SEED, 0)
        good = mi.gen_tid2eid(SEED, 0, VOCAB, cfg.E, cfg.k)
        bad_range = good.copy()
        bad_range[5, 2] = cfg.E
        bad_dup = good.copy()
        bad_dup[7, 1] = bad_dup[7, 0]
        for tab in (bad_range, bad_dup, np.zeros((0, cfg.k), np.int32)):
            with pytest.raises(MoEError) as e:
                ctx.load(0, router_w=W, router_bias=b, experts=ex, tid2eid=tab)
            assert e.value.status == MOE_EINVAL
        ctx.load(0, router_w=W, router_bias=b, experts=ex, tid2eid=good)
        x = to_dev_bf16(mi.gen_x(SEED, 0, 4, cfg.H))
        with pytest.raises(MoEError) as e:
            ctx.forward(x, 0, 1)
        assert e.value.status == MOE_EINVAL
        with pytest.raises(MoEError) as e:
            ctx.route(0, x)
        assert e.value.status == MOE_EINVAL
        small = mi.gen_tid2eid(SEED + 1, 0, 5, cfg.E, cfg.k)
        ctx.load(0, tid2eid=small)
        tok = np.array([0, 1, 4, 9], dtype=np.int32)
        ids, _, _, _ = ctx.route(0, x, token_ids=_dev_i32(tok))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids.cpu().numpy(), small[np.clip(tok, 0, 4)])
