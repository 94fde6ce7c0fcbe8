"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check compares the oracle with a library routine, a brute-force
enumeration, a closed form, or a byte count printed on the pages, so that a
dropped term, a wrong sign or index, a swapped nibble or a transposed operand
in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as mi
import oracle
from moe_inputs.configs import C1, C2, C2_Q2B64, C3, C3_Q2B64, C4, C5, CONFIGS, Q2B32, Q2B64, Q4B32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- decoding
def test_fp16_decode_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_value(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    lib = oracle.lib()
    got = np.array([lib.oracle_bf16(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])


ALL_FMTS = [Q4B32, Q2B32, Q2B64]
BW = {Q4B32: 32, Q2B32: 32, Q2B64: 64}  # weights per block


def _numpy_decode_block(block: np.ndarray, fmt: int) -> np.ndarray:
    """Independent numpy decoder of one canonical block (bit unpacking by numpy)."""
    d = float(block[:2].view(np.float16)[0])
    codes = block[2:]
    if fmt == Q4B32:
        q = np.stack([codes & 0xF, codes >> 4], axis=1).ravel().astype(np.int64)
        return d * (q - 8)
    q = np.stack([(codes >> s) & 3 for s in (0, 2, 4, 6)], axis=1).ravel().astype(np.int64)
    return d * (q - 2)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_block_decode_matches_numpy_decoder(fmt):
    ex = mi.gen_experts(7, 0, 0, 1, 256, 128, fmt, raw=True)
    bb = mi.block_bytes(fmt)
    assert mi.block_weights(fmt) == BW[fmt]
    blocks = ex.reshape(-1, bb)[:200]
    for blk in blocks:
        ref = _numpy_decode_block(blk, fmt)
        assert ref.shape == (BW[fmt],)
        got = np.array([oracle.block_weight(blk, fmt, j) for j in range(BW[fmt])])
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_matrix_decode_matches_numpy_decoder(fmt):
    """Whole G, U and D of one expert: row r, column c is element c % BW of
    block r * (K / BW) + c / BW of its matrix (numpy reshape, no oracle indexing)."""
    H, F = 256, 128
    ex = mi.gen_experts(8, 0, 0, 1, H, F, fmt, raw=True)
    bb, bw = mi.block_bytes(fmt), BW[fmt]
    blocks = ex.reshape(-1, bb)
    dec = np.stack([_numpy_decode_block(b, fmt) for b in blocks])  # [nblocks x bw]
    ng = F * H // bw
    G, U, D = oracle.expert_matrices(ex, H, F, fmt)
    np.testing.assert_array_equal(G, dec[:ng].reshape(F, H))
    np.testing.assert_array_equal(U, dec[ng:2 * ng].reshape(F, H))
    np.testing.assert_array_equal(D, dec[2 * ng:].reshape(H, F))


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_dequant_round_trip_on_grid(fmt):
    """Weights on the grid d*(q-o) re-quantise to identical bytes."""
    rng = np.random.default_rng(3)
    nq = 16 if fmt == Q4B32 else 4
    o = 8 if fmt == Q4B32 else 2
    qmax = 7 if fmt == Q4B32 else 1
    bw = BW[fmt]
    for _ in range(200):
        q = rng.integers(0, nq, size=bw)
        q[rng.integers(0, bw)] = o + qmax  # the block's absmax sits on code o+qmax
        q = np.where(np.abs(q - o) > qmax, o + qmax, q)
        d = float(np.float16(rng.uniform(1e-4, 1e-1)))
        w = d * (q - o).astype(np.float64)
        blk = mi.quantize_block(w, fmt)
        deq = np.array([oracle.block_weight(blk, fmt, j) for j in range(bw)])
        np.testing.assert_array_equal(deq, w)
        np.testing.assert_array_equal(mi.quantize_block(deq, fmt), blk)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_dequant_error_bound_off_grid(fmt):
    """Quantised N(0,0.02) draws decode within d/2 of the draw (no clamping
    inside the scale's range)."""
    qmax = 7 if fmt == Q4B32 else 1
    bw = BW[fmt]
    z = mi.normals(11, mi.TAG_EXPERT, 0, 0, 0, bw * 300).reshape(300, bw) * 0.02
    for w in z:
        blk = mi.quantize_block(w, fmt)
        d = oracle.fp16_value(int(blk[0]) | (int(blk[1]) << 8))
        deq = np.array([oracle.block_weight(blk, fmt, j) for j in range(bw)])
        amax = np.abs(w).max()
        inside = np.abs(w) <= d * qmax
        assert np.all(np.abs(w - deq)[inside] <= d / 2 + 1e-15)
        # clamped codes only occur where fp16 rounding put d*qmax below absmax
        assert np.all(np.abs(deq[~inside]) == d * qmax) and np.all(np.abs(w[~inside]) <= amax)


# ------------------------------------------------------------------ routing
def test_router_logits_match_numpy_matmul():
    cfg = C2
    x = mi.gen_x(1, 0, 4, cfg.H)
    W = mi.gen_router(1, 0, cfg.E, cfg.H)
    b = mi.gen_bias(1, 0, cfg.E, cfg.bias_kind, cfg.bias_param)
    got = oracle.router_logits(x, W, b)
    ref = oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(W).T + b.astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _brute_force_selected(l: np.ndarray, k: int) -> set:
    E = l.shape[0]
    sel = set()
    for e in range(E):
        better = sum(1 for e2 in range(E) if l[e2] > l[e] or (l[e2] == l[e] and e2 < e))
        if better < k:
            sel.add(e)
    return sel


@pytest.mark.parametrize("name", ["C1", "C2", "C4", "C5"])
def test_selection_matches_brute_force_rank_count(name):
    cfg = CONFIGS[name]
    T = min(cfg.T[-1], 24)
    layer = 3 if cfg.L > 3 else 0
    x = mi.gen_x(2, 0, T, cfg.H)
    W = mi.gen_router(2, layer, cfg.E, cfg.H)
    b = mi.gen_bias(2, layer, cfg.E, cfg.bias_kind, cfg.bias_param)
    lg = oracle.router_logits(x, W, b)
    ids, w = oracle.select_topk(lg, cfg.k)
    for t in range(T):
        assert set(ids[t].tolist()) == _brute_force_selected(lg[t], cfg.k)
        # selection order is (logit descending, id ascending): np.lexsort is the library reference
        order = np.lexsort((np.arange(cfg.E), -lg[t]))[: cfg.k]
        assert ids[t].tolist() == order.tolist()


def test_tie_break_lowest_id_at_boundary():
    # equal logits for experts 3 and 11 exactly at the k-th boundary
    E, k = 16, 4
    l = np.linspace(-1.0, 1.0, E)[::-1].copy()  # expert 0 best, descending
    l[3] = l[11] = 0.05
    l[[0, 1, 2]] = [2.0, 1.5, 1.0]
    l[[4, 5, 6, 7, 8, 9, 10, 12, 13, 14, 15]] = -np.arange(1, 12) * 0.1
    ids, w = oracle.select_topk(l[None, :], k)
    assert ids[0].tolist() == [0, 1, 2, 3]
    # the same tie produced through the router: duplicated router rows 3 and 11
    H = 64
    x = mi.gen_x(5, 0, 1, H)
    W = mi.gen_router(5, 0, E, H)
    W[11] = W[3]
    bias = np.zeros(E, dtype=np.float32)
    bias[3] = bias[11] = 50.0  # both far ahead of every other expert
    lg = oracle.router_logits(x, W, bias)
    assert lg[0, 3] == lg[0, 11]
    ids, w = oracle.select_topk(lg, 1)
    assert ids[0, 0] == 3 and w[0, 0] == 1.0
    ids, w = oracle.select_topk(lg, 2)
    assert ids[0].tolist() == [3, 11]
    assert w[0, 0] == w[0, 1] == 0.5


def test_weights_sum_to_one_and_special_cases():
    cfg = C2
    x = mi.gen_x(3, 0, 8, cfg.H)
    W = mi.gen_router(3, 0, cfg.E, cfg.H)
    b = mi.gen_bias(3, 0, cfg.E, cfg.bias_kind, cfg.bias_param)
    lg = oracle.router_logits(x, W, b)
    ids, w = oracle.select_topk(lg, cfg.k)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(w[:, :-1] >= w[:, 1:])  # descending with the logits
    # renormalised top-k softmax equals the softmax of the selected logits (closed form)
    sel = np.take_along_axis(lg, ids, axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-12, atol=0)
    # k = 1 gives weight exactly 1
    ids1, w1 = oracle.select_topk(lg, 1)
    assert np.all(w1 == 1.0)
    # k = E equals the full softmax (textbook routine)
    idsE, wE = oracle.select_topk(lg, cfg.E)
    full = scipy.special.softmax(lg, axis=1)
    np.testing.assert_allclose(wE, np.take_along_axis(full, idsE, axis=1), rtol=1e-12, atol=1e-300)


# -------------------------------------------------------------- permutation
def test_hash_routing_two_experts_is_the_logistic_function():
    """k = 2: the weights are sigmoid(l_a - l_b) and its complement (scipy)."""
    rng = np.random.default_rng(11)
    lg = rng.normal(0, 2, (64, 9))
    table = np.stack([rng.permutation(9)[:2] for _ in range(20)]).astype(np.int32)
    tok = rng.integers(0, 20, 64).astype(np.int32)
    ids, w = oracle.route_hash(lg, table, tok)
    np.testing.assert_array_equal(ids, table[tok])  # table order, not logit order
    la = lg[np.arange(64), ids[:, 0]]
    lb = lg[np.arange(64), ids[:, 1]]
    np.testing.assert_allclose(w[:, 0], scipy.special.expit(la - lb), rtol=0, atol=1e-14)
    np.testing.assert_allclose(w[:, 1], scipy.special.expit(lb - la), rtol=0, atol=1e-14)


def test_hash_routing_with_the_top_k_table_equals_score_routing():
    """A table whose row for each token is that token's score top-k gives the
    score-routing result (ids and weights), so the two weight rules agree."""
    rng = np.random.default_rng(12)
    T, E, k = 32, 40, 5
    lg = rng.normal(0, 1, (T, E))
    ids_s, w_s = oracle.select_topk(lg, k)
    ids_h, w_h = oracle.route_hash(lg, ids_s, np.arange(T, dtype=np.int32))
    np.testing.assert_array_equal(ids_h, ids_s)
    np.testing.assert_allclose(w_h, w_s, rtol=0, atol=1e-15)


def test_hash_routing_invariants():
    """Weights sum to 1, k = 1 gives exactly 1, a per-token shift of all logits
    and any change to the logits of experts outside the row leave them
    unchanged, and permuting a row permutes its weights the same way."""
    rng = np.random.default_rng(13)
    T, E, k, V = 24, 30, 4, 50
    lg = rng.normal(0, 3, (T, E))
    table = np.stack([rng.permutation(E)[:k] for _ in range(V)]).astype(np.int32)
    tok = rng.integers(0, V, T).astype(np.int32)
    ids, w = oracle.route_hash(lg, table, tok)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    _, w1 = oracle.route_hash(lg, table[:, :1].copy(), tok)
    assert np.all(w1 == 1.0)
    _, w_shift = oracle.route_hash(lg + rng.normal(0, 5, (T, 1)), table, tok)
    np.testing.assert_allclose(w_shift, w, rtol=0, atol=1e-13)
    lg2 = lg.copy()
    outside = np.ones((T, E), bool)
    outside[np.arange(T)[:, None], ids] = False
    lg2[outside] = rng.normal(0, 3, outside.sum())
    _, w_out = oracle.route_hash(lg2, table, tok)
    np.testing.assert_allclose(w_out, w, rtol=0, atol=1e-13)
    perm = rng.permutation(k)
    ids_p, w_p = oracle.route_hash(lg, table[:, perm].copy(), tok)
    np.testing.assert_array_equal(ids_p, ids[:, perm])
    np.testing.assert_allclose(w_p, w[:, perm], rtol=0, atol=1e-15)


@pytest.mark.parametrize("T,k,E", [(4, 2, 16), (4, 10, 512), (8, 6, 256), (4096, 6, 256), (1, 1, 1)])
def test_permutation_matches_stable_argsort(T, k, E):
    rng = np.random.default_rng(T * 1000 + k)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    off, perm, inv, active = oracle.permutation(ids, E)
    flat = ids.ravel()
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert off[-1] == T * k
    np.testing.assert_array_equal(inv[perm], np.arange(T * k))  # bijection, inv o perm = id
    np.testing.assert_array_equal(active, np.unique(flat))


# ------------------------------------------------------------------ the FFN
def _dense_ffn(G, U, D, x):
    g = G @ x
    u = U @ x
    return D @ (g * scipy.special.expit(g) * u)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_single_expert_equals_dense_ffn(fmt):
    """E = 1, k = 1: the layer is one dense FFN (numpy float64 matmuls)."""
    H, F = 256, 96 if BW[fmt] == 32 else 128
    ex = mi.gen_experts(4, 0, 0, 1, H, F, fmt)
    G, U, D = oracle.expert_matrices(ex, H, F, fmt)
    # the matrices decode the same through the independent numpy decoder
    bb = mi.block_bytes(fmt)
    np.testing.assert_array_equal(G.ravel()[:BW[fmt]], _numpy_decode_block(ex[:bb], fmt))
    x = mi.gen_x(4, 0, 3, H)
    W = mi.gen_router(4, 0, 1, H)
    y, ids, w, _ = oracle.moe_layer(x, H, F, 1, 0, 1, fmt, W, None, ex, len(ex))
    assert np.all(ids == 0) and np.all(w == 1.0)
    for t in range(3):
        ref = _dense_ffn(G, U, D, oracle.bf16_to_f64(x[t]))
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-15)
    out, h = oracle.expert_ffn(ex, H, F, fmt, oracle.bf16_to_f64(x[0]), want_h=True)
    g = G @ oracle.bf16_to_f64(x[0])
    np.testing.assert_allclose(h, g * scipy.special.expit(g) * (U @ oracle.bf16_to_f64(x[0])), rtol=1e-12, atol=1e-16)


def test_zero_input_gives_zero_output():
    cfg = C1
    W, b, ex = mi.layer_inputs(cfg, 1, 0)
    x = np.zeros((4, cfg.H), dtype=np.uint16)
    y, ids, w, lg = oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex, cfg.expert_bytes)
    assert np.all(y == 0.0)
    assert np.all(lg == 0.0) and ids.tolist() == [[0, 1]] * 4  # all logits tie: lowest ids


def _dense_layer(cfg, x, W, b, ex):
    """Brute force: every expert on every token, masked by the selection."""
    xd = oracle.bf16_to_f64(x)
    lg = xd @ oracle.bf16_to_f64(W).T + (b.astype(np.float64) if b is not None else 0.0)
    T = x.shape[0]
    y = np.zeros((T, cfg.H))
    nb = cfg.expert_bytes
    outs = []
    for e in range(cfg.E + cfg.S):
        G, U, D = oracle.expert_matrices(ex[e * nb:(e + 1) * nb], cfg.H, cfg.F, cfg.fmt)
        outs.append(np.stack([_dense_ffn(G, U, D, xd[t]) for t in range(T)]))
    for t in range(T):
        order = np.lexsort((np.arange(cfg.E), -lg[t]))
        mask = np.zeros(cfg.E)
        mask[order[: cfg.k]] = 1.0
        wsel = mask * np.exp(lg[t] - lg[t].max())
        wsel /= wsel.sum()
        for e in range(cfg.E):
            y[t] += wsel[e] * outs[e][t]
        if cfg.S:
            y[t] += outs[cfg.E][t]
    return y


def test_layer_equals_brute_force_dense_c1():
    cfg = C1
    W, b, ex = mi.layer_inputs(cfg, 1, 0)
    x = mi.gen_x(1, 0, 4, cfg.H)
    y, *_ = oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex, cfg.expert_bytes)
    np.testing.assert_allclose(y, _dense_layer(cfg, x, W, b, ex), rtol=1e-11, atol=1e-15)


def test_layer_with_shared_expert_equals_brute_force():
    from moe_inputs.configs import MoEConfig
    cfg = MoEConfig("tiny_shared", (5,), 128, 64, 8, 1, 3, 1, Q4B32, mi.BIAS_NORMAL, 0.5)
    W, b, ex = mi.layer_inputs(cfg, 9, 2)
    x = mi.gen_x(9, 1, 5, cfg.H)
    y, *_ = oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex, cfg.expert_bytes)
    np.testing.assert_allclose(y, _dense_layer(cfg, x, W, b, ex), rtol=1e-11, atol=1e-15)


def test_combine_with_arbitrary_routing_equals_dense():
    """The combine step on its own, as the hash-routed tests call it: ids in
    table order (not sorted, not the score top-k), weights that do not sum to
    1, a shared expert; equal to numpy's dense sum over the decoded matrices."""
    from moe_inputs.configs import MoEConfig
    cfg = MoEConfig("tiny_combine", (3,), 96, 64, 7, 1, 3, 1, Q2B32, mi.BIAS_NONE, 0.0)
    ex = mi.gen_experts(11, 0, 0, cfg.E + cfg.S, cfg.H, cfg.F, cfg.fmt)
    x = mi.gen_x(11, 0, 3, cfg.H)
    ids = np.array([[5, 0, 3], [6, 2, 1], [1, 4, 0]], dtype=np.int32)
    w = np.array([[0.5, 0.25, 1.5], [1.0, -0.75, 0.125], [2.0, 0.0, 0.3]])
    y = oracle.combine(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, ids, w, ex, cfg.expert_bytes)
    nb = cfg.expert_bytes
    mats = [oracle.expert_matrices(ex[e * nb:(e + 1) * nb], cfg.H, cfg.F, cfg.fmt) for e in range(cfg.E + 1)]
    for t in range(3):
        xd = oracle.bf16_to_f64(x[t])
        ref = sum(w[t, j] * _dense_ffn(*mats[ids[t, j]], xd) for j in range(cfg.k)) + _dense_ffn(*mats[cfg.E], xd)
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-15)


def test_residual_rounding_matches_torch():
    rng = np.random.default_rng(0)
    xb = mi.gen_x(1, 0, 2, 64)
    y = rng.normal(size=(2, 64)) * 0.3
    got = oracle.residual_bf16(xb, y)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float()
    ref = (xf + torch.from_numpy(y).float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)


# --------------------------------------------------------- chain pre-norm
def _bits(vals):
    return (np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_rmsnorm_closed_forms():
    # constant rows normalise to 1 (eps = 0), a (3, 4) row to (3, 4) / sqrt(12.5)
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(_bits([2.0] * 8), eps=0.0), _bits([1.0] * 8))
    got = oracle.bf16_to_f64(oracle.rmsnorm_bf16(_bits([3.0, 4.0]), eps=0.0))
    want = np.array([3.0, 4.0]) / np.sqrt(12.5)
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0**-9)
    # one element of 64 at 1, the rest 0: rms = 1/8, so the element becomes 8
    row = np.zeros(64, dtype=np.float32)
    row[5] = 1.0
    h = oracle.bf16_to_f64(oracle.rmsnorm_bf16(_bits(row), eps=0.0))
    assert h[5] == 8.0 and np.count_nonzero(h) == 1


def test_rmsnorm_matches_torch_rne_and_invariants():
    xb = mi.gen_x(3, 0, 4, 512)
    xf = oracle.bf16_to_f64(xb)
    h = oracle.rmsnorm_bf16(xb)
    r = xf / np.sqrt((xf**2).mean(axis=1, keepdims=True) + oracle.RMSNORM_EPS)
    ref = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(h, ref)
    hf = oracle.bf16_to_f64(h)
    assert np.all(np.abs(np.sqrt((hf**2).mean(axis=1)) - 1.0) < 2.0**-8)
    # exact invariants with eps = 0: a power-of-two scale drops out, the sign flips through
    h0 = oracle.rmsnorm_bf16(xb, eps=0.0)
    x8 = _bits(xf * 8.0)
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(x8, eps=0.0), h0)
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(xb ^ np.uint16(0x8000), eps=0.0), h0 ^ np.uint16(0x8000))


# --------------------------------------------------------- byte accounting
def test_byte_accounting_matches_pages():
    # DeepSeek-V4-Flash ("Strata 改源码去跑 DeepSeek V4 Flash？", section 二, GGUF
    # table): the Q4_K expert tensors total 145.125 GiB; q4b32 is the same 4.5
    # bits per weight, so 43 layers x 256 routed experts give exactly that.
    assert 43 * 256 * C4.expert_bytes == int(145.125 * 2**30)
    assert mi.expert_bytes(4096, 2048, Q4B32) == 14_155_776
    # Qwen3.8-Flash-Next (same page, section 三 item 4): the fixed per-expert blob
    # is 1,382,400 bytes = 3 x 2560 x 640 weights at 2.25 bits; q2b32 spends 2.5
    # bits, i.e. 10/9 of the blob.
    assert 3 * 2560 * 640 * 9 // 32 == 1_382_400
    assert C2.expert_bytes == 1_536_000 == 1_382_400 * 10 // 9
    # the teardown page ("Strata 引擎深度拆解", its addendum on the three-tier
    # VRAM/RAM/NVMe layout) puts one more GB of VRAM at roughly 700 more experts
    assert int(1e9 // 1_382_400) == 723
    # q2b64 (one fp16 scale per 64 two-bit codes) is exactly the blob, and the
    # 48 x 512 Qwen experts take the 34 GB of the Q2_0 tier (same page, section 一)
    assert C2_Q2B64.expert_bytes == C3_Q2B64.expert_bytes == 1_382_400
    assert mi.expert_bytes(2560, 640, Q2B64) == 1_382_400
    assert round(48 * 512 * C3_Q2B64.expert_bytes / 1e9) == 34


def test_c5_zipf_calibration_fixture():
    """The stored Zipf exponent was written by tests/golden/make_golden.py from the oracle."""
    with open(os.path.join(GOLDEN, "c5_zipf.json")) as f:
        rec = json.load(f)
    assert rec["s"] == C5.bias_param
    assert rec["max_tokens_per_expert"] > 500
    assert rec["previous_s_max"] <= 500
    assert sum(rec["histogram"]) == 4096 * 6


def test_selected_experts_helper_equals_full_layer():
    """The parity helper that generates only the selected experts (and the
    shared one) gives the full-layer oracle's output bit for bit."""
    from moe_inputs.configs import MoEConfig, Q2B32, Q4B32
    from parity import oracle_layer_selected
    for cfg in (MoEConfig("sel_q4s", (5,), 256, 96, 24, 1, 4, 3, Q4B32, mi.BIAS_NORMAL, 0.5),
                MoEConfig("sel_q2", (3,), 320, 64, 40, 0, 6, 2, Q2B32, mi.BIAS_ZIPF, 1.1)):
        for layer in range(cfg.L):
            W, b, ex = mi.layer_inputs(cfg, 4, layer)
            x = mi.gen_x(4, layer, cfg.T[0], cfg.H)
            y, ids, w, _ = oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex, cfg.expert_bytes)
            y2, ids2, w2 = oracle_layer_selected(x, cfg, 4, layer, W, b)
            np.testing.assert_array_equal(ids2, ids)
            np.testing.assert_array_equal(w2, w)
            np.testing.assert_array_equal(y2, y)
