"""GPU parity of the decode path (T <= 8) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from moe_inputs.configs import C1, C2, C4, MoEConfig, Q2B32, Q4B32

from parity import (W_TOL, assert_y_close, bf16_dev_to_bits, bf16_dev_to_f64, load_layer, min_routing_gap,
                    to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _check_layer(ctx, cfg, seed, layer, window, T, W, b, ex, what):
    import torch
    x = mi.gen_x(seed, window, T, cfg.H)
    xd = to_dev_bf16(x)
    print(f"[parity] {what} seed={seed} layer={layer} T={T}", flush=True)
    ids, w, offsets, perm = ctx.route(layer, xd)
    y = ctx.forward(xd, layer_begin=layer, layer_count=1)
    torch.cuda.synchronize()
    y_ref, ids_ref, w_ref, lg = oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex,
                                                 cfg.expert_bytes)
    off_ref, perm_ref, _, _ = oracle.permutation(ids_ref, cfg.E)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref, err_msg=f"{what}: ids")
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_ref, err_msg=f"{what}: offsets")
    np.testing.assert_array_equal(perm.cpu().numpy(), perm_ref, err_msg=f"{what}: perm")
    assert np.abs(w.cpu().numpy().astype(np.float64) - w_ref).max() <= W_TOL, f"{what}: weights"
    r, mx = assert_y_close(bf16_dev_to_f64(y), y_ref, what)
    print(f"[parity] {what}: rel-L2 {r:.2e} max-abs {mx:.2e} min-gap {min_routing_gap(lg, cfg.k):.2e}", flush=True)
    return y


def test_c1_tiny_layer(torch_cuda):
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = C1
    with MoEContext.from_config(cfg) as ctx:
        W, b, ex = load_layer(ctx, cfg, 1, 0)
        _check_layer(ctx, cfg, 1, 0, 0, 4, W, b, ex, "C1")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_c2_qwen_layer_window4(torch_cuda, seed):
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = C2
    with MoEContext.from_config(cfg) as ctx:
        W, b, ex = load_layer(ctx, cfg, seed, 0)
        _check_layer(ctx, cfg, seed, 0, 0, 4, W, b, ex, "C2")


SMALL_Q4_SHARED = MoEConfig("small_q4_shared", (8,), 512, 256, 24, 1, 4, 2, Q4B32, mi.BIAS_NORMAL, 0.5)
SMALL_Q2 = MoEConfig("small_q2", (8,), 640, 160, 40, 0, 6, 2, Q2B32, mi.BIAS_ZIPF, 1.1)
ODD_BLOCKS = MoEConfig("odd_blocks", (8,), 96, 224, 7, 1, 3, 1, Q2B32, mi.BIAS_NONE, 0.0)  # K/32 = 3 and 7


@pytest.mark.parametrize("cfg", [SMALL_Q4_SHARED, SMALL_Q2, ODD_BLOCKS], ids=lambda c: c.name)
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_small_configs_all_windows(torch_cuda, cfg, T):
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(cfg) as ctx:
        for layer in range(cfg.L):
            W, b, ex = load_layer(ctx, cfg, 5, layer)
            _check_layer(ctx, cfg, 5, layer, layer, T, W, b, ex, f"{cfg.name}/T{T}")


@pytest.mark.parametrize("cfg", [SMALL_Q4_SHARED, SMALL_Q2], ids=lambda c: c.name)
def test_raw_codes_cover_every_code_value(torch_cuda, cfg):
    """Uniform codes (0 included) and random-sign scales."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(cfg) as ctx:
        W, b, ex = load_layer(ctx, cfg, 9, 0, raw=True)
        for T in (1, 4, 8):
            _check_layer(ctx, cfg, 9, 0, T, T, W, b, ex, f"{cfg.name}/raw/T{T}")


def test_c4_deepseek_layer_with_shared_expert(torch_cuda):
    """One layer of the 256+1-expert q4b32 shape at windows 1 to 4 and 8 (the
    down projection's ring of in-flight chunks is 8 at a window of 1, 4 at 2,
    and 2 from 3 on)."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = C4
    with MoEContext.from_config(cfg, n_layers=1) as ctx:
        W, b, ex = load_layer(ctx, cfg, 2, 0)
        for T in (1, 2, 3, 4, 8):
            _check_layer(ctx, cfg, 2, 0, T, T, W, b, ex, f"C4/T{T}")


def test_determinism_bitwise(torch_cuda):
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = SMALL_Q2
    with MoEContext.from_config(cfg) as ctx:
        load_layer(ctx, cfg, 3, 0)
        load_layer(ctx, cfg, 3, 1)
        x = to_dev_bf16(mi.gen_x(3, 0, 8, cfg.H))
        outs = [bf16_dev_to_bits(ctx.forward(x, 0, 2, residual=True)) for _ in range(3)]
        assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_tie_break_duplicated_router_rows(torch_cuda):
    """Experts 3 and 11 with identical router rows and bias tie exactly; the lower id wins."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = MoEConfig("tie", (4,), 256, 64, 16, 0, 1, 1, Q4B32, mi.BIAS_NONE, 0.0)
    W = mi.gen_router(5, 0, cfg.E, cfg.H)
    W[11] = W[3]
    bias = np.zeros(cfg.E, dtype=np.float32)
    bias[3] = bias[11] = 50.0
    ex = mi.gen_experts(5, 0, 0, cfg.E, cfg.H, cfg.F, cfg.fmt)
    with MoEContext.from_config(cfg) as ctx:
        ctx.load(0, router_w=W, router_bias=bias, experts=ex)
        x = mi.gen_x(5, 0, 4, cfg.H)
        ids, w, _, _ = ctx.route(0, to_dev_bf16(x))
        assert ids.cpu().numpy().ravel().tolist() == [3, 3, 3, 3]
        assert np.all(w.cpu().numpy() == 1.0)
    cfg2 = MoEConfig("tie2", (4,), 256, 64, 16, 0, 2, 1, Q4B32, mi.BIAS_NONE, 0.0)
    with MoEContext.from_config(cfg2) as ctx:
        ctx.load(0, router_w=W, router_bias=bias, experts=ex)
        ids, w, _, _ = ctx.route(0, to_dev_bf16(mi.gen_x(5, 0, 4, cfg.H)))
        assert ids.cpu().numpy().tolist() == [[3, 11]] * 4
        assert np.all(w.cpu().numpy() == 0.5)


@pytest.mark.parametrize("nudge", [1, -1], ids=["up", "down"])
def test_near_tie_falls_back_to_exact_order(torch_cuda, nudge):
    """Experts 3 and 11 differ by one bf16 unit in one router weight and share a
    large bias: their logits differ by ~1e-4, far below what the fp32 selection
    keys resolve, so the kernel must select on the fp64 logits.  Ids and their
    order must equal the oracle's for every token (whichever of the two wins
    depends on the sign of that token's x element)."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = MoEConfig("near_tie", (8,), 256, 64, 16, 0, 2, 1, Q4B32, mi.BIAS_NONE, 0.0)
    W = mi.gen_router(6, 0, cfg.E, cfg.H)
    W[11] = W[3]
    W[11, 17] = np.uint16(int(W[3, 17]) + nudge)  # one unit in the last place of a bf16 (same sign)
    bias = np.zeros(cfg.E, dtype=np.float32)
    bias[3] = bias[11] = 50.0
    ex = mi.gen_experts(6, 0, 0, cfg.E, cfg.H, cfg.F, cfg.fmt)
    x = mi.gen_x(6, 0, 8, cfg.H)
    lg = oracle.router_logits(x, W, bias)
    assert np.all(lg[:, 3] != lg[:, 11]), "the nudge must separate the two logits"
    ids_ref, w_ref = oracle.select_topk(lg, cfg.k)
    with MoEContext.from_config(cfg) as ctx:
        ctx.load(0, router_w=W, router_bias=bias, experts=ex)
        ids, w, _, _ = ctx.route(0, to_dev_bf16(x))
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        assert np.abs(w.cpu().numpy().astype(np.float64) - w_ref).max() <= W_TOL
        assert set(map(tuple, ids_ref.tolist())) <= {(3, 11), (11, 3)}


def test_zero_tokens_and_error_paths(torch_cuda):
    import torch
    from quantized_expert_ffn_softmax_amd import (MOE_EINVAL, MOE_ERANGE, MOE_ESTATE, MoEContext, MoEError,
                                                  moe_forward, moe_load_experts)
    cfg = SMALL_Q4_SHARED
    with MoEContext.from_config(cfg) as ctx:
        x = to_dev_bf16(mi.gen_x(1, 0, 4, cfg.H))
        with pytest.raises(MoEError) as ei:
            ctx.forward(x)  # nothing loaded yet
        assert ei.value.status == MOE_ESTATE
        W, b, ex = mi.layer_inputs(cfg, 1, 0)
        ctx.load(0, router_w=W, router_bias=b)
        with pytest.raises(MoEError) as ei:
            ctx.forward(x)  # router loaded, experts not
        assert ei.value.status == MOE_ESTATE
        with pytest.raises(MoEError) as ei:
            moe_load_experts(ctx.handle, 0, experts=ex[:-1], expert_begin=0, expert_count=cfg.E + 1)
        assert ei.value.status == MOE_EINVAL
        ctx.load(0, experts=ex)
        y = torch.zeros_like(x)
        moe_forward(ctx.handle, x, y, 0)  # T = 0: no-op
        assert int(y.abs().sum().item()) == 0
        big = to_dev_bf16(mi.gen_x(1, 0, cfg.T[0] + 1, cfg.H))
        with pytest.raises(MoEError) as ei:
            ctx.forward(big)
        assert ei.value.status == MOE_ERANGE
        with pytest.raises(MoEError) as ei:
            moe_forward(ctx.handle, x, x, 4)  # y aliases x
        assert ei.value.status == MOE_EINVAL
        with pytest.raises(MoEError) as ei:
            moe_forward(ctx.handle, x, None, 4)
        assert ei.value.status == MOE_EINVAL
        # the context still works after rejected calls
        y = ctx.forward(x)
        torch.cuda.synchronize()
        y_ref, *_ = oracle.moe_layer(mi.gen_x(1, 0, 4, cfg.H), cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex,
                                     cfg.expert_bytes)
        assert_y_close(bf16_dev_to_f64(y), y_ref, "after errors")


def test_create_rejects_bad_geometry(torch_cuda):
    from quantized_expert_ffn_softmax_amd import MOE_EINVAL, MOE_ENOMEM, MOE_Q4B32 as Q4, MoEContext, MoEError
    for args in [(100, 64, 8, 0, 2, 1, Q4, 4), (128, 64, 8, 0, 9, 1, Q4, 4), (128, 64, 8, 2, 2, 1, Q4, 4),
                 (128, 64, 8, 0, 2, 1, 7, 4), (128, 64, 8, 0, 2, 1, Q4, 0), (8192, 64, 8, 0, 2, 1, Q4, 4),
                 (4096, 4096, 8, 0, 2, 1, Q4, 4)]:
        with pytest.raises(MoEError) as ei:
            MoEContext(*args)
        assert ei.value.status == MOE_EINVAL
    # an arena far beyond the device: ENOMEM, and nothing leaks across repeated attempts
    for _ in range(3):
        with pytest.raises(MoEError) as ei:
            MoEContext(4096, 2048, 1024, 1, 8, 64, Q4, 4)  # 64 x 1025 experts x 14.2 MB
        assert ei.value.status == MOE_ENOMEM


# The decode limits at once: 1024 experts (16 logits per lane), top-16, a
# shared expert, an 8-token window (128 pairs, up to 129 active experts),
# hidden 4096 (two 16-byte segments per lane in the router).
MAX_DECODE = MoEConfig("max_decode", (8,), 4096, 64, 1024, 1, 16, 1, Q2B32, mi.BIAS_ZIPF, 0.3)
# the largest expert (hidden 4096, FF 2048, q4b32) with top-16 and a shared
# expert: up to 129 active experts of 14.2 MB in one window of 8
MAX_FFN_DECODE = MoEConfig("max_ffn_decode", (8,), 4096, 2048, 256, 1, 16, 1, Q4B32, mi.BIAS_NORMAL, 0.5)


@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_at_the_size_limits(torch_cuda, T):
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = MAX_DECODE
    with MoEContext.from_config(cfg) as ctx:
        W, b, ex = load_layer(ctx, cfg, 12, 0)
        _check_layer(ctx, cfg, 12, 0, T, T, W, b, ex, f"max_decode/T{T}")


def test_decode_largest_experts_top16(torch_cuda):
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = MAX_FFN_DECODE
    with MoEContext.from_config(cfg) as ctx:
        W, b, ex = load_layer(ctx, cfg, 14, 0)
        for T in (4, 8):
            _check_layer(ctx, cfg, 14, 0, T, T, W, b, ex, f"max_ffn_decode/T{T}")


def test_two_contexts_interleaved(torch_cuda):
    """Two live contexts of different geometry and format (and a prefill-capable
    one) used in turn on one stream: each call matches the oracle and repeats its
    own first result bit for bit, so no state leaks between contexts."""
    import torch
    from quantized_expert_ffn_softmax_amd import MoEContext
    a_cfg, b_cfg = SMALL_Q4_SHARED, SMALL_Q2
    with MoEContext.from_config(a_cfg, max_tokens=64) as ca, MoEContext.from_config(b_cfg) as cb:
        a_in = load_layer(ca, a_cfg, 17, 0)
        b_in = load_layer(cb, b_cfg, 18, 0)
        first = {}
        for rnd in range(2):
            for name, ctx, cfg, inp, T in (("a4", ca, a_cfg, a_in, 4), ("b8", cb, b_cfg, b_in, 8),
                                            ("a40", ca, a_cfg, a_in, 40), ("b3", cb, b_cfg, b_in, 3)):
                x = mi.gen_x(19, 0, T, cfg.H)
                y = ctx.forward(to_dev_bf16(x))
                torch.cuda.synchronize()
                bits = bf16_dev_to_bits(y)
                if rnd == 0:
                    first[name] = bits
                    y_ref = oracle.moe_layer(x, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, *inp, cfg.expert_bytes)[0]
                    assert_y_close(bf16_dev_to_f64(y), y_ref, f"two contexts/{name}")
                else:
                    np.testing.assert_array_equal(bits, first[name], err_msg=f"two contexts/{name} repeat")
