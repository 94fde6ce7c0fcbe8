"""GPU parity of the q2b64 expert format (2-bit codes, one fp16 scale per 64
weights: 2.25 bits per weight, the size of the pages' 2-bit expert blob)
against the fp64 oracle, through the C ABI.

Covers the decode path (the Qwen shape at windows 1/4/8, small shapes at
every window class, padded K chunks holding half a 64-block, a shared
expert, raw codes covering every code value), the prefill path (several
128-row M-blocks, ragged N-tiles, padded K), a short teacher-forced chain with
the pre-norm and residual, and bitwise determinism."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from moe_inputs.configs import C2_Q2B64, C3_Q2B64, MoEConfig, Q2B64

from parity import (W_TOL, assert_y_close, bf16_dev_to_bits, bf16_dev_to_f64, load_layer, min_routing_gap,
                    to_dev_bf16)

pytestmark = pytest.mark.gpu

# H = 640: 20 blocks of 32, 5 full chunks; F = 192: 6 blocks, the second down
# chunk holds one 64-block and one zero-scale padding 64-block.
SMALL = MoEConfig("q2b64_small", (8,), 640, 192, 40, 0, 6, 2, Q2B64, mi.BIAS_ZIPF, 1.1)
# H = 320: the third gate/up chunk holds 64-block 4 and padding; F = 64: one
# half-padded down chunk; a shared expert.
ODD = MoEConfig("q2b64_odd", (8,), 320, 64, 9, 1, 3, 1, Q2B64, mi.BIAS_NONE, 0.0)


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
    print(f"[q2b64] {what} seed={seed} layer={layer} T={T}", flush=True)
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
    print(f"[q2b64] {what}: rel-L2 {r:.2e} max-abs {mx:.2e} min-gap {min_routing_gap(lg, cfg.k):.2e}", flush=True)
    return y


def test_expert_bytes_are_the_blob_size(torch_cuda):
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(C2_Q2B64, n_layers=1) as ctx:
        assert ctx.expert_bytes == 1_382_400 == C2_Q2B64.expert_bytes


def test_qwen_shape_decode_windows(torch_cuda):
    """512 experts, top-10, H 2560, F 640 at windows 1, 4, 8."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = C2_Q2B64
    with MoEContext.from_config(cfg, max_tokens=8) as ctx:
        W, b, ex = load_layer(ctx, cfg, 1, 0)
        for T in (1, 4, 8):
            _check_layer(ctx, cfg, 1, 0, T, T, W, b, ex, f"C2_q2b64/T{T}")


@pytest.mark.parametrize("cfg", [SMALL, ODD], ids=lambda c: c.name)
@pytest.mark.parametrize("T", [1, 3, 4, 5, 8])
def test_small_decode_all_window_classes(torch_cuda, cfg, T):
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(cfg) as ctx:
        for layer in range(cfg.L):
            W, b, ex = load_layer(ctx, cfg, 6, layer)
            _check_layer(ctx, cfg, 6, layer, layer, T, W, b, ex, f"{cfg.name}/T{T}")


def test_raw_codes_cover_every_code_value(torch_cuda):
    """Uniform codes (0 included) and random-sign scales, decode and prefill."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = SMALL
    with MoEContext.from_config(cfg, max_tokens=200, n_layers=1) as ctx:
        W, b, ex = load_layer(ctx, cfg, 9, 0, raw=True)
        for T in (1, 4, 8, 200):
            _check_layer(ctx, cfg, 9, 0, T, T, W, b, ex, f"{cfg.name}/raw/T{T}")


@pytest.mark.parametrize("cfg,T", [(SMALL, 600), (ODD, 300), (C2_Q2B64, 96)], ids=["small_T600", "odd_T300",
                                                                                  "qwen_T96"])
def test_prefill_full_output(torch_cuda, cfg, T):
    from quantized_expert_ffn_softmax_amd import MoEContext
    with MoEContext.from_config(cfg, max_tokens=T, n_layers=1) as ctx:
        W, b, ex = load_layer(ctx, cfg, 7, 0)
        _check_layer(ctx, cfg, 7, 0, 11, T, W, b, ex, f"{cfg.name}/prefill/T{T}")


def test_prefill_raw_codes_cover_every_code_value(torch_cuda):
    """Uniform 2-bit codes and random-sign 64-block scales through the grouped GEMMs."""
    from quantized_expert_ffn_softmax_amd import MoEContext
    for cfg, T in ((SMALL, 300), (ODD, 200)):
        with MoEContext.from_config(cfg, max_tokens=T, n_layers=1) as ctx:
            W, b, ex = load_layer(ctx, cfg, 9, 0, raw=True)
            _check_layer(ctx, cfg, 9, 0, 12, T, W, b, ex, f"{cfg.name}/prefill/raw/T{T}")


def test_short_chain_teacher_forced(torch_cuda):
    """Four Qwen-shaped q2b64 layers with the pre-norm and residual at window 4:
    per layer the routing matches the oracle on the GPU's own normalised input,
    the chain equals the composition of single-layer calls bit for bit, and the
    last layer's output matches the oracle."""
    import torch
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg, L, T = C3_Q2B64, 4, 4
    with MoEContext.from_config(cfg, n_layers=L, max_tokens=8) as ctx:
        inputs = [load_layer(ctx, cfg, 2, layer) for layer in range(L)]
        x0 = mi.gen_x(2, 3, T, cfg.H)
        y, th, tids, tw = ctx.forward(to_dev_bf16(x0), 0, L, residual=True, trace=True, prenorm=True)
        torch.cuda.synchronize()
        thb = bf16_dev_to_bits(th)
        x = x0
        for layer in range(L):
            W, b, ex = inputs[layer]
            ids_ref, w_ref = oracle.select_topk(oracle.router_logits(thb[layer], W, b), cfg.k)
            np.testing.assert_array_equal(tids[layer].cpu().numpy(), ids_ref, err_msg=f"layer {layer}: ids")
            assert np.abs(tw[layer].cpu().numpy().astype(np.float64) - w_ref).max() <= W_TOL
            xn = ctx.forward(to_dev_bf16(x), layer, 1, residual=True, prenorm=True)
            torch.cuda.synchronize()
            x = bf16_dev_to_bits(xn)
        np.testing.assert_array_equal(x, bf16_dev_to_bits(y), err_msg="chain output")
        W, b, ex = inputs[L - 1]
        y_last = ctx.forward(to_dev_bf16(thb[L - 1]), L - 1, 1)
        torch.cuda.synchronize()
        y_ref, _, _, _ = oracle.moe_layer(thb[L - 1], cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex,
                                          cfg.expert_bytes)
        r, mx = assert_y_close(bf16_dev_to_f64(y_last), y_ref, "chain last layer")
        print(f"[q2b64] chain of {L}: routing exact, chain = composition, last layer rel-L2 {r:.2e}", flush=True)


def test_determinism_bitwise(torch_cuda):
    import torch
    from quantized_expert_ffn_softmax_amd import MoEContext
    cfg = SMALL
    with MoEContext.from_config(cfg, max_tokens=300) as ctx:
        load_layer(ctx, cfg, 3, 0)
        load_layer(ctx, cfg, 3, 1)
        for T in (4, 300):
            xd = to_dev_bf16(mi.gen_x(3, 0, T, cfg.H))
            outs = []
            for _ in range(3):
                y = ctx.forward(xd, 0, 2, residual=True)
                torch.cuda.synchronize()
                outs.append(bf16_dev_to_bits(y))
            for o in outs[1:]:
                np.testing.assert_array_equal(o, outs[0], err_msg=f"T={T}")
