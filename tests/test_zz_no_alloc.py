"""moe_route_static (routing with the library's static device scratch, no
context, no allocation) against moe_route on a context holding the same
router, through the C ABI: two calls in a row, the second with a smaller
input (fewer tokens, then a smaller router), each bit-exact on ids, offsets
and perm and equal on the weights, and equal to the oracle's routing."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from moe_inputs.configs import C1, C2, MoEConfig, Q4B32

from parity import W_TOL, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _route_both(torch, cfg, W, b, x):
    import quantized_expert_ffn_softmax_amd as moe
    T = x.shape[0]
    xd = to_dev_bf16(x)
    with moe.MoEContext.from_config(cfg, max_tokens=8, n_layers=1) as ctx:
        ctx.load(0, router_w=W, router_bias=b)
        ids_c, w_c, off_c, perm_c = ctx.route(0, xd)
        torch.cuda.synchronize()
    Wd = torch.from_numpy(W.view(np.int16)).cuda()
    bd = torch.from_numpy(b).cuda()
    ids = torch.full((T, cfg.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, cfg.k), -7.0, dtype=torch.float32, device="cuda")
    off = torch.full((cfg.E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * cfg.k,), -7, dtype=torch.int32, device="cuda")
    moe.moe_route_static(xd, T, cfg.H, cfg.E, cfg.k, Wd, bd, ids, w, off, perm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_c.cpu().numpy(), err_msg=f"{cfg.name} T={T}: ids")
    np.testing.assert_array_equal(w.cpu().numpy(), w_c.cpu().numpy(), err_msg=f"{cfg.name} T={T}: weights")
    np.testing.assert_array_equal(off.cpu().numpy(), off_c.cpu().numpy(), err_msg=f"{cfg.name} T={T}: offsets")
    np.testing.assert_array_equal(perm.cpu().numpy(), perm_c.cpu().numpy(), err_msg=f"{cfg.name} T={T}: perm")
    ids_ref, w_ref = oracle.select_topk(oracle.router_logits(x, W, b), cfg.k)
    off_ref, perm_ref, _, _ = oracle.permutation(ids_ref, cfg.E)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_array_equal(off.cpu().numpy(), off_ref)
    np.testing.assert_array_equal(perm.cpu().numpy(), perm_ref)
    assert np.abs(w.cpu().numpy().astype(np.float64) - w_ref).max() <= W_TOL
    print(f"[static route] {cfg.name} T={T}: equal to moe_route and to the oracle", flush=True)


def test_static_route_matches_context_route(torch_cuda):
    torch = torch_cuda
    big = C2
    W = mi.gen_router(3, 0, big.E, big.H)
    b = mi.gen_bias(3, 0, big.E, big.bias_kind, big.bias_param)
    _route_both(torch, big, W, b, mi.gen_x(3, 0, 8, big.H))
    _route_both(torch, big, W, b, mi.gen_x(3, 1, 3, big.H))
    small = C1
    W1 = mi.gen_router(4, 0, small.E, small.H)
    b1 = mi.gen_bias(4, 0, small.E, mi.BIAS_NORMAL, 0.5)
    _route_both(torch, small, W1, b1, mi.gen_x(4, 0, 4, small.H))
    wide = MoEConfig("wide", (8,), 4096, 64, 1024, 0, 16, 1, Q4B32, mi.BIAS_ZIPF, 1.1)
    W2 = mi.gen_router(5, 0, wide.E, wide.H)
    b2 = mi.gen_bias(5, 0, wide.E, wide.bias_kind, wide.bias_param)
    _route_both(torch, wide, W2, b2, mi.gen_x(5, 0, 8, wide.H))
    _route_both(torch, small, W1, b1, mi.gen_x(4, 1, 2, small.H))
