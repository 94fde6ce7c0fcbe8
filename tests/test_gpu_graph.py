"""moe_forward captured into a HIP graph (torch.cuda.CUDAGraph on a
default-priority side stream): every replay must equal the eager result bit
for bit, with the program's own eager work and synchronisations between the
replays, and the replayed output must match the fp64 oracle (single layers:
within the rel-L2 / max-abs bar over the whole output; the two-layer chain:
its last layer teacher-forced on the captured call's own traced MoE input,
plus the residual stream).  The forward path records no memset and allocates
nothing, so the captured work is exactly the eager work."""
import numpy as np
import pytest

import moe_inputs as mi
from moe_inputs.configs import MoEConfig, Q2B32, Q4B32

import oracle
from parity import W_TOL, assert_y_close, bf16_dev_to_bits, bf16_dev_to_f64, load_layer, to_dev_bf16

pytestmark = pytest.mark.gpu

DEC = MoEConfig("graph_dec", (4,), 512, 256, 24, 1, 4, 2, Q4B32, mi.BIAS_NORMAL, 0.5)
PF = MoEConfig("graph_pf", (300,), 640, 160, 40, 0, 6, 1, Q2B32, mi.BIAS_ZIPF, 1.1)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("cfg,T,layers,flags", [(DEC, 4, 2, (True, True)), (DEC, 8, 1, (False, False)),
                                                (PF, 300, 1, (False, False))],
                         ids=["decode_chain_T4", "decode_T8", "prefill_T300"])
def test_graph_replay_equals_eager(torch_cuda, cfg, T, layers, flags):
    torch = torch_cuda
    from quantized_expert_ffn_softmax_amd import MoEContext
    residual, prenorm = flags
    with MoEContext.from_config(cfg, max_tokens=max(T, 8)) as ctx:
        inputs = [load_layer(ctx, cfg, 21, layer) for layer in range(cfg.L)]
        xh = mi.gen_x(21, 0, T, cfg.H)
        x = to_dev_bf16(xh)
        y = torch.empty_like(x)
        tx = torch.empty((layers, T, cfg.H), dtype=x.dtype, device=x.device)
        tids = torch.empty((layers, T, cfg.k), dtype=torch.int32, device=x.device)
        tw = torch.empty((layers, T, cfg.k), dtype=torch.float32, device=x.device)
        from quantized_expert_ffn_softmax_amd import MOE_FWD_PRENORM, MOE_FWD_RESIDUAL, moe_forward
        flags_i = (MOE_FWD_RESIDUAL if residual else 0) | (MOE_FWD_PRENORM if prenorm else 0)

        def fwd():
            moe_forward(ctx.handle, x, y, T, 0, layers, flags_i, tx, tids, tw)

        fwd()
        torch.cuda.synchronize()
        eager = bf16_dev_to_bits(y)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            g.capture_begin()
            fwd()
            g.capture_end()
        torch.cuda.current_stream().wait_stream(side)
        for rep in range(4):
            y.zero_()
            tx.zero_()
            # eager work of the program between replays
            other = ctx.forward(to_dev_bf16(mi.gen_x(21, 1 + rep, T, cfg.H)), 0, layers, residual=residual,
                                prenorm=prenorm)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(bf16_dev_to_bits(y), eager, err_msg=f"replay {rep}")
            assert not np.array_equal(bf16_dev_to_bits(other), eager)
        # the replayed result against the oracle, the last layer on its traced MoE input
        last = layers - 1
        h_last = bf16_dev_to_bits(tx)[last]
        W, b, ex = inputs[last]
        y_ref, ids_ref, w_ref, _ = oracle.moe_layer(h_last, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex,
                                                    cfg.expert_bytes)
        np.testing.assert_array_equal(tids[last].cpu().numpy(), ids_ref)
        assert np.abs(tw[last].cpu().numpy().astype(np.float64) - w_ref).max() <= W_TOL
        if layers == 1 and not residual:
            r, mx = assert_y_close(bf16_dev_to_f64(y), y_ref, "graph replay")
        else:
            # the stream entering the last layer, from an eager single-layer call (a chain equals the
            # composition of single-layer calls), plus the oracle's layer output
            x_prev = ctx.forward(x, 0, 1, residual=residual, prenorm=prenorm)
            torch.cuda.synchronize()
            if prenorm:
                # the captured last layer's MoE input is the pre-norm of that stream (within one bf16 ulp)
                hn = oracle.bf16_to_f64(oracle.rmsnorm_bf16(bf16_dev_to_bits(x_prev)))
                assert (np.abs(oracle.bf16_to_f64(h_last) - hn) <= np.abs(hn) * 2.0 ** -7).all()
            r, mx = assert_y_close(bf16_dev_to_f64(y), oracle.bf16_to_f64(bf16_dev_to_bits(x_prev)) + y_ref,
                                   "graph replay, chain output")
        print(f"[graph] {cfg.name} T={T} layers={layers}: replays equal eager; vs oracle rel-L2 {r:.2e} "
              f"max-abs {mx:.2e}", flush=True)


def test_library_chain_graph_replays(torch_cuda):
    """A decode chain (layer_count > 1) replays the library's own HIP graph,
    captured on the first call with a given set of buffers.  Calls that reuse
    the buffers with new contents, interleaved with eager work and a weight
    upload (which drops the cached graphs), equal the eager path (a profiled
    call runs eagerly) bit for bit, and the last layer matches the oracle on
    its traced input."""
    torch = torch_cuda
    from quantized_expert_ffn_softmax_amd import (MOE_FWD_PRENORM, MOE_FWD_PROFILE, MOE_FWD_RESIDUAL, MoEContext,
                                                  moe_forward)
    cfg = DEC
    T, layers = 4, 2
    with MoEContext.from_config(cfg, max_tokens=8) as ctx:
        inputs = [load_layer(ctx, cfg, 23, layer) for layer in range(cfg.L)]
        x = torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda")
        y = torch.empty_like(x)
        tx = torch.empty((layers, T, cfg.H), dtype=x.dtype, device=x.device)
        tids = torch.empty((layers, T, cfg.k), dtype=torch.int32, device=x.device)
        tw = torch.empty((layers, T, cfg.k), dtype=torch.float32, device=x.device)
        flags = MOE_FWD_RESIDUAL | MOE_FWD_PRENORM
        for rep in range(5):
            x.copy_(to_dev_bf16(mi.gen_x(23, rep, T, cfg.H)))
            if rep == 3:  # an upload drops the cached graphs; the next call captures again
                ctx.load(0, router_w=inputs[0][0], router_bias=inputs[0][1])
            moe_forward(ctx.handle, x, y, T, 0, layers, flags, tx, tids, tw)
            torch.cuda.synchronize()
            got = bf16_dev_to_bits(y)
            moe_forward(ctx.handle, x, y, T, 0, layers, flags | MOE_FWD_PROFILE, tx, tids, tw)
            torch.cuda.synchronize()
            ctx.profile_read()
            np.testing.assert_array_equal(got, bf16_dev_to_bits(y), err_msg=f"call {rep}: graph vs eager")
        h_last = bf16_dev_to_bits(tx)[layers - 1]
        W, b, ex = inputs[layers - 1]
        _, ids_ref, w_ref, _ = oracle.moe_layer(h_last, cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, cfg.fmt, W, b, ex,
                                                cfg.expert_bytes)
        np.testing.assert_array_equal(tids[layers - 1].cpu().numpy(), ids_ref)
        assert np.abs(tw[layers - 1].cpu().numpy().astype(np.float64) - w_ref).max() <= W_TOL
        print("[graph] library chain graph: 5 calls equal eager, routing of the last layer equals the oracle's",
              flush=True)
