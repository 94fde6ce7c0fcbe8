"""moe_forward captured into a HIP graph (torch.cuda.CUDAGraph on a
default-priority side stream): every replay must equal the eager result bit
for bit, with the program's own eager work and synchronisations between the
replays.  The forward path records no memset and allocates nothing, so the
captured work is exactly the eager work."""
import numpy as np
import pytest

import moe_inputs as mi
from moe_inputs.configs import MoEConfig, Q2B32, Q4B32

from parity import bf16_dev_to_bits, load_layer, to_dev_bf16

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
        for layer in range(cfg.L):
            load_layer(ctx, cfg, 21, layer)
        x = to_dev_bf16(mi.gen_x(21, 0, T, cfg.H))
        y = torch.empty_like(x)
        ctx.forward(x, 0, layers, residual=residual, prenorm=prenorm, y=y)
        torch.cuda.synchronize()
        eager = bf16_dev_to_bits(y)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            g.capture_begin()
            ctx.forward(x, 0, layers, residual=residual, prenorm=prenorm, y=y)
            g.capture_end()
        torch.cuda.current_stream().wait_stream(side)
        for rep in range(4):
            y.zero_()
            # eager work of the program between replays
            other = ctx.forward(to_dev_bf16(mi.gen_x(21, 1 + rep, T, cfg.H)), 0, layers, residual=residual,
                                prenorm=prenorm)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(bf16_dev_to_bits(y), eager, err_msg=f"replay {rep}")
            assert not np.array_equal(bf16_dev_to_bits(other), eager)
