"""Shared helpers of the parity tests: seeded inputs -> GPU and oracle, and the
comparison bar.

Bar (for every output of one call):
  * expert ids, offsets and permutation bit-exact;
  * routing weights |w_gpu - w_ref| <= 1e-6;
  * y: rel-L2 = ||y - y_ref||_2 / ||y_ref||_2 <= 5e-3 over the whole [T x H]
    output, and max |y - y_ref| <= 2e-2 * max |y_ref|.
"""
import numpy as np

import moe_inputs as mi

REL_L2_TOL = 5e-3
MAX_ABS_FRAC = 2e-2
W_TOL = 1e-6


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16).view(np.float32).astype(
        np.float64)


def bf16_dev_to_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16).copy()


def rel_l2(y, ref):
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_y_close(y, ref, what=""):
    r = rel_l2(y, ref)
    mx = float(np.abs(y - ref).max())
    lim = MAX_ABS_FRAC * float(np.abs(ref).max())
    assert r <= REL_L2_TOL, f"{what} rel-L2 {r:.3e} > {REL_L2_TOL}"
    assert mx <= lim, f"{what} max-abs {mx:.3e} > {lim:.3e}"
    return r, mx


def min_routing_gap(logits: np.ndarray, k: int) -> float:
    """Smallest gap among the k+1 largest logits of any token (how close the
    routing is to a tie)."""
    s = -np.sort(-logits, axis=1)[:, : k + 1]
    return float(np.min(s[:, :-1] - s[:, 1:]))


def load_layer(ctx, cfg, seed, layer, raw=False, staging_experts=None):
    W, b, ex = mi.layer_inputs(cfg, seed, layer, raw=raw)
    ctx.load(layer, router_w=W, router_bias=b, experts=ex)
    return W, b, ex


def oracle_layer_selected(x_bits, cfg, seed, layer, W, b, raw=False):
    """The oracle's layer output on x_bits with only the experts it selects
    (and the shared expert) generated: the same seeded bytes as the full
    layer, since every expert's bytes are keyed by (seed, layer, expert).
    Returns (y [T x H] float64, ids [T x k], w [T x k])."""
    import oracle
    ids, w = oracle.select_topk(oracle.router_logits(x_bits, W, b), cfg.k)
    uniq = np.unique(ids)
    remap = np.full(cfg.E, -1, dtype=np.int32)
    remap[uniq] = np.arange(len(uniq), dtype=np.int32)
    eb = cfg.expert_bytes
    ex = np.empty((len(uniq) + cfg.S) * eb, dtype=np.uint8)
    for i, e in enumerate(uniq):
        mi.gen_experts(seed, layer, int(e), 1, cfg.H, cfg.F, cfg.fmt, raw=raw, out=ex[i * eb:(i + 1) * eb])
    if cfg.S:
        mi.gen_experts(seed, layer, cfg.E, 1, cfg.H, cfg.F, cfg.fmt, raw=raw, out=ex[len(uniq) * eb:])
    y = oracle.combine(x_bits, cfg.H, cfg.F, len(uniq), cfg.S, cfg.k, cfg.fmt, remap[ids], w, ex, eb)
    return y, ids, w
