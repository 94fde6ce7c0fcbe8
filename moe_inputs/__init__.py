"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Only input generation lives here (see gen.c for the generator definition and
the canonical expert byte format).  Nothing in this package computes any part
of the MoE layer.
"""
import ctypes
import os

import numpy as np

from .configs import (BIAS_NONE, BIAS_NORMAL, BIAS_ZIPF, CONFIGS, Q2B32, Q2B64, Q4B32,  # noqa: F401
                      MoEConfig)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_inputs.so")

TAG_X = 1
TAG_ROUTER = 2
TAG_BIAS = 3
TAG_PERM = 4
TAG_EXPERT = 5
TAG_RAW = 6

_lib = None


def build(verbose: bool = False) -> str:
    """Compile gen.c into libmoe_inputs.so (gcc, OpenMP)."""
    import subprocess
    src = os.path.join(_HERE, "gen.c")
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-mavx2", "-fno-math-errno", "-fno-trapping-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, i32, i64, f64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        L.moe_gen_block_bytes.argtypes = [i32]
        L.moe_gen_block_bytes.restype = i64
        L.moe_gen_block_weights.argtypes = [i32]
        L.moe_gen_block_weights.restype = i32
        L.moe_gen_expert_bytes.argtypes = [i32, i32, i32]
        L.moe_gen_expert_bytes.restype = i64
        L.moe_gen_quantize_block.argtypes = [vp, i32, vp]
        L.moe_gen_normals.argtypes = [u64, u32, u32, u32, u64, u64, vp]
        L.moe_gen_bf16_normal.argtypes = [u64, u32, u32, u32, f64, u64, vp]
        L.moe_gen_x.argtypes = [u64, u32, i32, i32, vp]
        L.moe_gen_router.argtypes = [u64, u32, i32, i32, vp]
        L.moe_gen_bias.argtypes = [u64, u32, i32, i32, f64, vp]
        L.moe_gen_experts.argtypes = [u64, u32, i32, i32, i32, i32, i32, i32, vp]
        for f in ("moe_gen_quantize_block", "moe_gen_normals", "moe_gen_bf16_normal", "moe_gen_x",
                  "moe_gen_router", "moe_gen_bias", "moe_gen_experts"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def expert_bytes(H: int, F: int, fmt: int) -> int:
    return int(lib().moe_gen_expert_bytes(H, F, fmt))


def block_bytes(fmt: int) -> int:
    return int(lib().moe_gen_block_bytes(fmt))


def block_weights(fmt: int) -> int:
    return int(lib().moe_gen_block_weights(fmt))


def normals(seed: int, tag: int, a: int, b: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().moe_gen_normals(seed, tag, a, b, start, n, _ptr(out))
    return out


def quantize_block(w: np.ndarray, fmt: int) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float64)
    assert w.shape == (block_weights(fmt),)
    out = np.zeros(block_bytes(fmt), dtype=np.uint8)
    lib().moe_gen_quantize_block(_ptr(w), fmt, _ptr(out))
    return out


def gen_x(seed: int, window: int, T: int, H: int, out: np.ndarray = None) -> np.ndarray:
    """Activations [T x H] as bf16 bit patterns (uint16)."""
    if out is None:
        out = np.empty((T, H), dtype=np.uint16)
    lib().moe_gen_x(seed, window, T, H, _ptr(out))
    return out


def gen_router(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    """Router weights [E x H] as bf16 bit patterns (uint16)."""
    out = np.empty((E, H), dtype=np.uint16)
    lib().moe_gen_router(seed, layer, E, H, _ptr(out))
    return out


def gen_bias(seed: int, layer: int, E: int, kind: int, param: float) -> np.ndarray:
    out = np.zeros(E, dtype=np.float32)
    lib().moe_gen_bias(seed, layer, E, kind, float(param), _ptr(out))
    return out


def gen_experts(seed: int, layer: int, e_begin: int, count: int, H: int, F: int, fmt: int,
                raw: bool = False, out: np.ndarray = None) -> np.ndarray:
    """Canonical bytes of `count` experts starting at expert index e_begin.

    Expert index E (one past the routed experts) is the shared expert."""
    nb = expert_bytes(H, F, fmt)
    if nb < 0:
        raise ValueError("H and F must be positive multiples of 32")
    if out is None:
        out = np.empty(count * nb, dtype=np.uint8)
    assert out.nbytes >= count * nb and out.dtype == np.uint8
    lib().moe_gen_experts(seed, layer, e_begin, count, H, F, fmt, 1 if raw else 0, _ptr(out))
    return out


def gen_tid2eid(seed: int, layer: int, vocab: int, E: int, k: int) -> np.ndarray:
    """Hash-routing table [vocab x k] int32: every row k distinct expert ids in
    [0, E), a seeded uniform choice in a seeded order."""
    rng = np.random.default_rng([seed, layer, 0x7A1D])
    return np.argsort(rng.random((vocab, E)), axis=1)[:, :k].astype(np.int32)


def gen_token_ids(seed: int, window: int, T: int, vocab: int) -> np.ndarray:
    """Token ids [T] int32, uniform in [0, vocab)."""
    rng = np.random.default_rng([seed, window, 0x70C])
    return rng.integers(0, vocab, T).astype(np.int32)


def layer_inputs(cfg: MoEConfig, seed: int, layer: int, raw: bool = False):
    """Router weights, bias and every expert (routed then shared) of one layer."""
    W = gen_router(seed, layer, cfg.E, cfg.H)
    b = gen_bias(seed, layer, cfg.E, cfg.bias_kind, cfg.bias_param)
    ex = gen_experts(seed, layer, 0, cfg.E + cfg.S, cfg.H, cfg.F, cfg.fmt, raw)
    return W, b, ex
