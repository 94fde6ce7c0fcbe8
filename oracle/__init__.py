"""fp64 CPU oracle of the sparse-MoE expert-FFN layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never loads it and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C loops in double precision,
OpenMP over tokens and pairs); this module only marshals numpy arrays.
Every function follows the definition written at the top of moe_oracle.c;
parity of each function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py``.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
Q4B32, Q2B32, Q2B64 = 1, 2, 3
_lib = None


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "moe_oracle.c")
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", tmp, src, "-lm"]
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
        i32, i64, vp, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_bf16.restype = f64
        L.oracle_fp16.argtypes = [ctypes.c_uint16]
        L.oracle_fp16.restype = f64
        L.oracle_block_weight.argtypes = [vp, i32, i32]
        L.oracle_block_weight.restype = f64
        L.oracle_dequant_rows.argtypes = [vp, i32, i32, i32, vp]
        L.oracle_dequant_rows.restype = None
        L.oracle_expert_ffn.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.oracle_expert_ffn.restype = None
        L.oracle_router_logits.argtypes = [vp, i32, i32, vp, i32, vp, vp]
        L.oracle_router_logits.restype = None
        L.oracle_select_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_select_topk.restype = None
        L.oracle_route_hash.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_route_hash.restype = None
        L.oracle_permutation.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_permutation.restype = None
        L.oracle_combine.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp]
        L.oracle_combine.restype = None
        L.oracle_moe_layer.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp, vp, vp, vp]
        L.oracle_moe_layer.restype = None
        L.oracle_residual_bf16.argtypes = [ctypes.c_uint16, f64]
        L.oracle_residual_bf16.restype = ctypes.c_uint16
        L.oracle_rmsnorm_bf16.argtypes = [vp, i32, f64, vp]
        L.oracle_rmsnorm_bf16.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def num_threads() -> int:
    """OpenMP threads used by the oracle's parallel loops."""
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's later parallel loops (timing only; results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (a numpy restatement used by tests)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def block_weight(block: np.ndarray, fmt: int, j: int) -> float:
    block = np.ascontiguousarray(block, dtype=np.uint8)
    return float(lib().oracle_block_weight(_p(block), fmt, j))


def fp16_value(bits: int) -> float:
    return float(lib().oracle_fp16(bits))


def dequant_rows(blocks: np.ndarray, rows: int, K: int, fmt: int) -> np.ndarray:
    out = np.empty((rows, K), dtype=np.float64)
    lib().oracle_dequant_rows(_p(np.ascontiguousarray(blocks)), rows, K, fmt, _p(out))
    return out


def expert_matrices(expert: np.ndarray, H: int, F: int, fmt: int):
    """(G [FxH], U [FxH], D [HxF]) dequantised from one expert's canonical bytes."""
    bb = 10 if fmt == Q2B32 else 18
    bw = 64 if fmt == Q2B64 else 32
    ng = F * (H // bw) * bb
    e = np.ascontiguousarray(expert)
    G = dequant_rows(e[:ng], F, H, fmt)
    U = dequant_rows(e[ng:2 * ng], F, H, fmt)
    D = dequant_rows(e[2 * ng:], H, F, fmt)
    return G, U, D


def expert_ffn(expert: np.ndarray, H: int, F: int, fmt: int, x: np.ndarray, want_h: bool = False):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(H, dtype=np.float64)
    h = np.empty(F, dtype=np.float64) if want_h else None
    lib().oracle_expert_ffn(_p(np.ascontiguousarray(expert)), H, F, fmt, _p(x), _p(out), _p(h))
    return (out, h) if want_h else out


def router_logits(x_bits: np.ndarray, W_bits: np.ndarray, bias) -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    T, H = x_bits.shape
    E = W_bits.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float64)
    lib().oracle_router_logits(_p(x_bits), T, H, _p(W_bits), E, _p(b), _p(out))
    return out


def select_topk(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_select_topk(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def route_hash(logits: np.ndarray, table: np.ndarray, tok: np.ndarray):
    """Hash routing: ids[t] = table[tok[t]] (table order), weights = the
    softmax over all E logits renormalised over those ids."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    table = np.ascontiguousarray(table, dtype=np.int32)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    T, E = logits.shape
    k = table.shape[1]
    assert tok.shape == (T,) and tok.min() >= 0 and tok.max() < table.shape[0]
    assert table.min() >= 0 and table.max() < E
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_route_hash(_p(logits), T, E, k, _p(table), _p(tok), _p(ids), _p(w))
    return ids, w


def permutation(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    P = T * k
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(P, dtype=np.int32)
    inv = np.empty(P, dtype=np.int32)
    active = np.empty(E, dtype=np.int32)
    nact = np.zeros(1, dtype=np.int32)
    lib().oracle_permutation(_p(ids), T, k, E, _p(offsets), _p(perm), _p(inv), _p(active), _p(nact))
    return offsets, perm, inv, active[: int(nact[0])].copy()


def combine(x_bits, H, F, E, S, k, fmt, ids, w, experts, expert_bytes):
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    n = x_bits.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    y = np.empty((n, H), dtype=np.float64)
    lib().oracle_combine(_p(x_bits), n, H, F, E, S, k, fmt, _p(ids), _p(w), _p(np.ascontiguousarray(experts)),
                         expert_bytes, _p(y))
    return y


def moe_layer(x_bits, H, F, E, S, k, fmt, W_bits, bias, experts, expert_bytes):
    """Returns (y [T x H] float64, ids [T x k], w [T x k], logits [T x E])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T = x_bits.shape[0]
    y = np.empty((T, H), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lg = np.empty((T, E), dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().oracle_moe_layer(_p(x_bits), T, H, F, E, S, k, fmt, _p(np.ascontiguousarray(W_bits, dtype=np.uint16)),
                           _p(b), _p(np.ascontiguousarray(experts)), expert_bytes, _p(y), _p(ids), _p(w), _p(lg))
    return y, ids, w, lg


def residual_bf16(x_bits: np.ndarray, y: np.ndarray) -> np.ndarray:
    """x_{l+1} = bf16_rne(fp32(x_l) + fp32(y_l)) elementwise."""
    f = lib().oracle_residual_bf16
    xb = np.asarray(x_bits, dtype=np.uint16).ravel()
    yv = np.asarray(y, dtype=np.float64).ravel()
    out = np.array([f(int(a), float(b)) for a, b in zip(xb, yv)], dtype=np.uint16)
    return out.reshape(np.shape(x_bits))


RMSNORM_EPS = 1e-6


def rmsnorm_bf16(x_bits: np.ndarray, eps: float = RMSNORM_EPS) -> np.ndarray:
    """Per-token unit-gain RMS normalisation, rounded once to bf16 (rows of x)."""
    x = np.ascontiguousarray(np.atleast_2d(x_bits), dtype=np.uint16)
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        lib().oracle_rmsnorm_bf16(_p(x[t]), x.shape[1], eps, _p(out[t]))
    return out.reshape(np.shape(x_bits))

