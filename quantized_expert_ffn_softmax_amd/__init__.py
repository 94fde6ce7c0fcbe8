"""Python binding of libmoe, the MI355X sparse mixture-of-experts layer.

Thin argument marshalling over the C ABI declared in include/moe.h: every step
of the layer runs in the HIP kernels of libmoe.so.  PyTorch is used only for
device memory and streams.  There is no fallback: if libmoe.so is missing the
import of the library raises.

Module-level functions carry the C names (moe_create, moe_load_experts,
moe_route, moe_forward, moe_destroy); ``MoEContext`` wraps them for
convenience.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_ESTATE, MOE_ERANGE = 0, -1, -2, -3, -4, -5
MOE_Q4B32, MOE_Q2B32, MOE_Q2B64 = 1, 2, 3
MOE_FWD_RESIDUAL = 1
MOE_FWD_PROFILE = 2
MOE_FWD_PRENORM = 4
KERNEL_NAMES = {0: "router", 1: "topk_sort", 2: "gateup", 3: "down", 4: "combine", 5: "pf_router", 6: "pf_topk",
                7: "pf_sort", 8: "pf_gemm1", 9: "pf_gemm2", 10: "pf_combine", 11: "norm"}
MOE_ABI_VERSION = 2
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ENOMEM", -3: "MOE_EHIP", -4: "MOE_ESTATE", -5: "MOE_ERANGE"}

# Every symbol include/moe.h declares.
EXPORTED = ("moe_create", "moe_load_experts", "moe_route", "moe_forward", "moe_destroy", "moe_last_error",
            "moe_expert_bytes", "moe_memory_bytes", "moe_profile_read", "moe_route_static")


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("abi_version", "hidden", "ffn", "n_experts", "n_shared", "top_k",
                                                "n_layers", "quant", "max_tokens", "device")]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("expert_begin", ctypes.c_int32), ("expert_count", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("experts", ctypes.c_void_p),
                ("experts_bytes", ctypes.c_size_t), ("tid2eid", ctypes.c_void_p), ("vocab", ctypes.c_int32)]


class moe_fwd_args(ctypes.Structure):
    _fields_ = [("layer_begin", ctypes.c_int32), ("layer_count", ctypes.c_int32), ("T", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("trace_x", ctypes.c_void_p), ("trace_ids", ctypes.c_void_p), ("trace_w", ctypes.c_void_p),
                ("token_ids", ctypes.c_void_p)]


class moe_kernel_time(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("layer", ctypes.c_int32), ("ms", ctypes.c_float)]


class MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_expert_ffn_softmax_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.moe_create.argtypes = [ctypes.POINTER(moe_config), ctypes.POINTER(vp)]
        L.moe_load_experts.argtypes = [vp, ctypes.POINTER(moe_layer_weights)]
        L.moe_route.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, vp, vp]
        L.moe_forward.argtypes = [vp, ctypes.POINTER(moe_fwd_args), vp]
        L.moe_destroy.argtypes = [vp]
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_expert_bytes.argtypes = [i32, i32, i32]
        L.moe_expert_bytes.restype = ctypes.c_int64
        L.moe_memory_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]
        L.moe_profile_read.argtypes = [vp, ctypes.POINTER(moe_kernel_time), i32, ctypes.POINTER(i32)]
        L.moe_route_static.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        for f in ("moe_create", "moe_load_experts", "moe_route", "moe_forward", "moe_destroy", "moe_memory_bytes",
                  "moe_profile_read", "moe_route_static"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error().decode(errors="replace"))


def _dptr(t, itemsize=None, name="tensor"):
    """Device address of a contiguous GPU tensor (or None).  The library reads
    and writes these addresses from its kernels, so a host tensor, or elements
    of another width than the call's layout (2 bytes: bf16 activations and
    router weights; 4 bytes: int32 ids and fp32 weights), is rejected here."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if itemsize is not None and t.element_size() != itemsize:
        raise ValueError(f"{name} must have {itemsize}-byte elements, got {t.element_size()}")
    return t.data_ptr()


def _hptr(a):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("host arrays passed to libmoe must be C-contiguous")
    return a.ctypes.data


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------------ C names
def moe_expert_bytes(hidden, ffn, quant):
    return int(lib().moe_expert_bytes(hidden, ffn, quant))


def moe_create(hidden, ffn, n_experts, n_shared, top_k, n_layers, quant, max_tokens, device=0):
    cfg = moe_config(MOE_ABI_VERSION, hidden, ffn, n_experts, n_shared, top_k, n_layers, quant, max_tokens, device)
    h = ctypes.c_void_p()
    _check(lib().moe_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def moe_load_experts(ctx, layer, router_w=None, router_bias=None, experts=None, expert_begin=0, expert_count=0,
                     tid2eid=None):
    if tid2eid is not None and (tid2eid.dtype != np.int32 or tid2eid.ndim != 2):
        raise ValueError("tid2eid must be a [vocab x k] int32 array")
    w = moe_layer_weights(layer, expert_begin, expert_count, _hptr(router_w), _hptr(router_bias), _hptr(experts),
                          0 if experts is None else experts.nbytes, _hptr(tid2eid),
                          0 if tid2eid is None else tid2eid.shape[0])
    _check(lib().moe_load_experts(ctx, ctypes.byref(w)))


def moe_route(ctx, layer, x, T, ids, w, offsets=None, perm=None, stream=None, token_ids=None):
    _check(lib().moe_route(ctx, layer, _dptr(x, 2, "x"), T, _dptr(token_ids, 4, "token_ids"), _dptr(ids, 4, "ids"),
                           _dptr(w, 4, "w"), _dptr(offsets, 4, "offsets"), _dptr(perm, 4, "perm"), _stream(stream)))


def moe_route_static(x, T, hidden, n_experts, top_k, router_w, router_bias, ids, w, offsets=None, perm=None,
                     stream=None):
    """Decode-window routing on device router weights with the library's static scratch (no context, no
    allocation)."""
    _check(lib().moe_route_static(_dptr(x, 2, "x"), T, hidden, n_experts, top_k, _dptr(router_w, 2, "router_w"),
                                  _dptr(router_bias, 4, "router_bias"), _dptr(ids, 4, "ids"), _dptr(w, 4, "w"),
                                  _dptr(offsets, 4, "offsets"), _dptr(perm, 4, "perm"), _stream(stream)))


def moe_forward(ctx, x, y, T, layer_begin=0, layer_count=1, flags=0, trace_x=None, trace_ids=None, trace_w=None,
                stream=None, token_ids=None):
    a = moe_fwd_args(layer_begin, layer_count, T, flags, _dptr(x, 2, "x"), _dptr(y, 2, "y"),
                     _dptr(trace_x, 2, "trace_x"), _dptr(trace_ids, 4, "trace_ids"), _dptr(trace_w, 4, "trace_w"),
                     _dptr(token_ids, 4, "token_ids"))
    _check(lib().moe_forward(ctx, ctypes.byref(a), _stream(stream)))


def moe_destroy(ctx):
    _check(lib().moe_destroy(ctx))


def moe_memory_bytes(ctx):
    a, s = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().moe_memory_bytes(ctx, ctypes.byref(a), ctypes.byref(s)))
    return a.value, s.value


def moe_profile_read(ctx, cap=65536):
    """[(kernel_name, layer, ms), ...] of the profiled launches since the last read."""
    buf = (moe_kernel_time * cap)()
    n = ctypes.c_int32()
    _check(lib().moe_profile_read(ctx, buf, cap, ctypes.byref(n)))
    return [(KERNEL_NAMES.get(buf[i].kernel, buf[i].kernel), buf[i].layer, buf[i].ms) for i in range(n.value)]


# --------------------------------------------------------------- convenience
class MoEContext:
    """Owns one moe_ctx; tensors are torch CUDA tensors, weights numpy arrays."""

    def __init__(self, hidden, ffn, n_experts, n_shared, top_k, n_layers, quant, max_tokens, device=0):
        self.H, self.F, self.E, self.S, self.k, self.L = hidden, ffn, n_experts, n_shared, top_k, n_layers
        self.quant, self.max_tokens, self.device = quant, max_tokens, device
        self.handle = moe_create(hidden, ffn, n_experts, n_shared, top_k, n_layers, quant, max_tokens, device)

    @classmethod
    def from_config(cls, cfg, max_tokens=None, n_layers=None, device=0):
        return cls(cfg.H, cfg.F, cfg.E, cfg.S, cfg.k, n_layers or cfg.L, cfg.fmt, max_tokens or max(cfg.T), device)

    @property
    def expert_bytes(self):
        return moe_expert_bytes(self.H, self.F, self.quant)

    def load(self, layer, router_w=None, router_bias=None, experts=None, expert_begin=0, tid2eid=None):
        """tid2eid: None, or a [vocab x k] int32 table that makes the layer hash-routed."""
        count = 0 if experts is None else experts.nbytes // self.expert_bytes
        moe_load_experts(self.handle, layer, router_w, router_bias, experts, expert_begin, count, tid2eid)

    def _rows(self, x, token_ids=None, y=None):
        """T of an activation tensor [T, H]; y and token_ids must match it."""
        if x.dim() != 2 or x.shape[1] != self.H:
            raise ValueError(f"x must be [T, {self.H}], got {tuple(x.shape)}")
        T = x.shape[0]
        if y is not None and tuple(y.shape) != tuple(x.shape):
            raise ValueError(f"y must be {tuple(x.shape)}, got {tuple(y.shape)}")
        if token_ids is not None and token_ids.numel() < T:
            raise ValueError(f"token_ids holds {token_ids.numel()} ids for {T} tokens")
        return T

    def route(self, layer, x, stream=None, token_ids=None):
        import torch
        T = self._rows(x, token_ids)
        dev = x.device
        ids = torch.empty((T, self.k), dtype=torch.int32, device=dev)
        w = torch.empty((T, self.k), dtype=torch.float32, device=dev)
        offsets = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(T * self.k, dtype=torch.int32, device=dev)
        moe_route(self.handle, layer, x, T, ids, w, offsets, perm, stream, token_ids)
        return ids, w, offsets, perm

    def forward(self, x, layer_begin=0, layer_count=1, residual=False, trace=False, y=None, stream=None,
                profile=False, prenorm=False, token_ids=None):
        import torch
        T = self._rows(x, token_ids, y)
        if y is None:
            y = torch.empty_like(x)
        tx = tid = tw = None
        if trace:
            tx = torch.empty((layer_count, T, self.H), dtype=x.dtype, device=x.device)
            tid = torch.empty((layer_count, T, self.k), dtype=torch.int32, device=x.device)
            tw = torch.empty((layer_count, T, self.k), dtype=torch.float32, device=x.device)
        flags = ((MOE_FWD_RESIDUAL if residual else 0) | (MOE_FWD_PROFILE if profile else 0) |
                 (MOE_FWD_PRENORM if prenorm else 0))
        moe_forward(self.handle, x, y, T, layer_begin, layer_count, flags, tx, tid, tw, stream, token_ids)
        return (y, tx, tid, tw) if trace else y

    def profile_read(self):
        return moe_profile_read(self.handle)

    def memory_bytes(self):
        return moe_memory_bytes(self.handle)

    def close(self):
        if self.handle is not None:
            moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
