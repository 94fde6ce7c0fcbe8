"""The C-ABI library loads and exports every symbol include/moe.h declares (CPU only)."""
import ctypes
import os
import re

import pytest

import quantized_expert_ffn_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\S.*?\b(moe_[a-z_]+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary_calls():
    names = _declared_symbols()
    for f in ("moe_create", "moe_load_experts", "moe_route", "moe_forward", "moe_destroy", "moe_last_error"):
        assert f in names
    assert set(names) == set(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_host_only_calls_without_gpu():
    """Calls that touch no kernel: byte accounting, argument checks, NULL handling."""
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    assert moe.moe_expert_bytes(4096, 2048, moe.MOE_Q4B32) == 14_155_776
    assert moe.moe_expert_bytes(2560, 640, moe.MOE_Q2B32) == 1_536_000
    assert moe.moe_expert_bytes(100, 64, moe.MOE_Q4B32) == -1
    # q2b64: 2.25 bits per weight, hidden and ffn multiples of 64
    assert moe.moe_expert_bytes(2560, 640, moe.MOE_Q2B64) == 1_382_400
    assert moe.moe_expert_bytes(2560, 96, moe.MOE_Q2B64) == -1
    assert moe.moe_expert_bytes(128, 64, 4) == -1
    lib = moe.lib()
    assert lib.moe_destroy(None) == moe.MOE_OK
    assert lib.moe_forward(None, None, None) == moe.MOE_EINVAL
    assert lib.moe_route(None, 0, None, 1, None, None, None, None, None, None) == moe.MOE_EINVAL
    assert lib.moe_load_experts(None, None) == moe.MOE_EINVAL
    assert b"NULL" in lib.moe_last_error()
    # a bad geometry is rejected before any device is touched
    cfg = moe.moe_config(moe.MOE_ABI_VERSION, 100, 64, 8, 0, 2, 1, moe.MOE_Q4B32, 4, 0)
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(cfg), ctypes.byref(h)) == moe.MOE_EINVAL
    assert h.value is None
    cfg = moe.moe_config(99, 128, 64, 8, 0, 2, 1, moe.MOE_Q4B32, 4, 0)
    assert lib.moe_create(ctypes.byref(cfg), ctypes.byref(h)) == moe.MOE_EINVAL


def test_binding_struct_layouts_match_the_header(tmp_path):
    """The ctypes structures of the binding have the sizes and field offsets a C
    compiler gives the structures of include/moe.h."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "layout.c"
    fields = {"moe_config": ["abi_version", "max_tokens", "device"],
              "moe_layer_weights": ["layer", "router_w", "router_bias", "experts", "experts_bytes", "tid2eid", "vocab"],
              "moe_fwd_args": ["layer_begin", "flags", "x", "y", "trace_x", "trace_ids", "trace_w", "token_ids"],
              "moe_kernel_time": ["kernel", "layer", "ms"]}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "moe.h"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'    printf("{st} %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'    printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines += ["    return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(root, "include"), "-o", str(exe), str(src)], check=True)
    got = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines())
    for st, fs in fields.items():
        cls = getattr(moe, st)
        assert int(got[st]) == ctypes.sizeof(cls), st
        for f in fs:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, f"{st}.{f}"


def test_bench_refuses_more_than_one_gpu():
    """bench.py --gpus 2 exits with a message before touching a GPU."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_static_route_argument_checks():
    """moe_route_static validates before touching any device: window, geometry and top-k limits."""
    import quantized_expert_ffn_softmax_amd as moe
    lib = moe.lib()
    f = lib.moe_route_static
    assert f(None, 9, 256, 16, 2, None, None, None, None, None, None, None) == moe.MOE_ERANGE
    assert f(None, -1, 256, 16, 2, None, None, None, None, None, None, None) == moe.MOE_ERANGE
    assert f(None, 4, 100, 16, 2, None, None, None, None, None, None, None) == moe.MOE_EINVAL
    assert f(None, 4, 8192, 16, 2, None, None, None, None, None, None, None) == moe.MOE_EINVAL
    assert f(None, 4, 256, 0, 1, None, None, None, None, None, None, None) == moe.MOE_EINVAL
    assert f(None, 4, 256, 2000, 2, None, None, None, None, None, None, None) == moe.MOE_EINVAL
    assert f(None, 4, 256, 16, 17, None, None, None, None, None, None, None) == moe.MOE_EINVAL
    assert f(None, 4, 256, 8, 9, None, None, None, None, None, None, None) == moe.MOE_EINVAL
    assert f(None, 4, 256, 16, 2, None, None, None, None, None, None, None) == moe.MOE_EINVAL  # NULL pointers
    assert b"required" in lib.moe_last_error()
    assert f(None, 0, 4096, 1024, 16, None, None, None, None, None, None, None) == moe.MOE_OK  # T = 0: no-op


def test_binding_rejects_tensors_the_kernels_cannot_read():
    """Host tensors, non-contiguous views and elements of the wrong width are
    refused before any call reaches the library; activations must be [T, H]."""
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_forward(None, x, x, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_route(None, 0, x, 4, None, None)

    class Dev:  # stands for a device tensor: the checks read only these attributes
        is_cuda = True

        def __init__(self, size, contiguous=True):
            self.size, self.contiguous = size, contiguous

        def is_contiguous(self):
            return self.contiguous

        def element_size(self):
            return self.size

        def data_ptr(self):
            return 0x1000

    assert moe._dptr(None, 2, "x") is None
    assert moe._dptr(Dev(2), 2, "x") == 0x1000
    with pytest.raises(ValueError, match="2-byte"):
        moe._dptr(Dev(4), 2, "x")
    with pytest.raises(ValueError, match="contiguous"):
        moe._dptr(Dev(2, contiguous=False), 2, "x")
    ctx = moe.MoEContext.__new__(moe.MoEContext)
    ctx.H, ctx.handle = 64, None
    assert ctx._rows(x) == 4
    assert ctx._rows(x, torch.zeros(4, dtype=torch.int32), torch.zeros_like(x)) == 4
    with pytest.raises(ValueError, match=r"\[T, 64\]"):
        ctx._rows(torch.zeros((4, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"\[T, 64\]"):
        ctx._rows(torch.zeros(256, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y must be"):
        ctx._rows(x, y=torch.zeros((3, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="token_ids"):
        ctx._rows(x, torch.zeros(3, dtype=torch.int32))
