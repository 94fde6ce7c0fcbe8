"""Rules the product's sources and build keep (CPU only).

The HIP path and the oracle share no code and neither reaches the other; the
binding fails loudly when the HIP library is missing (no CPU fallback); every
HIP source is compiled for gfx950 with packed fp32 instructions disabled; the
sources avoid runtime features this design rules out (non-default stream
priorities, registering existing host memory, uncached device memory, memsets
on paths a caller may capture in a graph); nothing tracked runs a working file.
"""
import os
import re
import subprocess

import pytest

import quantized_expert_ffn_softmax_amd as moe
from quantized_expert_ffn_softmax_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_expert_ffn_softmax_amd")


def _files(top, suffixes):
    for d, dirs, fs in os.walk(top):
        dirs[:] = [x for x in dirs if x != "__pycache__"]
        for f in sorted(fs):
            if f.endswith(suffixes):
                yield os.path.join(d, f)


def _read(p):
    with open(p, encoding="utf-8") as f:
        return f.read()


def test_product_path_never_reaches_the_oracle():
    for p in list(_files(PKG, (".py", ".hip", ".h"))) + [os.path.join(ROOT, "include", "moe.h")]:
        assert not re.search(r"\boracle\b|liboracle", _read(p)), f"{p} names the oracle"


def test_oracle_never_reaches_the_hip_path():
    for p in _files(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        text = _read(p)
        assert "quantized_expert_ffn_softmax_amd" not in text and "libmoe" not in text, p
        assert not re.search(r"#include\s+\"[^\"]*(moe_device|moe_internal|moe\.h)", text), p


def test_binding_raises_without_the_hip_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "libmoe.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()


def test_every_hip_source_is_built_for_gfx950_without_packed_fp32():
    flags = " ".join(_build.FLAGS)
    assert "--offload-arch=gfx950" in flags
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in flags
    on_disk = sorted(os.path.basename(p) for p in _files(os.path.join(PKG, "csrc"), (".hip",)))
    assert sorted(os.path.basename(s) for s in _build.SOURCES) == on_disk


def test_sources_avoid_ruled_out_runtime_features():
    banned = re.compile(r"hipStreamCreateWithPriority|hipHostRegister|hipExtMallocWithFlags|MallocUncached"
                        r"|v_pk_(add|mul|fma)_f32|is_high_priority_stream|priority\s*=")
    for p in list(_files(PKG, (".py", ".hip", ".h"))) + [os.path.join(ROOT, "bench.py")]:
        m = banned.search(_read(p))
        assert m is None, f"{p}: {m.group(0) if m else ''}"


def test_no_memset_on_a_capturable_path():
    """The one hipMemsetAsync clears the router statistics during a weight
    upload, on the context's own upload stream; forward and routing calls
    (which a caller may capture in a HIP graph) record none."""
    hits = []
    for p in _files(os.path.join(PKG, "csrc"), (".hip", ".h")):
        for i, line in enumerate(_read(p).splitlines()):
            if "hipMemsetAsync" in line:
                hits.append((os.path.basename(p), line.strip()))
    assert hits == [("moe_prefill.hip", "hipError_t e = hipMemsetAsync(rstat, 0, 2 * sizeof(float), st);")]
    api = _read(os.path.join(PKG, "csrc", "moe_api.hip"))
    assert api.count("launch_router_stats(") == 1 and "c->load_stream" in api.split("launch_router_stats(")[1][:200]


def test_tracked_code_runs_no_working_file():
    try:
        tracked = subprocess.run(["git", "ls-files"], cwd=ROOT, capture_output=True, text=True, check=True).stdout
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("not a git checkout")
    for rel in tracked.split():
        if rel.endswith((".py", ".hip", ".h", ".c", ".sh", ".ini")) and not rel.endswith("test_build_rules.py"):
            assert "_work" not in _read(os.path.join(ROOT, rel)), rel
