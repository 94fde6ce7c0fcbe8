"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into libmoe.so.

    python -m quantized_expert_ffn_softmax_amd._build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["csrc/moe_api.hip", "csrc/moe_kernels.hip", "csrc/moe_prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-value",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, s) for s in SOURCES if os.path.exists(os.path.join(HERE, s))]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(os.path.dirname(HERE), "include"), "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    errs = [ln for ln in r.stderr.splitlines() if "error" in ln.lower()]
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
