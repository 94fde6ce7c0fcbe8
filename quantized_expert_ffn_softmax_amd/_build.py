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
    # MFMA results in VGPRs: the decode kernels scale every block product on the
    # VALU, and results in AGPRs would each need a v_accvgpr_read first
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-result", "-Wno-unused-value",
]


def build(verbose: bool = False) -> str:
    """Compiles every source to an object in parallel, then links libmoe.so."""
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    missing = [s for s in srcs if not os.path.exists(s)]
    if missing:
        raise RuntimeError(f"HIP sources missing: {missing}")
    inc = ["-I", os.path.join(os.path.dirname(HERE), "include")]
    objs, procs = [], []
    for src in srcs:
        obj = os.path.join(HERE, "_obj_" + os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + inc + ["-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    failed = False
    for p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out + err)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    for obj in objs:
        os.remove(obj)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    errs = [ln for ln in r.stderr.splitlines() if "error" in ln.lower()]
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
