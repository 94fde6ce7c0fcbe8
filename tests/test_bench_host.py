"""Host logic of bench.py that the reported numbers rest on (CPU only): the
HBM-traffic summary of two counter runs, and the code hash that ties a
traffic file to the kernels it was measured on."""
import argparse
import csv
import json
import os
import shutil

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


@pytest.fixture()
def fake_root(tmp_path, monkeypatch):
    """A copy of the kernel sources and an empty profiles/ under a temporary root."""
    src = os.path.join(ROOT, "quantized_expert_ffn_softmax_amd", "csrc")
    shutil.copytree(src, tmp_path / "quantized_expert_ffn_softmax_amd" / "csrc")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_traffic_summary_scales_each_counter_by_the_calibration_copy(fake_root):
    mb = 512
    gate = "void moe::k_gateup_decode<2, 5, 5, 1>(...)"
    # two gate/up dispatches per run, eight calibration copies (the largest eight count), small copies ignored
    fetch = [(gate, 10000.0), (gate, 12000.0)] + [("__amd_rocclr_copyBuffer", mb * 512.0)] * 8 + \
            [("__amd_rocclr_copyBuffer", 3.0)] * 4
    write = [(gate, 300.0), (gate, 100.0)] + [("__amd_rocclr_copyBuffer", mb * 1024.0)] * 8
    _csv(fake_root / "f.csv", "FETCH_SIZE", fetch + [("other", 1e9)])
    _csv(fake_root / "w.csv", "WRITE_SIZE", write)
    bench.summarize_pmc(argparse.Namespace(summarize_pmc=[str(fake_root / "f.csv"), str(fake_root / "w.csv"), mb],
                                           workload="C2"))
    out = json.load(open(fake_root / "profiles" / "gateup_traffic.json"))
    # FETCH reads half of the copy's bytes (x2), WRITE all of them (x1)
    assert out["scale_fetch"] == 2.0 and out["scale_write"] == 1.0
    assert out["fetch_kib_per_dispatch"] == 11000.0 and out["write_kib_per_dispatch"] == 200.0
    assert out["dispatches"] == [2, 2]
    assert out["bytes_per_launch"] == (11000.0 * 2 + 200.0) * 1024
    assert out["kernel_sha"] == bench.kernel_sha("moe_kernels.hip")


def test_traffic_summary_needs_the_calibration_copies(fake_root):
    gate = "moe::k_gateup_decode<2, 5, 5, 1>"
    _csv(fake_root / "f.csv", "FETCH_SIZE", [(gate, 1.0)] + [("__amd_rocclr_copyBuffer", 1.0)] * 7)
    _csv(fake_root / "w.csv", "WRITE_SIZE", [(gate, 1.0)] + [("__amd_rocclr_copyBuffer", 1.0)] * 8)
    with pytest.raises(SystemExit):
        bench.summarize_pmc(argparse.Namespace(summarize_pmc=[str(fake_root / "f.csv"), str(fake_root / "w.csv"),
                                                              512], workload="C2"))


def test_code_hash_ignores_comments_and_follows_code(fake_root):
    p = fake_root / "quantized_expert_ffn_softmax_amd" / "csrc" / "moe_kernels.hip"
    h0 = bench.kernel_sha("moe_kernels.hip")
    text = p.read_text(encoding="utf-8")
    p.write_text("// a new comment line\n\n" + text.replace("\n", "  \n", 3) + "\n/* and a block\n comment */\n",
                 encoding="utf-8")
    assert bench.kernel_sha("moe_kernels.hip") == h0
    p.write_text(text + "\nnamespace moe { constexpr int kProbe = 1; }\n", encoding="utf-8")
    assert bench.kernel_sha("moe_kernels.hip") != h0
    # a change to a shared device header drops both kernels' counters
    p.write_text(text, encoding="utf-8")
    hp = bench.kernel_sha("moe_prefill.hip")
    hdr = fake_root / "quantized_expert_ffn_softmax_amd" / "csrc" / "moe_device.h"
    hdr.write_text(hdr.read_text(encoding="utf-8") + "\nnamespace moe { constexpr int kProbe2 = 2; }\n",
                   encoding="utf-8")
    assert bench.kernel_sha("moe_kernels.hip") != h0 and bench.kernel_sha("moe_prefill.hip") != hp


def test_committed_traffic_files_match_the_current_code():
    """The traffic figures in profiles/ are used only while the code hashes as recorded."""
    for name, src in (("gateup_traffic.json", "moe_kernels.hip"), ("gemm1_traffic.json", "moe_prefill.hip")):
        rec = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert rec["kernel_sha"] == bench.kernel_sha(src), name
