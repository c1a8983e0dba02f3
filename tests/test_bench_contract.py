"""bench.py's host-side contract: one GPU only, and the algorithmic work figures it prices the
roofline with (checked against hand counts at the Mixtral prefill shape)."""
import json
import os
import subprocess
import sys

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in line and line["n_gpus"] == 2


def test_layer_work_mixtral_prefill():
    w = wl.get("mixtral_prefill")
    R = w.T * w.k                                   # no capacity: every assignment kept
    work = bench.layer_work(w, R, w.E)
    # gate/up: 2 products of d x d_e per kept row, 2 FLOPs per multiply-add
    assert work["flops_gate_up"] == 4 * 4096 * 14336 * 8192
    assert work["flops_down"] == 2 * 4096 * 14336 * 8192
    # bytes: every expert's gate and up weights once (bf16), x rows in, h rows out
    assert work["bytes_gate_up"] == 8 * 2 * 14336 * 4096 * 2 + 8192 * 4096 * 2 + 8192 * 14336 * 2
    assert work["bytes_down"] == 8 * 4096 * 14336 * 2 + 8192 * 14336 * 2 + 8192 * 4096 * 4


def test_layer_work_quantised_weights():
    w8 = wl.get("mixtral_decode_fp8")
    w4 = wl.get("mixtral_decode_mxfp4")
    R = w8.T * w8.k
    # FP8: one byte per weight plus a 4-byte scale per row; MXFP4: half a byte plus a scale byte per 32
    assert bench.layer_work(w8, R, 8)["bytes_gate_up"] == 8 * 2 * 14336 * (4096 + 4) + R * 4096 * 2 + R * 14336 * 2
    assert bench.layer_work(w4, R, 8)["bytes_gate_up"] == 8 * 2 * 14336 * 4096 * (0.5 + 1 / 32) + R * 4096 * 2 \
        + R * 14336 * 2
