"""Host-side checks of the measurement harness (no GPU): the single-GPU
refusal, the workloads' work and bytes against closed forms of their shapes,
and the committed HBM traffic summaries against each workload's compulsory
bytes."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import ATTN_WORKLOADS, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MiB = 1 << 20
L2_TOTAL = 8 * 4 * MiB          # eight XCDs with a 4 MiB L2 each


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
    assert r.stdout.strip() == "" or not r.stdout.lstrip().startswith("{")   # no bench line


# (flop, |A| + |B| bytes, |C| bytes) written out from each configuration's
# shape: 2*b*M*N*K multiply-adds counted twice, bf16 operands, fp32 or bf16 output.
CLOSED = {
    "gemm512": (2 * 512 ** 3, 2 * 2 * 512 * 512, 4 * 512 * 512),
    "sscore32x2048": (2 * 32 * 2048 * 2048 * 128, 2 * 2 * 32 * 2048 * 128, 4 * 32 * 2048 * 2048),
    "gemm8192": (2 * 8192 ** 3, 2 * 2 * 8192 * 8192, 2 * 8192 * 8192),
    "gemm65536x256x4096": (2 * 65536 * 256 * 4096, 2 * (65536 * 4096 + 4096 * 256), 4 * 65536 * 256),
    "gemm16384x8192x2048_colA": (2 * 16384 * 8192 * 2048, 2 * (16384 * 2048 + 2048 * 8192), 2 * 16384 * 8192),
    "gemm4096x2048x8192": (2 * 4096 * 2048 * 8192, 2 * (4096 * 8192 + 8192 * 2048), 2 * 4096 * 2048),
}


@pytest.mark.parametrize("name", sorted(CLOSED))
def test_workload_work_and_bytes_match_closed_forms(name):
    w = WORKLOADS[name]
    flop, ab, c = CLOSED[name]
    assert w.flop == flop
    assert w.bytes_a + w.bytes_b == ab
    assert w.bytes_c == c


def test_headline_figures():
    # the figures the measurement is quoted with
    assert WORKLOADS["gemm8192"].flop == pytest.approx(1.0995e12, rel=1e-4)
    s = WORKLOADS["sscore32x2048"]
    assert (s.bytes_a + s.bytes_b, s.bytes_c) == (32 * MiB, 512 * MiB)
    a = ATTN_WORKLOADS["attn32x2048"]
    assert a.flop == 2 * 32 * 2048 * 2048 * (128 + 128)
    # causal: query i sees i + 1 keys, so sum_i (i + 1) = L (L + 1) / 2 pairs
    assert ATTN_WORKLOADS["attn32x2048_causal"].flop == 2 * 32 * (2048 * 2049 // 2) * 256
    g = ATTN_WORKLOADS["attn32x2048_gqa8_causal"]
    assert g.bytes_in == 2 * (32 * 2048 * 128 + 4 * 2 * 2048 * 128)


def _summary(name):
    path = bench.traffic_file(name)
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    return vals


@pytest.mark.parametrize("name", sorted(WORKLOADS) + sorted(ATTN_WORKLOADS))
def test_traffic_summary_agrees_with_compulsory_bytes(name):
    vals = _summary(name)
    assert len(vals["kernel_source_sha256_16"]) == 16
    # a 1 GiB copy reads each byte twice by this counter and writes it once
    assert float(vals["copy_scale_factor"]) == pytest.approx(2.0, rel=0.01)
    assert float(vals["write_scale_factor"]) == pytest.approx(1.0, rel=0.01)
    rd, wr = float(vals["hbm_read_bytes_per_launch"]), float(vals["hbm_write_bytes_per_launch"])
    if name in WORKLOADS:
        w = WORKLOADS[name]
        comp_in, comp_out = w.bytes_a + w.bytes_b, w.bytes_c
    else:
        w = ATTN_WORKLOADS[name]
        comp_in, comp_out = w.bytes_in, w.bytes_out
    if name == "gemm4096x2048x8192":
        # split K, one step = the product kernel, which writes fp32 partial sums
        # (two chunks), and the reduction, which writes C
        comp_out = 2 * 4 * w.M * w.N + w.bytes_c
    # every output byte goes to memory exactly once
    assert wr == pytest.approx(comp_out, rel=0.02)
    # inputs larger than all the L2s together cannot come from L2 across launches
    if comp_in >= L2_TOTAL:
        assert rd >= 0.99 * comp_in
