"""CPU checks of bench.py's contract and of the byte and operation counts its
roofline line divides by (no GPU needed)."""
import dataclasses
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_expert_ffn_route_amd import synth  # noqa: E402


def _shape_only(s):
    """A Case with the workload's sizes and no data (the counts are given)."""
    return synth.Case(spec=s, x=np.zeros((s.T, s.H), np.uint16), expert_ids=None, expert_scales=None, w1=None,
                      w1s=None, w2=None, w2s=None)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=600)


def test_more_than_one_gpu_is_refused_before_any_work():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_config_one_gemm1_bytes_match_the_headline_figure():
    # the decode workload's GEMM1 moves, per touched expert, its gate and up
    # weights (2 I H bytes) and their scales (8 I), the shared expert's alike,
    # and per grouped row the int8 input row, its scale and the fp32 h row:
    # 59 touched experts and 72 rows give 1 008 501 024 bytes
    s = synth.WORKLOADS[1]
    case = _shape_only(s)
    counts = np.zeros(256, np.int32)
    counts[:59] = 1
    counts[:5] += 1  # 64 kept pairs over 59 experts
    _, g1, g2, touched, rows = bench.algorithmic_bytes(case, counts)
    H, I = 4096, 2048
    assert touched == 59 and rows == 64 + 8
    assert g1 == 60 * (2 * I * H + 8 * I) + 72 * (H + 4 + 4 * I) == 1_008_501_024
    assert g2 == 60 * (H * I + 4 * H) + 64 * (I + 4 + 2 * H) + 8 * (I + 4 + 2 * H)


def test_fp4_bytes_per_weight_element():
    s = synth.WORKLOADS[1]
    assert bench.weight_bytes_per_element(s) == 1.0
    assert bench.weight_bytes_per_element(dataclasses.replace(s, weight_format="mxfp4")) == 0.5 + 1 / 32


def test_gemm_ops_count_two_per_multiply_add():
    s = synth.WORKLOADS[4]
    case = _shape_only(s)
    counts = np.full(256, 16, np.int32)  # 4096 pairs
    g1, g2 = bench.gemm_ops(case, counts)
    rows = 4096 + 512
    assert g1 == 2 * rows * 2 * 2048 * 4096 and g2 == 2 * rows * 4096 * 2048
    assert bench.layer_ops(case, counts) == g1 + g2


def test_gemm_write_bytes_at_t512():
    # GEMM1 writes an fp32 h row of max(I, I_s) per grouped row, GEMM2 a bf16
    # row of H per routed row and per active token (z and share_output)
    s = synth.WORKLOADS[4]
    case = _shape_only(s)
    counts = np.full(256, 16, np.int32)  # 4096 routed rows
    w1, w2 = bench.gemm_write_bytes(case, counts)
    assert w1 == (4096 + 512) * 4 * 2048 == 37_748_736
    assert w2 == (4096 + 512) * 2 * 4096
    _, g1, g2, _, _ = bench.algorithmic_bytes(case, counts)
    assert w1 < g1 and w2 < g2
