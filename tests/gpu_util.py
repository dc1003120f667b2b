"""Shared GPU-side helpers of the parity tests: run the C ABI with every debug
buffer attached and compare it with the CPU oracle, stage by stage.

Tolerances (checked in compare()):
  - routing outputs, counts, offsets, row order: bit-exact
  - q_x, xs: bit-exact (pure IEEE fp32 operations on both sides)
  - acc1 (GEMM1 int32): bit-exact
  - h (SwiGLU, fp32): relative 1e-5 (the GPU's expf may differ from the host
    libm's in the last place)
  - q_h: differs by at most 1 on at most 0.1 % of elements; hs relative 1e-5
  - acc2 (GEMM2 int32) and z (bf16): bit-exact on every row whose q_h and hs
    equal the oracle's
  - output / share_output: max |gpu - ref| <= 2e-2 * max |ref| and
    sum |gpu - ref| / sum |ref| <= 5e-3
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_expert_ffn_route_amd as moe
import oracle
from moe_expert_ffn_route_amd import synth

F32 = synth.bf16_bits_to_f32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(case, tensors=None, dbg=True, stream=None, garbage_workspace=False, packed=False):
    dims = moe.dims_of_case(case)
    if tensors is None:
        tensors = moe.upload(case)
    if packed:
        tensors = moe.pack_weights(tensors)
        dims.weight_layout = moe.MOE_WEIGHT_PACKED
    runner = moe.Runner(dims)
    if garbage_workspace:
        runner.workspace.fill_(0xA5)
        runner.output.fill_(7)
        if runner.share_output is not None:
            runner.share_output.fill_(7)
    d, bufs = moe.debug_buffers(dims) if dbg else (None, {})
    runner(tensors, dbg=d, stream=stream)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in bufs.items()}
    res["output"] = runner.output.view(torch.int16).cpu().numpy().view(np.uint16)
    if runner.share_output is not None:
        res["share_output"] = runner.share_output.view(torch.int16).cpu().numpy().view(np.uint16)
    res["expert_token_nums"] = runner.expert_token_nums.cpu().numpy()
    if "z" in res:
        res["z"] = res["z"].view(np.uint16)
    return res


def out_close(got_bits, ref_bits, what):
    g = F32(got_bits).astype(np.float64)
    r = F32(ref_bits).astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - r)
    mx = np.abs(r).max() if r.size else 0.0
    assert err.max(initial=0.0) <= 2e-2 * mx + 1e-30, f"{what}: max err {err.max()} vs max|ref| {mx}"
    den = np.abs(r).sum()
    if den > 0:
        assert err.sum() / den <= 5e-3, f"{what}: mean rel err {err.sum() / den}"
    return float(err.max(initial=0.0)), float((g == r).mean()) if r.size else 1.0


def compare(case, gpu, ref, tokens=None):
    """Stage-by-stage comparison. `ref` is oracle.forward(case, tokens, trace=True)."""
    s = case.spec
    T, K, H = s.T, s.K, s.H
    # routing: always global
    P, Ta = ref["P"], ref["T_act"]
    nr = gpu["num_rows"]
    assert nr[0] == P and nr[1] == Ta and nr[2] == ref["n_bad"], (nr, P, Ta, ref["n_bad"])
    assert np.array_equal(gpu["expert_token_nums"], ref["expert_token_nums"])
    assert np.array_equal(gpu["group_offset"], ref["offsets"])
    assert np.array_equal(gpu["sorted_pair"][:P], ref["sorted_pair"])
    assert np.array_equal(gpu["row_of_pair"][: T * K], ref["row_of_pair"][: T * K])
    if s.I_s:
        assert np.array_equal(gpu["shared_token"][:Ta], ref["shared_token"])
    # rows the oracle computed
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    rop = ref["row_of_pair"][: T * K].reshape(T, K) if T else np.zeros((0, K), int)
    rows = [int(r) for t in toks for r in rop[t] if r >= 0]
    if s.I_s:
        act = np.ones(T, bool) if case.mask is None else case.mask.astype(bool)
        rank = np.cumsum(act) - 1
        rows += [P + int(rank[t]) for t in toks if act[t]]
    rows = np.array(sorted(rows), dtype=np.int64)
    stats = {}
    if len(rows):
        inter = np.where(rows < P, s.I, s.I_s)
        assert np.array_equal(gpu["q_x"][rows], ref["q_x"][rows]), "q_x"
        assert np.array_equal(gpu["xs"][rows], ref["xs"][rows]), "xs"
        Imax = max(s.I, s.I_s)
        for r, n in zip(rows, inter):
            assert np.array_equal(gpu["acc1"][r, :2 * n], ref["acc1"][r, :2 * n]), f"acc1 row {r}"
        hmask = np.arange(Imax)[None, :] < inter[:, None]
        hg, hr = gpu["h"][rows][hmask], ref["h"][rows][hmask]
        assert np.all(np.abs(hg - hr) <= 1e-5 * np.abs(hr) + 1e-30), "h"
        dq = np.abs(gpu["q_h"][rows].astype(int) - ref["q_h"][rows].astype(int))[hmask]
        assert dq.max(initial=0) <= 1, "q_h off by more than 1"
        frac = (dq > 0).mean() if dq.size else 0.0
        assert frac <= 1e-3, f"q_h differs on {frac:.2%}"
        assert np.all(np.abs(gpu["hs"][rows] - ref["hs"][rows]) <= 1e-5 * ref["hs"][rows])
        same = [r for r, n in zip(rows, inter)
                if np.array_equal(gpu["q_h"][r, :n], ref["q_h"][r, :n]) and gpu["hs"][r] == ref["hs"][r]]
        for r in same:
            assert np.array_equal(gpu["acc2"][r], ref["acc2"][r]), f"acc2 row {r}"
            assert np.array_equal(gpu["z"][r], ref["z"][r]), f"z row {r}"
        stats.update(rows=len(rows), rows_exact_qh=len(same), qh_diff_frac=float(frac))
    stats["output"] = out_close(gpu["output"][toks], ref["output"][toks], "output")
    if s.I_s:
        stats["share_output"] = out_close(gpu["share_output"][toks], ref["share_output"][toks], "share_output")
    return stats


def check(case, tokens=None, tensors=None, **kw):
    gpu = run_gpu(case, tensors=tensors, **kw)
    ref = oracle.forward(case, tokens=tokens, trace=True)
    return compare(case, gpu, ref, tokens), gpu, ref
