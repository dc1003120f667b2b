"""Shared GPU-side helpers of the parity tests: run the C ABI with every debug
buffer attached and compare it with the CPU oracle, stage by stage.

Tolerances (checked in compare()):
  - routing outputs, counts, offsets, row order: bit-exact
  - q_x, xs: bit-exact (pure IEEE fp32 operations on both sides)
  - acc1 (GEMM1 int32): bit-exact
  - h (SwiGLU, fp32): relative 1e-5 (the GPU's expf may differ from the host
    libm's in the last place)
  - q_h, hs: bit-exact against the oracle's quantisation of the GPU's own h;
    against the oracle's own trace q_h differs by at most 1 on at most 0.1 %
    of elements and hs by relative 1e-5
  - acc2 (GEMM2 int32) and z (bf16): bit-exact on every row, from the GPU's
    own q_h and hs (and against the oracle's trace on every row whose q_h
    and hs equal the oracle's)
  - output / share_output: max |gpu - ref| <= 2e-2 * max |ref| and
    sum |gpu - ref| / sum |ref| <= 5e-3
"""
from __future__ import annotations

import dataclasses
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


def with_floor_rows(case, zero=(), tiny=(), seed=0, cols=slice(None)):
    """x with token rows (or the columns `cols` of them) at the amax floor:
    `zero` rows all zero, `tiny` rows N(0, 1) * 3e-9 (|x| about 1e-8 at most,
    far below eps = 1e-6, also after smooth scales of at most 2). Every
    quantiser of those rows (or groups) then divides by eps instead of their
    maximum; whole floored rows give h rows of zero or about 1e-15, which take
    the floor again in requantisation."""
    x = case.x.copy()
    rng = np.random.default_rng(seed)
    for t in zero:
        x[t, cols] = 0
    for t in tiny:
        x[t, cols] = synth.f32_to_bf16_bits((rng.standard_normal(x[t, cols].shape) * 3e-9).astype(np.float32))
    return dataclasses.replace(case, x=x)


def grouped_row_tokens(case, ref):
    """Token of every grouped row: the routed pairs in the oracle's grouped
    order, then one shared-expert row per active token."""
    K, P = case.spec.K, ref["P"]
    n = P + (ref["T_act"] if case.spec.I_s else 0)
    return [int(ref["sorted_pair"][r]) // K if r < P else int(ref["shared_token"][r - P]) for r in range(n)]


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


def pack_reference(w, which):
    """The packed order written out with numpy, from its definition: 1 KB
    blocks per (tile, 64-byte step), lane l holding row l % 16, bytes
    16 (l / 16)..+16; a GEMM1 weight's gate and up tiles alternate."""
    G, n, k = w.shape
    t = w.reshape(G, n // 16, 16, k // 64, 4, 16)          # g, tile, row-in-tile, step, lane-group, byte
    t = t.transpose(0, 1, 3, 4, 2, 5)                      # g, tile, step, lane-group, row-in-tile, byte
    if which == moe.MOE_PACK_GMM1:                         # (gate, up) halves -> gate j, up j, gate j + 1, ...
        t = t.reshape(G, 2, n // 32, *t.shape[2:]).swapaxes(1, 2)
    return np.ascontiguousarray(t).reshape(-1)


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


def _routing_rows(case, gpu, ref, tokens):
    """Check the routing outputs (bit-exact) and return (grouped rows the
    oracle computed, tokens)."""
    s = case.spec
    T, K = s.T, s.K
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
    return np.array(sorted(rows), dtype=np.int64), toks


def _row_experts(case, gpu, rows, P):
    """Group index of each grouped row: the local expert of a routed row (from
    the GPU's own sorted_pair, which is checked bit-exactly first), E_loc for a
    shared row."""
    s = case.spec
    base = s.ep_rank * s.E_loc
    sp = gpu["sorted_pair"]
    ids = case.expert_ids.reshape(-1)
    return np.array([int(ids[sp[r]]) - base if r < P else s.E_loc for r in rows], dtype=np.int64)


def _gemm2_own_inputs(case, gpu, rows, P):
    """GEMM2 of every grouped row on the GPU's own requantised input: acc2 must
    equal the exact product of the GPU's q_h row and W2 (float64 sums of int8
    products are exact: |acc| <= I * 127^2 < 2^53), and z must equal
    bf16((float(acc2) * w2s) * row scale) with the GPU's hs (times the pair's
    routing weight, rounded once, with the fused route scale). Returns the
    number of rows checked."""
    s = case.spec
    groups = _row_experts(case, gpu, rows, P)
    qh, hs = gpu["q_h"], gpu["hs"].astype(np.float32)
    w_pair = case.expert_scales.reshape(-1).astype(np.float32)
    for g in np.unique(groups):
        rg = rows[groups == g]
        if g < s.E_loc:
            n, W, ws = s.I, case.w2[g], case.w2s[g]
        else:
            n, W, ws = s.I_s, case.sw2, case.sw2s
        exact = qh[rg, :n].astype(np.float64) @ W.astype(np.float64).T
        assert np.abs(exact).max(initial=0) < 2 ** 31
        exact = exact.astype(np.int64)
        got = gpu["acc2"][rg].astype(np.int64)
        bad = np.nonzero(~np.all(got == exact, axis=1))[0]
        assert bad.size == 0, f"acc2 row {int(rg[bad[0]])} (group {g}) differs from q_h x W2"
        rs = hs[rg]
        if s.fuse_route_scale and g < s.E_loc:
            rs = (rs * w_pair[gpu["sorted_pair"][rg]]).astype(np.float32)
        y = exact.astype(np.int32).astype(np.float32) * ws.astype(np.float32)[None, :]
        y = (y * rs[:, None]).astype(np.float32)
        zexp = synth.f32_to_bf16_bits(y)
        bad = np.nonzero(~np.all(gpu["z"][rg] == zexp, axis=1))[0]
        assert bad.size == 0, f"z row {int(rg[bad[0]])} (group {g}) is not bf16((acc2 * w2s) * hs)"
    return len(rows)


def compare(case, gpu, ref, tokens=None):
    """Stage-by-stage comparison. `ref` is oracle.forward(case, tokens, trace=True).

    Every grouped row of the computed tokens is checked at every stage: q_x,
    xs, acc1 against the oracle bit for bit; h against the oracle to
    relative 1e-5; q_h / hs bit for bit against the oracle's quantisation of
    the GPU's own h, and within 1 LSB of the oracle's trace; acc2 and z bit
    for bit from the GPU's own q_h / hs (where those equal the oracle's, also
    against the oracle's own acc2 and z); outputs within the block's
    tolerance."""
    s = case.spec
    P = ref["P"]
    rows, toks = _routing_rows(case, gpu, ref, tokens)
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
        # requantisation on the GPU's own h: the oracle's quantiser, bit for bit
        for r, n in zip(rows, inter):
            q_exp, hs_exp = oracle.quant_row(gpu["h"][r, :n], s.eps)
            assert np.array_equal(gpu["q_h"][r, :n], q_exp), f"q_h row {r} is not the quantisation of its h"
            assert gpu["hs"][r] == hs_exp, f"hs row {r} is not the scale of its h"
        dq = np.abs(gpu["q_h"][rows].astype(int) - ref["q_h"][rows].astype(int))[hmask]
        assert dq.max(initial=0) <= 1, "q_h off by more than 1"
        frac = (dq > 0).mean() if dq.size else 0.0
        assert frac <= 1e-3, f"q_h differs on {frac:.2%}"
        assert np.all(np.abs(gpu["hs"][rows] - ref["hs"][rows]) <= 1e-5 * ref["hs"][rows])
        checked = _gemm2_own_inputs(case, gpu, rows, P)
        same = [r for r, n in zip(rows, inter)
                if np.array_equal(gpu["q_h"][r, :n], ref["q_h"][r, :n]) and gpu["hs"][r] == ref["hs"][r]]
        for r in same:
            assert np.array_equal(gpu["acc2"][r], ref["acc2"][r]), f"acc2 row {r}"
            assert np.array_equal(gpu["z"][r], ref["z"][r]), f"z row {r}"
        stats.update(rows=len(rows), rows_gemm2_checked=checked, rows_exact_qh=len(same),
                     qh_diff_frac=float(frac))
    stats["output"] = out_close(gpu["output"][toks], ref["output"][toks], "output")
    if s.I_s:
        stats["share_output"] = out_close(gpu["share_output"][toks], ref["share_output"][toks], "share_output")
    return stats


def check(case, tokens=None, tensors=None, ref=None, **kw):
    """Run the GPU path and compare it with the oracle (computed here on the
    host's threads unless `ref` passes an earlier oracle run of the same
    case and tokens)."""
    gpu = run_gpu(case, tensors=tensors, **kw)
    if ref is None:
        ref = oracle.forward(case, tokens=tokens, trace=True, threads=oracle.default_threads())
    return compare(case, gpu, ref, tokens), gpu, ref


# ---------------------------------------------------------------- FP4 weights
#
# The FP8 x FP4 MFMA accumulates in fp32 with its own rounding, so the GEMM
# accumulators are not bit-exact; every later stage is checked bit-exactly
# (up to expf) on the GPU's own inputs, which pins each kernel separately:
#   - q_x, xs: bit-exact against the oracle (same fp32 operations);
#   - acc1, acc2: |gpu - exact| <= ACC_REL * sum_k |term_k|, where the exact
#     fp32-rounded sum and the magnitude sum come from oracle.gemm_mx on the
#     GPU's input codes (for the magnitude: signs cleared). The hardware's
#     own error is at most about 2^-13.5 of that sum per instruction (measured
#     on random operands); the bound leaves a factor 5 above it; a wrong lane,
#     block or scale mapping is off by O(1);
#   - h: SwiGLU of (acc1 * w1s) * xs, relative 1e-5 (expf);
#   - q_h, hs: bit-exact against the oracle's FP8 quantisation of the GPU's h;
#   - z: bf16((acc2 * w2s) * row scale), bit-exact;
#   - against the oracle's own trace: q_h codes within one E4M3 step;
#   - output / share_output: the block's output tolerance (out_close).
ACC_REL = 2.0 ** -11


def _e4m3_step(c):
    """Signed position of E4M3 codes on the grid (+0 and -0 both 0)."""
    c = np.asarray(c).astype(np.int32)
    m = c & 0x7F
    return np.where(c & 0x80, -m, m)


def _map_rows(fn, rows):
    """fn over every grouped row on the host's threads (the oracle's routines
    and numpy's kernels release the GIL); the first failing row's assertion
    propagates."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(oracle.default_threads()) as ex:
        return list(ex.map(fn, [int(r) for r in rows]))


def _mx_acc_check(got, codes, data, bscale, what):
    exact = oracle.gemm_mx(codes[None, :], data, bscale)[0]
    mag = oracle.gemm_mx((codes & 0x7F)[None, :], data & 0x77, bscale)[0]
    err = np.abs(got.astype(np.float64) - exact.astype(np.float64))
    bound = ACC_REL * mag.astype(np.float64) + 1e-30
    assert np.all(err <= bound), f"{what}: worst err/sum|terms| {np.max(err / (mag + 1e-30)):.3g}"
    return float(np.max(err / (mag.astype(np.float64) + 1e-30)))


def compare_mx(case, gpu, ref, tokens=None):
    """compare() for weight_format "mxfp4"."""
    s = case.spec
    K, H, P = s.K, s.H, ref["P"]
    rows, toks = _routing_rows(case, gpu, ref, tokens)
    stats = {}
    qx = gpu["q_x"].view(np.uint8)
    qh = gpu["q_h"].view(np.uint8)
    acc1 = gpu["acc1"].view(np.float32)
    acc2 = gpu["acc2"].view(np.float32)
    base = s.ep_rank * s.E_loc

    def row_check(r):
        worst = 0.0
        if r < P:
            p = int(gpu["sorted_pair"][r])
            e = int(case.expert_ids[p // K, p % K]) - base
            n = s.I
            w1, w1b, w1s = case.w1[e], case.w1b[e], case.w1s[e]
            w2, w2b, w2s = case.w2[e], case.w2b[e], case.w2s[e]
            rw = case.expert_scales[p // K, p % K]
        else:
            n = s.I_s
            w1, w1b, w1s, w2, w2b, w2s = case.sw1, case.sw1b, case.sw1s, case.sw2, case.sw2b, case.sw2s
            rw = None
        assert np.array_equal(qx[r], ref["q_x"][r]), f"q_x row {r}"
        assert gpu["xs"][r] == ref["xs"][r], f"xs row {r}"
        a1 = acc1[r, :2 * n]
        worst = max(worst, _mx_acc_check(a1, qx[r], w1, w1b, f"acc1 row {r}"))
        y = (a1 * w1s) * np.float32(gpu["xs"][r])
        h_exp = oracle.swiglu(y.astype(np.float32))
        hg = gpu["h"][r, :n]
        assert np.all(np.abs(hg - h_exp) <= 1e-5 * np.abs(h_exp) + 1e-30), f"h row {r}"
        q_exp, hs_exp = oracle.quant_row_fp8(hg, s.eps)
        assert np.array_equal(qh[r, :n], q_exp), f"q_h row {r}"
        assert gpu["hs"][r] == np.float32(hs_exp), f"hs row {r}"
        d = np.abs(_e4m3_step(qh[r, :n]) - _e4m3_step(ref["q_h"][r, :n]))
        assert d.max(initial=0) <= 1, f"q_h row {r} more than one E4M3 step from the oracle's"
        a2 = acc2[r, :H]
        worst = max(worst, _mx_acc_check(a2, qh[r, :n], w2, w2b, f"acc2 row {r}"))
        rs2 = np.float32(gpu["hs"][r])
        if s.fuse_route_scale and rw is not None:
            rs2 = np.float32(rs2 * np.float32(rw))
        z_exp = synth.f32_to_bf16_bits((a2 * w2s) * rs2)
        assert np.array_equal(gpu["z"][r], z_exp), f"z row {r}"
        return worst, float((d > 0).mean())

    res = _map_rows(row_check, rows)
    worst = max((w for w, _ in res), default=0.0)
    flips = [f for _, f in res]
    stats.update(rows=len(rows), acc_err_over_sum=worst, qh_step_frac=max(flips, default=0.0))
    stats["output"] = out_close(gpu["output"][toks], ref["output"][toks], "output")
    if s.I_s:
        stats["share_output"] = out_close(gpu["share_output"][toks], ref["share_output"][toks], "share_output")
    return stats


def check_mx(case, tokens=None, tensors=None, **kw):
    gpu = run_gpu(case, tensors=tensors, **kw)
    ref = oracle.forward(case, tokens=tokens, trace=True, threads=oracle.default_threads())
    return compare_mx(case, gpu, ref, tokens), gpu, ref


# -------------------------------------------------- group-wise activation scales
#
# quant_mode 2: the GPU dequantises each group's int32 partial exactly as the
# oracle does (p_g = (float(acc_g) * w_scale) * group_scale) but adds the p_g
# per wave, then over the waves, where the oracle adds them left to right; so
# the fp32 GEMM outputs are held to the bound of that reassociation,
# |gpu - oracle| <= 2 * n_groups * 2^-24 * sum_g |p_g|, with the p_g taken
# from numpy int64 products of the GPU's own codes. Every other stage is
# checked bit-exactly on the GPU's own inputs, as for FP4 weights.


def _group_terms(q, scales, W, ws, G):
    """float64 p_g [N, n_groups] of one row: int64 partial x weight scale x group scale."""
    n = len(scales)
    parts = np.stack([W[:, g * G:(g + 1) * G].astype(np.int64) @ q[g * G:(g + 1) * G].astype(np.int64)
                      for g in range(n)], axis=1).astype(np.float64)
    return parts * ws[:, None].astype(np.float64) * scales[None, :].astype(np.float64)


def _group_gemm_check(got, q, scales, W, ws, G, what):
    exact = oracle.gemm_i8_groups(q, scales, W, ws, G).astype(np.float64)
    terms = _group_terms(q, scales, W, ws, G)
    bound = 2 * terms.shape[1] * 2.0 ** -24 * np.abs(terms).sum(axis=1) + 1e-30
    err = np.abs(got.astype(np.float64) - exact)
    assert np.all(err <= bound), f"{what}: worst err / bound {np.max(err / bound):.3g}"
    return float(np.max(err / bound))


def compare_group(case, gpu, ref, tokens=None):
    """compare() for group-wise activation scales (quant_group > 0)."""
    s = case.spec
    K, H, P, G = s.K, s.H, ref["P"], s.quant_group
    rows, toks = _routing_rows(case, gpu, ref, tokens)
    acc1 = gpu["acc1"].view(np.float32)
    acc2 = gpu["acc2"].view(np.float32)
    base = s.ep_rank * s.E_loc

    def row_check(r):
        worst = 0.0
        if r < P:
            p = int(gpu["sorted_pair"][r])
            e = int(case.expert_ids[p // K, p % K]) - base
            n, w1, w1s, w2, w2s = s.I, case.w1[e], case.w1s[e], case.w2[e], case.w2s[e]
        else:
            n, w1, w1s, w2, w2s = s.I_s, case.sw1, case.sw1s, case.sw2, case.sw2s
        assert np.array_equal(gpu["q_x"][r], ref["q_x"][r]), f"q_x row {r}"
        assert np.array_equal(gpu["xs"][r], ref["xs"][r]), f"xs row {r}"
        y1 = acc1[r, :2 * n]
        worst = max(worst, _group_gemm_check(y1, gpu["q_x"][r], gpu["xs"][r], w1, w1s, G, f"acc1 row {r}"))
        h_exp = oracle.swiglu(y1.astype(np.float32))
        hg = gpu["h"][r, :n]
        assert np.all(np.abs(hg - h_exp) <= 1e-5 * np.abs(h_exp) + 1e-30), f"h row {r}"
        q_exp, hs_exp = oracle.quant_row_groups(hg, G, s.eps)
        assert np.array_equal(gpu["q_h"][r, :n], q_exp), f"q_h row {r}"
        assert np.array_equal(gpu["hs"][r, :n // G], hs_exp), f"hs row {r}"
        d = np.abs(gpu["q_h"][r, :n].astype(int) - ref["q_h"][r, :n].astype(int))
        assert d.max(initial=0) <= 1, f"q_h row {r} more than 1 from the oracle's"
        y2 = acc2[r, :H]
        worst = max(worst, _group_gemm_check(y2, gpu["q_h"][r, :n], gpu["hs"][r, :n // G], w2, w2s, G,
                                             f"acc2 row {r}"))
        assert np.array_equal(gpu["z"][r], synth.f32_to_bf16_bits(y2)), f"z row {r}"
        return worst, float((d > 0).mean())

    res = _map_rows(row_check, rows)
    worst = max((w for w, _ in res), default=0.0)
    flips = [f for _, f in res]
    stats = dict(rows=len(rows), acc_err_over_bound=worst, qh_diff_frac=max(flips, default=0.0))
    stats["output"] = out_close(gpu["output"][toks], ref["output"][toks], "output")
    if s.I_s:
        stats["share_output"] = out_close(gpu["share_output"][toks], ref["share_output"][toks], "share_output")
    return stats


def check_group(case, tokens=None, tensors=None, **kw):
    gpu = run_gpu(case, tensors=tensors, **kw)
    ref = oracle.forward(case, tokens=tokens, trace=True, threads=oracle.default_threads())
    return compare_group(case, gpu, ref, tokens), gpu, ref
