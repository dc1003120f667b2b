"""CPU checks of the GPU parity harness itself (tests/gpu_util.compare): fed
the oracle's own trace laid out as the GPU's debug dumps, it passes; a
GEMM2 mistake confined to a row whose requantised input legitimately
differs from the oracle's by one code is still caught, as is a wrong row
scale in z, a wrong requantisation of the GPU's own h, and a wrong acc1."""
import dataclasses

import numpy as np
import pytest

import oracle
from moe_expert_ffn_route_amd import synth
from gpu_util import compare


def _as_gpu(case, ref):
    """The oracle's trace in the layout run_gpu() returns."""
    s = case.spec
    T, K = s.T, s.K
    R = T * K + T
    g = {k: np.array(ref[k], copy=True) for k in ("q_x", "xs", "acc1", "h", "q_h", "hs", "acc2", "z",
                                                    "output", "expert_token_nums")}
    if s.I_s:
        g["share_output"] = ref["share_output"].copy()
    P = ref["P"]
    sp = np.full(max(1, T * K), -1, np.int32)
    sp[:P] = ref["sorted_pair"]
    g["sorted_pair"] = sp
    g["row_of_pair"] = ref["row_of_pair"].copy()
    g["group_offset"] = ref["offsets"].copy()
    st = np.full(max(1, T), -1, np.int32)
    st[:ref["T_act"]] = ref["shared_token"]
    g["shared_token"] = st
    g["num_rows"] = np.array([P, ref["T_act"], ref["n_bad"], 0], np.int32)
    assert g["q_x"].shape[0] == R
    return g


def _case(**kw):
    base = dict(name="harness", T=12, H=256, I=256, E_g=8, K=3, I_s=256, seed=9101)
    base.update(kw)
    return synth.make_case(synth.Spec(**base))


def _bump_qh(case, gpu, r):
    """Change one code of row r's q_h by one (a legitimate 1-LSB difference)
    and recompute that row's acc2 and z consistently from it."""
    s = case.spec
    P = int(gpu["num_rows"][0])
    n = s.I if r < P else s.I_s
    j = int(np.argmax(np.abs(gpu["q_h"][r, :n]) < 127))
    gpu["q_h"][r, j] += 1
    if r < P:
        p = int(gpu["sorted_pair"][r])
        e = int(case.expert_ids.reshape(-1)[p]) - s.ep_rank * s.E_loc
        W, ws = case.w2[e], case.w2s[e]
    else:
        W, ws = case.sw2, case.sw2s
    acc = gpu["q_h"][r, :n].astype(np.int64) @ W.astype(np.int64).T
    gpu["acc2"][r] = acc
    rs = np.float32(gpu["hs"][r])
    if s.fuse_route_scale and r < P:
        rs = np.float32(rs * np.float32(case.expert_scales.reshape(-1)[int(gpu["sorted_pair"][r])]))
    gpu["z"][r] = synth.f32_to_bf16_bits((acc.astype(np.int32).astype(np.float32) * ws) * rs)
    return j


@pytest.mark.parametrize("fused", [False, True])
def test_harness_accepts_the_oracle_and_catches_a_wrong_requant(fused):
    case = _case(fuse_route_scale=fused, active=10, smooth=True)
    ref = oracle.forward(case, trace=True)
    gpu = _as_gpu(case, ref)
    st = compare(case, gpu, ref)
    assert st["rows"] == st["rows_gemm2_checked"] == st["rows_exact_qh"]
    # a requantised code one off on one row, with acc2 and z consistent with
    # it: the requantisation check on the GPU's own h catches it
    r = 5
    gpu2 = _as_gpu(case, ref)
    _bump_qh(case, gpu2, r)
    with pytest.raises(AssertionError, match="q_h row 5 is not the quantisation"):
        compare(case, gpu2, ref)


def test_harness_catches_gemm2_error_on_a_row_with_a_differing_code(monkeypatch):
    case = _case()
    ref = oracle.forward(case, trace=True)
    r = 7
    gpu = _as_gpu(case, ref)
    _bump_qh(case, gpu, r)
    # accept the bumped code as a legitimate requantisation of this row
    real = oracle.quant_row

    def quant_row(v, eps=1e-6):
        q, sc = real(v, eps)
        if np.array_equal(v, gpu["h"][r, :len(v)]):
            q = gpu["q_h"][r, :len(v)].copy()
        return q, sc

    monkeypatch.setattr(oracle, "quant_row", quant_row)
    st = compare(case, gpu, ref)
    assert st["rows_exact_qh"] == st["rows"] - 1 and st["rows_gemm2_checked"] == st["rows"]
    bad = {k: v.copy() for k, v in gpu.items()}
    bad["acc2"][r, 3] += 1
    with pytest.raises(AssertionError, match=f"acc2 row {r}"):
        compare(case, bad, ref)
    bad = {k: v.copy() for k, v in gpu.items()}
    bad["z"][r, 9] ^= 1
    with pytest.raises(AssertionError, match=f"z row {r}"):
        compare(case, bad, ref)


def test_harness_catches_wrong_row_scale_and_acc1():
    case = _case(seed=9102)
    ref = oracle.forward(case, trace=True)
    gpu = _as_gpu(case, ref)
    bad = {k: v.copy() for k, v in gpu.items()}
    bad["hs"][2] = np.float32(bad["hs"][2] * 2)
    with pytest.raises(AssertionError):
        compare(case, bad, ref)
    bad = {k: v.copy() for k, v in gpu.items()}
    bad["acc1"][4, 1] += 1
    with pytest.raises(AssertionError, match="acc1 row 4"):
        compare(case, bad, ref)


def test_harness_covers_shared_rows():
    case = _case(seed=9103, I_s=512)
    ref = oracle.forward(case, trace=True)
    gpu = _as_gpu(case, ref)
    P = ref["P"]
    bad = {k: v.copy() for k, v in gpu.items()}
    bad["acc2"][P + 1, 0] -= 1
    with pytest.raises(AssertionError, match=f"acc2 row {P + 1}"):
        compare(case, bad, ref)
