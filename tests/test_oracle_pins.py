"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each `pin_*` function checks the oracle against a closed form, an invariant,
a special case that reduces to a textbook routine (numpy sort / integer
matmul, torch's SiLU in float64), an exact scaling law, or brute force on a
tiny input. They are plain functions so that test_oracle_mutants.py can run
them against deliberately broken copies of the oracle.

Sources: "FusedDeepMoE Kernel 深度分析报告" (sec. 1.2 signature, 4.1 dispatch,
4.2 combine, 6.1/6.2 epilogues, 7.2 BlockQuant, 9.1 math correspondence) and
"DeepSeek V4 Decode Optimization" sec. 0 (W8A8 contract; symmetric per-token
int8 quantisation is invariant to a positive scalar) and sec. 3.1 (group-wise
amax).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from moe_expert_ffn_route_amd import synth

F32 = synth.bf16_bits_to_f32


def small_spec(**kw):
    base = dict(name="pin", T=6, H=128, I=48, E_g=6, K=2, seed=77)
    base.update(kw)
    return synth.Spec(**base)


def run(case, **kw):
    return oracle.forward(case, **kw)


# ---------------------------------------------------------------- routing


def _route_bruteforce(ids, mask, E_g, ep_size, ep_rank):
    """Grouping by a comparison sort on (expert, pair id): numpy lexsort."""
    T, K = ids.shape
    E = E_g // ep_size
    p = np.arange(T * K)
    t = p // K
    g = ids.reshape(-1).astype(np.int64)
    act = np.ones(T * K, bool) if mask is None else mask[t].astype(bool)
    bad = act & ((g < 0) | (g >= E_g))
    e = g - ep_rank * E
    keep = act & ~bad & (e >= 0) & (e < E)
    kp, ke = p[keep], e[keep]
    order = kp[np.lexsort((kp, ke))]
    counts = np.bincount(ke, minlength=E).astype(np.int32)
    rop = np.full(T * K, -1, np.int32)
    rop[order] = np.arange(len(order), dtype=np.int32)
    return counts, order.astype(np.int32), rop, int(bad.sum())


def pin_route_bruteforce():
    rng = np.random.default_rng(5)
    cases = []
    for T, K, E_g, ep in [(0, 3, 8, 1), (1, 1, 1, 1), (1, 4, 8, 2), (13, 3, 16, 4), (64, 8, 256, 16),
                          (37, 6, 12, 3), (200, 8, 64, 1)]:
        ids = rng.integers(-2, E_g + 2, (T, K)).astype(np.int32)      # out-of-range and duplicates
        mask = (rng.random(T) < 0.7).astype(np.uint8) if T > 3 else None
        for r in range(ep):
            cases.append((ids, mask, E_g, ep, r))
    for ids, mask, E_g, ep, r in cases:
        T, K = ids.shape
        d = oracle.dims_of(T, 64, 64, K, E_g, 0, ep, r)
        got = oracle.route(d, ids, mask)
        counts, order, rop, bad = _route_bruteforce(ids, mask, E_g, ep, r)
        assert np.array_equal(got["counts"], counts)
        assert np.array_equal(got["sorted_pair"], order)
        assert np.array_equal(got["row_of_pair"], rop)
        assert got["n_bad"] == bad
        assert np.array_equal(got["offsets"], np.concatenate([[0], np.cumsum(counts)]))


def pin_route_count_invariant():
    # sum(expert_token_nums) = active tokens x top-k when every expert is local
    for i, spec in synth.WORKLOADS.items():
        x, ids, esc, mask, _, _ = synth.make_activations(spec)
        d = oracle.dims_of(spec.T, spec.H, spec.I, spec.K, spec.E_g, spec.I_s, spec.ep_size, spec.ep_rank)
        got = oracle.route(d, ids, mask)
        n_act = spec.T if mask is None else int(mask.sum())
        if spec.ep_size == 1:
            assert got["counts"].sum() == n_act * spec.K
        else:
            act = np.ones(spec.T, bool) if mask is None else mask.astype(bool)
            lo = spec.ep_rank * spec.E_loc
            local = (ids >= lo) & (ids < lo + spec.E_loc) & act[:, None]
            assert got["counts"].sum() == local.sum()
        # K distinct experts per token: no expert sees one token twice
        assert all(len(set(r)) == spec.K for r in ids.tolist())


# ----------------------------------------------------------- quantisation


def pin_quant_closed_forms():
    rng = np.random.default_rng(11)
    inv127 = np.float32(1) / np.float32(127)
    for n in (1, 7, 64, 512, 4096):
        v = rng.standard_normal(n).astype(np.float32) * np.float32(rng.uniform(0.01, 100))
        q, s = oracle.quant_row(v)
        i = int(np.argmax(np.abs(v)))
        assert q[i] == (127 if v[i] > 0 else -127)           # the row maximum maps to +-127
        assert s == np.float32(np.float32(np.abs(v).max()) * inv127)
        assert np.all(np.abs(q.astype(int)) <= 127)
        # rounding error bound: |q - v*127/a| <= 1/2 (+ fp32 slack)
        exact = v.astype(np.float64) * 127.0 / np.float64(np.abs(v).max())
        assert np.all(np.abs(q - exact) <= 0.5 + 1e-4)
        # symmetric: quant(-v) = -quant(v), same scale
        q2, s2 = oracle.quant_row(-v)
        assert np.array_equal(q2, -q) and s2 == s


def _tie_row():
    """A row with maximum 128 (so 1/max is exact) whose other entries land
    exactly on k + 1/2 after the x127 / max scaling."""
    vals, want = [np.float32(128)], [127]
    for m in range(-120, 120):
        v = np.float32(np.float32(128 * m + 64) / np.float32(127))
        if np.float32(v * np.float32(127)) == np.float32(128 * m + 64):
            vals.append(v)
            want.append(m if m % 2 == 0 else m + 1)      # ties to even
    return np.array(vals, np.float32), np.array(want, np.int8)


def pin_quant_ties_to_even():
    # CAST_RINT (FusedDeepMoE sec. 7.2): round to nearest, ties to even
    v, want = _tie_row()
    assert len(v) > 40
    q, s = oracle.quant_row(v)
    assert np.array_equal(q, want)


def pin_quant_zero_and_eps():
    eps = np.float32(1e-6)
    q, s = oracle.quant_row(np.zeros(33, np.float32), float(eps))
    assert np.all(q == 0)
    assert s == np.float32(eps * (np.float32(1) / np.float32(127)))
    # a row below the floor is scaled by eps, not by its own maximum
    v = np.array([2e-7, -1e-7, 0.0, 5e-8], np.float32)
    q, s = oracle.quant_row(v, float(eps))
    assert s == np.float32(eps * (np.float32(1) / np.float32(127)))
    assert np.array_equal(q, np.rint(v.astype(np.float64) * 127 / 1e-6).astype(np.int8))


def pin_quant_integer_rows():
    # integer rows whose maximum is 127 are reproduced exactly with scale 1
    rng = np.random.default_rng(12)
    for n in (2, 100, 1024):
        v = rng.integers(-127, 128, n).astype(np.float32)
        v[rng.integers(0, n)] = 127 * rng.choice([-1, 1])
        q, s = oracle.quant_row(v)
        assert np.array_equal(q.astype(np.float32), v)
        assert s == np.float32(1.0)


def pin_quant_pow2_invariance():
    # a positive scalar leaves the code unchanged; a power of two scales the
    # scale exactly ("DeepSeek V4 Decode Optimization", sec. 0 / 2.5)
    rng = np.random.default_rng(13)
    v = rng.standard_normal(777).astype(np.float32)
    q0, s0 = oracle.quant_row(v)
    for j in (-12, -3, -1, 1, 4, 20):
        q, s = oracle.quant_row(v * np.float32(2.0 ** j))
        assert np.array_equal(q, q0)
        assert s == np.float32(s0 * np.float32(2.0 ** j))


# ----------------------------------------------------------------- GEMMs


def pin_gemm_exact():
    rng = np.random.default_rng(14)
    for M, N, Kd in ((1, 1, 1), (5, 7, 300), (16, 33, 4096), (3, 2, 64)):
        A = rng.integers(-127, 128, (M, Kd)).astype(np.int8)
        B = rng.integers(-127, 128, (N, Kd)).astype(np.int8)
        C = oracle.gemm_i8(A, B)
        assert np.array_equal(C, A.astype(np.int64) @ B.astype(np.int64).T)
    A = np.full((2, 4096), -127, np.int8)
    C = oracle.gemm_i8(A, A)
    assert np.all(C == 4096 * 127 * 127)


# --------------------------------------------------------------- SwiGLU


def pin_swiglu_vs_torch():
    rng = np.random.default_rng(15)
    n = 4000
    y = (rng.standard_normal(2 * n) * 6).astype(np.float32)
    y[:8] = [0.0, -0.0, 80.0, -80.0, 1e-30, -1e-30, 20.0, -20.0]
    h = oracle.swiglu(y)
    t = torch.from_numpy(y.astype(np.float64))
    ref = (torch.nn.functional.silu(t[:n]) * t[n:]).numpy()
    assert np.all(np.abs(h - ref) <= 1e-6 * np.abs(ref) + 1e-37)


# --------------------------------------------- whole block: special cases


def _dense_case(T=6, H=128, I=48, seed=3, w1_pow=-18, w2_pow=-10):
    """One expert, top-1, routing weight 1, power-of-two scales, integer x rows
    with |max| = 127: q_x = x and xs = 1 exactly, so the block must equal the
    plain dense SwiGLU FFN up to the requantisation of h and the bf16 casts."""
    rng = np.random.default_rng(seed)
    spec = small_spec(T=T, H=H, I=I, E_g=1, K=1)
    xi = rng.integers(-127, 128, (T, H)).astype(np.float32)
    xi[np.arange(T), rng.integers(0, H, T)] = 127 * rng.choice([-1, 1], T)
    w1 = rng.integers(-127, 128, (1, 2 * I, H)).astype(np.int8)
    w2 = rng.integers(-127, 128, (1, H, I)).astype(np.int8)
    case = synth.Case(spec, synth.f32_to_bf16_bits(xi), np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32),
                      w1, np.full((1, 2 * I), 2.0 ** w1_pow, np.float32), w2,
                      np.full((1, H), 2.0 ** w2_pow, np.float32))
    return case, xi


def pin_dense_swiglu_ffn():
    for T, H, I in ((6, 128, 48), (3, 64, 96)):
        case, xi = _dense_case(T, H, I)
        res = run(case, trace=True)
        W1 = torch.from_numpy(case.w1[0].astype(np.float64)) * case.w1s[0, 0].item()
        W2 = torch.from_numpy(case.w2[0].astype(np.float64)) * case.w2s[0, 0].item()
        x = torch.from_numpy(xi.astype(np.float64))
        y = x @ W1.T
        href = torch.nn.functional.silu(y[:, :I]) * y[:, I:]
        ref = (href @ W2.T).numpy()
        out = F32(res["output"]).astype(np.float64)
        hs = res["hs"][:T].astype(np.float64)
        # |q_h*hs - h| <= hs/2 per element, plus fp32 rounding of h; bf16 half-ulp of the output
        bound = (np.abs(case.w2[0]).astype(np.float64).sum(1)[None, :] * case.w2s[0, 0]
                 * (0.5 * hs[:, None] + 1e-6 * np.abs(href.numpy()).max(1, keepdims=True))
                 + 2.0 ** -8 * np.abs(ref) + 1e-30)
        assert np.all(np.abs(out - ref) <= bound)
        # and the first stages are exact: q_x = x, xs = 1, acc1 = x W1^T
        assert np.array_equal(res["q_x"][:T].astype(np.float32), xi)
        assert np.all(res["xs"][:T] == 1.0)
        assert np.array_equal(res["acc1"][:T, :2 * I],
                              (xi.astype(np.int64) @ case.w1[0].astype(np.int64).T))


def _case(**kw):
    spec = small_spec(**kw)
    return synth.make_case(spec)


def _replace(case, **kw):
    return dataclasses.replace(case, **kw)


def pin_scale_linearity():
    c = _case(T=5, E_g=4, K=2, I_s=32)
    base = run(c)
    o0, s0 = F32(base["output"]), F32(base["share_output"])
    p8 = np.float32(8.0)
    # GEMM2 weight scales x 8 -> output x 8 (exact)
    r = run(_replace(c, w2s=c.w2s * p8, sw2s=c.sw2s * p8))
    assert np.array_equal(F32(r["output"]), o0 * p8) and np.array_equal(F32(r["share_output"]), s0 * p8)
    # up-half GEMM1 scales x 1/4 -> h x 1/4: q_h unchanged, output x 1/4
    w1s = c.w1s.copy()
    w1s[:, c.spec.I:] *= np.float32(0.25)
    r = run(_replace(c, w1s=w1s), trace=True)
    rb = run(c, trace=True)
    assert np.array_equal(r["q_h"], rb["q_h"])
    assert np.array_equal(F32(r["output"]), o0 * np.float32(0.25))
    # routing weights x 32 -> output x 32, shared output unchanged
    r = run(_replace(c, expert_scales=c.expert_scales * np.float32(32)))
    assert np.array_equal(F32(r["output"]), o0 * np.float32(32)) and np.array_equal(F32(r["share_output"]), s0)
    # negating the down projection negates the output
    r = run(_replace(c, w2=-c.w2, sw2=-c.sw2))
    assert np.array_equal(F32(r["output"]), -o0) and np.array_equal(F32(r["share_output"]), -s0)
    # the gate half is not linear: scaling it must change the result
    w1s = c.w1s.copy()
    w1s[:, : c.spec.I] *= np.float32(0.25)
    r = run(_replace(c, w1s=w1s))
    assert not np.array_equal(F32(r["output"]), o0 * np.float32(0.25))


def pin_permutation_invariance():
    c = _case(T=7, E_g=6, K=3, I_s=32)
    base = run(c)
    rng = np.random.default_rng(21)
    pi = rng.permutation(6)                    # expert e is renamed pi[e]
    inv = np.argsort(pi)
    c2 = _replace(c, expert_ids=pi[c.expert_ids].astype(np.int32), w1=c.w1[inv], w1s=c.w1s[inv],
                  w2=c.w2[inv], w2s=c.w2s[inv])
    r = run(c2)
    assert np.array_equal(r["output"], base["output"]) and np.array_equal(r["share_output"], base["share_output"])
    assert np.array_equal(r["expert_token_nums"][pi], base["expert_token_nums"])
    sg = rng.permutation(7)                    # token permutation
    c3 = _replace(c, x=c.x[sg], expert_ids=c.expert_ids[sg], expert_scales=c.expert_scales[sg])
    r = run(c3)
    assert np.array_equal(r["output"], base["output"][sg]) and np.array_equal(r["share_output"], base["share_output"][sg])


def pin_combine():
    # top-1 with weight 1: the output row is the expert's bf16 row itself
    c = _case(T=5, E_g=3, K=1)
    c = _replace(c, expert_scales=np.ones((5, 1), np.float32))
    r = run(c, trace=True)
    assert np.array_equal(r["output"], r["z"][r["row_of_pair"]])
    # top-4: the fp32 sum of weighted bf16 rows, within fp32 + one bf16 rounding
    c = _case(T=9, E_g=8, K=4)
    r = run(c, trace=True)
    z = F32(r["z"][r["row_of_pair"].reshape(9, 4)]).astype(np.float64)      # [T, K, H]
    w = c.expert_scales.astype(np.float64)[:, :, None]
    ref = (z * w).sum(1)
    bound = 2.0 ** -8 * np.abs(ref) + 4 * 2.0 ** -24 * np.abs(z * w).sum(1) + 1e-30
    assert np.all(np.abs(F32(r["output"]) - ref) <= bound)


def _bf16_rne(v32):
    """float32 -> bf16 bits, round to nearest even, through torch."""
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def pin_fused_route_scale():
    # "DeepSeek V4 Decode Optimization" sec. 2.3: the routing weight folded
    # into the GEMM2 row scale, combine only sums
    spec = small_spec(T=9, E_g=8, K=3, I_s=32, active=7, wseed=11)
    fused = dataclasses.replace(spec, fuse_route_scale=True)
    # (a) with unit weights the fused path is the plain path, bit for bit
    c1 = _replace(synth.make_case(spec), expert_scales=np.ones((9, 3), np.float32))
    c1f = _replace(synth.make_case(fused), expert_scales=np.ones((9, 3), np.float32))
    a, b = run(c1, trace=True), run(c1f, trace=True)
    assert np.array_equal(a["output"], b["output"]) and np.array_equal(a["z"], b["z"])
    assert np.array_equal(a["share_output"], b["share_output"])
    # (b) power-of-two weights scale the output exactly
    cf = synth.make_case(fused)
    r = run(cf, trace=True)
    r4 = run(_replace(cf, expert_scales=cf.expert_scales * np.float32(4.0)))
    assert np.array_equal(F32(r4["output"]), F32(r["output"]) * 4.0)
    assert np.array_equal(r4["share_output"], r["share_output"])
    # (c) each routed row's bf16 output is rounded from acc2 * w2s scaled by
    #     hs times the weight of that row's own (token, k) pair; torch rounds
    P = r["P"]
    w_pair = cf.expert_scales.reshape(-1)[r["sorted_pair"]].astype(np.float32)        # [P]
    e_row = np.repeat(np.arange(cf.spec.E_loc), r["expert_token_nums"])              # [P]
    y = r["acc2"][:P].astype(np.float32) * cf.w2s[e_row]
    y = y * (r["hs"][:P] * w_pair)[:, None]
    assert np.array_equal(r["z"][:P], _bf16_rne(y))
    # (d) each output is the plain fp32 sum over k of those rows
    zr = F32(r["z"][r["row_of_pair"].reshape(9, 3)]).astype(np.float64)
    zr[r["row_of_pair"].reshape(9, 3) < 0] = 0.0
    ref = zr.sum(1)
    bound = 2.0 ** -8 * np.abs(ref) + 4 * 2.0 ** -24 * np.abs(zr).sum(1) + 1e-30
    assert np.all(np.abs(F32(r["output"]) - ref) <= bound)


# -------------------------------------------- FP4 weights / FP8 activations
# OCP microscaling formats: E4M3 activations (torch.float8_e4m3fn is the
# reference), E2M1 weights (the spec's value table), E8M0 block scales 2^(e-127).

E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3_torch(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def pin_e4m3_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_to_f32(codes), _e4m3_torch(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # encoding: random values, exact ties, subnormals and the top of the range
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(4000).astype(np.float32) * np.float32(30),
                        rng.uniform(-2e-3, 2e-3, 1000).astype(np.float32),
                        (ref[ok][:-1] + np.diff(ref[ok])) / 2,           # midpoints of neighbouring codes
                        np.float32([448, -448, 463.9, 464, -464, 0.0, -0.0, 2 ** -10, 3 * 2 ** -10])]).astype(
        np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 464)]
    ours = oracle.f32_to_e4m3(v)
    tref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(_e4m3_torch(ours), _e4m3_torch(tref))
    # beyond the range the quantiser saturates
    assert np.array_equal(oracle.f32_to_e4m3(np.float32([500, -1e6])), np.uint8([0x7E, 0xFE]))


def pin_e2m1_values():
    vals = oracle.e2m1_to_f32(np.arange(16, dtype=np.uint8))
    assert np.array_equal(vals[:8], np.float32(E2M1_VALUES))
    assert np.array_equal(vals[8:], -np.float32(E2M1_VALUES))


def pin_fp8_quant_rules():
    rng = np.random.default_rng(8)
    v = rng.standard_normal(256).astype(np.float32)
    q, sc = oracle.quant_row_fp8(v)
    i = int(np.argmax(np.abs(v)))
    assert _e4m3_torch(q[i:i + 1])[0] == np.float32(448.0) * np.sign(v[i])
    assert np.float32(sc) == np.float32(np.float32(np.abs(v).max()) * np.float32(1.0 / 448.0))
    # every code is the nearest E4M3 value to v * 448 / amax (torch rounds)
    t = (v * np.float32(448.0)) * (np.float32(1.0) / np.float32(np.abs(v).max()))
    assert np.array_equal(_e4m3_torch(q), torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).float().numpy())
    # a power-of-two rescale leaves the codes and scales the row scale exactly
    q4, sc4 = oracle.quant_row_fp8(v * np.float32(4.0))
    assert np.array_equal(q4, q) and sc4 == sc * 4
    # an all-zero row: zero codes, scale eps / 448
    qz, scz = oracle.quant_row_fp8(np.zeros(64, np.float32), eps=1e-6)
    assert not qz.any() and np.float32(scz) == np.float32(np.float32(1e-6) * np.float32(1.0 / 448.0))


def pin_gemm_mx_exact():
    # every product and partial sum here is exact in float64, so numpy's
    # matmul of the decoded operands, rounded once to fp32, is the exact result
    rng = np.random.default_rng(9)
    M, N, K = 5, 24, 256
    A = rng.integers(0, 256, (M, K), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x3C                      # no NaN codes
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    S = rng.integers(120, 135, (N, K // 32), dtype=np.uint8)
    a = _e4m3_torch(A).astype(np.float64)
    nib = np.empty((N, K), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = B & 15, B >> 4        # element 2j in the low nibble
    table = np.array(E2M1_VALUES + [-x for x in E2M1_VALUES])
    b = table[nib] * np.repeat(2.0 ** (S.astype(np.float64) - 127), 32, axis=1)
    ref = (a @ b.T).astype(np.float32)
    assert np.array_equal(oracle.gemm_mx(A, B, S), ref)


def pin_mx_block_scale_linearity():
    # the up half's block scales + 1: h doubles, so the FP8 codes of h stay and
    # its row scale, every z row and the output double exactly
    spec = small_spec(T=7, H=128, I=64, E_g=4, K=2, I_s=64, weight_format="mxfp4", wseed=21)
    c = synth.make_case(spec)
    r = run(c, trace=True)
    w1b = c.w1b.copy()
    w1b[:, spec.I:] += 1
    sw1b = c.sw1b.copy()
    sw1b[spec.I_s:] += 1
    r2 = run(_replace(c, w1b=w1b, sw1b=sw1b), trace=True)
    rows = np.concatenate([np.arange(r["P"]), r["P"] + np.arange(r["T_act"])])
    assert np.array_equal(r2["q_h"][rows], r["q_h"][rows]) and np.array_equal(r2["hs"][rows], r["hs"][rows] * 2)
    assert np.array_equal(F32(r2["output"]), F32(r["output"]) * 2)
    assert np.array_equal(F32(r2["share_output"]), F32(r["share_output"]) * 2)
    # GEMM2's block scales + 1: its accumulators and outputs double
    r3 = run(_replace(c, w2b=c.w2b + 1, sw2b=c.sw2b + 1), trace=True)
    assert np.array_equal(r3["acc2"][rows], r["acc2"][rows] * 2)
    assert np.array_equal(F32(r3["output"]), F32(r["output"]) * 2)


def pin_mx_forward_stages():
    # the traced stages of a whole FP4-weight block agree with the helpers
    # pinned above, applied row by row in numpy
    spec = small_spec(T=6, H=128, I=64, E_g=3, K=2, I_s=64, weight_format="mxfp4", smooth=True, wseed=22)
    c = synth.make_case(spec)
    r = run(c, trace=True)
    e_row = np.repeat(np.arange(spec.E_loc), r["expert_token_nums"])
    for row in range(r["P"]):
        t = r["sorted_pair"][row] // spec.K
        v = F32(c.x[t]) * c.smooth[e_row[row]]
        q, sc = oracle.quant_row_fp8(v)
        assert np.array_equal(r["q_x"][row], q) and np.float32(r["xs"][row]) == np.float32(sc)
        acc = oracle.gemm_mx(q[None], c.w1[e_row[row]], c.w1b[e_row[row]])[0]
        assert np.array_equal(r["acc1"][row, :2 * spec.I], acc)


def pin_mask_and_ep_share():
    spec = small_spec(T=10, E_g=8, K=3, I_s=32, active=6, wseed=5)
    c = synth.make_case(spec)
    r = run(c, trace=True)
    off = c.mask == 0
    assert np.all(r["output"][off] == 0) and np.all(r["share_output"][off] == 0)
    assert r["expert_token_nums"].sum() == 6 * 3
    # active rows do not depend on the other tokens being masked
    full = run(_replace(c, mask=None))
    on = ~off
    assert np.array_equal(r["output"][on], full["output"][on])
    assert np.array_equal(r["share_output"][on], full["share_output"][on])
    # expert-parallel share: each rank keeps only its local pairs; every kept
    # pair's bf16 row equals the one computed with all experts local
    ft = run(_replace(c, mask=None), trace=True)
    parts = []
    for rank in range(2):
        sp = dataclasses.replace(spec, ep_size=2, ep_rank=rank, I_s=0, active=None)
        w = synth.make_weights(sp)
        cr = synth.Case(sp, c.x, c.expert_ids, c.expert_scales, *w)
        rr = run(cr, trace=True)
        kept = rr["row_of_pair"] >= 0
        assert np.array_equal(kept, (c.expert_ids.reshape(-1) // 4) == rank)
        assert np.array_equal(rr["z"][rr["row_of_pair"][kept]], ft["z"][ft["row_of_pair"][kept]])
        parts.append(F32(rr["output"]).astype(np.float64))
    tot = parts[0] + parts[1]
    ref = F32(ft["output"]).astype(np.float64)
    assert np.all(np.abs(tot - ref) <= 2.0 ** -7 * (np.abs(parts[0]) + np.abs(parts[1])) + 1e-30)


def pin_shared_matches_routed():
    # a shared expert with expert 0's weights reproduces expert 0's rows
    c = _case(T=6, E_g=3, K=2)
    c = _replace(c, spec=dataclasses.replace(c.spec, I_s=c.spec.I),
                 sw1=c.w1[0].copy(), sw1s=c.w1s[0].copy(), sw2=c.w2[0].copy(), sw2s=c.w2s[0].copy())
    r = run(c, trace=True)
    t, k = np.nonzero(c.expert_ids == 0)
    assert len(t) > 0
    rows = r["row_of_pair"][t * 2 + k]
    assert np.array_equal(r["share_output"][t], r["z"][rows])


def pin_smooth_scales():
    c = _case(T=6, E_g=4, K=2, I_s=32)
    base = run(c, trace=True)
    ones = np.ones((4, c.spec.H), np.float32)
    r = run(_replace(c, smooth=ones, share_smooth=np.ones(c.spec.H, np.float32)))
    assert np.array_equal(r["output"], base["output"]) and np.array_equal(r["share_output"], base["share_output"])
    # expert e's smooth row 2^j_e: codes unchanged, scale x 2^j_e, for the rows of expert e only
    j = np.array([-2, 1, 3, 0])
    sm = np.repeat((2.0 ** j).astype(np.float32)[:, None], c.spec.H, 1)
    r = run(_replace(c, smooth=sm), trace=True)
    P = base["P"]
    assert np.array_equal(r["q_x"][:P], base["q_x"][:P])
    e_of_row = np.repeat(np.arange(4), base["expert_token_nums"])
    assert np.array_equal(r["xs"][:P], base["xs"][:P] * (2.0 ** j[e_of_row]).astype(np.float32))
    # shared rows unaffected by the routed smooth scales
    Ta = base["T_act"]
    assert np.array_equal(r["q_x"][P:P + Ta], base["q_x"][P:P + Ta])
    assert np.array_equal(r["xs"][P:P + Ta], base["xs"][P:P + Ta])


def pin_subset_and_empty():
    c = _case(T=8, E_g=5, K=2, I_s=32)
    full = run(c)
    r = run(c, tokens=[6, 1, 3])
    for t in (6, 1, 3):
        assert np.array_equal(r["output"][t], full["output"][t])
        assert np.array_equal(r["share_output"][t], full["share_output"][t])
    c0 = _case(T=0, E_g=5, K=2, I_s=32)
    r = run(c0)
    assert r["output"].shape == (0, c0.spec.H) and np.all(r["expert_token_nums"] == 0)


# ------------------------------------------------ group-wise activation scales
# "DeepSeek V4 Decode Optimization" sec. 3.1: the amax narrowed from per row to
# per row and group, each group's INT32 partial dequantised by its own scale.


def pin_group_quant_closed_forms():
    rng = np.random.default_rng(31)
    G = 64
    v = rng.standard_normal(4 * G).astype(np.float32)
    v[G + 5] = 40.0                      # an outlier in group 1
    v[3 * G:] = 0.0                      # an all-zero group 3
    q, s = oracle.quant_row_groups(v, G, eps=1e-6)
    inv127 = np.float32(1.0) / np.float32(127.0)
    for g in range(4):
        vg, qg = v[g * G:(g + 1) * G], q[g * G:(g + 1) * G].astype(np.float64)
        a = max(np.float32(np.abs(vg).max()), np.float32(1e-6))
        assert s[g] == np.float32(a * inv127)                     # scale = a' * fl(1/127), per group
        if g < 3:
            assert abs(qg[int(np.argmax(np.abs(vg)))]) == 127     # the group max maps to +-127
        assert np.all(np.abs(qg * a / 127.0 - vg) <= a / 254.0 * (1 + 1e-6))  # half a step of its own group
    assert not q[3 * G:].any()
    # the outlier coarsens only its own group: the other groups' codes and
    # scales are those of the same row without it
    w = v.copy()
    w[G + 5] = 0.5
    q2, s2 = oracle.quant_row_groups(w, G, eps=1e-6)
    for g in (0, 2, 3):
        assert s2[g] == s[g] and np.array_equal(q2[g * G:(g + 1) * G], q[g * G:(g + 1) * G])
    assert s[1] > 5 * s2[1]


def pin_group_gemm_vs_float64():
    # each group's exact partial, dequantised by its own scale, summed: float64
    # sums of numpy integer matmuls bound the fp32 result
    rng = np.random.default_rng(32)
    G, K, N = 64, 512, 40
    a = rng.integers(-127, 128, K).astype(np.int8)
    B = rng.integers(-127, 128, (N, K)).astype(np.int8)
    a_sc = rng.uniform(1e-3, 1e-1, K // G).astype(np.float32)   # very different scales per group
    ws = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    y = oracle.gemm_i8_groups(a, a_sc, B, ws, G).astype(np.float64)
    parts = np.stack([(B[:, g * G:(g + 1) * G].astype(np.int64) @ a[g * G:(g + 1) * G].astype(np.int64))
                      for g in range(K // G)], axis=1).astype(np.float64)
    terms = parts * ws[:, None].astype(np.float64) * a_sc[None, :].astype(np.float64)
    ref = terms.sum(axis=1)
    bound = 3 * (K // G) * 2.0 ** -24 * np.abs(terms).sum(axis=1)
    assert np.all(np.abs(y - ref) <= bound)
    # one group alone: exactly the per-row dequant of its partial
    y1 = oracle.gemm_i8_groups(a[:G], a_sc[:1], B[:, :G].copy(), ws, G)
    assert np.array_equal(y1, (parts[:, 0].astype(np.float32) * ws) * a_sc[0])


def pin_group_single_group_is_row_mode():
    # a group spanning the whole row is the per-row mode, bit for bit; the
    # fp32 GEMM dumps then equal the per-row dequant of the int32 accumulators
    spec = small_spec(T=6, H=128, I=128, E_g=4, K=2, I_s=128, smooth=True, active=5, wseed=23)
    c = synth.make_case(spec)
    r1 = run(c, trace=True)
    r2 = run(_replace(c, spec=dataclasses.replace(spec, quant_group=128)), trace=True)
    for k in ("output", "share_output", "expert_token_nums"):
        assert np.array_equal(r2[k], r1[k]), k
    rows = np.concatenate([np.arange(r1["P"]), r1["P"] + np.arange(r1["T_act"])])
    for k in ("q_x", "q_h", "h", "z"):
        assert np.array_equal(r2[k][rows], r1[k][rows]), k
    assert np.array_equal(r2["xs"][rows, 0], r1["xs"][rows]) and np.array_equal(r2["hs"][rows, 0], r1["hs"][rows])
    e_row = np.repeat(np.arange(spec.E_loc), r1["expert_token_nums"])
    for row in range(r1["P"]):
        y = (r1["acc1"][row, :2 * spec.I].astype(np.float32) * c.w1s[e_row[row]]) * r1["xs"][row]
        assert np.array_equal(r2["acc1"][row, :2 * spec.I], y)


def pin_group_outlier_resolution():
    # one token with a large outlier: with 64-element groups only the outlier's
    # group loses resolution, so GEMM1's dequantised output stays about
    # sqrt(H / 64) = 4 times closer to the float64 product than with one scale
    # per row (the quantisation error of x is all that differs)
    spec = small_spec(T=1, H=1024, I=128, E_g=1, K=1, wseed=24)
    c = synth.make_case(spec)
    x = F32(c.x).copy()
    x[0, 7] = 200.0
    c = _replace(c, x=synth.f32_to_bf16_bits(x))
    y = (c.w1[0].astype(np.float64) @ F32(c.x).astype(np.float64)[0]) * c.w1s[0]
    r0 = run(c, trace=True)
    y0 = (r0["acc1"][0, :2 * spec.I].astype(np.float32) * c.w1s[0]) * r0["xs"][0]
    r1 = run(_replace(c, spec=dataclasses.replace(spec, quant_group=64)), trace=True)
    y1 = r1["acc1"][0, :2 * spec.I]
    e0, e1 = (np.linalg.norm(v.astype(np.float64) - y) / np.linalg.norm(y) for v in (y0, y1))
    assert e1 < 0.03 and e0 > 3 * e1, (e0, e1)


PINS = [pin_route_bruteforce, pin_route_count_invariant, pin_quant_closed_forms, pin_quant_ties_to_even, pin_quant_zero_and_eps,
        pin_quant_integer_rows, pin_quant_pow2_invariance, pin_gemm_exact, pin_swiglu_vs_torch,
        pin_dense_swiglu_ffn, pin_scale_linearity, pin_permutation_invariance, pin_combine,
        pin_mask_and_ep_share, pin_shared_matches_routed, pin_smooth_scales, pin_subset_and_empty,
        pin_fused_route_scale, pin_e4m3_codes_vs_torch, pin_e2m1_values, pin_fp8_quant_rules, pin_gemm_mx_exact,
        pin_mx_block_scale_linearity, pin_mx_forward_stages, pin_group_quant_closed_forms, pin_group_gemm_vs_float64,
        pin_group_single_group_is_row_mode, pin_group_outlier_resolution]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
