"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs, stage by stage (tolerances in gpu_util.py).

Small cases run the whole oracle (the tiny workload among them); they span
every work-item size (16-, 32- and 256-row chunks, several per expert, ragged
tails, the XCD-ordered tall items), masks, expert-parallel shares, smooth
scales, a shared expert whose intermediate differs from the routed one, the
fused route scale, requantisation in GEMM1's epilogue, seeded random shapes,
and the degenerate cases (T = 0, T = 1, every token masked, ids out of range,
duplicated ids, a token with non-finite inputs, rows at the amax floor,
exact rounding ties). The four larger workloads and
the compute-bound probe run at full size with every token through the oracle,
whose tokens are split over the host's threads. Graph replay, timing events,
dirty workspaces, shrinking batches, the cache warm and the read probe are
checked for changing nothing they should not.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_expert_ffn_route_amd as moe
import oracle
from moe_expert_ffn_route_amd import synth
from gpu_util import check, compare, grouped_row_tokens, pack_reference, run_gpu, say, with_floor_rows

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="parity", T=16, H=512, I=256, E_g=8, K=2, seed=101)
    base.update(kw)
    return synth.Spec(**base)


SMALL = {
    "cfg0_tiny": synth.WORKLOADS[0],
    "ragged_mask_smooth_shared": spec(T=37, H=768, I=512, I_s=256, E_g=16, K=4, active=29, smooth=True,
                                      share_smooth=True, seed=102),
    "ep_share_rank2": spec(T=50, H=512, I=512, E_g=32, K=6, ep_size=4, ep_rank=2, active=41, smooth=True, seed=103),
    "skew_multi_chunk": spec(T=200, H=256, I=256, E_g=8, K=2, routing="zipf", zipf_s=2.0, I_s=512, seed=104),
    "k1_single_expert": spec(T=70, H=256, I=256, E_g=1, K=1, seed=105),
    "k16": spec(T=9, H=512, I=256, E_g=16, K=16, I_s=256, seed=106),
    "t1": spec(T=1, H=1024, I=512, E_g=4, K=2, I_s=512, seed=107),
    "wide_hidden": spec(T=5, H=4096, I=256, E_g=4, K=2, I_s=256, seed=108),
    "wide_inter": spec(T=6, H=256, I=2048, E_g=4, K=2, I_s=768, seed=109),
    "t16_full_tiles": spec(T=16, H=512, I=512, E_g=2, K=2, I_s=256, seed=110),
    # more than 16 tokens with K step counts (H / 64 = 12, I / 64 = 4) that the
    # larger-batch kernel's 8-step weight ring does not divide
    "t40_short_ring": spec(T=40, H=768, I=256, E_g=4, K=2, I_s=768, seed=111),
    "t17_one_row_past_decode": spec(T=17, H=512, I=256, E_g=2, K=1, I_s=256, seed=112),
    # experts averaging 256 rows or more: every group is cut into tall work
    # items (256-row chunks, the last one ragged; rows past it repeat the
    # chunk's last row)
    "tall_ragged_shared": spec(T=300, H=512, I=256, E_g=2, K=2, I_s=256, seed=113),
    "tall_exact_one_chunk": spec(T=256, H=512, I=512, E_g=1, K=1, seed=114),
    # two full chunks of one expert; with I = 1024 a chunk has 8 groups of
    # weight tiles, so the two chunks of a group run 8 blocks apart
    "tall_two_chunks_grouped": spec(T=512, H=256, I=1024, E_g=1, K=1, I_s=256, seed=141),
    "tall_three_chunks_ragged": spec(T=700, H=512, I=256, E_g=1, K=1, seed=142),
    # the DeepSeek-V3 hidden size (H = 7168 = 28 x 256, not a power of two) on
    # each item size: decode with I = 2048, 32-row items, tall items
    "h7168_decode": spec(T=8, H=7168, I=2048, E_g=16, K=4, I_s=2048, seed=148),
    "h7168_wide": spec(T=40, H=7168, I=512, E_g=8, K=2, I_s=512, seed=149),
    "h7168_tall": spec(T=260, H=7168, I=512, E_g=1, K=1, seed=150),
    # decode batches at the production intermediate sizes (I = 1024, 2048):
    # masks, a shared expert, EP shares, smooth and fused route scales, T = 1
    # with K = 16, 16 tokens over 512 local experts with top-16 (272 chunks),
    # one expert with 16 rows, and the H = 4096 decode shape
    "dec_i1024_mask_shared": spec(T=12, H=512, I=1024, E_g=8, K=3, I_s=1024, active=9, seed=171),
    "dec_i2048_ep_smooth": spec(T=16, H=768, I=2048, E_g=32, K=6, ep_size=4, ep_rank=1, smooth=True, seed=172),
    "dec_fused_share_smooth": spec(T=8, H=512, I=1024, E_g=16, K=4, I_s=1024, fuse_route_scale=True,
                                   share_smooth=True, seed=173),
    "dec_t1_k16": spec(T=1, H=1024, I=1024, E_g=32, K=16, I_s=1024, seed=174),
    "dec_t16_k16_e512": spec(T=16, H=256, I=1024, E_g=512, K=16, seed=175),
    "dec_one_expert_16_rows": spec(T=16, H=512, I=1024, E_g=1, K=1, I_s=1024, seed=176),
    "dec_h4096": spec(T=8, H=4096, I=2048, E_g=16, K=8, I_s=2048, active=7, seed=177),
    # tall items with long contractions: GEMM1 over H = 8192 (128 stages of
    # the four-buffer copy ring), and GEMM2 over I = 4096 (its GEMM1 has 32
    # N groups; the shared expert's I_s = 512 takes a second GEMM2 launch)
    "tall_long_k_gemm1": spec(T=260, H=8192, I=512, E_g=1, K=1, seed=146),
    "tall_long_k_gemm2": spec(T=270, H=512, I=4096, E_g=1, K=1, I_s=512, seed=147),
    # XCD-ordered tall items: 4 experts of one or two ragged chunks (262, 279,
    # 244, 255 rows) and a shared expert of 3 chunks with I_s != I (a split
    # GEMM2): 36 GEMM1 items, so the first 32 are renumbered over the 8 XCDs
    # and the last 4 keep their order
    "tall_xcd_order_ragged_split": spec(T=520, H=1024, I=512, E_g=4, K=2, I_s=256, seed=145),
    "tall_mask_smooth_split_gemm2": spec(T=290, H=768, I=256, E_g=2, K=2, I_s=512, active=270, smooth=True,
                                         share_smooth=True, seed=115),
    "tall_skewed": spec(T=600, H=256, I=256, E_g=2, K=1, routing="zipf", zipf_s=2.0, I_s=256, seed=116),
    "tall_tail_two_tiles": spec(T=280, H=512, I=256, E_g=1, K=1, I_s=256, seed=117),
    # expert-parallel shares of a large batch: the item size follows the rows
    # this rank can expect (T*K / ep_rank_size), so 512 tokens over 8 experts
    # on 4 ranks take 32-row items, and 600 tokens on 1 of 2 experts tall ones
    "ep_share_t512_wide_items": spec(T=512, H=256, I=256, E_g=8, K=2, ep_size=4, ep_rank=3, I_s=256, seed=143),
    "ep_share_t600_tall_items": spec(T=600, H=256, I=256, E_g=2, K=2, ep_size=2, ep_rank=0, active=580,
                                     seed=144),
    # the routing weight folded into the GEMM2 row scale (combine only sums),
    # on each item size, with masks, an EP share, smooth scales and a split
    # GEMM2 (I_s != I)
    "fused_decode_shared_mask": spec(T=12, H=512, I=256, E_g=8, K=3, I_s=256, active=10, fuse_route_scale=True,
                                     seed=151),
    "fused_wide_ep_smooth": spec(T=60, H=512, I=256, E_g=16, K=4, ep_size=2, ep_rank=1, active=50, smooth=True,
                                 fuse_route_scale=True, seed=152),
    "fused_tall_split_gemm2": spec(T=300, H=512, I=256, E_g=2, K=2, I_s=512, fuse_route_scale=True, seed=153),
    # batches of at most 64 (token, k) pairs are routed by one wave: the
    # largest expert count (512 local experts, 8 per lane), 64 tokens of top-1
    # (32-row items, a shared expert of 64 rows in two chunks), masks, bad ids
    # and an EP share
    "wave_routing_e512_k16": spec(T=4, H=256, I=256, E_g=512, K=16, I_s=256, seed=181),
    "wave_routing_t64_k1_shared": spec(T=64, H=256, I=256, E_g=8, K=1, I_s=256, active=60, seed=182),
    "wave_routing_ep_share_mask": spec(T=21, H=512, I=256, E_g=64, K=3, ep_size=4, ep_rank=1, active=17,
                                       smooth=True, seed=183),
}


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_case_parity(name, packed):
    say(f"[parity] {name} packed={packed}: {SMALL[name]}")
    stats, _, _ = check(synth.make_case(SMALL[name]), packed=packed)
    say(f"[parity] {name}: {stats}")


# Requantisation in GEMM1's epilogue (requant_in_epilogue, decode GEMM): the
# last of a chunk's N-tile workgroups to arrive quantises the chunk's h rows.
# Cases: one chunk per expert with many N tiles, a shared expert whose
# intermediate differs (fewer arrivals for its chunk than the grid's N extent),
# masks, smooth scales, an EP share, the fused route scale, rows longer than
# the finaliser keeps in registers (I 4096 and 16384), T = 1, every token
# masked; a batch above 16 tokens (option ignored: the separate launch runs).
FIN = {
    "fin_decode_shared_mask_smooth": spec(T=12, H=512, I=512, E_g=8, K=3, I_s=256, active=10, smooth=True,
                                          share_smooth=True, requant_in_epilogue=True, seed=161),
    "fin_split_shared_larger": spec(T=16, H=768, I=256, E_g=4, K=2, I_s=768, requant_in_epilogue=True, seed=162),
    "fin_ep_share_fused": spec(T=9, H=512, I=256, E_g=32, K=6, ep_size=4, ep_rank=2, fuse_route_scale=True,
                               requant_in_epilogue=True, seed=163),
    "fin_long_rows_4096": spec(T=6, H=256, I=4096, E_g=4, K=2, I_s=2304, requant_in_epilogue=True, seed=164),
    "fin_long_rows_16384": spec(T=3, H=256, I=16384, E_g=2, K=1, I_s=512, requant_in_epilogue=True, seed=165),
    "fin_t1": spec(T=1, H=1024, I=512, E_g=4, K=2, I_s=512, requant_in_epilogue=True, seed=166),
    "fin_all_masked": spec(T=7, I_s=256, active=0, requant_in_epilogue=True, seed=167),
    "fin_ignored_above_16_tokens": spec(T=40, H=512, I=256, E_g=4, K=2, I_s=512, requant_in_epilogue=True,
                                        seed=168),
    "fin_decode_h4096": spec(T=8, H=4096, I=2048, E_g=16, K=4, I_s=2048, requant_in_epilogue=True, seed=169),
    "fin_i1024_mask": spec(T=12, H=512, I=1024, E_g=8, K=3, I_s=1024, active=9, requant_in_epilogue=True,
                               seed=170),
}


@pytest.mark.parametrize("packed", [True, False], ids=["packed", "rowmajor"])
@pytest.mark.parametrize("name", list(FIN))
def test_requant_in_epilogue_parity(name, packed):
    say(f"[parity] {name} packed={packed}: {FIN[name]}")
    case = synth.make_case(FIN[name])
    stats, gpu, ref = check(case, packed=packed)
    say(f"[parity] {name}: {stats}")
    # identical to the separate requantisation launch, bit for bit
    plain = run_gpu(dataclasses.replace(case, spec=dataclasses.replace(case.spec, requant_in_epilogue=False)),
                    packed=packed)
    for k in ("output", "share_output"):
        if gpu.get(k) is not None:
            assert np.array_equal(gpu[k], plain[k]), k
    P, Ta = int(gpu["num_rows"][0]), int(gpu["num_rows"][1])
    for r in range(P + (Ta if case.spec.I_s else 0)):  # rows in use
        n = case.spec.I if r < P else case.spec.I_s
        assert np.array_equal(gpu["q_h"][r, :n], plain["q_h"][r, :n]), f"q_h row {r}"
        assert gpu["hs"][r] == plain["hs"][r], f"hs row {r}"


# The production tile shapes (hidden 4096, intermediate 2048: one K batch per
# wave in GEMM1) at small T: 16-row chunks (T <= 16) and 32-row chunks
# (T > 16), including an expert with more than one chunk.
H4096 = {
    "h4096_t6_shared": spec(T=6, H=4096, I=2048, E_g=8, K=2, I_s=2048, seed=121),
    "h4096_mask_smooth": spec(T=10, H=4096, I=2048, E_g=4, K=2, active=7, smooth=True, seed=122),
    "h4096_mt4_shared": spec(T=40, H=4096, I=2048, E_g=4, K=2, I_s=2048, seed=123),
    "h4096_mt4_multichunk": spec(T=80, H=4096, I=2048, E_g=2, K=2, seed=124),
}


@pytest.mark.parametrize("packed", [True, False], ids=["packed", "rowmajor"])
@pytest.mark.parametrize("name", list(H4096))
def test_production_tile_parity(name, packed):
    say(f"[parity] {name} packed={packed}: {H4096[name]}")
    stats, gpu, _ = check(synth.make_case(H4096[name]), packed=packed)
    say(f"[parity] {name}: {stats}")


def _random_specs(n, seed=2024):
    """Seeded random small shapes over every option of the block: batch sizes
    on both sides of the decode / 32-row / 256-row work-item choice, hidden and
    intermediate sizes, a shared expert or none (with a differing
    intermediate), expert-parallel shares, masks, smooth scales, uniform and
    skewed routing, both weight layouts, the fused route scale."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E_g = int(rng.choice([1, 2, 4, 8, 16, 32]))
        ep = int(rng.choice([d for d in (1, 2, 4) if E_g % d == 0]))
        K = int(rng.integers(1, min(E_g, 8) + 1))
        T = int(rng.choice([1, 3, 8, 16, 17, 40, 100, 260, 300]))
        I_s = int(rng.choice([0, 256, 512]))
        kw = dict(name=f"random{i}", T=T, H=int(rng.choice([256, 512, 768, 1024])), I=int(rng.choice([256, 512])),
                  E_g=E_g, K=K, I_s=I_s, ep_size=ep, ep_rank=int(rng.integers(0, ep)),
                  routing=str(rng.choice(["uniform", "zipf"])), zipf_s=1.5, seed=200 + i)
        if rng.random() < 0.4:
            kw["active"] = int(rng.integers(0, T + 1))
        if rng.random() < 0.4:
            kw["smooth"] = True
        if I_s and rng.random() < 0.4:
            kw["share_smooth"] = True
        if rng.random() < 0.3:
            kw["fuse_route_scale"] = True
        out.append((synth.Spec(**kw), bool(i % 2)))
    # the same draws again with requantisation in GEMM1's epilogue (where it
    # applies: batches of at most 16 tokens)
    out += [(dataclasses.replace(sp, name=sp.name + "_fin", requant_in_epilogue=True), pk)
            for sp, pk in out if sp.T <= 16]
    return out


RANDOM = _random_specs(24)


@pytest.mark.parametrize("i", range(len(RANDOM)))
def test_random_shapes_parity(i):
    sp, packed = RANDOM[i]
    say(f"[parity] random {i} packed={packed}: {sp}")
    stats, _, _ = check(synth.make_case(sp), packed=packed)
    say(f"[parity] random {i}: {stats}")


@pytest.mark.parametrize("which", [1, 2], ids=["gmm1", "gmm2"])
@pytest.mark.parametrize("shape", [(1, 32, 64), (3, 96, 192), (2, 4096, 512), (1, 512, 2048)])
def test_pack_layout(shape, which):
    rng = np.random.default_rng(7)
    w = rng.integers(-127, 128, shape).astype(np.int8)
    d = moe.moe_w8a8_pack_weights(torch.from_numpy(w).cuda(), which)
    torch.cuda.synchronize()
    got = d.cpu().numpy().reshape(-1)
    assert np.array_equal(got, pack_reference(w, which))
    # spot checks straight from the header's definition: block (g, p, s), lane l, byte b
    G, n, k = shape
    for g, p, s, l, b in [(0, 0, 0, 0, 0), (G - 1, n // 16 - 1, k // 64 - 1, 63, 15), (G // 2, 1, 0, 17, 3)]:
        j = p if which == 2 else (p // 2 if p % 2 == 0 else n // 32 + p // 2)
        off = ((g * (n // 16) + p) * (k // 64) + s) * 1024 + 16 * l + b
        assert got[off] == w[g, 16 * j + l % 16, 64 * s + 16 * (l // 16) + b]


# Size limits of the C ABI: 512 local experts, top-16, hidden and intermediate
# 16384, and many routing rounds (32768 pairs); every token goes through the
# oracle.
LIMITS = {
    "e512_k16": (spec(T=64, H=256, I=256, E_g=512, K=16, I_s=256, seed=131), None),
    "hidden_16384": (spec(T=3, H=16384, I=256, E_g=4, K=2, I_s=256, seed=132), None),
    "inter_16384": (spec(T=3, H=256, I=16384, E_g=4, K=2, I_s=512, seed=133), None),
    "pairs_32768": (spec(T=2048, H=256, I=256, E_g=64, K=16, active=1900, seed=134), None),
    "t24_hidden_16384": (spec(T=24, H=16384, I=256, E_g=4, K=2, I_s=256, seed=135), None),
    "t24_inter_16384": (spec(T=24, H=256, I=16384, E_g=4, K=2, I_s=512, seed=136), None),
}


@pytest.mark.parametrize("packed", [True, False], ids=["packed", "rowmajor"])
@pytest.mark.parametrize("name", list(LIMITS))
def test_size_limits(name, packed):
    sp, tokens = LIMITS[name]
    say(f"[parity] {name} packed={packed}: {sp}")
    stats, _, _ = check(synth.make_case(sp), tokens=tokens, packed=packed)
    say(f"[parity] {name}: {stats}")


def test_zero_tokens():
    s = spec(T=0, I_s=256)
    c = synth.make_case(s)
    gpu = run_gpu(c)
    assert np.all(gpu["expert_token_nums"] == 0)
    assert gpu["num_rows"][0] == 0 and gpu["num_rows"][1] == 0


def test_all_tokens_masked():
    s = spec(T=12, I_s=256, active=0, smooth=True)
    c = synth.make_case(s)
    stats, gpu, _ = check(c)
    assert np.all(gpu["output"] == 0) and np.all(gpu["share_output"] == 0)


def test_out_of_range_ids_are_dropped_and_counted():
    c = synth.make_case(spec(T=20, E_g=8, K=3, I_s=256, seed=111))
    ids = c.expert_ids.copy()
    ids[3, 1] = -5
    ids[7, 0] = 8
    ids[11, 2] = 1 << 30
    c = dataclasses.replace(c, expert_ids=ids)
    stats, gpu, ref = check(c)
    assert gpu["num_rows"][2] == 3 == ref["n_bad"]


@pytest.mark.parametrize("T,packed,smooth", [(12, True, False), (12, False, True), (40, True, True),
                                             (40, False, False)],
                         ids=["decode", "decode_smooth_rowmajor", "wide_smooth", "wide_rowmajor"])
def test_amax_floor_rows(T, packed, smooth):
    c = synth.make_case(spec(T=T, H=512, I=256, E_g=8, K=3, I_s=256, smooth=smooth, share_smooth=smooth,
                             seed=120 + T))
    zero, tiny = [0, 5], [2, T - 1]
    c = with_floor_rows(c, zero=zero, tiny=tiny, seed=T)
    stats, gpu, ref = check(c, packed=packed)
    say(f"[parity] amax floor T={T}: {stats}")
    # every grouped row of a floored token has the scale eps / 127 in both
    # quantisations (its h is zero or about 1e-15) and, for an all-zero
    # token, zero codes
    floor = np.float32(np.float32(c.spec.eps) * np.float32(1.0 / 127.0))
    tok = grouped_row_tokens(c, ref)
    hit = [r for r in range(len(tok)) if tok[r] in zero + tiny]
    assert len(hit) >= len(zero + tiny)
    for r in hit:
        assert gpu["xs"][r] == floor, f"row {r} (token {tok[r]}): scale {gpu['xs'][r]} is not eps / 127"
        assert gpu["hs"][r] == floor, f"row {r} (token {tok[r]}): h scale {gpu['hs'][r]} is not eps / 127"
        if tok[r] in zero:
            assert not gpu["q_x"][r].any() and not gpu["q_h"][r].any()


INT8_TIES = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 6.5, 10.5, 62.5, 63.5, -0.5, -1.5, -2.5, -4.5, -63.5], np.float32)


@pytest.mark.parametrize("T", [12, 40], ids=["decode", "wide"])
def test_quant_ties_round_to_even(T):
    # a token row whose maximum is 127: (v * 127) * (1/127) is then exactly v
    # in fp32 for each v below, so every one of them is an exact tie, which
    # the quantiser rounds to even (np.rint), not away from zero
    c = synth.make_case(spec(T=T, H=512, I=256, E_g=8, K=3, I_s=256, seed=160 + T))
    t, n = 4, len(INT8_TIES)
    row = np.zeros(c.spec.H, np.float32)
    row[0], row[1:1 + n] = 127.0, INT8_TIES
    x = c.x.copy()
    x[t] = synth.f32_to_bf16_bits(row)
    c = dataclasses.replace(c, x=x)
    stats, gpu, ref = check(c)
    expect = np.rint(INT8_TIES).astype(np.int8)
    tok = grouped_row_tokens(c, ref)
    hit = [r for r in range(len(tok)) if tok[r] == t]
    assert hit
    for r in hit:
        assert gpu["q_x"][r, 0] == 127 and np.array_equal(gpu["q_x"][r, 1:1 + n], expect), f"row {r}"
        assert not gpu["q_x"][r, 1 + n:].any()


def test_duplicate_expert_in_topk():
    c = synth.make_case(spec(T=10, E_g=4, K=3, seed=112))
    ids = c.expert_ids.copy()
    ids[:, 1] = ids[:, 0]
    check(dataclasses.replace(c, expert_ids=ids))


@pytest.mark.parametrize("T,packed", [(12, True), (40, False)], ids=["decode", "wide"])
def test_non_finite_token_leaves_other_tokens_exact(T, packed):
    # a NaN and an infinity in one token's x make only that token's rows
    # unspecified: routing, and every stage of every other token, still match
    # the oracle (which is run on those tokens only)
    c = synth.make_case(spec(T=T, H=512, I=256, E_g=8, K=3, I_s=256, seed=118))
    x = c.x.copy()
    x[3, 5] = 0x7FC0   # bf16 NaN
    x[3, 17] = 0x7F80  # bf16 +inf
    others = [t for t in range(T) if t != 3]
    stats, gpu, _ = check(dataclasses.replace(c, x=x), tokens=others, packed=packed)
    assert stats["rows"] > 0


def test_deterministic_dirty_workspace_and_side_stream():
    c = synth.make_case(spec(T=33, H=512, I=512, E_g=8, K=4, I_s=256, seed=113))
    t = moe.upload(c)
    a = run_gpu(c, tensors=t)
    s = torch.cuda.Stream()
    b = run_gpu(c, tensors=t, garbage_workspace=True, stream=s)
    for k in ("output", "share_output", "expert_token_nums"):
        assert np.array_equal(a[k], b[k]), k
    # intermediates: only the defined part (rows in use; a shared row uses I_s columns)
    P, Ta = int(a["num_rows"][0]), int(a["num_rows"][1])
    for r in range(P + Ta):
        n = c.spec.I if r < P else c.spec.I_s
        for k, w in (("q_x", c.spec.H), ("acc1", 2 * n), ("h", n), ("q_h", n), ("acc2", c.spec.H)):
            assert np.array_equal(a[k][r, :w], b[k][r, :w]), (k, r)


GRAPH_CASES = {
    "decode": spec(T=12, H=512, I=256, E_g=8, K=2, I_s=256, active=10, seed=116),
    "decode_requant_in_epilogue": spec(T=12, H=512, I=256, E_g=8, K=2, I_s=512, active=10,
                                       requant_in_epilogue=True, seed=120),
    "wide": spec(T=40, H=512, I=256, E_g=8, K=2, I_s=512, active=37, seed=118),
    "tall": spec(T=300, H=512, I=256, E_g=2, K=2, I_s=256, seed=119),
}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_hip_graph_capture_and_replay(name):
    # the production path launches kernels only (no memset, no allocation), so
    # a caller can capture it; every replay must match the eager result, with
    # other eager work and synchronisations between replays (each GEMM kernel
    # family: decode, 32-row and 256-row work items)
    say(f"[graph] {name}: {GRAPH_CASES[name]}")
    c = synth.make_case(GRAPH_CASES[name])
    t = moe.pack_weights(moe.upload(c))
    dims = moe.dims_of_case(c)
    dims.weight_layout = moe.MOE_WEIGHT_PACKED
    runner = moe.Runner(dims)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        runner(t, stream=s)
    torch.cuda.synchronize()
    eager = (runner.output.clone(), runner.share_output.clone(), runner.expert_token_nums.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        runner(t, stream=s)
    for i in range(4):
        runner.output.fill_(3)
        runner.share_output.fill_(3)
        runner.expert_token_nums.fill_(-1)
        runner.workspace.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(runner.output, eager[0]), i
        assert torch.equal(runner.share_output, eager[1]), i
        assert torch.equal(runner.expert_token_nums, eager[2]), i


@pytest.mark.parametrize("I_s", [256, 512], ids=["split_gemm2", "one_gemm2"])
def test_timing_events(I_s):
    # stage events (markers between stages) and kernel events (bound to the
    # GEMM launches) leave the results unchanged; each GEMM's own duration
    # lies inside the markers around its stage
    import ctypes
    from moe_expert_ffn_route_amd import binding
    c = synth.make_case(spec(T=24, H=1024, I=512, E_g=16, K=4, I_s=I_s, seed=117))
    t = moe.pack_weights(moe.upload(c))
    dims = moe.dims_of_case(c)
    dims.weight_layout = moe.MOE_WEIGHT_PACKED
    runner = moe.Runner(dims)
    runner(t)
    torch.cuda.synchronize()
    plain = (runner.output.clone(), runner.share_output.clone())
    stage = [torch.cuda.Event(enable_timing=True) for _ in range(len(binding.STAGES) + 1)]
    kern = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in stage + kern:
        e.record()
    torch.cuda.synchronize()
    sa = (ctypes.c_void_p * len(stage))(*[e.cuda_event for e in stage])
    ka = (ctypes.c_void_p * 4)(*[e.cuda_event for e in kern])
    d = binding.Debug(stage_events=ctypes.cast(sa, ctypes.c_void_p).value,
                      kernel_events=ctypes.cast(ka, ctypes.c_void_p).value)
    runner.output.fill_(0)
    runner(t, dbg=d)
    torch.cuda.synchronize()
    assert torch.equal(runner.output, plain[0]) and torch.equal(runner.share_output, plain[1])
    g1 = binding.STAGES.index("gemm1")
    g2 = binding.STAGES.index("gemm2")
    k1, k2 = kern[0].elapsed_time(kern[1]), kern[2].elapsed_time(kern[3])
    s1, s2 = stage[g1].elapsed_time(stage[g1 + 1]), stage[g2].elapsed_time(stage[g2 + 1])
    say(f"[parity] gemm1 kernel {k1 * 1e3:.1f} us (stage {s1 * 1e3:.1f}), gemm2 {k2 * 1e3:.1f} us (stage {s2 * 1e3:.1f})")
    assert 0 < k1 <= s1 * 1.05 + 2e-3 and 0 < k2 <= s2 * 1.05 + 2e-3
    assert stage[g1].elapsed_time(kern[0]) >= -1e-3 and kern[1].elapsed_time(stage[g1 + 1]) >= -1e-3


def test_repeated_calls_shrinking_batch():
    # one workspace, a large call then a smaller one: nothing stale leaks
    big = spec(T=64, H=512, I=256, E_g=8, K=2, I_s=256, seed=114)
    small = dataclasses.replace(big, T=5, seed=115)
    cb, cs = synth.make_case(big), synth.make_case(small)
    dims_b = moe.dims_of_case(cb)
    runner = moe.Runner(dims_b)
    runner(moe.upload(cb))
    torch.cuda.synchronize()
    dims_s = moe.dims_of_case(cs)
    ts = moe.upload(cs)
    out = torch.empty((5, 512), dtype=torch.bfloat16, device="cuda")
    sout = torch.empty((5, 512), dtype=torch.bfloat16, device="cuda")
    etn = torch.empty(8, dtype=torch.int32, device="cuda")
    moe.moe_w8a8_forward(dims_s, output=out, share_output=sout, expert_token_nums=etn, workspace=runner.workspace,
                         **ts)
    torch.cuda.synchronize()
    ref = oracle.forward(cs)
    from gpu_util import out_close
    out_close(out.view(torch.int16).cpu().numpy().view(np.uint16), ref["output"], "output")
    out_close(sout.view(torch.int16).cpu().numpy().view(np.uint16), ref["share_output"], "share_output")
    assert np.array_equal(etn.cpu().numpy(), ref["expert_token_nums"])


# ------------------------------------------------------- full-size workloads

_WEIGHTS = {}


def weights_for(s):
    key = (s.weight_seed, s.H, s.I, s.E_g, s.ep_size, s.ep_rank)
    if key not in _WEIGHTS:
        say(f"[parity] generating weights {key}")
        w = synth.make_weights(s)
        _WEIGHTS.clear()
        _WEIGHTS[key] = w
    return _WEIGHTS[key]


# Every token of every workload goes through the oracle (split over the
# host's threads); 1, 3 and 4 share one set of weights. Configs 1 and 4 run
# both weight layouts against one oracle run.
FULL = (1, 2, 3, 4, 5)


@pytest.mark.parametrize("cfg", FULL)
def test_full_size_workload(cfg):
    s = synth.WORKLOADS[cfg]
    say(f"[parity] config {cfg} {s.name}: all {s.T} tokens")
    case = synth.workload_case(cfg, weights=weights_for(s))
    ref = oracle.forward(case, trace=True, threads=oracle.default_threads())
    say(f"[parity] config {cfg}: oracle done ({ref['P']} routed rows)")
    stats, gpu, _ = check(case, ref=ref, packed=True)
    say(f"[parity] config {cfg} packed: {stats}")
    if cfg in (1, 4):
        del gpu
        stats, gpu, _ = check(case, ref=ref, packed=False)
        say(f"[parity] config {cfg} row-major: {stats}")
    if cfg == 1:  # requantisation in GEMM1's epilogue
        del gpu
        fin = dataclasses.replace(case, spec=dataclasses.replace(case.spec, requant_in_epilogue=True))
        stats, gpu, _ = check(fin, ref=ref, packed=True)
        say(f"[parity] config {cfg} requant in GEMM1's epilogue: {stats}")
    assert stats["rows"] == ref["P"] + (ref["T_act"] if s.I_s else 0)
    del gpu, ref
    torch.cuda.empty_cache()


def test_cache_warm_changes_no_result():
    # the warm is a cache hint: warming the next layer's shared expert on a
    # second stream while this layer runs leaves every output bit unchanged,
    # and so does warming the weights this call is about to read
    c = synth.make_case(spec(T=8, H=1024, I=512, E_g=16, K=4, I_s=512, seed=171))
    t = moe.pack_weights(moe.upload(c))
    nxt = {k: v.clone() for k, v in t.items() if k.startswith("share_gmm") and v is not None}
    dims = moe.dims_of_case(c)
    dims.weight_layout = moe.MOE_WEIGHT_PACKED
    runner = moe.Runner(dims)
    runner(t)
    torch.cuda.synchronize()
    ref = (runner.output.clone(), runner.share_output.clone())
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    for i in range(3):
        runner.output.fill_(1)
        runner.share_output.fill_(1)
        ev = torch.cuda.Event()
        ev.record(main)
        side.wait_event(ev)
        moe.moe_w8a8_warm(nxt["share_gmm1_weight"], stream=side)
        moe.moe_w8a8_warm(t["gmm1_weight"], stream=side)
        runner(t, stream=main)
        torch.cuda.synchronize()
        assert torch.equal(runner.output, ref[0]) and torch.equal(runner.share_output, ref[1]), i
    # the warmed tensors themselves are untouched
    for k, v in nxt.items():
        assert torch.equal(v, t[k])


@pytest.mark.parametrize("nbytes", [16, 1024, 4096 + 48, 8 << 20, (64 << 20) + 16 * 37])
def test_read_probe_reads_and_changes_nothing(nbytes):
    # the bandwidth probe only reads: its range, and a guard band written
    # after it, keep every byte, for whole and ragged last wave passes
    buf = torch.randint(0, 256, (nbytes + 4096,), dtype=torch.uint8, device="cuda")
    ref = buf.clone()
    for _ in range(2):
        moe.moe_w8a8_read_probe(buf, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)


@pytest.mark.parametrize("items,dst_bytes", [(1, 0), (1, 4096), (16, 48 * 1024 + 16 * 7), (64, 1 << 20)])
def test_read_write_probe_writes_only_its_range(items, dst_bytes):
    # the read-and-write probe leaves its source unchanged and writes nothing
    # outside [dst, dst + dst_bytes): the guard band after the range keeps
    # every byte, also when the range does not split evenly over the items
    src_bytes = items * 256 * 1024
    src = torch.randint(0, 256, (src_bytes,), dtype=torch.uint8, device="cuda")
    dst = torch.randint(0, 256, (dst_bytes + 8192,), dtype=torch.uint8, device="cuda")
    src_ref, guard = src.clone(), dst[dst_bytes:].clone()
    for _ in range(2):
        moe.moe_w8a8_read_write_probe(src, src_bytes, dst, dst_bytes)
    torch.cuda.synchronize()
    assert torch.equal(src, src_ref)
    assert torch.equal(dst[dst_bytes:], guard)
