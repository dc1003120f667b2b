"""GPU parity of the FP4-weight / FP8-activation variant (weight_format
MOE_WEIGHT_MXFP4) against the CPU oracle's moe_oracle_forward_mx, stage by
stage (tolerances in gpu_util.compare_mx: FP8 codes, scales and every
epilogue bit-exact on the GPU's own inputs, the fp32 MFMA accumulators within
a bound relative to the sum of the magnitudes of their terms, outputs within
the block's output tolerance).

The cases span every K split of the MX kernel (8, 4 and 2 waves; one batch
per wave; 1-, 2- and 4-step batches over several passes), 16-row items
(decode) and 32-row items with several chunks per expert (batches above 16
tokens), masks, smooth scales, an expert-parallel share, a shared expert
whose intermediate differs (two GEMM2 launches), the fused route scale,
T = 0 and T = 1, and the full shapes of the decode workload (every token) and
of the T = 512 workload (32 tokens spread over the batch).
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_expert_ffn_route_amd as moe
from moe_expert_ffn_route_amd import synth
from gpu_util import check_mx, grouped_row_tokens, pack_reference, say, with_floor_rows

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="mx", T=8, H=512, I=256, E_g=8, K=2, seed=301, weight_format="mxfp4")
    base.update(kw)
    return synth.Spec(**base)


CASES = {
    # the tiny workload's shape (H / 128 = 4 steps: 4 waves x 1; I: 2 waves x 1)
    "tiny_shape": (spec(), None),
    # H 768 (6 steps: 2 waves x 3 passes), I 512 (4 waves), I_s 256: split GEMM2
    "shared_mask_smooth_split": (spec(T=12, H=768, I=512, I_s=256, E_g=16, K=4, active=10, smooth=True,
                                      share_smooth=True, seed=302), None),
    # H 1024 (8 steps: 4 waves x 2), an expert-parallel share, fused route scale
    "ep_share_fused": (spec(T=16, H=1024, I=256, E_g=32, K=6, ep_size=4, ep_rank=1, fuse_route_scale=True,
                            seed=303), None),
    # 40 tokens on 2 experts: two 32-row chunks per expert (the second with 8
    # rows: its second row tile is skipped), 16 GEMM1 N tiles, so the chunks of
    # one tile run 8 blocks apart
    "t40_multichunk_shared": (spec(T=40, H=512, I=256, E_g=2, K=2, I_s=256, seed=304), None),
    "t100_skewed_mask_fused": (spec(T=100, H=512, I=256, E_g=8, K=3, routing="zipf", zipf_s=1.5, active=90,
                                    I_s=512, fuse_route_scale=True, seed=305), [0, 7, 50, 99]),
    # K split beyond one batch per wave: H 9216 (72 steps: 4 waves x 9 passes
    # of 2 steps), I 12288 (96 steps: 4 waves x 6 passes of 4 steps)
    "long_k_gemm1": (spec(T=3, H=9216, I=256, E_g=4, K=2, I_s=256, seed=306), None),
    "long_k_gemm2": (spec(T=3, H=256, I=12288, E_g=4, K=2, I_s=512, seed=307), None),
    # 32-row items (T > 16) with long K: H 9216 (72 steps: 8 waves x 9
    # passes of 1 step), I 3072 (24 steps: 8 waves x 3)
    "t20_long_k_gemm1": (spec(T=20, H=9216, I=256, E_g=2, K=1, I_s=256, seed=313), None),
    "t24_mid_k_gemm2": (spec(T=24, H=256, I=3072, E_g=2, K=2, I_s=512, seed=314), None),
    # two-tile items on every weight-ring length of that kernel: H 768 (6
    # steps: a 2-step ring), I 512 (4 steps: a 4-step ring), I_s 256 (2
    # steps), and I 2048 (16 steps: an 8-step ring in two turns)
    "t40_rings_2_and_4": (spec(T=40, H=768, I=512, E_g=2, K=2, I_s=256, seed=315), None),
    "t36_ring_8_two_turns": (spec(T=36, H=1024, I=2048, E_g=2, K=2, I_s=1024, active=33, seed=316), None),
    # the DeepSeek-V3 hidden size H = 7168: 56 steps of 128, so the K-split
    # kernel's waves take 14 steps in 7 batches of 2, and the two-tile
    # kernel's 8-step ring turns 7 times
    "h7168_decode": (spec(T=8, H=7168, I=1024, E_g=8, K=3, I_s=512, seed=317), None),
    "h7168_two_tile": (spec(T=40, H=7168, I=512, E_g=2, K=2, I_s=256, seed=318), None),
    "t1": (spec(T=1, H=512, I=256, E_g=4, K=2, I_s=512, seed=308), None),
    # H 2048 (16 steps: 4 waves x 4), I 3072 (24 steps: 4 waves x 6)
    "mid_k": (spec(T=9, H=2048, I=3072, E_g=4, K=2, I_s=1024, seed=312), None),
    "t0": (spec(T=0, I_s=256, seed=309), None),
    "all_masked": (spec(T=6, I_s=256, active=0, seed=310), None),
    # the decode workload's shape: T 8, H 4096, I 2048, 256 experts, top-8,
    # shared expert 2048 (every token through the oracle)
    "decode_full_shape": (spec(T=8, H=4096, I=2048, E_g=256, K=8, I_s=2048, seed=1235), None),
    # the large-batch workload's shape (two-tile items): 32 tokens spread over
    # the batch through the oracle (the FP4 oracle decodes every code per
    # product, about 0.8 s per grouped row on one host thread)
    "t512_full_shape": (spec(T=512, H=4096, I=2048, E_g=256, K=8, I_s=2048, seed=1238, wseed=1235),
                        list(range(3, 512, 16))),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mx_parity(name):
    sp, tokens = CASES[name]
    say(f"[mx] {name}: {sp}")
    stats, _, _ = check_mx(synth.make_case(sp), tokens=tokens)
    say(f"[mx] {name}: {stats}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [12, 40], ids=["decode", "two_tile"])
def test_mx_amax_floor_rows(T):
    # rows at the amax floor: the FP8 quantisers divide by eps (scale
    # eps / 448) for x and again for h; all-zero rows give zero codes
    c = synth.make_case(spec(T=T, H=512, I=256, E_g=4, K=2, I_s=256, smooth=True, seed=330 + T))
    zero, tiny = [0, 7], [3, T - 1]
    c = with_floor_rows(c, zero=zero, tiny=tiny, seed=T)
    stats, gpu, ref = check_mx(c)
    say(f"[mx] amax floor T={T}: {stats}")
    floor = np.float32(np.float32(c.spec.eps) * np.float32(1.0 / 448.0))
    tok = grouped_row_tokens(c, ref)
    hit = [r for r in range(len(tok)) if tok[r] in zero + tiny]
    assert len(hit) >= len(zero + tiny)
    for r in hit:
        assert gpu["xs"][r] == floor and gpu["hs"][r] == floor, f"row {r} (token {tok[r]})"
        if tok[r] in zero:
            assert not gpu["q_x"][r].any() and not gpu["q_h"][r].any()


def _e4m3_ties():
    """Values v whose E4M3 encoding is an exact tie after the quantiser's
    fp32 steps with a row maximum of 448 ((v * 448) * (1/448) == v): the
    bf16-representable midpoints of neighbouring E4M3 values, subnormal ones
    included, and their negatives."""
    f = np.float32
    inv = f(1) / f(448)
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (vals[:-1] + vals[1:]) / 2
    out = [f(m) for m in mids
           if not (np.array([m], np.float32).view(np.uint32)[0] & 0xFFFF) and (f(m) * f(448)) * inv == f(m)]
    return np.array(out + [-v for v in out], np.float32)


@pytest.mark.parametrize("T", [12, 40], ids=["decode", "two_tile"])
def test_mx_quant_ties_round_to_even(T):
    # a token row whose maximum is 448: each value below lands exactly halfway
    # between two E4M3 values, which the encoder rounds to the even code (the
    # codes torch's float8_e4m3fn conversion gives)
    ties = _e4m3_ties()
    c = synth.make_case(spec(T=T, H=512, I=256, E_g=4, K=2, I_s=256, seed=340 + T))
    t, n = 5, len(ties)
    assert n >= 60
    row = np.zeros(c.spec.H, np.float32)
    row[0], row[1:1 + n] = 448.0, ties
    x = c.x.copy()
    x[t] = synth.f32_to_bf16_bits(row)
    c = dataclasses.replace(c, x=x)
    stats, gpu, ref = check_mx(c)
    expect = torch.from_numpy(ties).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    tok = grouped_row_tokens(c, ref)
    hit = [r for r in range(len(tok)) if tok[r] == t]
    assert hit
    for r in hit:
        codes = gpu["q_x"][r].view(np.uint8)
        assert codes[0] == 0x7E and np.array_equal(codes[1:1 + n], expect), f"row {r}"


def _random_specs(n, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E_g = int(rng.choice([2, 4, 8, 16]))
        ep = int(rng.choice([d for d in (1, 2) if E_g % d == 0]))
        T = int(rng.choice([1, 5, 8, 16, 17, 30, 40, 64]))
        kw = dict(name=f"mxrandom{i}", T=T, H=int(rng.choice([256, 512, 768, 1024, 1280])),
                  I=int(rng.choice([256, 512, 768])), E_g=E_g, K=int(rng.integers(1, min(E_g, 6) + 1)),
                  I_s=int(rng.choice([0, 256, 512])), ep_size=ep, ep_rank=int(rng.integers(0, ep)),
                  routing=str(rng.choice(["uniform", "zipf"])), seed=400 + i)
        if rng.random() < 0.4:
            kw["active"] = int(rng.integers(0, T + 1))
        if rng.random() < 0.4:
            kw["smooth"] = True
        if kw["I_s"] and rng.random() < 0.4:
            kw["share_smooth"] = True
        if rng.random() < 0.3:
            kw["fuse_route_scale"] = True
        out.append(spec(**kw))
    return out


# (batches above 16 tokens whose local experts can average 16 rows run the
# two-tile kernel: about a third of these draws)
RANDOM = _random_specs(14)


@pytest.mark.parametrize("i", range(len(RANDOM)))
def test_mx_random_shapes(i):
    say(f"[mx] random {i}: {RANDOM[i]}")
    stats, _, _ = check_mx(synth.make_case(RANDOM[i]))
    say(f"[mx] random {i}: {stats}")


def _scale_reference(bs, which):
    """The packed scale order from its definition: 64 bytes per (tile position,
    128-element step), byte l the scale of row l % 16 for block l / 16."""
    G, n, nb = bs.shape
    t = bs.reshape(G, n // 16, 16, nb // 4, 4)            # g, tile, row-in-tile, step, block
    t = t.transpose(0, 1, 3, 4, 2)                         # g, tile, step, block, row-in-tile
    if which == moe.MOE_PACK_GMM1:
        t = t.reshape(G, 2, n // 32, *t.shape[2:]).swapaxes(1, 2)
    return np.ascontiguousarray(t).reshape(-1)


@pytest.mark.parametrize("which", [1, 2], ids=["gmm1", "gmm2"])
@pytest.mark.parametrize("shape", [(1, 32, 128), (3, 96, 384), (2, 512, 4096)])
def test_pack_mx_layout(shape, which):
    G, n, k = shape
    rng = np.random.default_rng(11)
    data = rng.integers(0, 256, (G, n, k // 2), dtype=np.uint8)
    bs = rng.integers(0, 255, (G, n, k // 32), dtype=np.uint8)
    d = moe.moe_w8a8_pack_weights_mx(torch.from_numpy(data).cuda(), torch.from_numpy(bs).cuda(), which)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    assert got.size == moe.moe_w8a8_packed_mx_bytes(G, n, k)
    nd = G * n * k // 2
    assert np.array_equal(got[:nd], pack_reference(data.view(np.int8), which).view(np.uint8))
    assert np.array_equal(got[nd:], _scale_reference(bs, which))
    # spot checks from the header's definition: (g, tile position p, step s, byte l)
    for g, p, s, l in [(0, 0, 0, 0), (G - 1, n // 16 - 1, k // 128 - 1, 63), (G // 2, 1, 0, 17)]:
        j = p if which == 2 else (p // 2 if p % 2 == 0 else n // 32 + p // 2)
        assert got[nd + ((g * (n // 16) + p) * (k // 128) + s) * 64 + l] == bs[g, 16 * j + l % 16, 4 * s + l // 16]


@pytest.mark.parametrize("name", ["ep_share_fused", "t40_multichunk_shared"])
def test_mx_hip_graph_capture_and_replay(name):
    # the FP4 path launches kernels only, so a caller can capture it; every
    # replay must match the eager result, with other eager work and
    # synchronisations between the replays
    sp, _ = CASES[name]
    say(f"[mx graph] {name}: {sp}")
    c = synth.make_case(sp)
    t = moe.upload(c)
    runner = moe.Runner(moe.dims_of_case(c))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        runner(t, stream=s)
    torch.cuda.synchronize()
    eager = [runner.output.clone(), runner.expert_token_nums.clone()]
    if runner.share_output is not None:
        eager.append(runner.share_output.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        runner(t, stream=s)
    for i in range(4):
        runner.output.fill_(3)
        runner.expert_token_nums.fill_(-1)
        if runner.share_output is not None:
            runner.share_output.fill_(3)
        runner.workspace.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(runner.output, eager[0]), i
        assert torch.equal(runner.expert_token_nums, eager[1]), i
        if runner.share_output is not None:
            assert torch.equal(runner.share_output, eager[2]), i


def test_mx_two_tile_hip_graph_capture_and_replay():
    # the two-tile FP4 kernel launches kernels only: a captured forward
    # replays to the eager result, with other eager work between replays
    c = synth.make_case(spec(T=48, H=512, I=512, E_g=2, K=2, I_s=256, active=45, seed=320))
    t = moe.upload(c)
    runner = moe.Runner(moe.dims_of_case(c))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        runner(t, stream=s)
    torch.cuda.synchronize()
    eager = (runner.output.clone(), runner.share_output.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        runner(t, stream=s)
    for i in range(4):
        runner.output.fill_(3)
        runner.share_output.fill_(3)
        runner.workspace.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(runner.output, eager[0]) and torch.equal(runner.share_output, eager[1]), i
