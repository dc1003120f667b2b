"""GPU parity of group-wise activation scales (quant_mode 2, "DeepSeek V4
Decode Optimization" sec. 3.1) against the CPU oracle's quant_group mode,
stage by stage (gpu_util.compare_group: codes, group scales and epilogues
bit-exact on the GPU's own inputs; the fp32 GEMM outputs within the bound of
adding the same dequantised group partials in another order).

The cases cover the three group sizes (64, 128, 256), every K split the
group path takes (8, 4, 2 and 1 waves; a batch of whole groups, or one group
per batch over several passes), 16- and 32-row items with several chunks per
expert, masks, smooth scales, an EP share, a shared expert with a different
intermediate (two GEMM2 launches), T = 0 / 1, and the full shapes of the
decode workload and of the T = 512 workload (every token of both).
"""
import numpy as np
import pytest
import torch

from moe_expert_ffn_route_amd import synth
import moe_expert_ffn_route_amd as moe
from gpu_util import check_group, grouped_row_tokens, say, with_floor_rows

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="grp", T=8, H=512, I=256, E_g=8, K=2, seed=501, quant_group=128)
    base.update(kw)
    return synth.Spec(**base)


CASES = {
    # the tiny workload's shape: H 512 = 4 groups of 128 (4 waves x 1 group),
    # I 256 = 2 groups (2 waves)
    "tiny_g128": (spec(), None),
    # G 64: H 512 = 8 groups (8 waves x 1 step), I 256 = 4 groups (4 waves)
    "tiny_g64_shared": (spec(quant_group=64, I_s=512, seed=502), None),
    # G 256: I 256 is one group (one wave), H 1024 four (4 waves x 4 steps)
    "g256_one_group": (spec(H=1024, quant_group=256, I_s=256, seed=503), None),
    # H 768 = 6 groups of 128 (2 waves x 3 passes of 1 group), I 512, I_s 256
    "mask_smooth_split_gemm2": (spec(T=12, H=768, I=512, I_s=256, E_g=16, K=4, active=10, smooth=True,
                                     share_smooth=True, seed=504), None),
    "ep_share": (spec(T=16, H=1024, I=512, E_g=32, K=6, ep_size=4, ep_rank=1, active=13, smooth=True, seed=505),
                 None),
    # 40 tokens on 2 experts: 32-row items (two row tiles; the second chunk of
    # an expert has 8 rows, so its second tile is skipped), 16 N tiles
    "t40_multichunk": (spec(T=40, H=512, I=256, E_g=2, K=2, I_s=256, seed=506), None),
    # two row tiles with H 4096 (8 waves x 2 batches of 4 steps) and I 256
    # (2 waves x one 2-step group), and with H 768 (2 waves x 3 one-group
    # batches), smooth scales
    "t20_two_tiles_h4096": (spec(T=20, H=4096, I=256, E_g=1, K=1, I_s=256, seed=511), None),
    "t40_two_tiles_h768": (spec(T=40, H=768, I=512, E_g=2, K=2, I_s=256, smooth=True, seed=512), None),
    # many experts with few rows each at T > 16: 16-row items
    "t24_few_rows_per_expert": (spec(T=24, H=512, I=256, E_g=16, K=2, I_s=256, seed=513), None),
    # G 64 and H 9216: 144 groups, 8 waves x 18 passes of one group
    "long_k_g64": (spec(T=3, H=9216, I=256, E_g=4, K=2, I_s=256, quant_group=64, seed=507), None),
    # I 4096 with I_s 4352 and G 128: a routed GEMM2 batch holds 4 groups
    # (8 waves x 8 steps) but the h scale rows are 34 groups apart, so the
    # scales are loaded one by one; the shared GEMM2 (34 groups) runs on 2
    # waves x 17 passes of one group
    "scale_stride_34": (spec(T=5, H=256, I=4096, I_s=4352, E_g=2, K=1, seed=510), None),
    "t1": (spec(T=1, I_s=512, seed=508), None),
    "t0": (spec(T=0, I_s=256, seed=509), None),
    # 32-row items on the wide kernel with each group size (64: a 4-step
    # weight ring; 128 and 256: 8 steps), an EP share, masks and smooth
    # scales, a shared expert whose intermediate differs
    "wide_g64_ep_mask": (spec(T=48, H=1024, I=512, E_g=8, K=4, ep_size=2, ep_rank=1, active=44, smooth=True,
                              I_s=768, quant_group=64, seed=514), None),
    "wide_g128_shared_smooth": (spec(T=40, H=2048, I=1024, E_g=2, K=2, I_s=512, share_smooth=True,
                                     quant_group=128, seed=515), None),
    "wide_g256_long_k": (spec(T=36, H=4096, I=768, E_g=2, K=1, I_s=256, quant_group=256, seed=516), None),
    # the DeepSeek-V3 hidden size H = 7168 (56 groups of 128: 8 waves of 7
    # one-group batches) on 16-row and 32-row items
    "h7168_g128_decode": (spec(T=8, H=7168, I=1024, E_g=8, K=3, I_s=512, quant_group=128, seed=517), None),
    "h7168_g128_wide": (spec(T=40, H=7168, I=512, E_g=2, K=2, I_s=256, quant_group=128, seed=518), None),
    # the decode workload's shape with 128-element groups (every token)
    "decode_full_shape": (spec(T=8, H=4096, I=2048, E_g=256, K=8, I_s=2048, seed=1235), None),
    # the large-batch workload's shape (two-tile items), every token: all
    # 4608 grouped rows
    "t512_full_shape": (spec(T=512, H=4096, I=2048, E_g=256, K=8, I_s=2048, seed=1238, wseed=1235), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_group_parity(name):
    sp, tokens = CASES[name]
    say(f"[grp] {name}: {sp}")
    c = synth.make_case(sp)
    stats, _, _ = check_group(c, tokens=tokens, packed=True)
    say(f"[grp] {name}: {stats}")
    if name == "tiny_g128":  # row-major weights too
        stats, _, _ = check_group(c, tokens=tokens, packed=False)
        say(f"[grp] {name} row-major: {stats}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,G", [(12, 128), (40, 64)], ids=["decode_g128", "wide_g64"])
def test_group_amax_floor(T, G):
    # one group of a row at the amax floor: token 0's first group all zero,
    # token 2's second group far below eps; only those groups' scales are
    # eps / 127, the row's other groups keep their own
    c = synth.make_case(spec(T=T, H=512, I=256, E_g=4, K=2, I_s=256, quant_group=G, seed=530 + T))
    c = with_floor_rows(c, zero=[0], seed=T, cols=slice(0, G))
    c = with_floor_rows(c, tiny=[2], seed=T + 1, cols=slice(G, 2 * G))
    stats, gpu, ref = check_group(c, packed=True)
    say(f"[grp] amax floor T={T} G={G}: {stats}")
    floor = np.float32(np.float32(c.spec.eps) * np.float32(1.0 / 127.0))
    tok = grouped_row_tokens(c, ref)
    for r, t in enumerate(tok):
        if t == 0:
            assert gpu["xs"][r, 0] == floor and not gpu["q_x"][r, :G].any() and gpu["xs"][r, 1] > floor
        elif t == 2:
            assert gpu["xs"][r, 1] == floor and gpu["xs"][r, 0] > floor
    assert 0 in tok and 2 in tok


def _random_specs(n, seed=6060):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([64, 128, 256]))
        E_g = int(rng.choice([2, 4, 8, 16]))
        T = int(rng.choice([1, 5, 8, 16, 17, 30, 40, 64]))
        ep = int(rng.choice([d for d in (1, 2) if E_g % d == 0]))
        kw = dict(name=f"grprandom{i}", T=T, H=int(rng.choice([1, 2, 3, 4])) * 256 * (2 if G == 256 else 1),
                  I=int(rng.choice([256, 512])), E_g=E_g, K=int(rng.integers(1, min(E_g, 6) + 1)),
                  I_s=int(rng.choice([0, 256, 512])), routing=str(rng.choice(["uniform", "zipf"])),
                  ep_size=ep, ep_rank=int(rng.integers(0, ep)), quant_group=G, seed=600 + i)
        if rng.random() < 0.4:
            kw["active"] = int(rng.integers(0, T + 1))
        if rng.random() < 0.4:
            kw["smooth"] = True
        out.append(spec(**kw))
    return out


RANDOM = _random_specs(14)


@pytest.mark.parametrize("i", range(len(RANDOM)))
def test_group_random_shapes(i):
    say(f"[grp] random {i}: {RANDOM[i]}")
    stats, _, _ = check_group(synth.make_case(RANDOM[i]), packed=bool(i % 2))
    say(f"[grp] random {i}: {stats}")


def test_group_hip_graph_capture_and_replay():
    # group-wise scales launch kernels only: a captured forward replays to the
    # eager result, with other eager work between the replays
    c = synth.make_case(spec(T=20, H=768, I=512, E_g=4, K=2, I_s=256, active=18, smooth=True, seed=520))
    t = moe.upload(c)
    runner = moe.Runner(moe.dims_of_case(c))
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
