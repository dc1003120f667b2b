"""CPU checks that the seeded inputs follow the stated recipe (distributions,
shapes, distinct top-k experts, exact active counts, determinism, the shared
weight seed of the one-model workloads)."""
import dataclasses

import numpy as np

from moe_expert_ffn_route_amd import synth


def spec(**kw):
    base = dict(name="recipe", T=64, H=512, I=256, E_g=32, K=6, I_s=256, seed=901)
    base.update(kw)
    return synth.Spec(**base)


def test_same_seed_same_case():
    a, b = synth.make_case(spec()), synth.make_case(spec())
    for k in ("x", "expert_ids", "expert_scales", "w1", "w1s", "w2", "w2s", "sw1", "sw1s", "sw2", "sw2s"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    c = synth.make_case(spec(seed=902))
    assert not np.array_equal(a.x, c.x) and not np.array_equal(a.expert_ids, c.expert_ids)


def test_topk_ids_distinct_and_in_range():
    for routing in ("uniform", "zipf"):
        c = synth.make_case(spec(routing=routing, zipf_s=1.2))
        ids = c.expert_ids
        assert ids.shape == (64, 6) and ids.dtype == np.int32
        assert ids.min() >= 0 and ids.max() < 32
        assert all(len(set(row)) == 6 for row in ids.tolist())


def test_zipf_routing_is_skewed_and_uniform_is_not():
    u = np.bincount(synth.make_case(spec(T=512, K=2)).expert_ids.ravel(), minlength=32)
    z = np.bincount(synth.make_case(spec(T=512, K=2, routing="zipf", zipf_s=1.2)).expert_ids.ravel(), minlength=32)
    assert u.max() < 3 * u.mean()
    assert z.max() > 4 * z.mean() and (z == 0).sum() >= (u == 0).sum()


def test_routing_weights_are_a_softmax_over_k():
    w = synth.make_case(spec()).expert_scales
    assert w.dtype == np.float32 and np.all(w > 0)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_int8_weights_and_scales_follow_the_recipe():
    c = synth.make_case(spec())
    for w in (c.w1, c.w2, c.sw1, c.sw2):
        assert w.dtype == np.int8 and w.min() >= -127 and w.max() <= 127
        # clamp(rint(32 N(0, 1))): standard deviation near 32
        assert 29 < float(w.astype(np.float64).std()) < 35
    for s in (c.w1s, c.w2s, c.sw1s, c.sw2s):
        assert s.dtype == np.float32 and s.min() >= 1e-3 and s.max() <= 1e-2
    assert c.w1.shape == (32, 512, 512) and c.w2.shape == (32, 512, 256)
    assert c.sw1.shape == (512, 512) and c.sw2.shape == (512, 256)


def test_x_is_bf16_of_a_standard_normal():
    x = synth.bf16_bits_to_f32(synth.make_case(spec(T=256)).x).astype(np.float64)
    assert abs(x.mean()) < 0.02 and 0.97 < x.std() < 1.03
    # bf16: the low 16 bits of every fp32 value are zero
    assert np.all((x.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)


def test_mask_has_exactly_the_active_count_and_smooth_scales_their_range():
    c = synth.make_case(spec(active=41, smooth=True, share_smooth=True))
    assert c.mask.dtype == np.uint8 and int(c.mask.sum()) == 41 and set(np.unique(c.mask)) <= {0, 1}
    assert c.smooth.shape == (32, 512) and c.smooth.min() >= 0.5 and c.smooth.max() <= 2.0
    assert c.share_smooth.shape == (512,)


def test_one_model_workloads_share_their_weights():
    # the decode, Zipf and T = 512 workloads are one model: the same weight
    # seed, so expert g's weights are the same arrays in all three
    s1, s3, s4 = synth.WORKLOADS[1], synth.WORKLOADS[3], synth.WORKLOADS[4]
    assert s1.weight_seed == s3.weight_seed == s4.weight_seed
    small = [dataclasses.replace(s, H=256, I=256, I_s=256) for s in (s1, s3, s4)]
    w = [synth.expert_weights(s, 7) for s in small]
    for a, b in zip(w[0], w[1]):
        assert np.array_equal(a, b)
    for a, b in zip(w[0], w[2]):
        assert np.array_equal(a, b)
