"""The token-split (multi-threaded) oracle run equals the single-threaded run
bit for bit: every output, count and traced intermediate, on cases with a
shared expert, masks, smooth scales, an expert-parallel share, the FP4-weight
mode and group-wise scales. The parity tests and the benchmark's all-core CPU
baseline rely on this."""
import dataclasses

import numpy as np
import pytest

import oracle
from moe_expert_ffn_route_amd import synth


def spec(**kw):
    base = dict(name="thr", T=23, H=256, I=256, E_g=8, K=3, I_s=256, seed=9001)
    base.update(kw)
    return synth.Spec(**base)


CASES = {
    "shared_mask_smooth": spec(active=17, smooth=True, share_smooth=True),
    "ep_share_no_shared": spec(I_s=0, E_g=16, ep_size=4, ep_rank=3, seed=9002),
    "fused_route_scale": spec(fuse_route_scale=True, seed=9003),
    "zipf_subset": spec(T=40, routing="zipf", zipf_s=1.5, seed=9004),
    "group_wise": spec(quant_group=64, seed=9005),
    "fp4_weights": spec(T=9, weight_format="mxfp4", seed=9006),
}


def _same(a, b, key):
    if a is None or b is None:
        assert a is None and b is None, key
        return
    if isinstance(a, np.ndarray):
        assert a.dtype == b.dtype and a.shape == b.shape, key
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), key
    else:
        assert a == b, key


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("threads", [2, 5])
def test_threaded_equals_single(name, threads):
    case = synth.make_case(CASES[name])
    tokens = None if name != "zipf_subset" else [0, 3, 4, 9, 20, 39]
    one = oracle.forward(case, tokens=tokens, trace=True)
    many = oracle.forward(case, tokens=tokens, trace=True, threads=threads)
    assert set(one) == set(many)
    for k in one:
        _same(one[k], many[k], k)


def test_threads_more_than_tokens():
    case = synth.make_case(spec(T=2, seed=9007))
    one = oracle.forward(case)
    many = oracle.forward(case, threads=8)
    _same(one["output"], many["output"], "output")
    _same(one["share_output"], many["share_output"], "share_output")
