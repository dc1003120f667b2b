"""The oracle under the undefined-behaviour sanitizer (CPU only).

The oracle is rebuilt with gcc's UBSan and bounds checks (aborting on the
first finding) and run on the block's options and degenerate cases: every
result must be bit-identical to the ordinary build's, and no check may fire
(a finding aborts the test process).
"""
import dataclasses
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from moe_expert_ffn_route_amd import synth

GCC = shutil.which("gcc")


def spec(**kw):
    base = dict(name="ubsan", T=16, H=256, I=256, E_g=8, K=2, seed=301)
    base.update(kw)
    return synth.Spec(**base)


CASES = {
    "tiny": synth.WORKLOADS[0],
    "t0": spec(T=0),
    "t1_shared": spec(T=1, I_s=512),
    "all_masked": spec(T=9, active=0, I_s=256),
    "mask_smooth_shared_smooth": spec(T=37, H=512, I=512, I_s=256, E_g=16, K=4, active=29, smooth=True,
                                      share_smooth=True),
    "ep_share": spec(T=50, E_g=32, K=6, ep_size=4, ep_rank=3, active=41, smooth=True),
    "zipf_multi_chunk": spec(T=200, E_g=8, K=2, routing="zipf", zipf_s=2.0, I_s=512),
    "k16_e512": spec(T=20, E_g=512, K=16, I_s=256),
    "fused_route_scale": spec(T=30, E_g=16, K=4, I_s=256, active=25, fuse_route_scale=True),
    "mxfp4_weights": spec(T=12, E_g=8, K=3, I_s=256, active=10, smooth=True, weight_format="mxfp4"),
    "group_scales": spec(T=14, H=512, I=256, E_g=8, K=3, I_s=512, active=12, smooth=True, share_smooth=True,
                         quant_group=64),
}


@pytest.fixture(scope="module")
def ubsan_lib(tmp_path_factory):
    if GCC is None:
        pytest.skip("gcc not available")
    out = str(tmp_path_factory.mktemp("ubsan") / "libmoe_oracle_ubsan.so")
    flags = [f for f in oracle.CFLAGS if f != "-shared"]
    subprocess.check_call([GCC, *flags, "-shared", "-fsanitize=undefined,bounds,float-cast-overflow",
                           "-fno-sanitize-recover=all", "-static-libubsan", oracle.SRC, "-o", out, "-lm"])
    return out


def _same(a, b):
    for k, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[k]), k
        else:
            assert v == b[k], k


@pytest.mark.parametrize("name", list(CASES))
def test_oracle_clean_under_ubsan(ubsan_lib, name):
    case = synth.make_case(CASES[name])
    ref = oracle.forward(case, trace=True)
    with oracle.using(ubsan_lib):
        got = oracle.forward(case, trace=True)
    _same(ref, got)


def test_out_of_range_and_duplicate_ids_under_ubsan(ubsan_lib):
    case = synth.make_case(spec(T=12, E_g=8, K=3, I_s=256))
    ids = case.expert_ids.copy()
    ids[0, 0], ids[3, 2], ids[5, 1] = -1, 8, 1 << 30   # out of range: dropped and counted
    ids[7, :] = ids[7, 0]                               # one expert three times in a token
    case = dataclasses.replace(case, expert_ids=ids)
    ref = oracle.forward(case, trace=True)
    with oracle.using(ubsan_lib):
        got = oracle.forward(case, trace=True)
    _same(ref, got)
    assert ref["n_bad"] == 3
