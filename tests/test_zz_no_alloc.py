"""The entry point that allocates nothing (moe_w8a8_forward_noalloc, the
library's built-in per-device scratch array as workspace) against the
workspace entry point (moe_w8a8_forward) on the same inputs: outputs, counts
and every debug intermediate bit for bit, over two calls in a row, the second
with a smaller batch (the array keeps the first call's contents), and the
second also against the oracle."""
import numpy as np
import pytest
import torch

import moe_expert_ffn_route_amd as moe
import oracle
from moe_expert_ffn_route_amd import synth
from gpu_util import out_close, say

pytestmark = pytest.mark.gpu

BIG = synth.Spec("noalloc_big", T=40, H=512, I=256, E_g=16, K=4, I_s=256, active=37, smooth=True,
                 share_smooth=True, seed=7001)
SMALL = synth.Spec("noalloc_small", T=5, H=512, I=256, E_g=16, K=4, I_s=256, seed=7002)
DECODE = synth.Spec("noalloc_decode", T=8, H=1024, I=512, E_g=32, K=8, I_s=512, seed=7003)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _both(case, packed):
    """(workspace entry point, no-alloc entry point) results on one case."""
    t = moe.upload(case)
    dims = moe.dims_of_case(case)
    if packed:
        t = moe.pack_weights(t)
        dims.weight_layout = moe.MOE_WEIGHT_PACKED
    res = []
    for noalloc in (False, True):
        runner = moe.Runner(dims)  # outputs (and, for the first, the workspace)
        runner.output.fill_(7)
        if runner.share_output is not None:
            runner.share_output.fill_(7)
        d, bufs = moe.debug_buffers(dims)
        kw = dict(output=runner.output, share_output=runner.share_output,
                  expert_token_nums=runner.expert_token_nums, dbg=d, **t)
        if noalloc:
            moe.moe_w8a8_forward_noalloc(dims, **kw)
        else:
            moe.moe_w8a8_forward(dims, workspace=runner.workspace, workspace_bytes=runner.workspace_bytes, **kw)
        torch.cuda.synchronize()
        r = {k: v.cpu().numpy() for k, v in bufs.items()}
        r["output"] = _bits(runner.output)
        r["share_output"] = _bits(runner.share_output) if runner.share_output is not None else None
        r["expert_token_nums"] = runner.expert_token_nums.cpu().numpy()
        res.append(r)
    return res


def _same(a, b, case):
    s = case.spec
    for k in ("output", "share_output", "expert_token_nums", "num_rows", "group_offset"):
        if a[k] is None:
            assert b[k] is None
            continue
        assert np.array_equal(a[k], b[k]), k
    P, Ta = int(a["num_rows"][0]), int(a["num_rows"][1])
    assert np.array_equal(a["sorted_pair"][:P], b["sorted_pair"][:P])
    for r in range(P + (Ta if s.I_s else 0)):
        n = s.I if r < P else s.I_s
        for k, w in (("q_x", s.H), ("xs", None), ("acc1", 2 * n), ("h", n), ("q_h", n), ("hs", None),
                     ("acc2", s.H), ("z", s.H)):
            x, y = (a[k][r:r + 1], b[k][r:r + 1]) if w is None else (a[k][r, :w], b[k][r, :w])
            assert np.array_equal(np.ascontiguousarray(x).view(np.uint8), np.ascontiguousarray(y).view(np.uint8)), (k, r)


@pytest.mark.parametrize("packed", [True, False], ids=["packed", "rowmajor"])
def test_noalloc_equals_workspace_entry_two_calls(packed):
    for sp in (BIG, SMALL):  # the second call is smaller than the first
        say(f"[noalloc] {sp.name} packed={packed}")
        case = synth.make_case(sp)
        ws_res, na_res = _both(case, packed)
        _same(ws_res, na_res, case)
    ref = oracle.forward(case)
    out_close(na_res["output"], ref["output"], "output")
    out_close(na_res["share_output"], ref["share_output"], "share_output")


def test_noalloc_decode_shape_and_limit():
    case = synth.make_case(DECODE)
    ws_res, na_res = _both(case, True)
    _same(ws_res, na_res, case)
    # a batch whose workspace exceeds the built-in array is refused before launch
    big = moe.make_dims(num_tokens=512, hidden=4096, inter=2048, topk=8, moe_expert_num=256)
    assert moe.moe_w8a8_workspace_size(big) > moe.binding.NOALLOC_SCRATCH_BYTES
    dev = lambda n, dt: torch.zeros(n, dtype=dt, device="cuda")
    rc = moe.moe_w8a8_forward_noalloc(
        big, x=dev((512, 4096), torch.bfloat16), expert_ids=dev((512, 8), torch.int32),
        expert_scales=dev((512, 8), torch.float32), gmm1_weight=dev(16, torch.int8),
        gmm1_weight_scale=dev(4, torch.float32), gmm2_weight=dev(16, torch.int8),
        gmm2_weight_scale=dev(4, torch.float32), output=dev((512, 4096), torch.bfloat16),
        expert_token_nums=dev(256, torch.int32), check=False)
    assert rc == moe.binding.MOE_ERR_SCRATCH_LIMIT
