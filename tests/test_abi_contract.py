"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, its structs have the header's layout, and host-side argument
checks reject bad calls before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_expert_ffn_route_amd as moe
from moe_expert_ffn_route_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w8a8.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from moe_expert_ffn_route_amd import build
        build.build()
    return binding.library()


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"MOE_W8A8_API\s+[\w\s\*]+?\b(moe_w8a8_\w+)\s*\(", text)


def test_header_declares_the_binding_exports():
    assert sorted(declared_functions()) == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(lib, name)


def test_struct_layout_matches_header(tmp_path):
    fields_d = [f for f, _ in binding.Dims._fields_]
    fields_g = [f for f, _ in binding.Debug._fields_]
    prog = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe_w8a8.h"', 'int main(void){',
            'printf("%zu\\n", sizeof(moe_w8a8_dims_t));', 'printf("%zu\\n", sizeof(moe_w8a8_debug_t));']
    prog += [f'printf("%zu\\n", offsetof(moe_w8a8_dims_t, {f}));' for f in fields_d]
    prog += [f'printf("%zu\\n", offsetof(moe_w8a8_debug_t, {f}));' for f in fields_g]
    prog += ['return 0;}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    vals = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    assert vals[0] == ctypes.sizeof(binding.Dims) and vals[1] == ctypes.sizeof(binding.Debug)
    off = vals[2:]
    assert off[: len(fields_d)] == [getattr(binding.Dims, f).offset for f in fields_d]
    assert off[len(fields_d):] == [getattr(binding.Debug, f).offset for f in fields_g]


def good_dims(**kw):
    d = dict(num_tokens=8, hidden=512, inter=256, topk=2, moe_expert_num=8)
    d.update(kw)
    return moe.make_dims(**d)


def test_workspace_size(lib):
    n = moe.moe_w8a8_workspace_size(good_dims())
    assert n > 8 * 3 * 512  # at least the grouped int8 rows
    assert moe.moe_w8a8_workspace_size(good_dims(num_tokens=0)) >= 0
    big = moe.moe_w8a8_workspace_size(good_dims(num_tokens=512, hidden=4096, inter=2048, topk=8,
                                                moe_expert_num=256, share_inter=2048))
    assert big > moe.moe_w8a8_workspace_size(good_dims(num_tokens=8, hidden=4096, inter=2048, topk=8,
                                                       moe_expert_num=256, share_inter=2048))
    assert lib.moe_w8a8_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_w8a8_workspace_size(ctypes.byref(good_dims()), None) == binding.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(num_tokens=-1), binding.MOE_ERR_INVALID_ARG),
    (dict(hidden=0), binding.MOE_ERR_INVALID_ARG),
    (dict(topk=0), binding.MOE_ERR_INVALID_ARG),
    (dict(topk=17), binding.MOE_ERR_UNSUPPORTED),
    (dict(moe_expert_num=9, ep_rank_size=2), binding.MOE_ERR_INVALID_ARG),
    (dict(ep_rank_size=2, ep_rank_id=2), binding.MOE_ERR_INVALID_ARG),
    (dict(quant_mode=2), binding.MOE_ERR_UNSUPPORTED),
    (dict(amax_eps=0.0), binding.MOE_ERR_INVALID_ARG),
    (dict(amax_eps=float("nan")), binding.MOE_ERR_INVALID_ARG),
    (dict(hidden=320), binding.MOE_ERR_UNSUPPORTED),
    (dict(inter=100), binding.MOE_ERR_UNSUPPORTED),
    (dict(share_inter=64), binding.MOE_ERR_UNSUPPORTED),
    (dict(moe_expert_num=1024), binding.MOE_ERR_UNSUPPORTED),
    (dict(num_tokens=70000), binding.MOE_ERR_UNSUPPORTED),
    (dict(weight_layout=2), binding.MOE_ERR_INVALID_ARG),
    (dict(fuse_route_scale=2), binding.MOE_ERR_INVALID_ARG),
    (dict(fuse_route_scale=-1), binding.MOE_ERR_INVALID_ARG),
    (dict(weight_format=2), binding.MOE_ERR_INVALID_ARG),
    (dict(weight_format=1), binding.MOE_ERR_UNSUPPORTED),           # FP4 weights must be packed
    # group-wise activation scales: 64, 128 or 256 (H, I and I_s are
    # multiples of 256, so every allowed size divides them); INT8 weights and
    # the per-row route scale only
    (dict(quant_mode=2, quant_group=32), binding.MOE_ERR_UNSUPPORTED),
    (dict(quant_mode=2, quant_group=512), binding.MOE_ERR_UNSUPPORTED),
    (dict(quant_mode=2, quant_group=0), binding.MOE_ERR_UNSUPPORTED),
    (dict(quant_mode=2, quant_group=192), binding.MOE_ERR_UNSUPPORTED),
    (dict(quant_mode=2, quant_group=128, fuse_route_scale=1), binding.MOE_ERR_UNSUPPORTED),
    (dict(quant_mode=2, quant_group=128, weight_format=1, weight_layout=1), binding.MOE_ERR_UNSUPPORTED),
    (dict(quant_mode=3), binding.MOE_ERR_UNSUPPORTED),
])
def test_bad_dims_rejected(lib, kw, code):
    n = ctypes.c_size_t(0)
    assert lib.moe_w8a8_workspace_size(ctypes.byref(good_dims(**kw)), ctypes.byref(n)) == code


FAKE = 1 << 20  # a 256-aligned non-NULL address; never dereferenced: every call below fails validation


def call(lib, dims, **over):
    args = dict(x=FAKE, expert_ids=FAKE, expert_scales=FAKE, gmm1_weight=FAKE, gmm1_weight_scale=FAKE,
                gmm2_weight=FAKE, gmm2_weight_scale=FAKE, share_gmm1_weight=None, share_gmm1_weight_scale=None,
                share_gmm2_weight=None, share_gmm2_weight_scale=None, expert_smooth_scales=None,
                share_smooth_scales=None, x_active_mask=None, output=FAKE, share_output=None,
                expert_token_nums=FAKE, workspace=FAKE)
    ws = over.pop("workspace_bytes", 1 << 40)
    args.update(over)
    order = ["x", "expert_ids", "expert_scales", "gmm1_weight", "gmm1_weight_scale", "gmm2_weight",
             "gmm2_weight_scale", "share_gmm1_weight", "share_gmm1_weight_scale", "share_gmm2_weight",
             "share_gmm2_weight_scale", "expert_smooth_scales", "share_smooth_scales", "x_active_mask", "output",
             "share_output", "expert_token_nums", "workspace"]
    d = ctypes.byref(dims) if dims is not None else None
    return lib.moe_w8a8_forward(d, *[args[k] for k in order], ws, None, None)


@pytest.mark.parametrize("over,code", [
    (dict(x=None), binding.MOE_ERR_INVALID_ARG),
    (dict(expert_ids=None), binding.MOE_ERR_INVALID_ARG),
    (dict(output=None), binding.MOE_ERR_INVALID_ARG),
    (dict(expert_token_nums=None), binding.MOE_ERR_INVALID_ARG),
    (dict(x=FAKE + 8), binding.MOE_ERR_INVALID_ARG),                 # bf16 rows need 16-byte alignment
    (dict(gmm1_weight=FAKE + 4), binding.MOE_ERR_INVALID_ARG),
    (dict(expert_scales=FAKE + 2), binding.MOE_ERR_INVALID_ARG),
    (dict(share_gmm1_weight=FAKE), binding.MOE_ERR_INVALID_ARG),     # shared weights without share_inter
    (dict(share_smooth_scales=FAKE), binding.MOE_ERR_INVALID_ARG),
    (dict(workspace=None), binding.MOE_ERR_WORKSPACE),
    (dict(workspace_bytes=100), binding.MOE_ERR_WORKSPACE),
    (dict(workspace=FAKE + 128), binding.MOE_ERR_INVALID_ARG),
])
def test_forward_rejects_bad_arguments(lib, over, code):
    assert call(lib, good_dims(), **over) == code


def test_forward_rejects_bad_dims_and_shared_mismatch(lib):
    assert call(lib, None) == binding.MOE_ERR_INVALID_ARG
    assert call(lib, good_dims(quant_mode=0)) == binding.MOE_ERR_UNSUPPORTED
    # share_inter > 0 needs all four shared tensors and share_output
    sd = good_dims(share_inter=256)
    assert call(lib, sd) == binding.MOE_ERR_INVALID_ARG
    assert call(lib, sd, share_gmm1_weight=FAKE, share_gmm1_weight_scale=FAKE, share_gmm2_weight=FAKE,
                share_gmm2_weight_scale=FAKE) == binding.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("src,dst,g,n,k,which", [
    (None, FAKE, 1, 32, 64, 1), (FAKE, None, 1, 32, 64, 1), (FAKE, 2 * FAKE, 1, 16, 64, 1),
    (FAKE, 2 * FAKE, 1, 48, 64, 2), (FAKE, 2 * FAKE, 1, 32, 96, 1), (FAKE, 2 * FAKE, -1, 32, 64, 2),
    (FAKE + 8, 2 * FAKE, 1, 32, 64, 1), (FAKE, FAKE + 512, 1, 32, 64, 2), (FAKE, 2 * FAKE, 1, 32, 64, 0),
    (FAKE, 2 * FAKE, 1, 32, 64, 3)])
def test_pack_rejects_bad_arguments(lib, src, dst, g, n, k, which):
    assert lib.moe_w8a8_pack_weights(src, dst, g, n, k, which, None) == binding.MOE_ERR_INVALID_ARG


def test_group_mode_workspace(lib):
    # the per-row scales become H / G and max(I, I_s) / G per row
    d1 = good_dims(share_inter=512)
    d2 = good_dims(share_inter=512, quant_mode=2, quant_group=64)
    assert moe.moe_w8a8_workspace_size(d2) > moe.moe_w8a8_workspace_size(d1)
    assert moe.moe_w8a8_workspace_size(good_dims(quant_mode=2, quant_group=256)) > 0


def test_mx_workspace_and_packed_size(lib):
    mx = moe.moe_w8a8_workspace_size(good_dims(weight_format=1, weight_layout=1))
    assert mx > 0
    # 16 * (n/16) tiles x k/128 steps x (1024 element bytes + 64 scale bytes)
    assert moe.moe_w8a8_packed_mx_bytes(3, 64, 256) == 3 * 64 * (256 // 2 + 256 // 32)
    assert moe.moe_w8a8_packed_mx_bytes(0, 32, 128) == 0
    for g, n, k in ((1, 16, 128), (1, 32, 64), (-1, 32, 128), (1, 0, 128)):
        b = ctypes.c_size_t(0)
        assert lib.moe_w8a8_packed_mx_bytes(g, n, k, ctypes.byref(b)) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_w8a8_packed_mx_bytes(1, 32, 128, None) == binding.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("data,bs,dst,g,n,k,which", [
    (None, FAKE, 4 * FAKE, 1, 32, 128, 1), (FAKE, None, 4 * FAKE, 1, 32, 128, 1),
    (FAKE, 2 * FAKE, None, 1, 32, 128, 1), (FAKE, 2 * FAKE, 4 * FAKE, 1, 32, 64, 1),
    (FAKE, 2 * FAKE, 4 * FAKE, 1, 48, 128, 2), (FAKE, 2 * FAKE, 4 * FAKE, 1, 32, 128, 0),
    (FAKE + 8, 2 * FAKE, 4 * FAKE, 1, 32, 128, 1), (FAKE, 2 * FAKE, 4 * FAKE + 8, 1, 32, 128, 1),
    (FAKE, 2 * FAKE, FAKE + 1024, 1, 32, 128, 2),        # dst overlaps the elements
    (FAKE, 2 * FAKE, 2 * FAKE - 256, 1, 32, 128, 2)])    # dst overlaps the block scales
def test_pack_mx_rejects_bad_arguments(lib, data, bs, dst, g, n, k, which):
    assert lib.moe_w8a8_pack_weights_mx(data, bs, dst, g, n, k, which, None) == binding.MOE_ERR_INVALID_ARG


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -99):
        s = moe.moe_w8a8_status_string(code)
        assert isinstance(s, str) and s


def call_noalloc(lib, dims, **over):
    args = dict(x=FAKE, expert_ids=FAKE, expert_scales=FAKE, gmm1_weight=FAKE, gmm1_weight_scale=FAKE,
                gmm2_weight=FAKE, gmm2_weight_scale=FAKE, share_gmm1_weight=None, share_gmm1_weight_scale=None,
                share_gmm2_weight=None, share_gmm2_weight_scale=None, expert_smooth_scales=None,
                share_smooth_scales=None, x_active_mask=None, output=FAKE, share_output=None,
                expert_token_nums=FAKE)
    args.update(over)
    order = ["x", "expert_ids", "expert_scales", "gmm1_weight", "gmm1_weight_scale", "gmm2_weight",
             "gmm2_weight_scale", "share_gmm1_weight", "share_gmm1_weight_scale", "share_gmm2_weight",
             "share_gmm2_weight_scale", "expert_smooth_scales", "share_smooth_scales", "x_active_mask", "output",
             "share_output", "expert_token_nums"]
    d = ctypes.byref(dims) if dims is not None else None
    return lib.moe_w8a8_forward_noalloc(d, *[args[k] for k in order], None, None)


@pytest.mark.parametrize("over,code", [
    (dict(x=None), binding.MOE_ERR_INVALID_ARG),
    (dict(output=None), binding.MOE_ERR_INVALID_ARG),
    (dict(gmm1_weight=FAKE + 4), binding.MOE_ERR_INVALID_ARG),
    (dict(share_gmm1_weight=FAKE), binding.MOE_ERR_INVALID_ARG),
])
def test_noalloc_rejects_bad_arguments_before_any_hip_call(lib, over, code):
    # argument checks come before the library touches the device
    assert call_noalloc(lib, good_dims(), **over) == code
    assert call_noalloc(lib, None) == binding.MOE_ERR_INVALID_ARG
    assert call_noalloc(lib, good_dims(quant_mode=0)) == binding.MOE_ERR_UNSUPPORTED


def test_noalloc_scratch_limit(lib):
    # calls whose workspace exceeds the built-in array are rejected up front
    # with their own status; the decode and 128-token EP-share shapes fit
    big = good_dims(num_tokens=512, hidden=4096, inter=2048, topk=8, moe_expert_num=256, share_inter=2048)
    assert moe.moe_w8a8_workspace_size(big) > binding.NOALLOC_SCRATCH_BYTES
    share = dict(share_gmm1_weight=FAKE, share_gmm1_weight_scale=FAKE, share_gmm2_weight=FAKE,
                 share_gmm2_weight_scale=FAKE, share_output=FAKE)
    assert call_noalloc(lib, big, **share) == binding.MOE_ERR_SCRATCH_LIMIT
    assert "scratch" in moe.moe_w8a8_status_string(binding.MOE_ERR_SCRATCH_LIMIT)
    for T in (8, 128):
        d = good_dims(num_tokens=T, hidden=4096, inter=2048, topk=8, moe_expert_num=256, share_inter=2048)
        assert moe.moe_w8a8_workspace_size(d) <= binding.NOALLOC_SCRATCH_BYTES, T


def test_noalloc_scratch_size_matches_header():
    with open(HEADER) as f:
        m = re.search(r"#define MOE_W8A8_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("ptr,nbytes,code", [
    (None, 16, binding.MOE_ERR_INVALID_ARG), (FAKE + 8, 16, binding.MOE_ERR_INVALID_ARG),
    (FAKE, 24, binding.MOE_ERR_INVALID_ARG), (None, 0, binding.MOE_OK), (FAKE, 0, binding.MOE_OK)])
@pytest.mark.parametrize("entry", ["moe_w8a8_warm", "moe_w8a8_read_probe"])
def test_warm_and_read_probe_reject_bad_arguments(lib, entry, ptr, nbytes, code):
    # zero bytes is a no-op that launches nothing, whatever the pointer
    assert getattr(lib, entry)(ptr, nbytes, None) == code


KB256 = 256 * 1024


@pytest.mark.parametrize("src,src_bytes,dst,dst_bytes,code", [
    (None, KB256, None, 0, binding.MOE_ERR_INVALID_ARG),            # NULL source
    (FAKE + 8, KB256, None, 0, binding.MOE_ERR_INVALID_ARG),        # misaligned source
    (FAKE, KB256 + 16, None, 0, binding.MOE_ERR_INVALID_ARG),       # not whole 256 KB items
    (FAKE, KB256, None, 16, binding.MOE_ERR_INVALID_ARG),           # NULL destination
    (FAKE, KB256, FAKE + 8, 16, binding.MOE_ERR_INVALID_ARG),       # misaligned destination
    (FAKE, KB256, FAKE + 2 * KB256, 24, binding.MOE_ERR_INVALID_ARG),   # destination not whole 16 bytes
    (FAKE, KB256, FAKE + 2 * KB256, 2 * KB256, binding.MOE_ERR_INVALID_ARG),  # writes more than it reads
    (FAKE, KB256, FAKE + KB256 - 16, 32, binding.MOE_ERR_INVALID_ARG),  # destination overlaps the source
    (FAKE, 0, None, 16, binding.MOE_ERR_INVALID_ARG),               # writes with nothing read
    (None, 0, None, 0, binding.MOE_OK),                              # nothing at all: a no-op
])
def test_read_write_probe_rejects_bad_arguments(lib, src, src_bytes, dst, dst_bytes, code):
    assert lib.moe_w8a8_read_write_probe(src, src_bytes, dst, dst_bytes, None) == code
