"""ctypes binding of libmoe_w8a8 (include/moe_w8a8.h).

The entry points keep the C names: `moe_w8a8_workspace_size`,
`moe_w8a8_forward`, `moe_w8a8_status_string`. This module only marshals
arguments (torch device tensors -> device pointers, the current HIP stream);
every step of the block runs in the library's HIP kernels. There is no other
backend: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_w8a8.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_SCRATCH_LIMIT = -5
NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_W8A8_NOALLOC_SCRATCH_BYTES

EXPORTS = ("moe_w8a8_workspace_size", "moe_w8a8_forward", "moe_w8a8_forward_noalloc", "moe_w8a8_pack_weights",
           "moe_w8a8_packed_mx_bytes", "moe_w8a8_pack_weights_mx", "moe_w8a8_warm", "moe_w8a8_read_probe",
           "moe_w8a8_read_write_probe", "moe_w8a8_status_string")
MOE_WEIGHT_ROW_MAJOR, MOE_WEIGHT_PACKED = 0, 1
MOE_WEIGHT_INT8, MOE_WEIGHT_MXFP4 = 0, 1
MOE_PACK_GMM1, MOE_PACK_GMM2 = 1, 2


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {moe_w8a8_status_string(code)} ({code})")
        self.code = code


class Dims(ctypes.Structure):
    """moe_w8a8_dims_t"""
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("share_inter", ctypes.c_int32), ("topk", ctypes.c_int32), ("moe_expert_num", ctypes.c_int32),
                ("ep_rank_size", ctypes.c_int32), ("ep_rank_id", ctypes.c_int32), ("quant_mode", ctypes.c_int32),
                ("amax_eps", ctypes.c_float), ("weight_layout", ctypes.c_int32),
                ("fuse_route_scale", ctypes.c_int32), ("weight_format", ctypes.c_int32),
                ("quant_group", ctypes.c_int32), ("requant_in_epilogue", ctypes.c_int32)]

    @property
    def e_loc(self) -> int:
        return self.moe_expert_num // self.ep_rank_size


DEBUG_FIELDS = ("sorted_pair", "row_of_pair", "group_offset", "shared_token", "num_rows", "q_x", "xs", "acc1",
                "h", "q_h", "hs", "acc2", "z", "stage_events", "kernel_events")
STAGES = ("route_quant", "gemm1", "requant", "gemm2", "combine")


class Debug(ctypes.Structure):
    """moe_w8a8_debug_t"""
    _fields_ = [(n, ctypes.c_void_p) for n in DEBUG_FIELDS]


_lib = None


def library() -> ctypes.CDLL:
    """Open libmoe_w8a8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_expert_ffn_route_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.moe_w8a8_workspace_size.restype = ctypes.c_int
        L.moe_w8a8_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_w8a8_forward.restype = ctypes.c_int
        L.moe_w8a8_forward.argtypes = ([ctypes.POINTER(Dims)] + [P] * 18 + [ctypes.c_size_t, ctypes.POINTER(Debug), P])
        L.moe_w8a8_forward_noalloc.restype = ctypes.c_int
        L.moe_w8a8_forward_noalloc.argtypes = [ctypes.POINTER(Dims)] + [P] * 17 + [ctypes.POINTER(Debug), P]
        L.moe_w8a8_pack_weights.restype = ctypes.c_int
        L.moe_w8a8_pack_weights.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
        L.moe_w8a8_packed_mx_bytes.restype = ctypes.c_int
        L.moe_w8a8_packed_mx_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_size_t)]
        L.moe_w8a8_pack_weights_mx.restype = ctypes.c_int
        L.moe_w8a8_pack_weights_mx.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, P]
        L.moe_w8a8_warm.restype = ctypes.c_int
        L.moe_w8a8_warm.argtypes = [P, ctypes.c_size_t, P]
        L.moe_w8a8_read_probe.restype = ctypes.c_int
        L.moe_w8a8_read_probe.argtypes = [P, ctypes.c_size_t, P]
        L.moe_w8a8_read_write_probe.restype = ctypes.c_int
        L.moe_w8a8_read_write_probe.argtypes = [P, ctypes.c_size_t, P, ctypes.c_size_t, P]
        L.moe_w8a8_status_string.restype = ctypes.c_char_p
        L.moe_w8a8_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def make_dims(num_tokens, hidden, inter, topk, moe_expert_num, share_inter=0, ep_rank_size=1, ep_rank_id=0,
              quant_mode=1, amax_eps=1e-6, weight_layout=MOE_WEIGHT_ROW_MAJOR, fuse_route_scale=0,
              weight_format=MOE_WEIGHT_INT8, quant_group=0, requant_in_epilogue=0) -> Dims:
    return Dims(num_tokens, hidden, inter, share_inter, topk, moe_expert_num, ep_rank_size, ep_rank_id, quant_mode,
                amax_eps, weight_layout, fuse_route_scale, weight_format, quant_group, requant_in_epilogue)


def moe_w8a8_status_string(code: int) -> str:
    return library().moe_w8a8_status_string(code).decode()


def moe_w8a8_workspace_size(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    rc = library().moe_w8a8_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_workspace_size")
    return int(n.value)


def _stream(stream):
    """The HIP stream handle to pass: torch's current stream when None."""
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else stream


def moe_w8a8_pack_weights(src, which, dst=None, stream=None):
    """Pack an int8 weight tensor [groups, n, k] or [n, k] (device) into the
    kernels' streaming order; `which` is MOE_PACK_GMM1 for a gmm1 tensor and
    MOE_PACK_GMM2 for a gmm2 tensor. Returns dst (allocated like src if None)."""
    if dst is None:
        dst = torch.empty_like(src)
    shape = src.shape if src.dim() == 3 else (1, *src.shape)
    rc = library().moe_w8a8_pack_weights(_ptr(src), _ptr(dst), shape[0], shape[1], shape[2], which, _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_pack_weights")
    return dst


def moe_w8a8_warm(t, nbytes: Optional[int] = None, stream=None) -> None:
    """Warm the caches with a device tensor's bytes (or its first nbytes)."""
    n = t.numel() * t.element_size() if nbytes is None else nbytes
    rc = library().moe_w8a8_warm(_ptr(t), n, _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_warm")


def moe_w8a8_read_probe(t, nbytes: Optional[int] = None, stream=None) -> None:
    """Stream a device tensor's bytes (or its first nbytes) once and discard
    them (the read-bandwidth probe)."""
    n = t.numel() * t.element_size() if nbytes is None else nbytes
    rc = library().moe_w8a8_read_probe(_ptr(t), n, _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_read_probe")


def moe_w8a8_read_write_probe(src, src_bytes: int, dst=None, dst_bytes: int = 0, stream=None) -> None:
    """Read src_bytes of a device tensor in 256 KB work items and write dst_bytes
    of another (arbitrary values) in equal shares at the items' ends: the
    larger-batch GEMMs' read and write mix, for measurement."""
    rc = library().moe_w8a8_read_write_probe(_ptr(src), src_bytes, _ptr(dst), dst_bytes, _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_read_write_probe")


def moe_w8a8_packed_mx_bytes(groups: int, n: int, k: int) -> int:
    b = ctypes.c_size_t(0)
    rc = library().moe_w8a8_packed_mx_bytes(groups, n, k, ctypes.byref(b))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_packed_mx_bytes")
    return int(b.value)


def moe_w8a8_pack_weights_mx(data, block_scale, which, dst=None, stream=None):
    """Pack FP4 weights (uint8 E2M1 pairs [groups, n, k/2] or [n, k/2], E8M0
    block scales [.., n, k/32], device tensors) into one buffer for
    weight_format MOE_WEIGHT_MXFP4. Returns dst (uint8, allocated if None)."""
    shape = data.shape if data.dim() == 3 else (1, *data.shape)
    groups, n, k = shape[0], shape[1], 2 * shape[2]
    if dst is None:
        dst = torch.empty(moe_w8a8_packed_mx_bytes(groups, n, k), dtype=torch.uint8, device=data.device)
    rc = library().moe_w8a8_pack_weights_mx(_ptr(data), _ptr(block_scale), _ptr(dst), groups, n, k, which,
                                            _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_pack_weights_mx")
    return dst


def pack_weights(tensors: dict, stream=None) -> dict:
    """Return a copy of an upload() dict whose four weight tensors are packed."""
    out = dict(tensors)
    for k in ("gmm1_weight", "gmm2_weight", "share_gmm1_weight", "share_gmm2_weight"):
        if out.get(k) is not None:
            out[k] = moe_w8a8_pack_weights(out[k], MOE_PACK_GMM1 if "gmm1" in k else MOE_PACK_GMM2, stream=stream)
    return out


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors passed to libmoe_w8a8 must be device tensors")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe_w8a8 must be contiguous")
    return t.data_ptr()


def moe_w8a8_forward(dims: Dims, x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale, gmm2_weight,
                     gmm2_weight_scale, share_gmm1_weight=None, share_gmm1_weight_scale=None,
                     share_gmm2_weight=None, share_gmm2_weight_scale=None, expert_smooth_scales=None,
                     share_smooth_scales=None, x_active_mask=None, output=None, share_output=None,
                     expert_token_nums=None, workspace=None, workspace_bytes: Optional[int] = None,
                     dbg: Optional[Debug] = None, stream=None, check: bool = True) -> int:
    """Call the C entry point with device tensors (or raw device addresses).
    Returns the status code; raises MoeError on failure when check=True."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale, gmm2_weight, gmm2_weight_scale,
            share_gmm1_weight, share_gmm1_weight_scale, share_gmm2_weight, share_gmm2_weight_scale,
            expert_smooth_scales, share_smooth_scales, x_active_mask, output, share_output, expert_token_nums,
            workspace]
    rc = library().moe_w8a8_forward(ctypes.byref(dims), *[_ptr(a) for a in args], workspace_bytes,
                                    ctypes.byref(dbg) if dbg is not None else None, _stream(stream))
    if check and rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_forward")
    return rc


def moe_w8a8_forward_noalloc(dims: Dims, x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale,
                             gmm2_weight, gmm2_weight_scale, share_gmm1_weight=None, share_gmm1_weight_scale=None,
                             share_gmm2_weight=None, share_gmm2_weight_scale=None, expert_smooth_scales=None,
                             share_smooth_scales=None, x_active_mask=None, output=None, share_output=None,
                             expert_token_nums=None, dbg: Optional[Debug] = None, stream=None,
                             check: bool = True) -> int:
    """Call the entry point that takes no workspace (the library's built-in
    per-device scratch array). Returns the status code; raises MoeError on
    failure when check=True."""
    args = [x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale, gmm2_weight, gmm2_weight_scale,
            share_gmm1_weight, share_gmm1_weight_scale, share_gmm2_weight, share_gmm2_weight_scale,
            expert_smooth_scales, share_smooth_scales, x_active_mask, output, share_output, expert_token_nums]
    rc = library().moe_w8a8_forward_noalloc(ctypes.byref(dims), *[_ptr(a) for a in args],
                                            ctypes.byref(dbg) if dbg is not None else None, _stream(stream))
    if check and rc != MOE_OK:
        raise MoeError(rc, "moe_w8a8_forward_noalloc")
    return rc


# ---------------------------------------------------------------- helpers

def dims_of_case(case) -> Dims:
    """Dims of a moe_expert_ffn_route_amd.synth.Case."""
    return Dims(**case.dims)


def upload(case, device="cuda", weights=None) -> dict:
    """Copy a synth.Case's arrays to the device (weights may be passed in to
    reuse already resident tensors). Returns a dict of tensors keyed by the
    C argument names."""
    def t(a, dtype=None):
        if a is None:
            return None
        x = torch.from_numpy(a)
        if dtype is not None:
            x = x.view(dtype)
        return x.to(device, non_blocking=False).contiguous()

    d = dict(x=t(case.x, torch.bfloat16) if case.x.size else torch.empty(case.x.shape, dtype=torch.bfloat16,
                                                                          device=device),
             expert_ids=t(case.expert_ids), expert_scales=t(case.expert_scales),
             expert_smooth_scales=t(case.smooth), share_smooth_scales=t(case.share_smooth),
             x_active_mask=t(case.mask))
    if weights is None and case.w1b is None:
        weights = dict(gmm1_weight=t(case.w1), gmm1_weight_scale=t(case.w1s), gmm2_weight=t(case.w2),
                       gmm2_weight_scale=t(case.w2s), share_gmm1_weight=t(case.sw1),
                       share_gmm1_weight_scale=t(case.sw1s), share_gmm2_weight=t(case.sw2),
                       share_gmm2_weight_scale=t(case.sw2s))
    if weights is None and case.w1b is not None:
        # FP4 weights: element pairs and block scales packed into one buffer each
        weights = {}
        for name, data, bs in (("gmm1_weight", case.w1, case.w1b), ("gmm2_weight", case.w2, case.w2b),
                               ("share_gmm1_weight", case.sw1, case.sw1b),
                               ("share_gmm2_weight", case.sw2, case.sw2b)):
            if data is not None:
                weights[name] = moe_w8a8_pack_weights_mx(t(data), t(bs),
                                                         MOE_PACK_GMM1 if "gmm1" in name else MOE_PACK_GMM2)
        weights.update(gmm1_weight_scale=t(case.w1s), gmm2_weight_scale=t(case.w2s),
                       share_gmm1_weight_scale=t(case.sw1s), share_gmm2_weight_scale=t(case.sw2s))
        for k in ("share_gmm1_weight", "share_gmm2_weight"):
            weights.setdefault(k, None)
    d.update(weights)
    return d


class Runner:
    """Owns the outputs and workspace for repeated calls of one shape."""

    def __init__(self, dims: Dims, device="cuda"):
        self.dims = dims
        T, H = dims.num_tokens, dims.hidden
        self.output = torch.empty((T, H), dtype=torch.bfloat16, device=device)
        self.share_output = torch.empty((T, H), dtype=torch.bfloat16, device=device) if dims.share_inter else None
        self.expert_token_nums = torch.empty(dims.e_loc, dtype=torch.int32, device=device)
        self.workspace_bytes = moe_w8a8_workspace_size(dims)
        self.workspace = torch.empty(max(256, self.workspace_bytes), dtype=torch.uint8, device=device)
        assert self.workspace.data_ptr() % 256 == 0

    def __call__(self, tensors: dict, dbg: Optional[Debug] = None, stream=None):
        moe_w8a8_forward(self.dims, output=self.output, share_output=self.share_output,
                         expert_token_nums=self.expert_token_nums, workspace=self.workspace,
                         workspace_bytes=self.workspace_bytes, dbg=dbg, stream=stream, **tensors)
        return self.output, self.share_output, self.expert_token_nums


def debug_buffers(dims: Dims, device="cuda") -> tuple[Debug, dict]:
    """Allocate every intermediate buffer of moe_w8a8_debug_t."""
    T, K, H, E = dims.num_tokens, dims.topk, dims.hidden, dims.e_loc
    imax = max(dims.inter, dims.share_inter)
    R = T * K + T
    G = dims.quant_group if dims.quant_mode == 2 else 0
    ngx, ngh = (H // G, imax // G) if G else (1, 1)  # activation scales per row
    z = lambda *s, dt: torch.zeros(s, dtype=dt, device=device)
    bufs = dict(sorted_pair=z(max(1, T * K), dt=torch.int32), row_of_pair=z(max(1, T * K), dt=torch.int32),
                group_offset=z(E + 1, dt=torch.int32), shared_token=z(max(1, T), dt=torch.int32),
                num_rows=z(4, dt=torch.int32), q_x=z(max(1, R), H, dt=torch.int8),
                xs=z(max(1, R), ngx, dt=torch.float32) if G else z(max(1, R), dt=torch.float32),
                acc1=z(max(1, R), 2 * imax, dt=torch.int32), h=z(max(1, R), imax, dt=torch.float32),
                q_h=z(max(1, R), imax, dt=torch.int8),
                hs=z(max(1, R), ngh, dt=torch.float32) if G else z(max(1, R), dt=torch.float32),
                acc2=z(max(1, R), H, dt=torch.int32), z=z(max(1, R), H, dt=torch.int16))
    dbg = Debug(**{k: v.data_ptr() for k, v in bufs.items()})
    return dbg, bufs
