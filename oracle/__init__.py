"""CPU oracle of the W8A8 MoE expert block -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around `moe_oracle.c`, a plain single-threaded C model of the
block (see the header of that file for the passages each step follows). Only
`tests/`, the smoke entry and the benchmark's CPU-baseline leg may import this
package; the GPU library and its Python binding never do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (strict fp32: no contraction, no fast-math)."""
    hdr = os.path.join(HERE, "moe_oracle.h")
    fresh = (os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC)
             and os.path.getmtime(LIB) >= os.path.getmtime(hdr))
    if force or not fresh:
        tmp = LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("I_s", ctypes.c_int32), ("K", ctypes.c_int32), ("E_g", ctypes.c_int32),
                ("ep_size", ctypes.c_int32), ("ep_rank", ctypes.c_int32), ("eps", ctypes.c_float),
                ("fuse_route_scale", ctypes.c_int32), ("quant_group", ctypes.c_int32)]


class _Trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("sorted_pair", "row_of_pair", "offsets", "shared_token", "num_rows", "q_x", "xs",
                 "acc1", "h", "q_h", "hs", "acc2", "z")]


_lib = None


def load(path: str):
    """Open an oracle build and declare its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.moe_oracle_route.restype = ctypes.c_int32
    L.moe_oracle_route.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P]
    L.moe_oracle_quant_row.restype = None
    L.moe_oracle_quant_row.argtypes = [P, ctypes.c_int32, ctypes.c_float, P, P]
    L.moe_oracle_gemm_i8.restype = ctypes.c_int32
    L.moe_oracle_gemm_i8.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
    L.moe_oracle_swiglu.restype = None
    L.moe_oracle_swiglu.argtypes = [P, ctypes.c_int32, P]
    L.moe_oracle_forward.restype = ctypes.c_int32
    L.moe_oracle_forward.argtypes = [ctypes.POINTER(_Dims)] + [P] * 15 + [ctypes.c_int32] + [P] * 4
    L.moe_oracle_bf16_to_f32.restype = ctypes.c_float
    L.moe_oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.moe_oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.moe_oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    L.moe_oracle_forward_mx.restype = ctypes.c_int32
    L.moe_oracle_forward_mx.argtypes = [ctypes.POINTER(_Dims)] + [P] * 19 + [ctypes.c_int32] + [P] * 4
    L.moe_oracle_f32_to_e4m3.restype = ctypes.c_uint8
    L.moe_oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    L.moe_oracle_e4m3_to_f32.restype = ctypes.c_float
    L.moe_oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    L.moe_oracle_e2m1_to_f32.restype = ctypes.c_float
    L.moe_oracle_e2m1_to_f32.argtypes = [ctypes.c_uint8]
    L.moe_oracle_quant_row_fp8.restype = None
    L.moe_oracle_quant_row_fp8.argtypes = [P, ctypes.c_int32, ctypes.c_float, P, P]
    L.moe_oracle_gemm_mx.restype = None
    L.moe_oracle_gemm_mx.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
    L.moe_oracle_quant_row_groups.restype = None
    L.moe_oracle_quant_row_groups.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P, P]
    L.moe_oracle_gemm_i8_groups.restype = ctypes.c_int32
    L.moe_oracle_gemm_i8_groups.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
    return L


def lib():
    global _lib
    if _lib is None:
        _lib = load(build())
    return _lib


class using:
    """Context manager: route every call of this module to another oracle build
    (the tests use it to check that a deliberately broken copy fails its pins)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.prev = lib()
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def dims_of(T, H, I, K, E_g, I_s=0, ep_size=1, ep_rank=0, eps=1e-6, fuse_route_scale=False,
            quant_group=0) -> _Dims:
    return _Dims(T, H, I, I_s, K, E_g, ep_size, ep_rank, eps, int(bool(fuse_route_scale)), int(quant_group))


def _spec_dims(spec) -> _Dims:
    return dims_of(spec.T, spec.H, spec.I, spec.K, spec.E_g, spec.I_s, spec.ep_size, spec.ep_rank, spec.eps,
                   spec.fuse_route_scale, getattr(spec, "quant_group", 0))


def route(d: _Dims, expert_ids: np.ndarray, mask: Optional[np.ndarray] = None) -> dict:
    E = d.E_g // d.ep_size
    ids = _c(expert_ids, np.int32)
    m = _c(mask, np.uint8)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sp = np.zeros(max(1, d.T * d.K), np.int32)
    rop = np.zeros(max(1, d.T * d.K), np.int32)
    bad = ctypes.c_int32(0)
    P = lib().moe_oracle_route(ctypes.byref(d), _p(ids), _p(m), _p(counts), _p(offsets), _p(sp),
                               _p(rop), ctypes.addressof(bad))
    return dict(counts=counts, offsets=offsets, sorted_pair=sp[:P].copy(),
                row_of_pair=rop[: d.T * d.K].copy(), P=int(P), n_bad=int(bad.value))


def quant_row(v: np.ndarray, eps: float = 1e-6):
    v = _c(v, np.float32)
    q = np.zeros(v.shape[-1], np.int8)
    s = np.zeros(1, np.float32)
    lib().moe_oracle_quant_row(_p(v), v.shape[-1], eps, _p(q), _p(s))
    return q, np.float32(s[0])


def quant_rows(v: np.ndarray, eps: float = 1e-6):
    v = np.atleast_2d(_c(v, np.float32))
    q = np.zeros(v.shape, np.int8)
    s = np.zeros(v.shape[0], np.float32)
    for i in range(v.shape[0]):
        q[i], s[i] = quant_row(v[i], eps)
    return q, s


def gemm_i8(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C = A @ B.T exactly (A [M,K] int8, B [N,K] int8)."""
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    M, Kd = A.shape
    N = B.shape[0]
    C = np.zeros((M, N), np.int32)
    rc = lib().moe_oracle_gemm_i8(_p(A), _p(B), M, N, Kd, _p(C))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow")
    return C


def quant_row_groups(v: np.ndarray, G: int, eps: float = 1e-6):
    """Group-wise quantisation of one row: (codes, one scale per group of G)."""
    v = _c(v, np.float32)
    n = v.shape[-1]
    q = np.zeros(n, np.int8)
    s = np.zeros(n // G, np.float32)
    lib().moe_oracle_quant_row_groups(_p(v), n, G, eps, _p(q), _p(s))
    return q, s


def gemm_i8_groups(a: np.ndarray, a_scales: np.ndarray, B: np.ndarray, wscale: np.ndarray, G: int) -> np.ndarray:
    """One row through a GEMM with group-wise activation scales -> fp32 [N]."""
    a, B = _c(a, np.int8), _c(B, np.int8)
    a_scales, wscale = _c(a_scales, np.float32), _c(wscale, np.float32)
    N, Kd = B.shape
    y = np.zeros(N, np.float32)
    if lib().moe_oracle_gemm_i8_groups(_p(a), _p(a_scales), _p(B), _p(wscale), N, Kd, G, _p(y)) != 0:
        raise OverflowError("int32 partial overflow")
    return y


def swiglu(y: np.ndarray) -> np.ndarray:
    y = _c(y, np.float32)
    n = y.shape[-1] // 2
    h = np.zeros(n, np.float32)
    lib().moe_oracle_swiglu(_p(y), n, _p(h))
    return h


def bf16_to_f32(b: int) -> float:
    return lib().moe_oracle_bf16_to_f32(b)


def f32_to_bf16(f: float) -> int:
    return lib().moe_oracle_f32_to_bf16(f)


def default_threads() -> int:
    """Host threads for token-split oracle runs (at most 16)."""
    return max(1, min(16, os.cpu_count() or 1))


def forward(case, tokens: Optional[Sequence[int]] = None, trace: bool = False, threads: int = 1) -> dict:
    """Run the oracle on a synth.Case. tokens=None computes every output row.

    threads > 1 splits the tokens over that many host threads, each running
    the unchanged single-threaded C forward on its own token subset (ctypes
    releases the GIL). The C forward writes only the output and trace rows of
    the tokens it is given, so the threads share the per-row buffers (they
    write disjoint rows) and each gets its own routing outputs, which are
    identical and taken from the first thread. The result equals the
    single-threaded run bit for bit."""
    s = case.spec
    d = _spec_dims(s)
    T, H, K, E = s.T, s.H, s.K, s.E_loc
    Imax = max(s.I, s.I_s)
    rows_max = T * K + T
    out = np.zeros((T, H), np.uint16)
    sout = np.zeros((T, H), np.uint16) if s.I_s else None
    mx = getattr(s, "weight_format", "int8") == "mxfp4"
    G = getattr(s, "quant_group", 0)
    routing_keys = ("sorted_pair", "row_of_pair", "offsets", "shared_token", "num_rows")

    def routing_bufs():
        return dict(sorted_pair=np.full(max(1, T * K), -1, np.int32),
                    row_of_pair=np.full(max(1, T * K), -1, np.int32),
                    offsets=np.zeros(E + 1, np.int32), shared_token=np.full(max(1, T), -1, np.int32),
                    num_rows=np.zeros(3, np.int32))

    rows = {}
    if trace:
        rows = dict(q_x=np.zeros((rows_max, H), np.int8),
                    xs=np.zeros((rows_max, H // G), np.float32) if G else np.zeros(rows_max, np.float32),
                    acc1=np.zeros((rows_max, 2 * Imax), np.int32), h=np.zeros((rows_max, Imax), np.float32),
                    q_h=np.zeros((rows_max, Imax), np.int8),
                    hs=np.zeros((rows_max, Imax // G), np.float32) if G else np.zeros(rows_max, np.float32),
                    acc2=np.zeros((rows_max, H), np.int32), z=np.zeros((rows_max, H), np.uint16))
    if mx:
        keep = [_c(case.x, np.uint16), _c(case.expert_ids, np.int32), _c(case.expert_scales, np.float32),
                _c(case.w1, np.uint8), _c(case.w1b, np.uint8), _c(case.w1s, np.float32),
                _c(case.w2, np.uint8), _c(case.w2b, np.uint8), _c(case.w2s, np.float32),
                _c(case.sw1, np.uint8), _c(case.sw1b, np.uint8), _c(case.sw1s, np.float32),
                _c(case.sw2, np.uint8), _c(case.sw2b, np.uint8), _c(case.sw2s, np.float32),
                _c(case.smooth, np.float32), _c(case.share_smooth, np.float32), _c(case.mask, np.uint8)]
        fwd = lib().moe_oracle_forward_mx
    else:
        keep = [_c(case.x, np.uint16), _c(case.expert_ids, np.int32), _c(case.expert_scales, np.float32),
                _c(case.w1, np.int8), _c(case.w1s, np.float32), _c(case.w2, np.int8), _c(case.w2s, np.float32),
                _c(case.sw1, np.int8), _c(case.sw1s, np.float32), _c(case.sw2, np.int8), _c(case.sw2s, np.float32),
                _c(case.smooth, np.float32), _c(case.share_smooth, np.float32), _c(case.mask, np.uint8)]
        fwd = lib().moe_oracle_forward

    def run(sub):
        """One C forward over the token subset `sub` (None = all tokens)."""
        etn = np.zeros(E, np.int32)
        rb = routing_bufs() if trace else {}
        tr = _Trace(**{k: _p(v) for k, v in {**rb, **rows}.items()}) if trace else None
        rc = fwd(ctypes.byref(d), *[_p(a) for a in keep], _p(sub), 0 if sub is None else len(sub), _p(out),
                 _p(sout), _p(etn), ctypes.byref(tr) if tr is not None else None)
        if rc != 0:
            raise RuntimeError(f"oracle forward failed: {rc}")
        return etn, rb

    sub = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
    toks = np.arange(T, dtype=np.int32) if sub is None else sub
    n_thr = max(1, min(int(threads), len(toks)))
    if n_thr == 1:
        etn, rb = run(sub)
    else:
        from concurrent.futures import ThreadPoolExecutor
        parts = [np.ascontiguousarray(toks[i::n_thr]) for i in range(n_thr)]  # every token has K pairs
        with ThreadPoolExecutor(n_thr) as ex:
            results = list(ex.map(run, parts))
        etn, rb = results[0]
    res = dict(rb)
    res.update(rows)
    res.update(output=out, share_output=sout, expert_token_nums=etn)
    if trace:
        P, Ta = int(res["num_rows"][0]), int(res["num_rows"][1])
        res["sorted_pair"] = res["sorted_pair"][:P]
        res["shared_token"] = res["shared_token"][:Ta]
        res["P"], res["T_act"], res["n_bad"] = P, Ta, int(res["num_rows"][2])
        if mx:  # E4M3 codes and fp32 accumulators
            for k in ("q_x", "q_h"):
                res[k] = res[k].view(np.uint8)
        if mx or G:
            for k in ("acc1", "acc2"):
                res[k] = res[k].view(np.float32)
    return res


# FP8 / FP4 helpers of the FP4-weight variant (elementwise through the C oracle)
def f32_to_e4m3(a) -> np.ndarray:
    f = lib().moe_oracle_f32_to_e4m3
    a = np.asarray(a, np.float32)
    return np.array([f(float(v)) for v in a.reshape(-1)], np.uint8).reshape(a.shape)


def e4m3_to_f32(c) -> np.ndarray:
    f = lib().moe_oracle_e4m3_to_f32
    c = np.asarray(c, np.uint8)
    return np.array([f(int(v)) for v in c.reshape(-1)], np.float32).reshape(c.shape)


def e2m1_to_f32(c) -> np.ndarray:
    f = lib().moe_oracle_e2m1_to_f32
    c = np.asarray(c, np.uint8)
    return np.array([f(int(v)) for v in c.reshape(-1)], np.float32).reshape(c.shape)


def quant_row_fp8(v: np.ndarray, eps: float = 1e-6):
    v = np.ascontiguousarray(v, np.float32)
    q = np.zeros(v.shape, np.uint8)
    sc = np.zeros(1, np.float32)
    lib().moe_oracle_quant_row_fp8(_p(v), v.size, eps, _p(q), _p(sc))
    return q, float(sc[0])


def gemm_mx(A: np.ndarray, B: np.ndarray, S: np.ndarray) -> np.ndarray:
    """A [M, K] E4M3 codes, B [N, K/2] E2M1 pairs, S [N, K/32] E8M0 -> fp32 [M, N]."""
    A, B, S = (np.ascontiguousarray(x, np.uint8) for x in (A, B, S))
    M, K = A.shape
    N = B.shape[0]
    C = np.zeros((M, N), np.float32)
    lib().moe_oracle_gemm_mx(_p(A), _p(B), _p(S), M, N, K, _p(C))
    return C
