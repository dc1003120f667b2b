"""Seeded synthetic inputs for the W8A8 MoE expert block.

This module only draws inputs. It holds none of the block's arithmetic (no
quantisation, GEMM, activation or combine), so both the CPU oracle and the GPU
path can be fed from it without sharing any computation.

Workloads follow the decode shapes of the pages (FusedDeepMoE operator
signature, sec. 1.2 of "FusedDeepMoE Kernel 深度分析报告"; the W8A8 deployment
contract of "DeepSeek V4 Decode Optimization", sec. 0 "Freeze the deployment
contract first": 8 token rows, INT8 weights with FP32 per-output-channel
scales, per-token dynamic activation quantisation).

Distributions (one recipe for every case):
  x               bf16 = round-to-nearest-even of N(0, 1) in fp32
  expert weights  int8 = clamp(rint(32 * N(0, 1)), -127, 127)
  weight scales   fp32 ~ U[1e-3, 1e-2], one per output channel
  expert_ids      K distinct experts per token: uniform, or Zipf(s) over a
                  random permutation of the experts (weighted sampling without
                  replacement, Efraimidis-Spirakis keys)
  expert_scales   softmax over the K chosen experts of N(0, 1) logits
  smooth scales   fp32 ~ U[0.5, 2]
  x_active_mask   exactly `active` tokens set, at random positions
  FP4 weights     (weight_format "mxfp4") E2M1 codes uniform over all 16, two
                  per byte; E8M0 block scales (one per 32 K elements) uniform
                  over exponents 124..130 (2^-3 .. 2^3); fp32 per-channel
                  scales as above

Every array comes from its own numpy PCG64 stream keyed by
SeedSequence([seed, stream, index]); expert weights are drawn per global
expert id so that any subset can be materialised on its own.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# stream ids of SeedSequence([seed, stream, index])
S_IDS, S_ESCALE, S_X, S_W1, S_W1S, S_W2, S_W2S, S_MASK, S_SMOOTH = range(1, 10)
S_SW1, S_SW1S, S_SW2, S_SW2S, S_SSMOOTH, S_PERM = range(10, 16)
S_W1B, S_W2B, S_SW1B, S_SW2B = range(16, 20)

AMAX_EPS = 1e-6


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic workload."""
    name: str
    T: int            # tokens (rows of x)
    H: int            # hidden
    I: int            # routed expert intermediate; GEMM1 has 2*I outputs
    E_g: int          # global routed experts
    K: int            # top-k
    I_s: int = 0      # shared expert intermediate (0 = no shared expert)
    ep_size: int = 1  # expert-parallel group size: local experts = E_g / ep_size
    ep_rank: int = 0  # this rank owns [ep_rank*E_loc, (ep_rank+1)*E_loc)
    routing: str = "uniform"   # "uniform" | "zipf"
    zipf_s: float = 1.2
    active: Optional[int] = None   # number of active tokens (None = no mask)
    smooth: bool = False           # per-local-expert smooth scales [E_loc, H]
    share_smooth: bool = False     # shared-expert smooth scales [H]
    seed: int = 1234
    wseed: Optional[int] = None    # weight seed (defaults to seed)
    eps: float = AMAX_EPS
    fuse_route_scale: bool = False  # routing weight folded into the GEMM2 row scale
    weight_format: str = "int8"     # "int8" | "mxfp4" (FP4 weights, FP8 activations)
    quant_group: int = 0            # 0: one activation scale per row; G: per row and group of G
    requant_in_epilogue: bool = False  # requantise h in GEMM1's epilogue (decode GEMM) instead of its own launch

    @property
    def E_loc(self) -> int:
        return self.E_g // self.ep_size

    @property
    def weight_seed(self) -> int:
        return self.seed if self.wseed is None else self.wseed


# The five workloads (and a probe). Workloads 1, 3 and 4 are one model (same expert shapes),
# so they share a weight seed and one set of resident weights serves all three.
WORKLOADS = {
    0: Spec("tiny_w8a8_moe", T=8, H=512, I=256, E_g=8, K=2, seed=1234),
    1: Spec("v4flash_decode_t8", T=8, H=4096, I=2048, E_g=256, K=8, I_s=2048,
            seed=1235, wseed=1235),
    2: Spec("ep_rank_share_t128", T=128, H=4096, I=2048, E_g=256, K=8,
            ep_size=16, ep_rank=0, active=96, smooth=True, seed=1236),
    3: Spec("zipf_skew_t64", T=64, H=4096, I=2048, E_g=256, K=8, I_s=2048,
            routing="zipf", zipf_s=1.2, seed=1237, wseed=1235),
    4: Spec("large_batch_t512", T=512, H=4096, I=2048, E_g=256, K=8, I_s=2048,
            seed=1238, wseed=1235),
    # Supplementary compute-bound probe (not one of the pages' workloads):
    # every token picks all 8 experts, so each expert multiplies 512 rows and
    # the GEMMs do 2 * 512 int8 operations per weight byte, above the MI355X
    # ridge of about 625; it exercises the grouped GEMMs' MFMA throughput.
    5: Spec("mfma_probe_t512_e8", T=512, H=4096, I=2048, E_g=8, K=8, seed=1239),
}


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, index])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _int8_normal(rng: np.random.Generator, n: int) -> np.ndarray:
    z = rng.standard_normal(n, dtype=np.float32)
    z *= 32.0
    np.rint(z, out=z)
    np.clip(z, -127, 127, out=z)
    return z.astype(np.int8)


def _uniform_f32(rng: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, n).astype(np.float32)


def _fp4_pairs(rng: np.random.Generator, n: int) -> np.ndarray:
    """n / 2 bytes, each two E2M1 codes drawn uniformly over all 16."""
    return rng.integers(0, 256, n // 2, dtype=np.uint8)


def _e8m0(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(124, 131, n, dtype=np.uint8)


def _routing(spec: Spec) -> np.ndarray:
    """[T, K] int32 global expert ids, K distinct per token."""
    T, K, E = spec.T, spec.K, spec.E_g
    rng = _rng(spec.seed, S_IDS)
    if T == 0:
        return np.zeros((0, K), np.int32)
    if spec.routing == "uniform":
        keys = rng.random((T, E))
        ids = np.argsort(keys, axis=1, kind="stable")[:, :K]
    elif spec.routing == "zipf":
        perm = _rng(spec.seed, S_PERM).permutation(E)
        w = np.empty(E)
        w[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-spec.zipf_s)
        # weighted sampling without replacement: top-K of log(u)/w
        u = rng.random((T, E))
        keys = np.log(u) / w[None, :]
        ids = np.argsort(-keys, axis=1, kind="stable")[:, :K]
    else:
        raise ValueError(spec.routing)
    return ids.astype(np.int32)


def _expert_scales(spec: Spec) -> np.ndarray:
    rng = _rng(spec.seed, S_ESCALE)
    logits = rng.standard_normal((spec.T, spec.K))
    logits -= logits.max(axis=1, keepdims=True) if spec.T else 0
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p.astype(np.float32)


def expert_weights(spec: Spec, g: int):
    """Weights of global expert g: (w1 [2I,H] i8, w1s [2I] f32, w2 [H,I] i8, w2s [H] f32)."""
    s, H, I = spec.weight_seed, spec.H, spec.I
    w1 = _int8_normal(_rng(s, S_W1, g), 2 * I * H).reshape(2 * I, H)
    w1s = _uniform_f32(_rng(s, S_W1S, g), 2 * I, 1e-3, 1e-2)
    w2 = _int8_normal(_rng(s, S_W2, g), H * I).reshape(H, I)
    w2s = _uniform_f32(_rng(s, S_W2S, g), H, 1e-3, 1e-2)
    return w1, w1s, w2, w2s


def expert_weights_mx(spec: Spec, g: int):
    """FP4 weights of global expert g: (w1 [2I, H/2] u8, w1b [2I, H/32] u8,
    w1s [2I] f32, w2 [H, I/2] u8, w2b [H, I/32] u8, w2s [H] f32)."""
    s, H, I = spec.weight_seed, spec.H, spec.I
    w1 = _fp4_pairs(_rng(s, S_W1, g), 2 * I * H).reshape(2 * I, H // 2)
    w1b = _e8m0(_rng(s, S_W1B, g), 2 * I * H // 32).reshape(2 * I, H // 32)
    w1s = _uniform_f32(_rng(s, S_W1S, g), 2 * I, 1e-3, 1e-2)
    w2 = _fp4_pairs(_rng(s, S_W2, g), H * I).reshape(H, I // 2)
    w2b = _e8m0(_rng(s, S_W2B, g), H * I // 32).reshape(H, I // 32)
    w2s = _uniform_f32(_rng(s, S_W2S, g), H, 1e-3, 1e-2)
    return w1, w1b, w1s, w2, w2b, w2s


@dataclasses.dataclass
class Case:
    """One batch of inputs, all host numpy arrays in the ABI's layouts."""
    spec: Spec
    x: np.ndarray                 # uint16 bf16 bits [T, H]
    expert_ids: np.ndarray        # int32 [T, K] (global ids)
    expert_scales: np.ndarray     # fp32 [T, K]
    w1: np.ndarray                # int8 [E_loc, 2I, H]
    w1s: np.ndarray               # fp32 [E_loc, 2I]
    w2: np.ndarray                # int8 [E_loc, H, I]
    w2s: np.ndarray               # fp32 [E_loc, H]
    sw1: Optional[np.ndarray] = None   # int8 [2I_s, H]
    sw1s: Optional[np.ndarray] = None  # fp32 [2I_s]
    sw2: Optional[np.ndarray] = None   # int8 [H, I_s]
    sw2s: Optional[np.ndarray] = None  # fp32 [H]
    smooth: Optional[np.ndarray] = None        # fp32 [E_loc, H]
    share_smooth: Optional[np.ndarray] = None  # fp32 [H]
    mask: Optional[np.ndarray] = None          # uint8 [T]
    # weight_format "mxfp4": w1 / w2 / sw1 / sw2 hold E2M1 code pairs (uint8,
    # last dimension halved) and these their E8M0 block scales
    w1b: Optional[np.ndarray] = None   # uint8 [E_loc, 2I, H/32]
    w2b: Optional[np.ndarray] = None   # uint8 [E_loc, H, I/32]
    sw1b: Optional[np.ndarray] = None  # uint8 [2I_s, H/32]
    sw2b: Optional[np.ndarray] = None  # uint8 [H, I_s/32]

    @property
    def dims(self) -> dict:
        s = self.spec
        return dict(num_tokens=s.T, hidden=s.H, inter=s.I, share_inter=s.I_s, topk=s.K,
                    moe_expert_num=s.E_g, ep_rank_size=s.ep_size, ep_rank_id=s.ep_rank,
                    quant_mode=2 if s.quant_group else 1, amax_eps=s.eps, fuse_route_scale=int(s.fuse_route_scale),
                    weight_format=int(s.weight_format == "mxfp4"),
                    weight_layout=int(s.weight_format == "mxfp4"),  # FP4 weights are always packed
                    quant_group=s.quant_group, requant_in_epilogue=int(s.requant_in_epilogue))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_weights(spec: Spec, threads: Optional[int] = None):
    """All E_loc local experts, stacked: (w1, w1s, w2, w2s)."""
    E, H, I = spec.E_loc, spec.H, spec.I
    w1 = np.empty((E, 2 * I, H), np.int8)
    w2 = np.empty((E, H, I), np.int8)
    w1s = np.empty((E, 2 * I), np.float32)
    w2s = np.empty((E, H), np.float32)
    base = spec.ep_rank * E

    def fill(e):
        a, b, c, d = expert_weights(spec, base + e)
        w1[e], w1s[e], w2[e], w2s[e] = a, b, c, d

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(fill, range(E)))
    return w1, w1s, w2, w2s


def shared_weights(spec: Spec):
    if spec.I_s == 0:
        return None, None, None, None
    s, H, Is = spec.weight_seed, spec.H, spec.I_s
    sw1 = _int8_normal(_rng(s, S_SW1), 2 * Is * H).reshape(2 * Is, H)
    sw1s = _uniform_f32(_rng(s, S_SW1S), 2 * Is, 1e-3, 1e-2)
    sw2 = _int8_normal(_rng(s, S_SW2), H * Is).reshape(H, Is)
    sw2s = _uniform_f32(_rng(s, S_SW2S), H, 1e-3, 1e-2)
    return sw1, sw1s, sw2, sw2s


def make_activations(spec: Spec):
    """(x, expert_ids, expert_scales, mask, smooth, share_smooth) for one batch."""
    T, H = spec.T, spec.H
    x = f32_to_bf16_bits(_rng(spec.seed, S_X).standard_normal((T, H), dtype=np.float32))
    ids = _routing(spec)
    esc = _expert_scales(spec)
    mask = None
    if spec.active is not None:
        mask = np.zeros(T, np.uint8)
        on = _rng(spec.seed, S_MASK).permutation(T)[: spec.active]
        mask[on] = 1
    smooth = None
    if spec.smooth:
        smooth = _uniform_f32(_rng(spec.seed, S_SMOOTH), spec.E_loc * H, 0.5, 2.0).reshape(spec.E_loc, H)
    ssm = None
    if spec.share_smooth:
        ssm = _uniform_f32(_rng(spec.seed, S_SSMOOTH), H, 0.5, 2.0)
    return x, ids, esc, mask, smooth, ssm


def make_case_mx(spec: Spec) -> Case:
    """A case with FP4 weights (weight_format "mxfp4")."""
    x, ids, esc, mask, smooth, ssm = make_activations(spec)
    E, H, I, Is = spec.E_loc, spec.H, spec.I, spec.I_s
    w1 = np.empty((E, 2 * I, H // 2), np.uint8)
    w1b = np.empty((E, 2 * I, H // 32), np.uint8)
    w1s = np.empty((E, 2 * I), np.float32)
    w2 = np.empty((E, H, I // 2), np.uint8)
    w2b = np.empty((E, H, I // 32), np.uint8)
    w2s = np.empty((E, H), np.float32)

    def fill(e):
        w1[e], w1b[e], w1s[e], w2[e], w2b[e], w2s[e] = expert_weights_mx(spec, spec.ep_rank * E + e)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(E)))
    sw = [None] * 6
    if Is:
        s = spec.weight_seed
        sw = [_fp4_pairs(_rng(s, S_SW1), 2 * Is * H).reshape(2 * Is, H // 2),
              _e8m0(_rng(s, S_SW1B), 2 * Is * H // 32).reshape(2 * Is, H // 32),
              _uniform_f32(_rng(s, S_SW1S), 2 * Is, 1e-3, 1e-2),
              _fp4_pairs(_rng(s, S_SW2), H * Is).reshape(H, Is // 2),
              _e8m0(_rng(s, S_SW2B), H * Is // 32).reshape(H, Is // 32),
              _uniform_f32(_rng(s, S_SW2S), H, 1e-3, 1e-2)]
    return Case(spec, x, ids, esc, w1, w1s, w2, w2s, sw[0], sw[2], sw[3], sw[5], smooth, ssm, mask,
                w1b=w1b, w2b=w2b, sw1b=sw[1], sw2b=sw[4])


def make_case(spec: Spec, weights=None) -> Case:
    """Materialise a whole case. `weights` may pass a cached make_weights() result."""
    if spec.weight_format == "mxfp4":
        return make_case_mx(spec)
    x, ids, esc, mask, smooth, ssm = make_activations(spec)
    w1, w1s, w2, w2s = weights if weights is not None else make_weights(spec)
    sw1, sw1s, sw2, sw2s = shared_weights(spec)
    return Case(spec, x, ids, esc, w1, w1s, w2, w2s, sw1, sw1s, sw2, sw2s, smooth, ssm, mask)


def workload_case(i: int, weights=None) -> Case:
    return make_case(WORKLOADS[i], weights)
