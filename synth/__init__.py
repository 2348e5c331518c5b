"""Seeded synthetic inputs for the routed MoE layer.

This module is shared input infrastructure: the CPU oracle's tests and the GPU
path both draw their inputs from it, and it holds none of the layer's own
arithmetic.  It only produces random bytes, uniform integers and normal samples
and rounds normals to the storage type a workload names.  It never interprets
an MXFP4 code or scale: a uniformly random byte *is* two uniformly random
4-bit codes, and a uniformly random integer in [118, 127] *is* an E8M0 code.

Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
as easy as 1, 2, 3", SC 2011), driven through numpy's implementation.  Every
tensor draws from its own key (seed, stream id, sub-index), so any expert's
weights can be regenerated on its own and in any order.  Normals use the
Box-Muller transform on pairs of 53-bit uniforms (both branches).

Stream ids: x 0, router weight 1, gate codes 2, gate scales 3, up codes 4,
up scales 5, down codes 6, down scales 7 (FP16 weights use 2, 4, 6); INT4
group-32 zero points 8, 9, 10 and NVFP4 tensor scales 11, 12, 13 (gate, up,
down).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

STREAM_X = 0
STREAM_ROUTER = 1
STREAM_GATE = 2
STREAM_GATE_SCALE = 3
STREAM_UP = 4
STREAM_UP_SCALE = 5
STREAM_DOWN = 6
STREAM_DOWN_SCALE = 7
STREAM_ZERO = {"gate": 8, "up": 9, "down": 10}
STREAM_TENSOR_SCALE = {"gate": 11, "up": 12, "down": 13}

_M64 = (1 << 64) - 1


def _key(seed: int, stream: int, sub: int) -> list[int]:
    # Two 64-bit key words; distinct (seed, stream, sub) give distinct keys.
    return [((seed & 0xFFFFFFFF) << 32) | (stream & 0xFFFFFFFF), sub & _M64]


def _gen(seed: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=_key(seed, stream, sub)))


def random_bytes(seed: int, stream: int, n: int, sub: int = 0) -> np.ndarray:
    """n independent uniform bytes (uint8): the little-endian bytes of consecutive 64-bit outputs."""
    n = int(n)
    words = _gen(seed, stream, sub).bit_generator.random_raw((n + 7) // 8).astype("<u8")
    return words.view(np.uint8)[:n].copy()


def uniform_uint(seed: int, stream: int, n: int, lo: int, hi: int, sub: int = 0) -> np.ndarray:
    """n independent integers uniform in [lo, hi] (multiply-shift on 32 random bits), as int64."""
    g = _gen(seed, stream, sub)
    r = g.bit_generator.random_raw(int(n)).astype(np.uint64) >> np.uint64(32)
    span = np.uint64(hi - lo + 1)
    return (lo + ((r * span) >> np.uint64(32))).astype(np.int64)


def uniform(seed: int, stream: int, n: int, lo: float, hi: float, sub: int = 0) -> np.ndarray:
    """n independent float64 values uniform in [lo, hi) (53-bit uniforms)."""
    g = _gen(seed, stream, sub)
    u = (g.bit_generator.random_raw(int(n)) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    return lo + (hi - lo) * u


def normal(seed: int, stream: int, n: int, std: float = 1.0, sub: int = 0) -> np.ndarray:
    """n independent N(0, std^2) samples in float64.

    Box-Muller on pairs of 53-bit uniforms: pair i gives sample 2i (cosine branch) and
    sample 2i+1 (sine branch)."""
    n = int(n)
    m = (n + 1) // 2
    g = _gen(seed, stream, sub)
    raw = g.bit_generator.random_raw(2 * m).reshape(m, 2)
    u1 = ((raw[:, 0] >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)
    u2 = (raw[:, 1] >> np.uint64(11)).astype(np.float64) * (2.0 * math.pi / 9007199254740992.0)
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty((m, 2), dtype=np.float64)
    np.multiply(r, np.cos(u2), out=out[:, 0])
    np.multiply(r, np.sin(u2), out=out[:, 1])
    out = out.reshape(-1)[:n]
    if std != 1.0:
        out *= std
    return out


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 storage (via float32, round-to-nearest-even); uint16 bits."""
    f = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (f + np.uint64(0x7FFF) + ((f >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to IEEE binary16 storage (numpy's round-to-nearest-even); uint16 bits."""
    return np.asarray(a, dtype=np.float16).view(np.uint16)


# --------------------------------------------------------------------------------------------
# Workloads.  Shapes and value distributions of the routed-MoE layer configurations; every
# tensor is drawn with seed 0 unless a caller asks otherwise.
# --------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hidden: int            # H
    n_routed: int          # E
    top_k: int             # k
    n_shared: int          # S (always-on experts appended after the k routed slots)
    inter: int             # I, per-expert SwiGLU intermediate size
    weight_format: str     # "mxfp4", "fp16", "int4g32" or "nvfp4"
    act_dtype: str         # "bf16" or "fp16"
    router_std: float      # standard deviation of router weight entries
    zipf_s: float = 0.0    # >0: logit bias b_e = -s * ln(e + 1)
    weight_std: float = 0.02  # FP16 weights only
    scale_lo: int = 118    # E8M0 codes uniform in [scale_lo, scale_hi]
    scale_hi: int = 127
    dense_slices: bool = False  # FP16 dense FFN cut into all-active slices
    tokens: tuple = ()

    @property
    def n_experts(self) -> int:
        return self.n_routed + self.n_shared

    @property
    def k_total(self) -> int:
        return self.top_k + self.n_shared


WORKLOADS = {
    "tiny": Workload("tiny", 256, 8, 2, 0, 512, "mxfp4", "bf16", 0.02, tokens=(16,)),
    "decode": Workload("decode", 4096, 128, 8, 0, 1536, "mxfp4", "bf16", 0.02, tokens=(1, 8, 32, 64)),
    "prefill": Workload("prefill", 7168, 256, 8, 1, 2048, "mxfp4", "bf16", 0.02, zipf_s=1.2,
                        tokens=(8192,)),
    "dense_slices": Workload("dense_slices", 4096, 8, 8, 0, 2048, "fp16", "fp16", 0.0,
                             dense_slices=True, tokens=(1, 16, 128)),
    "sweep": Workload("sweep", 7168, 256, 8, 0, 2048, "mxfp4", "bf16", 1.0 / math.sqrt(7168.0),
                      tokens=(1, 8, 15, 32, 64, 88, 128, 176)),
}


def custom(name="custom", hidden=256, n_routed=8, top_k=2, n_shared=0, inter=512, weight_format="mxfp4",
           act_dtype="bf16", router_std=0.02, zipf_s=0.0, weight_std=0.02, scale_lo=118, scale_hi=127,
           dense_slices=False) -> Workload:
    return Workload(name, hidden, n_routed, top_k, n_shared, inter, weight_format, act_dtype, router_std,
                    zipf_s, weight_std, scale_lo, scale_hi, dense_slices, ())


@dataclasses.dataclass
class LayerInputs:
    """Host copies of one layer's inputs, in the exact storage the library consumes.

    x: uint16 [T][H] (bf16 or fp16 bits).  router: float32 [E][H].  bias: float32 [E] or None.
    MXFP4: *_codes uint8 [E'][N][K/2] (two codes per byte), *_scales uint8 [E'][N][K/32].
    FP16:  *_codes uint16 [E'][N][K] (binary16 bits), *_scales None.
    INT4_G32: *_codes uint8 [E'][N][K/2] (unsigned codes), *_scales uint16 [E'][N][K/32] (binary16
           bits), extras[m] uint8 [E'][N][ceil(K/64)] zero points (group 2j in the low nibble).
    NVFP4: *_codes uint8 [E'][N][K/2] (E2M1), *_scales uint8 [E'][N][K/16] (E4M3 bits),
           extras[m] float32 [E'] tensor scales.
    gate/up have N = I, K = H; down has N = H, K = I.
    """
    wl: Workload
    T: int
    x: np.ndarray
    router: Optional[np.ndarray]
    bias: Optional[np.ndarray]
    gate_codes: np.ndarray
    gate_scales: Optional[np.ndarray]
    up_codes: np.ndarray
    up_scales: Optional[np.ndarray]
    down_codes: np.ndarray
    down_scales: Optional[np.ndarray]
    extras: Optional[dict] = None


def make_x(wl: Workload, T: int, seed: int = 0) -> np.ndarray:
    z = normal(seed, STREAM_X, T * wl.hidden).reshape(T, wl.hidden)
    return to_bf16_bits(z) if wl.act_dtype == "bf16" else to_f16_bits(z)


def make_router(wl: Workload, seed: int = 0):
    if wl.dense_slices:
        return None, None
    w = normal(seed, STREAM_ROUTER, wl.n_routed * wl.hidden, std=wl.router_std)
    w = w.astype(np.float32).reshape(wl.n_routed, wl.hidden)
    bias = None
    if wl.zipf_s > 0:
        bias = (-wl.zipf_s * np.log(np.arange(wl.n_routed, dtype=np.float64) + 1.0)).astype(np.float32)
    return w, bias


def make_expert_matrix(wl: Workload, which: str, expert: int, seed: int = 0):
    """One expert's (codes, scales) for which in {"gate","up","down"}; scales None for FP16."""
    H, I = wl.hidden, wl.inter
    N, K = (I, H) if which in ("gate", "up") else (H, I)
    stream = {"gate": STREAM_GATE, "up": STREAM_UP, "down": STREAM_DOWN}[which]
    if wl.weight_format == "mxfp4":
        codes = random_bytes(seed, stream, N * K // 2, sub=expert).reshape(N, K // 2)
        sc = uniform_uint(seed, stream + 1, N * K // 32, wl.scale_lo, wl.scale_hi, sub=expert)
        return codes, sc.astype(np.uint8).reshape(N, K // 32)
    if wl.weight_format == "int4g32":
        codes = random_bytes(seed, stream, N * K // 2, sub=expert).reshape(N, K // 2)
        sc = to_f16_bits(uniform(seed, stream + 1, N * K // 32, INT4_SCALE_LO, INT4_SCALE_HI, sub=expert))
        return codes, sc.reshape(N, K // 32)
    if wl.weight_format == "nvfp4":
        codes = random_bytes(seed, stream, N * K // 2, sub=expert).reshape(N, K // 2)
        sc = uniform_uint(seed, stream + 1, N * K // 16, NVFP4_SCALE_CODE_LO, NVFP4_SCALE_CODE_HI, sub=expert)
        return codes, sc.astype(np.uint8).reshape(N, K // 16)
    z = normal(seed, stream, N * K, std=wl.weight_std, sub=expert).reshape(N, K)
    return to_f16_bits(z), None


# INT4 group-32: binary16 scales uniform in [0.002, 0.004) and zero points uniform in 0..15, so
# with uniform codes a weight (code - zero) * scale has a standard deviation of about 0.02.
INT4_SCALE_LO, INT4_SCALE_HI = 0.002, 0.004
# NVFP4: E4M3 scale codes uniform over 0x28 .. 0x3F (0.25 .. 1.875) and fp32 tensor scales
# uniform in [0.005, 0.01) per expert (weights of standard deviation about 0.02).
NVFP4_SCALE_CODE_LO, NVFP4_SCALE_CODE_HI = 0x28, 0x3F
NVFP4_TENSOR_SCALE_LO, NVFP4_TENSOR_SCALE_HI = 0.005, 0.01


def make_expert_extra(wl: Workload, which: str, expert: int, seed: int = 0):
    """INT4 group-32: the zero points of one expert's matrix ([N][ceil(K/64)] bytes, group 2j in
    the low nibble); NVFP4: its tensor scale (float32 scalar); None for other formats."""
    H, I = wl.hidden, wl.inter
    N, K = (I, H) if which in ("gate", "up") else (H, I)
    if wl.weight_format == "int4g32":
        g = K // 32
        z = uniform_uint(seed, STREAM_ZERO[which], N * g, 0, 15, sub=expert).reshape(N, g)
        if g % 2:
            z = np.concatenate([z, np.zeros((N, 1), np.int64)], axis=1)
        return (z[:, 0::2] | (z[:, 1::2] << 4)).astype(np.uint8)
    if wl.weight_format == "nvfp4":
        return np.float32(uniform(seed, STREAM_TENSOR_SCALE[which], 1, NVFP4_TENSOR_SCALE_LO, NVFP4_TENSOR_SCALE_HI,
                                  sub=expert)[0])
    return None


def make_dense_fp16(wl: Workload, seed: int = 0):
    """Unsliced dense FFN weights for the all-active-slices workload:
    gate, up: [n_slices*I][H]; down: [H][n_slices*I]; binary16 bits.
    Slice j of gate/up is rows [j*I, (j+1)*I); slice j of down is columns [j*I, (j+1)*I)."""
    assert wl.dense_slices and wl.weight_format == "fp16"
    H, Id = wl.hidden, wl.inter * wl.n_routed
    g = to_f16_bits(normal(seed, STREAM_GATE, Id * H, std=wl.weight_std)).reshape(Id, H)
    u = to_f16_bits(normal(seed, STREAM_UP, Id * H, std=wl.weight_std)).reshape(Id, H)
    d = to_f16_bits(normal(seed, STREAM_DOWN, H * Id, std=wl.weight_std)).reshape(H, Id)
    return g, u, d


def make_layer(wl: Workload, T: int, seed: int = 0, experts=None) -> LayerInputs:
    """All inputs of one layer call with T tokens.  experts: restrict weight generation to this
    iterable of expert ids (other experts are left zero) -- for sampled checks at full size."""
    x = make_x(wl, T, seed)
    router, bias = make_router(wl, seed)
    E2, H, I = wl.n_experts, wl.hidden, wl.inter
    if wl.dense_slices:
        g, u, d = make_dense_fp16(wl, seed)
        gate = np.ascontiguousarray(g.reshape(E2, I, H))
        up = np.ascontiguousarray(u.reshape(E2, I, H))
        down = np.ascontiguousarray(d.reshape(H, E2, I).transpose(1, 0, 2))
        return LayerInputs(wl, T, x, None, None, gate, None, up, None, down, None)
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    extras = None
    if wl.weight_format == "mxfp4":
        codes = {k: np.zeros((E2, n, kk // 2), np.uint8) for k, (n, kk) in shapes.items()}
        scales = {k: np.zeros((E2, n, kk // 32), np.uint8) for k, (n, kk) in shapes.items()}
    elif wl.weight_format == "int4g32":
        codes = {k: np.zeros((E2, n, kk // 2), np.uint8) for k, (n, kk) in shapes.items()}
        scales = {k: np.zeros((E2, n, kk // 32), np.uint16) for k, (n, kk) in shapes.items()}
        extras = {k: np.zeros((E2, n, (kk // 32 + 1) // 2), np.uint8) for k, (n, kk) in shapes.items()}
    elif wl.weight_format == "nvfp4":
        codes = {k: np.zeros((E2, n, kk // 2), np.uint8) for k, (n, kk) in shapes.items()}
        scales = {k: np.zeros((E2, n, kk // 16), np.uint8) for k, (n, kk) in shapes.items()}
        extras = {k: np.zeros(E2, np.float32) for k in shapes}
    else:
        codes = {k: np.zeros((E2, n, kk), np.uint16) for k, (n, kk) in shapes.items()}
        scales = {k: None for k in shapes}

    def fill(job):
        e, k = job
        c, s = make_expert_matrix(wl, k, e, seed)
        codes[k][e] = c
        if s is not None:
            scales[k][e] = s
        if extras is not None:
            extras[k][e] = make_expert_extra(wl, k, e, seed)

    jobs = [(e, k) for e in (range(E2) if experts is None else experts) for k in shapes]
    # every (expert, matrix) has its own generator key, so the order of the jobs does not matter
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, jobs))
    return LayerInputs(wl, T, x, router, bias, codes["gate"], scales["gate"], codes["up"], scales["up"],
                       codes["down"], scales["down"], extras)


def to_torch(L: LayerInputs, device) -> dict:
    """Upload LayerInputs to torch tensors on `device` (bf16/fp16 activations, uint8 codes and scales
    or fp16 weights, fp32 router).  For the all-active-slices workload the expert views are slices
    of the unsliced dense matrices: gate/up rows and down columns, exactly as stored densely."""
    import torch

    def t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)

    act = torch.bfloat16 if L.wl.act_dtype == "bf16" else torch.float16
    out = {"x": t(L.x).view(act), "router": t(L.router), "bias": t(L.bias), "weight_format": L.wl.weight_format}
    if L.wl.dense_slices:
        E2, I, H = L.gate_codes.shape
        g = t(L.gate_codes.reshape(E2 * I, H)).view(torch.float16)
        u = t(L.up_codes.reshape(E2 * I, H)).view(torch.float16)
        d = t(np.ascontiguousarray(L.down_codes.transpose(1, 0, 2)).reshape(H, E2 * I)).view(torch.float16)
        out.update(dense_gate=g, dense_up=u, dense_down=d,
                   gate=g.view(E2, I, H), up=u.view(E2, I, H),
                   down=d.as_strided((E2, H, I), (I, E2 * I, 1)),
                   gate_scales=None, up_scales=None, down_scales=None)
        return out
    if L.wl.weight_format == "fp16":
        out.update(gate=t(L.gate_codes).view(torch.float16), up=t(L.up_codes).view(torch.float16),
                   down=t(L.down_codes).view(torch.float16), gate_scales=None, up_scales=None, down_scales=None)
    elif L.extras is not None:
        out.update(gate=t(L.gate_codes), up=t(L.up_codes), down=t(L.down_codes),
                   gate_scales=t(L.gate_scales.view(np.uint8)), up_scales=t(L.up_scales.view(np.uint8)),
                   down_scales=t(L.down_scales.view(np.uint8)),
                   extras={k: t(v) for k, v in L.extras.items()})
    else:
        out.update(gate=t(L.gate_codes), up=t(L.up_codes), down=t(L.down_codes), gate_scales=t(L.gate_scales),
                   up_scales=t(L.up_scales), down_scales=t(L.down_scales))
    return out
