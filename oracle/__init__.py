"""fp64 CPU oracle of the routed Mixture-of-Experts FFN layer (numpy front end over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may
import it; the library in mxfp4_routed_expert_router_amd never does, and the oracle never imports
the library.  It shares no code with the HIP path; only the seeded input generator (synth) is
common to both.

What each function computes, and the passage of the pages it follows, is stated in moe_oracle.h
and moe_oracle.c.  Parity status: every function here is pinned by tests/test_oracle_pins.py to
values the pages fix, closed forms, library routines or brute force; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "moe_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

X_BF16, X_FP16 = 0, 1
W_MXFP4, W_FP16, W_INT4_G32, W_NVFP4 = 0, 1, 2, 3
W_FORMATS = {"mxfp4": W_MXFP4, "fp16": W_FP16, "int4g32": W_INT4_G32, "nvfp4": W_NVFP4}
MX_FP8_E4M3, MX_FP4_E2M1, MX_FP6_E2M3 = 1, 2, 3

_CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared"]


def build(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc (plain IEEE arithmetic: no fast-math, no FMA contraction)."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", *_CFLAGS, "-I", HERE, source, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


class _Proj(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("w_expert_stride", ctypes.c_int64), ("w_row_stride", ctypes.c_int64),
                ("s_expert_stride", ctypes.c_int64), ("s_row_stride", ctypes.c_int64),
                ("zeros", ctypes.c_void_p), ("z_expert_stride", ctypes.c_int64), ("z_row_stride", ctypes.c_int64),
                ("tensor_scale", ctypes.c_void_p)]


class _Weights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("n_experts", ctypes.c_int), ("hidden", ctypes.c_int),
                ("inter", ctypes.c_int), ("gate", _Proj), ("up", _Proj), ("down", _Proj)]


class ExpertWeights:
    """Holds the numpy arrays (kept alive) and the C struct describing them.

    codes: [E'][N][K/2] uint8 (MXFP4, INT4_G32, NVFP4) or [E'][N][K] uint16 (FP16), possibly a
    strided view whose innermost dimension is contiguous; scales: [E'][N][K/32] uint8 (MXFP4),
    [E'][N][K/32] binary16 bits as uint16 (INT4_G32), [E'][N][K/16] uint8 E4M3 (NVFP4) or None;
    extras (per projection, INT4_G32: zero points [E'][N][K/64] uint8; NVFP4: tensor scales [E']
    float32)."""

    def __init__(self, fmt, gate, gate_s, up, up_s, down, down_s, extras=None):
        extras = dict(extras or {})
        if fmt == W_NVFP4:
            extras = {k: np.ascontiguousarray(v, np.float32) for k, v in extras.items()}
        self.keep = [gate, gate_s, up, up_s, down, down_s, extras]
        E2, I = gate.shape[0], gate.shape[1]
        H = down.shape[1]
        self.n_experts, self.hidden, self.inter, self.fmt = E2, H, I, fmt

        def proj(c, s, ex):
            assert c.strides[-1] == c.itemsize
            p = _Proj()
            p.w = c.ctypes.data
            p.w_expert_stride, p.w_row_stride = c.strides[0], c.strides[1]
            if s is not None:
                assert s.strides[-1] == s.itemsize
                p.scales = s.ctypes.data
                p.s_expert_stride, p.s_row_stride = s.strides[0], s.strides[1]
            if ex is not None and fmt == W_INT4_G32:
                p.zeros = ex.ctypes.data
                p.z_expert_stride, p.z_row_stride = ex.strides[0], ex.strides[1]
            if ex is not None and fmt == W_NVFP4:
                p.tensor_scale = ex.ctypes.data
            return p

        self.c = _Weights(fmt, E2, H, I, proj(gate, gate_s, extras.get("gate")), proj(up, up_s, extras.get("up")),
                          proj(down, down_s, extras.get("down")))

    @classmethod
    def from_layer(cls, L) -> "ExpertWeights":
        fmt = W_FORMATS[L.wl.weight_format]
        return cls(fmt, L.gate_codes, L.gate_scales, L.up_codes, L.up_scales, L.down_codes, L.down_scales,
                   getattr(L, "extras", None))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        self.lib = lib
        d, i, vp = ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        lib.orc_e2m1.restype = d; lib.orc_e2m1.argtypes = [i]
        lib.orc_e8m0.restype = d; lib.orc_e8m0.argtypes = [i]
        lib.orc_mxfp4.restype = d; lib.orc_mxfp4.argtypes = [i, i]
        lib.orc_bf16.restype = d; lib.orc_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_f16.restype = d; lib.orc_f16.argtypes = [ctypes.c_uint16]
        lib.orc_silu.restype = d; lib.orc_silu.argtypes = [d]
        lib.orc_mxfp4_bits_per_weight.restype = d; lib.orc_mxfp4_bits_per_weight.argtypes = []
        lib.orc_int4g32_bits_per_weight.restype = d; lib.orc_int4g32_bits_per_weight.argtypes = []
        lib.orc_nvfp4_bits_per_weight.restype = d; lib.orc_nvfp4_bits_per_weight.argtypes = []
        lib.orc_mxfp4_bytes.restype = ctypes.c_int64
        lib.orc_mxfp4_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
        lib.orc_num_threads.restype = i; lib.orc_num_threads.argtypes = []
        lib.orc_set_num_threads.restype = None; lib.orc_set_num_threads.argtypes = [i]
        lib.orc_route.restype = None
        lib.orc_route.argtypes = [vp, i, i, i, vp, vp, i, i, i, d, vp, vp, vp, vp, vp]
        lib.orc_route_sigmoid.restype = None
        lib.orc_route_sigmoid.argtypes = [vp, i, i, i, vp, vp, i, i, i, d, d, d, vp, vp, vp, vp]
        lib.orc_bucket.restype = i
        lib.orc_bucket.argtypes = [vp, i, i, vp, vp, vp, vp]
        lib.orc_expert_apply.restype = None
        lib.orc_expert_apply.argtypes = [ctypes.POINTER(_Weights), i, vp, vp]
        lib.orc_expert_ffn.restype = None
        lib.orc_expert_ffn.argtypes = [vp, i, i, i, ctypes.POINTER(_Weights), vp, vp, vp, vp]
        lib.orc_combine.restype = None
        lib.orc_combine.argtypes = [vp, vp, i, i, i, vp, vp]
        lib.orc_layer_bruteforce.restype = None
        lib.orc_layer_bruteforce.argtypes = [vp, i, i, i, ctypes.POINTER(_Weights), vp, vp, vp]
        lib.orc_layer_dense_mixture.restype = None
        lib.orc_layer_dense_mixture.argtypes = [vp, i, i, i, ctypes.POINTER(_Weights), vp, vp, vp]
        lib.orc_dense_ffn_f16.restype = None
        lib.orc_dense_ffn_f16.argtypes = [vp, i, i, i, i, vp, vp, vp, vp]
        lib.orc_weight.restype = d
        lib.orc_weight.argtypes = [ctypes.POINTER(_Proj), i, i, i, i]
        lib.orc_mxfp4_decode_matrix.restype = None
        lib.orc_mxfp4_decode_matrix.argtypes = [vp, vp, i, i, vp]
        lib.orc_mx_bits.restype = i; lib.orc_mx_bits.argtypes = [i]
        lib.orc_mx_emax.restype = i; lib.orc_mx_emax.argtypes = [i]
        lib.orc_mx_value.restype = d; lib.orc_mx_value.argtypes = [i, i]
        lib.orc_mx_encode.restype = i; lib.orc_mx_encode.argtypes = [i, d]
        lib.orc_mx_scale_code.restype = i; lib.orc_mx_scale_code.argtypes = [i, d]
        lib.orc_mx_quantize.restype = None; lib.orc_mx_quantize.argtypes = [vp, i, i, i, vp, vp]
        lib.orc_mx_dequantize.restype = None; lib.orc_mx_dequantize.argtypes = [vp, vp, i, i, i, vp]
        lib.orc_expert_ffn_attenuated.restype = None
        lib.orc_expert_ffn_attenuated.argtypes = [vp, i, i, i, ctypes.POINTER(_Weights), i, vp, vp, vp, vp]
        lib.orc_row_factor.restype = d; lib.orc_row_factor.argtypes = [vp, i]
        lib.orc_combine_restore.restype = None
        lib.orc_combine_restore.argtypes = [vp, vp, i, i, i, i, vp, vp]
        lib.orc_expert_ffn_mx.restype = None
        lib.orc_expert_ffn_mx.argtypes = [vp, i, i, i, ctypes.POINTER(_Weights), i, vp, vp, vp, vp, vp]

    # ---- formats ----
    def e2m1(self, c: int) -> float: return self.lib.orc_e2m1(c)
    def e8m0(self, e: int) -> float: return self.lib.orc_e8m0(e)
    def mxfp4(self, c: int, e: int) -> float: return self.lib.orc_mxfp4(c, e)
    def bf16(self, b: int) -> float: return self.lib.orc_bf16(b)
    def f16(self, b: int) -> float: return self.lib.orc_f16(b)
    def silu(self, z: float) -> float: return self.lib.orc_silu(z)
    def bits_per_weight(self) -> float: return self.lib.orc_mxfp4_bits_per_weight()
    def int4g32_bits_per_weight(self) -> float: return self.lib.orc_int4g32_bits_per_weight()
    def nvfp4_bits_per_weight(self) -> float: return self.lib.orc_nvfp4_bits_per_weight()
    def mxfp4_bytes(self, n_rows: int, k: int) -> int: return self.lib.orc_mxfp4_bytes(n_rows, k)
    def num_threads(self) -> int: return self.lib.orc_num_threads()
    def set_num_threads(self, n: int) -> None: self.lib.orc_set_num_threads(n)

    def weight(self, W: "ExpertWeights", which: str, e: int, n: int, k: int) -> float:
        """Decoded element (n, k) of expert e's projection which in {gate, up, down}."""
        return self.lib.orc_weight(ctypes.byref(getattr(W.c, which)), W.fmt, e, n, k)

    def decode_matrix(self, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
        codes = np.ascontiguousarray(codes, np.uint8); scales = np.ascontiguousarray(scales, np.uint8)
        n, k = codes.shape[0], codes.shape[1] * 2
        out = np.empty((n, k), np.float64)
        self.lib.orc_mxfp4_decode_matrix(_p(codes), _p(scales), n, k, _p(out))
        return out

    # ---- MX activation formats ----
    def mx_bits(self, fmt: int) -> int: return self.lib.orc_mx_bits(fmt)
    def mx_emax(self, fmt: int) -> int: return self.lib.orc_mx_emax(fmt)
    def mx_value(self, fmt: int, code: int) -> float: return self.lib.orc_mx_value(fmt, code)
    def mx_encode(self, fmt: int, q: float) -> int: return self.lib.orc_mx_encode(fmt, q)
    def mx_scale_code(self, fmt: int, amax: float) -> int: return self.lib.orc_mx_scale_code(fmt, amax)

    def mx_quantize(self, v: np.ndarray, fmt: int):
        """[n][K] float64 -> (codes [n][K] uint8, one code per byte; scales [n][K/32] uint8)."""
        v = np.ascontiguousarray(v, np.float64)
        n, K = v.shape
        codes = np.empty((n, K), np.uint8); scales = np.empty((n, K // 32), np.uint8)
        self.lib.orc_mx_quantize(_p(v), n, K, fmt, _p(codes), _p(scales))
        return codes, scales

    def mx_dequantize(self, codes: np.ndarray, scales: np.ndarray, fmt: int) -> np.ndarray:
        codes = np.ascontiguousarray(codes, np.uint8); scales = np.ascontiguousarray(scales, np.uint8)
        n, K = codes.shape
        out = np.empty((n, K), np.float64)
        self.lib.orc_mx_dequantize(_p(codes), _p(scales), n, K, fmt, _p(out))
        return out

    def expert_ffn_mx(self, x: np.ndarray, x_fmt: int, k_total: int, W: ExpertWeights, act_fmt: int,
                      offsets: np.ndarray, sorted_slot: np.ndarray,
                      slot_mask: Optional[np.ndarray] = None, want_h: bool = False):
        """-> y_slots [T*k_total][H]; with want_h also the fp64 h before quantisation per sorted row
        [T*k_total][I] (NaN for rows not computed)."""
        x = np.ascontiguousarray(x, np.uint16)
        T = x.shape[0]
        offsets = np.ascontiguousarray(offsets, np.int32); sorted_slot = np.ascontiguousarray(sorted_slot, np.int32)
        mask = None if slot_mask is None else np.ascontiguousarray(slot_mask, np.uint8)
        y = np.full((T * k_total, W.hidden), np.nan)
        h = np.full((T * k_total, W.inter), np.nan) if want_h else None
        self.lib.orc_expert_ffn_mx(_p(x), x_fmt, T, k_total, ctypes.byref(W.c), act_fmt, _p(offsets),
                                   _p(sorted_slot), _p(mask), _p(y), _p(h))
        return (y, h) if want_h else y

    # ---- layer ----
    def route(self, x: np.ndarray, x_fmt: int, router: np.ndarray, bias: Optional[np.ndarray], top_k: int,
              n_shared: int = 0, tie_eps: float = 1e-6) -> dict:
        x = np.ascontiguousarray(x, np.uint16); router = np.ascontiguousarray(router, np.float32)
        bias = None if bias is None else np.ascontiguousarray(bias, np.float32)
        T, H = x.shape
        E = router.shape[0]
        kt = top_k + n_shared
        out = dict(logits=np.empty((T, E)), probs=np.empty((T, E)), ids=np.empty((T, kt), np.int32),
                   weights=np.empty((T, kt)), near_tie=np.zeros(T, np.uint8))
        self.lib.orc_route(_p(x), x_fmt, T, H, _p(router), _p(bias), E, top_k, n_shared, tie_eps,
                           _p(out["logits"]), _p(out["probs"]), _p(out["ids"]), _p(out["weights"]),
                           _p(out["near_tie"]))
        return out

    def route_sigmoid(self, x: np.ndarray, x_fmt: int, router: np.ndarray, sel_bias: Optional[np.ndarray],
                      top_k: int, n_shared: int = 0, routed_scale: float = 1.0, shared_weight: float = 1.0,
                      tie_eps: float = 1e-6) -> dict:
        """Sigmoid router (Cascadia Sec. 3.1) -> dict(scores, ids, weights, near_tie)."""
        x = np.ascontiguousarray(x, np.uint16); router = np.ascontiguousarray(router, np.float32)
        sel_bias = None if sel_bias is None else np.ascontiguousarray(sel_bias, np.float32)
        T, H = x.shape
        E = router.shape[0]
        kt = top_k + n_shared
        out = dict(scores=np.empty((T, E)), ids=np.empty((T, kt), np.int32), weights=np.empty((T, kt)),
                   near_tie=np.zeros(T, np.uint8))
        self.lib.orc_route_sigmoid(_p(x), x_fmt, T, H, _p(router), _p(sel_bias), E, top_k, n_shared, routed_scale,
                                   shared_weight, tie_eps, _p(out["scores"]), _p(out["ids"]), _p(out["weights"]),
                                   _p(out["near_tie"]))
        return out

    def bucket(self, ids: np.ndarray, n_buckets: int) -> dict:
        ids = np.ascontiguousarray(ids, np.int32).reshape(-1)
        n = ids.size
        out = dict(counts=np.empty(n_buckets, np.int32), offsets=np.empty(n_buckets + 1, np.int32),
                   sorted_slot=np.empty(n, np.int32), slot_pos=np.empty(n, np.int32))
        out["n_valid"] = self.lib.orc_bucket(_p(ids), n, n_buckets, _p(out["counts"]), _p(out["offsets"]),
                                             _p(out["sorted_slot"]), _p(out["slot_pos"]))
        return out

    def expert_apply(self, W: ExpertWeights, e: int, xv: np.ndarray) -> np.ndarray:
        xv = np.ascontiguousarray(xv, np.float64)
        out = np.empty(W.hidden, np.float64)
        self.lib.orc_expert_apply(ctypes.byref(W.c), e, _p(xv), _p(out))
        return out

    def expert_ffn(self, x: np.ndarray, x_fmt: int, k_total: int, W: ExpertWeights, offsets: np.ndarray,
                   sorted_slot: np.ndarray, slot_mask: Optional[np.ndarray] = None) -> np.ndarray:
        x = np.ascontiguousarray(x, np.uint16)
        T = x.shape[0]
        offsets = np.ascontiguousarray(offsets, np.int32); sorted_slot = np.ascontiguousarray(sorted_slot, np.int32)
        mask = None if slot_mask is None else np.ascontiguousarray(slot_mask, np.uint8)
        y = np.full((T * k_total, W.hidden), np.nan)
        self.lib.orc_expert_ffn(_p(x), x_fmt, T, k_total, ctypes.byref(W.c), _p(offsets), _p(sorted_slot),
                                _p(mask), _p(y))
        return y

    # ---- FP16 range management (Cascadia Sec. 3.3, Eq. 1) ----
    def expert_ffn_attenuated(self, x: np.ndarray, x_fmt: int, k_total: int, W: ExpertWeights, att_log2: int,
                              offsets: np.ndarray, sorted_slot: np.ndarray,
                              slot_mask: Optional[np.ndarray] = None) -> np.ndarray:
        """-> E(x) / 2^att_log2 per slot, [T*k_total][H] (NaN for rows not computed)."""
        x = np.ascontiguousarray(x, np.uint16)
        T = x.shape[0]
        offsets = np.ascontiguousarray(offsets, np.int32); sorted_slot = np.ascontiguousarray(sorted_slot, np.int32)
        mask = None if slot_mask is None else np.ascontiguousarray(slot_mask, np.uint8)
        y = np.full((T * k_total, W.hidden), np.nan)
        self.lib.orc_expert_ffn_attenuated(_p(x), x_fmt, T, k_total, ctypes.byref(W.c), att_log2, _p(offsets),
                                           _p(sorted_slot), _p(mask), _p(y))
        return y

    def row_factor(self, w: np.ndarray) -> float:
        w = np.ascontiguousarray(w, np.float64).reshape(-1)
        return self.lib.orc_row_factor(_p(w), w.size)

    def combine_restore(self, y_slots_att: np.ndarray, weights: np.ndarray, att_log2: int,
                        token_mask: Optional[np.ndarray] = None) -> np.ndarray:
        weights = np.ascontiguousarray(weights, np.float64)
        T, kt = weights.shape
        y_slots_att = np.ascontiguousarray(y_slots_att, np.float64).reshape(T * kt, -1)
        H = y_slots_att.shape[1]
        mask = None if token_mask is None else np.ascontiguousarray(token_mask, np.uint8)
        y = np.full((T, H), np.nan)
        self.lib.orc_combine_restore(_p(y_slots_att), _p(weights), T, kt, H, att_log2, _p(mask), _p(y))
        return y

    def combine(self, y_slots: np.ndarray, weights: np.ndarray, token_mask: Optional[np.ndarray] = None):
        weights = np.ascontiguousarray(weights, np.float64)
        T, kt = weights.shape
        y_slots = np.ascontiguousarray(y_slots, np.float64).reshape(T * kt, -1)
        H = y_slots.shape[1]
        mask = None if token_mask is None else np.ascontiguousarray(token_mask, np.uint8)
        y = np.full((T, H), np.nan)
        self.lib.orc_combine(_p(y_slots), _p(weights), T, kt, H, _p(mask), _p(y))
        return y

    def layer_bruteforce(self, x, x_fmt, W: ExpertWeights, ids, weights) -> np.ndarray:
        x = np.ascontiguousarray(x, np.uint16); ids = np.ascontiguousarray(ids, np.int32)
        weights = np.ascontiguousarray(weights, np.float64)
        T, kt = ids.shape
        y = np.empty((T, W.hidden))
        self.lib.orc_layer_bruteforce(_p(x), x_fmt, T, kt, ctypes.byref(W.c), _p(ids), _p(weights), _p(y))
        return y

    def layer_dense_mixture(self, x, x_fmt, W: ExpertWeights, ids, weights) -> np.ndarray:
        x = np.ascontiguousarray(x, np.uint16); ids = np.ascontiguousarray(ids, np.int32)
        weights = np.ascontiguousarray(weights, np.float64)
        T, kt = ids.shape
        y = np.empty((T, W.hidden))
        self.lib.orc_layer_dense_mixture(_p(x), x_fmt, T, kt, ctypes.byref(W.c), _p(ids), _p(weights), _p(y))
        return y

    def dense_ffn_f16(self, x, x_fmt, wg, wu, wd) -> np.ndarray:
        x = np.ascontiguousarray(x, np.uint16)
        wg, wu, wd = (np.ascontiguousarray(a, np.uint16) for a in (wg, wu, wd))
        T, H = x.shape
        I = wg.shape[0]
        y = np.empty((T, H))
        self.lib.orc_dense_ffn_f16(_p(x), x_fmt, T, H, I, _p(wg), _p(wu), _p(wd), _p(y))
        return y

    def layer(self, L, tie_eps: float = 1e-6, token_mask: Optional[np.ndarray] = None) -> dict:
        """route -> bucket -> grouped expert FFN -> combine on synth.LayerInputs L.  For the
        all-active-slices workload the ids are j and the weights 1 (no router).  token_mask limits
        the expert FFN and the combine to the given tokens (routing and bucketing stay whole)."""
        wl = L.wl
        x_fmt = X_BF16 if wl.act_dtype == "bf16" else X_FP16
        W = ExpertWeights.from_layer(L)
        if wl.dense_slices:
            kt = wl.n_experts
            r = dict(ids=np.tile(np.arange(kt, dtype=np.int32), (L.T, 1)), weights=np.ones((L.T, kt)),
                     near_tie=np.zeros(L.T, np.uint8), probs=None, logits=None)
        else:
            kt = wl.k_total
            r = self.route(L.x, x_fmt, L.router, L.bias, wl.top_k, wl.n_shared, tie_eps)
        b = self.bucket(r["ids"], wl.n_experts)
        slot_mask = None if token_mask is None else np.repeat(np.asarray(token_mask, np.uint8), kt)
        ys = self.expert_ffn(L.x, x_fmt, kt, W, b["offsets"], b["sorted_slot"], slot_mask)
        y = self.combine(ys, r["weights"], token_mask)
        return dict(route=r, bucket=b, y_slots=ys, y=y, weights=W)


_default: Optional[Oracle] = None


def load(path: Optional[str] = None) -> Oracle:
    """Load the built oracle (building it first only when no library exists yet)."""
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default
