"""Routed Mixture-of-Experts FFN layer for AMD Instinct MI355X (gfx950).

Thin Python binding of the C ABI in include/moe.h (libmoe.so, built from csrc/ by _build.py).  The
functions keep the C names and only marshal arguments: torch tensors provide device memory and the
current HIP stream; every step of the layer runs in the library's HIP kernels.  There is no CPU
fallback -- importing works anywhere, but any call raises when libmoe.so is missing or no GPU is
present.

    ids, w, probs = moe_route(x, w_router, top_k, bias, n_shared)     # router
    b = moe_bucket(ids, n_experts)                                     # group slots by expert
    y_slots = moe_expert_ffn(x, W, b.offsets, b.sorted_slot, k_total)  # SwiGLU experts
    y = moe_combine(y_slots, w)                                        # weighted combine, fp32
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libmoe.so")
ROOT = os.path.dirname(PKG)
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_ACT_BF16, MOE_ACT_FP16 = 0, 1
MOE_W_MXFP4, MOE_W_FP16, MOE_W_INT4_G32, MOE_W_NVFP4 = 0, 1, 2, 3
W_FORMATS = {"mxfp4": MOE_W_MXFP4, "fp16": MOE_W_FP16, "int4g32": MOE_W_INT4_G32, "nvfp4": MOE_W_NVFP4}
MOE_MX_FP8_E4M3, MOE_MX_FP4_E2M1, MOE_MX_FP6_E2M3 = 1, 2, 3
MX_FORMATS = {"fp8": MOE_MX_FP8_E4M3, "fp4": MOE_MX_FP4_E2M1, "fp6": MOE_MX_FP6_E2M3}

STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_BLOCK", 4: "MOE_ERR_ALIGN",
          5: "MOE_ERR_DTYPE", 6: "MOE_ERR_TOPK", 7: "MOE_ERR_WORKSPACE", 8: "MOE_ERR_HIP"}


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({text})")
        self.status = status


class moe_proj(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("w_expert_stride", ctypes.c_int64), ("w_row_stride", ctypes.c_int64),
                ("s_expert_stride", ctypes.c_int64), ("s_row_stride", ctypes.c_int64),
                ("zeros", ctypes.c_void_p), ("z_expert_stride", ctypes.c_int64), ("z_row_stride", ctypes.c_int64),
                ("tensor_scale", ctypes.c_void_p)]


class moe_expert_weights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("n_experts", ctypes.c_int), ("hidden", ctypes.c_int),
                ("inter", ctypes.c_int), ("gate", moe_proj), ("up", moe_proj), ("down", moe_proj)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it with `python -m mxfp4_routed_expert_router_amd._build` "
                               "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIBRARY)
        vp, i, st, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int64
        L.moe_status_str.restype = ctypes.c_char_p; L.moe_status_str.argtypes = [i]
        L.moe_abi_version.restype = i; L.moe_abi_version.argtypes = []
        L.moe_route_workspace_bytes.restype = st; L.moe_route_workspace_bytes.argtypes = [i, i, i]
        L.moe_route.restype = i
        L.moe_route.argtypes = [vp, i, i, i, vp, vp, i, i, i, vp, vp, vp, vp, st, vp]
        L.moe_route_bucket_workspace_bytes.restype = st
        L.moe_route_bucket_workspace_bytes.argtypes = [i, i, i, i, i]
        L.moe_route_bucket.restype = i
        L.moe_route_bucket.argtypes = [vp, i, i, i, vp, vp, i, i, i, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.POINTER(moe_expert_weights), vp, st, vp, st, vp]
        L.moe_route_sigmoid.restype = i
        L.moe_route_sigmoid.argtypes = [vp, i, i, i, vp, vp, i, i, i, ctypes.c_float, ctypes.c_float, vp, vp, vp,
                                        vp, st, vp]
        L.moe_row_shape.restype = i; L.moe_row_shape.argtypes = [i, ctypes.POINTER(ctypes.c_int), i]
        L.moe_pad_rows.restype = i; L.moe_pad_rows.argtypes = [vp, i, i, vp, vp, vp]
        L.moe_bucket_workspace_bytes.restype = st; L.moe_bucket_workspace_bytes.argtypes = [i, i]
        L.moe_bucket.restype = i
        L.moe_bucket.argtypes = [vp, i, i, vp, vp, vp, vp, vp, st, vp]
        L.moe_expert_ffn_workspace_bytes.restype = st
        L.moe_expert_ffn_workspace_bytes.argtypes = [i, i, ctypes.POINTER(moe_expert_weights)]
        L.moe_expert_ffn.restype = i
        L.moe_expert_ffn.argtypes = [vp, i, i, i, ctypes.POINTER(moe_expert_weights), vp, vp, vp, vp, st, vp]
        L.moe_expert_ffn_static.restype = i
        L.moe_expert_ffn_static.argtypes = [vp, i, i, i, ctypes.POINTER(moe_expert_weights), vp, vp, vp, vp]
        L.moe_expert_ffn_f16_workspace_bytes.restype = st
        L.moe_expert_ffn_f16_workspace_bytes.argtypes = [i, i, ctypes.POINTER(moe_expert_weights)]
        L.moe_expert_ffn_f16.restype = i
        L.moe_expert_ffn_f16.argtypes = [vp, i, i, i, ctypes.POINTER(moe_expert_weights), i, vp, vp, vp, vp, st, vp]
        L.moe_combine_restore.restype = i
        L.moe_combine_restore.argtypes = [vp, vp, i, i, i, i, vp, vp]
        L.moe_expert_ffn_plan.restype = i
        L.moe_expert_ffn_plan.argtypes = [i, i, i, ctypes.POINTER(moe_expert_weights), vp, vp, st, vp]
        L.moe_expert_ffn_gateup.restype = i
        L.moe_expert_ffn_gateup.argtypes = [vp, i, i, i, ctypes.POINTER(moe_expert_weights), vp, vp, vp, st, vp]
        L.moe_expert_ffn_down.restype = i
        L.moe_expert_ffn_down.argtypes = [i, i, i, ctypes.POINTER(moe_expert_weights), vp, vp, vp, vp, st, vp]
        L.moe_combine.restype = i
        L.moe_combine.argtypes = [vp, vp, i, i, i, vp, vp]
        L.moe_mxfp4_dequant.restype = i
        L.moe_mxfp4_dequant.argtypes = [vp, vp, i, i, i64, i64, vp, vp]
        L.moe_mx_row_bytes.restype = st; L.moe_mx_row_bytes.argtypes = [i, i]
        L.moe_mx_quantize.restype = i
        L.moe_mx_quantize.argtypes = [vp, i, i, i, i, vp, vp, vp]
        L.moe_expert_ffn_mx_workspace_bytes.restype = st
        L.moe_expert_ffn_mx_workspace_bytes.argtypes = [i, i, ctypes.POINTER(moe_expert_weights), i]
        L.moe_expert_ffn_mx_workspace_layout.restype = i
        L.moe_expert_ffn_mx_workspace_layout.argtypes = [i, i, ctypes.POINTER(moe_expert_weights), i,
                                                         ctypes.POINTER(ctypes.c_size_t)]
        L.moe_expert_ffn_mx.restype = i
        L.moe_expert_ffn_mx.argtypes = [vp, i, i, i, ctypes.POINTER(moe_expert_weights), i, vp, vp, vp, vp, st, vp]
        L.moe_stream_read.restype = i
        L.moe_stream_read.argtypes = [vp, st, vp, vp]
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MoEError(status, where, lib().moe_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _act_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return MOE_ACT_BF16
    if x.dtype == torch.float16:
        return MOE_ACT_FP16
    raise TypeError(f"activations must be bfloat16 or float16, got {x.dtype}")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes > 0 else None


class ExpertWeights:
    """Device weights of all experts of a layer, described for moe_expert_ffn.

    MXFP4: gate/up codes uint8 [E'][I][H/2], scales uint8 [E'][I][H/32]; down codes [E'][H][I/2],
    scales [E'][H][I/32].  FP16: gate/up float16 [E'][I][H], down [E'][H][I], scales None.
    INT4_G32 (fmt="int4g32"): codes as MXFP4, scales [E'][N][K/32] binary16 bits as uint8 pairs
    ([E'][N][K/16] uint8), extras {"gate"/"up"/"down": zero points uint8 [E'][N][ceil(K/64)]}.
    NVFP4 (fmt="nvfp4"): codes as MXFP4, scales uint8 E4M3 [E'][N][K/16], extras {matrix: fp32
    tensor scales [E']}.
    Any strided view whose last dimension is contiguous is accepted (slices of a larger matrix)."""

    def __init__(self, gate, gate_scales, up, up_scales, down, down_scales, fmt=None, extras=None):
        if fmt is None:
            fmt = MOE_W_FP16 if gate.dtype == torch.float16 else MOE_W_MXFP4
        elif isinstance(fmt, str):
            fmt = W_FORMATS[fmt]
        extras = dict(extras or {})
        self.extras = extras
        self.tensors = (gate, gate_scales, up, up_scales, down, down_scales)
        E2, I = gate.shape[0], gate.shape[1]
        H = down.shape[1]
        self.fmt, self.n_experts, self.hidden, self.inter = fmt, E2, H, I

        def proj(c, s, ex):
            p = moe_proj()
            p.w = c.data_ptr()
            es = c.element_size()
            p.w_expert_stride, p.w_row_stride = c.stride(0) * es, c.stride(1) * es
            if c.stride(2) != 1:
                raise ValueError("weight rows must be contiguous")
            if s is not None:
                p.scales = s.data_ptr()
                ss = s.element_size()
                p.s_expert_stride, p.s_row_stride = s.stride(0) * ss, s.stride(1) * ss
            if ex is not None and fmt == MOE_W_INT4_G32:
                p.zeros = ex.data_ptr()
                p.z_expert_stride, p.z_row_stride = ex.stride(0), ex.stride(1)
            if ex is not None and fmt == MOE_W_NVFP4:
                if ex.dtype != torch.float32 or not ex.is_contiguous():
                    raise ValueError("NVFP4 tensor scales must be a contiguous float32 tensor")
                p.tensor_scale = ex.data_ptr()
            return p

        self.c = moe_expert_weights(fmt, E2, H, I, proj(gate, gate_scales, extras.get("gate")),
                                    proj(up, up_scales, extras.get("up")), proj(down, down_scales, extras.get("down")))

    @property
    def device(self):
        return self.tensors[0].device

    def weight_bytes(self, experts=None) -> int:
        """Logical bytes (codes + scales) of the given experts (all when None)."""
        per = 0
        for t in self.tensors:
            if t is not None:
                per += t[0].numel() * t.element_size()
        n = self.n_experts if experts is None else len(experts)
        return per * n


# ----------------------------------------------------------------------------------------------------
def moe_route_workspace_bytes(T: int, H: int, E: int) -> int:
    return lib().moe_route_workspace_bytes(T, H, E)


def moe_route(x: torch.Tensor, w_router: torch.Tensor, top_k: int, logit_bias: Optional[torch.Tensor] = None,
              n_shared: int = 0, want_probs: bool = False, out=None, workspace=None):
    """-> (ids int32 [T][k'], weights fp32 [T][k'], probs fp32 [T][E] or None)."""
    T, H = x.shape
    E = w_router.shape[0]
    kt = top_k + n_shared
    dev = x.device
    if out is None:
        ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
        w = torch.empty((T, kt), dtype=torch.float32, device=dev)
        probs = torch.empty((T, E), dtype=torch.float32, device=dev) if want_probs else None
    else:
        ids, w, probs = out
    need = moe_route_workspace_bytes(T, H, E)
    ws = workspace if workspace is not None else _workspace(need, dev)
    _check(lib().moe_route(_ptr(x), _act_dtype(x), T, H, _ptr(w_router), _ptr(logit_bias), E, top_k, n_shared,
                           _ptr(ids), _ptr(w), _ptr(probs), _ptr(ws), 0 if ws is None else ws.numel(),
                           _stream(dev)), "moe_route")
    return ids, w, probs


def moe_route_bucket_workspace_bytes(T: int, H: int, E: int, top_k: int, n_shared: int = 0) -> int:
    return lib().moe_route_bucket_workspace_bytes(T, H, E, top_k, n_shared)


def moe_route_bucket(x: torch.Tensor, w_router: torch.Tensor, top_k: int, logit_bias: Optional[torch.Tensor],
                     n_shared: int, ids: torch.Tensor, weights: torch.Tensor, buckets: "Buckets",
                     W: Optional[ExpertWeights] = None, ffn_workspace: Optional[torch.Tensor] = None,
                     probs: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> None:
    """moe_route + moe_bucket (+ moe_expert_ffn_plan into ffn_workspace when W is given) in one call,
    into the caller's buffers."""
    T, H = x.shape
    E = w_router.shape[0]
    need = moe_route_bucket_workspace_bytes(T, H, E, top_k, n_shared)
    ws = workspace if workspace is not None else _workspace(need, x.device)
    _check(lib().moe_route_bucket(_ptr(x), _act_dtype(x), T, H, _ptr(w_router), _ptr(logit_bias), E, top_k, n_shared,
                                  _ptr(ids), _ptr(weights), _ptr(probs), _ptr(buckets.counts), _ptr(buckets.offsets),
                                  _ptr(buckets.sorted_slot), _ptr(buckets.slot_pos),
                                  None if W is None else ctypes.byref(W.c), _ptr(ffn_workspace),
                                  0 if ffn_workspace is None else ffn_workspace.numel(), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(x.device)), "moe_route_bucket")


def moe_route_sigmoid(x: torch.Tensor, w_router: torch.Tensor, top_k: int,
                      selection_bias: Optional[torch.Tensor] = None, n_shared: int = 0, routed_scale: float = 1.0,
                      shared_weight: float = 1.0, want_scores: bool = False, out=None, workspace=None):
    """Cascadia's sigmoid router -> (ids int32 [T][k'], weights fp32 [T][k'], scores fp32 [T][E] or None)."""
    T, H = x.shape
    E = w_router.shape[0]
    kt = top_k + n_shared
    dev = x.device
    if out is None:
        ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
        w = torch.empty((T, kt), dtype=torch.float32, device=dev)
        scores = torch.empty((T, E), dtype=torch.float32, device=dev) if want_scores else None
    else:
        ids, w, scores = out
    need = moe_route_workspace_bytes(T, H, E)
    ws = workspace if workspace is not None else _workspace(need, dev)
    _check(lib().moe_route_sigmoid(_ptr(x), _act_dtype(x), T, H, _ptr(w_router), _ptr(selection_bias), E, top_k,
                                   n_shared, routed_scale, shared_weight, _ptr(ids), _ptr(w), _ptr(scores), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(dev)), "moe_route_sigmoid")
    return ids, w, scores


def moe_row_shape(T: int, shapes) -> int:
    """Smallest supported row shape >= T (-1 if none)."""
    arr = (ctypes.c_int * len(shapes))(*shapes)
    return lib().moe_row_shape(T, arr, len(shapes))


def moe_pad_rows(n_rows: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor) -> None:
    """Rows >= n_rows[0] (a device int32 scalar) get zero weights and id -1, in place."""
    T, kt = ids.shape
    _check(lib().moe_pad_rows(_ptr(n_rows), T, kt, _ptr(ids), _ptr(weights), _stream(ids.device)), "moe_pad_rows")


@dataclass
class Buckets:
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_slot: torch.Tensor
    slot_pos: Optional[torch.Tensor]


def moe_bucket_workspace_bytes(n_slots: int, n_buckets: int) -> int:
    return lib().moe_bucket_workspace_bytes(n_slots, n_buckets)


def moe_bucket(ids: torch.Tensor, n_buckets: int, out: Optional[Buckets] = None, workspace=None) -> Buckets:
    n = ids.numel()
    dev = ids.device
    if out is None:
        out = Buckets(torch.empty(n_buckets, dtype=torch.int32, device=dev),
                      torch.empty(n_buckets + 1, dtype=torch.int32, device=dev),
                      torch.empty(n, dtype=torch.int32, device=dev),
                      torch.empty(n, dtype=torch.int32, device=dev))
    need = moe_bucket_workspace_bytes(n, n_buckets)
    ws = workspace if workspace is not None else _workspace(need, dev)
    _check(lib().moe_bucket(_ptr(ids), n, n_buckets, _ptr(out.counts), _ptr(out.offsets), _ptr(out.sorted_slot),
                            _ptr(out.slot_pos), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)),
           "moe_bucket")
    return out


def moe_expert_ffn_workspace_bytes(T: int, k_total: int, W: ExpertWeights) -> int:
    return lib().moe_expert_ffn_workspace_bytes(T, k_total, ctypes.byref(W.c))


def moe_expert_ffn(x: torch.Tensor, W: ExpertWeights, offsets: torch.Tensor, sorted_slot: torch.Tensor,
                   k_total: int, out: Optional[torch.Tensor] = None, workspace=None) -> torch.Tensor:
    """-> y_slots fp32 [T*k_total][hidden] (rows of dropped slots are left as allocated)."""
    T = x.shape[0]
    dev = x.device
    y = out if out is not None else torch.empty((T * k_total, W.hidden), dtype=torch.float32, device=dev)
    need = moe_expert_ffn_workspace_bytes(T, k_total, W)
    ws = workspace if workspace is not None else _workspace(need, dev)
    _check(lib().moe_expert_ffn(_ptr(x), _act_dtype(x), T, k_total, ctypes.byref(W.c), _ptr(offsets),
                                _ptr(sorted_slot), _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(dev)), "moe_expert_ffn")
    return y


MOE_FFN_STATIC_SCRATCH_BYTES = 16 << 20


def moe_expert_ffn_static(x: torch.Tensor, W: ExpertWeights, offsets: torch.Tensor, sorted_slot: torch.Tensor,
                          k_total: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_expert_ffn with the library's fixed device scratch array as its workspace (no workspace
    argument; calls needing more than MOE_FFN_STATIC_SCRATCH_BYTES are refused).  Only `out` may be
    allocated here, and only when the caller passes none."""
    T = x.shape[0]
    dev = x.device
    y = out if out is not None else torch.empty((T * k_total, W.hidden), dtype=torch.float32, device=dev)
    _check(lib().moe_expert_ffn_static(_ptr(x), _act_dtype(x), T, k_total, ctypes.byref(W.c), _ptr(offsets),
                                       _ptr(sorted_slot), _ptr(y), _stream(dev)), "moe_expert_ffn_static")
    return y


def moe_expert_ffn_plan(T: int, W: ExpertWeights, offsets: torch.Tensor, k_total: int,
                        workspace: torch.Tensor) -> None:
    """Step 1 of moe_expert_ffn: the tile schedule (from offsets) into `workspace`
    (moe_expert_ffn_workspace_bytes bytes), read by the two phases below."""
    xdt = MOE_ACT_FP16 if W.fmt == MOE_W_FP16 else MOE_ACT_BF16
    _check(lib().moe_expert_ffn_plan(xdt, T, k_total, ctypes.byref(W.c), _ptr(offsets), _ptr(workspace),
                                     workspace.numel(), _stream(offsets.device)),
           "moe_expert_ffn_plan")


def moe_expert_ffn_gateup(x: torch.Tensor, W: ExpertWeights, offsets: torch.Tensor, sorted_slot: torch.Tensor,
                          k_total: int, workspace: torch.Tensor) -> None:
    """Phase 1 of moe_expert_ffn: h into `workspace`, after moe_expert_ffn_plan on it."""
    T = x.shape[0]
    _check(lib().moe_expert_ffn_gateup(_ptr(x), _act_dtype(x), T, k_total, ctypes.byref(W.c), _ptr(offsets),
                                       _ptr(sorted_slot), _ptr(workspace), workspace.numel(), _stream(x.device)),
           "moe_expert_ffn_gateup")


def moe_expert_ffn_down(T: int, W: ExpertWeights, offsets: torch.Tensor, sorted_slot: torch.Tensor, k_total: int,
                        workspace: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """Phase 2 of moe_expert_ffn: y_slots from the h left in `workspace` by the gate/up phase."""
    xdt = MOE_ACT_FP16 if W.fmt == MOE_W_FP16 else MOE_ACT_BF16
    _check(lib().moe_expert_ffn_down(xdt, T, k_total, ctypes.byref(W.c), _ptr(offsets), _ptr(sorted_slot),
                                     _ptr(out), _ptr(workspace), workspace.numel(), _stream(out.device)),
           "moe_expert_ffn_down")
    return out


def moe_expert_ffn_f16_workspace_bytes(T: int, k_total: int, W: ExpertWeights) -> int:
    return lib().moe_expert_ffn_f16_workspace_bytes(T, k_total, ctypes.byref(W.c))


def moe_expert_ffn_f16(x: torch.Tensor, W: ExpertWeights, attenuation_log2: int, offsets: torch.Tensor,
                       sorted_slot: torch.Tensor, k_total: int, out: Optional[torch.Tensor] = None,
                       workspace=None) -> torch.Tensor:
    """Range-managed expert FFN (Cascadia Eq. 1): -> binary16 y_slots [T*k_total][hidden] holding
    E(x) / 2^attenuation_log2 (float16 tensor)."""
    T = x.shape[0]
    dev = x.device
    y = out if out is not None else torch.empty((T * k_total, W.hidden), dtype=torch.float16, device=dev)
    need = moe_expert_ffn_f16_workspace_bytes(T, k_total, W)
    ws = workspace if workspace is not None else _workspace(need, dev)
    _check(lib().moe_expert_ffn_f16(_ptr(x), _act_dtype(x), T, k_total, ctypes.byref(W.c), attenuation_log2,
                                    _ptr(offsets), _ptr(sorted_slot), _ptr(y), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(dev)), "moe_expert_ffn_f16")
    return y


def moe_combine_restore(y_slots: torch.Tensor, weights: torch.Tensor, attenuation_log2: int,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Eq. 1 combination of binary16 attenuated slots with row factors, restored to fp32 y [T][H]."""
    T, kt = weights.shape
    H = y_slots.shape[-1]
    y = out if out is not None else torch.empty((T, H), dtype=torch.float32, device=y_slots.device)
    _check(lib().moe_combine_restore(_ptr(y_slots), _ptr(weights), T, kt, H, attenuation_log2, _ptr(y),
                                     _stream(y_slots.device)), "moe_combine_restore")
    return y


def moe_combine(y_slots: torch.Tensor, weights: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, kt = weights.shape
    H = y_slots.shape[-1]
    y = out if out is not None else torch.empty((T, H), dtype=torch.float32, device=y_slots.device)
    _check(lib().moe_combine(_ptr(y_slots), _ptr(weights), T, kt, H, _ptr(y), _stream(y_slots.device)),
           "moe_combine")
    return y


def moe_mxfp4_dequant(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """[N][K/2] codes + [N][K/32] scales -> [N][K] bfloat16 (the FFN's decode primitive)."""
    N, K = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((N, K), dtype=torch.bfloat16, device=codes.device)
    _check(lib().moe_mxfp4_dequant(_ptr(codes), _ptr(scales), N, K, codes.stride(0), scales.stride(0), _ptr(out),
                                   _stream(codes.device)), "moe_mxfp4_dequant")
    return out


def moe_stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read every byte of the contiguous device tensor `buf` once with whole-line nontemporal loads
    (a measurement utility: timing it over a buffer far larger than the caches gives the practical
    HBM read rate).  `sink` is a one-element int32 device tensor whose contents are meaningless."""
    if not buf.is_contiguous() or sink.numel() < 1 or sink.dtype != torch.int32:
        raise ValueError("moe_stream_read: needs a contiguous buffer and an int32 sink")
    _check(lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf.device)),
           "moe_stream_read")


def _mx_fmt(fmt) -> int:
    return MX_FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def moe_mx_row_bytes(fmt, K: int) -> int:
    return lib().moe_mx_row_bytes(_mx_fmt(fmt), K)


def moe_mx_quantize(x: torch.Tensor, fmt) -> tuple:
    """[n][K] bf16/fp16 -> (packed codes uint8 [n][row bytes], E8M0 scales uint8 [n][K/32])."""
    n, K = x.shape
    f = _mx_fmt(fmt)
    codes = torch.empty((n, max(moe_mx_row_bytes(f, K), 1)), dtype=torch.uint8, device=x.device)
    scales = torch.empty((n, max(K // 32, 1)), dtype=torch.uint8, device=x.device)
    _check(lib().moe_mx_quantize(_ptr(x), _act_dtype(x), n, K, f, _ptr(codes), _ptr(scales), _stream(x.device)),
           "moe_mx_quantize")
    return codes, scales


def moe_expert_ffn_mx_workspace_bytes(T: int, k_total: int, W: ExpertWeights, fmt) -> int:
    return lib().moe_expert_ffn_mx_workspace_bytes(T, k_total, ctypes.byref(W.c), _mx_fmt(fmt))


def moe_expert_ffn_mx_workspace_layout(T: int, k_total: int, W: ExpertWeights, fmt) -> dict:
    """Byte offsets of the quantised x and h that moe_expert_ffn_mx leaves in its workspace."""
    offs = (ctypes.c_size_t * 4)()
    _check(lib().moe_expert_ffn_mx_workspace_layout(T, k_total, ctypes.byref(W.c), _mx_fmt(fmt), offs),
           "moe_expert_ffn_mx_workspace_layout")
    return dict(x_codes=offs[0], x_scales=offs[1], h_codes=offs[2], h_scales=offs[3])


def moe_expert_ffn_mx(x: torch.Tensor, W: ExpertWeights, fmt, offsets: torch.Tensor, sorted_slot: torch.Tensor,
                      k_total: int, out: Optional[torch.Tensor] = None, workspace=None) -> torch.Tensor:
    """MX mode of moe_expert_ffn (x and h quantised to the MX format `fmt`): -> y_slots fp32."""
    T = x.shape[0]
    dev = x.device
    f = _mx_fmt(fmt)
    y = out if out is not None else torch.empty((T * k_total, W.hidden), dtype=torch.float32, device=dev)
    need = moe_expert_ffn_mx_workspace_bytes(T, k_total, W, f)
    ws = workspace if workspace is not None else _workspace(need, dev)
    _check(lib().moe_expert_ffn_mx(_ptr(x), _act_dtype(x), T, k_total, ctypes.byref(W.c), f, _ptr(offsets),
                                   _ptr(sorted_slot), _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(dev)), "moe_expert_ffn_mx")
    return y


# ----------------------------------------------------------------------------------------------------
class MoELayer:
    """One routed-MoE layer with every intermediate buffer allocated once, so that forward() only
    enqueues the four library calls (capturable in a HIP graph)."""

    def __init__(self, W: ExpertWeights, T: int, top_k: int, n_shared: int = 0,
                 w_router: Optional[torch.Tensor] = None, logit_bias: Optional[torch.Tensor] = None,
                 mx=None):
        self.W, self.T, self.top_k, self.n_shared = W, T, top_k, n_shared
        self.mx = None if mx is None else _mx_fmt(mx)  # MX mode: activation format of the FFN
        self.w_router, self.logit_bias = w_router, logit_bias
        dev = W.device
        kt = top_k + n_shared
        self.k_total = kt
        H = W.hidden
        E = W.n_experts - n_shared
        self.dense = w_router is None  # all-active slices: caller-fixed ids j, weights 1
        if self.dense:
            self.ids = torch.arange(kt, dtype=torch.int32, device=dev).repeat(T, 1).contiguous()
            self.weights = torch.ones((T, kt), dtype=torch.float32, device=dev)
            self.route_ws = None
        else:
            self.ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
            self.weights = torch.empty((T, kt), dtype=torch.float32, device=dev)
            self.route_ws = _workspace(moe_route_bucket_workspace_bytes(T, H, E, top_k, n_shared), dev)
        n = T * kt
        self.buckets = Buckets(torch.empty(W.n_experts, dtype=torch.int32, device=dev),
                               torch.empty(W.n_experts + 1, dtype=torch.int32, device=dev),
                               torch.empty(n, dtype=torch.int32, device=dev),
                               torch.empty(n, dtype=torch.int32, device=dev))
        self.bucket_ws = _workspace(moe_bucket_workspace_bytes(n, W.n_experts), dev)
        self.y_slots = torch.empty((n, H), dtype=torch.float32, device=dev)
        self.ffn_ws = _workspace(moe_expert_ffn_workspace_bytes(T, kt, W) if self.mx is None
                                 else moe_expert_ffn_mx_workspace_bytes(T, kt, W, self.mx), dev)
        self.y = torch.empty((T, H), dtype=torch.float32, device=dev)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not self.dense and self.mx is None:
            # route, bucket and tile plan in one call, then the two FFN phases
            moe_route_bucket(x, self.w_router, self.top_k, self.logit_bias, self.n_shared, self.ids, self.weights,
                             self.buckets, self.W, self.ffn_ws, workspace=self.route_ws)
            moe_expert_ffn_gateup(x, self.W, self.buckets.offsets, self.buckets.sorted_slot, self.k_total, self.ffn_ws)
            moe_expert_ffn_down(self.T, self.W, self.buckets.offsets, self.buckets.sorted_slot, self.k_total,
                                self.ffn_ws, self.y_slots)
            return moe_combine(self.y_slots, self.weights, out=self.y)
        if not self.dense:
            moe_route(x, self.w_router, self.top_k, self.logit_bias, self.n_shared,
                      out=(self.ids, self.weights, None), workspace=self.route_ws)
        moe_bucket(self.ids, self.W.n_experts, out=self.buckets, workspace=self.bucket_ws)
        if self.mx is None:
            moe_expert_ffn(x, self.W, self.buckets.offsets, self.buckets.sorted_slot, self.k_total, out=self.y_slots,
                           workspace=self.ffn_ws)
        else:
            moe_expert_ffn_mx(x, self.W, self.mx, self.buckets.offsets, self.buckets.sorted_slot, self.k_total,
                              out=self.y_slots, workspace=self.ffn_ws)
        return moe_combine(self.y_slots, self.weights, out=self.y)


class FixedShapeLayer:
    """A routed-MoE layer run at fixed row shapes (Cascadia Sec. 3.2): for each supported shape S
    the five calls (route, pad, bucket, expert FFN, combine) on S rows are captured once in a HIP
    graph; a call with T rows copies them into the shape's input buffer, writes T to the device
    row count, replays the graph of the smallest S >= T and returns the first T rows of y.  The
    padding rows carry zero routing weights and invalid ids, so they cost no expert work and
    change no real row.  Buffers are allocated once here; forward() allocates nothing."""

    def __init__(self, W: ExpertWeights, shapes, top_k: int, w_router: torch.Tensor,
                 logit_bias: Optional[torch.Tensor] = None, n_shared: int = 0):
        self.shapes = sorted(set(int(s) for s in shapes))
        self.W, self.top_k, self.n_shared = W, top_k, n_shared
        self.w_router, self.logit_bias = w_router, logit_bias
        dev = W.device
        S = self.shapes[-1]
        kt = top_k + n_shared
        self.k_total = kt
        H = W.hidden
        E = W.n_experts - n_shared
        self.x = torch.zeros((S, H), dtype=torch.bfloat16 if W.fmt == MOE_W_MXFP4 else torch.float16, device=dev)
        self.n_rows = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ids = torch.empty((S, kt), dtype=torch.int32, device=dev)
        self.weights = torch.empty((S, kt), dtype=torch.float32, device=dev)
        self.route_ws = _workspace(max(moe_route_workspace_bytes(s, H, E) for s in self.shapes), dev)
        self.buckets = Buckets(torch.empty(W.n_experts, dtype=torch.int32, device=dev),
                               torch.empty(W.n_experts + 1, dtype=torch.int32, device=dev),
                               torch.empty(S * kt, dtype=torch.int32, device=dev), None)
        self.bucket_ws = _workspace(max(moe_bucket_workspace_bytes(s * kt, W.n_experts) for s in self.shapes), dev)
        self.ffn_ws = _workspace(max(moe_expert_ffn_workspace_bytes(s, kt, W) for s in self.shapes), dev)
        self.y_slots = torch.empty((S * kt, H), dtype=torch.float32, device=dev)
        self.y = torch.empty((S, H), dtype=torch.float32, device=dev)
        self.graphs = {}

    def run_shape(self, S: int) -> None:
        """Enqueue the five calls for row shape S (eager; also what each graph holds)."""
        kt = self.k_total
        ids, w = self.ids[:S], self.weights[:S]
        moe_route(self.x[:S], self.w_router, self.top_k, self.logit_bias, self.n_shared, out=(ids, w, None),
                  workspace=self.route_ws)
        moe_pad_rows(self.n_rows, ids, w)
        b = Buckets(self.buckets.counts, self.buckets.offsets, self.buckets.sorted_slot[:S * kt], None)
        moe_bucket(ids, self.W.n_experts, out=b, workspace=self.bucket_ws)
        moe_expert_ffn(self.x[:S], self.W, b.offsets, b.sorted_slot, kt, out=self.y_slots[:S * kt],
                       workspace=self.ffn_ws)
        moe_combine(self.y_slots[:S * kt], w, out=self.y[:S])

    def capture(self) -> None:
        """Capture one graph per shape (after one eager pass of each on a side stream)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for S in self.shapes:
                self.run_shape(S)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for S in self.shapes:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.run_shape(S)
            self.graphs[S] = g
        torch.cuda.synchronize()

    def forward(self, x: torch.Tensor, use_graph: bool = True) -> torch.Tensor:
        """y[:T] for the T rows of x (a view into the layer's output buffer, valid until the next call)."""
        T = x.shape[0]
        S = moe_row_shape(T, self.shapes)
        if S < 0:
            raise ValueError(f"{T} rows exceed the largest supported row shape {self.shapes[-1]}")
        self.x[:T].copy_(x)
        self.n_rows.fill_(T)
        if use_graph:
            if not self.graphs:
                self.capture()
            self.graphs[S].replay()
        else:
            self.run_shape(S)
        return self.y[:T]


__all__ = ["moe_route", "moe_route_sigmoid", "moe_route_bucket", "moe_route_bucket_workspace_bytes", "moe_bucket", "moe_expert_ffn", "moe_expert_ffn_static", "moe_expert_ffn_f16",
           "moe_expert_ffn_f16_workspace_bytes", "moe_combine_restore", "moe_expert_ffn_plan", "moe_expert_ffn_gateup",
           "moe_expert_ffn_down", "moe_combine", "moe_mxfp4_dequant", "moe_mx_quantize", "moe_mx_row_bytes",
           "moe_expert_ffn_mx", "moe_expert_ffn_mx_workspace_bytes", "moe_stream_read", "moe_expert_ffn_mx_workspace_layout",
           "moe_route_workspace_bytes", "moe_bucket_workspace_bytes", "moe_expert_ffn_workspace_bytes",
           "moe_row_shape", "moe_pad_rows", "ExpertWeights", "Buckets", "MoELayer", "FixedShapeLayer", "MoEError",
           "lib"]
