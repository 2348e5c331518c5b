"""The C ABI on the host: the library loads, exports every entry point include/moe.h declares, and
rejects bad arguments with the documented status before touching the GPU (no compute call here;
device pointers are fake addresses that validation never dereferences)."""
import ctypes
import re

import pytest

import mxfp4_routed_expert_router_amd as m

OK, NULL, SHAPE, BLOCK, ALIGN, DTYPE, TOPK, WORKSPACE = 0, 1, 2, 3, 4, 5, 6, 7
P = 0x7F0000000000  # a 256-byte aligned fake device address


def fake(off=0):
    return ctypes.c_void_p(P + off)


def declared_functions():
    text = open(m.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = m.lib()
    names = declared_functions()
    assert {"moe_route", "moe_bucket", "moe_expert_ffn", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_abi_version() == 2
    for s in range(9):
        assert L.moe_status_str(s)


def test_route_validation():
    L = m.lib()
    ws = fake(0x1000)
    r = lambda **k: L.moe_route(k.get("x", fake()), k.get("xdt", 0), k.get("T", 4), k.get("H", 64),
                                k.get("wr", fake(0x100)), None, k.get("E", 8), k.get("k", 2), k.get("S", 0),
                                k.get("ids", fake(0x200)), k.get("w", fake(0x300)), None, k.get("ws", ws),
                                k.get("wsb", 1 << 20), None)
    assert L.moe_route(None, 0, 0, 64, None, None, 8, 2, 0, None, None, None, None, 0, None) == OK  # T = 0
    assert r(T=-1) == SHAPE
    assert r(H=0) == SHAPE
    assert r(E=0) == SHAPE
    assert r(E=1025) == SHAPE
    assert r(S=-1) == SHAPE
    assert r(xdt=7) == DTYPE
    assert r(k=0) == TOPK
    assert r(k=9) == TOPK
    assert r(E=512, k=250, S=7) == TOPK
    assert r(x=None) == NULL
    assert r(wr=None) == NULL
    assert r(ids=None) == NULL
    assert r(x=fake(8)) == ALIGN
    assert r(wr=fake(0x102)) == ALIGN
    assert r(ws=None) == WORKSPACE
    need = L.moe_route_workspace_bytes(4, 64, 8)
    assert need > 0
    assert r(wsb=need - 1) == WORKSPACE
    assert r(ws=fake(0x1004), wsb=need) == ALIGN


def test_bucket_validation():
    L = m.lib()
    b = lambda **k: L.moe_bucket(k.get("ids", fake()), k.get("n", 100), k.get("nb", 8), k.get("c", fake(0x400)),
                                 k.get("o", fake(0x800)), k.get("s", fake(0xC00)), None, k.get("ws", None),
                                 k.get("wsb", 0), None)
    assert L.moe_bucket(None, 0, 8, None, None, None, None, None, 0, None) == OK
    assert b(n=-5) == SHAPE
    assert b(nb=0) == SHAPE
    assert b(nb=1025) == SHAPE
    assert b(ids=None) == NULL
    assert b(o=None) == NULL
    assert b(ids=fake(2)) == ALIGN
    assert L.moe_bucket_workspace_bytes(512, 8) == 0
    need = L.moe_bucket_workspace_bytes(5000, 8)
    assert need >= 4 * (5000 + 10 * 8)
    assert b(n=5000) == WORKSPACE
    assert b(n=5000, ws=fake(0x2000), wsb=need - 4) == WORKSPACE


def weights(fmt=m.MOE_W_MXFP4, E=4, H=64, I=96, **over):
    W = m.moe_expert_weights()
    W.fmt, W.n_experts, W.hidden, W.inter = fmt, E, H, I
    bpe = 2
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        p = getattr(W, name)
        p.w = P + 0x10000
        if fmt == m.MOE_W_MXFP4:
            p.scales = P + 0x20000
            p.w_row_stride, p.w_expert_stride = K // 2, N * K // 2
            p.s_row_stride, p.s_expert_stride = K // 32, N * K // 32
        else:
            p.scales = None
            p.w_row_stride, p.w_expert_stride = bpe * K, bpe * N * K
    for k, v in over.items():
        obj, field = k.split("__") if "__" in k else (None, k)
        if obj:
            setattr(getattr(W, obj), field, v)
        else:
            setattr(W, field, v)
    return W


def ffn(W, T=4, kt=2, xdt=0, x=None, ws=None, wsb=None):
    L = m.lib()
    need = L.moe_expert_ffn_workspace_bytes(T, kt, ctypes.byref(W))
    return L.moe_expert_ffn(x if x is not None else fake(), xdt, T, kt, ctypes.byref(W), fake(0x100), fake(0x200),
                            fake(0x300), ws if ws is not None else fake(0x4000), need if wsb is None else wsb, None)


def test_expert_ffn_validation():
    L = m.lib()
    assert L.moe_expert_ffn(None, 0, 0, 2, None, None, None, None, None, 0, None) == OK
    assert L.moe_expert_ffn(fake(), 0, 4, 2, None, fake(), fake(), fake(), fake(), 1 << 20, None) == NULL
    assert ffn(weights(hidden=48)) == BLOCK          # MXFP4 hidden not a multiple of 32
    assert ffn(weights(inter=80)) == BLOCK
    assert ffn(weights(fmt=m.MOE_W_FP16, hidden=48), xdt=1) == SHAPE
    assert ffn(weights(fmt=7)) == DTYPE
    assert ffn(weights(), xdt=1) == DTYPE            # MXFP4 needs bf16 activations
    assert ffn(weights(fmt=m.MOE_W_FP16), xdt=0) == DTYPE
    Wf = weights(fmt=m.MOE_W_FP16)
    Wf.gate.scales = P
    assert ffn(Wf, xdt=1) == DTYPE                   # FP16 weights take no scales
    assert ffn(weights(n_experts=0)) == SHAPE
    assert ffn(weights(n_experts=2000)) == SHAPE
    assert ffn(weights(), kt=0) == SHAPE
    assert ffn(weights(), T=-3) == SHAPE
    assert ffn(weights(gate__w=None)) == NULL
    assert ffn(weights(down__scales=None)) == NULL
    # MXFP4: a base or byte stride off the 16-byte grid starts inside a 32-value block
    assert ffn(weights(up__w=P + 8)) == BLOCK
    assert ffn(weights(gate__w_row_stride=40)) == BLOCK   # >= K/2 = 32 but not a multiple of 16
    assert ffn(weights(down__w_expert_stride=100 * 16 + 8)) == BLOCK
    # FP16 weights: the same offsets only break the 128-bit load alignment
    assert ffn(weights(fmt=m.MOE_W_FP16, up__w=P + 8), xdt=1) == ALIGN
    assert ffn(weights(fmt=m.MOE_W_FP16, down__w_expert_stride=100 * 16 + 8), xdt=1) == ALIGN
    assert ffn(weights(gate__w_row_stride=16)) == SHAPE   # rows would overlap
    assert ffn(weights(), x=fake(4)) == ALIGN
    assert ffn(weights(), ws=fake(0x4008)) == ALIGN
    W = weights()
    need = L.moe_expert_ffn_workspace_bytes(4, 2, ctypes.byref(W))
    assert need >= 4 * 4 * 2 * 96
    assert ffn(W, wsb=need - 1) == WORKSPACE
    # a slice of a larger MXFP4 projection that starts mid-block (8 bytes = 16 codes) is refused
    assert ffn(weights(down__w=P + 0x10000 + 8)) == BLOCK


def test_expert_ffn_plan_validation():
    L = m.lib()
    W = weights()
    need = L.moe_expert_ffn_workspace_bytes(4, 2, ctypes.byref(W))

    def plan(W, T=4, kt=2, xdt=0, off=fake(0x100), ws=fake(0x4000), wsb=need):
        return L.moe_expert_ffn_plan(xdt, T, kt, ctypes.byref(W), off, ws, wsb, None)

    assert L.moe_expert_ffn_plan(0, 0, 2, None, None, None, 0, None) == OK
    assert plan(W, off=None) == NULL
    assert plan(W, wsb=need - 1) == WORKSPACE
    assert plan(W, ws=fake(0x4008)) == ALIGN
    assert plan(W, off=fake(0x102)) == ALIGN
    assert plan(W, xdt=1) == DTYPE
    assert plan(weights(n_experts=0)) == SHAPE
    assert plan(W, kt=0) == SHAPE


def test_mx_validation():
    L = m.lib()
    FP8, FP4, FP6 = m.MOE_MX_FP8_E4M3, m.MOE_MX_FP4_E2M1, m.MOE_MX_FP6_E2M3
    assert [L.moe_mx_row_bytes(f, 256) for f in (FP8, FP4, FP6)] == [256, 128, 192]
    assert L.moe_mx_row_bytes(FP8, 48) == 0 and L.moe_mx_row_bytes(9, 256) == 0
    q = lambda **k: L.moe_mx_quantize(k.get("x", fake()), k.get("xdt", 0), k.get("n", 4), k.get("K", 256),
                                      k.get("f", FP8), k.get("c", fake(0x1000)), k.get("s", fake(0x2000)), None)
    assert L.moe_mx_quantize(None, 0, 0, 256, FP8, None, None, None) == OK
    assert q(n=-1) == SHAPE
    assert q(K=0) == SHAPE
    assert q(K=48) == BLOCK
    assert q(f=0) == DTYPE and q(f=4) == DTYPE and q(xdt=3) == DTYPE
    assert q(x=None) == NULL and q(c=None) == NULL and q(s=None) == NULL
    assert q(x=fake(8)) == ALIGN and q(c=fake(0x1008)) == ALIGN

    def mx(W, T=4, kt=2, f=FP6, xdt=0, ws=fake(0x4000), wsb=None, x=fake()):
        need = L.moe_expert_ffn_mx_workspace_bytes(T, kt, ctypes.byref(W), f)
        return L.moe_expert_ffn_mx(x, xdt, T, kt, ctypes.byref(W), f, fake(0x100), fake(0x200), fake(0x300),
                                   ws, need if wsb is None else wsb, None)

    W = weights(H=256, I=512, hidden=256, inter=512)
    for name, (N, K) in (("gate", (512, 256)), ("up", (512, 256)), ("down", (256, 512))):
        p = getattr(W, name)
        p.w_row_stride, p.w_expert_stride = K // 2, N * K // 2
        p.s_row_stride, p.s_expert_stride = K // 32, N * K // 32
    need = L.moe_expert_ffn_mx_workspace_bytes(4, 2, ctypes.byref(W), FP6)
    # x codes + x scales + h codes + h scales + tile table
    assert need >= 4 * 192 + 4 * 8 + 8 * 384 + 8 * 16
    assert L.moe_expert_ffn_mx(None, 0, 0, 2, None, FP6, None, None, None, None, 0, None) == OK
    assert mx(W, f=0) == DTYPE
    assert mx(W, xdt=1) == DTYPE
    assert mx(weights(fmt=m.MOE_W_FP16, hidden=256, inter=512), xdt=0) == DTYPE
    assert mx(W, wsb=need - 1) == WORKSPACE
    assert mx(W, ws=fake(0x4008)) == ALIGN
    assert mx(W, x=None) == NULL
    assert mx(weights(hidden=96, inter=512)) == SHAPE      # hidden not a multiple of 256
    assert mx(weights(hidden=256, inter=96)) == SHAPE      # inter not a multiple of 256
    W2 = weights(H=256, I=512, hidden=256, inter=512)
    W2.gate.s_row_stride = 10
    assert mx(W2) == ALIGN                                  # scale rows must be 4-byte aligned
    W3 = weights(H=256, I=512, hidden=256, inter=512)
    W3.up.scales = P + 0x20004
    assert mx(W3) == ALIGN
    offs = (ctypes.c_size_t * 4)()
    assert L.moe_expert_ffn_mx_workspace_layout(4, 2, ctypes.byref(W), FP6, offs) == OK
    assert 0 == offs[0] < offs[1] < offs[2] < offs[3] < need and all(o % 256 == 0 for o in offs)
    assert L.moe_expert_ffn_mx_workspace_layout(4, 2, ctypes.byref(W), 7, offs) == DTYPE
    assert L.moe_expert_ffn_mx_workspace_layout(0, 2, ctypes.byref(W), FP6, offs) == SHAPE
    assert L.moe_expert_ffn_mx_workspace_layout(4, 2, None, FP6, offs) == NULL


def test_combine_and_dequant_validation():
    L = m.lib()
    assert L.moe_combine(None, None, 0, 2, 64, None, None) == OK
    assert L.moe_combine(fake(), fake(0x100), 4, 2, 66, fake(0x200), None) == SHAPE
    assert L.moe_combine(fake(), fake(0x100), 4, 0, 64, fake(0x200), None) == SHAPE
    assert L.moe_combine(None, fake(0x100), 4, 2, 64, fake(0x200), None) == NULL
    assert L.moe_combine(fake(4), fake(0x100), 4, 2, 64, fake(0x200), None) == ALIGN
    assert L.moe_mxfp4_dequant(fake(), fake(0x100), 3, 48, 24, 2, fake(0x200), None) == BLOCK
    assert L.moe_mxfp4_dequant(fake(), fake(0x100), 3, 64, 16, 2, fake(0x200), None) == SHAPE
    assert L.moe_mxfp4_dequant(fake(8), fake(0x100), 3, 64, 32, 2, fake(0x200), None) == BLOCK
    assert L.moe_mxfp4_dequant(fake(), fake(0x100), 3, 64, 40, 2, fake(0x200), None) == BLOCK
    assert L.moe_mxfp4_dequant(fake(), fake(0x100), 3, 64, 32, 2, fake(0x208), None) == ALIGN
    assert L.moe_mxfp4_dequant(None, fake(0x100), 3, 64, 32, 2, fake(0x200), None) == NULL


def test_stream_read_validation():
    L = m.lib()
    assert L.moe_stream_read(None, 0, None, None) == OK           # nothing to read
    assert L.moe_stream_read(None, 64, fake(), None) == NULL
    assert L.moe_stream_read(fake(), 64, None, None) == NULL
    assert L.moe_stream_read(fake(8), 64, fake(0x100), None) == ALIGN
    assert L.moe_stream_read(fake(), 40, fake(0x100), None) == ALIGN


def test_workspace_queries_are_host_only():
    L = m.lib()
    assert L.moe_route_workspace_bytes(0, 64, 8) == 0
    assert L.moe_route_workspace_bytes(8192, 7168, 256) >= 4 * 8192 * 256
    W = weights(H=7168, I=2048, E=257)
    # two 16-bit h planes plus the tile table (16 bytes per tile of the bound)
    assert L.moe_expert_ffn_workspace_bytes(8192, 9, ctypes.byref(W)) >= 4 * 8192 * 9 * 2048 + 16 * 257


def test_expert_ffn_static_validation():
    """The no-allocation FFN: checks that come before the scratch array is looked up."""
    L = m.lib()
    assert L.moe_expert_ffn_static(None, 0, 0, 2, None, None, None, None, None) == OK     # T = 0
    assert L.moe_expert_ffn_static(fake(), 0, 4, 2, None, fake(), fake(), fake(), None) == NULL
    assert L.moe_expert_ffn_static(fake(), 0, -1, 2, ctypes.byref(weights()), fake(), fake(), fake(), None) == SHAPE
    W = weights(E=256, H=7168, I=2048)
    need = L.moe_expert_ffn_workspace_bytes(300, 8, ctypes.byref(W))
    assert need > m.MOE_FFN_STATIC_SCRATCH_BYTES
    assert L.moe_expert_ffn_static(fake(), 0, 300, 8, ctypes.byref(W), fake(0x100), fake(0x200), fake(0x300),
                                   None) == WORKSPACE


def test_range_path_validation():
    """moe_expert_ffn_f16 and moe_combine_restore (Cascadia Eq. 1) reject bad arguments on the host."""
    L = m.lib()
    W = weights()
    need = L.moe_expert_ffn_f16_workspace_bytes(4, 2, ctypes.byref(W))
    assert need >= 2 * 4 * 2 * 96 * 2

    def f16(W, n=4, T=4, kt=2, xdt=0, y=fake(0x300), ws=fake(0x4000), wsb=need):
        return L.moe_expert_ffn_f16(fake(), xdt, T, kt, ctypes.byref(W), n, fake(0x100), fake(0x200), y, ws, wsb,
                                    None)

    assert L.moe_expert_ffn_f16(None, 0, 0, 2, None, 4, None, None, None, None, 0, None) == OK
    assert f16(W, n=-1) == SHAPE and f16(W, n=31) == SHAPE
    assert f16(W, xdt=1) == DTYPE
    assert f16(W, y=None) == NULL
    assert f16(W, y=fake(0x301)) == ALIGN
    assert f16(W, wsb=need - 1) == WORKSPACE
    assert f16(weights(up__w=P + 8)) == BLOCK
    cr = lambda **k: L.moe_combine_restore(k.get("ys", fake()), k.get("w", fake(0x100)), k.get("T", 4), 2,
                                           k.get("H", 64), k.get("n", 4), k.get("y", fake(0x200)), None)
    assert L.moe_combine_restore(None, None, 0, 2, 64, 4, None, None) == OK
    assert cr(n=-2) == SHAPE and cr(n=31) == SHAPE and cr(H=66) == SHAPE
    assert cr(ys=None) == NULL
    assert cr(ys=fake(4)) == ALIGN and cr(y=fake(0x208)) == ALIGN


def test_row_shape_and_padding_validation():
    """moe_row_shape (host) picks the smallest supported shape that holds T; moe_pad_rows checks."""
    L = m.lib()
    assert m.moe_row_shape(5, [1, 2, 4, 8, 16]) == 8
    assert m.moe_row_shape(8, [16, 8, 1]) == 8
    assert m.moe_row_shape(0, [4, 2]) == 2
    assert m.moe_row_shape(17, [1, 16]) == -1
    assert m.moe_row_shape(3, [0, -2, 3]) == 3
    assert m.moe_row_shape(-1, [4]) == -1
    assert L.moe_row_shape(4, None, 3) == -1
    assert L.moe_pad_rows(None, 0, 2, None, None, None) == OK
    assert L.moe_pad_rows(fake(), -1, 2, fake(0x100), fake(0x200), None) == SHAPE
    assert L.moe_pad_rows(fake(), 8, 0, fake(0x100), fake(0x200), None) == SHAPE
    assert L.moe_pad_rows(None, 8, 2, fake(0x100), fake(0x200), None) == NULL
    assert L.moe_pad_rows(fake(), 8, 2, fake(0x102), fake(0x200), None) == ALIGN


def test_sigmoid_route_validation():
    L = m.lib()
    r = lambda **k: L.moe_route_sigmoid(k.get("x", fake()), 0, k.get("T", 4), 64, fake(0x100), None, k.get("E", 8),
                                        k.get("k", 2), k.get("S", 0), k.get("g", 1.0), k.get("sw", 1.0),
                                        fake(0x200), fake(0x300), None, fake(0x1000), 1 << 20, None)
    assert L.moe_route_sigmoid(None, 0, 0, 64, None, None, 8, 2, 0, 1.0, 1.0, None, None, None, None, 0, None) == OK
    assert r(k=0) == TOPK and r(k=9) == TOPK
    assert r(E=0) == SHAPE
    assert r(g=float("nan")) == SHAPE and r(sw=float("inf")) == SHAPE
    assert r(x=None) == NULL
    assert r(x=fake(8)) == ALIGN


def codec_weights(fmt, E=4, H=64, I=96):
    W = m.moe_expert_weights()
    W.fmt, W.n_experts, W.hidden, W.inter = fmt, E, H, I
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        p = getattr(W, name)
        p.w = P + 0x10000
        p.scales = P + 0x20000
        p.w_row_stride, p.w_expert_stride = K // 2, N * K // 2
        srow = 2 * (K // 32) if fmt == m.MOE_W_INT4_G32 else K // 16
        p.s_row_stride, p.s_expert_stride = srow, N * srow
        if fmt == m.MOE_W_INT4_G32:
            p.zeros = P + 0x30000
            p.z_row_stride, p.z_expert_stride = (K // 32 + 1) // 2, N * ((K // 32 + 1) // 2)
        else:
            p.tensor_scale = P + 0x40000
    return W


def test_codec_validation():
    """INT4 group-32 and NVFP4 weights: bf16 activations, their scale data required, 32-value
    groups (16 code bytes) never cut."""
    for fmt in (m.MOE_W_INT4_G32, m.MOE_W_NVFP4):
        W = codec_weights(fmt)
        assert ffn(W, xdt=1) == DTYPE
        W = codec_weights(fmt); W.gate.scales = None
        assert ffn(W) == NULL
        W = codec_weights(fmt, H=48)
        assert ffn(W) == BLOCK
        W = codec_weights(fmt); W.up.w = P + 0x10008
        assert ffn(W) == BLOCK
        W = codec_weights(fmt); W.down.s_row_stride = 1
        assert ffn(W) == SHAPE
    W = codec_weights(m.MOE_W_INT4_G32); W.gate.zeros = None
    assert ffn(W) == NULL
    W = codec_weights(m.MOE_W_NVFP4); W.down.tensor_scale = None
    assert ffn(W) == NULL
    W = codec_weights(m.MOE_W_NVFP4); W.down.tensor_scale = P + 0x40002
    assert ffn(W) == ALIGN


def test_route_bucket_validation():
    L = m.lib()
    need = L.moe_route_bucket_workspace_bytes(4, 64, 8, 2, 0)
    assert need >= L.moe_route_workspace_bytes(4, 64, 8)
    big = L.moe_route_bucket_workspace_bytes(3000, 64, 8, 2, 0)  # router partials + bucketing scratch
    assert big >= L.moe_route_workspace_bytes(3000, 64, 8) + L.moe_bucket_workspace_bytes(6000, 8)
    W = weights(E=8)

    def rb(T=4, E=8, k=2, S=0, Wp=None, ws=fake(0x8000), wsb=need, fws=fake(0x40000), fwsb=1 << 24, ids=fake(0x200)):
        return L.moe_route_bucket(fake(), 0, T, 64, fake(0x100), None, E, k, S, ids, fake(0x300), None,
                                  fake(0x400), fake(0x500), fake(0x600), None, Wp, fws, fwsb, ws, wsb, None)

    assert L.moe_route_bucket(None, 0, 0, 64, None, None, 8, 2, 0, None, None, None, None, None, None, None, None,
                              None, 0, None, 0, None) == OK
    assert rb(k=0) == TOPK and rb(E=0) == SHAPE
    assert rb(ids=None) == NULL and rb(ids=fake(0x202)) == ALIGN
    assert rb(wsb=need - 1) == WORKSPACE
    assert rb(Wp=ctypes.byref(weights(E=9))) == SHAPE            # n_experts must be E + n_shared
    assert rb(Wp=ctypes.byref(W), fwsb=16) == WORKSPACE          # the FFN workspace holds the tile table
