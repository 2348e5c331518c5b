"""Pins of the fp64 oracle to things other than itself.

Each check takes a loaded oracle.Oracle and raises AssertionError when the oracle disagrees with
what the pages, a closed form, a library routine or brute force fixes.  test_oracle_pins.py runs
them on the real oracle; test_oracle_mutants.py runs them on copies of the oracle with a planted
mistake and requires that every mutant fails at least one of them.

Independent references used here (none calls the oracle):
  * minifloat(): a generic sign/exponent/fraction decoder, itself checked against numpy's binary16
    and binary32 conversions over every bit pattern, then used with (2 exponent bits, 1 fraction
    bit, bias 1) -- the E2M1 layout -- and compared with the page's magnitude set.
  * np_decode(): numpy nibble unpacking and block scales built from binary32 bit patterns.
  * numpy matmul, scipy softmax/expit, numpy lexsort/argsort/bincount.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

import synth
from oracle import ExpertWeights, X_BF16, X_FP16, W_MXFP4, W_FP16, W_INT4_G32, W_NVFP4

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------------
# independent references
# ------------------------------------------------------------------------------------------------
def minifloat(bits: int, e_bits: int, m_bits: int, bias: int, inf_nan: bool) -> float:
    sign = (bits >> (e_bits + m_bits)) & 1
    ex = (bits >> m_bits) & ((1 << e_bits) - 1)
    fr = bits & ((1 << m_bits) - 1)
    if ex == 0:
        v = math.ldexp(fr, 1 - bias - m_bits)
    elif inf_nan and ex == (1 << e_bits) - 1:
        v = math.nan if fr else math.inf
    else:
        v = math.ldexp((1 << m_bits) + fr, ex - bias - m_bits)
    return -v if sign else v


E2M1_REF = np.array([minifloat(c, 2, 1, 1, False) for c in range(16)])


def scale_ref(e: np.ndarray) -> np.ndarray:
    """2^(e-127) built from binary32 bit patterns (exponent field e, or the subnormal 2^-127 for
    e = 0); e = 255 has no binary32 power of two and is handled by the caller."""
    e = np.asarray(e, np.uint32)
    bits = np.where(e == 0, np.uint32(0x00400000), e << np.uint32(23)).astype(np.uint32)
    return bits.view(np.float32).astype(np.float64)


def np_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[N][K/2] packed bytes + [N][K/32] scale codes -> [N][K] float64 (low nibble first)."""
    N = codes.shape[0]
    K = codes.shape[1] * 2
    c = np.stack([codes & 0x0F, codes >> 4], axis=-1).reshape(N, K)
    return E2M1_REF[c] * np.repeat(scale_ref(scales), 32, axis=1)


def np_act(x_bits: np.ndarray, fmt: int) -> np.ndarray:
    if fmt == X_FP16:
        return x_bits.view(np.float16).astype(np.float64)
    return (x_bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


E4M3_REF = np.array([minifloat(c, 4, 3, 7, False) for c in range(256)])  # 0x7F / 0xFF (NaN) unused


def np_decode_int4(codes, scales16, zeros):
    """[N][K/2] unsigned codes, [N][K/32] binary16 scale bits, [N][ceil(K/64)] packed zero points
    -> [N][K] float64 (code - zero) * scale, group g = k // 32."""
    N, K = codes.shape[0], codes.shape[1] * 2
    q = np.stack([codes & 0x0F, codes >> 4], axis=-1).reshape(N, K).astype(np.int64)
    z = np.stack([zeros & 0x0F, zeros >> 4], axis=-1).reshape(N, -1)[:, :K // 32].astype(np.int64)
    s = np.ascontiguousarray(scales16).view(np.float16).astype(np.float64)
    return (q - np.repeat(z, 32, axis=1)) * np.repeat(s, 32, axis=1)


def np_decode_nvfp4(codes, scales, ts):
    """[N][K/2] E2M1 codes, [N][K/16] E4M3 scale codes, tensor scale -> [N][K] float64."""
    N, K = codes.shape[0], codes.shape[1] * 2
    c = np.stack([codes & 0x0F, codes >> 4], axis=-1).reshape(N, K)
    return E2M1_REF[c] * np.repeat(E4M3_REF[scales], 16, axis=1) * float(ts)


def np_weights(L):
    """Dense float64 [E'][N][K] gate, up, down for synth.LayerInputs L."""
    if L.wl.weight_format == "mxfp4":
        dec = lambda c, s: np.stack([np_decode(c[e], s[e]) for e in range(c.shape[0])])
        return dec(L.gate_codes, L.gate_scales), dec(L.up_codes, L.up_scales), dec(L.down_codes, L.down_scales)
    if L.wl.weight_format == "int4g32":
        dec = lambda c, s, z: np.stack([np_decode_int4(c[e], s[e], z[e]) for e in range(c.shape[0])])
        return tuple(dec(getattr(L, m + "_codes"), getattr(L, m + "_scales"), L.extras[m]) for m in ("gate", "up", "down"))
    if L.wl.weight_format == "nvfp4":
        dec = lambda c, s, t: np.stack([np_decode_nvfp4(c[e], s[e], t[e]) for e in range(c.shape[0])])
        return tuple(dec(getattr(L, m + "_codes"), getattr(L, m + "_scales"), L.extras[m]) for m in ("gate", "up", "down"))
    f = lambda c: np.ascontiguousarray(c).view(np.float16).astype(np.float64)
    return f(L.gate_codes), f(L.up_codes), f(L.down_codes)


def np_silu(z):
    return z * scipy.special.expit(z)


def np_expert(Wg, Wu, Wd, X):
    """X [n][H] -> [n][H]: the SwiGLU expert on each row."""
    g = X @ Wg.T
    u = X @ Wu.T
    return (np_silu(g) * u) @ Wd.T


def np_route(x, fmt, router, bias, k):
    X = np_act(x, fmt)
    logits = X @ router.astype(np.float64).T
    if bias is not None:
        logits = logits + bias.astype(np.float64)
    p = scipy.special.softmax(logits, axis=1)
    T, E = p.shape
    order = np.stack([np.lexsort((np.arange(E), -p[t])) for t in range(T)])
    return logits, p, order


def close(a, b, rel=1e-10, what=""):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= rel * scale, f"{what}: max abs err {err:.3e} > {rel:.1e} * {scale:.3e}"


def small_layer(T=6, H=64, E=5, k=2, S=0, I=96, seed=3, zipf=0.0, router_std=0.3, fmt="mxfp4", scale=(118, 127)):
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, n_shared=S, inter=I, weight_format=fmt,
                      act_dtype="fp16" if fmt == "fp16" else "bf16", router_std=router_std, zipf_s=zipf,
                      weight_std=0.05, scale_lo=scale[0], scale_hi=scale[1])
    return synth.make_layer(wl, T, seed=seed)


# ------------------------------------------------------------------------------------------------
# number formats
# ------------------------------------------------------------------------------------------------
def check_minifloat_reference(o):
    """The generic decoder agrees with numpy on every binary16 and bfloat16 pattern."""
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f16 = bits.astype(np.uint16).view(np.float16).astype(np.float64)
        bf = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    for b in range(0, 65536, 7):  # every 7th pattern keeps this quick; all exponent fields are hit
        r16 = minifloat(b, 5, 10, 15, True)
        rbf = minifloat(b, 8, 7, 127, True)
        assert (math.isnan(r16) and math.isnan(f16[b])) or r16 == f16[b], b
        assert (math.isnan(rbf) and math.isnan(bf[b])) or rbf == bf[b], b


def check_e2m1(o):
    """v(c) for all 16 codes: the E2M1 layout, magnitudes equal to the page's set, bit 3 = sign."""
    g = golden("mxfp4_format.json")
    assert sorted(set(abs(v) for v in E2M1_REF)) == g["e2m1_magnitudes"]
    for c in range(16):
        v = o.e2m1(c)
        assert v == E2M1_REF[c] and math.copysign(1, v) == math.copysign(1, E2M1_REF[c]), (c, v)
    assert sorted(abs(o.e2m1(c)) for c in range(8)) == [abs(o.e2m1(c)) for c in range(8)]


def check_e8m0(o):
    """2^(e-127) against binary32 bit patterns (e in 0..254) and the closed form at e = 255."""
    ref = scale_ref(np.arange(255))
    for e in range(255):
        assert o.e8m0(e) == ref[e], e
    assert o.e8m0(255) == 2.0 ** 128


def check_mxfp4_table(o):
    """All 16 x 256 (code, scale) pairs against v(c) * 2^(e-127) evaluated two other ways."""
    g = golden("mxfp4_format.json")
    bias = g["scale_bias"]
    for e in range(256):
        s = 2.0 ** (e - bias)
        for c in range(16):
            v = o.mxfp4(c, e)
            assert v == E2M1_REF[c] * s == math.ldexp(E2M1_REF[c], e - bias), (c, e, v)


def check_bf16_f16(o):
    for b in list(range(0, 65536, 11)) + [0x0001, 0x03FF, 0x0400, 0x7BFF, 0x7C00, 0x8001, 0xFC00, 0x3C00]:
        r16 = minifloat(b, 5, 10, 15, True)
        v = o.f16(b)
        assert (math.isnan(v) and math.isnan(r16)) or v == r16, (b, v, r16)
        rbf = minifloat(b, 8, 7, 127, True)
        v = o.bf16(b)
        assert (math.isnan(v) and math.isnan(rbf)) or v == rbf, (b, v, rbf)


def check_storage(o):
    """4 + 8/32 = 4.25 bits per weight, and the byte counts of the workloads."""
    g = golden("mxfp4_format.json")
    assert o.bits_per_weight() == g["bits_per_weight"]
    for n, k in [(1, 32), (7, 96), (2048, 7168), (4096, 1536)]:
        assert o.mxfp4_bytes(n, k) * 8 == n * k * g["bits_per_weight"], (n, k)
    for case in golden("storage_sizes.json")["cases"]:
        H, I, E = case["hidden"], case["inter"], case["experts"]
        total = E * (2 * o.mxfp4_bytes(I, H) + o.mxfp4_bytes(H, I))
        assert total == case["bytes"], case
        if "code_bytes" in case:
            assert E * 3 * I * H // 2 == case["code_bytes"] and E * 3 * I * H // 32 == case["scale_bytes"]


def check_nibble_order(o):
    """Hand-packed row: low nibble first, sign in bit 3."""
    g = golden("nibble_order.json")
    codes = np.frombuffer(bytes.fromhex(g["bytes_hex"]), np.uint8).reshape(1, 16)
    scales = np.array([[g["scale_code"]]], np.uint8)
    got = o.decode_matrix(codes, scales)[0]
    want = np.array(g["values"])
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want)), got
    # element access used by the FFN: expert 0's gate = this row, in a 1-row, 32-column matrix
    gate = codes.reshape(1, 1, 16); gs = scales.reshape(1, 1, 1)
    down = np.zeros((1, 32, 1), np.uint8); ds = np.full((1, 32, 1), 127, np.uint8)
    W = ExpertWeights(W_MXFP4, gate, gs, gate, gs, down, ds)
    for k in range(32):
        v = o.weight(W, "gate", 0, 0, k)
        assert v == want[k] and np.signbit(v) == np.signbit(want[k]), (k, v)


def check_weight_access(o):
    """orc_weight equals the numpy decode at every element, for strided (sliced) views too."""
    L = small_layer(T=1, H=64, I=96, E=3)
    W = ExpertWeights.from_layer(L)
    Wg, Wu, Wd = np_weights(L)
    rng = np.random.default_rng(0)
    for _ in range(200):
        e = int(rng.integers(3)); n = int(rng.integers(96)); k = int(rng.integers(64))
        assert o.weight(W, "gate", e, n, k) == Wg[e, n, k]
        assert o.weight(W, "up", e, n, k) == Wu[e, n, k]
        assert o.weight(W, "down", e, k, n) == Wd[e, k, n]
    # a column slice of the down projection (as in the all-active-slices layout)
    big = L.down_codes  # [3][64][48]
    view = big[:, :, 16:32]  # columns 32..63 of each expert: bytes 16..31, blocks 1..1
    sv = L.down_scales[:, :, 1:2]
    Wv = ExpertWeights(W_MXFP4, L.gate_codes, L.gate_scales, L.up_codes, L.up_scales, view, sv)
    for e in range(3):
        for m in range(0, 64, 9):
            for n in range(32):
                assert o.weight(Wv, "down", e, m, n) == Wd[e, m, 32 + n]


def check_silu(o):
    for z in [-1000.0, -50.0, -3.5, -1e-9, 0.0, 1e-9, 0.7, 2.0, 30.0, 700.0, 1000.0]:
        v = o.silu(z)
        assert not math.isnan(v)
        ref = z * scipy.special.expit(z)
        assert abs(v - ref) <= 1e-15 * max(1.0, abs(ref)), (z, v, ref)
    assert o.silu(-1000.0) == 0.0


def check_decode_matrix(o):
    L = small_layer(T=1, H=96, I=64, E=2, scale=(0, 254))
    for e in range(2):
        assert np.array_equal(o.decode_matrix(L.gate_codes[e], L.gate_scales[e]),
                              np_decode(L.gate_codes[e], L.gate_scales[e]))


# ------------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------------
def check_router_vs_numpy(o):
    for (T, H, E, k, zipf) in [(9, 64, 7, 3, 0.0), (5, 96, 16, 4, 1.2), (4, 32, 3, 1, 0.0)]:
        L = small_layer(T=T, H=H, E=E, k=k, zipf=zipf, router_std=0.4)
        r = o.route(L.x, X_BF16, L.router, L.bias, k)
        logits, p, order = np_route(L.x, X_BF16, L.router, L.bias, k)
        close(r["logits"], logits, 1e-12, "logits")
        close(r["probs"], p, 1e-12, "probs")
        for t in range(T):
            if not r["near_tie"][t]:
                assert list(r["ids"][t]) == list(order[t, :k]), (t, r["ids"][t], order[t, :k])
            sel = p[t, r["ids"][t]]
            close(r["weights"][t], sel / sel.sum(), 1e-12, "weights")
            assert abs(r["weights"][t].sum() - 1.0) <= 1e-12


def check_router_tiebreak(o):
    """Equal probabilities: lowest index first; the token is flagged as a near tie."""
    H, E = 32, 6
    router = np.zeros((E, H), np.float32)
    router[1] = 0.25; router[4] = 0.25; router[2] = 0.5  # experts 1 and 4 tie, 2 leads
    x = synth.to_bf16_bits(np.ones((1, H)))
    r = o.route(x, X_BF16, router, None, 3)
    assert list(r["ids"][0]) == [2, 1, 4], r["ids"]
    r2 = o.route(x, X_BF16, router, None, 2)
    assert list(r2["ids"][0]) == [2, 1]
    assert r["near_tie"][0] == 1 and r2["near_tie"][0] == 1
    # a clear gap is not flagged
    router[4] = 0.0
    r3 = o.route(x, X_BF16, router, None, 2)
    assert list(r3["ids"][0]) == [2, 1] and r3["near_tie"][0] == 0


def check_router_k_equals_E(o):
    """k = E: every expert is selected, in descending-probability order, and w = p."""
    L = small_layer(T=5, H=64, E=6, k=6)
    r = o.route(L.x, X_BF16, L.router, None, 6)
    _, p, order = np_route(L.x, X_BF16, L.router, None, 6)
    for t in range(5):
        assert sorted(r["ids"][t]) == list(range(6))
        close(r["weights"][t], p[t, r["ids"][t]], 1e-12, "w=p")
        if not r["near_tie"][t]:
            assert list(r["ids"][t]) == list(order[t])


def check_router_shift_invariance(o):
    """Adding one constant to every logit (through the bias) changes neither p nor the choice."""
    L = small_layer(T=7, H=64, E=9, k=3, zipf=1.2)
    a = o.route(L.x, X_BF16, L.router, L.bias, 3)
    b = o.route(L.x, X_BF16, L.router, (L.bias + np.float32(2.5)).astype(np.float32), 3)
    close(a["probs"], b["probs"], 1e-12, "shift")
    assert np.array_equal(a["ids"], b["ids"])
    # the bias shapes the choice: without it the routing differs on this input
    c = o.route(L.x, X_BF16, L.router, None, 3)
    assert not np.array_equal(a["ids"], c["ids"])


def check_router_shared(o):
    """Cascadia's 6 routed + 2 shared = 8 selections per row; shared ids follow the routed ones."""
    g = golden("cascadia_routing.json")
    E, k = g["routed_experts"], g["top_k"]
    S = len(g["shared_ids"])
    L = small_layer(T=3, H=32, E=E, k=k, S=S)
    r = o.route(L.x, X_BF16, L.router, None, k, S)
    assert r["ids"].shape[1] == g["selections_per_row"]
    for t in range(3):
        assert list(r["ids"][t, k:]) == g["shared_ids"]
        assert all(0 <= i < E for i in r["ids"][t, :k])
        assert list(r["weights"][t, k:]) == [1.0] * S
        assert abs(r["weights"][t, :k].sum() - 1.0) <= 1e-12


# ------------------------------------------------------------------------------------------------
# bucketing
# ------------------------------------------------------------------------------------------------
def check_bucket(o):
    rng = np.random.default_rng(1)
    for n, nb in [(1, 1), (40, 7), (300, 33), (1000, 257)]:
        ids = rng.integers(0, nb, n).astype(np.int32)
        b = o.bucket(ids, nb)
        assert np.array_equal(b["counts"], np.bincount(ids, minlength=nb))
        assert np.array_equal(b["offsets"], np.concatenate([[0], np.cumsum(np.bincount(ids, minlength=nb))]))
        assert np.array_equal(b["sorted_slot"], np.argsort(ids, kind="stable"))
        assert np.array_equal(b["slot_pos"][b["sorted_slot"]], np.arange(n))
        assert b["n_valid"] == n


def check_bucket_invalid(o):
    ids = np.array([3, -1, 0, 9, 3, 2, 100], np.int32)
    b = o.bucket(ids, 4)
    assert list(b["counts"]) == [1, 0, 1, 2] and b["n_valid"] == 4
    assert list(b["sorted_slot"]) == [2, 5, 0, 4, -1, -1, -1]
    assert list(b["slot_pos"]) == [2, -1, 0, -1, 3, 1, -1]


# ------------------------------------------------------------------------------------------------
# expert FFN, combine, layer
# ------------------------------------------------------------------------------------------------
def check_expert_apply_vs_numpy(o):
    """One expert on one vector: the decode-in-reduction sums equal numpy matmuls over the
    numpy-decoded matrices (non-square H != I catches a transposed operand)."""
    for fmt in ("mxfp4", "fp16"):
        L = small_layer(T=3, H=64, I=96, E=3, fmt=fmt)
        W = ExpertWeights.from_layer(L)
        Wg, Wu, Wd = np_weights(L)
        xf = X_BF16 if fmt == "mxfp4" else X_FP16
        X = np_act(L.x, xf)
        for e in range(3):
            ref = np_expert(Wg[e], Wu[e], Wd[e], X)
            for t in range(3):
                close(o.expert_apply(W, e, X[t]), ref[t], 1e-11, f"expert {fmt} e={e}")


def check_layer_vs_numpy(o):
    """The whole oracle layer against numpy routing + per-token expert mixture."""
    for (T, H, E, k, S, I) in [(8, 64, 5, 2, 0, 96), (6, 32, 4, 3, 1, 64)]:
        L = small_layer(T=T, H=H, E=E, k=k, S=S, I=I)
        out = o.layer(L)
        _, p, order = np_route(L.x, X_BF16, L.router, L.bias, k)
        Wg, Wu, Wd = np_weights(L)
        X = np_act(L.x, X_BF16)
        ref = np.zeros((T, H))
        for t in range(T):
            sel = order[t, :k]
            w = p[t, sel] / p[t, sel].sum()
            for j, e in enumerate(sel):
                ref[t] += w[j] * np_expert(Wg[e], Wu[e], Wd[e], X[t:t + 1])[0]
            for s in range(S):
                e = E + s
                ref[t] += np_expert(Wg[e], Wu[e], Wd[e], X[t:t + 1])[0]
        keep = out["route"]["near_tie"] == 0
        close(out["y"][keep], ref[keep], 1e-10, "layer")


def check_layer_forms(o):
    """Grouped path (bucket + slots + combine) == per-token brute force == dense mixture."""
    L = small_layer(T=7, H=64, E=6, k=2, S=1, I=64)
    out = o.layer(L)
    r = out["route"]
    yb = o.layer_bruteforce(L.x, X_BF16, out["weights"], r["ids"], r["weights"])
    yc = o.layer_dense_mixture(L.x, X_BF16, out["weights"], r["ids"], r["weights"])
    close(out["y"], yb, 1e-12, "grouped vs brute force")
    close(out["y"], yc, 1e-12, "grouped vs dense mixture")


def check_single_expert_swiglu(o):
    """E = k = 1: the layer is the textbook SwiGLU FFN W_d[SiLU(W_g x) * W_u x]."""
    L = small_layer(T=4, H=64, E=1, k=1, I=96)
    out = o.layer(L)
    Wg, Wu, Wd = np_weights(L)
    X = np_act(L.x, X_BF16)
    close(out["y"], np_expert(Wg[0], Wu[0], Wd[0], X), 1e-11, "swiglu")
    assert np.all(out["route"]["weights"] == 1.0)


def check_combine(o):
    rng = np.random.default_rng(2)
    T, kt, H = 5, 3, 16
    ys = rng.standard_normal((T * kt, H))
    w1 = rng.standard_normal((T, kt)); w2 = rng.standard_normal((T, kt))
    ref = np.einsum("tj,tjh->th", w1, ys.reshape(T, kt, H))
    close(o.combine(ys, w1), ref, 1e-13, "combine")
    onehot = np.zeros((T, kt)); onehot[:, 1] = 1.0
    assert np.array_equal(o.combine(ys, onehot), ys.reshape(T, kt, H)[:, 1])
    close(o.combine(ys, 2.0 * w1 - 3.0 * w2), 2.0 * o.combine(ys, w1) - 3.0 * o.combine(ys, w2), 1e-12, "linear")


def check_dense_slices(o):
    """Eq. 2: the sum of 8 all-active unit-weight slices equals the unsliced dense FFN, and the
    unsliced FFN equals numpy's."""
    g = golden("dense_slices.json")
    ns = g["n_slices"]
    wl = synth.custom(hidden=64, n_routed=ns, top_k=ns, inter=32, weight_format="fp16", act_dtype="fp16",
                      weight_std=0.05, dense_slices=True)
    L = synth.make_layer(wl, 3, seed=5)
    wg, wu, wd = synth.make_dense_fp16(wl, seed=5)
    out = o.layer(L)
    assert np.all(out["route"]["weights"] == g["slice_weight"])
    dense = o.dense_ffn_f16(L.x, X_FP16, wg, wu, wd)
    close(out["y"], dense, 1e-12, "slices vs dense")
    f = lambda a: a.view(np.float16).astype(np.float64)
    close(dense, np_expert(f(wg), f(wu), f(wd), np_act(L.x, X_FP16)), 1e-12, "dense vs numpy")


def np_route_sigmoid(x, fmt, router, bias, k, gamma):
    X = np_act(x, fmt)
    sc = scipy.special.expit(X @ router.astype(np.float64).T)
    key = sc + (0.0 if bias is None else bias.astype(np.float64))
    T, E = sc.shape
    order = np.stack([np.lexsort((np.arange(E), -key[t])) for t in range(T)])
    sel = order[:, :k]
    s_sel = np.take_along_axis(sc, sel, axis=1)
    return sc, sel, gamma * s_sel / s_sel.sum(axis=1, keepdims=True)


def check_router_sigmoid_vs_numpy(o):
    """Sigmoid router (Cascadia Sec. 3.1): scores against scipy's expit of numpy logits, selection
    against a lexsort of score + bias, weights against gamma * s / sum s over the selection, and the
    Cascadia row of six routed plus two shared selections (ids 256 and 257) from the fixture."""
    g = golden("cascadia_routing.json")
    for (T, H, E, k, S, gamma, sw, bias_std) in [(9, 64, 20, 3, 0, 1.0, 1.0, 0.0), (7, 96, 33, 5, 2, 2.5, 1.0, 0.3),
                                                 (4, 32, g["routed_experts"], g["top_k"], len(g["shared_ids"]),
                                                  1.5, 0.75, 0.1)]:
        wl = synth.custom(hidden=H, n_routed=E, top_k=k, n_shared=S, router_std=0.4)
        x = synth.make_x(wl, T, seed=3)
        router, _ = synth.make_router(wl, seed=3)
        rng = np.random.default_rng(E)
        bias = (rng.standard_normal(E) * bias_std).astype(np.float32) if bias_std else None
        r = o.route_sigmoid(x, X_BF16, router, bias, k, S, gamma, sw)
        sc, sel, w = np_route_sigmoid(x, X_BF16, router, bias, k, gamma)
        close(r["scores"], sc, 1e-12, "sigmoid scores")
        keep = r["near_tie"] == 0
        assert np.array_equal(r["ids"][keep, :k], sel[keep])
        close(r["weights"][keep, :k], w[keep], 1e-12, "sigmoid weights")
        close(r["weights"][:, :k].sum(axis=1), np.full(T, gamma), 1e-12, "routed weights sum to gamma")
        assert np.all(r["ids"][:, k:] == np.arange(E, E + S)) and np.all(r["weights"][:, k:] == sw)
        if E == g["routed_experts"]:
            assert r["ids"].shape[1] == g["selections_per_row"]
            assert r["ids"][:, k:].tolist() == [g["shared_ids"]] * T


def check_router_sigmoid_bias_selects_only(o):
    """The bias moves the selection, never the weights: a large bias on one expert puts it in every
    row, with the weight its unbiased score earns; without bias the selection is the softmax
    router's (both scores are increasing in the logit)."""
    L = small_layer(T=10, H=64, E=16, k=4, router_std=0.4)
    bias = np.zeros(16, np.float32); bias[11] = 10.0
    r = o.route_sigmoid(L.x, X_BF16, L.router, bias, 4)
    sc = scipy.special.expit(np_act(L.x, X_BF16) @ L.router.astype(np.float64).T)
    assert np.all(r["ids"][:, 0] == 11)
    close(r["weights"][:, 0], sc[:, 11] / np.take_along_axis(sc, r["ids"][:, :4], axis=1).sum(axis=1), 1e-12,
          "forced expert weight")
    r0 = o.route_sigmoid(L.x, X_BF16, L.router, None, 4)
    rs = o.route(L.x, X_BF16, L.router, None, 4)
    keep = (r0["near_tie"] == 0) & (rs["near_tie"] == 0)
    assert np.array_equal(r0["ids"][keep], rs["ids"][keep])


# ------------------------------------------------------------------------------------------------
# Other weight codecs: Cascadia's group-32 INT4 and NVFP4
# ------------------------------------------------------------------------------------------------
def check_int4g32_storage(o):
    """4 + 16/32 + 4/32 bits per weight: with Cascadia's shapes (hidden 6144, expert width 3072,
    8 experts per row, 64 sparse layers) that is the page's 16.76 GB of active expert weights per
    token; an 8-bit zero point (4.75 bits) or none (4.5) would give 17.21 or 16.31 GB."""
    g = golden("cascadia_int4.json")
    bpw = o.int4g32_bits_per_weight()
    assert bpw == 4.625
    weights = g["sparse_layers"] * g["experts_per_row"] * 3 * g["hidden"] * g["expert_inter"]
    gb = lambda b: round(weights * b / 8 / 1e9, 2)
    assert gb(bpw) == g["active_expert_gb_per_token"]
    assert gb(4.0 + g["scale_bits"] / g["group"]) != g["active_expert_gb_per_token"]
    assert gb(4.0 + (g["scale_bits"] + 8) / g["group"]) != g["active_expert_gb_per_token"]


def check_int4g32_decode(o):
    """(code - zero) * scale for every code x every zero point under normal, subnormal, negative and
    largest binary16 scales, against numpy's own unpacking and float16 conversion; odd group counts
    (a half-used last zero-point byte) and strided rows."""
    sc = np.array([0.0029296875, 1.0, -2.5, 6.1e-5, 5.96e-8, 65504.0, -0.0, 3.0517578e-05], np.float16)
    q = np.arange(16)
    N, K = 16 * 16, 32 * len(sc)                       # row = (code, zero); group g uses scale g
    codes = np.zeros((N, K), np.uint8)
    zeros = np.zeros((N, len(sc)), np.uint8)
    for i, (c, z) in enumerate((c, z) for c in q for z in q):
        codes[i] = c
        zeros[i] = z
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    zp = (zeros[:, 0::2] | (zeros[:, 1::2] << 4)).astype(np.uint8)
    s16 = np.tile(sc.view(np.uint16), (N, 1))
    W = ExpertWeights(W_INT4_G32, packed[None], s16[None], packed[None], s16[None], packed[None], s16[None],
                      {"gate": zp[None], "up": zp[None], "down": zp[None]})  # only the gate is read
    ref = np_decode_int4(packed, s16, zp)
    for n in range(0, N, 7):
        for k in range(0, K, 5):
            v = o.weight(W, "gate", 0, n, k)
            assert v == ref[n, k] or (np.isnan(v) and np.isnan(ref[n, k])), (n, k, v, ref[n, k])
    # a synthetic layer: odd group count (K = 96 -> 3 groups), every element
    L = small_layer(T=3, H=96, E=2, k=1, I=64, fmt="int4g32")
    Wl = ExpertWeights.from_layer(L)
    Wg, Wu, Wd = np_weights(L)
    for e in range(2):
        for n in range(0, 64, 3):
            for k in range(96):
                assert o.weight(Wl, "gate", e, n, k) == Wg[e, n, k]
                assert o.weight(Wl, "up", e, n, k) == Wu[e, n, k]
        for n in range(0, 96, 5):
            for k in range(64):
                assert o.weight(Wl, "down", e, n, k) == Wd[e, n, k]


def check_nvfp4_format(o):
    """NVFP4: 4.5 bits per weight before the tensor scale (page); every E2M1 code under every
    non-NaN E4M3 scale code times a tensor scale, against the minifloat reference; a synthetic
    layer's every element against numpy."""
    g = golden("nvfp4_format.json")
    assert o.nvfp4_bits_per_weight() == g["bits_per_weight"]
    assert g["element_bits"] + 8 / g["block"] == g["bits_per_weight"]
    scodes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    N, K = 16, 16 * len(scodes)
    codes = np.repeat(np.arange(16, dtype=np.uint8)[:, None], K, axis=1)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.tile(scodes, (N, 1))
    ts = np.array([0.3125], np.float32)
    W = ExpertWeights(W_NVFP4, packed[None], scales[None], packed[None], scales[None], packed[None], scales[None],
                      {"gate": ts, "up": ts, "down": ts})
    ref = np_decode_nvfp4(packed, scales, ts[0])
    for n in range(N):
        for k in range(0, K, 3):
            assert o.weight(W, "gate", 0, n, k) == ref[n, k], (n, k)
    L = small_layer(T=3, H=64, E=2, k=1, I=96, fmt="nvfp4")
    Wl = ExpertWeights.from_layer(L)
    Wg, Wu, Wd = np_weights(L)
    for e in range(2):
        for n in range(0, 96, 7):
            for k in range(64):
                assert o.weight(Wl, "gate", e, n, k) == Wg[e, n, k] and o.weight(Wl, "up", e, n, k) == Wu[e, n, k]
        for n in range(0, 64, 5):
            for k in range(96):
                assert o.weight(Wl, "down", e, n, k) == Wd[e, n, k]


def check_codec_layers_vs_numpy(o):
    """The whole oracle layer with INT4 group-32 and NVFP4 experts against numpy routing and a
    per-token expert mixture over the numpy-decoded weights (one shared expert included)."""
    for fmt in ("int4g32", "nvfp4"):
        T, H, E, k, S, I = 7, 64, 5, 2, 1, 96
        L = small_layer(T=T, H=H, E=E, k=k, S=S, I=I, fmt=fmt)
        out = o.layer(L)
        xf = X_BF16
        _, p, order = np_route(L.x, xf, L.router, L.bias, k)
        Wg, Wu, Wd = np_weights(L)
        X = np_act(L.x, xf)
        ref = np.zeros((T, H))
        for t in range(T):
            sel = order[t, :k]
            w = p[t, sel] / p[t, sel].sum()
            for j, e in enumerate(list(sel) + list(range(E, E + S))):
                ref[t] += (w[j] if j < k else 1.0) * np_expert(Wg[e], Wu[e], Wd[e], X[t:t + 1])[0]
        keep = out["route"]["near_tie"] == 0
        close(out["y"][keep], ref[keep], 1e-10, f"layer {fmt}")


# ------------------------------------------------------------------------------------------------
# FP16 range management (Cascadia Sec. 3.3, Eq. 1)
# ------------------------------------------------------------------------------------------------
def check_eq1_row_factor(o):
    """F = 2^ceil(log2 max(1, sum |w|)): the fixture's hand-worked rows, and on random rows the
    defining property -- F is a power of two with F/2 < max(1, sum |w|) <= F -- checked with exact
    binary arithmetic (frexp) rather than log2."""
    g = golden("cascadia_range.json")
    for case in g["row_factor_cases"]:
        assert o.row_factor(np.array(case["weights"], np.float64)) == case["F"], case
    rng = np.random.default_rng(31)
    for _ in range(200):
        w = rng.standard_normal(rng.integers(1, 12)) * np.exp2(rng.integers(-4, 5))
        F = o.row_factor(w)
        m = max(1.0, float(np.sum(np.abs(w))))
        mant, ex = math.frexp(F)
        assert mant == 0.5 and F >= 1.0, F
        assert F / 2 < m <= F, (m, F)


def check_eq1_restores_plain_layer(o):
    """Eq. 1 preserves the function, and with powers of two and no overflow it does so exactly:
    the attenuated experts are the plain experts divided by A (printed example A_8 = 16) bit for
    bit, and the restored combine equals the plain combine bit for bit -- on rows whose weights
    sum to 1 (F = 1), 2 (one shared expert, F = 2) and 3 (two shared experts, F = 4)."""
    g = golden("cascadia_range.json")
    n = g["att_log2"]
    assert 2 ** n == g["A"]
    for S in (0, 1, 2):
        L = small_layer(T=6, H=64, E=5, k=2, S=S, I=96)
        W = ExpertWeights.from_layer(L)
        r = o.route(L.x, X_BF16, L.router, L.bias, 2, S)
        b = o.bucket(r["ids"], 5 + S)
        ys = o.expert_ffn(L.x, X_BF16, 2 + S, W, b["offsets"], b["sorted_slot"])
        ya = o.expert_ffn_attenuated(L.x, X_BF16, 2 + S, W, n, b["offsets"], b["sorted_slot"])
        assert np.array_equal(ya, ys / g["A"]), S
        F = np.array([o.row_factor(w) for w in r["weights"]])
        assert np.all(F == {0: 1.0, 1: 2.0, 2: 4.0}[S]), (S, F)
        y = o.combine(ys, r["weights"])
        yr = o.combine_restore(ya, r["weights"], n)
        assert np.array_equal(yr, y), S
        # the same steps in numpy, in the equation's order
        yt = np.einsum("tj,tjh->th", r["weights"] / F[:, None], ya.reshape(6, 2 + S, -1))
        close(yr, g["A"] * F[:, None] * yt, 1e-13, "eq1 numpy")
    # an FP16-weight layer (the arithmetic the equation is written for) and a larger exponent
    L = small_layer(T=4, H=64, E=3, k=2, S=1, I=64, fmt="fp16")
    W = ExpertWeights.from_layer(L)
    r = o.route(L.x, X_FP16, L.router, L.bias, 2, 1)
    b = o.bucket(r["ids"], 4)
    ys = o.expert_ffn(L.x, X_FP16, 3, W, b["offsets"], b["sorted_slot"])
    ya = o.expert_ffn_attenuated(L.x, X_FP16, 3, W, 9, b["offsets"], b["sorted_slot"])
    assert np.array_equal(ya * 512.0, ys)
    assert np.array_equal(o.combine_restore(ya, r["weights"], 9), o.combine(ys, r["weights"]))


# ------------------------------------------------------------------------------------------------
# MX activation formats (MX mode).  The pages fix only E2M1 + E8M0; these pins hold the oracle to
# the OCP MX element formats through independent decoders (minifloat, torch's float8_e4m3fn), to
# the nearest/ties-to-even/saturation rule by exhaustive comparison, and to the scale rule through
# exact binary fractions.
# ------------------------------------------------------------------------------------------------
MX_FORMATS = {o_fmt: spec for o_fmt, spec in [
    (1, dict(bits=8, e_bits=4, m_bits=3, bias=7, emax=8, vmax=448.0)),
    (2, dict(bits=4, e_bits=2, m_bits=1, bias=1, emax=2, vmax=6.0)),
    (3, dict(bits=6, e_bits=2, m_bits=3, bias=1, emax=2, vmax=7.5)),
]}


def mx_table(o, fmt):
    """Non-negative codes and values of a format (E4M3's NaN code 0x7F excluded)."""
    n = 1 << (MX_FORMATS[fmt]["bits"] - 1)
    codes = [c for c in range(n) if not (fmt == 1 and c == 0x7F)]
    return np.array(codes), np.array([o.mx_value(fmt, c) for c in codes])


def check_mx_tables(o):
    """Every code of every MX element format decodes as the generic minifloat decoder says (sign,
    exponent field with the format's bias, subnormals at field 0); E4M3 also against torch's
    float8_e4m3fn on all 256 patterns, with NaN exactly at S.1111.111; largest values 448, 6, 7.5."""
    import torch
    for fmt, sp in MX_FORMATS.items():
        for c in range(1 << sp["bits"]):
            v = o.mx_value(fmt, c)
            if fmt == 1 and (c & 0x7F) == 0x7F:
                assert math.isnan(v), c
                continue
            assert v == minifloat(c, sp["e_bits"], sp["m_bits"], sp["bias"], False), (fmt, c, v)
        _, vals = mx_table(o, fmt)
        assert vals.max() == sp["vmax"] and np.all(np.diff(vals) > 0), fmt
        assert o.mx_bits(fmt) == sp["bits"] and o.mx_emax(fmt) == sp["emax"]
        assert sp["vmax"] >= 2.0 ** sp["emax"] > sp["vmax"] / 2
    tv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    ov = np.array([o.mx_value(1, c) for c in range(256)])
    assert np.array_equal(np.isnan(tv), np.isnan(ov)) and np.array_equal(tv[~np.isnan(tv)], ov[~np.isnan(ov)])


def check_mx_encode_nearest(o):
    """Encoding picks the nearest value (exhaustive comparison with every code), an exact midpoint
    goes to the even code, values past the largest saturate to it, and the sign is the input's
    (including -0.0); E4M3 also equals torch's float8_e4m3fn conversion inside its range."""
    import torch
    rng = np.random.default_rng(11)
    for fmt, sp in MX_FORMATS.items():
        codes, vals = mx_table(o, fmt)
        mids = (vals[1:] + vals[:-1]) / 2
        q = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                            rng.uniform(0, sp["vmax"] * 1.3, 3000), [sp["vmax"] * 4, 1e30]])
        sign_bit = 1 << (sp["bits"] - 1)
        for v in q:
            c = o.mx_encode(fmt, float(v))
            assert c < sign_bit, (fmt, v, c)
            d = np.abs(vals - v)
            best = d.min()
            assert abs(o.mx_value(fmt, c) - v) == best, (fmt, v, c)
            ties = codes[d == best]
            if len(ties) > 1:
                assert c % 2 == 0 and c in ties, (fmt, v, c, ties)
            assert o.mx_encode(fmt, -float(v)) == c | sign_bit, (fmt, v)
        assert o.mx_encode(fmt, sp["vmax"] * 10) == codes[-1]
        assert o.mx_encode(fmt, -0.0) == sign_bit and o.mx_encode(fmt, 0.0) == 0
        assert o.mx_encode(fmt, -1e-30) == sign_bit
    q = rng.standard_normal(5000) * 60
    q = np.concatenate([q, (vals_e4 := mx_table(o, 1)[1]), (vals_e4[1:] + vals_e4[:-1]) / 2])
    q = q[np.abs(q) <= 448].astype(np.float32)
    tc = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    oc = np.array([o.mx_encode(1, float(v)) for v in q])
    assert np.array_equal(tc, oc)


def check_mx_scale_rule(o):
    """Scale code = floor(log2 amax) - emax + 127 for amax = (1 + j/8) 2^k (exact binary
    fractions, so floor(log2) is k), clamped to [0, 254]; an all-zero block takes code 0."""
    for fmt, sp in MX_FORMATS.items():
        for k in range(-140, 140, 3):
            for j in range(8):
                amax = math.ldexp(1.0 + j / 8.0, k)
                want = min(max(k - sp["emax"] + 127, 0), 254)
                assert o.mx_scale_code(fmt, amax) == want, (fmt, k, j)
        assert o.mx_scale_code(fmt, 0.0) == 0


def check_mx_quantize_fp8_vs_torch(o):
    """MXFP8 block quantisation against an independent torch formulation: per 32-block,
    X = 2^(floor(log2 amax) - 8) from torch.frexp, codes = float8_e4m3fn(clamp(v / X, +-448))."""
    import torch
    rng = np.random.default_rng(12)
    n, K = 6, 256
    v = rng.standard_normal((n, K)) * np.exp(rng.uniform(-6, 6, (n, K // 32))).repeat(32, axis=1)
    v[0, :32] = 0.0                                        # zero block
    v[1, 32:64] = np.float32(1.99) * 2.0 ** np.arange(32)  # wide range, top values saturate
    v[2, :32] = rng.choice([-3.0, -1.0, 0.5, 2.25, 448 / 256.0], 32)  # exact values and midpoints
    v = v.astype(np.float32).astype(np.float64)            # binary32 inputs, as the kernels see
    codes, scales = o.mx_quantize(v, 1)
    t = torch.from_numpy(v).reshape(n, K // 32, 32)
    amax = t.abs().amax(dim=2, keepdim=True)
    _, ex = torch.frexp(amax)
    sc = torch.where(amax > 0, (ex - 1 - 8 + 127).clamp(0, 254), torch.zeros_like(ex))
    X = torch.ldexp(torch.ones_like(amax), (sc - 127).to(torch.float64))
    tq = (t / X).clamp(-448, 448).float().to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, K).numpy()
    assert np.array_equal(scales, sc.reshape(n, K // 32).numpy().astype(np.uint8))
    # torch keeps +0 for -0.0 inputs in some paths; compare magnitudes there and signs elsewhere
    assert np.array_equal(codes & 0x7F, tq & 0x7F)
    nz = (codes & 0x7F) != 0
    assert np.array_equal(codes[nz], tq[nz])


def check_mx_quantize_blocks(o):
    """For every format: values that are representable at the block's own scale come back exactly;
    the block's largest element lands in the top binade [2^emax, vmax] (or saturates to vmax);
    every element is within half a spacing of its value; blocks are independent."""
    rng = np.random.default_rng(13)
    for fmt, sp in MX_FORMATS.items():
        codes_t, vals = mx_table(o, fmt)
        top = vals[vals >= 2.0 ** sp["emax"]]
        n, K = 4, 128
        S = rng.integers(-20, 20, (n, K // 32))
        pick = rng.choice(vals, (n, K)) * rng.choice([-1.0, 1.0], (n, K))
        pick[:, ::32] = rng.choice(top, (n, K // 32))        # each block holds a top-binade element
        v = pick * np.ldexp(1.0, S).repeat(32, axis=1)
        c, s = o.mx_quantize(v, fmt)
        assert np.array_equal(s.astype(int), S + 127), fmt
        assert np.array_equal(o.mx_dequantize(c, s, fmt), v), fmt
        w = rng.standard_normal((n, K)) * 3.0
        c, s = o.mx_quantize(w, fmt)
        d = o.mx_dequantize(c, s, fmt)
        X = np.ldexp(1.0, s.astype(int) - 127).repeat(32, axis=1)
        q = np.abs(w / X)
        for r in range(n):
            for b in range(K // 32):
                blk = q[r, 32 * b:32 * b + 32]
                m = np.argmax(blk)
                assert 2.0 ** sp["emax"] <= blk[m] < 2.0 ** (sp["emax"] + 1)
                assert abs(d[r, 32 * b + m]) / X[r, 32 * b] >= min(2.0 ** sp["emax"], sp["vmax"])
        qc = np.minimum(q, sp["vmax"]).reshape(-1)
        i_hi = np.searchsorted(vals, qc, side="left")          # first value >= q
        hi = vals[i_hi]
        lo = vals[np.maximum(np.searchsorted(vals, qc, side="right") - 1, 0)]  # last value <= q
        err = np.abs(np.abs(d / X).reshape(-1) - qc)
        assert np.all(err <= (hi - lo) / 2), fmt
        w2 = w.copy(); w2[:, 32:64] *= 1e6
        c2, s2 = o.mx_quantize(w2, fmt)
        assert np.array_equal(c2[:, :32], c[:, :32]) and np.array_equal(c2[:, 64:], c[:, 64:])


def check_expert_ffn_mx_vs_numpy(o):
    """The MX-mode grouped FFN equals numpy on the same steps: x rows and h rows through the
    (separately pinned) MX round trip, numpy matmuls over the numpy-decoded weights; non-square
    shapes and two experts with several slots each."""
    for fmt in (1, 2, 3):
        L = small_layer(T=5, H=64, I=96, E=3, k=2)
        W = ExpertWeights.from_layer(L)
        r = o.route(L.x, X_BF16, L.router, L.bias, 2)
        b = o.bucket(r["ids"], 3)
        ys, hp = o.expert_ffn_mx(L.x, X_BF16, 2, W, fmt, b["offsets"], b["sorted_slot"], want_h=True)
        Wg, Wu, Wd = np_weights(L)
        X = np_act(L.x, X_BF16)
        rt = lambda a: o.mx_dequantize(*o.mx_quantize(a, fmt), fmt)
        Xq = rt(X)
        for s in range(10):
            e, t = r["ids"].reshape(-1)[s], s // 2
            h = np_silu(Xq[t:t + 1] @ Wg[e].T) * (Xq[t:t + 1] @ Wu[e].T)
            close(ys[s], (rt(h) @ Wd[e].T)[0], 1e-10, f"mx ffn fmt={fmt} slot={s}")
            close(hp[b["slot_pos"][s]], h[0], 1e-12, f"mx ffn h before quantisation fmt={fmt} slot={s}")
        ye = o.expert_ffn(L.x, X_BF16, 2, W, b["offsets"], b["sorted_slot"])
        assert not np.allclose(ys, ye, rtol=0, atol=0)  # the round trips change the result


ALL_CHECKS = [
    check_minifloat_reference, check_e2m1, check_e8m0, check_mxfp4_table, check_bf16_f16, check_storage,
    check_nibble_order, check_weight_access, check_silu, check_decode_matrix,
    check_router_vs_numpy, check_router_tiebreak, check_router_k_equals_E, check_router_shift_invariance,
    check_router_shared, check_router_sigmoid_vs_numpy, check_router_sigmoid_bias_selects_only,
    check_bucket, check_bucket_invalid,
    check_expert_apply_vs_numpy, check_layer_vs_numpy, check_layer_forms, check_single_expert_swiglu,
    check_combine, check_dense_slices, check_eq1_row_factor, check_eq1_restores_plain_layer,
    check_int4g32_storage, check_int4g32_decode, check_nvfp4_format, check_codec_layers_vs_numpy,
    check_mx_tables, check_mx_encode_nearest, check_mx_scale_rule, check_mx_quantize_fp8_vs_torch,
    check_mx_quantize_blocks, check_expert_ffn_mx_vs_numpy,
]
