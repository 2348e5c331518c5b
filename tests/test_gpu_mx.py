"""MX mode on the GPU against the quantisation-aware fp64 oracle (needs an MI355X).

Bars: the activation quantiser's codes and E8M0 scales bit-exact (x is an exact input and both
sides decide each code on the same binary32 value), and the x codes the FFN call leaves in its
workspace likewise.  h is quantised from the kernel's fp32 h (FP8 x FP4 products are accumulated
by the matrix core at somewhat below fp32 precision) and by the oracle from its fp64 h, so an h
value lying on a rounding point may take the neighbouring code: the h codes read back from the
workspace must equal the oracle's except at such points (checked against the oracle's fp64 h),
and those must be rare.  Outputs are held to max-abs error <= 2e-2 x RMS of the MX oracle beyond
each element's flip budget (|W_down| times the change of the flipped h values, zero for rows whose
h matched).  The deviation of the MX mode from the exact oracle is printed, not asserted: it is
the price of the mode.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mxfp4_routed_expert_router_amd as moe
from gpu_support import DEV, LAYER_TOL, expert_weights, host_layer, note, require_gpu, rms_ratio

pytestmark = pytest.mark.gpu

FORMATS = {"fp8": (moe.MOE_MX_FP8_E4M3, oracle.MX_FP8_E4M3, 8), "fp6": (moe.MOE_MX_FP6_E2M3, oracle.MX_FP6_E2M3, 6),
           "fp4": (moe.MOE_MX_FP4_E2M1, oracle.MX_FP4_E2M1, 4)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def sync_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def unpack(packed: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Packed rows (the layout moe.h documents) -> one code per byte [n][K]."""
    n = packed.shape[0]
    if bits == 8:
        return packed[:, :K].copy()
    if bits == 4:
        return np.stack([packed & 0x0F, packed >> 4], axis=-1).reshape(n, -1)[:, :K]
    w = np.ascontiguousarray(packed.reshape(n, K // 32, 24)).view("<u8").astype(object)  # 3 words per block
    out = np.zeros((n, K // 32, 32), np.uint8)
    for j in range(32):
        bit = 6 * j
        v = w[:, :, bit // 64] >> (bit % 64)
        if bit % 64 > 58:
            v = v | (w[:, :, bit // 64 + 1] << (64 - bit % 64))
        out[:, :, j] = (v & 63).astype(np.uint8)
    return out.reshape(n, K)


def act_values(bits16: np.ndarray, fp16: bool) -> np.ndarray:
    if fp16:
        return bits16.view(np.float16).astype(np.float64)
    return (bits16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def special_x(n, K, fp16, seed=3):
    """bf16 (or fp16) rows with every interesting case: N(0,1) blocks at many magnitudes, an
    all-zero block, negative zeros, tiny (subnormal) values, values on rounding midpoints of the
    formats and blocks whose largest value lands on a power of two."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((n, K)) * np.exp2(rng.integers(-12, 12, (n, K // 32))).repeat(32, axis=1)
    v[0, :32] = 0.0
    v[0, 32:64] = -0.0
    v[0, 64:96] = rng.choice([1.0, 1.5, 2.0, 2.5, 3.0, 3.5, 5.0, 6.5, 7.25, 7.75, 0.0625, 0.1875], 32)
    v[0, 96:128] = rng.choice([1.0, 1.125, 0.5625, 4.5, 448.0, 464.0, 480.0, 240.0, 0.015625], 32)
    v[1, :32] = np.exp2(rng.integers(-140, -126, 32)) * rng.choice([-1.0, 1.0], 32)  # subnormal bf16
    v[1, 32:64] = 8.0
    v[1, 64:96] = -rng.random(32) * 1e-3
    if fp16:
        v = np.clip(v, -6e4, 6e4)
        return v.astype(np.float16).view(np.uint16)
    b = v.astype(np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)   # round to bf16
    b[0, 32:64] = 0x8000                                           # -0.0
    return b


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("fp16", [False, True], ids=["bf16", "fp16"])
def test_mx_quantize_bit_exact(orc, fmt, fp16):
    f_lib, f_orc, bits = FORMATS[fmt]
    n, K = 48, 2048
    note(f"mx quantize {fmt} {'fp16' if fp16 else 'bf16'} {n}x{K}")
    xb = special_x(n, K, fp16)
    codes, scales = orc.mx_quantize(act_values(xb, fp16), f_orc)
    xt = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.float16 if fp16 else torch.bfloat16)
    gc, gs = moe.moe_mx_quantize(xt, f_lib)
    got_c = unpack(sync_np(gc), K, bits)
    got_s = sync_np(gs)
    assert np.array_equal(got_s, scales), np.argwhere(got_s != scales)[:5]
    bad = np.argwhere(got_c != codes)
    assert bad.size == 0, [(tuple(i), got_c[tuple(i)], codes[tuple(i)]) for i in bad[:5]]


STEP_TOL = 0.02      # a differing h code is allowed only this close (in steps) to a rounding midpoint,
H_REL_TOL = 1e-4     # or this close relative to the block's largest |h| (the kernel's h error is absolute)
POW2_TOL = 1.5e-3    # a differing h scale only when amax is this close (in log2) to a power of two
FLIP_RATE = 2e-3     # at most this fraction of h values may differ (on the allowed points only)


def x_codes_from_ws(wsn, lay, T, H, bits):
    rb = H // 32 * 4 * bits
    c = wsn[lay["x_codes"]:lay["x_codes"] + T * rb].reshape(T, rb)
    return unpack(c, H, bits), wsn[lay["x_scales"]:lay["x_scales"] + T * H // 32].reshape(T, H // 32)


def h_codes_from_ws(wsn, lay, rows, I, bits):
    rb = I // 32 * 4 * bits
    c = np.stack([wsn[lay["h_codes"] + r * rb:lay["h_codes"] + (r + 1) * rb] for r in rows])
    s = np.stack([wsn[lay["h_scales"] + r * (I // 32):lay["h_scales"] + (r + 1) * (I // 32)] for r in rows])
    return unpack(c, I, bits), s


def value_table(orc, f_orc):
    n = 256 if f_orc == oracle.MX_FP8_E4M3 else (64 if f_orc == oracle.MX_FP6_E2M3 else 16)
    return np.array([orc.mx_value(f_orc, c) for c in range(n)])


def compare_h(orc, f_orc, h_pre, g_codes, g_scales):
    """GPU h codes/scales vs the oracle's quantisation of its fp64 h (rows aligned).  A differing
    value must be explainable by rounding: a scale one apart where amax sits on a power of two, or
    a code one step from the oracle's where the oracle's h lies on that step's midpoint; such points
    must be rare.  -> per row, {element: dequantised GPU h - dequantised oracle h} of its flips."""
    o_codes, o_scales = orc.mx_quantize(h_pre, f_orc)
    n, I = h_pre.shape
    val = value_table(orc, f_orc)
    flips = [dict() for _ in range(n)]
    n_diff = 0
    for r in range(n):
        for j in range(I // 32):
            sl = slice(32 * j, 32 * j + 32)
            Xo, Xg = 2.0 ** (int(o_scales[r, j]) - 127), 2.0 ** (int(g_scales[r, j]) - 127)
            if g_scales[r, j] != o_scales[r, j]:
                l2 = np.log2(np.max(np.abs(h_pre[r, sl])))
                assert abs(int(g_scales[r, j]) - int(o_scales[r, j])) == 1 and abs(l2 - np.round(l2)) <= POW2_TOL, \
                    (r, j, g_scales[r, j], o_scales[r, j], l2)
                for i in range(32):
                    flips[r][32 * j + i] = val[g_codes[r, 32 * j + i]] * Xg - val[o_codes[r, 32 * j + i]] * Xo
                n_diff += 32
                continue
            qmax = np.max(np.abs(h_pre[r, sl])) / Xo
            for i in np.nonzero(g_codes[r, sl] != o_codes[r, sl])[0]:
                vg, vo = val[g_codes[r, 32 * j + i]], val[o_codes[r, 32 * j + i]]
                if vg == vo:  # +0 and -0
                    continue
                q = h_pre[r, 32 * j + i] / Xo
                between = val[(val > min(vg, vo)) & (val < max(vg, vo))]
                tol = max(STEP_TOL * abs(vg - vo), H_REL_TOL * qmax)
                assert between.size == 0 and abs(q - (vg + vo) / 2) <= tol, (r, 32 * j + i, q, vg, vo, qmax)
                flips[r][32 * j + i] = (vg - vo) * Xo
                n_diff += 1
    assert n_diff <= FLIP_RATE * h_pre.size + 2, (n_diff, h_pre.size)
    return flips


def flip_budget(orc, L, e, flips, H):
    """|W_down[e]| @ |delta h| over the flipped elements: how far a row's y may move from the
    oracle's because its h took the other side of those rounding points (columns of W_down
    decoded by the oracle)."""
    budget = np.zeros(H)
    for n, dh in flips.items():
        b = n // 32
        col = orc.decode_matrix(np.ascontiguousarray(L.down_codes[e][:, 16 * b:16 * b + 16]),
                                np.ascontiguousarray(L.down_scales[e][:, b:b + 1]))[:, n % 32]
        budget += np.abs(col) * abs(dh)
    return budget


def excess_ratio(got, ref, budget):
    """max over elements of (|got - ref| - budget), over the RMS of ref."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref) - budget)) / max(rms, 1e-300)


def mx_ffn_case(orc, L, ids, fmt, sample_tokens=None):
    """GPU moe_expert_ffn_mx on the oracle's bucketing of ids vs the MX oracle: x codes bit-exact,
    h codes equal up to rounding-point flips, y_slots within the tolerance plus each row's flip
    budget.  The deviation from the exact oracle is printed."""
    f_lib, f_orc, bits = FORMATS[fmt]
    wl = L.wl
    T, H, I = L.T, wl.hidden, wl.inter
    kt = ids.shape[1]
    W = oracle.ExpertWeights.from_layer(L)
    b = orc.bucket(ids, wl.n_experts)
    mask = np.ones(T * kt, np.uint8)
    if sample_tokens is not None:
        mask = np.zeros(T, np.uint8); mask[sample_tokens] = 1
        mask = np.repeat(mask, kt)
    ref, h_pre = orc.expert_ffn_mx(L.x, oracle.X_BF16, kt, W, f_orc, b["offsets"], b["sorted_slot"], mask,
                                   want_h=True)
    t = synth.to_torch(L, DEV)
    Wt = expert_weights(t)
    ws = torch.empty(moe.moe_expert_ffn_mx_workspace_bytes(T, kt, Wt, f_lib), dtype=torch.uint8, device=DEV)
    y = moe.moe_expert_ffn_mx(t["x"], Wt, f_lib, torch.from_numpy(b["offsets"]).to(DEV),
                              torch.from_numpy(b["sorted_slot"]).to(DEV), kt, workspace=ws)
    got = sync_np(y)
    wsn = sync_np(ws)
    lay = moe.moe_expert_ffn_mx_workspace_layout(T, kt, Wt, f_lib)
    gxc, gxs = x_codes_from_ws(wsn, lay, T, H, bits)
    oxc, oxs = orc.mx_quantize(act_values(L.x, False), f_orc)
    assert np.array_equal(gxs, oxs) and np.array_equal(gxc, oxc)
    slots = np.nonzero(mask)[0]
    slots = slots[b["slot_pos"][slots] >= 0]
    rows = b["slot_pos"][slots]
    gh, ghs = h_codes_from_ws(wsn, lay, rows, I, bits)
    flips = compare_h(orc, f_orc, h_pre[rows], gh, ghs)
    ids_flat = ids.reshape(-1)
    budget = np.stack([flip_budget(orc, L, ids_flat[s], f, H) for s, f in zip(slots, flips)])
    err = excess_ratio(got[slots], ref[slots], budget)
    raw = rms_ratio(got[slots], ref[slots])
    exact = orc.expert_ffn(L.x, oracle.X_BF16, kt, W, b["offsets"], b["sorted_slot"], mask)
    dev_exact = rms_ratio(got[slots], exact[slots])
    n_flip = sum(len(f) for f in flips)
    note(f"  {fmt}: max-abs/rms vs MX oracle {raw:.3e} ({err:.3e} beyond the flip budget) over {slots.size} rows; "
         f"{n_flip} h values on a rounding point; vs exact oracle {dev_exact:.3e}")
    return err


MX_FFN_EDGE = [  # (T, H, I, E, k, id pattern)
    (16, 256, 512, 8, 2, "routed"),           # the tiny layer's shape
    (300, 256, 256, 3, 2, "routed"),          # ~200 rows per expert: a full 128-row tile + a ragged one
    (200, 512, 256, 4, 1, "one-expert"),      # 128 + 72 rows: 4 and 3 column tiles of 32
    (70, 256, 768, 3, 2, "two-experts"),      # 70 rows: 3 column tiles, the last one ragged
    (5, 256, 256, 50, 2, "routed"),           # most experts empty, one column tile each
    (33, 1024, 512, 2, 1, "routed"),          # 4 K steps in gate/up, 2 in down
]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("case", MX_FFN_EDGE, ids=[f"T{c[0]}-H{c[1]}-I{c[2]}-E{c[3]}-k{c[4]}-{c[5]}" for c in MX_FFN_EDGE])
def test_mx_expert_ffn_edges(orc, case, fmt):
    T, H, I, E, k, pattern = case
    note(f"mx expert ffn {fmt} {case}")
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, inter=I, router_std=0.3, weight_std=0.05)
    L = synth.make_layer(wl, T, seed=21)
    if pattern == "routed":
        ids = orc.route(L.x, oracle.X_BF16, L.router, L.bias, k)["ids"]
    elif pattern == "one-expert":
        ids = np.full((T, 1), 2, np.int32)
    else:
        ids = np.tile(np.array([0, 2], np.int32), (T, 1))
    assert mx_ffn_case(orc, L, ids, fmt) <= LAYER_TOL


MX_FFN_CASES = [("tiny", 16, None), ("decode", 64, [0, 33, 63])]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("name,T,sample", MX_FFN_CASES, ids=[f"{c[0]}-T{c[1]}" for c in MX_FFN_CASES])
def test_mx_expert_ffn(orc, name, T, sample, fmt):
    note(f"mx expert ffn {fmt} {name} T={T}")
    L = host_layer(name, T)
    wl = L.wl
    ids = orc.route(L.x, oracle.X_BF16, L.router, L.bias, wl.top_k, wl.n_shared)["ids"]
    assert mx_ffn_case(orc, L, ids, fmt, sample) <= LAYER_TOL


@pytest.mark.parametrize("fmt", ["fp6", "fp8", "fp4"])
def test_mx_layer_prefill(orc, fmt):
    """The whole prefill layer (T=8192, 256 routed + 1 shared expert, skewed routing) in MX mode,
    as the benchmark runs it; the oracle checks tokens of the hottest expert (its first and last
    128-row tiles) and of the coldest one, with the same h check as the FFN tests (tokens with an h
    value on a rounding point get the looser bound)."""
    f_lib, f_orc, bits = FORMATS[fmt]
    L = host_layer("prefill", 8192)
    wl = L.wl
    T, H, I = L.T, wl.hidden, wl.inter
    kt = wl.k_total
    note(f"mx layer prefill {fmt} T={T}")
    t = synth.to_torch(L, DEV)
    Wt = expert_weights(t)
    layer = moe.MoELayer(Wt, T, wl.top_k, wl.n_shared, t["router"], t["bias"], mx=f_lib)
    y = sync_np(layer.forward(t["x"]))
    wsn = sync_np(layer.ffn_ws)
    g_pos = sync_np(layer.buckets.slot_pos)
    r = orc.route(L.x, oracle.X_BF16, L.router, L.bias, wl.top_k, wl.n_shared)
    counts = np.bincount(r["ids"][:, :wl.top_k].reshape(-1), minlength=wl.n_routed)
    hot, cold = int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    has = lambda e: np.nonzero((r["ids"][:, :wl.top_k] == e).any(axis=1))[0]
    h = has(hot)
    last = (len(h) - 1) // 128 * 128  # first token of the hot expert's last 128-row tile
    sample = sorted(set(h[:3].tolist() + h[last:last + 2].tolist() + h[-2:].tolist() + has(cold)[:3].tolist()
                        + [0, T - 1]))
    sample = np.array([s for s in sample if r["near_tie"][s] == 0])
    note(f"  sampled tokens {sample.tolist()} (hot expert {hot}: {counts[hot]} tokens, cold {cold}: {counts[cold]})")
    b = orc.bucket(r["ids"], wl.n_experts)
    mask = np.zeros(T, np.uint8); mask[sample] = 1
    W = oracle.ExpertWeights.from_layer(L)
    ys, h_pre = orc.expert_ffn_mx(L.x, oracle.X_BF16, kt, W, f_orc, b["offsets"], b["sorted_slot"],
                                  np.repeat(mask, kt), want_h=True)
    ref = orc.combine(ys, r["weights"], mask)
    slots = (sample[:, None] * kt + np.arange(kt)).reshape(-1)
    lay = moe.moe_expert_ffn_mx_workspace_layout(T, kt, Wt, f_lib)
    gh, ghs = h_codes_from_ws(wsn, lay, g_pos[slots], I, bits)
    flips = compare_h(orc, f_orc, h_pre[b["slot_pos"][slots]], gh, ghs)
    ids_flat = r["ids"].reshape(-1)
    w_flat = r["weights"].reshape(-1)
    budget = np.zeros((len(sample), H))
    for q, (s, f) in enumerate(zip(slots, flips)):
        if f:
            budget[q // kt] += abs(w_flat[s]) * flip_budget(orc, L, ids_flat[s], f, H)
    err = excess_ratio(y[sample], ref[sample], budget)
    raw = rms_ratio(y[sample], ref[sample])
    note(f"  max-abs / rms vs MX oracle = {raw:.3e} ({err:.3e} beyond the flip budget) over {len(sample)} tokens; "
         f"{sum(len(f) for f in flips)} h values on a rounding point")
    assert err <= LAYER_TOL


def test_mx_deterministic():
    L = host_layer("tiny", 16)
    t = synth.to_torch(L, DEV)
    layer = moe.MoELayer(expert_weights(t), 16, 2, 0, t["router"], t["bias"], mx="fp6")
    a = sync_np(layer.forward(t["x"])).copy()
    b = sync_np(layer.forward(t["x"]))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_mx_zero_tokens():
    L = host_layer("tiny", 16)
    t = synth.to_torch(L, DEV)
    W = expert_weights(t)
    x0 = t["x"][:0]
    off = torch.zeros(9, dtype=torch.int32, device=DEV)
    y = moe.moe_expert_ffn_mx(x0, W, "fp6", off, torch.zeros(0, dtype=torch.int32, device=DEV), 2)
    assert y.shape == (0, 256)
    c, s = moe.moe_mx_quantize(x0, "fp8")
    torch.cuda.synchronize()


def test_mx_dropped_slots(orc):
    """Out-of-range ids: bucketing drops them, the MX FFN leaves their rows untouched and the
    valid rows still match the MX oracle exactly (MXFP6)."""
    L = host_layer("tiny", 16)
    r = orc.route(L.x, oracle.X_BF16, L.router, None, 2)
    ids = r["ids"].copy()
    ids[3, 1] = 8
    ids[7, 0] = -1
    t = synth.to_torch(L, DEV)
    b = moe.moe_bucket(torch.from_numpy(ids).to(DEV), 8)
    sentinel = torch.full((16 * 2, 256), 12345.0, dtype=torch.float32, device=DEV)
    y = moe.moe_expert_ffn_mx(t["x"], expert_weights(t), "fp6", b.offsets, b.sorted_slot, 2, out=sentinel)
    got = sync_np(y)
    ob = orc.bucket(ids, 8)
    W = oracle.ExpertWeights.from_layer(L)
    ref = orc.expert_ffn_mx(L.x, oracle.X_BF16, 2, W, oracle.MX_FP6_E2M3, ob["offsets"], ob["sorted_slot"])
    dropped = [3 * 2 + 1, 7 * 2 + 0]
    assert np.all(got[dropped] == 12345.0)
    keep = np.setdiff1d(np.arange(32), dropped)
    assert np.array_equal(got[keep], ref[keep].astype(np.float32))

