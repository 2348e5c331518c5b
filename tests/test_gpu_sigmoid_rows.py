"""Cascadia's sigmoid router and the fixed row-shape call on the GPU against the fp64 oracle
(needs an MI355X).

Sigmoid router (Cascadia Sec. 3.1): ids bit-exact on every token the oracle does not flag as a
near tie of its selection keys (valid top-k selections on flagged ones), sigmoid scores within
1e-5 absolute and 1e-4 relative, weights within 1e-5 x routed_scale; and a whole layer routed by
it (six routed plus two shared experts, as in Cascadia's rows) against the oracle's layer.

Fixed row shapes (Cascadia Sec. 3.2): the real rows of a padded call equal, bit for bit, the same
rows of an unpadded call at the same shape (padding changes nothing), they match the oracle on
the real tokens, and one captured graph per shape replays correctly for several row counts.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mxfp4_routed_expert_router_amd as moe
from gpu_support import (DEV, EXACT_TOL, LAYER_TOL, PROB_TOL, expert_weights, host_layer, note, require_gpu,
                         rms_ratio)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def sync_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def sel_bias(E, std, seed=17):
    if std == 0.0:
        return None
    return (np.random.default_rng(seed).standard_normal(E) * std).astype(np.float32)


def check_sigmoid(r, ids, w, sc, top_k, gamma):
    s = r["scores"]
    assert np.max(np.abs(sc - s)) <= PROB_TOL
    rel = float(np.max(np.abs(sc - s) / np.maximum(s, 1e-30)))
    note(f"  sigmoid scores: max relative error {rel:.2e}; near ties {int(r['near_tie'].sum())}")
    assert rel <= 1e-4
    ok = r["near_tie"] == 0
    assert np.array_equal(ids[ok], r["ids"][ok])
    assert np.max(np.abs(w[ok] - r["weights"][ok]), initial=0.0) <= PROB_TOL * max(1.0, abs(gamma))
    for t in np.nonzero(~ok)[0]:
        sel = ids[t, :top_k]
        assert len(set(sel.tolist())) == top_k
        assert abs(w[t, :top_k].sum() - gamma) <= 1e-5 * max(1.0, abs(gamma))


SIG_CASES = [  # (T, H, E, k, S, router_std, bias_std, gamma, shared_weight, x dtype)
    (176, 7168, 256, 6, 2, 1.0 / np.sqrt(7168), 0.02, 2.5, 1.0, "bf16"),   # Cascadia row: 6 routed + 2 shared
    (64, 4096, 128, 8, 0, 0.02, 0.0, 1.0, 1.0, "bf16"),
    (33, 96, 100, 5, 1, 0.3, 0.1, 1.5, 0.5, "fp16"),
    (5, 64, 1, 1, 0, 0.3, 0.0, 1.0, 1.0, "bf16"),
    (4, 64, 1024, 8, 0, 0.3, 0.05, 1.0, 1.0, "bf16"),
    (3, 64, 300, 200, 0, 0.3, 0.01, 1.0, 1.0, "bf16"),
]


@pytest.mark.parametrize("case", SIG_CASES, ids=[f"T{c[0]}-H{c[1]}-E{c[2]}-k{c[3]}-S{c[4]}-{c[9]}" for c in SIG_CASES])
def test_route_sigmoid(orc, case):
    T, H, E, k, S, rstd, bstd, gamma, sw, xdt = case
    note(f"sigmoid route {case}")
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, n_shared=S, router_std=rstd, act_dtype=xdt,
                      weight_format="mxfp4" if xdt == "bf16" else "fp16")
    x = synth.make_x(wl, T, seed=12)
    router, _ = synth.make_router(wl, seed=12)
    bias = sel_bias(E, bstd)
    xf = oracle.X_BF16 if xdt == "bf16" else oracle.X_FP16
    r = orc.route_sigmoid(x, xf, router, bias, k, S, gamma, sw)
    xt = torch.from_numpy(x).to(DEV).view(torch.bfloat16 if xdt == "bf16" else torch.float16)
    ids, w, sc = moe.moe_route_sigmoid(xt, torch.from_numpy(router).to(DEV), k,
                                       None if bias is None else torch.from_numpy(bias).to(DEV), S, gamma, sw,
                                       want_scores=True)
    ids, w, sc = sync_np(ids), sync_np(w), sync_np(sc)
    check_sigmoid(r, ids, w, sc, k, gamma)
    assert np.all(ids[:, k:] == np.arange(E, E + S)) and np.all(w[:, k:] == np.float32(sw))


def test_layer_sigmoid_router(orc):
    """A layer routed by the sigmoid router with six routed and two shared experts (MXFP4 weights):
    route -> bucket -> expert FFN -> combine against the oracle's same steps."""
    T, H, E, k, S, I = 40, 1024, 64, 6, 2, 512
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, n_shared=S, inter=I, router_std=0.05)
    L = synth.make_layer(wl, T, seed=13)
    bias = sel_bias(E, 0.02)
    gamma = 2.5
    r = orc.route_sigmoid(L.x, oracle.X_BF16, L.router, bias, k, S, gamma, 1.0)
    b = orc.bucket(r["ids"], E + S)
    W = oracle.ExpertWeights.from_layer(L)
    ref = orc.combine(orc.expert_ffn(L.x, oracle.X_BF16, k + S, W, b["offsets"], b["sorted_slot"]), r["weights"])
    t = synth.to_torch(L, DEV)
    ids, w, _ = moe.moe_route_sigmoid(t["x"], t["router"], k, torch.from_numpy(bias).to(DEV), S, gamma, 1.0)
    gb = moe.moe_bucket(ids, E + S)
    ys = moe.moe_expert_ffn(t["x"], expert_weights(t), gb.offsets, gb.sorted_slot, k + S)
    y = sync_np(moe.moe_combine(ys, w))
    keep = r["near_tie"] == 0
    err = rms_ratio(y[keep], ref[keep])
    note(f"  sigmoid-routed layer: max-abs / rms = {err:.3e} over {int(keep.sum())} tokens")
    assert err <= LAYER_TOL and err <= EXACT_TOL


# ------------------------------------------------------------------------------------------------
# fixed row shapes
# ------------------------------------------------------------------------------------------------
def make_fixed(L, shapes):
    wl = L.wl
    t = synth.to_torch(L, DEV)
    layer = moe.FixedShapeLayer(expert_weights(t), shapes, wl.top_k, t["router"], t["bias"], wl.n_shared)
    return layer, t


def oracle_rows(orc, L, T):
    """The oracle layer on the first T tokens of L, as a T-token call."""
    import dataclasses
    sub = dataclasses.replace(L, T=T, x=L.x[:T])
    out = orc.layer(sub)
    keep = out["route"]["near_tie"] == 0
    return out["y"], keep


@pytest.mark.parametrize("name,Tmax", [("decode", 64), ("sweep", 176)])
def test_padding_changes_no_real_row(orc, name, Tmax):
    """Shape 16, 5 real rows (then shape 64 / 176 with a ragged count): the padded call's real rows
    equal the unpadded call's at the same shape bit for bit, and the oracle's on those tokens."""
    L = host_layer(name, Tmax)
    shapes = [1, 16, Tmax]
    layer, t = make_fixed(L, shapes)
    for S, n in ((16, 5), (Tmax, Tmax - 3)):
        note(f"fixed shapes {name}: shape {S}, {n} real rows")
        layer.x[:S].copy_(t["x"][:S])
        layer.n_rows.fill_(S)                     # all rows real
        layer.run_shape(S)
        full = sync_np(layer.y[:S]).copy()
        layer.n_rows.fill_(n)                     # rows n.. are padding
        layer.run_shape(S)
        padded = sync_np(layer.y[:n]).copy()
        assert np.array_equal(padded.view(np.uint32), full[:n].view(np.uint32))
        ids = sync_np(layer.ids[:S])
        assert np.all(ids[n:] == -1) and np.all(sync_np(layer.weights[:S])[n:] == 0.0)
        ref, keep = oracle_rows(orc, L, n)
        err = rms_ratio(padded[keep], ref[keep])
        note(f"  vs oracle on the {n} real rows: max-abs / rms = {err:.3e}")
        assert err <= LAYER_TOL and err <= EXACT_TOL


def test_fixed_shape_graphs(orc):
    """One captured graph per shape; replays for 1, 3, 16, 9 and 1 real rows (the row count and the
    input rows change between replays) each equal the eager padded call bit for bit."""
    L = host_layer("decode", 32)
    layer, t = make_fixed(L, [1, 4, 16, 32])
    layer.capture()
    for n in (1, 3, 16, 9, 1, 32):
        x = t["x"][32 - n:].contiguous()          # different rows each time
        got = sync_np(layer.forward(x)).copy()
        eager = sync_np(layer.forward(x, use_graph=False)).copy()
        assert got.shape == (n, L.wl.hidden)
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), n
    import dataclasses
    sub = dataclasses.replace(L, T=9, x=np.ascontiguousarray(L.x[23:]))
    out = orc.layer(sub)
    got = sync_np(layer.forward(t["x"][23:].contiguous()))
    keep = out["route"]["near_tie"] == 0
    err = rms_ratio(got[keep], out["y"][keep])
    note(f"  graph replay, 9 rows vs oracle: {err:.3e}")
    assert err <= LAYER_TOL and err <= EXACT_TOL
