"""The range-managed FP16 path (Cascadia Sec. 3.3, Eq. 1) on the GPU against the fp64 oracle
(needs an MI355X).

moe_expert_ffn_f16 returns the attenuated expert outputs E(x) / A in binary16 (with h rounded to
binary16 on the way), moe_combine_restore divides each row's weights by its factor F, combines,
rounds the combination to binary16 and restores A F in fp32.  Bars: the binary16 slots against
the oracle's E / A, and the restored y against the oracle's plain layer output (which the oracle's
own Eq. 1 form reproduces bit for bit), both max-abs <= 2e-2 x RMS; three binary16 roundings
(h, the slots, the combination) cost about 1e-3 x RMS.  The MXFP4 workloads' expert outputs reach
8e5 to 2e6, far past binary16's 65504: there the attenuation is what keeps the path finite, and
the case without it is shown to overflow.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mxfp4_routed_expert_router_amd as moe
from gpu_support import DEV, LAYER_TOL, expert_weights, host_layer, note, require_gpu, rms_ratio, x_fmt

pytestmark = pytest.mark.gpu

F16_MAX = 65504.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def sync_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run_range(orc, L, n, ids=None, weights=None):
    """GPU Eq. 1 path on the oracle's routing and buckets -> (slots as fp64, y, oracle dict)."""
    wl = L.wl
    xf = x_fmt(wl)
    if ids is None:
        r = orc.route(L.x, xf, L.router, L.bias, wl.top_k, wl.n_shared)
        ids, weights = r["ids"], r["weights"]
    kt = ids.shape[1]
    b = orc.bucket(ids, wl.n_experts)
    W = oracle.ExpertWeights.from_layer(L)
    ref_att = orc.expert_ffn_attenuated(L.x, xf, kt, W, n, b["offsets"], b["sorted_slot"])
    ref_y = orc.combine(orc.expert_ffn(L.x, xf, kt, W, b["offsets"], b["sorted_slot"]), weights)
    t = synth.to_torch(L, DEV)
    Wt = expert_weights(t)
    ys = moe.moe_expert_ffn_f16(t["x"], Wt, n, torch.from_numpy(b["offsets"]).to(DEV),
                                torch.from_numpy(b["sorted_slot"]).to(DEV), kt)
    w32 = torch.from_numpy(np.ascontiguousarray(weights, np.float32)).to(DEV)
    y = moe.moe_combine_restore(ys, w32, n)
    return sync_np(ys).astype(np.float64), sync_np(y).astype(np.float64), ref_att, ref_y


@pytest.mark.parametrize("name,T,n", [("decode", 8, 4), ("tiny", 16, 0), ("sweep", 8, 6), ("decode", 64, 5)],
                         ids=["decode-T8-A16", "tiny-T16-A1", "sweep-T8-A64", "decode-T64-A32"])
def test_range_path(orc, name, T, n):
    """decode T=8 with the printed A = 16 (max |E| 8.4e5 becomes 5.3e4); the tiny layer needs no
    attenuation (max |E| 4.1e4); the sweep layer's 1.7e6 needs A = 64."""
    note(f"range path {name} T={T} A=2^{n}")
    L = host_layer(name, T)
    ys, y, ref_att, ref_y = run_range(orc, L, n)
    assert np.nanmax(np.abs(ref_att)) < F16_MAX
    e_slots = rms_ratio(ys, ref_att)
    e_y = rms_ratio(y, ref_y)
    note(f"  binary16 slots max-abs/rms = {e_slots:.3e}; restored y {e_y:.3e} (oracle max |E| "
         f"{np.nanmax(np.abs(ref_att)) * 2 ** n:.3e})")
    assert e_slots <= LAYER_TOL and e_y <= LAYER_TOL


def test_range_needs_attenuation(orc):
    """Without the attenuation the decode layer's expert outputs leave the binary16 range: every
    slot value past it comes out non-finite (infinite, or NaN where an infinite h meets
    infinities of both signs in the down projection) -- what Eq. 1 is for -- while A = 16 keeps
    every value finite."""
    L = host_layer("decode", 8)
    ys0, y0, ref0, _ = run_range(orc, L, 0)
    assert np.nanmax(np.abs(ref0)) > F16_MAX
    # past the binary16 rounding point 65520 by more than the path's own error (h is rounded to
    # binary16 on the way: about 3e-3 x RMS of E, a few hundred here, against a 2% margin of 1310)
    big = np.abs(ref0) > 65520.0 * 1.02
    assert big.any() and not np.any(np.isfinite(ys0[big]))
    note(f"  A = 1: {int(big.sum())} slot values past the binary16 range, all non-finite on the GPU")
    ys4, _, _, _ = run_range(orc, L, 4)
    assert np.all(np.isfinite(ys4))


def test_range_dense_slices_row_factor(orc):
    """The FP16 dense FFN as 8 all-active unit-weight slices: sum |w| = 8, so F = 8 divides every
    weight before the binary16 combination and is restored afterwards."""
    L = host_layer("dense_slices", 16)
    wl = L.wl
    ids = np.tile(np.arange(wl.n_experts, dtype=np.int32), (16, 1))
    w = np.ones((16, wl.n_experts))
    assert orc.row_factor(w[0]) == 8.0
    ys, y, ref_att, ref_y = run_range(orc, L, 0, ids, w)
    g, u, d = synth.make_dense_fp16(wl)
    dense = orc.dense_ffn_f16(L.x, oracle.X_FP16, g, u, d)
    e = rms_ratio(y, dense)
    note(f"  dense slices T=16: slots {rms_ratio(ys, ref_att):.3e}, y vs unsliced dense FFN {e:.3e}")
    assert e <= LAYER_TOL and rms_ratio(ys, ref_att) <= LAYER_TOL


def test_range_fp16_weights_beyond_f16(orc):
    """FP16 weights large enough that |h| passes 65504: the plain FFN's binary16 hi + lo pair of h
    cannot hold it (its documented limit), while the range path with A = 2^10 stays finite and
    within the bar."""
    H, I, E, k = 64, 64, 3, 2
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, inter=I, weight_format="fp16", act_dtype="fp16",
                      router_std=0.3, weight_std=16.0)
    L = synth.make_layer(wl, 24, seed=4)
    f = lambda a: np.ascontiguousarray(a).view(np.float16).astype(np.float64)
    X = f(L.x)
    with np.errstate(over="ignore"):
        hmax = max(np.max(np.abs((X @ f(L.gate_codes[e]).T) / (1 + np.exp(-(X @ f(L.gate_codes[e]).T)))
                                 * (X @ f(L.up_codes[e]).T))) for e in range(E))
    note(f"  max |h| over the experts {hmax:.3e}")
    assert hmax > F16_MAX
    ys, y, ref_att, ref_y = run_range(orc, L, 10)
    assert np.all(np.isfinite(ys)) and np.all(np.isfinite(y))
    e = rms_ratio(y, ref_y)
    note(f"  A = 2^10: slots {rms_ratio(ys, ref_att):.3e}, y {e:.3e}")
    assert e <= LAYER_TOL and rms_ratio(ys, ref_att) <= LAYER_TOL
    # the plain FFN on the same inputs (reported, not asserted: its h pair overflows)
    t = synth.to_torch(L, DEV)
    r = orc.route(L.x, oracle.X_FP16, L.router, L.bias, k)
    b = orc.bucket(r["ids"], E)
    yp = sync_np(moe.moe_expert_ffn(t["x"], expert_weights(t), torch.from_numpy(b["offsets"]).to(DEV),
                                    torch.from_numpy(b["sorted_slot"]).to(DEV), k))
    note(f"  plain FFN: {int(np.sum(~np.isfinite(yp)))} non-finite of {yp.size} outputs")
