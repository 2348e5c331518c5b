"""Cascadia's group-32 INT4 weights and NVFP4 weights on the GPU against the fp64 oracle (needs an
MI355X).  Both decode exactly into bf16 MFMA operands (INT4 as a high + low pair), so the exact
path's bars hold: max-abs error <= 2e-2 x RMS (the layer's tolerance) and <= 1e-3 x RMS."""
import numpy as np
import pytest
import torch

import oracle
import synth
import mxfp4_routed_expert_router_amd as moe
from gpu_support import DEV, EXACT_TOL, LAYER_TOL, expert_weights, note, require_gpu, rms_ratio

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


CODEC_CASES = [  # (T, H, I, E, S, k, pattern, sample)
    (37, 96, 160, 5, 0, 2, "routed", None),        # ragged H and I, an odd group count (3 along H)
    (200, 64, 96, 4, 0, 1, "one-expert", None),     # 200 rows of one expert: several tiles
    (40, 256, 128, 6, 1, 2, "routed", None),        # a shared expert
    (64, 4096, 1536, 128, 0, 8, "routed", [0, 1, 31, 32, 62, 63]),   # decode-sized experts
    (8, 7168, 2048, 256, 0, 8, "routed", None),     # the sweep's expert shape
]


@pytest.mark.parametrize("fmt", ["int4g32", "nvfp4"])
@pytest.mark.parametrize("case", CODEC_CASES, ids=[f"T{c[0]}-H{c[1]}-I{c[2]}-E{c[3]}+{c[4]}-k{c[5]}-{c[6]}" for c in CODEC_CASES])
def test_codec_expert_ffn(orc, case, fmt):
    T, H, I, E, S, k, pattern, sample = case
    note(f"codec ffn {fmt} {case}")
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, n_shared=S, inter=I, weight_format=fmt, router_std=0.3)
    L = synth.make_layer(wl, T, seed=23)
    if pattern == "routed":
        ids = orc.route(L.x, oracle.X_BF16, L.router, L.bias, k, S)["ids"]
    else:
        ids = np.full((T, 1), 2, np.int32)
    kt = ids.shape[1]
    b = orc.bucket(ids, wl.n_experts)
    mask = None
    if sample is not None:
        mask = np.zeros(T, np.uint8); mask[sample] = 1
        mask = np.repeat(mask, kt)
    W = oracle.ExpertWeights.from_layer(L)
    ref = orc.expert_ffn(L.x, oracle.X_BF16, kt, W, b["offsets"], b["sorted_slot"], mask)
    t = synth.to_torch(L, DEV)
    y = sync_np(moe.moe_expert_ffn(t["x"], expert_weights(t), torch.from_numpy(b["offsets"]).to(DEV),
                                   torch.from_numpy(b["sorted_slot"]).to(DEV), kt))
    rows = np.arange(T * kt) if mask is None else np.nonzero(mask)[0]
    err = rms_ratio(y[rows], ref[rows])
    note(f"  max-abs / rms = {err:.3e}")
    assert err <= LAYER_TOL and err <= EXACT_TOL


@pytest.mark.parametrize("fmt", ["int4g32", "nvfp4"])
def test_codec_layer(orc, fmt):
    """A whole layer (route, bucket, expert FFN, combine) with 64 routed experts, top-6 and two
    shared experts, as Cascadia's rows carry."""
    T, H, I, E, S, k = 48, 1024, 512, 64, 2, 6
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, n_shared=S, inter=I, weight_format=fmt, router_std=0.05)
    L = synth.make_layer(wl, T, seed=24)
    out = orc.layer(L)
    t = synth.to_torch(L, DEV)
    layer = moe.MoELayer(expert_weights(t), T, k, S, t["router"], t["bias"])
    y = sync_np(layer.forward(t["x"]))
    keep = out["route"]["near_tie"] == 0
    err = rms_ratio(y[keep], out["y"][keep])
    note(f"  {fmt} layer: max-abs / rms = {err:.3e} over {int(keep.sum())} tokens")
    assert err <= LAYER_TOL and err <= EXACT_TOL


def test_int4_range_path(orc):
    """Cascadia's own combination: INT4 group-32 experts on the range-managed binary16 path
    (Eq. 1) with A = 16."""
    T, H, I, E, k = 32, 512, 256, 16, 4
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, inter=I, weight_format="int4g32", router_std=0.1)
    L = synth.make_layer(wl, T, seed=25)
    r = orc.route(L.x, oracle.X_BF16, L.router, L.bias, k)
    b = orc.bucket(r["ids"], E)
    W = oracle.ExpertWeights.from_layer(L)
    ref_att = orc.expert_ffn_attenuated(L.x, oracle.X_BF16, k, W, 4, b["offsets"], b["sorted_slot"])
    ref_y = orc.combine_restore(ref_att, r["weights"], 4)
    t = synth.to_torch(L, DEV)
    ys = moe.moe_expert_ffn_f16(t["x"], expert_weights(t), 4, torch.from_numpy(b["offsets"]).to(DEV),
                                torch.from_numpy(b["sorted_slot"]).to(DEV), k)
    y = moe.moe_combine_restore(ys, torch.from_numpy(r["weights"].astype(np.float32)).to(DEV), 4)
    e1, e2 = rms_ratio(sync_np(ys).astype(np.float64), ref_att), rms_ratio(sync_np(y), ref_y)
    note(f"  INT4 range path: slots {e1:.3e}, y {e2:.3e}")
    assert e1 <= LAYER_TOL and e2 <= LAYER_TOL
