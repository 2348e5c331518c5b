"""HIP path against the fp64 oracle, stage by stage and end to end (needs an MI355X).

Bars: routing ids and bucket permutations bit-exact (near ties flagged by the oracle are checked
for validity instead); router probabilities and routing weights within 1e-5 absolute (and 1e-4
relative); expert FFN and layer outputs with max-abs error <= 2e-2 x RMS of the oracle output (the
layer's tolerance), and, as a regression bar for the exact path's own precision, <= 1e-3 x RMS.
Workloads are the seeded synthetic layers of synth.WORKLOADS plus ragged and degenerate shapes.
Every sweep batch (T = 1 ... 176) is checked on all of its slots and tokens except T = 88 (a
24-token sample); the prefill layer (T = 8192) on a sample of about 150 tokens that reaches the
first, a middle and the last 128-row tile of its hottest expert (all routing and bucketing is still
whole).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mxfp4_routed_expert_router_amd as moe
from gpu_support import (DEV, EXACT_TOL, LAYER_TOL, check_route, expert_weights, host_layer, note, require_gpu,
                         rms_ratio, x_fmt)

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


# ------------------------------------------------------------------------------------------------
# decode primitive
# ------------------------------------------------------------------------------------------------
def test_dequant_every_code_and_scale(orc):
    """All 256 byte values (every code in both nibbles) under every scale code 0..252, bit-exact."""
    K = 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (253, 1))          # [253][256] bytes
    scales = np.repeat(np.arange(253, dtype=np.uint8)[:, None], K // 32, axis=1)
    ref = orc.decode_matrix(codes, scales).astype(np.float32)           # exact in fp32
    ref_bits = ref.view(np.uint32)
    assert np.all(ref_bits & 0xFFFF == 0)                               # exact in bf16 too
    note("dequant: 253 scale codes x 512 elements")
    out = moe.moe_mxfp4_dequant(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    got = sync_np(out.view(torch.int16)).view(np.uint16)
    assert np.array_equal(got, (ref_bits >> 16).astype(np.uint16))


def test_dequant_strided_rows(orc):
    rng = np.random.default_rng(7)
    big = rng.integers(0, 256, (9, 48), dtype=np.uint8)                 # rows of 48 bytes
    sc = rng.integers(118, 128, (9, 5), dtype=np.uint8)
    dc = torch.from_numpy(big).to(DEV)[:, 16:48]                         # K = 64 codes, row stride 48 B
    ds = torch.from_numpy(sc).to(DEV)[:, 1:3]
    got = sync_np(moe.moe_mxfp4_dequant(dc, ds).float())
    ref = orc.decode_matrix(np.ascontiguousarray(big[:, 16:48]), np.ascontiguousarray(sc[:, 1:3]))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("where", ["first", "inner", "last"])
def test_stream_read_reaches_every_piece(where):
    """moe_stream_read (a measurement utility) reads the whole buffer: one 16-byte piece holds the
    value that makes the checksum write the sink, placed at the first piece, inside a later
    workgroup's 64 KB chunk (4096 pieces) or at the very last piece of a ragged size; every other
    piece is zero, so the sink holds that value exactly when that piece was read."""
    magic = 0x9E3779B9
    n16 = 4096 * 1024 + 1003                             # 1024 whole chunks plus a ragged tail
    idx = {"first": 0, "inner": 4096 * 517 + 2049, "last": n16 - 1}[where]
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_stream_read(buf, sink)
    assert int(sync_np(sink)[0]) == 0                    # all-zero buffer: nothing written
    buf[4 * idx] = np.int64(magic).astype(np.int32).item()
    moe.moe_stream_read(buf, sink)
    assert int(sync_np(sink)[0]) & 0xFFFFFFFF == magic
    note(f"stream read: piece {idx} of {n16} reached")


# ------------------------------------------------------------------------------------------------
# router
# ------------------------------------------------------------------------------------------------
ROUTE_CASES = ([("tiny", 16)] + [("decode", t) for t in (1, 8, 32, 64)]
               + [("sweep", t) for t in synth.WORKLOADS["sweep"].tokens] + [("prefill", 8192)])


def run_route(wl, x, router, bias):
    return moe.moe_route(x, router, wl.top_k, bias, wl.n_shared, want_probs=True)


@pytest.mark.parametrize("name,T", ROUTE_CASES, ids=[f"{n}-T{t}" for n, t in ROUTE_CASES])
def test_route(orc, name, T):
    wl = synth.WORKLOADS[name]
    note(f"route {name} T={T}")
    x = synth.make_x(wl, T)
    router, bias = synth.make_router(wl)
    r = orc.route(x, x_fmt(wl), router, bias, wl.top_k, wl.n_shared)
    xt = torch.from_numpy(x).to(DEV).view(torch.bfloat16)
    ids, w, probs = run_route(wl, xt, torch.from_numpy(router).to(DEV),
                              None if bias is None else torch.from_numpy(bias).to(DEV))
    flagged = check_route(r, sync_np(ids), sync_np(w), sync_np(probs), wl.top_k)
    note(f"  near ties flagged: {flagged} of {T}")


ROUTE_EDGE = [  # (T, H, E, k, S, router_std, zipf)
    (5, 64, 1, 1, 0, 0.3, 0.0),       # one expert
    (9, 32, 7, 7, 0, 0.5, 0.0),       # k = E, E not a multiple of 64
    (33, 96, 100, 5, 0, 0.3, 1.2),    # ragged H, biased logits
    (4, 64, 1024, 8, 0, 0.3, 0.0),    # maximum expert count
    (6, 64, 256, 6, 2, 0.3, 0.0),     # Cascadia: 6 routed + 2 shared selections
    (3, 64, 300, 200, 0, 0.3, 0.0),   # k > 64: selections spread over several lanes' registers
]


@pytest.mark.parametrize("case", ROUTE_EDGE, ids=[f"T{c[0]}-H{c[1]}-E{c[2]}-k{c[3]}-S{c[4]}" for c in ROUTE_EDGE])
def test_route_edges(orc, case):
    T, H, E, k, S, std, zipf = case
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, n_shared=S, inter=64, router_std=std, zipf_s=zipf)
    note(f"route edge {case}")
    x = synth.make_x(wl, T, seed=11)
    router, bias = synth.make_router(wl, seed=11)
    r = orc.route(x, oracle.X_BF16, router, bias, k, S)
    ids, w, probs = moe.moe_route(torch.from_numpy(x).to(DEV).view(torch.bfloat16), torch.from_numpy(router).to(DEV),
                                  k, None if bias is None else torch.from_numpy(bias).to(DEV), S, want_probs=True)
    check_route(r, sync_np(ids), sync_np(w), sync_np(probs), k)
    assert np.all(sync_np(ids)[:, k:] == np.arange(E, E + S))


# ------------------------------------------------------------------------------------------------
# bucketing
# ------------------------------------------------------------------------------------------------
def bucket_case_ids(kind):
    rng = np.random.default_rng(5)
    if kind == "prefill":
        wl = synth.WORKLOADS["prefill"]
        x = synth.make_x(wl, 8192)
        router, bias = synth.make_router(wl)
        return oracle.load().route(x, oracle.X_BF16, router, bias, wl.top_k, wl.n_shared)["ids"].reshape(-1), 257
    n, nb = {"one": (7, 1), "exact-chunk": (512, 128), "ragged": (513, 33), "sweep": (1408, 256),
             "four-chunks": (2048, 257), "five-chunks": (2049, 300), "max-buckets-fused": (1500, 1024),
             "max-buckets": (3000, 1024), "skew": (5000, 64)}[kind]
    ids = rng.integers(0, nb, n).astype(np.int32)
    if kind == "skew":
        ids[rng.random(n) < 0.9] = 3
    return ids, nb


@pytest.mark.parametrize("kind", ["one", "exact-chunk", "ragged", "sweep", "four-chunks", "five-chunks",
                                  "max-buckets-fused", "max-buckets", "skew", "prefill"])
def test_bucket(orc, kind):
    ids, nb = bucket_case_ids(kind)
    note(f"bucket {kind}: {ids.size} slots, {nb} buckets")
    ref = orc.bucket(ids, nb)
    b = moe.moe_bucket(torch.from_numpy(ids).to(DEV), nb)
    for f in ("counts", "offsets", "sorted_slot", "slot_pos"):
        assert np.array_equal(sync_np(getattr(b, f)), ref[f]), f


def test_bucket_drops_invalid_ids(orc):
    rng = np.random.default_rng(9)
    for n in (300, 2000):
        ids = rng.integers(0, 16, n).astype(np.int32)
        ids[::7] = -3
        ids[::11] = 99
        ref = orc.bucket(ids, 16)
        b = moe.moe_bucket(torch.from_numpy(ids).to(DEV), 16)
        for f in ("counts", "offsets", "sorted_slot", "slot_pos"):
            assert np.array_equal(sync_np(getattr(b, f)), ref[f]), (n, f)


# ------------------------------------------------------------------------------------------------
# expert FFN (fed the oracle's buckets) and combine (fed oracle slots and weights)
# ------------------------------------------------------------------------------------------------
def ffn_vs_oracle(orc, L, ids, sample_tokens=None):
    """GPU moe_expert_ffn on the oracle's bucketing of `ids` vs the oracle's y_slots."""
    wl = L.wl
    T = L.T
    kt = ids.shape[1]
    W = oracle.ExpertWeights.from_layer(L)
    b = orc.bucket(ids, wl.n_experts)
    mask = None
    if sample_tokens is not None:
        mask = np.zeros(T, np.uint8); mask[sample_tokens] = 1
        mask = np.repeat(mask, kt)
    ref = orc.expert_ffn(L.x, x_fmt(wl), kt, W, b["offsets"], b["sorted_slot"], mask)
    t = synth.to_torch(L, DEV)
    y = moe.moe_expert_ffn(t["x"], expert_weights(t), torch.from_numpy(b["offsets"]).to(DEV),
                           torch.from_numpy(b["sorted_slot"]).to(DEV), kt)
    got = sync_np(y)
    rows = np.arange(T * kt) if mask is None else np.nonzero(mask)[0]
    return rms_ratio(got[rows], ref[rows])


FFN_CASES = [("tiny", 16, None), ("decode", 1, None), ("decode", 8, None), ("decode", 64, None),
             ("dense_slices", 1, None), ("dense_slices", 16, [0, 9, 15]), ("dense_slices", 128, [0, 64, 127])]


@pytest.mark.parametrize("name,T,sample", FFN_CASES, ids=[f"{c[0]}-T{c[1]}" for c in FFN_CASES])
def test_expert_ffn(orc, name, T, sample):
    note(f"expert ffn {name} T={T}")
    L = host_layer(name, T)
    wl = L.wl
    if wl.dense_slices:
        ids = np.tile(np.arange(wl.n_experts, dtype=np.int32), (T, 1))
    else:
        ids = orc.route(L.x, x_fmt(wl), L.router, L.bias, wl.top_k, wl.n_shared)["ids"]
    err = ffn_vs_oracle(orc, L, ids, sample)
    note(f"  max-abs / rms = {err:.3e}")
    assert err <= LAYER_TOL
    assert err <= EXACT_TOL


FFN_EDGE = [  # (T, H, I, E, k, fmt, id pattern)
    (37, 96, 160, 5, 2, "mxfp4", "routed"),      # ragged H and I (not multiples of 128 / 64)
    (200, 64, 96, 4, 1, "mxfp4", "one-expert"),  # 200 rows in one expert: several tiles
    (40, 64, 64, 3, 2, "mxfp4", "two-experts"),  # 40 rows per expert: 2-tile path
    (23, 32, 32, 6, 3, "fp16", "routed"),        # smallest FP16 shapes
    (64, 256, 128, 9, 8, "fp16", "routed"),
    (3, 64, 64, 50, 2, "mxfp4", "routed"),       # most experts empty
    # many small tiles: the row-split streaming kernels (full-K streams per wave, shared LDS
    # activation stages), at 1, 2, 3 and 5 chunks of 128 and with ragged row counts
    (64, 128, 4096, 64, 4, "mxfp4", "routed"),
    (64, 384, 4096, 64, 4, "mxfp4", "routed"),
    (64, 4096, 256, 64, 4, "mxfp4", "routed"),
    (64, 4096, 640, 64, 4, "mxfp4", "routed"),
    (256, 1024, 992, 128, 8, "mxfp4", "routed"),
    (256, 992, 1024, 256, 8, "mxfp4", "routed"),
    # 17 and 21 chunks of 128: scale-table windows of 16 chunks, with the last one partly used
    (128, 2176, 1024, 128, 4, "mxfp4", "routed"),
    (128, 2688, 1024, 128, 4, "mxfp4", "routed"),
    # many rows per expert: the 64-token tile kernels, with partial sub-tiles and tiles
    (512, 256, 384, 4, 2, "mxfp4", "routed"),
    (300, 384, 256, 3, 2, "mxfp4", "routed"),
    (200, 128, 256, 4, 1, "mxfp4", "one-expert"),
    (70, 256, 128, 3, 2, "mxfp4", "two-experts"),
    # 7 and 9 chunks of 128 in gate/up: the three-deep weight ring ends with 4 and 3 chunks left
    # (5 on the prefill and dense workloads, 1 and 2 above)
    (200, 896, 256, 4, 1, "mxfp4", "one-expert"),
    (160, 1152, 128, 3, 2, "mxfp4", "routed"),
    # the same tile kernels on FP16 weights: ragged tiles, 3 and 5 chunks of 128
    (300, 384, 640, 3, 2, "fp16", "routed"),
    (200, 128, 256, 4, 1, "fp16", "one-expert"),
    # FP16 weights on the K-split streaming kernels (one 16-token tile per expert): 5 and 3 chunks
    # of 128 (the four waves' K shares 2, 2, 1, 0 and 1, 1, 1, 0), and 9 and 8 chunks
    (8, 640, 384, 6, 3, "fp16", "routed"),
    (16, 1152, 1024, 8, 2, "fp16", "routed"),
    # at most 4 tokens: the tiny kernels (4-row tiles; down: whole-K rows per wave, h in LDS;
    # gate/up for up to 2 tokens and H a multiple of 512: x in LDS, weights two chunk pairs deep, a
    # wave's K share rounded to whole pairs, so that H = 512 and 1536 leave the last waves empty) at
    # 1 to 16 chunks of 128 per wave; an expert chosen twice per token (8 rows: two tiles); I not a
    # multiple of 512, H not a multiple of 64 and I above 2048 (the K-split kernels instead)
    (1, 512, 512, 8, 4, "mxfp4", "routed"),
    (2, 1024, 1024, 16, 4, "mxfp4", "duplicate"),
    (2, 1536, 512, 4, 1, "mxfp4", "one-expert"),
    (4, 1536, 512, 4, 1, "mxfp4", "one-expert"),
    (2, 2560, 1536, 6, 2, "mxfp4", "routed"),
    (1, 128, 512, 8, 4, "mxfp4", "routed"),
    (2, 256, 1536, 8, 3, "mxfp4", "routed"),
    (3, 192, 2048, 16, 4, "mxfp4", "routed"),
    (4, 64, 512, 4, 4, "mxfp4", "duplicate"),
    (4, 128, 1024, 4, 1, "mxfp4", "one-expert"),
    (2, 128, 384, 8, 2, "mxfp4", "routed"),
    (4, 96, 512, 4, 2, "mxfp4", "routed"),
    (4, 128, 2560, 8, 2, "mxfp4", "routed"),
    # the tiny gate/up kernel near its LDS bound: x of two tokens at H = 22528 (88 KB), 44 chunks
    # of 128 per wave
    (2, 22528, 256, 4, 2, "mxfp4", "routed"),
]


@pytest.mark.parametrize("case", FFN_EDGE, ids=[f"T{c[0]}-H{c[1]}-I{c[2]}-E{c[3]}-k{c[4]}-{c[5]}-{c[6]}" for c in FFN_EDGE])
def test_expert_ffn_edges(orc, case):
    T, H, I, E, k, fmt, pattern = case
    note(f"expert ffn edge {case}")
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, inter=I, weight_format=fmt,
                      act_dtype="bf16" if fmt == "mxfp4" else "fp16", router_std=0.3, weight_std=0.05)
    L = synth.make_layer(wl, T, seed=21)
    if pattern == "routed":
        ids = orc.route(L.x, x_fmt(wl), L.router, L.bias, k)["ids"]
    elif pattern == "one-expert":
        ids = np.full((T, 1), 2, np.int32)
    elif pattern == "duplicate":
        ids = np.tile(np.array([0, 0, 1, 2][:k], np.int32), (T, 1))
    else:
        ids = np.tile(np.array([0, 2], np.int32), (T, 1))
    err = ffn_vs_oracle(orc, L, ids)
    note(f"  max-abs / rms = {err:.3e}")
    assert err <= LAYER_TOL
    assert err <= EXACT_TOL


# Wide matrices with about 16 rows per expert: enough row blocks for the 8-wave row-split kernels.
# Down at 5 and 7 chunks of 128 (pairs of steps whose second chunk is missing; the 7-chunk case
# also runs the steady loop); gate/up at 5 chunks (a last step with one chunk).  Sampled tokens
# keep the oracle to a few seconds.
FFN_WIDE = [(128, 16384, 640, 32, 4), (128, 16384, 896, 32, 4), (128, 640, 8192, 32, 4)]


@pytest.mark.parametrize("case", FFN_WIDE, ids=[f"T{c[0]}-H{c[1]}-I{c[2]}-E{c[3]}-k{c[4]}" for c in FFN_WIDE])
def test_expert_ffn_wide(orc, case):
    T, H, I, E, k = case
    note(f"expert ffn wide {case}")
    wl = synth.custom(hidden=H, n_routed=E, top_k=k, inter=I, weight_format="mxfp4", act_dtype="bf16",
                      router_std=0.3, weight_std=0.05)
    L = synth.make_layer(wl, T, seed=22)
    ids = orc.route(L.x, x_fmt(wl), L.router, L.bias, k)["ids"]
    err = ffn_vs_oracle(orc, L, ids, sample_tokens=[0, 1, 2, 40, 63, 64, 100, 126, 127])
    note(f"  max-abs / rms = {err:.3e}")
    assert err <= LAYER_TOL
    assert err <= EXACT_TOL


@pytest.mark.parametrize("T,kt,H", [(1, 8, 4096), (37, 3, 96), (176, 8, 7168), (5, 11, 256), (3, 16, 64)])
def test_combine(orc, T, kt, H):
    rng = np.random.default_rng(T)
    ys = rng.standard_normal((T * kt, H)).astype(np.float32) * 1e3
    w = rng.random((T, kt)).astype(np.float32)
    ref = orc.combine(ys.astype(np.float64), w.astype(np.float64))
    y = moe.moe_combine(torch.from_numpy(ys).to(DEV), torch.from_numpy(w).to(DEV))
    assert rms_ratio(sync_np(y), ref) <= 1e-5


# ------------------------------------------------------------------------------------------------
# end to end
# ------------------------------------------------------------------------------------------------
def gpu_layer(L):
    wl = L.wl
    t = synth.to_torch(L, DEV)
    layer = moe.MoELayer(expert_weights(t), L.T, wl.top_k if not wl.dense_slices else wl.n_experts,
                         wl.n_shared, None if wl.dense_slices else t["router"], t["bias"])
    return layer, t


LAYER_CASES = ([("tiny", 16, None)] + [("decode", T, None) for T in (1, 8, 32, 64)]
               + [("prefill", 8192, "hot-cold")]
               + [("dense_slices", T, None if T < 128 else [0, 127]) for T in (1, 16, 128)])


def prefill_sample(r, wl, T):
    """About 150 tokens of the prefill batch: tokens of the hottest routed expert from its first,
    a middle and its last 128-row tile (its bucket is sorted by token, so the i-th token holding it
    is sorted row i of that bucket), tokens of the least-loaded active expert, and a seeded
    spread of others."""
    counts = np.bincount(r["ids"][:, :wl.top_k].reshape(-1), minlength=wl.n_routed)
    hot, cold = int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    has = lambda e: np.nonzero((r["ids"][:, :wl.top_k] == e).any(axis=1))[0]
    h = has(hot)
    n = len(h)
    last_tile = (n - 1) // 128
    mid_tile = last_tile // 2
    picks = list(h[:4]) + list(h[mid_tile * 128:mid_tile * 128 + 4]) + [h[mid_tile * 128 + 127]]
    picks += list(h[last_tile * 128:last_tile * 128 + 2]) + list(h[-4:])
    picks += list(has(cold)[:4]) + [0, T - 1]
    rng = np.random.default_rng(8192)
    picks += list(rng.choice(T, 130, replace=False))
    sample = sorted(set(int(v) for v in picks))
    note(f"  sampled {len(sample)} tokens (hot expert {hot}: {counts[hot]} tokens, tiles 0, {mid_tile} and "
         f"{last_tile}; cold expert {cold}: {counts[cold]})")
    return sample


@pytest.mark.parametrize("name,T,sample", LAYER_CASES, ids=[f"{c[0]}-T{c[1]}" for c in LAYER_CASES])
def test_layer(orc, name, T, sample):
    note(f"layer {name} T={T}")
    L = host_layer(name, T)
    wl = L.wl
    layer, t = gpu_layer(L)
    y = sync_np(layer.forward(t["x"]))
    if wl.dense_slices:
        rows = np.arange(T) if sample is None else np.array(sample)
        g, u, d = synth.make_dense_fp16(wl)
        ref = orc.dense_ffn_f16(L.x[rows], oracle.X_FP16, g, u, d)
        err = rms_ratio(y[rows], ref)
    else:
        r = orc.route(L.x, x_fmt(wl), L.router, L.bias, wl.top_k, wl.n_shared)
        if sample == "hot-cold":
            sample = prefill_sample(r, wl, T)
        mask = None
        if sample is not None:
            mask = np.zeros(T, np.uint8); mask[sample] = 1
        out = orc.layer(L, token_mask=mask)
        rows = np.arange(T) if sample is None else np.array(sample)
        rows = rows[out["route"]["near_tie"][rows] == 0]
        err = rms_ratio(y[rows], out["y"][rows])
    note(f"  max-abs / rms = {err:.3e} over {len(rows)} tokens")
    assert err <= LAYER_TOL
    assert err <= EXACT_TOL


# The concurrency sweep (the benchmark's workload): one oracle run per batch serves two checks --
# the expert FFN fed the oracle's buckets against the oracle's y_slots (every valid slot), and the
# whole GPU layer (route, bucket, FFN, combine) against the oracle's y on every token that is not
# a near tie.  T = 88 uses a 24-token sample to keep the oracle's share of the run down.
SWEEP_SAMPLES = {88: [0, 1, 2, 3, 10, 20, 30, 40, 43, 44, 45, 50, 55, 60, 63, 64, 65, 70, 75, 80, 84, 85, 86, 87]}


@pytest.mark.parametrize("T", synth.WORKLOADS["sweep"].tokens, ids=[f"sweep-T{t}" for t in synth.WORKLOADS["sweep"].tokens])
def test_sweep_ffn_and_layer(orc, T):
    L = host_layer("sweep", T)
    wl = L.wl
    kt = wl.k_total
    sample = SWEEP_SAMPLES.get(T)
    mask = None
    if sample is not None:
        mask = np.zeros(T, np.uint8); mask[sample] = 1
    note(f"sweep T={T}: oracle on {T if sample is None else len(sample)} tokens")
    out = orc.layer(L, token_mask=mask)
    r, b = out["route"], out["bucket"]
    t = synth.to_torch(L, DEV)
    W = expert_weights(t)
    ys = sync_np(moe.moe_expert_ffn(t["x"], W, torch.from_numpy(b["offsets"]).to(DEV),
                                    torch.from_numpy(b["sorted_slot"]).to(DEV), kt))
    toks = np.arange(T) if sample is None else np.array(sample)
    slots = (toks[:, None] * kt + np.arange(kt)).reshape(-1)
    err_ffn = rms_ratio(ys[slots], out["y_slots"][slots])
    layer = moe.MoELayer(W, T, wl.top_k, wl.n_shared, t["router"], t["bias"])
    y = sync_np(layer.forward(t["x"]))
    rows = toks[r["near_tie"][toks] == 0]
    err = rms_ratio(y[rows], out["y"][rows])
    note(f"  ffn max-abs / rms = {err_ffn:.3e} over {len(slots)} slots; layer {err:.3e} over {len(rows)} tokens")
    for e in (err_ffn, err):
        assert e <= LAYER_TOL
        assert e <= EXACT_TOL


@pytest.mark.parametrize("name,T", [("tiny", 16), ("sweep", 176)])
def test_deterministic(name, T):
    L = host_layer(name, T)
    layer, t = gpu_layer(L)
    a = sync_np(layer.forward(t["x"])).copy()
    b = sync_np(layer.forward(t["x"]))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_zero_tokens():
    L = host_layer("tiny", 16)
    t = synth.to_torch(L, DEV)
    W = expert_weights(t)
    x0 = t["x"][:0]
    ids, w, _ = moe.moe_route(x0, t["router"], 2)
    b = moe.moe_bucket(ids, 8)
    y = moe.moe_expert_ffn(x0, W, b.offsets, b.sorted_slot, 2)
    assert moe.moe_combine(y, w).shape == (0, 256)
    torch.cuda.synchronize()


def test_invalid_ids_are_dropped_safely(orc):
    """Out-of-range ids: bucket drops them, the FFN skips them, valid slots are still exact."""
    L = host_layer("tiny", 16)
    r = orc.route(L.x, oracle.X_BF16, L.router, None, 2)
    ids = r["ids"].copy()
    ids[3, 1] = 8
    ids[7, 0] = -1
    t = synth.to_torch(L, DEV)
    b = moe.moe_bucket(torch.from_numpy(ids).to(DEV), 8)
    sentinel = torch.full((32, 256), 12345.0, device=DEV)
    y = sync_np(moe.moe_expert_ffn(t["x"], expert_weights(t), b.offsets, b.sorted_slot, 2, out=sentinel))
    ref_b = orc.bucket(ids, 8)
    ref = orc.expert_ffn(L.x, oracle.X_BF16, 2, oracle.ExpertWeights.from_layer(L), ref_b["offsets"],
                         ref_b["sorted_slot"])
    assert np.all(y[3 * 2 + 1] == 12345.0) and np.all(y[7 * 2 + 0] == 12345.0)
    valid = ref_b["slot_pos"] >= 0
    assert rms_ratio(y[valid], ref[valid]) <= LAYER_TOL


def test_split_phases_equal_fused_call():
    """moe_expert_ffn_plan, moe_expert_ffn_gateup then moe_expert_ffn_down == moe_expert_ffn, bit for bit."""
    L = host_layer("decode", 8)
    wl = L.wl
    t = synth.to_torch(L, DEV)
    W = expert_weights(t)
    ids, w, _ = moe.moe_route(t["x"], t["router"], wl.top_k)
    b = moe.moe_bucket(ids, wl.n_experts)
    a = moe.moe_expert_ffn(t["x"], W, b.offsets, b.sorted_slot, wl.top_k)
    ws = torch.empty(moe.moe_expert_ffn_workspace_bytes(8, wl.top_k, W), dtype=torch.uint8, device=DEV)
    moe.moe_expert_ffn_plan(8, W, b.offsets, wl.top_k, ws)
    moe.moe_expert_ffn_gateup(t["x"], W, b.offsets, b.sorted_slot, wl.top_k, ws)
    c = moe.moe_expert_ffn_down(8, W, b.offsets, b.sorted_slot, wl.top_k, ws, torch.empty_like(a))
    assert np.array_equal(sync_np(a).view(np.uint32), sync_np(c).view(np.uint32))


def test_stale_plan_stays_in_bounds():
    """A tile schedule planned for a larger batch, then used for a smaller one: every entry that
    names rows past the smaller batch reads as empty (no access outside the buffers), and the
    properly planned call afterwards is exact again."""
    L = host_layer("decode", 64)
    wl = L.wl
    t = synth.to_torch(L, DEV)
    W = expert_weights(t)
    ids, w, _ = moe.moe_route(t["x"], t["router"], wl.top_k)
    b = moe.moe_bucket(ids, wl.n_experts)
    ws = torch.empty(moe.moe_expert_ffn_workspace_bytes(64, wl.top_k, W), dtype=torch.uint8, device=DEV)
    moe.moe_expert_ffn_plan(64, W, b.offsets, wl.top_k, ws)
    T2 = 8
    x2 = t["x"][:T2].contiguous()
    ids2, _, _ = moe.moe_route(x2, t["router"], wl.top_k)
    b2 = moe.moe_bucket(ids2, wl.n_experts)
    out = torch.empty((T2 * wl.top_k, wl.hidden), dtype=torch.float32, device=DEV)
    moe.moe_expert_ffn_gateup(x2, W, b2.offsets, b2.sorted_slot, wl.top_k, ws)
    moe.moe_expert_ffn_down(T2, W, b2.offsets, b2.sorted_slot, wl.top_k, ws, out)
    torch.cuda.synchronize()
    ref = moe.moe_expert_ffn(x2, W, b2.offsets, b2.sorted_slot, wl.top_k)
    moe.moe_expert_ffn_plan(T2, W, b2.offsets, wl.top_k, ws)
    moe.moe_expert_ffn_gateup(x2, W, b2.offsets, b2.sorted_slot, wl.top_k, ws)
    moe.moe_expert_ffn_down(T2, W, b2.offsets, b2.sorted_slot, wl.top_k, ws, out)
    assert np.array_equal(sync_np(ref).view(np.uint32), sync_np(out).view(np.uint32))


@pytest.mark.parametrize("name,T", [("decode", 8), ("sweep", 176)])
def test_graph_replay_equals_eager(name, T):
    """One layer call captured in a HIP graph: each of several replays, with eager work and
    synchronisations between them, reproduces the eager result bit for bit."""
    note(f"graph replay {name} T={T}")
    L = host_layer(name, T)
    wl = L.wl
    t = synth.to_torch(L, DEV)
    layer = moe.MoELayer(expert_weights(t), T, wl.top_k, wl.n_shared, t["router"], t.get("bias"))
    x = t["x"]
    eager = sync_np(layer.forward(x)).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x)
    for r in range(3):
        layer.y.fill_(-1.0)                                   # eager work between replays
        other = torch.randn(1 << 20, device=DEV).sum()        # a library reduction on the stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = sync_np(layer.y)
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {r}"
        assert float(other) == float(other)


# ------------------------------------------------------------------------------------------------
# moe_route_bucket (router + bucketing + tile plan in one call) against the separate calls
# ------------------------------------------------------------------------------------------------
RB_CASES = [("tiny", 16), ("decode", 1), ("decode", 8), ("sweep", 1), ("sweep", 5), ("sweep", 8), ("sweep", 9),
            ("sweep", 176), ("sweep", 300), ("prefill", 8), ("prefill", 8192)]


@pytest.mark.parametrize("name,T", RB_CASES, ids=[f"{n}-T{t}" for n, t in RB_CASES])
def test_route_bucket_equals_separate_calls(name, T):
    """Same ids, weights, probabilities, bucket arrays and tile table bit for bit, and the same
    expert-FFN output, from one moe_route_bucket call as from moe_route -> moe_bucket ->
    moe_expert_ffn_plan: through the two-launch path (one selecting and bucketing workgroup) up to
    8 tokens -- sweep T = 8 and 9 sit on either side of the boundary, prefill T = 8 adds a shared
    expert -- and the separate kernels above it."""
    wl = synth.WORKLOADS[name]
    note(f"route_bucket {name} T={T}")
    import dataclasses
    base = host_layer(name, {"sweep": 176, "decode": 8, "tiny": 16, "prefill": 8192}[name])
    L = dataclasses.replace(base, T=T, x=synth.make_x(wl, T))  # the workload's weights, T new tokens
    t = synth.to_torch(L, DEV)
    W = expert_weights(t)
    E, k, S = wl.n_routed, wl.top_k, wl.n_shared
    kt = k + S
    ids_a, w_a, p_a = moe.moe_route(t["x"], t["router"], k, t["bias"], S, want_probs=True)
    b_a = moe.moe_bucket(ids_a, wl.n_experts)
    # zero-filled, so that the padding past the tile table compares equal too
    ws_a = torch.zeros(moe.moe_expert_ffn_workspace_bytes(T, kt, W), dtype=torch.uint8, device=DEV)
    moe.moe_expert_ffn_plan(T, W, b_a.offsets, kt, ws_a)
    ids_b = torch.full_like(ids_a, -7)
    w_b = torch.full_like(w_a, -7.0)
    p_b = torch.full_like(p_a, -7.0)
    b_b = moe.Buckets(*(torch.full_like(v, -7) for v in (b_a.counts, b_a.offsets, b_a.sorted_slot, b_a.slot_pos)))
    ws_b = torch.zeros_like(ws_a)
    for rep in range(2):  # the second call reuses the workspace
        moe.moe_route_bucket(t["x"], t["router"], k, t["bias"], S, ids_b, w_b, b_b, W, ws_b, probs=p_b)
        for a, b in ((ids_a, ids_b), (w_a, w_b), (p_a, p_b), (b_a.counts, b_b.counts), (b_a.offsets, b_b.offsets),
                     (b_a.sorted_slot, b_b.sorted_slot), (b_a.slot_pos, b_b.slot_pos)):
            assert np.array_equal(sync_np(a.view(torch.int32)), sync_np(b.view(torch.int32))), rep
    n_tab = ws_a.numel()
    plane = 2 * ((T * kt * W.inter * 2 + 255) // 256 * 256)
    assert np.array_equal(sync_np(ws_a[plane:]), sync_np(ws_b[plane:]))   # the tile tables
    moe.moe_expert_ffn_gateup(t["x"], W, b_a.offsets, b_a.sorted_slot, kt, ws_b)
    yb = moe.moe_expert_ffn_down(T, W, b_a.offsets, b_a.sorted_slot, kt, ws_b,
                                 torch.empty((T * kt, W.hidden), dtype=torch.float32, device=DEV))
    ya = moe.moe_expert_ffn(t["x"], W, b_a.offsets, b_a.sorted_slot, kt)
    assert np.array_equal(sync_np(ya).view(np.uint32), sync_np(yb).view(np.uint32))
    assert n_tab > plane
