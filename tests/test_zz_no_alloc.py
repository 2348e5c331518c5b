"""moe_expert_ffn_static (the entry point that allocates nothing: its workspace is a fixed device
array inside the library) against moe_expert_ffn on the same inputs, through the C ABI (needs an
MI355X).  Both run the same kernels, so the outputs must agree bit for bit: first on the 176-token
sweep batch, then, reusing the array, on a smaller batch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import mxfp4_routed_expert_router_amd as moe
from gpu_support import DEV, expert_weights, host_layer, note, require_gpu

pytestmark = pytest.mark.gpu


def test_static_scratch_matches_workspace_call():
    require_gpu()
    L = host_layer("sweep", 176)
    wl = L.wl
    kt = wl.k_total
    t = synth.to_torch(L, DEV)
    W = expert_weights(t)
    orc = oracle.load()
    for T in (176, 15):  # second call smaller: the array keeps the first call's contents
        note(f"no-alloc ffn: sweep T={T}")
        x = t["x"][:T].contiguous()
        r = orc.route(L.x[:T], oracle.X_BF16, L.router, L.bias, wl.top_k, wl.n_shared)
        b = orc.bucket(r["ids"], wl.n_experts)
        off = torch.from_numpy(b["offsets"]).to(DEV)
        ss = torch.from_numpy(b["sorted_slot"]).to(DEV)
        ref = moe.moe_expert_ffn(x, W, off, ss, kt)
        got = torch.full_like(ref, float("nan"))
        moe.moe_expert_ffn_static(x, W, off, ss, kt, out=got)
        torch.cuda.synchronize()
        a, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.all(np.isfinite(g))
        assert np.array_equal(a.view(np.uint32), g.view(np.uint32))
    # a call whose workspace would exceed the array is refused before anything is launched
    need = moe.moe_expert_ffn_workspace_bytes(300, kt, W)
    assert need > moe.MOE_FFN_STATIC_SCRATCH_BYTES
    xs = torch.empty((300, wl.hidden), dtype=torch.bfloat16, device=DEV)
    st = moe.lib().moe_expert_ffn_static(ctypes.c_void_p(xs.data_ptr()), 0, 300, kt, ctypes.byref(W.c),
                                         ctypes.c_void_p(off.data_ptr()), ctypes.c_void_p(ss.data_ptr()),
                                         ctypes.c_void_p(xs.data_ptr()), None)
    assert st == 7  # MOE_ERR_WORKSPACE
