"""moe_layer_step_noalloc, the layer step on the library's static device scratch (for callers that cannot
allocate), against moe_layer_step with a caller workspace: two calls in a row, the second with fewer tokens
(the scratch keeps the first call's contents), each bitwise equal to the workspace call, which the parity
tests hold to the oracle."""
import ctypes as C

import numpy as np
import pytest
import torch

import moe_synth as S
import sparse_moe_ffn_topk_amd as moe
from moe_testlib import REL_TOL, row_rel_err, to_device


def test_noalloc_rejects_more_than_its_scratch():
    # checked on the host before any device call: the grouped path's workspace for 512 Flint tokens is 48 MiB
    L = moe.load_library()
    cfg = moe.config_for(S.WORKLOADS["flint"])
    assert L.moe_workspace_bytes(C.byref(cfg), 512) > moe.NOALLOC_SCRATCH_BYTES
    lw = moe.LayerWeights(*([0x10000] * 8 + [0]))
    rc = L.moe_layer_step_noalloc(C.byref(cfg), C.byref(lw), C.c_void_p(0x20000), 512, C.c_void_p(0x30000), None,
                                  None, None)
    assert rc == -3 and "static scratch" in L.moe_last_error().decode()
    assert L.moe_layer_step_noalloc(C.byref(cfg), C.byref(lw), C.c_void_p(0x20000), 0, C.c_void_p(0x30000), None,
                                    None, None) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("name,T1,T2,norm", [("flint", 64, 1, True), ("ling", 9, 3, False), ("lfm25", 40, 8, False),
                                             ("flint", 8, 2, False)])
def test_noalloc_matches_layer_step(gpu, name, T1, T2, norm):
    import dataclasses
    wl = S.WORKLOADS[name]
    if norm:
        wl = dataclasses.replace(wl, norm_eps=1e-5)
    print(f"[case] noalloc {name} T={T1} then T={T2} norm={norm}", flush=True)
    w = to_device(S.make_layer(wl, layer=61))
    cfg = moe.config_for(wl)
    for T in (T1, T2):
        x = S.make_x(wl, tokens=T, layer=61, step=T).cuda()
        k = wl.top_k
        outs = []
        for noalloc in (False, True):
            resid = x.clone() if norm else torch.zeros_like(x)
            ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
            wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
            if noalloc:
                moe.layer_step_noalloc(cfg, w, resid if norm else x, resid, ids, wts)
            else:
                moe.layer_step(cfg, w, resid if norm else x, resid, ids, wts)
            torch.cuda.synchronize()
            outs.append((resid, ids, wts))
        (ra, ia, wa), (rb, ib, wb) = outs
        assert torch.equal(ia, ib) and torch.equal(wa, wb), f"T={T}: routing differs"
        assert torch.equal(ra, rb), f"T={T}: output differs"
        assert row_rel_err(rb.cpu().numpy(), ra.cpu().numpy()).max() <= REL_TOL
