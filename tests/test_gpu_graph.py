"""HIP-graph capture of the library's calls (as bench.py replays them):
every replay, with eager work and synchronizations in between, must write
exactly what the eager calls write."""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_04_amd")


def test_graph_replay_matches_eager():
    print("[case] graph replay: encode K/V + attend, hkv=2 ctx=4096 hq=8", flush=True)
    hkv, ctx, hq, d = 2, 4096, 8, 128
    w = synth.gqa_decode(hkv=hkv, ctx=ctx, hq=hq)
    kc = tq.Codec(d, tq.TQ_PROD, 4, w["codec"].flip, w["codec"].S)
    vc = tq.Codec(d, tq.TQ_MSE, 4, w["codec"].flip)
    k = torch.from_numpy(w["k"]).cuda()
    v = torch.from_numpy(w["v"]).cuda()
    q = torch.from_numpy(w["q"].reshape(1, hq, 1, d)).cuda()
    ws = torch.zeros((tq.attend_workspace_bytes(1, 1, hq, hkv, ctx, d),), dtype=torch.uint8,
                     device="cuda")
    kpk, vpk = tq.encode_kv(kc, vc, k, v)
    ref = tq.attend_decode(kc, vc, q, kpk, vpk, ctx, hkv, workspace=ws).clone()
    refs = [t.clone() for t in (kpk.idx, kpk.qjl, kpk.norm, kpk.rnorm, vpk.idx, vpk.norm)]
    torch.cuda.synchronize()

    out = torch.zeros_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tq.encode_kv(kc, None, k, None, kout=kpk)
        tq.encode_kv(None, vc, None, v, vout=vpk)
        tq.attend_decode(kc, vc, q, kpk, vpk, ctx, hkv, out=out, workspace=ws)
    torch.cuda.synchronize()
    planes = (kpk.idx, kpk.qjl, kpk.norm, kpk.rnorm, vpk.idx, vpk.norm)
    for rep in range(4):
        for t in planes:
            t.zero_()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(planes, refs):
            assert torch.equal(a, b), rep
        assert torch.equal(out, ref), rep
        # eager work between replays
        again = tq.attend_decode(kc, vc, q, kpk, vpk, ctx, hkv, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, ref), rep
