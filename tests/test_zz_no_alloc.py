"""The allocation-free attention entry point (tq_attend_decode_noalloc)
against tq_attend_decode: two calls in a row, the second on a smaller
input, each compared with the workspace call on the same codes (the same
kernels run, so outputs and scores must be identical; the parity bar of
1e-3 per row is checked against the oracle as well), and a request beyond
the fixed scratch rejected before any launch."""

import numpy as np
import pytest
import torch

import kv_cache_vector_04_amd as tq
import oracle
import synth
from parity import check_rows, check_scores, gpu_codes, to_np

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)


def _case(seed, batch, hkv, G, n_q, ctx, kb, vb):
    rng = np.random.default_rng(seed)
    d = 128
    k = rng.standard_t(3, (batch, hkv, ctx, d)).astype(np.float16)
    v = rng.standard_normal((batch, hkv, ctx, d)).astype(np.float16)
    q = rng.standard_normal((batch, hkv * G, n_q, d)).astype(np.float16)
    draws = synth.codec_draws(rng, d, m=d)
    kc = tq.Codec(d, tq.TQ_PROD, kb, draws.flip, draws.S)
    vc = tq.Codec(d, tq.TQ_MSE, vb, draws.flip)
    kp, vp = tq.encode_kv(kc, vc, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    return dict(q=torch.from_numpy(q).cuda(), kc=kc, vc=vc, kp=kp, vp=vp, ctx=ctx, hkv=hkv,
                draws=draws, batch=batch, hq=hkv * G, n_q=n_q)


def _oracle(c):
    d = 128
    B, hkv, ctx = c["batch"], c["hkv"], c["ctx"]

    def codes(pk, codec):
        g = gpu_codes(pk, d, codec.code_bits, codec.m if codec.mode == tq.TQ_PROD else None)
        out = {"idx": g["idx"].reshape(B, hkv, ctx, d), "norm": g["norm"].reshape(B, hkv, ctx)}
        if "sign" in g:
            out["sign"] = g["sign"].reshape(B, hkv, ctx, d)
            out["rnorm"] = g["rnorm"].reshape(B, hkv, ctx)
        return out
    kcent, _ = oracle.codebook(d, c["kc"].code_bits)
    vcent, _ = oracle.codebook(d, c["vc"].code_bits)
    return oracle.attention_from_codes(
        to_np(c["q"]).astype(np.float64), codes(c["kp"], c["kc"]), codes(c["vp"], c["vc"]),
        {"signs": c["draws"].flip, "centroids": kcent, "S": c["draws"].S.astype(np.float64)},
        {"signs": c["draws"].flip, "centroids": vcent}, return_scores=True)


def test_noalloc_matches_workspace_call_twice():
    cases = [("8 KV heads x 4096 tokens, G = 4, K b=4 / V b=4", (5, 1, 8, 4, 1, 4096, 4, 4)),
             ("smaller: 2 KV heads x 777 tokens, G = 2, 2 queries, K b=3 / V b=3",
              (6, 1, 2, 2, 2, 777, 3, 3))]
    for name, args in cases:
        say("noalloc vs workspace call: " + name)
        c = _case(*args)
        shape = (c["batch"], c["hq"], c["n_q"], 128)
        sshape = (c["batch"], c["hq"], c["n_q"], c["ctx"])
        out = torch.full(shape, np.nan, dtype=torch.float32, device="cuda")
        sc = torch.full(sshape, np.nan, dtype=torch.float32, device="cuda")
        tq.attend_decode_noalloc(c["kc"], c["vc"], c["q"], c["kp"], c["vp"], c["ctx"], c["hkv"], out,
                                 scores_out=sc)
        ref, ref_sc = tq.attend_decode(c["kc"], c["vc"], c["q"], c["kp"], c["vp"], c["ctx"], c["hkv"],
                                       want_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(sc, ref_sc)
        o_out, o_sc = _oracle(c)
        print("rows", check_rows(to_np(out), o_out), "scores", check_scores(to_np(sc), o_sc))


def test_noalloc_rejects_requests_beyond_the_scratch():
    say("noalloc: request beyond the fixed scratch")
    batch, n_q, hq, hkv, ctx, d = 8, 16, 64, 8, 65536, 128
    need = tq.attend_workspace_bytes(batch, n_q, hq, hkv, ctx, d)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    rng = np.random.default_rng(1)
    draws = synth.codec_draws(rng, d, m=d)
    kc = tq.Codec(d, tq.TQ_PROD, 4, draws.flip, draws.S)
    vc = tq.Codec(d, tq.TQ_MSE, 4, draws.flip)
    n = batch * hkv * ctx
    kp, vp = tq.Packed(kc, n), tq.Packed(vc, n)
    q = torch.zeros((batch, hq, n_q, d), dtype=torch.float16, device="cuda")
    out = torch.empty((batch, hq, n_q, d), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.attend_decode_noalloc(kc, vc, q, kp, vp, ctx, hkv, out)
    assert e.value.status == tq.TQ_ERR_TOO_LARGE
