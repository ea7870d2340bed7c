"""GPU attention-from-codes parity (tq_attend_decode)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_rows, check_scores, gpu_codes, to_np

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_04_amd")


def say(*a):
    print("[case]", *a, flush=True)


def _codes_4d(pk, codec, B, Hkv, ctx):
    g = gpu_codes(pk, codec.d, codec.code_bits, codec.m if codec.mode == tq.TQ_PROD else None)
    return {k: v.reshape((B, Hkv, ctx) + v.shape[1:]) for k, v in g.items()}


def _oracle_attention(q, kpk, vpk, kc, vc, draws, B, Hkv, ctx, q_rope_pos=None, scale=None):
    d = kc.d
    kcent, _ = oracle.codebook(d, kc.code_bits)
    vcent, _ = oracle.codebook(d, vc.code_bits)
    kb = {"signs": draws.flip, "centroids": kcent, "S": draws.S.astype(np.float64)}
    vb = {"signs": draws.flip, "centroids": vcent}
    q64 = q.astype(np.float64)
    if q_rope_pos is not None:
        q64 = oracle.rope_interleaved(q64, q_rope_pos)
    return oracle.attention_from_codes(q64, _codes_4d(kpk, kc, B, Hkv, ctx),
                                       _codes_4d(vpk, vc, B, Hkv, ctx), kb, vb, scale=scale,
                                       return_scores=True)


def _run(B, Hq, Hkv, ctx, nq, d, kbits, vbits, seed, dist="normal"):
    rng = np.random.default_rng(seed)
    if dist == "t":
        k = rng.standard_t(3, (B, Hkv, ctx, d)).astype(np.float16)
        v = rng.standard_t(3, (B, Hkv, ctx, d)).astype(np.float16)
    else:
        k = rng.standard_normal((B, Hkv, ctx, d)).astype(np.float16)
        v = rng.standard_normal((B, Hkv, ctx, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, nq, d)).astype(np.float16)
    draws = synth.codec_draws(rng, d, m=d)
    kc = tq.Codec(d, tq.TQ_PROD, kbits, draws.flip, draws.S)
    vc = tq.Codec(d, tq.TQ_MSE, vbits, draws.flip)
    kpk, vpk = tq.encode_kv(kc, vc, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    out, sc = tq.attend_decode(kc, vc, torch.from_numpy(q).cuda(), kpk, vpk, ctx, Hkv, want_scores=True)
    torch.cuda.synchronize()
    ref_out, ref_sc = _oracle_attention(q, kpk, vpk, kc, vc, draws, B, Hkv, ctx)
    e1 = check_scores(to_np(sc), ref_sc)
    e2 = check_rows(to_np(out), ref_out)
    return e1, e2


def test_attend_gqa_decode_full():
    say("attend gqa-decode: 32 q heads, 8 kv heads, ctx 32768, d 128, K prod b=4, V mse b=4")
    w = synth.gqa_decode()
    kc = tq.Codec(128, tq.TQ_PROD, 4, w["codec"].flip, w["codec"].S)
    vc = tq.Codec(128, tq.TQ_MSE, 4, w["codec"].flip)
    kpk, vpk = tq.encode_kv(kc, vc, torch.from_numpy(w["k"]).cuda(), torch.from_numpy(w["v"]).cuda())
    q = w["q"].reshape(1, 32, 1, 128)
    out, sc = tq.attend_decode(kc, vc, torch.from_numpy(q).cuda(), kpk, vpk, 32768, 8, want_scores=True)
    torch.cuda.synchronize()
    ref_out, ref_sc = _oracle_attention(q, kpk, vpk, kc, vc, w["codec"], 1, 8, 32768)
    print("scores (max row rel err, max elem err)", check_scores(to_np(sc), ref_sc),
          "| out max row rel err", check_rows(to_np(out), ref_out))


@pytest.mark.parametrize("B,Hq,Hkv,ctx,nq,d,kb,vb", [
    (1, 4, 4, 1, 1, 128, 4, 4),
    (1, 8, 2, 257, 1, 128, 3, 3),
    (2, 6, 3, 1000, 3, 128, 4, 4),
    (1, 16, 1, 4099, 2, 128, 3, 4),
    (1, 4, 2, 700, 5, 64, 3, 3),
    (2, 2, 2, 300, 17, 64, 2, 2),
    # 3-bit values with 1- and 3-bit key tables at d = 128: value words
    # loaded four tokens at a time
    (1, 8, 2, 1025, 1, 128, 2, 3),
    (2, 8, 2, 777, 2, 128, 4, 3),
])
def test_attend_shapes(B, Hq, Hkv, ctx, nq, d, kb, vb):
    say("attend B=%d Hq=%d Hkv=%d ctx=%d nq=%d d=%d kb=%d vb=%d" % (B, Hq, Hkv, ctx, nq, d, kb, vb))
    _run(B, Hq, Hkv, ctx, nq, d, kb, vb, seed=ctx + nq + d)


@pytest.mark.parametrize("nq", [1, 9])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kb", [2, 3, 4, 5])
@pytest.mark.parametrize("vb", [1, 2, 3, 4])
def test_attend_every_bit_width_pair(d, kb, vb, nq):
    """Every key width (1..4 table bits + the QJL bit) with every value
    width: each pair is its own kernel instance; two full tiles plus a
    ragged tail.  nq = 1 gives 2 query rows per KV head (the few-row decode
    kernel), nq = 9 gives 18 (the many-query kernels)."""
    say("attend every width d=%d kb=%d vb=%d nq=%d" % (d, kb, vb, nq))
    _run(1, 4, 2, 130, nq, d, kb, vb, seed=1000 + 10 * kb + vb + d + 7 * nq)


@pytest.mark.parametrize("kb", [4, 5])          # three and two code steps in flight per wave
@pytest.mark.parametrize("steps", [3, 4, 5])     # code steps per wave
def test_attend_load_ring_rounds(kb, steps):
    """One KV head spread over every CU, each workgroup's range holding
    8 x `steps` 16-token steps, so that each of its 8 waves runs `steps` of
    them: whole rounds of the load ring with no tail, and tails of one and
    two steps (the context follows the device's CU count)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ctx = cus * 8 * 16 * steps
    say("attend ring rounds: 4 q heads on 1 kv head, ctx %d (%d steps per wave), kb=%d" % (ctx, steps, kb))
    _run(1, 4, 1, ctx, 1, 128, kb, 4, seed=500 + 10 * steps + kb)


@pytest.mark.parametrize("d,nq", [(128, 1), (128, 3), (64, 1), (64, 4)])
def test_attend_query_rope_few_rows(d, nq):
    """RoPE on the queries in the few-row decode kernels (the matrix-core
    kernel at d = 128, the vector-ALU kernel at d = 64): query a of every head
    sits at position pos0 + a, here far enough out that the angle reduction
    matters."""
    B, Hq, Hkv, ctx, pos0 = 1, 8, 2, 1500, 4093
    say("attend query RoPE d=%d nq=%d pos0=%d" % (d, nq, pos0))
    rng = np.random.default_rng(40 + d + nq)
    k = rng.standard_normal((B, Hkv, ctx, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, ctx, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, nq, d)).astype(np.float16)
    draws = synth.codec_draws(rng, d, m=d)
    kc = tq.Codec(d, tq.TQ_PROD, 4, draws.flip, draws.S)
    vc = tq.Codec(d, tq.TQ_MSE, 4, draws.flip)
    kpk, vpk = tq.encode_kv(kc, vc, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    out, sc = tq.attend_decode(kc, vc, torch.from_numpy(q).cuda(), kpk, vpk, ctx, Hkv,
                               rope=(10000.0, pos0), want_scores=True)
    torch.cuda.synchronize()
    ref_out, ref_sc = _oracle_attention(q, kpk, vpk, kc, vc, draws, B, Hkv, ctx,
                                        q_rope_pos=pos0 + np.arange(nq))
    print("scores", check_scores(to_np(sc), ref_sc), "| out", check_rows(to_np(out), ref_out))


@pytest.mark.parametrize("d,nq", [(128, 1), (64, 2), (64, 9), (128, 9)])
def test_attend_fp32_queries_and_scale(d, nq):
    """fp32 queries and an explicit softmax scale in every attention kernel:
    the few-row decode kernels (G nq <= 16; d = 128 on the matrix cores, d = 64
    on the vector ALU) and the many-query kernels at d = 64 and 128."""
    B, Hq, Hkv, ctx, scale = 2, 4, 2, 700, 0.07
    say("attend fp32 q, scale %g: d=%d nq=%d" % (scale, d, nq))
    rng = np.random.default_rng(70 + d + nq)
    k = rng.standard_normal((B, Hkv, ctx, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, ctx, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, nq, d)).astype(np.float32)
    draws = synth.codec_draws(rng, d, m=d)
    kc = tq.Codec(d, tq.TQ_PROD, 3, draws.flip, draws.S)
    vc = tq.Codec(d, tq.TQ_MSE, 3, draws.flip)
    kpk, vpk = tq.encode_kv(kc, vc, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    out, sc = tq.attend_decode(kc, vc, torch.from_numpy(q).cuda(), kpk, vpk, ctx, Hkv, scale=scale,
                               want_scores=True)
    torch.cuda.synchronize()
    ref_out, ref_sc = _oracle_attention(q, kpk, vpk, kc, vc, draws, B, Hkv, ctx, scale=scale)
    print("scores", check_scores(to_np(sc), ref_sc), "| out", check_rows(to_np(out), ref_out))


def test_attend_heavy_tails():
    say("attend Student-t(3) 8x2 heads ctx 5000")
    _run(1, 8, 2, 5000, 1, 128, 4, 4, seed=11, dist="t")


def test_attend_esm2_bidirectional_slice():
    say("attend esm2 layer 0 batch 0: 20 heads, 1024 queries x 1024 keys, d 64, RoPE q and k")
    p = synth.esm2_params()
    lay = synth.esm2_layer(p, 0, device="cuda", batch=1)
    kc = tq.Codec(64, tq.TQ_PROD, 3, p["codec"].flip, p["codec"].S)
    vc = tq.Codec(64, tq.TQ_MSE, 3, p["codec"].flip)
    kpk, vpk = tq.encode_kv(kc, vc, lay["k"], lay["v"], rope=(10000.0, 1024))
    out = tq.attend_decode(kc, vc, lay["q"], kpk, vpk, 1024, 20, rope=(10000.0, 0))
    torch.cuda.synchronize()
    q = to_np(lay["q"])
    ref_out, _ = _oracle_attention(q, kpk, vpk, kc, vc, p["codec"], 1, 20, 1024,
                                   q_rope_pos=np.arange(1024))
    print("out max row rel err", check_rows(to_np(out), ref_out))


def test_attend_llama_decode_slice():
    say("attend llama layer 0: 8 q heads on 2 kv heads, ctx 131072, K prod b=3, V mse b=3")
    p = synth.llama_prefill_params()
    lay = synth.llama_prefill_layer(p, 0, device="cuda", heads=2)
    kc = tq.Codec(128, tq.TQ_PROD, 3, p["codec"].flip, p["codec"].S)
    vc = tq.Codec(128, tq.TQ_MSE, 3, p["codec"].flip)
    kpk, vpk = tq.encode_kv(kc, vc, lay["k"].contiguous(), lay["v"].contiguous())
    q = lay["q"][:8].reshape(1, 8, 1, 128).contiguous()
    out, sc = tq.attend_decode(kc, vc, q, kpk, vpk, 131072, 2, want_scores=True)
    torch.cuda.synchronize()
    ref_out, ref_sc = _oracle_attention(to_np(q), kpk, vpk, kc, vc, p["codec"], 1, 2, 131072)
    print("scores", check_scores(to_np(sc), ref_sc), "out", check_rows(to_np(out), ref_out))
