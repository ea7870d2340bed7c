"""The binding rejects mismatched sizes and buffers with ValueError before
any kernel runs: tq_packed carries no row count, so an undersized code plane,
a query of the wrong width or a caller-given output of the wrong shape or
type would otherwise reach the kernels and read or write past an end."""

import numpy as np
import pytest
import torch

import kv_cache_vector_04_amd as tq
import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)


@pytest.fixture(scope="module")
def setup():
    rng = np.random.default_rng(77)
    d, hkv, ctx, hq = 128, 2, 64, 8
    draws = synth.codec_draws(rng, d, m=d)
    kc = tq.Codec(d, tq.TQ_PROD, 4, draws.flip, draws.S)
    vc = tq.Codec(d, tq.TQ_MSE, 4, draws.flip)
    k = torch.from_numpy(rng.standard_normal((hkv * ctx, d)).astype(np.float16)).cuda()
    v = torch.from_numpy(rng.standard_normal((hkv * ctx, d)).astype(np.float16)).cuda()
    kp, vp = tq.encode_kv(kc, vc, k, v)
    q = torch.from_numpy(rng.standard_normal((1, hq, 1, d)).astype(np.float16)).cuda()
    torch.cuda.synchronize()
    return dict(d=d, hkv=hkv, ctx=ctx, hq=hq, kc=kc, vc=vc, k=k, v=v, kp=kp, vp=vp, q=q)


def test_encode_rejects_small_or_mismatched_outputs(setup):
    say("validation: encode_kv outputs")
    s = setup
    n = s["hkv"] * s["ctx"]
    with pytest.raises(ValueError):
        tq.encode_kv(s["kc"], None, s["k"], None, kout=tq.Packed(s["kc"], n - 1))
    with pytest.raises(ValueError):
        tq.encode_kv(None, s["vc"], None, s["v"], vout=tq.Packed(s["kc"], n))   # prod planes for mse
    c3 = tq.Codec(s["d"], tq.TQ_MSE, 3, np.zeros(s["d"], dtype=bool))
    with pytest.raises(ValueError):
        tq.encode_kv(None, s["vc"], None, s["v"], vout=tq.Packed(c3, n))      # 3-bit rows for 4-bit
    with pytest.raises(ValueError):
        tq.encode_kv(s["kc"], None, s["k"][:, :64].contiguous(), None)


def test_attend_rejects_bad_sizes(setup):
    say("validation: attend_decode")
    s = setup
    a = (s["kc"], s["vc"])
    with pytest.raises(ValueError):   # more tokens than the planes hold
        tq.attend_decode(*a, s["q"], s["kp"], s["vp"], s["ctx"] + 1, s["hkv"])
    with pytest.raises(ValueError):   # query width
        tq.attend_decode(*a, s["q"][..., :64].contiguous(), s["kp"], s["vp"], s["ctx"], s["hkv"])
    with pytest.raises(ValueError):   # hq not a multiple of hkv
        tq.attend_decode(*a, s["q"], s["kp"], s["vp"], s["ctx"] // 2, 3)
    with pytest.raises(ValueError):   # output of the wrong type / shape / device
        tq.attend_decode(*a, s["q"], s["kp"], s["vp"], s["ctx"], s["hkv"],
                         out=torch.empty((1, s["hq"], 1, s["d"]), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        tq.attend_decode(*a, s["q"], s["kp"], s["vp"], s["ctx"], s["hkv"],
                         out=torch.empty((1, s["hq"], 1, s["d"]), dtype=torch.float32))
    with pytest.raises(ValueError):   # keys and values swapped
        tq.attend_decode(*a, s["q"], s["vp"], s["kp"], s["ctx"], s["hkv"])
    with pytest.raises(ValueError):   # workspace too small
        tq.attend_decode(*a, s["q"], s["kp"], s["vp"], s["ctx"], s["hkv"],
                         workspace=torch.empty((16,), dtype=torch.uint8, device="cuda"))


def test_decode_and_scan_reject_short_planes(setup):
    say("validation: decode_kv and inner_product")
    s = setup
    n = s["hkv"] * s["ctx"]
    with pytest.raises(ValueError):
        tq.decode_kv(s["kc"], s["kp"], n + 1)
    with pytest.raises(ValueError):
        tq.inner_product(s["kc"], s["q"].reshape(-1, s["d"]).float(), s["kp"], n + 1)
    with pytest.raises(ValueError):
        tq.inner_product(s["kc"], s["q"].reshape(-1, s["d"])[:, :64].float().contiguous(), s["kp"], n)


def test_split_attention_rejects_scores_buffer(setup):
    say("validation: attend_split scores_out")
    rng = np.random.default_rng(3)
    flip = np.zeros(64, dtype=bool)
    S = rng.standard_normal((64, 64)).astype(np.float32)
    kc = tq.SplitCodec(tq.Codec(64, tq.TQ_PROD, 4, flip, S), tq.Codec(64, tq.TQ_PROD, 3, flip, S))
    vc = tq.SplitCodec(tq.Codec(64, tq.TQ_MSE, 4, flip), tq.Codec(64, tq.TQ_MSE, 3, flip))
    ctx, hkv, hq = 32, 1, 4
    x = torch.from_numpy(rng.standard_normal((hkv * ctx, 128)).astype(np.float16)).cuda()
    kp, vp = tq.encode_split(kc, vc, x, x)
    q = torch.from_numpy(rng.standard_normal((1, hq, 1, 128)).astype(np.float16)).cuda()
    with pytest.raises(ValueError):
        tq.attend_split(kc, vc, q, kp, vp, ctx, hkv, scores_out=torch.empty((1, hq, 1, ctx)))
    with pytest.raises(ValueError):
        tq.attend_split(kc, vc, q, kp, vp, ctx, hkv,
                        scores_out=torch.empty((1, hq, 1, ctx - 1), device="cuda"))
    with pytest.raises(ValueError):
        tq.attend_split(kc, vc, q, kp, vp, ctx + 1, hkv)
    out = tq.attend_split(kc, vc, q, kp, vp, ctx, hkv,
                          scores_out=torch.empty((1, hq, 1, ctx), device="cuda"))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_empty_batches_are_no_ops(setup):
    """Zero rows: encode and decode return empty results without a launch,
    and leave the existing codes untouched."""
    say("validation: zero-row encode / decode")
    s = setup
    d = s["d"]
    before = s["kp"].idx.clone()
    k0 = torch.empty((0, d), dtype=torch.float16, device="cuda")
    kp, vp = tq.encode_kv(s["kc"], s["vc"], k0, k0.clone())
    assert kp.n == 0 and vp.n == 0 and kp.idx.shape == (0, d * 3 // 8)
    assert tq.decode_kv(s["kc"], kp, 0).shape == (0, d)
    assert tq.decode_kv(s["vc"], s["vp"], 0, dtype=torch.float32).shape == (0, d)
    torch.cuda.synchronize()
    assert torch.equal(before, s["kp"].idx)
