"""Moments and structure of the seeded synthetic workloads."""

import math

import numpy as np
import pytest
from scipy import stats

import synth


def test_codec_unit_recipe():
    w = synth.codec_unit()
    assert w["keys"].shape == (4096, 128) and w["keys"].dtype == np.float32
    assert w["queries"].shape == (16, 128)
    n = np.linalg.norm(w["keys"].astype(np.float64), axis=1)
    assert np.allclose(n, w["norm_target"], rtol=1e-6)
    ln = np.log(n)
    # log-uniform on [ln 0.1, ln 10]: mean 0, variance (2 ln 10)^2 / 12
    assert abs(ln.mean()) < 4 * (2 * math.log(10) / math.sqrt(12)) / 64
    assert ln.min() >= math.log(0.1) - 1e-6 and ln.max() <= math.log(10) + 1e-6
    assert w["codec"].S.shape == (128, 128) and w["codec"].flip.dtype == bool
    again = synth.codec_unit()
    assert np.array_equal(again["keys"], w["keys"])


def test_gqa_decode_recipe_small():
    w = synth.gqa_decode(hkv=2, ctx=4096)
    k = w["k"].astype(np.float64)
    assert w["k"].dtype == np.float16 and k.shape == (2, 4096, 128)
    for h in range(2):
        ch = w["k_channels"][h]
        assert len(set(ch.tolist())) == 4
        rest = np.setdiff1d(np.arange(128), ch)
        # Student-t(3) quartiles are +-0.7649; outlier channels are x20
        q1, q3 = np.percentile(k[h][:, rest], [25, 75])
        assert q1 == pytest.approx(stats.t.ppf(0.25, 3), abs=0.02)
        assert q3 == pytest.approx(stats.t.ppf(0.75, 3), abs=0.02)
        ratio = np.median(np.abs(k[h][:, ch])) / np.median(np.abs(k[h][:, rest]))
        assert ratio == pytest.approx(20, rel=0.05)
    assert w["q"].shape == (32, 128) and w["q"].dtype == np.float16


def test_llama_prefill_recipe_slice():
    p = synth.llama_prefill_params()
    assert p["hot"].shape == (32, 1311)
    assert len(np.unique(p["hot"][0])) == 1311
    lay = synth.llama_prefill_layer(p, 0, heads=1, ctx=8192)
    k = lay["k"].float().numpy()[0]
    hot = p["hot"][0][p["hot"][0] < 8192]
    cold = np.setdiff1d(np.arange(8192), hot)
    est = k[cold].std(axis=0)
    assert np.allclose(est, p["std_k"][0, 0], rtol=0.08)
    assert k[hot].std() / k[cold].std() == pytest.approx(10, rel=0.1)


def test_esm2_recipe_slice():
    p = synth.esm2_params()
    lay = synth.esm2_layer(p, 0, batch=1)
    k = lay["k"].float().numpy()[0]
    h0 = p["heavy_k"][0, 0]
    assert np.std(k[0][:, h0]) == pytest.approx(15, rel=0.1)
    rest = np.setdiff1d(np.arange(64), h0)
    assert np.std(k[0][:, rest]) == pytest.approx(1, rel=0.05)


def test_vector_search_recipe_slice():
    p = synth.vector_search_params()
    w = synth.vector_search_data(p, n=2000, n_q=8)
    x = w["x"].numpy()
    assert x.shape == (2000, 1536)
    assert np.allclose(np.linalg.norm(x, axis=1), 1, atol=1e-5)
    # points cluster: cosine to their best centre is high
    mu = p["mu"] / np.linalg.norm(p["mu"], axis=1, keepdims=True)
    best = np.max(x @ mu.T, axis=1)
    assert np.median(best) > 0.9


def test_esm2_shape_matches_page_kv_size():
    """[TurboESM] "1. Il Problema": ESM-2 650M at 1024 tokens keeps about
    330 MB of FP32 KV cache; 33 layers x (K, V) x 1024 x (20 heads x 64) x 4 B
    is 330 MiB, the shape of the ESM-2 workload at batch 1."""
    with open(__import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "page_figures.txt")) as f:
        page_mb = [float(l.split()[1]) for l in f if l.startswith("esm2_650m_fp32_kv_1024_mb")][0]
    p = synth.esm2_params()
    nbytes = p["layers"] * 2 * p["seq"] * p["heads"] * p["d"] * 4
    assert nbytes == 346030080
    assert nbytes / 2 ** 20 == pytest.approx(page_mb, rel=1e-3)
