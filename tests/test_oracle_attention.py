"""Pins of the oracle's attention, RoPE and top-k.

* code-domain attention equals decode-then-attend with scipy's softmax;
* query head h reads KV head h // G only;
* RoPE keeps norms, matches the complex-number form, and rotated inner
  products depend only on the position difference ([TurboESM] "2.
  Metodologia", part A);
* top-k equals a brute-force selection with ties to the lower index.
"""

import math

import numpy as np
import pytest
from scipy import special

from oracle import (codebook, encode_prod, encode_mse, decode_prod, decode_mse,
                    attention_from_codes, attention_materialized, rope_interleaved,
                    rotate, top_k, inner_product_matrix)


def _make(B, Hq, Hkv, ctx, nq, d, kbits=3, vbits=3, seed=0):
    rng = np.random.default_rng(seed)
    kc, kt = codebook(d, kbits - 1)
    vc, vt = codebook(d, vbits)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    S = rng.standard_normal((d, d))
    k = rng.standard_normal((B, Hkv, ctx, d)) * 2
    v = rng.standard_normal((B, Hkv, ctx, d))
    q = rng.standard_normal((B, Hq, nq, d))
    kcodes = {"idx": np.zeros((B, Hkv, ctx, d), int), "sign": np.zeros((B, Hkv, ctx, d), np.uint8),
              "norm": np.zeros((B, Hkv, ctx)), "rnorm": np.zeros((B, Hkv, ctx))}
    vcodes = {"idx": np.zeros((B, Hkv, ctx, d), int), "norm": np.zeros((B, Hkv, ctx))}
    for b in range(B):
        for g in range(Hkv):
            e = encode_prod(k[b, g], signs, kc, kt, S)
            kcodes["idx"][b, g], kcodes["sign"][b, g] = e.idx, e.sign
            kcodes["norm"][b, g], kcodes["rnorm"][b, g] = e.norm, e.rnorm
            ev = encode_mse(v[b, g], signs, vt)
            vcodes["idx"][b, g], vcodes["norm"][b, g] = ev.idx, ev.norm
    kbook = {"signs": signs, "centroids": kc, "S": S}
    vbook = {"signs": signs, "centroids": vc}
    return q, kcodes, vcodes, kbook, vbook


@pytest.mark.parametrize("B,Hq,Hkv,ctx,nq,d", [(1, 4, 2, 5, 1, 8), (2, 4, 1, 7, 3, 16), (1, 2, 2, 1, 2, 8)])
def test_code_attention_equals_textbook(B, Hq, Hkv, ctx, nq, d):
    q, kc, vc, kb, vb = _make(B, Hq, Hkv, ctx, nq, d)
    out, scores = attention_from_codes(q, kc, vc, kb, vb, return_scores=True)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kh = decode_prod(kc["idx"][b, g], kc["sign"][b, g], kc["norm"][b, g], kc["rnorm"][b, g],
                             kb["signs"], kb["centroids"], kb["S"])
            vh = decode_mse(vc["idx"][b, g], vc["norm"][b, g], vb["signs"], vb["centroids"])
            s = q[b, h] @ kh.T / math.sqrt(d)
            assert np.allclose(scores[b, h], s, atol=1e-12)
            assert np.allclose(out[b, h], special.softmax(s, axis=-1) @ vh, atol=1e-12)
    assert np.allclose(attention_materialized(q, kc, vc, kb, vb), out, atol=1e-12)


def test_gqa_head_mapping():
    q, kc, vc, kb, vb = _make(1, 8, 2, 6, 1, 8, seed=3)
    base = attention_from_codes(q, kc, vc, kb, vb)
    kc2 = {k: v.copy() for k, v in kc.items()}
    kc2["norm"][0, 1] *= 3.0          # change KV head 1 only
    alt = attention_from_codes(q, kc2, vc, kb, vb)
    assert np.array_equal(alt[0, :4], base[0, :4])
    assert not np.allclose(alt[0, 4:], base[0, 4:])


def test_rope_matches_complex_form_and_is_relative():
    rng = np.random.default_rng(2)
    d = 64
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 100, 1023])
    y = rope_interleaved(x, pos)
    zc = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * 10000.0 ** (-np.arange(d // 2) * 2 / d))
    assert np.allclose(y[:, 0::2], zc.real, atol=1e-12) and np.allclose(y[:, 1::2], zc.imag, atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    ip = lambda i, j: float(rotate(rope_interleaved(q[None], [i]), signs)[0] @
                            rotate(rope_interleaved(k[None], [j]), signs)[0])
    ref = float(rope_interleaved(q[None], [3])[0] @ rope_interleaved(k[None], [10])[0])
    assert ip(3, 10) == pytest.approx(ref, abs=1e-12)       # rotation keeps it
    assert ip(3, 10) == pytest.approx(ip(103, 110), abs=1e-10)   # depends on j - i only
    assert ip(0, 7) == pytest.approx(ip(3, 10), abs=1e-10)


def test_top_k_brute_force_with_ties():
    rng = np.random.default_rng(5)
    s = rng.integers(0, 6, size=(4, 40)).astype(float)   # many ties
    ids, vals = top_k(s, 10)
    for a in range(4):
        pairs = sorted(range(40), key=lambda j: (-s[a, j], j))[:10]
        assert ids[a].tolist() == pairs
        assert vals[a].tolist() == [s[a, j] for j in pairs]


def test_inner_product_matrix_prod_and_mse():
    d = 16
    q, kc, vc, kb, vb = _make(1, 2, 1, 9, 2, d, seed=6)
    codes = {k: v[0, 0] for k, v in kc.items()}
    est = inner_product_matrix(q[0, 0], codes, kb)
    kh = decode_prod(codes["idx"], codes["sign"], codes["norm"], codes["rnorm"], kb["signs"], kb["centroids"], kb["S"])
    assert np.allclose(est, q[0, 0] @ kh.T, atol=1e-12)
