"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random arrays; it holds none of the codec's
arithmetic.  Both the CPU oracle (tests) and the GPU library (tests, bench)
consume exactly these arrays.  The codec's own random draws -- the sign
vector D of the randomized Walsh-Hadamard rotation and the QJL Gaussian
matrix S -- are drawn here as well and passed to both sides as inputs.

Seeding: one numpy SeedSequence(1000 + workload id) per workload, spawned
into independent PCG64 sub-streams (data, codec parameters, queries, ...).
Workloads too large for host generation draw their bulk arrays with a seeded
torch.Generator on the target device; their small parameters (channel
scales, outlier positions) still come from numpy.

Workload ids:
  1 codec unit: 4096 keys + 16 queries, d = 128, fp32
  2 GQA decode: 8 KV heads x 32768 tokens x 128, Student-t(3), fp16
  3 Llama-8B-shaped prefill: 32 layers x 8 heads x 131072 x 128, fp16
  4 ESM-2-shaped bidirectional: 33 layers x 64 batch x 20 heads x 1024 x 64
  5 vector search: 1e6 x 1536 unit vectors from a 64-centre mixture, fp32
"""

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np


def streams(workload, n):
    """n independent PCG64 generators for a workload id."""
    seqs = np.random.SeedSequence(1000 + int(workload)).spawn(n)
    return [np.random.Generator(np.random.PCG64(s)) for s in seqs]


def _torch_seed(rng):
    return int(rng.integers(0, 2**62))


@dataclass
class CodecDraws:
    """Random draws owned by one codec instance."""
    flip: np.ndarray                 # (d,) bool, True where D_i = -1
    S: Optional[np.ndarray] = None   # (m, d) float32, i.i.d. N(0, 1)


def codec_draws(rng, d, m=0):
    flip = rng.random(d) < 0.5
    S = rng.standard_normal((m, d)).astype(np.float32) if m else None
    return CodecDraws(flip=flip, S=S)


# --- workload 1: codec unit test ---------------------------------------

def codec_unit(n_keys=4096, n_queries=16, d=128):
    """Keys: i.i.d. N(0,1) fp32 rows rescaled to norms drawn log-uniform in
    [0.1, 10]; queries: i.i.d. N(0,1) fp32; one D and a d x d Gaussian S."""
    r_keys, r_norm, r_q, r_par = streams(1, 4)
    g = r_keys.standard_normal((n_keys, d)).astype(np.float32).astype(np.float64)
    target = np.exp(r_norm.uniform(math.log(0.1), math.log(10.0), n_keys))
    keys = (g / np.linalg.norm(g, axis=1, keepdims=True) * target[:, None]).astype(np.float32)
    queries = r_q.standard_normal((n_queries, d)).astype(np.float32)
    par = codec_draws(r_par, d, m=d)
    return {"keys": keys, "queries": queries, "codec": par, "norm_target": target}


# --- workload 2: GQA decode step ---------------------------------------

def gqa_decode(hkv=8, ctx=32768, d=128, hq=32, n_outlier=4, outlier_scale=20.0):
    """K and V of one layer, [hkv, ctx, d] fp16: i.i.d. Student-t(3) with, per
    head and per tensor, n_outlier distinct channels scaled by outlier_scale.
    One fp16 N(0,1) query token per query head.  K and V share one D; the
    QJL matrix S (d x d) belongs to K."""
    r_k, r_v, r_ch, r_q, r_par = streams(2, 5)
    out = {}
    for name, r in (("k", r_k), ("v", r_v)):
        x = r.standard_t(3.0, size=(hkv, ctx, d))
        chans = np.stack([r_ch.choice(d, n_outlier, replace=False) for _ in range(hkv)])
        for h in range(hkv):
            x[h, :, chans[h]] *= outlier_scale
        out[name] = x.astype(np.float16)
        out[name + "_channels"] = chans
    out["q"] = r_q.standard_normal((hq, d)).astype(np.float16)
    out["codec"] = codec_draws(r_par, d, m=d)
    return out


# --- workload 3: Llama-3.1-8B-shaped prefill ----------------------------

def llama_prefill_params(layers=32, hkv=8, d=128, ctx=131072, hot_frac=0.01):
    """Small parameters of workload 3: per (layer, head, channel) stds
    log-uniform in [0.05, 5], separately for K and V; per layer a set of
    round(hot_frac * ctx) token positions (shared by K, V and heads) that are
    scaled by 10; per layer a query seed; the codec draws."""
    r_sk, r_sv, r_pos, r_seed, r_par = streams(3, 5)
    lo, hi = math.log(0.05), math.log(5.0)
    std_k = np.exp(r_sk.uniform(lo, hi, (layers, hkv, d)))
    std_v = np.exp(r_sv.uniform(lo, hi, (layers, hkv, d)))
    n_hot = int(round(hot_frac * ctx))
    hot = np.stack([np.sort(r_pos.choice(ctx, n_hot, replace=False)) for _ in range(layers)])
    seeds = np.array([_torch_seed(r_seed) for _ in range(3 * layers)]).reshape(layers, 3)
    return {"std_k": std_k, "std_v": std_v, "hot": hot, "seeds": seeds,
            "codec": codec_draws(r_par, d, m=d), "ctx": ctx, "hkv": hkv, "d": d,
            "hq": 32}


def llama_prefill_layer(params, layer, device="cpu", heads=None, ctx=None):
    """K, V [heads, ctx, d] fp16 and q [32, d] fp16 of one layer, drawn with
    a seeded torch.Generator on `device`.  heads/ctx select a leading slice
    (the slice equals the corresponding part of the full draw)."""
    import torch
    d, full_ctx, hkv = params["d"], params["ctx"], params["hkv"]
    heads = hkv if heads is None else heads
    ctx = full_ctx if ctx is None else ctx
    out = {}
    for t, (name, std) in enumerate((("k", params["std_k"]), ("v", params["std_v"]))):
        g = torch.Generator(device=device)
        g.manual_seed(int(params["seeds"][layer, t]))
        x = torch.empty((hkv, full_ctx, d), dtype=torch.float32, device=device)
        x.normal_(generator=g)
        x = x[:heads, :ctx]
        x *= torch.as_tensor(std[layer, :heads], dtype=torch.float32, device=device)[:, None, :]
        hot = torch.as_tensor(params["hot"][layer], device=device)
        hot = hot[hot < ctx]
        x[:, hot, :] *= 10.0
        out[name] = x.to(torch.float16)
    g = torch.Generator(device=device)
    g.manual_seed(int(params["seeds"][layer, 2]))
    q = torch.empty((params["hq"], d), dtype=torch.float32, device=device)
    q.normal_(generator=g)
    out["q"] = q.to(torch.float16)
    return out


# --- workload 4: ESM-2-650M-shaped bidirectional attention ---------------

def esm2_params(layers=33, batch=64, heads=20, d=64, seq=1024, n_heavy=2,
                heavy_scale=15.0):
    """Per (layer, head) n_heavy distinct heavy channels (scaled by
    heavy_scale, separately chosen for K and V), a torch seed per layer, and
    the codec draws (m = d = 64)."""
    r_ch, r_seed, r_par = streams(4, 3)
    heavy_k = np.stack([[r_ch.choice(d, n_heavy, replace=False) for _ in range(heads)]
                        for _ in range(layers)])
    heavy_v = np.stack([[r_ch.choice(d, n_heavy, replace=False) for _ in range(heads)]
                        for _ in range(layers)])
    seeds = np.array([_torch_seed(r_seed) for _ in range(layers)])
    return {"heavy_k": heavy_k, "heavy_v": heavy_v, "seeds": seeds,
            "heavy_scale": heavy_scale, "codec": codec_draws(r_par, d, m=d),
            "layers": layers, "batch": batch, "heads": heads, "d": d, "seq": seq}


def esm2_layer(params, layer, device="cpu", batch=None):
    """Q, K, V [batch, heads, seq, d] fp16 of one layer (N(0,1); K and V with
    their heavy channels scaled).  `batch` selects a leading slice."""
    import torch
    B, H, S, d = params["batch"], params["heads"], params["seq"], params["d"]
    nb = B if batch is None else batch
    g = torch.Generator(device=device)
    g.manual_seed(int(params["seeds"][layer]))
    out = {}
    for name in ("q", "k", "v"):
        x = torch.empty((B, H, S, d), dtype=torch.float32, device=device)
        x.normal_(generator=g)
        x = x[:nb]
        if name != "q":
            heavy = params["heavy_" + name][layer]
            scale = torch.ones((H, d), dtype=torch.float32, device=device)
            for h in range(H):
                scale[h, torch.as_tensor(heavy[h], device=device)] = params["heavy_scale"]
            x = x * scale[None, :, None, :]
        out[name] = x.to(torch.float16)
    return out


# --- workload 5: vector search ----------------------------------------

def vector_search_params(n=1_000_000, n_q=1024, d=1536, centres=64, sigma=0.3):
    r_c, r_seed, r_par = streams(5, 3)
    mu = r_c.standard_normal((centres, d)).astype(np.float32)
    seeds = [_torch_seed(r_seed) for _ in range(2)]
    return {"mu": mu, "seeds": seeds, "n": n, "n_q": n_q, "d": d, "sigma": sigma,
            "codec": codec_draws(r_par, d, m=d)}


def vector_search_data(params, device="cpu", n=None, n_q=None):
    """Database [n, d] and queries [n_q, d], fp32 unit rows: mu_c + sigma *
    N(0, I) with the centre c uniform, then scaled to unit length.  n / n_q
    select a leading slice of the full draw order (rows are drawn in chunks,
    so a slice equals the leading rows of the full set)."""
    import torch
    n_full, nq_full, d = params["n"], params["n_q"], params["d"]
    n = n_full if n is None else n
    n_q = nq_full if n_q is None else n_q
    mu = torch.as_tensor(params["mu"], device=device)
    out = {}
    for key, rows, seed in (("x", n, params["seeds"][0]), ("q", n_q, params["seeds"][1])):
        g = torch.Generator(device=device)
        g.manual_seed(int(seed))
        chunks = []
        chunk = 65536
        for start in range(0, rows, chunk):
            cnt = min(chunk, rows - start)
            c = torch.randint(0, mu.shape[0], (chunk,), generator=g, device=device)
            e = torch.empty((chunk, d), dtype=torch.float32, device=device)
            e.normal_(generator=g)
            y = (mu[c] + params["sigma"] * e)[:cnt]
            chunks.append(y / torch.linalg.vector_norm(y, dim=1, keepdim=True))
        out[key] = torch.cat(chunks) if chunks else torch.empty((0, d), device=device)
    return out
