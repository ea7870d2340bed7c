"""Benchmark of the TurboQuant KV-cache codec hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input of
the single-layer GQA decode workload: 8 KV heads x 32768 tokens x d 128,
fp16 Student-t(3) K and V with 4 outlier channels per head scaled x20;
keys encoded TurboQuant_prod at 4 bits (3-bit table + 1-bit QJL, 128 x 128
Gaussian S), values TurboQuant_mse at 4 bits; then one decode step of 32
query heads attending over all 32768 tokens straight from the packed codes.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Inputs are resident in HBM before the timed region.  Eight input sets and
eight code sets rotate so that each encode reads its input from HBM and each
attention step reads codes written four steps earlier (more than the 256 MB
Infinity Cache has passed through since), not from the cache.

Each step is replayed from a HIP graph captured once per buffer set, so
that host launch overhead stays out of the timed loop.  Prints one JSON
line.  `value` is KV vectors encoded per second over whole steps (encode +
attention).  The per-kernel rates come from HIP events on the replay stream
around graphs holding one launch per buffer set; `roofline` describes the
kernel with the largest share of the step.  `cpu_baseline` times the fp64 CPU
oracle on a bounded sample of the same workload on this host.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "kv_cache_vector_04_amd", "csrc")
# rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the bench's kernels: its
# "per-launch:" lines give HBM bytes per launch (already scaled by the copy
# kernel calibration) and the hash of each kernel source they were taken on.
TRAFFIC_FILE = os.path.join(HERE, "profiles", "gqa_decode_step_hbm_traffic.md")


def source_hash(name):
    import hashlib
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(part):
    """HBM bytes per launch of `part` ("encode" or "attend") as the committed
    counter summary records them, or None when that summary was taken on
    other kernel sources than the ones built here (the kernel has changed
    since the counters were taken) or has no such line."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        f = line.split()
        if len(f) >= 4 and f[0] == "per-launch:" and f[1] == part:
            for src in f[3:]:
                name, _, h = src.partition("@")
                if not os.path.exists(os.path.join(CSRC, name)) or source_hash(name) != h:
                    return None
            return int(f[2])
    return None


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=10):
    """Device-to-device copy of a 1 GiB buffer (torch's copy kernel), timed
    with HIP events on the current stream: read + write bytes per second.
    Context for the HBM-bound kernels (the practical ceiling of a plain
    stream), not a peak."""
    a = torch.ones((nbytes // 4,), dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    return 2.0 * nbytes / dt / 1e9


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200 for gqa_decode, 3 for the others)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 20 for gqa_decode, 1 for the others)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=8)
    ap.add_argument("--workload", default="gqa_decode",
                    choices=("gqa_decode", "llama_prefill", "esm2", "vector_search", "fibquant",
                             "split"),
                    help="gqa_decode (the default bench line); llama_prefill (32 layers x 8 KV "
                         "heads x 131072 tokens, 3-bit, encode + one decode step per layer); "
                         "esm2 (33 layers x 64 x 20 heads x 1024 tokens, d64, RoPE keys, 3-bit, "
                         "encode + bidirectional attention); vector_search (1e6 x d1536 encode "
                         "+ 1024-query scan with top-10); fibquant (the GQA K/V, 2 x 262144 "
                         "rows d128, through the k = 2 vector code at N = 32, 2.5 bits, "
                         "encode + decode, with a sweep over N); split (the GQA step with "
                         "outlier-channel split codecs, 3/2 bits = 2.5 and 4/3 = 3.5, attention "
                         "through the materializing decoder)")
    a = ap.parse_args()
    heavy = a.workload != "gqa_decode"
    if a.steps is None:
        a.steps = 3 if heavy else 200
    if a.warmup is None:
        a.warmup = 1 if heavy else 20
    return a


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the codec shards by KV head or token range with no collective; "
              "see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import kv_cache_vector_04_amd as tq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.workload == "vector_search":
        return bench_search(a, torch, synth, tq, dev)
    if a.workload == "fibquant":
        return bench_fibquant(a, torch, synth, tq, dev)
    if a.workload == "split":
        return bench_split(a, torch, synth, tq, dev)
    if a.workload in ("llama_prefill", "esm2"):
        return bench_layers(a, torch, synth, tq, dev)
    hkv, ctx, d, hq = 8, 32768, 128, 32
    w = synth.gqa_decode(hkv=hkv, ctx=ctx, d=d, hq=hq)
    kc = tq.Codec(d, tq.TQ_PROD, 4, w["codec"].flip, w["codec"].S)
    vc = tq.Codec(d, tq.TQ_MSE, 4, w["codec"].flip)
    k0 = torch.from_numpy(w["k"]).to(dev)
    v0 = torch.from_numpy(w["v"]).to(dev)
    q = torch.from_numpy(w["q"].reshape(1, hq, 1, d)).to(dev)
    n = hkv * ctx
    S = a.sets
    ks = [k0.clone() for _ in range(S)]
    vs = [v0.clone() for _ in range(S)]
    kpk = [tq.Packed(kc, n, dev) for _ in range(S)]
    vpk = [tq.Packed(vc, n, dev) for _ in range(S)]
    out = torch.empty((1, hq, 1, d), dtype=torch.float32, device=dev)
    ws = torch.zeros((tq.attend_workspace_bytes(1, 1, hq, hkv, ctx, d),), dtype=torch.uint8, device=dev)
    del k0, v0

    # fill every code set once so that any attention step reads valid codes
    for i in range(S):
        tq.encode_kv(kc, vc, ks[i], vs[i], kout=kpk[i], vout=vpk[i])
    torch.cuda.synchronize()

    def enc(j):
        # keys and values in one call: one launch of the fused encoder
        tq.encode_kv(kc, vc, ks[j], vs[j], kout=kpk[j], vout=vpk[j])

    def enc_k(j):
        tq.encode_kv(kc, None, ks[j], None, kout=kpk[j])

    def enc_v(j):
        tq.encode_kv(None, vc, None, vs[j], vout=vpk[j])

    def attend(j):
        r = (j + S // 2) % S
        tq.attend_decode(kc, vc, q, kpk[r], vpk[r], ctx, hkv, out=out, workspace=ws)

    def step(j):
        enc(j)
        attend(j)

    # Two-pass baseline (context only, not part of the step): decode the same
    # codes to vectors with tq_decode_kv (K in fp32, so that the scores keep
    # fp32 accuracy; V in fp16), then plain softmax attention with torch
    # matmuls on the materialized vectors (right operands contiguous).
    G = hq // hkv
    khat = torch.empty((hkv, ctx, d), dtype=torch.float32, device=dev)
    vhat = torch.empty((hkv, ctx, d), dtype=torch.float16, device=dev)
    qt = q.reshape(hkv, G, d).float().transpose(1, 2).contiguous()             # [hkv, d, G]
    out2 = torch.empty((hkv, G, d), dtype=torch.float32, device=dev)

    def dec_k(j):
        tq.decode_kv(kc, kpk[(j + S // 2) % S], n, out=khat.view(n, d))

    def dec_v(j):
        tq.decode_kv(vc, vpk[(j + S // 2) % S], n, out=vhat.view(n, d))

    def two_pass(j):
        dec_k(j)
        dec_v(j)
        s_ = torch.matmul(khat, qt) * (1.0 / d ** 0.5)                          # [hkv, ctx, G] fp32
        p_ = torch.softmax(s_, dim=1).to(torch.float16).transpose(1, 2).contiguous()
        out2.copy_(torch.matmul(p_, vhat))

    for i in range(a.warmup):
        step(i % S)
    torch.cuda.synchronize()

    # One HIP graph per step (one per buffer set) takes the Python launch
    # overhead out of the timed loop; the library's launches are captured on
    # the capture stream like any other work.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    g_step = [capture(lambda j=j: step(j)) for j in range(S)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        g_step[i % S].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Per-kernel durations: HIP events on the capture-and-replay stream around
    # graphs that hold one launch per buffer set, replayed back to back.
    reps = max(2, a.steps // S)
    t_part = {}

    def time_parts(parts):
        graphs = {name: capture(lambda fn=fn: [fn(j) for j in range(S)]) for name, fn in parts}
        for name, g in graphs.items():
            g.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            t_part[name] = e0.elapsed_time(e1) * 1e-3 / (reps * S)     # seconds per launch

    time_parts((("encode", enc), ("encode_k", enc_k), ("encode_v", enc_v), ("attend", attend)))
    # the baseline last, so that its buffers and library set-up do not touch
    # the parts above; the matmul library sets itself up outside the capture
    two_pass(0)
    torch.cuda.synchronize()
    time_parts((("two_pass", two_pass), ("decode_k", dec_k), ("decode_v", dec_v)))

    ms_per_step = wall / a.steps * 1e3
    vectors = 2 * n

    # algorithmic bytes (see the design notes): per key 256 in + 72 out,
    # per value 256 in + 68 out; attention reads 140 B per token per KV head
    kbytes = n * (d * 2 + d * 3 // 8 + d // 8 + 8)
    vbytes = n * (d * 2 + d * 4 // 8 + 4)
    abytes = n * ((d * 3 // 8 + d // 8 + 8) + (d * 4 // 8 + 4))
    te, tk, tv, ta = t_part["encode"], t_part["encode_k"], t_part["encode_v"], t_part["attend"]
    t2 = t_part["two_pass"]
    # the last replay of the two-pass graph used buffer set S - 1: compare
    # with the fused attention over the same codes
    attend(S - 1)
    torch.cuda.synchronize()
    ref = out.reshape(hkv, G, d)
    diff = float(((out2 - ref).norm(dim=-1) / ref.norm(dim=-1).clamp_min(1e-30)).max())
    # decoder bytes per vector: packed codes in, d fp32 (K) or fp16 (V) out
    dkb = n * ((d * 3 // 8 + d // 8 + 8) + 4 * d)
    dvb = n * ((d * 4 // 8 + 4) + 2 * d)
    tdk, tdv = t_part["decode_k"], t_part["decode_v"]
    two = {"us": t2 * 1e6, "fused_speedup": t2 / ta, "max_row_rel_diff_vs_fused": diff,
           "decode_k": {"us": tdk * 1e6, "GB_per_s": dkb / tdk / 1e9,
                        "frac_of_hbm_peak": dkb / tdk / 1e9 / HBM_PEAK_GBS},
           "decode_v": {"us": tdv * 1e6, "GB_per_s": dvb / tdv / 1e9,
                        "frac_of_hbm_peak": dvb / tdv / 1e9 / HBM_PEAK_GBS},
           "note": "context, not in the step: tq_decode_kv of K (fp32) and V (fp16), then plain "
                   "softmax attention (torch matmuls, fp32 scores) on the materialized vectors"}
    enc = {"us": te * 1e6,
           "vectors_per_s": vectors / te,
           "GB_per_s": (kbytes + vbytes) / te / 1e9,
           "frac_of_hbm_peak": (kbytes + vbytes) / te / 1e9 / HBM_PEAK_GBS,
           "note": "one tq_encode_kv call with both codecs: one launch encodes keys and values",
           "us_k_alone": tk * 1e6, "us_v_alone": tv * 1e6}
    att = {"us": ta * 1e6, "GB_per_s": abytes / ta / 1e9,
           "frac_of_hbm_peak": abytes / ta / 1e9 / HBM_PEAK_GBS,
           "note": "one tq_attend_decode call: decode kernel + log-sum-exp merge kernel"}
    parts = {"encode": (te, kbytes + vbytes), "attend": (ta, abytes)}
    dom = max(parts, key=lambda p: parts[p][0])
    t_dom, b_dom = parts[dom]
    roof = {"kernel": {"encode": "encode_kv_half_kernel<128,3,4> (keys prod + values mse, fp16)",
                       "attend": "decode_mfma_kernel<3,4,8> + merge_kernel<128>"}[dom],
            "bound": "hbm", "achieved": b_dom / t_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": b_dom / t_dom / 1e9 / HBM_PEAK_GBS, "traffic": counter_traffic(dom)}

    res = {
        "metric": "KV vectors encoded/s and decode-attention GB/s over packed codes (% of HBM peak)",
        "value": vectors / (wall / a.steps), "unit": "vectors/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gqa-decode: 1 layer, 8 KV heads x 32768 tokens x d128 fp16 "
                               "Student-t(3) + 4 outlier channels x20; K prod b=4 (3+1 QJL, "
                               "128x128 S), V mse b=4; 32 query heads, 1 query token",
                   "vectors_per_step": vectors, "code_bytes_read_per_step": abytes,
                   "rotating_sets": S},
        "encode": enc, "attend": att, "two_pass_attention": two, "roofline": roof,
        "context": {"hbm_copy_GB_per_s": copy_bandwidth(torch, dev),
                    "note": "1 GiB device-to-device copy on this GPU (read + write bytes), "
                            "the practical ceiling of a plain stream; peak stays 8 TB/s"},
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"], orc = cpu_baseline(w)
        # agreement of this run's codes (buffer set 0) with the oracle's
        # encode of the same input, taken in the same run
        res["parity"] = oracle_agreement(w, orc, kpk[0], vpk[0], kc, vc)
    print(json.dumps(res), flush=True)


def bench_layers(a, torch, synth, tq, dev):
    """Many-layer workloads, all layers resident in HBM; a step is every
    layer's encode of K and V plus its attention from the fresh codes.

    llama_prefill: 32 layers x 8 KV heads x 131072 tokens x d128 fp16
      (per-channel stds log-uniform in [0.05, 5], 1% of tokens x10); K prod
      b=3 (2-bit table + 1-bit QJL), V mse b=3; one decode step of 32 query
      heads per layer over all 131072 tokens.
    esm2: 33 layers x batch 64 x 20 heads x 1024 tokens x d64 fp16 (2 heavy
      channels per head x15); RoPE (base 10000) on K before the rotation and
      on the queries; K prod b=3, V mse b=3; bidirectional attention of all
      1024 queries of every head over its 1024 keys."""
    if a.workload == "llama_prefill":
        P = synth.llama_prefill_params()
        L, hkv, d, ctx, hq = 32, P["hkv"], P["d"], P["ctx"], P["hq"]
        layers = [synth.llama_prefill_layer(P, l, device=dev) for l in range(L)]
        batch, n_q, heads, rope_k, rope_q = 1, 1, hkv, None, None
        qs = [x["q"].reshape(1, hq, 1, d) for x in layers]
        desc = ("llama-prefill: 32 layers x 8 KV heads x 131072 tokens x d128 fp16 (channel stds "
                "log-uniform [0.05,5], 1% hot tokens x10); K prod b=3 (2+1 QJL), V mse b=3; one "
                "decode step of 32 query heads per layer")
    else:
        P = synth.esm2_params()
        L, batch, heads, ctx, d = P["layers"], P["batch"], P["heads"], P["seq"], P["d"]
        layers = [synth.esm2_layer(P, l, device=dev) for l in range(L)]
        hkv, hq, n_q = heads, heads, ctx
        rope_k, rope_q = (10000.0, ctx), (10000.0, 0)
        qs = [x["q"] for x in layers]
        desc = ("esm2: 33 layers x 64 sequences x 20 heads x 1024 tokens x d64 fp16 (2 heavy "
                "channels per head x15); RoPE base 10000 on K and q; K prod b=3 (2+1 QJL), "
                "V mse b=3; bidirectional attention, 1024 x 1024 scores per head")
    n = batch * heads * ctx                     # vectors per tensor per layer
    kc = tq.Codec(d, tq.TQ_PROD, 3, P["codec"].flip, P["codec"].S)
    vc = tq.Codec(d, tq.TQ_MSE, 3, P["codec"].flip)
    kpk = [tq.Packed(kc, n, dev) for _ in range(L)]
    vpk = [tq.Packed(vc, n, dev) for _ in range(L)]
    outs = [torch.empty((batch, hq, n_q, d), dtype=torch.float32, device=dev) for _ in range(L)]
    ws = torch.zeros((tq.attend_workspace_bytes(batch, n_q, hq, hkv, ctx, d),), dtype=torch.uint8,
                     device=dev)

    def enc(l):
        # one call with both codecs: a single launch where the inputs allow it
        # (fp16 without RoPE: the Llama-shaped layers), else one per tensor
        tq.encode_kv(kc, vc, layers[l]["k"], layers[l]["v"], rope=rope_k, kout=kpk[l], vout=vpk[l])

    def attend(l):
        tq.attend_decode(kc, vc, qs[l], kpk[l], vpk[l], ctx, hkv, rope=rope_q, out=outs[l],
                         workspace=ws)

    for _ in range(a.warmup):
        for l in range(L):
            enc(l)
            attend(l)
    torch.cuda.synchronize()
    t = {"encode": [], "attend": []}
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for name, fn in (("encode", enc), ("attend", attend)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(L):
                fn(l)
            e1.record()
            torch.cuda.synchronize()
            t[name].append(e0.elapsed_time(e1) * 1e-3 / L)      # seconds per layer
    wall = time.perf_counter() - t0
    te, ta = (float(np.median(t[x])) for x in ("encode", "attend"))
    # algorithmic bytes per layer: fp16 in + packed out (encode), packed codes read (attention)
    kout = d * 2 // 8 + d // 8 + 8
    vout = d * 3 // 8 + 4
    kbytes, vbytes, abytes = n * (2 * d + kout), n * (2 * d + vout), n * (kout + vout)
    parts = {"encode": (te, kbytes + vbytes), "attend": (ta, abytes)}
    dom = max(parts, key=lambda x: parts[x][0])
    kname = {"encode": "encode_kv_half_kernel<128,2,3> (keys prod + values mse, one launch)"
                       if a.workload == "llama_prefill" else
                       "encode_kernel<64,2,prod,RoPE> + encode_half_kernel<64,3,mse>",
             "attend": "decode_mfma_kernel<2,3,8> + merge_kernel<128>"
                       if a.workload == "llama_prefill" else "attend_mq_kernel<2,3>"}[dom]
    roof = {"kernel": kname, "bound": "hbm", "achieved": parts[dom][1] / parts[dom][0] / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": parts[dom][1] / parts[dom][0] / 1e9 / HBM_PEAK_GBS, "traffic": None}
    if a.workload == "esm2" and dom == "attend":
        # every query meets every key: a matrix-core product, 6 d algorithmic
        # flops per (query, key) pair (<q, c>, <Sq, +-1>, the weighted value sum)
        flops = 6.0 * d * batch * heads * ctx * ctx
        roof = {"kernel": "attend_mq_kernel<2,3>", "bound": "mfma",
                "achieved": flops / ta / 1e12, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": flops / ta / 1e12 / MFMA_F16_PEAK_TFLOPS, "traffic": None}
    res = {
        "metric": "KV vectors encoded/s and decode-attention GB/s over packed codes (% of HBM peak)",
        "value": 2 * n * L / (wall / a.steps), "unit": "vectors/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": wall / a.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": {"workload": desc, "layers": L, "vectors_per_step": 2 * n * L},
        "encode": {"us_per_layer": te * 1e6, "vectors_per_s": 2 * n / te,
                   "frac_of_hbm_peak": (kbytes + vbytes) / te / 1e9 / HBM_PEAK_GBS,
                   "note": "one tq_encode_kv call with both codecs per layer"},
        "attend": {"us_per_layer": ta * 1e6, "GB_per_s": abytes / ta / 1e9,
                   "frac_of_hbm_peak": abytes / ta / 1e9 / HBM_PEAK_GBS},
        "roofline": roof,
    }
    if a.workload == "esm2":
        pairs = batch * heads * ctx * ctx
        res["attend"]["qk_pairs_per_s"] = pairs / ta
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_layers(a.workload, P, layers[0], d, ctx, heads)
    print(json.dumps(res), flush=True)


def cpu_baseline_layers(workload, P, lay, d, ctx, heads):
    """The fp64 numpy oracle on a bounded sample of a many-layer workload,
    timed on this host with the BLAS pool at every core of this process:
    llama_prefill: layer 0, KV heads 0-1 over all 131072 tokens (encode of
    their keys and values, then the decode step of their 8 query heads);
    esm2: layer 0, sequence 0 (RoPE and encode of the 20 heads' 1024 keys and
    values, then all 1024 x 1024 scores and outputs of every head).  Rates
    use the GPU's byte accounting."""
    import oracle
    from threadpoolctl import threadpool_limits
    cb = 2
    kc, kt = oracle.codebook(d, cb)
    vc, vt = oracle.codebook(d, 3)
    S = P["codec"].S.astype(np.float64)
    flip = P["codec"].flip
    if workload == "llama_prefill":
        nh, nq = 2, 1
        k = lay["k"][:nh].cpu().numpy().astype(np.float64)           # [2, ctx, d]
        v = lay["v"][:nh].cpu().numpy().astype(np.float64)
        q = lay["q"][:4 * nh].cpu().numpy().astype(np.float64).reshape(1, 4 * nh, 1, d)
        sample = ("layer 0, KV heads 0-1 x 131072 tokens: encode of 262144 keys + 262144 values, "
                  "then the decode step of their 8 query heads (fp64 numpy)")
    else:
        nh, nq = heads, ctx
        k = lay["k"][0].cpu().numpy().astype(np.float64)              # [20, 1024, 64]
        v = lay["v"][0].cpu().numpy().astype(np.float64)
        q = lay["q"][:1].cpu().numpy().astype(np.float64)             # [1, 20, 1024, 64]
        sample = ("layer 0, sequence 0: RoPE + encode of 20 x 1024 keys and values, then the "
                  "bidirectional attention of the 20 heads (1024 x 1024 scores each; fp64 numpy)")
    cores = _cores()
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        if workload == "esm2":
            pos = np.arange(ctx)
            k = oracle.rope_interleaved(k, pos)
            q = oracle.rope_interleaved(q, pos)
        ek = oracle.encode_prod(k.reshape(-1, d), flip, kc, kt, S, keep_z=False)
        ev = oracle.encode_mse(v.reshape(-1, d), flip, vt, keep_z=False)
        kcodes = {"idx": ek.idx.reshape(1, nh, ctx, d), "sign": ek.sign.reshape(1, nh, ctx, d),
                  "norm": ek.norm.reshape(1, nh, ctx), "rnorm": ek.rnorm.reshape(1, nh, ctx)}
        vcodes = {"idx": ev.idx.reshape(1, nh, ctx, d), "norm": ev.norm.reshape(1, nh, ctx)}
        oracle.attention_from_codes(q, kcodes, vcodes, {"signs": flip, "centroids": kc, "S": S},
                                    {"signs": flip, "centroids": vc})
        dt = time.perf_counter() - t0
    n = nh * ctx
    kout, vout = d * cb // 8 + d // 8 + 8, d * 3 // 8 + 4
    nbytes = n * (2 * d + kout) + n * (2 * d + vout) + n * (kout + vout)
    return {"value": 2 * n / dt, "unit": "vectors/s", "cores": int(cores), "kind": "oracle",
            "seconds": dt, "GB_per_s": nbytes / dt / 1e9, "sample": sample}


MFMA_F16_PEAK_TFLOPS = 2500.0


def bench_search(a, torch, synth, tq, dev):
    """Vector search: encode 1,000,000 unit vectors (d 1536, Gaussian mixture
    of 64 centres, sigma 0.3) with TurboQuant_prod at 2 bits (1-bit table +
    1536 QJL bits), then score 1024 fp32 queries against all rows from the
    codes and keep the top 10.  A step is encode + scan + top-10; the parts
    are timed with HIP events on the launch stream."""
    p = synth.vector_search_params()
    data = synth.vector_search_data(p, device=dev)
    n, nq, d = p["n"], p["n_q"], p["d"]
    codec = tq.Codec(d, tq.TQ_PROD, 2, p["codec"].flip, p["codec"].S)
    pk = tq.Packed(codec, n, dev)
    ew = torch.empty((tq.encode_workspace_bytes(codec, None, n),), dtype=torch.uint8, device=dev)
    sw = torch.empty((tq.inner_product_workspace_bytes(nq, n, d, 10),), dtype=torch.uint8, device=dev)
    ids = torch.empty((nq, 10), dtype=torch.int64, device=dev)
    vals = torch.empty((nq, 10), dtype=torch.float32, device=dev)

    def encode():
        tq.encode_kv(codec, None, data["x"], None, kout=pk, workspace=ew)

    def scan():
        tq.inner_product(codec, data["q"], pk, n, top_k=10, want_matrix=False, workspace=sw,
                         out_ids=ids, out_vals=vals)

    for _ in range(max(1, a.warmup)):
        encode()
        scan()
    torch.cuda.synchronize()
    t_enc, t_scan = [], []
    t0 = time.perf_counter()
    for _ in range(a.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        encode()
        e[1].record()
        scan()
        e[2].record()
        torch.cuda.synchronize()
        t_enc.append(e[0].elapsed_time(e[1]) * 1e-3)
        t_scan.append(e[1].elapsed_time(e[2]) * 1e-3)
    wall = time.perf_counter() - t0
    te, ts = float(np.median(t_enc)), float(np.median(t_scan))
    # algorithmic work: per vector 2 m d flops of S r (m = d) and 4 B d in +
    # 392 B out; per (query, row) pair 4 d flops (two d-long products) and
    # 392 B of codes per row once per query block of 32
    enc_flops = 2.0 * d * d * n
    enc_bytes = n * (4 * d + d // 8 + d // 8 + 8)
    scan_flops = 4.0 * d * n * nq
    enc = {"ms": te * 1e3, "vectors_per_s": n / te, "GB_per_s": enc_bytes / te / 1e9,
           "TFLOP_per_s": enc_flops / te / 1e12}
    sc = {"ms": ts * 1e3, "pairs_per_s": n * nq / ts, "TFLOP_per_s": scan_flops / ts / 1e12,
          "note": "query prep + MFMA scan + two-pass top-10"}
    dom_t, dom_f, dom = (ts, scan_flops, "wide_scan_kernel<1,prod> + top-10") if ts >= te else \
        (te, enc_flops, "wide_transform_kernel + wide_proj_kernel<signs>")
    roof = {"kernel": dom, "bound": "mfma", "achieved": dom_f / dom_t / 1e12,
            "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": dom_f / dom_t / 1e12 / MFMA_F16_PEAK_TFLOPS, "traffic": None}
    res = {
        "metric": "KV vectors encoded/s and decode-attention GB/s over packed codes (% of HBM peak)",
        "value": n / (wall / a.steps), "unit": "vectors/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": wall / a.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "vector-search: 1e6 x d1536 fp32 unit rows (64-centre Gaussian "
                               "mixture, sigma 0.3), prod b=2 (1-bit table + 1536 QJL bits); "
                               "1024 fp32 queries, top-10",
                   "vectors_per_step": n, "queries": nq},
        "encode": enc, "scan": sc, "roofline": roof,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_search(p, data)
    print(json.dumps(res), flush=True)


FP32_VECTOR_PEAK_TFLOPS = 157.3


def bench_fibquant(a, torch, synth, tq, dev, n_main=32, sweep=(4, 16, 32, 64, 256)):
    """FibQuant k = 2 over the GQA decode workload's K and V (8 KV heads x
    32768 tokens x 128, fp16): a step encodes both to block codes at
    N = 32 (2.5 bits per coordinate) and decodes both back to fp16.  From
    N = 64 up the encoder tests each block against its cell's candidate
    codewords (the search table), below it tests all N; the sweep also times
    the encoder that tests all N at every N.  Each
    part of each N is one HIP graph over the `--sets` input copies, timed
    with HIP events over replays.  Bytes per row: encode reads 2 d and
    writes d/2 log2(N)/8 + 4; decode the reverse."""
    w = synth.gqa_decode()
    d = 128
    S = a.sets
    k0 = torch.from_numpy(w["k"].reshape(-1, d)).to(dev)
    v0 = torch.from_numpy(w["v"].reshape(-1, d)).to(dev)
    xs = [t.clone() for _ in range(S) for t in (k0, v0)]
    n = k0.shape[0]
    flip = w["codec"].flip
    reps = max(2, a.steps // S)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def time_graph(fn, per):
        fn()
        torch.cuda.synchronize()
        g = capture(fn)
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (reps * per)

    def setup(nc, search=None):
        c = tq.VQCodec(d, nc, flip, search=search)
        bufs = [(torch.empty((n, c.row_bytes), dtype=torch.uint8, device=dev),
                 torch.empty((n,), dtype=torch.float32, device=dev),
                 torch.empty((n, d), dtype=torch.float16, device=dev)) for _ in range(2 * S)]

        def enc():
            for x, (i, nu, _) in zip(xs, bufs):
                tq.encode_vq(c, x, idx=i, norm=nu)

        def dec():
            for i, nu, o in bufs:
                tq.decode_vq(c, i, nu, n, out=o)
        return enc, dec

    rows_sweep = []
    step = None
    for nc in sweep:
        enc, dec = setup(nc)
        te, td = time_graph(enc, 2 * S), time_graph(dec, 2 * S)      # per tensor
        full_enc, _ = setup(nc, search=False)
        tf = time_graph(full_enc, 2 * S)
        bb = int(round(np.log2(nc)))
        row_b = 2 * d + d // 2 * bb // 8 + 4
        rows_sweep.append({"N": nc, "bits_per_coord": bb / 2.0,
                           "encode_us_per_tensor": te * 1e6, "encode_GB_per_s": n * row_b / te / 1e9,
                           "encode_full_search_us_per_tensor": tf * 1e6,
                           "decode_us_per_tensor": td * 1e6, "decode_GB_per_s": n * row_b / td / 1e9})
        if nc == n_main:
            step = (enc, dec)
    enc, dec = step
    g_step = capture(lambda: (enc(), dec()))
    g_step.replay()
    torch.cuda.synchronize()
    steps = max(1, a.steps // S)
    t0 = time.perf_counter()
    for _ in range(steps):
        g_step.replay()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / (steps * S)          # per K+V pair
    main_row = next(r for r in rows_sweep if r["N"] == n_main)
    te = main_row["encode_us_per_tensor"] * 1e-6
    ach = main_row["encode_GB_per_s"]
    roof = {"kernel": "encode_vq_kernel<128,5,_Float16>", "bound": "hbm",
            "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
            "traffic": None}
    res = {
        "metric": "KV vectors encoded/s and decode-attention GB/s over packed codes (% of HBM peak)",
        "value": 2 * n / wall, "unit": "vectors/s", "n_gpus": 1, "steps": steps * S,
        "warmup": a.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fibquant k=2 round trip: GQA decode K and V (8 KV heads x 32768 "
                               "tokens x d128, fp16 Student-t(3), 4 outlier channels x20), N=%d "
                               "(%.1f bits per coordinate), encode + decode to fp16" %
                               (n_main, np.log2(n_main) / 2),
                   "vectors_per_step": 2 * n, "input_sets": S},
        "sweep": rows_sweep, "roofline": roof,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_fibquant(w, n_main)
    print(json.dumps(res), flush=True)


def split_codecs(tq, rng, b_hi, b_lo, synth):
    """Key (prod) and value (mse) split codecs with fresh draws per half."""
    out = []
    for prod in (True, False):
        halves = []
        for b in (b_hi, b_lo):
            dr = synth.codec_draws(rng, 64, m=64 if prod else 0)
            halves.append(tq.Codec(64, tq.TQ_PROD if prod else tq.TQ_MSE, b, dr.flip,
                                   dr.S if prod else None))
        out.append(tq.SplitCodec(*halves))
    return out


def bench_split(a, torch, synth, tq, dev, main=(3, 2), sweep=((3, 2), (4, 3))):
    """Outlier-channel split over the GQA decode workload (8 KV heads x 32768
    tokens x 128, fp16 Student-t(3), four outlier channels x20 per head, 32
    query heads).  Each head's K and V channels are ordered once by the
    library's outlier rule on its first 4096 tokens (the offline permutation a
    model folds into its projection weights; the queries take their KV head's
    key order), outside the timed region.  A step: tq_encode_split of K and V
    (two launches, one per channel half), then tq_attend_split, attention of
    the 32 query heads straight from the split codes.  The two-pass path
    (tq_decode_split of both to fp32, then softmax(q K^T / sqrt d) V with fp32
    torch matmuls) is timed beside it for comparison.  The
    inputs rotate over `--sets` copies (more than the last-level cache); each
    part is one HIP graph per copy, timed with HIP events over replays.
    Quality: relMSE of the decoded K and V, the relative L2 error of the
    score matrix q K^T and the agreement of its top token with the
    unquantized one, beside whole-codec b = 2, 3, 4 (K prod, V mse) through
    the same decoder."""
    w = synth.gqa_decode()
    hkv, ctx, d, hq = 8, 32768, 128, 32
    G = hq // hkv
    kk, vv, qq = w["k"].copy(), w["v"].copy(), w["q"].reshape(hq, d).copy()
    for h in range(hkv):
        pk = tq.outlier_order(kk[h, :4096], 64)
        pv = tq.outlier_order(vv[h, :4096], 64)
        kk[h], vv[h] = kk[h][:, pk], vv[h][:, pv]
        qq[h * G:(h + 1) * G] = qq[h * G:(h + 1) * G][:, pk]
    n = hkv * ctx
    S = a.sets
    k0 = torch.from_numpy(kk.reshape(n, d)).to(dev)
    v0 = torch.from_numpy(vv.reshape(n, d)).to(dev)
    ks = [k0.clone() for _ in range(S)]
    vs = [v0.clone() for _ in range(S)]
    q = torch.from_numpy(qq.astype(np.float32)).to(dev).reshape(hkv, G, d)
    khat = torch.empty((n, d), dtype=torch.float32, device=dev)
    vhat = torch.empty((n, d), dtype=torch.float32, device=dev)
    kf, vf = k0.float().reshape(hkv, ctx, d), v0.float().reshape(hkv, ctx, d)
    out = torch.empty((hkv, G, d), dtype=torch.float32, device=dev)
    q4 = q.reshape(1, hq, 1, d).contiguous()
    out4 = torch.empty((1, hq, 1, d), dtype=torch.float32, device=dev)
    ws = torch.zeros((tq.attend_workspace_bytes(1, 1, hq, hkv, ctx, d),), dtype=torch.uint8, device=dev)

    def attn(kx, vx):
        # fp32 throughout (the transposed operand is an fp32 view)
        s_ = torch.matmul(q, kx.transpose(1, 2)) * (1.0 / d ** 0.5)
        return torch.matmul(torch.softmax(s_, dim=-1), vx)

    # The x20 outlier channels make the logits span tens of units, so the
    # softmax over 32768 tokens is close to one-hot and the attention output
    # is mostly the value of the top token: the score matrix's error and the
    # top-1 agreement measure the keys' effect, the relMSE of V the values'.
    s_ref = torch.matmul(q, kf.transpose(1, 2)).double()

    def quality(kh, vh):
        kh3, vh3 = kh.float().reshape(hkv, ctx, d), vh.float().reshape(hkv, ctx, d)
        rk = float((((kh3 - kf) ** 2).sum(-1) / (kf ** 2).sum(-1)).mean())
        rv = float((((vh3 - vf) ** 2).sum(-1) / (vf ** 2).sum(-1)).mean())
        sc = torch.matmul(q, kh3.transpose(1, 2)).double()
        se = float((sc - s_ref).norm() / s_ref.norm())
        top1 = float((sc.argmax(-1) == s_ref.argmax(-1)).double().mean())
        return {"relmse_k": rk, "relmse_v": rv, "score_rel_l2_err": se, "top1_agreement": top1}

    rng = np.random.default_rng(2024)
    codecs = {bb: split_codecs(tq, rng, bb[0], bb[1], synth) for bb in sweep}
    packs = {bb: [(tq.SplitPacked(codecs[bb][0], n, dev), tq.SplitPacked(codecs[bb][1], n, dev))
                  for _ in range(S)] for bb in sweep}

    def parts(bb):
        kc, vc = codecs[bb]

        def enc(j):
            kp, vp = packs[bb][j]
            tq.encode_split(kc, vc, ks[j], vs[j], kout=kp, vout=vp)

        def dec(j):
            kp, vp = packs[bb][j]
            tq.decode_split(kc, kp, n, out=khat)
            tq.decode_split(vc, vp, n, out=vhat)

        def att(j):
            out.copy_(attn(khat.reshape(hkv, ctx, d), vhat.reshape(hkv, ctx, d)))

        def fused(j):
            kp, vp = packs[bb][j]
            tq.attend_split(kc, vc, q4, kp, vp, ctx, hkv, out=out4, workspace=ws)
        return enc, dec, att, fused

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    reps = max(2, a.steps // S)

    def time_graph(g, per):
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (reps * per)

    def code_bytes(c):
        total = 0
        for h in (c.hi, c.lo):
            total += 64 * h.code_bits // 8 + 4 + (64 // 8 + 4 if h.mode == tq.TQ_PROD else 0)
        return total

    rows = []
    step_graphs = None
    for bb in sweep:
        enc, dec, att, fused = parts(bb)
        for j in range(S):          # eager warm-up (the matmul library sets up outside capture)
            enc(j)
            dec(j)
            att(j)
            fused(j)
        torch.cuda.synchronize()
        t = {name: time_graph(capture(lambda fn=fn: [fn(j) for j in range(S)]), S)
             for name, fn in (("encode", enc), ("decode", dec), ("attention", att),
                              ("fused", fused))}
        enc(0)
        dec(0)
        torch.cuda.synchronize()
        kc, vc = codecs[bb]
        eb = n * (2 * 2 * d + code_bytes(kc) + code_bytes(vc))
        db = n * (2 * 4 * d + code_bytes(kc) + code_bytes(vc))
        rows.append(dict({"bits_hi": bb[0], "bits_lo": bb[1], "bits_per_channel": (bb[0] + bb[1]) / 2.0,
                          "encode_us": t["encode"] * 1e6, "encode_GB_per_s": eb / t["encode"] / 1e9,
                          "encode_frac_of_hbm_peak": eb / t["encode"] / 1e9 / HBM_PEAK_GBS,
                          "attend_split_us": t["fused"] * 1e6,
                          "attend_split_GB_per_s": n * (code_bytes(kc) + code_bytes(vc)) / t["fused"] / 1e9,
                          "two_pass": {"decode_us": t["decode"] * 1e6,
                                       "decode_GB_per_s": db / t["decode"] / 1e9,
                                       "attention_us": t["attention"] * 1e6}},
                         **quality(khat, vhat)))
        # the fused output against the two-pass one on the same codes
        fused(0)
        dec(0)
        att(0)
        torch.cuda.synchronize()
        rows[-1]["fused_vs_two_pass_max_row_rel_diff"] = float(
            ((out4.reshape(hkv, G, d) - out).norm(dim=-1) / out.norm(dim=-1)).max())
        if bb == main:
            step_graphs = [capture(lambda j=j: (enc(j), fused(j))) for j in range(S)]
    uniform = []
    for b in (2, 3, 4):
        kc = tq.Codec(d, tq.TQ_PROD, b, w["codec"].flip, w["codec"].S)
        vc = tq.Codec(d, tq.TQ_MSE, b, w["codec"].flip)
        kp, vp = tq.encode_kv(kc, vc, k0, v0)
        tq.decode_kv(kc, kp, n, out=khat)
        tq.decode_kv(vc, vp, n, out=vhat)
        torch.cuda.synchronize()
        uniform.append(dict({"bits": b}, **quality(khat, vhat)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step_graphs[i % S].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mr = next(r for r in rows if (r["bits_hi"], r["bits_lo"]) == main)
    te = mr["encode_us"] * 1e-6
    eb = mr["encode_GB_per_s"] * 1e9 * te
    roof = {"kernel": "encode_kv_half_kernel<64, 2, 3> + <64, 1, 2> (one launch per channel half)",
            "bound": "hbm", "achieved": eb / te / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": eb / te / 1e9 / HBM_PEAK_GBS, "traffic": None}
    if mr["attend_split_us"] > mr["encode_us"]:
        roof = {"kernel": "decode_split_kernel<2, 1, 3, 2> + merge_kernel<128>", "bound": "hbm",
                "achieved": mr["attend_split_GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": mr["attend_split_GB_per_s"] / HBM_PEAK_GBS, "traffic": None}
    res = {
        "metric": "KV vectors encoded/s and decode-attention GB/s over packed codes (% of HBM peak)",
        "value": 2 * n / (wall / a.steps), "unit": "vectors/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": wall / a.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "outlier-channel split on the GQA decode step: 8 KV heads x 32768 "
                               "tokens x d128 fp16 Student-t(3), 4 outlier channels x20 per head, "
                               "32 query heads; K prod / V mse at %d bits on the 64 outlier-ordered "
                               "channels and %d on the rest (%.1f bits per channel); a step is "
                               "tq_encode_split + tq_attend_split (attention from the split codes)" %
                               (main[0], main[1], (main[0] + main[1]) / 2.0),
                   "vectors_per_step": 2 * n, "input_sets": S},
        "sweep": rows, "uniform_codecs": uniform, "roofline": roof,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_split(kk.reshape(n, d), vv.reshape(n, d), main)
    print(json.dumps(res), flush=True)


def cpu_baseline_split(k, v, bb, rows=262144):
    """The fp64 numpy oracle on a bounded sample: split encode + decode of the
    first `rows` keys (prod) and values (mse)."""
    import oracle
    from oracle import split as SP
    rng = np.random.default_rng(7)

    def half(bits, prod):
        signs = rng.integers(0, 2, 64).astype(bool)
        if prod:
            c, t = oracle.codebook(64, bits - 1)
            return {"signs": signs, "centroids": c, "thresholds": t, "S": rng.standard_normal((64, 64))}
        c, t = oracle.codebook(64, bits)
        return {"signs": signs, "centroids": c, "thresholds": t}
    kh, kl, vh, vl = half(bb[0], True), half(bb[1], True), half(bb[0], False), half(bb[1], False)
    t0 = time.perf_counter()
    for a in range(0, rows, 8192):
        ek = SP.encode_split_prod(k[a:a + 8192].astype(np.float64), 64, kh, kl)
        ev = SP.encode_split_mse(v[a:a + 8192].astype(np.float64), 64, vh, vl)
        SP.decode_split(ek, kh, kl)
        SP.decode_split(ev, vh, vl)
    dt = time.perf_counter() - t0
    return {"value": 2 * rows / dt, "unit": "vectors/s", "cores": _threads(), "kind": "oracle",
            "seconds": dt, "sample": "split %d/%d encode + decode of %d keys and %d values "
                                     "(fp64 numpy, blocks of 8192)" % (bb[0], bb[1], rows, rows)}


def cpu_baseline_fibquant(w, n_codes, rows=65536):
    """The fp64 numpy oracle on a bounded sample: encode + decode of the first
    `rows` keys and `rows` values (codebook built beforehand, untimed)."""
    import oracle
    d = 128
    code = oracle.fibquant_codebook(d, n_codes)
    flip = w["codec"].flip
    k = w["k"].reshape(-1, d)[:rows].astype(np.float64)
    v = w["v"].reshape(-1, d)[:rows].astype(np.float64)
    t0 = time.perf_counter()
    for x in (k, v):
        for a in range(0, rows, 4096):
            idx, nu, _ = oracle.encode_vq(x[a:a + 4096], flip, code)
            oracle.decode_vq(idx, nu, flip, code)
    dt = time.perf_counter() - t0
    return {"value": 2 * rows / dt, "unit": "vectors/s", "cores": _threads(), "kind": "oracle",
            "seconds": dt, "sample": "encode + decode of %d keys and %d values at N=%d "
                                     "(fp64 numpy, blocks of 4096 rows)" % (rows, rows, n_codes)}


def cpu_baseline_search(p, data, rows=65536, queries=16):
    """The fp64 numpy oracle on a bounded sample of the vector-search step:
    encode of the first `rows` rows (in blocks of 8192) and the scores and
    top-10 of `queries` queries against them."""
    import oracle
    d = p["d"]
    c, t = oracle.codebook(d, 1)
    S = p["codec"].S.astype(np.float64)
    flip = p["codec"].flip
    x = data["x"][:rows].cpu().numpy()
    q = data["q"][:queries].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    scores = []
    for a in range(0, rows, 8192):
        e = oracle.encode_prod(x[a:a + 8192].astype(np.float64), flip, c, t, S, keep_z=False)
        codes = {"idx": e.idx, "norm": e.norm, "sign": e.sign, "rnorm": e.rnorm}
        scores.append(oracle.inner_product_matrix(q, codes, {"signs": flip, "centroids": c, "S": S}))
    oracle.top_k(np.concatenate(scores, axis=1), 10)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "vectors/s", "cores": _threads(), "kind": "oracle",
            "seconds": dt, "sample": "encode of %d rows + scores and top-10 of %d queries over "
                                     "them (fp64 numpy)" % (rows, queries)}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max((i.get("num_threads", 1) for i in threadpool_info()), default=1))
    except Exception:
        return int(os.cpu_count())


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def _gqa_oracle_step(w, heads):
    """The oracle's whole step on KV heads 0..heads-1: encode of their keys
    (prod b=4) and values (mse b=4) over all 32768 tokens, then the attention
    of their 4 query heads each."""
    import oracle
    d, ctx = 128, 32768
    kc, kt = oracle.codebook(d, 3)
    vc, vt = oracle.codebook(d, 4)
    S = w["codec"].S.astype(np.float64)
    flip = w["codec"].flip
    k = w["k"][:heads].reshape(-1, d).astype(np.float64)
    v = w["v"][:heads].reshape(-1, d).astype(np.float64)
    q = w["q"][:4 * heads].astype(np.float64).reshape(1, 4 * heads, 1, d)
    t0 = time.perf_counter()
    ek = oracle.encode_prod(k, flip, kc, kt, S)
    ev = oracle.encode_mse(v, flip, vt)
    kcodes = {"idx": ek.idx.reshape(1, heads, ctx, d), "sign": ek.sign.reshape(1, heads, ctx, d),
              "norm": ek.norm.reshape(1, heads, ctx), "rnorm": ek.rnorm.reshape(1, heads, ctx)}
    vcodes = {"idx": ev.idx.reshape(1, heads, ctx, d), "norm": ev.norm.reshape(1, heads, ctx)}
    oracle.attention_from_codes(q, kcodes, vcodes, {"signs": flip, "centroids": kc, "S": S},
                                {"signs": flip, "centroids": vc})
    return time.perf_counter() - t0, ek, ev


def cpu_baseline(w):
    """The fp64 numpy oracle on a bounded sample of the same workload, timed
    on this host: the whole step (8 KV heads) with the BLAS pool at every
    core of this process (median of 3), and one KV head with one thread.
    Bytes are counted as for the GPU: 256 + 72 B per key and 256 + 68 B per
    value encoded, 140 B of codes per token and KV head attended.  Returns
    (baseline record, the oracle's codes of the full step)."""
    from threadpoolctl import threadpool_limits
    ctx = 32768
    per_head = ctx * ((256 + 72) + (256 + 68) + 140)
    cores = _cores()
    times = []
    with threadpool_limits(limits=cores):
        for _ in range(3):
            dt, ek, ev = _gqa_oracle_step(w, 8)
            times.append(dt)
    dt = float(np.median(times))
    with threadpool_limits(limits=1):
        dt1, _, _ = _gqa_oracle_step(w, 1)
    rec = {"value": 2 * 8 * ctx / dt, "unit": "vectors/s", "cores": int(cores), "kind": "oracle",
           "seconds": dt, "GB_per_s": 8 * per_head / dt / 1e9,
           "single_thread": {"value": 2 * ctx / dt1, "unit": "vectors/s", "cores": 1,
                             "seconds": dt1, "GB_per_s": per_head / dt1 / 1e9,
                             "sample": "one KV head: encode of 32768 keys + 32768 values and the "
                                       "attention of its 4 query heads (fp64 numpy, BLAS at 1 "
                                       "thread)"},
           "sample": "one full step (8 KV heads): encode of 262144 keys + 262144 values and the "
                     "attention of 32 query heads over 32768 tokens (fp64 numpy, BLAS at %d "
                     "threads), median of 3" % cores}
    return rec, (ek, ev)


def oracle_agreement(w, orc, kpk, vpk, kc, vc):
    """Code agreement between the GPU's packed keys and values (one buffer
    set of this run) and the oracle's encode of the same input: mismatch
    fractions of the codes, the fraction of coordinates whose fp64 rotated
    value lies within 1e-5 of a threshold (a property of the data), and the
    QJL sign bits against [S r >= 0] recomputed in fp64 from the GPU's own
    codes.  Every mismatch must lie inside the 1e-5 band."""
    import oracle
    ek, ev = orc
    d, band = 128, 1e-5
    kcb, kt = oracle.codebook(d, 3)
    _, vt = oracle.codebook(d, 4)
    S = w["codec"].S.astype(np.float64)
    host = lambda t: t.detach().cpu().numpy()
    out = {}
    for name, enc, pk, cb, t in (("K", ek, kpk, 3, kt), ("V", ev, vpk, 4, vt)):
        g = oracle.unpack_codes(host(pk.idx), d, cb)
        bad = g != enc.idx
        near = np.zeros(enc.z.shape, dtype=bool)
        for a in range(0, enc.z.shape[0], 16384):
            zz = enc.z[a:a + 16384]
            near[a:a + 16384] = np.min(np.abs(zz[..., None] - t), axis=-1) <= band
        out[name] = {"code_mismatch_frac": float(bad.mean()),
                     "mismatch_outside_band": int((bad & ~near).sum()),
                     "near_band_frac": float(near.mean()),
                     "rows_with_a_mismatch_frac": float(bad.any(axis=1).mean())}
        if name == "K":
            sign = oracle.unpack_bits(host(pk.qjl), d)
            p = oracle.qjl_projection(oracle.codec.residual_from_codes(enc.z, g, kcb), S)
            sb = sign != (p >= 0)
            out[name]["qjl_mismatch_frac"] = float(sb.mean())
            out[name]["qjl_mismatch_outside_band"] = int((sb & (np.abs(p) > band)).sum())
    out["note"] = ("GPU codes of one buffer set vs the fp64 oracle's encode of the same input; "
                   "rule: mismatches only within 1e-5 of a threshold, at most 1e-4 of codes")
    return out


if __name__ == "__main__":
    main()
