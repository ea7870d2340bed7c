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

# HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE passes of the
# current kernels, scaled by the runtime copy kernel's reading on a known
# 64 MiB copy (FETCH_SIZE x2.0, WRITE_SIZE x1.0); None where the kernel has
# changed since the counters were taken.
TRAFFIC = {"encode_k": (33138 * 2 + 18432) * 1024,
           "encode_v": (32852 * 2 + 17410) * 1024,
           "attend": (18334 * 2 + 520 + 365 * 2 + 16) * 1024}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=8)
    return ap.parse_args()


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

    def enc_k(j):
        tq.encode_kv(kc, None, ks[j], None, kout=kpk[j])

    def enc_v(j):
        tq.encode_kv(None, vc, None, vs[j], vout=vpk[j])

    def attend(j):
        r = (j + S // 2) % S
        tq.attend_decode(kc, vc, q, kpk[r], vpk[r], ctx, hkv, out=out, workspace=ws)

    def step(j):
        enc_k(j)
        enc_v(j)
        attend(j)

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
    g_parts = {name: capture(lambda fn=fn: [fn(j) for j in range(S)])
               for name, fn in (("encode_k", enc_k), ("encode_v", enc_v), ("attend", attend))}
    reps = max(2, a.steps // S)
    t_part = {}
    for name, g in g_parts.items():
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        t_part[name] = e0.elapsed_time(e1) * 1e-3 / (reps * S)     # seconds per launch

    ms_per_step = wall / a.steps * 1e3
    vectors = 2 * n

    # algorithmic bytes (see the design notes): per key 256 in + 72 out,
    # per value 256 in + 68 out; attention reads 140 B per token per KV head
    kbytes = n * (d * 2 + d * 3 // 8 + d // 8 + 8)
    vbytes = n * (d * 2 + d * 4 // 8 + 4)
    abytes = n * ((d * 3 // 8 + d // 8 + 8) + (d * 4 // 8 + 4))
    tk, tv, ta = t_part["encode_k"], t_part["encode_v"], t_part["attend"]
    enc = {"us_k": tk * 1e6, "us_v": tv * 1e6,
           "vectors_per_s": vectors / (tk + tv),
           "GB_per_s": (kbytes + vbytes) / (tk + tv) / 1e9,
           "frac_of_hbm_peak": (kbytes + vbytes) / (tk + tv) / 1e9 / HBM_PEAK_GBS}
    att = {"us": ta * 1e6, "GB_per_s": abytes / ta / 1e9,
           "frac_of_hbm_peak": abytes / ta / 1e9 / HBM_PEAK_GBS,
           "note": "one tq_attend_decode call: decode kernel + log-sum-exp merge kernel"}
    parts = {"encode_k": (tk, kbytes), "encode_v": (tv, vbytes), "attend": (ta, abytes)}
    dom = max(parts, key=lambda p: parts[p][0])
    t_dom, b_dom = parts[dom]
    roof = {"kernel": {"encode_k": "encode_half_kernel<128,3,prod> (keys, fp16)",
                       "encode_v": "encode_half_kernel<128,4,mse> (values, fp16)",
                       "attend": "decode_kernel<128,3,4> + merge_kernel<128>"}[dom],
            "bound": "hbm", "achieved": b_dom / t_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": b_dom / t_dom / 1e9 / HBM_PEAK_GBS, "traffic": TRAFFIC.get(dom)}

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
        "encode": enc, "attend": att, "roofline": roof,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


def cpu_baseline(w):
    """The fp64 numpy oracle on a bounded sample of the same workload: encode
    of KV heads 0..H-1 (all 32768 tokens, K prod b=4 and V mse b=4) and the
    attention of their query heads, timed on this host."""
    import oracle
    d, ctx = 128, 32768
    heads = 8
    kc, kt = oracle.codebook(d, 3)
    vc, vt = oracle.codebook(d, 4)
    S = w["codec"].S.astype(np.float64)
    flip = w["codec"].flip
    k = w["k"][:heads].reshape(-1, d).astype(np.float64)
    v = w["v"][:heads].reshape(-1, d).astype(np.float64)
    q = w["q"][:4 * heads].astype(np.float64).reshape(1, 4 * heads, 1, d)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        ek = oracle.encode_prod(k, flip, kc, kt, S)
        ev = oracle.encode_mse(v, flip, vt)
        kcodes = {"idx": ek.idx.reshape(1, heads, ctx, d), "sign": ek.sign.reshape(1, heads, ctx, d),
                  "norm": ek.norm.reshape(1, heads, ctx), "rnorm": ek.rnorm.reshape(1, heads, ctx)}
        vcodes = {"idx": ev.idx.reshape(1, heads, ctx, d), "norm": ev.norm.reshape(1, heads, ctx)}
        oracle.attention_from_codes(q, kcodes, vcodes, {"signs": flip, "centroids": kc, "S": S},
                                    {"signs": flip, "centroids": vc})
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = cores
    return {"value": 2 * heads * ctx / dt, "unit": "vectors/s", "cores": int(threads),
            "kind": "oracle", "seconds": dt,
            "sample": "one full step (%d KV heads): encode of %d keys + %d values and the "
                      "attention of %d query heads over 32768 tokens (fp64 numpy), median of 3" %
                      (heads, heads * ctx, heads * ctx, 4 * heads)}


if __name__ == "__main__":
    main()
