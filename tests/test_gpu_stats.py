"""The statistical validation harness against the GPU library: for each of
six synthetic regimes and both schemes (TQ-KV, TQ-QKV at 3 bits), the
per-seed metrics of the GPU (encode + tq_decode_kv, codec draws from
MT19937) and of the oracle (codec draws from PCG64) must not be separated
by a two-sample KS test ("Riepilogo Tecnico: Ablazione, Inferenza
Statistica e Validazione", "Configurazione Sperimentale")."""

import numpy as np
import pytest
import torch

import harness as H
from synth import regimes

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_04_amd")

BITS = 3
SEEDS = range(32)


def _gpu_run(regime, scheme, seeds):
    out = {}
    for s in seeds:
        k, v, q = H.data(regime, s)
        d = k.shape[-1]
        kd, vd = H.draws_for(scheme, H.codec_rng("mt19937", s), d)
        if scheme == "TQ-QKV":
            kc = tq.Codec(d, tq.TQ_PROD, BITS, kd.flip, kd.S)
        else:
            kc = tq.Codec(d, tq.TQ_MSE, BITS, kd.flip)
        vc = tq.Codec(d, tq.TQ_MSE, BITS, vd.flip)
        kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        kp = tq.encode_kv(kc, None, kt, None)[0] if scheme == "TQ-QKV" else tq.encode_kv(None, kc, None, kt)[1]
        _, vp = tq.encode_kv(None, vc, None, vt)
        kh = tq.decode_kv(kc, kp, k.shape[0], dtype=torch.float32).cpu().numpy()
        vh = tq.decode_kv(vc, vp, v.shape[0], dtype=torch.float32).cpu().numpy()
        for name, val in H.metrics(k, v, q, kh, vh).items():
            out.setdefault(name, []).append(val)
    return {name: np.array(vals) for name, vals in out.items()}


@pytest.mark.parametrize("regime", regimes.REGIMES)
@pytest.mark.parametrize("scheme", H.SCHEMES)
def test_gpu_and_oracle_metric_distributions_agree(regime, scheme):
    print("[case] stats %s %s, %d seeds" % (regime, scheme, len(SEEDS)), flush=True)
    g = _gpu_run(regime, scheme, SEEDS)
    o = H.oracle_run(regime, scheme, BITS, SEEDS, "pcg64")
    ps = {name: H.ks_p(o[name], g[name]) for name in o}
    print("  oracle means", {n: round(float(v.mean()), 5) for n, v in o.items()})
    print("  gpu means   ", {n: round(float(v.mean()), 5) for n, v in g.items()})
    print("  KS p", {n: round(p, 4) for n, p in ps.items()}, flush=True)
    for name, p in ps.items():
        assert p > 1e-3, (name, p)
