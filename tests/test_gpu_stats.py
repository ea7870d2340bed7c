"""The statistical validation harness against the GPU library: for each of
six synthetic regimes and each scheme (TQ-KV, TQ-QKV at 3 bits; FibQuant
N = 32 and the 3 / 2 outlier split at 2.5 bits), the
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


def _gpu_split(x, draws, prod):
    """Outlier-first order from the library's rule, split encode + decode,
    channels put back in the original order."""
    perm = tq.outlier_order(x, 64).astype(np.int64)
    mode = tq.TQ_PROD if prod else tq.TQ_MSE
    halves = [tq.Codec(64, mode, b, dr.flip, dr.S if prod else None) for b, dr in zip((3, 2), draws)]
    c = tq.SplitCodec(*halves)
    xt = torch.from_numpy(np.ascontiguousarray(x[:, perm])).cuda()
    pk = tq.encode_split(c, None, xt, None)[0] if prod else tq.encode_split(None, c, None, xt)[1]
    dec = tq.decode_split(c, pk, x.shape[0], dtype=torch.float32).cpu().numpy()
    out = np.empty_like(dec)
    out[:, perm] = dec
    return out


def _gpu_run_25(scheme, k, v, kd, vd):
    d = k.shape[-1]
    if scheme == "FQ":
        outs = []
        for x, dr in ((k, kd), (v, vd)):
            c = tq.VQCodec(d, 32, dr.flip)
            xt = torch.from_numpy(x).cuda()
            idx, nu = tq.encode_vq(c, xt)
            outs.append(tq.decode_vq(c, idx, nu, x.shape[0], dtype=torch.float32).cpu().numpy())
        return outs
    return _gpu_split(k, kd, True), _gpu_split(v, vd, False)


def _gpu_run(regime, scheme, seeds):
    out = {}
    for s in seeds:
        k, v, q = H.data(regime, s)
        d = k.shape[-1]
        kd, vd = H.draws_for(scheme, H.codec_rng("mt19937", s), d)
        if scheme in H.SCHEMES_25:
            kh, vh = _gpu_run_25(scheme, k, v, kd, vd)
            for name, val in H.metrics(k, v, q, kh, vh).items():
                out.setdefault(name, []).append(val)
            continue
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
@pytest.mark.parametrize("scheme", H.SCHEMES + H.SCHEMES_25)
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
