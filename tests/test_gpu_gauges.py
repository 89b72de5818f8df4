"""GPU parity with grouped orthogonal gauges as the basis ("Codec-Gauge:
Learning Compression-Friendly Gauges for Transformer KV Caches", Gauge
Parameterization and Training: block-diagonal G = diag(exp(A_k - A_k^T)) over
groups of g channels; Compression Conditions: the random-gauge and grouped
PCA/KLT controls).  The codec takes the gauge as its basis B = G^T; every
section must meet the per-section parity rules and the decode bound."""
import numpy as np
import pytest
import torch

import oracle as orc
import parity
from tensor_compression_amd import kvtc, synth

pytestmark = pytest.mark.gpu


def _basis(kind, g, cfg, k, v, lo):
    L, D = cfg["layers"], cfg["head_dim"]
    if kind == "klt":
        return orc.grouped_klt_basis(cfg, k, v, g, lo.mid_begin, lo.mid_end)
    B = np.zeros((L, 2, D, D), np.float32)
    for l in range(L):
        for s in range(2):
            G = orc.grouped_gauge(D, g, orc.random_gauge_generators(D, g, 0.5, seed=100 * l + 10 * s + g))
            B[l, s] = G.T.astype(np.float32)
    return B


@pytest.mark.parametrize("kind,g", [("random", 8), ("random", 16), ("random", 32), ("klt", 16)])
def test_grouped_gauge_parity(kind, g):
    w = synth.WORKLOADS["llama3_8b"]
    layers = 2
    K, V = synth.generate(w, device="cuda", tokens=1500, layers=layers, seed=9)
    T = K.shape[2]
    cfg = synth.oracle_config(w, layers=layers)
    k, v = synth.to_numpy_bits(K), synth.to_numpy_bits(V)
    lo = orc.layout(cfg, T)
    basis = _basis(kind, g, cfg, k, v, lo)
    plan = kvtc.Plan(cfg, torch.from_numpy(basis), max_tokens=T)
    ws = plan.workspace(T)
    data, st = plan.encode(K, V, ws)
    assert st == kvtc.OK, kvtc.STATUS[st]
    gbytes = data.cpu().numpy().tobytes()
    stats = plan.section_stats(ws, T, lo.n_sections)
    report = []
    for u in range(lo.n_sections):
        coef, _ = plan.coeffs(K, V, u, u + 1, lo.T_mid)
        parity.compare_section(orc, cfg, T, k, v, basis, gbytes, stats, u, gpu_coef=coef[0].cpu().numpy(),
                               report=report)
    assert sum(r["boundary_codes"] for r in report) <= parity.BOUNDARY_FRACTION * sum(r["codes"] for r in report)
    kd, vd, st2 = plan.decode(data, T, kvtc.FP32)
    assert st2 == kvtc.OK
    rk, rv = orc.decode(cfg, gbytes, basis, T)
    for got, ref, x in ((kd, rk, k), (vd, rv, v)):
        parity.compare_decode(got.cpu().numpy(), ref, parity.channel_rms(orc.bf16_bits_to_f32(x).reshape(x.shape)))
