"""GPU parity of the scalar quantisers on gauge coordinates ("Codec-Gauge:
Learning Compression-Friendly Gauges for Transformer KV Caches", Compression
Conditions: block-uniform ranges per T_b x d_l block, KIVI-style per-channel
key and per-token value ranges, the same bit settings), through the C ABI
(kvtc_sq_encode / kvtc_sq_decode) against the oracle's scalar quantisers.

Rules: ranges within the MFMA coefficient bound of the exact ones; codes
equal to the oracle's quantiser on the exact coefficients with the GPU's
ranges except within 1e-5 of a rounding boundary (<= 0.01%); the decode of
the GPU's codes and ranges within 1e-4 of the per-channel RMS of the
oracle's decode of the same codes and ranges; the bf16 output is the
round-to-nearest-even cast of the fp32 output."""
import numpy as np
import pytest
import torch

import oracle as orc
import parity
from tensor_compression_amd import kvtc, synth

pytestmark = pytest.mark.gpu

BLOCK, KIVI = kvtc.SQ_BLOCK, kvtc.SQ_KIVI


def _gauge_basis(cfg, g, seed=0):
    L, D = cfg["layers"], cfg["head_dim"]
    B = np.zeros((L, 2, D, D), np.float32)
    for l in range(L):
        for s in range(2):
            G = orc.grouped_gauge(D, g, orc.random_gauge_generators(D, g, 0.5, seed=seed + 100 * l + 10 * s + g))
            B[l, s] = G.T.astype(np.float32)
    return B


def _setup(tokens=1100, layers=2, seed=21, basis="random16", **over):
    w = synth.WORKLOADS["llama3_8b"]
    K, V = synth.generate(w, device="cuda", tokens=tokens, layers=layers, seed=seed)
    cfg = synth.oracle_config(w, layers=layers, **over)
    k, v = synth.to_numpy_bits(K), synth.to_numpy_bits(V)
    if basis == "klt16":
        B = orc.grouped_klt_basis(cfg, k, v, 16)
    elif basis == "pca":
        B = orc.fit_pca_basis(cfg, k, v)
    else:
        B = _gauge_basis(cfg, int(basis[len("random"):]))
        if cfg["basis_per_head"]:
            B = np.repeat(B[:, :, None], cfg["kv_heads"], axis=2).copy()
    plan = kvtc.Plan(cfg, torch.from_numpy(B), max_tokens=max(tokens, 1))
    return cfg, K, V, k, v, B, plan


def _roundtrip(cfg, sq, K, V, k, v, B, plan):
    T = K.shape[2]
    codes, ranges, st = plan.sq_encode(sq, K, V)
    assert st == 0, st
    nb, nr = orc.sq_sizes(cfg, sq, T)
    assert (codes.numel(), ranges.shape[0]) == (nb, nr)
    cg, rg = codes.cpu().numpy(), ranges.cpu().numpy()
    parity.check_sq(orc, cfg, sq, k, v, B, cg, rg, T)
    kd, vd = plan.sq_decode(sq, codes, ranges, T, kvtc.FP32)
    ko, vo = orc.sq_decode(cfg, sq, cg, rg, T, B)
    for got, ref, x in ((kd, ko, k), (vd, vo, v)):
        parity.compare_decode(got.cpu().numpy(), ref, parity.channel_rms(orc.bf16_bits_to_f32(x).reshape(x.shape)))
    return codes, ranges, kd, vd


@pytest.mark.parametrize("sq,basis", [
    (dict(kind=BLOCK, group=16, tile=16, bits_k=4, bits_v=4), "random16"),   # T_b 16, g 16
    (dict(kind=BLOCK, group=128, tile=64, bits_k=3, bits_v=3), "klt16"),     # one range per T_b x d_l
    (dict(kind=KIVI, group=32, tile=32, bits_k=2, bits_v=2), "random16"),    # KIVI 2-bit
    (dict(kind=KIVI, group=16, tile=64, bits_k=4, bits_v=6), "pca"),
    (dict(kind=BLOCK, group=8, tile=8, bits_k=8, bits_v=5), "random8"),
    (dict(kind=KIVI, group=2, tile=2, bits_k=7, bits_v=1), "random32"),
])
def test_sq_parity(sq, basis):
    cfg, K, V, k, v, B, plan = _setup(basis=basis)
    _roundtrip(cfg, sq, K, V, k, v, B, plan)


def test_sq_parity_interleaved_rope_per_head_basis():
    cfg, K, V, k, v, B, plan = _setup(tokens=700, basis="random16", rope_style=1, basis_per_head=1, seed=5)
    _roundtrip(cfg, dict(kind=KIVI, group=16, tile=16, bits_k=4, bits_v=4), K, V, k, v, B, plan)


@pytest.mark.parametrize("T", [1, 5, 64, 65, 127])
def test_sq_short_and_ragged(T):
    cfg, K, V, k, v, B, plan = _setup(tokens=T, layers=1, basis="random16", seed=T)
    for sq in (dict(kind=BLOCK, group=16, tile=16, bits_k=4, bits_v=3),
               dict(kind=KIVI, group=32, tile=64, bits_k=2, bits_v=4)):
        _roundtrip(cfg, sq, K, V, k, v, B, plan)


def test_sq_single_element_ranges():
    """tile 1 and group 1: every range holds one coefficient, whose step is
    0 and whose zero is the coefficient itself; decoding gives back the
    coefficients rounded to bf16 through the inverse gauge."""
    cfg, K, V, k, v, B, plan = _setup(tokens=200, layers=1, basis="random16")
    sq = dict(kind=BLOCK, group=1, tile=1, bits_k=3, bits_v=3)
    codes, ranges, kd, vd = _roundtrip(cfg, sq, K, V, k, v, B, plan)
    assert np.all(ranges[:, 1].cpu().numpy() == 0.0)
    assert not codes.cpu().numpy().any()


def test_sq_bf16_output_is_the_rounded_fp32_output():
    cfg, K, V, k, v, B, plan = _setup(tokens=300, layers=1, basis="random16")
    sq = dict(kind=KIVI, group=16, tile=32, bits_k=4, bits_v=4)
    codes, ranges, st = plan.sq_encode(sq, K, V)
    assert st == 0
    k32, v32 = plan.sq_decode(sq, codes, ranges, 300, kvtc.FP32)
    k16, v16 = plan.sq_decode(sq, codes, ranges, 300, kvtc.BF16)
    assert torch.equal(k32.to(torch.bfloat16), k16) and torch.equal(v32.to(torch.bfloat16), v16)


def test_sq_empty_call():
    cfg, K, V, k, v, B, plan = _setup(tokens=64, layers=1)
    sq = dict(kind=BLOCK, group=16, tile=16, bits_k=4, bits_v=4)
    assert plan.sq_sizes(sq, 0) == (0, 0)
    K0, V0 = K[:, :, :0].contiguous(), V[:, :, :0].contiguous()
    codes, ranges, st = plan.sq_encode(sq, K0, V0)
    assert st == 0 and codes.numel() == 0 and ranges.shape[0] == 0


def test_sq_nonfinite_input_is_reported():
    cfg, K, V, k, v, B, plan = _setup(tokens=200, layers=1)
    sq = dict(kind=KIVI, group=16, tile=16, bits_k=4, bits_v=4)
    V2 = V.clone()
    V2[0, 3, 150, 7] = float("inf")
    _, _, st = plan.sq_encode(sq, K, V2)
    assert st & (1 << kvtc.ERR_NONFINITE)
    K2 = K.clone()
    K2[0, 0, 10, 0] = float("nan")
    _, _, st = plan.sq_encode(sq, K2, V)
    assert st & (1 << kvtc.ERR_NONFINITE)
    _, _, st = plan.sq_encode(sq, K, V)  # the status word is cleared by each call
    assert st == 0


def test_sq_argument_checks():
    cfg, K, V, k, v, B, plan = _setup(tokens=128, layers=1)
    good = dict(kind=BLOCK, group=16, tile=16, bits_k=4, bits_v=4)
    for bad, want in ((dict(good, kind=3), kvtc.ERR_INVALID_ARG), (dict(good, group=3), kvtc.ERR_INVALID_ARG),
                      (dict(good, group=0), kvtc.ERR_INVALID_ARG), (dict(good, tile=0), kvtc.ERR_INVALID_ARG),
                      (dict(good, bits_k=9), kvtc.ERR_INVALID_ARG), (dict(good, bits_v=0), kvtc.ERR_INVALID_ARG),
                      (dict(good, tile=48), kvtc.ERR_UNSUPPORTED), (dict(good, tile=128), kvtc.ERR_UNSUPPORTED)):
        with pytest.raises(kvtc.KvtcError) as e:
            plan.sq_sizes(bad, 128)
        assert e.value.status == want, bad
    with pytest.raises(kvtc.KvtcError) as e:
        plan.sq_sizes(good, 129)  # beyond the plan's max_tokens
    assert e.value.status == kvtc.ERR_INVALID_ARG
    # capacity
    nb, nr = plan.sq_sizes(good, 128)
    codes = torch.empty(nb - 16, dtype=torch.uint8, device="cuda")
    ranges = torch.empty((nr, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(kvtc.KvtcError) as e:
        plan.sq_encode_async(good, K, V, codes, ranges, None)
    assert e.value.status == kvtc.ERR_CAPACITY
    # fp32 caches and WHT plans
    w = synth.WORKLOADS["tiny"]
    Kt, Vt = synth.generate(w, device="cuda", tokens=64)
    pt = kvtc.Plan(synth.oracle_config(w), torch.from_numpy(np.broadcast_to(
        np.eye(64, dtype=np.float32), (1, 2, 64, 64)).copy()), max_tokens=64)
    with pytest.raises(kvtc.KvtcError) as e:
        pt.sq_sizes(good, 64)
    assert e.value.status == kvtc.ERR_UNSUPPORTED
    wh = synth.WORKLOADS["hadamard_long"]
    ph = kvtc.Plan(synth.oracle_config(wh, layers=1), None, max_tokens=64)
    with pytest.raises(kvtc.KvtcError) as e:
        ph.sq_sizes(good, 64)
    assert e.value.status == kvtc.ERR_INVALID_ARG


def test_sq_full_size_sampled_layers():
    """The Llama-3-8B-shaped cache (32 layers x 8 KV heads x 4096 tokens,
    bf16) in the launch configuration of the benchmark; layers 0, 17 and 31
    checked against the oracle on a one-layer slice (sections are coded
    independently, so a layer's codes and ranges do not depend on the
    others)."""
    w = synth.WORKLOADS["llama3_8b"]
    K, V = synth.generate(w, device="cuda")
    cfg = synth.oracle_config(w)
    T = K.shape[2]
    B = _gauge_basis(cfg, 16, seed=7)
    plan = kvtc.Plan(cfg, torch.from_numpy(B), max_tokens=T)
    sq = dict(kind=BLOCK, group=16, tile=16, bits_k=4, bits_v=4)
    codes, ranges, st = plan.sq_encode(sq, K, V)
    assert st == 0
    kd, vd = plan.sq_decode(sq, codes, ranges, T, kvtc.BF16)
    c1 = dict(cfg, layers=1)
    nb1, nr1 = orc.sq_sizes(c1, sq, T)
    cg, rg = codes.cpu().numpy(), ranges.cpu().numpy()
    for l in (0, 17, 31):
        k1 = synth.to_numpy_bits(K[l:l + 1].contiguous())
        v1 = synth.to_numpy_bits(V[l:l + 1].contiguous())
        B1 = B[l:l + 1].copy()
        cl, rl = cg[l * nb1:(l + 1) * nb1], rg[l * nr1:(l + 1) * nr1]
        parity.check_sq(orc, c1, sq, k1, v1, B1, cl, rl, T)
        ko, vo = orc.sq_decode(c1, sq, cl, rl, T, B1)
        for got, ref, x in ((kd[l:l + 1], ko, k1), (vd[l:l + 1], vo, v1)):
            # bf16 output: the oracle's fp32 decode rounded the same way, within
            # the decode bound plus half a bf16 ulp
            g = got.float().cpu().numpy()
            rms = parity.channel_rms(orc.bf16_bits_to_f32(x).reshape(x.shape))
            err = np.abs(g.astype(np.float64) - ref)
            assert np.all(err <= 1e-4 * rms + 2.0 ** -8 * np.abs(ref) + 1e-30)
