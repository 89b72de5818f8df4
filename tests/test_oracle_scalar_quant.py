"""Pins of the oracle's scalar quantisers on gauge coordinates ("Codec-Gauge:
Learning Compression-Friendly Gauges for Transformer KV Caches", Compression
Conditions: block-uniform ranges per T_b x d_l block; KIVI-style per-channel
key and per-token value ranges; the same bit settings), CPU only.

Pins: the size arithmetic of the layout, lattice data that quantises without
loss, the min and max of every range landing on the end codes, the half-step
error bound in the coefficient domain, and that an outlier only widens the
ranges it belongs to (per channel for KIVI keys, per token for KIVI values,
per block for block-uniform)."""
import numpy as np
import pytest
import torch

from tensor_compression_amd import synth


def _cfg(orc, **over):
    w = synth.WORKLOADS["tiny"]
    cfg = synth.oracle_config(w, **over)
    return w, cfg


def test_layout_sizes(orc):
    w, cfg = _cfg(orc, layers=2)
    D, H, L = cfg["head_dim"], cfg["kv_heads"], cfg["layers"]
    T = 200
    for kind, g, tile, bk, bv in ((orc.SQ_BLOCK, 16, 64, 4, 3), (orc.SQ_KIVI, 32, 32, 4, 2)):
        sq = dict(kind=kind, group=g, tile=tile, bits_k=bk, bits_v=bv)
        nb, nr = orc.sq_sizes(cfg, sq, T)
        assert nb == L * H * T * D * (bk + bv) // 8
        nt = -(-T // tile)
        if kind == orc.SQ_BLOCK:
            assert nr == L * H * 2 * nt * (D // g)
        else:
            assert nr == L * H * (nt * D + T * (D // g))


def _lattice(orc, kind):
    """fp32 cache, no RoPE, identity basis, values on the integer lattice
    0..15 with both ends present in every range: 4-bit codes are exact."""
    w, cfg = _cfg(orc, rope_keys=0)
    D, T = cfg["head_dim"], 128
    rng = np.random.default_rng(4)
    x = rng.integers(0, 16, (1, 1, T, D)).astype(np.float32)
    x[..., 0, :] = 0.0
    x[..., 1, :] = 15.0
    x[..., :, 0] = 0.0  # per-token value ranges (KIVI) need both ends in each group
    x[..., :, 1] = 15.0
    if kind == orc.SQ_KIVI:
        for q in range(D // 16):
            x[..., :, 16 * q] = 0.0
            x[..., :, 16 * q + 1] = 15.0
    k = x.view(np.uint32).copy()
    v = (15.0 - x).astype(np.float32).view(np.uint32).copy()
    basis = np.broadcast_to(np.eye(D, dtype=np.float32), (1, 2, D, D)).copy()
    return cfg, k, v, basis, x


@pytest.mark.parametrize("kind", [1, 2])
def test_lattice_data_is_lossless(orc, kind):
    cfg, k, v, basis, x = _lattice(orc, kind)
    sq = dict(kind=kind, group=16, tile=64, bits_k=4, bits_v=4)
    codes, ranges = orc.sq_encode(cfg, sq, k, v, basis)
    ko, vo = orc.sq_decode(cfg, sq, codes, ranges, x.shape[2], basis)
    assert np.array_equal(ko, x) and np.array_equal(vo, 15.0 - x)
    # a range spans the lattice (zero 0, step 1) or is constant (step 0)
    full = (ranges[:, 0] == 0.0) & (ranges[:, 1] == 1.0)
    const = ranges[:, 1] == 0.0
    assert np.all(full | const) and full.any()


def _tiny(orc, kind, bits=(4, 3), g=16, tile=64):
    w, cfg = _cfg(orc)
    K, V = synth.generate(w, tokens=256)
    k, v = synth.to_numpy_bits(K), synth.to_numpy_bits(V)
    basis = orc.grouped_klt_basis(cfg, k, v, g)
    sq = dict(kind=kind, group=g, tile=tile, bits_k=bits[0], bits_v=bits[1])
    return cfg, sq, k, v, basis


def _unpack(codes, n, b):
    bits = np.unpackbits(codes, bitorder="little")[: n * b].reshape(n, b)
    return (bits.astype(np.uint32) << np.arange(b, dtype=np.uint32)).sum(axis=1)


@pytest.mark.parametrize("kind", [1, 2])
def test_range_ends_take_the_end_codes_and_half_step_bound(orc, kind):
    cfg, sq, k, v, basis = _tiny(orc, kind)
    T, D = k.shape[2], cfg["head_dim"]
    codes, ranges = orc.sq_encode(cfg, sq, k, v, basis)
    nk = T * D  # one layer, one head: section 0 keys, section 1 values
    for s, b in ((0, sq["bits_k"]), (1, sq["bits_v"])):
        c, _ = orc.section_coeffs(dict(cfg, sink_tokens=0, recent_tokens=0), k, v, basis, s)
        off_c = 0 if s == 0 else nk * sq["bits_k"] // 8
        q = _unpack(codes[off_c:], nk, b).reshape(T, D)
        nr0 = orc.sq_sizes(dict(cfg), dict(sq), T)[1]
        nt = -(-T // sq["tile"])
        g = sq["group"]
        if kind == 1:
            r_of = lambda t, i: (t // sq["tile"]) * (D // g) + i // g
            nr_k = nt * (D // g)
        else:
            r_of = (lambda t, i: (t // sq["tile"]) * D + i) if s == 0 else (lambda t, i: t * (D // g) + i // g)
            nr_k = nt * D
        rg = ranges[(0 if s == 0 else nr_k):]
        tt, ii = np.meshgrid(np.arange(T), np.arange(D), indexing="ij")
        ridx = np.vectorize(r_of)(tt, ii)
        zero, scale = rg[ridx, 0], rg[ridx, 1]
        chat = (q.astype(np.float64) * scale + zero)
        step = scale.astype(np.float64)
        # |c_hat - c| <= step / 2 (plus the fp32 roundings of zero and scale)
        assert np.all(np.abs(chat - c) <= 0.5 * step + 1e-5 * np.abs(c) + 1e-30)
        # every range's minimum maps to code 0 and its maximum to 2^b - 1
        for r in np.unique(ridx):
            sel = ridx == r
            if rg[r, 1] > 0:
                assert q[sel][np.argmin(c[sel])] == 0
                assert q[sel][np.argmax(c[sel])] == (1 << b) - 1


def test_kivi_outlier_stays_in_its_ranges(orc):
    cfg, sq, k, v, basis = _tiny(orc, 2)
    T, D = k.shape[2], cfg["head_dim"]
    _, r0 = orc.sq_encode(cfg, sq, k, v, basis)
    # an outlier token in V: in gauge coordinates it spreads over channels,
    # but only the value ranges of that token may change, and no key range
    v2 = orc.bf16_bits_to_f32(v).reshape(v.shape) if cfg["dtype"] == 1 else v.view(np.float32).copy()
    v2 = v2.copy()
    v2[0, 0, 100] *= 50.0
    v2 = v2.astype(np.float32).view(np.uint32)
    _, r1 = orc.sq_encode(cfg, sq, k, v2, basis)
    nt = -(-T // sq["tile"])
    nrk = nt * D
    g = sq["group"]
    assert np.array_equal(r0[:nrk], r1[:nrk])
    changed = np.nonzero((r0[nrk:] != r1[nrk:]).any(axis=1))[0]
    assert changed.size > 0 and np.all(changed // (D // g) == 100)


@pytest.mark.parametrize("kind", [1, 2])
def test_parity_rules_refuse_planted_mistakes(orc, kind):
    """The GPU parity rules accept the oracle's own output and refuse a code
    moved by one step away from a rounding boundary, a zero point moved
    beyond the coefficient bound and a scale off by more than its bound."""
    import parity
    cfg, sq, k, v, basis = _tiny(orc, kind)
    T = k.shape[2]
    codes, ranges = orc.sq_encode(cfg, sq, k, v, basis)
    parity.check_sq(orc, cfg, sq, k, v, basis, codes, ranges, T)
    bad = codes.copy()
    bad[100] ^= 0x10
    with pytest.raises(AssertionError):
        parity.check_sq(orc, cfg, sq, k, v, basis, bad, ranges, T)
    for col in (0, 1):
        r2 = ranges.copy()
        r2[3, col] += np.float32(1e-3) * max(abs(float(r2[3, 1])), 1e-3)
        with pytest.raises(AssertionError):
            parity.check_sq(orc, cfg, sq, k, v, basis, codes, r2, T)
