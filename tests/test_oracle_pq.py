"""Pins of the oracle's TTAS-X2 value path ("TTAS-X2: Extreme KV Cache
Compression for Large Language Models", 2.2 V Compression: RMS normalisation
per vector, Hadamard transform, two-level product quantisation with K1 = 256
and K2 = 64..512 centroids, fixed-budget outliers per head), CPU only.

Pins: the layout sizes; nearest-centroid choices against brute force in
numpy (bf16-rounded codebooks, lowest index on ties); the level-1 and
level-2 indices of a whole encode against brute force on the coefficients
the encoder keeps; the outlier selection against a sort of |y - y^| done in
numpy; a full outlier budget giving back the input within fp32 rounding
(the orthonormal Hadamard transform is its own inverse); the codebook-sum
decode against a numpy Hadamard matrix; an all-zero cache where every
distance ties; refusal of bad configurations and of a corrupt outlier index."""
import numpy as np
import pytest

from tensor_compression_amd import synth

P8 = dict(sub_dim=8, k1=32, k2=16, outliers=24, block_tokens=48)


def _bf16(a):
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _hadamard(D):
    i = np.arange(D)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return (1 - 2 * par).astype(np.float64) / np.sqrt(D)


def _setup(orc, T=100, D=64, seed=3, pq=P8, dtype=0):
    w = synth.WORKLOADS["tiny"]
    cfg = synth.oracle_config(w, head_dim=D, kv_heads=2, dtype=dtype)
    rng = np.random.default_rng(seed)
    L, H = cfg["layers"], cfg["kv_heads"]
    v = rng.normal(size=(L, H, T, D)).astype(np.float32)
    v[..., :3] *= 6.0  # a few loud channels
    M = D // pq["sub_dim"]
    cb1 = rng.normal(size=(L, M, pq["k1"], pq["sub_dim"])).astype(np.float32)
    cb2 = (0.3 * rng.normal(size=(L, M, pq["k2"], pq["sub_dim"]))).astype(np.float32)
    vb = v.view(np.uint32).copy() if dtype == 0 else None
    return cfg, v, vb, cb1, cb2


def _unpack(row, bit, nb):
    v = 0
    for e in range(nb):
        v |= ((int(row[(bit + e) >> 5]) >> ((bit + e) & 31)) & 1) << e
    return v


def test_layout_sizes(orc):
    cfg, *_ = _setup(orc)
    for pq, rw in ((dict(P8), (8 * (5 + 4) + 31) // 32), (dict(P8, sub_dim=16, k1=256, k2=512), (4 * 17 + 31) // 32)):
        got_rw, ns = orc.pq_sizes(cfg, pq, 100)
        assert got_rw == rw
        assert ns == cfg["layers"] * cfg["kv_heads"] * (-(-100 // pq["block_tokens"])) * pq["outliers"]


def test_nearest_is_the_brute_force_argmin(orc):
    rng = np.random.default_rng(7)
    for k, d in ((256, 8), (64, 8), (16, 16), (512, 4)):
        cb = rng.normal(size=(k, d)).astype(np.float32)
        cr = _bf16(cb).astype(np.float64)
        for _ in range(20):
            y = rng.normal(size=d).astype(np.float32)
            dist = ((y.astype(np.float64)[None, :] - cr) ** 2).sum(axis=1)
            assert orc.pq_nearest(y, cb) == int(np.argmin(dist))
    # exact ties: duplicated centroids go to the lower index
    cb = rng.normal(size=(8, 8)).astype(np.float32)
    cb[5] = cb[2]
    assert orc.pq_nearest(cb[2], cb) == 2
    # the codebook is held in bf16: a point on a rounded centroid is at distance 0
    cb = np.array([[1.0 + 2 ** -12] * 4, [1.0 + 2 ** -20] * 4], np.float32)
    y = np.full(4, 1.0 + 2 ** -12, np.float32)  # closer to centroid 0 unrounded
    assert orc.pq_nearest(y, cb) == 0  # both round to 1.0; the tie goes to index 0
    cb[0] = 1.5
    assert orc.pq_nearest(y, cb) == 1


def _full_y(orc, cfg, pq, vb, cb1, cb2, T):
    """Every coefficient y as the encoder computes it: with a budget of
    block_tokens x D every coefficient is an outlier, stored exactly."""
    full = dict(pq, outliers=pq["block_tokens"] * cfg["head_dim"])
    codes, rms, out = orc.pq_encode(cfg, full, vb, cb1, cb2)
    D = cfg["head_dim"]
    y = np.zeros((cfg["layers"], cfg["kv_heads"], T * D), np.float32)
    for l in range(cfg["layers"]):
        for h in range(cfg["kv_heads"]):
            o = out[l, h].reshape(-1, 2)
            o = o[o[:, 0] != 0xFFFFFFFF]
            assert o.shape[0] == T * D and np.array_equal(np.sort(o[:, 0]), np.arange(T * D))
            y[l, h, o[:, 0]] = o[:, 1].view(np.float32)
    return y.reshape(cfg["layers"], cfg["kv_heads"], T, D), codes, rms


def test_indices_are_nearest_on_the_coefficients(orc):
    cfg, v, vb, cb1, cb2 = _setup(orc)
    T, D, d = v.shape[2], cfg["head_dim"], P8["sub_dim"]
    M, b1, b2 = D // d, 5, 4
    y, codes, rms = _full_y(orc, cfg, P8, vb, cb1, cb2, T)
    # r and y as the pages define them (within fp rounding of an independent numpy evaluation)
    r = np.sqrt((v.astype(np.float64) ** 2).mean(axis=3))
    assert np.allclose(rms, r, rtol=1e-6)
    yn = (v / rms[..., None]).astype(np.float64) @ _hadamard(D).T
    assert np.allclose(y, yn, rtol=1e-5, atol=1e-6)
    c1, c2 = _bf16(cb1).astype(np.float64), _bf16(cb2).astype(np.float64)
    for l in range(cfg["layers"]):
        for h in range(cfg["kv_heads"]):
            for t in range(T):
                row = codes[l, h, t]
                for s in range(M):
                    ys = y[l, h, t, s * d:(s + 1) * d]
                    i1 = _unpack(row, s * b1, b1)
                    i2 = _unpack(row, M * b1 + s * b2, b2)
                    assert i1 == int(np.argmin(((ys[None] - c1[l, s]) ** 2).sum(1)))
                    e = (ys - _bf16(cb1)[l, s, i1]).astype(np.float64)
                    assert i2 == int(np.argmin(((e[None] - c2[l, s]) ** 2).sum(1)))


def test_outliers_are_the_largest_errors(orc):
    cfg, v, vb, cb1, cb2 = _setup(orc)
    T, D, d = v.shape[2], cfg["head_dim"], P8["sub_dim"]
    M, b1, b2 = D // d, 5, 4
    y, codes, rms = _full_y(orc, cfg, P8, vb, cb1, cb2, T)
    _, _, out = orc.pq_encode(cfg, P8, vb, cb1, cb2)
    c1, c2 = _bf16(cb1), _bf16(cb2)
    bt, B = P8["block_tokens"], P8["outliers"]
    for l in range(cfg["layers"]):
        for h in range(cfg["kv_heads"]):
            yh = np.zeros((T, D), np.float32)
            for t in range(T):
                for s in range(M):
                    i1 = _unpack(codes[l, h, t], s * b1, b1)
                    i2 = _unpack(codes[l, h, t], M * b1 + s * b2, b2)
                    yh[t, s * d:(s + 1) * d] = c1[l, s, i1] + c2[l, s, i2]
            mag = np.abs(y[l, h] - yh).ravel()
            for k in range(-(-T // bt)):
                lo, hi = k * bt * D, min(T, (k + 1) * bt) * D
                idx = np.arange(lo, hi)
                order = np.lexsort((idx, -mag[lo:hi]))  # |err| descending, index ascending
                want = np.sort(idx[order[:B]])
                got = out[l, h, k]
                assert np.array_equal(got[:, 0], want)
                assert np.array_equal(got[:, 1].view(np.float32), y[l, h].ravel()[want])


def test_full_budget_gives_back_the_input(orc):
    for dtype in (0, 1):
        cfg, v, vb, cb1, cb2 = _setup(orc, T=50, dtype=dtype)
        if dtype == 1:
            vb = (v.view(np.uint32) >> 16).astype(np.uint16)
            v = (vb.astype(np.uint32) << 16).view(np.float32)
        full = dict(P8, outliers=P8["block_tokens"] * cfg["head_dim"])
        codes, rms, out = orc.pq_encode(cfg, full, vb, cb1, cb2)
        x = orc.pq_decode(cfg, full, codes, rms, out, 50, cb1, cb2)
        assert np.allclose(x, v, rtol=2e-6, atol=2e-6 * np.abs(v).max())


def test_zero_budget_decode_is_the_codebook_sum(orc):
    cfg, v, vb, cb1, cb2 = _setup(orc)
    pq = dict(P8, outliers=0)
    T, D, d = v.shape[2], cfg["head_dim"], P8["sub_dim"]
    M, b1, b2 = D // d, 5, 4
    codes, rms, out = orc.pq_encode(cfg, pq, vb, cb1, cb2)
    assert out.size == 0
    x = orc.pq_decode(cfg, pq, codes, rms, out, T, cb1, cb2)
    c1, c2 = _bf16(cb1), _bf16(cb2)
    Hm = _hadamard(D)
    for l in range(cfg["layers"]):
        for h in range(cfg["kv_heads"]):
            for t in range(0, T, 7):
                yh = np.concatenate([c1[l, s, _unpack(codes[l, h, t], s * b1, b1)] +
                                     c2[l, s, _unpack(codes[l, h, t], M * b1 + s * b2, b2)] for s in range(M)])
                want = (Hm @ yh.astype(np.float64)) * rms[l, h, t]
                assert np.allclose(x[l, h, t], want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


def test_zero_cache_ties_take_the_lowest_indices(orc):
    cfg, v, vb, cb1, cb2 = _setup(orc, T=20)
    cb1[:, :, 5] = 0.0  # a zero centroid at 5 (and one at 9: the tie goes to 5)
    cb1[:, :, 9] = 0.0
    cb2[:, :, 2] = 0.0
    z = np.zeros_like(vb)
    pq = dict(P8, block_tokens=8)
    codes, rms, out = orc.pq_encode(cfg, pq, z, cb1, cb2)
    assert not rms.any()
    D, M = cfg["head_dim"], cfg["head_dim"] // 8
    for s in range(M):
        assert _unpack(codes[0, 0, 3], s * 5, 5) == 5
        assert _unpack(codes[0, 0, 3], M * 5 + s * 4, 4) == 2
    # every error is zero: each block keeps its first `outliers` coefficients
    for k in range(3):
        n = min(8, 20 - 8 * k) * D
        want = 8 * k * D + np.arange(min(pq["outliers"], n))
        assert np.array_equal(out[0, 0, k, : want.size, 0], want)
        assert not out[0, 0, k, :, 1].any()
    x = orc.pq_decode(cfg, pq, codes, rms, out, 20, cb1, cb2)
    assert not x.any()


def test_refusals(orc):
    cfg, v, vb, cb1, cb2 = _setup(orc)
    for bad in (dict(P8, k1=24), dict(P8, k2=1024), dict(P8, sub_dim=3), dict(P8, outliers=-1),
                dict(P8, block_tokens=0)):
        with pytest.raises(orc.OracleError):
            orc.pq_sizes(cfg, bad, 10)
    codes, rms, out = orc.pq_encode(cfg, P8, vb, cb1, cb2)
    bad = out.copy()
    bad[0, 0, 1, 0, 0] = 0  # an index of block 0 listed in block 1
    with pytest.raises(orc.OracleError):
        orc.pq_decode(cfg, P8, codes, rms, bad, v.shape[2], cb1, cb2)
    vn = v.copy()
    vn[0, 1, 7, 3] = np.inf
    with pytest.raises(orc.OracleError):
        orc.pq_encode(cfg, P8, vn.view(np.uint32), cb1, cb2)
