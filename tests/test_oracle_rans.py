"""Pins of the oracle's frequency tables and interleaved rANS coder:
exhaustive round trips, closed forms and the entropy bound (CPU only)."""
import itertools
import math

import numpy as np
import pytest


def test_freq_normalize_properties(orc):
    rng = np.random.default_rng(0)
    for sb in (8, 12, 15):
        M = 1 << sb
        for _ in range(200):
            k = int(rng.integers(1, 257))
            counts = np.zeros(256, np.uint32)
            idx = rng.choice(256, k, replace=False)
            counts[idx] = rng.geometric(rng.uniform(0.001, 0.9), k).astype(np.uint32)
            f = orc.freq_normalize(counts, sb)
            assert int(f.sum()) == M
            assert np.array_equal(f > 0, counts > 0)


def test_freq_normalize_closed_forms(orc):
    c = np.zeros(256, np.uint32)
    c[0], c[1] = 3, 1
    f = orc.freq_normalize(c, 12)
    assert f[0] == 3072 and f[1] == 1024 and f.sum() == 4096
    c = np.zeros(256, np.uint32)
    c[77] = 123
    f = orc.freq_normalize(c, 12)
    assert f[77] == 4096 and f.sum() == 4096  # a single symbol takes the whole range
    f = orc.freq_normalize(np.full(256, 5, np.uint32), 12)
    assert np.all(f == 16)
    assert np.all(orc.freq_normalize(np.zeros(256, np.uint32), 12) == 0)


def _round_trip(orc, sym, freq, lanes, sb=12):
    states, words = orc.rans_encode(sym, freq, sb, lanes)
    out = orc.rans_decode(states, words, freq, sym.size, sb, lanes)
    assert np.array_equal(out, sym)
    return states, words


def test_freq_normalize_rounds_half_up(orc):
    """Counts (2, 5, 2) of N = 9 at M = 256: n M / N = 56.9, 142.2, 56.9 round
    to 57, 142, 57, which already sum to M.  (Flooring would give 56, 142, 56
    and hand the deficit of 2 to the most frequent symbol: 56, 144, 56.)"""
    c = np.zeros(256, np.uint32)
    c[[3, 4, 5]] = [2, 5, 2]
    f = orc.freq_normalize(c, 8)
    assert list(f[[3, 4, 5]]) == [57, 142, 57] and int(f.sum()) == 256


def test_rans_exhaustive_tiny_alphabets(orc):
    """Every sequence of length 0..8 over alphabets of 1..3 symbols, with
    several tables and lane counts, round-trips exactly."""
    tables = {
        1: [{7: 4096}],
        2: [{0: 2048, 255: 2048}, {0: 4095, 1: 1}, {3: 1, 9: 4095}],
        3: [{0: 1, 1: 2, 2: 4093}, {5: 1365, 6: 1365, 7: 1366}, {0: 4000, 100: 95, 200: 1}],
    }
    for a, tbls in tables.items():
        for tbl in tbls:
            freq = np.zeros(256, np.uint16)
            for s, f in tbl.items():
                freq[s] = f
            alphabet = sorted(tbl)
            for n in range(9):
                for seq in itertools.product(alphabet, repeat=n):
                    sym = np.array(seq, np.uint8)
                    for lanes in (1, 2, 3, 16, 32):
                        _round_trip(orc, sym, freq, lanes)


def test_rans_single_symbol_emits_nothing(orc):
    freq = np.zeros(256, np.uint16)
    freq[42] = 4096
    sym = np.full(10000, 42, np.uint8)
    states, words = _round_trip(orc, sym, freq, 32)
    assert words.size == 0 and np.all(states == 65536)


@pytest.mark.parametrize("lanes", [1, 5, 16, 32])
def test_rans_uniform_table_closed_form(orc, lanes):
    """With f = 16 for all 256 symbols each symbol adds exactly 8 bits: lane j
    with n_j symbols emits floor(n_j / 2) words."""
    rng = np.random.default_rng(1)
    freq = np.full(256, 16, np.uint16)
    for N in (0, 1, 2, 63, 64, 1000, 4097):
        sym = rng.integers(0, 256, N).astype(np.uint8)
        _, words = _round_trip(orc, sym, freq, lanes)
        n_j = [len(range(j, N, lanes)) for j in range(lanes)]
        assert words.size == sum(n // 2 for n in n_j)


def test_rans_entropy_bound(orc):
    """Coded word bytes stay within 1% of the order-0 entropy of the input
    when the table is built from the input's own histogram."""
    rng = np.random.default_rng(2)
    for dist in ("geometric", "gauss", "skew", "uniform"):
        N = 1 << 18
        if dist == "geometric":
            sym = np.minimum(rng.geometric(0.05, N), 255).astype(np.uint8)
        elif dist == "gauss":
            sym = np.clip(np.rint(rng.standard_normal(N) * 20 + 128), 0, 255).astype(np.uint8)
        elif dist == "skew":
            p = np.exp(-np.arange(256) / 10.0)
            sym = rng.choice(256, N, p=p / p.sum()).astype(np.uint8)
        else:
            sym = rng.integers(0, 256, N).astype(np.uint8)
        counts = orc.byte_histogram(sym)
        freq = orc.freq_normalize(counts, 12)
        _, words = _round_trip(orc, sym, freq, 32)
        p = counts[counts > 0] / N
        H = -(p * np.log2(p)).sum()
        assert 2 * words.size <= 1.01 * N * H / 8, (dist, 2 * words.size, N * H / 8)


def test_rans_detects_damage(orc):
    rng = np.random.default_rng(3)
    sym = np.clip(np.rint(rng.standard_normal(5000) * 10 + 50), 0, 255).astype(np.uint8)
    freq = orc.freq_normalize(orc.byte_histogram(sym), 12)
    states, words = orc.rans_encode(sym, freq, 12, 32)
    with pytest.raises(orc.OracleError):
        orc.rans_decode(states, words[1:], freq, sym.size, 12, 32)  # truncated
    with pytest.raises(orc.OracleError):
        orc.rans_decode(states, np.concatenate([words, words[:1]]), freq, sym.size, 12, 32)
    bad = states.copy()
    bad[3] ^= 0x10
    try:
        out = orc.rans_decode(bad, words, freq, sym.size, 12, 32)
        assert not np.array_equal(out, sym)
    except orc.OracleError:
        pass
    bad_freq = freq.copy()
    bad_freq[int(np.argmax(freq))] += 1  # table no longer sums to 4096
    with pytest.raises(orc.OracleError):
        orc.rans_decode(states, words, bad_freq, sym.size, 12, 32)
