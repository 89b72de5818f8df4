"""GPU <-> oracle comparison rules, shared by the GPU tests.

Rules (per section, on identical inputs):
  * bit widths: the GPU's widths equal the oracle's greedy allocation run on
    the GPU's own variances (exact), and equal the oracle's widths on its own
    variances unless a near-tie at the allocation threshold is shown;
  * side information: zero and scale equal the oracle's side-information rule
    applied to the GPU's statistics and widths (exact);
  * coefficients: within the fp32 accumulation bound of the exact dot product;
  * codes: equal to the oracle's quantiser applied to the oracle's own
    coefficients with the GPU's side information, except where the oracle's
    pre-rounding value v lies within 1e-5 of a rounding boundary; such codes
    are counted and must stay at or below 0.01% of all codes;
  * rANS: every chunk record of the GPU container is reproduced bit-for-bit
    by the oracle coder from the record's own decoded bytes (same histogram,
    same table, same states and words);
  * decode: the GPU decoder's fp32 output is within 1e-4 of the per-channel
    RMS of the oracle decoder's output on the same container.
"""
from __future__ import annotations

import math

import numpy as np

BOUNDARY_TOL = 1e-5
BOUNDARY_FRACTION = 1e-4
DECODE_TOL = 1e-4


def _f32(x):
    return np.asarray(x, np.float32)


def rcp_of(scale: np.ndarray) -> np.ndarray:
    """fp32 1/scale with the guard of the side-information rule."""
    s = _f32(scale)
    with np.errstate(divide="ignore", over="ignore"):
        r = np.where(s > 0, np.float32(1.0) / np.where(s > 0, s, np.float32(1.0)), np.float32(0))
    r = _f32(r)
    bad = ~np.isfinite(r)
    r[bad] = 0
    return r


def coeff_bound(orc, cfg, k, v, basis, u, T):
    """Per-element bound on |c_gpu - c_exact| for the fp32 MFMA accumulation of
    the D exact products: 16 * 2^-24 * sum_j |x_j B_ji|.  Four chained
    32-product bf16 MFMA steps have measured up to 9.2 * 2^-24 * sum|x B|; the
    kernel re-computes codes exactly within 24 * 2^-24 * ||x||_2 ||B_i||_2 of a
    rounding boundary, which is never below this bound."""
    lo = orc.layout(cfg, T)
    x = np.abs(orc.section_rows(cfg, k, v, u, lo.mid_begin, lo.mid_end).astype(np.float64))
    H = cfg["kv_heads"]
    l, s, h = u // (2 * H), (u // H) % 2, u % H
    B = basis[l, s, h] if cfg["basis_per_head"] else basis[l, s]
    Bp = np.abs(orc.round_bf16(B) if cfg["dtype"] == 1 else B).astype(np.float64)
    return 16 * 2.0 ** -24 * (x @ Bp) + 1e-30


def compare_section(orc, cfg, T, k, v, basis, gpu_bytes, gpu_stats, u, gpu_coef=None, report=None):
    """Apply the parity rules to section u. Returns a dict of counters."""
    D = cfg["head_dim"]
    H = cfg["kv_heads"]
    s = (u // H) % 2
    lo = orc.layout(cfg, T)
    out = dict(section=u, near_tie=False, boundary_codes=0, codes=0, records=0)
    if lo.T_mid == 0:
        return out
    pc = orc.parse_container(gpu_bytes, cfg, T)
    bits_g = pc["bits"][u].astype(np.uint8)
    zero_g = pc["zero"][u]
    scale_g = pc["scale"][u]
    mu_g, var_g, mn_g, mx_g = (a[u] for a in gpu_stats)
    c, r = orc.section_coeffs(cfg, k, v, basis, u)
    mu_o, var_o, mn_o, mx_o = orc.stats(c)
    wht = cfg["transform"] == 1
    # -- coefficients: within the fp32 accumulation bound of the exact sum
    if wht:
        bound = np.zeros_like(c, dtype=np.float64)
        if gpu_coef is not None:
            assert np.array_equal(gpu_coef, c), "WHT coefficients must be exact"
    else:
        bound = coeff_bound(orc, cfg, k, v, basis, u, T)
        if gpu_coef is not None:
            err = np.abs(gpu_coef.astype(np.float64) - c)
            assert np.all(err <= bound), f"section {u}: coefficient error {float((err / bound).max())} x bound"
    # -- statistics: min/max move by at most the coefficient bound, the
    # variance by 2 sigma b + b^2 (b = the largest bound of the component)
    bmax = bound.max(axis=0)
    sc = np.maximum(np.abs(mn_o), np.abs(mx_o)).astype(np.float64)
    tiny = 1e-7 * sc + 1e-30
    assert np.all(np.abs(mn_g.astype(np.float64) - mn_o) <= bmax + tiny), f"section {u}: min"
    assert np.all(np.abs(mx_g.astype(np.float64) - mx_o) <= bmax + tiny), f"section {u}: max"
    vo = var_o.astype(np.float64)
    vtol = 2 * np.sqrt(vo) * bmax + bmax ** 2 + 1e-6 * vo + tiny ** 2
    assert np.all(np.abs(var_g.astype(np.float64) - vo) <= vtol), f"section {u}: var"
    # -- widths
    if not wht:
        budget = orc.budget(cfg["bits_k"] if s == 0 else cfg["bits_v"], D)
        assert np.array_equal(orc.alloc_greedy(var_g, budget, cfg["max_bits"]), bits_g), \
            f"section {u}: GPU allocation differs from greedy on its own variances"
        bits_o = orc.alloc_greedy(var_o, budget, cfg["max_bits"])
        if not np.array_equal(bits_o, bits_g):
            # near-tie: both allocations are optimal for variances that agree to
            # rounding; their modelled distortions must agree accordingly
            d_o = orc.distortion(var_o, bits_o)
            d_g = orc.distortion(var_o, bits_g)
            assert abs(d_g - d_o) <= 1e-5 * d_o, f"section {u}: allocation differs beyond a near-tie"
            out["near_tie"] = True
    # -- side information: the oracle's rule on the GPU's statistics
    if wht and s == 0:
        b = int(bits_g[0])
        amax = float(np.max(np.maximum(np.abs(mn_g), np.abs(mx_g))))
        Q = (1 << (b - 1)) - 1
        sc = np.float32(amax / Q)
        assert np.all(scale_g == sc), f"section {u}: symmetric scale"
        rcp = rcp_of(np.full(D, sc, np.float32))
        q_ref, v_ref = orc.quantize_sym(c, b, float(rcp[0]))
    else:
        z_r, s_r, rcp = orc.side_info(bits_g, mu_g, mn_g, mx_g)
        assert np.array_equal(z_r.view(np.uint32), zero_g.view(np.uint32)), f"section {u}: zero points"
        assert np.array_equal(s_r.view(np.uint32), scale_g.view(np.uint32)), f"section {u}: scales"
        q_ref, v_ref = orc.quantize(c, bits_g, zero_g, rcp)
    # -- codes
    q_g = orc.section_codes(cfg, gpu_bytes, basis, u, T)
    diff = q_g != q_ref
    if diff.any():
        vb = v_ref[diff].astype(np.float64)
        dist = np.abs(vb - (np.floor(vb) + 0.5))
        assert np.all(dist < BOUNDARY_TOL), \
            f"section {u}: {int(diff.sum())} codes differ, worst boundary distance {dist.max()}"
        assert np.all(np.abs(q_g[diff].astype(int) - q_ref[diff].astype(int)) == 1)
    out["boundary_codes"] = int(diff.sum())
    out["codes"] = int(q_g.size)
    # -- rANS records
    out["records"] = check_records(orc, cfg, gpu_bytes, u, T, bits_g)
    if report is not None:
        report.append(out)
    return out


def check_records(orc, cfg, data, u, T, bits):
    """Re-code every chunk record of section u with the oracle coder and
    require the identical bytes."""
    pc = orc.parse_container(data, cfg, T)
    lo = pc["layout"]
    buf = np.frombuffer(data, np.uint8)
    lanes, sb, D = cfg["rans_lanes"], cfg["rans_scale_bits"], cfg["head_dim"]
    n_rec = 0
    for ch in range(lo.chunks_per_sec):
        idx = u * lo.chunks_per_sec + ch
        off, size = int(pc["offsets"][idx]), int(pc["sizes"][idx])
        n = min(cfg["chunk_tokens"], lo.T_mid - ch * cfg["chunk_tokens"])
        ntiles = (n + cfg["tile_tokens"] - 1) // cfg["tile_tokens"]
        tile_n = [min(cfg["tile_tokens"], n - t * cfg["tile_tokens"]) for t in range(ntiles)]
        P = [orc.packed_bytes(bits, m) for m in tile_n]
        if sum(P) == 0:
            assert size == 0
            continue
        rec = buf[off: off + size]
        freq = rec[:512].view(np.uint16)
        nws = rec[512: 512 + 4 * ntiles].view(np.uint32)
        at = 512 + 4 * ntiles
        packed = []
        streams = []
        for t in range(ntiles):
            st = rec[at: at + 4 * lanes].view(np.uint32)
            nw = int(nws[t])
            wd = rec[at + 4 * lanes: at + 4 * lanes + 2 * nw].view(np.uint16)
            streams.append((st.copy(), wd.copy()))
            packed.append(orc.rans_decode(st, wd, freq, P[t], sb, lanes))
            at += 4 * lanes + 2 * nw + (2 if nw & 1 else 0)
        assert (at + 15) // 16 * 16 == size
        allp = np.concatenate(packed)
        f2 = orc.freq_normalize(orc.byte_histogram(allp), sb)
        assert np.array_equal(f2, freq), f"section {u} chunk {ch}: frequency table"
        for t in range(ntiles):
            st2, wd2 = orc.rans_encode(packed[t], freq, sb, lanes)
            assert np.array_equal(st2, streams[t][0]) and np.array_equal(wd2, streams[t][1]), \
                f"section {u} chunk {ch} tile {t}: rANS stream differs"
        n_rec += 1
    return n_rec


def channel_rms(x: np.ndarray) -> np.ndarray:
    """RMS over tokens per (layer, head, channel) of [L, H, T, D]."""
    return np.sqrt((x.astype(np.float64) ** 2).mean(axis=2, keepdims=True))


def compare_decode(gpu_out: np.ndarray, ref_out: np.ndarray, rms: np.ndarray, tol=DECODE_TOL):
    err = np.abs(gpu_out.astype(np.float64) - ref_out.astype(np.float64))
    lim = tol * rms + 1e-30
    bad = err > lim
    assert not bad.any(), f"{int(bad.sum())} decoded values beyond {tol} x channel RMS (worst {float((err / lim).max())}x)"


def nrmse(a, b) -> float:
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    return math.sqrt(float(((a - b) ** 2).sum() / max((a ** 2).sum(), 1e-300)))
