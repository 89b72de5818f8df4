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
  * records: every chunk record of the GPU container is reproduced
    bit-for-bit by the oracle from the codes the record decodes to (same
    tables, states, words, raw rows and mode), and the packed tiles the
    kernels exchange equal the oracle's packing of the codes;
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
    # -- widths (one budget over all sections: checked over the whole cache
    # by check_global_widths)
    if not wht and cfg.get("alloc_scope", 0) == 0:
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


def check_global_widths(orc, cfg, T, gpu_bytes, gpu_stats, k, v, basis):
    """One budget over all sections: the GPU's widths equal the greedy
    allocation over every component of the cache run on the GPU's own
    variances (exact), and agree with it on the oracle's variances up to a
    near-tie of equal modelled distortion."""
    lo = orc.layout(cfg, T)
    D = cfg["head_dim"]
    pc = orc.parse_container(gpu_bytes, cfg, T)
    bits_g = pc["bits"][: lo.n_sections].astype(np.uint8)
    var_g = gpu_stats[1][: lo.n_sections]
    budget = sum(orc.budget(cfg["bits_k"] if (u // cfg["kv_heads"]) % 2 == 0 else cfg["bits_v"], D)
                 for u in range(lo.n_sections))
    want = orc.alloc_greedy_heap(var_g, budget, cfg["max_bits"]).reshape(lo.n_sections, D)
    assert np.array_equal(want, bits_g), "GPU widths differ from the global greedy on its own variances"
    return bits_g, budget


def check_records(orc, cfg, data, u, T, bits):
    """Every chunk record of section u is the oracle's record of the codes it
    decodes to: identical codes give identical tables, states, words, raw
    rows and record mode."""
    pc = orc.parse_container(data, cfg, T)
    lo = pc["layout"]
    buf = np.frombuffer(data, np.uint8)
    n_rec = 0
    for ch in range(lo.chunks_per_sec):
        idx = u * lo.chunks_per_sec + ch
        off, size, mode = int(pc["offsets"][idx]), int(pc["sizes"][idx]), int(pc["modes"][idx])
        n = min(cfg["chunk_tokens"], lo.T_mid - ch * cfg["chunk_tokens"])
        rec = buf[off: off + size].tobytes()
        q = orc.chunk_decode(cfg, bits, rec, mode, n)
        rec2, mode2 = orc.chunk_encode(cfg, bits, q)
        assert mode2 == mode, f"section {u} chunk {ch}: record mode {mode}, oracle {mode2}"
        assert rec2 == rec, f"section {u} chunk {ch}: record bytes differ from the oracle's"
        n_rec += 1
    return n_rec


def blk_tokens(cfg):
    """Tokens of a transform work block (the chunk, at most 1024 tokens)."""
    return min(cfg["chunk_tokens"], 1024)


def check_packed_tiles(orc, cfg, T, bits, q, slots):
    """The packed tiles of a section in the workspace (`slots` [blocks, slot
    bytes]) are the oracle's packing of its codes q [T_mid, D], padding bits
    and words included."""
    lo = orc.layout(cfg, T)
    blk, tile = blk_tokens(cfg), cfg["tile_tokens"]
    for b in range(slots.shape[0]):
        at = 0
        for a in range(b * blk, min(lo.T_mid, (b + 1) * blk), tile):
            m = min(tile, lo.T_mid - a)
            want = orc.pack(q[a: a + m], bits).tobytes()
            got = slots[b, at: at + len(want)].tobytes()
            assert got == want, f"block {b} tile at token {a}: packed bytes differ from the oracle's packing"
            at += len(want)


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


# ---- scalar quantisers on gauge coordinates ------------------------------------

def sq_extents(sq, s):
    """(tokens, channels) of a range of section kind s (0 keys, 1 values)."""
    if sq["kind"] == 1:
        return sq["tile"], sq["group"]
    return (sq["tile"], 1) if s == 0 else (1, sq["group"])


def sq_section_offsets(cfg, sq, T, u):
    """(code byte offset, range offset) of section u."""
    D, H = cfg["head_dim"], cfg["kv_heads"]
    h, s, l = u % H, (u // H) % 2, u // (2 * H)
    cb = [T * D * sq["bits_k"] // 8, T * D * sq["bits_v"] // 8]
    nr = []
    for kind in (0, 1):
        te, ce = sq_extents(sq, kind)
        nr.append(-(-T // te) * (D // ce))

    def off(x):
        return l * H * (x[0] + x[1]) + (H * x[0] if s else 0) + h * x[s]
    return off(cb), off(nr)


def unpack_rows(buf, T, D, b):
    """Token-major rows of D b-bit codes, least significant bit first."""
    bits = np.unpackbits(np.asarray(buf, np.uint8), bitorder="little")[: T * D * b].reshape(T, D, b)
    return (bits.astype(np.uint32) << np.arange(b, dtype=np.uint32)).sum(axis=2)


def check_sq(orc, cfg, sq, k, v, basis, codes_g, ranges_g, T, report=None):
    """Parity rules of the scalar quantisers, per section:
      * ranges: zero within the coefficient bound of the range's exact
        minimum, scale within twice that bound / (2^b - 1) (plus fp32
        rounding) of the exact (max - min) / (2^b - 1);
      * codes: equal to the oracle's quantiser on the oracle's exact
        coefficients with the GPU's ranges, except where its pre-rounding
        value lies within 1e-5 of a rounding boundary (at most 0.01%)."""
    D, H = cfg["head_dim"], cfg["kv_heads"]
    full = dict(cfg, sink_tokens=0, recent_tokens=0)
    codes_g = np.asarray(codes_g, np.uint8)
    ranges_g = np.asarray(ranges_g, np.float32).reshape(-1, 2)
    n_sec = cfg["layers"] * 2 * H
    n_codes = n_boundary = 0
    for u in range(n_sec):
        s = (u // H) % 2
        b = sq["bits_k"] if s == 0 else sq["bits_v"]
        te, ce = sq_extents(sq, s)
        co, ro = sq_section_offsets(cfg, sq, T, u)
        nr = -(-T // te) * (D // ce)
        rg = ranges_g[ro: ro + nr]
        c, _ = orc.section_coeffs(full, k, v, basis, u)
        c = c[:T].astype(np.float32)
        bound = coeff_bound(orc, full, k, v, basis, u, T)[:T]
        tt, ii = np.meshgrid(np.arange(T), np.arange(D), indexing="ij")
        ridx = (tt // te) * (D // ce) + ii // ce
        mn = np.full(nr, np.inf)
        mx = np.full(nr, -np.inf)
        bm = np.zeros(nr)
        np.minimum.at(mn, ridx.ravel(), c.astype(np.float64).ravel())
        np.maximum.at(mx, ridx.ravel(), c.astype(np.float64).ravel())
        np.maximum.at(bm, ridx.ravel(), bound.ravel())
        tiny = 1e-7 * np.maximum(np.abs(mn), np.abs(mx)) + 1e-30
        zg, sg = rg[:, 0].astype(np.float64), rg[:, 1].astype(np.float64)
        assert np.all(np.abs(zg - mn) <= bm + tiny), f"section {u}: zero points"
        qm = float((1 << b) - 1)
        sref = (mx - mn) / qm
        assert np.all(np.abs(sg - sref) <= 2 * bm / qm + 2.0 ** -22 * sref + tiny / qm), f"section {u}: scales"
        # codes
        rcp = rcp_of(rg[:, 1])
        z32 = rg[:, 0][ridx]
        vref = ((c - z32).astype(np.float32) * rcp[ridx]).astype(np.float32)
        qref = np.clip(np.rint(vref), 0, qm).astype(np.uint32)
        nb = T * D * b // 8
        qg = unpack_rows(codes_g[co: co + nb], T, D, b)
        diff = qg != qref
        if diff.any():
            vb = vref[diff].astype(np.float64)
            dist = np.abs(vb - (np.floor(vb) + 0.5))
            assert np.all(dist < BOUNDARY_TOL), \
                f"section {u}: {int(diff.sum())} codes differ, worst boundary distance {dist.max()}"
            assert np.all(np.abs(qg[diff].astype(int) - qref[diff].astype(int)) == 1)
        n_codes += qg.size
        n_boundary += int(diff.sum())
    assert n_boundary <= BOUNDARY_FRACTION * max(n_codes, 1), f"{n_boundary} boundary codes of {n_codes}"
    if report is not None:
        report.append(dict(codes=n_codes, boundary_codes=n_boundary))
    return n_codes, n_boundary
