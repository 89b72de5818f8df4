"""GPU parity: the HIP path (through the C ABI) against the oracle on the same
seeded inputs.  Rules are in tests/parity.py."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import parity
from tensor_compression_amd import kvtc, synth
from tensor_compression_amd.calibrate import fit_pca_basis

pytestmark = pytest.mark.gpu


def _setup(name, tokens=None, layers=None, seed=None, workload=None, **over):
    w = synth.WORKLOADS[name] if workload is None else workload
    K, V = synth.generate(w, device="cuda", tokens=tokens, layers=layers, seed=seed)
    T = K.shape[2]
    cfg = synth.oracle_config(w, layers=K.shape[0], **over)
    k, v = synth.to_numpy_bits(K), synth.to_numpy_bits(V)
    basis = None
    if cfg["transform"] == 0:
        lo = orc.layout(cfg, T)
        t0, t1 = (0, T) if w.basis_from == "all" else (lo.mid_begin, max(lo.mid_end, lo.mid_begin + 1))
        basis = orc.fit_pca_basis(cfg, k, v, t0, min(t1, T))
    plan = kvtc.Plan(cfg, None if basis is None else torch.from_numpy(basis), max_tokens=max(T, 1))
    return cfg, T, K, V, k, v, basis, plan


def _encode(plan, K, V):
    T = K.shape[2]
    ws = plan.workspace(T)
    data, st = plan.encode(K, V, ws)
    return data.cpu().numpy().tobytes(), st, ws


def _full_parity(cfg, T, K, V, k, v, basis, plan, sections=None, decode_check=True):
    data, st, ws = _encode(plan, K, V)
    assert st == kvtc.OK, kvtc.STATUS[st]
    lo = orc.layout(cfg, T)
    stats = plan.section_stats(ws, T, lo.n_sections)
    secs = range(lo.n_sections) if sections is None else sections
    report = []
    for u in secs:
        coef, _ = plan.coeffs(K, V, u, u + 1, lo.T_mid)
        parity.compare_section(orc, cfg, T, k, v, basis, data, stats, u,
                               gpu_coef=coef[0].cpu().numpy(), report=report)
    total_codes = sum(r["codes"] for r in report)
    boundary = sum(r["boundary_codes"] for r in report)
    assert boundary <= parity.BOUNDARY_FRACTION * max(total_codes, 1)
    # the packed tiles the encoder's kernels exchanged are the oracle's packing
    # of the codes the container holds
    pc = orc.parse_container(data, cfg, T)
    codes = {u: orc.section_codes(cfg, data, basis, u, T) for u in secs} if lo.T_mid else {}
    for u in codes:
        parity.check_packed_tiles(orc, cfg, T, pc["bits"][u], codes[u], plan.packed_tiles(ws, T, u).cpu().numpy())
    if decode_check:
        wsd = plan.workspace(T)
        kd, vd, st2 = plan.decode(torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda(), T, kvtc.FP32, ws=wsd)
        assert st2 == kvtc.OK
        # and the record decoder rebuilds exactly those tiles
        for u in codes:
            parity.check_packed_tiles(orc, cfg, T, pc["bits"][u], codes[u],
                                      plan.packed_tiles(wsd, T, u).cpu().numpy())
        kd, vd = kd.cpu().numpy(), vd.cpu().numpy()
        H = cfg["kv_heads"]
        ref = orc.decode_sections(cfg, data, basis, 0, lo.n_sections, lo.T_mid) if sections is None else None
        for u in secs:
            l, s, h = u // (2 * H), (u // H) % 2, u % H
            if ref is not None:
                mid_ref = ref[u]
            else:
                mid_ref = orc.decode_sections(cfg, data, basis, u, u + 1, lo.T_mid)[0]
            src = k if s == 0 else v
            srcf = orc.bf16_bits_to_f32(src).reshape(src.shape) if cfg["dtype"] == 1 else src
            rms = np.sqrt((srcf[l, h].astype(np.float64) ** 2).mean(axis=0))
            got = (kd if s == 0 else vd)[l, h, lo.mid_begin: lo.mid_end]
            parity.compare_decode(got, mid_ref, rms[None, :])
        # raw windows restored bit-exactly (fp32 output of a bf16 cache widens exactly)
        for a, b in ((k, kd), (v, vd)):
            af = orc.bf16_bits_to_f32(a).reshape(a.shape) if cfg["dtype"] == 1 else a
            assert np.array_equal(af[:, :, : lo.s0], b[:, :, : lo.s0])
            assert np.array_equal(af[:, :, lo.mid_end:], b[:, :, lo.mid_end:])
    return data, report


# --------------------------------------------------------------------------- stages

def test_freq_tables_match_oracle():
    """The record encoder's normaliser on alphabets of 1..16 symbols."""
    rng = np.random.default_rng(0)
    cases, alpha = [], []
    for _ in range(400):
        A = int(rng.integers(1, 17))
        c = np.zeros(16, np.uint32)
        k = int(rng.integers(1, A + 1))
        c[rng.choice(A, k, replace=False)] = rng.geometric(rng.uniform(0.0005, 0.9), k)
        cases.append(c)
        alpha.append(A)
    for A in (1, 2, 4, 8, 16):  # single symbol, uniform, empty
        for c in (np.eye(16, dtype=np.uint32)[A - 1] * 77, np.r_[np.full(A, 3), np.zeros(16 - A)].astype(np.uint32),
                  np.zeros(16, np.uint32)):
            cases.append(c)
            alpha.append(A)
    counts = torch.from_numpy(np.stack(cases).astype(np.int32)).cuda()
    al = torch.tensor(alpha, dtype=torch.int32).cuda()
    for sb in (8, 10, 12):
        g = kvtc.freq_tables(counts, al, sb).cpu().numpy().view(np.uint16)
        for i, (c, A) in enumerate(zip(cases, alpha)):
            want = orc.freq_normalize(c[:A], sb)
            assert np.array_equal(g[i, :A], want), (sb, A, c)
            assert not g[i, A:].any()


# --------------------------------------------------------------------------- pipeline

def test_tiny_workload_parity():
    """1 layer, 1 head, head_dim 64, 256 tokens, fp32; fp32 MFMA path."""
    cfg, T, K, V, k, v, basis, plan = _setup("tiny")
    data, report = _full_parity(cfg, T, K, V, k, v, basis, plan)
    # the GPU decoder reads the oracle's container as well
    od = orc.encode(cfg, k, v, basis)
    kd, vd, st = plan.decode(torch.frombuffer(bytearray(od), dtype=torch.uint8).cuda(), T, kvtc.FP32)
    assert st == kvtc.OK
    ko, vo = orc.decode(cfg, od, basis, T)
    for a, b, src in ((kd.cpu().numpy(), ko, k), (vd.cpu().numpy(), vo, v)):
        parity.compare_decode(a, b, parity.channel_rms(src))


def test_llama_shaped_reduced_parity():
    """2 layers x 8 heads x 1500 tokens bf16: two chunks per section, a
    ragged last chunk and tile."""
    cfg, T, K, V, k, v, basis, plan = _setup("llama3_8b", tokens=1500, layers=2)
    _full_parity(cfg, T, K, V, k, v, basis, plan)


@pytest.mark.parametrize("bits", [1.0, 1.6, 2.0, 4.0])
def test_budget_sweep_parity(bits):
    """Qwen3-32B-shaped generator, 1 layer, 2200 tokens, the budget sweep."""
    cfg, T, K, V, k, v, basis, plan = _setup("qwen3_32b", tokens=2200, layers=1, bits_k=bits,
                                             bits_v=bits, chunk_tokens=512, tile_tokens=128)
    _full_parity(cfg, T, K, V, k, v, basis, plan)


@pytest.mark.parametrize("wht_keys", [1, 0])
def test_hadamard_path_parity(wht_keys):
    cfg, T, K, V, k, v, basis, plan = _setup("hadamard_long", tokens=1300, layers=2, wht_keys=wht_keys)
    _full_parity(cfg, T, K, V, k, v, basis, plan)


def test_interleaved_rope_per_head_basis():
    cfg, T, K, V, k, v, basis, plan = _setup("llama3_8b", tokens=700, layers=1, rope_style=1,
                                             basis_per_head=1, chunk_tokens=256, tile_tokens=64,
                                             rans_lanes=16)
    _full_parity(cfg, T, K, V, k, v, basis, plan)


@pytest.mark.parametrize("T", [0, 1, 20, 132, 133, 147, 148, 149, 1157])
def test_edge_lengths(T):
    """Empty, all-raw, one-token and ragged middles (sink 4, recent 128)."""
    w = synth.WORKLOADS["llama3_8b"]
    K, V = synth.generate(w, device="cuda", tokens=max(T, 1), layers=1)
    K, V = K[:, :, :T].contiguous(), V[:, :, :T].contiguous()
    cfg = synth.oracle_config(w, layers=1, head_dim=128, chunk_tokens=512, tile_tokens=128)
    k, v = synth.to_numpy_bits(K), synth.to_numpy_bits(V)
    Kb, Vb = synth.generate(w, device="cpu", tokens=600, layers=1)
    basis = orc.fit_pca_basis(cfg, synth.to_numpy_bits(Kb), synth.to_numpy_bits(Vb), 4, 472)
    plan = kvtc.Plan(cfg, torch.from_numpy(basis), max_tokens=2048)
    if T == 0:
        data, st, ws = _encode(plan, K, V)
        assert st == kvtc.OK and data == orc.encode(cfg, k, v, basis)
        return
    _full_parity(cfg, T, K, V, k, v, basis, plan)


@pytest.mark.parametrize("case", ["bf16_head_dim_64", "bf16_tile_32", "fp32_hadamard"])
def test_generic_kernel_configurations(case):
    """Configurations served by the generic transform kernels rather than the
    bf16 head_dim-128 ones: a bf16 head_dim-64 cache, 32-token tiles, and the
    Hadamard path on an fp32 cache."""
    import dataclasses
    if case == "bf16_head_dim_64":
        w = dataclasses.replace(synth.WORKLOADS["llama3_8b"], head_dim=64, rank=16)
        args = dict(tokens=900, layers=1, workload=w, head_dim=64, chunk_tokens=512, tile_tokens=128)
    elif case == "bf16_tile_32":
        args = dict(tokens=700, layers=1, chunk_tokens=256, tile_tokens=32)
    else:
        w = dataclasses.replace(synth.WORKLOADS["hadamard_long"], dtype="fp32")
        args = dict(tokens=900, layers=1, workload=w, dtype=0)
    name = "hadamard_long" if case == "fp32_hadamard" else "llama3_8b"
    cfg, T, K, V, k, v, basis, plan = _setup(name, **args)
    _full_parity(cfg, T, K, V, k, v, basis, plan)


def test_deterministic_container():
    cfg, T, K, V, k, v, basis, plan = _setup("llama3_8b", tokens=900, layers=1)
    d1, _, _ = _encode(plan, K, V)
    d2, _, _ = _encode(plan, K, V)
    assert d1 == d2


def test_damaged_containers_are_refused():
    cfg, T, K, V, k, v, basis, plan = _setup("llama3_8b", tokens=1200, layers=1)
    data, st, ws = _encode(plan, K, V)
    pc = orc.parse_container(data, cfg, T)
    rec = int(pc["offsets"][0])

    def status(d, n=None, TT=T):
        t = torch.frombuffer(bytearray(d), dtype=torch.uint8).cuda()
        shape = (1, cfg["kv_heads"], TT, cfg["head_dim"])
        ko = torch.empty(shape, dtype=torch.float32, device="cuda")
        vo = torch.empty(shape, dtype=torch.float32, device="cuda")
        ws2 = plan.workspace(TT)
        plan.decode_async(t, len(d) if n is None else n, TT, ko, vo, ws2, kvtc.FP32)
        torch.cuda.synchronize()
        return plan.result(ws2)[1]

    assert status(data) == kvtc.OK
    bad = bytearray(data); bad[1] ^= 0x20
    assert status(bad) == kvtc.ERR_CORRUPT                 # magic
    assert status(data, n=len(data) - 16) == kvtc.ERR_CORRUPT  # truncated
    assert status(data, n=200) == kvtc.ERR_CORRUPT
    assert status(data, TT=T - 1) == kvtc.ERR_CORRUPT      # header T mismatch
    bad = bytearray(data); bad[176] ^= 1
    assert status(bad) == kvtc.ERR_CORRUPT                 # basis fingerprint
    bad = bytearray(data); bad[rec + 5] ^= 0x10
    assert status(bad) == kvtc.ERR_CORRUPT                 # frequency table sum
    bad = bytearray(data); bad[pc["layout"].n_sections * 0 + 256] = 9  # a width above max_bits
    assert status(bad) == kvtc.ERR_CORRUPT
    # flipped stream words of the first tile: the final-state and word-count
    # checks catch nearly all of them
    assert int(pc["modes"][0]) == 0
    bits0 = pc["bits"][0]
    tb = sum(2 * (1 << orc.sym_bits(int(b))) for b in bits0 if orc.sym_bits(int(b)))
    tb = (tb + 3) // 4 * 4
    ntiles = -(-min(cfg["chunk_tokens"], pc["layout"].T_mid) // cfg["tile_tokens"])
    nw0 = int(np.frombuffer(data[rec + tb: rec + tb + 4], np.uint32)[0])
    w0 = rec + tb + 4 * ntiles + 4 * cfg["rans_lanes"]
    rng = np.random.default_rng(0)
    caught = 0
    for pos in rng.integers(w0, w0 + 2 * nw0, 12):
        bad = bytearray(data); bad[pos] ^= 0x5A
        caught += status(bad) == kvtc.ERR_CORRUPT
    assert caught == 12  # the record checksum catches every one
    # every byte of the container is under a checksum: the side information
    # (zero points and scales), the raw windows, the directory, the records
    # and the checksum field itself; the oracle refuses the same damage
    h = np.frombuffer(data[:256], np.uint8)
    side_off, raw_off, raw_bytes, dir_off, chunks_off = (
        int(h[a: a + 8].view(np.uint64)[0]) for a in (120, 136, 144, 152, 160))
    regions = [(side_off + 128, raw_off), (raw_off, raw_off + raw_bytes), (dir_off, chunks_off),
               (chunks_off, len(data)), (200, 216)]
    for a, b in regions:
        for pos in rng.integers(a, b, 3):
            bad = bytearray(data); bad[int(pos)] ^= 1 << int(rng.integers(0, 8))
            assert status(bad) == kvtc.ERR_CORRUPT, (a, b, int(pos))
            assert orc.decode_status(cfg, bytes(bad), basis, T) == orc.ERR_CORRUPT
    d0 = orc_dir_off(data)
    for mode in (1, 2):  # a record mode that disagrees with the record, or none at all
        bad = bytearray(data); bad[d0 + 12: d0 + 16] = np.uint32(mode).tobytes()
        assert status(bad) == kvtc.ERR_CORRUPT
        assert orc.decode_status(cfg, bytes(bad), basis, T) == orc.ERR_CORRUPT
    # a directory offset near 2^64 (16-byte aligned) would wrap an
    # offset + size bound; it is refused before the record is read
    bad = bytearray(data)
    bad[orc_dir_off(data): orc_dir_off(data) + 8] = np.uint64(2 ** 64 - 256).tobytes()
    assert status(bad) == kvtc.ERR_CORRUPT
    assert orc.decode_status(cfg, bytes(bad), basis, T) == orc.ERR_CORRUPT
    # the oracle agrees on the same damage
    bad = bytearray(data); bad[rec + 5] ^= 0x10
    assert orc.decode_status(cfg, bytes(bad), basis, T) == orc.ERR_CORRUPT


def orc_dir_off(data):
    """Byte offset of the chunk directory, from the container header."""
    return int(np.frombuffer(data[152:160], np.uint64)[0])


def test_short_output_reports_capacity():
    """An output with room for the header, directory and raw windows but not
    for every record: the device reports KVTC_ERR_CAPACITY and no container
    size, and writes nothing past the capacity it was given."""
    cfg, T, K, V, k, v, basis, plan = _setup("llama3_8b", tokens=1200, layers=1)
    data, st, ws = _encode(plan, K, V)
    assert st == kvtc.OK
    pc = orc.parse_container(data, cfg, T)
    chunks_off = int(pc["chunks_off"])
    assert len(data) > chunks_off + 64
    for cap in (chunks_off, (chunks_off + len(data)) // 2, len(data) - 1):
        buf = torch.full((len(data) + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
        ws2 = plan.workspace(T)
        plan.encode_async(K, V, buf[:cap], ws2)
        torch.cuda.synchronize()
        n, st2 = plan.result(ws2)
        assert st2 == kvtc.ERR_CAPACITY, (cap, st2)
        assert n == 0
        assert bool((buf[cap:] == 0xA5).all()), cap
    # the full capacity still encodes the same container
    buf = torch.full((len(data),), 0xA5, dtype=torch.uint8, device="cuda")
    ws3 = plan.workspace(T)
    plan.encode_async(K, V, buf, ws3)
    torch.cuda.synchronize()
    n, st3 = plan.result(ws3)
    assert st3 == kvtc.OK and n == len(data)
    assert buf.cpu().numpy().tobytes() == data


def test_nonfinite_middle_is_reported():
    cfg, T, K, V, k, v, basis, plan = _setup("llama3_8b", tokens=600, layers=1)
    K2 = K.clone()
    K2[0, 3, 200, 7] = float("nan")
    _, st, _ = _encode(plan, K2, V)
    assert st == kvtc.ERR_NONFINITE
    K3 = K.clone()
    K3[0, 1, 2, 5] = float("inf")  # sink window: passes through
    K3[0, 2, T - 3, 6] = float("nan")  # recent window
    data, st, _ = _encode(plan, K3, V)
    assert st == kvtc.OK
    kd, vd, st = plan.decode(torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda(), T, kvtc.BF16)
    assert st == kvtc.OK
    assert torch.isinf(kd[0, 1, 2, 5]) and torch.isnan(kd[0, 2, T - 3, 6])


def test_bf16_output_within_one_ulp():
    cfg, T, K, V, k, v, basis, plan = _setup("llama3_8b", tokens=800, layers=1)
    data, st, _ = _encode(plan, K, V)
    t = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
    k32, v32, _ = plan.decode(t, T, kvtc.FP32)
    k16, v16, _ = plan.decode(t, T, kvtc.BF16)
    assert torch.equal(k32.to(torch.bfloat16), k16) and torch.equal(v32.to(torch.bfloat16), v16)
    ko, vo = orc.decode(cfg, data, basis, T, orc.BF16)
    for g, o, src in ((k16, ko, k), (v16, vo, v)):
        gf = g.float().cpu().numpy().astype(np.float64)
        of = orc.bf16_bits_to_f32(o).reshape(o.shape).astype(np.float64)
        rms = parity.channel_rms(orc.bf16_bits_to_f32(src).reshape(src.shape))
        # the fp32 results agree to 1e-4 RMS; rounding each to bf16 adds at most one bf16 ulp
        ulp = np.spacing(np.maximum(np.abs(gf), np.abs(of)).astype(np.float32)).astype(np.float64) * 2 ** 16
        assert np.all(np.abs(gf - of) <= 1e-4 * rms + ulp)


# --------------------------------------------------------------------------- full size

def _full_size_sampled(name, fixed_secs, n_random, ratio_range, seed=7, **over):
    """A workload at its full size in the benchmark's launch configuration:
    the whole cache is coded and decoded on the GPU and the oracle checks
    sampled sections (statistics, widths, side information, coefficients,
    codes, rANS records and the decoded middle)."""
    w = synth.WORKLOADS[name]
    K, V = synth.generate(w, device="cuda")
    T = K.shape[2]
    cfg = synth.oracle_config(w, **over)
    lo = orc.layout(cfg, T)
    basis_t = fit_pca_basis(K, V, cfg, lo.mid_begin, lo.mid_end) if cfg["transform"] == 0 else None
    basis = None if basis_t is None else basis_t.cpu().numpy()
    plan = kvtc.Plan(cfg, basis_t, max_tokens=T)
    ws = plan.workspace(T)
    data_t, st = plan.encode(K, V, ws)
    assert st == kvtc.OK, kvtc.STATUS[st]
    data = data_t.cpu().numpy().tobytes()
    stats = plan.section_stats(ws, T, lo.n_sections)
    k, v = synth.to_numpy_bits(K), synth.to_numpy_bits(V)
    rng = np.random.default_rng(seed)
    secs = sorted(set(fixed_secs + [int(x) for x in rng.integers(0, lo.n_sections, n_random)]))
    kd, vd, st = plan.decode(data_t, T, kvtc.FP32)
    assert st == kvtc.OK, kvtc.STATUS[st]
    H = w.kv_heads
    report = []
    for u in secs:
        coef, _ = plan.coeffs(K, V, u, u + 1, lo.T_mid)
        parity.compare_section(orc, cfg, T, k, v, basis, data, stats, u,
                               gpu_coef=coef[0].cpu().numpy(), report=report)
        del coef
        mid_ref = orc.decode_sections(cfg, data, basis, u, u + 1, lo.T_mid)[0]
        l, s, h = u // (2 * H), (u // H) % 2, u % H
        src = k if s == 0 else v
        srcf = orc.bf16_bits_to_f32(src[l, h]).reshape(T, -1)
        rms = np.sqrt((srcf.astype(np.float64) ** 2).mean(axis=0))
        got = (kd if s == 0 else vd)[l, h, lo.mid_begin: lo.mid_end].cpu().numpy()
        parity.compare_decode(got, mid_ref, rms[None, :])
        # raw windows of the sampled head restored bit-exactly
        srcw = orc.bf16_bits_to_f32(src[l, h]).reshape(T, -1)
        dec = (kd if s == 0 else vd)[l, h]
        assert np.array_equal(srcw[: lo.s0], dec[: lo.s0].cpu().numpy())
        assert np.array_equal(srcw[lo.mid_end:], dec[lo.mid_end:].cpu().numpy())
    codes = sum(r["codes"] for r in report)
    assert sum(r["boundary_codes"] for r in report) <= parity.BOUNDARY_FRACTION * codes
    ratio = (K.numel() + V.numel()) * 2 / len(data)
    assert ratio_range[0] < ratio < ratio_range[1], ratio


def test_llama3_8b_full_size_sampled():
    """32 layers x 8 heads x 4096 tokens bf16 at 2 bits/comp."""
    _full_size_sampled("llama3_8b", [0, 7, 8, 255, 256, 511], 4, (5.0, 10.0))


@pytest.mark.timeout(900)
def test_llama3_8b_full_size_every_section_decoded():
    """The full Llama-3-8B-shaped cache in the benchmark's launch configuration:
    every one of its 512 sections, decoded on the GPU, is within the decode
    bound of the oracle's decode of the same container, and the raw windows
    come back bit-exactly."""
    w = synth.WORKLOADS["llama3_8b"]
    K, V = synth.generate(w, device="cuda")
    T = K.shape[2]
    cfg = synth.oracle_config(w)
    lo = orc.layout(cfg, T)
    basis_t = fit_pca_basis(K, V, cfg, lo.mid_begin, lo.mid_end)
    basis = basis_t.cpu().numpy()
    plan = kvtc.Plan(cfg, basis_t, max_tokens=T)
    data_t, st = plan.encode(K, V, plan.workspace(T))
    assert st == kvtc.OK, kvtc.STATUS[st]
    data = data_t.cpu().numpy().tobytes()
    kd, vd, st = plan.decode(data_t, T, kvtc.FP32)
    assert st == kvtc.OK, kvtc.STATUS[st]
    kd, vd = kd.cpu().numpy(), vd.cpu().numpy()
    k, v = synth.to_numpy_bits(K), synth.to_numpy_bits(V)
    del K, V, data_t
    ref = orc.decode_sections(cfg, data, basis, 0, lo.n_sections, lo.T_mid)
    L, H = w.layers, w.kv_heads
    for l in range(L):
        for s, (src, dec) in enumerate(((k, kd), (v, vd))):
            srcf = orc.bf16_bits_to_f32(src[l]).reshape(src.shape[1:])  # [H, T, D]
            rms = np.sqrt((srcf.astype(np.float64) ** 2).mean(axis=1))  # [H, D]
            for h in range(H):
                u = (l * 2 + s) * H + h
                parity.compare_decode(dec[l, h, lo.mid_begin: lo.mid_end], ref[u], rms[h][None, :])
            assert np.array_equal(srcf[:, : lo.s0], dec[l, :, : lo.s0])
            assert np.array_equal(srcf[:, lo.mid_end:], dec[l, :, lo.mid_end:])


def test_qwen3_32b_full_size_sampled():
    """64 layers x 8 heads x 32768 tokens bf16 at 2 bits/comp (the 8.6 GB
    cache); first, last and layer-boundary sections plus random ones."""
    _full_size_sampled("qwen3_32b", [0, 15, 16, 1023], 2, (6.0, 12.0), seed=3)


@pytest.mark.timeout(900)
def test_hadamard_long_full_size_sampled():
    """32 layers x 8 heads x 131072 tokens bf16 on the Hadamard path (keys 4
    bits, values 2 bits); WHT coefficients and codes are exact."""
    _full_size_sampled("hadamard_long", [0, 8, 511], 2, (4.0, 10.0), seed=5)
