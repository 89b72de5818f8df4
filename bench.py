#!/usr/bin/env python
"""Benchmark: KVTC-style encode + decode of a KV cache on one MI355X.

One step = kvtc_encode + kvtc_decode of the whole cache (every phase of the
coded path) with inputs resident in HBM.  Default workload: a
Llama-3-8B-shaped cache, 32 layers x 8 KV heads x 4096 tokens x head_dim 128,
bf16, 2 bits per component, sink 4 / recent 128, per-layer PCA basis.  The
cache is synthetic (seeded low-rank latent + noise, RoPE on keys; see
tensor_compression_amd/synth.py) and the basis is calibrated on it before
timing.

Prints one JSON line.  `value` is raw KV bytes / (encode + decode time) in
GB/s.  `roofline` is the dominant kernel's algorithmic bytes per launch over
its HIP-event-timed average duration against the 8 TB/s HBM3E peak;
`path_roofline` does the same for the whole step (algorithmic bytes
2 x (raw + container)).  `cpu_baseline` times the CPU oracle on a bounded
slice of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "encode+decode GB/s of raw bf16 KV at 2 bits/comp; ratio; % HBM roofline"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA of the MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--bits", type=float, default=None, help="bits per component (K and V)")
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--chunk-tokens", type=int, default=4096)
    ap.add_argument("--tile-tokens", type=int, default=256)
    ap.add_argument("--alloc-scope", type=int, default=0,
                    help="0: each section spends its own bit budget; 1: one budget over all sections")
    ap.add_argument("--cpu-layers", type=int, default=8,
                    help="layers of the workload the CPU oracle baseline codes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-phase event pass")
    ap.add_argument("--seqs", type=int, default=None, help="sequences of a paged workload")
    ap.add_argument("--sq", choices=("block", "kivi"), default=None,
                    help="time the scalar quantisers on gauge coordinates instead of the codec")
    ap.add_argument("--sq-group", type=int, default=16, help="channels per range (block, KIVI values)")
    ap.add_argument("--sq-tile", type=int, default=16, help="tokens per range (block, KIVI keys)")
    ap.add_argument("--sq-bits", type=int, default=4, help="bits per coefficient (keys and values)")
    ap.add_argument("--pq", action="store_true",
                    help="time the TTAS-X2 value path (two-level product quantisation) instead of the codec")
    ap.add_argument("--pq-k1", type=int, default=256)
    ap.add_argument("--pq-k2", type=int, default=64)
    ap.add_argument("--pq-outliers", type=int, default=64, help="outliers per (layer, head) and block")
    ap.add_argument("--pq-block", type=int, default=1024, help="tokens per outlier block")
    ap.add_argument("--ceilings", action="store_true",
                    help="time plain read, write and copy kernels over 520 MB (the practical HBM ceilings) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy kernel of known size (for scaling HBM counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a per-kernel table from a rocprofv3 --stats output folder and exit")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-kernel mean counters from a rocprofv3 --pmc csv folder and exit")
    ap.add_argument("--traffic-table", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the per-phase HBM traffic table from FETCH_SIZE and WRITE_SIZE "
                         "rocprofv3 --pmc csv folders of a --copy-calibration run and exit")
    return ap.parse_args()


# Phase -> (kernels, sources they are built from).  The roofline's `traffic`
# is taken from the committed counter summary only while these sources are
# unchanged since the counters were read.
PHASE_KERNELS = {
    "enc_stats": (("k_unrope128", "k_enc128"), ("kernels_encode.hip",)),
    "enc_quant_pack": (("k_quant128",), ("kernels_quant.hip",)),
    "rans_encode": (("k_rans_enc_recs",), ("kernels_rans.hip",)),
    "assemble": (("k_scan", "k_copy_records"), ("kernels_rans.hip",)),
    "enc_checksum": (("k_csum_part", "k_csum_final"), ("kernels_rans.hip",)),
    "dec_checksum": (("k_csum_part", "k_csum_final"), ("kernels_rans.hip",)),
    "rans_decode": (("k_rans_dec_recs",), ("kernels_rans.hip",)),
    "dec_transform": (("k_dec_pca128",), ("kernels_decode.hip",)),
    # scalar quantisers on gauge coordinates (bench.py --sq)
    "sq_encode": (("k_sq_clear", "k_sq_enc128"), ("kernels_sq.hip",)),
    "sq_decode": (("k_sq_dec128",), ("kernels_sq.hip",)),
    # TTAS-X2 value path (bench.py --pq)
    "pq_encode": (("k_pq_prep", "k_pq_enc", "k_pq_merge"), ("kernels_pq.hip",)),
    "pq_decode": (("k_pq_prep", "k_pq_dec"), ("kernels_pq.hip",)),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama3_8b.md")
TRAFFIC_FILE_SQ = os.path.join(ROOT, "profiles", "hbm_traffic_sq_llama3_8b.md")
TRAFFIC_FILE_PQ = os.path.join(ROOT, "profiles", "hbm_traffic_pq_llama3_8b.md")
# plain VALU lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
COPY_CAL_BYTES = 1 << 28  # fp32 elements read and written by the calibration copy


def source_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in tuple(files) + ("kvtc_internal.h",):
        with open(os.path.join(ROOT, "tensor_compression_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(phase, path=TRAFFIC_FILE):
    """HBM bytes per launch of the phase's kernels from the committed counter
    summary (rows `| phase | ... | bytes | digest |`), or None when absent or
    taken on different kernel sources."""
    if phase not in PHASE_KERNELS or not os.path.exists(path):
        return None
    want = source_digest(PHASE_KERNELS[phase][1])
    with open(path) as fh:
        for line in fh:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 6 and cells[0] == phase:
                try:
                    nbytes = float(cells[4])
                except ValueError:
                    return None
                return nbytes if cells[5] == want else None
    return None


def _short_kernel(name: str) -> str:
    n = name.split("(")[0].replace("void ", "")
    return n.replace("kvtc::", "")


def summarize_trace(d):
    """Per-kernel calls / mean / min / max (us) from rocprofv3 --stats."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((_short_kernel(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                             float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda r: -r[1] * r[2])
    print("| kernel | calls | avg (us) | min (us) | max (us) | % time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r[0]} | {r[1]} | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.1f} | {r[5]:.1f} |")


def pmc_means(d, counter):
    """Mean of `counter` per dispatch, per kernel, from a rocprofv3 --pmc csv folder."""
    import collections
    import csv
    import glob
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    per[_short_kernel(r["Kernel_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def traffic_table(fetch_dir, write_dir):
    """Per-phase HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the phase's kernels, each scaled by the ratio of the known
    bytes of the calibration copy to what the same counter read for it."""
    fetch, write = pmc_means(fetch_dir, "FETCH_SIZE"), pmc_means(write_dir, "WRITE_SIZE")
    cal = [k for k in fetch if "bitwise_not" in k]
    if not cal or cal[0] not in write:
        raise SystemExit("no calibration copy kernel in the counter folders (run with --copy-calibration)")
    known_kib = COPY_CAL_BYTES / 1024.0
    ff, fw = known_kib / fetch[cal[0]], known_kib / write[cal[0]]
    print(f"Calibration: the copy kernel moves {COPY_CAL_BYTES} B each way; FETCH_SIZE read "
          f"{fetch[cal[0]]:.1f} KiB (factor {ff:.4f}), WRITE_SIZE read {write[cal[0]]:.1f} KiB "
          f"(factor {fw:.4f}).")
    print()
    print("| kernel | FETCH_SIZE (KiB/dispatch) | WRITE_SIZE (KiB/dispatch) |")
    print("|---|---|---|")
    for k in sorted(fetch):
        if k.startswith("k_"):
            print(f"| {k} | {fetch[k]:.1f} | {write.get(k, 0.0):.1f} |")
    print()
    print("| phase | kernels | fetch bytes | write bytes | traffic bytes | sources digest |")
    print("|---|---|---|---|---|---|")
    for ph, (kernels, files) in PHASE_KERNELS.items():
        names = [k for k in fetch if any(k == b or k.startswith(b + "<") for b in kernels)]
        if not names:
            continue
        fb = sum(fetch[k] for k in names) * ff * 1024
        wb = sum(write.get(k, 0.0) for k in names) * fw * 1024
        print(f"| {ph} | {' + '.join(sorted(names))} | {fb:.0f} | {wb:.0f} | {fb + wb:.0f} | "
              f"{source_digest(files)} |")


def summarize_pmc(d):
    """Mean counter value per dispatch, per kernel, from rocprofv3 --pmc csv."""
    import collections
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                acc[(_short_kernel(r["Kernel_Name"]), r["Counter_Name"])][r["Dispatch_Id"]] += \
                    float(r["Counter_Value"])
    print("| kernel | counter | dispatches | mean per dispatch |")
    print("|---|---|---|---|")
    for (k, c), per in sorted(acc.items()):
        print(f"| {k} | {c} | {len(per)} | {sum(per.values()) / len(per):.6g} |")


def copy_calibration():
    """A plain copy-like kernel of known traffic: out = ~x over 2^28 bytes of
    int32, read once and written once (torch's bitwise_not kernel, which
    nothing else here launches)."""
    import torch
    x = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.bitwise_not(x, out=y)
    torch.cuda.synchronize()


def ceilings():
    """Practical HBM rates of plain torch kernels over 520 MiB (about the bytes
    of one pass over the Llama-3-8B middle): a fill (write) and a copy (read +
    write, both counted).  Printed as a markdown table."""
    import torch
    n = 520 << 20
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    cases = [("write (fill_)", n, lambda: y.fill_(7)),
             ("copy (copy_, read + write)", 2 * n, lambda: y.copy_(x))]
    print("| kernel | bytes moved | us | TB/s |")
    print("|---|---|---|---|")
    for name, moved, fn in cases:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            fn()
        b.record()
        b.synchronize()
        us = a.elapsed_time(b) / 20 * 1e3
        print(f"| {name} | {moved / 1e6:.0f} MB | {us:.1f} | {moved / us / 1e6:.2f} |")


def layout(cfg, T):
    s0 = min(cfg["sink_tokens"], T)
    mid_end = max(s0, T - cfg["recent_tokens"])
    return s0, mid_end


def packed_bytes_total(bits, cfg, T_mid):
    """Packed payload bytes of all sections from their bit widths [n_sec, D]."""
    import numpy as np
    ct, tt = cfg["chunk_tokens"], cfg["tile_tokens"]
    tiles = []
    for c0 in range(0, T_mid, ct):
        n = min(ct, T_mid - c0)
        for t0 in range(0, n, tt):
            tiles.append(min(tt, n - t0))
    total = 0
    b = bits.astype(np.int64)
    for m in set(tiles):
        cnt = tiles.count(m)
        total += cnt * int((4 * ((m * b + 31) // 32) * (b > 0)).sum())
    return total


def cpu_baseline(w, cfg, K, V, basis, layers):
    """The oracle as it stands, single-threaded, on the first `layers` layers."""
    import numpy as np

    import oracle
    from tensor_compression_amd import synth
    layers = max(1, min(layers, K.shape[0]))
    k = synth.to_numpy_bits(K[:layers])
    v = synth.to_numpy_bits(V[:layers])
    b = basis[:layers].cpu().numpy()
    c1 = dict(cfg, layers=layers)
    oracle.lib()
    t0 = time.perf_counter()
    data = oracle.encode(c1, k, v, b)
    t1 = time.perf_counter()
    oracle.decode(c1, data, b, K.shape[2], oracle.BF16)
    t2 = time.perf_counter()
    raw = k.nbytes + v.nbytes
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": raw / (t2 - t0) / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "host_cpus": os.cpu_count(), "host_cpu_model": model,
        "sample": f"{layers} of {K.shape[0]} layers ({layers * 2 * K.shape[1]} sections, "
                  f"{raw} raw bytes): oracle encode {t1 - t0:.2f} s + decode {t2 - t1:.2f} s, "
                  "single thread, throughput extrapolates linearly in sections",
        "encode_s": t1 - t0, "decode_s": t2 - t1,
    }


def run_paged(args, w):
    """The paged ragged batch: one step = kvtc_encode_paged + kvtc_decode_paged
    of the whole batch (decode writes back into the same pools, which a
    second copy of would not fit next to the workspace)."""
    import numpy as np
    import torch

    import oracle
    from tensor_compression_amd import kvtc, synth
    from tensor_compression_amd.calibrate import fit_pca_basis

    n_seqs = args.seqs if args.seqs is not None else w.n_seqs
    lens = synth.ragged_lengths(w, n_seqs)
    over = dict(chunk_tokens=args.chunk_tokens, tile_tokens=args.tile_tokens, alloc_scope=args.alloc_scope)
    if args.bits is not None:
        over.update(bits_k=args.bits, bits_v=args.bits)
    kp, vp, table, lens = synth.generate_paged(w, device="cuda", lengths=lens, layers=args.layers)
    L, P, H, _, D = kp.shape
    cfg = synth.oracle_config(w, layers=L, **over)
    # shared per-layer basis, fitted on the longest of the first eight sequences
    z0 = int(np.argmax(lens[:8]))
    Kz, Vz = synth.gather_paged(kp, table, z0, lens[z0]), synth.gather_paged(vp, table, z0, lens[z0])
    s0, mid_end = layout(cfg, lens[z0])
    basis = fit_pca_basis(Kz, Vz, cfg, s0, mid_end)
    del Kz, Vz
    plan = kvtc.Plan(cfg, basis, max_tokens=max(lens))
    ws_bytes, cap = plan.sizes_paged(lens)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    # the worst-case container capacity assumes every rANS stream expands; when
    # that does not fit next to the pools and the workspace, take what is free
    # (an encode that overflows reports KVTC_ERR_CAPACITY)
    free = torch.cuda.mem_get_info()[0] - (2 << 30)
    cap = int(min(cap, free))
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    table_d = table.cuda()
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")

    def step():
        plan.encode_paged_async(kp, vp, table_d, lens, lens_d, out, ws)
        plan.decode_paged_async(out, cap, kp, vp, table_d, lens, lens_d, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    plan.encode_paged_async(kp, vp, table_d, lens, lens_d, out, ws)
    torch.cuda.synchronize()
    nbytes, st = plan.result(ws)
    if st != kvtc.OK:
        raise SystemExit(f"device status: {kvtc.STATUS[st]}")
    phases = {}
    if not args.no_profile:
        plan.profile(True)
        for _ in range(max(1, min(args.steps, 3))):
            plan.encode_paged_async(kp, vp, table_d, lens, lens_d, out, ws)
            for name, ms in plan.profile_read():
                phases.setdefault(name, []).append(ms)
            plan.decode_paged_async(out, cap, kp, vp, table_d, lens, lens_d, ws)
            for name, ms in plan.profile_read():
                phases.setdefault(name, []).append(ms)
        plan.profile(False)
    ph_ms = {k: float(np.mean(v)) for k, v in phases.items()}
    tok = int(sum(lens))
    raw = tok * L * H * D * 2 * kp.element_size()
    res = {
        "metric": METRIC + " (paged ragged batch)",
        "value": raw / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {n_seqs} sequences, lengths U[{w.min_len}, {w.max_len}] ({tok} tokens), "
                        f"16-token pages, {L} layers x {H} KV heads x head_dim {D}, bf16, {cfg['bits_k']:g} "
                        f"bits/comp, shared per-layer PCA basis",
            "sequences": n_seqs, "tokens": tok, "layers": L, "kv_heads": H, "head_dim": D,
            "pool_pages": P, "bits_per_component": cfg["bits_k"],
        },
        "raw_bytes": raw, "container_bytes": nbytes, "compression_ratio": raw / nbytes,
        "bits_per_value": 8.0 * nbytes / (raw / kp.element_size()),
        "phases_ms": ph_ms,
        "path_roofline": {
            "bound": "hbm", "algorithmic_bytes": 2 * (raw + nbytes),
            "achieved": 2 * (raw + nbytes) / (ms_per_step * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": 2 * (raw + nbytes) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        },
        "workspace_bytes": ws_bytes, "container_capacity": cap, "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        # the oracle on the first two layers of the first sequence
        T0 = lens[0]
        k = synth.to_numpy_bits(synth.gather_paged(kp[:2], table, 0, T0))
        v = synth.to_numpy_bits(synth.gather_paged(vp[:2], table, 0, T0))
        c1 = dict(cfg, layers=2)
        b = basis[:2].cpu().numpy()
        oracle.lib()
        t_a = time.perf_counter()
        data = oracle.encode(c1, k, v, b)
        t_b = time.perf_counter()
        oracle.decode(c1, data, b, T0, oracle.BF16)
        t_c = time.perf_counter()
        res["cpu_baseline"] = {
            "value": (k.nbytes + v.nbytes) / (t_c - t_a) / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"sequence 0 ({T0} tokens), layers 0-1 of {L}: oracle encode {t_b - t_a:.2f} s + decode "
                      f"{t_c - t_b:.2f} s, single thread; the decode overwrote the pools, so the sample is the "
                      "reconstruction of the first step",
        }
    print(json.dumps(res), flush=True)


def run_sq(args, w):
    """The scalar quantisers on gauge coordinates: one step = kvtc_sq_encode
    + kvtc_sq_decode of the whole cache with a grouped random gauge (g = 16)
    as the basis.  Each call is one launch (plus a one-word status clear
    before the encoder), timed with HIP events on the launch stream."""
    import numpy as np
    import torch

    from tensor_compression_amd import kvtc, synth
    from tensor_compression_amd.calibrate import grouped_random_gauge

    K, V = synth.generate(w, device="cuda", tokens=args.tokens, layers=args.layers)
    L, H, T, D = K.shape
    cfg = synth.oracle_config(w, layers=L)
    basis = grouped_random_gauge(L, D, 16, 0.5, seed=1)
    B = basis.numpy()
    plan = kvtc.Plan(cfg, basis, max_tokens=T)
    sq = dict(kind=kvtc.SQ_BLOCK if args.sq == "block" else kvtc.SQ_KIVI, group=args.sq_group,
              tile=args.sq_tile, bits_k=args.sq_bits, bits_v=args.sq_bits)
    nb, nr = plan.sq_sizes(sq, T)
    codes = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ranges = torch.empty((nr, 2), dtype=torch.float32, device="cuda")
    status = torch.zeros(4, dtype=torch.int32, device="cuda")
    kd, vd = torch.empty_like(K), torch.empty_like(V)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def step(times=None):
        ev[0].record(stream)
        plan.sq_encode_async(sq, K, V, codes, ranges, status, stream)
        ev[1].record(stream)
        plan.sq_decode_async(sq, codes, ranges, T, kd, vd, kvtc.BF16, stream)
        ev[2].record(stream)
        if times is not None:
            torch.cuda.synchronize()
            times.append((ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.sq_encode_async(sq, K, V, codes, ranges, status, stream)
        plan.sq_decode_async(sq, codes, ranges, T, kd, vd, kvtc.BF16, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    if int(status[0].item()) != 0:
        raise SystemExit(f"device status {int(status[0].item())}")
    times = []
    for _ in range(args.steps):
        step(times)
    t_enc = float(np.mean([t[0] for t in times]))
    t_dec = float(np.mean([t[1] for t in times]))
    raw = (K.numel() + V.numel()) * K.element_size()
    stored = nb + 8 * nr
    alg = {"sq_encode": raw + stored, "sq_decode": stored + raw}
    ms = {"sq_encode": t_enc, "sq_decode": t_dec}
    dom = max(ms, key=lambda k: ms[k])
    ach = alg[dom] / (ms[dom] * 1e-3) / 1e9

    def nrmse(a, b):
        a, b = a.float(), b.float()
        return math.sqrt(float(((a - b) ** 2).sum()) / max(float((a ** 2).sum()), 1e-300))

    res = {
        "metric": f"scalar-quantiser ({args.sq}) encode+decode GB/s of raw bf16 KV",
        "value": raw / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {L} layers x {H} KV heads x {T} tokens x head_dim {D}, bf16, "
                        f"{args.sq} quantiser, {args.sq_bits} bits, group {args.sq_group}, tile {args.sq_tile}, "
                        "grouped random gauge g = 16",
            "layers": L, "kv_heads": H, "tokens": T, "head_dim": D, "sq": sq,
        },
        "raw_bytes": raw, "code_bytes": nb, "range_bytes": 8 * nr, "compression_ratio": raw / stored,
        "bits_per_value": 8.0 * stored / (K.numel() + V.numel()),
        "nrmse_k": nrmse(K, kd), "nrmse_v": nrmse(V, vd),
        "phases_ms": ms,
        "roofline": {"bound": "hbm", "kernel": dom, "kernels": ["k_sq_enc128" if dom == "sq_encode" else "k_sq_dec128"],
                     "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": traffic_from_profile(dom, TRAFFIC_FILE_SQ), "algorithmic_bytes": alg[dom],
                     "avg_ms": ms[dom]},
        "path_roofline": {"bound": "hbm", "algorithmic_bytes": 2 * (raw + stored),
                          "achieved": 2 * (raw + stored) / (ms_per_step * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s",
                          "frac": 2 * (raw + stored) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "mfma_roofline": {k: {"flops": 2 * D * (K.numel() + V.numel()),
                              "achieved_tflops": 2 * D * (K.numel() + V.numel()) / (ms[k] * 1e-3) / 1e12,
                              "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                              "frac": 2 * D * (K.numel() + V.numel()) / (ms[k] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
                          for k in ms},
    }
    if not args.no_cpu_baseline:
        import oracle
        nl = max(1, min(2, L))
        k = synth.to_numpy_bits(K[:nl])
        v = synth.to_numpy_bits(V[:nl])
        c1 = dict(cfg, layers=nl)
        oracle.lib()
        t_a = time.perf_counter()
        cg, rg = oracle.sq_encode(c1, sq, k, v, B[:nl])
        t_b = time.perf_counter()
        oracle.sq_decode(c1, sq, cg, rg, T, B[:nl])
        t_c = time.perf_counter()
        res["cpu_baseline"] = {
            "value": (k.nbytes + v.nbytes) / (t_c - t_a) / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{nl} of {L} layers: oracle encode {t_b - t_a:.2f} s + decode {t_c - t_b:.2f} s, "
                      "single thread",
        }
    print(json.dumps(res), flush=True)


def run_pq(args, w):
    """The TTAS-X2 value path: one step = kvtc_pq_encode + kvtc_pq_decode of
    the whole cache's values with k-means codebooks fitted on them before
    timing (keys take the codec's 4-bit path, not timed here).  Each call is a
    prep launch plus the encoder and the outlier merge (or the decoder),
    timed with HIP events on the launch stream."""
    import numpy as np
    import torch

    from tensor_compression_amd import calibrate, kvtc, synth

    K, V = synth.generate(w, device="cuda", tokens=args.tokens, layers=args.layers)
    del K
    L, H, T, D = V.shape
    cfg = synth.oracle_config(w, layers=L, transform=1, bits_k=4.0, bits_v=2.0, wht_keys=0)
    plan = kvtc.Plan(cfg, None, max_tokens=T)
    pq = dict(sub_dim=8, k1=args.pq_k1, k2=args.pq_k2, outliers=args.pq_outliers, block_tokens=args.pq_block)
    cb1, cb2 = calibrate.train_pq_codebooks(V, pq, iters=6, seed=0)
    c1, c2 = cb1.cuda(), cb2.cuda()
    nb, ns, wb = plan.pq_sizes(pq, T)
    codes, rms, outl, ws = plan.pq_buffers(pq, T)
    ws_d = torch.empty_like(ws)
    status = torch.zeros(4, dtype=torch.int32, device="cuda")
    status_d = torch.zeros(4, dtype=torch.int32, device="cuda")
    vd = torch.empty_like(V)
    stream = torch.cuda.current_stream()

    def enc():
        plan.pq_encode_async(pq, c1, c2, V, codes, rms, outl, ws, status, stream)

    def dec():
        plan.pq_decode_async(pq, c1, c2, codes, rms, outl, T, vd, ws_d, status_d, kvtc.BF16, stream)

    for _ in range(args.warmup):
        enc()
        dec()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        enc()
        dec()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    if int(status[0].item()) or int(status_d[0].item()):
        raise SystemExit(f"device status {int(status[0].item())} / {int(status_d[0].item())}")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    te, td = [], []
    for _ in range(args.steps):
        ev[0].record(stream)
        enc()
        ev[1].record(stream)
        dec()
        ev[2].record(stream)
        torch.cuda.synchronize()
        te.append(ev[0].elapsed_time(ev[1]))
        td.append(ev[1].elapsed_time(ev[2]))
    ms = {"pq_encode": float(np.mean(te)), "pq_decode": float(np.mean(td))}
    raw = V.numel() * V.element_size()
    stored = nb + 4 * L * H * T + 8 * ns
    N = L * H * T
    # the search is VALU work: at least one fused score and one running
    # minimum per candidate centroid, per subvector and level
    ops = 2 * N * (D // 8) * (pq["k1"] + pq["k2"])
    ach = ops / (ms["pq_encode"] * 1e-3) / 1e12
    dec_bytes = stored + raw
    vf = V.float()
    nrmse_v = math.sqrt(float(((vf - vd.float()) ** 2).sum()) / max(float((vf ** 2).sum()), 1e-300))
    res = {
        "metric": "TTAS-X2 value path encode+decode GB/s of raw bf16 V",
        "value": raw / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": f"{w.name} values: {L} layers x {H} KV heads x {T} tokens x head_dim {D}, bf16, "
                        f"RMS + WHT + two-level PQ (8-channel subvectors, K1 {pq['k1']}, K2 {pq['k2']}), "
                        f"{pq['outliers']} outliers per head and {pq['block_tokens']} tokens, k-means codebooks",
            "layers": L, "kv_heads": H, "tokens": T, "head_dim": D, "pq": pq,
        },
        "raw_bytes": raw, "code_bytes": nb, "rms_bytes": 4 * N, "outlier_bytes": 8 * ns,
        "compression_ratio": raw / stored, "bits_per_value": 8.0 * stored / V.numel(), "nrmse_v": nrmse_v,
        "phases_ms": ms,
        "roofline": {"bound": "alu", "kernel": "pq_encode", "kernels": ["k_pq_enc"], "achieved": ach,
                     "peak": VALU_PEAK_TOPS, "unit": "T VALU op/s", "frac": ach / VALU_PEAK_TOPS,
                     "traffic": traffic_from_profile("pq_encode", TRAFFIC_FILE_PQ), "algorithmic_ops": ops,
                     "avg_ms": ms["pq_encode"]},
        "decode_roofline": {"bound": "hbm", "kernel": "pq_decode", "algorithmic_bytes": dec_bytes,
                            "achieved": dec_bytes / (ms["pq_decode"] * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": dec_bytes / (ms["pq_decode"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                            "traffic": traffic_from_profile("pq_decode", TRAFFIC_FILE_PQ)},
    }
    if not args.no_cpu_baseline:
        import oracle
        v1 = synth.to_numpy_bits(V[:1])
        c_one = dict(cfg, layers=1)
        oracle.lib()
        t_a = time.perf_counter()
        oc, orms, oo = oracle.pq_encode(c_one, pq, v1, cb1[:1].numpy(), cb2[:1].numpy())
        t_b = time.perf_counter()
        oracle.pq_decode(c_one, pq, oc, orms, oo, T, cb1[:1].numpy(), cb2[:1].numpy())
        t_c = time.perf_counter()
        res["cpu_baseline"] = {
            "value": v1.nbytes / (t_c - t_a) / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of {L} ({H} heads x {T} tokens of values): oracle encode {t_b - t_a:.2f} s + "
                      f"decode {t_c - t_b:.2f} s, single thread",
        }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.traffic_table:
        traffic_table(*args.traffic_table)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} (world size {world}) "
              "is not supported -- sections shard across GPUs without communication, see the "
              "design notes", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from tensor_compression_amd import kvtc, synth
    from tensor_compression_amd.calibrate import fit_pca_basis

    kvtc.lib()  # fail loudly if the HIP library is missing
    torch.cuda.init()
    if args.ceilings:
        ceilings()
        return
    if args.copy_calibration:
        copy_calibration()
    w = synth.WORKLOADS[args.workload]
    if args.sq:
        run_sq(args, w)
        return
    if args.pq:
        run_pq(args, w)
        return
    if w.n_seqs > 0:
        run_paged(args, w)
        return
    over = dict(chunk_tokens=args.chunk_tokens, tile_tokens=args.tile_tokens)
    if args.bits is not None:
        over.update(bits_k=args.bits, bits_v=args.bits)
    K, V = synth.generate(w, device="cuda", tokens=args.tokens, layers=args.layers)
    L, H, T, D = K.shape
    cfg = synth.oracle_config(w, layers=L, **over)
    s0, mid_end = layout(cfg, T)
    basis = fit_pca_basis(K, V, cfg, s0, mid_end) if cfg["transform"] == 0 else None
    plan = kvtc.Plan(cfg, basis, max_tokens=T)
    ws_bytes, cap = plan.sizes(T)
    ws_e = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    kd = torch.empty_like(K)
    vd = torch.empty_like(V)
    out_dtype = kvtc.BF16 if K.dtype == torch.bfloat16 else kvtc.FP32
    # two copies of the cache at different addresses, coded by turns: no step
    # finds its input left in the 256 MB memory-side cache by the step before
    # (the decoder streams its rows past that cache), as with a fresh cache
    inputs = ((K, V), (K.clone(), V.clone()))
    turn = [0]

    def next_input():
        kv = inputs[turn[0] & 1]
        turn[0] += 1
        return kv

    def step():
        k_in, v_in = next_input()
        plan.encode_async(k_in, v_in, out, ws_e)
        plan.decode_async(out, cap, T, kd, vd, ws_d, out_dtype)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    nbytes, st_e = plan.result(ws_e)
    refined = plan.exact_recomputed(ws_e)
    _, st_d = plan.result(ws_d)
    if st_e != kvtc.OK or st_d != kvtc.OK:
        raise SystemExit(f"device status: encode {kvtc.STATUS[st_e]}, decode {kvtc.STATUS[st_d]}")

    raw = (K.numel() + V.numel()) * K.element_size()
    nvals = K.numel() + V.numel()

    # per-phase HIP-event timing, encode and decode of every step separately
    phases = {}
    if not args.no_profile:
        plan.profile(True)
        for _ in range(args.steps):
            k_in, v_in = next_input()
            plan.encode_async(k_in, v_in, out, ws_e)
            for name, ms in plan.profile_read():
                phases.setdefault(name, []).append(ms)
            plan.decode_async(out, cap, T, kd, vd, ws_d, out_dtype)
            for name, ms in plan.profile_read():
                phases.setdefault(name, []).append(ms)
        plan.profile(False)
    ph_ms = {k: float(np.mean(v)) for k, v in phases.items()}
    t_enc = sum(ph_ms.get(k, 0.0) for k in ("copy_raw", "enc_stats", "enc_alloc", "enc_quant_pack",
                                             "rans_encode", "assemble", "enc_checksum"))
    t_dec = sum(ph_ms.get(k, 0.0) for k in ("dec_check", "dec_checksum", "rans_decode", "dec_transform",
                                             "copy_raw_out"))

    # container accounting from the side records (bits) and the header
    blob_head = out[: 256].cpu().numpy()
    chunks_off = int(blob_head[160:168].view(np.uint64)[0])
    side = out[256: 256 + L * 2 * H * 9 * D].cpu().numpy().reshape(L * 2 * H, 9 * D)
    bits = side[:, :D]
    T_mid = mid_end - s0
    P = packed_bytes_total(bits, cfg, T_mid)
    C_rec = nbytes - chunks_off
    N_mid = L * 2 * H * T_mid * D
    e = K.element_size()
    alg = {  # minimum bytes each phase must move
        "enc_stats": N_mid * e,
        "enc_quant_pack": N_mid * e + P,
        "rans_encode": P + C_rec,
        "assemble": 2 * C_rec,
        "rans_decode": C_rec + P,
        "dec_transform": P + N_mid * e,
    }
    dom = max((k for k in alg if k in ph_ms), key=lambda k: ph_ms[k]) if ph_ms else None

    # reconstruction quality on the GPU
    def nrmse(a, b):
        a = a.float()
        b = b.float()
        return math.sqrt(float(((a - b) ** 2).sum()) / max(float((a ** 2).sum()), 1e-300))

    res = {
        "metric": METRIC,
        "value": raw / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if K.dtype == torch.bfloat16 else "fp32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {L} layers x {H} KV heads x {T} tokens x head_dim {D}, "
                        f"{w.dtype}, {cfg['bits_k']:g} bits/comp, sink {cfg['sink_tokens']}, "
                        f"recent {cfg['recent_tokens']}, {'PCA' if cfg['transform'] == 0 else 'WHT'}",
            "layers": L, "kv_heads": H, "tokens": T, "head_dim": D,
            "bits_per_component": cfg["bits_k"], "chunk_tokens": cfg["chunk_tokens"],
            "tile_tokens": cfg["tile_tokens"], "rans_lanes": cfg["rans_lanes"],
            "rans_scale_bits": cfg["rans_scale_bits"], "alloc_scope": cfg.get("alloc_scope", 0),
        },
        "raw_bytes": raw,
        "container_bytes": nbytes,
        "compression_ratio": raw / nbytes,
        "bits_per_value": 8.0 * nbytes / nvals,
        "exact_recomputed_codes": refined,
        "nrmse_k": nrmse(K, kd),
        "nrmse_v": nrmse(V, vd),
        "encode_gbps_events": raw / (t_enc * 1e-3) / 1e9 if t_enc else None,
        "decode_gbps_events": raw / (t_dec * 1e-3) / 1e9 if t_dec else None,
        "phases_ms": ph_ms,
        "path_roofline": {
            "bound": "hbm", "algorithmic_bytes": 2 * (raw + nbytes),
            "achieved": 2 * (raw + nbytes) / (ms_per_step * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": 2 * (raw + nbytes) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        },
        "wall_s": wall,
    }
    if dom:
        ach = alg[dom] / (ph_ms[dom] * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": dom, "kernels": list(PHASE_KERNELS[dom][0]),
                           "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBPS, "traffic": traffic_from_profile(dom),
                           "algorithmic_bytes": alg[dom], "avg_ms": ph_ms[dom]}
        # the same measure for every phase with a defined minimum traffic
        res["phase_roofline"] = {
            k: {"algorithmic_bytes": alg[k], "avg_ms": ph_ms[k],
                "frac": alg[k] / (ph_ms[k] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "traffic": traffic_from_profile(k)}
            for k in alg if k in ph_ms}
    if cfg["transform"] == 0 and ph_ms:
        # the projections are the path's dense contractions: 2 D flops per
        # coefficient (bf16 MFMA, fp32 accumulation) in the statistics pass,
        # again in the quantiser (it recomputes rather than stores them) and
        # in the inverse projection of the decoder
        # (the quantiser and the decoder project only the components that
        # carry codes: 2 D flops per coded coefficient)
        coded = int((bits > 0).sum()) * T_mid
        flops = {"enc_stats": 2 * D * N_mid, "enc_quant_pack": 2 * D * coded, "dec_transform": 2 * D * coded}
        res["mfma_roofline"] = {
            k: {"flops": flops[k], "achieved_tflops": flops[k] / (ph_ms[k] * 1e-3) / 1e12,
                "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                "frac": flops[k] / (ph_ms[k] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
            for k in flops if k in ph_ms}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, cfg, K, V, basis, args.cpu_layers) \
            if basis is not None else None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
