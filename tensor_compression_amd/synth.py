"""Seeded synthetic KV caches and the workload catalogue.

This module only draws inputs: it holds none of the codec's arithmetic and
is shared by the oracle tests, the GPU parity tests and the benchmark.

The caches stand in for real model captures, which are not available: the
pages measure on caches of Qwen3-32B ("TTAS-X2", 4 Memory Analysis) and of
the models listed on the Codec-Gauge page ("Evaluation Design").  Shapes
follow those models; the content is a low-rank Gaussian latent with noise,
which gives the PCA basis something to find.

Generator, per (layer l, K/V s), drawn in this order with one
``torch.Generator`` (layer-major, K before V):
  1. mixing M in R^{D x r}, entries N(0, 1/r);
  2. channel scales g_j = exp(N(0, 1)) (log-normal), then 2 distinct random
     channels multiplied by 20 (outliers) -- when ``scales`` is set;
  3. per head: latents z_t ~ N(0, I_r), noise eps ~ N(0, noise^2);
  x_t = g * (M z_t + eps).
Keys are then rotated with RoPE at their positions: this models what the
attention layer did before the cache was exported (the codec undoes it).  The
rotation here is the model-side one, written with torch's own ops.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    kv_heads: int
    head_dim: int
    tokens: int
    dtype: str  # "fp32" | "bf16"
    rank: int
    scales: bool
    outliers: int
    theta: float
    sink: int
    recent: int
    bits_k: float
    bits_v: float
    lanes: int
    transform: str = "pca"  # "pca" | "wht"
    noise: float = 0.05
    seed: int = 0
    basis_from: str = "mid"  # rows the basis is fitted on: "all" tokens or the coded "mid"dle
    bits_sweep: tuple = field(default_factory=tuple)
    n_seqs: int = 0  # ragged paged batch when > 0
    min_len: int = 0
    max_len: int = 0
    page_tokens: int = 16


WORKLOADS = {
    # 1 layer, 1 KV head, head_dim 64, 256 tokens, fp32; rank-8 latent with a
    # fixed random 64x8 mixing and N(0, 0.05) noise; keys RoPE'd (theta 1e4);
    # basis fitted on the same tensor; sink 4, recent 16, 4 bits/comp,
    # 12-bit rANS scale, 16 lanes, seed 0.
    "tiny": Workload("tiny", 1, 1, 64, 256, "fp32", 8, False, 0, 1e4, 4, 16, 4.0, 4.0, 16,
                     basis_from="all"),
    # Llama-3-8B-shaped cache: 32 layers, 8 KV heads, head_dim 128, 4096 tokens,
    # bf16; rank-32 latent, log-normal channel scales, 2 outlier channels x20;
    # theta 5e5; sink 4, recent 128, 2 bits/comp, per-layer basis.
    "llama3_8b": Workload("llama3_8b", 32, 8, 128, 4096, "bf16", 32, True, 2, 5e5, 4, 128, 2.0,
                          2.0, 32),
    # Qwen3-32B-shaped cache: 64 layers, 8 KV heads, head_dim 128, 32768 tokens,
    # bf16, the Llama-shaped generator; budgets 1 / 1.6 / 2 / 4 bits/comp.
    "qwen3_32b": Workload("qwen3_32b", 64, 8, 128, 32768, "bf16", 32, True, 2, 5e5, 4, 128, 2.0,
                          2.0, 32, bits_sweep=(1.0, 1.6, 2.0, 4.0)),
    # Hadamard path, long context: 32 layers, 8 KV heads, head_dim 128,
    # 131072 tokens, bf16; RMS normalisation + 128-point WHT; keys 4-bit with a
    # per-head scale, values 2-bit per component.
    "hadamard_long": Workload("hadamard_long", 32, 8, 128, 131072, "bf16", 32, True, 2, 5e5, 4,
                              128, 4.0, 2.0, 32, transform="wht"),
    # Ragged paged batch: 256 sequences, lengths uniform in [512, 8192], 16-token
    # pages; 32 layers, 8 KV heads, head_dim 128, bf16; shared per-layer basis;
    # 2 bits/comp; each sequence coded independently.
    "ragged_paged": Workload("ragged_paged", 32, 8, 128, 0, "bf16", 32, True, 2, 5e5, 4, 128, 2.0,
                             2.0, 32, n_seqs=256, min_len=512, max_len=8192, seed=0),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def model_rope(x: torch.Tensor, positions: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotate [..., T, D] rows by RoPE at `positions` (half-split pairs j, j+D/2),
    the convention of Llama/Qwen-style attention layers."""
    D = x.shape[-1]
    h = D // 2
    inv = theta ** (-torch.arange(h, dtype=torch.float64, device=x.device) * 2.0 / D)
    ang = positions.to(torch.float64)[:, None] * inv[None, :]
    cos = torch.cos(ang).to(torch.float32)
    sin = torch.sin(ang).to(torch.float32)
    a, b = x[..., :h], x[..., h:]
    return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1)


def _layer_params(gen, D, r, scales, outliers, device):
    M = torch.randn(D, r, generator=gen, device=device, dtype=torch.float32) / math.sqrt(r)
    g = torch.ones(D, device=device, dtype=torch.float32)
    if scales:
        g = torch.exp(torch.randn(D, generator=gen, device=device, dtype=torch.float32))
    if outliers:
        idx = torch.randperm(D, generator=gen, device=device)[:outliers]
        g[idx] = g[idx] * 20.0
    return M, g


def generate(w: Workload, device: str = "cpu", tokens: int | None = None,
             layers: int | None = None, seed: int | None = None):
    """K, V as [L, H, T, D] tensors of the workload dtype on `device`.

    `tokens` / `layers` override the shape (reduced-size parity cases)."""
    T = w.tokens if tokens is None else tokens
    L = w.layers if layers is None else layers
    H, D, r = w.kv_heads, w.head_dim, w.rank
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w.dtype)
    K = torch.empty(L, H, T, D, dtype=dt, device=device)
    V = torch.empty(L, H, T, D, dtype=dt, device=device)
    pos = torch.arange(T, device=device)
    for l in range(L):
        for s, dst in ((0, K), (1, V)):
            M, g = _layer_params(gen, D, r, w.scales, w.outliers, device)
            z = torch.randn(H, T, r, generator=gen, device=device, dtype=torch.float32)
            eps = torch.randn(H, T, D, generator=gen, device=device, dtype=torch.float32) * w.noise
            x = (z @ M.T + eps) * g
            if s == 0:
                x = model_rope(x, pos, w.theta)
            dst[l] = x.to(dt)
            del z, eps, x
    return K, V


def ragged_lengths(w: Workload, n_seqs: int | None = None, seed: int = 1):
    """Sequence lengths uniform in [min_len, max_len] (inclusive), seeded."""
    n = w.n_seqs if n_seqs is None else n_seqs
    gen = torch.Generator()
    gen.manual_seed(seed)
    return torch.randint(w.min_len, w.max_len + 1, (n,), generator=gen).tolist()


def page_permutation(n_pages: int, seed: int = 2):
    gen = torch.Generator()
    gen.manual_seed(seed)
    return torch.randperm(n_pages, generator=gen)


def generate_paged(w: Workload, device: str = "cpu", lengths=None, layers: int | None = None,
                   seed: int | None = None, spare_pages: int = 0):
    """A ragged batch in 16-token pages: pools [L, P, H, 16, D] (workload
    dtype, zero where no token lives), page_table [n_seqs, max_pages] int32
    (-1 past a sequence's pages) and the lengths.

    The per-layer mixing and channel scales are drawn first (layer-major, K
    before V) and shared by every sequence and head, as a shared per-layer
    basis implies; then each sequence draws its latents and noise in order.
    Pages are handed out by a seeded permutation of the pool."""
    lens = list(ragged_lengths(w) if lengths is None else lengths)
    L = w.layers if layers is None else layers
    H, D, r, pt = w.kv_heads, w.head_dim, w.rank, w.page_tokens
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w.dtype)
    params = [[_layer_params(gen, D, r, w.scales, w.outliers, device) for _ in range(2)] for _ in range(L)]
    n_pg = [(T + pt - 1) // pt for T in lens]
    n_pages = sum(n_pg) + spare_pages
    perm = page_permutation(max(n_pages, 1))
    max_pages = max(max(n_pg), 1)
    table = torch.full((len(lens), max_pages), -1, dtype=torch.int32)
    at = 0
    for z, n in enumerate(n_pg):
        table[z, :n] = perm[at: at + n].to(torch.int32)
        at += n
    pools = [torch.zeros(L, max(n_pages, 1), H, pt, D, dtype=dt, device=device) for _ in range(2)]
    for z, T in enumerate(lens):
        if T == 0:
            continue
        pages = table[z, : n_pg[z]].to(device=device, dtype=torch.long)
        pos = torch.arange(T, device=device)
        for l in range(L):
            for s in range(2):
                M, g = params[l][s]
                zl = torch.randn(H, T, r, generator=gen, device=device, dtype=torch.float32)
                eps = torch.randn(H, T, D, generator=gen, device=device, dtype=torch.float32) * w.noise
                x = (zl @ M.T + eps) * g
                if s == 0:
                    x = model_rope(x, pos, w.theta)
                xp = torch.zeros(H, n_pg[z] * pt, D, dtype=dt, device=device)
                xp[:, :T] = x.to(dt)
                pools[s][l, pages] = xp.view(H, n_pg[z], pt, D).permute(1, 0, 2, 3)
    return pools[0], pools[1], table, lens


def gather_paged(pool: torch.Tensor, table: torch.Tensor, z: int, T: int) -> torch.Tensor:
    """Sequence z of a page pool as a contiguous [L, H, T, D] tensor."""
    L, _, H, pt, D = pool.shape
    n = (T + pt - 1) // pt
    pages = table[z, :n].to(device=pool.device, dtype=torch.long)
    x = pool[:, pages].permute(0, 2, 1, 3, 4).reshape(L, H, n * pt, D)
    return x[:, :, :T].contiguous()


def to_numpy_bits(x: torch.Tensor):
    """Host copy for the oracle: fp32 as float32, bf16 as its uint16 bit pattern."""
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    return x.numpy()


def oracle_config(w: Workload, **over) -> dict:
    """The codec configuration of a workload as a plain dict of field names
    (each side converts it to its own struct)."""
    cfg = dict(
        layers=w.layers, kv_heads=w.kv_heads, head_dim=w.head_dim,
        dtype=0 if w.dtype == "fp32" else 1, transform=0 if w.transform == "pca" else 1,
        sink_tokens=w.sink, recent_tokens=w.recent, bits_k=w.bits_k, bits_v=w.bits_v,
        max_bits=8, rope_keys=1, rope_style=0, rope_theta=w.theta, rans_scale_bits=12,
        rans_lanes=w.lanes, chunk_tokens=4096, tile_tokens=256, basis_per_head=0, wht_keys=1,
    )
    cfg.update(over)
    return cfg
