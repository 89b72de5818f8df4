"""Offline calibration of the PCA basis (an input of the method: the KVTC
explainer's "The Tradeoff Is Real" -- the codec needs calibration).

The basis is the uncentered second-moment eigenbasis that the Codec-Gauge
page uses for its PCA/KLT control ("Compression Conditions"), per layer and
K/V (shared by the heads of a layer, or per head), fitted on keys with RoPE
undone.  This runs once per model, before any plan is built, with PyTorch
linear algebra; it is not part of the coded path.
"""
from __future__ import annotations

import math

import torch


def _unrotate(x: torch.Tensor, positions: torch.Tensor, theta: float, style: int) -> torch.Tensor:
    D = x.shape[-1]
    h = D // 2
    inv = theta ** (-torch.arange(h, dtype=torch.float64, device=x.device) * 2.0 / D)
    ang = positions.to(torch.float64)[:, None] * inv[None, :]
    c = torch.cos(ang).to(torch.float32)
    s = torch.sin(ang).to(torch.float32)
    if style == 0:
        a, b = x[..., :h], x[..., h:]
        return torch.cat([a * c + b * s, b * c - a * s], dim=-1)
    a, b = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = a * c + b * s
    out[..., 1::2] = b * c - a * s
    return out


def fit_pca_basis(K: torch.Tensor, V: torch.Tensor, cfg: dict, t0: int = 0,
                  t1: int | None = None) -> torch.Tensor:
    """fp32 basis [L, 2, D, D] (or [L, 2, H, D, D]); column i is component i,
    in descending eigenvalue order, largest-magnitude entry positive."""
    L, H, T, D = K.shape
    t1 = T if t1 is None else t1
    per_head = bool(cfg.get("basis_per_head", 0))
    out_shape = (L, 2, H, D, D) if per_head else (L, 2, D, D)
    out = torch.empty(out_shape, dtype=torch.float32, device=K.device)
    pos = torch.arange(t0, t1, device=K.device)
    for l in range(L):
        for s, src in ((0, K), (1, V)):
            x = src[l, :, t0:t1].to(torch.float32)
            if s == 0 and cfg.get("rope_keys", 1):
                x = _unrotate(x, pos, cfg["rope_theta"], cfg.get("rope_style", 0))
            x = x.to(torch.float64)
            if per_head:
                for h in range(H):
                    out[l, s, h] = _eig(x[h].T @ x[h] / max(x.shape[1], 1))
            else:
                xs = x.reshape(-1, D)
                out[l, s] = _eig(xs.T @ xs / max(xs.shape[0], 1))
    return out


def _eig(S: torch.Tensor) -> torch.Tensor:
    w, V = torch.linalg.eigh(S)
    order = torch.argsort(-w, stable=True)
    V = V[:, order]
    idx = torch.argmax(V.abs(), dim=0)
    sign = torch.sign(V[idx, torch.arange(V.shape[1], device=V.device)])
    sign[sign == 0] = 1
    return (V * sign).to(torch.float32)


def grouped_random_gauge(layers: int, D: int, g: int, scale: float = 0.5, seed: int = 0) -> torch.Tensor:
    """A seeded grouped gauge as a basis [layers, 2, D, D] (Codec-Gauge,
    Gauge Parameterization: block-diagonal exp(A - A^T) over groups of g
    channels; the random-gauge control of Compression Conditions).  The
    frame is Z = G X, so the basis (column i = component i) is B = G^T.  The
    generators A are N(0, scale^2); learning them is not part of the codec."""
    gen = torch.Generator().manual_seed(seed)
    out = torch.zeros((layers, 2, D, D), dtype=torch.float64)
    for l in range(layers):
        for s in range(2):
            A = torch.randn((D // g, g, g), generator=gen, dtype=torch.float64) * scale
            G = torch.matrix_exp(A - A.transpose(1, 2))
            for k in range(D // g):
                out[l, s, k * g:(k + 1) * g, k * g:(k + 1) * g] = G[k].T
    return out.to(torch.float32)


def hadamard(D: int, dtype=torch.float64, device="cpu") -> torch.Tensor:
    """Orthonormal Walsh-Hadamard matrix in Sylvester order."""
    i = torch.arange(D, device=device)
    bits = (i[:, None] & i[None, :]).to(torch.int64)
    par = torch.zeros_like(bits)
    while bool(bits.any()):
        par ^= bits & 1
        bits >>= 1
    return (1 - 2 * par).to(dtype) / math.sqrt(D)


def _kmeans(x: torch.Tensor, k: int, iters: int, gen: torch.Generator) -> torch.Tensor:
    """Lloyd's k-means on rows of x [N, d] (fp32), seeded with k distinct rows
    (repeated when N < k)."""
    N = x.shape[0]
    pick = torch.randperm(N, generator=gen)[:k]
    if pick.numel() < k:
        pick = pick.repeat((k + N - 1) // N)[:k]
    cent = x[pick.to(x.device)].clone()
    for _ in range(iters):
        a = torch.cdist(x, cent).argmin(1)
        s = torch.zeros_like(cent).index_add_(0, a, x)
        n = torch.bincount(a, minlength=k).to(x.dtype)
        keep = n > 0
        cent[keep] = s[keep] / n[keep, None]
    return cent


def train_pq_codebooks(V: torch.Tensor, pq: dict, iters: int = 8, seed: int = 0, max_rows: int = 65536):
    """Two-level product-quantisation codebooks for the TTAS-X2 value path
    (TTAS-X2 2.2: per-vector RMS normalisation, Hadamard transform, then
    product quantisation with K1 and K2 centroids per subspace), trained by
    k-means per layer and subspace on V [L, H, T, D]; level 2 on the level-1
    residuals (centroids rounded to bf16, as the codec holds them).  Returns
    fp32 (cb1 [L, M, k1, d], cb2 [L, M, k2, d]).  Set-up, not the coded path."""
    L, H, T, D = V.shape
    d, k1, k2 = pq["sub_dim"], pq["k1"], pq["k2"]
    M = D // d
    gen = torch.Generator().manual_seed(seed)
    Hm = hadamard(D, torch.float64, V.device)
    cb1 = torch.empty((L, M, k1, d), dtype=torch.float32)
    cb2 = torch.empty((L, M, k2, d), dtype=torch.float32)
    for l in range(L):
        x = V[l].reshape(-1, D).to(torch.float64)
        if x.shape[0] > max_rows:
            x = x[torch.randperm(x.shape[0], generator=gen)[:max_rows].to(x.device)]
        r = torch.sqrt((x * x).mean(1, keepdim=True))
        xn = torch.where(r > 0, x / torch.where(r > 0, r, torch.ones_like(r)), torch.zeros_like(x))
        y = (xn @ Hm.T).to(torch.float32)
        for s in range(M):
            ys = y[:, s * d:(s + 1) * d].contiguous()
            c1 = _kmeans(ys, k1, iters, gen).to(torch.bfloat16).to(torch.float32)
            e = ys - c1[torch.cdist(ys, c1).argmin(1)]
            c2 = _kmeans(e, k2, iters, gen)
            cb1[l, s] = c1.cpu()
            cb2[l, s] = c2.cpu()
    return cb1, cb2
