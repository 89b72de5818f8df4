"""Offline calibration of the PCA basis (an input of the method: the KVTC
explainer's "The Tradeoff Is Real" -- the codec needs calibration).

The basis is the uncentered second-moment eigenbasis that the Codec-Gauge
page uses for its PCA/KLT control ("Compression Conditions"), per layer and
K/V (shared by the heads of a layer, or per head), fitted on keys with RoPE
undone.  This runs once per model, before any plan is built, with PyTorch
linear algebra; it is not part of the coded path.
"""
from __future__ import annotations

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
