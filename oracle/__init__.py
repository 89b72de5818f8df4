"""KVTC oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, single-threaded CPU implementation of KVTC-style transform
coding (C in ``kvtc_oracle.c``, wrapped here with ctypes), used to check the
HIP library.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP
library and imports nothing from it.

Method sources are cited by page title and section; see ``kvtc_oracle.h``.

The PCA basis is an *input* of the method (the explainer's "The Tradeoff Is
Real": the codec "needs calibration"); :func:`fit_pca_basis` computes the
uncentered second-moment eigenbasis that the Codec-Gauge page defines for its
PCA/KLT control ("Compression Conditions"), per layer and K/V, from rows that
the oracle itself un-rotates.  The eigendecomposition is numpy's ``eigh`` in
fp64 (a library primitive).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvtc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvtc_oracle.so")

FP32, BF16 = 0, 1
PCA, WHT = 0, 1
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_CORRUPT, ERR_NONFINITE = range(6)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "CAPACITY", 4: "CORRUPT",
                5: "NONFINITE"}


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what}: {STATUS_NAMES.get(status, status)}")
        self.status = status


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("transform", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32), ("recent_tokens", ctypes.c_int32),
        ("bits_k", ctypes.c_float), ("bits_v", ctypes.c_float), ("max_bits", ctypes.c_int32),
        ("rope_keys", ctypes.c_int32), ("rope_style", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("rans_scale_bits", ctypes.c_int32),
        ("rans_lanes", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32), ("basis_per_head", ctypes.c_int32),
        ("wht_keys", ctypes.c_int32), ("alloc_scope", ctypes.c_int32),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2, no fp contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f32, f64, u64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_double, ctypes.c_uint64)
        sig = {
            "orc_f32_to_bf16": (ctypes.c_uint16, [f32]),
            "orc_bf16_to_f32": (f32, [ctypes.c_uint16]),
            "orc_rope_table": (None, [i32, i32, f64, P, P]),
            "orc_rope_inverse": (None, [P, P, i32, i32, P, P]),
            "orc_rope_forward": (None, [P, P, i32, i32, P, P]),
            "orc_project": (None, [P, P, i32, P]),
            "orc_unproject": (None, [P, P, i32, P]),
            "orc_rms": (f32, [P, i32]),
            "orc_wht": (None, [P, i32, P]),
            "orc_stats": (None, [P, i64, i32, P, P, P, P]),
            "orc_budget": (i32, [f32, i32]),
            "orc_alloc_greedy": (None, [P, i32, i32, i32, P]),
            "orc_alloc_greedy_heap": (None, [P, ctypes.c_int64, ctypes.c_int64, i32, P]),
            "orc_checksum": (None, [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P]),
            "orc_sq_check": (i32, [P, P]),
            "orc_sq_code_bytes": (ctypes.c_int64, [P, P, i32]),
            "orc_sq_range_pairs": (ctypes.c_int64, [P, P, i32]),
            "orc_sq_encode": (i32, [P, P, P, P, i32, P, P, P]),
            "orc_sq_decode": (i32, [P, P, P, P, i32, P, P, P]),
            "orc_pq_check": (i32, [P, P]),
            "orc_pq_row_words": (i32, [P, P]),
            "orc_pq_outlier_slots": (ctypes.c_int64, [P, P, i32]),
            "orc_pq_nearest": (i32, [P, P, i32, i32]),
            "orc_pq_encode": (i32, [P, P, P, i32, P, P, P, P, P]),
            "orc_pq_decode": (i32, [P, P, P, P, P, i32, P, P, P]),
            "orc_alloc_dp": (f64, [P, i32, i32, i32, P]),
            "orc_distortion": (f64, [P, P, i32]),
            "orc_side_info": (None, [P, P, P, P, i32, P, P, P]),
            "orc_quantize": (None, [P, i64, i32, P, P, P, P, P]),
            "orc_quantize_sym": (None, [P, i64, i32, i32, f32, P, P]),
            "orc_packed_bytes": (i64, [P, i32, i64]),
            "orc_pack": (None, [P, i64, i32, P, P]),
            "orc_unpack": (None, [P, i64, i32, P, P]),
            "orc_freq_normalize": (None, [P, i32, i32, P]),
            "orc_sym_bits": (i32, [i32]),
            "orc_raw_bits": (i32, [i32]),
            "orc_rans_encode_seq": (i64, [i64, P, P, P, P, P, i32, i32, P, P, i64]),
            "orc_rans_decode_seq": (ctypes.c_int, [i64, P, P, P, P, i32, i32, P, P, i64, P]),
            "orc_chunk_encode": (i64, [P, P, P, i32, P, i64, P]),
            "orc_chunk_decode": (ctypes.c_int, [P, P, P, i64, i32, i32, P]),
            "orc_rans_encode": (i64, [P, i64, P, i32, i32, P, P, i64]),
            "orc_rans_decode": (ctypes.c_int, [P, P, i64, P, i32, i32, i64, P]),
            "orc_check_config": (ctypes.c_int, [P]),
            "orc_fnv1a64": (u64, [u64, P, i64]),
            "orc_fingerprint": (u64, [P, P]),
            "orc_max_container_bytes": (i64, [P, i32]),
            "orc_encode": (ctypes.c_int, [P, P, P, i32, P, P, i64, P]),
            "orc_decode": (ctypes.c_int, [P, P, P, i64, P, P, i32]),
            "orc_decode_sections": (ctypes.c_int, [P, P, P, i64, i32, i32, P]),
            "orc_section_rows": (ctypes.c_int, [P, P, P, i32, i32, i32, i32, P]),
            "orc_section_codes": (ctypes.c_int, [P, P, P, i64, i32, P]),
            "orc_section_coeffs": (ctypes.c_int, [P, P, P, i32, P, i32, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    # data_as keeps a reference to the array, so a temporary passed straight
    # into a call (np.ascontiguousarray(...) of a strided view) stays alive
    # until the call returns
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# configuration
# --------------------------------------------------------------------------

CONFIG_FIELDS = [f for f, _ in _Cfg._fields_]

SQ_BLOCK, SQ_KIVI = 1, 2


class _SqCfg(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("group", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("bits_k", ctypes.c_int32), ("bits_v", ctypes.c_int32)]


def make_cfg(cfg: dict) -> _Cfg:
    """Fill the oracle's config struct from a plain dict of its field names."""
    c = _Cfg()
    for f in CONFIG_FIELDS:
        setattr(c, f, cfg.get(f, 0) if f == "alloc_scope" else cfg[f])
    return c


# --------------------------------------------------------------------------
# numeric primitives
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    return np.array([lib().orc_f32_to_bf16(float(v)) for v in x], dtype=np.uint16)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) -> fp32, vectorised in numpy
    (checked against the C routine in the tests)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    upper = u >> 16
    lower = u & 0xFFFF
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    upper = upper + up.astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    upper = np.where(nan, (u >> 16) | 0x40, upper)
    return (upper.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rope_table(T: int, D: int, theta: float):
    cos = np.zeros((T, D // 2), np.float32)
    sin = np.zeros((T, D // 2), np.float32)
    lib().orc_rope_table(T, D, theta, _p(cos), _p(sin))
    return cos, sin


def rope_inverse(y: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray, style: int = 0):
    y = np.ascontiguousarray(y, np.float32)
    x = np.zeros_like(y)
    lib().orc_rope_inverse(_p(y), _p(x), y.shape[-1], style,
                           _p(np.ascontiguousarray(cos_row, np.float32)),
                           _p(np.ascontiguousarray(sin_row, np.float32)))
    return x


def rope_forward(x: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray, style: int = 0):
    x = np.ascontiguousarray(x, np.float32)
    y = np.zeros_like(x)
    lib().orc_rope_forward(_p(x), _p(y), x.shape[-1], style,
                           _p(np.ascontiguousarray(cos_row, np.float32)),
                           _p(np.ascontiguousarray(sin_row, np.float32)))
    return y


def project(x: np.ndarray, Bp: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    Bp = np.ascontiguousarray(Bp, np.float32)
    c = np.zeros_like(x)
    lib().orc_project(_p(x), _p(Bp), x.shape[-1], _p(c))
    return c


def unproject(chat: np.ndarray, Bp: np.ndarray) -> np.ndarray:
    chat = np.ascontiguousarray(chat, np.float32)
    Bp = np.ascontiguousarray(Bp, np.float32)
    x = np.zeros_like(chat)
    lib().orc_unproject(_p(chat), _p(Bp), chat.shape[-1], _p(x))
    return x


def rms(x: np.ndarray) -> float:
    x = np.ascontiguousarray(x, np.float32)
    return float(lib().orc_rms(_p(x), x.shape[-1]))


def wht(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    y = np.zeros_like(x)
    lib().orc_wht(_p(x), x.shape[-1], _p(y))
    return y


# --------------------------------------------------------------------------
# statistics / allocation / quantiser
# --------------------------------------------------------------------------

def stats(c: np.ndarray):
    c = np.ascontiguousarray(c, np.float32)
    N, D = c.shape
    mu, var, mn, mx = (np.zeros(D, np.float32) for _ in range(4))
    lib().orc_stats(_p(c), N, D, _p(mu), _p(var), _p(mn), _p(mx))
    return mu, var, mn, mx


def budget(bits: float, D: int) -> int:
    return int(lib().orc_budget(bits, D))


def alloc_greedy(var: np.ndarray, budget_: int, max_bits: int) -> np.ndarray:
    var = np.ascontiguousarray(var, np.float32)
    bits = np.zeros(var.shape[0], np.uint8)
    lib().orc_alloc_greedy(_p(var), var.shape[0], budget_, max_bits, _p(bits))
    return bits


def alloc_greedy_heap(var: np.ndarray, budget_: int, max_bits: int) -> np.ndarray:
    """Greedy allocation over any number of components (all sections of a
    cache under one budget), heap-ordered; equal to alloc_greedy."""
    var = np.ascontiguousarray(var, np.float32).reshape(-1)
    bits = np.zeros(var.shape[0], np.uint8)
    lib().orc_alloc_greedy_heap(_p(var), var.shape[0], int(budget_), max_bits, _p(bits))
    return bits


def alloc_dp(var: np.ndarray, budget_: int, max_bits: int):
    var = np.ascontiguousarray(var, np.float32)
    bits = np.zeros(var.shape[0], np.uint8)
    d = lib().orc_alloc_dp(_p(var), var.shape[0], budget_, max_bits, _p(bits))
    return d, bits


def distortion(var: np.ndarray, bits: np.ndarray) -> float:
    var = np.ascontiguousarray(var, np.float32)
    bits = np.ascontiguousarray(bits, np.uint8)
    return float(lib().orc_distortion(_p(var), _p(bits), var.shape[0]))


def side_info(bits, mu, mn, mx):
    D = len(bits)
    bits = np.ascontiguousarray(bits, np.uint8)
    zero, scale, rcp = (np.zeros(D, np.float32) for _ in range(3))
    lib().orc_side_info(_p(bits), _p(np.ascontiguousarray(mu, np.float32)),
                        _p(np.ascontiguousarray(mn, np.float32)),
                        _p(np.ascontiguousarray(mx, np.float32)), D, _p(zero), _p(scale), _p(rcp))
    return zero, scale, rcp


def quantize(c, bits, zero, rcp):
    c = np.ascontiguousarray(c, np.float32)
    N, D = c.shape
    q = np.zeros((N, D), np.uint8)
    v = np.zeros((N, D), np.float32)
    lib().orc_quantize(_p(c), N, D, _p(np.ascontiguousarray(bits, np.uint8)),
                       _p(np.ascontiguousarray(zero, np.float32)),
                       _p(np.ascontiguousarray(rcp, np.float32)), _p(q), _p(v))
    return q, v


def quantize_sym(c, b: int, rcp: float):
    c = np.ascontiguousarray(c, np.float32)
    N, D = c.shape
    q = np.zeros((N, D), np.uint8)
    v = np.zeros((N, D), np.float32)
    lib().orc_quantize_sym(_p(c), N, D, b, rcp, _p(q), _p(v))
    return q, v


# --------------------------------------------------------------------------
# packing / rANS
# --------------------------------------------------------------------------

def packed_bytes(bits, ntok: int) -> int:
    bits = np.ascontiguousarray(bits, np.uint8)
    return int(lib().orc_packed_bytes(_p(bits), len(bits), ntok))


def pack(q: np.ndarray, bits) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    ntok, D = q.shape
    bits = np.ascontiguousarray(bits, np.uint8)
    out = np.zeros(max(packed_bytes(bits, ntok), 1), np.uint8)
    lib().orc_pack(_p(q), ntok, D, _p(bits), _p(out))
    return out[: packed_bytes(bits, ntok)]


def unpack(data: np.ndarray, ntok: int, bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, np.uint8)
    D = len(bits)
    data = np.ascontiguousarray(data, np.uint8)
    if data.size == 0:
        data = np.zeros(1, np.uint8)
    q = np.zeros((ntok, D), np.uint8)
    lib().orc_unpack(_p(data), ntok, D, _p(bits), _p(q))
    return q


def freq_normalize(counts, scale_bits: int = 12) -> np.ndarray:
    """Frequencies (sum 2^scale_bits) of an alphabet of len(counts) <= 256 symbols."""
    counts = np.ascontiguousarray(counts, np.uint32)
    assert counts.ndim == 1 and 1 <= counts.size <= 256
    f = np.zeros(counts.size, np.uint16)
    lib().orc_freq_normalize(_p(counts), counts.size, scale_bits, _p(f))
    return f


def sym_bits(b: int) -> int:
    return int(lib().orc_sym_bits(int(b)))


def raw_bits(b: int) -> int:
    return int(lib().orc_raw_bits(int(b)))


def rans_encode_seq(sym, lane, tab, n_sym, freqs, scale_bits: int = 12, lanes: int = 32):
    """Interleaved rANS over a symbol sequence in decoding order, with a lane
    and a table (offset into `freqs`, n_sym entries) per symbol."""
    sym = np.ascontiguousarray(sym, np.uint8)
    N = sym.size
    lane = np.ascontiguousarray(lane, np.uint8)
    tab = np.ascontiguousarray(tab, np.int32)
    n_sym = np.ascontiguousarray(n_sym, np.int32)
    freqs = np.ascontiguousarray(freqs, np.uint16)
    states = np.zeros(lanes, np.uint32)
    cap = rans_words_cap(N, lanes, scale_bits)
    words = np.zeros(max(cap, 1), np.uint16)
    one8, one32 = np.zeros(1, np.uint8), np.zeros(1, np.int32)
    n = lib().orc_rans_encode_seq(N, _p(sym if N else one8), _p(lane if N else one8),
                                  _p(tab if N else one32), _p(n_sym if N else one32), _p(freqs),
                                  scale_bits, lanes, _p(states), _p(words), cap)
    if n < 0:
        raise OracleError(ERR_CAPACITY, "rans_encode_seq")
    return states, words[:n].copy()


def rans_decode_seq(states, words, lane, tab, n_sym, freqs, scale_bits: int = 12, lanes: int = 32):
    lane = np.ascontiguousarray(lane, np.uint8)
    N = lane.size
    tab = np.ascontiguousarray(tab, np.int32)
    n_sym = np.ascontiguousarray(n_sym, np.int32)
    states = np.ascontiguousarray(states, np.uint32)
    words = np.ascontiguousarray(words, np.uint16)
    wbuf = words if words.size else np.zeros(1, np.uint16)
    out = np.zeros(max(N, 1), np.uint8)
    one8, one32 = np.zeros(1, np.uint8), np.zeros(1, np.int32)
    st = lib().orc_rans_decode_seq(N, _p(lane if N else one8), _p(tab if N else one32),
                                   _p(n_sym if N else one32), _p(np.ascontiguousarray(freqs, np.uint16)),
                                   scale_bits, lanes, _p(states), _p(wbuf), words.size, _p(out))
    if st != OK:
        raise OracleError(st, "rans_decode_seq")
    return out[:N]


def chunk_encode(cfg: dict, bits, q) -> tuple:
    """(record bytes, mode) of one chunk's codes q[n, D] (mode 0 coded, 1 packed)."""
    c = make_cfg(cfg)
    q = np.ascontiguousarray(q, np.uint8)
    n, D = q.shape
    bits = np.ascontiguousarray(bits, np.uint8)
    cap = 4 * n * D + 4096
    out = np.zeros(cap, np.uint8)
    mode = ctypes.c_int32(0)
    size = lib().orc_chunk_encode(ctypes.byref(c), _p(bits), _p(q if q.size else np.zeros(1, np.uint8)),
                                  n, _p(out), cap, ctypes.byref(mode))
    if size < 0:
        raise OracleError(ERR_CAPACITY, "chunk_encode")
    return out[:size].tobytes(), mode.value


def chunk_decode(cfg: dict, bits, rec: bytes, mode: int, n: int) -> np.ndarray:
    c = make_cfg(cfg)
    D = cfg["head_dim"]
    buf = np.frombuffer(bytes(rec), np.uint8).copy()
    q = np.zeros((max(n, 1), D), np.uint8)
    st = lib().orc_chunk_decode(ctypes.byref(c), _p(np.ascontiguousarray(bits, np.uint8)),
                                _p(buf if buf.size else np.zeros(1, np.uint8)), buf.size, mode, n, _p(q))
    if st != OK:
        raise OracleError(st, "chunk_decode")
    return q[:n]


def byte_histogram(sym: np.ndarray) -> np.ndarray:
    return np.bincount(np.asarray(sym, np.uint8).ravel(), minlength=256).astype(np.uint32)


def rans_words_cap(N: int, lanes: int, scale_bits: int) -> int:
    return (N * (scale_bits + 1)) // 16 + 2 * lanes + 2


def rans_encode(sym: np.ndarray, freq: np.ndarray, scale_bits: int = 12, lanes: int = 32):
    sym = np.ascontiguousarray(sym, np.uint8)
    if sym.size == 0:
        sym = np.zeros(0, np.uint8)
    N = sym.size
    states = np.zeros(lanes, np.uint32)
    cap = rans_words_cap(N, lanes, scale_bits)
    words = np.zeros(max(cap, 1), np.uint16)
    buf = sym if N else np.zeros(1, np.uint8)
    n = lib().orc_rans_encode(_p(buf), N, _p(np.ascontiguousarray(freq, np.uint16)), scale_bits,
                              lanes, _p(states), _p(words), cap)
    if n < 0:
        raise OracleError(ERR_CAPACITY, "rans_encode")
    return states, words[:n].copy()


def rans_decode(states, words, freq, N: int, scale_bits: int = 12, lanes: int = 32):
    states = np.ascontiguousarray(states, np.uint32)
    words = np.ascontiguousarray(words, np.uint16)
    wbuf = words if words.size else np.zeros(1, np.uint16)
    out = np.zeros(max(N, 1), np.uint8)
    st = lib().orc_rans_decode(_p(states), _p(wbuf), words.size,
                               _p(np.ascontiguousarray(freq, np.uint16)), scale_bits, lanes, N,
                               _p(out))
    if st != OK:
        raise OracleError(st, "rans_decode")
    return out[:N]


# --------------------------------------------------------------------------
# container encode / decode
# --------------------------------------------------------------------------

def _tensor_ptr(x: np.ndarray, dtype: int):
    if dtype == BF16:
        assert x.dtype == np.uint16, "bf16 tensors are passed as their uint16 bit patterns"
    else:
        assert x.dtype == np.float32
    return _p(np.ascontiguousarray(x))


def check_config(cfg: dict) -> int:
    c = make_cfg(cfg)
    return int(lib().orc_check_config(ctypes.byref(c)))


def checksum(data: bytes, skip_from: int = 0, skip_to: int = 0) -> tuple[int, int]:
    """(A, B): plain and position-weighted sums of the 32-bit words mod 2^61 - 1."""
    buf = np.frombuffer(bytes(data), np.uint8).copy()
    a = ctypes.c_uint64(0)
    b = ctypes.c_uint64(0)
    lib().orc_checksum(_p(buf), len(buf), skip_from, skip_to, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def sq_sizes(cfg: dict, sq: dict, T: int) -> tuple[int, int]:
    """(code bytes, (zero, scale) pairs) of the scalar-quantiser path."""
    c, q = make_cfg(cfg), _SqCfg(**sq)
    return (int(lib().orc_sq_code_bytes(ctypes.byref(c), ctypes.byref(q), T)),
            int(lib().orc_sq_range_pairs(ctypes.byref(c), ctypes.byref(q), T)))


def sq_encode(cfg: dict, sq: dict, k, v, basis) -> tuple[np.ndarray, np.ndarray]:
    """Scalar quantisers on gauge coordinates ([CG] Compression Conditions):
    (codes uint8, ranges float32 [pairs, 2])."""
    c, q = make_cfg(cfg), _SqCfg(**sq)
    T = k.shape[2]
    nb, nr = sq_sizes(cfg, sq, T)
    if nb < 0:
        raise OracleError(ERR_INVALID_ARG, "sq_encode")
    codes = np.zeros(max(nb, 1), np.uint8)
    ranges = np.zeros((max(nr, 1), 2), np.float32)
    kk, vv = np.ascontiguousarray(k), np.ascontiguousarray(v)
    b = np.ascontiguousarray(basis, np.float32)
    st = lib().orc_sq_encode(ctypes.byref(c), ctypes.byref(q), _p(kk), _p(vv), T, _p(b), _p(codes), _p(ranges))
    if st != OK:
        raise OracleError(st, "sq_encode")
    return codes[:nb], ranges[:nr]


def sq_decode(cfg: dict, sq: dict, codes, ranges, T: int, basis) -> tuple[np.ndarray, np.ndarray]:
    c, q = make_cfg(cfg), _SqCfg(**sq)
    shape = (cfg["layers"], cfg["kv_heads"], T, cfg["head_dim"])
    ko, vo = np.zeros(shape, np.float32), np.zeros(shape, np.float32)
    cs = np.ascontiguousarray(codes, np.uint8)
    rg = np.ascontiguousarray(ranges, np.float32)
    b = np.ascontiguousarray(basis, np.float32)
    st = lib().orc_sq_decode(ctypes.byref(c), ctypes.byref(q), _p(cs), _p(rg), T, _p(b), _p(ko), _p(vo))
    if st != OK:
        raise OracleError(st, "sq_decode")
    return ko, vo


class _PqCfg(ctypes.Structure):
    _fields_ = [("sub_dim", ctypes.c_int32), ("k1", ctypes.c_int32), ("k2", ctypes.c_int32),
                ("outliers", ctypes.c_int32), ("block_tokens", ctypes.c_int32)]


def pq_sizes(cfg: dict, pq: dict, T: int) -> tuple[int, int]:
    """(u32 words per token row, outlier slots) of the TTAS-X2 value path."""
    c, q = make_cfg(cfg), _PqCfg(**pq)
    rw = int(lib().orc_pq_row_words(ctypes.byref(c), ctypes.byref(q)))
    ns = int(lib().orc_pq_outlier_slots(ctypes.byref(c), ctypes.byref(q), T))
    if rw < 0 or ns < 0:
        raise OracleError(ERR_INVALID_ARG, "pq_sizes")
    return rw, ns


def pq_nearest(y, cb) -> int:
    """Index of the nearest bf16-rounded centroid of cb [k, d] to y [d]
    ([TTAS] 2.2 product quantisation; fp64 distance, lowest index on ties)."""
    y = np.ascontiguousarray(y, np.float32)
    cb = np.ascontiguousarray(cb, np.float32)
    return int(lib().orc_pq_nearest(_p(y), _p(cb), cb.shape[0], cb.shape[1]))


def pq_encode(cfg: dict, pq: dict, v, cb1, cb2):
    """TTAS-X2 value path ([TTAS] 2.2): (codes u32 [L,H,T,row_words], rms f32
    [L,H,T], outliers u32 [L,H,blocks,budget,2])."""
    c, q = make_cfg(cfg), _PqCfg(**pq)
    L, H, T = cfg["layers"], cfg["kv_heads"], v.shape[2]
    rw, ns = pq_sizes(cfg, pq, T)
    nblk = -(-T // pq["block_tokens"])
    codes = np.zeros((L, H, T, rw), np.uint32)
    rms_ = np.zeros((L, H, T), np.float32)
    outl = np.zeros((L, H, nblk, pq["outliers"], 2), np.uint32)
    vv = np.ascontiguousarray(v)
    a1, a2 = np.ascontiguousarray(cb1, np.float32), np.ascontiguousarray(cb2, np.float32)
    st = lib().orc_pq_encode(ctypes.byref(c), ctypes.byref(q), _p(vv), T, _p(a1), _p(a2), _p(codes), _p(rms_),
                             _p(outl) if outl.size else None)
    if st != OK:
        raise OracleError(st, "pq_encode")
    return codes, rms_, outl


def pq_decode(cfg: dict, pq: dict, codes, rms_, outl, T: int, cb1, cb2) -> np.ndarray:
    c, q = make_cfg(cfg), _PqCfg(**pq)
    out = np.zeros((cfg["layers"], cfg["kv_heads"], T, cfg["head_dim"]), np.float32)
    cs = np.ascontiguousarray(codes, np.uint32)
    rs = np.ascontiguousarray(rms_, np.float32)
    ol = np.ascontiguousarray(outl, np.uint32)
    a1, a2 = np.ascontiguousarray(cb1, np.float32), np.ascontiguousarray(cb2, np.float32)
    st = lib().orc_pq_decode(ctypes.byref(c), ctypes.byref(q), _p(cs), _p(rs), _p(ol) if ol.size else None, T,
                             _p(a1), _p(a2), _p(out))
    if st != OK:
        raise OracleError(st, "pq_decode")
    return out


def fnv1a64(data: bytes, h: int = 0xCBF29CE484222325) -> int:
    buf = np.frombuffer(bytes(data), np.uint8).copy()
    return int(lib().orc_fnv1a64(h, _p(buf) if buf.size else None, buf.size))


def fingerprint(cfg: dict, basis: np.ndarray | None) -> int:
    c = make_cfg(cfg)
    b = None if basis is None else np.ascontiguousarray(basis, np.float32)
    return int(lib().orc_fingerprint(ctypes.byref(c), _p(b)))


def max_container_bytes(cfg: dict, T: int) -> int:
    c = make_cfg(cfg)
    return int(lib().orc_max_container_bytes(ctypes.byref(c), T))


def encode(cfg: dict, k: np.ndarray, v: np.ndarray, basis: np.ndarray | None) -> bytes:
    """k, v: [L, H, T, D] (float32, or uint16 bf16 bit patterns)."""
    c = make_cfg(cfg)
    T = k.shape[2]
    cap = max_container_bytes(cfg, T)
    if cap < 0:
        raise OracleError(ERR_INVALID_ARG, "encode")
    out = np.zeros(cap, np.uint8)
    n = ctypes.c_int64(0)
    b = None if basis is None else np.ascontiguousarray(basis, np.float32)
    kk = np.ascontiguousarray(k)
    vv = np.ascontiguousarray(v)
    st = lib().orc_encode(ctypes.byref(c), _tensor_ptr(kk, cfg["dtype"]),
                          _tensor_ptr(vv, cfg["dtype"]), T, _p(b), _p(out), cap, ctypes.byref(n))
    if st != OK:
        raise OracleError(st, "encode")
    return out[: n.value].tobytes()


def decode(cfg: dict, data: bytes, basis: np.ndarray | None, T: int, out_dtype: int = FP32):
    c = make_cfg(cfg)
    shape = (cfg["layers"], cfg["kv_heads"], T, cfg["head_dim"])
    npdt = np.float32 if out_dtype == FP32 else np.uint16
    k = np.zeros(shape, npdt)
    v = np.zeros(shape, npdt)
    buf = np.frombuffer(data, np.uint8).copy()
    b = None if basis is None else np.ascontiguousarray(basis, np.float32)
    st = lib().orc_decode(ctypes.byref(c), _p(b), _p(buf), buf.size, _p(k), _p(v), out_dtype)
    if st != OK:
        raise OracleError(st, "decode")
    return k, v


def decode_status(cfg: dict, data: bytes, basis: np.ndarray | None, T: int) -> int:
    """Status of a full decode (used by corruption tests)."""
    try:
        decode(cfg, data, basis, T)
    except OracleError as e:
        return e.status
    return OK


def decode_sections(cfg: dict, data: bytes, basis, sec_begin: int, sec_end: int, T_mid: int):
    c = make_cfg(cfg)
    out = np.zeros((sec_end - sec_begin, max(T_mid, 1), cfg["head_dim"]), np.float32)
    buf = np.frombuffer(data, np.uint8).copy()
    b = None if basis is None else np.ascontiguousarray(basis, np.float32)
    st = lib().orc_decode_sections(ctypes.byref(c), _p(b), _p(buf), buf.size, sec_begin, sec_end,
                                   _p(out))
    if st != OK:
        raise OracleError(st, "decode_sections")
    return out[:, :T_mid]


def section_codes(cfg: dict, data: bytes, basis, section: int, T: int) -> np.ndarray:
    """Codes [T_mid, D] of one section, read back from a container."""
    c = make_cfg(cfg)
    lo = layout(cfg, T)
    q = np.zeros((max(lo.T_mid, 1), cfg["head_dim"]), np.uint8)
    buf = np.frombuffer(data, np.uint8).copy()
    b = None if basis is None else np.ascontiguousarray(basis, np.float32)
    st = lib().orc_section_codes(ctypes.byref(c), _p(b), _p(buf), buf.size, section, _p(q))
    if st != OK:
        raise OracleError(st, "section_codes")
    return q[: lo.T_mid]


def section_rows(cfg: dict, k, v, section: int, t0: int, t1: int) -> np.ndarray:
    c = make_cfg(cfg)
    T = k.shape[2]
    out = np.zeros((max(t1 - t0, 1), cfg["head_dim"]), np.float32)
    st = lib().orc_section_rows(ctypes.byref(c), _tensor_ptr(np.ascontiguousarray(k), cfg["dtype"]),
                                _tensor_ptr(np.ascontiguousarray(v), cfg["dtype"]), T, section,
                                t0, t1, _p(out))
    if st != OK:
        raise OracleError(st, "section_rows")
    return out[: t1 - t0]


def section_coeffs(cfg: dict, k, v, basis, section: int):
    """(coefficients [T_mid, D], r [T_mid]) of one section as the encoder computes them."""
    c = make_cfg(cfg)
    T = k.shape[2]
    lo = layout(cfg, T)
    out = np.zeros((max(lo.T_mid, 1), cfg["head_dim"]), np.float32)
    r = np.zeros(max(lo.T_mid, 1), np.float32)
    b = None if basis is None else np.ascontiguousarray(basis, np.float32)
    st = lib().orc_section_coeffs(ctypes.byref(c), _tensor_ptr(np.ascontiguousarray(k), cfg["dtype"]),
                                  _tensor_ptr(np.ascontiguousarray(v), cfg["dtype"]), T, _p(b),
                                  section, _p(out), _p(r))
    if st != OK:
        raise OracleError(st, "section_coeffs")
    return out[: lo.T_mid], r[: lo.T_mid]


@dataclass
class Layout:
    T: int
    s0: int
    mid_begin: int
    mid_end: int
    T_mid: int
    W_eff: int
    n_sections: int
    chunks_per_sec: int


def layout(cfg: dict, T: int) -> Layout:
    """Region split ([KVTC] "How the Pipeline Works"): sink [0, S'), middle
    [S', max(S', T - W)), recent window after it."""
    s0 = min(cfg["sink_tokens"], T)
    mid_end = max(s0, T - cfg["recent_tokens"])
    T_mid = mid_end - s0
    nsec = cfg["layers"] * 2 * cfg["kv_heads"]
    cps = (T_mid + cfg["chunk_tokens"] - 1) // cfg["chunk_tokens"] if T_mid > 0 else 0
    return Layout(T, s0, s0, mid_end, T_mid, T - mid_end, nsec, cps)


def parse_container(data: bytes, cfg: dict, T: int) -> dict:
    """Section records (bits, zero, scale) and directory of a container, read
    with plain numpy views (for parity tests)."""
    lo = layout(cfg, T)
    D = cfg["head_dim"]
    buf = np.frombuffer(data, np.uint8)
    hdr = buf[:256]
    side_off = int(hdr[120:128].view(np.uint64)[0])
    dir_off = int(hdr[152:160].view(np.uint64)[0])
    chunks_off = int(hdr[160:168].view(np.uint64)[0])
    total = int(hdr[168:176].view(np.uint64)[0])
    recs = buf[side_off: side_off + lo.n_sections * 9 * D].reshape(lo.n_sections, 9 * D)
    bits = recs[:, :D].copy()
    zero = recs[:, D: 5 * D].copy().view(np.float32)
    scale = recs[:, 5 * D: 9 * D].copy().view(np.float32)
    nch = lo.n_sections * lo.chunks_per_sec
    d = buf[dir_off: dir_off + 32 * nch].reshape(max(nch, 0), 32)
    offs = d[:, :8].copy().view(np.uint64).ravel()
    sizes = d[:, 8:12].copy().view(np.uint32).ravel()
    modes = d[:, 12:16].copy().view(np.uint32).ravel()
    csums = d[:, 16:32].copy().view(np.uint64).reshape(-1, 2)
    return dict(bits=bits, zero=zero, scale=scale, offsets=offs, sizes=sizes, modes=modes, csums=csums,
                fixed_csum=(int(hdr[200:208].view(np.uint64)[0]), int(hdr[208:216].view(np.uint64)[0])),
                chunks_off=chunks_off, total=total, layout=lo,
                fingerprint=int(hdr[176:184].view(np.uint64)[0]))


# --------------------------------------------------------------------------
# calibration (offline input of the method)
# --------------------------------------------------------------------------

def fit_pca_basis(cfg: dict, k, v, t0: int | None = None, t1: int | None = None) -> np.ndarray:
    """Uncentered second-moment eigenbasis per (layer, K/V) -- or per head when
    cfg["basis_per_head"] -- over rows t0..t1 (keys un-rotated by the oracle).
    Columns are components in descending eigenvalue order; each column's
    largest-magnitude entry is made positive.  Returns fp32
    [L, 2, D, D] (or [L, 2, H, D, D])."""
    L, H, T, D = cfg["layers"], cfg["kv_heads"], k.shape[2], cfg["head_dim"]
    t0 = 0 if t0 is None else t0
    t1 = T if t1 is None else t1
    per_head = bool(cfg["basis_per_head"])
    out = np.zeros((L, 2, H, D, D) if per_head else (L, 2, D, D), np.float32)
    for l in range(L):
        for s in range(2):
            acc = np.zeros((D, D), np.float64)
            n = 0
            for h in range(H):
                u = (l * 2 + s) * H + h
                x = section_rows(cfg, k, v, u, t0, t1).astype(np.float64)
                if per_head:
                    out[l, s, h] = _eig_basis(x.T @ x / max(x.shape[0], 1))
                else:
                    acc += x.T @ x
                    n += x.shape[0]
            if not per_head:
                out[l, s] = _eig_basis(acc / max(n, 1))
    return out


def gauge_block(A: np.ndarray) -> np.ndarray:
    """One orthogonal gauge block G = exp(A - A^T) ("Codec-Gauge: Learning
    Compression-Friendly Gauges for Transformer KV Caches", Gauge
    Parameterization and Training: a skew-symmetric generator per channel
    group), in fp64 by the matrix exponential of scipy."""
    from scipy.linalg import expm
    A = np.asarray(A, np.float64)
    return expm(A - A.T)


def grouped_gauge(D: int, g: int, generators) -> np.ndarray:
    """Block-diagonal gauge G = diag(exp(A_k - A_k^T)) over D / g groups of g
    consecutive channels (same page, Gauge Parameterization: groups of g
    channels, g in {8, 16, 32}); `generators` is [D / g, g, g] (the learned
    parameters; here any given matrices, training is not part of the codec).
    The frame is Z = G X, so as a basis (column i = component i) it enters
    the pipeline as B = G^T.  Returns fp64 [D, D]."""
    assert D % g == 0
    G = np.zeros((D, D), np.float64)
    for k in range(D // g):
        G[k * g:(k + 1) * g, k * g:(k + 1) * g] = gauge_block(generators[k])
    return G


def random_gauge_generators(D: int, g: int, scale: float, seed: int) -> np.ndarray:
    """Seeded normal generators [D / g, g, g] of standard deviation `scale`:
    the random-gauge control of the same page (Compression Conditions)."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, scale, (D // g, g, g))


def grouped_klt_basis(cfg: dict, k, v, g: int, t0: int | None = None, t1: int | None = None) -> np.ndarray:
    """The PCA/KLT control at group granularity (same page, Compression
    Conditions: the uncentered second-moment eigenbasis computed per layer,
    K/V and group): within each group of g consecutive channels the
    eigenvectors of that group's block of the second moment, descending.
    Block-diagonal fp32 [L, 2, D, D] like fit_pca_basis."""
    full = fit_pca_basis(dict(cfg, basis_per_head=0), k, v, t0, t1)  # only for the shape
    L, D = cfg["layers"], cfg["head_dim"]
    H, T = cfg["kv_heads"], k.shape[2]
    t0 = 0 if t0 is None else t0
    t1 = T if t1 is None else t1
    out = np.zeros_like(full)
    for l in range(L):
        for s in range(2):
            acc = np.zeros((D, D), np.float64)
            n = 0
            for h in range(H):
                x = section_rows(cfg, k, v, (l * 2 + s) * H + h, t0, t1).astype(np.float64)
                acc += x.T @ x
                n += x.shape[0]
            S = acc / max(n, 1)
            for q in range(D // g):
                sl = slice(q * g, (q + 1) * g)
                out[l, s, sl, sl] = _eig_basis(S[sl, sl])
    return out


def _eig_basis(S: np.ndarray) -> np.ndarray:
    w, V = np.linalg.eigh(S)
    order = np.argsort(-w, kind="stable")
    V = V[:, order]
    idx = np.argmax(np.abs(V), axis=0)
    sign = np.sign(V[idx, np.arange(V.shape[1])])
    sign[sign == 0] = 1
    return (V * sign).astype(np.float32)


def eig_values(cfg: dict, k, v, l: int, s: int, t0=None, t1=None) -> np.ndarray:
    """Eigenvalues (descending) of the pooled uncentered second moment of (l, s)."""
    H, T, D = cfg["kv_heads"], k.shape[2], cfg["head_dim"]
    t0 = 0 if t0 is None else t0
    t1 = T if t1 is None else t1
    acc = np.zeros((D, D), np.float64)
    n = 0
    for h in range(H):
        x = section_rows(cfg, k, v, (l * 2 + s) * H + h, t0, t1).astype(np.float64)
        acc += x.T @ x
        n += x.shape[0]
    return np.sort(np.linalg.eigvalsh(acc / n))[::-1]
