"""Thin ctypes binding of libkvtc (declared in include/kvtc.h).

Argument marshalling only: every step of encode and decode runs in the HIP
kernels of ``libkvtc.so``.  PyTorch supplies device memory and the current
stream.  The library must have been built (``tensor_compression_amd.build``);
there is no fallback path and loading raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvtc.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_CORRUPT, ERR_NONFINITE, ERR_HIP = range(7)
FP32, BF16 = 0, 1
PCA, WHT = 0, 1
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "CAPACITY", 4: "CORRUPT",
          5: "NONFINITE", 6: "HIP"}


class KvtcError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: KVTC_{STATUS.get(status, status)}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("transform", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32), ("recent_tokens", ctypes.c_int32),
        ("bits_k", ctypes.c_float), ("bits_v", ctypes.c_float), ("max_bits", ctypes.c_int32),
        ("rope_keys", ctypes.c_int32), ("rope_style", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("rans_scale_bits", ctypes.c_int32),
        ("rans_lanes", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32), ("basis_per_head", ctypes.c_int32),
        ("wht_keys", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
    ]


EXPORTS = {
    # name: (restype, argtypes)
    "kvtc_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kvtc_plan_mem_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
    "kvtc_plan": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]),
    "kvtc_plan_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "kvtc_plan_fingerprint": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64)]),
    "kvtc_workspace_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]),
    "kvtc_encode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]),
    "kvtc_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]),
    "kvtc_workspace_size_paged": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                                 ctypes.POINTER(ctypes.c_size_t),
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "kvtc_encode_paged": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "kvtc_decode_paged": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "kvtc_result": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64),
                                   ctypes.POINTER(ctypes.c_int32)]),
    "kvtc_encode_counters": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.POINTER(ctypes.c_uint64)]),
    "kvtc_profile_enable": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kvtc_profile_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_float),
                                         ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_int32)]),
    "kvtc_test_section_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p]),
    "kvtc_test_coeffs": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kvtc_test_rans_encode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "kvtc_test_rans_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "kvtc_test_freq_table": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Open libkvtc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m tensor_compression_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != OK:
        raise KvtcError(st, what)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    assert t.is_contiguous()
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_config(cfg: dict, max_tokens: int) -> Config:
    c = Config()
    for f, _ in Config._fields_:
        if f == "max_tokens":
            c.max_tokens = max_tokens
        else:
            setattr(c, f, cfg[f])
    return c


class Plan:
    """A plan: configuration, operand-precision basis and RoPE table in device
    memory owned by this object."""

    def __init__(self, cfg: dict, basis: torch.Tensor | None, max_tokens: int, device="cuda"):
        self.cfg = dict(cfg)
        self.max_tokens = max_tokens
        self.device = torch.device(device)
        self._c = make_config(cfg, max_tokens)
        n = ctypes.c_size_t(0)
        _check(lib().kvtc_plan_mem_size(ctypes.byref(self._c), ctypes.byref(n)), "kvtc_plan_mem_size")
        self.mem = torch.empty(n.value, dtype=torch.uint8, device=self.device)
        b = None
        if basis is not None:
            b = basis.to(device=self.device, dtype=torch.float32).contiguous()
        h = ctypes.c_void_p()
        _check(lib().kvtc_plan(ctypes.byref(self._c), _ptr(b), _ptr(self.mem), n.value, _stream(),
                               ctypes.byref(h)), "kvtc_plan")
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            lib().kvtc_plan_destroy(h)
            self.handle = None

    def fingerprint(self) -> int:
        v = ctypes.c_uint64(0)
        _check(lib().kvtc_plan_fingerprint(self.handle, ctypes.byref(v)), "kvtc_plan_fingerprint")
        return v.value

    def sizes(self, T: int):
        ws = ctypes.c_size_t(0)
        mc = ctypes.c_size_t(0)
        _check(lib().kvtc_workspace_size(self.handle, T, ctypes.byref(ws), ctypes.byref(mc)),
               "kvtc_workspace_size")
        return ws.value, mc.value

    def workspace(self, T: int) -> torch.Tensor:
        ws, _ = self.sizes(T)
        return torch.empty(ws, dtype=torch.uint8, device=self.device)

    def encode_async(self, K: torch.Tensor, V: torch.Tensor, out: torch.Tensor, ws: torch.Tensor,
                     stream=None):
        T = K.shape[2]
        _check(lib().kvtc_encode(self.handle, _ptr(K), _ptr(V), T, _ptr(out), out.numel(), _ptr(ws),
                                 ws.numel(), _stream(stream)), "kvtc_encode")

    def decode_async(self, data: torch.Tensor, nbytes: int, T: int, k_out: torch.Tensor,
                     v_out: torch.Tensor, ws: torch.Tensor, out_dtype: int | None = None,
                     stream=None):
        od = out_dtype if out_dtype is not None else (BF16 if k_out.dtype == torch.bfloat16 else FP32)
        _check(lib().kvtc_decode(self.handle, _ptr(data), nbytes, T, _ptr(k_out), _ptr(v_out), od,
                                 _ptr(ws), ws.numel(), _stream(stream)), "kvtc_decode")

    def result(self, ws: torch.Tensor):
        n = ctypes.c_uint64(0)
        st = ctypes.c_int32(0)
        _check(lib().kvtc_result(self.handle, _ptr(ws), ctypes.byref(n), ctypes.byref(st)),
               "kvtc_result")
        return n.value, st.value

    def exact_recomputed(self, ws: torch.Tensor) -> int:
        n = ctypes.c_uint64(0)
        _check(lib().kvtc_encode_counters(self.handle, _ptr(ws), ctypes.byref(n)),
               "kvtc_encode_counters")
        return n.value

    # convenience wrappers (synchronising)
    def encode(self, K: torch.Tensor, V: torch.Tensor, ws: torch.Tensor | None = None):
        """Encode and return (container bytes on the device, device status)."""
        T = K.shape[2]
        wsz, cap = self.sizes(T)
        ws = ws if ws is not None else torch.empty(wsz, dtype=torch.uint8, device=self.device)
        out = torch.empty(cap, dtype=torch.uint8, device=self.device)
        self.encode_async(K, V, out, ws)
        torch.cuda.current_stream().synchronize()
        n, st = self.result(ws)
        return out[:n], st

    def decode(self, data: torch.Tensor, T: int, out_dtype: int = FP32,
               ws: torch.Tensor | None = None):
        """Decode and return (K, V, device status)."""
        shape = (self.cfg["layers"], self.cfg["kv_heads"], T, self.cfg["head_dim"])
        dt = torch.float32 if out_dtype == FP32 else torch.bfloat16
        k = torch.empty(shape, dtype=dt, device=self.device)
        v = torch.empty(shape, dtype=dt, device=self.device)
        ws = ws if ws is not None else self.workspace(T)
        self.decode_async(data, data.numel(), T, k, v, ws, out_dtype)
        torch.cuda.current_stream().synchronize()
        _, st = self.result(ws)
        return k, v, st

    # paged ragged batches: pools [L, P, H, 16, D], page_table [n_seqs, max_pages]
    # int32 on the device, seq_lens as a host list (copied to the device here)
    def sizes_paged(self, seq_lens):
        lens = (ctypes.c_int32 * len(seq_lens))(*[int(x) for x in seq_lens])
        ws = ctypes.c_size_t(0)
        mc = ctypes.c_size_t(0)
        _check(lib().kvtc_workspace_size_paged(self.handle, len(seq_lens), lens, ctypes.byref(ws),
                                               ctypes.byref(mc)), "kvtc_workspace_size_paged")
        return ws.value, mc.value

    @staticmethod
    def _paged_args(k_pool, page_table, seq_lens, seq_lens_dev):
        lens = (ctypes.c_int32 * len(seq_lens))(*[int(x) for x in seq_lens])
        assert page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous()
        assert seq_lens_dev.dtype == torch.int32 and seq_lens_dev.numel() == len(seq_lens)
        return k_pool.shape[1], page_table.shape[1], lens

    def encode_paged_async(self, k_pool, v_pool, page_table, seq_lens, seq_lens_dev, out, ws, stream=None):
        P, max_pages, lens = self._paged_args(k_pool, page_table, seq_lens, seq_lens_dev)
        _check(lib().kvtc_encode_paged(self.handle, _ptr(k_pool), _ptr(v_pool), P, _ptr(page_table), max_pages,
                                       _ptr(seq_lens_dev), lens, len(seq_lens), _ptr(out), out.numel(), _ptr(ws),
                                       ws.numel(), _stream(stream)), "kvtc_encode_paged")

    def decode_paged_async(self, data, nbytes, k_pool, v_pool, page_table, seq_lens, seq_lens_dev, ws,
                           stream=None):
        P, max_pages, lens = self._paged_args(k_pool, page_table, seq_lens, seq_lens_dev)
        _check(lib().kvtc_decode_paged(self.handle, _ptr(data), nbytes, _ptr(k_pool), _ptr(v_pool), P,
                                       _ptr(page_table), max_pages, _ptr(seq_lens_dev), lens, len(seq_lens),
                                       _ptr(ws), ws.numel(), _stream(stream)), "kvtc_decode_paged")

    # profiling
    def profile(self, on: bool = True):
        _check(lib().kvtc_profile_enable(self.handle, 1 if on else 0), "kvtc_profile_enable")

    def profile_read(self):
        """[(phase name, ms)] of the last encode or decode (synchronises)."""
        ms = (ctypes.c_float * 24)()
        names = (ctypes.c_char_p * 24)()
        n = ctypes.c_int32(0)
        _check(lib().kvtc_profile_read(self.handle, 24, ms, names, ctypes.byref(n)),
               "kvtc_profile_read")
        return [(names[i].decode(), float(ms[i])) for i in range(n.value)]

    # parity hooks
    def section_stats(self, ws: torch.Tensor, T: int, n_sections: int):
        D = self.cfg["head_dim"]
        arrs = [(ctypes.c_float * (n_sections * D))() for _ in range(4)]
        _check(lib().kvtc_test_section_stats(self.handle, _ptr(ws), T, *arrs), "section_stats")
        import numpy as np
        return [np.ctypeslib.as_array(a).reshape(n_sections, D).copy() for a in arrs]

    def coeffs(self, K: torch.Tensor, V: torch.Tensor, sec_begin: int, sec_end: int, T_mid: int):
        D = self.cfg["head_dim"]
        n = sec_end - sec_begin
        out = torch.zeros((n, max(T_mid, 1), D), dtype=torch.float32, device=self.device)
        r = torch.zeros((n, max(T_mid, 1)), dtype=torch.float32, device=self.device)
        _check(lib().kvtc_test_coeffs(self.handle, _ptr(K), _ptr(V), K.shape[2], sec_begin, sec_end,
                                      _ptr(out), _ptr(r), _stream()), "kvtc_test_coeffs")
        torch.cuda.current_stream().synchronize()
        return out[:, :T_mid], r[:, :T_mid]


def rans_encode(sym: torch.Tensor, freq: torch.Tensor, scale_bits: int, lanes: int):
    """Device single-stream coder (parity hook): returns (states, words)."""
    N = sym.numel()
    cap = (N * (scale_bits + 1)) // 16 + 2 * lanes + 2
    dev = freq.device
    states = torch.zeros(lanes, dtype=torch.int32, device=dev)
    words = torch.zeros(max(cap, 1), dtype=torch.int16, device=dev)
    nw = torch.zeros(1, dtype=torch.int64, device=dev)
    symb = sym if N else torch.zeros(1, dtype=torch.uint8, device=dev)
    _check(lib().kvtc_test_rans_encode(_ptr(symb), N, _ptr(freq), scale_bits, lanes, _ptr(states),
                                       _ptr(words), cap, _ptr(nw), _stream()), "rans_encode")
    torch.cuda.current_stream().synchronize()
    n = int(nw.item())
    return states, words[:max(n, 0)], n


def rans_decode(states: torch.Tensor, words: torch.Tensor, freq: torch.Tensor, N: int,
                scale_bits: int, lanes: int):
    dev = freq.device
    out = torch.zeros(max(N, 1), dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    wb = words if words.numel() else torch.zeros(1, dtype=torch.int16, device=dev)
    _check(lib().kvtc_test_rans_decode(_ptr(states), _ptr(wb), words.numel(), _ptr(freq), scale_bits,
                                       lanes, N, _ptr(out), _ptr(st), _stream()), "rans_decode")
    torch.cuda.current_stream().synchronize()
    return out[:N], int(st.item())


def freq_table(counts: torch.Tensor, scale_bits: int):
    f = torch.zeros(256, dtype=torch.int16, device=counts.device)
    _check(lib().kvtc_test_freq_table(_ptr(counts), scale_bits, _ptr(f), _stream()), "freq_table")
    torch.cuda.current_stream().synchronize()
    return f
