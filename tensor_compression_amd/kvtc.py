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
SQ_BLOCK, SQ_KIVI = 1, 2
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
        ("alloc_scope", ctypes.c_int32),
    ]


class SqConfig(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("group", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("bits_k", ctypes.c_int32), ("bits_v", ctypes.c_int32)]


class PqConfig(ctypes.Structure):
    _fields_ = [("sub_dim", ctypes.c_int32), ("k1", ctypes.c_int32), ("k2", ctypes.c_int32),
                ("outliers", ctypes.c_int32), ("block_tokens", ctypes.c_int32)]


def make_pq_config(pq: dict) -> PqConfig:
    return PqConfig(pq["sub_dim"], pq["k1"], pq["k2"], pq["outliers"], pq["block_tokens"])


def make_sq_config(sq: dict) -> SqConfig:
    return SqConfig(sq["kind"], sq["group"], sq["tile"], sq["bits_k"], sq["bits_v"])


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
    "kvtc_decode_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p]),
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
    "kvtc_test_freq_tables": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "kvtc_test_packed_tiles": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kvtc_test_rope": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "kvtc_test_alloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "kvtc_test_quant_pack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "kvtc_test_dequant_project": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int32, ctypes.c_void_p]),
    "kvtc_pq_sizes": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.POINTER(ctypes.c_size_t)]),
    "kvtc_pq_encode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "kvtc_pq_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "kvtc_sq_sizes": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "kvtc_sq_encode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "kvtc_sq_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
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
        elif f == "alloc_scope":
            c.alloc_scope = cfg.get("alloc_scope", 0)
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

    def decode_noalloc_async(self, data: torch.Tensor, nbytes: int, T: int, k_out: torch.Tensor,
                             v_out: torch.Tensor, status: torch.Tensor | None, out_dtype: int = FP32,
                             stream=None):
        """kvtc_decode_noalloc: decode in the library's fixed device array;
        the status word goes to `status` (device int32 [1]) when given."""
        _check(lib().kvtc_decode_noalloc(self.handle, _ptr(data), nbytes, T, _ptr(k_out), _ptr(v_out),
                                         out_dtype, _ptr(status), _stream(stream)), "kvtc_decode_noalloc")

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

    def packed_tiles(self, ws: torch.Tensor, T: int, section: int) -> torch.Tensor:
        """The packed tiles of one section left in ws by the last encode (or
        decode), as its work-block slots hold them: uint8 [blocks, slot bytes]."""
        nb, sb = ctypes.c_int32(0), ctypes.c_size_t(0)
        _check(lib().kvtc_test_packed_tiles(self.handle, _ptr(ws), T, section, None, 0, ctypes.byref(nb),
                                            ctypes.byref(sb), _stream()), "kvtc_test_packed_tiles")
        out = torch.zeros(max(nb.value * sb.value, 1), dtype=torch.uint8, device=self.device)
        _check(lib().kvtc_test_packed_tiles(self.handle, _ptr(ws), T, section, _ptr(out), out.numel(), None, None,
                                            _stream()), "kvtc_test_packed_tiles")
        torch.cuda.current_stream().synchronize()
        return out[: nb.value * sb.value].view(nb.value, sb.value)


    def rope_stage(self, K: torch.Tensor, ws: torch.Tensor, T_mid: int) -> torch.Tensor:
        """kvtc_test_rope: the middle keys un-rotated, bf16 bits int16 [L, H, T_mid, D]."""
        L, H, T, D = K.shape
        out = torch.zeros((L, H, max(T_mid, 1), D), dtype=torch.int16, device=self.device)
        _check(lib().kvtc_test_rope(self.handle, _ptr(K), T, _ptr(ws), ws.numel(), _ptr(out), out.numel() * 2,
                                    _stream()), "kvtc_test_rope")
        torch.cuda.current_stream().synchronize()
        return out[:, :, :T_mid]

    def alloc_stage(self, T: int, stats, ws: torch.Tensor):
        """kvtc_test_alloc: host stats float32 [n_sections, D, 4] -> (widths u8,
        zero f32, scale f32), each [n_sections, D]."""
        import numpy as np
        st = np.ascontiguousarray(stats, np.float32)
        n, D = st.shape[0], st.shape[1]
        side = torch.zeros(n * 9 * D, dtype=torch.uint8, device=self.device)
        _check(lib().kvtc_test_alloc(self.handle, T, st.ctypes.data_as(ctypes.c_void_p), _ptr(ws), ws.numel(),
                                     _ptr(side), side.numel(), _stream()), "kvtc_test_alloc")
        torch.cuda.current_stream().synchronize()
        rec = side.cpu().numpy().reshape(n, 9 * D)
        return rec[:, :D].copy(), rec[:, D: 5 * D].copy().view(np.float32), rec[:, 5 * D:].copy().view(np.float32)

    def quant_pack_stage(self, K: torch.Tensor, V: torch.Tensor, ws: torch.Tensor, out: torch.Tensor):
        """kvtc_test_quant_pack: encode passes up to packing; section records
        into `out`, packed tiles left in ws."""
        _check(lib().kvtc_test_quant_pack(self.handle, _ptr(K), _ptr(V), K.shape[2], _ptr(out), out.numel(),
                                          _ptr(ws), ws.numel(), _stream()), "kvtc_test_quant_pack")
        torch.cuda.current_stream().synchronize()

    def dequant_project_stage(self, side: torch.Tensor, T: int, ws: torch.Tensor, k_out: torch.Tensor,
                              v_out: torch.Tensor, out_dtype: int):
        """kvtc_test_dequant_project: the decode transform from ws's packed
        tiles and the section records in `side` into the middle rows."""
        _check(lib().kvtc_test_dequant_project(self.handle, _ptr(side), side.numel(), T, _ptr(ws), ws.numel(),
                                               _ptr(k_out), _ptr(v_out), out_dtype, _stream()),
               "kvtc_test_dequant_project")
        torch.cuda.current_stream().synchronize()

    # ---- scalar quantisers on gauge coordinates (kvtc_sq_*)

    def sq_sizes(self, sq: dict, T: int):
        """(code bytes, range pairs) of a kvtc_sq_encode call over T tokens."""
        c = make_sq_config(sq)
        nb, nr = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _check(lib().kvtc_sq_sizes(self.handle, ctypes.byref(c), T, ctypes.byref(nb), ctypes.byref(nr)),
               "kvtc_sq_sizes")
        return nb.value, nr.value

    def sq_encode_async(self, sq: dict, K: torch.Tensor, V: torch.Tensor, codes: torch.Tensor,
                        ranges: torch.Tensor, status: torch.Tensor | None, stream=None):
        c = make_sq_config(sq)
        _check(lib().kvtc_sq_encode(self.handle, ctypes.byref(c), _ptr(K), _ptr(V), K.shape[2], _ptr(codes),
                                    codes.numel(), _ptr(ranges), ranges.numel() // 2, _ptr(status),
                                    _stream(stream)), "kvtc_sq_encode")

    def sq_encode(self, sq: dict, K: torch.Tensor, V: torch.Tensor):
        """kvtc_sq_encode: returns (codes uint8, ranges float32 [pairs, 2],
        status word)."""
        T = K.shape[2]
        nb, nr = self.sq_sizes(sq, T)
        codes = torch.empty(max(nb, 16), dtype=torch.uint8, device=self.device)
        ranges = torch.empty((max(nr, 1), 2), dtype=torch.float32, device=self.device)
        status = torch.zeros(4, dtype=torch.int32, device=self.device)
        self.sq_encode_async(sq, K, V, codes, ranges, status)
        torch.cuda.synchronize(self.device)
        return codes[:nb], ranges[:nr], int(status[0].item())

    def sq_decode_async(self, sq: dict, codes: torch.Tensor, ranges: torch.Tensor, T: int,
                        k_out: torch.Tensor, v_out: torch.Tensor, out_dtype: int = FP32, stream=None):
        c = make_sq_config(sq)
        _check(lib().kvtc_sq_decode(self.handle, ctypes.byref(c), _ptr(codes), codes.numel(), _ptr(ranges),
                                    ranges.numel() // 2, T, _ptr(k_out), _ptr(v_out), out_dtype,
                                    _stream(stream)), "kvtc_sq_decode")

    def sq_decode(self, sq: dict, codes: torch.Tensor, ranges: torch.Tensor, T: int, out_dtype: int = FP32):
        """kvtc_sq_decode into new [L, H, T, D] tensors of out_dtype."""
        c = self.cfg
        shape = (c["layers"], c["kv_heads"], T, c["head_dim"])
        dt = torch.float32 if out_dtype == FP32 else torch.bfloat16
        k_out = torch.empty(shape, dtype=dt, device=self.device)
        v_out = torch.empty(shape, dtype=dt, device=self.device)
        self.sq_decode_async(sq, codes, ranges, T, k_out, v_out, out_dtype)
        torch.cuda.synchronize(self.device)
        return k_out, v_out

    # ---- TTAS-X2 value path (kvtc_pq_*)

    def pq_sizes(self, pq: dict, T: int):
        """(code bytes, outlier slots, workspace bytes) of a call over T tokens."""
        c = make_pq_config(pq)
        a, b, w = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
        _check(lib().kvtc_pq_sizes(self.handle, ctypes.byref(c), T, ctypes.byref(a), ctypes.byref(b),
                                   ctypes.byref(w)), "kvtc_pq_sizes")
        return a.value, b.value, w.value

    def pq_buffers(self, pq: dict, T: int):
        """Fresh device buffers (codes u32, rms f32, outliers u32 [slots, 2], workspace)."""
        nb, ns, wb = self.pq_sizes(pq, T)
        L, H = self.cfg["layers"], self.cfg["kv_heads"]
        codes = torch.zeros(max(nb // 4, 4), dtype=torch.int32, device=self.device)
        rms = torch.zeros(max(L * H * T, 4), dtype=torch.float32, device=self.device)
        outl = torch.zeros((max(ns, 2), 2), dtype=torch.int32, device=self.device)
        ws = torch.empty(max(wb, 256), dtype=torch.uint8, device=self.device)
        return codes, rms, outl, ws

    def pq_encode_async(self, pq: dict, cb1, cb2, V, codes, rms, outl, ws, status, stream=None):
        c = make_pq_config(pq)
        _check(lib().kvtc_pq_encode(self.handle, ctypes.byref(c), _ptr(cb1), _ptr(cb2), _ptr(V), V.shape[2],
                                    _ptr(codes), codes.numel() * 4, _ptr(rms), rms.numel(), _ptr(outl),
                                    outl.numel() // 2, _ptr(ws), ws.numel(), _ptr(status), _stream(stream)),
               "kvtc_pq_encode")

    def pq_decode_async(self, pq: dict, cb1, cb2, codes, rms, outl, T, v_out, ws, status, out_dtype=FP32,
                        stream=None):
        c = make_pq_config(pq)
        _check(lib().kvtc_pq_decode(self.handle, ctypes.byref(c), _ptr(cb1), _ptr(cb2), _ptr(codes),
                                    codes.numel() * 4, _ptr(rms), _ptr(outl), outl.numel() // 2, T, _ptr(v_out),
                                    out_dtype, _ptr(ws), ws.numel(), _ptr(status), _stream(stream)),
               "kvtc_pq_decode")

    def pq_encode(self, pq: dict, cb1, cb2, V):
        """kvtc_pq_encode: (codes [L,H,T,row_words] u32 as int32, rms [L,H,T],
        outliers [L,H,blocks,budget,2] as int32, status word)."""
        L, H, T = V.shape[0], V.shape[1], V.shape[2]
        nb, ns, _ = self.pq_sizes(pq, T)
        codes, rms, outl, ws = self.pq_buffers(pq, T)
        status = torch.zeros(4, dtype=torch.int32, device=self.device)
        self.pq_encode_async(pq, cb1, cb2, V, codes, rms, outl, ws, status)
        torch.cuda.synchronize(self.device)
        nblk = -(-T // pq["block_tokens"])
        rw = nb // (4 * L * H * T) if T else 0
        return (codes[: nb // 4].reshape(L, H, T, rw), rms[: L * H * T].reshape(L, H, T),
                outl[:ns].reshape(L, H, nblk, pq["outliers"], 2), int(status[0].item()))

    def pq_decode(self, pq: dict, cb1, cb2, codes, rms, outl, T: int, out_dtype: int = FP32):
        """kvtc_pq_decode into a new [L, H, T, D] tensor; returns (values, status word)."""
        c = self.cfg
        dt = torch.float32 if out_dtype == FP32 else torch.bfloat16
        v_out = torch.empty((c["layers"], c["kv_heads"], T, c["head_dim"]), dtype=dt, device=self.device)
        _, _, wb = self.pq_sizes(pq, T)
        ws = torch.empty(max(wb, 256), dtype=torch.uint8, device=self.device)
        status = torch.zeros(4, dtype=torch.int32, device=self.device)
        o = outl.contiguous() if outl.numel() else torch.zeros((2, 2), dtype=torch.int32, device=self.device)
        self.pq_decode_async(pq, cb1, cb2, codes.contiguous(), rms.contiguous(), o, T, v_out, ws, status, out_dtype)
        torch.cuda.synchronize(self.device)
        return v_out, int(status[0].item())


def freq_tables(counts: torch.Tensor, alphabet: torch.Tensor, scale_bits: int):
    """Device normaliser of the record encoder on n tables: counts int32
    [n, 16], alphabet sizes int32 [n] -> frequencies int16 [n, 16]."""
    n = alphabet.numel()
    f = torch.zeros((max(n, 1), 16), dtype=torch.int16, device=counts.device)
    _check(lib().kvtc_test_freq_tables(_ptr(counts), _ptr(alphabet), n, scale_bits, _ptr(f), _stream()),
           "freq_tables")
    torch.cuda.current_stream().synchronize()
    return f[:n]
