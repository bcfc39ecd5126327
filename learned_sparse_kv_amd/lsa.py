"""ctypes binding of liblsa.so: the C-ABI in include/lsa.h, same names.

Argument marshalling only: torch tensors become device pointers, the
current torch stream becomes the hipStream_t, and a non-zero status raises
LsaError.  Every step of the path runs in the HIP library; if it is not built
the import fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsa.so")

LSA_F32, LSA_BF16, LSA_FP8_E4M3FN = 0, 1, 2
LSA_MAX_BATCH = 64
LSA_CHUNK = 64

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported dtype or shape",
           -3: "slot pool capacity exceeded", -4: "workspace too small", -5: "HIP runtime error"}


class LsaError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn}: {_STATUS.get(code, code)} ({code})")
        self.code = code


class lsa_geom(C.Structure):
    _fields_ = [("batch", C.c_int32), ("chunk", C.c_int32), ("window", C.c_int32),
                ("seq_len", C.c_void_p), ("hist_tokens", C.c_void_p), ("chunk_cap", C.c_int32),
                ("recent_cap", C.c_int32)]


class lsa_kv_layout(C.Structure):
    _fields_ = [("kv_dtype", C.c_int), ("Dk", C.c_int32), ("Dv", C.c_int32),
                ("v_off", C.c_int32), ("row_bytes", C.c_int64), ("page_bytes", C.c_int64),
                ("ikey_off", C.c_int64)]


class lsa_gather_stats(C.Structure):
    _fields_ = [("fetched", C.c_int64), ("resident", C.c_int64), ("evicted", C.c_int64),
                ("copies", C.c_int64), ("bytes", C.c_int64)]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


class lsa_ctx_desc(C.Structure):
    _fields_ = [("geom", lsa_geom), ("H", C.c_int32), ("d", C.c_int32), ("q_dt", C.c_int),
                ("idx_dt", C.c_int), ("Hq", C.c_int32), ("k", C.c_int32),
                ("kv", lsa_kv_layout), ("sm_scale", C.c_float), ("theta", C.c_float),
                ("recent", C.c_void_p), ("ikey_scale", C.c_void_p), ("pool", C.c_void_p),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t), ("n_layers", C.c_int32),
                ("growing", C.c_int32)]


class lsa_trigger_in(C.Structure):
    _fields_ = [("kic", C.c_void_p), ("kic_scale", C.c_void_p), ("q", C.c_void_p),
                ("w", C.c_void_p), ("bias", C.c_void_p)]


class lsa_window_in(C.Structure):
    _fields_ = [("steps", C.c_int32), ("q_refine", C.c_void_p), ("w_refine", C.c_void_p),
                ("q_attn", C.c_void_p), ("next", C.POINTER(lsa_trigger_in)),
                ("new_rows", C.c_void_p), ("commit_ikeys", C.c_void_p),
                ("commit_ikey_scale", C.c_void_p)]


class lsa_window_out(C.Structure):
    _fields_ = [("out", C.c_void_p), ("lse", C.c_void_p), ("topk_idx", C.c_void_p),
                ("topk_cnt", C.c_void_p), ("sel_cnt", C.c_void_p),
                ("stats", lsa_gather_stats)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m learned_sparse_kv_amd.build` (no fallback path exists)")
    lib = C.CDLL(_LIB_PATH)
    P, I32, I64, F, SZ, I = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t, C.c_int
    G = C.POINTER(lsa_geom)
    sig = {
        "lsa_status_str": ([I], C.c_char_p),
        "lsa_score_ws_bytes": ([G, I32], SZ),
        "lsa_score_chunks": ([G, P, I, P, P, I32, I32, P, I, P, P, P, SZ, P], I),
        "lsa_select_threshold": ([G, P, F, P, P, P], I),
        "lsa_score_chunks_union": ([G, I32, P, I, P, P, I32, I32, P, I, P, P, P, SZ, P], I),
        "lsa_score_chunks_sigmoid": ([G, P, I, P, P, F, I32, I32, P, I, P, P, P], I),
        "lsa_select_ranked": ([G, P, I, P, P, P, P], I),
        "lsa_append_kv": ([G, C.POINTER(lsa_kv_layout), P, P, P], I),
        "lsa_commit_chunk": ([G, C.POINTER(lsa_kv_layout), P, P, P, I, I32, P, P, P, P, P, P, P, P, P], I),
        "lsa_chunk_mass_ws_bytes": ([G, I32, I32], SZ),
        "lsa_chunk_attn_mass": ([G, P, I32, I32, C.POINTER(lsa_kv_layout), P, P, P, F, P, P, P, SZ, P],
                                I),
        "lsa_refine_ws_bytes": ([G, I32], SZ),
        "lsa_topk_refine": ([G, P, P, P, I64, I64, P, I, P, P, I, P, I32, I32, I32, P, P, P, SZ,
                             P], I),
        "lsa_attn_ws_bytes": ([G, C.POINTER(lsa_kv_layout), I32, I32, I32], SZ),
        "lsa_sparse_decode_attn": ([G, P, I32, C.POINTER(lsa_kv_layout), P, P, P, P, P, I32, F, P,
                                    P, I32, P, SZ, P], I),
        "lsa_pool_create": ([C.POINTER(P), G, P, I32, I64, P, I32], I),
        "lsa_pool_destroy": ([P], None),
        "lsa_gather_kv": ([P, P, P, P, P, P, P, P, P, C.POINTER(lsa_gather_stats)], I),
        "lsa_ctx_ws_bytes": ([C.POINTER(lsa_ctx_desc)], SZ),
        "lsa_ctx_create": ([C.POINTER(P), C.POINTER(lsa_ctx_desc)], I),
        "lsa_ctx_destroy": ([P], None),
        "lsa_ctx_prime": ([P, C.POINTER(lsa_trigger_in), P, P, C.POINTER(lsa_window_out)], I),
        "lsa_step64": ([P, C.POINTER(lsa_window_in), C.POINTER(lsa_window_out), P, P], I),
        "lsa_ctx_state": ([P, P, P, P], I),
        "lsa_timing_enable": ([I32], I),
        "lsa_timing_only": ([C.c_char_p], I),
        "lsa_timing_every": ([I32], I),
        "lsa_timing_reset": ([], None),
        "lsa_timing_read": ([C.c_char_p, C.POINTER(I64), C.POINTER(C.c_double)], I),
        "lsa_stream_read": ([P, SZ, P, P], I),
        "lsa_tune_set": ([I, I32], I),
        "lsa_attn_noalloc_max_bytes": ([], SZ),
        "lsa_sparse_decode_attn_noalloc": ([G, P, I32, C.POINTER(lsa_kv_layout), P, P, P, P, P, I32, F,
                                            P, P, I32, P], I),
        "lsa_device_status": ([P, C.POINTER(C.c_uint32)], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def lib():
    return _lib


# ---------------------------------------------------------------- marshalling
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return int(t)


def _stream(s=None):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def _check(fn, code):
    if code != 0:
        raise LsaError(fn, code)


class Geom:
    """lsa_geom plus the host arrays it points to.  hist_tokens, chunk_cap and
    recent_cap describe a growing context (None / 0: packed layout)."""

    def __init__(self, seq_len, window: int, chunk: int = LSA_CHUNK, hist_tokens=None,
                 chunk_cap: int = 0, recent_cap: int = 0):
        self.seq_len = np.ascontiguousarray(seq_len, dtype=np.int32)
        self.hist_tokens = None if hist_tokens is None else np.ascontiguousarray(hist_tokens, dtype=np.int32)
        self.s = lsa_geom(len(self.seq_len), chunk, window, self.seq_len.ctypes.data,
                          None if self.hist_tokens is None else self.hist_tokens.ctypes.data,
                          int(chunk_cap), int(recent_cap))

    @property
    def ref(self):
        return C.byref(self.s)


def kv_layout(kv_dtype, Dk, Dv, v_off, row_bytes, page_bytes, ikey_off):
    return lsa_kv_layout(kv_dtype, Dk, Dv, v_off, row_bytes, page_bytes, ikey_off)


# ---------------------------------------------------------------- entry points
def lsa_score_ws_bytes(g: Geom, d: int) -> int:
    return _lib.lsa_score_ws_bytes(g.ref, d)


def lsa_score_chunks(g: Geom, q, q_dt, w, bias, H, d, kic, kic_dt, kic_scale, z, ws, stream=None):
    _check("lsa_score_chunks",
           _lib.lsa_score_chunks(g.ref, _ptr(q), q_dt, _ptr(w), _ptr(bias), H, d, _ptr(kic), kic_dt,
                                 _ptr(kic_scale), _ptr(z), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)))


def lsa_score_chunks_union(g: Geom, q, q_dt, w, bias, H, d, kic, kic_dt, kic_scale, z, ws,
                           stream=None):
    """q, w, bias, kic, kic_scale: equal-length lists of per-layer tensors
    (kic_scale entries may be None unless kic_dt is fp8)."""
    n = len(q)
    arr = lambda xs: (C.c_void_p * n)(*[_ptr(x) for x in xs])
    _check("lsa_score_chunks_union",
           _lib.lsa_score_chunks_union(g.ref, n, arr(q), q_dt, arr(w), arr(bias), H, d, arr(kic), kic_dt,
                                       arr(kic_scale), _ptr(z), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)))


def lsa_score_chunks_sigmoid(g: Geom, q, q_dt, w, bias, theta, H, d, kic, kic_dt, kic_scale, S, stream=None):
    _check("lsa_score_chunks_sigmoid",
           _lib.lsa_score_chunks_sigmoid(g.ref, _ptr(q), q_dt, _ptr(w), _ptr(bias), float(theta), H, d,
                                         _ptr(kic), kic_dt, _ptr(kic_scale), _ptr(S), _stream(stream)))


def lsa_append_kv(g: Geom, kv: lsa_kv_layout, rows, recent, stream=None):
    _check("lsa_append_kv", _lib.lsa_append_kv(g.ref, C.byref(kv), _ptr(rows), _ptr(recent), _stream(stream)))


def lsa_commit_chunk(g: Geom, kv: lsa_kv_layout, recent_src, recent_dst, cold, idx_dt, d, new_ikeys,
                     new_ikey_scale, ikey_scale, new_kic, new_kic_scale, kic, kic_scale, stream=None):
    """Returns the new hist_tokens (host int32 array)."""
    out = np.zeros(g.s.batch, np.int32)
    _check("lsa_commit_chunk",
           _lib.lsa_commit_chunk(g.ref, C.byref(kv), _ptr(recent_src), _ptr(recent_dst), _ptr(cold), idx_dt, d,
                                 _ptr(new_ikeys), _ptr(new_ikey_scale), _ptr(ikey_scale), _ptr(new_kic),
                                 _ptr(new_kic_scale), _ptr(kic), _ptr(kic_scale), out.ctypes.data,
                                 _stream(stream)))
    return out


RANK_SMALLEST_U32, RANK_LARGEST_F32 = 0, 1


def lsa_select_ranked(g: Geom, keys, kind, m, sel_ids, sel_cnt, stream=None):
    m = np.ascontiguousarray(m, dtype=np.int32)
    _check("lsa_select_ranked",
           _lib.lsa_select_ranked(g.ref, _ptr(keys), int(kind), m.ctypes.data, _ptr(sel_ids),
                                  _ptr(sel_cnt), _stream(stream)))


def lsa_chunk_mass_ws_bytes(g: Geom, Hq, n_steps):
    return _lib.lsa_chunk_mass_ws_bytes(g.ref, Hq, n_steps)


def lsa_chunk_attn_mass(g: Geom, q, Hq, n_steps, kv: lsa_kv_layout, pages, page_table, recent, sm_scale,
                        mass, rec_mass, ws, stream=None):
    _check("lsa_chunk_attn_mass",
           _lib.lsa_chunk_attn_mass(g.ref, _ptr(q), Hq, n_steps, C.byref(kv), _ptr(pages),
                                    _ptr(page_table), _ptr(recent), float(sm_scale), _ptr(mass),
                                    _ptr(rec_mass), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def lsa_select_threshold(g: Geom, z, theta, sel_ids, sel_cnt, stream=None):
    _check("lsa_select_threshold",
           _lib.lsa_select_threshold(g.ref, _ptr(z), float(theta), _ptr(sel_ids), _ptr(sel_cnt),
                                     _stream(stream)))


def lsa_refine_ws_bytes(g: Geom, k: int) -> int:
    return _lib.lsa_refine_ws_bytes(g.ref, k)


def lsa_topk_refine(g: Geom, sel_ids, sel_cnt, pages, page_bytes, ikey_off, page_table, idx_dt,
                    ikey_scale, q, q_dt, w, H, d, k, topk_idx, topk_cnt, ws, stream=None):
    _check("lsa_topk_refine",
           _lib.lsa_topk_refine(g.ref, _ptr(sel_ids), _ptr(sel_cnt), _ptr(pages), page_bytes,
                                ikey_off, _ptr(page_table), idx_dt, _ptr(ikey_scale), _ptr(q), q_dt,
                                _ptr(w), H, d, k, _ptr(topk_idx), _ptr(topk_cnt), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))


def lsa_attn_ws_bytes(g: Geom, kv: lsa_kv_layout, Hq, k, n_splits=0) -> int:
    return _lib.lsa_attn_ws_bytes(g.ref, C.byref(kv), Hq, k, n_splits)


def lsa_sparse_decode_attn(g: Geom, q, Hq, kv: lsa_kv_layout, pages, page_table, recent, topk_idx,
                           topk_cnt, k, sm_scale, out, lse, n_splits, ws, stream=None):
    _check("lsa_sparse_decode_attn",
           _lib.lsa_sparse_decode_attn(g.ref, _ptr(q), Hq, C.byref(kv), _ptr(pages),
                                       _ptr(page_table), _ptr(recent), _ptr(topk_idx),
                                       _ptr(topk_cnt), k, float(sm_scale), _ptr(out), _ptr(lse),
                                       n_splits, _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)))


def lsa_attn_noalloc_max_bytes() -> int:
    return _lib.lsa_attn_noalloc_max_bytes()


def lsa_sparse_decode_attn_noalloc(g: Geom, q, Hq, kv: lsa_kv_layout, pages, page_table, recent, topk_idx,
                                   topk_cnt, k, sm_scale, out, lse, n_splits, stream=None):
    _check("lsa_sparse_decode_attn_noalloc",
           _lib.lsa_sparse_decode_attn_noalloc(g.ref, _ptr(q), Hq, C.byref(kv), _ptr(pages),
                                               _ptr(page_table), _ptr(recent), _ptr(topk_idx),
                                               _ptr(topk_cnt), k, float(sm_scale), _ptr(out), _ptr(lse),
                                               n_splits, _stream(stream)))


class Pool:
    """lsa_pool_create / lsa_gather_kv / lsa_pool_destroy."""

    def __init__(self, g: Geom, slot_mem, slots_per_req, page_bytes, cold, cold_on_host):
        self.g, self._keep = g, (slot_mem, cold)
        h = C.c_void_p()
        _check("lsa_pool_create", _lib.lsa_pool_create(C.byref(h), g.ref, _ptr(slot_mem),
                                                        slots_per_req, page_bytes, _ptr(cold),
                                                        int(cold_on_host)))
        self.h = h

    def gather(self, sel_ids, sel_cnt, keep_ids, keep_cnt, page_table, copy_stream=None,
               wait_event=None, done_event=None):
        st = lsa_gather_stats()
        _check("lsa_gather_kv",
               _lib.lsa_gather_kv(self.h, _ptr(sel_ids), _ptr(sel_cnt), _ptr(keep_ids),
                                  _ptr(keep_cnt), _ptr(page_table), _stream(copy_stream),
                                  _event(wait_event), _event(done_event), C.byref(st)))
        return st.as_dict()

    def close(self):
        if getattr(self, "h", None):
            _lib.lsa_pool_destroy(self.h)
            self.h = None

    __del__ = close


def lsa_gather_kv(pool: Pool, *a, **kw):
    return pool.gather(*a, **kw)


def _event(e):
    if e is None:
        return None
    if isinstance(e, torch.cuda.Event):
        return e.cuda_event
    return int(e)


def trigger_ptr(trig):
    """Pointer to the first lsa_trigger_in of a struct or of an array of them."""
    if trig is None:
        return None
    if isinstance(trig, lsa_trigger_in):
        return C.pointer(trig)
    return C.cast(trig, C.POINTER(lsa_trigger_in))


class Ctx:
    """lsa_ctx_create / lsa_ctx_prime / lsa_step64 / lsa_ctx_destroy."""

    def __init__(self, desc: lsa_ctx_desc, keep=()):
        self.desc, self._keep = desc, keep
        h = C.c_void_p()
        _check("lsa_ctx_create", _lib.lsa_ctx_create(C.byref(h), C.byref(desc)))
        self.h = h

    def prime(self, trig, main=None, copy=None, sel_cnt=None):
        """trig: one lsa_trigger_in, or a ctypes array of one per indexer layer."""
        out = lsa_window_out()
        out.sel_cnt = _ptr(sel_cnt)
        _check("lsa_ctx_prime", _lib.lsa_ctx_prime(self.h, trigger_ptr(trig), _stream(main),
                                                   _stream(copy), C.byref(out)))
        return out.stats.as_dict()

    def step64(self, win: lsa_window_in, out: lsa_window_out, main=None, copy=None):
        _check("lsa_step64", _lib.lsa_step64(self.h, C.byref(win), C.byref(out), _stream(main),
                                             _stream(copy)))
        return out.stats.as_dict()

    def state(self):
        """(seq_len, hist_tokens, recent_first) as host int32 arrays [B]."""
        B = self.desc.geom.batch
        L, rs, rf = (np.zeros(B, np.int32) for _ in range(3))
        _check("lsa_ctx_state", _lib.lsa_ctx_state(self.h, _ptr(L), _ptr(rs), _ptr(rf)))
        return L, rs, rf

    def close(self):
        if getattr(self, "h", None):
            _lib.lsa_ctx_destroy(self.h)
            self.h = None

    __del__ = close


def lsa_ctx_ws_bytes(desc: lsa_ctx_desc) -> int:
    return _lib.lsa_ctx_ws_bytes(C.byref(desc))


def lsa_step64(ctx: Ctx, win, out, main=None, copy=None):
    return ctx.step64(win, out, main, copy)


# ---------------------------------------------------------------- diagnostics
KERNELS = ("k_fuse_query", "k_score", "k_select", "k_select_tiles", "k_refine", "k_topk", "k_refine_mfma",
           "k_band_fine", "k_band_list", "k_topk_band", "k_attn_mla", "k_attn_f32", "k_attn_merge",
           "k_gather", "k_stream_read", "k_score_sig", "k_select_ranked", "k_chunk_ml",
           "k_append_kv", "k_commit_chunk", "k_commit_page", "k_compact_recent", "k_resolve_sel",
           "k_key_norm2")


def lsa_timing_enable(on: bool):
    _check("lsa_timing_enable", _lib.lsa_timing_enable(1 if on else 0))


def lsa_timing_only(kernel=None):
    _check("lsa_timing_only", _lib.lsa_timing_only(kernel.encode() if kernel else None))


def lsa_timing_every(n: int):
    _check("lsa_timing_every", _lib.lsa_timing_every(int(n)))


def lsa_timing_reset():
    _lib.lsa_timing_reset()


def lsa_timing_read(kernel: str):
    n, ms = C.c_int64(), C.c_double()
    _check("lsa_timing_read", _lib.lsa_timing_read(kernel.encode(), C.byref(n), C.byref(ms)))
    return int(n.value), float(ms.value)


def lsa_stream_read(src, nbytes: int, sink, stream=None):
    _check("lsa_stream_read", _lib.lsa_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)))


TUNE_REFINE_BLOCKS, TUNE_ATTN_PAIR_POLLS = 0, 1


def lsa_tune_set(knob: int, value: int):
    """Launch-shape override (value < 0: the library's own choice)."""
    _check("lsa_tune_set", _lib.lsa_tune_set(int(knob), int(value)))


def lsa_device_status(stream=None):
    """(status code, flags) of the device error word; clears it.  Does not
    raise: a set word returns LSA_ERR_HIP (-5) with its flags."""
    f = C.c_uint32(0)
    code = _lib.lsa_device_status(_stream(stream), C.byref(f))
    return int(code), int(f.value)
