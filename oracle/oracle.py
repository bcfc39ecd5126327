"""Python access to the CPU oracle (lsa_oracle.c) and the pool simulation.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library; both read the same input bytes produced by the seeded
generator.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB = os.path.join(_HERE, "liblsa_oracle.so")
# -ffp-contract=off and no fast-math: every fp32 operation is the one written.
# -mfma lets fmaf() compile to the hardware fused multiply-add (same IEEE
# result as the library call, much faster).
CFLAGS = ["-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-std=c11"]


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Batch(C.Structure):
    _fields_ = [("B", C.c_int32), ("C", C.c_int32), ("W", C.c_int32),
                ("seq_len", C.c_void_p),
                ("H", C.c_int32), ("d", C.c_int32), ("q_dt", C.c_int32), ("idx_dt", C.c_int32),
                ("Hq", C.c_int32), ("Dk", C.c_int32), ("Dv", C.c_int32), ("kv_dt", C.c_int32),
                ("v_off", C.c_int32),
                ("kv_row_bytes", C.c_int64), ("page_bytes", C.c_int64), ("ikey_off", C.c_int64),
                ("kic", C.c_void_p), ("kic_scale", C.c_void_p), ("pages", C.c_void_p),
                ("ikey_scale", C.c_void_p), ("recent", C.c_void_p)]


_lib = None


def load(path: str):
    """Load an oracle build (the default one, or a test's variant) and bind it."""
    global _lib
    _lib = C.CDLL(path)
    P, I32, I64, F, D = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_double
    _lib.lsao_decode.argtypes = [C.c_int, P, I64, P]
    _lib.lsao_decode.restype = I64
    _lib.lsao_geometry.argtypes = [I32, I32, I32, P]
    _lib.lsao_score_select.argtypes = [C.POINTER(Batch), P, P, P, F, P, P, P]
    _lib.lsao_score_select.restype = C.c_int
    _lib.lsao_score_select_union.argtypes = [C.POINTER(Batch), I32, P, P, P, P, P, F, P, P, P]
    _lib.lsao_score_select_union.restype = C.c_int
    _lib.lsao_score_select_sigmoid.argtypes = [C.POINTER(Batch), P, P, P, F, P, P, P]
    _lib.lsao_score_select_sigmoid.restype = C.c_int
    _lib.lsao_sigmoid.argtypes = [F]
    _lib.lsao_sigmoid.restype = F
    _lib.lsao_refine_topk.argtypes = [C.POINTER(Batch), I32, P, I32, P, P, I32, P, P]
    _lib.lsao_refine_topk.restype = I32
    _lib.lsao_attend.argtypes = [C.POINTER(Batch), I32, P, I32, P, D, P, P]
    _lib.lsao_attend.restype = C.c_int
    _lib.lsao_decode_units.argtypes = [C.POINTER(Batch), I32, P, P, P, P, P, P, P, I32, D,
                                       P, P, P, P, I32]
    _lib.lsao_decode_units.restype = C.c_int
    _lib.lsao_chunk_mass.argtypes = [C.POINTER(Batch), I32, I32, P, D, P, P, I32]
    _lib.lsao_chunk_mass.restype = C.c_int
    _lib.lsao_max_threads.restype = C.c_int
    return _lib


def lib():
    return _lib if _lib is not None else load(build())


def _p(a):
    return None if a is None else a.ctypes.data


def decode(dt: int, raw: np.ndarray) -> np.ndarray:
    raw = np.ascontiguousarray(raw)
    n = raw.size
    out = np.empty(n, dtype=np.float32)
    lib().lsao_decode(dt, _p(raw), n, _p(out))
    return out.reshape(raw.shape)


def geometry(L: int, C_: int, W: int):
    g = np.zeros(3, dtype=np.int64)
    lib().lsao_geometry(L, C_, W, _p(g))
    return int(g[0]), int(g[1]), int(g[2])


class Oracle:
    """Oracle bound to one set of generated inputs (keeps arrays alive)."""

    def __init__(self, inp, kic=None, kic_scale=None):
        cfg = inp.cfg
        self.inp, self.cfg = inp, cfg
        self._keep = dict(
            seq_len=np.ascontiguousarray(inp["seq_len"], dtype=np.int32),
            kic=np.ascontiguousarray(inp["kic"] if kic is None else kic),
            kic_scale=np.ascontiguousarray(inp["kic_scale"] if kic_scale is None else kic_scale),
            pages=np.ascontiguousarray(inp["pages"]),
            ikey_scale=np.ascontiguousarray(inp["ikey_scale"]),
            recent=np.ascontiguousarray(inp["recent"]),
        )
        k = self._keep
        fp8 = cfg.idx_dtype == 2
        self.batch = Batch(cfg.batch, cfg.chunk, cfg.window, _p(k["seq_len"]),
                           cfg.H, cfg.d, cfg.q_dtype, cfg.idx_dtype,
                           cfg.Hq, cfg.Dk, cfg.Dv, cfg.kv_dtype, cfg.v_off,
                           cfg.kv_row_bytes, cfg.page_bytes, cfg.ikey_off,
                           _p(k["kic"]), _p(k["kic_scale"]) if fp8 else None, _p(k["pages"]),
                           _p(k["ikey_scale"]) if fp8 else None, _p(k["recent"]))
        self.n_total = int(sum(geometry(int(L), cfg.chunk, cfg.window)[1] for L in k["seq_len"]))

    def score_select(self, theta: float = 0.0, q=None, w=None, bias=None):
        inp = self.inp
        q = np.ascontiguousarray(inp["q_coarse"] if q is None else q)
        w = np.ascontiguousarray(inp["w_coarse"] if w is None else w, dtype=np.float32)
        bias = np.ascontiguousarray(inp["bias"] if bias is None else bias, dtype=np.float32)
        n = max(self.n_total, 1)
        z = np.zeros(n, np.float32)
        sel = np.full(n, -1, np.int32)
        cnt = np.zeros(self.cfg.batch, np.int32)
        rc = lib().lsao_score_select(C.byref(self.batch), _p(q), _p(w), _p(bias),
                                     np.float32(theta), _p(z), _p(sel), _p(cnt))
        assert rc == 0
        return z[:self.n_total], sel[:self.n_total], cnt

    def score_select_sigmoid(self, theta: float = 0.5, q=None, w=None, bias=None):
        """Per-head sigmoid score S_c (probabilities) and the chunks with
        S_c > theta.  Returns (S, sel, cnt)."""
        inp = self.inp
        q = np.ascontiguousarray(inp["q_coarse"] if q is None else q)
        w = np.ascontiguousarray(inp["w_coarse"] if w is None else w, dtype=np.float32)
        bias = np.ascontiguousarray(inp["bias"] if bias is None else bias, dtype=np.float32)
        n = max(self.n_total, 1)
        S = np.zeros(n, np.float32)
        sel = np.full(n, -1, np.int32)
        cnt = np.zeros(self.cfg.batch, np.int32)
        rc = lib().lsao_score_select_sigmoid(C.byref(self.batch), _p(q), _p(w), _p(bias),
                                             np.float32(theta), _p(S), _p(sel), _p(cnt))
        assert rc == 0
        return S[:self.n_total], sel[:self.n_total], cnt

    def score_select_union(self, layers, theta: float = 0.0):
        """OR-mode union over indexer layers.  layers: list of dicts with
        q_coarse, w_coarse, bias, kic, kic_scale.  Returns (zmax, sel, cnt)."""
        n = max(self.n_total, 1)
        keep = [{k: np.ascontiguousarray(v) for k, v in lay.items()} for lay in layers]
        for lay in keep:
            lay["w_coarse"] = np.ascontiguousarray(lay["w_coarse"], dtype=np.float32)
            lay["bias"] = np.ascontiguousarray(lay["bias"], dtype=np.float32)
            lay["kic_scale"] = np.ascontiguousarray(lay["kic_scale"], dtype=np.float32)
        nl = len(keep)
        arr = lambda key: (C.c_void_p * nl)(*[_p(lay[key]) for lay in keep])
        zmax = np.zeros(n, np.float32)
        sel = np.full(n, -1, np.int32)
        cnt = np.zeros(self.cfg.batch, np.int32)
        rc = lib().lsao_score_select_union(C.byref(self.batch), nl, arr("q_coarse"), arr("w_coarse"),
                                           arr("bias"), arr("kic"), arr("kic_scale"), np.float32(theta),
                                           _p(zmax), _p(sel), _p(cnt))
        assert rc == 0
        return zmax[:self.n_total], sel[:self.n_total], cnt

    def refine_topk(self, r: int, sel_r, q_r, w_r, k: int, want_scores=False):
        sel_r = np.ascontiguousarray(sel_r, dtype=np.int32)
        q_r = np.ascontiguousarray(q_r)
        w_r = np.ascontiguousarray(w_r, dtype=np.float32)
        topk = np.zeros(max(k, 1), np.int32)
        sc = np.zeros(max(len(sel_r) * self.cfg.chunk, 1), np.float32) if want_scores else None
        kc = lib().lsao_refine_topk(C.byref(self.batch), r, _p(sel_r), len(sel_r), _p(q_r),
                                    _p(w_r), k, _p(topk), _p(sc))
        assert kc >= 0
        if want_scores:
            return topk[:kc], sc[:len(sel_r) * self.cfg.chunk]
        return topk[:kc]

    def attend(self, r: int, topk, q_r, sm: float):
        topk = np.ascontiguousarray(topk, dtype=np.int32)
        q_r = np.ascontiguousarray(q_r)
        out = np.zeros((self.cfg.Hq, self.cfg.Dv), np.float64)
        lse = np.zeros(self.cfg.Hq, np.float64)
        rc = lib().lsao_attend(C.byref(self.batch), r, _p(topk) if len(topk) else None,
                               len(topk), _p(q_r), float(sm), _p(out), _p(lse))
        assert rc == 0
        return out, lse

    def decode_units(self, units, sel, cnt, k: int, sm: float, q_refine=None, w_refine=None,
                     q_attn=None, threads: int = 0):
        """units: list of (request, step).  Returns topk list, out, lse."""
        inp, cfg = self.inp, self.cfg
        ur = np.ascontiguousarray([u[0] for u in units], dtype=np.int32)
        us = np.ascontiguousarray([u[1] for u in units], dtype=np.int32)
        qr = np.ascontiguousarray(inp["q_refine"] if q_refine is None else q_refine)
        wr = np.ascontiguousarray(inp["w_refine"] if w_refine is None else w_refine,
                                  dtype=np.float32)
        qa = np.ascontiguousarray(inp["q_attn"] if q_attn is None else q_attn)
        n = len(units)
        tk = np.zeros((n, max(k, 1)), np.int32)
        tc = np.zeros(n, np.int32)
        out = np.zeros((n, cfg.Hq, cfg.Dv), np.float64)
        lse = np.zeros((n, cfg.Hq), np.float64)
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        if sel.size == 0:
            sel = np.zeros(1, np.int32)
        cnt = np.ascontiguousarray(cnt, dtype=np.int32)
        rc = lib().lsao_decode_units(C.byref(self.batch), n, _p(ur), _p(us), _p(sel), _p(cnt),
                                     _p(qr), _p(wr), _p(qa), k, float(sm), _p(tk), _p(tc),
                                     _p(out), _p(lse), threads)
        assert rc == 0
        return [tk[i, :tc[i]].copy() for i in range(n)], out, lse


    def chunk_mass(self, r: int, q_steps, sm: float, threads: int = 0):
        """Attention mass of every history chunk of request r under the full
        softmax of each given step's queries (q_steps [n_steps, Hq, Dk] in the
        KV dtype), summed over steps and heads.  Returns (mass [N] float64,
        recent-window mass)."""
        q = np.ascontiguousarray(q_steps)
        n_steps = q.shape[0]
        n = int(self.inp["n_hist"][r])
        mass = np.zeros(max(n, 1), np.float64)
        rec = np.zeros(1, np.float64)
        rc = lib().lsao_chunk_mass(C.byref(self.batch), r, n_steps, _p(q), float(sm), _p(mass),
                                   _p(rec), threads)
        assert rc == 0
        return mass[:n], float(rec[0])


# ------------------------------------------------------------------ policies
# The pages compare LSA with a recency-only scheme (the recent 8K only), a
# scheme that keeps a random 10 % of the history chunks, and an oracle that
# keeps the top 50 / 25 / 10 % of history chunks by true attention weight
# (cjcn.com.cn explainer, sections 五 and 六).  Readings: a policy keeping
# pct percent of N chunks keeps ceil(N * pct / 100) of them; the random
# policy keeps the chunks with the smallest of N uniformly drawn 32-bit keys
# (a uniform sample without replacement); the oracle policy keeps the
# chunks of largest mass; ties go to the lower chunk index; the kept chunks
# are listed ascending.

def policy_count(n: int, pct: int) -> int:
    return (int(n) * int(pct) + 99) // 100


def select_smallest(keys, m: int):
    """The m chunks of smallest key, ties to the lower index, ascending."""
    keys = np.asarray(keys)
    order = np.lexsort((np.arange(len(keys)), keys))
    return np.sort(order[:m]).astype(np.int32)


def select_largest(mass, m: int):
    """The m chunks of largest mass, ties to the lower index, ascending."""
    mass = np.asarray(mass, dtype=np.float64)
    order = np.lexsort((np.arange(len(mass)), -mass))
    return np.sort(order[:m]).astype(np.int32)


def mass_recall(mass, sel) -> float:
    """Share of the history chunks' attention mass held by the chunks in sel."""
    mass = np.asarray(mass, dtype=np.float64)
    tot = mass.sum()
    return float(mass[np.asarray(sel, dtype=np.int64)].sum() / tot) if tot > 0 else 0.0


def sigmoid(x: float) -> float:
    """The oracle's fp32 sigmoid of the per-head score (exposed for its pins)."""
    return float(lib().lsao_sigmoid(np.float32(x)))


def pool_sim(selections, capacity: int):
    """Slot-pool residency over windows, one window ahead (plain sets).

    selections: list over windows m = 0.. of the selected chunk-id sets of
    one request.  Window m's chunks must be resident while window m runs and
    window m+1's chunks are fetched during it, so after the fetch for m+1
    the resident set is S_m | S_{m+1} (everything else was evicted) and the
    fetch copies S_{m+1} minus what was resident (S_{m-1} | S_m).  The first
    fetch (m = 0) starts from an empty pool.  Returns per fetch the number of
    copied chunks; raises OverflowError when S_m | S_{m+1} exceeds capacity.
    """
    misses = []
    prev = set()            # S_{m-1}
    cur = set()             # S_m
    for m, s in enumerate(selections):
        s = set(int(x) for x in s)
        resident = prev | cur
        if len(cur | s) > capacity:
            raise OverflowError(f"fetch {m}: {len(cur | s)} chunks > capacity {capacity}")
        misses.append(len(s - resident))
        prev, cur = cur, s
    return misses
