"""Device plumbing around the C-ABI: upload generated inputs, size
workspaces, call the entry points.  No step of the method runs here."""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import lsa
from . import synth

_TORCH_DT = {synth.F32: torch.float32, synth.BF16: torch.int16, synth.FP8: torch.uint8}


def _dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def _pinned(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = a
    return t


def _ws(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class DeviceInputs:
    """Generated inputs resident on the GPU (cold tier in HBM or pinned host)."""

    def __init__(self, inp, device="cuda", host_cold=None):
        cfg = inp.cfg
        self.inp, self.cfg, self.device = inp, cfg, device
        self.geom = lsa.Geom(inp["seq_len"], cfg.window, cfg.chunk)
        self.B = cfg.batch
        self.nh = int(inp["chunk_off"][-1])
        self.kic = [_dev(k, device) for k in inp["kic_windows"]]
        self.kic_scale = [_dev(s, device) for s in inp["kic_scale_windows"]]
        self.q_coarse = _dev(inp["q_coarse"], device)
        self.w_coarse = _dev(inp["w_coarse"], device)
        self.bias = _dev(inp["bias"], device)
        self.host_cold = cfg.host_cold if host_cold is None else host_cold
        if self.host_cold:
            self.pages = _pinned(inp["pages"].reshape(-1))
        else:
            self.pages = _dev(inp["pages"].reshape(-1), device)
        self.ikey_scale = _dev(inp["ikey_scale"], device)
        self.recent = _dev(inp["recent"].reshape(-1), device)
        self.q_refine = _dev(inp["q_refine"], device)
        self.w_refine = _dev(inp["w_refine"], device)
        self.q_attn = _dev(inp["q_attn"], device)
        self.kv = lsa.kv_layout(cfg.kv_dtype, cfg.Dk, cfg.Dv, cfg.v_off, cfg.kv_row_bytes,
                                cfg.page_bytes, cfg.ikey_off)

    # ---- single entry points ----
    def score_select(self, theta=0.0, window=0, stream=None):
        cfg, d = self.cfg, self.device
        z = torch.empty(max(self.nh, 1), dtype=torch.float32, device=d)
        sel = torch.full((max(self.nh, 1),), -1, dtype=torch.int32, device=d)
        cnt = torch.zeros(self.B, dtype=torch.int32, device=d)
        ws = _ws(lsa.lsa_score_ws_bytes(self.geom, cfg.d), d)
        lsa.lsa_score_chunks(self.geom, self.q_coarse, cfg.q_dtype, self.w_coarse, self.bias,
                             cfg.H, cfg.d, self.kic[window], cfg.idx_dtype,
                             self.kic_scale[window], z, ws, stream)
        lsa.lsa_select_threshold(self.geom, z, theta, sel, cnt, stream)
        return z[:self.nh], sel, cnt

    def score_select_sigmoid(self, theta=0.5, window=0, q=None, w=None, bias=None, stream=None):
        """Per-head sigmoid score S and the chunks with S > theta; q, w, bias
        (host arrays) replace the request's own when given."""
        cfg, d = self.cfg, self.device
        q = self.q_coarse if q is None else _dev(q, d)
        w = self.w_coarse if w is None else _dev(np.ascontiguousarray(w, dtype=np.float32), d)
        bias = self.bias if bias is None else _dev(np.ascontiguousarray(bias, dtype=np.float32), d)
        S = torch.empty(max(self.nh, 1), dtype=torch.float32, device=d)
        sel = torch.full((max(self.nh, 1),), -1, dtype=torch.int32, device=d)
        cnt = torch.zeros(self.B, dtype=torch.int32, device=d)
        lsa.lsa_score_chunks_sigmoid(self.geom, q, cfg.q_dtype, w, bias, theta, cfg.H, cfg.d,
                                     self.kic[window], cfg.idx_dtype, self.kic_scale[window], S, stream)
        lsa.lsa_select_threshold(self.geom, S, theta, sel, cnt, stream)
        return S[:self.nh], sel, cnt

    def select_ranked(self, keys, kind, m, stream=None):
        """The m[r] best history chunks of each request by key (host array
        or device tensor), ties to the lower chunk, ascending."""
        d = self.device
        if isinstance(keys, np.ndarray):
            keys = _dev(np.ascontiguousarray(keys), d)
        sel = torch.full((max(self.nh, 1),), -1, dtype=torch.int32, device=d)
        cnt = torch.zeros(self.B, dtype=torch.int32, device=d)
        lsa.lsa_select_ranked(self.geom, keys, kind, m, sel, cnt, stream)
        return sel, cnt

    def chunk_mass(self, q_steps=None, pages=None, page_table=None, stream=None):
        """Attention mass of every history chunk under the full softmax of
        the given steps' queries ([n_steps, B, Hq, Dk]; all the inputs'
        steps by default), and each request's recent-window mass."""
        cfg, d = self.cfg, self.device
        q = self.q_attn if q_steps is None else q_steps
        pages = self.pages if pages is None else pages
        n_steps = q.shape[0]
        mass = torch.empty(max(self.nh, 1), dtype=torch.float32, device=d)
        rec = torch.empty(self.B, dtype=torch.float32, device=d)
        ws = _ws(lsa.lsa_chunk_mass_ws_bytes(self.geom, cfg.Hq, n_steps), d)
        lsa.lsa_chunk_attn_mass(self.geom, q, cfg.Hq, n_steps, self.kv, pages, page_table, self.recent,
                                cfg.sm_scale, mass, rec, ws, stream)
        return mass[:self.nh], rec

    def score_select_union(self, layers, theta=0.0, stream=None):
        """OR-mode union over indexer layers (list of dicts with q_coarse,
        w_coarse, bias, kic, kic_scale as host arrays)."""
        cfg, d = self.cfg, self.device
        dev = [{k: torch.from_numpy(np.ascontiguousarray(v)).to(d) for k, v in lay.items()} for lay in layers]
        z = torch.empty(max(self.nh, 1), dtype=torch.float32, device=d)
        sel = torch.full((max(self.nh, 1),), -1, dtype=torch.int32, device=d)
        cnt = torch.zeros(self.B, dtype=torch.int32, device=d)
        ws = _ws(lsa.lsa_score_ws_bytes(self.geom, cfg.d), d)
        lsa.lsa_score_chunks_union(self.geom, [x["q_coarse"] for x in dev], cfg.q_dtype,
                                   [x["w_coarse"] for x in dev], [x["bias"] for x in dev], cfg.H, cfg.d,
                                   [x["kic"] for x in dev], cfg.idx_dtype, [x["kic_scale"] for x in dev],
                                   z, ws, stream)
        lsa.lsa_select_threshold(self.geom, z, theta, sel, cnt, stream)
        return z[:self.nh], sel, cnt

    def refine_topk(self, sel, cnt, step, k, pages=None, page_table=None, stream=None):
        cfg, d = self.cfg, self.device
        pages = self.pages if pages is None else pages
        topk = torch.full((self.B, k), -1, dtype=torch.int32, device=d)
        tcnt = torch.zeros(self.B, dtype=torch.int32, device=d)
        ws = _ws(lsa.lsa_refine_ws_bytes(self.geom, k), d)
        lsa.lsa_topk_refine(self.geom, sel, cnt, pages, cfg.page_bytes, cfg.ikey_off, page_table,
                            cfg.idx_dtype, self.ikey_scale, self.q_refine[step], cfg.q_dtype,
                            self.w_refine[step], cfg.H, cfg.d, k, topk, tcnt, ws, stream)
        return topk, tcnt

    def attend(self, topk, tcnt, step, k, n_splits=0, pages=None, page_table=None, stream=None,
               q=None):
        cfg, d = self.cfg, self.device
        pages = self.pages if pages is None else pages
        odt = torch.float32 if cfg.kv_dtype == synth.F32 else torch.int16
        out = torch.empty((self.B, cfg.Hq, cfg.Dv), dtype=odt, device=d)
        lse = torch.empty((self.B, cfg.Hq), dtype=torch.float32, device=d)
        ws = _ws(lsa.lsa_attn_ws_bytes(self.geom, self.kv, cfg.Hq, k, n_splits), d)
        qa = self.q_attn[step] if q is None else q
        lsa.lsa_sparse_decode_attn(self.geom, qa, cfg.Hq, self.kv, pages, page_table,
                                   self.recent, topk, tcnt, k, cfg.sm_scale, out, lse, n_splits,
                                   ws, stream)
        return out, lse


def out_to_f32(out: torch.Tensor, cfg) -> np.ndarray:
    o = out.cpu()
    if cfg.kv_dtype == synth.F32:
        return o.numpy().astype(np.float64)
    return o.view(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)


class Pipeline:
    """The window pipeline (lsa_ctx_* / lsa_step64) over DeviceInputs."""

    def __init__(self, dev: DeviceInputs, k=None, slots_per_req=None, theta=0.0):
        cfg = dev.cfg
        self.dev, self.cfg = dev, cfg
        self.k = cfg.topk if k is None else k
        spr = cfg.slots_per_req if slots_per_req is None else slots_per_req
        spr = max(1, min(spr, max(int(dev.inp["n_hist"].max()), 1)))
        self.spr = spr
        self.slots = torch.empty(cfg.batch * spr * cfg.page_bytes, dtype=torch.uint8,
                                 device=dev.device)
        self.pool = lsa.Pool(dev.geom, self.slots, spr, cfg.page_bytes, dev.pages,
                             dev.host_cold)
        desc = lsa.lsa_ctx_desc()
        desc.geom = dev.geom.s
        desc.H, desc.d, desc.q_dt, desc.idx_dt = cfg.H, cfg.d, cfg.q_dtype, cfg.idx_dtype
        desc.Hq, desc.k = cfg.Hq, self.k
        desc.kv = dev.kv
        desc.sm_scale, desc.theta = cfg.sm_scale, theta
        desc.recent = dev.recent.data_ptr()
        desc.ikey_scale = dev.ikey_scale.data_ptr()
        desc.pool = self.pool.h.value
        nbytes = lsa.lsa_ctx_ws_bytes(desc)
        if nbytes == 0:
            raise lsa.LsaError("lsa_ctx_ws_bytes", -1)
        self.ws = _ws(nbytes, dev.device)
        desc.ws, desc.ws_bytes = self.ws.data_ptr(), self.ws.numel()
        self.ctx = lsa.Ctx(desc, keep=(dev,))
        self.copy_stream = torch.cuda.Stream(device=dev.device)
        self.sel_cnt = np.zeros(cfg.batch, dtype=np.int32)

    def trigger(self, window: int) -> lsa.lsa_trigger_in:
        d = self.dev
        w = window % len(d.kic)
        return lsa.lsa_trigger_in(d.kic[w].data_ptr(), d.kic_scale[w].data_ptr(),
                                  d.q_coarse.data_ptr(), d.w_coarse.data_ptr(), d.bias.data_ptr())

    def prime(self, main=None):
        self._trig0 = self.trigger(0)
        st = self.ctx.prime(self._trig0, main, self.copy_stream, self.sel_cnt)
        return st, self.sel_cnt.copy()

    def window(self, m: int, step0: int, steps: int, out, lse=None, topk=None, tcnt=None,
               last=False, main=None):
        """Run window m (steps [step0, step0+steps) of the query arrays)."""
        d = self.dev
        nxt = None if last else self.trigger(m + 1)
        self._nxt = nxt
        qr = d.q_refine[step0:step0 + steps]
        wr = d.w_refine[step0:step0 + steps]
        qa = d.q_attn[step0:step0 + steps]
        win = lsa.lsa_window_in(steps, qr.data_ptr(), wr.data_ptr(), qa.data_ptr(),
                                C.pointer(nxt) if nxt is not None else None)
        wo = lsa.lsa_window_out()
        wo.out = out.data_ptr()
        wo.lse = lse.data_ptr() if lse is not None else None
        wo.topk_idx = topk.data_ptr() if topk is not None else None
        wo.topk_cnt = tcnt.data_ptr() if tcnt is not None else None
        wo.sel_cnt = self.sel_cnt.ctypes.data
        st = self.ctx.step64(win, wo, main, self.copy_stream)
        return st, self.sel_cnt.copy()

    def close(self):
        torch.cuda.synchronize()
        self.ctx.close()
        self.pool.close()
