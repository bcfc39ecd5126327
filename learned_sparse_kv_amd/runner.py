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

    def __init__(self, dev: DeviceInputs, k=None, slots_per_req=None, theta=0.0, n_layers=1):
        cfg = dev.cfg
        self.dev, self.cfg = dev, cfg
        self.n_layers = n_layers
        # indexer layers beyond the inputs' own (the same for every window)
        self.extra_layers = []
        if n_layers > 1:
            for lay in synth.indexer_layers(dev.inp, n_layers)[1:]:
                self.extra_layers.append({key: _dev(np.ascontiguousarray(v), dev.device)
                                          for key, v in lay.items()})
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
        desc.n_layers = n_layers
        nbytes = lsa.lsa_ctx_ws_bytes(desc)
        if nbytes == 0:
            raise lsa.LsaError("lsa_ctx_ws_bytes", -1)
        self.ws = _ws(nbytes, dev.device)
        desc.ws, desc.ws_bytes = self.ws.data_ptr(), self.ws.numel()
        self.ctx = lsa.Ctx(desc, keep=(dev,))
        self.copy_stream = torch.cuda.Stream(device=dev.device)
        self.sel_cnt = np.zeros(cfg.batch, dtype=np.int32)

    def trigger(self, window: int):
        """The window's trigger: one lsa_trigger_in per indexer layer (the
        inputs' own indexer first, with that window's KIComp)."""
        d = self.dev
        w = window % len(d.kic)
        trig = (lsa.lsa_trigger_in * self.n_layers)()
        trig[0] = lsa.lsa_trigger_in(d.kic[w].data_ptr(), d.kic_scale[w].data_ptr(),
                                     d.q_coarse.data_ptr(), d.w_coarse.data_ptr(), d.bias.data_ptr())
        for l, lay in enumerate(self.extra_layers, start=1):
            trig[l] = lsa.lsa_trigger_in(lay["kic"].data_ptr(), lay["kic_scale"].data_ptr(),
                                         lay["q_coarse"].data_ptr(), lay["w_coarse"].data_ptr(),
                                         lay["bias"].data_ptr())
        return trig

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
        win = lsa.lsa_window_in(steps, qr.data_ptr(), wr.data_ptr(), qa.data_ptr(), lsa.trigger_ptr(nxt))
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


def token_row(inp, r: int, s: int) -> np.ndarray:
    """Stored bytes of token s's KV row of request r (history page or recent)."""
    cfg = inp.cfg
    rs = int(inp["rs"][r])
    if s < rs:
        pg = inp["pages"][int(inp["chunk_off"][r]) + s // cfg.chunk]
        o = (s % cfg.chunk) * cfg.kv_row_bytes
        return pg[o:o + cfg.kv_row_bytes]
    return inp["recent"][int(inp["rec_off"][r]) + s - rs]


def growing_state(full, L0, n_windows: int, recent_cap: int):
    """Host arrays of a growing-context run over the tokens of `full` (inputs
    generated at the final context lengths L0 + 64 * n_windows), in the
    fixed-capacity layout (chunk_cap chunks, recent_cap recent rows per
    request): the cold-tier pages, KIComp rows and scales of the history at
    L0, the recent rows, each step's appended row, and per window the index
    keys, KIComp row and scales of the chunk each request commits then (the
    recent region's oldest full chunk, once it holds W + 64 rows)."""
    cfg = full.cfg
    C, W, B = cfg.chunk, cfg.window, cfg.batch
    L = np.asarray(L0, np.int64).copy()
    if not np.array_equal(L + C * n_windows, np.asarray(full["seq_len"], np.int64)):
        raise ValueError("full must hold the contexts L0 + 64 * n_windows")
    rs0 = C * (np.maximum(L - W, 0) // C)
    chunk_cap = max(int(np.max(full["n_hist"])), 1)
    rb, pb = cfg.kv_row_bytes, cfg.page_bytes
    kb = cfg.d * synth.ELEM_BYTES[cfg.idx_dtype]
    pages = np.zeros((B * chunk_cap, pb), np.uint8)
    kic = np.zeros((B * chunk_cap, kb), np.uint8)
    ksc = np.ones(B * chunk_cap, np.float32)
    isc = np.ones(B * chunk_cap, np.float32)
    rec = np.zeros((B * recent_cap, rb), np.uint8)
    fk = full["kic_windows"][0].reshape(int(full["chunk_off"][-1]), -1).view(np.uint8)
    for r in range(B):
        f0, n0, o = int(full["chunk_off"][r]), int(rs0[r]) // C, r * chunk_cap
        pages[o:o + n0] = full["pages"][f0:f0 + n0]
        kic[o:o + n0] = fk[f0:f0 + n0]
        ksc[o:o + n0] = full["kic_scale_windows"][0][f0:f0 + n0]
        isc[o:o + n0] = full["ikey_scale"][f0:f0 + n0]
        for i, t in enumerate(range(int(rs0[r]), int(L[r]))):
            rec[r * recent_cap + i] = token_row(full, r, t)
    T = C * n_windows
    app = np.zeros((T, B, rb), np.uint8)
    for t in range(T):
        for r in range(B):
            app[t, r] = token_row(full, r, int(L[r]) + t)
    nik = np.zeros((n_windows, B, C * kb), np.uint8)
    nkc = np.zeros((n_windows, B, kb), np.uint8)
    nis = np.ones((n_windows, B), np.float32)
    nks = np.ones((n_windows, B), np.float32)
    commits = np.zeros((n_windows, B), bool)
    rs = rs0.copy()
    for m in range(n_windows):
        Lm = L + C * (m + 1)
        for r in range(B):
            if Lm[r] - rs[r] >= W + C:
                c = int(full["chunk_off"][r]) + int(rs[r]) // C
                nik[m, r] = full["pages"][c, cfg.ikey_off:cfg.ikey_off + C * kb]
                nkc[m, r] = fk[c]
                nis[m, r] = full["ikey_scale"][c]
                nks[m, r] = full["kic_scale_windows"][0][c]
                commits[m, r] = True
                rs[r] += C
    return dict(L0=L, rs0=rs0, chunk_cap=chunk_cap, pages=pages, kic=kic, kic_scale=ksc,
                ikey_scale=isc, recent=rec, app=app, nik=nik, nkc=nkc, nis=nis, nks=nks,
                commits=commits)


class Growing:
    """Growing-context decode over the tokens of `full` (inputs generated at
    the final context lengths), one entry point per step.  The run starts at
    contexts L0 and adds one token per step; every 64 steps (a window) it
    scores and selects the current history, and at the end of each window it
    commits the recent region's oldest full chunk into the history.  Device
    state uses fixed capacities per request (chunk_cap chunks, recent_cap
    recent rows): a cold tier of pages, KIComp rows and scales, and two recent
    buffers used in turn."""

    def __init__(self, full, L0, n_windows: int, device="cuda"):
        cfg = full.cfg
        C, W = cfg.chunk, cfg.window
        self.full, self.cfg, self.device, self.B = full, cfg, device, cfg.batch
        self.recent_cap = W + 2 * C
        st = growing_state(full, L0, n_windows, self.recent_cap)
        self.L, self.rs = st["L0"].copy(), st["rs0"].copy()
        self.n_windows = n_windows
        self.chunk_cap = st["chunk_cap"]
        B = self.B
        d = device
        self.pages = _dev(st["pages"].reshape(-1), d)
        self.kic, self.kic_scale = _dev(st["kic"].reshape(-1), d), _dev(st["kic_scale"], d)
        self.ikey_scale = _dev(st["ikey_scale"], d)
        rec = st["recent"]
        self.recent = [_dev(rec.reshape(-1), d), torch.zeros(rec.size, dtype=torch.uint8, device=d)]
        self.app = _dev(st["app"], d)
        self.nik, self.nkc = _dev(st["nik"], d), _dev(st["nkc"], d)
        self.nis, self.nks = _dev(st["nis"], d), _dev(st["nks"], d)
        self.q_coarse, self.w_coarse = _dev(full["q_coarse"], d), _dev(full["w_coarse"], d)
        self.bias = _dev(full["bias"], d)
        self.q_refine, self.w_refine = _dev(full["q_refine"], d), _dev(full["w_refine"], d)
        self.q_attn = _dev(full["q_attn"], d)
        self.kv = lsa.kv_layout(cfg.kv_dtype, cfg.Dk, cfg.Dv, cfg.v_off, cfg.kv_row_bytes,
                                cfg.page_bytes, cfg.ikey_off)
        self.cur = 0
        self.t = 0
        self.n_q = int(full["q_attn"].shape[0])  # per-step queries are reused cyclically past this
        self.sel = torch.full((B * self.chunk_cap,), -1, dtype=torch.int32, device=d)
        self.cnt = torch.zeros(B, dtype=torch.int32, device=d)
        self.z = torch.empty(B * self.chunk_cap, dtype=torch.float32, device=d)
        self._ws = {}
        self._k = None

    def _scratch(self, name, nbytes):
        w = self._ws.get(name)
        if w is None or w.numel() < nbytes:
            w = _ws(nbytes, self.device)
            self._ws[name] = w
        return w

    def _outputs(self, k):
        if self._k != k:
            cfg, d = self.cfg, self.device
            odt = torch.float32 if cfg.kv_dtype == synth.F32 else torch.int16
            self._topk = torch.full((self.B, k), -1, dtype=torch.int32, device=d)
            self._tcnt = torch.zeros(self.B, dtype=torch.int32, device=d)
            self._out = torch.empty((self.B, cfg.Hq, cfg.Dv), dtype=odt, device=d)
            self._lse = torch.empty((self.B, cfg.Hq), dtype=torch.float32, device=d)
            self._k = k
        return self._topk, self._tcnt, self._out, self._lse

    def geom(self):
        return lsa.Geom(self.L, self.cfg.window, self.cfg.chunk, hist_tokens=self.rs,
                        chunk_cap=self.chunk_cap, recent_cap=self.recent_cap)

    def trigger(self, theta=0.0, stream=None):
        """Score and select the current history (the window's trigger)."""
        cfg, g = self.cfg, self.geom()
        ws = self._scratch("score", lsa.lsa_score_ws_bytes(g, cfg.d))
        lsa.lsa_score_chunks(g, self.q_coarse, cfg.q_dtype, self.w_coarse, self.bias, cfg.H, cfg.d,
                             self.kic, cfg.idx_dtype, self.kic_scale, self.z, ws, stream)
        lsa.lsa_select_threshold(g, self.z, theta, self.sel, self.cnt, stream)
        return self.sel, self.cnt

    def step(self, k, stream=None):
        """One decode step: append the next token, refine and top-k over the
        window's selection, attend over the top-k and the grown recent region."""
        cfg, t = self.cfg, self.t
        tq = t % self.n_q
        self.L += 1
        g = self.geom()
        lsa.lsa_append_kv(g, self.kv, self.app[t], self.recent[self.cur], stream)
        topk, tcnt, out, lse = self._outputs(k)
        ws = self._scratch("refine", lsa.lsa_refine_ws_bytes(g, k))
        lsa.lsa_topk_refine(g, self.sel, self.cnt, self.pages, cfg.page_bytes, cfg.ikey_off, None,
                            cfg.idx_dtype, self.ikey_scale, self.q_refine[tq], cfg.q_dtype,
                            self.w_refine[tq], cfg.H, cfg.d, k, topk, tcnt, ws, stream)
        ws = self._scratch("attn", lsa.lsa_attn_ws_bytes(g, self.kv, cfg.Hq, k, 0))
        lsa.lsa_sparse_decode_attn(g, self.q_attn[tq], cfg.Hq, self.kv, self.pages, None,
                                   self.recent[self.cur], topk, tcnt, k, cfg.sm_scale, out, lse, 0, ws,
                                   stream)
        self.t += 1
        return topk, tcnt, out, lse

    def commit(self, m: int, stream=None):
        """End of window m: the oldest full recent chunk joins the history."""
        cfg, g = self.cfg, self.geom()
        self.rs = lsa.lsa_commit_chunk(g, self.kv, self.recent[self.cur], self.recent[1 - self.cur],
                                       self.pages, cfg.idx_dtype, cfg.d, self.nik[m], self.nis[m],
                                       self.ikey_scale, self.nkc[m], self.nks[m], self.kic,
                                       self.kic_scale, stream).astype(np.int64)
        self.cur = 1 - self.cur
        return self.rs


class GrowingPipeline:
    """Growing-context decode through the window pipeline (lsa_step64 with
    growing set) over the tokens of `full`, from contexts L0, n_windows
    windows of 64 steps.  Every trigger uses the request's own coarse query
    and the KIComp rows of the history it scores; before window m's call the
    KIComp rows (and scales) of the chunks committed in window m go into the
    trigger's arrays, since the next trigger scores them."""

    def __init__(self, full, L0, n_windows: int, host_cold=True, k=None, slots_per_req=None,
                 theta=0.0, device="cuda"):
        cfg = full.cfg
        self.full, self.cfg, self.B, self.device = full, cfg, cfg.batch, device
        C, W = cfg.chunk, cfg.window
        L0 = np.asarray(L0, np.int64)
        rs0 = C * (np.maximum(L0 - W, 0) // C)
        rmax = max(W + 63, int((L0 - rs0).max())) + 64
        self.recent_cap = 2 * rmax
        st = growing_state(full, L0, n_windows, self.recent_cap)
        self.st, self.n_windows, self.chunk_cap = st, n_windows, st["chunk_cap"]
        d = device
        self.geom = lsa.Geom(st["L0"], W, C, hist_tokens=st["rs0"], chunk_cap=self.chunk_cap,
                             recent_cap=self.recent_cap)
        self.pages = _pinned(st["pages"].reshape(-1)) if host_cold else _dev(st["pages"].reshape(-1), d)
        self.kic, self.kic_scale = _dev(st["kic"].reshape(-1), d), _dev(st["kic_scale"], d)
        self.ikey_scale = _dev(st["ikey_scale"], d)
        self.recent = _dev(st["recent"].reshape(-1), d)
        self.app = _dev(st["app"], d)
        self.nik, self.nis = _dev(st["nik"], d), _dev(st["nis"], d)
        self.nkc, self.nks = _dev(st["nkc"], d), _dev(st["nks"], d)
        # KIComp rows each window commits: (row in kic, window, request)
        self.kic_rows = []
        n = (st["rs0"] // C).astype(np.int64)
        for m in range(n_windows):
            rows = [(r * self.chunk_cap + int(n[r]), r) for r in range(self.B) if st["commits"][m, r]]
            n = n + st["commits"][m]
            self.kic_rows.append((torch.tensor([x[0] for x in rows], dtype=torch.int64, device=d),
                                  torch.tensor([x[1] for x in rows], dtype=torch.int64, device=d)))
        self.q_coarse, self.w_coarse = _dev(full["q_coarse"], d), _dev(full["w_coarse"], d)
        self.bias = _dev(full["bias"], d)
        self.q_refine, self.w_refine = _dev(full["q_refine"], d), _dev(full["w_refine"], d)
        self.q_attn = _dev(full["q_attn"], d)
        self.n_q = int(full["q_attn"].shape[0])
        self.kv = lsa.kv_layout(cfg.kv_dtype, cfg.Dk, cfg.Dv, cfg.v_off, cfg.kv_row_bytes,
                                cfg.page_bytes, cfg.ikey_off)
        self.k = cfg.topk if k is None else k
        spr = cfg.slots_per_req if slots_per_req is None else slots_per_req
        self.spr = max(1, min(spr, self.chunk_cap))
        self.slots = torch.empty(self.B * self.spr * cfg.page_bytes, dtype=torch.uint8, device=d)
        self.pool = lsa.Pool(self.geom, self.slots, self.spr, cfg.page_bytes, self.pages, host_cold)
        desc = lsa.lsa_ctx_desc()
        desc.geom = self.geom.s
        desc.H, desc.d, desc.q_dt, desc.idx_dt = cfg.H, cfg.d, cfg.q_dtype, cfg.idx_dtype
        desc.Hq, desc.k = cfg.Hq, self.k
        desc.kv = self.kv
        desc.sm_scale, desc.theta = cfg.sm_scale, theta
        desc.recent = self.recent.data_ptr()
        desc.ikey_scale = self.ikey_scale.data_ptr()
        desc.pool = self.pool.h.value
        desc.n_layers = 1
        desc.growing = 1
        nbytes = lsa.lsa_ctx_ws_bytes(desc)
        if nbytes == 0:
            raise lsa.LsaError("lsa_ctx_ws_bytes", -1)
        self.ws = _ws(nbytes, d)
        desc.ws, desc.ws_bytes = self.ws.data_ptr(), self.ws.numel()
        self.ctx = lsa.Ctx(desc, keep=(self,))
        self.copy_stream = torch.cuda.Stream(device=d)
        self.sel_cnt = np.zeros(self.B, dtype=np.int32)
        self.trig = lsa.lsa_trigger_in(self.kic.data_ptr(), self.kic_scale.data_ptr(),
                                       self.q_coarse.data_ptr(), self.w_coarse.data_ptr(),
                                       self.bias.data_ptr())

    def prime(self, main=None):
        st = self.ctx.prime(self.trig, main, self.copy_stream, self.sel_cnt)
        return st, self.sel_cnt.copy()

    def window(self, m: int, out, lse=None, topk=None, tcnt=None, last=False, main=None):
        """Window m: 64 steps (queries of steps 64 m .. 64 m + 63, cyclic past
        the inputs' own), appending app[64 m + j] at step j."""
        rows, reqs = self.kic_rows[m]
        if len(rows):  # the next trigger scores the chunks this window commits
            kb = self.kic.numel() // (self.B * self.chunk_cap)
            self.kic.view(-1, kb).index_copy_(0, rows, self.nkc[m].index_select(0, reqs))
            self.kic_scale.index_copy_(0, rows, self.nks[m].index_select(0, reqs))
        t0 = (64 * m) % self.n_q
        if t0 + 64 > self.n_q:
            raise ValueError("the inputs hold too few steps of queries for a whole window")
        win = lsa.lsa_window_in(64, self.q_refine[t0].data_ptr(), self.w_refine[t0].data_ptr(),
                                self.q_attn[t0].data_ptr(), None if last else lsa.trigger_ptr(self.trig),
                                self.app[64 * m].data_ptr(), self.nik[m].data_ptr(),
                                self.nis[m].data_ptr())
        wo = lsa.lsa_window_out()
        wo.out = out.data_ptr()
        wo.lse = lse.data_ptr() if lse is not None else None
        wo.topk_idx = topk.data_ptr() if topk is not None else None
        wo.topk_cnt = tcnt.data_ptr() if tcnt is not None else None
        wo.sel_cnt = self.sel_cnt.ctypes.data
        st = self.ctx.step64(win, wo, main, self.copy_stream)
        return st, self.sel_cnt.copy()

    def state(self):
        return self.ctx.state()

    def close(self):
        torch.cuda.synchronize()
        self.ctx.close()
        self.pool.close()
