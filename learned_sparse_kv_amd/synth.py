"""Seeded synthetic inputs for the LSA decode hot path.

This module only draws random numbers and lays them out in the byte layout
that the C-ABI (include/lsa.h) and the CPU oracle both read.  It performs no
step of the method: no scoring, selection, refinement, top-k or attention.
The one piece of arithmetic it does on method quantities is computing the
direction used to *plant* relevant chunks (the fused coarse query, in
float64), which is part of the input recipe, not of the result.

Recipe (one ``numpy.random.SeedSequence`` per config, spawned per tensor and
per request, PCG64 streams):

* KIComp rows ~ N(0, 1/d); a random ``planted`` share of history chunks get
  ``+2.0 * u`` added, u the unit direction of sum_h w_h q_h.
* coarse query q_h ~ N(0, H/4) per element, w_h = 1/H, b = -1.0.  The fused
  query then has per-element variance 1/4, unplanted logits are ~N(-1, 1/4)
  (about 2.3 % of them exceed 0) and planted logits sit far above 0.
  With ``signed_weights`` the head weights (coarse and per step) are drawn
  U(-1, 1) per head and scaled so that sum_h w_h^2 = 1/H as for 1/H (so the
  fused query keeps its variance), and each request's bias is drawn
  U(-1.25, -0.75): weights of both signs that are not powers of two.
* per-token index keys ~ N(0, 1/d); refine queries ~ N(0, 1), w = 1/H.
* attention queries and KV ~ N(0, 1); separate K and V for the fp32 config,
  a 576-wide latent row (value = first 512) otherwise.
* bf16 by round-to-nearest-even; fp8 E4M3FN per chunk block with scale
  s = max|x| / 448 and byte = RNE(x / s) (saturated to +-448).
* drift (multi-window runs): per window, ``round(drift/2 * N_hist)`` planted
  chunks are un-planted and as many new ones planted.

Layout (per request r with context L_r, chunk C, recent window W):
rs_r = C*floor(max(L_r - W, 0)/C) history tokens in N_r = rs_r/C chunks, and
R_r = L_r - rs_r recent tokens.  Arrays over chunks are concatenated over
requests (``[sum N_r, ...]``), recent rows likewise (``[sum R_r, row]``).
A page holds one chunk: C KV rows, then C index-key rows.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

F32, BF16, FP8 = 0, 1, 2          # dtype codes shared with the C-ABI enum
ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1}


@dataclasses.dataclass
class LsaConfig:
    name: str
    seed: int
    batch: int
    seq_lens: tuple | None          # None: drawn from len_range
    len_range: tuple = (0, 0)
    chunk: int = 64
    window: int = 8192
    H: int = 64                     # indexer heads
    d: int = 128                    # indexer dim
    q_dtype: int = BF16             # indexer query dtype
    idx_dtype: int = BF16           # KIComp and per-token index key dtype
    planted: float = 0.12
    topk: int = 2048
    Hq: int = 64
    Dk: int = 576
    Dv: int = 512
    kv_dtype: int = BF16
    separate_v: bool = False        # True: K row and V row stored side by side
    steps: int = 64
    windows: int = 1                # KIComp versions (drift between them)
    drift: float = 0.0
    host_cold: bool = False         # cold tier lives in pinned host memory
    slots_per_req: int = 1024
    signed_weights: bool = False    # head weights U(-1, 1) (scaled), bias per request

    # ---- layout sizes (byte layout of the ABI) ----
    @property
    def kv_row_elems(self) -> int:
        return self.Dk + (self.Dv if self.separate_v else 0)

    @property
    def kv_row_bytes(self) -> int:
        return self.kv_row_elems * ELEM_BYTES[self.kv_dtype]

    @property
    def ikey_row_bytes(self) -> int:
        return self.d * ELEM_BYTES[self.idx_dtype]

    @property
    def page_bytes(self) -> int:
        return self.chunk * (self.kv_row_bytes + self.ikey_row_bytes)

    @property
    def ikey_off(self) -> int:
        return self.chunk * self.kv_row_bytes

    @property
    def v_off(self) -> int:
        return self.Dk if self.separate_v else 0

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.Dk)))


def layout(cfg: LsaConfig, seq_lens):
    """Chunk/recent counts and offsets implied by the layout contract."""
    L = np.asarray(seq_lens, dtype=np.int64)
    C, W = cfg.chunk, cfg.window
    rs = C * (np.maximum(L - W, 0) // C)
    n_hist = rs // C
    n_rec = L - rs
    chunk_off = np.concatenate([[0], np.cumsum(n_hist)]).astype(np.int64)
    rec_off = np.concatenate([[0], np.cumsum(n_rec)]).astype(np.int64)
    return rs, n_hist, n_rec, chunk_off, rec_off


# ----------------------------------------------------------------------------
# encoders (input casting only)
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_fp8_blocks(x: np.ndarray):
    """x: [nblk, ...] float; per-block scale max|x|/448; returns (bytes, scale)."""
    xb = x.reshape(x.shape[0], -1).astype(np.float32)
    amax = np.abs(xb).max(axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    y = np.clip(xb / scale[:, None], -448.0, 448.0).astype(np.float32)
    enc = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return enc.reshape(x.shape), scale


def encode(x: np.ndarray, dt: int):
    if dt == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dt == BF16:
        return to_bf16_bits(x)
    raise ValueError("use to_fp8_blocks for fp8")


def decode_query_f64(q_enc: np.ndarray, dt: int) -> np.ndarray:
    """Value of an encoded query (for the planting direction only)."""
    if dt == F32:
        return q_enc.astype(np.float64)
    return (q_enc.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------
def config(k: int) -> LsaConfig:
    if k == 0:
        return LsaConfig("cfg0_tiny_f32_16k", 0, 1, (16384,), window=2048, H=4, d=64,
                         q_dtype=F32, idx_dtype=F32, planted=0.12, topk=512, Hq=8,
                         Dk=128, Dv=128, kv_dtype=F32, separate_v=True, steps=64)
    if k == 1:
        return LsaConfig("cfg1_bf16_64k", 1, 1, (65536,))
    if k == 2:
        return LsaConfig("cfg2_bf16_ragged16_32k-128k", 2, 16, None, len_range=(32768, 131072))
    if k == 3:
        return LsaConfig("cfg3_fp8idx_500k_b4", 3, 4, (512000,) * 4, idx_dtype=FP8,
                         planted=0.08)
    if k == 4:
        return LsaConfig("cfg4_step64_500k_b8_hostcold", 4, 8, (512000,) * 8, idx_dtype=FP8,
                         planted=0.08, steps=256, windows=5, drift=0.02, host_cold=True)
    raise KeyError(k)


def config_2u() -> LsaConfig:
    """cfg 2 with every context fixed to 131,072 tokens (clean 128K point)."""
    c = config(2)
    return dataclasses.replace(c, name="cfg2u_bf16_128k_b16", seq_lens=(131072,) * 16)


def seq_lens_of(cfg: LsaConfig):
    if cfg.seq_lens is not None:
        return np.asarray(cfg.seq_lens, dtype=np.int64)
    ss = np.random.SeedSequence([cfg.seed, 0xC0FFEE])
    rng = np.random.Generator(np.random.PCG64(ss))
    lo, hi = cfg.len_range
    raw = rng.integers(lo, hi + 1, size=cfg.batch)
    return (cfg.chunk * np.rint(raw / cfg.chunk)).astype(np.int64)


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------
_T_KIC, _T_PLANT, _T_QC, _T_IKEY, _T_KVH, _T_KVR, _T_QR, _T_QA, _T_DRIFT = range(9)
_T_LAYER = 100  # tensor ids of indexer layer l >= 1: _T_LAYER + 10 l + {0: KIComp, 1: planted, 2: query, 3: weights}
_T_POLICY = 200  # random-policy keys of window w: _T_POLICY + w
_T_FOCUS = 300
_T_WC, _T_WR = 400, 402  # signed coarse weights (and biases), refine weights


def _rng(root: np.random.SeedSequence, tensor: int, req: int = 0):
    ss = np.random.SeedSequence(root.entropy, spawn_key=(tensor, req))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _signed_weights(rng, shape):
    """Head weights (last axis) of both signs: U(-1, 1), scaled per row so
    that sum_h w_h^2 = 1/H, as for the uniform weights 1/H."""
    u = rng.uniform(-1.0, 1.0, size=shape)
    H = shape[-1]
    u /= np.sqrt(H * (u * u).sum(axis=-1, keepdims=True))
    return u.astype(np.float32)


def _coarse_weights(cfg, root, tensor, B, H):
    """Coarse head weights [B, H] and biases [B] of one indexer layer."""
    if not cfg.signed_weights:
        return np.full((B, H), 1.0 / H, dtype=np.float32), np.full((B,), -1.0, dtype=np.float32)
    w, b = np.zeros((B, H), np.float32), np.zeros(B, np.float32)
    for r in range(B):
        rng = _rng(root, tensor, r)  # the request's weights, then its bias
        w[r] = _signed_weights(rng, (H,))
        b[r] = rng.uniform(-1.25, -0.75)
    return w, b


class Inputs(dict):
    """Dict of numpy arrays plus the config and the layout sizes."""


def generate(cfg: LsaConfig, steps: int | None = None, threads: int = 8) -> Inputs:
    steps = cfg.steps if steps is None else steps
    L = seq_lens_of(cfg)
    rs, n_hist, n_rec, chunk_off, rec_off = layout(cfg, L)
    B, C, H, d = cfg.batch, cfg.chunk, cfg.H, cfg.d
    NH, NR = int(chunk_off[-1]), int(rec_off[-1])
    root = np.random.SeedSequence(cfg.seed)
    out = Inputs()
    out.cfg = cfg
    out.update(seq_len=L.astype(np.int32), chunk_off=chunk_off, rec_off=rec_off,
               rs=rs, n_hist=n_hist, n_rec=n_rec)

    # ---- coarse query, head weights, bias ----
    q_raw = np.stack([_normal(_rng(root, _T_QC, r), (H, d), std=np.sqrt(H / 4.0))
                      for r in range(B)])
    out["q_coarse"] = encode(q_raw, cfg.q_dtype)
    out["w_coarse"], out["bias"] = _coarse_weights(cfg, root, _T_WC, B, H)
    qv = decode_query_f64(out["q_coarse"], cfg.q_dtype)
    u = np.einsum("bh,bhd->bd", out["w_coarse"].astype(np.float64), qv)
    u /= np.linalg.norm(u, axis=1, keepdims=True)

    # ---- KIComp (one version per window; drift between versions) ----
    kic_noise = np.zeros((NH, d), dtype=np.float32)
    planted_sets = [[None] * B for _ in range(cfg.windows)]
    for r in range(B):
        n = int(n_hist[r])
        kic_noise[chunk_off[r]:chunk_off[r + 1]] = _normal(_rng(root, _T_KIC, r), (n, d),
                                                           std=1.0 / np.sqrt(d))
        prng = _rng(root, _T_PLANT, r)
        n_pl = int(round(cfg.planted * n))
        cur = np.sort(prng.choice(n, size=n_pl, replace=False)) if n else np.zeros(0, np.int64)
        planted_sets[0][r] = cur
        drng = _rng(root, _T_DRIFT, r)
        n_sw = int(round(cfg.drift / 2 * n))
        for m in range(1, cfg.windows):
            if n_sw > 0 and n > 0:
                drop = drng.choice(cur, size=min(n_sw, len(cur)), replace=False)
                rest = np.setdiff1d(np.arange(n), cur)
                add = drng.choice(rest, size=min(n_sw, len(rest)), replace=False)
                cur = np.sort(np.union1d(np.setdiff1d(cur, drop), add))
            planted_sets[m][r] = cur
    kic_list, kic_scale_list = [], []
    for m in range(cfg.windows):
        rows = kic_noise.copy()
        for r in range(B):
            idx = chunk_off[r] + planted_sets[m][r]
            rows[idx] += (2.0 * u[r]).astype(np.float32)
        if cfg.idx_dtype == FP8:
            enc, sc = to_fp8_blocks(rows)
        else:
            enc, sc = encode(rows, cfg.idx_dtype), np.ones(NH, np.float32)
        kic_list.append(enc)
        kic_scale_list.append(sc)
    out["kic"] = kic_list[0]
    out["kic_scale"] = kic_scale_list[0]
    out["kic_windows"] = kic_list
    out["kic_scale_windows"] = kic_scale_list
    out["planted"] = planted_sets

    # ---- pages: [NH, page_bytes]: C KV rows then C index-key rows ----
    pages = np.empty((NH, cfg.page_bytes), dtype=np.uint8)
    ikey_scale = np.ones(NH, dtype=np.float32)

    def fill_request(r):
        n = int(n_hist[r])
        if n == 0:
            return
        base = int(chunk_off[r])
        kv_rng = _rng(root, _T_KVH, r)
        ik_rng = _rng(root, _T_IKEY, r)
        blk = 256  # chunks per block, bounds the float32 temporaries
        for c0 in range(0, n, blk):
            c1 = min(n, c0 + blk)
            nb = c1 - c0
            kv = _normal(kv_rng, (nb, C, cfg.kv_row_elems))
            kv_enc = encode(kv, cfg.kv_dtype).reshape(nb, -1).view(np.uint8)
            ik = _normal(ik_rng, (nb, C, d), std=1.0 / np.sqrt(d))
            if cfg.idx_dtype == FP8:
                ik_enc, sc = to_fp8_blocks(ik)
                ikey_scale[base + c0:base + c1] = sc
            else:
                ik_enc = encode(ik, cfg.idx_dtype)
            pg = pages[base + c0:base + c1]
            pg[:, :cfg.ikey_off] = kv_enc
            pg[:, cfg.ikey_off:] = ik_enc.reshape(nb, -1).view(np.uint8)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill_request, range(B)))
    out["pages"] = pages
    out["ikey_scale"] = ikey_scale

    # ---- recent KV rows [NR, kv_row_bytes] ----
    recent = np.empty((NR, cfg.kv_row_bytes), dtype=np.uint8)
    for r in range(B):
        x = _normal(_rng(root, _T_KVR, r), (int(n_rec[r]), cfg.kv_row_elems))
        enc = np.ascontiguousarray(encode(x, cfg.kv_dtype)).view(np.uint8)
        recent[rec_off[r]:rec_off[r + 1]] = enc.reshape(int(n_rec[r]), cfg.kv_row_bytes)
    out["recent"] = recent

    # ---- per-step refine and attention queries ----
    qr = _normal(_rng(root, _T_QR), (steps, B, H, d))
    out["q_refine"] = encode(qr, cfg.q_dtype)
    if cfg.signed_weights:
        out["w_refine"] = _signed_weights(_rng(root, _T_WR), (steps, B, H))
    else:
        out["w_refine"] = np.full((steps, B, H), 1.0 / H, dtype=np.float32)
    qa = _normal(_rng(root, _T_QA), (steps, B, cfg.Hq, cfg.Dk))
    out["q_attn"] = encode(qa, cfg.kv_dtype)
    return out


def small_config(name="small_bf16", seed=11, seq_lens=(5000, 3000), window=1024, idx=BF16,
                 topk=256, steps=3, H=8, d=128, Hq=64, Dk=576, Dv=512, kv=BF16,
                 separate_v=False, planted=0.12, q_dtype=None, signed_weights=False) -> LsaConfig:
    """Parity-test shapes: several tiles and a ragged tail, seconds on the CPU."""
    return LsaConfig(name, seed, len(seq_lens), tuple(seq_lens), window=window, H=H, d=d,
                     q_dtype=(F32 if kv == F32 else BF16) if q_dtype is None else q_dtype,
                     idx_dtype=idx, planted=planted, topk=topk, Hq=Hq, Dk=Dk, Dv=Dv,
                     kv_dtype=kv, separate_v=separate_v, steps=steps,
                     signed_weights=signed_weights)


def attention_focus(inp: Inputs, boost: float = 2.5, window: int = 0) -> Inputs:
    """A copy of inp in which attention prefers the planted chunks of the
    given window, as the method presumes (the indexer predicts the history
    the next steps attend to).  Per request, one seeded unit direction v_r
    (Dk dims) is added with weight a = sqrt(boost / sm) to the key part of
    every KV row of those chunks and to every attention query, so that
    sm * q . k rises by about boost (natural-log units) for their tokens.
    Only pages and q_attn change; the copy owns new arrays for them."""
    cfg = inp.cfg
    if cfg.kv_dtype != BF16:
        raise ValueError("attention_focus writes bf16 rows")
    root = np.random.SeedSequence(cfg.seed)
    a = np.sqrt(boost / cfg.sm_scale)
    C, Dk, rw = cfg.chunk, cfg.Dk, cfg.kv_row_bytes // 2
    out = Inputs(inp)
    out.cfg = cfg
    pages = inp["pages"].copy()
    qa = (inp["q_attn"].astype(np.uint32) << 16).view(np.float32).copy()
    for r in range(cfg.batch):
        v = _rng(root, _T_FOCUS, r).standard_normal(Dk)
        v = (v / np.linalg.norm(v) * a).astype(np.float32)
        qa[:, r] += v
        pl = np.asarray(inp["planted"][window][r], dtype=np.int64)
        if len(pl) == 0:
            continue
        rows = pages[int(inp["chunk_off"][r]) + pl, :cfg.ikey_off].view(np.uint16).reshape(len(pl), C, rw)
        k = (rows[:, :, :Dk].astype(np.uint32) << 16).view(np.float32) + v
        rows[:, :, :Dk] = to_bf16_bits(k)
        pages[int(inp["chunk_off"][r]) + pl, :cfg.ikey_off] = rows.reshape(len(pl), -1).view(np.uint8)
    out["pages"] = pages
    out["q_attn"] = to_bf16_bits(qa)
    return out


def policy_keys(inp: Inputs, window: int = 0) -> np.ndarray:
    """Uniform 32-bit keys, one per history chunk ([sum N] uint32, one stream
    per request and window): keeping the chunks of smallest key is a uniform
    random sample without replacement (the random-share policy)."""
    cfg = inp.cfg
    root = np.random.SeedSequence(cfg.seed)
    n_hist = inp["n_hist"]
    out = np.zeros(int(inp["chunk_off"][-1]), np.uint32)
    for r in range(cfg.batch):
        a, n = int(inp["chunk_off"][r]), int(n_hist[r])
        out[a:a + n] = _rng(root, _T_POLICY + window, r).integers(0, 2 ** 32, n, dtype=np.uint32)
    return out


def indexer_layers(inp: Inputs, n_layers: int = 3, window: int = 0):
    """Coarse-indexer inputs of n_layers independent memory indexers (the
    pages place three, at layers 10, 12 and 20).  Layer 0 is the inputs' own
    indexer; layer l >= 1 draws its own coarse query (same law), its own
    KIComp noise, and its own planted chunks (same rate, drawn independently,
    so the layers' selections overlap only partly).  Returns a list of dicts
    with q_coarse, w_coarse, bias, kic, kic_scale for the given window."""
    cfg = inp.cfg
    B, H, d = cfg.batch, cfg.H, cfg.d
    chunk_off, n_hist = inp["chunk_off"], inp["n_hist"]
    NH = int(chunk_off[-1])
    root = np.random.SeedSequence(cfg.seed)
    layers = [dict(q_coarse=inp["q_coarse"], w_coarse=inp["w_coarse"], bias=inp["bias"],
                   kic=inp["kic_windows"][window], kic_scale=inp["kic_scale_windows"][window])]
    for l in range(1, n_layers):
        t = _T_LAYER + 10 * l
        q_raw = np.stack([_normal(_rng(root, t + 2, r), (H, d), std=np.sqrt(H / 4.0)) for r in range(B)])
        q_enc = encode(q_raw, cfg.q_dtype)
        w, bias = _coarse_weights(cfg, root, t + 3, B, H)
        qv = decode_query_f64(q_enc, cfg.q_dtype)
        u = np.einsum("bh,bhd->bd", w.astype(np.float64), qv)
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        rows = np.zeros((NH, d), dtype=np.float32)
        for r in range(B):
            n = int(n_hist[r])
            rows[chunk_off[r]:chunk_off[r + 1]] = _normal(_rng(root, t, r), (n, d), std=1.0 / np.sqrt(d))
            if n:
                pl = np.sort(_rng(root, t + 1, r).choice(n, size=int(round(cfg.planted * n)), replace=False))
                rows[chunk_off[r] + pl] += (2.0 * u[r]).astype(np.float32)
        if cfg.idx_dtype == FP8:
            enc, sc = to_fp8_blocks(rows)
        else:
            enc, sc = encode(rows, cfg.idx_dtype), np.ones(NH, np.float32)
        layers.append(dict(q_coarse=q_enc, w_coarse=w, bias=bias, kic=enc, kic_scale=sc))
    return layers
