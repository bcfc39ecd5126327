"""Shared test helpers: tiny custom inputs built on the seeded generator."""
import dataclasses

import numpy as np

from learned_sparse_kv_amd import synth


def tiny_cfg(**kw):
    """A very small f32 configuration (C=4) for brute-force checks."""
    base = dict(name="tiny", seed=5, batch=2, seq_lens=(40, 23), chunk=4, window=8, H=3, d=5,
                q_dtype=synth.F32, idx_dtype=synth.F32, planted=0.25, topk=6, Hq=2, Dk=6,
                Dv=6, kv_dtype=synth.F32, separate_v=True, steps=2)
    base.update(kw)
    cfg = synth.LsaConfig(**base)
    return cfg


def tiny_inputs(**kw):
    """Tiny inputs with head weights that differ per head, request and step."""
    cfg = tiny_cfg(**kw)
    inp = synth.generate(cfg)
    rng = np.random.default_rng(cfg.seed + 100)
    inp["w_coarse"] = rng.uniform(-1.0, 1.0, inp["w_coarse"].shape).astype(np.float32)
    inp["w_refine"] = rng.uniform(-1.0, 1.0, inp["w_refine"].shape).astype(np.float32)
    inp["bias"] = rng.uniform(-1.0, 1.0, inp["bias"].shape).astype(np.float32)
    return inp


def with_cfg(inp, **kw):
    inp.cfg = dataclasses.replace(inp.cfg, **kw)
    return inp


def kv_rows(inp, r):
    """Decoded K and V rows of request r for tokens [0, L) (test-side reader)."""
    from oracle import oracle
    cfg = inp.cfg
    L = int(inp["seq_len"][r])
    rs, nh, nr = oracle.geometry(L, cfg.chunk, cfg.window)
    c0, q0 = int(inp["chunk_off"][r]), int(inp["rec_off"][r])
    rows = []
    for s in range(L):
        if s < rs:
            pg = inp["pages"][c0 + s // cfg.chunk]
            raw = pg[(s % cfg.chunk) * cfg.kv_row_bytes:(s % cfg.chunk + 1) * cfg.kv_row_bytes]
        else:
            raw = inp["recent"][q0 + s - rs]
        dt = {0: np.float32, 1: np.uint16}[cfg.kv_dtype]
        rows.append(oracle.decode(cfg.kv_dtype, raw.view(dt)).astype(np.float64))
    rows = np.stack(rows)
    K = rows[:, :cfg.Dk]
    V = rows[:, cfg.v_off:cfg.v_off + cfg.Dv]
    return K, V


def dense_attention(q, K, V, sm):
    """Textbook softmax attention in float64: q [Hq, Dk], K [n, Dk], V [n, Dv]."""
    x = sm * (q @ K.T)
    m = x.max(axis=1, keepdims=True)
    p = np.exp(x - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ V) / l, (m + np.log(l))[:, 0]


def stored_row(inp, r, s):
    """Stored bytes of token s's KV row of request r (its page or the recent rows)."""
    cfg = inp.cfg
    rs = int(inp["rs"][r])
    if s < rs:
        o = (s % cfg.chunk) * cfg.kv_row_bytes
        return inp["pages"][int(inp["chunk_off"][r]) + s // cfg.chunk][o:o + cfg.kv_row_bytes]
    return inp["recent"][int(inp["rec_off"][r]) + s - rs]


def growing_snapshot(full, r, L, rs):
    """Request r of `full` (inputs generated at the final contexts) as a
    growing-context run holds it at context L with history boundary rs:
    history chunks [0, rs/C) with their pages, KIComp rows and scales,
    tokens [rs, L) as recent rows, and the request's per-step queries.  One
    request, packed; the window is L - rs so the geometry puts rs there."""
    cfg = full.cfg
    C = cfg.chunk
    n = rs // C
    sc = dataclasses.replace(cfg, batch=1, seq_lens=(L,), window=L - rs)
    inp = synth.Inputs()
    inp.cfg = sc
    f0 = int(full["chunk_off"][r])
    inp.update(seq_len=np.array([L], np.int32), chunk_off=np.array([0, n], np.int64),
               rec_off=np.array([0, L - rs], np.int64), rs=np.array([rs], np.int64),
               n_hist=np.array([n], np.int64), n_rec=np.array([L - rs], np.int64))
    inp["pages"] = np.ascontiguousarray(full["pages"][f0:f0 + n])
    inp["ikey_scale"] = np.ascontiguousarray(full["ikey_scale"][f0:f0 + n])
    inp["kic"] = np.ascontiguousarray(full["kic_windows"][0][f0:f0 + n])
    inp["kic_scale"] = np.ascontiguousarray(full["kic_scale_windows"][0][f0:f0 + n])
    inp["recent"] = np.stack([stored_row(full, r, s) for s in range(rs, L)])
    for key in ("q_coarse", "w_coarse", "bias"):
        inp[key] = np.ascontiguousarray(full[key][r:r + 1])
    for key in ("q_refine", "w_refine", "q_attn"):
        inp[key] = np.ascontiguousarray(full[key][:, r:r + 1])
    return inp
