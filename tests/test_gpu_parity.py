"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Bars (the decode hot path's stated targets):
  * chunk logits z bit-identical, selected chunk ids and counts exact;
  * top-k token indices and counts exact;
  * attention output within max relative error 1e-5 (fp32 rows) or 2e-2
    (bf16 rows; 6e-2 allowed with fp8 index keys, which only change which
    tokens are selected), measured per (request, step, head) vector as
    max_i |o_i - r_i| / max_i |r_i|; lse within a small absolute bound.
"""
import numpy as np
import pytest
import torch

from learned_sparse_kv_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu

F32, BF16, FP8 = synth.F32, synth.BF16, synth.FP8


def _runner():
    from learned_sparse_kv_amd import runner
    return runner


def _lsa():
    from learned_sparse_kv_amd import lsa
    return lsa


def small(kind):
    """Parity-test configurations; a "_sw" suffix gives the same shapes with
    signed head weights that are not powers of two and a bias per request."""
    if kind.endswith("_sw"):
        return synth.dataclasses.replace(small(kind[:-3]), signed_weights=True, name=kind)
    if kind == "f32":
        return synth.small_config("f32_small", 21, (5000, 2100, 700), window=1024, idx=F32, kv=F32,
                                  H=4, d=64, Hq=8, Dk=128, Dv=128, separate_v=True, topk=256,
                                  steps=2)
    if kind == "bf16":
        return synth.small_config("bf16_small", 22, (9000, 4100, 300), window=1024, idx=BF16, H=16,
                                  topk=256, steps=2)
    if kind == "fp8":
        return synth.small_config("fp8_small", 23, (9000, 6500), window=1024, idx=FP8, H=16,
                                  topk=512, steps=2)
    if kind == "bf16_h8":  # head count off the matrix-core path: the VALU refine
        return synth.small_config("bf16_h8", 25, (7000, 2500), window=1024, idx=BF16, H=8,
                                  topk=256, steps=2)
    if kind == "bf16_qf32":  # fp32 queries: the one-lane-per-chunk sigmoid score
        return synth.small_config("bf16_qf32", 26, (6000, 2500), window=1024, idx=BF16, H=16,
                                  topk=256, steps=1, q_dtype=F32)
    if kind == "fp8_qf32":
        return synth.small_config("fp8_qf32", 27, (6000, 4000), window=1024, idx=FP8, H=16,
                                  topk=256, steps=1, q_dtype=F32)
    if kind == "bf16_hq32":  # 32 attention heads: the wave-pair attention kernel
        return synth.small_config("bf16_hq32", 28, (6000, 2600, 500), window=1024, idx=BF16, H=16,
                                  Hq=32, topk=256, steps=2)
    if kind == "bf16_h128":
        return synth.small_config("bf16_h128", 24, (4000,), window=512, idx=BF16, H=16, Hq=128,
                                  topk=128, steps=1)
    raise KeyError(kind)


def tol_of(cfg):
    if cfg.kv_dtype == F32:
        return 1e-5, 1e-5
    return (6e-2 if cfg.idx_dtype == FP8 else 2e-2), 2e-3


def rel_err(got, ref):
    return (np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30))


_cache = {}


def config_of(kind):
    if not kind.startswith("cfg"):
        return small(kind)
    cfg = synth.config(int(kind[3]))
    if kind.endswith("_sw"):
        cfg = synth.dataclasses.replace(cfg, signed_weights=True, name=cfg.name + "_sw")
    return cfg


def setup(kind):
    """Inputs, device copies and oracle of a kind.  Small kinds stay cached;
    a full-size config replaces every other full-size one."""
    if kind not in _cache:
        cfg = config_of(kind)
        steps = None if not kind.startswith("cfg") else 2
        inp = synth.generate(cfg, steps=steps)
        print(f"[setup] {kind}: lens={list(inp['seq_len'])} n_hist={list(inp['n_hist'])}",
              flush=True)
        if kind.startswith("cfg"):
            for k in [k for k in _cache if k.startswith("cfg")]:
                del _cache[k]
        _cache[kind] = (inp, _runner().DeviceInputs(inp), oracle.Oracle(inp))
    return _cache[kind]


SMALL = ["f32", "bf16", "fp8", "bf16_h128", "bf16_h8"]
SIGNED = [k + "_sw" for k in SMALL] + ["cfg3_sw"]


@pytest.mark.parametrize("kind", SMALL + ["cfg0", "cfg1", "cfg2", "cfg3"] + SIGNED)
def test_score_select_bitexact(kind):
    inp, dev, o = setup(kind)
    z, sel, cnt = dev.score_select()
    torch.cuda.synchronize()
    z_o, sel_o, cnt_o = o.score_select()
    assert np.array_equal(z.cpu().numpy().view(np.uint32), z_o.view(np.uint32))
    c = cnt.cpu().numpy()
    assert np.array_equal(c, cnt_o)
    s = sel.cpu().numpy()
    for r in range(inp.cfg.batch):
        a = int(inp["chunk_off"][r])
        assert np.array_equal(s[a:a + c[r]], sel_o[a:a + c[r]])


def _units(inp, full):
    B, S = inp.cfg.batch, inp["q_refine"].shape[0]
    if full:
        return [(r, j) for r in range(B) for j in range(S)]
    # full-size configs: a few sampled units (first, last and a middle request)
    rs = sorted({0, B // 2, B - 1})
    return [(r, j % S) for j, r in enumerate(rs)]


@pytest.mark.parametrize("kind", SMALL + ["bf16_hq32", "cfg0", "cfg1", "cfg2", "cfg3"] + SIGNED)
def test_refine_topk_and_attention(kind):
    inp, dev, o = setup(kind)
    cfg = inp.cfg
    full = not kind.startswith("cfg") or kind == "cfg0"
    z, sel, cnt = dev.score_select()
    _, sel_o, cnt_o = o.score_select()
    units = _units(inp, full)
    tk_o, out_o, lse_o = o.decode_units(units, sel_o, cnt_o, cfg.topk, cfg.sm_scale)
    tol, lse_tol = tol_of(cfg)
    worst = 0.0
    for u, (r, j) in enumerate(units):
        print(f"[unit] {kind} request={r} step={j}", flush=True)
        topk, tcnt = dev.refine_topk(sel, cnt, j, cfg.topk)
        out, lse = dev.attend(topk, tcnt, j, cfg.topk)
        torch.cuda.synchronize()
        tc = tcnt.cpu().numpy()
        assert tc[r] == len(tk_o[u])
        assert np.array_equal(topk.cpu().numpy()[r, :tc[r]], tk_o[u])
        got = _runner().out_to_f32(out, cfg)[r]
        err = rel_err(got, out_o[u])
        worst = max(worst, float(err.max()))
        assert err.max() <= tol, (kind, r, j, float(err.max()))
        assert np.abs(lse.cpu().numpy()[r] - lse_o[u]).max() <= lse_tol * max(1.0, np.abs(lse_o[u]).max())
    print(f"[result] {kind} worst rel err {worst:.3e}", flush=True)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_full_selection_is_full_attention(kind):
    """theta = -inf and k >= |T|: every history token plus the recent window."""
    inp, dev, o = setup(kind)
    cfg = inp.cfg
    k = int(inp["n_hist"].max()) * 64 + 64
    z, sel, cnt = dev.score_select(theta=float("-inf"))
    _, sel_o, cnt_o = o.score_select(theta=float("-inf"))
    assert np.array_equal(cnt.cpu().numpy(), inp["n_hist"].astype(np.int32))
    topk, tcnt = dev.refine_topk(sel, cnt, 0, k)
    out, lse = dev.attend(topk, tcnt, 0, k)
    torch.cuda.synchronize()
    units = [(r, 0) for r in range(cfg.batch)]
    tk_o, out_o, lse_o = o.decode_units(units, sel_o, cnt_o, k, cfg.sm_scale)
    got = _runner().out_to_f32(out, cfg)
    tol, _ = tol_of(cfg)
    for r in range(cfg.batch):
        assert tcnt.cpu().numpy()[r] == inp["rs"][r]
        assert rel_err(got[r], out_o[r]).max() <= tol


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_no_selection_is_recent_window(kind):
    inp, dev, o = setup(kind)
    cfg = inp.cfg
    z, sel, cnt = dev.score_select(theta=float("inf"))
    assert int(cnt.sum()) == 0
    topk, tcnt = dev.refine_topk(sel, cnt, 1, cfg.topk)
    out, lse = dev.attend(topk, tcnt, 1, cfg.topk)
    torch.cuda.synchronize()
    assert int(tcnt.sum()) == 0
    _, sel_o, cnt_o = o.score_select(theta=float("inf"))
    units = [(r, 1) for r in range(cfg.batch)]
    _, out_o, _ = o.decode_units(units, sel_o, cnt_o, cfg.topk, cfg.sm_scale)
    got = _runner().out_to_f32(out, cfg)
    tol, _ = tol_of(cfg)
    for r in range(cfg.batch):
        assert rel_err(got[r], out_o[r]).max() <= tol


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_split_count_invariance_and_determinism(kind):
    inp, dev, o = setup(kind)
    cfg = inp.cfg
    z, sel, cnt = dev.score_select()
    topk, tcnt = dev.refine_topk(sel, cnt, 0, cfg.topk)
    outs = []
    for ns in (0, 1, 3, 0):
        out, lse = dev.attend(topk, tcnt, 0, cfg.topk, n_splits=ns)
        outs.append(_runner().out_to_f32(out, cfg))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[3])  # same launch twice: bitwise
    tol, _ = tol_of(cfg)
    for x in outs[1:3]:
        assert rel_err(x, outs[0]).max() <= tol


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_attention_output_at_unaligned_address(kind):
    """The output pointer carries no alignment promise: the same launch with
    the output one element past a 16-byte boundary gives the same values
    (the merge then stores element by element)."""
    inp, dev, o = setup(kind)
    cfg = inp.cfg
    lsa = _lsa()
    z, sel, cnt = dev.score_select()
    topk, tcnt = dev.refine_topk(sel, cnt, 0, cfg.topk)
    ref, _ = dev.attend(topk, tcnt, 0, cfg.topk)
    odt = torch.float32 if kind == "f32" else torch.int16
    n = dev.B * cfg.Hq * cfg.Dv
    buf = torch.zeros(n + 8, dtype=odt, device="cuda")
    out = buf[1:1 + n].view(dev.B, cfg.Hq, cfg.Dv)
    assert out.data_ptr() % 16 != 0
    lse = torch.empty((dev.B, cfg.Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(lsa.lsa_attn_ws_bytes(dev.geom, dev.kv, cfg.Hq, cfg.topk, 0), dtype=torch.uint8,
                     device="cuda")
    lsa.lsa_sparse_decode_attn(dev.geom, dev.q_attn[0], cfg.Hq, dev.kv, dev.pages, None, dev.recent, topk,
                               tcnt, cfg.topk, cfg.sm_scale, out, lse, 0, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), ref.cpu())
    assert torch.count_nonzero(buf[:1]) == 0 and torch.count_nonzero(buf[1 + n:]) == 0


def test_topk_k1_and_k_exceeding_candidates():
    inp, dev, o = setup("bf16")
    cfg = inp.cfg
    z, sel, cnt = dev.score_select()
    _, sel_o, cnt_o = o.score_select()
    for k in (1, 7, 100000):
        topk, tcnt = dev.refine_topk(sel, cnt, 1, k)
        torch.cuda.synchronize()
        for r in range(cfg.batch):
            a = int(inp["chunk_off"][r])
            want = o.refine_topk(r, sel_o[a:a + cnt_o[r]], inp["q_refine"][1, r],
                                 inp["w_refine"][1, r], k)
            got = topk.cpu().numpy()[r, :tcnt.cpu().numpy()[r]]
            assert np.array_equal(got, want), (k, r)


@pytest.mark.parametrize("host_cold,variant", [(False, "band"), (True, "band"), (True, "valu"),
                                               (True, "union3")])
def test_window_pipeline_matches_oracle(host_cold, variant):
    """lsa_step64 over three windows with drift: per-window outputs and
    per-fetch copy counts against the oracle and the pool simulation.  The
    "valu" variant (8 indexer heads, bf16 keys, signed head weights) takes the
    pipeline's vector-ALU refine instead of the matrix-core band; "union3"
    selects, at every trigger, the OR union over three indexer layers."""
    R = _runner()
    n_layers = 3 if variant == "union3" else 1
    if variant in ("band", "union3"):
        cfg = synth.small_config("pipe", 31, (12000, 7000), window=1024, idx=FP8, H=16, topk=256,
                                 steps=6, planted=0.10)
    else:
        cfg = synth.small_config("pipe_valu", 33, (12000, 7000), window=1024, idx=BF16, H=8, topk=256,
                                 steps=6, planted=0.10, signed_weights=True)
    cfg = synth.dataclasses.replace(cfg, windows=4, drift=0.10, host_cold=host_cold,
                                    slots_per_req=80)
    inp = synth.generate(cfg)
    dev = R.DeviceInputs(inp)
    pipe = R.Pipeline(dev, n_layers=n_layers)
    B, S = cfg.batch, 2  # two steps per window
    st0, cnt0 = pipe.prime()
    sels, fetched = [], [st0["fetched"]]
    windows = 3
    outs = torch.empty((windows, S, B, cfg.Hq, cfg.Dv), dtype=torch.int16, device="cuda")
    tks = torch.empty((windows, S, B, cfg.topk), dtype=torch.int32, device="cuda")
    tcs = torch.empty((windows, S, B), dtype=torch.int32, device="cuda")
    for m in range(windows):
        st, _ = pipe.window(m, m * S, S, outs[m], topk=tks[m], tcnt=tcs[m], last=(m == windows - 1))
        if m < windows - 1:
            fetched.append(st["fetched"])
    torch.cuda.synchronize()
    # oracle: per-window selection with that window's KIComp, then the steps
    per_req_sets = [[] for _ in range(B)]
    tol, _ = tol_of(cfg)
    for m in range(windows):
        o = oracle.Oracle(inp, kic=inp["kic_windows"][m], kic_scale=inp["kic_scale_windows"][m])
        if n_layers > 1:
            _, sel_o, cnt_o = o.score_select_union(synth.indexer_layers(inp, n_layers, window=m))
        else:
            _, sel_o, cnt_o = o.score_select()
        for r in range(B):
            a = int(inp["chunk_off"][r])
            per_req_sets[r].append(set(sel_o[a:a + cnt_o[r]].tolist()))
        units = [(r, m * S + j) for j in range(S) for r in range(B)]
        tk_o, out_o, _ = o.decode_units(units, sel_o, cnt_o, cfg.topk, cfg.sm_scale)
        got = R.out_to_f32(outs[m].reshape(S * B, cfg.Hq, cfg.Dv), cfg)
        tk = tks[m].cpu().numpy().reshape(S * B, -1)
        tc = tcs[m].cpu().numpy().reshape(-1)
        for u, (r, jj) in enumerate(units):
            assert np.array_equal(tk[u, :tc[u]], tk_o[u]), (m, r, jj)
            assert rel_err(got[u], out_o[u]).max() <= tol
    sim = [oracle.pool_sim(per_req_sets[r], pipe.spr) for r in range(B)]
    want = [sum(sim[r][m] for r in range(B)) for m in range(windows)]
    assert fetched == want
    pipe.close()


@pytest.mark.parametrize("workload,n_layers", [(4, 1), (2, 1), (4, 3)])
def test_window_pipeline_full_size_sampled(workload, n_layers):
    """lsa_step64 at full size, 64 steps per window as the bench times it,
    over two windows with 2 % drift: the 500K-token batch of 8 (fp8 index
    keys, pinned-host cold tier), also with every trigger selecting the OR
    union of three indexer layers (slots for a window's 2,200 or so chunks), and
    the ragged 32K-128K batch of 16 (bf16 index keys, HBM cold tier).
    Sampled (request, step) units against the oracle (top-k bit for bit,
    attention within tolerance) and every window's fetch count against the
    pool simulation."""
    R = _runner()
    cfg = synth.dataclasses.replace(synth.config(workload), windows=3, drift=0.02)
    if n_layers > 1:
        cfg = synth.dataclasses.replace(cfg, slots_per_req=3072)
    inp = synth.generate(cfg, steps=64, threads=16)
    dev = R.DeviceInputs(inp)
    pipe = R.Pipeline(dev, n_layers=n_layers)
    B, S, windows = cfg.batch, 64, 2
    print(f"[setup] {cfg.name}: n_hist={list(inp['n_hist'])} slots/request={pipe.spr}", flush=True)
    st0, _ = pipe.prime()
    fetched = [st0["fetched"]]
    outs = torch.empty((windows, S, B, cfg.Hq, cfg.Dv), dtype=torch.int16, device="cuda")
    tks = torch.empty((windows, S, B, cfg.topk), dtype=torch.int32, device="cuda")
    tcs = torch.empty((windows, S, B), dtype=torch.int32, device="cuda")
    for m in range(windows):
        print(f"[window] {m}", flush=True)
        st, _ = pipe.window(m, 0, S, outs[m], topk=tks[m], tcnt=tcs[m], last=(m == windows - 1))
        if m < windows - 1:
            fetched.append(st["fetched"])
    torch.cuda.synchronize()
    tol, _ = tol_of(cfg)
    per_req_sets = [[] for _ in range(B)]
    samples = [[(0, 0), (B // 2, 31), (B - 1, S - 1)], [(1, 63), (B - 2, 1)]]
    for m in range(windows):
        o = oracle.Oracle(inp, kic=inp["kic_windows"][m], kic_scale=inp["kic_scale_windows"][m])
        if n_layers > 1:
            _, sel_o, cnt_o = o.score_select_union(synth.indexer_layers(inp, n_layers, window=m))
        else:
            _, sel_o, cnt_o = o.score_select()
        for r in range(B):
            a = int(inp["chunk_off"][r])
            per_req_sets[r].append(set(sel_o[a:a + cnt_o[r]].tolist()))
        tk_o, out_o, _ = o.decode_units(samples[m], sel_o, cnt_o, cfg.topk, cfg.sm_scale)
        for u, (r, j) in enumerate(samples[m]):
            print(f"[unit] window={m} request={r} step={j}", flush=True)
            tc = int(tcs[m, j, r].item())
            assert tc == len(tk_o[u]), (m, r, j)
            assert np.array_equal(tks[m, j, r, :tc].cpu().numpy(), tk_o[u]), (m, r, j)
            got = R.out_to_f32(outs[m, j, r:r + 1], cfg)[0]
            err = float(rel_err(got, out_o[u]).max())
            assert err <= tol, (m, r, j, err)
    sim = [oracle.pool_sim(per_req_sets[r], pipe.spr) for r in range(B)]
    assert fetched == [sum(sim[r][m] for r in range(B)) for m in range(windows)]
    pipe.close()


def test_topk_all_ties_zero_query():
    """q = 0 makes every refine score +0: the k lowest candidate tokens."""
    inp, dev, o = setup("fp8")
    cfg = inp.cfg
    z, sel, cnt = dev.score_select()
    _, sel_o, cnt_o = o.score_select()
    saved = dev.q_refine.clone()
    dev.q_refine.zero_()
    try:
        topk, tcnt = dev.refine_topk(sel, cnt, 0, cfg.topk)
        torch.cuda.synchronize()
    finally:
        dev.q_refine.copy_(saved)
    for r in range(cfg.batch):
        a = int(inp["chunk_off"][r])
        toks = [c * 64 + t for c in sel_o[a:a + cnt_o[r]] for t in range(64)]
        want = toks[:cfg.topk]
        got = topk.cpu().numpy()[r, :tcnt.cpu().numpy()[r]]
        assert list(got) == want


@pytest.mark.parametrize("kind", ["f32", "bf16", "fp8", "cfg3", "bf16_sw", "fp8_sw", "cfg3_sw"])
def test_score_union_bitexact(kind):
    """OR-mode union over three indexer layers: the combined logits bitwise,
    the selected ids and counts exactly."""
    inp, dev, o = setup(kind)
    layers = synth.indexer_layers(inp, 3)
    z, sel, cnt = dev.score_select_union(layers)
    torch.cuda.synchronize()
    z_o, sel_o, cnt_o = o.score_select_union(layers)
    assert np.array_equal(z.cpu().numpy().view(np.uint32), z_o.view(np.uint32))
    c = cnt.cpu().numpy()
    assert np.array_equal(c, cnt_o)
    s = sel.cpu().numpy()
    for r in range(inp.cfg.batch):
        a = int(inp["chunk_off"][r])
        assert np.array_equal(s[a:a + c[r]], sel_o[a:a + c[r]])
    # one layer through the union entry point is the single-layer scoring
    z1, _, c1 = dev.score_select_union(layers[:1])
    z0, _, c0 = dev.score_select()
    torch.cuda.synchronize()
    assert np.array_equal(z1.cpu().numpy().view(np.uint32), z0.cpu().numpy().view(np.uint32))
    assert np.array_equal(c1.cpu().numpy(), c0.cpu().numpy())


def _sig_bound(inp, q, w, bias):
    """Per-chunk bound on |S' - S| that the matrix-core sigmoid score states
    (two ulps per operation, Cauchy-Schwarz, 1/4-Lipschitz sigmoid, 2^-14 per
    head for the two sigmoids), in float64 from the decoded inputs."""
    cfg = inp.cfg
    u2, d, H = 2.0 ** -22, cfg.d, cfg.H
    gam = lambda n: n * u2 / (1 - n * u2)
    qv = oracle.decode(cfg.q_dtype, q).astype(np.float64).reshape(cfg.batch, H, d)
    kic = inp["kic_windows"][0]
    kv = oracle.decode(cfg.idx_dtype, kic).astype(np.float64).reshape(-1, d)
    sc = inp["kic_scale_windows"][0].astype(np.float64) if cfg.idx_dtype == FP8 else np.ones(len(kv))
    E = np.zeros(len(kv))
    for r in range(cfg.batch):
        a, n = int(inp["chunk_off"][r]), int(inp["n_hist"][r])
        if n == 0:
            continue
        wa = np.abs(w[r].astype(np.float64))
        x = sc[a:a + n, None] * (kv[a:a + n] @ qv[r].T) + float(bias[r])
        da = np.abs(sc[a:a + n]) * 2 * gam(d) * np.linalg.norm(kv[a:a + n], axis=1) * \
            (wa * np.linalg.norm(qv[r], axis=1)).sum()
        dx = da + 4 * u2 * (np.abs(x) @ wa + da)
        E[a:a + n] = 0.25 * dx + wa.sum() * (2.0 ** -14 + 2 * gam(H + 24))
    return E * 1.01


def _check_sigmoid(inp, dev, o, q=None, w=None, bias=None, exact=False):
    q = inp["q_coarse"] if q is None else q
    w = inp["w_coarse"] if w is None else w
    bias = inp["bias"] if bias is None else bias
    S, sel, cnt = dev.score_select_sigmoid(q=q, w=w, bias=bias)
    torch.cuda.synchronize()
    S_o, sel_o, cnt_o = o.score_select_sigmoid(q=q, w=w, bias=bias)
    S = S.cpu().numpy()
    c = cnt.cpu().numpy()
    assert np.array_equal(c, cnt_o)
    s = sel.cpu().numpy()
    for r in range(inp.cfg.batch):
        a = int(inp["chunk_off"][r])
        assert np.array_equal(s[a:a + c[r]], sel_o[a:a + c[r]])
    if exact:
        assert np.array_equal(S.view(np.uint32), S_o.view(np.uint32))
        return S, S_o, 0
    E = _sig_bound(inp, q, w, bias)
    err = np.abs(S.astype(np.float64) - S_o)
    assert np.all(err <= E), (err.max(), E[np.argmax(err - E)])
    # an output this close to the threshold cannot be an unchecked S': it
    # is the canonical value
    w1 = np.abs(np.asarray(w, np.float64)).sum(axis=1).min()
    near = np.abs(S.astype(np.float64) - 0.5) <= w1 * 2.0 ** -14
    assert np.array_equal(S[near].view(np.uint32), S_o[near].view(np.uint32))
    return S, S_o, int(near.sum())


SIG_EXACT = ["f32", "bf16_qf32", "fp8_qf32", "f32_sw", "fp8_qf32_sw"]  # fp32 queries: one lane per chunk
SIG_MFMA = ["bf16", "fp8", "bf16_h128", "bf16_h8", "cfg1", "cfg3", "bf16_sw", "fp8_sw", "bf16_h8_sw",
            "cfg3_sw"]


@pytest.mark.parametrize("kind", SIG_EXACT)
def test_score_sigmoid_exact_path(kind):
    """Per-head sigmoid score, fp32 queries: S bitwise, the chunks above 0.5 exactly."""
    inp, dev, o = setup(kind)
    _check_sigmoid(inp, dev, o, exact=True)


@pytest.mark.parametrize("kind", SIG_MFMA)
def test_score_sigmoid_matrix_core(kind):
    """Matrix-core sigmoid score: the fetched set exactly, S within its bound,
    canonical where it sits near the threshold."""
    inp, dev, o = setup(kind)
    _check_sigmoid(inp, dev, o)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "bf16_h8"])
def test_score_sigmoid_near_threshold(kind):
    """Queries scaled by 2^-16 and zero bias: every S sits within about 1e-5
    of 0.5, inside the bound, so (nearly) every chunk takes the canonical
    re-score and the fetch decisions turn on the last bits."""
    inp, dev, o = setup(kind)
    q = inp["q_coarse"]
    qs = synth.to_bf16_bits((q.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** -16))
    bias = np.zeros_like(inp["bias"])
    S, S_o, near = _check_sigmoid(inp, dev, o, q=qs, bias=bias)
    assert near >= 0.9 * len(S)
    assert 0 < int((S_o > 0.5).sum()) < len(S)


# ------------------------------------------------- comparison policies
def _segments(inp):
    return [(int(inp["chunk_off"][r]), int(inp["n_hist"][r])) for r in range(inp.cfg.batch)]


@pytest.mark.parametrize("kind", ["bf16", "fp8", "cfg3"])
def test_select_ranked_bitexact(kind):
    """Smallest-key and largest-value selections against the oracle's sorts:
    uniform keys, keys with heavy ties, fp32 values with ties and signed
    zeros; shares 0, 10, 25, 50 and 100 %, and a count above N."""
    inp, dev, o = setup(kind)
    lsa = _lsa()
    rng = np.random.default_rng(7)
    uni = synth.policy_keys(inp)
    tied = (uni % 7).astype(np.uint32)
    vals = (rng.integers(-3, 40, len(uni)) / 7.0).astype(np.float32)
    vals[rng.random(len(uni)) < 0.1] = -0.0
    cases = [(uni, lsa.RANK_SMALLEST_U32, oracle.select_smallest),
             (tied, lsa.RANK_SMALLEST_U32, oracle.select_smallest),
             (vals, lsa.RANK_LARGEST_F32, oracle.select_largest)]
    for keys, rk, ref in cases:
        for pct in (0, 10, 25, 50, 100, 101):
            m = [oracle.policy_count(n, pct) + (5 if pct == 101 else 0) for _, n in _segments(inp)]
            sel, cnt = dev.select_ranked(keys, rk, m)
            torch.cuda.synchronize()
            s, c = sel.cpu().numpy(), cnt.cpu().numpy()
            for r, (a, n) in enumerate(_segments(inp)):
                want = ref(keys[a:a + n], min(m[r], n))
                assert c[r] == len(want), (rk, pct, r)
                assert np.array_equal(s[a:a + c[r]], want), (rk, pct, r)


# Scores come from bf16 rows and queries with fp32 accumulation over 576
# products: |dx| <= gamma(576) sum|q k| sm (u = 2^-23 covers a truncating
# accumulation), about 1.3e-3 for N(0, 1) data at sm = 1/24, so a chunk's
# exp and the log-sum-exp each move by that much; the fp32 sums over steps
# and heads add less than 3e-4.  5e-3 relative holds with room.
MASS_RTOL = 5e-3


@pytest.mark.parametrize("kind", ["bf16", "bf16_h128", "cfg3"])
def test_chunk_mass_parity(kind):
    """Attention mass per history chunk under the full softmax of every step
    of the inputs, against the oracle; mass + recent = steps * heads; and the
    top-share selection by the GPU's mass differs from the oracle's only
    among chunks tied with the boundary within the tolerance."""
    inp, dev, o = setup(kind)
    lsa = _lsa()
    cfg = inp.cfg
    mass, rec = dev.chunk_mass()
    torch.cuda.synchronize()
    mass, rec = mass.cpu().numpy().astype(np.float64), rec.cpu().numpy().astype(np.float64)
    units = inp["q_attn"].shape[0] * cfg.Hq
    for r, (a, n) in enumerate(_segments(inp)):
        assert abs(mass[a:a + n].sum() + rec[r] - units) <= 1e-3 * units
    reqs = [0] if kind.startswith("cfg") else range(cfg.batch)
    for r in reqs:
        a, n = _segments(inp)[r]
        mo, ro = o.chunk_mass(r, np.ascontiguousarray(inp["q_attn"][:, r]), cfg.sm_scale)
        np.testing.assert_allclose(mass[a:a + n], mo, rtol=MASS_RTOL, atol=1e-9 * units)
        assert abs(rec[r] - ro) <= MASS_RTOL * ro + 1e-9 * units
        for pct in (10, 25, 50):
            m = oracle.policy_count(n, pct)
            if m == 0 or m == n:
                continue
            mg = torch.from_numpy(np.zeros(max(dev.nh, 1), np.float32)).cuda()
            mg[a:a + n] = torch.from_numpy(mass[a:a + n].astype(np.float32)).cuda()
            ms = [0] * cfg.batch
            ms[r] = m
            sel, cnt = dev.select_ranked(mg, lsa.RANK_LARGEST_F32, ms)
            torch.cuda.synchronize()
            got = set(sel.cpu().numpy()[a:a + int(cnt.cpu().numpy()[r])].tolist())
            want = set(oracle.select_largest(mo, m).tolist())
            edge = np.sort(mo)[::-1][m - 1]
            for c in got ^ want:
                assert abs(mo[c] - edge) <= 2 * MASS_RTOL * edge, (pct, c, mo[c], edge)


# ------------------------------------------------- growing context
def _check_growing_pipeline(cfg, full, L0, nw, k, host_cold, spr, att_steps=(0, 1, 40, 63)):
    """Run nw windows of lsa_step64 with a growing context and check, per
    window, the selection counts, every step's top-k (bit-exact) and sampled
    steps' attention against the oracle on the packed state of that step,
    the fetch counts against the pool simulation, and the end state (lengths,
    committed pages and scales, recent rows) against the generated data.
    Window m's selection is the trigger over the history at window m's start
    (with the chunks window m - 1 committed), scored one window ahead."""
    from tests import helpers
    R = _runner()
    B = cfg.batch
    gp = R.GrowingPipeline(full, L0, nw, host_cold=host_cold, k=k, slots_per_req=spr)
    outs = torch.empty((nw, 64, B, cfg.Hq, cfg.Dv), dtype=torch.int16, device="cuda")
    lses = torch.empty((nw, 64, B, cfg.Hq), dtype=torch.float32, device="cuda")
    tks = torch.empty((nw, 64, B, k), dtype=torch.int32, device="cuda")
    tcs = torch.empty((nw, 64, B), dtype=torch.int32, device="cuda")
    st0, cnt0 = gp.prime()
    fetched, cnts, starts = [st0["fetched"]], [cnt0], []
    for m in range(nw):
        L, rs, rf = gp.state()
        starts.append((L.copy(), rs.copy(), rf.copy()))
        print(f"[pgrow] {cfg.name} window {m}: L={list(L)} rs={list(rs)} recent_first={list(rf)}", flush=True)
        st, cnt = gp.window(m, outs[m], lse=lses[m], topk=tks[m], tcnt=tcs[m], last=(m == nw - 1))
        if m < nw - 1:
            fetched.append(st["fetched"])
            cnts.append(cnt)
    torch.cuda.synchronize()
    tol, lse_tol = tol_of(cfg)
    sets = [[] for _ in range(B)]
    tk_all, tc_all = tks.cpu().numpy(), tcs.cpu().numpy()
    lse_all = lses.cpu().numpy()
    for m in range(nw):
        L_m, rs_m, _ = starts[m]
        got_att = {j: R.out_to_f32(outs[m, j], cfg) for j in att_steps}
        for r in range(B):
            snap = helpers.growing_snapshot(full, r, int(L_m[r]), int(rs_m[r]))
            _, sel_o, cnt_o = oracle.Oracle(snap).score_select()
            assert cnts[m][r] == cnt_o[0], (m, r)
            sel_r = np.ascontiguousarray(sel_o[:cnt_o[0]])
            sets[r].append(set(sel_r.tolist()))
            for j in range(64):
                t = 64 * m + j
                sj = helpers.growing_snapshot(full, r, int(L_m[r]) + j + 1, int(rs_m[r]))
                o = oracle.Oracle(sj)
                want = o.refine_topk(0, sel_r, sj["q_refine"][t, 0], sj["w_refine"][t, 0], k)
                assert tc_all[m, j, r] == len(want), (m, j, r)
                assert np.array_equal(tk_all[m, j, r, :len(want)], want), (m, j, r)
                if j in got_att:
                    ref, lse_ref = o.attend(0, want, sj["q_attn"][t, 0], cfg.sm_scale)
                    assert rel_err(got_att[j][r], ref).max() <= tol, (m, j, r)
                    assert np.abs(lse_all[m, j, r] - lse_ref).max() <= lse_tol * max(1.0, np.abs(lse_ref).max())
    sim = [oracle.pool_sim(sets[r], gp.spr) for r in range(B)]
    assert fetched == [sum(sim[r][m] for r in range(B)) for m in range(nw)]
    L, rs, rf = gp.state()
    assert np.array_equal(L, full["seq_len"]) and np.array_equal(rs, full["rs"])
    pages = gp.pages.cpu().numpy().reshape(B * gp.chunk_cap, -1)
    isc = gp.ikey_scale.cpu().numpy()
    rec = gp.recent.cpu().numpy().reshape(B * gp.recent_cap, -1)
    for r in range(B):
        c0, n, a = int(full["chunk_off"][r]), int(full["n_hist"][r]), r * gp.chunk_cap
        assert np.array_equal(pages[a:a + n], full["pages"][c0:c0 + n]), r
        assert np.array_equal(isc[a:a + n], full["ikey_scale"][c0:c0 + n]), r
        q0, nr, b = int(full["rec_off"][r]), int(full["n_rec"][r]), r * gp.recent_cap + int(rf[r])
        assert np.array_equal(rec[b:b + nr], full["recent"][q0:q0 + nr]), r
    gp.close()
    return starts


@pytest.mark.parametrize("idx,host_cold", [("bf16", True), ("fp8", True), ("fp8", False)])
def test_window_pipeline_growing_matches_oracle(idx, host_cold):
    """lsa_step64 with a growing context: three windows of 64 steps on
    ragged requests (two commit a chunk in every window, one only in the
    last), the pinned-host or HBM cold tier."""
    W, k, nw = 1024, 256, 3
    L0 = [5000, 3100, 900]
    dt = BF16 if idx == "bf16" else FP8
    cfg = synth.small_config("pgrow_" + idx, 41 if idx == "bf16" else 42, tuple(L + 64 * nw for L in L0),
                             window=W, idx=dt, H=16, topk=k, steps=64 * nw)
    full = synth.generate(cfg)
    _check_growing_pipeline(cfg, full, L0, nw, k, host_cold, spr=64)


def test_window_pipeline_growing_moves_recent_rows():
    """A growing context run long enough that the recent rows reach the end
    of their area and move back to its start (a short window: 128 tokens)."""
    W, k, nw = 128, 64, 7
    L0 = [2000, 1100, 100]
    cfg = synth.small_config("pgrow_move", 43, tuple(L + 64 * nw for L in L0), window=W, idx=FP8,
                             H=16, topk=k, steps=64 * nw)
    full = synth.generate(cfg)
    starts = _check_growing_pipeline(cfg, full, L0, nw, k, True, spr=32, att_steps=(0, 63))
    rf = np.array([s[2] for s in starts])  # recent_first at each window's start
    assert (np.diff(rf, axis=0) < 0).any(), rf  # some request's rows moved back


# ------------------------------------------------- growing context
@pytest.mark.parametrize("idx", ["bf16", "fp8"])
def test_growing_context_matches_oracle(idx):
    """Two windows of growing-context decode (one token appended per step,
    the oldest full recent chunk committed at each window's end) on ragged
    requests, one too short to commit: every trigger's selection and every
    step's top-k bit-exact against the oracle on the packed state of that
    step, attention within tolerance on sampled steps, and the end state
    (history pages, KIComp rows, recent rows) equal to the generated data."""
    from tests import helpers
    runner = _runner()
    W, k, nw = 1024, 256, 2
    L0 = [5000, 3100, 900]
    dt = BF16 if idx == "bf16" else FP8
    cfg = synth.small_config("grow_" + idx, 31 if idx == "bf16" else 32, tuple(L + 64 * nw for L in L0),
                             window=W, idx=dt, H=16, topk=k, steps=64 * nw)
    full = synth.generate(cfg)
    g = runner.Growing(full, L0, nw)
    tol, lse_tol = tol_of(cfg)
    t = 0
    for m in range(nw):
        L_trig, rs_m = g.L.copy(), g.rs.copy()
        print(f"[grow] {idx} window {m}: L={list(L_trig)} rs={list(rs_m)}", flush=True)
        sel, cnt = g.trigger()
        torch.cuda.synchronize()
        s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
        sel_ref = []
        for r in range(cfg.batch):
            snap = helpers.growing_snapshot(full, r, int(L_trig[r]), int(rs_m[r]))
            _, sel_o, cnt_o = oracle.Oracle(snap).score_select()
            a = r * g.chunk_cap
            assert c_h[r] == cnt_o[0], (m, r)
            assert np.array_equal(s_h[a:a + c_h[r]], sel_o[:cnt_o[0]]), (m, r)
            sel_ref.append(np.ascontiguousarray(sel_o[:cnt_o[0]]))
        for j in range(64):
            topk, tcnt, out, lse = g.step(k)
            torch.cuda.synchronize()
            tk, tc = topk.cpu().numpy(), tcnt.cpu().numpy()
            check_att = j in (0, 1, 40, 63)
            got = runner.out_to_f32(out, cfg) if check_att else None
            for r in range(cfg.batch):
                snap = helpers.growing_snapshot(full, r, int(L_trig[r]) + j + 1, int(rs_m[r]))
                o = oracle.Oracle(snap)
                want = o.refine_topk(0, sel_ref[r], snap["q_refine"][t, 0], snap["w_refine"][t, 0], k)
                assert tc[r] == len(want), (m, j, r)
                assert np.array_equal(tk[r, :tc[r]], want), (m, j, r)
                if check_att:
                    ref, lse_ref = o.attend(0, want, snap["q_attn"][t, 0], cfg.sm_scale)
                    assert rel_err(got[r], ref).max() <= tol, (m, j, r)
                    assert np.abs(lse.cpu().numpy()[r] - lse_ref).max() <= lse_tol * max(1.0, np.abs(lse_ref).max())
            t += 1
        g.commit(m)
    torch.cuda.synchronize()
    assert np.array_equal(g.L, full["seq_len"]) and np.array_equal(g.rs, full["rs"])
    pages = g.pages.cpu().numpy().reshape(cfg.batch * g.chunk_cap, -1)
    kic = g.kic.cpu().numpy().reshape(cfg.batch * g.chunk_cap, -1)
    rec = g.recent[g.cur].cpu().numpy().reshape(cfg.batch * g.recent_cap, -1)
    fk = full["kic_windows"][0].reshape(int(full["chunk_off"][-1]), -1).view(np.uint8)
    for r in range(cfg.batch):
        c0, n, a = int(full["chunk_off"][r]), int(full["n_hist"][r]), r * g.chunk_cap
        assert np.array_equal(pages[a:a + n], full["pages"][c0:c0 + n]), r
        assert np.array_equal(kic[a:a + n], fk[c0:c0 + n]), r
        q0, nr = int(full["rec_off"][r]), int(full["n_rec"][r])
        assert np.array_equal(rec[r * g.recent_cap:r * g.recent_cap + nr], full["recent"][q0:q0 + nr]), r
