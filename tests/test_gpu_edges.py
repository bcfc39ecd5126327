"""GPU parity at the edges of the method and of the kernels, through the C-ABI.

  * the threshold at a logit of exactly +0 / -0 and at the smallest
    subnormals (strict "exceeds 0.5");
  * the matrix-core refine pass when one wave walks more than 128 chunks
    (its 64-chunk index window moves while chunks are in flight);
  * the exact top-k's radix fallbacks: many uncertain band entries in LDS,
    and a band too long for LDS;
  * the slot pool's capacity error (nothing changes) and the gathers after it;
  * a bounded wait that runs out is reported, not returned silently;
  * an empty attended set (no recent token, nothing selected).
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


def rel_err(got, ref):
    return (np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30))


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ------------------------------------------------------------- threshold at 0
@pytest.mark.parametrize("idx", ["f32", "bf16", "fp8"])
def test_threshold_at_zero_logit(idx):
    """Chunks whose KIComp row is zero have z = fma(s, +0, b): +0 for b = +0
    and for b = -0 (+0 + -0 = +0), never selected (strict); the smallest
    positive subnormal bias gives the smallest positive z, selected; its
    negative is not.  Logits bitwise and selections exactly as the oracle's,
    with subnormals kept on the GPU."""
    dt = {"f32": F32, "bf16": BF16, "fp8": FP8}[idx]
    kw = dict(idx=F32, kv=F32, H=4, d=64, Hq=8, Dk=128, Dv=128, separate_v=True) if dt == F32 else dict(idx=dt, H=16)
    cfg = synth.small_config("zero_" + idx, 51, (6000, 5000, 4000, 3000), window=1024, topk=128, steps=1,
                             signed_weights=True, **kw)
    inp = synth.generate(cfg)
    tiny = np.array([1], np.uint32).view(np.float32)[0]
    inp["bias"] = np.array([0.0, -0.0, tiny, -tiny], np.float32)
    kic = inp["kic_windows"][0]
    assert kic is inp["kic"]
    rows = []
    for r in range(cfg.batch):
        a, n = int(inp["chunk_off"][r]), int(inp["n_hist"][r])
        ev = a + np.arange(0, n, 2)
        kic[ev] = 0
        rows.append(np.arange(0, n, 2))
    dev = _runner().DeviceInputs(inp)
    z, sel, cnt = dev.score_select()
    torch.cuda.synchronize()
    z_o, sel_o, cnt_o = oracle.Oracle(inp).score_select()
    z_h, s_h, c_h = z.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(_bits(z_h), _bits(z_o))
    assert np.array_equal(c_h, cnt_o)
    want_bits = [0x00000000, 0x00000000, 0x00000001, 0x80000001]
    for r in range(cfg.batch):
        a = int(inp["chunk_off"][r])
        assert np.array_equal(s_h[a:a + c_h[r]], sel_o[a:a + c_h[r]]), r
        assert np.all(_bits(z_h[a + rows[r]]) == want_bits[r]), r
        chosen = set(s_h[a:a + c_h[r]].tolist())
        zero_rows = set(rows[r].tolist())
        if r == 2:
            assert zero_rows <= chosen
        else:
            assert not (zero_rows & chosen), r


# ------------------------------------------------ long walks of the refine pass
@pytest.mark.parametrize("idx,blocks", [("fp8", 1), ("bf16", 1), ("fp8", 5), ("bf16", 7)])
def test_refine_one_block_per_request(idx, blocks):
    """Few refine blocks per request (forced), so each wave walks dozens to
    more than 128 of the request's chunks and its 64-chunk index window moves
    while the next chunk's key rows are in flight; the chunks left over after
    the whole-chunk rounds are split into 16-token parts, a run of which can
    span two chunks.  Every chunk selected, signed head weights: the top-k
    bit for bit as the oracle's, and as the default launch shape's."""
    lsa = _lsa()
    dt = FP8 if idx == "fp8" else BF16
    cfg = synth.small_config("walk_" + idx, 52, (44000, 30000), window=1024, idx=dt, H=16, topk=512,
                             steps=2, signed_weights=True)
    inp = synth.generate(cfg)
    dev = _runner().DeviceInputs(inp)
    o = oracle.Oracle(inp)
    z, sel, cnt = dev.score_select(theta=float("-inf"))
    _, sel_o, cnt_o = o.score_select(theta=float("-inf"))
    assert int(cnt_o[0]) // 4 >= 128
    for j in range(2):
        lsa.lsa_tune_set(lsa.TUNE_REFINE_BLOCKS, blocks)
        try:
            topk1, tcnt1 = dev.refine_topk(sel, cnt, j, cfg.topk)
            torch.cuda.synchronize()
        finally:
            lsa.lsa_tune_set(lsa.TUNE_REFINE_BLOCKS, -1)
        topk0, tcnt0 = dev.refine_topk(sel, cnt, j, cfg.topk)
        torch.cuda.synchronize()
        for r in range(cfg.batch):
            a = int(inp["chunk_off"][r])
            want = o.refine_topk(r, sel_o[a:a + cnt_o[r]], inp["q_refine"][j, r], inp["w_refine"][j, r],
                                 cfg.topk)
            print(f"[walk] {idx} blocks={blocks} step={j} request={r} candidates={int(cnt_o[r]) * 64}",
                  flush=True)
            got1 = topk1.cpu().numpy()[r, :int(tcnt1[r])]
            got0 = topk0.cpu().numpy()[r, :int(tcnt0[r])]
            assert np.array_equal(got1, want), (j, r)
            assert np.array_equal(got0, want), (j, r)


# ----------------------------------------------------- radix paths of the top-k
def _all_ties(inp, dev, theta, k):
    """Zero refine queries make every score +0: the top-k is the k lowest
    candidate tokens.  Returns (got, want) per request."""
    _, sel_o, cnt_o = oracle.Oracle(inp).score_select(theta=theta)
    z, sel, cnt = dev.score_select(theta=theta)
    saved = dev.q_refine.clone()
    dev.q_refine.zero_()
    try:
        topk, tcnt = dev.refine_topk(sel, cnt, 0, k)
        torch.cuda.synchronize()
    finally:
        dev.q_refine.copy_(saved)
    out = []
    for r in range(inp.cfg.batch):
        a = int(inp["chunk_off"][r])
        toks = [int(c) * 64 + t for c in sel_o[a:a + cnt_o[r]] for t in range(64)]
        out.append((list(topk.cpu().numpy()[r, :int(tcnt[r])]), toks[:k], len(toks)))
    return out


@pytest.mark.parametrize("case", ["lds", "global"])
def test_topk_all_ties_radix_paths(case):
    """Every candidate selected and every score tied: all of them are in the
    band and uncertain, more than the direct ranking takes, so the exact
    top-k runs its radix select -- over the band in LDS (at most 8,192
    entries) or, for a longer band, over the lists in global memory."""
    if case == "lds":
        cfg = synth.small_config("ties_lds", 53, (9000, 6500), window=1024, idx=FP8, H=16, topk=512, steps=1,
                                 signed_weights=True)
    else:
        cfg = synth.small_config("ties_glob", 54, (12500, 9900), window=1024, idx=BF16, H=16, topk=700,
                                 steps=1, signed_weights=True)
    inp = synth.generate(cfg)
    dev = _runner().DeviceInputs(inp)
    for r, (got, want, m) in enumerate(_all_ties(inp, dev, float("-inf"), cfg.topk)):
        print(f"[ties] {case} request={r} band={m}", flush=True)
        assert (m <= 8192) == (case == "lds") and m > 1024
        assert got == want, r


def test_topk_all_ties_500k():
    """All scores tied at the 500K-token, batch-4 shape (about 50K candidates
    per request): the global-memory radix path at full size."""
    cfg = synth.config(3)
    inp = synth.generate(cfg, steps=1)
    dev = _runner().DeviceInputs(inp)
    for r, (got, want, m) in enumerate(_all_ties(inp, dev, 0.0, cfg.topk)):
        print(f"[ties] 500k request={r} band={m}", flush=True)
        assert m > 8192
        assert got == want, r


# ------------------------------------------------------------- pool capacity
@pytest.mark.parametrize("host_cold", [False, True])
def test_pool_capacity_error_leaves_pool_unchanged(host_cold):
    """A selection (with the kept set) larger than a request's slots returns
    LSA_ERR_CAPACITY before anything changes: the page table stays, and the
    next gathers fetch exactly what the pool simulation says, with every
    resident slot holding its chunk's cold page."""
    lsa = _lsa()
    cfg = synth.small_config("pool", 55, (9000, 6500), window=1024, idx=FP8, H=16, topk=128, steps=1)
    inp = synth.generate(cfg)
    dev = _runner().DeviceInputs(inp, host_cold=host_cold)
    B, pb, spr = cfg.batch, cfg.page_bytes, 12
    nh = dev.nh
    off = [int(x) for x in inp["chunk_off"]]
    slots = torch.zeros(B * spr * pb, dtype=torch.uint8, device="cuda")
    pool = lsa.Pool(dev.geom, slots, spr, pb, dev.pages, host_cold)
    pt = torch.full((nh,), -7, dtype=torch.int32, device="cuda")
    cs = torch.cuda.Stream()

    def ids(per_req):
        sel = np.full(nh, -1, np.int32)
        cnt = np.zeros(B, np.int32)
        for r, lst in enumerate(per_req):
            sel[off[r]:off[r] + len(lst)] = lst
            cnt[r] = len(lst)
        return sel, cnt

    def check_slots(per_req):
        torch.cuda.synchronize()
        p, sl = pt.cpu().numpy(), slots.cpu().numpy().reshape(B * spr, pb)
        for r, lst in enumerate(per_req):
            for c in range(int(inp["n_hist"][r])):
                if c in lst:
                    assert 0 <= p[off[r] + c] - r * spr < spr
                    assert np.array_equal(sl[p[off[r] + c]], inp["pages"][off[r] + c]), (r, c)
                else:
                    assert p[off[r] + c] == -1, (r, c)

    s_a = [list(range(10)), [5, 7]]
    sel_a, cnt_a = ids(s_a)
    st = pool.gather(sel_a, cnt_a, None, None, pt, cs)
    assert st["fetched"] == 12
    check_slots(s_a)
    before = pt.cpu().clone()
    # 13 chunks for request 1 alone
    sel_x, cnt_x = ids([[1], list(range(20, 33))])
    with pytest.raises(lsa.LsaError) as e:
        pool.gather(sel_x, cnt_x, None, None, pt, cs)
    assert e.value.code == -3
    # 5 new chunks next to the 10 kept ones of request 0
    sel_y, cnt_y = ids([list(range(20, 25)), [5, 7]])
    with pytest.raises(lsa.LsaError) as e:
        pool.gather(sel_y, cnt_y, sel_a, cnt_a, pt, cs)
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert torch.equal(pt.cpu(), before)
    # valid again: two new chunks for request 0 with its ten kept, and a new
    # selection for request 1 that replaces its old one
    s_b = [[20, 21], [6, 7, 8]]
    sel_b, cnt_b = ids(s_b)
    st = pool.gather(sel_b, cnt_b, sel_a, cnt_a, pt, cs)
    sims = [oracle.pool_sim([set(s_a[r]), set(s_b[r])], spr) for r in range(B)]
    assert st["fetched"] == sum(s[1] for s in sims)
    check_slots(s_b)
    # the selection in use before stays resident (kept), the rest is released
    assert st["resident"] == len(set(s_a[0]) | set(s_b[0])) + len(set(s_a[1]) | set(s_b[1]))
    pool.close()


# --------------------------------------------------------- bounded wait report
def test_attention_wait_expiry_is_reported():
    """The bf16 attention kernel that splits the dims over wave pairs (head
    counts that are multiples of 32 but not of 64) bounds each wait for the
    partner wave; with the bound forced to zero polls every wait runs out at
    once (the kernel still finishes), and lsa_device_status reports it
    (LSA_ERR_HIP, bit 0) and clears it.  With the default bound the same
    launch is clean and gives the reference output bit for bit."""
    lsa = _lsa()
    R = _runner()
    cfg = synth.small_config("expiry", 56, (9000, 4100), window=1024, idx=BF16, H=16, topk=256, steps=1,
                             Hq=32)
    inp = synth.generate(cfg)
    dev = R.DeviceInputs(inp)
    assert lsa.lsa_device_status() == (0, 0)
    z, sel, cnt = dev.score_select()
    topk, tcnt = dev.refine_topk(sel, cnt, 0, cfg.topk)
    ref, ref_lse = dev.attend(topk, tcnt, 0, cfg.topk)
    assert lsa.lsa_device_status() == (0, 0)
    lsa.lsa_tune_set(lsa.TUNE_ATTN_PAIR_POLLS, 0)
    try:
        dev.attend(topk, tcnt, 0, cfg.topk)
        code, flags = lsa.lsa_device_status()
    finally:
        lsa.lsa_tune_set(lsa.TUNE_ATTN_PAIR_POLLS, -1)
    assert code == -5 and flags & 1
    assert lsa.lsa_device_status() == (0, 0)
    out, lse = dev.attend(topk, tcnt, 0, cfg.topk)
    assert lsa.lsa_device_status() == (0, 0)
    assert torch.equal(out.cpu(), ref.cpu()) and torch.equal(lse.cpu(), ref_lse.cpu())


def test_window_pipeline_reports_wait_expiry():
    """lsa_step64 returns LSA_ERR_HIP from the call after a window that ran out
    of a bounded wait (that call's window still runs); the report covers that
    window only, and the windows after it are clean."""
    lsa = _lsa()
    R = _runner()
    cfg = synth.small_config("pipe_expiry", 57, (9000, 7000), window=1024, idx=FP8, H=16, topk=256, steps=2,
                             planted=0.10, Hq=96)
    cfg = synth.dataclasses.replace(cfg, windows=4, slots_per_req=80)
    inp = synth.generate(cfg)
    pipe = R.Pipeline(R.DeviceInputs(inp))
    B = cfg.batch
    out = torch.empty((2, B, cfg.Hq, cfg.Dv), dtype=torch.int16, device="cuda")
    pipe.prime()
    lsa.lsa_tune_set(lsa.TUNE_ATTN_PAIR_POLLS, 0)
    try:
        pipe.window(0, 0, 2, out)          # its waits run out
    finally:
        lsa.lsa_tune_set(lsa.TUNE_ATTN_PAIR_POLLS, -1)
    with pytest.raises(lsa.LsaError) as e:
        pipe.window(1, 0, 2, out)          # sees window 0's report
    assert e.value.code == -5
    # the pipeline took the word over at the end of window 0
    assert lsa.lsa_device_status() == (0, 0)
    pipe.window(2, 0, 2, out)              # clean again
    pipe.window(3, 0, 2, out, last=True)
    assert lsa.lsa_device_status() == (0, 0)
    pipe.close()


# --------------------------------------------------------- empty attended set
@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_empty_attended_set(kv):
    """A request whose recent region is empty (window 0, context a multiple of
    64) and whose selection is empty attends to nothing: its output is zero
    and its lse -inf, as the oracle defines it; the other request (56 recent
    tokens) is unaffected."""
    R = _runner()
    kw = dict(idx=F32, kv=F32, H=4, d=64, Hq=8, Dk=128, Dv=128, separate_v=True) if kv == "f32" else dict(idx=BF16, H=16)
    cfg = synth.small_config("empty_" + kv, 58, (4096, 3000), window=0, topk=64, steps=1, **kw)
    inp = synth.generate(cfg)
    assert list(inp["n_rec"]) == [0, 56]
    dev = R.DeviceInputs(inp)
    o = oracle.Oracle(inp)
    z, sel, cnt = dev.score_select(theta=float("inf"))
    topk, tcnt = dev.refine_topk(sel, cnt, 0, cfg.topk)
    out, lse = dev.attend(topk, tcnt, 0, cfg.topk)
    torch.cuda.synchronize()
    _, sel_o, cnt_o = o.score_select(theta=float("inf"))
    _, out_o, lse_o = o.decode_units([(0, 0), (1, 0)], sel_o, cnt_o, cfg.topk, cfg.sm_scale)
    got = R.out_to_f32(out, cfg)
    l = lse.cpu().numpy()
    assert np.all(out_o[0] == 0) and np.all(np.isneginf(lse_o[0]))
    assert np.all(got[0] == 0) and np.all(np.isneginf(l[0]))
    tol = 1e-5 if kv == "f32" else 2e-2
    assert rel_err(got[1], out_o[1]).max() <= tol
