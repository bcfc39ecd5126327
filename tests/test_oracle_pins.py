"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against brute force with exact rationals, a
textbook routine, a closed form or an invariant of the method, chosen so that
a dropped term, a wrong sign or index, or a transposed operand fails one of
them.  CPU only.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from learned_sparse_kv_amd import synth
from oracle import oracle
from tests import helpers

U = 2.0 ** -24  # unit roundoff of binary32


def gamma(n):
    return n * U / (1 - n * U)


# ---------------------------------------------------------------- PIN-1 decode
def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode(synth.FP8, codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan_codes = {0x7F, 0xFF}
    for c in range(256):
        if c in nan_codes:
            assert math.isnan(mine[c]), c
        else:
            assert mine[c] == ref[c] and np.signbit(mine[c]) == np.signbit(ref[c]), c
    # closed forms: largest normal, smallest subnormal, one
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x38] == 1.0


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode(synth.BF16, codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    same = (mine.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


# ---------------------------------------------------------------- geometry
@pytest.mark.parametrize("L,C,W,exp", [
    (16384, 64, 2048, (14336, 224, 2048)),
    (5000, 64, 1024, (3968, 62, 1032)),
    (512000, 64, 8192, (503808, 7872, 8192)),
    (100, 64, 1024, (0, 0, 100)),
    (1024 + 63, 64, 1024, (0, 0, 1087)),
    (1024 + 64, 64, 1024, (64, 1, 1024)),
])
def test_geometry_closed_form(L, C, W, exp):
    assert oracle.geometry(L, C, W) == exp


def test_generator_layout_agrees_with_oracle_geometry():
    inp = synth.generate(synth.small_config(seq_lens=(5000, 3000, 700)))
    for r, L in enumerate(inp["seq_len"]):
        rs, nh, nr = oracle.geometry(int(L), 64, 1024)
        assert (inp["rs"][r], inp["n_hist"][r], inp["n_rec"][r]) == (rs, nh, nr)


# ---------------------------------------------------------------- PIN-2/3 score, select
def _exact_logits(inp):
    cfg = inp.cfg
    q = oracle.decode(cfg.q_dtype, inp["q_coarse"]).reshape(cfg.batch, cfg.H, cfg.d)
    kic = oracle.decode(cfg.idx_dtype, inp["kic"]).reshape(-1, cfg.d)
    out, bound = [], []
    for r in range(cfg.batch):
        c0, c1 = inp["chunk_off"][r], inp["chunk_off"][r + 1]
        w = inp["w_coarse"][r]
        for c in range(c0, c1):
            s = Fraction(float(inp["kic_scale"][c])) if cfg.idx_dtype == synth.FP8 else 1
            acc = Fraction(0)
            mag = Fraction(0)
            for i in range(cfg.d):
                qb = sum(Fraction(float(w[h])) * Fraction(float(q[r, h, i])) for h in range(cfg.H))
                qa = sum(abs(Fraction(float(w[h])) * Fraction(float(q[r, h, i]))) for h in range(cfg.H))
                acc += qb * Fraction(float(kic[c, i]))
                mag += qa * abs(Fraction(float(kic[c, i])))
            b = Fraction(float(inp["bias"][r]))
            out.append(b + s * acc)
            bound.append(gamma(cfg.H + cfg.d + 2) * float(abs(s) * mag + abs(b)))
    return out, bound


@pytest.mark.parametrize("idx", [synth.F32, synth.FP8])
def test_score_brute_force_exact(idx):
    inp = helpers.tiny_inputs(idx_dtype=idx, d=7, H=4)
    o = oracle.Oracle(inp)
    z, sel, cnt = o.score_select()
    exact, bound = _exact_logits(inp)
    assert len(z) == len(exact) > 0
    for zi, ei, bi in zip(z, exact, bound):
        assert abs(float(zi) - float(ei)) <= bi + 1e-300, (zi, float(ei), bi)


def test_score_exact_by_construction_is_bitwise():
    """Small integers and power-of-two weights: every fp32 step is exact."""
    inp = helpers.tiny_inputs(d=6, H=4)
    rng = np.random.default_rng(3)
    cfg = inp.cfg
    inp["q_coarse"] = rng.integers(-8, 9, size=inp["q_coarse"].shape).astype(np.float32)
    inp["w_coarse"] = np.array([[0.5, 0.25, 2.0, 1.0]] * cfg.batch, np.float32)
    inp["kic"] = rng.integers(-8, 9, size=inp["kic"].shape).astype(np.float32)
    inp["bias"] = np.array([-3.0, 5.0], np.float32)
    z, _, _ = oracle.Oracle(inp).score_select()
    exact, _ = _exact_logits(inp)
    assert [float(v) for v in z] == [float(e) for e in exact]


def test_score_special_cases():
    inp = helpers.tiny_inputs(H=1, d=5)
    inp["w_coarse"][:] = 1.0
    z, _, _ = oracle.Oracle(inp).score_select()
    q = inp["q_coarse"].astype(np.float64)
    kic = inp["kic"].astype(np.float64)
    for r in range(2):
        for c in range(inp["chunk_off"][r], inp["chunk_off"][r + 1]):
            ref = float(np.float32(np.dot(q[r, 0], kic[c]) + inp["bias"][r]))
            assert abs(z[c] - ref) <= 4 * U * (np.abs(q[r, 0] * kic[c]).sum() + 1)
    inp["kic"][:] = 0.0
    z, _, _ = oracle.Oracle(inp).score_select()
    for r in range(2):
        assert (z[inp["chunk_off"][r]:inp["chunk_off"][r + 1]] == inp["bias"][r]).all()


def test_select_is_exactly_strict_threshold():
    inp = synth.generate(synth.small_config(seq_lens=(9000, 4000)))
    o = oracle.Oracle(inp)
    z, sel, cnt = o.score_select()
    for r in range(2):
        c0, c1 = inp["chunk_off"][r], inp["chunk_off"][r + 1]
        want = [c for c in range(c1 - c0) if z[c0 + c] > 0.0]
        assert list(sel[c0:c0 + cnt[r]]) == want
        # sigmoid(z) > 0.5 exactly when z > 0
        assert all((1 / (1 + math.exp(-float(z[c0 + c]))) > 0.5) == (z[c0 + c] > 0)
                   for c in range(c1 - c0) if abs(z[c0 + c]) > 1e-12)
    _, _, cnt_none = o.score_select(theta=float("inf"))
    _, sel_all, cnt_all = o.score_select(theta=float("-inf"))
    assert (cnt_none == 0).all()
    assert list(cnt_all) == list(inp["n_hist"])
    assert list(sel_all[:cnt_all[0]]) == list(range(cnt_all[0]))


def test_select_zero_logit_not_selected():
    inp = helpers.tiny_inputs()
    inp["kic"][:] = 0.0
    inp["bias"][:] = 0.0                 # z = +0 exactly
    z, sel, cnt = oracle.Oracle(inp).score_select()
    assert (z == 0).all() and (cnt == 0).all()
    inp["bias"][:] = np.float32(1e-45)   # smallest subnormal above 0
    _, _, cnt = oracle.Oracle(inp).score_select()
    assert list(cnt) == list(inp["n_hist"])


# ---------------------------------------------------------------- PIN-4/5 refine, top-k
def _exact_refine(inp, r, sel_r, q_r, w_r):
    cfg = inp.cfg
    C = cfg.chunk
    q = oracle.decode(cfg.q_dtype, q_r).reshape(cfg.H, cfg.d).astype(np.float64)
    c0 = inp["chunk_off"][r]
    res, bnd = [], []
    for c in sel_r:
        pg = inp["pages"][c0 + c]
        eb = synth.ELEM_BYTES[cfg.idx_dtype]
        raw = pg[cfg.ikey_off:]
        dt = {0: np.float32, 1: np.uint16, 2: np.uint8}[cfg.idx_dtype]
        keys = oracle.decode(cfg.idx_dtype, raw.view(dt)).reshape(C, cfg.d)
        s = Fraction(float(inp["ikey_scale"][c0 + c])) if cfg.idx_dtype == synth.FP8 else 1
        for t in range(C):
            I = Fraction(0)
            mag = 0.0
            for h in range(cfg.H):
                a = sum(Fraction(float(q[h, i])) * Fraction(float(keys[t, i])) for i in range(cfg.d))
                I += Fraction(float(w_r[h])) * max(a, Fraction(0))
                mag += abs(float(w_r[h])) * float(np.abs(q[h] * keys[t]).sum())
            res.append(s * I)
            bnd.append(gamma(cfg.H + cfg.d + 2) * float(abs(s)) * mag)
    return res, bnd


@pytest.mark.parametrize("idx", [synth.F32, synth.FP8])
def test_refine_brute_force_exact(idx):
    inp = helpers.tiny_inputs(idx_dtype=idx, H=3, d=5)
    o = oracle.Oracle(inp)
    _, sel, cnt = o.score_select(theta=float("-inf"))
    for r in range(2):
        c0 = inp["chunk_off"][r]
        sel_r = sel[c0:c0 + cnt[r]]
        q_r, w_r = inp["q_refine"][1, r], inp["w_refine"][1, r]
        topk, sc = o.refine_topk(r, sel_r, q_r, w_r, k=6, want_scores=True)
        exact, bnd = _exact_refine(inp, r, sel_r, q_r, w_r)
        assert len(sc) == len(exact) == 4 * len(sel_r)
        for a, e, b in zip(sc, exact, bnd):
            assert abs(float(a) - float(e)) <= b + 1e-300
        # top-k by the exact scores (no near-ties in this data)
        toks = [c * 4 + t for c in sel_r for t in range(4)]
        order = sorted(range(len(toks)), key=lambda i: (-exact[i], toks[i]))
        kth = sorted(exact, reverse=True)
        if len(kth) > 6:
            # either an exact tie at 0 (both sides hold +0 exactly, the lower
            # token wins) or a gap wider than the rounding bound
            assert (kth[5] == kth[6] == 0) or float(kth[5] - kth[6]) > 2 * max(bnd)
        want = sorted(toks[i] for i in order[:6])
        assert list(topk) == want


def test_refine_single_head_is_relu_dot():
    inp = helpers.tiny_inputs(H=1, d=5)
    o = oracle.Oracle(inp)
    _, sel, cnt = o.score_select(theta=float("-inf"))
    q_r = inp["q_refine"][0, 0]
    _, sc = o.refine_topk(0, sel[:cnt[0]], q_r, np.ones(1, np.float32), k=3, want_scores=True)
    for i, c in enumerate(np.repeat(sel[:cnt[0]], 4)):
        t = i % 4
        key = inp["pages"][c][inp.cfg.ikey_off:].view(np.float32).reshape(4, 5)[t]
        ref = max(float(np.dot(q_r[0].astype(np.float64), key.astype(np.float64))), 0.0)
        assert abs(sc[i] - ref) <= 8 * U * float(np.abs(q_r[0] * key).sum())


def test_topk_matches_textbook_sort_and_ties():
    inp = synth.generate(synth.small_config(seq_lens=(9000,), H=4, d=32, Hq=2, Dk=64, Dv=64))
    o = oracle.Oracle(inp)
    _, sel, cnt = o.score_select()
    sel_r = sel[:cnt[0]]
    toks = [c * 64 + t for c in sel_r for t in range(64)]
    q_r, w_r = inp["q_refine"][0, 0], inp["w_refine"][0, 0]
    for k in (1, 17, 256, len(toks) - 1, len(toks), len(toks) + 5):
        topk, sc = o.refine_topk(0, sel_r, q_r, w_r, k=k, want_scores=True)
        want = sorted(sorted(range(len(toks)), key=lambda i: (-sc[i], toks[i]))[:k])
        assert list(topk) == [toks[i] for i in want]
    # all scores equal (q = 0): the k lowest token indices
    zq = np.zeros_like(q_r)
    topk = o.refine_topk(0, sel_r, zq, w_r, k=100)
    assert list(topk) == toks[:100]
    # empty candidate set
    assert len(o.refine_topk(0, sel_r[:0], q_r, w_r, k=100)) == 0


# ---------------------------------------------------------------- PIN-6/7/8 attention
def _units_all(inp, theta, k):
    o = oracle.Oracle(inp)
    _, sel, cnt = o.score_select(theta=theta)
    units = [(r, j) for r in range(inp.cfg.batch) for j in range(inp.cfg.steps)]
    topk, out, lse = o.decode_units(units, sel, cnt, k, inp.cfg.sm_scale)
    return units, topk, out, lse


@pytest.mark.parametrize("kind", ["f32_sep", "bf16_latent"])
def test_full_selection_equals_dense_attention(kind):
    if kind == "f32_sep":
        inp = helpers.tiny_inputs()
    else:
        inp = synth.generate(synth.small_config(seq_lens=(700, 1500), window=256, H=2, d=16,
                                                Hq=4, steps=2))
    cfg = inp.cfg
    units, topk, out, lse = _units_all(inp, float("-inf"), k=10 ** 6)
    for u, (r, j) in enumerate(units):
        K, V = helpers.kv_rows(inp, r)
        q = oracle.decode(cfg.kv_dtype, inp["q_attn"][j, r]).reshape(cfg.Hq, cfg.Dk)
        o_ref, lse_ref = helpers.dense_attention(q.astype(np.float64), K, V, cfg.sm_scale)
        assert len(topk[u]) == inp["rs"][r]
        np.testing.assert_allclose(out[u], o_ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[u], lse_ref, rtol=1e-12)


def test_no_selection_equals_sliding_window_attention():
    inp = synth.generate(synth.small_config(seq_lens=(3000, 1100), window=512, H=2, d=16,
                                            Hq=4, steps=2))
    cfg = inp.cfg
    units, topk, out, lse = _units_all(inp, float("inf"), k=64)
    for u, (r, j) in enumerate(units):
        assert len(topk[u]) == 0
        K, V = helpers.kv_rows(inp, r)
        rs = inp["rs"][r]
        q = oracle.decode(cfg.kv_dtype, inp["q_attn"][j, r]).reshape(cfg.Hq, cfg.Dk)
        o_ref, lse_ref = helpers.dense_attention(q.astype(np.float64), K[rs:], V[rs:], cfg.sm_scale)
        np.testing.assert_allclose(out[u], o_ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[u], lse_ref, rtol=1e-12)


def test_attention_closed_forms():
    inp = helpers.tiny_inputs(seq_lens=(1, 23))
    cfg = inp.cfg
    o = oracle.Oracle(inp)
    # |A| = 1: output is that V row exactly, lse = sm * q . k
    q = inp["q_attn"][0, 0]
    out, lse = o.attend(0, [], q, cfg.sm_scale)
    K, V = helpers.kv_rows(inp, 0)
    assert (out == V[0][None, :]).all()
    np.testing.assert_allclose(lse, cfg.sm_scale * (q.astype(np.float64) @ K[0]), rtol=1e-14)
    # Q = 0: mean of the attended V rows, lse = ln |A|
    _, sel, cnt = o.score_select(theta=float("-inf"))
    c0 = inp["chunk_off"][1]
    topk = o.refine_topk(1, sel[c0:c0 + cnt[1]], inp["q_refine"][0, 1], inp["w_refine"][0, 1], 3)
    out, lse = o.attend(1, topk, np.zeros_like(inp["q_attn"][0, 1]), cfg.sm_scale)
    K, V = helpers.kv_rows(inp, 1)
    rs = inp["rs"][1]
    rows = list(topk) + list(range(rs, 23))
    np.testing.assert_allclose(out, np.broadcast_to(V[rows].mean(axis=0), out.shape), rtol=1e-12)
    np.testing.assert_allclose(lse, np.log(len(rows)), rtol=1e-14)


def test_attention_empty_set_is_empty_sum():
    """No recent token (window 0, context a multiple of the chunk) and an
    empty top-k: the attended set is empty, and the output is the value of an
    empty sum (0) with lse = ln 0 = -inf; one attended token in the other
    request still gives that token's V row exactly."""
    inp = helpers.tiny_inputs(seq_lens=(8, 9), window=0)
    cfg = inp.cfg
    assert list(inp["n_rec"]) == [0, 1]
    o = oracle.Oracle(inp)
    out, lse = o.attend(0, [], inp["q_attn"][0, 0], cfg.sm_scale)
    assert out.shape == (cfg.Hq, cfg.Dv) and np.all(out == 0) and np.all(np.isneginf(lse))
    _, sel, cnt = o.score_select(theta=float("inf"))
    _, outs, lses = o.decode_units([(0, 0), (1, 1)], sel, cnt, cfg.topk, cfg.sm_scale)
    assert np.all(outs[0] == 0) and np.all(np.isneginf(lses[0]))
    K, V = helpers.kv_rows(inp, 1)
    assert (outs[1] == V[8][None, :]).all()


# ---------------------------------------------------------------- PIN-10 pool
def test_pool_sim_closed_forms():
    s = [set(range(10)), set(range(10)), set(range(10))]
    assert oracle.pool_sim(s, 10) == [10, 0, 0]
    s = [set(range(0, 5)), set(range(5, 10)), set(range(10, 15))]
    assert oracle.pool_sim(s, 10) == [5, 5, 5]
    # a chunk dropped for one window and re-selected while still resident
    s = [{1, 2}, {2, 3}, {1, 3}]
    assert oracle.pool_sim(s, 4) == [2, 1, 0]
    s = [{1, 2}, {3, 4}, {5, 6}, {1, 2}]
    assert oracle.pool_sim(s, 4) == [2, 2, 2, 2]
    with pytest.raises(OverflowError):
        oracle.pool_sim([set(range(6)), set(range(3, 10))], 8)


# ---------------------------------------------------------------- PIN-11 determinism
def test_oracle_deterministic_across_threads():
    inp = synth.generate(synth.small_config(seq_lens=(6000, 2500), H=4, d=32, Hq=8, steps=2))
    o = oracle.Oracle(inp)
    _, sel, cnt = o.score_select()
    units = [(r, j) for r in range(2) for j in range(2)]
    a = o.decode_units(units, sel, cnt, 256, inp.cfg.sm_scale, threads=1)
    b = o.decode_units(units, sel, cnt, 256, inp.cfg.sm_scale, threads=4)
    for x, y in zip(a[0], b[0]):
        assert (x == y).all()
    assert (a[1] == b[1]).all() and (a[2] == b[2]).all()


# ---------------------------------------------------------------- generator recipe
def test_generator_selection_rate_cfg0():
    """cfg 0: 12 % planted, all planted chunks selected, ~2 % leakage."""
    inp = synth.generate(synth.config(0), steps=1)
    z, sel, cnt = oracle.Oracle(inp).score_select()
    n = int(inp["n_hist"][0])
    planted = set(inp["planted"][0][0].tolist())
    chosen = set(sel[:cnt[0]].tolist())
    assert planted <= chosen
    leak = len(chosen - planted) / (n - len(planted))
    assert 0.0 <= leak < 0.08
    assert 0.10 <= cnt[0] / n <= 0.20


# ------------------------------------------------ NEXT-1 OR-union over layers
def _single_layer(inp, lay, theta=0.0):
    o = oracle.Oracle(inp, kic=lay["kic"], kic_scale=lay["kic_scale"])
    return o.score_select(theta=theta, q=lay["q_coarse"], w=lay["w_coarse"], bias=lay["bias"])


@pytest.mark.parametrize("idx", [synth.F32, synth.BF16, synth.FP8])
def test_union_is_union_of_single_layers(idx):
    """The OR-mode union equals the set union of the three single-layer
    selections, and its logit is the per-chunk max of theirs, bitwise."""
    inp = synth.generate(synth.small_config(seq_lens=(9000, 4000), idx=idx, H=4, d=64))
    lays = synth.indexer_layers(inp, 3)
    zm, sel, cnt = oracle.Oracle(inp).score_select_union(lays)
    singles = [_single_layer(inp, lay) for lay in lays]
    assert np.array_equal(zm.view(np.uint32),
                          np.maximum.reduce([s[0] for s in singles]).view(np.uint32))
    for r in range(inp.cfg.batch):
        c0 = inp["chunk_off"][r]
        want = sorted(set().union(*[set(s[1][c0:c0 + s[2][r]].tolist()) for s in singles]))
        assert sel[c0:c0 + cnt[r]].tolist() == want
        # the union is strictly larger than every single layer here
        assert all(cnt[r] > s[2][r] for s in singles)


def test_union_special_cases():
    inp = synth.generate(synth.small_config(seq_lens=(9000, 4000), H=4, d=64))
    lays = synth.indexer_layers(inp, 3)
    o = oracle.Oracle(inp)
    z0, sel0, cnt0 = _single_layer(inp, lays[0])
    # one layer, and three copies of it: the single-layer selection, bitwise
    for group in ([lays[0]], [lays[0]] * 3):
        zm, sel, cnt = o.score_select_union(group)
        assert np.array_equal(zm.view(np.uint32), z0.view(np.uint32))
        assert np.array_equal(cnt, cnt0)
        assert all(np.array_equal(sel[c:c + n], sel0[c:c + n]) for c, n in zip(inp["chunk_off"], cnt0))
    # a layer that never fires changes nothing
    dead = dict(lays[2], bias=np.full_like(lays[2]["bias"], -1e30))
    _, sel_a, cnt_a = o.score_select_union(lays[:2])
    _, sel_b, cnt_b = o.score_select_union(lays[:2] + [dead])
    assert np.array_equal(cnt_a, cnt_b)
    assert all(np.array_equal(sel_a[c:c + n], sel_b[c:c + n]) for c, n in zip(inp["chunk_off"], cnt_a))
    # thresholds at the ends
    _, _, cnt_none = o.score_select_union(lays, theta=float("inf"))
    _, _, cnt_all = o.score_select_union(lays, theta=float("-inf"))
    assert (cnt_none == 0).all() and list(cnt_all) == list(inp["n_hist"])


# ------------------------------------------------- NEXT-2 per-head sigmoid score
def test_sigmoid_against_double_and_closed_forms():
    """The oracle's written-out fp32 sigmoid against the double-precision
    1/(1+exp(-x)): within a few ulp plus the conditioning of forming
    t = x log2(e) in fp32 (its rounding, |t| 2^-24, becomes a relative error
    of ln 2 |t| 2^-24 in e^-x), up to |x| = 88; exact at 0; 1 beyond 17 and 0
    below -89."""
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.uniform(-20, 20, 20000), rng.uniform(-88, 88, 5000),
                         [0.25, 0.5, 1.0, -1.0, 3.0, -7.5]]).astype(np.float32)
    for x in xs:
        s = oracle.sigmoid(float(x))
        ref = 1.0 / (1.0 + math.exp(-float(x)))
        tol = 3e-7 + abs(float(x)) * 1.4427 * 2 ** -23
        assert abs(s - ref) <= tol * ref, (float(x), s, ref)
    assert oracle.sigmoid(0.0) == 0.5 and oracle.sigmoid(-0.0) == 0.5
    assert oracle.sigmoid(17.0) == 1.0 and oracle.sigmoid(1e30) == 1.0
    assert oracle.sigmoid(-89.0) == 0.0 and oracle.sigmoid(-1e30) == 0.0
    # symmetry sigma(x) + sigma(-x) = 1 to a few ulp
    for x in rng.uniform(-15, 15, 2000).astype(np.float32):
        assert abs(oracle.sigmoid(float(x)) + oracle.sigmoid(-float(x)) - 1.0) <= 3e-7


def _exact_sigmoid_scores(inp):
    """S_c with exact rational dot products and a double sigmoid, and a bound
    on the fp32 result's distance from it."""
    cfg = inp.cfg
    q = oracle.decode(cfg.q_dtype, inp["q_coarse"]).reshape(cfg.batch, cfg.H, cfg.d)
    kic = oracle.decode(cfg.idx_dtype, inp["kic"]).reshape(-1, cfg.d)
    out, bound = [], []
    for r in range(cfg.batch):
        b = float(inp["bias"][r])
        for c in range(inp["chunk_off"][r], inp["chunk_off"][r + 1]):
            s = float(inp["kic_scale"][c]) if cfg.idx_dtype == synth.FP8 else 1.0
            tot, err = 0.0, 0.0
            for h in range(cfg.H):
                a = sum(Fraction(float(q[r, h, i])) * Fraction(float(kic[c, i])) for i in range(cfg.d))
                mag = sum(abs(float(q[r, h, i]) * float(kic[c, i])) for i in range(cfg.d))
                x = float(s * a + Fraction(b))
                sig = 1.0 / (1.0 + math.exp(-x))
                w = float(inp["w_coarse"][r, h])
                tot += w * sig
                dx = gamma(cfg.d + 2) * (abs(s) * mag + abs(b))
                err += abs(w) * (dx / 4 + 4e-7 * sig + 1e-38)
            out.append(tot)
            bound.append(err + gamma(cfg.H + 1) * tot + 1e-38)
    return out, bound


@pytest.mark.parametrize("idx", [synth.F32, synth.FP8])
def test_sigmoid_score_brute_force(idx):
    inp = helpers.tiny_inputs(idx_dtype=idx, d=7, H=4)
    rng = np.random.default_rng(9)
    inp["w_coarse"] = rng.uniform(0.05, 0.5, size=inp["w_coarse"].shape).astype(np.float32)
    inp["bias"] = np.array([0.3, -0.7], np.float32)
    S, sel, cnt = oracle.Oracle(inp).score_select_sigmoid()
    exact, bound = _exact_sigmoid_scores(inp)
    assert len(S) == len(exact) > 0
    for si, ei, bi in zip(S, exact, bound):
        assert abs(float(si) - ei) <= bi, (si, ei, bi)
    for r in range(inp.cfg.batch):
        c0 = inp["chunk_off"][r]
        n = inp["chunk_off"][r + 1] - c0
        assert sel[c0:c0 + cnt[r]].tolist() == [c for c in range(n) if S[c0 + c] > 0.5]


def test_sigmoid_score_special_cases():
    inp = helpers.tiny_inputs(H=4, d=5)
    inp["w_coarse"][:] = 0.25
    inp["kic"][:] = 0.0
    for b, want_sel in [(0.0, False), (1e-3, True), (-1e-3, False)]:
        inp["bias"][:] = b
        S, sel, cnt = oracle.Oracle(inp).score_select_sigmoid()
        # every head sees x = b: S = 4 * 0.25 * sigmoid(b) = sigmoid(b), exactly
        assert (S == np.float32(oracle.sigmoid(b))).all()
        assert list(cnt) == (list(inp["n_hist"]) if want_sel else [0] * inp.cfg.batch)
    # a chunk aligned with every head's query is selected, its negation is not
    inp = helpers.tiny_inputs(H=2, d=4)
    inp["w_coarse"][:] = 0.5
    inp["bias"][:] = 0.0
    inp["q_coarse"][:] = 1.0
    inp["kic"][:] = 0.5
    inp["kic"][1::2] = -0.5
    S, sel, cnt = oracle.Oracle(inp).score_select_sigmoid()
    assert (S[0::2] > 0.5).all() and (S[1::2] < 0.5).all()


# ------------------------------------------- NEXT-3 comparison policies
def _q_steps(inp, r):
    return np.ascontiguousarray(inp["q_attn"][:, r])


@pytest.mark.parametrize("kind", ["f32_sep", "bf16_latent"])
def test_chunk_mass_brute_force(kind):
    """Per-chunk attention mass against a dense fp64 softmax over every token
    (numpy matrix product, then per-chunk sums of the probabilities)."""
    if kind == "f32_sep":
        inp = helpers.tiny_inputs()
    else:
        inp = synth.generate(synth.small_config(seq_lens=(700, 1500), window=256, H=2, d=16,
                                                Hq=4, steps=2))
    cfg = inp.cfg
    o = oracle.Oracle(inp)
    for r in range(cfg.batch):
        K, _ = helpers.kv_rows(inp, r)
        q = oracle.decode(cfg.kv_dtype, _q_steps(inp, r)).astype(np.float64).reshape(-1, cfg.Dk)
        x = cfg.sm_scale * (q @ K.T)                        # [steps*Hq, L]
        p = np.exp(x - x.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        rs, n = int(inp["rs"][r]), int(inp["n_hist"][r])
        want = p[:, :rs].sum(axis=0).reshape(n, cfg.chunk).sum(axis=1)
        mass, rec = o.chunk_mass(r, _q_steps(inp, r), cfg.sm_scale)
        np.testing.assert_allclose(mass, want, rtol=1e-11, atol=1e-15)
        assert math.isclose(rec, p[:, rs:].sum(), rel_tol=1e-11)


def test_chunk_mass_total_and_closed_forms():
    inp = helpers.tiny_inputs(seq_lens=(40, 23, 64))
    cfg = inp.cfg
    o = oracle.Oracle(inp)
    for r in range(cfg.batch):
        q = _q_steps(inp, r)
        L, rs = int(inp["seq_len"][r]), int(inp["rs"][r])
        units = q.shape[0] * cfg.Hq
        mass, rec = o.chunk_mass(r, q, cfg.sm_scale)
        # every softmax sums to one
        assert math.isclose(mass.sum() + rec, units, rel_tol=1e-13)
        # Q = 0: every token gets 1/L of each unit
        mass0, rec0 = o.chunk_mass(r, np.zeros_like(q), cfg.sm_scale)
        np.testing.assert_allclose(mass0, units * cfg.chunk / L, rtol=1e-13)
        assert math.isclose(rec0, units * (L - rs) / L, rel_tol=1e-13)
    # one token whose key lies along every query: its chunk takes all the mass
    inp = helpers.tiny_inputs(seq_lens=(40, 23))
    cfg = inp.cfg
    r, tok = 0, 13                                   # chunk 3, a history token
    q = np.zeros_like(_q_steps(inp, r))
    q[..., 0] = 1.0
    pages = inp["pages"].view(np.float32).reshape(inp["pages"].shape[0], -1)
    rw = cfg.kv_row_bytes // 4                       # a page starts with its C KV rows
    pages[tok // cfg.chunk, (tok % cfg.chunk) * rw] = 1e4
    mass, rec = oracle.Oracle(inp).chunk_mass(r, q, cfg.sm_scale)
    units = q.shape[0] * cfg.Hq
    assert mass[tok // cfg.chunk] > units * (1 - 1e-12) and mass.argmax() == tok // cfg.chunk


def test_chunk_mass_deterministic_across_threads():
    inp = synth.generate(synth.small_config(seq_lens=(900,), window=256, H=2, d=16, Hq=4,
                                            steps=2))
    o = oracle.Oracle(inp)
    a = o.chunk_mass(0, _q_steps(inp, 0), inp.cfg.sm_scale, threads=1)
    b = o.chunk_mass(0, _q_steps(inp, 0), inp.cfg.sm_scale, threads=4)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1]


def test_policy_selections_textbook():
    rng = np.random.default_rng(3)
    for n in (0, 1, 7, 100, 1000):
        keys = rng.integers(0, 50, n).astype(np.uint32)   # many ties
        mass = rng.integers(0, 50, n).astype(np.float32) / 7
        for pct in (10, 25, 50, 100):
            m = oracle.policy_count(n, pct)
            assert m == -(-n * pct // 100) and m >= n * pct / 100 > m - 1 or n == 0
            want_s = sorted(sorted(range(n), key=lambda c: (int(keys[c]), c))[:m])
            want_l = sorted(sorted(range(n), key=lambda c: (-float(mass[c]), c))[:m])
            assert oracle.select_smallest(keys, m).tolist() == want_s
            assert oracle.select_largest(mass, m).tolist() == want_l
    # all equal: the lowest indices; zero and all
    assert oracle.select_smallest(np.zeros(9, np.uint32), 4).tolist() == [0, 1, 2, 3]
    assert oracle.select_largest(np.ones(9, np.float32), 4).tolist() == [0, 1, 2, 3]
    assert oracle.select_largest(np.arange(5.0), 0).tolist() == []
    assert oracle.select_largest(np.arange(5.0), 5).tolist() == [0, 1, 2, 3, 4]
    # recall: everything is 1, nothing is 0, the top half of a ramp is 3/4
    mass = np.arange(1, 9, dtype=np.float64)
    assert oracle.mass_recall(mass, range(8)) == 1.0 and oracle.mass_recall(mass, []) == 0.0
    assert math.isclose(oracle.mass_recall(mass, oracle.select_largest(mass, 4)), 26 / 36)


# ------------------------------------------------- NEXT-4 growing context
def test_growing_snapshot_at_the_final_state_is_the_generated_request():
    """The test-side snapshot of a growing run, taken at a request's final
    context and boundary, holds exactly the generator's packed data of that
    request; at an earlier state its rows are the same tokens' rows."""
    cfg = synth.small_config("grow", 31, (2200, 1500), window=512, H=4, d=64, steps=2)
    full = synth.generate(cfg)
    o_full = oracle.Oracle(full)
    z_full, _, cnt_full = o_full.score_select()
    for r in range(cfg.batch):
        L, rs = int(full["seq_len"][r]), int(full["rs"][r])
        snap = helpers.growing_snapshot(full, r, L, rs)
        c0, n = int(full["chunk_off"][r]), int(full["n_hist"][r])
        assert np.array_equal(snap["pages"], full["pages"][c0:c0 + n])
        q0 = int(full["rec_off"][r])
        assert np.array_equal(snap["recent"], full["recent"][q0:q0 + L - rs])
        z, _, cnt = oracle.Oracle(snap).score_select()
        assert np.array_equal(z.view(np.uint32), z_full[c0:c0 + n].view(np.uint32)) and cnt[0] == cnt_full[r]
        # 100 tokens earlier, two chunks fewer in the history: same rows, moved
        early = helpers.growing_snapshot(full, r, L - 100, rs - 128)
        K_e, _ = helpers.kv_rows(early, 0)
        K_f, _ = helpers.kv_rows(full, r)
        assert np.array_equal(K_e, K_f[:L - 100])
