"""The allocation-free attention entry point (lsa_sparse_decode_attn_noalloc)
against the workspace entry point (lsa_sparse_decode_attn), through the C-ABI:
the same outputs bit for bit on two calls in a row, the second smaller, and
a clear error (nothing enqueued) when the partials exceed its scratch."""
import numpy as np
import pytest
import torch

from learned_sparse_kv_amd import synth

pytestmark = pytest.mark.gpu


def _both(cfg):
    from learned_sparse_kv_amd import lsa, runner
    inp = synth.generate(cfg)
    dev = runner.DeviceInputs(inp)
    z, sel, cnt = dev.score_select()
    topk, tcnt = dev.refine_topk(sel, cnt, 0, cfg.topk)
    ref, ref_lse = dev.attend(topk, tcnt, 0, cfg.topk)
    odt = torch.float32 if cfg.kv_dtype == synth.F32 else torch.int16
    out = torch.full((dev.B, cfg.Hq, cfg.Dv), 7, dtype=odt, device="cuda")
    lse = torch.full((dev.B, cfg.Hq), 7.0, dtype=torch.float32, device="cuda")
    lsa.lsa_sparse_decode_attn_noalloc(dev.geom, dev.q_attn[0], cfg.Hq, dev.kv, dev.pages, None, dev.recent,
                                       topk, tcnt, cfg.topk, cfg.sm_scale, out, lse, 0)
    torch.cuda.synchronize()
    return ref.cpu(), ref_lse.cpu(), out.cpu(), lse.cpu()


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_noalloc_attention_matches_workspace_entry_point(kv):
    if kv == "bf16":
        big = synth.small_config("na_big", 61, (9000, 4100, 300), window=1024, H=16, topk=256, steps=1)
        small = synth.small_config("na_small", 62, (3000,), window=512, H=16, topk=64, steps=1)
    else:
        kw = dict(idx=synth.F32, kv=synth.F32, H=4, d=64, Hq=8, Dk=128, Dv=128, separate_v=True)
        big = synth.small_config("na_big32", 63, (5000, 2100, 700), window=1024, topk=256, steps=1, **kw)
        small = synth.small_config("na_small32", 64, (1500,), window=256, topk=32, steps=1, **kw)
    for cfg in (big, small):
        ref, ref_lse, out, lse = _both(cfg)
        print(f"[noalloc] {cfg.name} batch={cfg.batch}", flush=True)
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), cfg.name


def test_noalloc_attention_rejects_oversize():
    """64 requests of 500K tokens need about 42 MB of partials, more than the
    32 MiB scratch: LSA_ERR_WORKSPACE before anything is enqueued."""
    from learned_sparse_kv_amd import lsa
    B, L, k, Hq = 64, 512000, 2048, 64
    g = lsa.Geom(np.full(B, L, np.int32), 8192)
    kv = lsa.kv_layout(synth.BF16, 576, 512, 0, 1152, 64 * 1152 + 64 * 128, 64 * 1152)
    assert lsa.lsa_attn_ws_bytes(g, kv, Hq, k, 0) > lsa.lsa_attn_noalloc_max_bytes()
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(lsa.LsaError) as e:
        lsa.lsa_sparse_decode_attn_noalloc(g, dummy, Hq, kv, dummy, None, dummy, dummy, dummy, k, 0.04,
                                           dummy, None, 0)
    assert e.value.code == -4
