"""The allocation-free decode entry point on the GPU: its output equals the workspace
entry point's on the same inputs, over two calls in a row (the second one smaller), both
of which use the library's per-GPU static array."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import io_aware_exact_attention_amd as mi

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, d, lens, seed, paged):
    cfg = ai.DecodeCfg("noalloc", B=B, Hq=Hq, Hkv=Hkv, d=d, seed=seed, paged=paged)
    lens = np.asarray(lens, np.int32)
    q = ai.decode_q(cfg)
    maxlen = int(lens.max())
    if paged:
        lay = ai.paged_layout(lens, 16, seed, extra_pages=3)
        kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
        vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
        table = torch.from_numpy(lay.block_table).cuda()
    else:
        kc = ai.build_contig_cache(cfg, ai.T_K, lens, maxlen)
        vc = ai.build_contig_cache(cfg, ai.T_V, lens, maxlen)
        table = None
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
        torch.bfloat16).cuda()
    return cfg, dev(q), dev(kc), dev(vc), table, torch.from_numpy(lens).cuda(), maxlen


def _both(cfg, q, kc, vc, table, seq, maxlen, splits):
    o1 = torch.empty_like(q)
    l1 = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    ws = mi.decode_workspace(cfg.B, cfg.Hq, cfg.d, maxlen, splits, q.device)
    mi.attn_fwd_decode(q, kc, vc, table, seq, o1, l1, maxlen, cfg.scale, splits, ws)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    mi.attn_fwd_decode_noalloc(q, kc, vc, table, seq, o2, l2, maxlen, cfg.scale, splits)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


@pytest.mark.parametrize("paged", [True, False])
def test_noalloc_decode_equals_workspace_decode_on_two_calls(paged):
    # first call: many chunks (fills much of the array); second: a smaller batch, shorter
    # sequences, a different split count, reusing the array the first call left behind
    big = _case(6, 32, 8, 128, [9000, 1, 4097, 0, 20000, 333], 950, paged)
    small = _case(2, 8, 2, 64, [300, 77], 951, paged)
    for (cfg, q, kc, vc, table, seq, maxlen), splits in ((big, 0), (small, 3)):
        print(f"noalloc decode B={cfg.B} Hq={cfg.Hq} d={cfg.d} paged={paged} splits={splits}",
              flush=True)
        o1, l1, o2, l2 = _both(cfg, q, kc, vc, table, seq, maxlen, splits)
        assert torch.equal(o1, o2), "outputs differ from the workspace entry point"
        assert torch.equal(l1, l2), "LSE differs from the workspace entry point"


def test_noalloc_decode_refuses_partials_beyond_the_array():
    cfg, q, kc, vc, table, seq, maxlen = _case(1, 4, 1, 64, [5], 952, True)
    need = mi.attn_decode_workspace_bytes(64, 64, 128, 1 << 17, 128)
    assert need > mi.ATTN_DECODE_NOALLOC_MAX_BYTES
    qb = torch.zeros(64, 64, 128, dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros(1, 8, 16, 128, dtype=torch.bfloat16, device="cuda")
    tb = torch.zeros(64, (1 << 17) // 16, dtype=torch.int32, device="cuda")
    sl = torch.ones(64, dtype=torch.int32, device="cuda")
    with pytest.raises(mi.AttnError):
        mi.attn_fwd_decode_noalloc(qb, kb, kb, tb, sl, torch.empty_like(qb), None, 1 << 17,
                                   0.1, 128)
