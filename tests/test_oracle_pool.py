"""The oracle's process pool (CPU): whole-output comparison and the timed legs."""
import numpy as np

import attn_inputs as ai
from oracle import attention_decode, attention_prefill
from oracle import pool


def oracle_as_gpu_output(cfg):
    q, k, v = ai.prefill_inputs(cfg)
    ro, rl = attention_prefill(ai.bf16_bits_to_f64(q), ai.bf16_bits_to_f64(k),
                               ai.bf16_bits_to_f64(v), cfg.scale, cfg.causal)
    return ai.to_bf16_bits(ro.astype(np.float32)), rl.astype(np.float32), ro, rl


def test_whole_output_check_matches_a_direct_comparison():
    cfg = ai.CONFIGS["tiny_prefill"]
    o_bits, lse, ro, rl = oracle_as_gpu_output(cfg)
    r = pool.check_prefill_heads("tiny_prefill", o_bits, lse)
    err = np.abs(ai.bf16_bits_to_f64(o_bits) - ro)
    assert r["n"] == err.size
    assert r["max_abs"] == err.max()
    assert np.isclose(r["mean_abs"], err.mean(), rtol=1e-12)
    assert r["lse_max_abs"] == np.abs(lse.astype(np.float64) - rl).max()
    assert r["finite"]
    # bf16 rounding of the output only
    assert r["max_abs"] <= 2.0 ** -8 * np.abs(ro).max()


def test_whole_output_check_finds_a_planted_error():
    # one wrong element (a causal row past the first 1,024-row block would need a bigger
    # config; the tiny one has 512 rows) and one non-finite element elsewhere
    cfg = ai.CONFIGS["tiny_prefill"]
    o_bits, lse, _, _ = oracle_as_gpu_output(cfg)
    bad = o_bits.copy()
    x = ai.bf16_bits_to_f32(bad[0, 2, 300, 17:18])[0]
    bad[0, 2, 300, 17] = ai.to_bf16_bits(np.array([x + 0.5], np.float32))[0]
    r = pool.check_prefill_heads("tiny_prefill", bad, lse)
    assert r["max_at"] == (0, 2, 300, 17) and r["max_abs"] > 0.49
    bad[0, 3, 10, 5] = np.uint16(0x7FC0)
    assert not pool.check_prefill_heads("tiny_prefill", bad, lse, heads=[(0, 3)])["finite"]


def test_causal_block_against_its_visible_keys_equals_the_full_rows():
    # the pool evaluates rows [i0, i1) of a causal head against keys [0, i1 + Nk - Nq)
    # only; that is the definition because every later key is masked for those rows
    from oracle import attention_rows
    q, k, v = ai.custom_prefill(seed=77, B=1, Hq=1, Hkv=1, Nq=300, Nk=700, d=64)
    Q, K, V = (ai.bf16_bits_to_f64(x[0, 0]) for x in (q, k, v))
    rows = np.arange(100, 200)
    full = attention_rows(Q[rows], K, V, 0.125, True, rows, 300)
    part = attention_rows(Q[rows], K[:200 + 400], V[:200 + 400], 0.125, True, rows, 200)
    # (equal up to summation order: the masked keys add exact zeros)
    assert np.abs(full[0] - part[0]).max() <= 1e-13
    assert np.abs(full[1] - part[1]).max() <= 1e-13


def test_timed_legs_run():
    cfg = ai.CONFIGS["tiny_prefill"]
    q, k, v = ai.prefill_inputs(cfg)
    r = pool.time_prefill(q, k, v, cfg.scale, True, [(0, h) for h in range(cfg.Hq)])
    assert r["units"] == cfg.Hq and r["seconds"] > 0 and 1 <= r["workers"] <= 16
    dc = ai.DecodeCfg("pool", B=2, Hq=8, Hkv=2, d=64, seed=3, paged=True, len_range=(1, 300))
    lens = ai.decode_lengths(dc)
    lay = ai.paged_layout(lens, 16, dc.seed)
    kp = ai.build_paged_cache(dc, ai.T_K, lens, lay, pad_bits=np.uint16(0))
    vp = ai.build_paged_cache(dc, ai.T_V, lens, lay, pad_bits=np.uint16(0))
    r = pool.time_decode(ai.decode_q(dc), kp, vp, lay.block_table, lens, dc.scale,
                         [(b, h) for b in range(2) for h in range(2)])
    assert r["units"] == 4 and r["seconds"] > 0
