"""GPU parity: libmiattn (through the C-ABI binding) against the fp64 CPU oracle.

Bar, for bf16 inputs with fp32 accumulation, O compared after upcasting the GPU's bf16
output: max abs error <= 2e-2, mean abs error <= 2e-3, LSE max abs error <= 1e-3.
Small shapes and the full-size prefill workloads are compared element by element over the
whole output (the full sizes through the oracle's process pool); the largest decode and
FP8 workloads on sampled heads and rows the oracle computes one by one.
Set MIATTN_PARITY_LOG=<path> to append every case's errors as JSON lines.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import attn_inputs as ai
import io_aware_exact_attention_amd as mi
from oracle import pool as oracle_pool
from oracle import (attention_backward, attention_decode, attention_decode_fp8,
                    attention_prefill, attention_prefill_fp8, attention_prefill_paged,
                    attention_prefill_paged_fp8, attention_prefill_varlen,
                    attention_prefill_varlen_fp8, attention_rows, e4m3_value, gather_paged)

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN, TOL_LSE = 2e-2, 2e-3, 1e-3


def dev(bits, dtype=torch.bfloat16):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def f64(bits):
    return ai.bf16_bits_to_f64(bits)


def log_case(label, **kv):
    path = os.environ.get("MIATTN_PARITY_LOG")
    print(label, kv, flush=True)
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": label, **kv}) + "\n")


def check(label, o_gpu, lse_gpu, o_ref, lse_ref, lse_tol=TOL_LSE):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    l = lse_gpu.float().cpu().numpy().astype(np.float64)
    assert o.shape == o_ref.shape and l.shape == lse_ref.shape
    err = np.abs(o - o_ref)
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(l) == fin).all(), f"{label}: LSE finiteness differs"
    assert (l[~fin] == lse_ref[~fin]).all()
    lerr = float(np.abs(l[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    log_case(label, max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max_abs=lerr,
             **({} if lse_tol == TOL_LSE else {"lse_tol": lse_tol}))
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    assert err.max() <= TOL_MAX, f"{label}: max abs {err.max():.3e}"
    assert err.mean() <= TOL_MEAN, f"{label}: mean abs {err.mean():.3e}"
    assert lerr <= lse_tol, f"{label}: lse max abs {lerr:.3e} (tolerance {lse_tol:.3e})"


def run_prefill(q, k, v, causal, scale):
    o, lse = mi.prefill(dev(q).reshape(q.shape), dev(k).reshape(k.shape),
                        dev(v).reshape(v.shape), causal, scale)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------------ prefill, whole outputs
def test_prefill_tiny_config():
    cfg = ai.CONFIGS["tiny_prefill"]
    q, k, v = ai.prefill_inputs(cfg)
    o, lse = run_prefill(q, k, v, cfg.causal, cfg.scale)
    ro, rl = attention_prefill(f64(q), f64(k), f64(v), cfg.scale, cfg.causal)
    check("tiny_prefill", o, lse, ro, rl)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 17, 63, 65, 127, 129, 1000])
def test_prefill_ragged_lengths(N, causal, d):
    q, k, v = ai.custom_prefill(seed=1000 + N, B=1, Hq=2, Hkv=2, Nq=N, Nk=N, d=d)
    scale = 1 / math.sqrt(d)
    o, lse = run_prefill(q, k, v, causal, scale)
    ro, rl = attention_prefill(f64(q), f64(k), f64(v), scale, causal)
    check(f"prefill N={N} causal={causal} d={d}", o, lse, ro, rl)


@pytest.mark.parametrize("Nq,Nk", [(1, 300), (77, 300), (128, 1000), (200, 201), (5, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_fewer_queries_than_keys(Nq, Nk, causal):
    q, k, v = ai.custom_prefill(seed=2000 + Nq, B=1, Hq=2, Hkv=1, Nq=Nq, Nk=Nk, d=128)
    o, lse = run_prefill(q, k, v, causal, 0.09)
    ro, rl = attention_prefill(f64(q), f64(k), f64(v), 0.09, causal)
    check(f"prefill Nq={Nq} Nk={Nk} causal={causal}", o, lse, ro, rl)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (8, 2), (8, 8), (6, 3)])
def test_prefill_gqa_and_batch(Hq, Hkv):
    q, k, v = ai.custom_prefill(seed=3000 + Hq * 10 + Hkv, B=3, Hq=Hq, Hkv=Hkv, Nq=150, Nk=150,
                                d=64)
    o, lse = run_prefill(q, k, v, True, 0.125)
    ro, rl = attention_prefill(f64(q), f64(k), f64(v), 0.125, True)
    check(f"prefill GQA Hq={Hq} Hkv={Hkv} B=3", o, lse, ro, rl)
    # GQA equals repeated-head MHA bit for bit (same arithmetic per head)
    G = Hq // Hkv
    o2, lse2 = run_prefill(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), True, 0.125)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.6])
def test_prefill_scale_values(scale):
    q, k, v = ai.custom_prefill(seed=4000, B=1, Hq=2, Hkv=2, Nq=190, Nk=190, d=64)
    o, lse = run_prefill(q, k, v, True, scale)
    ro, rl = attention_prefill(f64(q), f64(k), f64(v), float(np.float32(scale)), True)
    check(f"prefill scale={scale}", o, lse, ro, rl)


def test_prefill_worked_example_and_first_row():
    # q = e0, keys (0, e0), values (1, 5), scale ln 3: weights (1/4, 3/4), O = 4, LSE = ln 4
    d = 64
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, 2, d), np.float32)
    k[0, 0, 1, 0] = 1.0
    v = np.stack([np.ones(d), 5 * np.ones(d)]).astype(np.float32)[None, None]
    qb, kb, vb = ai.to_bf16_bits(q), ai.to_bf16_bits(k), ai.to_bf16_bits(v)
    o, lse = run_prefill(qb, kb, vb, True, float(np.float32(math.log(3.0))))
    out = o.float().cpu().numpy()[0, 0]
    # causal row 0 sees only key 0: exactly V[0]
    assert (out[0] == 1.0).all()
    assert np.abs(out[1] - 4.0).max() <= TOL_MAX
    assert abs(float(lse[0, 0, 1]) - math.log(4.0)) <= TOL_LSE
    assert abs(float(lse[0, 0, 0]) - 0.0) <= 1e-6


def test_prefill_causal_first_row_is_exact_and_runs_are_deterministic():
    q, k, v = ai.custom_prefill(seed=5000, B=2, Hq=4, Hkv=4, Nq=300, Nk=300, d=128)
    o1, l1 = run_prefill(q, k, v, True, 0.088)
    o2, l2 = run_prefill(q, k, v, True, 0.088)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    vv = dev(v).reshape(v.shape)
    assert torch.equal(o1[:, :, 0], vv[:, :, 0])


def test_prefill_constant_values():
    q, k, _ = ai.custom_prefill(seed=5100, B=1, Hq=2, Hkv=2, Nq=260, Nk=260, d=64)
    vrow = ai.to_bf16_bits(np.random.default_rng(1).standard_normal(64).astype(np.float32))
    v = np.broadcast_to(vrow, (1, 2, 260, 64)).copy()
    o, _ = run_prefill(q, k, v, True, 0.125)
    ref = np.broadcast_to(f64(vrow), (1, 2, 260, 64))
    assert np.abs(o.float().cpu().numpy() - ref).max() <= 1e-2


# ------------------------------------------------------------------ prefill, full sizes
def whole_prefill_check(name, o, lse):
    """Every output of a full-size prefill workload against the oracle, head by head in
    the oracle's process pool (each worker regenerates its head's inputs from the seeds)."""
    o_bits = o.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    gl = lse.cpu().numpy()
    r = oracle_pool.check_prefill_heads(name, o_bits, gl,
                                        progress=lambda m: print(m, flush=True))
    log_case(name + " (whole output)", max_abs=r["max_abs"], mean_abs=r["mean_abs"],
             lse_max_abs=r["lse_max_abs"], n=r["n"], max_at=list(r["max_at"]))
    cfg = ai.CONFIGS[name]
    assert r["n"] == cfg.B * cfg.Hq * cfg.Nq * cfg.d
    assert r["finite"]
    assert r["max_abs"] <= TOL_MAX and r["mean_abs"] <= TOL_MEAN and r["lse_max_abs"] <= TOL_LSE


@pytest.mark.parametrize("name", ["llama2_7b_prefill", "llama2_7b_prefill_noncausal"])
def test_prefill_llama2_shape(name):
    cfg = ai.CONFIGS[name]
    q, k, v = ai.prefill_inputs(cfg)
    o, lse = run_prefill(q, k, v, cfg.causal, cfg.scale)
    whole_prefill_check(name, o, lse)


def test_prefill_long_context_32k():
    # every row of every head; a block of 1,024 causal rows is compared against the keys
    # it can see (~9 TFLOP of fp64 oracle work over the pool)
    cfg = ai.CONFIGS["long_prefill_32k"]
    q, k, v = ai.prefill_inputs(cfg)
    o, lse = run_prefill(q, k, v, cfg.causal, cfg.scale)
    del q, k, v
    whole_prefill_check("long_prefill_32k", o, lse)


# ------------------------------------------------------------------ decode
def make_decode(B, Hq, Hkv, d, lens, seed, paged, extra_pages=3, fp8=False):
    cfg = ai.DecodeCfg("case", B=B, Hq=Hq, Hkv=Hkv, d=d, seed=seed, paged=paged, kv_fp8=fp8)
    lens = np.asarray(lens, np.int32)
    q = ai.decode_q(cfg)
    maxlen = max(int(lens.max()), 1)
    if paged:
        lay = ai.paged_layout(lens, 16, seed, extra_pages=extra_pages)
        kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
        vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
        table = lay.block_table
    else:
        kc = ai.build_contig_cache(cfg, ai.T_K, lens, maxlen)
        vc = ai.build_contig_cache(cfg, ai.T_V, lens, maxlen)
        table = None
    return cfg, q, kc, vc, lens, table, maxlen


def run_decode(q, kc, vc, lens, table, maxlen, scale, num_splits=0):
    o, lse = mi.decode(dev(q).reshape(q.shape), dev(kc).reshape(kc.shape),
                       dev(vc).reshape(vc.shape), torch.from_numpy(lens).cuda(), maxlen,
                       block_table=None if table is None else torch.from_numpy(table).cuda(),
                       scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def decode_ref(q, kc, vc, lens, table, scale):
    return attention_decode(f64(q), f64(kc), f64(vc), lens, scale, table, 16)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 0, 3])
def test_decode_edge_lengths(paged, d, splits):
    lens = [0, 1, 15, 16, 17, 31, 33, 1000]
    cfg, q, kc, vc, lens, table, maxlen = make_decode(8, 8, 2, d, lens, 600 + d, paged)
    o, lse = run_decode(q, kc, vc, lens, table, maxlen, cfg.scale, splits)
    ro, rl = decode_ref(q, kc, vc, lens, table, cfg.scale)
    check(f"decode edge paged={paged} d={d} splits={splits}", o, lse, ro, rl)
    assert (o[0] == 0).all() and torch.isinf(lse[0]).all()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (32, 1), (10, 2), (64, 2)])
def test_decode_group_sizes(Hq, Hkv):
    lens = [300, 77, 1]
    cfg, q, kc, vc, lens, table, maxlen = make_decode(3, Hq, Hkv, 128, lens, 700 + Hq, True)
    o, lse = run_decode(q, kc, vc, lens, table, maxlen, cfg.scale, 2)
    ro, rl = decode_ref(q, kc, vc, lens, table, cfg.scale)
    check(f"decode Hq={Hq} Hkv={Hkv}", o, lse, ro, rl)


def test_decode_paged_equals_contiguous_and_split_invariance():
    lens = [5000, 2048, 333, 4097]
    cfgc, q, kc, vc, lens_, _, maxlen = make_decode(4, 16, 4, 128, lens, 800, False)
    cfgp, q2, kp, vp, _, table, _ = make_decode(4, 16, 4, 128, lens, 800, True)
    assert (q == q2).all()
    ref = decode_ref(q, kc, vc, lens_, None, cfgc.scale)
    outs = {}
    for s in (1, 0, 5, 40):
        oc, lc = run_decode(q, kc, vc, lens_, None, maxlen, cfgc.scale, s)
        op, lp = run_decode(q, kp, vp, lens_, table, maxlen, cfgc.scale, s)
        assert torch.equal(oc, op) and torch.equal(lc, lp), f"paged != contiguous at splits={s}"
        check(f"decode splits={s}", oc, lc, *ref)
        outs[s] = oc.float()
    for s in (0, 5, 40):
        assert (outs[s] - outs[1]).abs().max().item() <= 2e-2


def test_decode_is_last_row_of_causal_prefill():
    n, H, d = 777, 4, 128
    q, k, v = ai.custom_prefill(seed=900, B=1, Hq=H, Hkv=H, Nq=n, Nk=n, d=d)
    op, lp = run_prefill(q, k, v, True, 0.088)
    qd = q[:, :, -1]
    od, ld = run_decode(qd, k, v, np.array([n], np.int32), None, n, 0.088, 3)
    assert (od.float() - op[:, :, -1].float()).abs().max().item() <= 2e-2
    assert (ld - lp[:, :, -1]).abs().max().item() <= 1e-3


@pytest.fixture(scope="module")
def cfg4_inputs():
    cfg = ai.CONFIGS["gqa_decode_contig"]
    lens = ai.decode_lengths(cfg)
    q = ai.decode_q(cfg)
    kc = ai.build_contig_cache(cfg, ai.T_K, lens, cfg.fixed_len)
    vc = ai.build_contig_cache(cfg, ai.T_V, lens, cfg.fixed_len)
    return cfg, q, kc, vc, lens


def test_decode_gqa_contiguous_config(cfg4_inputs):
    cfg, q, kc, vc, lens = cfg4_inputs
    o, lse = run_decode(q, kc, vc, lens, None, cfg.fixed_len, cfg.scale)
    o2, lse2 = run_decode(q, kc, vc, lens, None, cfg.fixed_len, cfg.scale)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    ro, rl = decode_ref(q, kc, vc, lens, None, cfg.scale)
    check("gqa_decode_contig", o, lse, ro, rl)


def test_decode_paged_config():
    cfg = ai.CONFIGS["paged_gqa_decode"]
    lens = ai.decode_lengths(cfg)
    lay = ai.paged_layout(lens, cfg.page_size, cfg.seed)
    q = ai.decode_q(cfg)
    kp = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
    vp = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
    maxlen = int(lens.max())
    o, lse = run_decode(q, kp, vp, lens, lay.block_table, maxlen, cfg.scale)
    ro, rl = decode_ref(q, kp, vp, lens, lay.block_table, cfg.scale)
    check("paged_gqa_decode", o, lse, ro, rl)


# ------------------------------------------------------------------ decode over an FP8 cache
def run_decode_fp8(q, kc, vc, lens, table, maxlen, scale, k_scale=ai.FP8_K_SCALE,
                   v_scale=ai.FP8_V_SCALE, num_splits=0):
    o, lse = mi.decode_fp8(dev(q).reshape(q.shape), torch.from_numpy(kc).cuda(),
                           torch.from_numpy(vc).cuda(), torch.from_numpy(lens).cuda(), maxlen,
                           k_scale, v_scale,
                           block_table=None if table is None else torch.from_numpy(table).cuda(),
                           scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def decode_fp8_ref(q, kc, vc, lens, table, scale, k_scale=ai.FP8_K_SCALE,
                   v_scale=ai.FP8_V_SCALE):
    return attention_decode_fp8(f64(q), kc, vc, lens, scale, k_scale, v_scale, table, 16)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 0, 3])
def test_decode_fp8_edge_lengths(paged, d, splits):
    lens = [0, 1, 15, 16, 17, 31, 33, 1000]
    cfg, q, kc, vc, lens, table, maxlen = make_decode(8, 8, 2, d, lens, 1600 + d, paged, fp8=True)
    assert kc.dtype == np.uint8
    o, lse = run_decode_fp8(q, kc, vc, lens, table, maxlen, cfg.scale, num_splits=splits)
    ro, rl = decode_fp8_ref(q, kc, vc, lens, table, cfg.scale)
    check(f"decode fp8 edge paged={paged} d={d} splits={splits}", o, lse, ro, rl)
    assert (o[0] == 0).all() and torch.isinf(lse[0]).all()


@pytest.mark.parametrize("Hq,Hkv", [(32, 1), (10, 2)])
def test_decode_fp8_group_sizes(Hq, Hkv):
    cfg, q, kc, vc, lens, table, maxlen = make_decode(3, Hq, Hkv, 128, [300, 77, 1], 1700 + Hq,
                                                      True, fp8=True)
    o, lse = run_decode_fp8(q, kc, vc, lens, table, maxlen, cfg.scale, num_splits=2)
    ro, rl = decode_fp8_ref(q, kc, vc, lens, table, cfg.scale)
    check(f"decode fp8 Hq={Hq} Hkv={Hkv}", o, lse, ro, rl)


@pytest.mark.parametrize("paged", [False, True])
def test_decode_fp8_unit_scales_equal_bf16_decode_of_widened_cache(paged):
    """With unit scales the FP8 path must give the bf16 path's bits on the bf16 widening of
    the same codes (E4M3 values are exact in bf16), which pins the widening and its byte
    order; every code except the two NaNs occurs in the random cache."""
    cfg, q, kc, vc, lens, table, maxlen = make_decode(4, 16, 4, 128, [700, 64, 1, 2100], 1800,
                                                      paged, fp8=True)
    rng = np.random.default_rng(5)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    live = kc != 0x7F
    kc = np.where(live, rng.choice(codes, kc.shape), kc).astype(np.uint8)
    vc = np.where(live, rng.choice(codes, vc.shape), vc).astype(np.uint8)
    widen = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.bfloat16).cuda()
    for s in (1, 0, 7):
        o8, l8 = run_decode_fp8(q, kc, vc, lens, table, maxlen, 0.01, 1.0, 1.0, s)
        ob, lb = mi.decode(dev(q).reshape(q.shape), widen(kc), widen(vc),
                           torch.from_numpy(lens).cuda(), maxlen,
                           block_table=None if table is None else torch.from_numpy(table).cuda(),
                           scale=0.01, num_splits=s)
        torch.cuda.synchronize()
        assert torch.equal(o8, ob) and torch.equal(l8, lb), f"fp8 != bf16 widening at splits={s}"
    ro, rl = decode_fp8_ref(q, kc, vc, lens, table, 0.01, 1.0, 1.0)
    # the bar is set for V of order one; these codes reach 448, so O and the reference are
    # divided by 128 (exact) first
    check(f"decode fp8 unit scales paged={paged}", o8.float() / 128, l8, ro / 128, rl)


@pytest.mark.parametrize("scale,k_scale,v_scale", [(-0.09, 0.02, 0.5), (0.2, 3.0, 0.001),
                                                   (0.0884, 2.0 ** -7, 2.0 ** 5)])
def test_decode_fp8_scale_values(scale, k_scale, v_scale):
    cfg, q, kc, vc, lens, table, maxlen = make_decode(2, 8, 2, 64, [513, 40], 1900, True,
                                                      fp8=True)
    o, lse = run_decode_fp8(q, kc, vc, lens, table, maxlen, scale, k_scale, v_scale)
    ro, rl = decode_fp8_ref(q, kc, vc, lens, table, scale, k_scale, v_scale)
    # V = v_scale * codes, where the codes are N(0,1) draws / FP8_V_SCALE: outputs and their
    # errors scale with v_scale / FP8_V_SCALE, which the bar (set for V of order one) divides out
    norm = v_scale / ai.FP8_V_SCALE
    check(f"decode fp8 scale={scale} ks={k_scale} vs={v_scale}", o.float() / norm, lse,
          ro / norm, rl)


def test_decode_fp8_paged_equals_contiguous():
    lens = [5000, 2048, 333, 4097]
    cfgc, q, kc, vc, lens_, _, maxlen = make_decode(4, 16, 4, 128, lens, 1950, False, fp8=True)
    _, q2, kp, vp, _, table, _ = make_decode(4, 16, 4, 128, lens, 1950, True, fp8=True)
    assert (q == q2).all()
    ref = decode_fp8_ref(q, kc, vc, lens_, None, cfgc.scale)
    for s in (0, 5):
        oc, lc = run_decode_fp8(q, kc, vc, lens_, None, maxlen, cfgc.scale, num_splits=s)
        op, lp = run_decode_fp8(q, kp, vp, lens_, table, maxlen, cfgc.scale, num_splits=s)
        assert torch.equal(oc, op) and torch.equal(lc, lp), f"paged != contiguous at splits={s}"
        check(f"decode fp8 splits={s}", oc, lc, *ref)


def test_decode_fp8_paged_config():
    cfg = ai.CONFIGS["paged_gqa_decode_fp8"]
    lens = ai.decode_lengths(cfg)
    lay = ai.paged_layout(lens, cfg.page_size, cfg.seed)
    q = ai.decode_q(cfg)
    kp = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
    vp = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
    maxlen = int(lens.max())
    o, lse = run_decode_fp8(q, kp, vp, lens, lay.block_table, maxlen, cfg.scale)
    ro, rl = decode_fp8_ref(q, kp, vp, lens, lay.block_table, cfg.scale)
    check("paged_gqa_decode_fp8", o, lse, ro, rl)


# ------------------------------------------------------------------ chunked prefill, paged cache
def make_chunk(B, Hq, Hkv, d, lens, Nq, seed, extra_pages=3):
    """Chunk queries plus a paged cache whose unused slots and pages hold NaN."""
    cfg = ai.DecodeCfg("chunk", B=B, Hq=Hq, Hkv=Hkv, d=d, seed=seed, paged=True, chunk=Nq)
    lens = np.asarray(lens, np.int32)
    q = ai.chunk_q(cfg)
    lay = ai.paged_layout(lens, 16, seed, extra_pages=extra_pages)
    kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
    vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
    return cfg, q, kc, vc, lens, lay.block_table


def run_chunk(q, kc, vc, lens, table, causal, scale):
    o, lse = mi.prefill_paged(dev(q).reshape(q.shape), dev(kc).reshape(kc.shape),
                              dev(vc).reshape(vc.shape), torch.from_numpy(table).cuda(),
                              torch.from_numpy(lens).cuda(), int(lens.max()), causal, scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Nq,lens", [(1, (1, 17, 300)), (77, (77, 200, 1000)),
                                     (256, (256, 300, 1031)), (300, (300, 301, 700))])
def test_prefill_paged_chunks(d, causal, Nq, lens):
    cfg, q, kc, vc, lens, table = make_chunk(3, 4, 2, d, lens, Nq, seed=2000 + Nq + d)
    scale = 1 / math.sqrt(d)
    o, lse = run_chunk(q, kc, vc, lens, table, causal, scale)
    ro, rl = attention_prefill_paged(f64(q), f64(kc), f64(vc), table, lens, scale, causal)
    check(f"prefill_paged d={d} causal={causal} Nq={Nq} lens={tuple(int(x) for x in lens)}",
          o, lse, ro, rl)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paged_kv_lens_clamped(causal):
    # kv_lens live on the device, so the host cannot check them: the kernel clamps each to
    # [Nq, max_kv_len].  The cache holds (77, 700, 700) tokens; the call passes 10 (below
    # Nq) and 5000 (above max_kv_len = 700, whose block-table row has 44 entries), and must
    # equal the call with the clamped lengths.
    Nq = 77
    cfg, q, kc, vc, lens, table = make_chunk(3, 4, 2, 128, (77, 700, 700), Nq, seed=2150)
    assert table.shape[1] == 44
    bad = np.asarray([10, 5000, 700], np.int32)
    o, lse = mi.prefill_paged(dev(q).reshape(q.shape), dev(kc).reshape(kc.shape),
                              dev(vc).reshape(vc.shape), torch.from_numpy(table).cuda(),
                              torch.from_numpy(bad).cuda(), 700, causal, 0.09)
    torch.cuda.synchronize()
    ro, rl = attention_prefill_paged(f64(q), f64(kc), f64(vc), table, lens, 0.09, causal)
    check(f"prefill_paged clamped kv_lens causal={causal}", o, lse, ro, rl)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paged_equals_contiguous_prefill(causal):
    # one sequence: the same key/value rows through the paged and the contiguous kernel
    cfg, q, kc, vc, lens, table = make_chunk(1, 8, 2, 128, (1000,), 333, seed=2100)
    o_p, l_p = run_chunk(q, kc, vc, lens, table, causal, 0.088)
    k = np.stack([np.stack([gather_paged(kc, table, 0, h, 1000, 16) for h in range(2)])])
    v = np.stack([np.stack([gather_paged(vc, table, 0, h, 1000, 16) for h in range(2)])])
    o_c, l_c = run_prefill(q, k, v, causal, 0.088)
    assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c)


def test_chunked_prefill_paged_config():
    cfg = ai.CONFIGS["chunked_prefill_paged"]
    lens = ai.decode_lengths(cfg)
    q = ai.chunk_q(cfg)
    lay = ai.paged_layout(lens, 16, cfg.seed)
    kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
    vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
    o, lse = run_chunk(q, kc, vc, lens, lay.block_table, True, cfg.scale)
    go = o.float().cpu().numpy().astype(np.float64)
    gl = lse.float().cpu().numpy().astype(np.float64)
    G = cfg.Hq // cfg.Hkv
    errs, lerrs = [], []
    for b in range(cfg.B):  # one query head per sequence, every row of it
        h = (5 * b + 3) % cfg.Hq
        kvh = h // G
        n = int(lens[b])
        K = f64(gather_paged(kc, lay.block_table, b, kvh, n, 16))
        V = f64(gather_paged(vc, lay.block_table, b, kvh, n, 16))
        rows = np.arange(cfg.chunk)
        ro, rl = attention_rows(f64(q[b, h]), K, V, cfg.scale, True, rows, cfg.chunk)
        errs.append(np.abs(go[b, h] - ro))
        lerrs.append(np.abs(gl[b, h] - rl))
    err, lerr = np.concatenate([e.ravel() for e in errs]), np.concatenate(lerrs)
    log_case("chunked_prefill_paged (sampled)", max_abs=float(err.max()),
             mean_abs=float(err.mean()), lse_max_abs=float(lerr.max()), n=int(err.size))
    assert np.isfinite(go).all()
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN and lerr.max() <= TOL_LSE


# ------------------------------------------------------------------ fp16 entry points
def dev16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16)
    return t.cuda()


def h64(bits):
    return ai.f16_bits_to_f64(bits)


def run_prefill16(q, k, v, causal, scale):
    o, lse = mi.prefill(dev16(q).reshape(q.shape), dev16(k).reshape(k.shape),
                        dev16(v).reshape(v.shape), causal, scale)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    return o, lse


@pytest.mark.parametrize("N,Nk,causal,d", [(1, 1, True, 64), (65, 65, False, 128),
                                           (129, 129, True, 128), (1000, 1000, True, 64),
                                           (300, 300, False, 64), (100, 700, True, 128),
                                           (77, 300, False, 128)])
def test_prefill_f16_shapes(N, Nk, causal, d):
    q, k, v = ai.custom_prefill(seed=5200 + N + d, B=1, Hq=2, Hkv=2, Nq=N, Nk=Nk, d=d, f16=True)
    scale = 1 / math.sqrt(d)
    o, lse = run_prefill16(q, k, v, causal, scale)
    ro, rl = attention_prefill(h64(q), h64(k), h64(v), scale, causal)
    check(f"prefill f16 Nq={N} Nk={Nk} causal={causal} d={d}", o, lse, ro, rl)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.6])
def test_prefill_f16_gqa_and_scale(scale):
    q, k, v = ai.custom_prefill(seed=5300, B=2, Hq=8, Hkv=2, Nq=190, Nk=190, d=64, f16=True)
    o, lse = run_prefill16(q, k, v, True, scale)
    ro, rl = attention_prefill(h64(q), h64(k), h64(v), float(np.float32(scale)), True)
    check(f"prefill f16 GQA scale={scale}", o, lse, ro, rl)


def test_prefill_f16_rising_scores_redo_every_tile():
    """Scores that rise by ~40 (natural log units) from one 64-key tile to the next: each
    new tile's weights against the previous tile's max would be ~2^58, far past fp16, so
    the fp16 kernel must redo every tile against a fresh max (its bound is 2^15)."""
    d, N = 64, 512
    rng = np.random.default_rng(11)
    u = np.zeros(d, np.float32)
    u[0] = 1.0
    t = np.arange(N, dtype=np.float32) * np.float32(40.0 / 64.0)   # score of key j
    k = ai.to_f16_bits(t[:, None] * u[None, :] + rng.standard_normal((N, d)).astype(np.float32)
                       * np.float32(0.01))
    q = ai.to_f16_bits(np.tile(u, (N, 1)))
    v = ai.to_f16_bits(rng.standard_normal((N, d)).astype(np.float32))
    q, k, v = q[None, None], k[None, None], v[None, None]
    for causal in (False, True):
        o, lse = run_prefill16(q, k, v, causal, 1.0)
        ro, rl = attention_prefill(h64(q), h64(k), h64(v), 1.0, causal)
        check(f"prefill f16 rising scores causal={causal}", o, lse, ro, rl)


def test_prefill_f16_llama2_shape():
    cfg = ai.CONFIGS["llama2_7b_prefill_f16"]
    q, k, v = ai.prefill_inputs(cfg)
    o, lse = run_prefill16(q, k, v, cfg.causal, cfg.scale)
    whole_prefill_check("llama2_7b_prefill_f16", o, lse)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paged_f16_chunks(causal):
    cfg = ai.DecodeCfg("chunk16", B=3, Hq=4, Hkv=2, d=128, seed=5400, paged=True, chunk=77,
                       f16=True)
    lens = np.array([77, 200, 1000], np.int32)
    q = ai.chunk_q(cfg)
    lay = ai.paged_layout(lens, 16, cfg.seed, extra_pages=3)
    kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
    vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
    o, lse = mi.prefill_paged(dev16(q).reshape(q.shape), dev16(kc).reshape(kc.shape),
                              dev16(vc).reshape(vc.shape),
                              torch.from_numpy(lay.block_table).cuda(),
                              torch.from_numpy(lens).cuda(), int(lens.max()), causal, 0.088)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    ro, rl = attention_prefill_paged(h64(q), h64(kc), h64(vc), lay.block_table, lens, 0.088,
                                     causal)
    check(f"prefill_paged f16 causal={causal}", o, lse, ro, rl)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("splits", [1, 0])
def test_decode_f16(paged, splits):
    lens = [0, 1, 17, 33, 1000, 4097]
    cfg = ai.DecodeCfg("dec16", B=6, Hq=16, Hkv=4, d=128, seed=5500, paged=paged, f16=True)
    lens = np.asarray(lens, np.int32)
    q = ai.decode_q(cfg)
    maxlen = int(lens.max())
    if paged:
        lay = ai.paged_layout(lens, 16, cfg.seed, extra_pages=3)
        kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
        vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
        table = lay.block_table
    else:
        kc = ai.build_contig_cache(cfg, ai.T_K, lens, maxlen)
        vc = ai.build_contig_cache(cfg, ai.T_V, lens, maxlen)
        table = None
    o, lse = mi.decode(dev16(q).reshape(q.shape), dev16(kc).reshape(kc.shape),
                       dev16(vc).reshape(vc.shape), torch.from_numpy(lens).cuda(), maxlen,
                       block_table=None if table is None else torch.from_numpy(table).cuda(),
                       scale=cfg.scale, num_splits=splits)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    ro, rl = attention_decode(h64(q), h64(kc), h64(vc), lens, cfg.scale, table, 16)
    check(f"decode f16 paged={paged} splits={splits}", o, lse, ro, rl)
    assert (o[0] == 0).all() and torch.isinf(lse[0]).all()


# ------------------------------------------------------------------ backward
# Bar for gradients (the forward bar is for outputs of order one; gradients have no fixed
# scale, so errors are measured relative to the reference gradient's size): per tensor,
# max|err| <= 2e-2 * max(max|ref|, 1e-2) and mean|err| <= 1e-2 * max(mean|ref|, 1e-2).
# Derivation: P and dS are rounded to bf16 before their products (relative 2^-9 each) and
# the outputs are bf16 (relative 2^-9), so the expected relative error is a few times
# 2^-9 ~ 0.2-0.6%.  The 1e-2 floor covers gradients that vanish exactly (one visible key,
# scale 0): there the kernel's dS is the difference of rowsum(dO*O), with O the forward's
# bf16 output, and rowsum(P*dP), which differ by ~2^-9 of dO*V, not by zero.
BWD_REL_MAX, BWD_REL_MEAN, BWD_FLOOR = 2e-2, 1e-2, 1e-2


def check_grads(label, got, ref):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        x = g.float().cpu().numpy().astype(np.float64)
        assert x.shape == r.shape, (name, x.shape, r.shape)
        assert np.isfinite(x).all(), f"{label} {name}: non-finite"
        err = np.abs(x - r)
        scale_max = max(np.abs(r).max(), BWD_FLOOR)
        scale_mean = max(np.abs(r).mean(), BWD_FLOOR)
        log_case(f"{label} {name}", rel_max=float(err.max() / scale_max),
                 rel_mean=float(err.mean() / scale_mean), ref_max=float(scale_max))
        assert err.max() <= BWD_REL_MAX * scale_max, f"{label} {name}: max {err.max():.3e}"
        assert err.mean() <= BWD_REL_MEAN * scale_mean, f"{label} {name}: mean {err.mean():.3e}"


def run_bwd(q, k, v, do, causal, scale, f16=False):
    to = dev16 if f16 else dev
    dq_, dk_, dv_ = (to(x).reshape(x.shape) for x in (q, k, v))
    o, lse = mi.prefill(dq_, dk_, dv_, causal, scale)
    gdo = to(do).reshape(do.shape)
    grads = mi.backward(dq_, dk_, dv_, o, lse, gdo, causal, scale)
    torch.cuda.synchronize()
    assert all(g.dtype == dq_.dtype for g in grads)
    return grads


def bwd_inputs(seed, B, Hq, Hkv, Nq, Nk, d, f16=False):
    q, k, v = ai.custom_prefill(seed=seed, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, f16=f16)
    do = ai.prefill_dout(ai.PrefillCfg("bwd", B, Hq, Hkv, Nq, Nk, d, True, seed, 1.0, f16))
    return q, k, v, do


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (17, 17), (65, 65), (130, 130), (300, 300),
                                   (64, 200), (100, 333)])
def test_backward_shapes(Nq, Nk, causal, d):
    q, k, v, do = bwd_inputs(7000 + Nq + Nk + d, 1, 2, 2, Nq, Nk, d)
    scale = 1 / math.sqrt(d)
    got = run_bwd(q, k, v, do, causal, scale)
    ref = attention_backward(f64(q), f64(k), f64(v), f64(do), scale, causal)
    check_grads(f"bwd Nq={Nq} Nk={Nk} causal={causal} d={d}", got, ref)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.6])
def test_backward_gqa_and_scale(scale):
    q, k, v, do = bwd_inputs(7100, 2, 8, 2, 150, 150, 64)
    got = run_bwd(q, k, v, do, True, scale)
    ref = attention_backward(f64(q), f64(k), f64(v), f64(do), float(np.float32(scale)), True)
    if scale == 0.0:
        assert (got[0] == 0).all() and (got[1] == 0).all()   # dQ = dK = 0 exactly
        ref = (ref[0], ref[1], ref[2])
        check_grads("bwd GQA scale=0 (dv)", got[2:], ref[2:])
        return
    check_grads(f"bwd GQA scale={scale}", got, ref)


@pytest.mark.parametrize("Nq,Nk,causal,d", [(1, 1, True, 64), (130, 130, True, 128),
                                            (300, 300, False, 64), (100, 333, True, 128),
                                            (65, 200, False, 128)])
def test_backward_f16_shapes(Nq, Nk, causal, d):
    q, k, v, do = bwd_inputs(7300 + Nq + Nk + d, 1, 2, 2, Nq, Nk, d, f16=True)
    scale = 1 / math.sqrt(d)
    got = run_bwd(q, k, v, do, causal, scale, f16=True)
    ref = attention_backward(h64(q), h64(k), h64(v), h64(do), scale, causal)
    check_grads(f"bwd f16 Nq={Nq} Nk={Nk} causal={causal} d={d}", got, ref)


def test_backward_f16_gqa():
    q, k, v, do = bwd_inputs(7400, 2, 8, 2, 150, 150, 64, f16=True)
    got = run_bwd(q, k, v, do, True, -0.2, f16=True)
    ref = attention_backward(h64(q), h64(k), h64(v), h64(do), float(np.float32(-0.2)), True)
    check_grads("bwd f16 GQA scale=-0.2", got, ref)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_odd_group_size(causal):
    """Three query heads per KV head: dK and dV sum over the group."""
    q, k, v, do = bwd_inputs(7450, 2, 6, 2, 200, 233 if not causal else 200, 128)
    got = run_bwd(q, k, v, do, causal, 0.07)
    ref = attention_backward(f64(q), f64(k), f64(v), f64(do), float(np.float32(0.07)), causal)
    check_grads(f"bwd Hq=6 Hkv=2 causal={causal}", got, ref)


def test_backward_is_deterministic():
    q, k, v, do = bwd_inputs(7200, 1, 4, 2, 700, 700, 128)
    g1 = run_bwd(q, k, v, do, True, 0.09)
    g2 = run_bwd(q, k, v, do, True, 0.09)
    for a_, b_ in zip(g1, g2):
        assert torch.equal(a_, b_)


def test_backward_llama2_shape():
    cfg = ai.CONFIGS["llama2_7b_prefill"]
    q, k, v = ai.prefill_inputs(cfg)
    do = ai.prefill_dout(cfg)
    dq, dk, dv = run_bwd(q, k, v, do, cfg.causal, cfg.scale)
    got = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    for (b, h) in [(0, 0), (3, 31), (2, 9)]:
        ref = attention_backward(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]),
                                 f64(v[b:b + 1, h:h + 1]), f64(do[b:b + 1, h:h + 1]),
                                 cfg.scale, cfg.causal)
        check_grads(f"bwd llama2 head ({b},{h})",
                    [torch.from_numpy(x[b:b + 1, h:h + 1]) for x in got], ref)


# ------------------------------------------------------------------ varlen (ragged) prefill
def run_varlen(q, k, v, cu_q, cu_k, causal, scale, f16=False):
    mq = int(np.diff(cu_q).max())
    mk = int(np.diff(cu_k).max())
    to = dev16 if f16 else dev
    o, lse = mi.prefill_varlen(to(q).reshape(q.shape), to(k).reshape(k.shape),
                               to(v).reshape(v.shape), torch.from_numpy(cu_q).cuda(),
                               torch.from_numpy(cu_k).cuda(), max(mq, 1), max(mk, 1), causal,
                               scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens_q,lens_k", [
    ([1, 255, 256, 257, 700], [1, 255, 256, 257, 700]),        # self-attention, tile edges
    ([5, 0, 300, 64], [40, 17, 300, 1000]),                      # Nq < Nk, an empty chunk
    ([513], [513]),
])
def test_prefill_varlen(d, causal, lens_q, lens_k):
    q, k, v, cu_q, cu_k = ai.varlen_inputs(7500 + d + len(lens_q), lens_q, lens_k, 4, 2, d)
    scale = 1 / math.sqrt(d)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, causal, scale)
    ro, rl = attention_prefill_varlen(f64(q), f64(k), f64(v), cu_q, cu_k, scale, causal)
    check(f"varlen d={d} causal={causal} lens_q={lens_q} lens_k={lens_k}", o, lse, ro, rl)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_varlen_f16(causal, d):
    lens_q, lens_k = [3, 0, 300, 129], [40, 17, 300, 600]
    q, k, v, cu_q, cu_k = ai.varlen_inputs(7550 + d, lens_q, lens_k, 4, 2, d, f16=True)
    scale = 1 / math.sqrt(d)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, causal, scale, f16=True)
    assert o.dtype == torch.float16
    ro, rl = attention_prefill_varlen(h64(q), h64(k), h64(v), cu_q, cu_k, scale, causal)
    check(f"varlen f16 d={d} causal={causal}", o, lse, ro, rl)


def test_prefill_varlen_odd_group_size():
    lens_q, lens_k = [70, 300, 1], [70, 450, 20]
    q, k, v, cu_q, cu_k = ai.varlen_inputs(7580, lens_q, lens_k, 6, 2, 128)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True, 0.1)
    ro, rl = attention_prefill_varlen(f64(q), f64(k), f64(v), cu_q, cu_k, float(np.float32(0.1)),
                                      True)
    check("varlen Hq=6 Hkv=2", o, lse, ro, rl)


@pytest.mark.parametrize("B", [64, 65])
def test_prefill_varlen_many_sequences(B):
    """Up to 64 sequences, each workgroup finds its (sequence, query tile) from the
    cumulative lengths, over a grid sized from the total; beyond 64 the grid covers the
    longest sequence for each.  Empty sequences and tile-edge lengths included."""
    rng = np.random.default_rng(7800 + B)
    lens = [int(x) for x in rng.integers(0, 600, B)]
    lens[3], lens[10], lens[11], lens[B - 1] = 0, 256, 257, 512
    q, k, v, cu_q, cu_k = ai.varlen_inputs(7800 + B, lens, lens, 8, 2, 64)
    for causal in (True, False):
        o, lse = run_varlen(q, k, v, cu_q, cu_k, causal, 0.125)
        ro, rl = attention_prefill_varlen(f64(q), f64(k), f64(v), cu_q, cu_k, 0.125, causal)
        check(f"varlen B={B} causal={causal}", o, lse, ro, rl)


def test_prefill_varlen_sequence_without_keys():
    q, k, v, cu_q, cu_k = ai.varlen_inputs(7600, [10, 20], [30, 0], 2, 2, 64)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, False, 0.125)
    assert (o[10:] == 0).all() and torch.isinf(lse[:, 10:]).all()
    ro, rl = attention_prefill_varlen(f64(q), f64(k), f64(v), cu_q, cu_k, 0.125, False)
    check("varlen sequence without keys", o, lse, ro, rl)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_varlen_single_sequence_equals_dense(causal):
    """One sequence packed along tokens is the dense prefill with the layout transposed:
    the same tiles in the same order, so the same bits."""
    n, Hq, Hkv, d = 777, 8, 2, 128
    q, k, v, cu_q, cu_k = ai.varlen_inputs(7700, [n], [n], Hq, Hkv, d)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, causal, 0.09)
    qd = np.ascontiguousarray(q.transpose(1, 0, 2))[None]
    kd = np.ascontiguousarray(k.transpose(1, 0, 2))[None]
    vd = np.ascontiguousarray(v.transpose(1, 0, 2))[None]
    od, ld = run_prefill(qd, kd, vd, causal, 0.09)
    assert torch.equal(o, od[0].transpose(0, 1)) and torch.equal(lse, ld[0])


def test_prefill_varlen_config_sampled():
    cfg = ai.CONFIGS["varlen_prefill"]
    lens = ai.varlen_lengths(cfg.seed, cfg.B, *cfg.len_range)
    q, k, v, cu_q, cu_k = ai.varlen_inputs(cfg.seed, lens, lens, cfg.Hq, cfg.Hkv, cfg.d)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True, cfg.scale)
    go, gl = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(19)
    errs, lerrs = [], []
    G = cfg.Hq // cfg.Hkv
    for b in rng.choice(cfg.B, 4, replace=False):
        qs, qe = int(cu_q[b]), int(cu_q[b + 1])
        n = qe - qs
        for h in rng.choice(cfg.Hq, 2, replace=False):
            rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 32)]))
            ro, rl = attention_rows(f64(q[qs + rows, h]), f64(k[qs:qe, h // G]),
                                    f64(v[qs:qe, h // G]), cfg.scale, True, rows, n)
            errs.append(np.abs(go[qs + rows, h] - ro).ravel())
            lerrs.append(np.abs(gl[h, qs + rows] - rl).ravel())
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    log_case("varlen_prefill (sampled)", max_abs=float(err.max()), mean_abs=float(err.mean()),
             lse_max_abs=float(lerr.max()))
    assert np.isfinite(go).all()
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN and lerr.max() <= TOL_LSE


# ------------------------------------------------------------------ bad page-table entries
def test_out_of_range_page_ids_are_clamped_into_the_pool():
    """Table entries outside [0, num_pages) are clamped to the nearest end on the device
    (negative ids, read as unsigned, to num_pages - 1): the result equals, bit for bit, a
    run whose table holds num_pages - 1 there, and every other sequence's result is the
    same as with a valid table.  (Caches padded with zeros so that all results are
    finite.)"""
    zero = np.uint16(0)
    lens = np.array([300, 77, 500], np.int32)
    cfg = ai.DecodeCfg("clamp", B=3, Hq=8, Hkv=2, d=128, seed=1990, paged=True)
    lay = ai.paged_layout(lens, 16, cfg.seed, extra_pages=3)
    q = ai.decode_q(cfg)
    kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay, pad_bits=zero)
    vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay, pad_bits=zero)
    last = kc.shape[0] - 1
    bad, clamped = lay.block_table.copy(), lay.block_table.copy()
    bad[0, 1], bad[0, 3] = -1, kc.shape[0] + 5
    clamped[0, 1], clamped[0, 3] = last, last
    maxlen = int(lens.max())
    o_ok, l_ok = run_decode(q, kc, vc, lens, lay.block_table, maxlen, cfg.scale, 2)
    o_bad, l_bad = run_decode(q, kc, vc, lens, bad, maxlen, cfg.scale, 2)
    o_cl, l_cl = run_decode(q, kc, vc, lens, clamped, maxlen, cfg.scale, 2)
    assert torch.equal(o_bad, o_cl) and torch.equal(l_bad, l_cl)
    assert torch.equal(o_ok[1:], o_bad[1:]) and torch.equal(l_ok[1:], l_bad[1:])
    # the same for chunked prefill against the paged cache
    ccfg = ai.DecodeCfg("clamp_chunk", B=3, Hq=4, Hkv=2, d=128, seed=1991, paged=True, chunk=77)
    clay = ai.paged_layout(lens, 16, ccfg.seed, extra_pages=3)
    cq = ai.chunk_q(ccfg)
    ckc = ai.build_paged_cache(ccfg, ai.T_K, lens, clay, pad_bits=zero)
    cvc = ai.build_paged_cache(ccfg, ai.T_V, lens, clay, pad_bits=zero)
    clast = ckc.shape[0] - 1
    cbad, ccl = clay.block_table.copy(), clay.block_table.copy()
    cbad[0, 2], cbad[2, 5] = -7, ckc.shape[0] + 100
    ccl[0, 2], ccl[2, 5] = clast, clast
    ok = run_chunk(cq, ckc, cvc, lens, clay.block_table, True, 0.09)
    bd = run_chunk(cq, ckc, cvc, lens, cbad, True, 0.09)
    cl = run_chunk(cq, ckc, cvc, lens, ccl, True, 0.09)
    assert torch.equal(bd[0], cl[0]) and torch.equal(bd[1], cl[1])
    assert torch.equal(ok[0][1], bd[0][1]) and torch.equal(ok[1][1], bd[1][1])


# ------------------------------------------------------------------ seeded random shapes
# Shapes drawn from fixed seeds (so every run tests the same cases): batch, heads, group
# size, lengths, head dimension, masking and scale all vary together, at sizes the oracle
# finishes in well under a second each.
def _random_shape(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 3, 4, 8]))
    Hkv = int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    Nk = int(rng.integers(1, 700))
    Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 700))
    scale = float(np.float32(rng.choice([1 / math.sqrt(d), 0.3, -0.15])))
    return dict(B=int(rng.integers(1, 4)), Hq=G * Hkv, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d,
                causal=causal, scale=scale)


@pytest.mark.parametrize("seed", list(range(9100, 9116)))
def test_prefill_random_shapes(seed):
    s = _random_shape(seed)
    q, k, v = ai.custom_prefill(seed=seed, B=s["B"], Hq=s["Hq"], Hkv=s["Hkv"], Nq=s["Nq"],
                                Nk=s["Nk"], d=s["d"])
    o, lse = run_prefill(q, k, v, s["causal"], s["scale"])
    ro, rl = attention_prefill(f64(q), f64(k), f64(v), s["scale"], s["causal"])
    check(f"prefill random seed={seed} {s}", o, lse, ro, rl)


@pytest.mark.parametrize("seed", list(range(9200, 9212)))
def test_decode_random_shapes(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 5, 8, 16, 24]))
    Hkv = int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 7))
    lens = rng.integers(0, 3000, size=B)
    paged = bool(rng.integers(0, 2))
    splits = int(rng.choice([0, 1, 2, 7]))
    cfg, q, kc, vc, lens, table, maxlen = make_decode(B, G * Hkv, Hkv, d, lens, seed, paged)
    o, lse = run_decode(q, kc, vc, lens, table, maxlen, cfg.scale, splits)
    ro, rl = decode_ref(q, kc, vc, lens, table, cfg.scale)
    check(f"decode random seed={seed} B={B} Hq={G * Hkv} Hkv={Hkv} d={d} paged={paged} "
          f"splits={splits}", o, lse, ro, rl)


@pytest.mark.parametrize("seed", list(range(9300, 9308)))
def test_prefill_varlen_random_shapes(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    G = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    lens_k = rng.integers(1, 600, size=B)
    lens_q = np.array([int(rng.integers(0, n + 1)) for n in lens_k]) if causal \
        else rng.integers(0, 600, size=B)
    q, k, v, cu_q, cu_k = ai.varlen_inputs(seed, lens_q, lens_k, G * Hkv, Hkv, d)
    if cu_q[-1] == 0:
        pytest.skip("no queries drawn")
    o, lse = run_varlen(q, k, v, cu_q, cu_k, causal, 1 / math.sqrt(d))
    ro, rl = attention_prefill_varlen(f64(q), f64(k), f64(v), cu_q, cu_k,
                                      float(np.float32(1 / math.sqrt(d))), causal)
    check(f"varlen random seed={seed} lens_q={lens_q.tolist()} lens_k={lens_k.tolist()} "
          f"Hq={G * Hkv} Hkv={Hkv} d={d} causal={causal}", o, lse, ro, rl)


@pytest.mark.parametrize("seed", list(range(9400, 9408)))
def test_prefill_paged_random_shapes(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    Nq = int(rng.integers(1, 400))
    lens = Nq + rng.integers(0, 1200, size=B)  # every context holds the Nq chunk queries
    causal = bool(rng.integers(0, 2))
    cfg, q, kc, vc, lens, table = make_chunk(B, G * Hkv, Hkv, d, lens, Nq, seed=seed)
    scale = float(np.float32(rng.choice([1 / math.sqrt(d), -0.1])))
    o, lse = run_chunk(q, kc, vc, lens, table, causal, scale)
    ro, rl = attention_prefill_paged(f64(q), f64(kc), f64(vc), table, lens, scale, causal)
    check(f"prefill_paged random seed={seed} B={B} Hq={G * Hkv} Hkv={Hkv} d={d} Nq={Nq} "
          f"lens={lens.tolist()} causal={causal}", o, lse, ro, rl)


@pytest.mark.parametrize("seed", list(range(9500, 9508)))
def test_backward_random_shapes(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 3, 4]))
    Hkv = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    Nk = int(rng.integers(1, 400))
    Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 400))
    B = int(rng.integers(1, 3))
    scale = float(np.float32(rng.choice([1 / math.sqrt(d), 0.2, -0.1])))
    q, k, v, do = bwd_inputs(seed, B, G * Hkv, Hkv, Nq, Nk, d)
    got = run_bwd(q, k, v, do, causal, scale)
    ref = attention_backward(f64(q), f64(k), f64(v), f64(do), scale, causal)
    check_grads(f"bwd random seed={seed} B={B} Hq={G * Hkv} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} "
                f"causal={causal} scale={scale}", got, ref)


@pytest.mark.parametrize("seed", list(range(9600, 9606)))
def test_decode_fp8_random_shapes(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 4, 8, 20]))
    Hkv = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 6))
    lens = rng.integers(0, 2500, size=B)
    paged = bool(rng.integers(0, 2))
    cfg, q, kc, vc, lens, table, maxlen = make_decode(B, G * Hkv, Hkv, d, lens, seed, paged,
                                                      fp8=True)
    o, lse = run_decode_fp8(q, kc, vc, lens, table, maxlen, cfg.scale)
    ro, rl = decode_fp8_ref(q, kc, vc, lens, table, cfg.scale)
    check(f"decode fp8 random seed={seed} B={B} Hq={G * Hkv} Hkv={Hkv} d={d} paged={paged}",
          o, lse, ro, rl)


@pytest.mark.parametrize("seed", list(range(9700, 9706)))
def test_prefill_f16_random_shapes(seed):
    s = _random_shape(seed)
    q, k, v = ai.custom_prefill(seed=seed, B=s["B"], Hq=s["Hq"], Hkv=s["Hkv"], Nq=s["Nq"],
                                Nk=s["Nk"], d=s["d"], f16=True)
    o, lse = run_prefill16(q, k, v, s["causal"], s["scale"])
    ro, rl = attention_prefill(h64(q), h64(k), h64(v), s["scale"], s["causal"])
    check(f"prefill f16 random seed={seed} {s}", o, lse, ro, rl)


# ------------------------------------------------------------------ FP8 prefill
def run_prefill_fp8(q, k, v, causal, scale, qs, ks, vs):
    t = lambda c: torch.from_numpy(np.ascontiguousarray(c)).cuda()
    o, lse = mi.prefill_fp8(t(q), t(k), t(v), qs, ks, vs, causal, scale)
    torch.cuda.synchronize()
    return o, lse


def fp8_case(seed, B, Hq, Hkv, Nq, Nk, d, q_mult=1.0):
    return ai.custom_prefill(seed=seed, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, q_mult=q_mult,
                             fp8=True)


QS, KS, VS = ai.FP8_Q_SCALE, ai.FP8_K_SCALE, ai.FP8_V_SCALE


@pytest.mark.parametrize("N,Nk,causal,d", [(1, 1, True, 64), (1, 1, False, 128),
                                            (17, 17, False, 128), (65, 65, True, 64),
                                            (129, 300, True, 128), (200, 201, False, 64),
                                            (300, 1000, False, 128), (1000, 1000, True, 128),
                                            (257, 513, True, 64)])
def test_prefill_fp8_shapes(N, Nk, causal, d):
    q, k, v = fp8_case(12000 + N, 1, 2, 2, N, Nk, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_prefill_fp8(q, k, v, causal, scale, QS, KS, VS)
    assert o.dtype == torch.bfloat16
    ro, rl = attention_prefill_fp8(q, k, v, scale, QS, KS, VS, causal)
    check(f"prefill fp8 N={N} Nk={Nk} causal={causal} d={d}", o, lse, ro, rl)


# The bar is absolute, for outputs of unit scale: v_scale stays near FP8_V_SCALE so that the
# dequantised V (and O) keep magnitudes of about 1.  The last set (q_scale = k_scale = 0.1)
# makes scores of tens: it is held to the accumulation bound below, the others to 1e-3.
@pytest.mark.parametrize("scale,qs,ks,vs,large", [(0.125, QS, KS, VS, False),
                                                   (-0.09, 0.02, 0.01, 0.02, False),
                                                   (0.0, QS, KS, VS, False),
                                                   (0.3, 0.05, 0.004, 0.0021, False),
                                                   (0.05, 0.1, 0.1, 0.01, True)])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3)])
def test_prefill_fp8_gqa_and_scales(Hq, Hkv, scale, qs, ks, vs, large):
    q, k, v = fp8_case(12500 + Hq, 3, Hq, Hkv, 190, 260, 128)
    o, lse = run_prefill_fp8(q, k, v, True, scale, qs, ks, vs)
    ro, rl = attention_prefill_fp8(q, k, v, float(np.float32(scale)), float(np.float32(qs)),
                                   float(np.float32(ks)), float(np.float32(vs)), True)
    check(f"prefill fp8 GQA Hq={Hq} Hkv={Hkv} scales={(scale, qs, ks, vs)}", o, lse, ro, rl,
          fp8_lse_tol(q, k, scale, qs, ks) if large else TOL_LSE)


# The FP8 matrix core sums the 64 products of one MFMA with reduced precision: its error
# is at most 2^-11 of the largest product (test_fp8_matrix_core_accumulation_bound pins
# that through the FP8 prefill entry point).  A score therefore carries an error of at most
# (d/64) * 2^-11 * max_d |c q_d k_d| on top of the fp32 path's, which the LSE inherits.  For
# unit-scale scores (the workloads' draws) that is far inside the plain 1e-3 bar, which
# those cases keep; the cases built to have large scores (tens to hundreds) are held to
# 1e-3 plus that bound instead.
def fp8_lse_tol(q, k, scale, qs, ks):
    s32 = lambda x: float(np.float32(x))
    Q = np.abs(s32(qs) * e4m3_value(q)).max(axis=2)     # [B, Hq, d]: max |q_d| of each head
    K = np.abs(s32(ks) * e4m3_value(k)).max(axis=2)     # [B, Hkv, d]
    G = q.shape[1] // k.shape[1]
    maxprod = max(float((Q[b, h] * K[b, h // G]).max())
                  for b in range(q.shape[0]) for h in range(q.shape[1]))
    return TOL_LSE + (q.shape[3] // 64) * 2.0 ** -11 * abs(s32(scale)) * maxprod


def test_prefill_fp8_large_scores_within_the_accumulation_bound():
    q, k, v = fp8_case(12550, 2, 4, 2, 190, 260, 128)
    scale, qs, ks, vs = 0.3, 1.0, 0.004, 0.0021
    o, lse = run_prefill_fp8(q, k, v, True, scale, qs, ks, vs)
    s32 = lambda x: float(np.float32(x))
    ro, rl = attention_prefill_fp8(q, k, v, s32(scale), s32(qs), s32(ks), s32(vs), True)
    assert np.abs(rl).max() > 50          # the scores really are large
    check("prefill fp8 large scores", o, lse, ro, rl, fp8_lse_tol(q, k, scale, qs, ks))


def test_fp8_matrix_core_accumulation_bound():
    # One query and one key per head, non-causal, unit scales: the LSE is then the score
    # q . k exactly as the FP8 matrix core returns it (one MFMA of 64 products at d=64, two
    # accumulated in fp32 at d=128), times log2(e) and then ln 2 in fp32.  Codes are drawn
    # uniformly over every non-NaN E4M3 code for half the heads and as E4M3 roundings of
    # 16*N(0,1) for the other half.
    rng = np.random.default_rng(4242)
    H = 2048
    for d in (64, 128):
        nonnan = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
        uni = rng.choice(nonnan, size=(2, H // 2, d))
        gau = ai.to_e4m3_codes((16 * rng.standard_normal((2, H // 2, d))).astype(np.float32))
        codes = np.concatenate([uni, gau], axis=1)
        q = np.ascontiguousarray(codes[0].reshape(1, H, 1, d))
        k = np.ascontiguousarray(codes[1].reshape(1, H, 1, d))
        v = np.zeros_like(k)
        _, lse = run_prefill_fp8(q, k, v, False, 1.0, 1.0, 1.0, 1.0)
        prod = e4m3_value(q[0, :, 0]) * e4m3_value(k[0, :, 0])          # [H, d], exact
        exact = prod.sum(axis=1)                                         # fp64, exact here
        chunk_max = np.abs(prod.reshape(H, d // 64, 64)).max(axis=2)     # per MFMA
        got = lse.cpu().numpy()[0, :, 0].astype(np.float64)
        err = np.abs(got - exact)
        # 2^-11 of each MFMA's largest product, plus the epilogue's fp32 roundings
        bound = 2.0 ** -11 * chunk_max.sum(axis=1) + 2.0 ** -21 * np.abs(exact)
        rel = err / np.maximum(chunk_max.sum(axis=1), 1e-30)
        log_case(f"fp8 matrix core accumulation d={d}", max_err_over_max_product=float(rel.max()),
                 bound=2.0 ** -11)
        assert (err <= bound).all(), f"d={d}: worst {rel.max():.3e} of the largest product"


def test_prefill_fp8_gqa_equals_repeated_heads_and_is_deterministic():
    q, k, v = fp8_case(12600, 2, 8, 2, 300, 300, 64)
    o, lse = run_prefill_fp8(q, k, v, True, 0.125, QS, KS, VS)
    o2, lse2 = run_prefill_fp8(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), True, 0.125,
                               QS, KS, VS)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o3, lse3 = run_prefill_fp8(q, k, v, True, 0.125, QS, KS, VS)
    assert torch.equal(o, o3) and torch.equal(lse, lse3)


def test_prefill_fp8_peaky_rows():
    # queries scaled by 4 before quantising: rows dominated by a few keys
    q, k, v = fp8_case(12700, 1, 4, 4, 700, 700, 128, q_mult=4.0)
    o, lse = run_prefill_fp8(q, k, v, True, 0.088, QS, KS, VS)
    ro, rl = attention_prefill_fp8(q, k, v, float(np.float32(0.088)), QS, KS, VS, True)
    # queries x4: scores of about 4x the unit-scale workloads' (a large-score case)
    check("prefill fp8 peaky rows", o, lse, ro, rl, fp8_lse_tol(q, k, 0.088, QS, KS))


@pytest.mark.parametrize("seed", list(range(9800, 9808)))
def test_prefill_fp8_random_shapes(seed):
    s = _random_shape(seed)
    q, k, v = fp8_case(seed, s["B"], s["Hq"], s["Hkv"], s["Nq"], s["Nk"], s["d"])
    o, lse = run_prefill_fp8(q, k, v, s["causal"], s["scale"], QS, KS, VS)
    ro, rl = attention_prefill_fp8(q, k, v, s["scale"], QS, KS, VS, s["causal"])
    check(f"prefill fp8 random seed={seed} {s}", o, lse, ro, rl)


def test_prefill_fp8_llama2_shape():
    cfg = ai.CONFIGS["llama2_7b_prefill_fp8"]
    qs, ks, vs = ai.prefill_scales(cfg)
    q, k, v = ai.prefill_inputs(cfg)
    o, lse = run_prefill_fp8(q, k, v, cfg.causal, cfg.scale, qs, ks, vs)
    rng = np.random.default_rng(17)
    go, gl = o.float().cpu().numpy(), lse.cpu().numpy()
    errs, lerrs = [], []
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            full = (b, h) in {(0, 0), (3, 31), (2, 9)}
            rows = np.arange(cfg.Nq) if full else np.unique(np.concatenate(
                [[0, cfg.Nq - 1], rng.integers(0, cfg.Nq, 16)]))
            Q = qs * e4m3_value(q[b, h, rows])
            K, V = ks * e4m3_value(k[b, h]), vs * e4m3_value(v[b, h])
            ro, rl = attention_rows(Q, K, V, cfg.scale, cfg.causal, rows, cfg.Nq)
            errs.append(np.abs(go[b, h, rows] - ro).ravel())
            lerrs.append(np.abs(gl[b, h, rows] - rl).ravel())
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    log_case("llama2_7b_prefill_fp8 (sampled)", max_abs=float(err.max()),
             mean_abs=float(err.mean()), lse_max_abs=float(lerr.max()), n=int(err.size))
    assert np.isfinite(go).all()
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN and lerr.max() <= TOL_LSE


# ------------------------------------------------------------------ FP8 chunked prefill
def make_chunk_fp8(B, Hq, Hkv, d, lens, Nq, seed, extra_pages=3):
    """FP8 chunk queries plus an FP8 paged cache whose unused slots and pages hold the NaN
    code."""
    cfg = ai.DecodeCfg("chunk8", B=B, Hq=Hq, Hkv=Hkv, d=d, seed=seed, paged=True, chunk=Nq,
                       kv_fp8=True)
    lens = np.asarray(lens, np.int32)
    lay = ai.paged_layout(lens, 16, seed, extra_pages=extra_pages)
    return (cfg, ai.chunk_q(cfg), ai.build_paged_cache(cfg, ai.T_K, lens, lay),
            ai.build_paged_cache(cfg, ai.T_V, lens, lay), lens, lay.block_table)


def run_chunk_fp8(q, kc, vc, lens, table, causal, scale, qs=QS, ks=KS, vs=VS):
    t = lambda c: torch.from_numpy(np.ascontiguousarray(c)).cuda()
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    mi.attn_fwd_prefill_paged_fp8(t(q), t(kc), t(vc), t(table), t(lens), o, lse, int(lens.max()),
                                  causal, scale, qs, ks, vs)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Nq,lens", [(1, (1, 17, 300)), (77, (77, 200, 1000)),
                                     (256, (256, 300, 1031)), (300, (300, 301, 700))])
def test_prefill_paged_fp8_chunks(d, causal, Nq, lens):
    cfg, q, kc, vc, lens, table = make_chunk_fp8(3, 4, 2, d, lens, Nq, seed=2400 + Nq + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_chunk_fp8(q, kc, vc, lens, table, causal, scale)
    ro, rl = attention_prefill_paged_fp8(q, kc, vc, table, lens, scale, QS, KS, VS, causal)
    check(f"prefill_paged_fp8 d={d} causal={causal} Nq={Nq} "
          f"lens={tuple(int(x) for x in lens)}", o, lse, ro, rl)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paged_fp8_equals_dense_fp8_prefill(causal):
    # every sequence as long as the chunk (self-attention over the chunk): the paged result
    # equals the dense FP8 prefill of the same codes bit for bit
    B, Hq, Hkv, d, N = 2, 4, 2, 128, 300
    cfg, q, kc, vc, lens, table = make_chunk_fp8(B, Hq, Hkv, d, (N, N), N, seed=2450)
    o, lse = run_chunk_fp8(q, kc, vc, lens, table, causal, 0.09)
    kd = np.stack([np.stack([gather_paged(kc, table, b, h, N, 16) for h in range(Hkv)])
                   for b in range(B)])
    vd = np.stack([np.stack([gather_paged(vc, table, b, h, N, 16) for h in range(Hkv)])
                   for b in range(B)])
    od, ld = run_prefill_fp8(q, kd, vd, causal, 0.09, QS, KS, VS)
    assert torch.equal(o, od) and torch.equal(lse, ld)


def test_chunked_prefill_paged_fp8_config():
    cfg = ai.CONFIGS["chunked_prefill_paged_fp8"]
    lens = ai.decode_lengths(cfg)
    q = ai.chunk_q(cfg)
    lay = ai.paged_layout(lens, 16, cfg.seed)
    kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
    vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
    o, lse = run_chunk_fp8(q, kc, vc, lens, lay.block_table, True, cfg.scale)
    go = o.float().cpu().numpy().astype(np.float64)
    gl = lse.float().cpu().numpy().astype(np.float64)
    G = cfg.Hq // cfg.Hkv
    errs, lerrs = [], []
    for b in range(cfg.B):  # one query head per sequence, every row of it
        h = (5 * b + 3) % cfg.Hq
        kvh = h // G
        n = int(lens[b])
        K = KS * e4m3_value(gather_paged(kc, lay.block_table, b, kvh, n, 16))
        V = VS * e4m3_value(gather_paged(vc, lay.block_table, b, kvh, n, 16))
        rows = np.arange(cfg.chunk)
        ro, rl = attention_rows(QS * e4m3_value(q[b, h]), K, V, cfg.scale, True, rows,
                                cfg.chunk)
        errs.append(np.abs(go[b, h] - ro))
        lerrs.append(np.abs(gl[b, h] - rl))
    err, lerr = np.concatenate([e.ravel() for e in errs]), np.concatenate(lerrs)
    log_case("chunked_prefill_paged_fp8 (sampled)", max_abs=float(err.max()),
             mean_abs=float(err.mean()), lse_max_abs=float(lerr.max()), n=int(err.size))
    assert np.isfinite(go).all()
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN and lerr.max() <= TOL_LSE


# ------------------------------------------------------------------ FP8 varlen prefill
def run_varlen_fp8(q, k, v, cu_q, cu_k, causal, scale):
    t = lambda c: torch.from_numpy(np.ascontiguousarray(c)).cuda()
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device="cuda")
    lq, lk = np.diff(cu_q), np.diff(cu_k)
    mi.attn_fwd_prefill_varlen_fp8(t(q), t(k), t(v), o, lse, t(cu_q), t(cu_k), int(lq.max()),
                                   int(lk.max()), causal, scale, QS, KS, VS)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_varlen_fp8(d, causal):
    lens_k = [1, 300, 77, 513, 64, 2]
    lens_q = [1, 300, 10, 257, 0, 2] if causal else [5, 300, 77, 100, 64, 1]
    q, k, v, cu_q, cu_k = ai.varlen_inputs(13000 + d, lens_q, lens_k, 4, 2, d, fp8=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_varlen_fp8(q, k, v, cu_q, cu_k, causal, scale)
    ro, rl = attention_prefill_varlen_fp8(q, k, v, cu_q, cu_k, scale, QS, KS, VS, causal)
    check(f"prefill_varlen_fp8 d={d} causal={causal}", o, lse, ro, rl)


def test_prefill_varlen_fp8_equals_dense_fp8_prefill():
    # each packed sequence equals the dense FP8 prefill of its own draws, bit for bit
    lens = [300, 129, 1]
    q, k, v, cu_q, cu_k = ai.varlen_inputs(13100, lens, lens, 4, 2, 128, fp8=True)
    o, lse = run_varlen_fp8(q, k, v, cu_q, cu_k, True, 0.09)
    for b, n in enumerate(lens):
        s = slice(cu_q[b], cu_q[b + 1])
        qd = np.ascontiguousarray(q[s].transpose(1, 0, 2))[None]
        kd = np.ascontiguousarray(k[s].transpose(1, 0, 2))[None]
        vd = np.ascontiguousarray(v[s].transpose(1, 0, 2))[None]
        od, ld = run_prefill_fp8(qd, kd, vd, True, 0.09, QS, KS, VS)
        assert torch.equal(o[s], od[0].transpose(0, 1)), b
        assert torch.equal(lse[:, s], ld[0]), b
