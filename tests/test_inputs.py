"""Checks of the seeded input generators and work counting (CPU only)."""
import numpy as np
import pytest
import torch

import attn_inputs as ai


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 3,
                        rng.uniform(-1e30, 1e30, 1000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], np.float32)])
    # exact ties: low 16 bits == 0x8000, with both parities of the kept lsb
    ties = (np.arange(64, dtype=np.uint32) << 17 | 0x3F808000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = ai.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = ai.bf16_bits_to_f64(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_streams_are_deterministic_and_independent():
    a = ai.normal_bf16(5, ai.T_K, 1, 2, (8, 4))
    b = ai.normal_bf16(5, ai.T_K, 1, 2, (8, 4))
    c = ai.normal_bf16(5, ai.T_V, 1, 2, (8, 4))
    np.testing.assert_array_equal(a, b)
    assert (a != c).any()


def test_prefill_q_multiplier_applied_before_rounding():
    cfg = ai.PrefillCfg("t", 1, 1, 1, 4, 4, 8, True, seed=9, q_mult=3.0)
    q = ai.prefill_head(cfg, ai.T_Q, 0, 0)
    x = np.random.default_rng(np.random.SeedSequence([9, ai.T_Q, 0, 0])).standard_normal(
        (4, 8), dtype=np.float32) * np.float32(3.0)
    np.testing.assert_array_equal(q, ai.to_bf16_bits(x))


def test_paged_layout_is_a_partition_of_the_pool():
    lens = np.array([17, 1, 32, 0, 100], np.int32)
    lay = ai.paged_layout(lens, 16, seed=3, extra_pages=3)
    used = []
    for b, n in enumerate(lens):
        nb = (n + 15) // 16
        row = lay.block_table[b]
        assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
        used += row[:nb].tolist()
    assert len(used) == len(set(used)) == sum((n + 15) // 16 for n in lens)
    assert max(used) < lay.num_pages


def test_paged_cache_holds_logical_rows():
    cfg = ai.DecodeCfg("t", B=2, Hq=4, Hkv=2, d=8, seed=11, paged=True, len_range=(3, 40))
    lens = ai.decode_lengths(cfg)
    lay = ai.paged_layout(lens, 16, cfg.seed)
    pool = ai.build_paged_cache(cfg, ai.T_K, lens, lay)
    for b in range(2):
        for h in range(2):
            rows = ai.decode_kv_logical(cfg, ai.T_K, b, h, int(lens[b]))
            for t in range(int(lens[b])):
                np.testing.assert_array_equal(pool[lay.block_table[b, t // 16], h, t % 16], rows[t])


def test_pair_counts_match_the_pages():
    # N^2 counts printed on the page "Flash Attention: GPU 메모리_IO를 최적화하는...",
    # section "왜 Flash Attention이 필요한가?": 512 tokens -> about 262,000 weights,
    # 4096 tokens -> about 16,000,000.
    assert ai.visible_pairs(512, 512, False) == 262_144
    assert abs(ai.visible_pairs(4096, 4096, False) - 16_000_000) / 16e6 < 0.05
    # causal: 1 + 2 + ... + N
    assert ai.visible_pairs(512, 512, True) == 512 * 513 // 2
    assert ai.visible_pairs(3, 10, True) == 8 + 9 + 10
    with pytest.raises(ValueError):
        ai.visible_pairs(4, 3, True)


def test_config_work_figures():
    c1 = ai.CONFIGS["tiny_prefill"]
    assert ai.prefill_flops(c1) == 4 * 64 * 4 * 131_328
    c2 = ai.CONFIGS["llama2_7b_prefill"]
    assert ai.prefill_flops(c2) == 137_506_062_336
    assert ai.prefill_flops(ai.CONFIGS["llama2_7b_prefill_noncausal"]) == 274_877_906_944
    assert ai.prefill_flops(ai.CONFIGS["long_prefill_32k"]) == 8_796_361_457_664
    c4 = ai.CONFIGS["gqa_decode_contig"]
    assert ai.decode_bytes(c4, ai.decode_lengths(c4)) == 2_148_540_672


# ----------------------------------------------------------------------------- FP8 E4M3 codes
def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(400_000) * np.exp(rng.uniform(-14, 7, 400_000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    np.testing.assert_array_equal(ai.to_e4m3_codes(x), _torch_e4m3(x))
    # exact midpoints between neighbouring finite codes: ties go to the even code
    vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mid = (vals[:-1] + vals[1:]) / 2
    assert (mid.astype(np.float32).astype(np.float64) == mid).all()
    both = np.concatenate([mid, -mid]).astype(np.float32)
    codes = ai.to_e4m3_codes(both)
    np.testing.assert_array_equal(codes, _torch_e4m3(both))
    assert (codes % 2 == 0).all()


def test_e4m3_saturates_and_keeps_signed_zero():
    x = np.array([448.0, 460.0, 1e6, -1e6, 0.0, -0.0, 2.0 ** -10, 2.0 ** -9], np.float32)
    np.testing.assert_array_equal(ai.to_e4m3_codes(x),
                                  np.array([0x7E, 0x7E, 0x7E, 0xFE, 0, 0x80, 0, 1], np.uint8))


def test_fp8_cache_quantises_the_bf16_workload_draws():
    cfg = ai.DecodeCfg("t", B=2, Hq=4, Hkv=2, d=8, seed=11, paged=True, len_range=(3, 40),
                       kv_fp8=True)
    lens = ai.decode_lengths(cfg)
    rows = ai.decode_kv_logical(cfg, ai.T_V, 1, 1, int(lens[1]))
    x = np.random.default_rng(np.random.SeedSequence([11, ai.T_V, 1, 1])).standard_normal(
        (int(lens[1]), 8), dtype=np.float32)
    assert rows.dtype == np.uint8
    np.testing.assert_array_equal(rows, _torch_e4m3(x / np.float32(ai.FP8_V_SCALE)))
    lay = ai.paged_layout(lens, 16, cfg.seed)
    pool = ai.build_paged_cache(cfg, ai.T_V, lens, lay)
    assert pool.dtype == np.uint8
    for t in range(int(lens[1])):
        np.testing.assert_array_equal(pool[lay.block_table[1, t // 16], 1, t % 16], rows[t])
    # unused slots of a partly filled page hold the E4M3 NaN code
    n = int(lens[1])
    if n % 16:
        assert (pool[lay.block_table[1, n // 16], 1, n % 16:] == 0x7F).all()
    assert ai.kv_scale(cfg, ai.T_K) == ai.FP8_K_SCALE != ai.FP8_V_SCALE
    base = ai.CONFIGS["paged_gqa_decode"]
    f8 = ai.CONFIGS["paged_gqa_decode_fp8"]
    np.testing.assert_array_equal(ai.decode_lengths(base), ai.decode_lengths(f8))
    lb = ai.decode_lengths(base)
    kv = 2 * int(lb.sum()) * base.Hkv * base.d
    assert ai.decode_bytes(base, lb) - ai.decode_bytes(f8, lb) == kv


def test_fp8_prefill_quantises_the_bf16_workload_draws():
    base = ai.PrefillCfg("t", B=1, Hq=2, Hkv=1, Nq=40, Nk=56, d=8, causal=True, seed=12,
                         q_mult=2.0)
    f8 = ai.PrefillCfg("t", B=1, Hq=2, Hkv=1, Nq=40, Nk=56, d=8, causal=True, seed=12,
                       q_mult=2.0, fp8=True)
    qs, ks, vs = ai.prefill_scales(f8)
    assert (qs, ks, vs) == (ai.FP8_Q_SCALE, ai.FP8_K_SCALE, ai.FP8_V_SCALE)
    assert ai.prefill_scales(base) == (1.0, 1.0, 1.0)
    q, k, v = ai.prefill_inputs(f8)
    assert q.dtype == k.dtype == v.dtype == np.uint8
    draw = lambda t, h, n, m=1.0: np.random.default_rng(np.random.SeedSequence(
        [12, t, 0, h])).standard_normal((n, 8), dtype=np.float32) * np.float32(m)
    np.testing.assert_array_equal(q[0, 1], _torch_e4m3(draw(ai.T_Q, 1, 40, 2.0) / np.float32(qs)))
    np.testing.assert_array_equal(k[0, 0], _torch_e4m3(draw(ai.T_K, 0, 56) / np.float32(ks)))
    np.testing.assert_array_equal(v[0, 0], _torch_e4m3(draw(ai.T_V, 0, 56) / np.float32(vs)))
    # one byte per input element, two per output element
    full = ai.CONFIGS["llama2_7b_prefill_fp8"]
    elems = full.B * full.Hq * full.Nq * full.d
    assert ai.prefill_bytes(full) == 3 * elems + 2 * elems + full.B * full.Hq * full.Nq * 4
    assert ai.prefill_flops(full) == ai.prefill_flops(ai.CONFIGS["llama2_7b_prefill"])


def test_fp8_chunk_queries_quantise_the_bf16_chunk_draws():
    base = ai.CONFIGS["chunked_prefill_paged"]
    f8 = ai.CONFIGS["chunked_prefill_paged_fp8"]
    np.testing.assert_array_equal(ai.decode_lengths(base), ai.decode_lengths(f8))
    small = ai.DecodeCfg("t", B=2, Hq=2, Hkv=1, d=8, seed=13, paged=True, chunk=5, kv_fp8=True)
    q = ai.chunk_q(small)
    assert q.dtype == np.uint8 and q.shape == (2, 2, 5, 8)
    x = np.random.default_rng(np.random.SeedSequence([13, ai.T_Q, 1, 0])).standard_normal(
        (5, 8), dtype=np.float32)
    np.testing.assert_array_equal(q[1, 0], _torch_e4m3(x / np.float32(ai.FP8_Q_SCALE)))


def test_fp8_varlen_inputs_pack_the_dense_fp8_streams():
    q, k, v, cu_q, cu_k = ai.varlen_inputs(14, [5, 9], [7, 9], 2, 1, 8, fp8=True)
    assert q.dtype == k.dtype == v.dtype == np.uint8
    cfg = ai.PrefillCfg("t", 1, 2, 1, 9, 9, 8, True, 14, fp8=True)
    dq, dk, dv = ai.prefill_inputs(cfg)
    # sequence 1 has 9 query and 9 key rows: batch index 1 of the streams
    np.testing.assert_array_equal(q[5:14, 1], ai.normal_e4m3(14, ai.T_Q, 1, 1, (9, 8), ai.FP8_Q_SCALE))
    np.testing.assert_array_equal(k[7:16, 0], ai.normal_e4m3(14, ai.T_K, 1, 0, (9, 8), ai.FP8_K_SCALE))
    np.testing.assert_array_equal(v[0:7, 0], ai.normal_e4m3(14, ai.T_V, 0, 0, (7, 8), ai.FP8_V_SCALE))
    np.testing.assert_array_equal(dq[0, 0], ai.normal_e4m3(14, ai.T_Q, 0, 0, (9, 8), ai.FP8_Q_SCALE))


# ----------------------------------------------------------------------------- fp16 rounding
def test_f16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 3,
                        rng.uniform(-6e4, 6e4, 1000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-6).astype(np.float32),  # subnormals
                        np.array([0.0, -0.0, 1.0, 65504.0, 2.0 ** -24], np.float32)])
    # exact ties halfway between neighbouring fp16 values, both parities of the kept bit
    ties = ((np.arange(64, dtype=np.uint32) << 13) | np.uint32(0x3F801000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = ai.to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(ai.f16_bits_to_f64(ours),
                                  torch.from_numpy(x).to(torch.float16).double().numpy())


def test_f16_variant_rounds_the_same_draws():
    a16 = ai.normal_bf16(5, ai.T_K, 1, 2, (8, 4), f16=True)
    x = np.random.default_rng(np.random.SeedSequence([5, ai.T_K, 1, 2])).standard_normal(
        (8, 4), dtype=np.float32)
    np.testing.assert_array_equal(a16, ai.to_f16_bits(x))
    cfg = ai.CONFIGS["llama2_7b_prefill_f16"]
    assert cfg.f16 and cfg.seed == ai.CONFIGS["llama2_7b_prefill"].seed
    q16 = ai.prefill_head(cfg, ai.T_Q, 0, 3)
    q = ai.prefill_head(ai.CONFIGS["llama2_7b_prefill"], ai.T_Q, 0, 3)
    # the two roundings of one draw differ by at most half a bf16 ulp plus half an fp16 ulp
    d = np.abs(ai.f16_bits_to_f64(q16) - ai.bf16_bits_to_f64(q))
    assert (d <= np.abs(ai.bf16_bits_to_f64(q)) * (2.0 ** -8 + 2.0 ** -11) + 2.0 ** -24).all()
    dc = ai.DecodeCfg("t", B=1, Hq=2, Hkv=1, d=8, seed=3, paged=False, fixed_len=5, f16=True)
    assert (ai.build_contig_cache(dc, ai.T_K, np.array([3], np.int32), 5)[0, 0, 3:]
            == ai.F16_NAN).all()


def test_varlen_inputs_pack_the_dense_streams():
    q, k, v, cu_q, cu_k = ai.varlen_inputs(9, [3, 0, 5], [4, 2, 6], 4, 2, 8)
    assert q.shape == (8, 4, 8) and k.shape == (12, 2, 8)
    assert cu_q.tolist() == [0, 3, 3, 8] and cu_k.tolist() == [0, 4, 6, 12]
    np.testing.assert_array_equal(q[3:8, 1], ai.normal_bf16(9, ai.T_Q, 2, 1, (5, 8)))
    np.testing.assert_array_equal(v[4:6, 0], ai.normal_bf16(9, ai.T_V, 1, 0, (2, 8)))
    q16, k16, _, _, _ = ai.varlen_inputs(9, [3, 0, 5], [4, 2, 6], 4, 2, 8, f16=True)
    np.testing.assert_array_equal(k16[6:12, 1], ai.normal_bf16(9, ai.T_K, 2, 1, (6, 8), f16=True))
    assert not np.array_equal(q16, q)
    lens = ai.varlen_lengths(8, 16, 256, 4096)
    assert lens.shape == (16,) and lens.min() >= 256 and lens.max() <= 4096
    assert ai.varlen_flops([2, 3], [2, 5], 1, 1, True) == 4 * (3 + 3 + 4 + 5)
