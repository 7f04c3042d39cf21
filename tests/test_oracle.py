"""Pins for the CPU oracle: brute force, closed forms, invariants (CPU only).

Each test checks the oracle against something other than itself, chosen so that a
plausible slip (a dropped term, a wrong sign or index, a transposed operand, a
mis-aligned causal mask, a wrong head mapping) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_decode, attention_prefill, attention_prefill_paged,
                    attention_probabilities, attention_rows, brute_force_attention,
                    merge_partials, online_attention, softmax_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("Nq,Nk,d,causal", [
    (1, 1, 1, False), (3, 5, 2, False), (5, 5, 3, True), (4, 7, 4, True), (8, 8, 4, True),
    (2, 8, 3, False), (6, 6, 1, True)])
def test_matches_brute_force(Nq, Nk, d, causal):
    q, k, v = rnd(1, Nq, d), rnd(2, Nk, d), rnd(3, Nk, d)
    scale = 0.7
    o, lse = attention_prefill(q[None, None], k[None, None], v[None, None], scale, causal)
    bo, bl = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=0, atol=1e-12)


def test_brute_force_batched_gqa():
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 3, 6, 2
    q, k, v = rnd(4, B, Hq, Nq, d), rnd(5, B, Hkv, Nk, d), rnd(6, B, Hkv, Nk, d)
    o, lse = attention_prefill(q, k, v, 0.5, True)
    for b in range(B):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            bo, bl = brute_force_attention(q[b, h].tolist(), k[b, kvh].tolist(),
                                           v[b, kvh].tolist(), 0.5, True)
            np.testing.assert_allclose(o[b, h], bo, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[b, h], bl, atol=1e-12, rtol=0)


def test_row_blocking_does_not_change_result():
    q, k, v = rnd(7, 1, 2, 37, 4), rnd(8, 1, 2, 37, 4), rnd(9, 1, 2, 37, 4)
    a = attention_prefill(q, k, v, 0.3, True, row_block=1024)
    b = attention_prefill(q, k, v, 0.3, True, row_block=5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- worked example
def test_worked_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    o, lse = attention_prefill(q, k, v, g["scale"], False)
    assert abs(o[0, 0, 0, 0] - g["expected_o"][0][0]) <= g["tolerance"] * 4
    assert abs(lse[0, 0, 0] - g["expected_lse"][0]) <= g["tolerance"] * 2


# ----------------------------------------------------------------------------- closed forms
def test_single_key_returns_that_value():
    q, k, v = rnd(10, 1, 1, 1, 8), rnd(11, 1, 1, 1, 8), rnd(12, 1, 1, 1, 8)
    o, lse = attention_prefill(q, k, v, 0.25, False)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])
    assert lse[0, 0, 0] == pytest.approx(0.25 * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_mean_of_visible_values(causal):
    Nq, Nk, d = 6, 9, 3
    q, k, v = rnd(13, Nq, d), rnd(14, Nk, d), rnd(15, Nk, d)
    o, lse = attention_prefill(q[None, None], k[None, None], v[None, None], 0.0, causal)
    for i in range(Nq):
        n = (i + Nk - Nq + 1) if causal else Nk
        np.testing.assert_allclose(o[0, 0, i], v[:n].mean(axis=0), atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_key_rows_give_uniform_weights(causal):
    Nq, Nk, d = 5, 8, 4
    q, v = rnd(16, Nq, d), rnd(17, Nk, d)
    krow = rnd(18, d)
    k = np.tile(krow, (Nk, 1))
    scale = 0.9
    o, lse = attention_prefill(q[None, None], k[None, None], v[None, None], scale, causal)
    for i in range(Nq):
        n = (i + Nk - Nq + 1) if causal else Nk
        np.testing.assert_allclose(o[0, 0, i], v[:n].mean(axis=0), atol=1e-13)
        assert lse[0, 0, i] == pytest.approx(scale * q[i] @ krow + math.log(n), abs=1e-13)


# ----------------------------------------------------------------------------- causal mask
def test_causal_first_row_is_first_value():
    N, d = 16, 8
    q, k, v = rnd(19, N, d), rnd(20, N, d), rnd(21, N, d)
    o, lse = attention_prefill(q[None, None], k[None, None], v[None, None], 0.4, True)
    np.testing.assert_array_equal(o[0, 0, 0], v[0])
    assert lse[0, 0, 0] == pytest.approx(0.4 * q[0] @ k[0], abs=1e-15)


def test_causal_row_i_is_noncausal_over_prefix():
    N, d = 12, 5
    q, k, v = rnd(22, N, d), rnd(23, N, d), rnd(24, N, d)
    o, lse = attention_prefill(q[None, None], k[None, None], v[None, None], 0.6, True)
    for i in range(N):
        bo, bl = brute_force_attention([q[i].tolist()], k[:i + 1].tolist(), v[:i + 1].tolist(),
                                       0.6, False)
        np.testing.assert_allclose(o[0, 0, i], bo[0], atol=1e-12)
        assert lse[0, 0, i] == pytest.approx(bl[0], abs=1e-12)


def test_causal_bottom_right_alignment():
    # Nq < Nk: the last query row sees every key, the first sees Nk - Nq + 1 keys.
    Nq, Nk, d = 3, 10, 4
    q, k, v = rnd(25, Nq, d), rnd(26, Nk, d), rnd(27, Nk, d)
    o, _ = attention_prefill(q[None, None], k[None, None], v[None, None], 0.5, True)
    full, _ = attention_prefill(q[None, None], k[None, None], v[None, None], 0.5, False)
    np.testing.assert_allclose(o[0, 0, -1], full[0, 0, -1], atol=1e-14)
    first, _ = attention_rows(q[:1], k[:Nk - Nq + 1], v[:Nk - Nq + 1], 0.5, False,
                              np.arange(1), 1)
    np.testing.assert_allclose(o[0, 0, 0], first[0], atol=1e-14)


def test_causal_rejects_more_queries_than_keys():
    with pytest.raises(ValueError):
        attention_prefill(rnd(1, 1, 1, 4, 2), rnd(2, 1, 1, 3, 2), rnd(3, 1, 1, 3, 2), 1.0, True)


# ----------------------------------------------------------------------------- softmax invariants
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k = rnd(28, 9, 4), rnd(29, 9, 4)
    p = attention_probabilities(q, k, 1.3, causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert (p >= 0).all()
    if causal:
        assert (np.triu(p, 1) == 0).all()


def test_constant_values_give_constant_output():
    q, k = rnd(30, 1, 1, 7, 4), rnd(31, 1, 1, 7, 4)
    vrow = rnd(32, 4)
    v = np.tile(vrow, (1, 1, 7, 1))
    for causal in (False, True):
        o, _ = attention_prefill(q, k, v, 0.8, causal)
        np.testing.assert_allclose(o[0, 0], np.tile(vrow, (7, 1)), atol=1e-14)


def test_score_shift_invariance():
    s = rnd(33, 4, 6)
    c = rnd(34, 4)[:, None] * 50.0
    p0, m0, l0 = softmax_rows(s)
    p1, m1, l1 = softmax_rows(s + c)
    np.testing.assert_allclose(p1, p0, atol=1e-14)
    np.testing.assert_allclose(m1 + np.log(l1), m0 + np.log(l0) + c[:, 0], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    # Adding u to every key row adds scale * q.u to a whole score row.
    q, k, v = rnd(35, 6, 4), rnd(36, 6, 4), rnd(37, 6, 4)
    u = rnd(38, 4)
    scale = 0.7
    o0, l0 = attention_prefill(q[None, None], k[None, None], v[None, None], scale, causal)
    o1, l1 = attention_prefill(q[None, None], (k + u)[None, None], v[None, None], scale, causal)
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(l1[0, 0], l0[0, 0] + scale * q @ u, atol=1e-13)


def test_lse_bounds_and_convex_hull():
    Nq, Nk, d = 8, 11, 3
    q, k, v = rnd(39, Nq, d), rnd(40, Nk, d), rnd(41, Nk, d)
    scale = 1.1
    for causal in (False, True):
        o, lse = attention_prefill(q[None, None], k[None, None], v[None, None], scale, causal)
        for i in range(Nq):
            n = (i + Nk - Nq + 1) if causal else Nk
            s = scale * (k[:n] @ q[i])
            assert s.max() - 1e-12 <= lse[0, 0, i] <= s.max() + math.log(n) + 1e-12
            assert (o[0, 0, i] >= v[:n].min(axis=0) - 1e-12).all()
            assert (o[0, 0, i] <= v[:n].max(axis=0) + 1e-12).all()


def test_noncausal_key_permutation_equivariance():
    q, k, v = rnd(42, 5, 4), rnd(43, 9, 4), rnd(44, 9, 4)
    perm = np.random.default_rng(45).permutation(9)
    o0, l0 = attention_prefill(q[None, None], k[None, None], v[None, None], 0.5, False)
    o1, l1 = attention_prefill(q[None, None], k[perm][None, None], v[perm][None, None], 0.5, False)
    np.testing.assert_allclose(o1, o0, atol=1e-14)
    np.testing.assert_allclose(l1, l0, atol=1e-14)


def test_swapping_k_and_v_roles_is_detected():
    # A transposed operand (using V where K belongs) must change the result.
    q, k, v = rnd(46, 4, 4), rnd(47, 6, 4), rnd(48, 6, 4)
    o, _ = attention_prefill(q[None, None], k[None, None], v[None, None], 0.5, False)
    bad, _ = attention_prefill(q[None, None], v[None, None], k[None, None], 0.5, False)
    assert np.abs(o - bad).max() > 1e-3


# ----------------------------------------------------------------------------- online recurrence
@pytest.mark.parametrize("causal", [False, True])
def test_online_one_block_equals_two_pass(causal):
    q, k, v = rnd(49, 10, 4), rnd(50, 10, 4), rnd(51, 10, 4)
    o2, l2 = attention_prefill(q[None, None], k[None, None], v[None, None], 0.9, causal)
    o1, l1 = online_attention(q, k, v, 0.9, causal, block=10)
    np.testing.assert_allclose(o1, o2[0, 0], atol=1e-15, rtol=0)
    np.testing.assert_allclose(l1, l2[0, 0], atol=1e-15, rtol=0)


@pytest.mark.parametrize("block", [1, 3, 4, 7, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_online_many_blocks_equals_two_pass(block, causal):
    Nq, Nk = 9, 13
    q, k, v = rnd(52, Nq, 5) * 3, rnd(53, Nk, 5), rnd(54, Nk, 5)
    o2, l2 = attention_prefill(q[None, None], k[None, None], v[None, None], 0.8, causal)
    o1, l1 = online_attention(q, k, v, 0.8, causal, block=block)
    np.testing.assert_allclose(o1, o2[0, 0], atol=1e-12)
    np.testing.assert_allclose(l1, l2[0, 0], atol=1e-12)


# ----------------------------------------------------------------------------- GQA
def test_gqa_equals_repeated_heads():
    B, Hq, Hkv, N, d = 2, 6, 2, 7, 4
    q, k, v = rnd(55, B, Hq, N, d), rnd(56, B, Hkv, N, d), rnd(57, B, Hkv, N, d)
    o, lse = attention_prefill(q, k, v, 0.5, True)
    G = Hq // Hkv
    o2, lse2 = attention_prefill(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.5, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # a wrong mapping (h % Hkv) gives a different answer on these inputs
    o3, _ = attention_prefill(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), 0.5, True)
    assert np.abs(o3 - o).max() > 1e-3


# ----------------------------------------------------------------------------- decode
def _decode_case(seed=60, B=3, Hq=4, Hkv=2, d=4, lens=(5, 1, 9), ps=4):
    rng = np.random.default_rng(seed)
    Nmax = max(lens)
    q = rng.standard_normal((B, Hq, d))
    kc = np.full((B, Hkv, Nmax + 2, d), np.nan)
    vc = np.full((B, Hkv, Nmax + 2, d), np.nan)
    for b, n in enumerate(lens):
        kc[b, :, :n] = rng.standard_normal((Hkv, n, d))
        vc[b, :, :n] = rng.standard_normal((Hkv, n, d))
    return q, kc, vc, np.array(lens, np.int32)


def _to_paged(kc, lens, ps, perm_seed):
    B, Hkv, _, d = kc.shape
    nblk = [(n + ps - 1) // ps for n in lens]
    P = sum(nblk) + 2
    perm = np.random.default_rng(perm_seed).permutation(P)
    table = np.full((B, max(nblk)), -1, np.int32)
    pad = 0x7F if kc.dtype == np.uint8 else np.nan   # never-read slots hold NaN
    pool = np.full((P, Hkv, ps, d), pad, kc.dtype)
    off = 0
    for b, n in enumerate(lens):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
        for t in range(n):
            pool[table[b, t // ps], :, t % ps] = kc[b, :, t]
    return pool, table


def test_decode_matches_brute_force_and_ignores_padding():
    q, kc, vc, lens = _decode_case()
    o, lse = attention_decode(q, kc, vc, lens, 0.5)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for b, n in enumerate(lens):
        for h in range(4):
            kvh = h // 2
            bo, bl = brute_force_attention([q[b, h].tolist()], kc[b, kvh, :n].tolist(),
                                           vc[b, kvh, :n].tolist(), 0.5, False)
            np.testing.assert_allclose(o[b, h], bo[0], atol=1e-12)
            assert lse[b, h] == pytest.approx(bl[0], abs=1e-12)


def test_decode_is_last_row_of_causal_prefill():
    rng = np.random.default_rng(61)
    n, d = 11, 4
    Q, K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    op, lp = attention_prefill(Q[None, None], K[None, None], V[None, None], 0.7, True)
    od, ld = attention_decode(Q[-1][None, None], K[None, None], V[None, None],
                              np.array([n], np.int32), 0.7)
    np.testing.assert_allclose(od[0, 0], op[0, 0, -1], atol=1e-14)
    assert ld[0, 0] == pytest.approx(lp[0, 0, -1], abs=1e-14)
    # bottom-right: one causal query against n keys is the decode row too
    o1, l1 = attention_prefill(Q[-1][None, None, None], K[None, None], V[None, None], 0.7, True)
    np.testing.assert_allclose(o1[0, 0, 0], od[0, 0], atol=1e-14)


def test_paged_equals_contiguous_and_page_order_is_irrelevant():
    q, kc, vc, lens = _decode_case(seed=62, lens=(7, 4, 13))
    o0, l0 = attention_decode(q, kc, vc, lens, 0.6)
    for seed in (1, 2):
        kp, table = _to_paged(kc, lens, 4, seed)
        vp, table2 = _to_paged(vc, lens, 4, seed)
        assert (table == table2).all()
        o1, l1 = attention_decode(q, kp, vp, lens, 0.6, block_table=table, page_size=4)
        np.testing.assert_array_equal(o1, o0)
        np.testing.assert_array_equal(l1, l0)


def test_decode_zero_length():
    q, kc, vc, _ = _decode_case()
    o, lse = attention_decode(q, kc, vc, np.array([0, 1, 0], np.int32), 0.5)
    assert (o[0] == 0).all() and (lse[0] == -np.inf).all()
    assert (o[2] == 0).all() and np.isfinite(lse[1]).all()


# ----------------------------------------------------------------------------- split + merge
def test_merge_of_halves_equals_full_row():
    rng = np.random.default_rng(63)
    q, k, v = rng.standard_normal((1, 6)), rng.standard_normal((20, 6)), rng.standard_normal((20, 6))
    full_o, full_l = attention_rows(q, k, v, 0.4, False, np.arange(1), 1)
    for cuts in ([7], [1, 19], [3, 9, 15]):
        edges = [0] + cuts + [20]
        parts = [attention_rows(q, k[a:b], v[a:b], 0.4, False, np.arange(1), 1)
                 for a, b in zip(edges[:-1], edges[1:])]
        o, l = merge_partials(np.stack([p[0][0] for p in parts]), np.array([p[1][0] for p in parts]))
        np.testing.assert_allclose(o, full_o[0], atol=1e-14)
        assert l == pytest.approx(full_l[0], abs=1e-13)


def test_merge_with_empty_split_is_identity():
    o = np.array([[1.0, 2.0], [9.0, 9.0]])
    r, l = merge_partials(o, np.array([0.3, -np.inf]))
    np.testing.assert_array_equal(r, o[0])
    assert l == 0.3
    r, l = merge_partials(o, np.array([-np.inf, -np.inf]))
    assert (r == 0).all() and l == -np.inf


# ----------------------------------------------------------- chunked prefill, paged cache
def _chunk_case(seed=70, B=3, Hq=4, Hkv=2, d=4, lens=(9, 5, 14), Nq=5, ps=4):
    q_full, kc, vc, lens = _decode_case(seed=seed, B=B, Hq=Hq, Hkv=Hkv, d=d, lens=lens, ps=ps)
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((B, Hq, Nq, d))
    return q, kc, vc, lens


@pytest.mark.parametrize("causal", [False, True])
def test_chunk_rows_equal_bottom_rows_of_full_prefill(causal):
    # the chunk's queries are the last Nq tokens: their rows of a full prefill over the
    # whole sequence (queries for every position) must equal the chunked result
    q, kc, vc, lens = _chunk_case()
    kp, table = _to_paged(kc, lens, 4, 3)
    vp, _ = _to_paged(vc, lens, 4, 3)
    o, lse = attention_prefill_paged(q, kp, vp, table, lens, 0.8, causal, page_size=4)
    rng = np.random.default_rng(5)
    Nq = q.shape[2]
    for b, n in enumerate(lens):
        qf = rng.standard_normal((1, 4, n, 4))
        qf[0, :, n - Nq:] = q[b]
        of, lf = attention_prefill(qf, kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], 0.8, causal)
        np.testing.assert_allclose(o[b], of[0, :, n - Nq:], atol=1e-13)
        np.testing.assert_allclose(lse[b], lf[0, :, n - Nq:], atol=1e-13)


def test_chunk_last_row_is_paged_decode():
    q, kc, vc, lens = _chunk_case(seed=72)
    kp, table = _to_paged(kc, lens, 4, 4)
    vp, _ = _to_paged(vc, lens, 4, 4)
    o, lse = attention_prefill_paged(q, kp, vp, table, lens, 0.6, True, page_size=4)
    od, ld = attention_decode(q[:, :, -1], kp, vp, lens, 0.6, block_table=table, page_size=4)
    np.testing.assert_allclose(o[:, :, -1], od, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, -1], ld, atol=1e-14)


def test_chunk_first_row_of_a_whole_sequence_is_first_value():
    # kv_lens == Nq: the chunk is the whole sequence and causal row 0 sees key 0 only
    q, kc, vc, _ = _chunk_case(seed=74)
    lens = np.array([5, 5, 5], np.int32)
    kp, table = _to_paged(kc, lens, 4, 5)
    vp, _ = _to_paged(vc, lens, 4, 5)
    o, lse = attention_prefill_paged(q, kp, vp, table, lens, 0.9, True, page_size=4)
    for b in range(3):
        for h in range(4):
            np.testing.assert_array_equal(o[b, h, 0], vc[b, h // 2, 0])
            assert lse[b, h, 0] == pytest.approx(0.9 * q[b, h, 0] @ kc[b, h // 2, 0], abs=1e-14)


def test_chunk_equal_keys_give_mean_of_visible_values():
    q, kc, vc, lens = _chunk_case(seed=76)
    Nq = q.shape[2]
    kc[:] = np.where(np.isnan(kc), np.nan, 0.25)  # every live key row equal
    kp, table = _to_paged(kc, lens, 4, 6)
    vp, _ = _to_paged(vc, lens, 4, 6)
    o, lse = attention_prefill_paged(q, kp, vp, table, lens, 1.0, True, page_size=4)
    for b, n in enumerate(lens):
        for h in range(4):
            for i in range(Nq):
                vis = n - Nq + i + 1
                np.testing.assert_allclose(o[b, h, i], vc[b, h // 2, :vis].mean(axis=0), atol=1e-13)
                assert lse[b, h, i] == pytest.approx(q[b, h, i].sum() * 0.25 + math.log(vis),
                                                     abs=1e-13)


def test_chunk_page_order_is_irrelevant_and_padding_unread():
    q, kc, vc, lens = _chunk_case(seed=78)
    outs = []
    for seed in (7, 8):
        kp, table = _to_paged(kc, lens, 4, seed)
        vp, _ = _to_paged(vc, lens, 4, seed)
        outs.append(attention_prefill_paged(q, kp, vp, table, lens, 0.5, True, page_size=4))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    assert np.isfinite(outs[0][0]).all()


def test_chunk_rejects_context_shorter_than_chunk():
    q, kc, vc, lens = _chunk_case(seed=80)
    kp, table = _to_paged(kc, lens, 4, 9)
    vp, _ = _to_paged(vc, lens, 4, 9)
    with pytest.raises(ValueError):
        attention_prefill_paged(q, kp, vp, table, np.array([4, 5, 14], np.int32), 0.5, True,
                                page_size=4)


# ----------------------------------------------------------------------------- FP8 KV cache
def test_e4m3_values_match_torch_for_every_code():
    import torch
    from oracle import e4m3_value
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert (np.isnan(ours) == np.isnan(ref)).all()
    assert np.flatnonzero(np.isnan(ours)).tolist() == [0x7F, 0xFF]
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    assert (np.signbit(ours[fin]) == np.signbit(ref[fin])).all()


def test_e4m3_closed_forms():
    from oracle import e4m3_value
    cases = {0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x08: 2.0 ** -6, 0x3C: 1.5, 0x40: 2.0, 0x00: 0.0, 0x77: 240.0}
    got = e4m3_value(np.array(list(cases), np.uint8))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    assert np.signbit(e4m3_value(np.array([0x80], np.uint8)))[0]
    # every finite code is a round trip through the (independent) input encoder
    import attn_inputs as ai
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    np.testing.assert_array_equal(ai.to_e4m3_codes(e4m3_value(codes).astype(np.float32)), codes)


def _fp8_case(seed, B=3, Hq=4, Hkv=2, d=5, lens=(6, 0, 9)):
    rng = np.random.default_rng(seed)
    nmax = max(lens)
    q = rng.standard_normal((B, Hq, d))
    codes = [c for c in range(256) if c & 0x7F != 0x7F]
    kc = rng.choice(codes, (B, Hkv, nmax + 2, d)).astype(np.uint8)
    vc = rng.choice(codes, (B, Hkv, nmax + 2, d)).astype(np.uint8)
    for b, n in enumerate(lens):       # slots past the length hold the NaN code
        kc[b, :, n:] = 0x7F
        vc[b, :, n:] = 0xFF
    return q, kc, vc, np.array(lens, np.int32)


def test_fp8_decode_matches_brute_force_on_torch_dequantised_cache():
    import torch
    from oracle import attention_decode_fp8
    q, kc, vc, lens = _fp8_case(71)
    ks, vs = 0.0173, 0.031
    o, lse = attention_decode_fp8(q, kc, vc, lens, 0.45, ks, vs)
    deq = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    assert (o[1] == 0).all() and (lse[1] == -np.inf).all()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        for h in range(4):
            K = (ks * deq(kc[b, h // 2, :n])).tolist()
            V = (vs * deq(vc[b, h // 2, :n])).tolist()
            bo, bl = brute_force_attention([q[b, h].tolist()], K, V, 0.45, False)
            np.testing.assert_allclose(o[b, h], bo[0], rtol=1e-12, atol=1e-14)
            assert lse[b, h] == pytest.approx(bl[0], abs=1e-12)


def test_fp8_scales_fold_into_the_softmax_scale_and_the_output():
    from oracle import attention_decode_fp8
    q, kc, vc, lens = _fp8_case(72)
    o0, l0 = attention_decode_fp8(q, kc, vc, lens, 0.3 * 0.02, 1.0, 1.0)
    o1, l1 = attention_decode_fp8(q, kc, vc, lens, 0.3, 0.02, 1.0)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=1e-12, atol=1e-13)
    o2, l2 = attention_decode_fp8(q, kc, vc, lens, 0.3, 0.02, 0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(l2, l1)
    # the two scales are not interchangeable
    o3, _ = attention_decode_fp8(q, kc, vc, lens, 0.3, 0.125, 0.02)
    assert np.abs(o3 - o2).max() > 1e-3


def test_fp8_paged_equals_contiguous():
    from oracle import attention_decode_fp8
    q, kc, vc, lens = _fp8_case(73, lens=(7, 4, 13))
    o0, l0 = attention_decode_fp8(q, kc, vc, lens, 0.6, 0.05, 0.07)
    kp, table = _to_paged(kc, lens, 4, 3)
    vp, _ = _to_paged(vc, lens, 4, 3)
    o1, l1 = attention_decode_fp8(q, kp, vp, lens, 0.6, 0.05, 0.07, block_table=table,
                                  page_size=4)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)


# ----------------------------------------------------------------------------- FP8 prefill
def _fp8_prefill_case(seed, B=2, Hq=4, Hkv=2, Nq=5, Nk=7, d=3):
    rng = np.random.default_rng(seed)
    codes = [c for c in range(256) if c & 0x7F != 0x7F]
    qc = rng.choice(codes, (B, Hq, Nq, d)).astype(np.uint8)
    kc = rng.choice(codes, (B, Hkv, Nk, d)).astype(np.uint8)
    vc = rng.choice(codes, (B, Hkv, Nk, d)).astype(np.uint8)
    return qc, kc, vc


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill_matches_brute_force_on_torch_dequantised_inputs(causal):
    import torch
    from oracle import attention_prefill_fp8
    qc, kc, vc = _fp8_prefill_case(81)
    qs, ks, vs = 0.011, 0.0173, 0.031
    o, lse = attention_prefill_fp8(qc, kc, vc, 0.45, qs, ks, vs, causal)
    deq = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    for b in range(2):
        for h in range(4):
            bo, bl = brute_force_attention((qs * deq(qc[b, h])).tolist(),
                                           (ks * deq(kc[b, h // 2])).tolist(),
                                           (vs * deq(vc[b, h // 2])).tolist(), 0.45, causal)
            np.testing.assert_allclose(o[b, h], np.array(bo), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[b, h], np.array(bl), rtol=1e-12, atol=1e-12)


def test_fp8_prefill_scales_fold_into_the_softmax_scale_and_the_output():
    from oracle import attention_prefill_fp8
    qc, kc, vc = _fp8_prefill_case(82)
    o0, l0 = attention_prefill_fp8(qc, kc, vc, 0.3 * 0.02 * 0.05, 1.0, 1.0, 1.0, True)
    o1, l1 = attention_prefill_fp8(qc, kc, vc, 0.3, 0.02, 0.05, 1.0, True)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=1e-12, atol=1e-13)
    # Q and K scales enter only through their product
    o2, l2 = attention_prefill_fp8(qc, kc, vc, 0.3, 0.05, 0.02, 1.0, True)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)
    # the V scale multiplies O and leaves LSE alone
    o3, l3 = attention_prefill_fp8(qc, kc, vc, 0.3, 0.02, 0.05, 0.125, True)
    np.testing.assert_allclose(o3, 0.125 * o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(l3, l1)
    # and is not interchangeable with the K scale
    o4, _ = attention_prefill_fp8(qc, kc, vc, 0.3, 0.02, 0.125, 0.05, True)
    assert np.abs(o4 - o3).max() > 1e-3


def test_fp8_prefill_negated_query_codes_equal_a_negated_scale():
    # flipping bit 7 of every Q code negates Q exactly (sign-magnitude format)
    from oracle import attention_prefill_fp8
    qc, kc, vc = _fp8_prefill_case(83)
    o0, l0 = attention_prefill_fp8(qc ^ np.uint8(0x80), kc, vc, 0.4, 0.02, 0.05, 0.1, False)
    o1, l1 = attention_prefill_fp8(qc, kc, vc, -0.4, 0.02, 0.05, 0.1, False)
    np.testing.assert_allclose(o0, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l0, l1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_paged_prefill_equals_dense_fp8_prefill_of_each_sequence(causal):
    # the chunk's queries against each sequence's gathered context (NaN codes in every
    # unused slot) equal the dense FP8 prefill over that context
    from oracle import attention_prefill_fp8, attention_prefill_paged_fp8
    rng = np.random.default_rng(91)
    codes = [c for c in range(256) if c & 0x7F != 0x7F]
    lens = np.array([7, 3, 13], np.int32)
    Nq = 3
    qc = rng.choice(codes, (3, 4, Nq, 5)).astype(np.uint8)
    kc = rng.choice(codes, (3, 2, 13, 5)).astype(np.uint8)
    vc = rng.choice(codes, (3, 2, 13, 5)).astype(np.uint8)
    kp, table = _to_paged(kc, lens, 4, 11)
    vp, _ = _to_paged(vc, lens, 4, 11)
    o, lse = attention_prefill_paged_fp8(qc, kp, vp, table, lens, 0.4, 0.02, 0.03, 0.05, causal,
                                         page_size=4)
    assert np.isfinite(o).all()
    for b, n in enumerate(lens):
        od, ld = attention_prefill_fp8(qc[b:b + 1], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], 0.4,
                                       0.02, 0.03, 0.05, causal)
        np.testing.assert_allclose(o[b], od[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b], ld[0], rtol=1e-12, atol=1e-12)


def test_fp8_paged_prefill_matches_brute_force_on_torch_dequantised_inputs():
    import torch
    from oracle import attention_prefill_paged_fp8
    rng = np.random.default_rng(92)
    codes = [c for c in range(256) if c & 0x7F != 0x7F]
    lens = np.array([6, 9], np.int32)
    qc = rng.choice(codes, (2, 2, 4, 3)).astype(np.uint8)
    kc = rng.choice(codes, (2, 1, 9, 3)).astype(np.uint8)
    vc = rng.choice(codes, (2, 1, 9, 3)).astype(np.uint8)
    kp, table = _to_paged(kc, lens, 4, 12)
    vp, _ = _to_paged(vc, lens, 4, 12)
    o, lse = attention_prefill_paged_fp8(qc, kp, vp, table, lens, 0.3, 0.011, 0.017, 0.029, True,
                                         page_size=4)
    deq = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    for b, n in enumerate(lens):
        for h in range(2):
            bo, bl = brute_force_attention((0.011 * deq(qc[b, h])).tolist(),
                                           (0.017 * deq(kc[b, 0, :n])).tolist(),
                                           (0.029 * deq(vc[b, 0, :n])).tolist(), 0.3, True)
            np.testing.assert_allclose(o[b, h], np.array(bo), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[b, h], np.array(bl), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_varlen_prefill_equals_dense_fp8_prefill_of_each_sequence(causal):
    from oracle import attention_prefill_fp8, attention_prefill_varlen_fp8
    rng = np.random.default_rng(93)
    codes = [c for c in range(256) if c & 0x7F != 0x7F]
    lens_q, lens_k = [2, 0, 5], [4, 3, 5]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    qc = rng.choice(codes, (int(cu_q[-1]), 4, 3)).astype(np.uint8)
    kc = rng.choice(codes, (int(cu_k[-1]), 2, 3)).astype(np.uint8)
    vc = rng.choice(codes, (int(cu_k[-1]), 2, 3)).astype(np.uint8)
    o, lse = attention_prefill_varlen_fp8(qc, kc, vc, cu_q, cu_k, 0.4, 0.02, 0.03, 0.05, causal)
    for b in range(3):
        if lens_q[b] == 0:
            continue
        sq, sk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        od, ld = attention_prefill_fp8(qc[sq].transpose(1, 0, 2)[None], kc[sk].transpose(1, 0, 2)[None],
                                       vc[sk].transpose(1, 0, 2)[None], 0.4, 0.02, 0.03, 0.05, causal)
        np.testing.assert_allclose(o[sq], od[0].transpose(1, 0, 2), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[:, sq], ld[0], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- backward
def _bwd_case(seed, B=1, Hq=2, Hkv=1, Nq=5, Nk=7, d=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, Nq, d)), rng.standard_normal((B, Hkv, Nk, d)),
            rng.standard_normal((B, Hkv, Nk, d)), rng.standard_normal((B, Hq, Nq, d)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,Nq,Nk", [(2, 2, 6, 6), (4, 2, 5, 9), (3, 1, 1, 4)])
def test_backward_matches_torch_autograd(causal, Hq, Hkv, Nq, Nk):
    """Autograd through torch's own fp64 matmul and softmax on the plain definition."""
    import torch
    from oracle import attention_backward
    q, k, v, do = _bwd_case(80 + Nq, 2, Hq, Hkv, Nq, Nk, 4)
    scale = 0.7
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    kr, vr = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
    s = scale * tq @ kr.transpose(-1, -2)
    if causal:
        vis = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq)
        s = s.masked_fill(~vis, float("-inf"))
    o = torch.softmax(s, dim=-1) @ vr
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    """Central differences of L = sum(dO * O) in every input coordinate."""
    from oracle import attention_backward
    q, k, v, do = _bwd_case(91, 1, 2, 1, 4, 5, 3)
    scale = 0.9
    loss = lambda q_, k_, v_: float((attention_prefill(q_, k_, v_, scale, causal)[0] * do).sum())
    grads = attention_backward(q, k, v, do, scale, causal)
    h = 1e-6
    for x, g, idx in ((q, grads[0], 0), (k, grads[1], 1), (v, grads[2], 2)):
        fd = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[idx], args_m[idx] = xp, xm
            fd[pos] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7)


def test_backward_single_key_and_zero_scale():
    from oracle import attention_backward
    # one key: O = V[0] for every row, so dV[0] = sum of dO rows and dQ = dK = 0
    q, k, v, do = _bwd_case(92, 1, 2, 2, 4, 1, 3)
    dq, dk, dv = attention_backward(q, k, v, do, 0.8, False)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0, :, 0], do[0].sum(axis=1), atol=1e-14)
    # scale 0: uniform weights over the visible keys; dQ = dK = 0 and
    # dV_j = sum over the queries i that see key j of dO_i / (number of keys i sees)
    q, k, v, do = _bwd_case(93, 1, 1, 1, 5, 7, 3)
    for causal in (False, True):
        dq, dk, dv = attention_backward(q, k, v, do, 0.0, causal)
        assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
        n_vis = np.array([7 - 5 + i + 1 if causal else 7 for i in range(5)])
        want = np.zeros((7, 3))
        for i in range(5):
            for j in range(n_vis[i]):
                want[j] += do[0, 0, i] / n_vis[i]
        np.testing.assert_allclose(dv[0, 0], want, atol=1e-14)


def test_backward_gqa_is_sum_over_repeated_heads():
    from oracle import attention_backward
    q, k, v, do = _bwd_case(94, 2, 6, 2, 5, 8, 4)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, True)
    dq2, dk2, dv2 = attention_backward(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), do,
                                       0.5, True)
    np.testing.assert_allclose(dq, dq2, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(2, 2, 3, 8, 4).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(2, 2, 3, 8, 4).sum(axis=2), atol=1e-13)


def test_backward_row_term_equals_do_dot_o():
    """rowsum(P * dP) = rowsum(dO * O): the row term a kernel can take from O instead of P."""
    from oracle.attention import attention_scores
    q, k, v, do = _bwd_case(95, 1, 1, 1, 6, 9, 4)
    for causal in (False, True):
        p, _, _ = softmax_rows(attention_scores(q[0, 0], k[0, 0], 0.6, causal, np.arange(6), 6))
        o = p @ v[0, 0]
        dp = do[0, 0] @ v[0, 0].T
        np.testing.assert_allclose((p * dp).sum(axis=1), (do[0, 0] * o).sum(axis=1),
                                   atol=1e-13)


# ----------------------------------------------------------------------------- varlen
def _varlen_case(seed, lens_q, lens_k, Hq=2, Hkv=1, d=3):
    rng = np.random.default_rng(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return (rng.standard_normal((tq, Hq, d)), rng.standard_normal((tk, Hkv, d)),
            rng.standard_normal((tk, Hkv, d)), cu_q, cu_k)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_brute_force_per_sequence(causal):
    from oracle import attention_prefill_varlen
    lens_q, lens_k = [3, 1, 4, 2], [5, 1, 4, 6]
    q, k, v, cu_q, cu_k = _varlen_case(101, lens_q, lens_k, Hq=4, Hkv=2)
    o, lse = attention_prefill_varlen(q, k, v, cu_q, cu_k, 0.8, causal)
    for b in range(4):
        for h in range(4):
            qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            bo, bl = brute_force_attention(q[qs:qe, h].tolist(), k[ks:ke, h // 2].tolist(),
                                           v[ks:ke, h // 2].tolist(), 0.8, causal)
            np.testing.assert_allclose(o[qs:qe, h], np.array(bo), atol=1e-12)
            np.testing.assert_allclose(lse[h, qs:qe], np.array(bl), atol=1e-12)


def test_varlen_sequence_order_and_empty_sequences():
    from oracle import attention_prefill_varlen
    lens_q, lens_k = [3, 0, 5, 2], [4, 2, 5, 0]
    q, k, v, cu_q, cu_k = _varlen_case(102, lens_q, lens_k)
    o, lse = attention_prefill_varlen(q, k, v, cu_q, cu_k, 0.5, False)
    # the empty-query sequence writes nothing; the key-less one gives O = 0, LSE = -inf
    assert (o[cu_q[3]:cu_q[4]] == 0).all() and (lse[:, cu_q[3]:cu_q[4]] == -np.inf).all()
    # reversing the sequence order reverses the outputs' blocks
    order = [3, 2, 1, 0]
    qb = [q[cu_q[b]:cu_q[b + 1]] for b in order]
    kb = [k[cu_k[b]:cu_k[b + 1]] for b in order]
    vb = [v[cu_k[b]:cu_k[b + 1]] for b in order]
    cq = np.concatenate([[0], np.cumsum([lens_q[b] for b in order])]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum([lens_k[b] for b in order])]).astype(np.int32)
    o2, l2 = attention_prefill_varlen(np.concatenate(qb), np.concatenate(kb), np.concatenate(vb),
                                      cq, ck, 0.5, False)
    for i, b in enumerate(order):
        np.testing.assert_array_equal(o2[cq[i]:cq[i + 1]], o[cu_q[b]:cu_q[b + 1]])
        np.testing.assert_array_equal(l2[:, cq[i]:cq[i + 1]], lse[:, cu_q[b]:cu_q[b + 1]])
