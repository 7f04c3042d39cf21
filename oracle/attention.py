"""CPU oracle for exact attention, numpy float64.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call anything in this package.  The GPU product
path never routes through it, and it shares no code with the GPU path.

What it computes is the plain definition of attention,
    O = softmax(scale * Q K^T [+ causal mask]) V,
from the page "FlashAttention 완전 정리" (cell-devlog), section "Attention이 뭔가"
(what attention is): the formula softmax(Q K^T / sqrt(d_k)) V, with Q K^T the
all-pairs similarity matrix, softmax turning each row into probabilities, and the
product with V the weighted sum.  It is run the way the same page's section
"문제 — Attention은 메모리 병목이다" (attention is memory-bound) lays out standard
attention: materialise S = Q K^T, take the row softmax of S, multiply by V.  The
fused method reaches the same result (same page, section on FlashAttention 1:
"accuracy unchanged, not an approximation"), so this definition is the parity
target.

Readings where the pages are silent (each one also listed in the design notes):
  * scale is an explicit argument (the pages write 1/sqrt(d_k); the flash_attn_func
    call on the page "메모리 장벽을 넘어" (tiptinker), section on the forward pass,
    defaults softmax_scale to None);
  * causal masking is aligned bottom-right: key j is visible to query i iff
    j <= i + (Nk - Nq); causal with Nq > Nk is rejected;
  * grouped-query heads: query head h reads KV head h // (Hq / Hkv);
  * LSE = m + ln(l), natural log, over the visible keys only;
  * layout [B, H, N, d] for Q, K, V, O;
  * a decode step is one query row per sequence attending to the first
    seqlens[b] cached keys; seqlens[b] == 0 gives O = 0 and LSE = -inf.

Parity status: every function here is pinned by tests/test_oracle.py against
brute force, closed forms and invariants (no function is parity unpinned).
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Prefill: three passes over a materialised score matrix
# ---------------------------------------------------------------------------
def _causal_visible(rows: np.ndarray, Nq: int, Nk: int) -> np.ndarray:
    """Boolean [len(rows), Nk]: key j visible to query row i iff j <= i + (Nk - Nq)."""
    j = np.arange(Nk)[None, :]
    return j <= (rows[:, None] + (Nk - Nq))


def attention_scores(q_rows: np.ndarray, k: np.ndarray, scale: float, causal: bool,
                     rows: np.ndarray, Nq: int) -> np.ndarray:
    """Pass 1: S = scale * Q K^T for the given query rows, masked entries -inf."""
    s = scale * (q_rows @ k.T)
    if causal:
        s = np.where(_causal_visible(rows, Nq, k.shape[0]), s, -np.inf)
    return s


def softmax_rows(s: np.ndarray):
    """Pass 2: row softmax of S.  Returns (P, m, l) with m the row max,
    l = sum exp(S - m) and P = exp(S - m) / l (the m, f, l of the page
    "Flash Attention: GPU 메모리_IO를 최적화하는..." (holysheep), section
    "수학적 원리: Online Softmax 알고리즘" (math: online softmax))."""
    m = s.max(axis=1, keepdims=True)
    f = np.exp(s - m)
    l = f.sum(axis=1, keepdims=True)
    return f / l, m[:, 0], l[:, 0]


def attention_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool, rows: np.ndarray, Nq: int):
    """Attention for selected query rows of one head.

    q_rows [R, d] are queries with indices ``rows`` (0-based, out of Nq);
    k, v [Nk, d].  Returns (O [R, d], LSE [R]) in float64.
    """
    s = attention_scores(q_rows, k, scale, causal, rows, Nq)
    p, m, l = softmax_rows(s)
    o = p @ v                                           # pass 3
    lse = m + np.log(l)
    return o, lse


def attention_prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      causal: bool, row_block: int = 1024):
    """Full prefill.  q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] (float64 holding the exact
    input values).  Returns O [B,Hq,Nq,d] and LSE [B,Hq,Nq], float64.

    Rows are processed in blocks of ``row_block`` only to bound the size of the
    materialised S; each block is the full three-pass computation for its rows.
    """
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    G = Hq // Hkv
    o = np.empty((B, Hq, Nq, d))
    lse = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            for i0 in range(0, Nq, row_block):
                rows = np.arange(i0, min(Nq, i0 + row_block))
                o[b, h, rows], lse[b, h, rows] = attention_rows(
                    q[b, h, rows], k[b, kvh], v[b, kvh], scale, causal, rows, Nq)
    return o, lse


def attention_probabilities(q: np.ndarray, k: np.ndarray, scale: float, causal: bool):
    """P for one head, q [Nq,d], k [Nk,d]: the softmax rows pass 2 produces."""
    rows = np.arange(q.shape[0])
    p, _, _ = softmax_rows(attention_scores(q, k, scale, causal, rows, q.shape[0]))
    return p


# ---------------------------------------------------------------------------
# Decode: one query per sequence against the first seqlens[b] cached keys
# ---------------------------------------------------------------------------
def gather_paged(pool: np.ndarray, block_table: np.ndarray, b: int, kvh: int, length: int,
                 page_size: int) -> np.ndarray:
    """Rows 0..length-1 of sequence b, KV head kvh, from a paged pool
    [num_pages, Hkv, page_size, d]: token t lives in page block_table[b, t // page_size],
    slot t % page_size (the paged KV cache of the page "메모리 장벽을 넘어" (tiptinker),
    section "2. FlashInfer" (PagedAttention integration))."""
    t = np.arange(length)
    pages = block_table[b, t // page_size]
    return pool[pages, kvh, t % page_size]


def attention_decode(q: np.ndarray, kcache: np.ndarray, vcache: np.ndarray,
                     seqlens: np.ndarray, scale: float, block_table: np.ndarray | None = None,
                     page_size: int = 16):
    """q [B,Hq,d].  Contiguous cache (block_table None): k/vcache [B,Hkv,Nmax,d];
    paged: [num_pages,Hkv,page_size,d] with block_table [B, max_blocks].
    Returns O [B,Hq,d], LSE [B,Hq] (float64)."""
    B, Hq, d = q.shape
    Hkv = kcache.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        for kvh in range(Hkv):
            if block_table is None:
                K = kcache[b, kvh, :n]
                V = vcache[b, kvh, :n]
            else:
                K = gather_paged(kcache, block_table, b, kvh, n, page_size)
                V = gather_paged(vcache, block_table, b, kvh, n, page_size)
            hs = slice(kvh * G, (kvh + 1) * G)
            ob, lb = attention_rows(q[b, hs], K, V, scale, False, np.arange(G), G)
            o[b, hs], lse[b, hs] = ob, lb
    return o, lse


# ---------------------------------------------------------------------------
# Variable-length (ragged) batch packed along tokens
# ---------------------------------------------------------------------------
def attention_prefill_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q: np.ndarray,
                             cu_k: np.ndarray, scale: float, causal: bool):
    """A ragged batch (the continuous-batching shape of the page "Transformers optimization
    overview", section on continuous batching) packed along tokens: q [total_q, Hq, d],
    k, v [total_k, Hkv, d]; sequence b owns query rows cu_q[b]:cu_q[b+1] and key rows
    cu_k[b]:cu_k[b+1], and its queries attend only to its own keys (bottom-right causal per
    sequence).  A sequence without keys gets O = 0, LSE = -inf.  Returns O [total_q, Hq, d]
    and LSE [Hq, total_q] (float64)."""
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.zeros((total_q, Hq, d))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        nq, nk = qe - qs, ke - ks
        if nq == 0 or nk == 0:
            continue
        if causal and nq > nk:
            raise ValueError("causal attention needs Nq <= Nk in every sequence")
        rows = np.arange(nq)
        for h in range(Hq):
            o[qs:qe, h], lse[h, qs:qe] = attention_rows(q[qs:qe, h], k[ks:ke, h // G],
                                                        v[ks:ke, h // G], scale, causal, rows, nq)
    return o, lse


# ---------------------------------------------------------------------------
# Backward: gradients of the definition
# ---------------------------------------------------------------------------
def attention_backward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                            scale: float, causal: bool):
    """Gradients of one head of O = softmax(scale * Q K^T [+ mask]) V (the definition of
    the page "FlashAttention 완전 정리" (cell-devlog), section "Attention이 뭔가") with
    respect to Q, K and V, for the output gradient dO.  The pages only say that the fused
    method recomputes the attention matrix in its backward pass instead of storing it
    (page "메모리 장벽을 넘어" (tiptinker), section "1. FlashAttention": tiling and
    recomputation); the gradients themselves are plain calculus:
        P  = softmax rows of S,  S = scale * Q K^T (masked entries -inf)
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian applied row by row)
        dQ = scale * dS K,   dK = scale * dS^T Q
    q, do [Nq, d]; k, v [Nk, d].  Returns dq [Nq, d], dk, dv [Nk, d] (float64)."""
    rows = np.arange(q.shape[0])
    p, _, _ = softmax_rows(attention_scores(q, k, scale, causal, rows, q.shape[0]))
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                       scale: float, causal: bool):
    """Backward of attention_prefill: q, do [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d].  With grouped
    query heads, a KV head's dK and dV are the sums over the query heads that read it
    (head h reads KV head h // (Hq / Hkv)).  Returns dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d]."""
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and Nq > k.shape[2]:
        raise ValueError("causal attention needs Nq <= Nk")
    G = Hq // Hkv
    dq = np.empty(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            gq, gk, gv = attention_backward_head(q[b, h], k[b, kvh], v[b, kvh], do[b, h],
                                                 scale, causal)
            dq[b, h] = gq
            dk[b, kvh] += gk
            dv[b, kvh] += gv
    return dq, dk, dv


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache
# ---------------------------------------------------------------------------
def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """float64 value of OCP FP8 E4M3 codes (the 8-bit format of a compressed KV cache,
    page "메모리 장벽을 넘어" (tiptinker), section "2. FlashInfer"; the pages do not spell
    the format out, so the OCP 8-bit floating point definition is used): bit 7 sign,
    bits 6..3 exponent e with bias 7, bits 2..0 mantissa m;
      e == 0:            (-1)^s * (m / 8) * 2^-6      (zero and subnormals)
      e == 15 and m == 7: NaN                          (no infinities)
      otherwise:          (-1)^s * (1 + m / 8) * 2^(e - 7)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def attention_decode_fp8(q: np.ndarray, kcodes: np.ndarray, vcodes: np.ndarray,
                         seqlens: np.ndarray, scale: float, k_scale: float, v_scale: float,
                         block_table: np.ndarray | None = None, page_size: int = 16):
    """Decode over an FP8 KV cache with one scale per tensor: the cached K is
    k_scale * e4m3_value(kcodes) and V is v_scale * e4m3_value(vcodes) (per-tensor
    scaling is a reading: the pages give no scale convention).  The caches are laid out
    as in attention_decode (codes instead of values); only the live rows of each
    (sequence, KV head) are dequantised, then attention is the plain definition.
    Returns O [B,Hq,d], LSE [B,Hq] (float64)."""
    B, Hq, d = q.shape
    Hkv = kcodes.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        for kvh in range(Hkv):
            if block_table is None:
                kc, vc = kcodes[b, kvh, :n], vcodes[b, kvh, :n]
            else:
                kc = gather_paged(kcodes, block_table, b, kvh, n, page_size)
                vc = gather_paged(vcodes, block_table, b, kvh, n, page_size)
            K = k_scale * e4m3_value(kc)
            V = v_scale * e4m3_value(vc)
            hs = slice(kvh * G, (kvh + 1) * G)
            o[b, hs], lse[b, hs] = attention_rows(q[b, hs], K, V, scale, False, np.arange(G), G)
    return o, lse


def attention_prefill_fp8(qcodes: np.ndarray, kcodes: np.ndarray, vcodes: np.ndarray,
                          scale: float, q_scale: float, k_scale: float, v_scale: float,
                          causal: bool, row_block: int = 1024):
    """Prefill over FP8 inputs with one scale per tensor (the FP8 support that the page
    "FlashAttention 완전 정리" (cell-devlog), section "FlashAttention 버전별 발전", subsection
    "FlashAttention 3", lists; the pages give no format or scale convention, so the reading is
    OCP E4M3 codes with per-tensor scales, as for the FP8 cache): Q is
    q_scale * e4m3_value(qcodes), K and V likewise with k_scale and v_scale, laid out as in
    attention_prefill.  The result is the plain definition on those dequantised values.
    Returns O [B,Hq,Nq,d], LSE [B,Hq,Nq] (float64)."""
    Q = q_scale * e4m3_value(qcodes)
    K = k_scale * e4m3_value(kcodes)
    V = v_scale * e4m3_value(vcodes)
    return attention_prefill(Q, K, V, scale, causal, row_block)


def attention_prefill_paged(q: np.ndarray, kpool: np.ndarray, vpool: np.ndarray,
                            block_table: np.ndarray, kv_lens: np.ndarray, scale: float,
                            causal: bool, page_size: int = 16, row_block: int = 1024):
    """Chunked (append) prefill against a paged cache: the Nq queries of sequence b are its
    last Nq tokens and attend to its first kv_lens[b] cached keys (chunked prefill in the
    continuous-batching section of the page "Transformers optimization overview"; the
    paged cache of the page "메모리 장벽을 넘어" (tiptinker), section "2. FlashInfer").

    q [B,Hq,Nq,d]; pools [num_pages,Hkv,page_size,d]; block_table [B, max_blocks];
    kv_lens [B] with Nq <= kv_lens[b].  Causal alignment is bottom-right, so query i sees
    keys 0 .. kv_lens[b] - Nq + i.  Returns O [B,Hq,Nq,d], LSE [B,Hq,Nq] (float64).
    """
    B, Hq, Nq, d = q.shape
    Hkv = kpool.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.empty((B, Hq, Nq, d))
    lse = np.empty((B, Hq, Nq))
    for b in range(B):
        n = int(kv_lens[b])
        if n < Nq:
            raise ValueError("each kv_lens[b] must be >= Nq")
        for kvh in range(Hkv):
            K = gather_paged(kpool, block_table, b, kvh, n, page_size)
            V = gather_paged(vpool, block_table, b, kvh, n, page_size)
            for h in range(kvh * G, (kvh + 1) * G):
                for i0 in range(0, Nq, row_block):
                    rows = np.arange(i0, min(Nq, i0 + row_block))
                    o[b, h, rows], lse[b, h, rows] = attention_rows(
                        q[b, h, rows], K, V, scale, causal, rows, Nq)
    return o, lse


# ---------------------------------------------------------------------------
# Combining partial results over disjoint key sets
# ---------------------------------------------------------------------------
def attention_prefill_paged_fp8(qcodes: np.ndarray, kpool: np.ndarray, vpool: np.ndarray,
                                block_table: np.ndarray, kv_lens: np.ndarray, scale: float,
                                q_scale: float, k_scale: float, v_scale: float, causal: bool,
                                page_size: int = 16):
    """Chunked prefill (attention_prefill_paged) over FP8 inputs: the queries and the paged
    pools hold E4M3 codes with one scale per tensor, read as in attention_prefill_fp8 (the
    pools as the FP8 cache of attention_decode_fp8).  Only the live rows a sequence
    gathers reach the arithmetic, so codes in unused slots never matter.
    Returns O [B,Hq,Nq,d], LSE [B,Hq,Nq] (float64)."""
    Q = q_scale * e4m3_value(qcodes)
    K = k_scale * e4m3_value(kpool)
    V = v_scale * e4m3_value(vpool)
    return attention_prefill_paged(Q, K, V, block_table, kv_lens, scale, causal, page_size)


def attention_prefill_varlen_fp8(qcodes: np.ndarray, kcodes: np.ndarray, vcodes: np.ndarray,
                                 cu_q: np.ndarray, cu_k: np.ndarray, scale: float,
                                 q_scale: float, k_scale: float, v_scale: float, causal: bool):
    """Ragged batch (attention_prefill_varlen) over FP8 inputs: the packed tensors hold E4M3
    codes with one scale per tensor, read as in attention_prefill_fp8.
    Returns O [total_q, Hq, d], LSE [Hq, total_q] (float64)."""
    return attention_prefill_varlen(q_scale * e4m3_value(qcodes), k_scale * e4m3_value(kcodes),
                                    v_scale * e4m3_value(vcodes), cu_q, cu_k, scale, causal)


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine attention results computed over disjoint key subsets of one row.

    o_parts [S, d] are the per-subset normalised outputs, lse_parts [S] their
    log-sum-exps (-inf for an empty subset).  From l = sum exp(x - m) (page
    "Flash Attention: GPU 메모리_IO를 최적화하는...", section on online softmax),
    the subset with statistics (m_s, l_s) contributes exp(lse_s) = exp(m_s) l_s to the
    full row's normaliser, so the full row is the exp(lse_s)-weighted mean of the
    o_s and its LSE is ln sum exp(lse_s).
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = np.max(lse_parts)
    if M == -np.inf:
        return np.zeros(o_parts.shape[1:]), -np.inf
    w = np.exp(lse_parts - M)
    W = w.sum()
    return (w[:, None] * o_parts).sum(axis=0) / W, M + math.log(W)


# ---------------------------------------------------------------------------
# Twins used only to check the oracle itself
# ---------------------------------------------------------------------------
def brute_force_attention(q, k, v, scale: float, causal: bool):
    """Pure-Python scalar attention for tiny inputs (lists or arrays of one head:
    q [Nq][d], k [Nk][d], v [Nk][d]).  math.exp and math.fsum, no numpy.
    Returns (O as nested lists, LSE as a list)."""
    Nq, Nk = len(q), len(k)
    d = len(q[0])
    out, lses = [], []
    for i in range(Nq):
        scores = []
        for j in range(Nk):
            if causal and j > i + (Nk - Nq):
                continue
            scores.append((j, float(scale) * math.fsum(float(q[i][t]) * float(k[j][t])
                                                       for t in range(d))))
        mx = max(s for _, s in scores)
        wts = [(j, math.exp(s - mx)) for j, s in scores]
        tot = math.fsum(w for _, w in wts)
        out.append([math.fsum(w * float(v[j][c]) for j, w in wts) / tot for c in range(d)])
        lses.append(mx + math.log(tot))
    return out, lses


def online_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                     block: int):
    """One head, key blocks of size ``block`` visited in order with the online-softmax
    recurrence (page "FlashAttention 완전 정리", section "Tiling": track the running max
    per block and update earlier partial results as each block arrives):

        m' = max(m, rowmax S_j)
        l' = exp(m - m') l + rowsum exp(S_j - m')
        A' = exp(m - m') A + exp(S_j - m') V_j
    and O = A / l at the end.  Used only to check the two-pass oracle."""
    Nq, d = q.shape
    Nk = k.shape[0]
    rows = np.arange(Nq)
    m = np.full(Nq, -np.inf)
    l = np.zeros(Nq)
    acc = np.zeros((Nq, d))
    for j0 in range(0, Nk, block):
        j1 = min(Nk, j0 + block)
        s = scale * (q @ k[j0:j1].T)
        if causal:
            vis = np.arange(j0, j1)[None, :] <= (rows[:, None] + (Nk - Nq))
            s = np.where(vis, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        # rows with no visible key so far keep m = -inf; guard the -inf - -inf case
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        p = np.exp(s - safe[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
    return acc / l[:, None], m + np.log(l)
