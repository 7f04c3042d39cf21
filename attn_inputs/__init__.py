"""Seeded synthetic inputs for the attention workloads.

This module is shared by the CPU oracle side and the GPU side, and by nothing
else.  It holds no attention arithmetic: only random draws, the rounding of those
draws to bfloat16, the workload table, the paged-cache layout (which page holds
which token) and the counting of work units used to express throughput.

Every tensor slice is drawn from its own counter-keyed stream
``numpy.random.SeedSequence([seed, tensor, b, h])`` so that any single head of a
full-size workload can be regenerated on its own (the oracle checks sampled
heads of the large workloads without drawing the whole tensor).

Value recipe (all workloads): i.i.d. float32 N(0, 1) draws, optionally multiplied
by a constant in float32, rounded to bfloat16 with round-to-nearest-even (to IEEE
fp16, also nearest-even, for the fp16 variants: the same draws, rounded differently).  An FP8
KV cache holds the same draws divided (in float32) by a per-tensor scale and rounded
to OCP FP8 E4M3 codes (round-to-nearest-even, saturating at +-448); the value a code
stands for is that scale times the code's E4M3 value.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Stream identifiers inside one workload seed.
T_Q, T_K, T_V, T_LEN, T_PERM, T_DO = 0, 1, 2, 3, 4, 5

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)

# Per-tensor scales of the FP8 KV caches: a code c of the K (V) cache stands for
# FP8_K_SCALE * e4m3(c) (FP8_V_SCALE * e4m3(c)).  Chosen so that N(0, 1) draws use the
# E4M3 range up to about 8 (6) standard deviations; the two differ so that a swapped
# pair of scales shows.
FP8_K_SCALE = float(np.float32(8.0 / 448.0))
FP8_V_SCALE = float(np.float32(6.0 / 448.0))
# Scale of FP8 prefill queries (K and V use the two above).
FP8_Q_SCALE = float(np.float32(7.0 / 448.0))


# ----------------------------------------------------------------------------
# bfloat16 rounding of float32 draws
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs are finite draws; NaN and
    infinity are not produced by the generators and are not handled here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE fp16 (numpy's conversion: nearest, ties to even),
    returned as uint16 bit patterns.  The draws stay far inside the fp16 range."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of fp16 bit patterns to float64."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bits_to_f64(bits: np.ndarray, f16: bool) -> np.ndarray:
    """Exact widening of 16-bit patterns of either element type."""
    return f16_bits_to_f64(bits) if f16 else bf16_bits_to_f64(bits)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; no infinities), round to nearest with ties to even, magnitudes
    above 448 (the largest finite E4M3 value) saturating to 448.

    Normal range (|x| >= 2^-6): the float32 mantissa is rounded to 3 bits by adding a
    bias below bit 20, as for bfloat16 above, and the exponent re-biased.  Subnormal
    range: the code is the integer rint(|x| * 2^9), in units of 2^-9.  Returns uint8
    codes; NaN is never produced (inputs are finite draws).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(448.0))
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(20)) & np.uint32(1)
    r = (u + np.uint32(0x7FFFF) + lsb) & np.uint32(0xFFF00000)
    exp = (r >> np.uint32(23)).astype(np.int32) - 127
    normal_code = ((exp + 7) << 3) | ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    sub_code = np.rint(a.astype(np.float64) * 512.0).astype(np.int32)
    code = np.where(a < np.float32(2.0 ** -6), sub_code, normal_code)
    sign = np.signbit(x).astype(np.int32) << 7
    return (code | sign).astype(np.uint8)


def _stream(seed: int, tensor: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor, b, h]))


def normal_bf16(seed: int, tensor: int, b: int, h: int, shape, mult: float = 1.0,
                f16: bool = False) -> np.ndarray:
    """One head's slice: float32 N(0,1) draws (times ``mult`` in float32), rounded to bf16
    bits (to fp16 bits when ``f16``)."""
    x = _stream(seed, tensor, b, h).standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return to_f16_bits(x) if f16 else to_bf16_bits(x)


def normal_e4m3(seed: int, tensor: int, b: int, h: int, shape, scale: float,
                mult: float = 1.0) -> np.ndarray:
    """One head's slice of an FP8 tensor: the float32 N(0,1) draws of ``normal_bf16`` (same
    stream, times ``mult`` in float32), divided by ``scale`` in float32, as E4M3 codes."""
    x = _stream(seed, tensor, b, h).standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return to_e4m3_codes(x / np.float32(scale))


# ----------------------------------------------------------------------------
# Workload table
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class PrefillCfg:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    q_mult: float = 1.0
    f16: bool = False             # fp16 elements instead of bf16
    fp8: bool = False             # Q, K, V as E4M3 codes with FP8_Q/K/V_SCALE (O bf16)

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the float32 value both sides receive."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


@dataclass(frozen=True)
class DecodeCfg:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    seed: int
    paged: bool
    page_size: int = 16
    fixed_len: int = 0            # every sequence this long (contiguous workload)
    len_range: tuple = (0, 0)     # inclusive uniform range of lengths (paged workload)
    chunk: int = 0                # chunked prefill: new tokens (queries) per sequence
    kv_fp8: bool = False          # K/V cache as E4M3 codes with FP8_K_SCALE / FP8_V_SCALE
    f16: bool = False             # fp16 Q and cache instead of bf16 (not with kv_fp8)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


CONFIGS = {
    # Tiny prefill: correctness-sized, several tiles and heads.
    "tiny_prefill": PrefillCfg("tiny_prefill", B=1, Hq=4, Hkv=4, Nq=512, Nk=512, d=64,
                               causal=True, seed=1),
    # Llama-2-7B-shaped prefill (32 heads x d=128), causal and non-causal on the same tensors.
    "llama2_7b_prefill": PrefillCfg("llama2_7b_prefill", B=4, Hq=32, Hkv=32, Nq=2048, Nk=2048,
                                    d=128, causal=True, seed=2),
    "llama2_7b_prefill_noncausal": PrefillCfg("llama2_7b_prefill_noncausal", B=4, Hq=32, Hkv=32,
                                              Nq=2048, Nk=2048, d=128, causal=False, seed=2),
    # The same draws rounded to fp16 (the fp16 entry points).
    "llama2_7b_prefill_f16": PrefillCfg("llama2_7b_prefill_f16", B=4, Hq=32, Hkv=32, Nq=2048,
                                        Nk=2048, d=128, causal=True, seed=2, f16=True),
    # The same shape over FP8 (E4M3) Q, K, V with one scale per tensor.
    "llama2_7b_prefill_fp8": PrefillCfg("llama2_7b_prefill_fp8", B=4, Hq=32, Hkv=32, Nq=2048,
                                        Nk=2048, d=128, causal=True, seed=2, fp8=True),
    # Long-context prefill, Q scaled by 3 before rounding so softmax rows are peaky.
    "long_prefill_32k": PrefillCfg("long_prefill_32k", B=1, Hq=32, Hkv=32, Nq=32768, Nk=32768,
                                   d=128, causal=True, seed=3, q_mult=3.0),
    # GQA decode on a contiguous cache, every sequence 8192 tokens long.
    "gqa_decode_contig": DecodeCfg("gqa_decode_contig", B=64, Hq=32, Hkv=8, d=128, seed=4,
                                   paged=False, fixed_len=8192),
    # Paged GQA decode, 16-token pages, lengths uniform in [1024, 131072].
    "paged_gqa_decode": DecodeCfg("paged_gqa_decode", B=8, Hq=32, Hkv=8, d=128, seed=5,
                                  paged=True, page_size=16, len_range=(1024, 131072)),
    # The paged decode workload (same lengths and page layout) over an FP8 E4M3 cache.
    "paged_gqa_decode_fp8": DecodeCfg("paged_gqa_decode_fp8", B=8, Hq=32, Hkv=8, d=128,
                                      seed=5, paged=True, page_size=16,
                                      len_range=(1024, 131072), kv_fp8=True),
    # Ragged batch of prompts (self-attention, causal) packed along tokens: 16 sequences
    # of 256..4096 tokens, Llama-2-style GQA heads.  B, Hq, Hkv, d as listed; the lengths
    # come from varlen_lengths(seed, B, *len_range).
    "varlen_prefill": DecodeCfg("varlen_prefill", B=16, Hq=32, Hkv=8, d=128, seed=8,
                                paged=False, len_range=(256, 4096)),
    # Chunked prefill against a paged cache: 512 new tokens per sequence appended to
    # contexts (which already hold them) of 2048..16384 tokens, Llama-2-style GQA heads.
    "chunked_prefill_paged": DecodeCfg("chunked_prefill_paged", B=8, Hq=32, Hkv=8, d=128,
                                       seed=6, paged=True, page_size=16,
                                       len_range=(2048, 16384), chunk=512),
    # The same chunked prefill over FP8 queries and an FP8 paged cache.
    "chunked_prefill_paged_fp8": DecodeCfg("chunked_prefill_paged_fp8", B=8, Hq=32, Hkv=8,
                                           d=128, seed=6, paged=True, page_size=16,
                                           len_range=(2048, 16384), chunk=512, kv_fp8=True),
}


# ----------------------------------------------------------------------------
# Prefill inputs
# ----------------------------------------------------------------------------
def prefill_scales(cfg: PrefillCfg):
    """(q_scale, k_scale, v_scale) of an FP8 prefill workload; 1.0 each otherwise."""
    if not cfg.fp8:
        return 1.0, 1.0, 1.0
    return FP8_Q_SCALE, FP8_K_SCALE, FP8_V_SCALE


def prefill_head(cfg: PrefillCfg, tensor: int, b: int, h: int) -> np.ndarray:
    """bf16 bits of one head: Q [Nq, d] for tensor T_Q, K/V [Nk, d] for T_K/T_V (fp16 bits
    when cfg.f16; E4M3 codes of the same draws over the tensor's scale when cfg.fp8)."""
    if cfg.fp8:
        sc = prefill_scales(cfg)[tensor]
        if tensor == T_Q:
            return normal_e4m3(cfg.seed, T_Q, b, h, (cfg.Nq, cfg.d), sc, cfg.q_mult)
        return normal_e4m3(cfg.seed, tensor, b, h, (cfg.Nk, cfg.d), sc)
    if tensor == T_Q:
        return normal_bf16(cfg.seed, T_Q, b, h, (cfg.Nq, cfg.d), cfg.q_mult, cfg.f16)
    return normal_bf16(cfg.seed, tensor, b, h, (cfg.Nk, cfg.d), f16=cfg.f16)


def prefill_inputs(cfg: PrefillCfg):
    """Whole tensors as bf16 bits (fp16 bits, E4M3 codes): q [B,Hq,Nq,d], k and v
    [B,Hkv,Nk,d]."""
    q = np.empty((cfg.B, cfg.Hq, cfg.Nq, cfg.d), np.uint8 if cfg.fp8 else np.uint16)
    k = np.empty((cfg.B, cfg.Hkv, cfg.Nk, cfg.d), np.uint8 if cfg.fp8 else np.uint16)
    v = np.empty_like(k)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            q[b, h] = prefill_head(cfg, T_Q, b, h)
        for h in range(cfg.Hkv):
            k[b, h] = prefill_head(cfg, T_K, b, h)
            v[b, h] = prefill_head(cfg, T_V, b, h)
    return q, k, v


def prefill_dout(cfg: PrefillCfg) -> np.ndarray:
    """Output gradient dO [B, Hq, Nq, d] for the backward: bf16 bits (fp16 when cfg.f16)
    of N(0,1) draws from its own stream."""
    do = np.empty((cfg.B, cfg.Hq, cfg.Nq, cfg.d), np.uint16)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            do[b, h] = normal_bf16(cfg.seed, T_DO, b, h, (cfg.Nq, cfg.d), f16=cfg.f16)
    return do


def custom_prefill(seed: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                   q_mult: float = 1.0, f16: bool = False, fp8: bool = False):
    """Inputs for an arbitrary prefill shape (edge cases), same recipe."""
    cfg = PrefillCfg("custom", B, Hq, Hkv, Nq, Nk, d, True, seed, q_mult, f16, fp8)
    return prefill_inputs(cfg)


# ----------------------------------------------------------------------------
# Variable-length (ragged) prefill inputs
# ----------------------------------------------------------------------------
def varlen_inputs(seed: int, lens_q, lens_k, Hq: int, Hkv: int, d: int, f16: bool = False,
                  fp8: bool = False):
    """Packed ragged batch: q [total_q, Hq, d], k, v [total_k, Hkv, d] bf16 bits (fp16 when
    f16; E4M3 codes over FP8_Q/K/V_SCALE when fp8) and the cumulative lengths cu_q, cu_k
    (int32 [B+1]).  Sequence b, head h draws its rows from the same per-(b, h) streams as
    the dense layout does, so each sequence equals a dense prefill input of its own length."""
    lens_q = np.asarray(lens_q, np.int64)
    lens_k = np.asarray(lens_k, np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    dt = np.uint8 if fp8 else np.uint16
    q = np.empty((int(cu_q[-1]), Hq, d), dt)
    k = np.empty((int(cu_k[-1]), Hkv, d), dt)
    v = np.empty_like(k)

    def draw(tensor, b, h, n):
        if fp8:
            sc = {T_Q: FP8_Q_SCALE, T_K: FP8_K_SCALE, T_V: FP8_V_SCALE}[tensor]
            return normal_e4m3(seed, tensor, b, h, (n, d), sc)
        return normal_bf16(seed, tensor, b, h, (n, d), f16=f16)

    for b in range(len(lens_q)):
        for h in range(Hq):
            q[cu_q[b]:cu_q[b + 1], h] = draw(T_Q, b, h, int(lens_q[b]))
        for h in range(Hkv):
            k[cu_k[b]:cu_k[b + 1], h] = draw(T_K, b, h, int(lens_k[b]))
            v[cu_k[b]:cu_k[b + 1], h] = draw(T_V, b, h, int(lens_k[b]))
    return q, k, v, cu_q, cu_k


def varlen_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """B sequence lengths uniform in [lo, hi] from the lengths stream."""
    return _stream(seed, T_LEN).integers(lo, hi, size=B, endpoint=True).astype(np.int32)


# ----------------------------------------------------------------------------
# Decode inputs
# ----------------------------------------------------------------------------
def decode_lengths(cfg: DecodeCfg) -> np.ndarray:
    """KV length of every sequence, int32 [B]."""
    if not cfg.paged:
        return np.full(cfg.B, cfg.fixed_len, np.int32)
    lo, hi = cfg.len_range
    return _stream(cfg.seed, T_LEN).integers(lo, hi, size=cfg.B, endpoint=True).astype(np.int32)


def decode_q(cfg: DecodeCfg) -> np.ndarray:
    """q [B, Hq, d] bf16 bits."""
    q = np.empty((cfg.B, cfg.Hq, cfg.d), np.uint16)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            q[b, h] = normal_bf16(cfg.seed, T_Q, b, h, (cfg.d,), f16=cfg.f16)
    return q


def kv_scale(cfg: DecodeCfg, tensor: int) -> float:
    """Per-tensor scale of an FP8 cache (1.0 for a bf16 cache)."""
    if not cfg.kv_fp8:
        return 1.0
    return FP8_K_SCALE if tensor == T_K else FP8_V_SCALE


F16_NAN = np.uint16(0x7E00)


def kv_pad(cfg: DecodeCfg):
    """NaN of the cache's element type: fills slots that must never be read."""
    if cfg.kv_fp8:
        return E4M3_NAN
    return F16_NAN if cfg.f16 else BF16_NAN


def decode_kv_logical(cfg: DecodeCfg, tensor: int, b: int, kvh: int, length: int) -> np.ndarray:
    """The first ``length`` cached K (or V) rows of sequence b, KV head kvh: [length, d]
    bf16 bits, or E4M3 codes for an FP8 cache."""
    if cfg.kv_fp8:
        return normal_e4m3(cfg.seed, tensor, b, kvh, (length, cfg.d), kv_scale(cfg, tensor))
    return normal_bf16(cfg.seed, tensor, b, kvh, (length, cfg.d), f16=cfg.f16)


@dataclass
class PagedLayout:
    """Which physical page holds which 16-token block of which sequence."""
    page_size: int
    num_pages: int
    max_blocks: int
    block_table: np.ndarray = field(repr=False)   # int32 [B, max_blocks], -1 = unused


def paged_layout(lengths: np.ndarray, page_size: int, seed: int, max_blocks: int | None = None,
                 extra_pages: int = 0) -> PagedLayout:
    """Pool of sum(ceil(len/page)) pages (+ ``extra_pages`` never referenced); sequence b takes a
    consecutive slice of a seeded random permutation of the pool."""
    nblk = [(int(n) + page_size - 1) // page_size for n in lengths]
    total = sum(nblk)
    num_pages = total + extra_pages
    mb = max(max(nblk) if nblk else 1, 1) if max_blocks is None else max_blocks
    perm = _stream(seed, T_PERM).permutation(num_pages).astype(np.int32)
    table = np.full((len(lengths), mb), -1, np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    return PagedLayout(page_size, num_pages, mb, table)


def build_contig_cache(cfg: DecodeCfg, tensor: int, lengths: np.ndarray, max_len: int,
                       pad_bits=None) -> np.ndarray:
    """[B, Hkv, max_len, d] bits (uint16 bf16, or uint8 E4M3 codes for an FP8 cache);
    slots at or past lengths[b] hold ``pad_bits`` (default: the element type's NaN)."""
    pad = kv_pad(cfg) if pad_bits is None else pad_bits
    c = np.full((cfg.B, cfg.Hkv, max_len, cfg.d), pad, type(kv_pad(cfg)))
    for b in range(cfg.B):
        n = int(lengths[b])
        for h in range(cfg.Hkv):
            c[b, h, :n] = decode_kv_logical(cfg, tensor, b, h, n)
    return c


def build_paged_cache(cfg: DecodeCfg, tensor: int, lengths: np.ndarray, layout: PagedLayout,
                      pad_bits=None) -> np.ndarray:
    """[num_pages, Hkv, page_size, d] bits (as in build_contig_cache); unused slots and
    pages hold ``pad_bits`` (default: the element type's NaN)."""
    ps = layout.page_size
    pad = kv_pad(cfg) if pad_bits is None else pad_bits
    etype = type(kv_pad(cfg))
    pool = np.full((layout.num_pages, cfg.Hkv, ps, cfg.d), pad, etype)
    for b in range(cfg.B):
        n = int(lengths[b])
        nblk = (n + ps - 1) // ps
        pages = layout.block_table[b, :nblk]
        for h in range(cfg.Hkv):
            rows = decode_kv_logical(cfg, tensor, b, h, n)
            padded = np.full((nblk * ps, cfg.d), pad, etype)
            padded[:n] = rows
            pool[pages, h] = padded.reshape(nblk, ps, cfg.d)
    return pool


# ----------------------------------------------------------------------------
# Work counting (for throughput figures; no attention arithmetic)
# ----------------------------------------------------------------------------
def visible_pairs(Nq: int, Nk: int, causal: bool) -> int:
    """Number of (query, key) pairs a row-wise softmax sees.  Causal masking is
    aligned bottom-right: key j is visible to query i iff j <= i + (Nk - Nq)."""
    if not causal:
        return Nq * Nk
    if Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    off = Nk - Nq
    # row i sees i + off + 1 keys (never more than Nk since i <= Nq - 1)
    return Nq * (off + 1) + Nq * (Nq - 1) // 2


def prefill_flops(cfg: PrefillCfg) -> int:
    """Algorithmic FLOPs: 2*d for Q.K^T plus 2*d for P.V per visible pair."""
    return 4 * cfg.d * cfg.B * cfg.Hq * visible_pairs(cfg.Nq, cfg.Nk, cfg.causal)


def backward_flops(cfg: PrefillCfg) -> int:
    """Algorithmic FLOPs of the backward: five products of 2*d per visible pair each
    (dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q, and S = Q K^T recomputed), i.e.
    2.5x the forward's count; the second recomputation of S and dP that a two-pass
    kernel does is not counted."""
    return 10 * cfg.d * cfg.B * cfg.Hq * visible_pairs(cfg.Nq, cfg.Nk, cfg.causal)


def prefill_bytes(cfg: PrefillCfg) -> int:
    """Algorithmic HBM bytes: Q, K, V read once, O written once, LSE written once (FP8
    inputs are 1 byte per element; O is 2 bytes either way)."""
    eb = 1 if cfg.fp8 else 2
    q = cfg.B * cfg.Hq * cfg.Nq * cfg.d
    kv = 2 * cfg.B * cfg.Hkv * cfg.Nk * cfg.d * eb
    return q * eb + kv + q * 2 + cfg.B * cfg.Hq * cfg.Nq * 4


def decode_bytes(cfg: DecodeCfg, lengths: np.ndarray) -> int:
    """Algorithmic HBM bytes of one decode step: K and V of the live tokens, Q, O,
    LSE, the lengths and (paged) the live block-table entries."""
    tot = int(np.sum(lengths, dtype=np.int64))
    kv = 2 * tot * cfg.Hkv * cfg.d * (1 if cfg.kv_fp8 else 2)
    qo = 2 * cfg.B * cfg.Hq * cfg.d * 2
    lse = cfg.B * cfg.Hq * 4
    lens = cfg.B * 4
    table = 0
    if cfg.paged:
        table = 4 * sum((int(n) + cfg.page_size - 1) // cfg.page_size for n in lengths)
    return kv + qo + lse + lens + table


def decode_flops(cfg: DecodeCfg, lengths: np.ndarray) -> int:
    return 4 * cfg.d * cfg.Hq * int(np.sum(lengths, dtype=np.int64))


def varlen_flops(lens_q, lens_k, Hq: int, d: int, causal: bool) -> int:
    """Algorithmic FLOPs of a ragged batch: 4*d per visible pair of each sequence."""
    return 4 * d * Hq * sum(visible_pairs(int(a), int(b), causal) for a, b in zip(lens_q, lens_k)
                            if a > 0)


def chunk_q(cfg: DecodeCfg) -> np.ndarray:
    """Chunked-prefill queries [B, Hq, chunk, d] bf16 bits (with an FP8 cache: E4M3 codes
    of the same draws over FP8_Q_SCALE)."""
    q = np.empty((cfg.B, cfg.Hq, cfg.chunk, cfg.d), np.uint8 if cfg.kv_fp8 else np.uint16)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            if cfg.kv_fp8:
                q[b, h] = normal_e4m3(cfg.seed, T_Q, b, h, (cfg.chunk, cfg.d), FP8_Q_SCALE)
            else:
                q[b, h] = normal_bf16(cfg.seed, T_Q, b, h, (cfg.chunk, cfg.d), f16=cfg.f16)
    return q


def chunk_prefill_flops(cfg: DecodeCfg, lengths: np.ndarray, causal: bool = True) -> int:
    """Algorithmic FLOPs of a chunked prefill: 4*d per visible pair, the chunk's queries
    being the last ``chunk`` positions of each sequence."""
    pairs = sum(visible_pairs(cfg.chunk, int(n), causal) for n in lengths)
    return 4 * cfg.d * cfg.Hq * pairs
