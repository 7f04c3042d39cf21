/*
 * miattn — fused exact attention forward for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Computes O = softmax(scale * Q K^T [+ causal mask]) V without ever writing the
 * N x N score matrix to memory: key/value tiles are streamed through on-chip memory
 * and the softmax is accumulated online (running row max m, running sum l, rescaled
 * partial output).
 *
 * Sources for what is computed:
 *  - the definition softmax(Q K^T / sqrt(d_k)) V: page "FlashAttention 완전 정리"
 *    (cell-devlog), section "Attention이 뭔가" (what attention is);
 *  - tiling with the score matrix kept on chip, and the online softmax that makes the
 *    blockwise result exact: same page, section "FlashAttention의 핵심 아이디어 —
 *    Tiling" (core idea: tiling); m, f, l definitions: page "Flash Attention: GPU
 *    메모리_IO를 최적화하는 어텐션 메커니즘 완전 가이드" (holysheep), section
 *    "수학적 원리: Online Softmax 알고리즘";
 *  - separate prefill and decode kernels, decode as a single query against a growing
 *    KV cache, and paged KV caches: page "메모리 장벽을 넘어: LLM 연산자 가속 라이브러리
 *    심층 분석" (tiptinker), section "2. FlashInfer";
 *  - the call shape (q, k, v, softmax_scale, causal) and the caller-side checks (device
 *    tensors, bf16, contiguous memory): same page, section "최적화된 어텐션 순전파
 *    (Forward Pass)".
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE memory owned by the caller.  The library never
 *    allocates, frees or synchronises; every call is asynchronous on `stream`
 *    (0 = the null stream) and its outputs are valid once the stream reaches it.
 *  - Tensors are dense, contiguous, row-major, in the layouts stated per argument; no
 *    strides are taken.  bf16 and fp16 tensors are passed as `const void*` (16-bit
 *    patterns); the entry points with the _f16 suffix take IEEE fp16 where the others
 *    take bf16.
 *    Outputs must not alias inputs.
 *  - Every call returns an attn_status_t.  Arguments are validated before any HIP call;
 *    a failed validation launches nothing.  Nothing throws across this interface.
 *  - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 *  - Causal masking is aligned bottom-right: key j is visible to query i iff
 *    j <= i + (Nk - Nq).  Causal with Nq > Nk is rejected.
 *  - LSE is the natural-log log-sum-exp of the scaled visible scores of a row,
 *    m + ln(l), in fp32.
 *  - Supported head dimensions: d in {64, 128}.  Inputs must be finite.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, non-finite scale */
  ATTN_ERR_UNSUPPORTED = 2,      /* d not in {64,128}, page_size != 16, too large a grid */
  ATTN_ERR_WORKSPACE = 3,        /* decode workspace missing or too small */
  ATTN_ERR_HIP = 4               /* the HIP runtime reported a launch error */
} attn_status_t;

/*
 * Prefill: many queries per sequence.
 *
 * Defined by: the forward call of the page "메모리 장벽을 넘어: LLM 연산자 가속 라이브러리
 * 심층 분석" (tiptinker), section "최적화된 어텐션 순전파 (Forward Pass)" (q, k, v, a softmax
 * scale and a causal flag; bf16 device tensors in contiguous memory), computing the
 * attention of the page "FlashAttention 완전 정리" (cell-devlog), section "Attention이
 * 뭔가", tile by tile as in its section "FlashAttention의 핵심 아이디어 — Tiling" (Q, K,
 * V read once and O written once; the score matrix never leaves the chip).  The layout is
 * [B, H, N, d] as in that page's scaled-dot-product example (the tiptinker page's call
 * documents [B, N, H, d]; the two conflict and [B, H, N, d] is kept).  Dropout, which that
 * call also takes, is not offered (probability 0).
 *
 *   q    [B, Hq,  Nq, d] bf16, 16-byte aligned
 *   k, v [B, Hkv, Nk, d] bf16, 16-byte aligned
 *   o    [B, Hq,  Nq, d] bf16 (written), 16-byte aligned
 *   lse  [B, Hq,  Nq]    fp32 (written) or NULL to skip it, 4-byte aligned
 *   causal != 0 applies the bottom-right causal mask.
 *   scale multiplies Q K^T before the softmax (usually 1/sqrt(d)); any finite value.
 *
 * Errors: INVALID_ARGUMENT for a null q/k/v/o, misalignment, any size < 1,
 * Hq % Hkv != 0, causal with Nq > Nk, non-finite scale; UNSUPPORTED for d not in
 * {64,128}, a grid beyond 2^31-1 workgroups, or Nk*d*2 beyond 2^31-1 bytes (one head's
 * K must fit a 32-bit buffer range); HIP if the launch fails.
 */
int attn_fwd_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                     hipStream_t stream);

/* attn_fwd_prefill with q, k, v and o in IEEE fp16 instead of bf16: the same layouts,
 * arguments and errors.  The products run on the fp16 MFMA with fp32 accumulation, P is
 * rounded to fp16 (nearest even) before P*V and o is rounded to fp16 (nearest even).  Each
 * output row is a convex combination of V rows, so it stays in fp16 range when V does. */
int attn_fwd_prefill_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         hipStream_t stream);

/*
 * Prefill over FP8 inputs: attn_fwd_prefill with q, k and v stored as OCP FP8 E4M3 codes
 * (1 byte per element, the format of attn_fwd_decode_fp8) and one scale per tensor, so
 * the query is q_scale * e4m3(code), and likewise the key (k_scale) and value (v_scale).
 * The FP8 support of the page "FlashAttention 완전 정리" (cell-devlog), section
 * "FlashAttention 버전별 발전", subsection "FlashAttention 3".  Q K^T runs on the FP8
 * matrix cores: every product is exact, but the matrix core sums each group of 64 products
 * with reduced precision (measured errors up to about 2^-11 of the group's largest
 * product, far above fp32 rounding).  V is widened to bf16 exactly, P is rounded to
 * bf16 (nearest even) before P*V, and o is bf16 as in attn_fwd_prefill.
 *
 *   q    [B, Hq,  Nq, d] uint8 codes, 16-byte aligned
 *   k, v [B, Hkv, Nk, d] uint8 codes, 16-byte aligned
 *   o    [B, Hq,  Nq, d] bf16 (written), 16-byte aligned
 *   lse  [B, Hq,  Nq]    fp32 (written) or NULL, of the dequantised scores
 *   q_scale, k_scale, v_scale  finite and > 0.
 *   All other arguments are those of attn_fwd_prefill.
 *
 * Errors: those of attn_fwd_prefill (with Nk*d beyond 2^31-1 bytes for UNSUPPORTED),
 * plus INVALID_ARGUMENT for a non-finite or non-positive q_scale, k_scale or v_scale, or
 * when |scale| * q_scale * k_scale overflows float.
 */
int attn_fwd_prefill_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         float q_scale, float k_scale, float v_scale, hipStream_t stream);

/*
 * Chunked (append) prefill against a paged KV cache: the Nq newest tokens of every
 * sequence attend to that sequence's whole cached context, which already holds their
 * own keys and values as its last Nq tokens.  This is the prefill step of chunked
 * prefill / continuous batching (page "Transformers optimization overview", section on
 * continuous batching) over a paged cache (page "메모리 장벽을 넘어" (tiptinker),
 * section "2. FlashInfer", PagedAttention integration).  Query i of sequence b sits at
 * position kv_lens[b] - Nq + i; causal != 0 lets it see keys 0 .. that position.
 *
 *   q      [B, Hq, Nq, d] bf16, 16-byte aligned
 *   kcache, vcache [num_pages, Hkv, page_size, d] bf16, 16-byte aligned, page_size == 16
 *   block_table [B, max_blocks_per_seq] int32, DEVICE memory: token t of sequence b is
 *          slot t % 16 of page block_table[b, t / 16].  Entries for tokens < kv_lens[b]
 *          must lie in [0, num_pages); other entries are never read.  Entries outside
 *          that range are clamped into it on the device: the result is then unspecified,
 *          but no read leaves the cache.
 *   kv_lens [B] int32, DEVICE memory, each in [Nq, max_kv_len] (not read on the host);
 *          a value outside that range is clamped into it on the device: the result is
 *          then unspecified, but no read leaves the block table or the cache.
 *   o      [B, Hq, Nq, d] bf16 (written), 16-byte aligned
 *   lse    [B, Hq, Nq] fp32 (written) or NULL
 *   Needs max_blocks_per_seq >= ceil(max_kv_len / 16).  Cache rows at or past
 *   kv_lens[b] are never read.
 *
 * Errors: INVALID_ARGUMENT for a null required pointer, misalignment, any size < 1,
 * Hq % Hkv != 0, Nq > max_kv_len, max_blocks_per_seq too small, non-finite scale;
 * UNSUPPORTED for d not in {64,128}, page_size != 16 or a grid beyond 2^31-1
 * workgroups; HIP if the launch fails.
 */
int attn_fwd_prefill_paged(const void* q, const void* kcache, const void* vcache,
                           const int32_t* block_table, const int32_t* kv_lens, void* o,
                           float* lse, int B, int Hq, int Hkv, int Nq, int d, int max_kv_len,
                           int page_size, int max_blocks_per_seq, int num_pages, int causal,
                           float scale, hipStream_t stream);

/*
 * Chunked prefill against an FP8 paged cache: attn_fwd_prefill_paged with the caches in
 * the E4M3 format and per-tensor scales of attn_fwd_decode_fp8 (the cache that FP8 decode
 * reads) and the queries as E4M3 codes with their own scale, computed as
 * attn_fwd_prefill_fp8 computes (Q K^T on the FP8 matrix cores, V widened to bf16, bf16
 * P and o).
 *
 *   q      [B, Hq, Nq, d] uint8 codes, 16-byte aligned
 *   kcache, vcache [num_pages, Hkv, 16, d] uint8 codes, 16-byte aligned
 *   o      [B, Hq, Nq, d] bf16 (written)
 *   q_scale, k_scale, v_scale  finite and > 0.
 *   All other arguments, the table and length contracts and the outputs are those of
 *   attn_fwd_prefill_paged.
 *
 * Errors: those of attn_fwd_prefill_paged, plus INVALID_ARGUMENT for a non-finite or
 * non-positive scale, or when |scale| * q_scale * k_scale overflows float.
 */
int attn_fwd_prefill_paged_fp8(const void* q, const void* kcache, const void* vcache,
                               const int32_t* block_table, const int32_t* kv_lens, void* o,
                               float* lse, int B, int Hq, int Hkv, int Nq, int d, int max_kv_len,
                               int page_size, int max_blocks_per_seq, int num_pages, int causal,
                               float scale, float q_scale, float k_scale, float v_scale,
                               hipStream_t stream);

/* attn_fwd_prefill_paged with fp16 q, caches and o (as in attn_fwd_prefill_f16). */
int attn_fwd_prefill_paged_f16(const void* q, const void* kcache, const void* vcache,
                               const int32_t* block_table, const int32_t* kv_lens, void* o,
                               float* lse, int B, int Hq, int Hkv, int Nq, int d, int max_kv_len,
                               int page_size, int max_blocks_per_seq, int num_pages, int causal,
                               float scale, hipStream_t stream);

/*
 * Variable-length (ragged) batched prefill: B sequences of different lengths packed along
 * the token axis, the batch shape of continuous batching (page "Transformers optimization
 * overview", section on continuous batching).  Sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b], cu_seqlens_k[b+1]);
 * its queries attend only to its own keys (bottom-right aligned when causal, per sequence).
 *
 *   q, o   [total_q, Hq, d] bf16 (token-major)      k, v  [total_k, Hkv, d] bf16
 *   lse    [Hq, total_q] fp32 (written) or NULL
 *   cu_seqlens_q, cu_seqlens_k  [B + 1] int32, DEVICE memory (not read on the host):
 *          cu[0] = 0, non-decreasing, cu[B] = total.  Sequence lengths must not exceed
 *          max_seqlen_q / max_seqlen_k.  The grid is sized on the host from these
 *          arguments (up to 64 sequences: floor((total_q + 255*B) / 256) query tiles
 *          per head, mapped to sequences on the device; beyond 64: max_seqlen_q's tiles
 *          for every sequence), so lengths that break these rules leave some rows
 *          unwritten, but never make a read or write leave the tensors.  A sequence
 *          with queries needs at least one key (and, when causal, at least as many keys as queries: a causal
 *          row that sees no key gets undefined values); one with no queries is skipped.
 *          Values are clamped to [0, total] on the device, so no value reads outside the
 *          tensors; a sequence with no keys gets o = 0 and lse = -inf.
 *
 * Errors: INVALID_ARGUMENT for a null required pointer, misalignment, any size < 1,
 * Hq % Hkv != 0, a max length above its total, a non-finite scale; UNSUPPORTED for d not
 * in {64,128} or a grid beyond 2^31-1 workgroups; HIP if the launch fails.
 */
int attn_fwd_prefill_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                            int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                            int max_seqlen_k, int d, int causal, float scale,
                            hipStream_t stream);

/*
 * Variable-length prefill over FP8 inputs: attn_fwd_prefill_varlen with q, k and v packed
 * as E4M3 codes (the token-major layouts, one byte per element) and the per-tensor scales
 * of attn_fwd_prefill_fp8, computed as attn_fwd_prefill_fp8 computes; o is bf16.
 *
 * Errors: those of attn_fwd_prefill_varlen, plus INVALID_ARGUMENT for a non-finite or
 * non-positive q_scale, k_scale or v_scale, or when |scale| * q_scale * k_scale overflows
 * float.
 */
int attn_fwd_prefill_varlen_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                int max_seqlen_k, int d, int causal, float scale, float q_scale,
                                float k_scale, float v_scale, hipStream_t stream);

/* attn_fwd_prefill_varlen with fp16 q, k, v and o (as in attn_fwd_prefill_f16). */
int attn_fwd_prefill_varlen_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                int max_seqlen_k, int d, int causal, float scale,
                                hipStream_t stream);

/*
 * Decode: one query per sequence against the sequence's KV cache, split along the
 * KV length into chunks whose partial results are merged by log-sum-exp.
 *
 * Defined by: the page "메모리 장벽을 넘어: LLM 연산자 가속 라이브러리 심층 분석"
 * (tiptinker), section "2. FlashInfer": decode as a separate kernel in which the newest
 * token's query attends to the KV cache of everything before it, with the cache held in
 * fixed-size pages (PagedAttention) reached through a per-sequence page table.  The
 * chunked split and its merge are not on the pages: a chunk's (m, l) and partial output
 * combine exactly under the m, f, l definitions of the page "Flash Attention: GPU
 * 메모리_IO를 최적화하는 어텐션 메커니즘 완전 가이드" (holysheep), section "수학적 원리:
 * Online Softmax 알고리즘".
 *
 *   q        [B, Hq, d] bf16
 *   o        [B, Hq, d] bf16 (written)
 *   lse      [B, Hq] fp32 (written) or NULL
 *   seqlens  [B] int32, DEVICE memory, each in [0, max_seqlen] (not read on the host);
 *            seqlens[b] == 0 gives o = 0 and lse = -inf for that sequence.
 *   Contiguous cache (block_table == NULL):
 *     kcache, vcache [B, Hkv, max_seqlen, d] bf16; token t of sequence b is row t.
 *     page_size, max_blocks_per_seq and num_pages are ignored.
 *   Paged cache (block_table != NULL):
 *     kcache, vcache [num_pages, Hkv, page_size, d] bf16 with page_size == 16;
 *     block_table [B, max_blocks_per_seq] int32, DEVICE memory; token t of sequence b
 *     is slot t % page_size of page block_table[b, t / page_size].  Entries for
 *     tokens < seqlens[b] must lie in [0, num_pages); other entries are never read.
 *     Entries outside that range are clamped into it on the device: the result is then
 *     unspecified, but no read leaves the cache.
 *     Needs max_blocks_per_seq >= ceil(max_seqlen / page_size).
 *   Cache rows at or past seqlens[b] are never read (they may hold anything).
 *   num_splits: number of KV chunks per sequence; 0 picks one automatically.  The
 *     count actually used is attn_decode_num_splits(...) of the same arguments.
 *   workspace: device scratch of at least attn_decode_workspace_bytes(...) bytes,
 *     16-byte aligned; may be NULL when that size is 0.  Its contents on entry do
 *     not matter; calls that share one workspace must be ordered on one stream.
 *
 * Errors: INVALID_ARGUMENT for a null required pointer, misalignment, any size < 1,
 * Hq % Hkv != 0, max_blocks_per_seq too small, num_splits < 0, non-finite scale;
 * UNSUPPORTED for d not in {64,128} or page_size != 16; WORKSPACE when the workspace
 * is missing or too small; HIP if a launch fails.
 */
int attn_fwd_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                    int B, int Hq, int Hkv, int d, int max_seqlen, int page_size,
                    int max_blocks_per_seq, int num_pages, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size in bytes of the per-GPU array that attn_fwd_decode_noalloc keeps its split-KV
 * partials in: 32 MiB. */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)

/*
 * attn_fwd_decode without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops that must not call hipMalloc, and
 * harnesses that forbid allocation.  The call itself calls no hipMalloc, hipFree or other
 * allocating routine.
 *
 * The split-KV partials go to a static device array of ATTN_DECODE_NOALLOC_MAX_BYTES that
 * the library holds on every GPU it runs on until the process ends (one copy per GPU,
 * looked up once per device on that device's first call).  Arguments, layouts, chunking,
 * outputs and results are those of attn_fwd_decode with the same arguments; the need is
 * attn_decode_workspace_bytes of them (for the call's own Hkv), and a call whose need
 * exceeds ATTN_DECODE_NOALLOC_MAX_BYTES returns WORKSPACE without launching anything.
 * Nothing in the array has to start at zero (every partial the merge reads is written by
 * the same call).  All calls on one GPU share its array: calls that may overlap on one GPU
 * (different streams without ordering between them) race and give wrong results.
 *
 * Errors: those of attn_fwd_decode (WORKSPACE as above); HIP if the array's device address
 * cannot be obtained or a launch fails.
 */
int attn_fwd_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* block_table, const int32_t* seqlens, void* o,
                            float* lse, int B, int Hq, int Hkv, int d, int max_seqlen,
                            int page_size, int max_blocks_per_seq, int num_pages, float scale,
                            int num_splits, hipStream_t stream);

/* attn_fwd_decode with fp16 q, caches and o (as in attn_fwd_prefill_f16): the same
 * layouts, chunking, workspace and errors. */
int attn_fwd_decode_f16(const void* q, const void* kcache, const void* vcache,
                        const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                        int B, int Hq, int Hkv, int d, int max_seqlen, int page_size,
                        int max_blocks_per_seq, int num_pages, float scale, int num_splits,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode over an FP8 KV cache: attn_fwd_decode with K and V stored as OCP FP8 E4M3 codes
 * (1 byte per element: sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities; codes 0x7F and 0xFF are NaN) and one scale per tensor, so the cached key
 * is k_scale * e4m3(code) and the cached value v_scale * e4m3(code).  Compressed (FP8)
 * KV caches, which halve the bytes decode streams: page "메모리 장벽을 넘어: LLM 연산자
 * 가속 라이브러리 심층 분석" (tiptinker), section "2. FlashInfer".
 *
 *   kcache, vcache  uint8 codes in the layouts of attn_fwd_decode ([B, Hkv, max_seqlen, d]
 *                   contiguous, or [num_pages, Hkv, 16, d] paged), 16-byte aligned.
 *   k_scale, v_scale  finite and > 0.
 *   All other arguments, the chunking (attn_decode_num_splits), the workspace
 *   (attn_decode_workspace_bytes) and the outputs are those of attn_fwd_decode.
 *
 * Errors: those of attn_fwd_decode, plus INVALID_ARGUMENT for a non-finite or
 * non-positive k_scale or v_scale, or when |scale| * k_scale overflows float.
 */
int attn_fwd_decode_fp8(const void* q, const void* kcache, const void* vcache,
                        const int32_t* block_table, const int32_t* seqlens, void* o,
                        float* lse, int B, int Hq, int Hkv, int d, int max_seqlen,
                        int page_size, int max_blocks_per_seq, int num_pages, float scale,
                        float k_scale, float v_scale, int num_splits, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Number of KV chunks attn_fwd_decode (and its _f16 and _fp8 variants) uses for these arguments
 * (num_splits 0 = auto).
 * Returns 0 for invalid arguments.  Pure host arithmetic; no HIP call. */
int attn_decode_num_splits(int B, int Hq, int Hkv, int d, int max_seqlen, int num_splits);

/* Workspace bytes that suffice for attn_fwd_decode (and its _f16 and _fp8 variants) with
 * these B, Hq, d, max_seqlen and num_splits (0 = auto) and any valid Hkv: fp32 partial
 * outputs and log-sum-exps, B*Hq*splits*(d+1)*4 rounded up to 256, where splits is the
 * largest chunk count the plan picks for any Hkv dividing Hq (the automatic plan uses more
 * chunks when fewer KV heads fill the grid), or 0 when one chunk always suffices.  The
 * count for a given Hkv is attn_decode_num_splits.
 * Returns 0 for invalid arguments (any size < 1, num_splits < 0).  Pure host arithmetic;
 * no HIP call. */
size_t attn_decode_workspace_bytes(int B, int Hq, int d, int max_seqlen, int num_splits);

/*
 * Backward of attn_fwd_prefill (bf16): the gradients dq, dk, dv of the attention output
 * for the output gradient dout, recomputing the attention weights tile by tile from the
 * forward's LSE instead of storing them (tiling and recomputation: page "메모리 장벽을
 * 넘어: LLM 연산자 가속 라이브러리 심층 분석" (tiptinker), section "1. FlashAttention").
 * The gradients are those of O = softmax(scale * Q K^T [+ causal mask]) V:
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),  dQ = scale * dS K,  dK = scale * dS^T Q,
 * with dK, dV of a KV head summed over the query heads that read it.
 *
 *   q, o, dout, dq  [B, Hq, Nq, d] bf16      k, v, dk, dv  [B, Hkv, Nk, d] bf16
 *   lse             [B, Hq, Nq] fp32: the LSE attn_fwd_prefill wrote for
 *                   the same q, k, v, causal and scale (o likewise its output).
 *   workspace       at least attn_bwd_workspace_bytes(B, Hq, Nq) bytes of device memory,
 *                   16-byte aligned; its contents on entry do not matter.  Calls sharing it
 *                   must be ordered on one stream.
 *   dq, dk, dv are written in full (no accumulation into existing contents).  Results are
 *   deterministic: no atomics are used.
 *
 * Errors: INVALID_ARGUMENT for a null or misaligned pointer, any size < 1, Hq % Hkv != 0,
 * causal with Nq > Nk, a non-finite scale; UNSUPPORTED for d not in {64,128}, a grid
 * beyond 2^31-1 workgroups, or one head's rows beyond 2^31-1 bytes; WORKSPACE when the
 * workspace is missing or too small; HIP if a launch fails.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
             hipStream_t stream);

/* attn_bwd with fp16 q, k, v, o, dout, dq, dk and dv (the backward of attn_fwd_prefill_f16);
 * products take fp16 operands, accumulation and the softmax terms stay fp32. */
int attn_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Workspace bytes attn_bwd (and attn_bwd_f16) needs: B*Hq*Nq*8 (two fp32 row terms per
 * query, rowsum(dO * O) and -LSE*log2(e)) rounded up to 256.  Returns 0 for invalid
 * arguments.  Pure host arithmetic; no HIP call. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq);

/* Static, human-readable text for a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
