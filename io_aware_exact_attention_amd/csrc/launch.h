// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk;
  float c;        // |scale| * log2(e)
  int negate_q;   // scale < 0: Q's sign is flipped on load (exact) so c >= 0
  int num_qtiles; // filled by launch_prefill
  int total_wg;   // filled by launch_prefill
  int head_group; // filled by launch_prefill: heads whose query tiles are interleaved
  // Paged K/V (block_table non-null): k, v are [pages, Hkv, 16, d] pools, sequence b has
  // kv_lens[b] keys (its last Nq are the queries' own positions) in pages
  // block_table[b, 0 .. max_blocks); Nk is then the largest kv_lens value.
  const int32_t* block_table;
  const int32_t* kv_lens;
  int max_blocks;
  uint32_t page_max;  // num_pages - 1: page ids are clamped to it
  int f16;  // Q, K, V, O are fp16 (else bf16)
  // FP8 (dense or paged layout): Q, K, V are E4M3 codes, O is bf16; c then carries the Q and
  // K scales, and v_scale multiplies the normalised output.
  int fp8;
  float v_scale;
  // Varlen (cu_q non-null): q, o are [total_q, Hq, D] and k, v [total_k, Hkv, D], sequence
  // b owning rows [cu_q[b], cu_q[b+1]) and [cu_k[b], cu_k[b+1]); lse is [Hq, total_q].
  // Nq and Nk are then the longest sequence's lengths.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
};

struct DecodeParams {
  const uint16_t* q;
  const void* kc;  // bf16, or E4M3 codes when kv_fp8
  const void* vc;
  const int32_t* block_table;  // null: contiguous cache
  const int32_t* seqlens;
  uint16_t* o;
  float* lse;
  float* ws_o;    // [B, Hq, num_splits, d] fp32 partial outputs (num_splits > 1)
  float* ws_lse;  // [B, Hq, num_splits] fp32 partial log-sum-exps
  int B, Hq, Hkv, G, ngroups;
  int max_seqlen;  // row count of the contiguous cache
  int max_blocks;  // block-table row length (paged)
  uint32_t page_max;  // num_pages - 1 (paged): page ids are clamped to it
  int num_splits, chunk;
  float c;        // |scale| * log2(e), times the K scale of an FP8 cache
  int negate_q;
  int kv_fp8;     // K/V caches hold E4M3 codes
  float v_scale;  // FP8 cache: multiplies the normalised output
  int f16;        // Q, O and the cache are fp16 (else bf16; never with kv_fp8)
};

// Queries one prefill workgroup owns (8 waves of 32): the grid has ceil(Nq / this) query
// tiles per head.
constexpr int kPrefillRows = 256;
// Queries (dQ pass) or keys (dK/dV pass) one backward workgroup owns.
constexpr int kBwdRows = 128;

// Query heads sharing one KV head that a decode workgroup serves at once.
constexpr int kDecodeHeadsPerGroup = 16;
// Keys one decode wave consumes per step; chunks are multiples of it.
constexpr int kDecodeBlock = 32;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeMaxSplits = 1024;  // chunks per sequence, at most

// Backward (bf16 or fp16): gradients of the prefill attention.  Layouts as for prefill; dvec and
// nlse are [B, Hq, Nq] fp32 workspace arrays for -D = -rowsum(dO * O) and -LSE * log2(e),
// written by the first kernel and read by the second.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;  // [B, Hq, Nq] natural-log log-sum-exp of the forward
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dvec;
  float* nlse;
  int B, Hq, Hkv, Nq, Nk;
  float scale;  // signed softmax scale
  float c;      // scale * log2(e), signed
  int f16;      // fp16 tensors (else bf16)
};

hipError_t launch_prefill(PrefillParams p, int d, int causal, hipStream_t stream);
hipError_t launch_backward(const BwdParams& p, int d, int causal, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream);

// Bytes of the per-GPU static array that holds the split-KV partials of the
// allocation-free decode entry point.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
// Device address of that array on the current device (looked up once per device).
hipError_t decode_scratch(void** ptr);

}  // namespace miattn
