// C-ABI entry points of libmiattn: argument validation (before any HIP call), launch
// planning (kernel instance, grid, decode chunking, workspace layout) and launch on the
// caller's stream.  The library never allocates, frees or synchronises.
//
// The caller-side checks mirror the ones shown before the forward call on the page
// "메모리 장벽을 넘어: LLM 연산자 가속 라이브러리 심층 분석" (tiptinker), section
// "최적화된 어텐션 순전파 (Forward Pass)": device tensors, bf16, contiguous memory.  Here
// they are reported as status codes instead of silent casts and copies.

#include <cmath>
#include <cstdint>

#include "../../include/miattn.h"
#include "launch.h"

static_assert(miattn::kDecodeScratchBytes == ATTN_DECODE_NOALLOC_MAX_BYTES,
              "the header states the size of the allocation-free decode's array");

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Decode chunking: chunk = ceil(max_seqlen / splits) rounded up to a whole number of
// 32-key blocks; the split count actually used is ceil(max_seqlen / chunk).
struct Plan {
  int splits;
  int chunk;
};

constexpr int kTargetChunk = 1024;      // keys per chunk in the automatic plan
constexpr int kMinWorkgroups = 2048;    // ~8 per compute unit on 256 CUs
constexpr int kMinChunk = 256;          // smallest chunk the plan uses to reach that

bool decode_sizes_ok(int B, int Hq, int Hkv, int d, int max_seqlen) {
  if (B < 1 || Hq < 1 || Hkv < 1 || max_seqlen < 1) return false;
  if (Hq % Hkv) return false;
  (void)d;
  return true;
}

Plan plan_decode(int B, int Hq, int Hkv, int max_seqlen, int num_splits) {
  const int G = Hq / Hkv;
  const int ngroups = (G + miattn::kDecodeHeadsPerGroup - 1) / miattn::kDecodeHeadsPerGroup;
  int want = num_splits;
  if (want <= 0) {
    // chunks of ~kTargetChunk keys; shorter ones (down to kMinChunk) only when the grid
    // would otherwise have fewer than kMinWorkgroups workgroups
    const long base = (long)B * Hkv * ngroups;
    long s = ((long)max_seqlen + kTargetChunk - 1) / kTargetChunk;
    if (base * s < kMinWorkgroups) {
      const long cap = ((long)max_seqlen + kMinChunk - 1) / kMinChunk;
      s = (kMinWorkgroups + base - 1) / base;
      if (s > cap) s = cap;
    }
    want = (int)(s < 1 ? 1 : s);
  }
  if (want > miattn::kDecodeMaxSplits) want = miattn::kDecodeMaxSplits;
  const int blk = miattn::kDecodeBlock;
  long chunk = ((long)max_seqlen + want - 1) / want;
  chunk = (chunk + blk - 1) / blk * blk;
  const int splits = (int)(((long)max_seqlen + chunk - 1) / chunk);
  return Plan{splits, (int)chunk};
}

size_t workspace_for(int B, int Hq, int d, const Plan& pl) {
  if (pl.splits <= 1) return 0;
  const size_t n = (size_t)B * Hq * pl.splits;
  const size_t bytes = n * (size_t)d * 4 + n * 4;
  return (bytes + 255) / 256 * 256;
}

// Both decode entry points: the cache element type (bf16 or E4M3 codes) changes the
// kernel instance, the exponent scale (times k_scale) and the output scale (v_scale).
int decode_impl(const void* q, const void* kcache, const void* vcache,
                const int32_t* block_table, const int32_t* seqlens, void* o, float* lse, int B,
                int Hq, int Hkv, int d, int max_seqlen, int page_size, int max_blocks_per_seq,
                int num_pages, float scale, bool fp8, bool f16, float k_scale, float v_scale,
                int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream,
                bool static_scratch = false) {
  if (!q || !kcache || !vcache || !seqlens || !o) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kcache, 16) || !aligned(vcache, 16) || !aligned(o, 16) ||
      !aligned(seqlens, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  if (!decode_sizes_ok(B, Hq, Hkv, d, max_seqlen) || d < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (num_splits < 0 || !std::isfinite(scale)) return ATTN_ERR_INVALID_ARGUMENT;
  if (block_table) {
    if (!aligned(block_table, 4) || num_pages < 1) return ATTN_ERR_INVALID_ARGUMENT;
    if (page_size != 16) return ATTN_ERR_UNSUPPORTED;
    if (max_blocks_per_seq < (max_seqlen + page_size - 1) / page_size)
      return ATTN_ERR_INVALID_ARGUMENT;
  }
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  const int ngroups = (G + miattn::kDecodeHeadsPerGroup - 1) / miattn::kDecodeHeadsPerGroup;
  if (B > 65535 || (long)Hkv * ngroups > 65535 || (long)B * Hq > 0x7fffffffL)
    return ATTN_ERR_UNSUPPORTED;

  const Plan pl = plan_decode(B, Hq, Hkv, max_seqlen, num_splits);
  const size_t need = workspace_for(B, Hq, d, pl);
  if (static_scratch && need) {
    // the library's per-GPU array instead of a caller workspace (after all validation)
    if (need > miattn::kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
    if (miattn::decode_scratch(&workspace) != hipSuccess) return ATTN_ERR_HIP;
    workspace_bytes = miattn::kDecodeScratchBytes;
  }
  if (need) {
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  }

  miattn::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kc = kcache;
  p.vc = vcache;
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.ws_o = need ? static_cast<float*>(workspace) : nullptr;
  p.ws_lse = need ? p.ws_o + (size_t)B * Hq * pl.splits * d : nullptr;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = G; p.ngroups = ngroups;
  p.max_seqlen = max_seqlen;
  p.max_blocks = block_table ? max_blocks_per_seq : 0;
  p.page_max = block_table ? (uint32_t)(num_pages - 1) : 0u;
  p.num_splits = pl.splits;
  p.chunk = pl.chunk;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  if (fp8) p.c *= k_scale;
  if (!std::isfinite(p.c)) return ATTN_ERR_INVALID_ARGUMENT;
  p.negate_q = scale < 0.f;
  p.kv_fp8 = fp8;
  p.f16 = f16;
  p.v_scale = v_scale;
  (void)hipGetLastError();
  return miattn::launch_decode(p, d, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// The prefill entry points (bf16 or fp16 elements).
// (and, with fp8, the FP8 one: E4M3 q, k, v with per-tensor scales, bf16 o).
int prefill_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int Nq, int Nk, int d, int causal, float scale, bool f16,
                 hipStream_t stream, bool fp8 = false, float q_scale = 1.f,
                 float k_scale = 1.f, float v_scale = 1.f) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (Hq % Hkv) return ATTN_ERR_INVALID_ARGUMENT;
  if (causal && Nq > Nk) return ATTN_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const long qtiles = (Nq + miattn::kPrefillRows - 1) / miattn::kPrefillRows;
  if (qtiles * (long)Hq * B > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;
  if ((long)B * Hq > 0x7fffffffL || (long)B * Hkv > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;
  if (fp8 && !(std::isfinite(q_scale) && q_scale > 0.f && std::isfinite(k_scale) &&
               k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return ATTN_ERR_INVALID_ARGUMENT;
  // one head's K (or V) must fit a buffer descriptor's 32-bit byte range
  if ((long)Nk * d * (fp8 ? 1 : 2) > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;

  miattn::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  if (fp8) p.c *= q_scale * k_scale;
  if (!std::isfinite(p.c)) return ATTN_ERR_INVALID_ARGUMENT;
  p.negate_q = scale < 0.f;
  p.f16 = f16;
  p.fp8 = fp8;
  p.v_scale = v_scale;
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  return miattn::launch_prefill(p, d, causal ? 1 : 0, stream) == hipSuccess ? ATTN_OK
                                                                             : ATTN_ERR_HIP;
}

int prefill_paged_impl(const void* q, const void* kcache, const void* vcache,
                       const int32_t* block_table, const int32_t* kv_lens, void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int d, int max_kv_len, int page_size,
                       int max_blocks_per_seq, int num_pages, int causal, float scale, bool f16,
                       hipStream_t stream, bool fp8 = false, float q_scale = 1.f,
                       float k_scale = 1.f, float v_scale = 1.f) {
  if (!q || !kcache || !vcache || !block_table || !kv_lens || !o) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kcache, 16) || !aligned(vcache, 16) || !aligned(o, 16) ||
      !aligned(block_table, 4) || !aligned(kv_lens, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || d < 1 || max_kv_len < 1 || num_pages < 1)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (Hq % Hkv || Nq > max_kv_len || !std::isfinite(scale)) return ATTN_ERR_INVALID_ARGUMENT;
  if (page_size != 16) return ATTN_ERR_UNSUPPORTED;
  if (max_blocks_per_seq < (max_kv_len + 15) / 16) return ATTN_ERR_INVALID_ARGUMENT;
  if (fp8 && !(std::isfinite(q_scale) && q_scale > 0.f && std::isfinite(k_scale) &&
               k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const long qtiles = (Nq + miattn::kPrefillRows - 1) / miattn::kPrefillRows;
  if (qtiles * (long)Hq * B > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;

  miattn::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(kcache);
  p.v = static_cast<const uint16_t*>(vcache);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = max_kv_len;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  p.negate_q = scale < 0.f;
  p.block_table = block_table;
  p.kv_lens = kv_lens;
  p.max_blocks = max_blocks_per_seq;
  p.page_max = (uint32_t)(num_pages - 1);
  p.f16 = f16;
  if (fp8) p.c *= q_scale * k_scale;
  if (!std::isfinite(p.c)) return ATTN_ERR_INVALID_ARGUMENT;
  p.fp8 = fp8;
  p.v_scale = v_scale;
  (void)hipGetLastError();
  return miattn::launch_prefill(p, d, causal ? 1 : 0, stream) == hipSuccess ? ATTN_OK
                                                                             : ATTN_ERR_HIP;
}

// The varlen entry points (bf16 or fp16 elements).
int prefill_varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int Hq,
                        int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                        int d, int causal, float scale, bool f16, hipStream_t stream,
                        bool fp8 = false, float q_scale = 1.f, float k_scale = 1.f,
                        float v_scale = 1.f) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  if (B < 1 || Hq < 1 || Hkv < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 ||
      max_seqlen_k < 1 || d < 1)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (Hq % Hkv || max_seqlen_q > total_q || max_seqlen_k > total_k || !std::isfinite(scale))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (fp8 && !(std::isfinite(q_scale) && q_scale > 0.f && std::isfinite(k_scale) &&
               k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const long qtiles = (max_seqlen_q + miattn::kPrefillRows - 1) / miattn::kPrefillRows;
  if (qtiles * (long)Hq * B > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;
  // 64 key rows of the packed K (row stride Hkv*d*2 bytes) must fit a buffer descriptor
  if (64L * Hkv * d * 2 > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;

  miattn::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = max_seqlen_q; p.Nk = max_seqlen_k;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  p.negate_q = scale < 0.f;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  p.f16 = f16;
  if (fp8) p.c *= q_scale * k_scale;
  if (!std::isfinite(p.c)) return ATTN_ERR_INVALID_ARGUMENT;
  p.fp8 = fp8;
  p.v_scale = v_scale;
  (void)hipGetLastError();
  return miattn::launch_prefill(p, d, causal ? 1 : 0, stream) == hipSuccess ? ATTN_OK
                                                                             : ATTN_ERR_HIP;
}

// The backward entry points (bf16 or fp16 tensors).
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
             bool f16, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (Hq % Hkv || (causal && Nq > Nk) || !std::isfinite(scale)) return ATTN_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const long qtiles = (Nq + miattn::kBwdRows - 1) / miattn::kBwdRows;
  const long ktiles = (Nk + miattn::kBwdRows - 1) / miattn::kBwdRows;
  if (qtiles * (long)Hq * B > 0x7fffffffL || ktiles * (long)Hkv * B > 0x7fffffffL)
    return ATTN_ERR_UNSUPPORTED;
  // one head's K (or Q) rows must fit a buffer descriptor's 32-bit byte range
  if ((long)Nk * d * 2 > 0x7fffffffL || (long)Nq * d * 2 > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Nq);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;

  miattn::BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.dvec = static_cast<float*>(workspace);
  p.nlse = p.dvec + (size_t)B * Hq * Nq;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  // A zero scale makes every weight exp2(-LSE log2 e).  A tiny exponent scale gives the same
  // fp32 weights and keeps (+-inf) * c infinite, which the masking relies on.
  if (p.c == 0.f) p.c = 1e-30f;
  p.f16 = f16;
  (void)hipGetLastError();
  return miattn::launch_backward(p, d, causal ? 1 : 0, stream) == hipSuccess ? ATTN_OK
                                                                               : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int attn_fwd_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                     hipStream_t stream) {
  return prefill_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, false, stream);
}

int attn_fwd_prefill_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         hipStream_t stream) {
  return prefill_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, true, stream);
}

int attn_fwd_prefill_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         float q_scale, float k_scale, float v_scale, hipStream_t stream) {
  return prefill_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, false, stream, true,
                      q_scale, k_scale, v_scale);
}

int attn_fwd_prefill_paged(const void* q, const void* kcache, const void* vcache,
                           const int32_t* block_table, const int32_t* kv_lens, void* o,
                           float* lse, int B, int Hq, int Hkv, int Nq, int d, int max_kv_len,
                           int page_size, int max_blocks_per_seq, int num_pages, int causal,
                           float scale, hipStream_t stream) {
  return prefill_paged_impl(q, kcache, vcache, block_table, kv_lens, o, lse, B, Hq, Hkv, Nq, d,
                            max_kv_len, page_size, max_blocks_per_seq, num_pages, causal, scale,
                            false, stream);
}

int attn_fwd_prefill_paged_fp8(const void* q, const void* kcache, const void* vcache,
                               const int32_t* block_table, const int32_t* kv_lens, void* o,
                               float* lse, int B, int Hq, int Hkv, int Nq, int d, int max_kv_len,
                               int page_size, int max_blocks_per_seq, int num_pages, int causal,
                               float scale, float q_scale, float k_scale, float v_scale,
                               hipStream_t stream) {
  return prefill_paged_impl(q, kcache, vcache, block_table, kv_lens, o, lse, B, Hq, Hkv, Nq, d,
                            max_kv_len, page_size, max_blocks_per_seq, num_pages, causal, scale,
                            false, stream, true, q_scale, k_scale, v_scale);
}

int attn_fwd_prefill_paged_f16(const void* q, const void* kcache, const void* vcache,
                               const int32_t* block_table, const int32_t* kv_lens, void* o,
                               float* lse, int B, int Hq, int Hkv, int Nq, int d, int max_kv_len,
                               int page_size, int max_blocks_per_seq, int num_pages, int causal,
                               float scale, hipStream_t stream) {
  return prefill_paged_impl(q, kcache, vcache, block_table, kv_lens, o, lse, B, Hq, Hkv, Nq, d,
                            max_kv_len, page_size, max_blocks_per_seq, num_pages, causal, scale,
                            true, stream);
}

int attn_fwd_prefill_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                            int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                            int max_seqlen_k, int d, int causal, float scale,
                            hipStream_t stream) {
  return prefill_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q,
                             total_k, max_seqlen_q, max_seqlen_k, d, causal, scale, false, stream);
}

int attn_fwd_prefill_varlen_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                int max_seqlen_k, int d, int causal, float scale, float q_scale,
                                float k_scale, float v_scale, hipStream_t stream) {
  return prefill_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q,
                             total_k, max_seqlen_q, max_seqlen_k, d, causal, scale, false, stream,
                             true, q_scale, k_scale, v_scale);
}

int attn_fwd_prefill_varlen_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                int max_seqlen_k, int d, int causal, float scale,
                                hipStream_t stream) {
  return prefill_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q,
                             total_k, max_seqlen_q, max_seqlen_k, d, causal, scale, true, stream);
}

int attn_decode_num_splits(int B, int Hq, int Hkv, int d, int max_seqlen, int num_splits) {
  if (!decode_sizes_ok(B, Hq, Hkv, d, max_seqlen) || num_splits < 0) return 0;
  return plan_decode(B, Hq, Hkv, max_seqlen, num_splits).splits;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int d, int max_seqlen, int num_splits) {
  if (B < 1 || Hq < 1 || d < 1 || max_seqlen < 1 || num_splits < 0) return 0;
  // The automatic plan depends on the KV-head count (fewer KV heads, more chunks), which
  // this call does not take: return the largest need over every Hkv that divides Hq.
  size_t most = 0;
  for (int hkv = 1; hkv <= Hq; ++hkv) {
    if (Hq % hkv) continue;
    const size_t w = workspace_for(B, Hq, d, plan_decode(B, Hq, hkv, max_seqlen, num_splits));
    if (w > most) most = w;
  }
  return most;
}

int attn_fwd_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                    int B, int Hq, int Hkv, int d, int max_seqlen, int page_size,
                    int max_blocks_per_seq, int num_pages, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, kcache, vcache, block_table, seqlens, o, lse, B, Hq, Hkv, d, max_seqlen,
                     page_size, max_blocks_per_seq, num_pages, scale, false, false, 1.f, 1.f,
                     num_splits, workspace, workspace_bytes, stream);
}

int attn_fwd_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* block_table, const int32_t* seqlens, void* o,
                            float* lse, int B, int Hq, int Hkv, int d, int max_seqlen,
                            int page_size, int max_blocks_per_seq, int num_pages, float scale,
                            int num_splits, hipStream_t stream) {
  return decode_impl(q, kcache, vcache, block_table, seqlens, o, lse, B, Hq, Hkv, d, max_seqlen,
                     page_size, max_blocks_per_seq, num_pages, scale, false, false, 1.f, 1.f,
                     num_splits, nullptr, 0, stream, true);
}

int attn_fwd_decode_f16(const void* q, const void* kcache, const void* vcache,
                        const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                        int B, int Hq, int Hkv, int d, int max_seqlen, int page_size,
                        int max_blocks_per_seq, int num_pages, float scale, int num_splits,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, kcache, vcache, block_table, seqlens, o, lse, B, Hq, Hkv, d, max_seqlen,
                     page_size, max_blocks_per_seq, num_pages, scale, false, true, 1.f, 1.f,
                     num_splits, workspace, workspace_bytes, stream);
}

int attn_fwd_decode_fp8(const void* q, const void* kcache, const void* vcache,
                        const int32_t* block_table, const int32_t* seqlens, void* o,
                        float* lse, int B, int Hq, int Hkv, int d, int max_seqlen,
                        int page_size, int max_blocks_per_seq, int num_pages, float scale,
                        float k_scale, float v_scale, int num_splits, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) ||
      !(v_scale > 0.f))
    return ATTN_ERR_INVALID_ARGUMENT;
  return decode_impl(q, kcache, vcache, block_table, seqlens, o, lse, B, Hq, Hkv, d, max_seqlen,
                     page_size, max_blocks_per_seq, num_pages, scale, true, false, k_scale, v_scale,
                     num_splits, workspace, workspace_bytes, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq) {
  if (B < 1 || Hq < 1 || Nq < 1) return 0;
  const size_t bytes = (size_t)B * Hq * Nq * 8;
  return (bytes + 255) / 256 * 256;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                  workspace, workspace_bytes, false, stream);
}

int attn_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                  workspace, workspace_bytes, true, stream);
}

}  // extern "C"
