// gfx950 (CDNA4) device helpers shared by the attention kernels: MFMA wrappers, the
// transposing LDS read, bf16 packing, workgroup placement across XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Word 3 of a buffer resource descriptor on gfx9-family chips: 32-bit data format, raw
// (stride 0) addressing.  Buffer loads past num_records return zeros.
constexpr int kBufferFlags = 0x00020000;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max used for exponentiation is only moved up when a row's true max
// exceeds it by more than this many powers of two; exp2 arguments therefore stay
// <= kRescaleLog2 and P <= 2^kRescaleLog2, far from fp32/bf16 overflow.  In exact
// arithmetic the result does not depend on which reference max is used.
constexpr float kRescaleLog2 = 8.0f;
// Prefill variant of the same idea: a tile's weights are formed against the current
// reference max and only redone against a fresh one when their sum exceeds the element
// type's kRedoBound (or is not finite).  Weights then stay below that bound, so P, O and
// l cannot overflow for any input that the exact softmax can handle.

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// supplies the address of 4 consecutive bf16 holding row i/4, columns 4*(i%4)..+3 of a
// 4x16 block; lane i receives column i of that block (rows 0..3).
//
// The restrict-qualified pointer gives each such read an alias scope of its own.  The
// compiler then does not make the read wait for every LDS DMA (buffer_load ... lds) still in
// flight; kernels that fill LDS by DMA order those writes and the reads themselves, with
// explicit vmcnt waits followed by a workgroup barrier.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// 16-byte LDS read (ds_read_b128) with the same alias-scope property as lds_read_tr.
__device__ __forceinline__ bf16x8 lds_read_b128(const char* __restrict__ p) {
  return *(const bf16x8*)p;
}

// 16-byte LDS read of four floats, with the same alias-scope property as lds_read_tr.
__device__ __forceinline__ f32x4 lds_read_f32x4(const char* __restrict__ p) {
  return *(const f32x4*)p;
}

// Workgroup barrier that is also a hard scheduling boundary: no instruction (memory or
// ALU) is moved across it.  Unlike __syncthreads() it is no memory fence, so it does not
// wait for the LDS DMA a wave has in flight for a later tile: kernels order those writes
// with explicit vmcnt waits before it.
__device__ __forceinline__ void block_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane LDS DMA (buffer_load_dwordx4 ... lds): lane l reads
// base + voff[l] (bytes) and the wave's 1 KB lands contiguously at dst, lane l at
// dst + 16*l.  The descriptor covers nbytes from base; reads beyond it return zeros.
// Counted by vmcnt like any vector-memory load.
__device__ __forceinline__ void lds_dma16(const void* base, int nbytes, uint32_t voff,
                                          lds_void* dst) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// The same with 4 bytes per lane (buffer_load_dword ... lds): the wave's 256 bytes land
// contiguously at dst, lane l at dst + 4*l.
__device__ __forceinline__ void lds_dma4(const void* base, int nbytes, uint32_t voff,
                                         lds_void* dst) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
}

// 16-byte buffer load into registers: reads base + off (bytes) when off < nbytes, else
// returns zeros.  CPOL is the instruction's cache-policy field (0: default).
template <int CPOL = 0>
__device__ __forceinline__ u32x4 buffer_load16(const void* base, int nbytes, int off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, kBufferFlags);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL));
}

__device__ __forceinline__ bf16x8 concat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Four E4M3 codes (byte k of x is code k) as four bf16, code k in element k:
// v_cvt_scalef32_pk_bf16_fp8 with unit scale on the low, then the high code pair.  Every
// E4M3 value is exact in bf16.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t x) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// acc + lo(x) + hi(x) for a packed bf16 pair x (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t x, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), ones, acc, false);
}

// Element types of Q, K, V and O.  Operand registers and LDS hold raw 16-bit patterns
// (typed bf16x8 throughout); the type decides the MFMA instruction, how P and O are
// rounded from fp32 (nearest even either way) and how far a prefill tile's unnormalised
// weights may grow before the tile is redone against a fresh row max.
//
// MFMA lane layouts (the same for both element types):
//   mfma32: D = A(32x16) * B(16x32) + C.  Lane l holds A[l%32][8*(l/32) .. +7],
//           B[8*(l/32) .. +7][l%32] and C[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator r.
//   mfma16: D = A(16x32) * B(32x16) + C.  Lane l holds A[l%16][8*(l/16) .. +7],
//           B[8*(l/16) .. +7][l%16] and C[4*(l/16) + r][l%16] in accumulator r.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct ElemBf16 {
  static constexpr bool kFp8 = false;
  // weights stay below 2^32: far inside the fp32 and bf16 ranges
  static constexpr float kRedoBound = 4294967296.0f;
  static __device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  // acc + both halves of a packed pair
  static __device__ __forceinline__ float add2(uint32_t x, float acc) { return add_bf16x2(x, acc); }
  // acc + x.lo*y.lo + x.hi*y.hi, both elements widened exactly to fp32
  static __device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    acc = fmaf(__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, y << 16), acc);
    return fmaf(__builtin_bit_cast(float, x & 0xffff0000u),
                __builtin_bit_cast(float, y & 0xffff0000u), acc);
  }
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};

struct ElemF16 {
  static constexpr bool kFp8 = false;
  // fp16 tops out at 65504, so a tile's weights (each at most their sum) stay below 2^15
  static constexpr float kRedoBound = 32768.0f;
  static __device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // v_cvt_pk_f16_f32
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f16x2 v;
    v[0] = (_Float16)a;
    v[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  // v_dot2_f32_f16 against (1, 1)
  static __device__ __forceinline__ float add2(uint32_t x, float acc) {
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), ones, acc, false);
  }
  // acc + x.lo*y.lo + x.hi*y.hi (v_dot2_f32_f16: the fp16 products are exact in fp32)
  static __device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), acc,
                                  false);
  }
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

// FP8 prefill: Q, K and V arrive as OCP E4M3 codes.  Q.K^T runs on the FP8 matrix cores;
// V is widened to bf16 in LDS (exactly), so P, the P.V products and O are bf16 as for
// ElemBf16.
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct ElemFp8 : ElemBf16 {
  static constexpr bool kFp8 = true;
  // D = A(32x64) * B(64x32) + C on E4M3 operands (v_mfma_f32_32x32x64_f8f6f4, both formats
  // E4M3, no block scales).  Lane l holds 32 codes of row l%32 of A and of column l%32 of
  // B; the K index a byte stands for may be any assignment shared by A and B in which
  // lanes l and l+32 hold complementary halves.  C is laid out as for mfma32.
  static __device__ __forceinline__ f32x16 mfma_qk(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

// LDS tiles of D-wide bf16/fp16 rows (ROWB = 2*D bytes, unpadded) used by the prefill and
// backward kernels.
// XOR applied to the 16-byte chunk index of row R.  Chosen so that both LDS read
// patterns are free of bank conflicts: the K operand read (16 lanes, 16 different rows,
// same chunk) and the transposing V read (4 consecutive rows x 4 consecutive chunks).
template <int D>
__device__ __forceinline__ int chunk_swizzle(int R) {
  if constexpr (D == 128) return ((R & 3) << 2) | ((R >> 2) & 3);
  else return (((R >> 1) & 1) << 2) | ((R >> 2) & 3);
}

// Row index within a 32-key block that the MFMA A operand of lane l loads, chosen so
// that accumulator r of lane group g holds key 16*(r/8) + 8*g + r%8: with that order
// the 8 accumulators a lane contributes to one 16-key PV step are 8 consecutive keys.
__device__ __forceinline__ int swap_bits_2_3(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt lgkmcnt(0): this wave's LDS writes (and reads) have completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_xor(float x, int m) { return __shfl_xor(x, m, 64); }

}  // namespace miattn
