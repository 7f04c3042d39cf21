// Backward of the fused attention, gfx950: dQ, dK, dV from Q, K, V, O, dO and the
// forward's log-sum-exp, recomputing the attention weights tile by tile instead of
// storing them.
//
// With S = scale*Q K^T (masked), P = exp(S - LSE) row by row (the forward's softmax, the
// row statistics taken from the stored LSE), the gradients are
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O) = rowsum(P * dP),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// and a KV head's dK, dV sum over the query heads that read it.  Two kernels, each a pass
// over the score matrix in 64-row tiles staged through LDS by DMA (a two-stage ring in
// the dQ pass, three stages in the dK/dV pass):
//
//  bwd_dq_kernel    a workgroup of 4 waves owns 128 queries of one head (32 per wave, on
//                   lanes) and streams the head's K and V tiles:
//                     S^T = K Q^T, dP^T = V dO^T   (K, V rows from LDS; Q^T, dO^T in registers)
//                     dQ^T += K^T dS^T             (K^T by transposing LDS reads)
//                   It also forms D for its rows (from its dO and O rows) for the second
//                   kernel.
//  bwd_dkdv_kernel  a workgroup of 4 waves owns 128 keys of one KV head (32 per wave, on
//                   lanes) and streams Q and dO tiles of every query head of the group:
//                     S = Q K^T, dP = dO V^T       (Q, dO rows from LDS; K^T, V^T in registers)
//                     dV^T += dO^T P, dK^T += Q^T dS  (dO^T, Q^T by transposing LDS reads)
// Neither writes the other's outputs, so no atomics are used and results are
// deterministic.  The work is 2.5x the forward's products (five N x N x d products
// against two) plus one extra product each for recomputing S and dP in the second pass.
//
// Method: the pages describe the fused method as tiling plus recomputation, the attention
// matrix being recomputed in the backward pass rather than stored (page "메모리 장벽을
// 넘어: LLM 연산자 가속 라이브러리 심층 분석" (tiptinker), section "1. FlashAttention");
// the gradients are those of the definition on the page "FlashAttention 완전 정리"
// (cell-devlog), section "Attention이 뭔가".

#include <type_traits>

#include "gfx950_common.h"
#include "launch.h"

namespace miattn {

template <int D>
struct BwdShape {
  static constexpr int kWaves = 4;
  static constexpr int ROWB = D * 2;                   // bytes per row in LDS (swizzled)
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int TROWS = 64;                     // rows per streamed tile
  static constexpr int TILE = TROWS * ROWB;
  static constexpr int DMA = TILE / 16 / (64 * kWaves);  // 16-byte DMA ops per thread per tensor
  static constexpr int ROWS_WG = 32 * kWaves;          // queries (dQ) or keys (dK/dV) per workgroup
  static_assert(ROWS_WG == kBwdRows, "host grid guards assume kBwdRows rows per workgroup");
  static_assert(TILE % (16 * 64 * kWaves) == 0, "tile must split evenly over threads");
};

// Lane-constant LDS offsets shared by both kernels (relative to a tile's start).
template <int D>
struct TileOffsets {
  using S = BwdShape<D>;
  int row[D / 16];       // A operand from rows: row swap23(lane%32), logical chunk 2*st + g
  int tr[D / 32][2];     // A operand by transposing reads: rows 8g + 4h + (i16 >> 2)
  int dma[S::DMA];       // source offset of this thread's DMA chunk i
  __device__ __forceinline__ TileOffsets(int lane, int wave) {
    const int g = lane >> 5;
    {
      const int R = swap_bits_2_3(lane & 31);
      const int sw = chunk_swizzle<D>(R);
#pragma unroll
      for (int st = 0; st < D / 16; ++st) row[st] = R * S::ROWB + (((2 * st + g) ^ sw) << 4);
    }
    const int i16 = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int R = 8 * (q4 >> 1) + 4 * h + (i16 >> 2);
      const int sw = chunk_swizzle<D>(R);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * (q4 & 1) + ((i16 & 3) >> 1);
        tr[db][h] = R * S::ROWB + ((c ^ sw) << 4) + ((i16 & 1) << 3);
      }
    }
    // DMA: instruction i of this wave fills 1 KB block i*kWaves + wave of the tile; lane l
    // fetches the chunk that belongs at LDS position l of that block (rows are swizzled).
#pragma unroll
    for (int i = 0; i < S::DMA; ++i) {
      const int p = (i * S::kWaves + wave) * 64 + lane;
      const int R = p / S::CPR;
      dma[i] = R * S::ROWB + (((p % S::CPR) ^ chunk_swizzle<D>(R)) << 4);
    }
  }
  // The 8 rows 16*t4 + 8g .. +7 of column block db, transposed: an MFMA A operand whose
  // k index runs over those rows.
  __device__ __forceinline__ bf16x8 trans(const char* tile, int db, int t4) const {
    return concat(lds_read_tr(tile + tr[db][0] + t4 * 16 * S::ROWB),
                  lds_read_tr(tile + tr[db][1] + t4 * 16 * S::ROWB));
  }
};

// One row's 8 elements d = 16*s + 8*g .. +7 (the B operand layout of a row held on a lane).
__device__ __forceinline__ u32x4 load_row_chunk(const uint16_t* row, int s, int g) {
  return *(const u32x4*)(row + 16 * s + 8 * g);
}

// acc + the dot product of two rows' 8 elements
template <typename E>
__device__ __forceinline__ float dot8(u32x4 x, u32x4 y, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = E::dot2(x[e], y[e], acc);
  return acc;
}

// A wave's 32 rows of output written through LDS as whole rows, 16 bytes per lane.  Row r
// lives in lanes r (columns 32*db + 8*a4 + 0..3) and r + 32 (+4..7) of the accumulators
// acc[db][4*a4 .. 4*a4+3], the MFMA layout; written times mul in the element type.  Stored
// straight from that layout, every store instruction would scatter 16-byte pieces over 32
// rows.
// stage: this wave's kStagedBytes of LDS, no longer read by any wave; out0: the wave's first
// row; rows: how many of the 32 rows exist.  One wave's LDS writes and reads execute in
// order, so the wave needs no barrier of its own.
template <int D>
constexpr int kStagedRowBytes = 2 * D + 16;  // rows padded by 16 bytes
template <int D>
constexpr int kStagedBytes = 32 * kStagedRowBytes<D>;
template <int D, typename E>
__device__ __forceinline__ void store_rows_staged(char* stage, uint16_t* out0,
                                                  const f32x16 (&acc)[D / 32], float mul,
                                                  int g, int lane, int rows) {
  constexpr int RB = kStagedRowBytes<D>;
  char* srow = stage + (lane & 31) * RB;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const u32x2 w = {E::pack2(acc[db][4 * a4 + 0] * mul, acc[db][4 * a4 + 1] * mul),
                       E::pack2(acc[db][4 * a4 + 2] * mul, acc[db][4 * a4 + 3] * mul)};
      *(u32x2*)(srow + 2 * (32 * db + 8 * a4 + 4 * g)) = w;
    }
#pragma unroll
  for (int i = 0; i < 32 * (D / 8) / 64; ++i) {
    const int idx = 64 * i + lane;  // 16-byte chunk of the wave's block
    const int r = idx / (D / 8), ch = idx % (D / 8);
    const u32x4 w = *(const u32x4*)(stage + r * RB + 16 * ch);
    if (r < rows) *(u32x4*)(out0 + (size_t)r * D + 8 * ch) = w;
  }
}

// Requires the dK and dV accumulators to sit in the accumulation registers (AGPRs) here.
// The loop of bwd_dkdv_kernel calls it at the top of a tile and after each half's score
// products; without it the register allocator gives the first half's scores the first
// dV, dK blocks' registers and moves those blocks to vector registers and back at every
// tile (64 extra moves), which also leaves fewer vector registers for the read-ahead.
template <int N>
__device__ __forceinline__ void pin_acc(f32x16 (&x)[N], f32x16 (&y)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    asm volatile("" : "+a"(x[i]));
    asm volatile("" : "+a"(y[i]));
  }
}

// ------------------------------------------------------------------------------ dQ
template <int D, bool CAUSAL, typename E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams a) {
  using S = BwdShape<D>;
  constexpr int STAGE = 2 * S::TILE;  // K tile, V tile
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;

  // workgroup -> (query tile, head): all heads' tiles of one rank, the causal last tile
  // (the one that sees the most keys) first
  const int BH = a.B * a.Hq;
  const int nqt = (a.Nq + S::ROWS_WG - 1) / S::ROWS_WG;
  const int bh = blockIdx.x % BH;
  const int rank = blockIdx.x / BH;
  const int qtile = CAUSAL ? nqt - 1 - rank : rank;
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int kvh = hq / (a.Hq / a.Hkv);
  const int off = a.Nk - a.Nq;  // bottom-right causal alignment
  const int m0 = qtile * S::ROWS_WG;
  const int qrow = m0 + 32 * wave + (lane & 31);
  const bool qvalid = qrow < a.Nq;
  const size_t rowi = (size_t)bh * a.Nq + min(qrow, a.Nq - 1);

  // Q^T and dO^T operands (row held on the lane) and D = rowsum(dO * O) of this row
  bf16x8 qop[D / 16], doop[D / 16];
  float dpart = 0.f;
  {
    const uint16_t* qr = a.q + rowi * D;
    const uint16_t* dr = a.dout + rowi * D;
    const uint16_t* orw = a.o + rowi * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 wq = load_row_chunk(qr, s, g), wd = load_row_chunk(dr, s, g);
      const u32x4 wo = load_row_chunk(orw, s, g);
      if (!qvalid) wq = wd = u32x4{0, 0, 0, 0};
      dpart = dot8<E>(wd, wo, dpart);
      qop[s] = __builtin_bit_cast(bf16x8, wq);
      doop[s] = __builtin_bit_cast(bf16x8, wd);
    }
  }
  const float Dq = dpart + wave_xor(dpart, 32);
  if (g == 0 && qvalid) {
    a.dvec[rowi] = -Dq;                     // the dK/dV pass starts its dP sums from -D
    a.nlse[rowi] = -a.lse[rowi] * kLog2e;  // the exponent offset the dK/dV pass adds
  }
  const float lse2 = qvalid ? a.lse[rowi] * kLog2e : INFINITY;

  const int kend = CAUSAL ? min(a.Nk, min(m0 + S::ROWS_WG, a.Nq) + off) : a.Nk;
  const int ntiles = (kend + S::TROWS - 1) / S::TROWS;
  const int lim = CAUSAL ? min(a.Nk - 1, qrow + off) : a.Nk - 1;  // last visible key
  // the last key every row of this wave sees, and the score that hides a key
  const int lim_all = CAUSAL ? min(a.Nk - 1, m0 + 32 * wave + off) : a.Nk - 1;
  const float s_hidden = a.c > 0.f ? -INFINITY : INFINITY;
  // the last key any real row of this wave sees (-1: the wave holds padding rows only)
  const int wrow0 = m0 + 32 * wave;
  const int last_vis = wrow0 >= a.Nq ? -1
                       : CAUSAL ? min(a.Nk - 1, min(wrow0 + 31, a.Nq - 1) + off)
                                : a.Nk - 1;

  const TileOffsets<D> to(lane, wave);
  const uint16_t* Kh = a.k + (size_t)(b * a.Hkv + kvh) * a.Nk * D;
  const uint16_t* Vh = a.v + (size_t)(b * a.Hkv + kvh) * a.Nk * D;
  auto issue = [&](int j) {
    const int n0 = j * S::TROWS;
    char* st = smem + (j & 1) * STAGE;
    const int nbytes = __builtin_amdgcn_readfirstlane((a.Nk - n0) * S::ROWB);
#pragma unroll
    for (int i = 0; i < S::DMA; ++i) {
      const int blk = i * S::kWaves + wave;
      lds_dma16(Kh + (size_t)n0 * D, nbytes, to.dma[i], (lds_void*)(st + blk * 1024));
      lds_dma16(Vh + (size_t)n0 * D, nbytes, to.dma[i], (lds_void*)(st + S::TILE + blk * 1024));
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  if (ntiles > 0) issue(0);
  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) {
      issue(j + 1);
      wait_vmcnt<2 * S::DMA>();
    } else {
      wait_vmcnt<0>();
    }
    block_barrier();
    // A tile past the last key any row of this wave sees adds nothing to its dQ: the wave
    // skips it, which frees its SIMD for the other workgroup's wave there.
    if (j * S::TROWS <= last_vis) {
      const char* st = smem + (j & 1) * STAGE;
      // One operand stream per tile: S^T and dP^T for the tile's two 32-key halves (K and V
      // rows against Q^T, dO^T in registers), the weights, then dQ^T += K^T dS^T (K^T by
      // transposing reads).  The LDS reads run kLead MFMAs ahead of their use, across the
      // weights.
      constexpr int NS = 4 * (D / 16);  // S and dP MFMAs: 2 halves x D/16 steps x 2
      constexpr int NM = NS + 4 * (D / 32);
      constexpr int kLead = 4;
      // operand of MFMA m: (half kb, step t) pairs of S (even) and dP (odd), then (16-key
      // step t4, block db) of dQ
      auto load = [&](int m) -> bf16x8 {
        if (m < NS) {
          const int kb = m / (2 * (D / 16)), t = (m >> 1) % (D / 16);
          return lds_read_b128(st + ((m & 1) ? S::TILE : 0) + to.row[t] + kb * 32 * S::ROWB);
        }
        const int x = m - NS;
        return to.trans(st, x % (D / 32), x / (D / 32));
      };
      bf16x8 ops[NM];
  #pragma unroll
      for (int m = 0; m < kLead; ++m) ops[m] = load(m);
      f32x16 s[2], dp[2];
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = dp[kb] = f32x16{};
  #pragma unroll
      for (int m = 0; m < NS; ++m) {
        if (m + kLead < NM) ops[m + kLead] = load(m + kLead);
        const int kb = m / (2 * (D / 16)), t = (m >> 1) % (D / 16);
        if (m & 1) dp[kb] = E::mfma32(ops[m], doop[t], dp[kb]);
        else s[kb] = E::mfma32(ops[m], qop[t], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // dS^T = P^T * (dP^T - D), P^T = exp(S - LSE); accumulator r of half kb is key
      // j*64 + 32*kb + 16*(r/8) + 8*g + r%8
      uint32_t pk[2][8];
      const int kbase = j * S::TROWS + 8 * g;
      // Only a tile past some row's last visible key needs the mask: there the hidden scores
      // are replaced by an infinity of the sign that sends S*c to -inf (c is never 0), so
      // their weights come out 0.
      if (j * S::TROWS + S::TROWS - 1 > lim_all) {
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + 32 * kb + 16 * (r >> 3) + (r & 7);
            s[kb][r] = key <= lim ? s[kb][r] : s_hidden;
          }
      }
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int r = 2 * jj;
          const float p0 = fast_exp2(fmaf(s[kb][r], a.c, -lse2));
          const float p1 = fast_exp2(fmaf(s[kb][r + 1], a.c, -lse2));
          pk[kb][jj] = E::pack2(p0 * (dp[kb][r] - Dq), p1 * (dp[kb][r + 1] - Dq));
        }
      // dQ^T += K^T dS^T in 16-key steps
  #pragma unroll
      for (int x = 0; x < NM - NS; ++x) {
        const int m = NS + x;
        if (m + kLead < NM) ops[m + kLead] = load(m + kLead);
        const int t4 = x / (D / 32), db = x % (D / 32);
        const u32x4 pw = {pk[t4 >> 1][4 * (t4 & 1) + 0], pk[t4 >> 1][4 * (t4 & 1) + 1],
                          pk[t4 >> 1][4 * (t4 & 1) + 2], pk[t4 >> 1][4 * (t4 & 1) + 3]};
        acc[db] = E::mfma32(ops[m], __builtin_bit_cast(bf16x8, pw), acc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    block_barrier();  // every wave is done with this stage before it is refilled
  }

  // every wave passed the loop's last barrier, and no DMA is in flight: the buffers are free
  static_assert(S::kWaves * kStagedBytes<D> <= 2 * STAGE, "dQ staging must fit the LDS");
  store_rows_staged<D, E>(smem + wave * kStagedBytes<D>,
                          a.dq + ((size_t)bh * a.Nq + m0 + 32 * wave) * D, acc, a.scale, g,
                          lane, min(32, a.Nq - (m0 + 32 * wave)));
}

// ------------------------------------------------------------------------------ dK, dV
template <int D, bool CAUSAL, typename E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams a) {
  using S = BwdShape<D>;
  constexpr int STAGE = 2 * S::TILE + 512;  // Q tile, dO tile, LSE and D of the tile's rows
  constexpr int NST = 3;                    // ring stages: two tiles in flight
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;

  // workgroup -> (key tile, KV head): all heads' tiles of one rank, the first key tile
  // (under causal masking the one that most queries see) first
  const int BH = a.B * a.Hkv;
  const int bh = blockIdx.x % BH;
  const int ktile = blockIdx.x / BH;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int off = a.Nk - a.Nq;
  const int k0 = ktile * S::ROWS_WG;
  const int key = k0 + 32 * wave + (lane & 31);
  const bool kvalid = key < a.Nk;
  const size_t rowk = (size_t)bh * a.Nk + min(key, a.Nk - 1);

  // K^T and V^T operands: this lane's key row
  bf16x8 kop[D / 16], vop[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 wk = load_row_chunk(a.k + rowk * D, s, g), wv = load_row_chunk(a.v + rowk * D, s, g);
    if (!kvalid) wk = wv = u32x4{0, 0, 0, 0};
    kop[s] = __builtin_bit_cast(bf16x8, wk);
    vop[s] = __builtin_bit_cast(bf16x8, wv);
  }

  // query tiles: those with a query that sees one of this workgroup's keys, per head
  const int qt0 = CAUSAL ? max(0, k0 - off) / S::TROWS : 0;
  const int nqt = (a.Nq + S::TROWS - 1) / S::TROWS;
  const int per_head = nqt - qt0;
  const int iters = G * per_head;

  const TileOffsets<D> to(lane, wave);
  // byte offset of ring stage k (a uniform value whose range the compiler can see, so that
  // constant offsets fold into the LDS instructions)
  auto stage_off = [](int k) {
    return (unsigned)__builtin_amdgcn_readfirstlane(k * STAGE) & 0x1ffffu;
  };
  auto issue = [&](int it, int stage) {
    const int h = kvh * G + it / per_head;
    const int q0 = (qt0 + it % per_head) * S::TROWS;
    const size_t r0 = (size_t)(b * a.Hq + h) * a.Nq + q0;
    char* st = smem + stage_off(stage);
    const int nbytes = __builtin_amdgcn_readfirstlane((a.Nq - q0) * S::ROWB);
#pragma unroll
    for (int i = 0; i < S::DMA; ++i) {
      const int blk = i * S::kWaves + wave;
      lds_dma16(a.q + r0 * D, nbytes, to.dma[i], (lds_void*)(st + blk * 1024));
      lds_dma16(a.dout + r0 * D, nbytes, to.dma[i], (lds_void*)(st + S::TILE + blk * 1024));
    }
    // -LSE*log2(e) and D of the tile's 64 rows: one 4-byte-per-lane DMA each (rows past Nq
    // read as zeros)
    const int fbytes = __builtin_amdgcn_readfirstlane((a.Nq - q0) * 4);
    if (wave == 0) lds_dma4(a.nlse + r0, fbytes, lane * 4, (lds_void*)(st + 2 * S::TILE));
    if (wave == 1) lds_dma4(a.dvec + r0, fbytes, lane * 4, (lds_void*)(st + 2 * S::TILE + 256));
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dk[i] = dv[i] = f32x16{};

  // Stage (it + 2) % NST, refilled at the top of iteration it, was last read in iteration
  // it - 1, which ended with a barrier.
  // Waves 0 and 1 issue one more DMA per tile (the row statistics) than the count the
  // waits allow for, so their waits cover one more instruction than needed.
  if (iters > 0) issue(0, 0);
  if (iters > 1) issue(1, 1);
  // the tile loop in the wave's phase order (below); each order has a loop of its own so
  // that the register allocator treats the two separately
  auto run = [&](auto order_tag) {
  int cur = 0;  // ring stage of tile it
  for (int it = 0; it < iters; ++it) {
    if (it + 2 < iters) {
      issue(it + 2, cur == 0 ? 2 : cur - 1);
      wait_vmcnt<4 * S::DMA>();
    } else if (it + 1 < iters) {
      wait_vmcnt<2 * S::DMA>();
    } else {
      wait_vmcnt<0>();
    }
    block_barrier();
    pin_acc(dk, dv);
    const char* st = smem + stage_off(cur);
    const float* nl_t = (const float*)(st + 2 * S::TILE);
    const float* d_t = (const float*)(st + 2 * S::TILE + 256);
    const int q0 = (qt0 + it % per_head) * S::TROWS;
    // One operand stream per tile, in four phases of P MFMAs: a query half's S and dP
    // products (Q and dO rows against K^T, V^T in registers) or its dV and dK products (dO^T
    // and Q^T by transposing reads), with the half's weights formed between the two.  Even
    // waves take the order S0 W0 D0 S1 W1 D1, odd waves S0 S1 W0 D0 W1 D1, so that the
    // waves of a workgroup, which start each tile together at the barrier, do not all ask
    // the LDS for operands at once while it sits idle during their weights.  The LDS reads
    // run kLead MFMAs ahead of their use, across the phases.
    constexpr int P = D / 8;  // S, dP x D/16 steps, or dV, dK x 2 query steps x D/32 blocks
    constexpr int NM = 4 * P;
    constexpr int kLead = 8;
    f32x16 sc[2], dpc[2];
    uint32_t ppk[2][8], dpk[2][8];
    f32x4 NL[2][4], ND[2][4];
    // the row statistics of half h (-LSE*log2(e) and -D), read a phase before its S and dP
    // products: the dP sums start from -D, so that they end as dP - D
    auto read_stats = [&](int h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = 32 * h + 8 * g + 4 * (i & 1) + 16 * (i >> 1);
        NL[h][i] = lds_read_f32x4((const char*)(nl_t + o));
        ND[h][i] = lds_read_f32x4((const char*)(d_t + o));
      }
    };
    // P = exp2(S*c - LSE*log2(e)) and dS = P * (dP - D) of half h, packed; accumulator r is
    // query q0 + 32*h + 16*(r/8) + 8*g + r%8.  Only the causal triangle needs a mask (MASK:
    // the half has a pair above it), applied by setting the exponent to -inf.  Rows past Nq
    // need none: their Q, dO, LSE and D rows are staged as zeros, so P = 1 and dS = 0 there
    // and both meet a zero dO or Q row.  Lanes of keys past Nk hold zero K and V rows;
    // whatever they compute stays in their own accumulator column, which is not stored.
    auto weights = [&](int h, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        float pv[2], dsv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * jj + e;
          float x = fmaf(sc[h][r], a.c, NL[h][r >> 2][r & 3]);
          if (MASK) {
            const int qi = q0 + 32 * h + 8 * g + 16 * (r >> 3) + (r & 7);
            x = key <= qi + off ? x : -INFINITY;
          }
          pv[e] = fast_exp2(x);
          dsv[e] = pv[e] * dpc[h][r];
        }
        ppk[h][jj] = E::pack2(pv[0], pv[1]);
        dpk[h][jj] = E::pack2(dsv[0], dsv[1]);
      }
    };
    // half h has a (query, key) pair above the causal diagonal unless its first query sees
    // the wave's last key (wave-uniform)
    auto diagonal = [&](int h) { return CAUSAL && k0 + 32 * wave + 31 > q0 + 32 * h + off; };
    auto tile = [&](auto order_tag) {
      constexpr bool ALT = decltype(order_tag)::value;
      // phase ph: S and dP products (else dV and dK) of half half_of(ph); the weights of
      // half w_after(ph) (if >= 0) follow it
      auto is_s = [](int ph) { return ALT ? ph < 2 : (ph & 1) == 0; };
      auto half_of = [](int ph) { return ALT ? ph & 1 : ph >> 1; };
      auto w_after = [](int ph) { return ph == 2 ? 1 : ph == (ALT ? 1 : 0) ? 0 : -1; };
      // the phase at whose start the statistics of half h are read (h = 0: the tile's start)
      auto stats_at = [](int h) { return h == 0 || ALT ? 0 : 1; };
      // operand of MFMA m: S (even) and dP (odd) steps, or (query step t, block db) pairs
      // of dV (even) and dK (odd)
      auto load = [&](int m) -> bf16x8 {
        const int ph = m / P, x = m % P, h = half_of(ph);
        if (is_s(ph))
          return lds_read_b128(st + ((x & 1) ? S::TILE : 0) + to.row[x >> 1] +
                               h * 32 * S::ROWB);
        return to.trans(st + ((x & 1) ? 0 : S::TILE), (x >> 1) % (D / 32),
                        2 * h + x / (2 * (D / 32)));
      };
      bf16x8 ops[NM];
#pragma unroll
      for (int m = 0; m < kLead; ++m) ops[m] = load(m);
#pragma unroll
      for (int ph = 0; ph < 4; ++ph) {
        const int h = half_of(ph), wh = w_after(ph);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (stats_at(hh) == ph) read_stats(hh);
        if (is_s(ph)) {
          sc[h] = f32x16{};
#pragma unroll
          for (int r = 0; r < 16; ++r) dpc[h][r] = ND[h][r >> 2][r & 3];
        }
#pragma unroll
        for (int x = 0; x < P; ++x) {
          const int m = ph * P + x;
          if (m + kLead < NM) ops[m + kLead] = load(m + kLead);
          if (is_s(ph)) {
            if (x & 1) dpc[h] = E::mfma32(ops[m], vop[x >> 1], dpc[h]);
            else sc[h] = E::mfma32(ops[m], kop[x >> 1], sc[h]);
          } else {
            // dV^T += dO^T P and dK^T += Q^T dS, 16-query step t
            const int t = x / (2 * (D / 32)), db = (x >> 1) % (D / 32);
            if (x & 1) {
              const u32x4 w = {dpk[h][4 * t], dpk[h][4 * t + 1], dpk[h][4 * t + 2],
                               dpk[h][4 * t + 3]};
              dk[db] = E::mfma32(ops[m], __builtin_bit_cast(bf16x8, w), dk[db]);
            } else {
              const u32x4 w = {ppk[h][4 * t], ppk[h][4 * t + 1], ppk[h][4 * t + 2],
                               ppk[h][4 * t + 3]};
              dv[db] = E::mfma32(ops[m], __builtin_bit_cast(bf16x8, w), dv[db]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (wh >= 0) {
          pin_acc(dk, dv);
          if (diagonal(wh)) weights(wh, std::integral_constant<bool, true>{});
          else weights(wh, std::integral_constant<bool, false>{});
        }
      }
    };
    tile(order_tag);
    block_barrier();  // every wave is done with this stage before it is refilled
    cur = cur == NST - 1 ? 0 : cur + 1;
  }
  };
  if (wave & 1) run(std::integral_constant<bool, true>{});
  else run(std::integral_constant<bool, false>{});

  // every wave passed the loop's last barrier, and no DMA is in flight: the ring is free
  static_assert(2 * S::kWaves * kStagedBytes<D> <= NST * STAGE, "dK/dV staging must fit the LDS");
  {
    const size_t out = ((size_t)bh * a.Nk + k0 + 32 * wave) * D;
    const int rows = min(32, a.Nk - (k0 + 32 * wave));
    char* st = smem + 2 * wave * kStagedBytes<D>;
    store_rows_staged<D, E>(st, a.dk + out, dk, a.scale, g, lane, rows);
    store_rows_staged<D, E>(st + kStagedBytes<D>, a.dv + out, dv, 1.f, g, lane, rows);
  }
}

template <int D, bool CAUSAL, typename E>
static hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  using S = BwdShape<D>;
  const int nqt = (p.Nq + S::ROWS_WG - 1) / S::ROWS_WG;
  const int nkt = (p.Nk + S::ROWS_WG - 1) / S::ROWS_WG;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, E>), dim3(nqt * p.B * p.Hq), dim3(256), 0, stream,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, E>), dim3(nkt * p.B * p.Hkv), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_bwd_e(const BwdParams& p, int d, int causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_bwd_d<64, true, E>(p, stream) : launch_bwd_d<64, false, E>(p, stream);
  return causal ? launch_bwd_d<128, true, E>(p, stream) : launch_bwd_d<128, false, E>(p, stream);
}

hipError_t launch_backward(const BwdParams& p, int d, int causal, hipStream_t stream) {
  return p.f16 ? launch_bwd_e<ElemF16>(p, d, causal, stream)
               : launch_bwd_e<ElemBf16>(p, d, causal, stream);
}

}  // namespace miattn
