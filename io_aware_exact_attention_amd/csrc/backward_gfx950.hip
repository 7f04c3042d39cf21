// Backward of the fused attention, gfx950: dQ, dK, dV from Q, K, V, O, dO and the
// forward's log-sum-exp, recomputing the attention weights tile by tile instead of
// storing them.
//
// With S = scale*Q K^T (masked), P = exp(S - LSE) row by row (the forward's softmax, the
// row statistics taken from the stored LSE), the gradients are
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O) = rowsum(P * dP),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// and a KV head's dK, dV sum over the query heads that read it.  Two kernels, each a pass
// over the score matrix in 64-row tiles staged through LDS by DMA (double-buffered):
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

// Stores a lane's 32 x D accumulator block (rows on lanes, columns 32*db + 8*(r/4) +
// 4*g + r%4 in accumulator r of block db), times mul, in the element type into row `out`.
template <int D, typename E>
__device__ __forceinline__ void store_row(uint16_t* out, const f32x16 (&acc)[D / 32], float mul,
                                          int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const u32x2 w = {E::pack2(acc[db][4 * a4 + 0] * mul, acc[db][4 * a4 + 1] * mul),
                       E::pack2(acc[db][4 * a4 + 2] * mul, acc[db][4 * a4 + 3] * mul)};
      *(u32x2*)(out + 32 * db + 8 * a4 + 4 * g) = w;
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
    a.dvec[rowi] = Dq;
    a.nlse[rowi] = -a.lse[rowi] * kLog2e;  // the exponent offset the dK/dV pass adds
  }
  const float lse2 = qvalid ? a.lse[rowi] * kLog2e : INFINITY;

  const int kend = CAUSAL ? min(a.Nk, min(m0 + S::ROWS_WG, a.Nq) + off) : a.Nk;
  const int ntiles = (kend + S::TROWS - 1) / S::TROWS;
  const int lim = CAUSAL ? min(a.Nk - 1, qrow + off) : a.Nk - 1;  // last visible key

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
    __syncthreads();
    const char* st = smem + (j & 1) * STAGE;
    // S^T and dP^T for the tile's two 32-key halves
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 ka = lds_read_b128(st + to.row[t] + kb * 32 * S::ROWB);
        const bf16x8 va = lds_read_b128(st + S::TILE + to.row[t] + kb * 32 * S::ROWB);
        s[kb] = E::mfma32(ka, qop[t], s[kb]);
        dp[kb] = E::mfma32(va, doop[t], dp[kb]);
      }
    }
    // dS^T = P^T * (dP^T - D), P^T = exp(S - LSE); accumulator r of half kb is key
    // j*64 + 32*kb + 16*(r/8) + 8*g + r%8
    uint32_t pk[2][8];
    const int kbase = j * S::TROWS + 8 * g;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = 2 * jj;
        const int key = kbase + 32 * kb + 16 * (r >> 3) + (r & 7);
        float p0 = fast_exp2(fmaf(s[kb][r], a.c, -lse2));
        float p1 = fast_exp2(fmaf(s[kb][r + 1], a.c, -lse2));
        p0 = key <= lim ? p0 : 0.f;
        p1 = key + 1 <= lim ? p1 : 0.f;
        pk[kb][jj] = E::pack2(p0 * (dp[kb][r] - Dq), p1 * (dp[kb][r + 1] - Dq));
      }
    // dQ^T += K^T dS^T in 16-key steps
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const u32x4 pw = {pk[t4 >> 1][4 * (t4 & 1) + 0], pk[t4 >> 1][4 * (t4 & 1) + 1],
                        pk[t4 >> 1][4 * (t4 & 1) + 2], pk[t4 >> 1][4 * (t4 & 1) + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = E::mfma32(to.trans(st, db, t4), __builtin_bit_cast(bf16x8, pw), acc[db]);
    }
    __syncthreads();  // every wave is done with this stage before it is refilled
  }

  if (qvalid) store_row<D, E>(a.dq + ((size_t)bh * a.Nq + qrow) * D, acc, a.scale, g);
}

// ------------------------------------------------------------------------------ dK, dV
template <int D, bool CAUSAL, typename E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams a) {
  using S = BwdShape<D>;
  constexpr int STAGE = 2 * S::TILE + 512;  // Q tile, dO tile, LSE and D of the tile's rows
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

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
  auto issue = [&](int it) {
    const int h = kvh * G + it / per_head;
    const int q0 = (qt0 + it % per_head) * S::TROWS;
    const size_t r0 = (size_t)(b * a.Hq + h) * a.Nq + q0;
    char* st = smem + (it & 1) * STAGE;
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

  if (iters > 0) issue(0);
  for (int it = 0; it < iters; ++it) {
    if (it + 1 < iters) {
      issue(it + 1);
      wait_vmcnt<2 * S::DMA>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    const char* st = smem + (it & 1) * STAGE;
    const float* nl_t = (const float*)(st + 2 * S::TILE);
    const float* d_t = (const float*)(st + 2 * S::TILE + 256);
    const int q0 = (qt0 + it % per_head) * S::TROWS;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      // S and dP for 32 queries; accumulator r is query q0 + 32*qh + 16*(r/8) + 8*g + r%8
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 qa = lds_read_b128(st + to.row[t] + qh * 32 * S::ROWB);
        const bf16x8 da = lds_read_b128(st + S::TILE + to.row[t] + qh * 32 * S::ROWB);
        s = E::mfma32(qa, kop[t], s);
        dp = E::mfma32(da, vop[t], dp);
      }
      const int qb = 32 * qh + 8 * g;
      const f32x4 NL[4] = {*(const f32x4*)(nl_t + qb), *(const f32x4*)(nl_t + qb + 4),
                           *(const f32x4*)(nl_t + qb + 16), *(const f32x4*)(nl_t + qb + 20)};
      const f32x4 Dv[4] = {*(const f32x4*)(d_t + qb), *(const f32x4*)(d_t + qb + 4),
                           *(const f32x4*)(d_t + qb + 16), *(const f32x4*)(d_t + qb + 20)};
      uint32_t ppk[8], dpk[8];
      // P = exp2(S*c - LSE*log2(e)) and dS = P * (dP - D); MASK zeroes the pairs that are
      // outside the causal triangle or past Nq, Nk
      auto weights = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          float pv[2], dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 2 * jj + e;
            const float p = fast_exp2(fmaf(s[r], a.c, NL[r >> 2][r & 3]));
            if (MASK) {
              const int qi = q0 + qb + 16 * (r >> 3) + (r & 7);
              const bool vis = kvalid && qi < a.Nq && (!CAUSAL || key <= qi + off);
              pv[e] = vis ? p : 0.f;
            } else {
              pv[e] = p;
            }
            dsv[e] = pv[e] * (dp[r] - Dv[r >> 2][r & 3]);
          }
          ppk[jj] = E::pack2(pv[0], pv[1]);
          dpk[jj] = E::pack2(dsv[0], dsv[1]);
        }
      };
      // every pair of this wave's 32 keys and the half's 32 queries is visible when the
      // half's rows are all below Nq, the wave's keys all below Nk and, under causal
      // masking, the half's first query sees the wave's last key (wave-uniform)
      const int kmax = k0 + 32 * wave + 31;
      const int qfirst = q0 + 32 * qh;
      const bool all_visible =
          qfirst + 31 < a.Nq && kmax < a.Nk && (!CAUSAL || kmax <= qfirst + off);
      if (all_visible) weights(std::integral_constant<bool, false>{});
      else weights(std::integral_constant<bool, true>{});
      // dV^T += dO^T P and dK^T += Q^T dS in 16-query steps
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 pw = {ppk[4 * t], ppk[4 * t + 1], ppk[4 * t + 2], ppk[4 * t + 3]};
        const u32x4 dw = {dpk[4 * t], dpk[4 * t + 1], dpk[4 * t + 2], dpk[4 * t + 3]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = E::mfma32(to.trans(st + S::TILE, db, 2 * qh + t),
                             __builtin_bit_cast(bf16x8, pw), dv[db]);
          dk[db] = E::mfma32(to.trans(st, db, 2 * qh + t), __builtin_bit_cast(bf16x8, dw),
                             dk[db]);
        }
      }
    }
    __syncthreads();  // every wave is done with this stage before it is refilled
  }

  if (kvalid) {
    const size_t out = ((size_t)bh * a.Nk + key) * D;
    store_row<D, E>(a.dk + out, dk, a.scale, g);
    store_row<D, E>(a.dv + out, dv, 1.f, g);
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
