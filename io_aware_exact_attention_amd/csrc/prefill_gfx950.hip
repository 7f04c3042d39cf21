// Prefill: fused exact attention forward for many queries per sequence, gfx950.
//
// One workgroup (8 waves, one workgroup per CU) owns BM = 256 queries of one
// (batch, head); each wave owns 32 of them.  Key/value tiles of BN = 64 rows stream from
// HBM straight into a 4-stage LDS ring (buffer_load_dwordx4 ... lds, issued two tiles ahead,
// no register staging).  Per tile and wave:
//   S^T = K_t Q^T       32x32x16 MFMA (bf16, or fp16 for fp16 inputs); K rows from LDS,
//                       Q^T held in registers.
//                       Keys land in accumulator registers, queries on lanes, so the
//                       row max / row sum of a query are in-lane plus one exchange.
//   online softmax      running max m and sum l per query; P = exp2(S*c - m*c)
//                       rounded to bf16.
//   O^T += V_t^T P^T    V^T read from LDS with the transposing LDS read, P^T straight
//                       from the S^T accumulators (no LDS round trip).
// The N x N score matrix never leaves registers.
//
// The 8 waves form two groups of 4 (one wave of each group per SIMD) that run half a
// tile apart: while one group issues the MFMAs of a tile (P.V of the previous tile,
// then Q.K^T of the current one), the other group does the softmax VALU work, so the
// matrix cores and the vector ALUs of every SIMD are busy at the same time.  Slots are
// separated by workgroup barriers.
//
// Method: page "FlashAttention 완전 정리" (cell-devlog), section "FlashAttention의 핵심
// 아이디어 — Tiling": loop over Q blocks and K/V blocks in on-chip memory, reading Q, K,
// V once and writing O once; the per-block softmax there is read as the online softmax
// the same section describes (track the running max per block, update the earlier
// partial result as each block arrives), with m, f, l as defined on the page "Flash
// Attention: GPU 메모리_IO를 최적화하는..." (holysheep), section "Online Softmax".
// Sequence-length parallelism (independent query-tile workgroups) follows the same
// page's "FlashAttention 2" subsection; the overlap of data movement with the matrix
// units that its "FlashAttention 3" subsection (and the page "메모리 장벽을 넘어",
// section "FlashAttention-3가 다른 이유") describes for Hopper is done here with LDS
// DMA prefetch and the two-group schedule.

#include <algorithm>
#include <type_traits>

#include "gfx950_common.h"
#include "launch.h"

namespace miattn {

// F8: the ring holds E4M3 K and V tiles (D bytes per row); each V tile is widened to a
// bf16 tile of ROWB-byte rows in one of two buffers after the ring, which the P.V reads use.
template <int D, bool F8 = false>
struct PrefillShape {
  static constexpr int kWaves = 8;
  static constexpr int BM = 32 * kWaves;        // queries per workgroup
  static_assert(BM == kPrefillRows, "host grid guards assume kPrefillRows queries per tile");
  static constexpr int BN = 64;                 // keys per tile
  static constexpr int ROWB = D * 2;            // bytes per bf16 K/V row in LDS (swizzled)
  static constexpr int CPR = D / 8;             // 16-byte chunks per bf16 row
  static constexpr int KROWB = F8 ? D : ROWB;   // bytes per row of a ring tile
  static constexpr int TILE = BN * KROWB;       // bytes of one K (or V) tile in the ring
  static constexpr int STAGES = 4;
  static constexpr int STAGE = 2 * TILE;        // K tile then V tile
  static constexpr int RING = STAGES * STAGE;
  static constexpr int VTILE = BN * ROWB;       // F8: one widened V tile
  static constexpr int LDS = RING + (F8 ? 2 * VTILE : 0);
  // bf16/fp16: 16-byte loads per thread per tensor and tile
  static constexpr int DMA = F8 ? 1 : TILE / 16 / (64 * kWaves);
  // 1 KB LDS DMA blocks per wave and tile (K and V)
  static constexpr int LOADS_PER_TILE = 2 * TILE / 1024 / kWaves;
  static_assert(F8 || TILE % (16 * 64 * kWaves) == 0, "tile must split evenly over threads");
  static_assert((2 * TILE) % (1024 * kWaves) == 0, "tile must split evenly over waves");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// F8 ring K tiles: XOR applied to the 16-byte chunk index of row R (D-byte rows), chosen
// so that the K operand read (16 lanes, rows swap_bits_2_3(0..15), one chunk) touches 16
// different 16-byte bank groups, as does each group of 8 of those lanes within 128 bytes.
template <int D>
__device__ __forceinline__ int chunk_swizzle_f8(int R) {
  const int b0 = R & 1, b1 = (R >> 1) & 1, b2 = (R >> 2) & 1, b3 = (R >> 3) & 1;
  if constexpr (D == 128) return b1 | (b3 << 1) | ((b0 ^ b2) << 2);
  else return b3 | ((b1 ^ b2) << 1);
}

// Order in which workgroups take (query tile, head) pairs.  Workgroup p runs on XCD
// p % 8.  When the B*Hq heads split evenly over the 8 XCDs, XCD x owns a contiguous block
// of them, so a head's K/V (and those of heads sharing a KV head) are read through one L2.
// Within its block the XCD walks groups of head_group heads; inside a group the query
// tiles go out by rank (rank 0 of every head in the group, then rank 1, ...).  Rank 0 is
// the last query tile under causal masking, the one that sees the most keys, so each
// group's long tiles start first and its short ones fill in behind them.  head_group is
// sized so that a group's K/V fit in one XCD's L2.  With heads that do not split evenly
// the same grouping runs over all heads, without the XCD blocks.
struct WorkItem {
  int qrank;
  int bh;
};

__device__ __forceinline__ WorkItem prefill_work_item(int p, int BH, int nq, int hg) {
  int nh = BH, k = p, hbase = 0;
  if ((BH & 7) == 0) {
    nh = BH >> 3;
    k = p >> 3;
    hbase = (p & 7) * nh;
  }
  const int gsize = hg * nq;
  const int gidx = k / gsize;
  const int r = k - gidx * gsize;
  const int hcount = min(hg, nh - gidx * hg);
  WorkItem w;
  w.qrank = r / hcount;
  w.bh = hbase + gidx * hg + (r - w.qrank * hcount);
  return w;
}

// Work order for chunked prefill over a paged cache, where contexts differ in length.
// When Hq splits over the 8 XCDs, XCD x owns query heads [x*Hq/8, (x+1)*Hq/8) of every
// sequence (with grouped heads that keeps one KV head's pages in one L2), and within the
// XCD the sequences go out longest context first.  Sequences are ranked by kv_lens with
// one load per lane and cross-lane reads (up to 64 sequences; beyond that, batch order).
struct PagedItem {
  int b, hq, qrank;
};

// `mine` is lane l's sequence length (for l < B).
__device__ __forceinline__ int sequence_of_rank(int r, int B, int mine, int lane) {
  if (B > 64) return r;
  int rank = 0;
  for (int j = 0; j < B; ++j) {
    const int o = __builtin_amdgcn_readlane(mine, j);
    rank += (o > mine) || (o == mine && j < lane);
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && rank == r);
  return (int)__builtin_ctzll(hit);
}

__device__ __forceinline__ PagedItem paged_work_item(int p, int B, int Hq, int nq, int mine,
                                                     int lane) {
  int r, hq, qr;
  if ((Hq & 7) == 0) {
    const int hpx = Hq >> 3;
    const int k = p >> 3;
    r = k / (hpx * nq);
    const int rem = k - r * (hpx * nq);
    hq = (p & 7) * hpx + rem / nq;
    qr = rem % nq;
  } else {
    r = p / (Hq * nq);
    const int rem = p - r * (Hq * nq);
    hq = rem / nq;
    qr = rem % nq;
  }
  PagedItem it;
  it.b = sequence_of_rank(r, B, mine, lane);
  it.hq = hq;
  it.qrank = qr;
  return it;
}

// Work order for a ragged (varlen) batch of at most 64 sequences, with no idle workgroups.
// The grid holds, per query head, a bound on the batch's query tiles that the host knows
// without reading the lengths: floor((total_q + B*(BM-1)) / BM).  Sequences are ranked by
// key count, longest first, as above; in that order sequence b takes hpx * ntiles_b
// consecutive slots of every XCD's list (its heads outer, its query tiles inner), where
// ntiles_b = ceil(nq_b / BM).  Lane l holds sequence l's query tiles and key count; a
// workgroup past the batch's last tile gets b = -1.
__device__ __forceinline__ PagedItem varlen_work_item(int p, int B, int Hq, int ntiles,
                                                      int mine, int lane) {
  int hpx = Hq, k = p, hbase = 0;
  if ((Hq & 7) == 0) {
    hpx = Hq >> 3;
    k = p >> 3;
    hbase = (p & 7) * hpx;
  }
  const int w = lane < B ? hpx * ntiles : 0;  // this lane's sequence's slots
  int before = 0;                             // slots of the sequences ranked ahead of it
  for (int j = 0; j < B; ++j) {
    const int o = __builtin_amdgcn_readlane(mine, j);
    const int wj = __builtin_amdgcn_readlane(w, j);
    before += ((o > mine) || (o == mine && j < lane)) ? wj : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(w > 0 && k >= before && k < before + w);
  PagedItem it;
  if (hit == 0) {
    it.b = -1;
    it.hq = it.qrank = 0;
    return it;
  }
  it.b = (int)__builtin_ctzll(hit);
  const int rem = k - __builtin_amdgcn_readlane(before, it.b);
  const int nt = __builtin_amdgcn_readlane(ntiles, it.b);
  it.hq = hbase + rem / nt;
  it.qrank = rem % nt;
  return it;
}

// Layouts: dense [B, H, N, D] (PAGED and VARLEN false); PAGED: K/V in the paged cache,
// kv_lens per sequence; VARLEN: sequences packed along the token axis, [total, H, D], with
// cumulative lengths cu_q, cu_k.
// F8 (E = ElemFp8, any layout): Q, K, V are E4M3 codes; Q.K^T runs on the FP8 MFMA, V is
// widened to bf16 in LDS, and O is scaled by v_scale.
template <int D, bool CAUSAL, bool PAGED, bool VARLEN, typename E>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams a) {
  constexpr bool F8 = E::kFp8;
  using S = PrefillShape<D, F8>;
  __shared__ __attribute__((aligned(1024))) char smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;   // ping-pong group
  const int g = lane >> 5;     // which half of the keys / head dim this lane's operands hold

  // --- workgroup -> (query tile, head, batch)
  int hq, b, qrank;
  if (VARLEN && a.B <= 64) {
    // lane l: sequence l's query tiles and key count (the clamped lengths used below)
    int ntiles = 0, mine = -1;
    if (lane < a.B) {
      const int qs = min(max(a.cu_q[lane], 0), a.total_q);
      const int ks = min(max(a.cu_k[lane], 0), a.total_k);
      ntiles = (min(max(a.cu_q[lane + 1], qs), a.total_q) - qs + S::BM - 1) / S::BM;
      mine = min(max(a.cu_k[lane + 1], ks), a.total_k) - ks;
    }
    const PagedItem pi = varlen_work_item(blockIdx.x, a.B, a.Hq, ntiles, mine, lane);
    if (pi.b < 0) return;  // past the batch's last query tile
    hq = pi.hq;
    b = pi.b;
    qrank = pi.qrank;
  } else if (PAGED || VARLEN) {
    int mine = -1;  // lane l: length of sequence l, the key count that ranks sequences
    if (lane < a.B)
      mine = PAGED ? a.kv_lens[lane] : a.cu_k[lane + 1] - a.cu_k[lane];
    const PagedItem pi = paged_work_item(blockIdx.x, a.B, a.Hq, a.num_qtiles, mine, lane);
    hq = pi.hq;
    b = pi.b;
    qrank = pi.qrank;
  } else {
    const WorkItem wi = prefill_work_item(blockIdx.x, a.B * a.Hq, a.num_qtiles, a.head_group);
    hq = wi.bh % a.Hq;
    b = wi.bh / a.Hq;
    qrank = wi.qrank;
  }
  // Queries and keys of this sequence.  Dense: Nq and Nk.  Paged: Nq and the sequence's
  // context length (which includes the Nq new queries as its last tokens).  Varlen: the
  // sequence's rows [cu[b], cu[b+1]) of the packed tensors, clamped to the totals so that
  // no cumulative-length value can send a read outside them.
  // (paged: kv_lens[b] clamped into [Nq, max_kv_len], so that no value sends a block-table
  // read past the sequence's row)
  int nq = a.Nq, nk = PAGED ? min(max(a.kv_lens[b], a.Nq), a.Nk) : a.Nk;
  int q_start = 0, k_start = 0;
  if (VARLEN) {
    q_start = min(max(a.cu_q[b], 0), a.total_q);
    nq = min(max(a.cu_q[b + 1], q_start), a.total_q) - q_start;
    k_start = min(max(a.cu_k[b], 0), a.total_k);
    nk = min(max(a.cu_k[b + 1], k_start), a.total_k) - k_start;
  }
  // Varlen query tiles are counted per sequence (beyond 64 sequences the grid covers the
  // longest for each); the causal order is reversed per sequence so that each one's
  // heaviest tile goes first.
  const int nqt = VARLEN ? (nq + S::BM - 1) / S::BM : a.num_qtiles;
  if (VARLEN && qrank >= nqt) return;
  const int qtile = CAUSAL ? (nqt - 1 - qrank) : qrank;
  const int kvh = hq / (a.Hq / a.Hkv);
  const int m0 = qtile * S::BM;
  const int off = nk - nq;  // bottom-right causal alignment

  // Row strides in elements: one head's consecutive query (key) rows.
  const size_t qstride = VARLEN ? (size_t)a.Hq * D : D;
  const size_t kstride = VARLEN ? (size_t)a.Hkv * D : D;
  const uint16_t* __restrict__ Qh =
      VARLEN ? a.q + ((size_t)q_start * a.Hq + hq) * D : a.q + (size_t)(b * a.Hq + hq) * a.Nq * D;
  const uint16_t* __restrict__ Kh =
      PAGED ? a.k
            : (VARLEN ? a.k + ((size_t)k_start * a.Hkv + kvh) * D
                      : a.k + (size_t)(b * a.Hkv + kvh) * a.Nk * D);
  const uint16_t* __restrict__ Vh =
      PAGED ? a.v
            : (VARLEN ? a.v + ((size_t)k_start * a.Hkv + kvh) * D
                      : a.v + (size_t)(b * a.Hkv + kvh) * a.Nk * D);
  // F8: the same tensors as one byte per element (paged: the pools); varlen rows are still
  // qstride (kstride) elements, now bytes, apart
  const uint8_t* __restrict__ Q8h =
      (const uint8_t*)a.q + (VARLEN ? ((size_t)q_start * a.Hq + hq) * D
                                    : (size_t)(b * a.Hq + hq) * a.Nq * D);
  const uint8_t* __restrict__ K8h =
      (const uint8_t*)a.k + (PAGED ? 0
                             : VARLEN ? ((size_t)k_start * a.Hkv + kvh) * D
                                      : (size_t)(b * a.Hkv + kvh) * a.Nk * D);
  const uint8_t* __restrict__ V8h =
      (const uint8_t*)a.v + (PAGED ? 0
                             : VARLEN ? ((size_t)k_start * a.Hkv + kvh) * D
                                      : (size_t)(b * a.Hkv + kvh) * a.Nk * D);

  // keys the workgroup needs: everything, or up to the diagonal of its last query
  int kend = nk;
  if (CAUSAL) kend = min(nk, min(m0 + S::BM, nq) - 1 + off + 1);
  const int ntiles = (kend + S::BN - 1) / S::BN;
  if (VARLEN && ntiles <= 0) {
    // no visible key (a sequence without keys): O = 0, LSE = -inf
    for (int idx = tid; idx < S::BM * (D / 8); idx += 64 * S::kWaves) {
      const int row = m0 + idx / (D / 8);
      if (row < nq)
        *(u32x4*)(a.o + ((size_t)(q_start + row) * a.Hq + hq) * D + (idx % (D / 8)) * 8) =
            u32x4{0, 0, 0, 0};
    }
    if (a.lse && tid < S::BM && m0 + tid < nq)
      a.lse[(size_t)hq * a.total_q + q_start + m0 + tid] = -INFINITY;
    return;
  }

  // This wave's 32 query rows: group 0 holds the first 128 rows of the tile, group 1 the
  // last 128, one 32-row block per SIMD in each.  Under causal masking group 0's rows then
  // stop seeing keys two tiles before group 1's, and in those last tiles each slot has
  // only one role (group 1's MFMAs or group 1's softmax), which runs without the other
  // contending for the SIMD.
  const int wrow0 = m0 + 32 * (4 * grp + (wave & 3));

  // --- LDS DMA of one K/V tile (buffer_load ... lds): wave-instruction i of this wave
  // fills 1 KB of the stage; lane l fetches the chunk that belongs at LDS position l of
  // that KB.  The buffer descriptor of tile j starts at its first key row and covers the
  // rows left, so rows past Nk read as zeros (their scores are masked).  The per-lane
  // offsets are the same for every tile; all per-tile address work is scalar.
  // (Varlen rows are kstride apart in memory; the LDS layout is the same.)
  const int krow_bytes = VARLEN ? (int)kstride * 2 : S::ROWB;
  constexpr int NOFF = F8 ? S::LOADS_PER_TILE : S::DMA;
  uint32_t dma_off[NOFF];
  if constexpr (F8) {
    // block blk = i*kWaves + wave of the stage: K blocks (swizzled rows) first, then the V
    // blocks, which keep the rows' byte order (the widening reads them linearly)
    const int row8 = VARLEN ? (int)kstride : D;  // bytes between consecutive key rows
#pragma unroll
    for (int i = 0; i < NOFF; ++i) {
      const int blk = i * S::kWaves + wave;
      if (blk < S::TILE / 1024) {
        const int p = blk * 64 + lane, R = p / (D / 16);
        dma_off[i] = R * row8 + (((p % (D / 16)) ^ chunk_swizzle_f8<D>(R)) << 4);
      } else {
        const int p = (blk - S::TILE / 1024) * 64 + lane;
        dma_off[i] = VARLEN ? (p / (D / 16)) * row8 + (p % (D / 16)) * 16 : p * 16;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < S::DMA; ++i) {
      const int p = (i * S::kWaves + wave) * 64 + lane;
      const int R = p / S::CPR;
      dma_off[i] = R * krow_bytes + (((p % S::CPR) ^ chunk_swizzle<D>(R)) << 4);
    }
  }
  // Paged cache [pages, Hkv, 16, D]: each 1 KB DMA block (RPB rows) lies inside one
  // 16-token page and gets its own descriptor.  The page ids of a tile's blocks are read
  // with scalar loads one tile ahead of its DMA.
  // (F8: 1024 / D rows of E4M3 codes, block blk of a stage covering K rows when blk < NB8
  // and V rows otherwise)
  constexpr int RPB = F8 ? 1024 / D : 1024 / S::ROWB;
  constexpr int NB8 = S::TILE / 1024;
  // The table is read through the constant address space: it does not change during the
  // kernel, and wave-uniform loads from there are scalar loads.
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const_i32* tbl = (const_i32*)(PAGED ? a.block_table + (size_t)b * a.max_blocks : nullptr);
  int pg_next[NOFF];
  auto fetch_pages = [&](int j) {
#pragma unroll
    for (int i = 0; i < NOFF; ++i) {
      const int blk = i * S::kWaves + wave;
      const int tok0 = j * S::BN + (F8 ? blk % NB8 : blk) * RPB;
      // clamped into the pool: a bad table entry reads a wrong page, never memory outside
      pg_next[i] = tok0 < nk ? (int)min((uint32_t)tbl[tok0 >> 4], a.page_max) : 0;
    }
  };
  if (PAGED) fetch_pages(0);
  auto issue_tile = [&](int j) {
    const int n0 = j * S::BN;
    char* st = smem + (j & (S::STAGES - 1)) * S::STAGE;
    if constexpr (F8 && PAGED) {
      int pg[NOFF];
#pragma unroll
      for (int i = 0; i < NOFF; ++i) pg[i] = pg_next[i];
      fetch_pages(j + 1);
#pragma unroll
      for (int i = 0; i < NOFF; ++i) {
        const int blk = i * S::kWaves + wave;
        const int bi = blk % NB8;  // block index within its K or V tile
        const int tok0 = n0 + bi * RPB;
        const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(RPB, nk - tok0)) * D);
        const size_t off = ((size_t)pg[i] * a.Hkv + kvh) * 16 * D + (size_t)(tok0 & 15) * D;
        lds_dma16((blk < NB8 ? K8h : V8h) + off, nbytes, dma_off[i] - bi * 1024,
                  (lds_void*)(st + blk * 1024));
      }
    } else if constexpr (F8) {
      // varlen: the range ends with the sequence's last key row inside this tile
      const int nbytes =
          VARLEN ? __builtin_amdgcn_readfirstlane((min(nk - n0, S::BN) - 1) * (int)kstride + D)
                 : (nk - n0) * D;
      const uint8_t* kt = K8h + (size_t)n0 * (VARLEN ? kstride : D);
      const uint8_t* vt = V8h + (size_t)n0 * (VARLEN ? kstride : D);
#pragma unroll
      for (int i = 0; i < NOFF; ++i) {
        const int blk = i * S::kWaves + wave;
        lds_dma16(blk < S::TILE / 1024 ? kt : vt, nbytes, dma_off[i],
                  (lds_void*)(st + blk * 1024));
      }
    } else if (PAGED) {
      int pg[S::DMA];
#pragma unroll
      for (int i = 0; i < S::DMA; ++i) pg[i] = pg_next[i];
      fetch_pages(j + 1);
#pragma unroll
      for (int i = 0; i < S::DMA; ++i) {
        const int blk = i * S::kWaves + wave;
        const int tok0 = n0 + blk * RPB;
        // wave-uniform; readfirstlane keeps the byte count, and so the descriptor, scalar
        const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(RPB, nk - tok0)) * S::ROWB);
        const size_t off = ((size_t)pg[i] * a.Hkv + kvh) * 16 * D + (size_t)(tok0 & 15) * D;
        const uint32_t lo = dma_off[i] - blk * 1024;  // offset within the block
        lds_dma16(Kh + off, nbytes, lo, (lds_void*)(st + blk * 1024));
        lds_dma16(Vh + off, nbytes, lo, (lds_void*)(st + S::TILE + blk * 1024));
      }
    } else if (VARLEN) {
      // the range ends with the sequence's last key row inside this tile, so rows past it
      // (the next sequence's) read as zeros
      const int rows = min(nk - n0, S::BN);
      const int nbytes = __builtin_amdgcn_readfirstlane((rows - 1) * krow_bytes + S::ROWB);
      const uint16_t* kt = Kh + (size_t)n0 * kstride;
      const uint16_t* vt = Vh + (size_t)n0 * kstride;
#pragma unroll
      for (int i = 0; i < S::DMA; ++i) {
        const int blk = i * S::kWaves + wave;
        lds_dma16(kt, nbytes, dma_off[i], (lds_void*)(st + blk * 1024));
        lds_dma16(vt, nbytes, dma_off[i], (lds_void*)(st + S::TILE + blk * 1024));
      }
    } else {
      const int nbytes = (nk - n0) * (D * 2);
      const uint16_t* kt = Kh + (size_t)n0 * D;
      const uint16_t* vt = Vh + (size_t)n0 * D;
#pragma unroll
      for (int i = 0; i < S::DMA; ++i) {
        const int blk = i * S::kWaves + wave;
        lds_dma16(kt, nbytes, dma_off[i], (lds_void*)(st + blk * 1024));
        lds_dma16(vt, nbytes, dma_off[i], (lds_void*)(st + S::TILE + blk * 1024));
      }
    }
  };

  // --- Q^T operand: lane holds query row qrow, head-dim slots 16*s + 8*g .. +7.
  // F8: 32 codes per 64-dim step s, head-dim slots 64*s + 16*g .. +15 and 64*s + 32 + 16*g
  // .. +15 (the K operand reads the same slots of its key rows).
  const int qrow = wrow0 + (lane & 31);
  using QOp = std::conditional_t<F8, i32x8, bf16x8>;
  QOp qop[F8 ? D / 64 : D / 16];
  if constexpr (F8) {
    const uint32_t flip = a.negate_q ? 0x80808080u : 0u;
    const u32x4* src = (const u32x4*)(Q8h + (size_t)min(qrow, nq - 1) * (VARLEN ? qstride : D));
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      u32x4 w0 = src[4 * s + g], w1 = src[4 * s + 2 + g];
      if (qrow >= nq) w0 = w1 = u32x4{0, 0, 0, 0};
      w0 ^= flip;
      w1 ^= flip;
      qop[s] = i32x8{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3],
                     (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
    }
  } else {
    const uint32_t flip = a.negate_q ? 0x80008000u : 0u;
    const u32x4* src = (const u32x4*)(Qh + (size_t)min(qrow, nq - 1) * qstride);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 w = src[2 * s + g];
      if (qrow >= nq) w = u32x4{0, 0, 0, 0};
      w ^= flip;
      qop[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Q loads are issued first, so the wait below covers exactly Q and tile 0.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (ntiles > 0) issue_tile(0);
  if (ntiles > 1) issue_tile(1);

  // --- lane-constant LDS offsets (within a stage)
  int koff[D / 16];  // K operand: row swap23(lane%32), logical chunk 2*st + g
  if constexpr (F8) {
    // E4M3 K: step st (64 dims) reads logical chunks 4*st + g and 4*st + 2 + g
    const int R = swap_bits_2_3(lane & 31);
    const int sw = chunk_swizzle_f8<D>(R);
#pragma unroll
    for (int st = 0; st < D / 64; ++st)
#pragma unroll
      for (int h = 0; h < 2; ++h) koff[2 * st + h] = R * D + (((4 * st + 2 * h + g) ^ sw) << 4);
  } else {
    const int R = swap_bits_2_3(lane & 31);
    const int sw = chunk_swizzle<D>(R);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) koff[st] = R * S::ROWB + (((2 * st + g) ^ sw) << 4);
  }
  // V^T operand via transposing reads: rows 8g + 4h + (i16>>2), relative to the stage
  // (F8: to the widened tile)
  int voff[D / 32][2];
  {
    const int i16 = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int R = 8 * (q4 >> 1) + 4 * h + (i16 >> 2);
      const int sw = chunk_swizzle<D>(R);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int c = 4 * db + 2 * (q4 & 1) + ((i16 & 3) >> 1);
        voff[db][h] = (F8 ? 0 : S::TILE) + R * S::ROWB + ((c ^ sw) << 4) + ((i16 & 1) << 3);
      }
    }
  }

  const float c = a.c;      // |scale| * log2(e)
  float m_run = -INFINITY;  // reference max (raw score units) of this lane's query
  // Sums over this lane's half of the keys: of the unrounded weights (for the LSE) and of
  // the rounded weights the P.V products consume (for normalising O, which then is an
  // exact convex combination of the V rows under those weights).
  float l_ex = 0.f;
  float l_rd = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  f32x16 sacc[2] = {f32x16{}, f32x16{}};
  uint32_t pk[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) pk[i][j] = 0;

  // --- MFMA slot: P.V of tile jpv (V^T through transposing reads, P^T from registers)
  // then S^T = K Q^T of tile jqk (two 32-key halves).  The operand reads run kLead MFMAs
  // ahead as one stream across both parts; the first kLead P.V operands are read during
  // the preceding softmax slot, so the matrix core starts on arrival.
  constexpr int NPV = 4 * (D / 32);  // P.V MFMAs per tile: 16-key steps x 32-dim blocks
  // Q.K^T operand reads per tile: 16-dim steps x key halves, one read per MFMA; F8: 64-dim
  // steps x key halves x the two 16-byte reads of one MFMA operand
  constexpr int NQK = F8 ? D / 16 : 2 * (D / 16);
  constexpr int kLead = 6;
  bf16x8 pre[kLead];
#pragma unroll
  for (int i = 0; i < kLead; ++i) pre[i] = bf16x8{};
  auto stage = [&](int j) -> const char* { return smem + (j & (S::STAGES - 1)) * S::STAGE; };
  // where the P.V reads of tile j find V: its ring stage, or (F8) its widened buffer
  auto vstage = [&](int j) -> const char* {
    if constexpr (F8) return smem + S::RING + (j & 1) * S::VTILE;
    else return stage(j);
  };
  auto pv_operand = [&](const char* st, int m) -> bf16x8 {
    const int t4 = m / (D / 32), db = m % (D / 32);
    return concat(lds_read_tr(st + voff[db][0] + t4 * 16 * S::ROWB),
                  lds_read_tr(st + voff[db][1] + t4 * 16 * S::ROWB));
  };
  auto qk_operand = [&](const char* st, int m) -> bf16x8 {
    if constexpr (F8) {
      // read m: MFMA t = m/2 (key half t%2, step t/2), 16-byte half m%2
      const int t = m >> 1;
      return lds_read_b128(st + koff[2 * (t >> 1) + (m & 1)] + (t & 1) * 32 * D);
    } else {
      return lds_read_b128(st + koff[m >> 1] + (m & 1) * 32 * S::ROWB);
    }
  };
  // F8: widen V tile j (E4M3 in its ring stage, rows in byte order) into its bf16 buffer in
  // the layout the transposing P.V reads expect.  Widening happens in even slots, where
  // group 0 issues MFMAs and group 1 runs the softmax; group 0's 256 threads do it all
  // (D/4 codes each), which keeps the softmax slot's vector work unchanged.  Part i
  // (i < D/32) widens D/32 codes per thread; the parts run inside group 0's MFMA slot, one
  // after every few MFMAs, where their few vector and LDS instructions hide in the MFMAs'
  // shadow.
  auto widen_part = [&](int j, int i) {
    if constexpr (F8) {
      const char* src = stage(j) + S::TILE;
      char* dst = smem + S::RING + (j & 1) * S::VTILE;
      // unit u: bf16 chunk c of row R (its 8 codes at byte 8c of the code row).  16
      // consecutive lanes read 128 contiguous bytes of codes, and 8 consecutive lanes write
      // the chunks c..c+7 of one row, a contiguous 128-byte half after the XOR: neither
      // access pattern has a bank conflict.
      const int u = tid + 256 * i;
      const int R = u / (D / 8), c = u % (D / 8);
      const u32x2 w = *(const u32x2*)(src + R * D + 8 * c);
      const u32x2 e0 = e4m3x4_to_bf16x4(w[0]), e1 = e4m3x4_to_bf16x4(w[1]);
      *(u32x4*)(dst + R * S::ROWB + ((c ^ chunk_swizzle<D>(R)) << 4)) =
          u32x4{e0[0], e0[1], e1[0], e1[1]};
    }
  };
  auto prefetch_pv = [&](int j) {
    const char* st = vstage(j);
#pragma unroll
    for (int i = 0; i < kLead; ++i) pre[i] = pv_operand(st, i);
  };
  // WIDEN (F8, group 0): V tile jqk is widened in parts between the MFMAs
  auto mfma_slot = [&](int jpv, int jqk, auto pv_tag, auto qk_tag, auto widen_tag) {
    constexpr bool DO_PV = decltype(pv_tag)::value;
    constexpr bool DO_QK = decltype(qk_tag)::value;
    constexpr bool WIDEN = F8 && decltype(widen_tag)::value;
    constexpr int P0 = DO_PV ? NPV : 0;
    constexpr int M = P0 + (DO_QK ? NQK : 0);
    constexpr int MPW = M / (D / 32);  // MFMAs per widening part
    const char* sv = vstage(jpv);
    const char* sk = stage(jqk);
    // The wave of the other group on this SIMD runs the softmax meanwhile.  The SIMD's
    // arbiter would favour the older of the two waves whenever both can issue; a raised
    // priority lets this wave's MFMAs issue as soon as their operands are there, and the
    // softmax's vector instructions fill the cycles in between.
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    auto load = [&](int m) -> bf16x8 {
      if (m < P0) return pv_operand(sv, m);
      return qk_operand(sk, m - P0);
    };
    // (an FP8 d = 64 slot without P.V has fewer operand reads than the read-ahead depth)
    constexpr int L0 = kLead < M ? kLead : M;
    bf16x8 ops[M];
#pragma unroll
    for (int m = 0; m < L0; ++m) ops[m] = DO_PV ? pre[m] : load(m);
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    // P.V also adds the tile's rounded weights to l_rd (one dot product with (1, 1) per
    // packed pair, one per P.V MFMA), so O is normalised by exactly the weights it summed
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (m + kLead < M) ops[m + kLead] = load(m + kLead);
      if (m < P0) {
        const int t4 = m / (D / 32), db = m % (D / 32);
        const u32x4 pw = {pk[t4 >> 1][4 * (t4 & 1) + 0], pk[t4 >> 1][4 * (t4 & 1) + 1],
                          pk[t4 >> 1][4 * (t4 & 1) + 2], pk[t4 >> 1][4 * (t4 & 1) + 3]};
        oacc[db] = E::mfma32(ops[m], __builtin_bit_cast(bf16x8, pw), oacc[db]);
        if constexpr (NPV == 16) {
          if (m & 1) r1 = E::add2(pk[m >> 3][m & 7], r1);
          else r0 = E::add2(pk[m >> 3][m & 7], r0);
        } else if (m < 16) {
          // (d = 64: 8 P.V MFMAs, two pairs each)
          r0 = E::add2(pk[m >> 3][m & 7], r0);
          r1 = E::add2(pk[(m + 8) >> 3][(m + 8) & 7], r1);
        }
      } else if constexpr (F8) {
        const int q = m - P0;
        if (q & 1) {
          const int t = q >> 1;
          const i32x8 kop = __builtin_bit_cast(
              i32x8, __builtin_shufflevector(ops[m - 1], ops[m], 0, 1, 2, 3, 4, 5, 6, 7, 8, 9,
                                             10, 11, 12, 13, 14, 15));
          if (t & 1) s1 = E::mfma_qk(kop, qop[t >> 1], s1);
          else s0 = E::mfma_qk(kop, qop[t >> 1], s0);
        }
      } else {
        const int q = m - P0;
        if (q & 1) s1 = E::mfma32(ops[m], qop[q >> 1], s1);
        else s0 = E::mfma32(ops[m], qop[q >> 1], s0);
      }
      if (WIDEN && m % MPW == MPW - 1) widen_part(jqk, m / MPW);
    }
    // issue order: [the first kLead Q.K^T reads when nothing was prefetched], then per MFMA
    // m the reads of operand m + kLead (two transposing reads for P.V, one for Q.K^T)
    if (!DO_PV) __builtin_amdgcn_sched_group_barrier(0x100, L0, 0);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      // (F8: a Q.K^T MFMA follows every second read)
      if (!F8 || m < P0 || ((m - P0) & 1)) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < P0 && (NPV == 16 || m < 8)) __builtin_amdgcn_sched_group_barrier(0x002, NPV == 16 ? 1 : 2, 0);
      const int n = m + kLead;
      if (n < P0) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (n < M) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (DO_QK) {
      sacc[0] = s0;
      sacc[1] = s1;
    }
    if (DO_PV) l_rd += r0 + r1;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  // Online softmax of tile j held in sacc; MASK applies the causal diagonal and the ragged
  // key tail.  The weights are formed against the current reference max m_run first.  The
  // max is only recomputed, the two lanes of a query exchange theirs and O and l are
  // rescaled, when the tile's weight sum exceeds E::kRedoBound (the reference has fallen
  // far behind the scores) or could not be formed at all.  On the first tile m_run is -inf,
  // so every weight is +inf or NaN and that path runs.  Otherwise the weights stay at most
  // E::kRedoBound, inside the range of fp32 and of the element type, and the result is the
  // same softmax.
  const int lim = CAUSAL ? min(nk - 1, qrow + off) : nk - 1;  // last visible key
  auto softmax = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (MASK) {
      // key kbase + o is visible when o <= lim - kbase; o is a small constant per register,
      // so each score costs one compare with an inline constant and one select
      const int vis = lim - (j * S::BN + 8 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[kb][r] = (kb * 32 + 16 * (r >> 3) + (r & 7) > vis) ? -INFINITY : sacc[kb][r];
    }
    // P = exp2(S*c - m*c) -> bf16 pairs, and the tile's sum of the unrounded weights (the
    // sum of the rounded pairs is taken in the MFMA slot that consumes them)
    auto weights = [&]() {
      const float nmc = -(m_run * c);
      float ex0, ex1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p0 = fast_exp2(fmaf(sacc[kb][2 * jj], c, nmc));
          const float p1 = fast_exp2(fmaf(sacc[kb][2 * jj + 1], c, nmc));
          pk[kb][jj] = E::pack2(p0, p1);
          if (kb == 0 && jj == 0) {
            ex0 = p0;
            ex1 = p1;
          } else {
            ex0 += p0;
            ex1 += p1;
          }
        }
      return ex0 + ex1;
    };
    float ts = weights();
    if (__builtin_amdgcn_ballot_w64(!(ts <= E::kRedoBound))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = fmaxf(mx, wave_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * c);
      m_run = m_new;
      l_ex *= alpha;
      l_rd *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      ts = weights();
    }
    l_ex += ts;
  };

  // Slot bookkeeping shared by both groups.  Slot 2j: tile j+2 is prefetched into the
  // stage tile j-2 used (F8: and V tile j is widened).  End of slot 2j+1: tile j+1 must be
  // resident.
  auto slot_begin = [&](int s) {
    if ((s & 1) == 0 && (s >> 1) + 2 < ntiles) issue_tile((s >> 1) + 2);
  };
  auto slot_end = [&](int s) {
    if (s & 1) {
      const int jw = (s + 1) >> 1;
      if (jw + 1 < ntiles) wait_vmcnt<S::LOADS_PER_TILE>();
      else wait_vmcnt<0>();
    } else if constexpr (F8) {
      wait_lgkmcnt0();  // the widened V is in LDS before any wave reads it
    }
    block_barrier();
  };

  // This wave's tiles, from its own rows (the last real one: rows past nq are never
  // stored):
  //   [0, jv)  every key visible to every row (tile 0 is masked all the same: peeled);
  //   [jv, jd) the causal diagonal of some row, or the ragged end of the keys: masked;
  //   [jd, n)  no key visible to any row: skipped, the wave only issues its share of the
  //            K/V DMA (FP8, group 0: and widens the V tiles, which group 1 may still
  //            read) and passes the barriers.  Skipping is exact: those weights are 0.
  const int n = ntiles;
  int jd = n;
  int jv = nk / S::BN;
  if (CAUSAL) {
    const int last = min(wrow0 + 31, nq - 1);
    jv = min(jv, max(wrow0 + off + 1, 0) / S::BN);
    jd = min(n, wrow0 >= nq ? 1 : max(last + off, 0) / S::BN + 1);
  } else if (wrow0 >= nq) {
    jd = 1;
  }
  jd = max(jd, 1);
  jv = max(1, min(jv, jd));

  // tile 0 resident before slot 0
  if (ntiles > 1) wait_vmcnt<S::LOADS_PER_TILE>(); else wait_vmcnt<0>();
  block_barrier();

  // Group 0: slot 2j = MFMA (P.V of j-1, Q.K^T of j); slot 2j+1 = softmax of j and the
  // first P.V operands of j.  Group 1 runs one slot behind.  The first tile and the
  // wave's last live tile (jd - 1) are peeled; slots past it keep only the DMA and the
  // barriers, so every wave passes 2n+2 barriers.
  std::integral_constant<bool, false> no;
  std::integral_constant<bool, true> yes;
  auto idle_slots = [&](int s0) {
    for (int s = s0; s < 2 * n + 2; ++s) {
      slot_begin(s);
      if constexpr (F8) {
        // group 0's even slot 2j: widen V tile j (with no MFMAs to hide behind)
        if (grp == 0 && (s & 1) == 0 && (s >> 1) < n) {
#pragma unroll
          for (int i = 0; i < D / 32; ++i) widen_part(s >> 1, i);
        }
      }
      slot_end(s);
    }
  };
  if (grp == 0) {
    slot_begin(0);
    mfma_slot(0, 0, no, yes, yes);
    slot_end(0);
    slot_begin(1);
    prefetch_pv(0);
    softmax(0, yes);
    slot_end(1);
    auto iter = [&](int j, auto mask_tag) {
      slot_begin(2 * j);
      mfma_slot(j - 1, j, yes, yes, yes);
      slot_end(2 * j);
      slot_begin(2 * j + 1);
      prefetch_pv(j);
      softmax(j, mask_tag);
      slot_end(2 * j + 1);
    };
    for (int j = 1; j < jv; ++j) iter(j, no);
    for (int j = jv; j < jd; ++j) iter(j, yes);
    slot_begin(2 * jd);
    if (F8 && jd < n) mfma_slot(jd - 1, jd, yes, no, yes);  // and widen V tile jd
    else mfma_slot(jd - 1, 0, yes, no, no);
    slot_end(2 * jd);
    idle_slots(2 * jd + 1);
  } else {
    slot_begin(0);
    slot_end(0);
    slot_begin(1);
    mfma_slot(0, 0, no, yes, no);
    slot_end(1);
    // iteration j runs the softmax of tile j-1: masked for tile 0 and tiles >= jv
    auto iter = [&](int j, auto mask_tag) {
      slot_begin(2 * j);
      prefetch_pv(j - 1);
      softmax(j - 1, mask_tag);
      slot_end(2 * j);
      slot_begin(2 * j + 1);
      mfma_slot(j - 1, j, yes, yes, no);
      slot_end(2 * j + 1);
    };
    if (jd > 1) iter(1, yes);
    for (int j = 2; j < min(jv + 1, jd); ++j) iter(j, no);
    for (int j = max(jv + 1, 2); j < jd; ++j) iter(j, yes);
    slot_begin(2 * jd);
    prefetch_pv(jd - 1);
    softmax(jd - 1, yes);
    slot_end(2 * jd);
    slot_begin(2 * jd + 1);
    mfma_slot(jd - 1, 0, yes, no, no);
    slot_end(2 * jd + 1);
    idle_slots(2 * jd + 2);
  }

  // --- epilogue: O = acc / (sum of rounded weights) -> bf16; LSE = m*scale + ln l with l
  // the sum of the unrounded weights
  const float l_tot = l_ex + wave_xor(l_ex, 32);
  const float l_rtot = l_rd + wave_xor(l_rd, 32);
  // O leaves through LDS: stored straight from the MFMA layout, every store instruction
  // would scatter 16-byte pieces over 32 rows.  After the last barrier no wave reads the
  // ring any more, so each wave stages its 32 x D block there (rows padded by 16 bytes)
  // and writes whole rows, 16 bytes per lane.  One wave's LDS writes and reads execute in
  // order, so the wave needs no barrier of its own.
  constexpr int OROWB = 2 * D + 16;
  static_assert(S::kWaves * 32 * OROWB <= S::LDS, "O staging must fit the LDS");
  char* ostage = smem + wave * 32 * OROWB;
  {
    const float inv = (F8 ? a.v_scale : 1.f) / l_rtot;
    char* srow = ostage + (lane & 31) * OROWB;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int dv = 32 * db + 8 * a4 + 4 * g;
        const u32x2 w = {E::pack2(oacc[db][4 * a4 + 0] * inv, oacc[db][4 * a4 + 1] * inv),
                         E::pack2(oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv)};
        *(u32x2*)(srow + 2 * dv) = w;
      }
  }
#pragma unroll
  for (int i = 0; i < 32 * (D / 8) / 64; ++i) {
    const int idx = 64 * i + lane;  // 16-byte chunk of the wave's block
    const int r = idx / (D / 8), ch = idx % (D / 8);
    const int row = wrow0 + r;
    const u32x4 w = *(const u32x4*)(ostage + r * OROWB + 16 * ch);
    if (row < nq) {
      uint16_t* orow = VARLEN ? a.o + ((size_t)(q_start + row) * a.Hq + hq) * D
                              : a.o + ((size_t)(b * a.Hq + hq) * a.Nq + row) * D;
      *(u32x4*)(orow + 8 * ch) = w;
    }
  }
  if (qrow < nq && g == 0 && a.lse)
    a.lse[VARLEN ? (size_t)hq * a.total_q + q_start + qrow
                 : (size_t)(b * a.Hq + hq) * a.Nq + qrow] = (m_run * c + log2f(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, typename E>
static hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  if (p.block_table)
    hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, true, false, E>), dim3(p.total_wg), dim3(512),
                       0, stream, p);
  else if (p.cu_q)
    hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, false, true, E>), dim3(p.total_wg), dim3(512),
                       0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, false, false, E>), dim3(p.total_wg), dim3(512),
                       0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_f8(const PrefillParams& p, hipStream_t stream) {
  if (p.block_table)
    hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, true, false, ElemFp8>), dim3(p.total_wg),
                       dim3(512), 0, stream, p);
  else if (p.cu_q)
    hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, false, true, ElemFp8>), dim3(p.total_wg),
                       dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<D, CAUSAL, false, false, ElemFp8>), dim3(p.total_wg),
                       dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_e(const PrefillParams& p, int d, int causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_one<64, true, E>(p, stream) : launch_one<64, false, E>(p, stream);
  return causal ? launch_one<128, true, E>(p, stream) : launch_one<128, false, E>(p, stream);
}

hipError_t launch_prefill(PrefillParams p, int d, int causal, hipStream_t stream) {
  constexpr int BM = PrefillShape<128>::BM;
  p.num_qtiles = (p.Nq + BM - 1) / BM;
  p.total_wg = p.num_qtiles * p.Hq * p.B;
  // ragged batch of at most 64 sequences: the tile bound of varlen_work_item per head
  if (p.cu_q && p.B <= 64) {
    const long tiles = ((long)p.total_q + (long)p.B * (BM - 1)) / BM;
    p.total_wg = (int)std::min<long>(tiles * p.Hq, (long)p.total_wg);
  }
  // A zero scale makes every visible weight 1.  A tiny positive exponent scale gives the
  // same fp32 weights (2^(tiny) rounds to 1) while keeping -inf * c = -inf for masked
  // keys, so the kernel needs no separate zero-weight select.
  if (!(p.c > 0.f)) p.c = 1e-30f;
  // Heads per dispatch group: as many as keep the group's K and V within 4 MiB (one
  // XCD's L2), at least 1, at most the heads one XCD owns.
  {
    const int BH = p.B * p.Hq;
    const int nh = (BH % 8 == 0) ? BH / 8 : BH;
    const double kv_bytes = 2.0 * p.Nk * d * (p.fp8 ? 1.0 : 2.0);
    int hg = (int)((4.0 * 1024 * 1024) / kv_bytes);
    p.head_group = hg < 1 ? 1 : (hg > nh ? nh : hg);
  }
  if (p.fp8) {
    if (d == 64) return causal ? launch_f8<64, true>(p, stream) : launch_f8<64, false>(p, stream);
    return causal ? launch_f8<128, true>(p, stream) : launch_f8<128, false>(p, stream);
  }
  return p.f16 ? launch_e<ElemF16>(p, d, causal, stream) : launch_e<ElemBf16>(p, d, causal, stream);
}

}  // namespace miattn
