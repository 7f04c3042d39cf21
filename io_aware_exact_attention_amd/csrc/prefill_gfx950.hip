// Prefill: fused exact attention forward for many queries per sequence, gfx950.
//
// One workgroup (4 waves) owns BM = 128 consecutive queries of one (batch, head); each
// wave owns 32 of them.  Key/value tiles of BN = 64 rows stream HBM -> registers -> LDS,
// double-buffered so the loads of tile t+1 are in flight while tile t is computed.  Per
// tile and wave:
//   S^T = K_t Q^T       32x32x16 bf16 MFMA; K rows from LDS, Q^T held in registers.
//                       Keys land in accumulator registers, queries on lanes, so the
//                       row max / row sum of a query are mostly in-lane.
//   online softmax      running max m and sum l per query; P = exp2(S*c - m*c)
//                       rounded to bf16; l accumulates the rounded P.
//   O^T += V_t^T P^T    V^T read from LDS with the transposing LDS read, P^T straight
//                       from the S^T accumulators (no LDS round trip).
// The N x N score matrix never leaves registers.
//
// Method: page "FlashAttention 완전 정리" (cell-devlog), section "FlashAttention의 핵심
// 아이디어 — Tiling": loop over Q blocks and K/V blocks in on-chip memory, reading Q, K,
// V once and writing O once; the per-block softmax there is read as the online softmax
// the same section describes (track the running max per block, update the earlier
// partial result as each block arrives), with m, f, l as defined on the page "Flash
// Attention: GPU 메모리_IO를 최적화하는..." (holysheep), section "Online Softmax".
// Sequence-length parallelism (independent query-tile workgroups) follows the same
// page's "FlashAttention 2" subsection; the load/compute overlap its "FlashAttention 3"
// subsection describes is done here with a register-staged LDS double buffer.

#include "gfx950_common.h"
#include "launch.h"

namespace miattn {

template <int D>
struct PrefillShape {
  static constexpr int kWaves = 4;
  static constexpr int BM = 32 * kWaves;       // queries per workgroup
  static constexpr int BN = 64;                // keys per tile
  static constexpr int KSTR = D * 2 + 16;      // LDS bytes per K row (pad: conflict-free b128 reads)
  static constexpr int VSTR = D * 2 + 64;      // LDS bytes per V row (pad: conflict-free tr reads)
  static constexpr int KTILE = BN * KSTR;
  static constexpr int VTILE = BN * VSTR;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CHUNKS = BN * D / 8;    // 16-byte chunks per K (or V) tile
  static constexpr int CPT = CHUNKS / (64 * kWaves);
  static_assert(CHUNKS % (64 * kWaves) == 0, "tile must split evenly over threads");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Row index within a 32-key block that the MFMA A operand of lane l loads, chosen so
// that accumulator r of lane group g holds key 16*(r/8) + 8*g + r%8: with that order
// the 8 accumulators a lane contributes to one 16-key PV step are 8 consecutive keys.
__device__ __forceinline__ int swap_bits_2_3(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams a) {
  using S = PrefillShape<D>;
  __shared__ __attribute__((aligned(16))) char smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;  // which half of the keys / head dim this lane's operands hold

  // --- workgroup -> (query tile, head, batch); XCD-grouped, heaviest causal tiles first
  const int L = xcd_remap(blockIdx.x, a.total_wg);
  const int qi = L % a.num_qtiles;
  const int bh = L / a.num_qtiles;
  const int hq = bh % a.Hq;
  const int b = bh / a.Hq;
  const int qtile = CAUSAL ? (a.num_qtiles - 1 - qi) : qi;
  const int kvh = hq / (a.Hq / a.Hkv);
  const int m0 = qtile * S::BM;
  const int off = a.Nk - a.Nq;  // bottom-right causal alignment

  const uint16_t* __restrict__ Qh = a.q + (size_t)(b * a.Hq + hq) * a.Nq * D;
  const uint16_t* __restrict__ Kh = a.k + (size_t)(b * a.Hkv + kvh) * a.Nk * D;
  const uint16_t* __restrict__ Vh = a.v + (size_t)(b * a.Hkv + kvh) * a.Nk * D;

  // keys this workgroup needs: everything, or up to the diagonal of its last query
  int kend = a.Nk;
  if (CAUSAL) kend = min(a.Nk, min(m0 + S::BM, a.Nq) - 1 + off + 1);
  const int ntiles = (kend + S::BN - 1) / S::BN;

  // keys this wave needs (it skips tiles wholly above its diagonal, and everything when
  // all its rows are padding past Nq)
  const int wrow0 = m0 + 32 * wave;
  int wkend = 0;
  if (wrow0 < a.Nq) wkend = CAUSAL ? min(a.Nk, min(wrow0 + 31, a.Nq - 1) + off + 1) : a.Nk;

  // --- Q^T operand: lane holds query row qrow, head-dim slots 16*s + 8*g .. +7
  const int qrow = wrow0 + (lane & 31);
  bf16x8 qop[D / 16];
  {
    const uint32_t flip = a.negate_q ? 0x80008000u : 0u;
    const u32x4* src = (const u32x4*)(Qh + (size_t)min(qrow, a.Nq - 1) * D);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 w = src[2 * s + g];
      if (qrow >= a.Nq) w = u32x4{0, 0, 0, 0};
      w ^= flip;
      qop[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // --- K/V tile staging: thread owns CPT 16-byte chunks of each tile
  u32x4 kreg[S::CPT], vreg[S::CPT];
  auto load_tile = [&](int t) {
    const int n0 = t * S::BN;
#pragma unroll
    for (int i = 0; i < S::CPT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / 8), ch = c % (D / 8);
      const int key = n0 + row;
      if (key < a.Nk) {
        kreg[i] = *(const u32x4*)(Kh + (size_t)key * D + ch * 8);
        vreg[i] = *(const u32x4*)(Vh + (size_t)key * D + ch * 8);
      } else {  // ragged tail: zero rows (their scores are masked, 0 * V stays finite)
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kb = smem + buf * S::STAGE;
    char* vb = kb + S::KTILE;
#pragma unroll
    for (int i = 0; i < S::CPT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / 8), ch = c % (D / 8);
      *(u32x4*)(kb + row * S::KSTR + ch * 16) = kreg[i];
      *(u32x4*)(vb + row * S::VSTR + ch * 16) = vreg[i];
    }
  };

  const float c = a.c;  // |scale| * log2(e)
  float m_run = -INFINITY;  // reference max (raw score units) of this lane's query
  float l_run = 0.f;        // sum of bf16-rounded P over this lane's half of the keys
  float l_ex = 0.f;         // sum of unrounded P (for the LSE)
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};

  // lane-constant parts of the LDS addresses
  const int krow_l = swap_bits_2_3(lane & 31);
  const int i16 = lane & 15, q4 = lane >> 4;
  const int vrow_l = 8 * (q4 >> 1) + (i16 >> 2);
  const int vcol_l = 16 * (q4 & 1) + 4 * (i16 & 3);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);
    const int n0 = t * S::BN;

    if (n0 < wkend) {
      const char* kb = smem + (t & 1) * S::STAGE;
      const char* vb = kb + S::KTILE;

      // S^T = K Q^T for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb_ = 0; kb_ < 2; ++kb_) {
        s[kb_] = f32x16{};
        const char* kp = kb + (kb_ * 32 + krow_l) * S::KSTR + g * 16;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          const bf16x8 ka = *(const bf16x8*)(kp + st * 32);
          s[kb_] = mfma_32x32x16(ka, qop[st], s[kb_]);
        }
      }

      // causal mask on tiles crossing this wave's diagonal; ragged key tail
      const bool masked = (n0 + S::BN > a.Nk) || (CAUSAL && n0 + S::BN - 1 > wrow0 + off);
      const int lim = CAUSAL ? min(a.Nk - 1, qrow + off) : a.Nk - 1;  // last visible key
      const int kbase = n0 + 8 * g;
      if (masked) {
#pragma unroll
        for (int kb_ = 0; kb_ < 2; ++kb_)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kbase + kb_ * 32 + 16 * (r >> 3) + (r & 7) > lim) s[kb_][r] = -INFINITY;
      }

      // online softmax: tile max, lazy rescale of the running state
      float mx = -INFINITY;
#pragma unroll
      for (int kb_ = 0; kb_ < 2; ++kb_)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb_][r]);
      mx = fmaxf(mx, wave_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const bool grow = (m_run == -INFINITY) || ((m_new - m_run) * c > kRescaleLog2);
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha =
            grow ? (m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * c)) : 1.f;
        m_run = grow ? m_new : m_run;
        l_run *= alpha;
        l_ex *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      }
      const float mc = m_run * c;

      // P = exp2(S*c - m*c) -> bf16 pairs.  The sum that normalises O accumulates the
      // rounded values (O is then an exact convex combination of the V rows under the
      // weights the MFMA used); the LSE uses the sum of the unrounded values.
      uint32_t pk[2][8];
      float ex0 = 0.f, ex1 = 0.f;
#pragma unroll
      for (int kb_ = 0; kb_ < 2; ++kb_)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float p0 = fast_exp2(fmaf(s[kb_][2 * j], c, -mc));
          float p1 = fast_exp2(fmaf(s[kb_][2 * j + 1], c, -mc));
          if (masked) {  // exact zeros for masked keys (also when c == 0)
            const int k0 = kbase + kb_ * 32 + 16 * ((2 * j) >> 3) + ((2 * j) & 7);
            p0 = k0 > lim ? 0.f : p0;
            p1 = k0 + 1 > lim ? 0.f : p1;
          }
          pk[kb_][j] = pack_bf16x2(p0, p1);
          l_run = add_bf16x2(pk[kb_][j], l_run);
          ex0 += p0;
          ex1 += p1;
        }
      l_ex += ex0 + ex1;

      // O^T += V^T P^T, four 16-key steps
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const u32x4 pw = {pk[t4 >> 1][4 * (t4 & 1) + 0], pk[t4 >> 1][4 * (t4 & 1) + 1],
                          pk[t4 >> 1][4 * (t4 & 1) + 2], pk[t4 >> 1][4 * (t4 & 1) + 3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const char* vp = vb + (16 * t4 + vrow_l) * S::VSTR + vcol_l * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x4 lo = lds_read_tr(vp + db * 64);
          const bf16x4 hi = lds_read_tr(vp + db * 64 + 4 * S::VSTR);
          oacc[db] = mfma_32x32x16(concat(lo, hi), pb, oacc[db]);
        }
      }
    }

    if (more) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // --- epilogue: O = acc / l -> bf16; LSE = m*scale + ln l
  const float l_tot = l_run + wave_xor(l_run, 32);
  const float l_lse = l_ex + wave_xor(l_ex, 32);
  if (qrow < a.Nq) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.o + ((size_t)(b * a.Hq + hq) * a.Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int dv = 32 * db + 8 * a4 + 4 * g;
        const u32x2 w = {pack_bf16x2(oacc[db][4 * a4 + 0] * inv, oacc[db][4 * a4 + 1] * inv),
                         pack_bf16x2(oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv)};
        *(u32x2*)(orow + dv) = w;
      }
    if (g == 0 && a.lse)
      a.lse[(size_t)(b * a.Hq + hq) * a.Nq + qrow] = (m_run * c + log2f(l_lse)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, CAUSAL>), dim3(p.total_wg), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill(PrefillParams p, int d, int causal, hipStream_t stream) {
  p.num_qtiles = (p.Nq + PrefillShape<128>::BM - 1) / PrefillShape<128>::BM;
  p.total_wg = p.num_qtiles * p.Hq * p.B;
  if (d == 64) return causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
  return causal ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
}

}  // namespace miattn
