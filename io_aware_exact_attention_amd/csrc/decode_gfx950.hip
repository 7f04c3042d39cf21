// Decode: one query per sequence against its KV cache (contiguous or paged), gfx950.
//
// The KV length of every sequence is cut into chunks of `chunk` tokens.  One workgroup
// (4 waves) handles one (chunk, KV head, batch) and serves all query heads that share
// that KV head (up to 16 per workgroup), so every cached K/V byte is read from HBM once.
// Each wave takes every 4th 32-key block of the chunk: the block is loaded with
// coalesced 16-byte loads (16 lanes per 256-byte row, one block ahead in registers),
// staged in the wave's own LDS slice, and consumed by 16x16x32 bf16 MFMAs:
//   S^T = K_blk Q^T  (queries on lanes, keys in accumulators), online softmax,
//   O^T += V_blk^T P^T (V^T through the transposing LDS read).
// The four waves' states are merged in LDS.  With one chunk the workgroup writes O and
// LSE; otherwise it writes its chunk's normalised fp32 output and log-sum-exp, and the
// merge kernel combines the chunks of a row by log-sum-exp.
//
// Method: decode as a single query against the growing K/V cache, paged KV caches and a
// decode kernel separate from prefill: page "메모리 장벽을 넘어: LLM 연산자 가속 라이브러리
// 심층 분석" (tiptinker), section "2. FlashInfer".  The online softmax is the one of the
// page "FlashAttention 완전 정리" (cell-devlog), section "Tiling"; the chunk merge follows
// from the m, l definitions on the page "Flash Attention: GPU 메모리_IO를 최적화하는..."
// (holysheep), section "Online Softmax": a chunk with statistics (m_s, l_s) contributes
// exp(m_s) l_s = exp(lse_s) to the row's normaliser.

#include "gfx950_common.h"
#include "launch.h"

namespace miattn {

template <int D>
struct DecodeShape {
  static constexpr int BLK = kDecodeBlock;                 // keys per wave step
  static constexpr int KSTR = D * 2 + 16;                  // conflict-free b128 reads
  static constexpr int VSTR = D * 2 + 32;                  // conflict-free tr reads
  static constexpr int WAVE_LDS = BLK * (KSTR + VSTR);
  static constexpr int LDS = kDecodeWaves * WAVE_LDS;
  static constexpr int CPL = BLK * D / 8 / 64;             // 16-byte chunks per lane per tensor
  static constexpr int RED = kDecodeWaves * kDecodeHeadsPerGroup * (D + 3) * 4;
  static_assert(RED <= LDS, "reduction scratch fits in the staging LDS");
};

template <int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(DecodeParams a) {
  using S = DecodeShape<D>;
  constexpr int NH = kDecodeHeadsPerGroup;
  __shared__ __attribute__((aligned(16))) char smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x;
  const int kvh = blockIdx.y / a.ngroups;
  const int grp = blockIdx.y % a.ngroups;
  const int b = blockIdx.z;

  const int len = min(a.seqlens[b], a.max_seqlen);  // never read past the cache bound
  const int t0 = split * a.chunk;
  const int col = lane & 15;             // query head within this workgroup's group
  const int hl = grp * NH + col;
  const bool colvalid = hl < a.G;
  const int hq = kvh * a.G + min(hl, a.G - 1);

  if (t0 >= len) {
    // empty chunk: nothing to contribute.  With a single chunk this is an empty
    // sequence and its result is O = 0, LSE = -inf.
    if (a.num_splits == 1) {
      for (int idx = tid; idx < NH * D / 8; idx += 256) {
        const int h = idx / (D / 8), ch = idx % (D / 8);
        if (grp * NH + h < a.G)
          *(u32x4*)(a.o + ((size_t)b * a.Hq + kvh * a.G + grp * NH + h) * D + ch * 8) =
              u32x4{0, 0, 0, 0};
      }
      if (a.lse && tid < NH && grp * NH + tid < a.G)
        a.lse[(size_t)b * a.Hq + kvh * a.G + grp * NH + tid] = -INFINITY;
    }
    return;
  }
  const int t1 = min(len, t0 + a.chunk);

  // Q^T operand: lane holds head hl, head-dim slots 32*s + 8*(lane/16) .. +7
  const int g4 = lane >> 4;
  bf16x8 qop[D / 32];
  {
    const uint32_t flip = a.negate_q ? 0x80008000u : 0u;
    const u32x4* src = (const u32x4*)(a.q + ((size_t)b * a.Hq + hq) * D);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      u32x4 w = src[4 * s + g4];
      if (!colvalid) w = u32x4{0, 0, 0, 0};
      w ^= flip;
      qop[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const size_t kv_stride_tok = (size_t)D;
  const uint16_t* kbase_c = a.kc + ((size_t)b * a.Hkv + kvh) * a.max_seqlen * D;
  const uint16_t* vbase_c = a.vc + ((size_t)b * a.Hkv + kvh) * a.max_seqlen * D;
  const int32_t* table = PAGED ? a.block_table + (size_t)b * a.max_blocks : nullptr;

  // Page ids of a 32-key block starting at tb (two 16-token pages, wave-uniform, so
  // scalar loads).  They are fetched one block ahead of the K/V loads that use them.
  auto block_pages = [&](int tb, int& p0, int& p1) {
    if (PAGED && tb < t1) {
      p0 = table[tb >> 4];
      p1 = tb + 16 < t1 ? table[(tb >> 4) + 1] : p0;
    }
  };
  // one 32-key block: lane owns CPL chunks of K and of V (row = idx / (D/8))
  u32x4 kr[S::CPL], vr[S::CPL];
  auto load_block = [&](int tb, int p0, int p1) {
#pragma unroll
    for (int i = 0; i < S::CPL; ++i) {
      const int cidx = lane + 64 * i;
      const int row = cidx / (D / 8), ch = cidx % (D / 8);
      const int tok = tb + row;
      if (tok < t1) {
        size_t off;
        if (PAGED) {
          const int page = (i * 64) / (D / 8) < 16 ? p0 : p1;  // row < 16 <=> first page
          off = (((size_t)page * a.Hkv + kvh) * 16 + (tok & 15)) * D + ch * 8;
          kr[i] = *(const u32x4*)(a.kc + off);
          vr[i] = *(const u32x4*)(a.vc + off);
        } else {
          off = (size_t)tok * kv_stride_tok + ch * 8;
          kr[i] = *(const u32x4*)(kbase_c + off);
          vr[i] = *(const u32x4*)(vbase_c + off);
        }
      } else {
        kr[i] = u32x4{0, 0, 0, 0};
        vr[i] = u32x4{0, 0, 0, 0};
      }
    }
  };

  char* kls = smem + wave * S::WAVE_LDS;
  char* vls = kls + S::BLK * S::KSTR;
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < S::CPL; ++i) {
      const int cidx = lane + 64 * i;
      const int row = cidx / (D / 8), ch = cidx % (D / 8);
      *(u32x4*)(kls + row * S::KSTR + ch * 16) = kr[i];
      *(u32x4*)(vls + row * S::VSTR + ch * 16) = vr[i];
    }
  };

  const float c = a.c;
  float m_run = -INFINITY;
  float l_run = 0.f;  // sum of bf16-rounded P (normalises O)
  float l_ex = 0.f;   // sum of unrounded P (for the LSE)
  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{};

  const int i16 = lane & 15;
  const char* kp_l = kls + i16 * S::KSTR + g4 * 16;
  const char* vp_l = vls + (4 * g4 + (i16 >> 2)) * S::VSTR + 4 * (i16 & 3) * 2;

  const int nblk = (t1 - t0 + S::BLK - 1) / S::BLK;
  int bi = wave;
  int pg0 = 0, pg1 = 0, npg0 = 0, npg1 = 0;
  block_pages(t0 + S::BLK * bi, pg0, pg1);
  block_pages(t0 + S::BLK * (bi + kDecodeWaves), npg0, npg1);
  if (bi < nblk) load_block(t0 + S::BLK * bi, pg0, pg1);
  for (; bi < nblk; bi += kDecodeWaves) {
    const int tb = t0 + S::BLK * bi;
    store_block();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (bi + kDecodeWaves < nblk) {
      load_block(tb + kDecodeWaves * S::BLK, npg0, npg1);
      block_pages(tb + 2 * kDecodeWaves * S::BLK, npg0, npg1);
    }

    // S^T = K Q^T: two 16-key halves
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4{};
#pragma unroll
      for (int st = 0; st < D / 32; ++st) {
        const bf16x8 ka = *(const bf16x8*)(kp_l + h * 16 * S::KSTR + st * 64);
        s[h] = mfma_16x16x32(ka, qop[st], s[h]);
      }
    }
    // accumulator r of half h is key tb + 16*h + 4*g4 + r
    const bool tail = tb + S::BLK > t1;
    if (tail) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tb + 16 * h + 4 * g4 + r >= t1) s[h][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, wave_xor(mx, 16));
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
      for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;
    }
    const float mc = m_run * c;
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float p0 = fast_exp2(fmaf(s[h][2 * j], c, -mc));
        float p1 = fast_exp2(fmaf(s[h][2 * j + 1], c, -mc));
        if (tail) {
          const int k0 = tb + 16 * h + 4 * g4 + 2 * j;
          p0 = k0 >= t1 ? 0.f : p0;
          p1 = k0 + 1 >= t1 ? 0.f : p1;
        }
        pk[2 * h + j] = pack_bf16x2(p0, p1);
        l_run = add_bf16x2(pk[2 * h + j], l_run);
        l_ex += p0 + p1;
      }
    // P^T operand: k-slots 8*g4 + e <-> keys 4*g4 + e (e < 4), 16 + 4*g4 + e - 4 (e >= 4)
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const bf16x4 lo = lds_read_tr(vp_l + db * 32);
      const bf16x4 hi = lds_read_tr(vp_l + db * 32 + 16 * S::VSTR);
      oacc[db] = mfma_16x16x32(concat(lo, hi), pb, oacc[db]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves' states (LDS reused as fp32 scratch)
  float l_col = l_run + wave_xor(l_run, 16);
  l_col += wave_xor(l_col, 32);
  float e_col = l_ex + wave_xor(l_ex, 16);
  e_col += wave_xor(e_col, 32);
  __syncthreads();
  float* red_m = (float*)smem;                          // [waves][NH]
  float* red_l = red_m + kDecodeWaves * NH;             // [waves][NH]
  float* red_e = red_l + kDecodeWaves * NH;             // [waves][NH]
  float* red_o = red_e + kDecodeWaves * NH;             // [waves][NH][D]
  if (g4 == 0) {
    red_m[wave * NH + col] = m_run;
    red_l[wave * NH + col] = l_col;
    red_e[wave * NH + col] = e_col;
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * NH + col) * D + 16 * db + 4 * g4 + r] = oacc[db][r];
  __syncthreads();

  for (int idx = tid; idx < NH * D; idx += 256) {
    const int h = idx / D, dv = idx % D;
    if (grp * NH + h >= a.G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, red_m[w * NH + h]);
    float Lsum = 0.f, Esum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float mw = red_m[w * NH + h];
      const float al = mw == -INFINITY ? 0.f : fast_exp2((mw - M) * c);
      Lsum += al * red_l[w * NH + h];
      Esum += al * red_e[w * NH + h];
      acc += al * red_o[(w * NH + h) * D + dv];
    }
    const float out = acc / Lsum;
    const float lse_nat = (M * c + log2f(Esum)) * kLn2;
    const size_t row = (size_t)b * a.Hq + kvh * a.G + grp * NH + h;
    if (a.num_splits == 1) {
      a.o[row * D + dv] = __builtin_bit_cast(uint16_t, (__bf16)out);
      if (dv == 0 && a.lse) a.lse[row] = lse_nat;
    } else {
      a.ws_o[(row * a.num_splits + split) * D + dv] = out;
      if (dv == 0) a.ws_lse[row * a.num_splits + split] = lse_nat;
    }
  }
}

// One wave per (batch, query head) row: combine the row's non-empty chunks.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B * a.Hq) return;
  const int b = row / a.Hq;
  const int len = min(a.seqlens[b], a.max_seqlen);
  const int n = min(a.num_splits, (len + a.chunk - 1) / a.chunk);
  uint16_t* orow = a.o + (size_t)row * D;
  if (n <= 0) {
    for (int dv = lane; dv < D; dv += 64) orow[dv] = 0;
    if (lane == 0 && a.lse) a.lse[row] = -INFINITY;
    return;
  }
  const float* lrow = a.ws_lse + (size_t)row * a.num_splits;
  const float* prow = a.ws_o + (size_t)row * a.num_splits * D;
  float M = -INFINITY;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, lrow[s]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, wave_xor(M, m));
  float W = 0.f;
  float acc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.f;
  for (int s = 0; s < n; ++s) {
    const float w = fast_exp2((lrow[s] - M) * kLog2e);
    W += w;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) acc[i] += w * prow[(size_t)s * D + lane + 64 * i];
  }
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
    orow[lane + 64 * i] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] / W));
  if (lane == 0 && a.lse) a.lse[row] = M + logf(W);
}

template <int D>
static hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.num_splits, p.Hkv * p.ngroups, p.B);
  if (p.block_table)
    hipLaunchKernelGGL((decode_split_kernel<D, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, false>), grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits == 1) return e;
  const int rows = p.B * p.Hq;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace miattn
