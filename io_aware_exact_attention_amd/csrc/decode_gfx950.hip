// Decode: one query per sequence against its KV cache (contiguous or paged), gfx950.
//
// The KV length of every sequence is cut into chunks of `chunk` tokens.  One workgroup
// (4 waves) handles one (chunk, KV head, batch) and serves all query heads that share
// that KV head (up to 16 per workgroup), so every cached K/V byte is read from HBM once.
// Each wave takes every 4th 32-key block of the chunk: the block is loaded with coalesced
// 16-byte buffer loads (16 lanes per 256-byte row; two blocks ahead in registers, three for
// an FP8 cache), staged in the wave's own LDS slice, and consumed by 16x16x32 MFMAs (bf16,
// or fp16 for fp16 inputs):
//   S^T = K_blk Q^T  (queries on lanes, keys in accumulators), online softmax,
//   O^T += V_blk^T P^T (V^T through the transposing LDS read).
// The four waves' states are merged in LDS.  With one chunk the workgroup writes O and
// LSE; otherwise it writes its chunk's normalised fp32 output and log-sum-exp, and the
// merge kernel combines the chunks of a row by log-sum-exp.
//
// FP8 cache (F8): K and V hold OCP E4M3 codes with one scale per tensor.  A block is read
// with the same 16-byte buffer loads (half as many) and each code is widened to bf16 in
// registers before the LDS store, which is exact, so the LDS and MFMA path is the bf16
// one.  The K scale is folded into the exponent scale c by the host; the V scale
// multiplies the normalised output.  Compressed (FP8) KV caches: page "메모리 장벽을
// 넘어" (tiptinker), section "2. FlashInfer".
//
// Method: decode as a single query against the growing K/V cache, paged KV caches and a
// decode kernel separate from prefill: page "메모리 장벽을 넘어: LLM 연산자 가속 라이브러리
// 심층 분석" (tiptinker), section "2. FlashInfer".  The online softmax is the one of the
// page "FlashAttention 완전 정리" (cell-devlog), section "Tiling"; the chunk merge follows
// from the m, l definitions on the page "Flash Attention: GPU 메모리_IO를 최적화하는..."
// (holysheep), section "Online Softmax": a chunk with statistics (m_s, l_s) contributes
// exp(m_s) l_s = exp(lse_s) to the row's normaliser.

#include <mutex>

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

constexpr int kDecodeSetsF8 = 3;  // FP8 blocks in flight per wave
// Cache policy of the K/V loads: nt (non-temporal), the hint for data read once per step.
// The KV cache is streamed once per decode step and nothing rereads it; with nt the
// decode reads 6-8% faster than with the default policy (paged 5.95 vs 5.52 TB/s,
// contiguous 6.25 vs 5.86 TB/s).
constexpr int kKvLoadPolicy = 2;

template <int D, bool PAGED, bool F8, typename E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(DecodeParams a) {
  using S = DecodeShape<D>;
  constexpr int EB = F8 ? 1 : 2;  // bytes per cached element
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

  const char* kbase_c = (const char*)a.kc + ((size_t)b * a.Hkv + kvh) * a.max_seqlen * D * EB;
  const char* vbase_c = (const char*)a.vc + ((size_t)b * a.Hkv + kvh) * a.max_seqlen * D * EB;
  const int32_t* table = PAGED ? a.block_table + (size_t)b * a.max_blocks : nullptr;

  // The wave takes the chunk's 32-key blocks wave, wave + W, wave + 2W, ...; block i
  // starts at key tbk(i).
  constexpr int W = kDecodeWaves;
  auto tbk = [&](int i) { return t0 + S::BLK * i; };

  // Page ids of the wave's blocks come from one vector load per window of 32 blocks:
  // lane 2*j + h holds the page of 16-token group h of the window's j-th block (0 past
  // the chunk end).  A block's two ids are then read with v_readlane, which keeps page
  // lookups out of the scalar-load counter that every LDS wait also drains.
  int pg_lane = 0;
  int pg_win = -1;
  auto block_pages = [&](int i, int& p0, int& p1) {
    if (PAGED) {
      const int j = (i - wave) / W;  // the wave's j-th block (i = wave + W*j)
      if ((j >> 5) != pg_win) {
        pg_win = j >> 5;
        const int tg = tbk(wave + W * (32 * pg_win + (lane >> 1))) + 16 * (lane & 1);
        pg_lane = tg < t1 ? table[tg >> 4] : 0;
      }
      // page ids are clamped into the pool: a bad table entry reads a wrong page, never
      // memory outside the cache
      p0 = (int)min((uint32_t)__builtin_amdgcn_readlane(pg_lane, 2 * (j & 31)), a.page_max);
      p1 = (int)min((uint32_t)__builtin_amdgcn_readlane(pg_lane, 2 * (j & 31) + 1), a.page_max);
    }
  };
  // One 32-key block = two 16-token groups (a page of the paged cache, 16 consecutive
  // rows of the contiguous one).  Each group is read through a buffer descriptor whose
  // range ends at the chunk's last key, so rows past it read as zeros.  Lane l owns the
  // 16-byte chunks l + 64*i of the block: offset 16*l + 1024*(i mod LC/2) within group
  // i / (LC/2).  LC, the loaded chunks per lane and tensor, is half as large for codes.
  constexpr int LC = F8 ? S::CPL / 2 : S::CPL;
  constexpr int HALF = LC / 2;
  auto load_block = [&](u32x4 (&kr)[LC], u32x4 (&vr)[LC], int tb, int p0, int p1) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tg = tb + 16 * h;
      const int rows = max(0, min(16, t1 - tg));
      const char* kg;
      const char* vg;
      if (PAGED) {
        const size_t off = ((size_t)(h ? p1 : p0) * a.Hkv + kvh) * 16 * D * EB;
        kg = (const char*)a.kc + off;
        vg = (const char*)a.vc + off;
      } else {
        kg = kbase_c + (size_t)tg * D * EB;
        vg = vbase_c + (size_t)tg * D * EB;
      }
      // wave-uniform by construction; readfirstlane keeps it in an SGPR so the descriptor
      // is scalar (a descriptor the compiler sees in VGPRs costs a loop per load)
      const int nbytes = __builtin_amdgcn_readfirstlane(rows * D * EB);
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        kr[h * HALF + i] = buffer_load16<kKvLoadPolicy>(kg, nbytes, lane * 16 + 1024 * i);
        vr[h * HALF + i] = buffer_load16<kKvLoadPolicy>(vg, nbytes, lane * 16 + 1024 * i);
      }
    }
  };

  char* kls = smem + wave * S::WAVE_LDS;
  char* vls = kls + S::BLK * S::KSTR;
  // chunk l + 64*i is row l/(D/8) + i*RPI, column chunk l%(D/8)
  constexpr int RPI = 64 / (D / 8);
  char* kst = kls + (lane / (D / 8)) * S::KSTR + (lane % (D / 8)) * 16;
  char* vst = vls + (lane / (D / 8)) * S::VSTR + (lane % (D / 8)) * 16;
  // codes: chunk l + 64*i is row l/(D/16) + i*RPI8, codes 16*(l%(D/16)) .. +15, which
  // widen to the two bf16 chunks 2*(l%(D/16)) and 2*(l%(D/16)) + 1 of that row
  constexpr int RPI8 = 64 / (D / 16);
  char* kst8 = kls + (lane / (D / 16)) * S::KSTR + (lane % (D / 16)) * 32;
  char* vst8 = vls + (lane / (D / 16)) * S::VSTR + (lane % (D / 16)) * 32;
  auto widen_store = [&](char* dst, const u32x4& w) {
    const u32x2 c0 = e4m3x4_to_bf16x4(w[0]), c1 = e4m3x4_to_bf16x4(w[1]);
    const u32x2 c2 = e4m3x4_to_bf16x4(w[2]), c3 = e4m3x4_to_bf16x4(w[3]);
    *(u32x4*)dst = u32x4{c0[0], c0[1], c1[0], c1[1]};
    *(u32x4*)(dst + 16) = u32x4{c2[0], c2[1], c3[0], c3[1]};
  };
  auto store_block = [&](const u32x4 (&kr)[LC], const u32x4 (&vr)[LC]) {
#pragma unroll
    for (int i = 0; i < LC; ++i) {
      if (F8) {
        widen_store(kst8 + i * RPI8 * S::KSTR, kr[i]);
        widen_store(vst8 + i * RPI8 * S::VSTR, vr[i]);
      } else {
        *(u32x4*)(kst + i * RPI * S::KSTR) = kr[i];
        *(u32x4*)(vst + i * RPI * S::VSTR) = vr[i];
      }
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
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // S^T, online softmax and O^T += V^T P^T for the block staged in this wave's LDS
  auto compute = [&](int tb) {
    // S^T = K Q^T: two 16-key halves
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4{};
#pragma unroll
      for (int st = 0; st < D / 32; ++st) {
        const bf16x8 ka = *(const bf16x8*)(kp_l + h * 16 * S::KSTR + st * 64);
        s[h] = E::mfma16(ka, qop[st], s[h]);
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
        pk[2 * h + j] = E::pack2(p0, p1);
        l_run = E::add2(pk[2 * h + j], l_run);
        l_ex += p0 + p1;
      }
    // P^T operand: k-slots 8*g4 + e <-> keys 4*g4 + e (e < 4), 16 + 4*g4 + e - 4 (e >= 4)
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const bf16x4 lo = lds_read_tr(vp_l + db * 32);
      const bf16x4 hi = lds_read_tr(vp_l + db * 32 + 16 * S::VSTR);
      oacc[db] = E::mfma16(concat(lo, hi), pb, oacc[db]);
    }
  };

  // The wave takes blocks wave, wave + W, wave + 2W, ... with NS blocks in flight: while
  // one is consumed, the next NS are loading into registers (the NS register sets rotate).
  // Codes take half the registers of bf16, so the FP8 instance keeps more blocks in flight.
  constexpr int NS = F8 ? kDecodeSetsF8 : 2;
  u32x4 kr[NS][LC], vr[NS][LC];
  int bi = wave;
  int pn0 = 0, pn1 = 0;  // pages of the next block to load
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    block_pages(bi + s * W, pn0, pn1);
    if (bi + s * W < nblk) load_block(kr[s], vr[s], tbk(bi + s * W), pn0, pn1);
  }
  block_pages(bi + NS * W, pn0, pn1);
  for (;;) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (bi >= nblk) goto merge;
      store_block(kr[s], vr[s]);
      wave_sync();
      if (bi + NS * W < nblk) load_block(kr[s], vr[s], tbk(bi + NS * W), pn0, pn1);
      block_pages(bi + (NS + 1) * W, pn0, pn1);
      compute(tbk(bi));
      wave_sync();
      bi += W;
    }
  }

merge:
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
    const float out = F8 ? acc / Lsum * a.v_scale : acc / Lsum;
    const float lse_nat = (M * c + log2f(Esum)) * kLn2;
    const size_t row = (size_t)b * a.Hq + kvh * a.G + grp * NH + h;
    if (a.num_splits == 1) {
      a.o[row * D + dv] = E::bits(out);
      if (dv == 0 && a.lse) a.lse[row] = lse_nat;
    } else {
      a.ws_o[(row * a.num_splits + split) * D + dv] = out;
      if (dv == 0) a.ws_lse[row * a.num_splits + split] = lse_nat;
    }
  }
}

// One workgroup per (batch, query head) row combines the row's non-empty chunks.  Thread
// (sub, dv) of the kMergeThreads sums chunks sub, sub + kMergeSub, ... for head-dim dv, so
// a thread issues few, independent loads; the row's chunk LSEs are staged in LDS first
// and the kMergeSub partial sums are combined in LDS.
constexpr int kMergeThreads = 512;

template <int D, typename E>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeParams a) {
  constexpr int kMergeSub = kMergeThreads / D;
  __shared__ float s_lse[kDecodeMaxSplits];
  __shared__ float s_acc[kMergeSub][D];
  __shared__ float s_w[kMergeSub];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / a.Hq;
  const int len = min(a.seqlens[b], a.max_seqlen);
  const int n = min(a.num_splits, (len + a.chunk - 1) / a.chunk);
  uint16_t* orow = a.o + (size_t)row * D;
  if (n <= 0) {
    if (tid < D) orow[tid] = 0;
    if (tid == 0 && a.lse) a.lse[row] = -INFINITY;
    return;
  }
  const float* lrow = a.ws_lse + (size_t)row * a.num_splits;
  const float* prow = a.ws_o + (size_t)row * a.num_splits * D;
  for (int s = tid; s < n; s += kMergeThreads) s_lse[s] = lrow[s];
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, s_lse[s]);
  const int sub = tid / D, dv = tid % D;
  float acc = 0.f, W = 0.f;
#pragma unroll 8
  for (int s = sub; s < n; s += kMergeSub) {
    const float w = fast_exp2((s_lse[s] - M) * kLog2e);
    W += w;
    acc += w * prow[(size_t)s * D + dv];
  }
  s_acc[sub][dv] = acc;
  if (dv == 0) s_w[sub] = W;
  __syncthreads();
  if (tid < D) {
    float t = 0.f, wt = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeSub; ++k) {
      t += s_acc[k][tid];
      wt += s_w[k];
    }
    orow[tid] = E::bits(t / wt);
    if (tid == 0 && a.lse) a.lse[row] = M + logf(wt);
  }
}

template <int D, bool F8, typename E>
static hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.num_splits, p.Hkv * p.ngroups, p.B);
  if (p.block_table)
    hipLaunchKernelGGL((decode_split_kernel<D, true, F8, E>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, false, F8, E>), grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits == 1) return e;
  const int rows = p.B * p.Hq;
  hipLaunchKernelGGL((decode_merge_kernel<D, E>), dim3(rows), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

// Split-KV partials of the allocation-free decode entry point: one fixed-size array per
// GPU, which the library holds until the process ends.  Host code never uses the name
// `scratch` as an address (in host code it is only a stand-in for the symbol): it asks
// the runtime for the array's device address once per device, with that device current,
// and uses that address from then on.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// The FP8 cache widens to bf16 and is paired with bf16 Q and O only.
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream) {
  if (p.kv_fp8)
    return d == 64 ? launch_d<64, true, ElemBf16>(p, stream) : launch_d<128, true, ElemBf16>(p, stream);
  if (p.f16)
    return d == 64 ? launch_d<64, false, ElemF16>(p, stream) : launch_d<128, false, ElemF16>(p, stream);
  return d == 64 ? launch_d<64, false, ElemBf16>(p, stream) : launch_d<128, false, ElemBf16>(p, stream);
}

}  // namespace miattn
