// mq_gemm.hip -- MFMA path for prefill and batches the skinny and GEMV paths do not take.
//
// Y[m, n] = sum_k X[m, k] * w_hat[n, k].  Per 64-wide k step a workgroup
//  * copies its X tile (BM x 64, fp16/bf16) global -> VGPR -> LDS,
//  * loads the packed planes of its weight tile (BN rows x two 32-code units),
//    rebuilds and slices the codes in VGPRs and dequantizes them exactly in
//    fp32 (w_hat = v*s + (delta - z)*s, all terms exact for an fp16 scale and
//    an integer zero point), rounds once to the activation dtype and writes
//    the tile to LDS,
//  * runs v_mfma_f32_16x16x32_{bf16,f16} from LDS with fp32 accumulators.
// LDS is double buffered: the next step's global loads are issued before the
// current step's MFMAs and its dequantization is written to the other buffer
// afterwards, so one barrier per step suffices.
//
// This is the pages' fused dequantize-and-multiply design for prefill and
// larger batches (MatGPTQ "Efficient and Accurate Inference over Nested
// Quantized Models", section 4: on-the-fly dequantization, fp32
// accumulation; prefill support, contribution 3) mapped onto gfx950 matrix
// cores: tiles are multiples of the 16x16x32 MFMA block, a wave owns a
// (BM/WM) x (BN/WN) sub-tile, and workgroups that share weight tiles are
// placed on the same XCD so the tiles are read from one L2.
//
// Split-k (when the caller provides a workspace): blockIdx.y selects a k
// range, partial tiles go to workspace[split][m][n] in fp32, and a second
// kernel sums the splits in a fixed order, so results stay deterministic.
#include <type_traits>

#include "mq_common.h"
#include "mq_kernels.h"

namespace mq {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int BK = 64;
// The weight tile in LDS is fragment-major: a 16-row x 32-k block is 1 KB and
// lane l of an MFMA operand read owns 16 bytes of it (row 16b + l % 16, k
// 8 (l / 16) .. + 7 of the block's k half), so every fragment read is one
// contiguous 1 KB per wave.  The X tile is row-major with an xor swizzle
// instead (see store_x), which lets its global loads take a whole row's k
// slice per eight lanes.  ds_write_b128 serves eight consecutive lanes per
// clock on gfx950, so the swizzles keep each such group on distinct banks.

struct GemmArgs {
  const void* x;
  void* y;        // [m, n] in x's dtype, or fp32 workspace [splits][m][n]
  PlanePtrs pl;
  const uint16_t* scales;
  const uint16_t* zeros;
  int m, n, k, group;
  int tiles_m, tiles_n;
  int ksteps_per_split;
  int to_workspace;
};

template <int BF16>
__device__ __forceinline__ floatx4 mfma16x16x32(const uint4& a, const uint4& b, const floatx4& c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Per-thread state of one workgroup tile.  Helpers are force-inlined member
// functions (not lambdas capturing arrays by reference), so the staging
// arrays are scalarised into registers instead of living in memory.
template <int R, int ROUND, int BF16, int BM, int BN, int WM, int WN>
struct GemmTile {
  static constexpr int T = 64 * WM * WN;
  static constexpr int NP = planes_needed(R, ROUND);
  static constexpr int FM = BM / WM / 16;
  static constexpr int FN = BN / WN / 16;
  static constexpr int CX = (BM * 8 + T - 1) / T;  // 16-byte X chunks per thread per step
  static constexpr int CW = BN * 2 / T;             // (row, unit) weight items per thread per step
  static_assert(CW >= 1 && CW * T == BN * 2, "W tile split");
  static constexpr float kDelta = ROUND ? 0.0f : prefix_delta(R);

  const GemmArgs& a;
  int tid, m0, n0, gpr;
  size_t upr;
  // staging registers: the X tile one k step ahead, the weight planes (from
  // HBM, longer latency) two steps ahead in two slots
  // X staging slots: two (X issued two steps ahead) when the register budget
  // allows it, i.e. for widths with at most three planes; one otherwise
  static constexpr int XD = NP <= 3 ? 2 : 1;
  uint4 xreg[XD][CX];
  uint32_t wrec[2][CW][kUnitWords];
  uint16_t sraw[2][CW], zraw[2][CW];
  floatx4 acc[FM][FN];

  __device__ __forceinline__ GemmTile(const GemmArgs& args, int t, int m0_, int n0_) : a(args), tid(t), m0(m0_), n0(n0_) {
    upr = (size_t)(a.k >> 5);
    gpr = a.k / a.group;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // X chunk c (16 B) is row c / 8, k 8 (c % 8) .. + 7: eight consecutive lanes
  // read one row's 128-byte k slice, so the vector cache sees one request per
  // row instead of one per lane.  Unconditional loads from clamped addresses:
  // X rows past m only feed output rows that are never stored.
  template <int XS>
  __device__ __forceinline__ void load_x(int kt) {
    const int k0 = kt * BK;
    const uint16_t* xg = static_cast<const uint16_t*>(a.x);
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int c = (tid + i * T) % (BM * 8);
      const int row = c >> 3, col = 8 * (c & 7);
      const int mrow = min(m0 + row, a.m - 1);
      xreg[XS % XD][i] = *reinterpret_cast<const uint4*>(xg + (size_t)mrow * a.k + k0 + col);
    }
  }
  // the X tile in LDS is row-major, eight 16-byte chunks per row, with chunk
  // c of row r stored at position c ^ (r % 8): the staging writes (eight
  // lanes per row) and the MFMA fragment reads (sixteen rows, one chunk
  // each) then both spread over all banks
  template <int XS>
  __device__ __forceinline__ void store_x(uint4* as) {
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int c = tid + i * T;
      if ((BM * 8) % T == 0 || c < BM * 8) as[(c >> 3) * 8 + ((c & 7) ^ ((c >> 3) & 7))] = xreg[XS % XD][i];
    }
  }
  // weight item it -> (row it / 2, unit it % 2): a lane pair reads one row's two
  // units, i.e. 16 contiguous bytes of a 2-bit plane
  template <int SLOT>
  __device__ __forceinline__ void load_w(int kt) {
    const int gk = (kt * BK) / a.group;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int it = tid + i * T;
      const int row = it >> 1, u = it & 1;
      const int nrow = min(n0 + row, a.n - 1);  // clamped; the output column is never stored
      const size_t unit = (size_t)nrow * upr + (size_t)(kt * 2 + u);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (kPlaneBits[p] == 2) {
          uint2 v = reinterpret_cast<const uint2*>(a.pl.p[p])[unit];
          wrec[SLOT][i][kUnitOff[p]] = v.x;
          wrec[SLOT][i][kUnitOff[p] + 1] = v.y;
        } else {
          wrec[SLOT][i][kUnitOff[p]] = a.pl.p[p][unit];
        }
      }
      const size_t g = (size_t)nrow * gpr + (size_t)gk;
      sraw[SLOT][i] = a.scales[g];
      zraw[SLOT][i] = a.zeros[g];
    }
  }
  // rebuild, slice and dequantize (exactly, in fp32) the staged weights, round
  // once to the MFMA dtype and write them to the LDS tile bs[BN/16][2][64]
  template <int SLOT>
  __device__ __forceinline__ void store_w(uint4* bs) {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int it = tid + i * T;
      const int row = it >> 1, u = it & 1;
      const float s = h2f(sraw[SLOT][i]);
      const float cz = (kDelta - h2f(zraw[SLOT][i])) * s;  // exact
      const uint32_t* rec = wrec[SLOT][i];
      uint32_t bytes[8];
      bytes[0] = assemble_word<NP, 0>(rec);
      bytes[1] = assemble_word<NP, 1>(rec);
      bytes[2] = assemble_word<NP, 2>(rec);
      bytes[3] = assemble_word<NP, 3>(rec);
      bytes[4] = assemble_word<NP, 4>(rec);
      bytes[5] = assemble_word<NP, 5>(rec);
      bytes[6] = assemble_word<NP, 6>(rec);
      bytes[7] = assemble_word<NP, 7>(rec);
      uint32_t h[16];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t v = slice_bytes<R, ROUND>(bytes[j]);
        const float w0 = fmaf((float)(v & 0xFFu), s, cz);
        const float w1 = fmaf((float)((v >> 8) & 0xFFu), s, cz);
        const float w2 = fmaf((float)((v >> 16) & 0xFFu), s, cz);
        const float w3 = fmaf((float)(v >> 24), s, cz);
        h[2 * j] = BF16 ? pack_bf16x2(w0, w1) : pack_f16x2(w0, w1);
        h[2 * j + 1] = BF16 ? pack_bf16x2(w2, w3) : pack_f16x2(w2, w3);
      }
      // 8-k chunk j of this row's k half u is lane (row % 16) + 16 j of block (row / 16, u)
      // (positions in the second k half are xor-ed with 4 so that the lane
      // pair of a row writes to different banks)
      uint4* dst = bs + ((row >> 4) * 2 + u) * 64 + ((row & 15) ^ (4 * u));
      dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
      dst[16] = make_uint4(h[4], h[5], h[6], h[7]);
      dst[32] = make_uint4(h[8], h[9], h[10], h[11]);
      dst[48] = make_uint4(h[12], h[13], h[14], h[15]);
    }
  }
  // MFMAs of one 32-wide k half from LDS tiles as[BM][8], bs[BN/16][2][64]
  __device__ __forceinline__ void mma_half(const uint4* as, const uint4* bs, int kh, int lane, int wm, int wn) {
    {
      uint4 bfr[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = bs[((wn * FN + j) * 2 + kh) * 64 + (lane ^ (4 * kh))];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 af = as[((wm * FM + i) * 16 + (lane & 15)) * 8 + ((kh * 4 + (lane >> 4)) ^ (lane & 7))];
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<BF16>(af, bfr[j], acc[i][j]);
      }
    }
  }
};

template <int R, int ROUND, int BF16, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs a) {
  using Tile = GemmTile<R, ROUND, BF16, BM, BN, WM, WN>;
  constexpr int FM = Tile::FM, FN = Tile::FN;
  // double-buffered LDS tiles: X swizzled row-major, weights fragment-major
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN / 16 * 2 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  // ---- tile selection: workgroups sharing a weight tile land on one XCD ----
  const int G = a.tiles_m * a.tiles_n;
  int logical = blockIdx.x;
  if ((G & 7) == 0) logical = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int tm = logical % a.tiles_m, tn = logical / a.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int KT = a.k / BK;
  const int kt_begin = blockIdx.y * a.ksteps_per_split;
  const int kt_end = min(KT, kt_begin + a.ksteps_per_split);

  Tile t(a, tid, m0, n0);

  if (kt_begin < kt_end) {
    const int klast = kt_end - 1;
    constexpr int XD = Tile::XD;
    t.template load_w<0>(kt_begin);
    t.template load_x<0>(kt_begin);
    t.template load_w<1>(min(kt_begin + 1, klast));
    if constexpr (XD == 2) t.template load_x<1>(min(kt_begin + 1, klast));
    t.template store_x<0>(As[0]);
    t.template store_w<0>(Bs[0]);
    __syncthreads();
    // Two k steps per trip so the LDS buffer and the staging slots are
    // compile-time constants.  Step kt computes from buffer kt & 1, issues the
    // weights for kt + 2 (into the slot that held kt) and X for kt + XD, then
    // writes step kt + 1 (weights loaded a step earlier, X loaded XD - 1 steps
    // earlier) into the other buffer.  Past the last step the loads repeat
    // the last step (in bounds) and nothing more is stored.
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
      {
        const bool has_next = kt + 1 < kt_end;
        if constexpr (XD == 2) t.template load_x<0>(min(kt + 2, klast));
        else if (has_next) t.template load_x<0>(kt + 1);
        t.template load_w<0>(min(kt + 2, klast));
        t.mma_half(As[0], Bs[0], 0, lane, wm, wn);
        t.mma_half(As[0], Bs[0], 1, lane, wm, wn);
        if (has_next) {
          t.template store_x<1>(As[1]);
          t.template store_w<1>(Bs[1]);
        }
        __syncthreads();
      }
      if (kt + 1 < kt_end) {
        const bool has_next = kt + 2 < kt_end;
        if constexpr (XD == 2) t.template load_x<1>(min(kt + 3, klast));
        else if (has_next) t.template load_x<0>(kt + 2);
        t.template load_w<1>(min(kt + 3, klast));
        t.mma_half(As[1], Bs[1], 0, lane, wm, wn);
        t.mma_half(As[1], Bs[1], 1, lane, wm, wn);
        if (has_next) {
          t.template store_x<0>(As[0]);
          t.template store_w<0>(Bs[0]);
        }
        __syncthreads();
      }
    }
  }

  // ---- epilogue: lane holds D[4*(lane/16) + v][lane % 16] of each block ----
  const int mbase = m0 + wm * (BM / WM) + (lane >> 4) * 4;
  const int nbase = n0 + wn * (BN / WN) + (lane & 15);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = nbase + j * 16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = mbase + i * 16 + v;
        if (m < a.m && n < a.n) {
          const float val = t.acc[i][j][v];
          if (a.to_workspace) {
            static_cast<float*>(a.y)[((size_t)blockIdx.y * a.m + m) * a.n + n] = val;
          } else {
            uint16_t* y = static_cast<uint16_t*>(a.y) + (size_t)m * a.n + n;
            *y = (uint16_t)((BF16 ? pack_bf16x2(val, 0.f) : pack_f16x2(val, 0.f)) & 0xFFFFu);
          }
        }
      }
    }
  }
}

// Fixed-order sum of the split-k partials, then one rounding to the output dtype.
template <int BF16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int splits, size_t mn,
                                                            uint16_t* __restrict__ y) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= mn) return;
  // loads are issued eight at a time; the sum is still taken in split order
  float t = 0.f;
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ws[(size_t)(s + j) * mn + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) t += v[j];
  }
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = s + j < splits ? ws[(size_t)(s + j) * mn + i] : 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (s + j < splits) t += v[j];
  y[i] = (uint16_t)((BF16 ? pack_bf16x2(t, 0.f) : pack_f16x2(t, 0.f)) & 0xFFFFu);
}

// ----------------------------------------------------------------------------
// tile configurations and planning
// ----------------------------------------------------------------------------
struct TileCfg {
  int bm, bn;
};
constexpr TileCfg kCfgs[] = {
    {256, 256},  // 0: prefill, 8 waves (2 x 4), wave tile 128 x 64
    {128, 256},  // 1: 8 waves (2 x 4), wave tile 64 x 64
    {64, 256},   // 2: 4 waves (1 x 4), wave tile 64 x 64
    {32, 256},   // 3: 4 waves (1 x 4), wave tile 32 x 64
    {16, 256},   // 4: 4 waves (1 x 4), wave tile 16 x 64
    {128, 128},  // 5: 4 waves (2 x 2), wave tile 64 x 64
    {256, 128},  // 6: 4 waves (2 x 2), wave tile 128 x 64 (accumulators in AGPRs)
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
constexpr int kCUs = 256;
constexpr int kMaxSplits = 16;

static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

static int tiles_of(int cfg, int m, int n) { return cdiv(m, kCfgs[cfg].bm) * cdiv(n, kCfgs[cfg].bn); }

static int pick_cfg(int m, int n) {
  if (m <= 16) return 4;
  if (m <= 32) return 3;
  if (m <= 64) return 2;
  if (m <= 128) return 1;
  return 0;  // 256 x 256: half the dequantization per MAC of a 128-row tile
}

// workgroups of a configuration that fit one CU's LDS (double-buffered X and W tiles)
static int blocks_per_cu(int cfg) {
  const int lds = 2 * (kCfgs[cfg].bm + kCfgs[cfg].bn) * BK * 2;
  const int b = (160 * 1024) / lds;
  return b < 1 ? 1 : (b > 2 ? 2 : b);
}

// When the tiles alone do not fill the GPU, split k to minimise (rounds of
// workgroups over the CUs) x (k steps per split):
// at most 16 splits of at least 8 k steps each; ties go to fewer splits, since
// every split adds workspace traffic and a reduction.  So a split count whose
// workgroups spill into a second, mostly idle round loses to a smaller one
// that fits in a single round.
static int pick_splits(int cfg, int m, int n, int k) {
  const int tiles = tiles_of(cfg, m, n);
  const int KT = k / BK;
  if (tiles * 8 >= kCUs * 7) return 1;  // the tiles alone fill the GPU
  const int slots = kCUs * blocks_per_cu(cfg);
  int best_s = 1;
  long best = (long)cdiv(tiles, slots) * KT;
  for (int s = 2; s <= kMaxSplits && KT / s >= 8; ++s) {
    const long t = (long)cdiv((long)tiles * s, slots) * cdiv(KT, s);
    if (t < best) {
      best = t;
      best_s = s;
    }
  }
  return best_s;
}

size_t gemm_workspace_bytes(int m, int n, int k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  const int cfg = pick_cfg(m, n);
  const int s = pick_splits(cfg, m, n, k);
  return s > 1 ? (size_t)s * (size_t)m * (size_t)n * sizeof(float) : 0;
}

GemmPlan plan_gemm(int m, int n, int k, size_t workspace_bytes) {
  GemmPlan p;
  p.cfg = pick_cfg(m, n);
  p.splits = pick_splits(p.cfg, m, n, k);
  if (p.splits > 1 && workspace_bytes < (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float)) {
    // no room to split: a smaller tile gives more workgroups instead
    p.splits = 1;
    if (p.cfg == 0 && tiles_of(0, m, n) * 8 < kCUs * 7) p.cfg = 5;
  }
  return p;
}

template <int R, int ROUND, int BF16, int BM, int BN, int WM, int WN>
static hipError_t gemm_launch_cfg(const GemmArgs& ga, int splits, hipStream_t s) {
  dim3 grid((unsigned)(ga.tiles_m * ga.tiles_n), (unsigned)splits);
  hipLaunchKernelGGL((gemm_kernel<R, ROUND, BF16, BM, BN, WM, WN>), grid, dim3(64 * WM * WN), 0, s, ga);
  return hipGetLastError();
}

template <int R, int ROUND, int BF16>
static hipError_t gemm_launch_t(const GemmArgs& ga, int cfg, int splits, hipStream_t s) {
  switch (cfg) {
    case 0: return gemm_launch_cfg<R, ROUND, BF16, 256, 256, 2, 4>(ga, splits, s);
    case 1: return gemm_launch_cfg<R, ROUND, BF16, 128, 256, 2, 4>(ga, splits, s);
    case 2: return gemm_launch_cfg<R, ROUND, BF16, 64, 256, 1, 4>(ga, splits, s);
    case 3: return gemm_launch_cfg<R, ROUND, BF16, 32, 256, 1, 4>(ga, splits, s);
    case 4: return gemm_launch_cfg<R, ROUND, BF16, 16, 256, 1, 4>(ga, splits, s);
    case 5: return gemm_launch_cfg<R, ROUND, BF16, 128, 128, 2, 2>(ga, splits, s);
    default: return gemm_launch_cfg<R, ROUND, BF16, 256, 128, 2, 2>(ga, splits, s);
  }
}

template <int R, int ROUND>
static hipError_t gemm_launch_d(const GemmArgs& ga, int bf16, int cfg, int splits, hipStream_t s) {
  return bf16 ? gemm_launch_t<R, ROUND, 1>(ga, cfg, splits, s) : gemm_launch_t<R, ROUND, 0>(ga, cfg, splits, s);
}

hipError_t launch_gemm(const LinearArgs& la, const GemmPlan& plan, void* workspace, hipStream_t s) {
  GemmArgs ga;
  ga.x = la.x;
  ga.pl = la.pl;
  ga.scales = la.scales;
  ga.zeros = la.zeros;
  ga.m = la.m;
  ga.n = la.n;
  ga.k = la.k;
  ga.group = la.group;
  ga.tiles_m = cdiv(la.m, kCfgs[plan.cfg].bm);
  ga.tiles_n = cdiv(la.n, kCfgs[plan.cfg].bn);
  const int KT = la.k / BK;
  const int splits = plan.splits;
  ga.ksteps_per_split = cdiv(KT, splits);
  ga.to_workspace = splits > 1;
  ga.y = splits > 1 ? workspace : la.y;
  hipError_t e;
#define MQ_GEMM_CASE(RR)                                                                   \
  case RR:                                                                                 \
    e = la.round_rule ? gemm_launch_d<RR, 1>(ga, la.bf16, plan.cfg, splits, s)             \
                      : gemm_launch_d<RR, 0>(ga, la.bf16, plan.cfg, splits, s);            \
    break;
  switch (la.r) {
    MQ_GEMM_CASE(2)
    MQ_GEMM_CASE(3)
    MQ_GEMM_CASE(4)
    MQ_GEMM_CASE(6)
    MQ_GEMM_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MQ_GEMM_CASE
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(static_cast<const float*>(workspace), splits, (size_t)la.m * (size_t)la.n, la.y,
                              la.bf16, s);
}

hipError_t launch_splitk_reduce(const float* ws, int splits, size_t mn, void* y, int bf16, hipStream_t s) {
  const unsigned blocks = (unsigned)((mn + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3(blocks), dim3(256), 0, s, ws, splits, mn,
                       static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<0>, dim3(blocks), dim3(256), 0, s, ws, splits, mn,
                       static_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace mq
