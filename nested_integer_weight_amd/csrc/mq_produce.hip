// mq_produce.hip -- the nested parent producer: scale search and cross-width
// code choice ("MatGPTQ: Efficient and Accurate Inference over Nested
// Quantized Models", section 3.2 points 1 and 2, Appendix A.2 Algorithms 1
// and 2), data-free (no Hessian error propagation).
//
// Every decision is an fp32 comparison of sums whose terms and order are fixed:
//   d = w - w_hat,  t = lambda_r * (d * d),  e = e + t  (widths in the given
//   order; in the scale search, the group's weights in index order, widths
//   innermost),
// each operation rounded on its own; ties go to the first candidate.  w_hat =
// s * (v - z) is exact in fp32 (fp16 scale, integer zero point, half-integer
// slice value).  Contraction into fused multiply-adds is switched off for this
// file so the compiler keeps those roundings, and fp32 division is the
// correctly rounded one.
#include "mq_common.h"
#include "mq_kernels.h"

#pragma clang fp contract(off)

namespace mq {
namespace {

// Per-width slice constants, host-derived (all uniform in the kernels).
struct Widths {
  int nr;
  int mask[kMaxProduceWidths];   // true prefix: q & mask keeps the top r bits
  float delta[kMaxProduceWidths];// true prefix: centre offset (2^(8-r) - 1) / 2
  int half[kMaxProduceWidths];   // rounded slices: 2^(8-r-1) (0 at r = 8)
  int shift[kMaxProduceWidths];  // 8 - r
  int cmax[kMaxProduceWidths];   // rounded slice: 2^r - 1; unclamped: 2^r
  float lam[kMaxProduceWidths];
};

// The width-slot-i level of code q (an integer that identifies the
// reconstructed value: the kept top bits, or the rounded code) and that
// level's value v_r(q) in code space.
template <int RULE>
__device__ __forceinline__ int slice_level(int q, const Widths& W, int i) {
  if constexpr (RULE == kRulePrefix) return q & W.mask[i];
  else return min((q + W.half[i]) >> W.shift[i], W.cmax[i]);
}
template <int RULE>
__device__ __forceinline__ float level_value(int lv, const Widths& W, int i) {
  if constexpr (RULE == kRulePrefix) return (float)lv + W.delta[i];
  else return (float)(lv << W.shift[i]);
}
template <int RULE>
__device__ __forceinline__ float slice_value(int q, const Widths& W, int i) {
  return level_value<RULE>(slice_level<RULE>(q, W, i), W, i);
}

__device__ __forceinline__ float weighted_term(float w, float s, float z, float v, float lam) {
  float w_hat = s * (v - z);  // exact
  float d = w - w_hat;
  float dd = d * d;
  return lam * dd;
}

// fp32 -> fp16 bit pattern, one round to nearest even
__device__ __forceinline__ uint16_t f2h_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// ----------------------------------------------------------------------------
// Algorithm 1: one thread per (group, candidate); the block's groups are
// staged in LDS.  Candidate i shrinks the min-max range [min(0, min w),
// max(0, max w)] by p_i = 1 - i / grid_den.
// ----------------------------------------------------------------------------
constexpr int kSearchThreads = 256;

template <int RULE, int NR>
__global__ __launch_bounds__(kSearchThreads) void scale_search_kernel(
    const float* __restrict__ w, size_t n_groups, int group, int groups_per_block, int n_grid, int grid_den,
    Widths W, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
  extern __shared__ float smem[];
  const int stride = group + 4;                          // keeps the groups' rows on different banks
  float* err = smem + (size_t)groups_per_block * stride;  // [groups_per_block][n_grid]
  const size_t g0 = (size_t)blockIdx.x * groups_per_block;
  const int gb_here = (int)min((size_t)groups_per_block, n_groups - g0);
  const int tid = threadIdx.x;

  // stage the groups (float4 loads; group % 64 == 0)
  const int q4 = group / 4;
  for (int e = tid; e < gb_here * q4; e += kSearchThreads) {
    int gb = e / q4, j4 = e - gb * q4;
    float4 v = reinterpret_cast<const float4*>(w + (g0 + gb) * (size_t)group)[j4];
    float* dst = smem + gb * stride + 4 * j4;
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
  __syncthreads();

  const int pairs = gb_here * n_grid;
  if (tid < pairs) {
    const int gb = tid / n_grid, i = tid - gb * n_grid;
    const float* wg = smem + gb * stride;
    float lo = 0.0f, hi = 0.0f;
    for (int j = 0; j < group; ++j) {
      lo = fminf(lo, wg[j]);
      hi = fmaxf(hi, wg[j]);
    }
    const float p = 1.0f - (float)i / (float)grid_den;
    const float lo_p = p * lo, hi_p = p * hi;
    uint16_t sb = f2h_bits((hi_p - lo_p) / 255.0f);
    if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;  // 1.0
    const float s = h2f(sb);
    const float z = fminf(fmaxf(rintf(-lo_p / s), 0.0f), 255.0f) + 0.0f;  // +0, never -0
    // The nearest code needs rint of the correctly rounded w / s.  With the
    // reciprocal r = RN(1 / s), y = RN(w r) is within 4 units in the last
    // place of RN(w / s) (two roundings of 2^-24 each, plus the quotient's
    // own), so rint(y) is the same integer unless a half-integer lies within
    // that distance of y; only then (about one weight in 4000) is the quotient
    // divided out.  Beyond |y| = 600 both clamp to the same code (|z| <= 255).
    const float rs = 1.0f / s;
    // v_r(q) - z for the true prefix as float(q & mask) + (delta_r - z): exact
    float cz[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) cz[t] = W.delta[t] - z;
    float acc = 0.0f;
    for (int j = 0; j < group; ++j) {
      const float wj = wg[j];
      const float y = wj * rs;
      const float ay = fabsf(y);
      float qf = rintf(y);
      if (fabsf((y - floorf(y)) - 0.5f) <= ay * 0x1p-21f && ay <= 600.0f) qf = rintf(wj / s);
      const int q = (int)fminf(fmaxf(qf + z, 0.0f), 255.0f);
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        float vz;  // v_r(q) - z, exact
        if constexpr (RULE == kRulePrefix) vz = (float)(q & W.mask[t]) + cz[t];
        else vz = slice_value<RULE>(q, W, t) - z;
        const float d = wj - s * vz;
        const float dd = d * d;
        acc = acc + W.lam[t] * dd;
      }
    }
    err[gb * n_grid + i] = acc;
  }
  __syncthreads();

  // first minimum over the candidates of each group; its (s, z) is recomputed
  if (tid < gb_here) {
    const float* eg = err + tid * n_grid;
    int best = 0;
    float be = eg[0];
    for (int i = 1; i < n_grid; ++i)
      if (eg[i] < be) { be = eg[i]; best = i; }
    const float* wg = smem + tid * stride;
    float lo = 0.0f, hi = 0.0f;
    for (int j = 0; j < group; ++j) {
      lo = fminf(lo, wg[j]);
      hi = fmaxf(hi, wg[j]);
    }
    const float p = 1.0f - (float)best / (float)grid_den;
    const float lo_p = p * lo, hi_p = p * hi;
    uint16_t sb = f2h_bits((hi_p - lo_p) / 255.0f);
    if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;
    const float s = h2f(sb);
    const float z = fminf(fmaxf(rintf(-lo_p / s), 0.0f), 255.0f) + 0.0f;
    scales[g0 + tid] = sb;
    zeros[g0 + tid] = f2h_bits(z);  // integer 0..255: exact
  }
}

// ----------------------------------------------------------------------------
// Algorithm 2: one thread per four consecutive weights (one group), every
// code q = 0..255 scored in order.  q is uniform across the wave, so each
// width's level and its "level changed" test run on the scalar unit; a term
// is recomputed only when its width's level changes (the term depends on q
// only through that level, so the values are those of scoring every q).
// ----------------------------------------------------------------------------
constexpr int kChooseThreads = 256;

template <int RULE, int NR>
__global__ __launch_bounds__(kChooseThreads) void choose_codes_kernel(
    const float* __restrict__ w, size_t n_quads, int group, Widths W, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, uint32_t* __restrict__ codes) {
  const size_t u = (size_t)blockIdx.x * kChooseThreads + threadIdx.x;
  if (u >= n_quads) return;
  const float4 w4 = reinterpret_cast<const float4*>(w)[u];
  const size_t g = (u * 4) / (size_t)group;
  const float s = h2f(scales[g]);
  const float z = h2f(zeros[g]);
  const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
  float term[NR][4];
  int level[NR];
  float best[4];
  int bq[4];
#pragma unroll
  for (int t = 0; t < NR; ++t) level[t] = -1;
#pragma unroll
  for (int b = 0; b < 4; ++b) { best[b] = 0.0f; bq[b] = 0; }

  for (int q = 0; q < 256; ++q) {
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const int lv = slice_level<RULE>(q, W, t);  // uniform: scalar unit
      if (lv != level[t]) {
        level[t] = lv;
        const float v = level_value<RULE>(lv, W, t);
#pragma unroll
        for (int b = 0; b < 4; ++b) term[t][b] = weighted_term(wv[b], s, z, v, W.lam[t]);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float e = term[0][b];
#pragma unroll
      for (int t = 1; t < NR; ++t) e = e + term[t][b];
      if (q == 0 || e < best[b]) { best[b] = e; bq[b] = q; }
    }
  }
  codes[u] = (uint32_t)bq[0] | ((uint32_t)bq[1] << 8) | ((uint32_t)bq[2] << 16) | ((uint32_t)bq[3] << 24);
}

Widths make_widths(const int* widths, const float* lambdas, int nr, int rule) {
  Widths W{};
  W.nr = nr;
  for (int t = 0; t < nr; ++t) {
    const int r = widths[t], sh = 8 - r;
    W.shift[t] = sh;
    W.mask[t] = (0xFF << sh) & 0xFF;
    W.delta[t] = 0.5f * (float)((1 << sh) - 1);
    W.half[t] = sh > 0 ? 1 << (sh - 1) : 0;
    W.cmax[t] = (rule == kRuleExtra && r < 8) ? (1 << r) : (1 << r) - 1;
    W.lam[t] = lambdas[t];
  }
  return W;
}

}  // namespace

// Groups per search block: as many as the candidates leave threads for (at
// most 16), within 60 KiB of LDS (group + 4 floats of weights and n_grid
// floats of errors per group).
static int produce_groups_per_block(int group, int n_grid) {
  const int by_lds = (int)((60u << 10) / (sizeof(float) * (size_t)(group + 4 + n_grid)));
  return max(1, min(min(16, kSearchThreads / n_grid), by_lds));
}

template <int RULE, int NR>
static hipError_t produce_launch(const float* w, int n, int k, int group, const Widths& W, int n_grid, int grid_den,
                                 uint8_t* codes, uint16_t* scales, uint16_t* zeros, hipStream_t s) {
  const size_t n_groups = (size_t)n * (size_t)(k / group);
  const int gpb = produce_groups_per_block(group, n_grid);
  const size_t blocks = (n_groups + gpb - 1) / gpb;
  const size_t lds = sizeof(float) * (size_t)gpb * (size_t)(group + 4 + n_grid);
  hipLaunchKernelGGL((scale_search_kernel<RULE, NR>), dim3((unsigned)blocks), dim3(kSearchThreads), lds, s, w,
                     n_groups, group, gpb, n_grid, grid_den, W, scales, zeros);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n_quads = (size_t)n * (size_t)k / 4;
  const size_t cblocks = (n_quads + kChooseThreads - 1) / kChooseThreads;
  hipLaunchKernelGGL((choose_codes_kernel<RULE, NR>), dim3((unsigned)cblocks), dim3(kChooseThreads), 0, s, w,
                     n_quads, group, W, scales, zeros, reinterpret_cast<uint32_t*>(codes));
  return hipGetLastError();
}

template <int RULE>
static hipError_t produce_rule(const float* w, int n, int k, int group, const Widths& W, int n_grid, int grid_den,
                               uint8_t* codes, uint16_t* scales, uint16_t* zeros, hipStream_t s) {
  switch (W.nr) {
    case 1: return produce_launch<RULE, 1>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
    case 2: return produce_launch<RULE, 2>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
    case 3: return produce_launch<RULE, 3>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
    case 4: return produce_launch<RULE, 4>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
    case 5: return produce_launch<RULE, 5>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_produce(const float* w, int n, int k, int group, const int* widths, const float* lambdas, int nr,
                          int rule, int n_grid, int grid_den, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                          hipStream_t s) {
  const Widths W = make_widths(widths, lambdas, nr, rule);
  if (rule == kRuleExtra) return produce_rule<kRuleExtra>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
  if (rule == kRuleRound) return produce_rule<kRuleRound>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
  return produce_rule<kRulePrefix>(w, n, k, group, W, n_grid, grid_den, codes, scales, zeros, s);
}

}  // namespace mq
