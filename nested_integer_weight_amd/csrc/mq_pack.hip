// mq_pack.hip -- parent packer and the slice / dequant export kernels.
//
// Packing follows MatGPTQ ("Efficient and Accurate Inference over Nested
// Quantized Models", section 4): the 8-bit codes are split offline into five
// MSB-first bit-plane buffers (bits 1-2, 3, 4, 5-6, 7-8) so that a width-r
// call reads only the leading planes.  The in-unit bit order is this
// library's own (see mq_common.h): it lets one shift and one mask per plane
// rebuild four codes as bytes.
//
// The export kernels rebuild codes through exactly the same device helpers
// (assemble_word, slice_pairs / slice_bytes / slice_f32x4) that the GEMV and
// the GEMM use.
#include "mq_common.h"
#include "mq_kernels.h"

namespace mq {

// One thread per (row, 32-code unit).
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, size_t n_units,
                                                   int units_per_row, uint32_t* __restrict__ p0,
                                                   uint32_t* __restrict__ p1, uint32_t* __restrict__ p2,
                                                   uint32_t* __restrict__ p3, uint32_t* __restrict__ p4) {
  size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= n_units) return;
  const uint4* src = reinterpret_cast<const uint4*>(codes + u * 32);
  uint4 a = src[0], b = src[1];
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t two[3][2] = {{0, 0}, {0, 0}, {0, 0}};  // planes 0, 3, 4
  uint32_t one[2] = {0, 0};                         // planes 1, 2
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    uint32_t c = (w[t / 4] >> (8 * (t % 4))) & 0xFFu;
    int word = t / 16;
    int pos2 = 8 * (t % 4) + 2 * ((t % 16) / 4);
    int pos1 = 8 * (t % 4) + t / 4;
    two[0][word] |= ((c >> 6) & 3u) << pos2;
    two[1][word] |= ((c >> 2) & 3u) << pos2;
    two[2][word] |= (c & 3u) << pos2;
    one[0] |= ((c >> 5) & 1u) << pos1;
    one[1] |= ((c >> 4) & 1u) << pos1;
  }
  reinterpret_cast<uint2*>(p0)[u] = make_uint2(two[0][0], two[0][1]);
  p1[u] = one[0];
  p2[u] = one[1];
  reinterpret_cast<uint2*>(p3)[u] = make_uint2(two[1][0], two[1][1]);
  reinterpret_cast<uint2*>(p4)[u] = make_uint2(two[2][0], two[2][1]);
  (void)units_per_row;
}

// Load the first NP planes of unit u into an 8-word unit record.
template <int NP>
__device__ __forceinline__ void load_unit(const PlanePtrs& pl, size_t u, uint32_t* rec) {
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (kPlaneBits[p] == 2) {
      uint2 v = reinterpret_cast<const uint2*>(pl.p[p])[u];
      rec[kUnitOff[p]] = v.x;
      rec[kUnitOff[p] + 1] = v.y;
    } else {
      rec[kUnitOff[p]] = pl.p[p][u];
    }
  }
}

template <int NP, int J = 0>
__device__ __forceinline__ void assemble_unit(const uint32_t* rec, uint32_t* out) {
  if constexpr (J < 8) {
    out[J] = assemble_word<NP, J>(rec);
    assemble_unit<NP, J + 1>(rec, out);
  }
}

template <int R, int RULE>
__global__ __launch_bounds__(256) void slice_kernel(PlanePtrs pl, size_t n_units, uint8_t* __restrict__ out) {
  constexpr int NP = planes_needed(R, RULE);
  size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= n_units) return;
  uint32_t rec[kUnitWords];
  load_unit<NP>(pl, u, rec);
  uint32_t bytes[8];
  assemble_unit<NP>(rec, bytes);
  uint32_t res[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (RULE == kRuleExtra && R < 8) {
      // the unclamped code reaches 2^r: taken from the 16-bit lanes (the low
      // 8 - r bits of each lane are zero, so the shifts move no bits between lanes)
      uint32_t lo, hi;
      slice_pairs<R, RULE>(bytes[j], lo, hi);
      lo >>= 8 - R;
      hi >>= 8 - R;
      res[j] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);  // codes <= 128 fit a byte
    } else {
      uint32_t v = slice_bytes<R, RULE>(bytes[j]);
      if constexpr (!RULE) v &= rep4((0xFFu << (8 - R)) & 0xFFu);  // exactly r bits
      res[j] = (v >> (8 - R)) & rep4(0xFFu >> (8 - R));                // r-bit code
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(out + u * 32);
  dst[0] = make_uint4(res[0], res[1], res[2], res[3]);
  dst[1] = make_uint4(res[4], res[5], res[6], res[7]);
}

// out_dtype: 0 = f32, 1 = f16, 2 = bf16
template <int R, int RULE, int OUT>
__global__ __launch_bounds__(256) void dequant_kernel(PlanePtrs pl, size_t n_units, int units_per_row,
                                                      int groups_per_row, int units_per_group,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ zeros,
                                                      void* __restrict__ out) {
  constexpr int NP = planes_needed(R, RULE);
  size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= n_units) return;
  size_t row = u / (size_t)units_per_row;
  int col_unit = (int)(u - row * (size_t)units_per_row);
  size_t g = row * (size_t)groups_per_row + (size_t)(col_unit / units_per_group);
  float s = h2f(scales[g]);
  float z = h2f(zeros[g]);
  float c = ((RULE ? 0.0f : prefix_delta(R)) - z) * s;  // exact: half-integer * fp16
  uint32_t rec[kUnitWords];
  load_unit<NP>(pl, u, rec);
  uint32_t bytes[8];
  assemble_unit<NP>(rec, bytes);
  float w[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v[4];
    slice_f32x4<R, RULE>(bytes[j], v);
#pragma unroll
    for (int b = 0; b < 4; ++b) w[4 * j + b] = fmaf(v[b], s, c);
  }
  if constexpr (OUT == 0) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + u * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else {
    uint32_t h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      h[i] = (OUT == 1) ? pack_f16x2(w[2 * i], w[2 * i + 1]) : pack_bf16x2(w[2 * i], w[2 * i + 1]);
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + u * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
  }
}

// ----------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------
static inline unsigned blocks_for(size_t n, unsigned t) { return (unsigned)((n + t - 1) / t); }

hipError_t launch_pack(const uint8_t* codes, int n, int k, uint32_t* const planes[5], hipStream_t s) {
  size_t n_units = (size_t)n * (size_t)(k / 32);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks_for(n_units, 256)), dim3(256), 0, s, codes, n_units, k / 32,
                     planes[0], planes[1], planes[2], planes[3], planes[4]);
  return hipGetLastError();
}

template <int R, int RULE>
static void slice_dispatch_r(const PlanePtrs& pl, size_t n_units, uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL((slice_kernel<R, RULE>), dim3(blocks_for(n_units, 256)), dim3(256), 0, s, pl, n_units,
                     out);
}

hipError_t launch_slice(const PlanePtrs& pl, int n, int k, int r, int rule, uint8_t* out, hipStream_t s) {
  size_t n_units = (size_t)n * (size_t)(k / 32);
#define MQ_SLICE_CASE(RR)                                                   \
  case RR:                                                                  \
    if (rule == kRuleExtra) slice_dispatch_r<RR, kRuleExtra>(pl, n_units, out, s); \
    else if (rule == kRuleRound) slice_dispatch_r<RR, kRuleRound>(pl, n_units, out, s);     \
    else slice_dispatch_r<RR, kRulePrefix>(pl, n_units, out, s);                        \
    break;
  switch (r) {
    MQ_SLICE_CASE(2)
    MQ_SLICE_CASE(3)
    MQ_SLICE_CASE(4)
    MQ_SLICE_CASE(6)
    MQ_SLICE_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MQ_SLICE_CASE
  return hipGetLastError();
}

template <int R, int RULE>
static void dequant_dispatch_r(const PlanePtrs& pl, int n, int k, int group, const uint16_t* sc,
                               const uint16_t* zr, int out_dtype, void* out, hipStream_t s) {
  size_t n_units = (size_t)n * (size_t)(k / 32);
  dim3 grid(blocks_for(n_units, 256)), block(256);
  int upr = k / 32, gpr = k / group, upg = group / 32;
  if (out_dtype == 0)
    hipLaunchKernelGGL((dequant_kernel<R, RULE, 0>), grid, block, 0, s, pl, n_units, upr, gpr, upg, sc, zr, out);
  else if (out_dtype == 1)
    hipLaunchKernelGGL((dequant_kernel<R, RULE, 1>), grid, block, 0, s, pl, n_units, upr, gpr, upg, sc, zr, out);
  else
    hipLaunchKernelGGL((dequant_kernel<R, RULE, 2>), grid, block, 0, s, pl, n_units, upr, gpr, upg, sc, zr, out);
}

hipError_t launch_dequant(const PlanePtrs& pl, int n, int k, int r, int rule, int group,
                          const uint16_t* scales, const uint16_t* zeros, int out_dtype, void* out,
                          hipStream_t s) {
#define MQ_DQ_CASE(RR)                                                                              \
  case RR:                                                                                          \
    if (rule == kRuleExtra)                                                                        \
      dequant_dispatch_r<RR, kRuleExtra>(pl, n, k, group, scales, zeros, out_dtype, out, s);       \
    else if (rule == kRuleRound)                                                                        \
      dequant_dispatch_r<RR, kRuleRound>(pl, n, k, group, scales, zeros, out_dtype, out, s);            \
    else                                                                                            \
      dequant_dispatch_r<RR, kRulePrefix>(pl, n, k, group, scales, zeros, out_dtype, out, s);           \
    break;
  switch (r) {
    MQ_DQ_CASE(2)
    MQ_DQ_CASE(3)
    MQ_DQ_CASE(4)
    MQ_DQ_CASE(6)
    MQ_DQ_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MQ_DQ_CASE
  return hipGetLastError();
}

}  // namespace mq
