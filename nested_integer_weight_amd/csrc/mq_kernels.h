// mq_kernels.h -- host-side launchers implemented in the .hip files.  Every
// launcher assumes validated arguments (mq_api.hip validates) and returns
// hipGetLastError() after its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mq_common.h"

namespace mq {

hipError_t launch_pack(const uint8_t* codes, int n, int k, uint32_t* const planes[5], hipStream_t s);
hipError_t launch_slice(const PlanePtrs& pl, int n, int k, int r, int round_rule, uint8_t* out,
                        hipStream_t s);
hipError_t launch_dequant(const PlanePtrs& pl, int n, int k, int r, int round_rule, int group,
                          const uint16_t* scales, const uint16_t* zeros, int out_dtype, void* out,
                          hipStream_t s);

struct LinearArgs {
  const void* x;
  void* y;
  PlanePtrs pl;
  const uint16_t* scales;
  const uint16_t* zeros;
  int m, n, k, group, r, round_rule;
  int bf16;  // 1: x/y are bf16, 0: fp16
};

// register GEMV: fp16 activations with m <= 4, bf16 activations with m == 1,
// k <= kGemvMaxK (one lane per 64-code slice, at most 4 waves per row)
constexpr int kGemvMaxM = 4;
constexpr int kGemvMaxK = 16384;
__host__ inline bool gemv_eligible(int m, int k, int bf16) {
  return m >= 1 && k <= kGemvMaxK && (bf16 ? m == 1 : m <= kGemvMaxM);
}
hipError_t launch_gemv(const LinearArgs& a, hipStream_t s);
// up to kGemvMaxBatch independent GEMV-eligible calls that share m, k, width,
// rule, group and dtype, in one launch (no call may read or write another's
// output)
constexpr int kGemvMaxBatch = 4;
hipError_t launch_gemv_batch(const LinearArgs* a, int ncalls, hipStream_t s);

// MFMA skinny path (weights dequantized straight into MFMA operand registers,
// activations shared through LDS): 2 <= m <= 64 with k a multiple of 256.
constexpr int kSkinnyMaxM = 64;
__host__ inline bool skinny_eligible(int m, int k) { return m >= 2 && m <= kSkinnyMaxM && k % 256 == 0; }
struct SkinnyPlan {
  int splits;            // k ranges (1 = no workspace)
  int rounds_per_split;  // 256-wide k rounds per range
  int nt;                // 16-row tiles per wave: 1 (64-row workgroups) or 2 (128-row)
  int kh;                // teams of 4 waves per workgroup splitting its k range (1 or 2)
  int run;               // 64-code runs per lane, row and round (1 or 2)
};
SkinnyPlan plan_skinny(int m, int n, int k, int group, int planes);
size_t skinny_workspace_bytes(int m, int n, int k);
hipError_t launch_skinny(const LinearArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s);

// fixed-order sum of fp32 split-k partials ws[splits][mn] rounded once into y (fp16 or bf16)
hipError_t launch_splitk_reduce(const float* ws, int splits, size_t mn, void* y, int bf16, hipStream_t s);

// MFMA GEMM (dequantized weight tiles in LDS), any m >= 1.
struct GemmPlan {
  int cfg;       // tile configuration index
  int splits;    // split-k factor (1 = no workspace)
};
GemmPlan plan_gemm(int m, int n, int k, size_t workspace_bytes);
size_t gemm_workspace_bytes(int m, int n, int k);
hipError_t launch_gemm(const LinearArgs& a, const GemmPlan& plan, void* workspace, hipStream_t s);

}  // namespace mq
