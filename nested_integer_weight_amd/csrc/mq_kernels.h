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
hipError_t launch_slice(const PlanePtrs& pl, int n, int k, int r, int rule, uint8_t* out,
                        hipStream_t s);
hipError_t launch_dequant(const PlanePtrs& pl, int n, int k, int r, int rule, int group,
                          const uint16_t* scales, const uint16_t* zeros, int out_dtype, void* out,
                          hipStream_t s);

struct LinearArgs {
  const void* x;
  void* y;
  PlanePtrs pl;
  const uint16_t* scales;
  const uint16_t* zeros;
  int m, n, k, group, r;
  int rule;  // kRulePrefix, kRuleRound or kRuleExtra
  int bf16;  // 1: x/y are bf16, 0: fp16
};

// register GEMV: fp16 activations with m <= 4, bf16 activations with m == 1,
// k <= kGemvMaxK (one lane per 64-code slice, at most 4 waves per row)
constexpr int kGemvMaxM = 4;
constexpr int kGemvMaxK = 16384;
__host__ inline bool gemv_eligible(int m, int k, int bf16) {
  return m >= 1 && k <= kGemvMaxK && (bf16 ? m == 1 : m <= kGemvMaxM);
}
// Up to kGemvMaxCalls independent GEMV-eligible calls that share m, rule and
// dtype (any width, n, k, group) in one launch.  No call may write what
// another call of the launch reads or writes.
constexpr int kGemvMaxCalls = 32;
hipError_t launch_gemv_multi(const LinearArgs* a, int ncalls, hipStream_t s);

// MFMA skinny path (weights dequantized straight into MFMA operand registers,
// activations shared through LDS): 2 <= m <= 64 with k a multiple of 256.
constexpr int kSkinnyMaxM = 64;
// (true prefix and rounded slice; the unclamped rule takes the GEMM)
__host__ inline bool skinny_shape(int m, int k) { return m >= 2 && m <= kSkinnyMaxM && k % 256 == 0; }
__host__ inline bool skinny_eligible(int m, int k, int rule) { return skinny_shape(m, k) && rule != kRuleExtra; }
struct SkinnyPlan {
  int splits;            // k ranges (1 = no workspace)
  int rounds_per_split;  // 256-wide k rounds per range
  int nt;                // 16-row tiles per wave: 1 (64-row workgroups; the only plan taken)
  int kh;                // teams of 4 waves per workgroup splitting its k range (1 or 2)
  int run;               // 64-code runs per lane, row and round (1 or 2)
};
SkinnyPlan plan_skinny(int m, int n, int k, int group, int planes);
size_t skinny_workspace_bytes(int m, int n, int k);
hipError_t launch_skinny(const LinearArgs& a, void* workspace, size_t workspace_bytes, hipStream_t s);
// Up to kSkinnyMaxCalls independent skinny calls of one launch shape (same m,
// width, rule, dtype and planned row tiles, teams and run length) in one
// launch.  Each call keeps its own plan; a call with a k split takes the next
// 256-byte-aligned part of the workspace (and runs unsplit when that part
// does not fit, as a single call would), and its partial sums are reduced
// after the launch.
constexpr int kSkinnyMaxCalls = 8;
__host__ inline size_t ws_align(size_t b) { return (b + 255) & ~(size_t)255; }
bool same_skinny_launch(const LinearArgs& a, const LinearArgs& b);
size_t skinny_call_workspace(const LinearArgs& a);  // bytes of its k split, 0 when it does not split
hipError_t launch_skinny_multi(const LinearArgs* a, int ncalls, void* workspace, size_t workspace_bytes,
                               hipStream_t s);

// fixed-order sum of fp32 split-k partials ws[splits][mn] rounded once into y (fp16 or bf16)
hipError_t launch_splitk_reduce(const float* ws, int splits, size_t mn, void* y, int bf16, hipStream_t s);

// MFMA GEMM (dequantized weight tiles in LDS), any m >= 1, k <= kMaxLinearK
// (its 32-bit byte offsets into a 256-row activation window).
constexpr int kMaxLinearK = 1 << 22;
struct GemmPlan {
  int cfg;       // tile configuration index
  int splits;    // split-k factor (1 = no workspace)
};
GemmPlan plan_gemm(int m, int n, int k, size_t workspace_bytes);
// Up to kGemmMaxCalls independent calls of the prefill tile (m > 128) with the
// same width, rule and dtype in one launch, none split over k.  Every output
// sums its k steps in the same order whatever the tile configuration, split
// or launch, so a call's result equals that of mq_linear without a workspace.
// Worth it when the calls' tiles together fill the GPU (kGemmBatchMinTiles).
constexpr int kGemmMaxCalls = 32;
constexpr int kGemmBatchMinTiles = 224;
bool gemm_batchable(const LinearArgs& a);
bool same_gemm_launch(const LinearArgs& a, const LinearArgs& b);
int gemm_tiles(const LinearArgs& a);
hipError_t launch_gemm_multi(const LinearArgs* a, int ncalls, hipStream_t s);
size_t gemm_workspace_bytes(int m, int n, int k);
hipError_t launch_gemm(const LinearArgs& a, const GemmPlan& plan, void* workspace, hipStream_t s);

// Parent producer: scale search, then the cross-width code choice, for
// nr <= kMaxProduceWidths distinct widths (validated by the caller).
constexpr int kMaxProduceWidths = 5;
constexpr int kMaxProduceGroup = 1024;
constexpr int kMaxProduceGrid = 256;
hipError_t launch_produce(const float* w, int n, int k, int group, const int* widths, const float* lambdas, int nr,
                          int rule, int n_grid, int grid_den, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                          hipStream_t s);

}  // namespace mq
