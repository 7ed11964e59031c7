// mq_gemm.hip -- MFMA path for prefill and batches the skinny and GEMV paths do not take.
//
// Y[m, n] = sum_k X[m, k] * w_hat[n, k].  Per 64-wide k step a workgroup
//  * copies its X tile (BM x 64, fp16/bf16) global -> VGPR -> LDS,
//  * loads the packed planes of its weight tile (BN rows x two 32-code units)
//    and, at the first step of each quantization group, the group's scale and
//    zero point, rebuilds and slices the codes in VGPRs and dequantizes them
//    exactly in fp32 (w_hat = v*s + (delta - z)*s, exact for an fp16 scale
//    and an integer zero point; computed from the exact fp16 halves 1024 + v
//    with one fma per weight), rounds once to the activation dtype and
//    writes the tile to LDS,
//  * runs v_mfma_f32_16x16x32_{bf16,f16} from LDS with fp32 accumulators.
// LDS is double buffered, so one barrier per step suffices: a step computes
// from one buffer pair while the next step's tiles are written to the other.
// In the eight-wave prefill tile half the waves stage the next step before
// their MFMAs and half after, so on every SIMD one wave's dequantization
// overlaps the other wave's matrix work.  Operands are read with buffer loads
// from per-workgroup windows (scalar bases, fixed 32-bit lane offsets, the k
// step in the scalar offset).
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
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

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

// Raw buffer descriptor of a workgroup's window of an operand: the base in
// scalar registers (read-first-lane), no stride, 4 GiB - 1 bytes.  Lanes then
// address the window with 32-bit byte offsets that stay fixed over the k loop,
// and the k step goes into the scalar offset, so the loop keeps no 64-bit
// addresses in vector registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window_rsrc(const void* base) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), (short)0, -1, 0x00020000);
}

// Per-thread state of one workgroup tile.  Helpers are force-inlined member
// functions (not lambdas capturing arrays by reference), so the staging
// arrays are scalarised into registers instead of living in memory.
template <int R, int RULE, int BF16, int BM, int BN, int WM, int WN>
struct GemmTile {
  static constexpr int T = 64 * WM * WN;
  static constexpr int NP = planes_needed(R, RULE);
  static constexpr int FM = BM / WM / 16;
  static constexpr int FN = BN / WN / 16;
  static constexpr int CX = (BM * 8 + T - 1) / T;  // 16-byte X chunks per thread per step
  static constexpr int CW = BN * 2 / T;             // (row, unit) weight items per thread per step
  static_assert(CW >= 1 && CW * T == BN * 2, "W tile split");
  static constexpr float kDelta = RULE ? 0.0f : prefix_delta(R);

  int tid;
  // descriptors of the workgroup's windows (X rows from m0, weight rows from n0)
  __amdgpu_buffer_rsrc_t rx, rp[NP], rs, rz;
  int xoff[CX];           // byte offset of the thread's X chunks in the window at k = 0
  int woff[CW], goff[CW];  // byte offsets of its weight items (1-bit plane units) and their groups
  int gsteps;              // k steps per group
  int kfirst;              // first k step of the workgroup's range
  // staging registers: the X tile one k step ahead, the weight planes two
  // steps ahead in two slots
  uint4 xreg[CX];
  uint32_t wrec[2][CW][kUnitWords];
  uint16_t sraw[2][CW], zraw[2][CW];
  // scale and zero point of the last step written to LDS: a step in the same
  // group as its predecessor takes them from here instead of loading them
  uint16_t scur[CW], zcur[CW];
  floatx4 acc[FM][FN];

  __device__ __forceinline__ GemmTile(const GemmArgs& a, int t, int m0, int n0) : tid(t) {
    const int upr = a.k >> 5, gpr = a.k / a.group;
    rx = window_rsrc(static_cast<const uint16_t*>(a.x) + (size_t)m0 * a.k);
#pragma unroll
    for (int p = 0; p < NP; ++p) rp[p] = window_rsrc(a.pl.p[p] + (size_t)n0 * upr * kPlaneBits[p]);
    rs = window_rsrc(a.scales + (size_t)n0 * gpr);
    rz = window_rsrc(a.zeros + (size_t)n0 * gpr);
    // X chunk c (16 B) is row c / 8, k 8 (c % 8) .. + 7: eight consecutive
    // lanes read one row's 128-byte k slice.  Rows past m are clamped to
    // m - 1: they only feed output rows that are never stored.
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int c = (tid + i * T) % (BM * 8);
      const int row = min(c >> 3, a.m - 1 - m0);
      xoff[i] = (row * a.k + 8 * (c & 7)) * 2;
    }
    // weight item it -> (row it / 2, unit it % 2): a lane pair reads one
    // row's two units, i.e. 16 contiguous bytes of a 2-bit plane; rows past n
    // are clamped (their output columns are never stored)
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int it = tid + i * T;
      const int row = min(it >> 1, a.n - 1 - n0);
      woff[i] = (row * upr + (it & 1)) * 4;
      goff[i] = row * gpr * 2;
    }
    gsteps = a.group / BK;
    kfirst = 0;
#pragma unroll
    for (int i = 0; i < CW; ++i) scur[i] = zcur[i] = 0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  __device__ __forceinline__ void load_x(int kt) {
#pragma unroll
    for (int i = 0; i < CX; ++i)
      xreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], kt * BK * 2, 0));
  }
  // the X tile in LDS is row-major, eight 16-byte chunks per row, with chunk
  // c of row r stored at position c ^ (r % 8): the staging writes (eight
  // lanes per row) and the MFMA fragment reads (sixteen rows, one chunk
  // each) then both spread over all banks
  __device__ __forceinline__ void store_x(uint4* as) {
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int c = tid + i * T;
      if ((BM * 8) % T == 0 || c < BM * 8) as[(c >> 3) * 8 + ((c & 7) ^ ((c >> 3) & 7))] = xreg[i];
    }
  }
  // does step kt start a group (or the range), so that it loads its own scale and zero point?
  __device__ __forceinline__ bool own_sz(int kt) const { return kt == kfirst || kt % gsteps == 0; }
  template <int SLOT>
  __device__ __forceinline__ void load_w(int kt) {
    const int gk = kt / gsteps;
    const bool sz = own_sz(kt);
#pragma unroll
    for (int i = 0; i < CW; ++i) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (kPlaneBits[p] == 2) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rp[p], woff[i] * 2, kt * 16, 0);
          wrec[SLOT][i][kUnitOff[p]] = v[0];
          wrec[SLOT][i][kUnitOff[p] + 1] = v[1];
        } else {
          wrec[SLOT][i][kUnitOff[p]] = __builtin_amdgcn_raw_buffer_load_b32(rp[p], woff[i], kt * 8, 0);
        }
      }
      if (sz) {
        sraw[SLOT][i] = __builtin_amdgcn_raw_buffer_load_b16(rs, goff[i], gk * 2, 0);
        zraw[SLOT][i] = __builtin_amdgcn_raw_buffer_load_b16(rz, goff[i], gk * 2, 0);
      }
    }
  }
  // rebuild, slice and dequantize (exactly, in fp32) the staged weights, round
  // once to the MFMA dtype and write them to the LDS tile bs[BN/16][2][64]
  // (step kt: the step whose weights slot SLOT holds; steps are written in order)
  template <int SLOT>
  __device__ __forceinline__ void store_w(uint4* bs, int kt) {
    const bool sz = own_sz(kt);
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int it = tid + i * T;
      const int row = it >> 1, u = it & 1;
      if (sz) {
        scur[i] = sraw[SLOT][i];
        zcur[i] = zraw[SLOT][i];
      }
      const float s = h2f(scur[i]);
      const float cz = (kDelta - h2f(zcur[i])) * s;  // exact
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
      if constexpr (RULE != kRuleExtra || R == 8) {
        // slice values v <= 255: v_perm puts each byte under an fp16 exponent
        // byte, giving the exact halves 1024 + v, and one fma per weight with
        // the 1024 folded into the constant, (1024 + v) s + (cz - 1024 s),
        // gives v s + cz exactly (the constant needs at most 24 significant
        // bits, the result at most 21)
        const float c1 = cz - 1024.0f * s;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = slice_bytes<R, RULE>(bytes[j]);
          const f16x2_t p0 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u));
          const f16x2_t p1 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u));
          const float w0 = fmaf((float)p0[0], s, c1);
          const float w1 = fmaf((float)p0[1], s, c1);
          const float w2 = fmaf((float)p1[0], s, c1);
          const float w3 = fmaf((float)p1[1], s, c1);
          h[2 * j] = BF16 ? pack_bf16x2(w0, w1) : pack_f16x2(w0, w1);
          h[2 * j + 1] = BF16 ? pack_bf16x2(w2, w3) : pack_f16x2(w2, w3);
        }
      } else {
        // the unclamped slice reaches 256: through fp32 lanes
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float v[4];
          slice_f32x4<R, RULE>(bytes[j], v);
          const float w0 = fmaf(v[0], s, cz);
          const float w1 = fmaf(v[1], s, cz);
          const float w2 = fmaf(v[2], s, cz);
          const float w3 = fmaf(v[3], s, cz);
          h[2 * j] = BF16 ? pack_bf16x2(w0, w1) : pack_f16x2(w0, w1);
          h[2 * j + 1] = BF16 ? pack_bf16x2(w2, w3) : pack_f16x2(w2, w3);
        }
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
  // the MFMAs of one 64-wide k step from LDS tiles as[BM][8], bs[BN/16][2][64]
  __device__ __forceinline__ void mma(const uint4* as, const uint4* bs, int lane, int wm, int wn) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
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

  // The k loop over [kb, ke), two steps per trip so the LDS buffer and the
  // staging slots are compile-time constants; one barrier per step.  Step kt
  // computes from buffers kt & 1 (As[b], Bs[b] with b relative to kb) and
  // writes step kt + 1 (X loaded a step earlier, weights two) into the other
  // pair.  Past the last step the loads repeat the last step (in bounds) and
  // the stores go to the pair no later step reads.
  //
  // compute_first: every step issues its loads, runs its MFMAs, then stages.
  // stage_first: every step stages, issues its loads, then runs its MFMAs.
  // Waves of the two orders on one SIMD overlap one wave's staging with the
  // other's MFMAs; both touch only the pair the order assigns to the step.
  __device__ __forceinline__ void compute_first(uint4* as0, uint4* as1, uint4* bs0, uint4* bs1, int kb, int ke,
                                                int lane, int wm, int wn) {
    const int kl = ke - 1;
    kfirst = kb;
    load_w<0>(kb);
    load_x(kb);
    load_w<1>(min(kb + 1, kl));
    store_x(as0);
    store_w<0>(bs0, kb);
    __syncthreads();
    for (int kt = kb; kt < ke; kt += 2) {
      load_x(min(kt + 1, kl));
      load_w<0>(min(kt + 2, kl));
      mma(as0, bs0, lane, wm, wn);
      store_x(as1);
      store_w<1>(bs1, min(kt + 1, kl));
      __syncthreads();
      if (kt + 1 < ke) {
        load_x(min(kt + 2, kl));
        load_w<1>(min(kt + 3, kl));
        mma(as1, bs1, lane, wm, wn);
        store_x(as0);
        store_w<0>(bs0, min(kt + 2, kl));
        __syncthreads();
      }
    }
  }
  __device__ __forceinline__ void stage_first(uint4* as0, uint4* as1, uint4* bs0, uint4* bs1, int kb, int ke,
                                              int lane, int wm, int wn) {
    const int kl = ke - 1;
    kfirst = kb;
    load_w<0>(kb);
    load_x(kb);
    load_w<1>(min(kb + 1, kl));
    store_x(as0);
    store_w<0>(bs0, kb);
    load_x(min(kb + 1, kl));
    __syncthreads();
    for (int kt = kb; kt < ke; kt += 2) {
      store_x(as1);
      store_w<1>(bs1, min(kt + 1, kl));
      load_x(min(kt + 2, kl));
      load_w<0>(min(kt + 2, kl));
      mma(as0, bs0, lane, wm, wn);
      __syncthreads();
      if (kt + 1 < ke) {
        store_x(as0);
        store_w<0>(bs0, min(kt + 2, kl));
        load_x(min(kt + 3, kl));
        load_w<1>(min(kt + 3, kl));
        mma(as1, bs1, lane, wm, wn);
        __syncthreads();
      }
    }
  }
};

// PP = 1 (eight-wave tiles): waves 4..7 take the stage-first order, so each
// SIMD holds one wave of either order (waves are placed on the SIMDs in turn).
// `block` is the workgroup's tile index within its call, `split` its k range.
template <int R, int RULE, int BF16, int BM, int BN, int WM, int WN, int PP>
__device__ __forceinline__ void gemm_body(const GemmArgs& a, int block, int split, uint4 (&As)[2][BM * 8],
                                          uint4 (&Bs)[2][BN / 16 * 2 * 64]) {
  using Tile = GemmTile<R, RULE, BF16, BM, BN, WM, WN>;
  static_assert(!PP || WM * WN == 8, "two orders need two waves per SIMD");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;

  // ---- tile selection: workgroups sharing a weight tile land on one XCD ----
  // (consecutive workgroups go to the eight XCDs in turn; a call's first
  // workgroup is on XCD 0)
  const int G = a.tiles_m * a.tiles_n;
  int logical = block;
  if ((G & 7) == 0) logical = (block & 7) * (G >> 3) + (block >> 3);
  const int tm = logical % a.tiles_m, tn = logical / a.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int KT = a.k / BK;
  const int kt_begin = split * a.ksteps_per_split;
  const int kt_end = min(KT, kt_begin + a.ksteps_per_split);

  // every k range is non-empty (the launcher sizes grid.y so)
  Tile t(a, tid, m0, n0);
  if (PP && (wave >> 2) == 1)
    t.stage_first(As[0], As[1], Bs[0], Bs[1], kt_begin, kt_end, lane, wm, wn);
  else
    t.compute_first(As[0], As[1], Bs[0], Bs[1], kt_begin, kt_end, lane, wm, wn);

  // ---- epilogue: lane holds D[4*(lane/16) + v][lane % 16] of each block ----
  constexpr int FM = Tile::FM, FN = Tile::FN;
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
            static_cast<float*>(a.y)[((size_t)split * a.m + m) * a.n + n] = val;
          } else {
            uint16_t* y = static_cast<uint16_t*>(a.y) + (size_t)m * a.n + n;
            *y = (uint16_t)((BF16 ? pack_bf16x2(val, 0.f) : pack_f16x2(val, 0.f)) & 0xFFFFu);
          }
        }
      }
    }
  }
}

template <int R, int RULE, int BF16, int BM, int BN, int WM, int WN, int PP>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs a) {
  // double-buffered LDS tiles: X swizzled row-major, weights fragment-major
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN / 16 * 2 * 64];
  gemm_body<R, RULE, BF16, BM, BN, WM, WN, PP>(a, (int)blockIdx.x, (int)blockIdx.y, As, Bs);
}

// Independent calls of one launch class (width, rule, dtype, tile
// configuration) in one launch, each without a k split: call i owns the
// workgroups blk0[i] .. blk0[i] + tiles_i - 1 (blk0[i] a multiple of 8, so
// the XCD grouping of a single launch is kept; the workgroups in between
// exit at once).  A workgroup's call is found by a scalar search.
struct GemmLaunch {
  GemmArgs c[kGemmMaxCalls];
  int blk0[kGemmMaxCalls];
  int ncalls;
};

template <int R, int RULE, int BF16, int BM, int BN, int WM, int WN, int PP>
__global__ __launch_bounds__(64 * WM * WN) void gemm_multi_kernel(GemmLaunch L) {
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN / 16 * 2 * 64];
  const int b = (int)blockIdx.x;
  int ci = 0;
  while (ci + 1 < L.ncalls && b >= L.blk0[ci + 1]) ++ci;
  const GemmArgs& a = L.c[ci];
  const int local = b - L.blk0[ci];
  if (local >= a.tiles_m * a.tiles_n) return;  // alignment padding: no tile
  gemm_body<R, RULE, BF16, BM, BN, WM, WN, PP>(a, local, 0, As, Bs);
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
    {256, 256},  // 0: prefill, 8 waves (4 x 2), wave tile 64 x 128, two step orders
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

template <int R, int RULE, int BF16, int BM, int BN, int WM, int WN, int PP = 0>
static hipError_t gemm_launch_cfg(const GemmArgs& ga, int splits, hipStream_t s) {
  dim3 grid((unsigned)(ga.tiles_m * ga.tiles_n), (unsigned)splits);
  hipLaunchKernelGGL((gemm_kernel<R, RULE, BF16, BM, BN, WM, WN, PP>), grid, dim3(64 * WM * WN), 0, s, ga);
  return hipGetLastError();
}

template <int R, int RULE, int BF16>
static hipError_t gemm_launch_t(const GemmArgs& ga, int cfg, int splits, hipStream_t s) {
  switch (cfg) {
    case 0: return gemm_launch_cfg<R, RULE, BF16, 256, 256, 4, 2, 1>(ga, splits, s);
    case 1: return gemm_launch_cfg<R, RULE, BF16, 128, 256, 2, 4>(ga, splits, s);
    case 2: return gemm_launch_cfg<R, RULE, BF16, 64, 256, 1, 4>(ga, splits, s);
    case 3: return gemm_launch_cfg<R, RULE, BF16, 32, 256, 1, 4>(ga, splits, s);
    case 4: return gemm_launch_cfg<R, RULE, BF16, 16, 256, 1, 4>(ga, splits, s);
    case 5: return gemm_launch_cfg<R, RULE, BF16, 128, 128, 2, 2>(ga, splits, s);
    default: return gemm_launch_cfg<R, RULE, BF16, 256, 128, 2, 2>(ga, splits, s);
  }
}

template <int R, int RULE>
static hipError_t gemm_launch_d(const GemmArgs& ga, int bf16, int cfg, int splits, hipStream_t s) {
  return bf16 ? gemm_launch_t<R, RULE, 1>(ga, cfg, splits, s) : gemm_launch_t<R, RULE, 0>(ga, cfg, splits, s);
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
  // k ranges of cdiv(KT, plan.splits) steps; only as many as hold a step
  // (at most plan.splits, so the workspace is large enough)
  ga.ksteps_per_split = cdiv(KT, plan.splits);
  const int splits = cdiv(KT, ga.ksteps_per_split);
  ga.to_workspace = splits > 1;
  ga.y = splits > 1 ? workspace : la.y;
  hipError_t e;
#define MQ_GEMM_CASE(RR)                                                                            \
  case RR:                                                                                          \
    e = la.rule == kRuleExtra ? gemm_launch_d<RR, kRuleExtra>(ga, la.bf16, plan.cfg, splits, s)   \
        : la.rule == kRuleRound ? gemm_launch_d<RR, kRuleRound>(ga, la.bf16, plan.cfg, splits, s)        \
                               : gemm_launch_d<RR, kRulePrefix>(ga, la.bf16, plan.cfg, splits, s);      \
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

bool gemm_batchable(const LinearArgs& a) { return a.m > 0 && pick_cfg(a.m, a.n) == 0; }
bool same_gemm_launch(const LinearArgs& a, const LinearArgs& b) {
  return gemm_batchable(a) && gemm_batchable(b) && a.r == b.r && a.rule == b.rule && a.bf16 == b.bf16;
}
int gemm_tiles(const LinearArgs& a) { return tiles_of(pick_cfg(a.m, a.n), a.m, a.n); }

template <int R, int RULE, int BF16>
static hipError_t gemm_multi_launch_t(const GemmLaunch& L, int blocks, hipStream_t s) {
  hipLaunchKernelGGL((gemm_multi_kernel<R, RULE, BF16, 256, 256, 4, 2, 1>), dim3((unsigned)blocks), dim3(512), 0, s,
                     L);
  return hipGetLastError();
}

hipError_t launch_gemm_multi(const LinearArgs* la, int ncalls, hipStream_t s) {
  if (ncalls < 1 || ncalls > kGemmMaxCalls) return hipErrorInvalidValue;
  // calls with the longest k first, so the workgroups with the most steps
  // start first and the launch's tail is short
  int ord[kGemmMaxCalls];
  for (int i = 0; i < ncalls; ++i) {
    if (!same_gemm_launch(la[0], la[i])) return hipErrorInvalidValue;
    int p = i;
    while (p > 0 && la[ord[p - 1]].k < la[i].k) {
      ord[p] = ord[p - 1];
      --p;
    }
    ord[p] = i;
  }
  GemmLaunch L;
  int blocks = 0;
  for (int q = 0; q < ncalls; ++q) {
    const int i = ord[q];
    GemmArgs& ga = L.c[q];
    ga.x = la[i].x;
    ga.y = la[i].y;
    ga.pl = la[i].pl;
    ga.scales = la[i].scales;
    ga.zeros = la[i].zeros;
    ga.m = la[i].m;
    ga.n = la[i].n;
    ga.k = la[i].k;
    ga.group = la[i].group;
    ga.tiles_m = cdiv(la[i].m, kCfgs[0].bm);
    ga.tiles_n = cdiv(la[i].n, kCfgs[0].bn);
    ga.ksteps_per_split = la[i].k / BK;
    ga.to_workspace = 0;
    L.blk0[q] = (blocks + 7) & ~7;
    blocks = L.blk0[q] + ga.tiles_m * ga.tiles_n;
  }
  L.ncalls = ncalls;
  const LinearArgs& a = la[0];
#define MQ_GEMM_MULTI_CASE(RR)                                                                        \
  case RR:                                                                                            \
    if (a.rule == kRuleExtra)                                                                         \
      return a.bf16 ? gemm_multi_launch_t<RR, kRuleExtra, 1>(L, blocks, s)                            \
                    : gemm_multi_launch_t<RR, kRuleExtra, 0>(L, blocks, s);                           \
    if (a.rule == kRuleRound)                                                                         \
      return a.bf16 ? gemm_multi_launch_t<RR, kRuleRound, 1>(L, blocks, s)                            \
                    : gemm_multi_launch_t<RR, kRuleRound, 0>(L, blocks, s);                           \
    return a.bf16 ? gemm_multi_launch_t<RR, kRulePrefix, 1>(L, blocks, s)                             \
                  : gemm_multi_launch_t<RR, kRulePrefix, 0>(L, blocks, s);
  switch (a.r) {
    MQ_GEMM_MULTI_CASE(2)
    MQ_GEMM_MULTI_CASE(3)
    MQ_GEMM_MULTI_CASE(4)
    MQ_GEMM_MULTI_CASE(6)
    MQ_GEMM_MULTI_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MQ_GEMM_MULTI_CASE
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
