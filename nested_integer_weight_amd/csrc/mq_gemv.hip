// mq_gemv.hip -- decode path (m <= 4): stream the bit planes, rebuild and
// slice the codes in registers, contract with register-resident activations,
// reduce across lanes with a transposing butterfly.
//
// The pages' small-batch design streams weights straight from memory because
// decoding at batch <= 4 is memory-bandwidth bound (MatGPTQ "Efficient and
// Accurate Inference over Nested Quantized Models", section 4, third
// component).  On gfx950 this becomes:
//  * every lane owns a fixed 64-code k-slice (two packing units) and walks a
//    block of output rows, so its slice of X is loaded once into VGPRs and
//    reused for every row; per row a lane issues one 16-byte load per 2-bit
//    plane and one 8-byte load per 1-bit plane, and the 64 lanes of a wave
//    cover consecutive slices, so each load instruction reads contiguous bytes;
//  * fp16 activations: a code byte v becomes the exact fp16 1024+v with one
//    v_perm_b32 (the byte under an 0x64 exponent byte) and v_dot2_f32_f16
//    accumulates X.(1024+v) in fp32; the 1024 and the zero point are removed
//    per (row, slice) with the slice's sum of X:
//      y += s * (sum_k X_k (1024 + v_k) - (1024 + z - delta) * sum_k X_k)
//    which equals s * sum_k X_k (v_k + delta - z) (scale and zero point are
//    shared by the whole 64-code slice because group % 64 == 0);
//  * bf16 activations: X is held as fp32 and codes are converted with
//    v_cvt_f32_ubyte, accumulating with fp32 FMA;
//  * a lane's per-row partials are summed over the lanes of the row with a
//    transposing butterfly (each exchange halves the values a lane holds),
//    then across waves through LDS when a row spans several waves.
#include "mq_common.h"
#include "mq_kernels.h"

namespace mq {

struct GemvArgs {
  const void* x;
  void* y;
  PlanePtrs pl;
  const uint16_t* scales;
  const uint16_t* zeros;
  int m, n, k, group;
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Transposing butterfly stage with xor-offset O on VC values per lane.
template <int VC, int O>
__device__ __forceinline__ void butterfly(float* acc, int lane) {
  if constexpr (O >= 1) {
    if constexpr (VC > 1) {
      constexpr int H = VC / 2;
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float keep = up ? acc[i + H] : acc[i];
        const float send = up ? acc[i] : acc[i + H];
        acc[i] = keep + __shfl_xor(send, O, 64);
      }
      butterfly<H, O / 2>(acc, lane);
    } else {
      acc[0] += __shfl_xor(acc[0], O, 64);
      butterfly<1, O / 2>(acc, lane);
    }
  }
}

template <int R, int ROUND, int MT, int BF16, int ROWS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  constexpr int NP = planes_needed(R, ROUND);
  constexpr int RB = (NP <= 2) ? ROWS : 4;  // rows whose loads are issued together
  constexpr int V = ROWS * MT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int slice = tid;  // a row spans the whole workgroup
  const int S = a.k >> 6;
  const bool valid = slice < S;
  const int slice_c = valid ? slice : 0;
  const size_t upr = (size_t)(a.k >> 5);               // units per row
  const int gpr = a.k / a.group;
  const int gidx = (slice_c * 64) / a.group;
  const size_t row0 = (size_t)blockIdx.x * (size_t)ROWS;

  // ---- activations of this slice, once per workgroup ----
  uint32_t xr[BF16 ? 1 : MT][32];
  float xf[BF16 ? MT : 1][BF16 ? 64 : 1];
  float xs[MT];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    const bool mok = valid && mm < a.m;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) +
                                                      (size_t)(mok ? mm : 0) * a.k + (size_t)slice_c * 64);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = mok ? src[i] : make_uint4(0, 0, 0, 0);
      uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo, hi;
        if constexpr (BF16) {
          lo = __builtin_bit_cast(float, w4[j] << 16);
          hi = __builtin_bit_cast(float, w4[j] & 0xFFFF0000u);
          xf[mm][8 * i + 2 * j] = lo;
          xf[mm][8 * i + 2 * j + 1] = hi;
        } else {
          xr[mm][4 * i + j] = w4[j];
          f16x2_t h = __builtin_bit_cast(f16x2_t, w4[j]);
          lo = (float)h.x;
          hi = (float)h.y;
        }
        sum += lo + hi;
      }
    }
    xs[mm] = sum;
  }

  float acc[V];
  constexpr float kDelta = ROUND ? 0.0f : prefix_delta(R);

#pragma unroll
  for (int i0 = 0; i0 < ROWS; i0 += RB) {
    uint32_t rec[RB][2][kUnitWords];
    uint16_t sraw[RB], zraw[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      size_t row = row0 + (size_t)(i0 + i);
      if (row >= (size_t)a.n) row = (size_t)a.n - 1;  // clamp loads; stores are guarded
      const size_t unit = row * upr + (size_t)slice_c * 2;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (kPlaneBits[p] == 2) {
          uint4 v = *reinterpret_cast<const uint4*>(a.pl.p[p] + unit * 2);
          rec[i][0][kUnitOff[p]] = v.x;
          rec[i][0][kUnitOff[p] + 1] = v.y;
          rec[i][1][kUnitOff[p]] = v.z;
          rec[i][1][kUnitOff[p] + 1] = v.w;
        } else {
          uint2 v = *reinterpret_cast<const uint2*>(a.pl.p[p] + unit);
          rec[i][0][kUnitOff[p]] = v.x;
          rec[i][1][kUnitOff[p]] = v.y;
        }
      }
      sraw[i] = a.scales[row * gpr + gidx];
      zraw[i] = a.zeros[row * gpr + gidx];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float dot[MT];
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) dot[mm] = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t bytes[8];
        bytes[0] = assemble_word<NP, 0>(rec[i][u]);
        bytes[1] = assemble_word<NP, 1>(rec[i][u]);
        bytes[2] = assemble_word<NP, 2>(rec[i][u]);
        bytes[3] = assemble_word<NP, 3>(rec[i][u]);
        bytes[4] = assemble_word<NP, 4>(rec[i][u]);
        bytes[5] = assemble_word<NP, 5>(rec[i][u]);
        bytes[6] = assemble_word<NP, 6>(rec[i][u]);
        bytes[7] = assemble_word<NP, 7>(rec[i][u]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (BF16) {
            uint32_t v = slice_bytes<R, ROUND>(bytes[j]);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              float fv = (float)((v >> (8 * b)) & 0xFFu);
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) dot[mm] = fmaf(fv, xf[mm][32 * u + 4 * j + b], dot[mm]);
            }
          } else {
            uint32_t lo, hi;
            if constexpr (ROUND && R < 8) {
              slice_pairs<R, ROUND>(bytes[j], lo, hi);
              lo |= 0x64006400u;
              hi |= 0x64006400u;
            } else {
              lo = __builtin_amdgcn_perm(0x64646464u, bytes[j], 0x04010400u);
              hi = __builtin_amdgcn_perm(0x64646464u, bytes[j], 0x04030402u);
            }
            const f16x2_t hl = __builtin_bit_cast(f16x2_t, lo);
            const f16x2_t hh = __builtin_bit_cast(f16x2_t, hi);
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) {
              dot[mm] = __builtin_amdgcn_fdot2(hl, __builtin_bit_cast(f16x2_t, xr[mm][16 * u + 2 * j]), dot[mm], false);
              dot[mm] = __builtin_amdgcn_fdot2(hh, __builtin_bit_cast(f16x2_t, xr[mm][16 * u + 2 * j + 1]), dot[mm], false);
            }
          }
        }
      }
      const float s = h2f(sraw[i]);
      const float c = (BF16 ? 0.0f : 1024.0f) + h2f(zraw[i]) - kDelta;
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) acc[(i0 + i) * MT + mm] = valid ? s * fmaf(-c, xs[mm], dot[mm]) : 0.f;
    }
  }

  // ---- transposing butterfly over the 64 lanes of the wave ----
  // Stage o (32, 16, ...) halves the values a lane holds: the lower lane of
  // each pair keeps the first half and the upper lane the second half, each
  // adding its partner's copy.  After log2(V) stages lane l holds the sum of
  // value (l >> (6 - log2 V)) over the lanes that share its upper bits; the
  // remaining stages are plain xor-reductions.
  constexpr int T = (V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
  static_assert((1 << T) == V, "values per lane must be a power of two");
  butterfly<V, 32>(acc, lane);
  const int idx = lane >> (6 - T);
  const bool holder = (lane & ((1 << (6 - T)) - 1)) == 0;

  auto store = [&](int id, float val) {
    const int i = id / MT, mm = id % MT;
    const size_t row = row0 + (size_t)i;
    if (row < (size_t)a.n && mm < a.m) {
      uint16_t* y = static_cast<uint16_t*>(a.y) + (size_t)mm * a.n + row;
      if constexpr (BF16) *y = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
      else *y = (uint16_t)(pack_f16x2(val, 0.f) & 0xFFFFu);
    }
  };

  const int nwaves = blockDim.x >> 6;
  if (nwaves == 1) {
    if (holder) store(idx, acc[0]);
  } else {
    // a row spans several waves: combine the per-wave sums through LDS
    extern __shared__ float red[];  // [waves][V]
    const int wave = tid >> 6;
    if (holder) red[wave * V + idx] = acc[0];
    __syncthreads();
    if (tid < V) {
      float t = 0.f;
      for (int w = 0; w < nwaves; ++w) t += red[w * V + tid];
      store(tid, t);
    }
  }
}

template <int R, int ROUND, int MT, int BF16>
static hipError_t gemv_launch_t(const LinearArgs& la, hipStream_t s) {
  constexpr int ROWS = (MT >= 4) ? 4 : 8;
  GemvArgs a;
  a.x = la.x;
  a.y = la.y;
  a.pl = la.pl;
  a.scales = la.scales;
  a.zeros = la.zeros;
  a.m = la.m;
  a.n = la.n;
  a.k = la.k;
  a.group = la.group;
  const int S = la.k / 64;
  const int threads = ((S + 63) / 64) * 64;  // one lane per 64-code slice, whole waves
  const unsigned blocks = (unsigned)((la.n + ROWS - 1) / ROWS);
  const size_t lds = (threads > 64) ? (size_t)(threads / 64) * ROWS * MT * sizeof(float) : 0;
  hipLaunchKernelGGL((gemv_kernel<R, ROUND, MT, BF16, ROWS>), dim3(blocks), dim3(threads), lds, s, a);
  return hipGetLastError();
}

template <int R, int ROUND, int BF16>
static hipError_t gemv_launch_m(const LinearArgs& a, hipStream_t s) {
  if constexpr (BF16) {
    return gemv_launch_t<R, ROUND, 1, 1>(a, s);  // bf16: m == 1 only
  } else {
    switch (a.m) {
      case 1: return gemv_launch_t<R, ROUND, 1, 0>(a, s);
      case 2: return gemv_launch_t<R, ROUND, 2, 0>(a, s);
      default: return gemv_launch_t<R, ROUND, 4, 0>(a, s);
    }
  }
}

template <int R, int ROUND>
static hipError_t gemv_launch_d(const LinearArgs& a, hipStream_t s) {
  return a.bf16 ? gemv_launch_m<R, ROUND, 1>(a, s) : gemv_launch_m<R, ROUND, 0>(a, s);
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t s) {
#define MQ_GEMV_CASE(RR) \
  case RR: return a.round_rule ? gemv_launch_d<RR, 1>(a, s) : gemv_launch_d<RR, 0>(a, s);
  switch (a.r) {
    MQ_GEMV_CASE(2)
    MQ_GEMV_CASE(3)
    MQ_GEMV_CASE(4)
    MQ_GEMV_CASE(6)
    MQ_GEMV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MQ_GEMV_CASE
}

}  // namespace mq
