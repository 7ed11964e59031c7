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

// fp16 value of a 2-bit field that sits at mantissa bit P of each half of a
// word: with exponent field 25 - P the half equals 2^(10 - P) + field.
template <int P>
__host__ __device__ constexpr uint32_t field2_magic() {
  return ((25u - P) << 10) | ((25u - P) << 26);
}
// gfx9 VOP3 encodings take no literal and read at most one SGPR, so the
// exponent pattern is kept in a VGPR and the mask in an SGPR: one v_and_or_b32.
template <uint32_t C>
__device__ __forceinline__ uint32_t vgpr_const() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(C));
  return r;
}
template <int P>
__device__ __forceinline__ uint32_t field2_to_f16x2(uint32_t w, uint32_t magic_v) {
  constexpr uint32_t mask = (3u << P) | (3u << (P + 16));
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic_v));
  return r;
}

// value of quad lane t in every lane of the quad (DPP quad_perm [t,t,t,t]);
// t is a constant after unrolling
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int t) {
  switch (t) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, false);
  }
}

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// SZ4 (group == 128, even groups per row): the scales and zeros of four rows
// come in with one dword load per lane (quad lane t fetches the two groups of
// its quad for row t) and DPP quad broadcasts hand every lane its own value;
// otherwise each row costs two 16-bit loads per lane.
// XW = 1: the workgroup's lanes cover one row's slices (several waves when
// k > 4096) and walk ROWS rows.  XW = 4 (k <= 4096, one wave per row): four
// waves with ROWS rows each share a workgroup, and the workgroup stages the
// activations once through LDS instead of every wave reading all of X.
template <int R, int ROUND, int MT, int BF16, int ROWS, int SZ4, int XW>
__device__ __forceinline__ void gemv_body(const GemvArgs a, const unsigned blk) {
  constexpr int NP = planes_needed(R, ROUND);
  // width 2, true prefix, fp16: fields go straight from the plane-0 word to
  // fp16 with one and-or per pair (no byte assembly)
  constexpr bool FAST2 = (R == 2 && !ROUND && !BF16);
  // rows per load batch: batch b + 1 is in flight while batch b is computed.
  // Narrow widths carry few bytes per row, so all rows of the block are
  // requested at once to keep enough bytes in flight; wide ones use small
  // batches, which shortens the compute tail after the last bytes arrive.
  constexpr int RB = NP <= 3 ? ROWS : 2;
  constexpr int NB = ROWS / RB;
  static_assert(NB * RB == ROWS, "row batches");
  constexpr int V = ROWS * MT;

  const int tid = XW > 1 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;  // lane of the row's slices
  const int lane = tid & 63;
  const int S = a.k >> 6;
  const bool valid = tid < S;            // one lane per 64-code slice; a row spans the workgroup
  const int slice = valid ? tid : 0;
  const size_t upr = (size_t)(a.k >> 5);  // units per row
  const int gpr = a.k / a.group;
  const int gidx = (slice * 64) / a.group;
  const size_t row0 = ((size_t)blk * XW + (XW > 1 ? (threadIdx.x >> 6) : 0)) * (size_t)ROWS;

  // ---- 1. issue the activation loads of this slice ----
  // (unconditional loads from clamped addresses; invalid lanes/tokens are
  // zeroed at first use so no load waits behind a branch)
  uint4 xraw[MT][8];
  constexpr int XC = XW > 1 ? (MT * 512) / (64 * XW) : 1;  // 16-byte X chunks per thread when staged
  uint4 xst[XC];
  if constexpr (XW == 1) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const int mc = mm < a.m ? mm : 0;
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)mc * a.k +
                                                        (size_t)slice * 64);
#pragma unroll
      for (int i = 0; i < 8; ++i) xraw[mm][i] = src[i];
    }
  } else {
    // chunk c = (token mm, slice sl, piece i) with consecutive threads on
    // consecutive 16-byte pieces of X; clamped reads for idle slices/tokens
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int c = (int)threadIdx.x + 64 * XW * j;
      const int mm = c >> 9, sl = (c >> 3) & 63, i = c & 7;
      const int mc = mm < a.m ? mm : 0;
      const int sc = sl < S ? sl : 0;
      xst[j] = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)mc * a.k +
                                              (size_t)sc * 64)[i];
    }
  }

  // ---- 2. issue the plane loads of the first row batch ----
  uint32_t rec[2][RB][2][kUnitWords];
  uint16_t sraw[2][SZ4 ? 1 : RB], zraw[2][SZ4 ? 1 : RB];
  uint32_t sq[SZ4 ? ROWS / 4 : 1], zq[SZ4 ? ROWS / 4 : 1];  // all rows' quads, loaded once
  static_assert(!SZ4 || ROWS % 4 == 0, "quad scale loads cover rows in fours");
  const int qgrp = ((tid >> 6) << 5) + 2 * (lane >> 2);       // first of the quad's two groups
  const int qgrp_c = qgrp <= gpr - 2 ? qgrp : gpr - 2;          // clamp for idle lanes
  const int sz_shift = 16 * ((lane >> 1) & 1);                  // this lane's half of the dword
  auto load_batch = [&](int buf, int b) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      size_t row = row0 + (size_t)(b * RB + i);
      if (row >= (size_t)a.n) row = (size_t)a.n - 1;  // clamp loads; stores are guarded
      const size_t unit = row * upr + (size_t)slice * 2;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (kPlaneBits[p] == 2) {
          const stream_u32x4 v = stream_load16(a.pl.p[p] + unit * 2);
          rec[buf][i][0][kUnitOff[p]] = v.x;
          rec[buf][i][0][kUnitOff[p] + 1] = v.y;
          rec[buf][i][1][kUnitOff[p]] = v.z;
          rec[buf][i][1][kUnitOff[p] + 1] = v.w;
        } else {
          const stream_u32x2 v = stream_load8(a.pl.p[p] + unit);
          rec[buf][i][0][kUnitOff[p]] = v.x;
          rec[buf][i][1][kUnitOff[p]] = v.y;
        }
      }
      if constexpr (!SZ4) {
        sraw[buf][i] = a.scales[row * gpr + gidx];
        zraw[buf][i] = a.zeros[row * gpr + gidx];
      }
    }
  };
  load_batch(0, 0);
  if constexpr (SZ4) {
#pragma unroll
    for (int q = 0; q < ROWS / 4; ++q) {
      size_t row = row0 + (size_t)(4 * q + (lane & 3));
      if (row >= (size_t)a.n) row = (size_t)a.n - 1;
      sq[q] = *reinterpret_cast<const uint32_t*>(a.scales + row * gpr + qgrp_c);
      zq[q] = *reinterpret_cast<const uint32_t*>(a.zeros + row * gpr + qgrp_c);
    }
  }
  if constexpr (XW > 1) {
    // [token][piece][slice]: a wave's reads of one piece are 64 consecutive
    // 16-byte entries
    __shared__ uint4 xlds[MT * 8 * 64];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int c = (int)threadIdx.x + 64 * XW * j;
      xlds[((c >> 9) * 8 + (c & 7)) * 64 + ((c >> 3) & 63)] = xst[j];
    }
    __syncthreads();
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
      for (int i = 0; i < 8; ++i) xraw[mm][i] = xlds[(mm * 8 + i) * 64 + lane];
  }

  // ---- 3. activations: register layout, slice sums ----
  constexpr uint32_t kOnes = 0x3C003C00u;  // (1.0, 1.0) in fp16
  uint32_t xr[BF16 ? 1 : MT][32];           // fp16 pairs, natural k order or FAST2 pair order
  float xf[BF16 ? MT : 1][BF16 ? 64 : 1];
  float xs[MT];                             // sum of the slice's X
  float xc[MT];                             // FAST2: sum of X times the fp16 field offsets
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    const uint32_t keep = (valid && mm < a.m) ? 0xFFFFFFFFu : 0u;
    uint32_t w[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w[4 * i] = xraw[mm][i].x & keep;
      w[4 * i + 1] = xraw[mm][i].y & keep;
      w[4 * i + 2] = xraw[mm][i].z & keep;
      w[4 * i + 3] = xraw[mm][i].w & keep;
    }
    if constexpr (BF16) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        xf[mm][2 * i] = __builtin_bit_cast(float, w[i] << 16);
        xf[mm][2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
        sum += xf[mm][2 * i] + xf[mm][2 * i + 1];
      }
      xs[mm] = sum;
    } else {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) sum = dot2h(w[i], kOnes, sum);
      xs[mm] = sum;
      if constexpr (FAST2) {
        // pair idx of plane-0 word (u, d): (b, q) = (idx / 4, idx % 4) holds codes
        // t0 = 32u + 16d + 4q + b (low half) and t0 + 2 (high half)
        float c = 0.f;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
          for (int idx = 0; idx < 8; ++idx) {
            const int b = idx / 4, q = idx % 4;
            const int t0 = 16 * wd + 4 * q + b;
            const uint32_t sel = (b == 0) ? 0x05040100u : 0x07060302u;
            const uint32_t pr = __builtin_amdgcn_perm(w[t0 / 2 + 1], w[t0 / 2], sel);
            xr[mm][8 * wd + idx] = pr;
            const int P = 8 * b + 2 * q;
            const int Pp = (idx < 5) ? P : P - 10;     // field bit after the optional shift by 10
            const uint32_t off = (uint32_t)(25 - Pp) << 10;  // fp16 2^(10 - Pp)
            c = dot2h(pr, off | (off << 16), c);
          }
        }
        xc[mm] = c;
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) xr[mm][i] = w[i];
      }
    }
  }

  float acc[V];
  constexpr float kDelta = ROUND ? 0.0f : prefix_delta(R);
  uint32_t mg0 = 0, mg2 = 0, mg4 = 0, mg6 = 0, mg8 = 0;
  if constexpr (FAST2) {
    mg0 = vgpr_const<field2_magic<0>()>();
    mg2 = vgpr_const<field2_magic<2>()>();
    mg4 = vgpr_const<field2_magic<4>()>();
    mg6 = vgpr_const<field2_magic<6>()>();
    mg8 = vgpr_const<field2_magic<8>()>();
  }

  // ---- 4. rows: batch b computes while batch b+1 is in flight ----
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int cur = b & 1;
    if (b + 1 < NB) load_batch(cur ^ 1, b + 1);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float dot[MT];
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) dot[mm] = 0.f;
      if constexpr (FAST2) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const uint32_t w = rec[cur][i][wd / 2][kUnitOff[0] + (wd & 1)];
          const uint32_t ws = w >> 10;
          uint32_t h[8];
          h[0] = field2_to_f16x2<0>(w, mg0);
          h[1] = field2_to_f16x2<2>(w, mg2);
          h[2] = field2_to_f16x2<4>(w, mg4);
          h[3] = field2_to_f16x2<6>(w, mg6);
          h[4] = field2_to_f16x2<8>(w, mg8);
          h[5] = field2_to_f16x2<0>(ws, mg0);
          h[6] = field2_to_f16x2<2>(ws, mg2);
          h[7] = field2_to_f16x2<4>(ws, mg4);
#pragma unroll
          for (int idx = 0; idx < 8; ++idx)
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) dot[mm] = dot2h(h[idx], xr[mm][8 * wd + idx], dot[mm]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t bytes[8];
          bytes[0] = assemble_word<NP, 0>(rec[cur][i][u]);
          bytes[1] = assemble_word<NP, 1>(rec[cur][i][u]);
          bytes[2] = assemble_word<NP, 2>(rec[cur][i][u]);
          bytes[3] = assemble_word<NP, 3>(rec[cur][i][u]);
          bytes[4] = assemble_word<NP, 4>(rec[cur][i][u]);
          bytes[5] = assemble_word<NP, 5>(rec[cur][i][u]);
          bytes[6] = assemble_word<NP, 6>(rec[cur][i][u]);
          bytes[7] = assemble_word<NP, 7>(rec[cur][i][u]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (BF16) {
              const uint32_t v = slice_bytes<R, ROUND>(bytes[j]);
#pragma unroll
              for (int bb = 0; bb < 4; ++bb) {
                const float fv = (float)((v >> (8 * bb)) & 0xFFu);
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) dot[mm] = fmaf(fv, xf[mm][32 * u + 4 * j + bb], dot[mm]);
              }
            } else {
              uint32_t lo, hi;
              if constexpr (ROUND && R < 8) {
                slice_pairs<R, ROUND>(bytes[j], lo, hi);
                lo |= 0x64006400u;
                hi |= 0x64006400u;
              } else {
                // byte under an 0x64 exponent byte: the exact fp16 1024 + v
                lo = __builtin_amdgcn_perm(0x64646464u, bytes[j], 0x04010400u);
                hi = __builtin_amdgcn_perm(0x64646464u, bytes[j], 0x04030402u);
              }
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) {
                dot[mm] = dot2h(lo, xr[mm][16 * u + 2 * j], dot[mm]);
                dot[mm] = dot2h(hi, xr[mm][16 * u + 2 * j + 1], dot[mm]);
              }
            }
          }
        }
      }
      float s, z;
      if constexpr (SZ4) {
        const int ri = b * RB + i;  // row within the workgroup's block
        const uint32_t sd = quad_bcast(sq[ri / 4], ri % 4);
        const uint32_t zd = quad_bcast(zq[ri / 4], ri % 4);
        s = h2f((uint16_t)(sd >> sz_shift));
        z = h2f((uint16_t)(zd >> sz_shift));
      } else {
        s = h2f(sraw[cur][i]);
        z = h2f(zraw[cur][i]);
      }
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        float t;
        if constexpr (FAST2) {
          // sum_k X (2^(10-P) + f) - xc = sum_k X f;  v = 64 f
          t = fmaf(64.0f, dot[mm] - xc[mm], (kDelta - z) * xs[mm]);
        } else if constexpr (BF16) {
          t = fmaf(kDelta - z, xs[mm], dot[mm]);
        } else {
          t = fmaf(-(1024.0f + z - kDelta), xs[mm], dot[mm]);
        }
        acc[(b * RB + i) * MT + mm] = valid ? s * t : 0.f;
      }
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
  if (XW > 1 || nwaves == 1) {
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

template <int R, int ROUND, int MT, int BF16, int ROWS, int SZ4, int XW>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  gemv_body<R, ROUND, MT, BF16, ROWS, SZ4, XW>(a, blockIdx.x);
}

// Several independent calls of one shape class (same m, k, width, rule,
// group, dtype) in one launch: workgroup b serves the call whose block range
// holds b.  One launch then streams the bytes of all of them, so the launch
// ramp and drain are paid once.
struct GemvBatch {
  GemvArgs call[kGemvMaxBatch];
  int first_block[kGemvMaxBatch];  // first workgroup of each call
  int ncalls;
};

template <int R, int ROUND, int MT, int BF16, int ROWS, int SZ4, int XW>
__global__ __launch_bounds__(256) void gemv_batch_kernel(GemvBatch b) {
  int c = 0;
#pragma unroll
  for (int i = 1; i < kGemvMaxBatch; ++i)
    if (i < b.ncalls && (int)blockIdx.x >= b.first_block[i]) c = i;
  gemv_body<R, ROUND, MT, BF16, ROWS, SZ4, XW>(b.call[c], blockIdx.x - (unsigned)b.first_block[c]);
}

template <int R, int ROUND, int MT, int BF16, int SZ4, int XW, int ROWS>
static void gemv_launch_k(const GemvBatch& b, int ncalls, unsigned blocks, int threads, size_t lds, hipStream_t s) {
  if (ncalls == 1)
    hipLaunchKernelGGL((gemv_kernel<R, ROUND, MT, BF16, ROWS, SZ4, XW>), dim3(blocks), dim3(threads), lds, s, b.call[0]);
  else
    hipLaunchKernelGGL((gemv_batch_kernel<R, ROUND, MT, BF16, ROWS, SZ4, XW>), dim3(blocks), dim3(threads), lds, s, b);
}

template <int R, int ROUND, int MT, int BF16>
static hipError_t gemv_launch_t(const LinearArgs* la, int ncalls, hipStream_t s) {
  constexpr int ROWS = (MT >= 4) ? 4 : 8;
  // every call of a batch shares k and group, hence the workgroup shape
  const int S = la[0].k / 64;
  const int xw = S <= 64 ? 4 : 1;  // four row groups share the staged X when a row fits one wave
  GemvBatch b;
  unsigned blocks = 0;
  for (int i = 0; i < ncalls; ++i) {
    GemvArgs& a = b.call[i];
    a.x = la[i].x;
    a.y = la[i].y;
    a.pl = la[i].pl;
    a.scales = la[i].scales;
    a.zeros = la[i].zeros;
    a.m = la[i].m;
    a.n = la[i].n;
    a.k = la[i].k;
    a.group = la[i].group;
    b.first_block[i] = (int)blocks;
    blocks += (unsigned)((la[i].n + xw * ROWS - 1) / (xw * ROWS));
  }
  for (int i = ncalls; i < kGemvMaxBatch; ++i) {
    b.call[i] = b.call[0];
    b.first_block[i] = (int)blocks;
  }
  b.ncalls = ncalls;
  const int gpr = la[0].k / la[0].group;
  const bool sz4 = la[0].group == 128 && gpr % 2 == 0;
  if (xw == 4) {
    if (sz4) gemv_launch_k<R, ROUND, MT, BF16, 1, 4, ROWS>(b, ncalls, blocks, 256, 0, s);
    else gemv_launch_k<R, ROUND, MT, BF16, 0, 4, ROWS>(b, ncalls, blocks, 256, 0, s);
  } else {
    const int threads = ((S + 63) / 64) * 64;  // one lane per 64-code slice, whole waves
    const size_t lds = (size_t)(threads / 64) * ROWS * MT * sizeof(float);
    if (sz4) gemv_launch_k<R, ROUND, MT, BF16, 1, 1, ROWS>(b, ncalls, blocks, threads, lds, s);
    else gemv_launch_k<R, ROUND, MT, BF16, 0, 1, ROWS>(b, ncalls, blocks, threads, lds, s);
  }
  return hipGetLastError();
}

template <int R, int ROUND, int BF16>
static hipError_t gemv_launch_m(const LinearArgs* a, int n, hipStream_t s) {
  if constexpr (BF16) {
    return gemv_launch_t<R, ROUND, 1, 1>(a, n, s);  // bf16: m == 1 only
  } else {
    switch (a[0].m) {
      case 1: return gemv_launch_t<R, ROUND, 1, 0>(a, n, s);
      case 2: return gemv_launch_t<R, ROUND, 2, 0>(a, n, s);
      default: return gemv_launch_t<R, ROUND, 4, 0>(a, n, s);
    }
  }
}

template <int R, int ROUND>
static hipError_t gemv_launch_d(const LinearArgs* a, int n, hipStream_t s) {
  return a[0].bf16 ? gemv_launch_m<R, ROUND, 1>(a, n, s) : gemv_launch_m<R, ROUND, 0>(a, n, s);
}

hipError_t launch_gemv_batch(const LinearArgs* a, int ncalls, hipStream_t s) {
  if (ncalls < 1 || ncalls > kGemvMaxBatch) return hipErrorInvalidValue;
#define MQ_GEMV_CASE(RR) \
  case RR: return a[0].round_rule ? gemv_launch_d<RR, 1>(a, ncalls, s) : gemv_launch_d<RR, 0>(a, ncalls, s);
  switch (a[0].r) {
    MQ_GEMV_CASE(2)
    MQ_GEMV_CASE(3)
    MQ_GEMV_CASE(4)
    MQ_GEMV_CASE(6)
    MQ_GEMV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MQ_GEMV_CASE
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t s) { return launch_gemv_batch(&a, 1, s); }

}  // namespace mq
