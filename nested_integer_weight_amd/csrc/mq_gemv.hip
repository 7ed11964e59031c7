// mq_gemv.hip -- decode path (m <= 4): stream the bit planes of one or more
// independent layer calls in one launch, rebuild and slice the codes in
// registers, contract with register-resident activations, reduce across lanes
// with a transposing butterfly.
//
// The pages' small-batch design streams the weights straight from memory,
// because decoding at batch <= 4 is bound by memory bandwidth (MatGPTQ
// "Efficient and Accurate Inference over Nested Quantized Models", section
// 4, third component).  On gfx950:
//  * Work items.  Every call's output rows are cut into items of 4 / W row
//    groups x sets x ROWS rows; a row group is W waves (W = 1, 2 or 4 by k),
//    each lane owning a fixed 64-code k-slice of the group's rows, so its
//    slice of X sits in VGPRs for every row it walks.  A row group walks its
//    rows in sets of ROWS (8, or 4 at four tokens and in launches of few
//    items, which then have twice the waves), one reduction per set; launches
//    with many items take two sets per item, which halves the share of the
//    activation set-up per row and still leaves several workgroups per CU.
//    One 256-thread
//    workgroup per item; a launch covers the items of up to kGemvMaxCalls
//    calls of one rule, m and dtype (any width, n, k and group), found by a
//    scalar search of the kernel arguments; the call's width selects the
//    code path of the workgroup.  Independent calls (gate, up and down of an FFN, a whole
//    Mix'n'Match pass at its per-layer widths) then share one launch ramp
//    and drain.
//  * Loads.  Buffer loads: the row group's first row is the base of a
//    descriptor in scalar registers, the row a scalar offset and the lane's
//    slice a vector offset, so no vector instruction computes an address.
//    Per row a lane reads one 16-byte piece per 2-bit plane and one 8-byte
//    piece per 1-bit plane (consecutive lanes on consecutive pieces: every
//    load instruction reads contiguous bytes), plus the 16-bit scale and zero
//    point of its slice's group.  Rows go in small batches, the next batches
//    in flight while one is computed.
//  * fp16 activations: a code byte v becomes the exact fp16 1024 + v with one
//    v_perm_b32 and v_dot2_f32_f16 accumulates X.(1024 + v) in fp32; the 1024
//    and the zero point are removed per (row, slice) with the slice's sum of X:
//      y += s * (sum_k X_k (1024 + v_k) - (1024 + z - delta) * sum_k X_k)
//    (scale and zero point are shared by the 64-code slice: group % 64 == 0).
//    At width 2 under the true prefix, each 2-bit field goes straight to an
//    exact fp16 2^(10-P) + f with one v_and_or_b32 and a per-position
//    exponent, and the offsets are removed with a precomputed sum.
//  * bf16 activations: X is held as fp32 and codes are converted with
//    v_cvt_f32_ubyte, accumulating with fp32 FMA.
//  * A lane's per-row partials are summed over the wave with a transposing
//    butterfly, then across the W waves of a row group through LDS.
// Each output row is computed by one workgroup in a fixed order, so results
// do not depend on which calls share a launch.
#include "mq_common.h"
#include "mq_kernels.h"

namespace mq {

namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// One call of a launch.  The geometry fields are derived on the host, so the
// kernel does no integer division.
struct GemvCall {
  const uint16_t* x;
  uint16_t* y;
  const uint32_t* p[kPlanes];
  const uint16_t* s;
  const uint16_t* z;
  int n, k;
  int r;      // width (the kernel branches on it per workgroup)
  int item0;  // first item of the call
  int wlog;   // log2 of the waves sharing a row (W = 1, 2 or 4)
  int sets;   // row sets of ROWS rows that a row group walks (1, 2 or 4)
  int rpi;    // rows per item: (4 / W) row groups x sets x ROWS
  int gpr;    // quantization groups per row, k / group
  int gmul;   // slice -> group index: (slice * gmul) >> 16 == slice / (group / 64)
};

struct GemvLaunch {
  GemvCall c[kGemvMaxCalls];
  int ncalls, m;
};

// waves that share one row (a lane per 64-code slice): 1, 2 or 4
__host__ __device__ inline int waves_per_row(int k) {
  const int w = ((k >> 6) + 63) >> 6;
  return w >= 3 ? 4 : w;
}

// Rows per wave: eight, or four for four tokens (the transposing butterfly
// reduces ROWS x tokens <= 32 values per lane) and in launches of few items.
__host__ __device__ constexpr int gemv_rows(int mt) { return mt >= 4 ? 4 : 8; }

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

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// a value known to be the same in every lane, moved to a scalar register
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Raw buffer descriptor (gfx9 data format word, no stride, 4 GiB - 1 bytes of
// records) at `base`.  The base is wave-uniform; it is passed through
// readfirstlane so that the descriptor is built in scalar registers (one the
// compiler believed divergent would be wrapped in a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), (short)0, -1, 0x00020000);
}
// cache-policy operand of the buffer loads: nontemporal (streamed once)
constexpr int kNontemporal = 2;

template <int R, int RULE, int MT, int BF16, int ROWS>
struct GemvWave {
  static constexpr int NP = planes_needed(R, RULE);
  static constexpr bool FAST2 = (R == 2 && !RULE && !BF16);
  static constexpr int V = ROWS * MT;
  // Rows are loaded and computed in batches of RB rows (two for widths of up
  // to three planes, one for wider ones), PD batches in flight.  Measured on
  // the 8B FFN shapes against deeper and shallower batches; larger batches
  // let the compiler convert every staged row before the first dot product
  // and lower the occupancy.
  static constexpr int RB = NP <= 3 ? 2 : 1;
  static constexpr int NB = ROWS / RB;
  static constexpr int PD = NP == 4 ? 3 : 2;
  static constexpr float kDelta = RULE ? 0.0f : prefix_delta(R);
  static_assert((V & (V - 1)) == 0 && V <= 32, "values per lane must be a power of two");
  static_assert(NB * RB == ROWS, "row batches");

  const GemvCall& C;
  int wave, lane, wsl, row0, slice, valid;
  __amdgpu_buffer_rsrc_t rp[NP], rs, rz;
  int vplane2, vplane1, vgroup;  // per-lane byte offsets
  uint32_t rec[PD][RB][2][kUnitWords];
  f16x2_t sz[PD][RB];
  uint32_t xr[BF16 ? 1 : MT][32];
  float xf[BF16 ? MT : 1][BF16 ? 64 : 1];
  float xs[MT], xc[MT];
  float acc[V];

  // Row group (wave >> wlog) of the item takes ROWS rows; its W waves split
  // the row's 64-code slices.
  __device__ __forceinline__ GemvWave(const GemvCall& call, int it, int w, int l) : C(call), wave(w), lane(l) {
    wsl = wave & ((1 << C.wlog) - 1);
    row0 = (it - C.item0) * C.rpi + (wave >> C.wlog) * ROWS * C.sets;
    const int sl = (wsl << 6) + lane;
    valid = sl < (C.k >> 6);
    slice = valid ? sl : 0;
    // descriptors based at the row group's first row (clamped to the matrix)
    const int base = min(row0, C.n - 1);
#pragma unroll
    for (int p = 0; p < NP; ++p)
      rp[p] = buffer_rsrc(reinterpret_cast<const char*>(C.p[p]) +
                          (size_t)base * (size_t)(C.k >> (kPlaneBits[p] == 2 ? 2 : 3)));
    rs = buffer_rsrc(C.s + (size_t)base * C.gpr);
    rz = buffer_rsrc(C.z + (size_t)base * C.gpr);
    vplane2 = slice * 16;
    vplane1 = slice * 8;
    vgroup = ((slice * C.gmul) >> 16) * 2;
  }

  // Issue the plane, scale and zero loads of batch b of row set `set` into
  // buffer BUF.  Rows past n are clamped to n - 1 (their results are not
  // stored).
  template <int BUF>
  __device__ __forceinline__ void load_batch(int set, int b) {
    const int base = min(row0, C.n - 1);
    const int rb2 = C.k >> 2, rb1 = C.k >> 3;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int r = min(row0 + set * ROWS + b * RB + i, C.n - 1) - base;  // uniform
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (kPlaneBits[p] == 2) {
          const stream_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rp[p], vplane2, r * rb2, kNontemporal);
          rec[BUF][i][0][kUnitOff[p]] = v.x;
          rec[BUF][i][0][kUnitOff[p] + 1] = v.y;
          rec[BUF][i][1][kUnitOff[p]] = v.z;
          rec[BUF][i][1][kUnitOff[p] + 1] = v.w;
        } else {
          const stream_u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rp[p], vplane1, r * rb1, kNontemporal);
          rec[BUF][i][0][kUnitOff[p]] = v.x;
          rec[BUF][i][1][kUnitOff[p]] = v.y;
        }
      }
      sz[BUF][i].x = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs, vgroup, r * C.gpr * 2, 0));
      sz[BUF][i].y = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rz, vgroup, r * C.gpr * 2, 0));
    }
  }

  // Activations of this lane's slice in register form: fp16 pairs (natural
  // k order, or the field order of the width-2 fast path) or fp32 for bf16,
  // the slice's sum of X and, for the fast path, the sum of X times the fp16
  // field offsets.  w0[mm] holds the slice's 64 halves of token mm.  Lanes
  // past the row's last slice and tokens past m hold copies of real
  // activations; what they compute is dropped (the per-row select of
  // compute_batch, the token check of the store), so nothing is masked here.
  __device__ __forceinline__ void x_setup(const uint32_t (&w0)[MT][32]) {
    constexpr uint32_t kOnes = 0x3C003C00u;  // (1.0, 1.0) in fp16
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const uint32_t (&w)[32] = w0[mm];
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
          float cs = 0.f;
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
              const int Pp = (idx < 5) ? P : P - 10;         // field bit after the optional shift by 10
              const uint32_t off = (uint32_t)(25 - Pp) << 10;  // fp16 2^(10 - Pp)
              cs = dot2h(pr, off | (off << 16), cs);
            }
          }
          xc[mm] = cs;
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) xr[mm][i] = w[i];
        }
      }
    }
  }

  // dot products of batch b (buffer BUF) into acc
  template <int BUF>
  __device__ __forceinline__ void compute_batch(int b) {
    uint32_t mg0 = 0, mg2 = 0, mg4 = 0, mg6 = 0, mg8 = 0;
    if constexpr (FAST2) {
      mg0 = vgpr_const<field2_magic<0>()>();
      mg2 = vgpr_const<field2_magic<2>()>();
      mg4 = vgpr_const<field2_magic<4>()>();
      mg6 = vgpr_const<field2_magic<6>()>();
      mg8 = vgpr_const<field2_magic<8>()>();
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float dot[MT];
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) dot[mm] = 0.f;
      if constexpr (FAST2) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const uint32_t w = rec[BUF][i][wd / 2][kUnitOff[0] + (wd & 1)];
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
          bytes[0] = assemble_word<NP, 0>(rec[BUF][i][u]);
          bytes[1] = assemble_word<NP, 1>(rec[BUF][i][u]);
          bytes[2] = assemble_word<NP, 2>(rec[BUF][i][u]);
          bytes[3] = assemble_word<NP, 3>(rec[BUF][i][u]);
          bytes[4] = assemble_word<NP, 4>(rec[BUF][i][u]);
          bytes[5] = assemble_word<NP, 5>(rec[BUF][i][u]);
          bytes[6] = assemble_word<NP, 6>(rec[BUF][i][u]);
          bytes[7] = assemble_word<NP, 7>(rec[BUF][i][u]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (BF16) {
              float fv[4];
              slice_f32x4<R, RULE>(bytes[j], fv);
#pragma unroll
              for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) dot[mm] = fmaf(fv[bb], xf[mm][32 * u + 4 * j + bb], dot[mm]);
              }
            } else {
              uint32_t lo, hi;
              if constexpr (RULE && R < 8) {
                slice_pairs<R, RULE>(bytes[j], lo, hi);
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
      const float s = (float)sz[BUF][i].x;
      const float z = (float)sz[BUF][i].y;
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        float t;
        if constexpr (FAST2) {
          // sum_k X (2^(10-P) + f) - xc = sum_k X f;  v = 64 f
          t = fmaf(64.0f, dot[mm] - xc[mm], (kDelta - z) * xs[mm]);
        } else if constexpr (BF16) {
          t = fmaf(kDelta - z, xs[mm], dot[mm]);
        } else {
          // z + (1024 - delta) is exact (an integer plus a value on a 0.5
          // grid, below 2^11) and takes one addition
          t = fmaf(-(z + (1024.0f - kDelta)), xs[mm], dot[mm]);
        }
        acc[(b * RB + i) * MT + mm] = valid ? s * t : 0.f;
      }
    }
  }

  template <int B>
  __device__ __forceinline__ void issue(int set) {
    if constexpr (B < PD) {
      load_batch<B>(set, B);
      issue<B + 1>(set);
    }
  }
  // Batch B of row set `set` computes from buffer B % PD, which then takes
  // the batch PD later: in this set, or the first ones of the next set (NB is
  // a multiple of PD, so every set uses the buffers in the same order).
  template <int B>
  __device__ __forceinline__ void run(int set) {
    if constexpr (B < NB) {
      compute_batch<B % PD>(B);
      if constexpr (B + PD < NB) {
        load_batch<B % PD>(set, B + PD);
      }
      run<B + 1>(set);
    }
  }

  // Sum acc over the wave (and the row group's waves through `red`) and
  // store the results of row set `set`.  `red` holds two slots used by
  // alternate sets: a slot is written again two sets later, after the
  // barrier of the set in between, which its readers reach only when done.
  __device__ __forceinline__ void finish(float* red, int m, int set) {
    // after log2(V) butterfly stages lane l holds the sum of value
    // l >> (6 - log2 V) over the lanes that share its upper bits
    constexpr int T = (V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
    butterfly<V, 32>(acc, lane);
    const int idx = lane >> (6 - T);
    const bool holder = (lane & ((1 << (6 - T)) - 1)) == 0;
    auto store = [&](int id, float val) {
      const int row = row0 + set * ROWS + id / MT, mm = id % MT;
      if (row < C.n && mm < m) {
        uint16_t* y = C.y + (size_t)mm * C.n + row;
        if constexpr (BF16) *y = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
        else *y = (uint16_t)(pack_f16x2(val, 0.f) & 0xFFFFu);
      }
    };
    if (C.wlog == 0) {
      if (holder) store(idx, acc[0]);
    } else {
      float* slot = red + (set & 1) * (4 * V);
      if (holder) slot[wave * V + idx] = acc[0];
      __syncthreads();
      if (wsl == 0 && lane < V) {
        float t = 0.f;
        for (int w = 0; w < (1 << C.wlog); ++w) t += slot[(wave + w) * V + lane];
        store(lane, t);
      }
    }
  }
};

// One workgroup per item: the item's call is found by a scalar search of the
// kernel arguments.  A row group of one wave (k <= 4096) shares the
// activations of its call with the other three waves through LDS; wider rows
// split the slices over 2 or 4 waves and each lane loads its own.
template <int R, int RULE, int MT, int BF16, int ROWS>
__device__ __forceinline__ void gemv_item(const GemvLaunch& a, const GemvCall& C, int it, float* red, uint4* xlds) {
  using Wave = GemvWave<R, RULE, MT, BF16, ROWS>;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int lane = (int)(threadIdx.x & 63);
  Wave w(C, it, wave, lane);
  // the weight loads go out first; the activations are read while they fly
  w.template issue<0>(0);
  uint32_t xw[MT][32];
  if (C.wlog == 0) {
    // chunk j of thread t: piece (t + 256 j) of the [token][slice][piece] X
    // block (16-byte pieces, consecutive threads on consecutive pieces)
    constexpr int XC = (MT * 512) / 256;
    const int S = C.k >> 6;
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int cidx = (int)threadIdx.x + 256 * j;
      const int mm = cidx >> 9, sl = (cidx >> 3) & 63, i = cidx & 7;
      const int mc = mm < a.m ? mm : 0;
      const int sc = sl < S ? sl : 0;
      xlds[((cidx >> 9) * 8 + (cidx & 7)) * 64 + ((cidx >> 3) & 63)] =
          reinterpret_cast<const uint4*>(C.x + (size_t)mc * C.k + (size_t)sc * 64)[i];
    }
    __syncthreads();
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = xlds[(mm * 8 + i) * 64 + lane];
        xw[mm][4 * i] = v.x;
        xw[mm][4 * i + 1] = v.y;
        xw[mm][4 * i + 2] = v.z;
        xw[mm][4 * i + 3] = v.w;
      }
  } else {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const int mc = mm < a.m ? mm : 0;
      const uint4* src = reinterpret_cast<const uint4*>(C.x + (size_t)mc * C.k + (size_t)w.slice * 64);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = src[i];
        xw[mm][4 * i] = v.x;
        xw[mm][4 * i + 1] = v.y;
        xw[mm][4 * i + 2] = v.z;
        xw[mm][4 * i + 3] = v.w;
      }
    }
  }
  w.x_setup(xw);
  // a rolled loop: the kernel holds every width's code path, and unrolling
  // the sets would outgrow the instruction cache
#pragma unroll 1
  for (int set = 0; set < C.sets; ++set) {
    if (set) w.template issue<0>(set);
    w.template run<0>(set);
    w.finish(red, a.m, set);
  }
}

// One workgroup per item: the item's call is found by a scalar search of the
// kernel arguments, and its width picks the code path (uniform over the
// workgroup), so one launch can hold calls of every width.
template <int RULE, int MT, int BF16, int ROWS>
__global__ __launch_bounds__(256) void gemv_multi_kernel(GemvLaunch a) {
  __shared__ float red[2 * 4 * ROWS * MT];  // two slots of [wave][value]
  __shared__ uint4 xlds[MT * 8 * 64];  // [token][piece][slice] for one-wave rows
  const int it = (int)blockIdx.x;
  int c = 0;
  while (c + 1 < a.ncalls && it >= a.c[c + 1].item0) ++c;
  const GemvCall& C = a.c[c];
  switch (C.r) {
    case 2: gemv_item<2, RULE, MT, BF16, ROWS>(a, C, it, red, xlds); break;
    case 3: gemv_item<3, RULE, MT, BF16, ROWS>(a, C, it, red, xlds); break;
    case 4: gemv_item<4, RULE, MT, BF16, ROWS>(a, C, it, red, xlds); break;
    case 6: gemv_item<6, RULE, MT, BF16, ROWS>(a, C, it, red, xlds); break;
    default: gemv_item<8, RULE, MT, BF16, ROWS>(a, C, it, red, xlds); break;
  }
}

int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// Row sets per item for a launch of `items1` one-set items: two sets spread
// the activation set-up over twice the rows, one keeps enough workgroups to
// fill the chip and balance its tail.  Measured on the 8B FFN decode step
// (7040 one-set items: 1 set 101.7 us, 2 sets 98.6 us, 4 sets 99.4 us) and on
// its single-width launches (1408 items: 2 sets no faster, 4 sets slower).
int gemv_sets(int items1) { return items1 >= 4096 ? 2 : 1; }

template <int RULE, int MT, int BF16, int ROWS>
hipError_t gemv_launch_r(const LinearArgs* la, int ncalls, int sets, hipStream_t s) {
  GemvLaunch a;
  int items = 0;
  for (int i = 0; i < ncalls; ++i) {
    GemvCall& c = a.c[i];
    c.x = static_cast<const uint16_t*>(la[i].x);
    c.y = static_cast<uint16_t*>(la[i].y);
    for (int p = 0; p < kPlanes; ++p) c.p[p] = la[i].pl.p[p];
    c.s = la[i].scales;
    c.z = la[i].zeros;
    c.n = la[i].n;
    c.k = la[i].k;
    c.r = la[i].r;
    c.item0 = items;
    const int W = waves_per_row(la[i].k);
    c.wlog = W == 1 ? 0 : W == 2 ? 1 : 2;
    c.sets = sets;
    c.rpi = (4 / W) * ROWS * sets;
    c.gpr = la[i].k / la[i].group;
    // exact for slice < 256 and group / 64 <= 256: the rounding error of the
    // multiplier stays below 1 / (group / 64)
    c.gmul = (65536 + la[i].group / 64 - 1) / (la[i].group / 64);
    items += cdiv(la[i].n, c.rpi);
  }
  for (int i = ncalls; i < kGemvMaxCalls; ++i) a.c[i] = a.c[ncalls - 1];
  a.ncalls = ncalls;
  a.m = la[0].m;
  hipLaunchKernelGGL((gemv_multi_kernel<RULE, MT, BF16, ROWS>), dim3((unsigned)items), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Launches of few items (fewer than kGemvFewItems 8-row items) take 4-row
// waves: twice the waves, and so twice the loads in flight, for the same bytes.
// Measured: the Llama-3.1-8B attention projections at M = 1 (q, k, v and o in
// one launch, 320 items) 4-8% faster at r >= 3 (4% slower at r = 2, where the
// per-item set-up weighs more), their dependent q/k/v-then-o block up to 15%
// faster; the FFN down (512 items, four waves per row) and gate+up (896)
// launches 2-15% slower.  A lane's partial sums meet in the same butterfly
// tree at either row count, so results do not depend on the choice.
constexpr int kGemvFewItems = 448;

template <int RULE, int MT, int BF16>
hipError_t gemv_launch_t(const LinearArgs* la, int ncalls, hipStream_t s) {
  constexpr int ROWS = gemv_rows(MT);
  int items1 = 0;
  for (int i = 0; i < ncalls; ++i) items1 += cdiv(la[i].n, (4 / waves_per_row(la[i].k)) * ROWS);
  if constexpr (ROWS == 8) {
    if (items1 < kGemvFewItems) return gemv_launch_r<RULE, MT, BF16, 4>(la, ncalls, 1, s);
  }
  return gemv_launch_r<RULE, MT, BF16, ROWS>(la, ncalls, gemv_sets(items1), s);
}

template <int RULE, int BF16>
hipError_t gemv_launch_m(const LinearArgs* a, int n, hipStream_t s) {
  if constexpr (BF16) {
    return gemv_launch_t<RULE, 1, 1>(a, n, s);  // bf16: m == 1 only
  } else {
    switch (a[0].m) {
      case 1: return gemv_launch_t<RULE, 1, 0>(a, n, s);
      case 2: return gemv_launch_t<RULE, 2, 0>(a, n, s);
      default: return gemv_launch_t<RULE, 4, 0>(a, n, s);
    }
  }
}

template <int RULE>
hipError_t gemv_launch_d(const LinearArgs* a, int n, hipStream_t s) {
  return a[0].bf16 ? gemv_launch_m<RULE, 1>(a, n, s) : gemv_launch_m<RULE, 0>(a, n, s);
}

}  // namespace

hipError_t launch_gemv_multi(const LinearArgs* a, int ncalls, hipStream_t s) {
  if (ncalls < 1 || ncalls > kGemvMaxCalls) return hipErrorInvalidValue;
  for (int i = 0; i < ncalls; ++i) {
    const int r = a[i].r;
    if ((r != 2 && r != 3 && r != 4 && r != 6 && r != 8) || a[i].rule != a[0].rule || a[i].m != a[0].m ||
        a[i].bf16 != a[0].bf16)
      return hipErrorInvalidValue;
  }
  return a[0].rule == kRuleExtra   ? gemv_launch_d<kRuleExtra>(a, ncalls, s)
         : a[0].rule == kRuleRound ? gemv_launch_d<kRuleRound>(a, ncalls, s)
                                   : gemv_launch_d<kRulePrefix>(a, ncalls, s);
}

}  // namespace mq
