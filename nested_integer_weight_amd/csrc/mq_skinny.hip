// mq_skinny.hip -- MFMA path for small decode batches (2 <= m <= 64).
//
// Y[m, n] = sum_k X[m, k] * w_hat[n, k] with the weights streamed straight from
// the bit planes into MFMA operand registers: no LDS round trip and no
// workgroup barrier for the weights, which are the HBM stream at these batch
// sizes.  Only the activations (a few KB per round) go through LDS, because
// every wave of a workgroup uses the same X slice.
//
// Work split.  A workgroup has 4 waves; wave w owns output rows
// n0 + 16 NT w + 16 t + c (t < NT; c = lane % 16; the planner takes NT = 1,
// 64-row workgroups).  The k range of a workgroup
// is walked in rounds of 256: in a round, lane group g = lane / 16 owns the
// 64 consecutive codes [64 g, 64 g + 64) of each of its rows, i.e. one
// 16-byte load per 2-bit plane and one 8-byte load per 1-bit plane.  MFMA
// k-step i (0..7) of v_mfma_f32_16x16x32_{f16,bf16} takes from lane group g
// the codes [64 g + 8 i, 64 g + 8 i + 8); the activation fragments in LDS
// use the same k order, so every product pairs X[m, k] with w_hat[n, k].
// A 64-code chunk never straddles a quantization group (group % 64 == 0),
// so each lane needs one scale and zero point per row and round.
//
// Operand values.  The weight operand is w_hat = s * (v - z) (+ delta_r for
// the true-prefix rule, MatGPTQ "Efficient and Accurate Inference over
// Nested Quantized Models", section 3, reconstruction with the centring
// offset) rounded once to the activation dtype:
//   fp16: the byte v becomes the exact half 1024 + v (v_perm with an 0x64
//         exponent byte); subtracting 1024 and adding (delta - z) are exact
//         in half precision (|v - z + delta| <= 255.5 on a 0.5 grid), and the
//         multiply by the fp16 scale rounds once to nearest even -- the same
//         value as rounding the exact product.
//   bf16: exact in fp32 (v * s + (delta - z) * s), then one RNE to bf16.
// Accumulation is fp32 in the MFMA.
//
// Split-k: a workgroup's flat index picks its call, then its row block and k
// range there; with more than one range the fp32 partial tiles go to the
// call's part of the workspace, [split][m][n], and the fixed-order reduction
// kernel of the GEMM path sums them, so results stay deterministic.
// Independent calls of one launch shape share a launch (one ramp and drain).

#include "mq_common.h"
#include "mq_kernels.h"

namespace mq {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// native vectors, not HIP's uint4/uint2 structs: copies of those go through
// memcpy and would pin the staging registers in memory
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
// 16-row output tiles per wave: NT = 1 (64 output rows per workgroup, the
// planner's choice) or NT = 2 (128 rows)
template <int NT>
constexpr int cols_per_block() { return 16 * NT * kWaves; }
constexpr int kRound = 256;                   // k per round at one chunk per lane

struct SkinnyArgs {
  const uint16_t* x;
  void* y;  // [m, n] in x's dtype, or fp32 workspace [splits][m][n]
  PlanePtrs pl;
  const uint16_t* scales;
  const uint16_t* zeros;
  int m, n, k, group;
  int rounds_per_split;
  int to_workspace;
};

// The calls of one launch: call i owns the flat workgroups blk0[i] ..
// blk0[i] + gx[i] * splits_i - 1, row block fastest.  All calls share the
// kernel's template shape (width, rule, dtype, m tiles, row tiles, teams,
// run length).
struct SkinnyLaunch {
  SkinnyArgs c[kSkinnyMaxCalls];
  int gx[kSkinnyMaxCalls];
  int blk0[kSkinnyMaxCalls];
  int ncalls;
};

template <int BF16>
__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  }
}

// RNE(s * (v - z + delta)) for two code bytes given as the halves 1024 + v.
// With an integer offset (delta = 0: the rounded slice, and the full-width
// prefix) c holds -(1024 + z), an integer below 2048 and so exact in half
// precision, and one exact addition gives v - z; otherwise c = delta - z and
// the 1024 goes first.
template <bool INT_OFFSET>
__device__ __forceinline__ uint32_t dq_f16x2(uint32_t magic_pair, f16x2 c, f16x2 s) {
  f16x2 v = __builtin_bit_cast(f16x2, magic_pair);
  if constexpr (!INT_OFFSET) {
    const f16x2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    v = v - k1024;  // exact: the code value
  }
  v = v + c;  // exact: v - z + delta
  v = v * s;  // the one rounding
  return __builtin_bit_cast(uint32_t, v);
}

// RUN = 64-code runs per lane, row and round: a round covers RUN * 256 codes,
// i.e. RUN * 64 bytes of every 2-bit plane row.  RUN = 2 reads whole 128-byte
// lines per row and round.
// XB = X buffers per team: 2 (the next round's X is staged while the current
// one is read) or 1 (staged after a barrier that follows the reads, when two
// buffers of long rounds would not fit in LDS)
template <int R, int RULE, int BF16, int MT, int NT, int RUN, int XB>
struct SkinnyWave {
  static constexpr int NP = planes_needed(R, RULE);
  static constexpr float kDelta = RULE ? 0.0f : prefix_delta(R);
  static constexpr int KR = kRound * RUN;     // codes per round
  static constexpr int KS = 8 * RUN;          // MFMA k-steps per round
  static constexpr int CPR = KR / 8;          // 16-byte X chunks per activation row and round
  static constexpr int XPIECES = 2 * MT * RUN;  // 16-byte X pieces per thread per round

  // weight slots in flight: rounds with few planes carry little data, so they
  // are loaded two rounds ahead; wider ones one round ahead
  // (bf16 at one m tile with two row tiles is the exception: its fp32 operand
  // arithmetic leaves no room for a third slot without spilling)
  static constexpr int kSlots = (NP <= 3 && !(BF16 && MT == 1 && NT == 2)) ? 3 : 2;

  const SkinnyArgs a;  // by value: a reference would make the compiler keep a copy in memory
  int tid, lane, g, c, nw, kb0;
  size_t upr;
  int gpr;
  // weights of one round per slot: [slot][tile][unit][word]
  uint32_t rec[kSlots][NT][2 * RUN][kUnitWords];
  // raw fp16 bits of scale and zero, zero-extended by the load itself (no
  // arithmetic before use, so the loads stay in flight)
  uint32_t sraw[kSlots][NT], zraw[kSlots][NT];
  u32x4 xreg[XPIECES];
  f32x4 acc[MT][NT];

  __device__ __forceinline__ SkinnyWave(const SkinnyArgs& args, int t, int n0, int kbase) : a(args), tid(t), kb0(kbase) {
    lane = t & 63;
    g = lane >> 4;
    c = lane & 15;
    nw = n0 + 16 * NT * (t >> 6);
    upr = (size_t)(a.k >> 5);
    gpr = a.k / a.group;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // X piece p = tid + 256 j is 16-byte chunk q = p % CPR of row p / CPR of
  // the round: CPR consecutive lanes read one row's contiguous round slice.
  // The chunk holds k = 8 q .. 8 q + 7, i.e. k-step i = q % KS of lane group
  // q / KS, so it goes to LDS block (m tile, k step) = (row / 16, i) at
  // fragment position 16 (q / KS) + row % 16, xor-ed with i % 8: the eight
  // consecutive lanes that one ds_write_b128 clock serves then hit distinct
  // banks, and the fragment reads (lane ^ (i % 8)) stay contiguous per 8
  // lanes.  Rows past m are clamped; they only feed output rows that are not
  // stored.
  __device__ __forceinline__ void load_x(int rnd) {
    const int kr = kb0 + rnd * KR;
#pragma unroll
    for (int j = 0; j < XPIECES; ++j) {
      const int p = tid + 256 * j;
      const int row = min(p / CPR, a.m - 1);
      xreg[j] = *reinterpret_cast<const u32x4*>(a.x + (size_t)row * a.k + kr + 8 * (p % CPR));
    }
  }
  __device__ __forceinline__ void store_x(u32x4* xs) {
#pragma unroll
    for (int j = 0; j < XPIECES; ++j) {
      const int p = tid + 256 * j;
      const int row = p / CPR, q = p % CPR;
      const int i = q % KS;
      xs[((row >> 4) * KS + i) * 64 + (((q / KS) * 16 + (row & 15)) ^ (i & 7))] = xreg[j];
    }
  }

  // plane words, scale and zero of row tile T for the round starting at code kc
  template <int SLOT, int T>
  __device__ __forceinline__ void load_w_tile(int kc) {
    const int row = min(nw + 16 * T + c, a.n - 1);
    // first unit of the chunk: a multiple of 2 RUN (k % KR == 0), so the
    // vector loads below are aligned to their size
    const size_t u0 = (size_t)row * upr + (size_t)(kc >> 5);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (kPlaneBits[p] == 2) {
#pragma unroll
        for (int h = 0; h < RUN; ++h) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(a.pl.p[p] + 2 * (u0 + 2 * h));
          rec[SLOT][T][2 * h][kUnitOff[p]] = v.x;
          rec[SLOT][T][2 * h][kUnitOff[p] + 1] = v.y;
          rec[SLOT][T][2 * h + 1][kUnitOff[p]] = v.z;
          rec[SLOT][T][2 * h + 1][kUnitOff[p] + 1] = v.w;
        }
      } else if constexpr (RUN == 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(a.pl.p[p] + u0);
        rec[SLOT][T][0][kUnitOff[p]] = v.x;
        rec[SLOT][T][1][kUnitOff[p]] = v.y;
        rec[SLOT][T][2][kUnitOff[p]] = v.z;
        rec[SLOT][T][3][kUnitOff[p]] = v.w;
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(a.pl.p[p] + u0);
        rec[SLOT][T][0][kUnitOff[p]] = v.x;
        rec[SLOT][T][1][kUnitOff[p]] = v.y;
      }
    }
    const size_t gi = (size_t)row * gpr + (size_t)(kc / a.group);
    sraw[SLOT][T] = a.scales[gi];
    zraw[SLOT][T] = a.zeros[gi];
  }
  template <int SLOT>
  __device__ __forceinline__ void load_w(int rnd) {
    const int kc = kb0 + rnd * KR + 64 * RUN * g;  // first code of this lane's chunk
    load_w_tile<SLOT, 0>(kc);
    if constexpr (NT == 2) load_w_tile<SLOT, 1>(kc);
  }

  // weight operand of MFMA k-step I for row tile T: codes [8 I, 8 I + 8) of the chunk
  // (a chunk of 64 RUN codes lies in one quantization group: group % (64 RUN) == 0)
  // (every array index here is a compile-time constant, so the staging arrays
  // stay in registers)
  template <int SLOT, int I, int T>
  __device__ __forceinline__ u32x4 w_frag() const {
    const uint32_t* u = rec[SLOT][T][I >> 2];
    constexpr int J0 = 2 * (I & 3);
    const uint32_t w0 = slice_bytes<R, RULE>(assemble_word<NP, J0>(u));
    const uint32_t w1 = slice_bytes<R, RULE>(assemble_word<NP, J0 + 1>(u));
    if constexpr (BF16) {
      const float s = h2f((uint16_t)sraw[SLOT][T]);
      const float cz = (kDelta - h2f((uint16_t)zraw[SLOT][T])) * s;  // exact
      u32x4 f;
      f.x = pack_bf16x2(fmaf((float)(w0 & 0xFFu), s, cz), fmaf((float)((w0 >> 8) & 0xFFu), s, cz));
      f.y = pack_bf16x2(fmaf((float)((w0 >> 16) & 0xFFu), s, cz), fmaf((float)(w0 >> 24), s, cz));
      f.z = pack_bf16x2(fmaf((float)(w1 & 0xFFu), s, cz), fmaf((float)((w1 >> 8) & 0xFFu), s, cz));
      f.w = pack_bf16x2(fmaf((float)((w1 >> 16) & 0xFFu), s, cz), fmaf((float)(w1 >> 24), s, cz));
      return f;
    } else {
      const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sraw[SLOT][T]);
      constexpr bool kInt = kDelta == 0.0f;
      // exact: |delta - z| <= 255.5, and 1024 + z <= 1279 for the integer form
      const _Float16 ch = (_Float16)((kInt ? -1024.0f : kDelta) - h2f((uint16_t)zraw[SLOT][T]));
      const f16x2 s2 = {sh, sh};
      const f16x2 c2 = {ch, ch};
      u32x4 f;
      f.x = dq_f16x2<kInt>(__builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u), c2, s2);
      f.y = dq_f16x2<kInt>(__builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u), c2, s2);
      f.z = dq_f16x2<kInt>(__builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u), c2, s2);
      f.w = dq_f16x2<kInt>(__builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u), c2, s2);
      return f;
    }
  }

  template <int SLOT, int I>
  __device__ __forceinline__ void kstep(const u32x4* xs) {
    if constexpr (NT == 2) {
      const u32x4 wf0 = w_frag<SLOT, I, 0>();
      const u32x4 wf1 = w_frag<SLOT, I, NT - 1>();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 xf = xs[(mt * KS + I) * 64 + (lane ^ (I & 7))];
        acc[mt][0] = mfma<BF16>(xf, wf0, acc[mt][0]);
        acc[mt][NT - 1] = mfma<BF16>(xf, wf1, acc[mt][NT - 1]);
      }
    } else {
      const u32x4 wf0 = w_frag<SLOT, I, 0>();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 xf = xs[(mt * KS + I) * 64 + (lane ^ (I & 7))];
        acc[mt][0] = mfma<BF16>(xf, wf0, acc[mt][0]);
      }
    }
  }

  template <int SLOT, int I = 0>
  __device__ __forceinline__ void compute(const u32x4* xs) {
    if constexpr (I < KS) {
      kstep<SLOT, I>(xs);
      compute<SLOT, I + 1>(xs);
    }
  }

  // Round rnd computes from slot SLOT and LDS buffer rnd & 1 (the only buffer
  // when XB = 1).  It first issues the X loads of round rnd + 1 and then the
  // weight loads of round rnd + kSlots - 1 (into the slot of round rnd - 1),
  // in that order, so that staging X at the end of the round waits for the X
  // loads only and the weights stay in flight across the barrier(s).  Past the
  // last round the loads repeat it.
  template <int SLOT>
  __device__ __forceinline__ void round(int rnd, int last, u32x4* xs0, u32x4* xs1) {
    load_x(min(rnd + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    load_w<(SLOT + kSlots - 1) % kSlots>(min(rnd + kSlots - 1, last));
    compute<SLOT>((rnd & 1) ? xs1 : xs0);
    if constexpr (XB == 1) {
      __syncthreads();
      store_x(xs0);
    } else {
      store_x((rnd & 1) ? xs0 : xs1);
    }
    __syncthreads();
  }

  __device__ __forceinline__ void run(int nr, u32x4* xs0, u32x4* xs1) {
    const int last = nr - 1;
    load_x(0);
    __builtin_amdgcn_sched_barrier(0);
    load_w<0>(0);
    if constexpr (kSlots == 3) load_w<1>(min(1, last));
    store_x(xs0);
    __syncthreads();
    int r = 0;
    if constexpr (kSlots == 3) {
      for (; r + 2 < nr; r += 3) {
        round<0>(r, last, xs0, xs1);
        round<1>(r + 1, last, xs0, xs1);
        round<2>(r + 2, last, xs0, xs1);
      }
      if (r < nr) round<0>(r, last, xs0, xs1);
      if (r + 1 < nr) round<1>(r + 1, last, xs0, xs1);
    } else {
      for (; r + 1 < nr; r += 2) {
        round<0>(r, last, xs0, xs1);
        round<1>(r + 1, last, xs0, xs1);
      }
      if (r < nr) round<0>(r, last, xs0, xs1);
    }
  }
};

// two X buffers per team unless two teams with long rounds at three or four
// m tiles need one each to stay within 128 KB of LDS
template <int MT, int KH, int RUN>
constexpr int x_buffers() { return (KH == 2 && RUN == 2 && MT >= 3) ? 1 : 2; }

// KH teams of 4 waves share a workgroup and split its k range: team 0 takes
// the first ceil(nr / KH) rounds, team 1 the rest, each with its own X
// buffers, and team 1 hands its partial tiles to team 0 through LDS at the
// end.  With one workgroup per CU this puts two waves on every SIMD, so one
// wave's operand arithmetic overlaps the other's weight loads, and twice the
// weight bytes are in flight per CU.
// Two waves per SIMD is enough to cover the latency with the prefetch above;
// asking for more would make the compiler spill the staging registers.
template <int R, int RULE, int BF16, int MT, int NT, int KH, int RUN>
__global__ __launch_bounds__(256 * KH) __attribute__((amdgpu_waves_per_eu(2, 2))) void skinny_kernel(SkinnyLaunch L) {
  constexpr int KR = kRound * RUN;
  constexpr int XB = x_buffers<MT, KH, RUN>();
  __shared__ u32x4 Xs[KH][XB][MT * 8 * RUN * 64];
  // the call this workgroup serves, and its row block and k range there
  int ci = 0;
  while (ci + 1 < L.ncalls && (int)blockIdx.x >= L.blk0[ci + 1]) ++ci;
  const SkinnyArgs& a = L.c[ci];
  const int local = (int)blockIdx.x - L.blk0[ci];
  const int by = local / L.gx[ci];
  const int bx = local - by * L.gx[ci];
  const int team = KH == 2 ? (int)(threadIdx.x >> 8) : 0;
  const int tid = threadIdx.x & 255;
  const int n0 = bx * cols_per_block<NT>();
  const int ks = by * a.rounds_per_split * KR;
  const int nr_all = min(a.rounds_per_split, (a.k - ks) / KR);
  const int nr0 = (nr_all + KH - 1) / KH;
  const int nr = team == 0 ? nr0 : nr_all - nr0;
  SkinnyWave<R, RULE, BF16, MT, NT, RUN, XB> w(a, tid, n0, ks + team * nr0 * KR);
  if (nr > 0) w.run(nr, Xs[team][0], Xs[team][XB - 1]);
  const int lane = tid & 63;
  if constexpr (KH == 2) {
    // run() passes 1 + (3 - XB) nr barriers (none for nr = 0); team 1, which
    // may have one round fewer, passes the missing ones here so that the two
    // teams' barriers pair up
    constexpr int BPR = 3 - XB;  // barriers per round
    const int pad = (nr0 > 0 ? 1 + BPR * nr0 : 0) - (nr > 0 ? 1 + BPR * nr : 0);
    for (int i = 0; i < pad; ++i) __syncthreads();
    // every wave is past its last round: team 1's X buffers are free
    f32x4* part = reinterpret_cast<f32x4*>(&Xs[1][0][0]);
    const int wt = tid >> 6;
    if (team == 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) part[((wt * MT + mt) * NT + t) * 64 + lane] = w.acc[mt][t];
    }
    __syncthreads();
    if (team == 1) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) w.acc[mt][t] += part[((wt * MT + mt) * NT + t) * 64 + lane];
  }
  // lane holds D[4 (lane / 16) + v][lane % 16] of every (m tile, row tile)
  const int nb = n0 + 16 * NT * (tid >> 6) + (lane & 15);
  const int mb = 4 * (lane >> 4);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int nn = nb + 16 * t;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int mm = 16 * mt + mb + v;
        if (mm < a.m && nn < a.n) {
          const float val = w.acc[mt][t][v];
          if (a.to_workspace) {
            static_cast<float*>(a.y)[((size_t)by * a.m + mm) * a.n + nn] = val;
          } else {
            uint16_t* y = static_cast<uint16_t*>(a.y) + (size_t)mm * a.n + nn;
            *y = (uint16_t)((BF16 ? pack_bf16x2(val, 0.f) : pack_f16x2(val, 0.f)) & 0xFFFFu);
          }
        }
      }
    }
  }
}

// about one workgroup per CU: measured against 448 and 896 at m = 8 and 64,
// fewer, longer k ranges win (less split-k traffic, fewer workgroup prologues)
constexpr int kTargetBlocks = 224;

int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// workgroup shapes that are instantiated: two teams need two m tiles, long
// runs at three or four m tiles come with two teams, and the X buffers
// (KH teams x XB x MT tiles x KS steps x 1 KB) fit in 128 KB
template <int MT, int KH, int RUN>
constexpr bool shape_ok() {
  return !(MT == 1 && KH == 2) && (RUN == 1 || MT <= 2 || (MT == 3 && KH == 2)) &&
         KH * x_buffers<MT, KH, RUN>() * MT * RUN <= 16;
}

template <int R, int RULE, int BF16, int MT, int NT, int KH, int RUN>
hipError_t launch_k(const SkinnyLaunch& sa, dim3 grid, hipStream_t s) {
  if constexpr (shape_ok<MT, KH, RUN>()) {
    hipLaunchKernelGGL((skinny_kernel<R, RULE, BF16, MT, NT, KH, RUN>), grid, dim3(256 * KH), 0, s, sa);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int R, int RULE, int BF16, int NT, int KH, int RUN>
hipError_t launch_t(const SkinnyLaunch& sa, int mt, dim3 grid, hipStream_t s) {
  switch (mt) {
    case 1: return launch_k<R, RULE, BF16, 1, NT, KH, RUN>(sa, grid, s);
    case 2: return launch_k<R, RULE, BF16, 2, NT, KH, RUN>(sa, grid, s);
    case 3: return launch_k<R, RULE, BF16, 3, NT, KH, RUN>(sa, grid, s);
    default: return launch_k<R, RULE, BF16, 4, NT, KH, RUN>(sa, grid, s);
  }
}

// (the planner takes 64-row workgroups, NT = 1, only)
template <int R, int RULE, int BF16>
hipError_t launch_b(const SkinnyLaunch& sa, int mt, const SkinnyPlan& p, dim3 grid, hipStream_t s) {
  if (p.nt != 1) return hipErrorInvalidValue;
  if (p.run == 2) return p.kh == 2 ? launch_t<R, RULE, BF16, 1, 2, 2>(sa, mt, grid, s)
                                   : launch_t<R, RULE, BF16, 1, 1, 2>(sa, mt, grid, s);
  return p.kh == 2 ? launch_t<R, RULE, BF16, 1, 2, 1>(sa, mt, grid, s)
                   : launch_t<R, RULE, BF16, 1, 1, 1>(sa, mt, grid, s);
}

template <int R, int RULE>
hipError_t launch_d(const SkinnyLaunch& sa, int bf16, int mt, const SkinnyPlan& p, dim3 grid, hipStream_t s) {
  return bf16 ? launch_b<R, RULE, 1>(sa, mt, p, grid, s) : launch_b<R, RULE, 0>(sa, mt, p, grid, s);
}

}  // namespace

SkinnyPlan plan_skinny(int m, int n, int k, int group, int planes) {
  SkinnyPlan p;
  // 128-code runs per lane when the groups and k allow it: 9-16% faster at
  // one m tile; at two and three m tiles only from three planes up (r = 2
  // and 3 lose up to 8%, r = 8 gains 7-9%); at four m tiles the longer rounds
  // need more registers than two waves per SIMD leave.  Long runs go with
  // 64-row workgroups.
  const int mt = cdiv(m, 16);
  p.run = (group % 128 == 0 && k % (2 * kRound) == 0 && (mt == 1 || (mt <= 3 && planes >= 3))) ? 2 : 1;
  // 64-row workgroups throughout: the independent calls of a decode step
  // (gate, up, down) then share one launch shape and so one launch; with
  // shared launches this was 4-10% faster at m = 64 and 4-7% at m = 32 (r = 2)
  // than 128-row workgroups for narrow n.
  p.nt = 1;
  const int rounds = k / (kRound * p.run);
  const int blocks_n = p.nt == 1 ? cdiv(n, cols_per_block<1>()) : cdiv(n, cols_per_block<2>());
  int s = cdiv(kTargetBlocks, blocks_n);
  if (s > rounds) s = rounds;
  if (s < 1) s = 1;
  p.rounds_per_split = cdiv(rounds, s);
  p.splits = cdiv(rounds, p.rounds_per_split);
  // two teams per workgroup from two m tiles up: measured 4-8% faster at
  // m = 32 and 64; at one m tile neither form wins consistently.  With long
  // runs at three m tiles each team keeps one X buffer (128 KB of LDS).
  p.kh = m > 16 ? 2 : 1;
  return p;
}

size_t skinny_workspace_bytes(int m, int n, int k) {
  if (!skinny_shape(m, k)) return 0;
  // the k split depends on the run length, which depends on the group and
  // the width: size for the larger of the two plans
  const SkinnyPlan p1 = plan_skinny(m, n, k, 64, 1);
  const SkinnyPlan p2 = plan_skinny(m, n, k, 128, 5);
  const int splits = p1.splits > p2.splits ? p1.splits : p2.splits;
  return splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * sizeof(float) : 0;
}

SkinnyPlan plan_skinny_call(const LinearArgs& la) {
  return plan_skinny(la.m, la.n, la.k, la.group, planes_needed(la.r, la.rule));
}

size_t skinny_call_workspace(const LinearArgs& la) {
  const SkinnyPlan p = plan_skinny_call(la);
  return p.splits > 1 ? (size_t)p.splits * (size_t)la.m * (size_t)la.n * sizeof(float) : 0;
}

bool same_skinny_launch(const LinearArgs& a, const LinearArgs& b) {
  if (a.m != b.m || a.r != b.r || a.rule != b.rule || a.bf16 != b.bf16) return false;
  const SkinnyPlan p = plan_skinny_call(a), q = plan_skinny_call(b);
  return p.nt == q.nt && p.kh == q.kh && p.run == q.run;
}

hipError_t launch_skinny_multi(const LinearArgs* la, int ncalls, void* workspace, size_t workspace_bytes,
                               hipStream_t s) {
  if (ncalls < 1 || ncalls > kSkinnyMaxCalls) return hipErrorInvalidValue;
  for (int i = 0; i < ncalls; ++i)
    if (la[i].rule == kRuleExtra || !same_skinny_launch(la[0], la[i])) return hipErrorInvalidValue;
  SkinnyLaunch L;
  SkinnyPlan plan[kSkinnyMaxCalls];
  size_t ws_off[kSkinnyMaxCalls];
  size_t used = 0;
  int blocks = 0;
  for (int i = 0; i < ncalls; ++i) {
    SkinnyPlan p = plan_skinny_call(la[i]);
    const size_t need = p.splits > 1 ? (size_t)p.splits * (size_t)la[i].m * (size_t)la[i].n * sizeof(float) : 0;
    ws_off[i] = ws_align(used);
    if (need && (!workspace || ws_off[i] + need > workspace_bytes)) {
      // not enough workspace for this call's k split: one range
      p.splits = 1;
      p.rounds_per_split = la[i].k / (kRound * p.run);
    }
    if (p.splits > 1) used = ws_off[i] + need;
    plan[i] = p;
    SkinnyArgs& sa = L.c[i];
    sa.x = static_cast<const uint16_t*>(la[i].x);
    sa.pl = la[i].pl;
    sa.scales = la[i].scales;
    sa.zeros = la[i].zeros;
    sa.m = la[i].m;
    sa.n = la[i].n;
    sa.k = la[i].k;
    sa.group = la[i].group;
    sa.rounds_per_split = p.rounds_per_split;
    sa.to_workspace = p.splits > 1;
    sa.y = p.splits > 1 ? static_cast<void*>(static_cast<char*>(workspace) + ws_off[i]) : la[i].y;
    L.gx[i] = cdiv(la[i].n, p.nt == 1 ? cols_per_block<1>() : cols_per_block<2>());
    L.blk0[i] = blocks;
    blocks += L.gx[i] * p.splits;
  }
  L.ncalls = ncalls;
  const int mt = cdiv(la[0].m, 16);
  const dim3 grid((unsigned)blocks);
  hipError_t e;
#define MQ_SK_CASE(RR)                                                                  \
  case RR:                                                                              \
    e = la[0].rule ? launch_d<RR, 1>(L, la[0].bf16, mt, plan[0], grid, s)               \
                   : launch_d<RR, 0>(L, la[0].bf16, mt, plan[0], grid, s);              \
    break;
  switch (la[0].r) {
    MQ_SK_CASE(2)
    MQ_SK_CASE(3)
    MQ_SK_CASE(4)
    MQ_SK_CASE(6)
    MQ_SK_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MQ_SK_CASE
  if (e != hipSuccess) return e;
  for (int i = 0; i < ncalls && e == hipSuccess; ++i)
    if (plan[i].splits > 1)
      e = launch_splitk_reduce(static_cast<const float*>(L.c[i].y), plan[i].splits,
                               (size_t)la[i].m * (size_t)la[i].n, la[i].y, la[i].bf16, s);
  return e;
}

hipError_t launch_skinny(const LinearArgs& la, void* workspace, size_t workspace_bytes, hipStream_t s) {
  return launch_skinny_multi(&la, 1, workspace, workspace_bytes, s);
}

}  // namespace mq
