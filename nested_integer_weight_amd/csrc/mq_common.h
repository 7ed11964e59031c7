// mq_common.h -- device-side layout and slicing helpers shared by every libmq
// kernel (packer, slice/dequant exports, GEMV, MFMA GEMM).
//
// Bit planes (MatGPTQ "Efficient and Accurate Inference over Nested Quantized
// Models", section 4: buffers for bits 1-2, 3, 4, 5-6, 7-8 from the MSB):
//   plane 0: bits 7..6   plane 1: bit 5   plane 2: bit 4
//   plane 3: bits 3..2   plane 4: bits 1..0
// Each plane is [n][k/32] units of 32 consecutive codes of one row.  A unit is
// two 32-bit words for a 2-bit plane and one word for a 1-bit plane.
//
// Within a unit, code t (0..31) of a 2-bit plane lives in word t/16 at bit
//   8*(t%4) + 2*((t%16)/4)
// and code t of a 1-bit plane lives at bit
//   8*(t%4) + t/4.
// So for output word j (codes 4j..4j+3) one shift of the plane word by a
// constant and one mask put the four codes' fields straight into their
// natural place inside four bytes: after OR-ing the planes a unit becomes the
// 32 truncated codes as bytes in k order.  No field ever crosses a byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kPlanes = 5;
constexpr int kPlaneBits[kPlanes] = {2, 1, 1, 2, 2};
// code bit index of each plane's lowest bit
constexpr int kPlaneLsb[kPlanes] = {6, 5, 4, 2, 0};
// offset of each plane's words in a packed "unit record" of 8 words
constexpr int kUnitOff[kPlanes] = {0, 2, 3, 4, 6};
constexpr int kUnitWords = 8;

__host__ __device__ constexpr int planes_for_bits(int bits) {
  return bits <= 2 ? 1 : bits == 3 ? 2 : bits == 4 ? 3 : bits <= 6 ? 4 : 5;
}
// leading bits covered by the first P planes
__host__ __device__ constexpr int bits_of_planes(int P) {
  return P <= 0 ? 0 : P == 1 ? 2 : P == 2 ? 3 : P == 3 ? 4 : P == 4 ? 6 : 8;
}
// Slicing rules, the RULE template parameter of every kernel (the values of
// mq_rule in mq.h):
//   kRulePrefix MatGPTQ true prefix: the r most significant bits, + delta_r
//   kRuleRound  MatQuant: round half up on the (r+1)-th bit, clamp to 2^r - 1
//   kRuleExtra  Extra-Precision MatQuant: the same rounding without the clamp,
//               2^r + 1 levels, values up to 256
constexpr int kRulePrefix = 0, kRuleRound = 1, kRuleExtra = 2;

// planes read by a width-r call: the true prefix reads r bits, both rounded
// rules r + 1 (r < 8), each rounded up to a plane boundary
__host__ __device__ constexpr int planes_needed(int r, int rule) {
  return planes_for_bits((rule && r < 8) ? r + 1 : r);
}
__host__ __device__ constexpr uint32_t rep4(uint32_t b) { return b * 0x01010101u; }

template <int SH>
__device__ __forceinline__ uint32_t shift_signed(uint32_t v) {
  if constexpr (SH >= 0) return v << SH; else return v >> (-SH);
}

// (a & mask) | c in one v_and_or_b32: gfx9 VOP3 encodings take no literal, so
// the mask is handed over in an SGPR and the accumulator stays in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
}

// Plane P's word for output word J (codes 4J..4J+3 of a unit) shifted so the
// four codes' fields sit at their code-bit position inside each byte.
template <int P, int J>
__device__ __forceinline__ uint32_t plane_shifted(const uint32_t* unit) {
  if constexpr (kPlaneBits[P] == 2) {
    return shift_signed<kPlaneLsb[P] - 2 * (J % 4)>(unit[kUnitOff[P] + J / 4]);
  } else {
    return shift_signed<kPlaneLsb[P] - J>(unit[kUnitOff[P]]);
  }
}
template <int P>
__host__ __device__ constexpr uint32_t plane_mask() {
  return rep4((kPlaneBits[P] == 2 ? 3u : 1u) << kPlaneLsb[P]);
}

template <int NP, int J, int P = 0>
__device__ __forceinline__ uint32_t assemble_word_impl(const uint32_t* unit, uint32_t acc) {
  if constexpr (P >= NP) {
    return acc;
  } else {
    return assemble_word_impl<NP, J, P + 1>(unit, and_or(plane_shifted<P, J>(unit), plane_mask<P>(), acc));
  }
}

// Output word J of a unit from its first NP planes: four codes as bytes with
// the planes' bits in place and all lower bits zero.
template <int NP, int J>
__device__ __forceinline__ uint32_t assemble_word(const uint32_t* unit) {
  return assemble_word_impl<NP, J, 1>(unit, plane_shifted<0, J>(unit) & plane_mask<0>());
}

// Value of the r-bit slice in the 8-bit code space for four codes packed in
// one word (bytes as assembled from the planes), before any centring offset:
//   kRulePrefix: v = (q >> (8-r)) << (8-r)                        (<= 255)
//   kRuleRound:  v = min(round_half_up(q / 2^(8-r)), 2^r - 1) << (8-r)
//   kRuleExtra:  v = round_half_up(q / 2^(8-r)) << (8-r)           (<= 256)
// The rounding can overflow a byte, so it is evaluated in 16-bit lanes:
// `lo`/`hi` receive codes {0,1} and {2,3} as u16 pairs.
template <int R, int RULE>
__device__ __forceinline__ void slice_pairs(uint32_t bytes, uint32_t& lo, uint32_t& hi) {
  // v_perm_b32 selector: byte 0x0c yields 0x00
  lo = __builtin_amdgcn_perm(0u, bytes, 0x0c010c00u);
  hi = __builtin_amdgcn_perm(0u, bytes, 0x0c030c02u);
  if constexpr (RULE && R < 8) {
    constexpr uint32_t keep = (0xFFu << (7 - R)) & 0xFFu;  // top r+1 bits
    constexpr uint32_t half = 1u << (7 - R);               // the (r+1)-th bit
    constexpr uint32_t lim = 256u - (1u << (8 - R));       // (2^r - 1) << (8-r)
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 a = __builtin_bit_cast(u16x2, lo & (keep * 0x10001u));
    u16x2 b = __builtin_bit_cast(u16x2, hi & (keep * 0x10001u));
    const u16x2 hv = {(unsigned short)half, (unsigned short)half};
    a = a + (a & hv);
    b = b + (b & hv);
    if constexpr (RULE == kRuleRound) {
      const u16x2 lv = {(unsigned short)lim, (unsigned short)lim};
      a = __builtin_elementwise_min(a, lv);
      b = __builtin_elementwise_min(b, lv);
    }
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
  }
}

// Same slice, kept as four bytes (v <= 255: not for the unclamped rule).
template <int R, int RULE>
__device__ __forceinline__ uint32_t slice_bytes(uint32_t bytes) {
  static_assert(RULE != kRuleExtra || R == 8, "the unclamped slice reaches 256: use slice_pairs");
  if constexpr (RULE && R < 8) {
    uint32_t lo, hi;
    slice_pairs<R, RULE>(bytes, lo, hi);
    return __builtin_amdgcn_perm(hi, lo, 0x06040200u);
  } else {
    return bytes;
  }
}

// The four slice values of a word as floats, for every rule.
template <int R, int RULE>
__device__ __forceinline__ void slice_f32x4(uint32_t bytes, float* f) {
  if constexpr (RULE == kRuleExtra && R < 8) {
    uint32_t lo, hi;
    slice_pairs<R, RULE>(bytes, lo, hi);
    f[0] = (float)(lo & 0xFFFFu);
    f[1] = (float)(lo >> 16);
    f[2] = (float)(hi & 0xFFFFu);
    f[3] = (float)(hi >> 16);
  } else {
    const uint32_t v = slice_bytes<R, RULE>(bytes);
    f[0] = (float)(v & 0xFFu);
    f[1] = (float)((v >> 8) & 0xFFu);
    f[2] = (float)((v >> 16) & 0xFFu);
    f[3] = (float)(v >> 24);
  }
}

// centring offset delta_r = (2^(8-r) - 1) / 2 of the true-prefix rule
__host__ __device__ constexpr float prefix_delta(int r) {
  return (float)((1 << (8 - r)) - 1) * 0.5f;
}

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Round-to-nearest-even fp32 -> bf16 for finite values.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Weight planes are streamed: every byte is read once per call, so their
// loads carry the nontemporal hint, which keeps them from displacing reused
// data in the caches (measured on plain 4 KB-row streams of 117 and 235 MB:
// 6.2-6.4 TB/s with the hint against 5.5 without).
typedef uint32_t stream_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t stream_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ stream_u32x4 stream_load16(const uint32_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const stream_u32x4*>(p));
}
__device__ __forceinline__ stream_u32x2 stream_load8(const uint32_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const stream_u32x2*>(p));
}

struct PlanePtrs {
  const uint32_t* p[kPlanes];
};

// word offset of (row, unit) in plane p
__device__ __forceinline__ size_t plane_word(int p, size_t row, size_t unit, size_t units_per_row) {
  return (row * units_per_row + unit) * (size_t)kPlaneBits[p];
}

}  // namespace mq
