// mq_api.hip -- the C ABI declared in include/mq.h: host-side validation,
// kernel choice, launches.  No memory is allocated and no state is kept.
#include <stdint.h>

#include "../../include/mq.h"
#include "mq_kernels.h"

namespace {

using namespace mq;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_width(int r) { return r == 2 || r == 3 || r == 4 || r == 6 || r == 8; }

mq_status check_shape(int n, int k) {
  if (n <= 0 || k <= 0) return MQ_EINVAL;
  if (k % 64) return MQ_ESHAPE;
  return MQ_OK;
}

mq_status check_group(int k, int group) {
  if (group <= 0) return MQ_ESHAPE;
  if (group % 64 || k % group) return MQ_ESHAPE;
  return MQ_OK;
}

// validate the packed parent for a width-r call and collect its plane pointers
mq_status check_packed(const mq_packed* w, int r, int rule, PlanePtrs* out) {
  if (!w) return MQ_EINVAL;
  mq_status st = check_shape(w->n, w->k);
  if (st != MQ_OK) return st;
  if (rule != MQ_PREFIX && rule != MQ_ROUND) return MQ_ERULE;
  if (!valid_width(r)) return MQ_EWIDTH;
  const int np = planes_needed(r, rule == MQ_ROUND);
  for (int p = 0; p < MQ_NPLANES; ++p) {
    out->p[p] = static_cast<const uint32_t*>(w->plane[p]);
    if (p < np) {
      if (!w->plane[p]) return MQ_ENOPLANE;
      if (!aligned16(w->plane[p])) return MQ_EALIGN;
    }
  }
  return MQ_OK;
}

mq_status check_scales(const mq_packed* w, int group, const uint16_t* scales, const uint16_t* zeros) {
  mq_status st = check_group(w->k, group);
  if (st != MQ_OK) return st;
  if (!scales || !zeros) return MQ_EINVAL;
  if (!aligned16(scales) || !aligned16(zeros)) return MQ_EALIGN;
  return MQ_OK;
}

mq_status validate_linear(const void* x, int x_dtype, int m, const mq_packed* w, int r, int rule, int group,
                          const uint16_t* scales, const uint16_t* zeros, void* y, PlanePtrs* pl) {
  if (m < 0) return MQ_EINVAL;
  mq_status st = check_packed(w, r, rule, pl);
  if (st != MQ_OK) return st;
  st = check_scales(w, group, scales, zeros);
  if (st != MQ_OK) return st;
  if (x_dtype != MQ_F16 && x_dtype != MQ_BF16) return MQ_EDTYPE;
  if (m == 0) return MQ_OK;
  if (!x || !y) return MQ_EINVAL;
  if (!aligned16(x) || !aligned16(y)) return MQ_EALIGN;
  // kernels index with 64-bit offsets; keep grid dimensions in range
  if ((long long)m * (long long)w->n > (1LL << 46) || (long long)w->n * (long long)w->k > (1LL << 46))
    return MQ_ESIZE;
  return MQ_OK;
}

mq_status run_linear(const void* x, int x_dtype, int m, const mq_packed* w, int r, int rule, int group,
                     const uint16_t* scales, const uint16_t* zeros, void* y, void* workspace,
                     size_t workspace_bytes, const PlanePtrs& pl, hipStream_t s) {
  if (m == 0) return MQ_OK;
  LinearArgs a;
  a.x = x;
  a.y = y;
  a.pl = pl;
  a.scales = scales;
  a.zeros = zeros;
  a.m = m;
  a.n = w->n;
  a.k = w->k;
  a.group = group;
  a.r = r;
  a.round_rule = rule == MQ_ROUND;
  a.bf16 = x_dtype == MQ_BF16;
  hipError_t e;
  if (gemv_eligible(m, w->k, a.bf16)) {
    e = launch_gemv(a, s);
  } else if (skinny_eligible(m, w->k)) {
    const bool ws_ok = workspace && aligned16(workspace);
    e = launch_skinny(a, ws_ok ? workspace : nullptr, ws_ok ? workspace_bytes : 0, s);
  } else {
    GemmPlan plan = plan_gemm(m, w->n, w->k, workspace ? workspace_bytes : 0);
    if (plan.splits > 1 && !aligned16(workspace)) plan.splits = 1;
    e = launch_gemm(a, plan, workspace, s);
  }
  return e == hipSuccess ? MQ_OK : MQ_EHIP;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

size_t x_bytes(const mq_call& c) { return (size_t)c.m * (size_t)c.w->k * 2; }
size_t y_bytes(const mq_call& c) { return (size_t)c.m * (size_t)c.w->n * 2; }

// May call d join a single GEMV launch with call c (c issued before d)?  They
// must share the shape class of the launch (m, k, width, rule, group, dtype)
// and be independent: neither output may overlap the other call's input or
// output, so running both at once gives what running them in order gives.
bool can_batch(const mq_call& c, const mq_call& d) {
  if (c.m != d.m || c.m == 0 || c.w->k != d.w->k || c.r != d.r || c.rule != d.rule || c.group != d.group ||
      c.x_dtype != d.x_dtype)
    return false;
  if (!gemv_eligible(c.m, c.w->k, c.x_dtype == MQ_BF16)) return false;
  return !overlaps(c.y, y_bytes(c), d.x, x_bytes(d)) && !overlaps(d.y, y_bytes(d), c.x, x_bytes(c)) &&
         !overlaps(c.y, y_bytes(c), d.y, y_bytes(d));
}

LinearArgs gemv_args(const mq_call& c, const PlanePtrs& pl) {
  LinearArgs a;
  a.x = c.x;
  a.y = c.y;
  a.pl = pl;
  a.scales = c.scales;
  a.zeros = c.zeros;
  a.m = c.m;
  a.n = c.w->n;
  a.k = c.w->k;
  a.group = c.group;
  a.r = c.r;
  a.round_rule = c.rule == MQ_ROUND;
  a.bf16 = c.x_dtype == MQ_BF16;
  return a;
}

}  // namespace

extern "C" {

const char* mq_status_str(mq_status s) {
  switch (s) {
    case MQ_OK: return "MQ_OK";
    case MQ_EINVAL: return "MQ_EINVAL: null pointer or invalid size";
    case MQ_EWIDTH: return "MQ_EWIDTH: width must be 2, 3, 4, 6 or 8";
    case MQ_ESHAPE: return "MQ_ESHAPE: k % 64, group % 64, k % group or packed shape mismatch";
    case MQ_EALIGN: return "MQ_EALIGN: device pointer not 16-byte aligned";
    case MQ_ENOPLANE: return "MQ_ENOPLANE: a plane needed by (width, rule) is NULL";
    case MQ_EDTYPE: return "MQ_EDTYPE: unsupported dtype";
    case MQ_EHIP: return "MQ_EHIP: kernel launch failed";
    case MQ_ERULE: return "MQ_ERULE: rule must be MQ_PREFIX or MQ_ROUND";
    case MQ_ESIZE: return "MQ_ESIZE: size out of range";
  }
  return "MQ_UNKNOWN";
}

size_t mq_plane_bytes(int32_t n, int32_t k, int32_t plane) {
  if (plane < 0 || plane >= MQ_NPLANES || check_shape(n, k) != MQ_OK) return 0;
  return (size_t)n * (size_t)k * (size_t)kPlaneBits[plane] / 8;
}

int32_t mq_planes_needed(int32_t r, int32_t rule) {
  if (!valid_width(r) || (rule != MQ_PREFIX && rule != MQ_ROUND)) return -1;
  return planes_needed(r, rule == MQ_ROUND);
}

mq_status mq_pack_parent(const uint8_t* codes, int32_t n, int32_t k, const mq_packed* out, void* stream) {
  if (!codes || !out) return MQ_EINVAL;
  mq_status st = check_shape(n, k);
  if (st != MQ_OK) return st;
  if (out->n != n || out->k != k) return MQ_ESHAPE;
  if (!aligned16(codes)) return MQ_EALIGN;
  uint32_t* planes[MQ_NPLANES];
  for (int p = 0; p < MQ_NPLANES; ++p) {
    if (!out->plane[p]) return MQ_ENOPLANE;
    if (!aligned16(out->plane[p])) return MQ_EALIGN;
    planes[p] = static_cast<uint32_t*>(out->plane[p]);
  }
  return launch_pack(codes, n, k, planes, static_cast<hipStream_t>(stream)) == hipSuccess ? MQ_OK : MQ_EHIP;
}

size_t mq_linear_workspace_bytes(int32_t m, int32_t n, int32_t k) {
  if (check_shape(n, k) != MQ_OK || m <= 0) return 0;
  if (m <= kGemvMaxM && k <= kGemvMaxK && m == 1) return 0;
  // the dtype is not known here: fp16 batches of up to 4 rows take the GEMV
  // (no workspace), bf16 ones the skinny path, so size for the latter
  if (skinny_eligible(m, k)) return skinny_workspace_bytes(m, n, k);
  return gemm_workspace_bytes(m, n, k);
}

mq_status mq_linear(const void* x, int32_t x_dtype, int32_t m, const mq_packed* w, int32_t r, int32_t rule,
                    int32_t group, const uint16_t* scales, const uint16_t* zeros, void* y, void* workspace,
                    size_t workspace_bytes, void* stream) {
  PlanePtrs pl;
  mq_status st = validate_linear(x, x_dtype, m, w, r, rule, group, scales, zeros, y, &pl);
  if (st != MQ_OK) return st;
  return run_linear(x, x_dtype, m, w, r, rule, group, scales, zeros, y, workspace, workspace_bytes, pl,
                    static_cast<hipStream_t>(stream));
}

mq_status mq_linear_mixed(const mq_call* calls, int32_t n_calls, void* workspace, size_t workspace_bytes,
                          int32_t* failed_call, void* stream) {
  if (failed_call) *failed_call = -1;
  if (n_calls < 0 || (n_calls > 0 && !calls)) return MQ_EINVAL;
  for (int32_t i = 0; i < n_calls; ++i) {
    const mq_call& c = calls[i];
    PlanePtrs pl;
    mq_status st = validate_linear(c.x, c.x_dtype, c.m, c.w, c.r, c.rule, c.group, c.scales, c.zeros, c.y, &pl);
    if (st != MQ_OK) {
      if (failed_call) *failed_call = i;
      return st;
    }
  }
  for (int32_t i = 0; i < n_calls;) {
    const mq_call& c = calls[i];
    PlanePtrs pl;
    validate_linear(c.x, c.x_dtype, c.m, c.w, c.r, c.rule, c.group, c.scales, c.zeros, c.y, &pl);
    // consecutive independent GEMV calls of one shape class share a launch
    int32_t j = i + 1;
    while (j < n_calls && j - i < kGemvMaxBatch) {
      bool ok = true;
      for (int32_t t = i; t < j && ok; ++t) ok = can_batch(calls[t], calls[j]);
      if (!ok) break;
      ++j;
    }
    mq_status st;
    if (j - i > 1) {
      LinearArgs la[kGemvMaxBatch];
      for (int32_t t = i; t < j; ++t) {
        PlanePtrs plt;
        const mq_call& ct = calls[t];
        validate_linear(ct.x, ct.x_dtype, ct.m, ct.w, ct.r, ct.rule, ct.group, ct.scales, ct.zeros, ct.y, &plt);
        la[t - i] = gemv_args(ct, plt);
      }
      st = launch_gemv_batch(la, j - i, static_cast<hipStream_t>(stream)) == hipSuccess ? MQ_OK : MQ_EHIP;
    } else {
      st = run_linear(c.x, c.x_dtype, c.m, c.w, c.r, c.rule, c.group, c.scales, c.zeros, c.y, workspace,
                      workspace_bytes, pl, static_cast<hipStream_t>(stream));
    }
    if (st != MQ_OK) {
      if (failed_call) *failed_call = i;
      return st;
    }
    i = j;
  }
  return MQ_OK;
}

mq_status mq_slice_codes(const mq_packed* w, int32_t r, int32_t rule, uint8_t* codes_out, void* stream) {
  PlanePtrs pl;
  mq_status st = check_packed(w, r, rule, &pl);
  if (st != MQ_OK) return st;
  if (!codes_out) return MQ_EINVAL;
  if (!aligned16(codes_out)) return MQ_EALIGN;
  return launch_slice(pl, w->n, w->k, r, rule == MQ_ROUND, codes_out, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MQ_OK
             : MQ_EHIP;
}

mq_status mq_dequant(const mq_packed* w, int32_t r, int32_t rule, int32_t group, const uint16_t* scales,
                     const uint16_t* zeros, int32_t out_dtype, void* w_out, void* stream) {
  PlanePtrs pl;
  mq_status st = check_packed(w, r, rule, &pl);
  if (st != MQ_OK) return st;
  st = check_scales(w, group, scales, zeros);
  if (st != MQ_OK) return st;
  if (out_dtype != MQ_F32 && out_dtype != MQ_F16 && out_dtype != MQ_BF16) return MQ_EDTYPE;
  if (!w_out) return MQ_EINVAL;
  if (!aligned16(w_out)) return MQ_EALIGN;
  return launch_dequant(pl, w->n, w->k, r, rule == MQ_ROUND, group, scales, zeros, out_dtype, w_out,
                        static_cast<hipStream_t>(stream)) == hipSuccess
             ? MQ_OK
             : MQ_EHIP;
}

}  // extern "C"
