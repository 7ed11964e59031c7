// mq_api.hip -- the C ABI declared in include/mq.h: host-side validation,
// kernel choice, launches.  No memory is allocated; the only state is the
// per-device address of the static scratch array of mq_linear_noalloc.
#include <stdint.h>

#include <atomic>

#include "../../include/mq.h"
#include "mq_kernels.h"

namespace {

using namespace mq;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_width(int r) { return r == 2 || r == 3 || r == 4 || r == 6 || r == 8; }

bool valid_rule(int rule) { return rule == MQ_PREFIX || rule == MQ_ROUND || rule == MQ_ROUND_EXTRA; }

// the kernels' rule constants are the mq_rule values
static_assert(MQ_PREFIX == kRulePrefix && MQ_ROUND == kRuleRound && MQ_ROUND_EXTRA == kRuleExtra, "rule values");

mq_status check_shape(int n, int k) {
  if (n <= 0 || k <= 0) return MQ_EINVAL;
  if (k % 64) return MQ_ESHAPE;
  // 2^40 codes (a 1 TB parent) keeps every per-unit grid far below 2^31 workgroups
  if ((uint64_t)n * (uint64_t)k > (1ull << 40)) return MQ_ESIZE;
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
  if (!valid_rule(rule)) return MQ_ERULE;
  if (!valid_width(r)) return MQ_EWIDTH;
  const int np = planes_needed(r, rule);
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
  // the GEMM addresses a workgroup's 256 activation rows with 32-bit byte offsets
  if (w->k > kMaxLinearK) return MQ_ESIZE;
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
  a.rule = rule;
  a.bf16 = x_dtype == MQ_BF16;
  hipError_t e;
  if (gemv_eligible(m, w->k, a.bf16)) {
    e = launch_gemv_multi(&a, 1, s);
  } else if (skinny_eligible(m, w->k, rule)) {
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

// Does call c write anything that call d reads or writes?  d reads x, the
// planes its width needs, the scales and the zero points, and writes y.
bool writes_into(const mq_call& c, const mq_call& d) {
  const size_t yc = y_bytes(c);
  if (overlaps(c.y, yc, d.x, x_bytes(d)) || overlaps(c.y, yc, d.y, y_bytes(d))) return true;
  const size_t sz = (size_t)d.w->n * (size_t)(d.w->k / d.group) * 2;
  if (overlaps(c.y, yc, d.scales, sz) || overlaps(c.y, yc, d.zeros, sz)) return true;
  const int np = planes_needed(d.r, d.rule);
  for (int p = 0; p < np; ++p)
    if (overlaps(c.y, yc, d.w->plane[p], (size_t)d.w->n * (size_t)d.w->k * kPlaneBits[p] / 8)) return true;
  return false;
}

// Calls that neither write what the other reads or writes give the same
// results in any order or at the same time.
bool independent(const mq_call& c, const mq_call& d) { return !writes_into(c, d) && !writes_into(d, c); }

// The launch class of a GEMV-eligible call: calls of one class (any width
// and shape) can share a GEMV launch.
bool same_gemv_class(const mq_call& c, const mq_call& d) {
  return c.m == d.m && c.rule == d.rule && c.x_dtype == d.x_dtype;
}
bool gemv_call(const mq_call& c) { return c.m > 0 && gemv_eligible(c.m, c.w->k, c.x_dtype == MQ_BF16); }
bool skinny_call(const mq_call& c) { return c.m > 0 && !gemv_call(c) && skinny_eligible(c.m, c.w->k, c.rule); }

LinearArgs call_args(const mq_call& c, const PlanePtrs& pl) {
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
  a.rule = c.rule;
  a.bf16 = c.x_dtype == MQ_BF16;
  return a;
}

PlanePtrs planes_of(const mq_call& c) {
  PlanePtrs pl;
  for (int p = 0; p < MQ_NPLANES; ++p) pl.p[p] = static_cast<const uint32_t*>(c.w->plane[p]);
  return pl;
}

// calls looked at together when forming launches
constexpr int kWindow = 256;

// ---------------------------------------------------------------------------
// Scratch for mq_linear_noalloc: the split-k partial sums of callers that
// cannot allocate.  Every device the library runs on holds its own copy until
// the process ends.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[MQ_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on device dev, which must be the current device.
mq_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MQ_EINVAL;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MQ_EHIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MQ_OK;
}

}  // namespace

extern "C" {

const char* mq_status_str(int32_t s) {
  switch (s) {
    case MQ_OK: return "MQ_OK";
    case MQ_EINVAL: return "MQ_EINVAL: null pointer or invalid size";
    case MQ_EWIDTH: return "MQ_EWIDTH: width must be 2, 3, 4, 6 or 8";
    case MQ_ESHAPE: return "MQ_ESHAPE: k % 64, group % 64, k % group or packed shape mismatch";
    case MQ_EALIGN: return "MQ_EALIGN: device pointer not 16-byte aligned";
    case MQ_ENOPLANE: return "MQ_ENOPLANE: a plane needed by (width, rule) is NULL";
    case MQ_EDTYPE: return "MQ_EDTYPE: unsupported dtype";
    case MQ_EHIP: return "MQ_EHIP: kernel launch failed";
    case MQ_ERULE: return "MQ_ERULE: rule must be MQ_PREFIX, MQ_ROUND or MQ_ROUND_EXTRA";
    case MQ_ESIZE: return "MQ_ESIZE: size out of range";
  }
  return "MQ_UNKNOWN";
}

size_t mq_plane_bytes(int32_t n, int32_t k, int32_t plane) {
  if (plane < 0 || plane >= MQ_NPLANES || check_shape(n, k) != MQ_OK) return 0;
  return (size_t)n * (size_t)k * (size_t)kPlaneBits[plane] / 8;
}

int32_t mq_planes_needed(int32_t r, int32_t rule) {
  if (!valid_width(r) || !valid_rule(rule)) return -1;
  return planes_needed(r, rule);
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
  // the unclamped rule takes the GEMM at these m as well: size for either
  if (skinny_shape(m, k)) {
    const size_t a = skinny_workspace_bytes(m, n, k), b = gemm_workspace_bytes(m, n, k);
    return a > b ? a : b;
  }
  return gemm_workspace_bytes(m, n, k);
}

size_t mq_linear_mixed_workspace_bytes(const mq_call* calls, int32_t n_calls) {
  if (!calls || n_calls <= 0) return 0;
  size_t single = 0, skinny_sum = 0;
  for (int32_t i = 0; i < n_calls; ++i) {
    const mq_call& c = calls[i];
    if (!c.w || c.m <= 0 || c.w->n <= 0 || c.w->k <= 0 || c.group <= 0 || !valid_width(c.r) || !valid_rule(c.rule))
      continue;
    const size_t one = mq_linear_workspace_bytes(c.m, c.w->n, c.w->k);
    if (one > single) single = one;
    if (skinny_call(c)) skinny_sum = ws_align(skinny_sum) + skinny_call_workspace(call_args(c, planes_of(c)));
  }
  return single > skinny_sum ? single : skinny_sum;
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

mq_status mq_linear_noalloc(const void* x, int32_t x_dtype, int32_t m, const mq_packed* w, int32_t r,
                            int32_t rule, int32_t group, const uint16_t* scales, const uint16_t* zeros, void* y,
                            void* stream) {
  PlanePtrs pl;
  mq_status st = validate_linear(x, x_dtype, m, w, r, rule, group, scales, zeros, y, &pl);
  if (st != MQ_OK) return st;
  if (m == 0) return MQ_OK;
  if (mq_linear_workspace_bytes(m, w->n, w->k) > (size_t)MQ_NOALLOC_SCRATCH_BYTES) return MQ_ESIZE;
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MQ_EHIP;
  if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return MQ_EHIP;
  if (sdev != dev) return MQ_EINVAL;
  void* ws = nullptr;
  st = scratch_on(dev, &ws);
  if (st != MQ_OK) return st;
  return run_linear(x, x_dtype, m, w, r, rule, group, scales, zeros, y, ws, (size_t)MQ_NOALLOC_SCRATCH_BYTES, pl,
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
  // Runs of consecutive, pairwise independent calls: inside a run the order
  // does not matter, so every GEMV-eligible call of one class (m, rule,
  // dtype) goes into one launch, whatever its width and shape, skinny calls of
  // one launch shape share launches, and the other calls run one by one.
  // Runs follow each other in stream order.
  for (int32_t i = 0; i < n_calls;) {
    int32_t j = i + 1;
    while (j < n_calls && j - i < kWindow) {
      bool ok = true;
      for (int32_t t = i; t < j && ok; ++t) ok = independent(calls[t], calls[j]);
      if (!ok) break;
      ++j;
    }
    bool done[kWindow] = {};
    for (int32_t t = i; t < j; ++t) {
      if (done[t - i]) continue;
      const mq_call& c = calls[t];
      mq_status st;
      if (gemv_call(c)) {
        LinearArgs la[kGemvMaxCalls];
        int nl = 0;
        for (int32_t u = t; u < j && nl < kGemvMaxCalls; ++u) {
          if (done[u - i] || !gemv_call(calls[u]) || !same_gemv_class(c, calls[u])) continue;
          la[nl++] = call_args(calls[u], planes_of(calls[u]));
          done[u - i] = true;
        }
        st = launch_gemv_multi(la, nl, static_cast<hipStream_t>(stream)) == hipSuccess ? MQ_OK : MQ_EHIP;
      } else if (skinny_call(c)) {
        // skinny calls of one launch shape share a launch; a call with a k
        // split joins only where its part of the workspace fits (or where it
        // would not fit even alone), so every call keeps the plan it has as a
        // single call and the results are those of single calls
        const bool ws_ok = workspace && aligned16(workspace);
        const size_t ws_b = ws_ok ? workspace_bytes : 0;
        LinearArgs la[kSkinnyMaxCalls];
        const LinearArgs a0 = call_args(c, planes_of(c));
        int nl = 0;
        size_t used = 0;
        for (int32_t u = t; u < j && nl < kSkinnyMaxCalls; ++u) {
          if (done[u - i] || !skinny_call(calls[u])) continue;
          const LinearArgs au = call_args(calls[u], planes_of(calls[u]));
          if (!same_skinny_launch(a0, au)) continue;
          const size_t need = skinny_call_workspace(au);
          if (need && need <= ws_b) {
            if (ws_align(used) + need > ws_b) continue;  // joins a later launch
            used = ws_align(used) + need;
          }
          la[nl++] = au;
          done[u - i] = true;
        }
        st = launch_skinny_multi(la, nl, ws_ok ? workspace : nullptr, ws_b, static_cast<hipStream_t>(stream)) ==
                     hipSuccess
                 ? MQ_OK
                 : MQ_EHIP;
      } else {
        // prefill-tile calls of one width, rule and dtype share a launch
        // without a k split when their tiles together fill the GPU; any
        // other call runs alone (split over k where the workspace allows)
        const LinearArgs a0 = call_args(c, planes_of(c));
        LinearArgs la[kGemmMaxCalls];
        int32_t idx[kGemmMaxCalls];
        int nl = 0, tiles = 0;
        if (gemm_batchable(a0)) {
          // the class's calls in this run, cut into launches of equal size
          int cnt = 0;
          for (int32_t u = t; u < j; ++u)
            if (!done[u - i] && !gemv_call(calls[u]) && !skinny_call(calls[u]) &&
                same_gemm_launch(a0, call_args(calls[u], planes_of(calls[u]))))
              ++cnt;
          const int nlaunch = (cnt + kGemmMaxCalls - 1) / kGemmMaxCalls;
          const int per = (cnt + nlaunch - 1) / (nlaunch > 0 ? nlaunch : 1);
          for (int32_t u = t; u < j && nl < per; ++u) {
            if (done[u - i] || gemv_call(calls[u]) || skinny_call(calls[u])) continue;
            const LinearArgs au = call_args(calls[u], planes_of(calls[u]));
            if (!same_gemm_launch(a0, au)) continue;
            idx[nl] = u;
            la[nl++] = au;
            tiles += gemm_tiles(au);
          }
        }
        if (nl >= 2 && tiles >= kGemmBatchMinTiles) {
          for (int q = 0; q < nl; ++q) done[idx[q] - i] = true;
          st = launch_gemm_multi(la, nl, static_cast<hipStream_t>(stream)) == hipSuccess ? MQ_OK : MQ_EHIP;
        } else {
          done[t - i] = true;
          st = run_linear(c.x, c.x_dtype, c.m, c.w, c.r, c.rule, c.group, c.scales, c.zeros, c.y, workspace,
                          workspace_bytes, planes_of(c), static_cast<hipStream_t>(stream));
        }
      }
      if (st != MQ_OK) {
        if (failed_call) *failed_call = t;
        return st;
      }
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
  return launch_slice(pl, w->n, w->k, r, rule, codes_out, static_cast<hipStream_t>(stream)) == hipSuccess
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
  return launch_dequant(pl, w->n, w->k, r, rule, group, scales, zeros, out_dtype, w_out,
                        static_cast<hipStream_t>(stream)) == hipSuccess
             ? MQ_OK
             : MQ_EHIP;
}

mq_status mq_produce_parent(const float* w, int32_t n, int32_t k, int32_t group, const int32_t* widths,
                            const float* lambdas, int32_t n_widths, int32_t rule, int32_t n_grid, int32_t grid_den,
                            uint8_t* codes, uint16_t* scales, uint16_t* zeros, void* stream) {
  if (!w || !codes || !scales || !zeros || !widths || !lambdas) return MQ_EINVAL;
  mq_status st = check_shape(n, k);
  if (st != MQ_OK) return st;
  st = check_group(k, group);
  if (st != MQ_OK) return st;
  if (group > kMaxProduceGroup) return MQ_ESHAPE;
  if ((uint64_t)n * (uint64_t)k > (1ull << 36)) return MQ_ESIZE;  // keeps every grid below 2^31 workgroups
  if (!valid_rule(rule)) return MQ_ERULE;
  if (n_widths < 1 || n_widths > kMaxProduceWidths) return MQ_EINVAL;
  for (int i = 0; i < n_widths; ++i) {
    if (!valid_width(widths[i])) return MQ_EWIDTH;
    for (int j = 0; j < i; ++j)
      if (widths[j] == widths[i]) return MQ_EWIDTH;
    const float l = lambdas[i];
    if (!(l >= 0.0f) || !(l <= 3.0e38f)) return MQ_EINVAL;  // finite, not negative, not NaN
  }
  if (grid_den < 1 || n_grid < 1 || n_grid > grid_den || n_grid > kMaxProduceGrid) return MQ_EINVAL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned16(zeros)) return MQ_EALIGN;
  int wv[kMaxProduceWidths];
  for (int i = 0; i < n_widths; ++i) wv[i] = widths[i];
  return launch_produce(w, n, k, group, wv, lambdas, n_widths, rule, n_grid, grid_den, codes, scales, zeros,
                        static_cast<hipStream_t>(stream)) == hipSuccess
             ? MQ_OK
             : MQ_EHIP;
}

}  // extern "C"
