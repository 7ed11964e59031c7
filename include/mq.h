/*
 * mq.h -- C ABI of libmq, the sliced-precision quantized linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 *   Y = X . dequant(slice_r(Q_c))^T
 *
 * One unsigned c = 8-bit parent code tensor Q_c [n, k] with one fp16 scale s
 * and one integer-valued fp16 zero point z per group of `group` consecutive
 * input (k) indices of an output row serves every width r in {2, 3, 4, 6, 8}
 * by taking the most significant bits of each code.  The scale and zero point
 * are shared by all widths ("Matryoshka Quantization | Summary", section 3.2
 * "MatQuant"; "MatGPTQ: Efficient and Accurate Inference over Nested
 * Quantized Models", section 1 and section 3.2).
 *
 * Slicing rules (MQ_RULE):
 *   MQ_ROUND  -- MatQuant (summary page, section 3.2; MatGPTQ App. A.1):
 *                code = clamp(round(q / 2^(8-r)), 0, 2^r - 1), ties upward
 *                (the (r+1)-th most significant bit decides);
 *                v = code * 2^(8-r).  Reads r+1 bits per weight (r < 8).
 *   MQ_PREFIX -- MatGPTQ true prefix (MatGPTQ App. A.1):
 *                code = q >> (8-r);  v = code * 2^(8-r) + delta_r,
 *                delta_r = (2^(8-r) - 1) / 2 (centre of the cell).
 *                Reads exactly r bits per weight.
 *   At r = 8 both rules are the identity v = q.
 * Dequantization: w_hat = s * (v - z).  With an fp16 scale and an integer
 * zero point this is exact in fp32.
 *
 * Bit planes (MatGPTQ section 4 "Fast Matryoshka Kernels": five buffers with
 * bits 1-2, 3, 4, 5-6 and 7-8 counted from the most significant bit):
 *   plane 0: code bits 7..6   (2 bits/weight)
 *   plane 1: code bit  5      (1 bit/weight)
 *   plane 2: code bit  4      (1 bit/weight)
 *   plane 3: code bits 3..2   (2 bits/weight)
 *   plane 4: code bits 1..0   (2 bits/weight)
 * A width-r call reads planes 0..P-1 only, P = mq_planes_needed(r, rule):
 * PREFIX r = 2,3,4,6,8 -> P = 1,2,3,4,5; ROUND r = 2,3,4,6 -> P = 2,3,4,5.
 * Each plane is a row-major [n][k/32] array of 32-code units (8 bytes for a
 * 2-bit plane, 4 bytes for a 1-bit plane).  Inside a unit, the 32 codes'
 * fields are interleaved so that shifting a unit word and masking it yields
 * four consecutive codes' bits already in place inside four bytes (the exact
 * bit positions are an implementation detail; only mq_pack_parent writes
 * them).  A plane that a call does not need may be NULL, so a caller can keep
 * only the first planes resident and pay only for an r-bit footprint.
 *
 * Layouts and types of the other operands:
 *   codes   uint8 [n, k] row-major, values 0..255.
 *   scales  fp16 bit patterns [n, k/group] row-major, finite and nonzero.
 *   zeros   fp16 bit patterns [n, k/group] row-major, integer values 0..255.
 *   x       [m, k] row-major, MQ_F16 or MQ_BF16.
 *   y       [m, n] row-major, same dtype as x; overwritten, not accumulated.
 *
 * Shape rules: n >= 1, k >= 64, k % 64 == 0, group % 64 == 0, k % group == 0,
 * m >= 0 (m == 0 is a no-op).  Every device pointer must be 16-byte aligned.
 *
 * Ownership and threading: the caller allocates and owns every buffer,
 * including the optional split-K workspace of mq_linear.  The library
 * allocates no memory, keeps no global state and is thread-safe.  `stream` is
 * a hipStream_t (NULL = the default stream); every call is asynchronous and
 * stream-ordered.  Results are bitwise deterministic for identical inputs and
 * identical workspace sizes.
 *
 * Errors: every argument is validated on the host before any HIP call; on a
 * failed check the call returns the status and launches nothing.  MQ_EHIP is
 * returned when a launch reports an error (hipGetLastError).  Device faults
 * are asynchronous and surface at the caller's next synchronisation.  The
 * library never prints, aborts or throws.
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MQ_OK = 0,
  MQ_EINVAL = 1,     /* null pointer, negative or zero size, m < 0          */
  MQ_EWIDTH = 2,     /* r not in {2,3,4,6,8}                                 */
  MQ_ESHAPE = 3,     /* k % 64, group % 64, k % group, packed n/k mismatch   */
  MQ_EALIGN = 4,     /* a device pointer is not 16-byte aligned              */
  MQ_ENOPLANE = 5,   /* a plane that (r, rule) needs is NULL                 */
  MQ_EDTYPE = 6,     /* dtype not allowed for this argument                  */
  MQ_EHIP = 7,       /* a kernel launch failed                               */
  MQ_ERULE = 8,      /* rule not MQ_PREFIX or MQ_ROUND                       */
  MQ_ESIZE = 9       /* a size exceeds what the kernels index (see below)    */
} mq_status;

typedef enum { MQ_F32 = 0, MQ_F16 = 1, MQ_BF16 = 2 } mq_dtype;
typedef enum { MQ_PREFIX = 0, MQ_ROUND = 1 } mq_rule;

#define MQ_NPLANES 5

/* A packed parent: the shape of Q_c and five device plane pointers.  The
 * struct itself lives in host memory; plane[p] may be NULL when the plane is
 * not resident. */
typedef struct {
  int32_t n, k;
  void* plane[MQ_NPLANES];
} mq_packed;

/* One layer-matrix call of mq_linear_mixed (host memory). */
typedef struct {
  const void* x;
  int32_t x_dtype;           /* mq_dtype */
  int32_t m;
  const mq_packed* w;
  int32_t r;
  int32_t rule;              /* mq_rule */
  int32_t group;
  const uint16_t* scales;
  const uint16_t* zeros;
  void* y;
} mq_call;

/* Human-readable name of a status (static string, never NULL). */
const char* mq_status_str(mq_status s);

/* Bytes of plane `plane` (0..4) for an [n, k] parent: n*k*bits/8, with
 * bits = 2,1,1,2,2.  Returns 0 for an invalid plane index or shape.  Pure,
 * host only. */
size_t mq_plane_bytes(int32_t n, int32_t k, int32_t plane);

/* Number of leading planes that a width-r call with `rule` reads, or -1 if
 * (r, rule) is invalid.  Pure, host only. */
int32_t mq_planes_needed(int32_t r, int32_t rule);

/* Pack: codes [n, k] (device) -> out->plane[0..4] (device, caller-allocated,
 * mq_plane_bytes each; all five must be non-NULL).  out->n/out->k must equal
 * n/k.  One pass over the codes (MatGPTQ section 1 contribution 3 "efficient
 * packing"; section 4, plane split done offline). */
mq_status mq_pack_parent(const uint8_t* codes, int32_t n, int32_t k, const mq_packed* out,
                         void* stream);

/* Workspace bytes that let mq_linear split the k reduction across
 * workgroups for this shape (0 when it never splits).  Pure, host only. */
size_t mq_linear_workspace_bytes(int32_t m, int32_t n, int32_t k);

/* The layer: y[m, n] = sum_k x[m, k] * w_hat[n, k] with w_hat the width-r
 * slice of `w` under `rule`, fp32 accumulation, result rounded once to the
 * dtype of x (MatGPTQ section 4: fp16/bf16 inputs, fp32 accumulation; the
 * nn.Linear orientation).  `workspace` (device, may be NULL) of
 * `workspace_bytes` lets the dispatcher split k for shapes with few output
 * tiles; with less than mq_linear_workspace_bytes() it does not split.
 * Kernel choice: m <= 4 streams the planes with a register GEMV; larger m runs
 * the MFMA GEMM that dequantizes weight tiles into LDS. */
mq_status mq_linear(const void* x, int32_t x_dtype, int32_t m, const mq_packed* w, int32_t r,
                    int32_t rule, int32_t group, const uint16_t* scales, const uint16_t* zeros,
                    void* y, void* workspace, size_t workspace_bytes, void* stream);

/* Mix'n'Match ("Matryoshka Quantization | Summary", section 4.3): n_calls
 * layer matrices, each at its own width, issued in order on one stream and
 * sharing one workspace.  All calls are validated before the first launch; an
 * invalid call returns its status and nothing is launched.  *failed_call (if
 * not NULL) receives the index of the first invalid call, else -1.
 * Consecutive calls that take the register GEMV with the same m, k, width,
 * rule, group and dtype, and whose outputs overlap neither each other nor the
 * others' inputs, run in one launch (up to 4 calls; e.g. the gate and up
 * projections of a decode step).  The results are those of issuing the calls
 * in order; a launch error reports the first call of its launch. */
mq_status mq_linear_mixed(const mq_call* calls, int32_t n_calls, void* workspace,
                          size_t workspace_bytes, int32_t* failed_call, void* stream);

/* Test support (same device functions as the GEMMs).
 * mq_slice_codes: codes_out [n, k] uint8 = the r-bit code (0..2^r - 1).
 * mq_dequant: w_out [n, k] of dtype out_dtype (F32 exact; F16/BF16 one
 * round-to-nearest-even from the exact value). */
mq_status mq_slice_codes(const mq_packed* w, int32_t r, int32_t rule, uint8_t* codes_out,
                         void* stream);
mq_status mq_dequant(const mq_packed* w, int32_t r, int32_t rule, int32_t group,
                     const uint16_t* scales, const uint16_t* zeros, int32_t out_dtype,
                     void* w_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
