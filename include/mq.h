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
 *                v = code * 2^(8-r).  Needs r+1 bits per weight (r < 8);
 *                at plane granularity it reads the planes that cover them:
 *                3, 4, 6 and 8 bits at r = 2, 3, 4 and 6.
 *   MQ_PREFIX -- MatGPTQ true prefix (MatGPTQ App. A.1):
 *                code = q >> (8-r);  v = code * 2^(8-r) + delta_r,
 *                delta_r = (2^(8-r) - 1) / 2 (centre of the cell).
 *                Reads exactly r bits per weight.
 *   MQ_ROUND_EXTRA -- Extra-Precision MatQuant ("Matryoshka Quantization |
 *                Summary", section 7 "Errata": the slice without the clamp):
 *                code = round(q / 2^(8-r)), ties upward, in 0..2^r (2^r + 1
 *                levels); v = code * 2^(8-r), up to 256 (unsigned 234 at r = 2
 *                gives 256).  Reads the same planes as MQ_ROUND.  The pages
 *                give no storage format for the extra bit (they describe it
 *                only as sparse, about 2.05 bits per weight at r = 2); here the
 *                value is rebuilt from the r + 1 bits the planes hold.
 *   At r = 8 every rule is the identity v = q.
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
 * PREFIX r = 2,3,4,6,8 -> P = 1,2,3,4,5; ROUND and ROUND_EXTRA r = 2,3,4,6
 * -> P = 2,3,4,5.
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
 * n * k <= 2^40 (MQ_ESIZE), m >= 0 (m == 0 is a no-op); the layer calls
 * (mq_linear, mq_linear_noalloc, mq_linear_mixed) also need k <= 2^22
 * (MQ_ESIZE).  Every device pointer must be 16-byte aligned.
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
  MQ_ERULE = 8,      /* rule not MQ_PREFIX, MQ_ROUND or MQ_ROUND_EXTRA       */
  MQ_ESIZE = 9       /* a size exceeds what the kernels index (see below)    */
} mq_status;

typedef enum { MQ_F32 = 0, MQ_F16 = 1, MQ_BF16 = 2 } mq_dtype;
typedef enum { MQ_PREFIX = 0, MQ_ROUND = 1, MQ_ROUND_EXTRA = 2 } mq_rule;

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

/* Human-readable name of a status value (static string, never NULL;
 * "MQ_UNKNOWN" for a value that is not an mq_status).  Takes a plain int so
 * that any value may be passed. */
const char* mq_status_str(int32_t s);

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
 * Kernel choice: fp16 x with m <= 4 and bf16 x with m == 1 (k <= 16384)
 * stream the planes with a register GEMV; other m in 2..64 with k % 256 == 0
 * take the skinny MFMA path (weights dequantized straight into MFMA operand
 * registers; not for MQ_ROUND_EXTRA); everything else runs the MFMA GEMM
 * that dequantizes weight tiles into LDS. */
mq_status mq_linear(const void* x, int32_t x_dtype, int32_t m, const mq_packed* w, int32_t r,
                    int32_t rule, int32_t group, const uint16_t* scales, const uint16_t* zeros,
                    void* y, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mq_linear
 * with the split-k workspace taken from a static array in the library
 * instead of a caller argument.  Calls no hipMalloc, hipFree or allocating
 * routine.  The array is MQ_NOALLOC_SCRATCH_BYTES per device, held from the
 * library's load until the process ends; its address is looked up once per
 * device on the first call there.  Returns MQ_ESIZE when the shape needs more
 * split-k workspace than that (mq_linear_workspace_bytes(m, n, k) >
 * MQ_NOALLOC_SCRATCH_BYTES), and MQ_EINVAL when `stream` does not belong to
 * the current device.  Every call on a device shares that device's array:
 * calls that overlap in time on one device (different streams, or different
 * threads on unordered streams) race and must be ordered by the caller.  The
 * array keeps the last call's partial sums; every call overwrites the part it
 * reads.  Results are those of mq_linear with a workspace of
 * MQ_NOALLOC_SCRATCH_BYTES bytes, bit for bit. */
#define MQ_NOALLOC_SCRATCH_BYTES (64u << 20)
mq_status mq_linear_noalloc(const void* x, int32_t x_dtype, int32_t m, const mq_packed* w, int32_t r,
                            int32_t rule, int32_t group, const uint16_t* scales, const uint16_t* zeros, void* y,
                            void* stream);

/* Mix'n'Match ("Matryoshka Quantization | Summary", section 4.3): n_calls
 * layer matrices, each at its own width, issued on one stream and sharing one
 * workspace.  All calls are validated before the first launch; an invalid call
 * returns its status and nothing is launched.  *failed_call (if not NULL)
 * receives the index of the first invalid call, else -1.
 * The list is cut into runs of consecutive calls that are pairwise
 * independent (no call writes memory that another call of the run reads or
 * writes: x, the planes its width needs, scales, zeros, y).  Runs execute in
 * order.  Inside a run, every call that takes the register GEMV (fp16 x with
 * m <= 4, bf16 x with m == 1, k <= 16384) with the same m, rule and dtype
 * joins one launch (up to 32 calls of any width and shape, e.g. the gate, up
 * and down projections of a decode step, or the projections of several
 * Mix'n'Match blocks at their own widths); skinny-path calls (see mq_linear) with the same m,
 * width, rule, dtype and planned workgroup shape join one launch too (up to
 * 8 calls), each keeping its own k split as long as the workspace holds all
 * of them (mq_linear_mixed_workspace_bytes); calls on the MFMA GEMM's prefill
 * tile (m > 128) with the same width, rule and dtype join launches without a k
 * split (up to 32 calls each, the run's calls of that class cut into launches
 * of equal size) when their output tiles of 256 x 256 number at least 224,
 * which fills the GPU without splitting; the other calls run one by one.
 * The results are those of issuing the calls in order, bit for bit, except
 * that a call in a shared GEMM launch gives the result of mq_linear without a
 * workspace (also bit for bit; with a workspace mq_linear may split k, which
 * changes the summation order within the tolerance).  A launch error reports
 * the first call of its launch. */
mq_status mq_linear_mixed(const mq_call* calls, int32_t n_calls, void* workspace,
                          size_t workspace_bytes, int32_t* failed_call, void* stream);

/* Workspace bytes with which mq_linear_mixed gives every call of `calls` the
 * k split it has as a single call, also where several split calls share a
 * launch: the larger of the single-call need and the 256-byte-aligned sum over
 * the calls that take the skinny MFMA path.  Pure, host only (reads the call
 * structs, not the device buffers); invalid entries count as 0. */
size_t mq_linear_mixed_workspace_bytes(const mq_call* calls, int32_t n_calls);

/* Test support (same device functions as the GEMMs).
 * mq_slice_codes: codes_out [n, k] uint8 = the r-bit code (0..2^r - 1; 0..2^r
 * for MQ_ROUND_EXTRA).
 * mq_dequant: w_out [n, k] of dtype out_dtype (F32 exact; F16/BF16 one
 * round-to-nearest-even from the exact value). */
mq_status mq_slice_codes(const mq_packed* w, int32_t r, int32_t rule, uint8_t* codes_out,
                         void* stream);
mq_status mq_dequant(const mq_packed* w, int32_t r, int32_t rule, int32_t group,
                     const uint16_t* scales, const uint16_t* zeros, int32_t out_dtype,
                     void* w_out, void* stream);

/* Parent producer: the nested 8-bit parent of an fp32 weight matrix, without
 * calibration data ("MatGPTQ: Efficient and Accurate Inference over Nested
 * Quantized Models", section 3.2 points 1 and 2; Appendix A.2, Algorithms 1
 * and 2; the Hessian-weighted error propagation of point 3 needs calibration
 * activations and is not part of it).
 *
 *   w       fp32 [n, k] row-major (device), finite, with every group's
 *           (max(0, max w) - min(0, min w)) / 255 below the fp16 maximum.
 *   widths  host array of n_widths (1..5) distinct target widths in
 *           {2, 3, 4, 6, 8}; lambdas: host array of their weights (finite,
 *           >= 0), in the same order.
 *   rule    the slice each width is reconstructed with (mq_rule).
 *   codes   uint8 [n, k] (device), written: the parent codes.
 *   scales, zeros: fp16 bit patterns [n, k/group] (device), written.
 *
 * Scale search (Algorithm 1): per group, candidate i = 0 .. n_grid - 1
 * shrinks the range [min(0, min w), max(0, max w)] by p_i = 1 - i / grid_den
 * (1 <= n_grid <= grid_den, n_grid <= 256) and takes s = fp16((p hi - p lo) /
 * 255) (1 if that is zero) and z = clamp(rint(-p lo / s), 0, 255); every
 * weight is coded to the nearest code clamp(rint(w / s) + z, 0, 255) and the
 * candidate scores sum_j sum_r lambda_r (w_j - s (v_r(q_j) - z))^2.  The
 * candidate with the smallest score (the first on ties) is kept.
 * Code choice (Algorithm 2): per weight, the code q in 0..255 with the
 * smallest sum_r lambda_r (w - s (v_r(q) - z))^2 (the first on ties).
 * Decisions are fp32 comparisons with every operation rounded on its own, in
 * this order: d = w - w_hat, t = lambda_r * (d * d), running sum over the
 * widths in the given order (and, in the search, over the group's weights in
 * index order, widths innermost).  The pages store the error matrix in fp32.
 *
 * Shape rules as for the layer, plus group <= 1024 (MQ_ESHAPE) and n * k <=
 * 2^36 (MQ_ESIZE).  MQ_EINVAL for
 * a bad n_widths, lambda, n_grid or grid_den; MQ_EWIDTH for a width outside
 * {2,3,4,6,8} or repeated.  Two launches on `stream`; no workspace. */
mq_status mq_produce_parent(const float* w, int32_t n, int32_t k, int32_t group, const int32_t* widths,
                            const float* lambdas, int32_t n_widths, int32_t rule, int32_t n_grid,
                            int32_t grid_den, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
