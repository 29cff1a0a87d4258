/*
 * qlinear.h -- C ABI of the group-wise weight-only quantized linear layer
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 *   y[m, n] = sum_k x[m, k] * w[n, k]  (+ bias[n])        (y = x W^T)
 * where W [N, K] is stored quantized in one of four formats and w is its
 * dequantized value.  The formats and their dequantization rules:
 *
 *   QP_FMT_AFFINE  MLX-style group affine codes (HF Transformers "Metal"
 *                  quantization page: weights packed into uint32 tensors with
 *                  per-group scales and biases, bits 2/4/8, group size default
 *                  64, fused dequantize + matmul "affine_qmm_t"):
 *                      w = q * scale + bias,  q unsigned b-bit.
 *   QP_FMT_Q4K     Q4_K-style nested "superscale" int4 (ExecuTorch PR #20571,
 *                  "Quant schema update", int4 bullet): group 32, super-block
 *                  256; scale = uint8 code * fp16 step, zero = uint8 code *
 *                  fp16 step, the two steps of a super-block packed in one
 *                  32-bit word; 4.625 bits per weight:
 *                      w = (q - zc*zstep) * (sc*sstep),  q in [0, 15].
 *   QP_FMT_Q6K     Q6_K-style symmetric int6 (same page, int6 bullet): group
 *                  16, super-block 256, scale = int8 code * fp16 step, no
 *                  zero; 6.5625 bits per weight:
 *                      w = q * (sc*step),  q in [-32, 31], sc in [0, 127].
 *   QP_FMT_SYM4    symmetric int4 in an int8 carrier, qmin = -7, qmax = 7
 *                  (ExecuTorch PR #16577, description), fp32 scale per output
 *                  channel (group_size = K) or per group:
 *                      w = q * scale.
 *
 * Quantization rules (qpack_quantize) -- per group along K of each row, every
 * step one IEEE fp32 operation, codes rounded half-to-even and clamped:
 *   AFFINE: lo = min w, hi = max w; scale = meta(fl32(fl32(hi-lo)/(2^b-1)));
 *           bias = meta(lo); q = scale == 0 ? 0 :
 *           clamp(rint(fl32(fl32(w - bias)/scale)), 0, 2^b-1), using the
 *           stored (meta-rounded) scale and bias.
 *   Q4K:    lo = min(min w, 0), hi = max(max w, 0); s = fl32(fl32(hi-lo)/15);
 *           z = fl32(-lo/s); q = clamp(rint(fl32(fl32(w-lo)/s)), 0, 15)
 *           (s == 0 -> q = z = 0).  Then per super-block of 256:
 *           sstep = fp16(fl32(max s / 255)), sc = clamp(rint(fl32(s/sstep)),
 *           0, 255) (0 if sstep == 0); zstep, zc likewise from z.
 *   Q6K:    s = fl32(max|w| / 31); q = clamp(rint(fl32(w/s)), -32, 31);
 *           step = fp16(fl32(max s / 127)), sc = clamp(rint(fl32(s/step)),
 *           0, 127).
 *   SYM4:   s = fl32(max|w| / 7) (fp32, stored); q = clamp(rint(fl32(w/s)),
 *           -7, 7).
 *   fp16 conversions keep subnormals (the nested steps usually are).
 *
 * Storage (all buffers row-major, N leading, caller-owned device memory):
 *   qweight     uint32 [N, K*b/32]: code k of a row at word k/(32/b), bits
 *               [b*(k % (32/b)), +b) -- least-significant first along K.
 *               SYM4 stores u = q + 8.  Q6K: low nibble of u = q + 32,
 *               [N, K/8].
 *   qweight_hi  Q6K only: high 2 bits of u = q + 32, uint32 [N, K/16], same
 *               bit order.  NULL otherwise.
 *   scales      AFFINE: fp16|bf16 [N, K/gs];  Q4K: uint8 [N, K/32];
 *               Q6K: int8 [N, K/16];  SYM4: fp32 [N, K/gs].
 *   zeros       AFFINE: biases fp16|bf16 [N, K/gs];  Q4K: uint8 zero codes
 *               [N, K/32];  NULL otherwise.
 *   steps       Q4K: uint32 [N, K/256], low 16 bits = fp16 scale step, high
 *               16 bits = fp16 zero step;  Q6K: fp16 [N, K/256];  NULL
 *               otherwise.
 *
 * Conventions for every entry point
 * ---------------------------------
 *   * Pointers to weights, activations and outputs are device pointers and
 *     must be 16-byte aligned; the caller owns every buffer; the library
 *     keeps no state between calls apart from the per-thread error message.
 *   * Buffers are read in 16-byte units: each input buffer (weights, bias,
 *     activations) must be allocated up to the next multiple of 16 bytes of
 *     its size (hipMalloc and torch allocations always are).  Only the
 *     bytes of the stated size are used.
 *   * `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; a status other than QP_OK means that nothing
 *     was enqueued and qpack_last_error() names the reason.
 *   * Validation happens on the host before any launch: shape divisibility
 *     (K % group_size, whole 16-byte chunks of codes along K, K % 256 for the
 *     nested formats), supported (fmt, bits, group_size, dtype) combinations,
 *     alignment, N, K, M > 0.
 *   * Inputs must be finite; non-finite weights or activations give
 *     unspecified results.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QP_ABI_VERSION 1

typedef enum {
  QP_OK = 0,
  QP_EINVAL = 1,        /* NULL descriptor/pointer, bad enum value          */
  QP_ESHAPE = 2,        /* N, K, M or group sizes that do not tile          */
  QP_EUNSUPPORTED = 3,  /* valid but not implemented combination           */
  QP_EALIGN = 4,        /* a pointer is not 16-byte aligned                 */
  QP_EHIP = 5           /* the HIP runtime reported an error at launch      */
} qp_status;

typedef enum {
  QP_FMT_AFFINE = 0,
  QP_FMT_Q4K = 1,
  QP_FMT_Q6K = 2,
  QP_FMT_SYM4 = 3
} qp_format;

typedef enum { QP_F16 = 0, QP_BF16 = 1, QP_F32 = 2 } qp_dtype;

/* Which kernel family qlinear_forward_kernel uses. */
typedef enum {
  QP_KERNEL_AUTO = 0,      /* M <= 8: qGEMV; from M = 2 (per-channel SYM4,
                              4-bit AFFINE), 5 (8-bit AFFINE) or 3 (other formats)
                              up to M = 16: MFMA qGEMV when K % 128 == 0;
                              larger M: qGEMM up to
                              K = 8192 (per-channel SYM4: 2^20), the MFMA
                              qGEMV beyond                                    */
  QP_KERNEL_GEMV = 1,      /* decode-shaped kernel, any M (processed 8 at once) */
  QP_KERNEL_GEMM = 2,      /* prefill-shaped MFMA kernel, any M; fp16-rounded
                              weights, so K % 64 == 0 and K <= 8192, where it
                              meets the output bound; per-channel SYM4 runs
                              on exact codes, K <= 2^20                       */
  QP_KERNEL_GEMV_MFMA = 3  /* MFMA qGEMV on exact codes, any M (tiles of 16
                              activation rows), K % 128 == 0, every buffer
                              < 2 GiB                                         */
} qp_kernel;

typedef struct {
  int32_t fmt;          /* qp_format                                         */
  int32_t bits;         /* AFFINE: 2, 4 or 8; Q4K: 4; Q6K: 6; SYM4: 4         */
  int32_t group_size;   /* AFFINE: 32, 64, 128; Q4K: 32; Q6K: 16;
                           SYM4: K (per output channel) or 32, 64, 128       */
  int32_t super_block;  /* Q4K, Q6K: 256; AFFINE, SYM4: 0                     */
  int32_t meta_dtype;   /* AFFINE: QP_F16 or QP_BF16; others: ignored         */
  int32_t reserved;     /* must be 0                                         */
  int64_t N;            /* output features (rows of W)                       */
  int64_t K;            /* input features (columns of W)                     */
} qp_desc;

typedef struct {
  void* qweight;
  void* qweight_hi;
  void* scales;
  void* zeros;
  void* steps;
} qp_weights;

/* Version of this ABI (QP_ABI_VERSION). */
int32_t qpack_abi_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on the same thread. */
const char* qpack_last_error(void);

/* Host only.  Byte sizes of the five buffers {qweight, qweight_hi, scales,
 * zeros, steps} for `d` (0 for an unused buffer).  Bits per weight of the
 * layout = 8 * sum(bytes) / (N*K): 4.625 for Q4K and 6.5625 for Q6K (the
 * superscale page's accounting), b + 32/gs for AFFINE. */
qp_status qpack_sizes(const qp_desc* d, size_t bytes_out[5]);

/* Quantize W (device fp32 [N, K], row-major) into `out`, whose buffers must
 * have the sizes qpack_sizes gives.  Bit-exact with the rules above. */
qp_status qpack_quantize(const qp_desc* d, const float* W, const qp_weights* out,
                         void* stream);

/* AFFINE only: quantize W like qpack_quantize, but with the zero point
 * (bias) of every group chosen by Half-Quadratic Quantization (HQQ, Badri
 * and Shaji 2023), the "hqq" quantization-parameter option that ExecuTorch
 * PR #17235's review ("Metal backend: Add Metal int4 quantization support
 * to Parakeet") asks for on the Metal int4 affine weights.  The scale is the
 * min/max scale of qpack_quantize; per group, starting from z0 = -bias/s in
 * code units, `iters` updates
 *     q = clamp(rint(w/s + z), 0, 2^b - 1),  e = w - (q - z)*s,
 *     W_e = sign(e)*max(|e| - |e|^(lp_norm - 1)/beta, 0),
 *     z <- mean(q - (w - W_e)/s),  beta <- kappa*beta
 * run, the iterate with the smallest sum |e| is kept (the start included),
 * the stored bias is meta(-z*s), and the codes are then rounded against the
 * stored scale and bias as in qpack_quantize, so every forward kernel reads
 * the result unchanged.  Every step is one fp32 operation in that order;
 * |e|^(lp_norm - 1) is computed in fp64 and rounded once; group sums run in
 * ascending k.  The method's defaults: iters 20, lp_norm 0.7, beta 10,
 * kappa 1.01.  Errors: QP_EUNSUPPORTED for another format; QP_EINVAL for
 * iters outside [0, 10000], lp_norm outside (0, 1], a non-positive or
 * non-finite beta or kappa, and the checks of qpack_quantize.  Buffers as
 * for qpack_quantize (qweight_hi and steps unused); asynchronous on
 * `stream`.  Off the forward path: one thread per group. */
qp_status qpack_quantize_hqq(const qp_desc* d, const float* W, const qp_weights* out,
                             int32_t iters, float lp_norm, float beta, float kappa,
                             void* stream);

/* Expand the packed codes of `w` into `codes` (device [N, K] bytes): uint8
 * q for AFFINE and Q4K, int8 q for Q6K and SYM4 (SYM4 gives the int8 carrier
 * form of the a8w4 page, values in [-7, 7]). */
qp_status qpack_unpack_codes(const qp_desc* d, const qp_weights* w, void* codes,
                             void* stream);

/* Pack codes (device [N, K] bytes, as qpack_unpack_codes writes them) into
 * out->qweight (and out->qweight_hi for Q6K); metadata buffers are not
 * touched.  Codes outside the format's range are masked to the field width
 * (unspecified result, no error). */
qp_status qpack_pack_codes(const qp_desc* d, const void* codes,
                           const qp_weights* out, void* stream);

/* Fused-N concatenation: the layers w_in[0 .. parts-1] (descriptors d_in,
 * same format, bits, group size, super-block, metadata dtype and K as d_out)
 * stacked along N into `out` (d_out->N = the sum of their N), so that one
 * forward call computes all of them (e.g. the q, k and v projections): the
 * superscale page concatenates coalesced int4 weights along N for the same
 * reason.  Every buffer is N-leading with a fixed byte count per row, so
 * each part's bytes are copied right after the previous part's
 * (hipMemcpyAsync on `stream`, device to device); `out` must not overlap the
 * inputs.  Asynchronous like the other calls. */
qp_status qpack_concat_n(const qp_desc* d_out, int32_t parts, const qp_desc* d_in,
                         const qp_weights* w_in, const qp_weights* out, void* stream);

/* Re-encode plain per-group metadata into the nested superscale form of
 * `d` (QP_FMT_Q4K or QP_FMT_Q6K).  ExecuTorch PR #20571, "[cuda] Nested
 * Superscale Quantization for CUDA Weights (int4 / int6)": the original int4
 * and int6 tensors are converted into Q4_K / Q6_K and the k-quant pipeline
 * reused; "Analysis": the codes stay identical to the source values and only
 * the metadata is re-quantized.  Plain forms: int4 codes u in [0, 15] with
 * w = (u - z) * s per group of 32; int6 codes q in [-32, 31] with w = q * s
 * per group of 16.
 *   s: device fp32 [N, K/32] (Q4K) or [N, K/16] (Q6K) group scales, >= 0;
 *   z: device fp32 [N, K/32] zero points in code units, >= 0 (Q4K), NULL
 *      for Q6K;
 *   out: scales, steps (and zeros for Q4K) of the sizes qpack_sizes gives;
 *      qweight / qweight_hi are not touched -- pack the unchanged codes with
 *      qpack_pack_codes;
 *   bad: optional device int32 (NULL to skip); set to 1 (never cleared) if
 *      any input is negative or not finite, which is encoded as 0.
 * Per super-block of 256 weights: step = fp16(fl32(max / L)) and code =
 * clamp(rint(fl32(v / step)), 0, L), 0 when the step is 0, with L = 255
 * (Q4K scale and zero codes) or 127 (Q6K scale code) -- the rule of the
 * nested quantizers, whose own plain stage feeds it. */
qp_status qpack_encode_nested(const qp_desc* d, const float* s, const float* z,
                              const qp_weights* out, int32_t* bad, void* stream);

/* Dequantize into W_out (device [N, K] of out_dtype).  QP_F32 gives the fp32
 * evaluation of the format's rule in the order written above (exact for Q6K;
 * the exact value rounded once for AFFINE and SYM4; for Q4K the difference
 * q - zero is rounded once before the product).  QP_F16 / QP_BF16 round that
 * fp32 value to nearest-even. */
qp_status qpack_dequantize(const qp_desc* d, const qp_weights* w, void* W_out,
                           int32_t out_dtype, void* stream);

/* y [M, N] (y_dtype, row-major) = x [M, K] (x_dtype, row-major) * W^T
 * (+ bias [N], x_dtype, or NULL).  x_dtype: QP_F16 or QP_BF16.  y_dtype:
 * QP_F16, QP_BF16 or QP_F32.  Accumulation is fp32.
 * The qGEMV (QP_KERNEL_GEMV) and the MFMA qGEMV (QP_KERNEL_GEMV_MFMA) use
 * the codes exactly, in products with the activations in their own type,
 * and apply each group's scale and offset in fp32.  The qGEMM
 * (QP_KERNEL_GEMM) runs on fp16 MFMA: each weight is dequantized and
 * rounded once to fp16 inside the kernel (scales, zero points and weights
 * are assumed to lie in the fp16 normal range) -- except per-channel SYM4,
 * whose codes q are fp16-exact and whose channel scale multiplies the fp32
 * sum -- and each activation row is
 * scaled by a power of two that brings its largest magnitude into fp16
 * range before it is converted (undone in fp32 after the sums), so every
 * finite bf16 activation is taken.  To hold the per-row exponents without a
 * workspace the qGEMM writes them into y before it computes; y's contents
 * are undefined until the call completes.  QP_KERNEL_AUTO picks by M and K as
 * listed under qp_kernel.
 * Where the qGEMM's 224-row tiling applies (qlinear_workspace_bytes > 0),
 * this call takes that workspace stream-ordered from a memory pool the
 * library keeps per device (created on first use, keeping what it served
 * for reuse until the process ends: about 2 (K + 2) bytes per activation
 * row) and returns it on `stream` after the qGEMM, so calls on different
 * streams never share it; under stream capture, or when the pool cannot
 * serve the request, it runs the workspace-free 256-row tiling instead
 * (same contract, slower).  Callers that manage memory themselves use
 * qlinear_forward_ws; callers that cannot allocate, qlinear_forward_static. */
qp_status qlinear_forward(const qp_desc* d, const void* x, int32_t x_dtype,
                          int64_t M, const qp_weights* w, const void* bias,
                          void* y, int32_t y_dtype, void* stream);

/* qlinear_forward with the kernel family chosen by the caller (qp_kernel). */
qp_status qlinear_forward_kernel(const qp_desc* d, const void* x,
                                 int32_t x_dtype, int64_t M,
                                 const qp_weights* w, const void* bias, void* y,
                                 int32_t y_dtype, int32_t kernel, void* stream);

/* Host only.  Bytes of device workspace that qlinear_forward_ws can use for
 * these arguments (the kernel is chosen as in qlinear_forward_kernel).  The
 * qGEMM has a second tiling, 224 weight rows per block instead of 256, for
 * shapes whose block count it spreads better over the 256 compute units
 * (N = 14336 at M = 2048: 512 blocks, two full waves, instead of 448, 1.75
 * waves); it reads the activations staged once as fp16 in MFMA fragment
 * order, ceil(M / 16) * 16 * K * 2 bytes, followed by one int32 prescale
 * exponent per staged row (ceil(M / 16) * 16 * 4 bytes).  0 when the call
 * would not use it (another kernel, 256-row tiles, or more than 2^31 staged
 * bytes).  The
 * argument checks of the forward call apply. */
qp_status qlinear_workspace_bytes(const qp_desc* d, int32_t x_dtype, int64_t M,
                                  int32_t kernel, size_t* bytes);

/* qlinear_forward_kernel with a caller-owned device workspace (16-byte
 * aligned).  When qlinear_workspace_bytes gives n > 0, a non-NULL workspace
 * of at least n bytes selects the 224-row-tile qGEMM: a staging kernel
 * writes the workspace, then the qGEMM reads it, both on `stream`; a
 * smaller non-zero size is QP_EINVAL.  Same numerics as the 256-row-tile
 * qGEMM (fp16 operands, fp32 accumulation) with another MFMA shape, so the
 * two agree up to the order of fp32 additions.  The workspace is busy until
 * this call's kernels finish on `stream`: work on other streams must not
 * use it meanwhile.  With n == 0 or a NULL workspace the call is
 * qlinear_forward_kernel. */
qp_status qlinear_forward_ws(const qp_desc* d, const void* x, int32_t x_dtype,
                             int64_t M, const qp_weights* w, const void* bias,
                             void* y, int32_t y_dtype, int32_t kernel,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc):
 * qlinear_forward_ws without a workspace argument.  Where the call would use
 * a workspace (see qlinear_workspace_bytes) it uses the library's static
 * device scratch instead: 40 MiB per GPU, held from the library's load until
 * the process ends, so ceil(M / 16) * 16 * (2 K + 4) bytes <= 40 MiB (e.g.
 * M = 2048 at K = 8192); a larger staging need is QP_EUNSUPPORTED and
 * nothing is enqueued.  Allocates nothing (no hipMalloc, no allocating library call);
 * the scratch's device address is looked up once per device on the first
 * call, with that device current.  Every call on a GPU shares that GPU's
 * scratch: calls that overlap on one GPU (other streams, other threads)
 * race, so serialize them.  The staging kernel writes every byte the qGEMM
 * reads, so stale contents from an earlier call are never used.  Other
 * arguments, numerics and errors as qlinear_forward_ws. */
qp_status qlinear_forward_static(const qp_desc* d, const void* x, int32_t x_dtype,
                                 int64_t M, const qp_weights* w, const void* bias,
                                 void* y, int32_t y_dtype, int32_t kernel,
                                 void* stream);

/* a8w4: int8 activations x symmetric int4 weights (ExecuTorch PR #16577,
 * "Arm backend: Support a8w4 for convolution and linear": int4 weights in
 * an int8 container with qmin = -7, qmax = 7, and 8-bit activations).
 *
 * qpack_quantize_activations: per-token symmetric int8 (the page does not
 * fix the activation rule; this one is per row m):
 *   xs[m] = fl32(max_k |x[m, k]| / 127),
 *   xq[m, k] = xs[m] == 0 ? 0 : clamp(rint(fl32(x[m, k] / xs[m])), -127, 127),
 * each step one IEEE fp32 operation, ties to even.  x: [M, K] x_dtype
 * (QP_F16 / QP_BF16); xq: int8 [M, K]; xs: fp32 [M]; device pointers,
 * 16-byte aligned, caller-owned. */
qp_status qpack_quantize_activations(const void* x, int32_t x_dtype, int64_t M,
                                     int64_t K, void* xq, float* xs, void* stream);

/* qlinear_forward_a8w4: y [M, N] = xs[m] * s_n * sum_k xq[m, k] * q[n, k]
 * (+ bias [N], fp32, or NULL), for weights in the SYM4 format with one fp32
 * scale s_n per output channel (group_size = K; q = u - 8 from the stored
 * nibbles).  The integer sums are exact (int8 matrix cores, int32 per K
 * split, int64 across splits); the scaling is done in fp64 in the order
 * ((sum * xs[m]) * s_n) + bias and rounded once to fp32, then to y_dtype
 * (QP_F16, QP_BF16, QP_F32) to nearest-even.  Needs K % 128 == 0 and xq and
 * the codes each below 2 GiB; other SYM4 group sizes and formats are
 * QP_EUNSUPPORTED. */
qp_status qlinear_forward_a8w4(const qp_desc* d, const void* xq, const float* xs,
                               int64_t M, const qp_weights* w, const float* bias,
                               void* y, int32_t y_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
