// C ABI of libqlinear: argument validation, error reporting and dispatch to
// the HIP kernels.  The contract of every entry point is documented in
// include/qlinear.h.  Shape rules follow the pages: K divisible by the group
// size and by whole packed words (the Metal export path filters out layers
// whose weights are not divisible by 8); for the nested superscale formats
// K % 256 == 0 and one step per 256-weight super-block, with detailed
// messages on failure (ExecuTorch PR #20571 review: kernel-side validation).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/qlinear.h"
#include "qp_internal.hpp"

namespace {

thread_local std::string g_err;

qp_status fail(qp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

qp_status ok() {
  g_err.clear();
  return QP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the descriptor and copies it into the internal form.
qp_status check_desc(const qp_desc* d, qp::Desc* out) {
  if (!d) return fail(QP_EINVAL, "descriptor is NULL");
  if (d->reserved != 0) return fail(QP_EINVAL, "qp_desc.reserved must be 0");
  if (d->N <= 0 || d->K <= 0)
    return fail(QP_ESHAPE, "N and K must be positive (N=%lld, K=%lld)", (long long)d->N,
                (long long)d->K);
  if (d->N > (int64_t(1) << 31) || d->K > (int64_t(1) << 24))
    return fail(QP_EUNSUPPORTED, "N must be <= 2^31 and K <= 2^24 (N=%lld, K=%lld)",
                (long long)d->N, (long long)d->K);
  const int64_t N = d->N, K = d->K;
  const int gs = d->group_size;
  switch (d->fmt) {
    case QP_FMT_AFFINE: {
      if (d->bits != 2 && d->bits != 4 && d->bits != 8)
        return fail(QP_EUNSUPPORTED, "AFFINE bits must be 2, 4 or 8 (got %d)", d->bits);
      if (gs != 32 && gs != 64 && gs != 128)
        return fail(QP_EUNSUPPORTED, "AFFINE group_size must be 32, 64 or 128 (got %d)", gs);
      if (d->meta_dtype != QP_F16 && d->meta_dtype != QP_BF16)
        return fail(QP_EUNSUPPORTED, "AFFINE meta_dtype must be QP_F16 or QP_BF16 (got %d)",
                    d->meta_dtype);
      if (d->super_block != 0)
        return fail(QP_EINVAL, "AFFINE has no super-block (super_block must be 0, got %d)",
                    d->super_block);
      if (K % gs)
        return fail(QP_ESHAPE, "K=%lld is not a multiple of group_size=%d", (long long)K, gs);
      const int chunk = 128 / d->bits;  // codes per 16-byte chunk
      if (K % chunk)
        return fail(QP_ESHAPE, "K=%lld must be a multiple of %d for %d-bit codes (16-byte chunks)",
                    (long long)K, chunk, d->bits);
      break;
    }
    case QP_FMT_Q4K:
      if (d->bits != 4 || gs != 32 || d->super_block != 256)
        return fail(QP_EUNSUPPORTED,
                    "Q4K needs bits=4, group_size=32, super_block=256 (got %d, %d, %d)", d->bits,
                    gs, d->super_block);
      if (K % 256)
        return fail(QP_ESHAPE, "Q4K needs K %% 256 == 0 (K=%lld, n_super=K/256)", (long long)K);
      break;
    case QP_FMT_Q6K:
      if (d->bits != 6 || gs != 16 || d->super_block != 256)
        return fail(QP_EUNSUPPORTED,
                    "Q6K needs bits=6, group_size=16, super_block=256 (got %d, %d, %d)", d->bits,
                    gs, d->super_block);
      if (K % 256)
        return fail(QP_ESHAPE, "Q6K needs K %% 256 == 0 (K=%lld, n_super=K/256)", (long long)K);
      break;
    case QP_FMT_SYM4:
      if (d->bits != 4 || d->super_block != 0)
        return fail(QP_EUNSUPPORTED, "SYM4 needs bits=4 and super_block=0 (got %d, %d)", d->bits,
                    d->super_block);
      if (K % 32)
        return fail(QP_ESHAPE, "SYM4 needs K %% 32 == 0 (K=%lld)", (long long)K);
      if (!(gs == K || gs == 32 || gs == 64 || gs == 128))
        return fail(QP_EUNSUPPORTED, "SYM4 group_size must be K or 32, 64, 128 (got %d)", gs);
      if (K % gs)
        return fail(QP_ESHAPE, "K=%lld is not a multiple of group_size=%d", (long long)K, gs);
      break;
    default:
      return fail(QP_EINVAL, "unknown format %d", d->fmt);
  }
  out->fmt = d->fmt;
  out->bits = d->bits;
  out->gs = gs;
  out->sb = d->super_block;
  out->meta = d->meta_dtype;
  out->N = N;
  out->K = K;
  return QP_OK;
}

void sizes_of(const qp::Desc& d, size_t b[5]) {
  const size_t N = (size_t)d.N, K = (size_t)d.K;
  for (int i = 0; i < 5; ++i) b[i] = 0;
  switch (d.fmt) {
    case QP_FMT_AFFINE:
      b[0] = N * K * d.bits / 8;
      b[2] = N * (K / d.gs) * 2;
      b[3] = N * (K / d.gs) * 2;
      break;
    case QP_FMT_Q4K:
      b[0] = N * K / 2;
      b[2] = N * K / 32;
      b[3] = N * K / 32;
      b[4] = N * (K / 256) * 4;
      break;
    case QP_FMT_Q6K:
      b[0] = N * K / 2;
      b[1] = N * K / 4;
      b[2] = N * K / 16;
      b[4] = N * (K / 256) * 2;
      break;
    default:
      b[0] = N * K / 2;
      b[2] = N * (K / d.gs) * 4;
      break;
  }
}

const char* kBufName[5] = {"qweight", "qweight_hi", "scales", "zeros", "steps"};

// Every buffer the format uses must be a non-NULL, 16-byte aligned pointer.
qp_status check_weights(const qp::Desc& d, const qp_weights* w, bool codes_only) {
  if (!w) return fail(QP_EINVAL, "weights struct is NULL");
  size_t b[5];
  sizes_of(d, b);
  const void* p[5] = {w->qweight, w->qweight_hi, w->scales, w->zeros, w->steps};
  for (int i = 0; i < 5; ++i) {
    if (!b[i] || (codes_only && i >= 2)) continue;
    if (!p[i]) return fail(QP_EINVAL, "%s is NULL but the format needs %zu bytes", kBufName[i], b[i]);
    if (!aligned16(p[i])) return fail(QP_EALIGN, "%s is not 16-byte aligned", kBufName[i]);
  }
  return QP_OK;
}

qp::Bufs bufs_of(const qp_weights* w) {
  return qp::Bufs{w->qweight, w->qweight_hi, w->scales, w->zeros, w->steps};
}

qp_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QP_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// The qGEMM addresses a block's 256 activation rows through a 32-bit buffer
// resource (256 * K * 2 bytes), hence K <= 2^22.
bool gemm_ok(const qp::Desc& d) { return d.K % 64 == 0 && d.K <= (int64_t(1) << 22); }

}  // namespace

extern "C" {

int32_t qpack_abi_version(void) { return QP_ABI_VERSION; }

const char* qpack_last_error(void) { return g_err.c_str(); }

qp_status qpack_sizes(const qp_desc* d, size_t bytes_out[5]) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if (!bytes_out) return fail(QP_EINVAL, "bytes_out is NULL");
  sizes_of(dd, bytes_out);
  return ok();
}

qp_status qpack_quantize(const qp_desc* d, const float* W, const qp_weights* out, void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if (!W) return fail(QP_EINVAL, "W is NULL");
  if (!aligned16(W)) return fail(QP_EALIGN, "W is not 16-byte aligned");
  if ((st = check_weights(dd, out, false)) != QP_OK) return st;
  (void)hipGetLastError();
  return hip_status(qp::launch_quantize(dd, W, out->qweight, out->qweight_hi, out->scales,
                                        out->zeros, out->steps, (hipStream_t)stream),
                    "qpack_quantize launch");
}

qp_status qpack_unpack_codes(const qp_desc* d, const qp_weights* w, void* codes, void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if ((st = check_weights(dd, w, true)) != QP_OK) return st;
  if (!codes) return fail(QP_EINVAL, "codes is NULL");
  if (!aligned16(codes)) return fail(QP_EALIGN, "codes is not 16-byte aligned");
  (void)hipGetLastError();
  return hip_status(qp::launch_unpack(dd, bufs_of(w), codes, (hipStream_t)stream),
                    "qpack_unpack_codes launch");
}

qp_status qpack_pack_codes(const qp_desc* d, const void* codes, const qp_weights* out,
                           void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if ((st = check_weights(dd, out, true)) != QP_OK) return st;
  if (!codes) return fail(QP_EINVAL, "codes is NULL");
  if (!aligned16(codes)) return fail(QP_EALIGN, "codes is not 16-byte aligned");
  (void)hipGetLastError();
  return hip_status(
      qp::launch_pack(dd, codes, out->qweight, out->qweight_hi, (hipStream_t)stream),
      "qpack_pack_codes launch");
}

qp_status qpack_dequantize(const qp_desc* d, const qp_weights* w, void* W_out, int32_t out_dtype,
                           void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if ((st = check_weights(dd, w, false)) != QP_OK) return st;
  if (out_dtype != QP_F16 && out_dtype != QP_BF16 && out_dtype != QP_F32)
    return fail(QP_EINVAL, "out_dtype must be QP_F16, QP_BF16 or QP_F32 (got %d)", out_dtype);
  if (!W_out) return fail(QP_EINVAL, "W_out is NULL");
  if (!aligned16(W_out)) return fail(QP_EALIGN, "W_out is not 16-byte aligned");
  (void)hipGetLastError();
  return hip_status(qp::launch_dequant(dd, bufs_of(w), W_out, out_dtype, (hipStream_t)stream),
                    "qpack_dequantize launch");
}

}  // extern "C"

namespace {

enum Use { USE_GEMV, USE_SKINNY, USE_GEMM };

// Checks the forward arguments that do not involve a workspace and picks the
// kernel family.
qp_status plan_forward(const qp_desc* d, qp::Desc* dd, int32_t x_dtype, int64_t M,
                       int32_t kernel, Use* use, size_t nbytes[5]) {
  qp_status st = check_desc(d, dd);
  if (st != QP_OK) return st;
  if (M <= 0) return fail(QP_ESHAPE, "M must be positive (got %lld)", (long long)M);
  if (M > (int64_t(1) << 24)) return fail(QP_EUNSUPPORTED, "M must be <= 2^24");
  if (x_dtype != QP_F16 && x_dtype != QP_BF16)
    return fail(QP_EINVAL, "x_dtype must be QP_F16 or QP_BF16 (got %d)", x_dtype);
  if (kernel != QP_KERNEL_AUTO && kernel != QP_KERNEL_GEMV && kernel != QP_KERNEL_GEMM &&
      kernel != QP_KERNEL_GEMV_MFMA)
    return fail(QP_EINVAL, "unknown kernel selector %d", kernel);
  if (kernel == QP_KERNEL_GEMM && !gemm_ok(*dd))
    return fail(QP_EUNSUPPORTED, "the qGEMM kernel needs K %% 64 == 0 and K <= 2^22 (K=%lld)",
                (long long)dd->K);
  sizes_of(*dd, nbytes);
  bool small_bufs = (size_t)M * (size_t)dd->K * 2 < (size_t(1) << 31);
  for (int i = 0; i < 5; ++i) small_bufs = small_bufs && nbytes[i] < (size_t(1) << 31);
  const bool gemv_fits = qp::gemv_supported(*dd) && small_bufs;
  const bool skinny_fits = qp::skinny_supported(*dd) && M <= 16 && small_bufs;
  if (kernel == QP_KERNEL_GEMV && !gemv_fits)
    return fail(QP_EUNSUPPORTED,
                "the qGEMV kernel needs K <= its register plan (K=%lld) and every buffer < 2 GiB",
                (long long)dd->K);
  if (kernel == QP_KERNEL_GEMV_MFMA && !skinny_fits)
    return fail(QP_EUNSUPPORTED,
                "the MFMA qGEMV kernel needs M <= 16, K %% 128 == 0 and every buffer < 2 GiB "
                "(M=%lld, K=%lld)",
                (long long)M, (long long)dd->K);
  if (kernel == QP_KERNEL_AUTO) {
    // The MFMA qGEMV dequantizes each weight once instead of doing one dot
    // product per activation row.  Where it takes over (measured on
    // 8192 x 8192 layers): 2 rows for per-channel SYM4 (exact codes), 4 for
    // Q6K (costly 6-bit dequantization), 3 for the others.
    int64_t mfma_from = 3;
    if (dd->fmt == qp::SYM4 && dd->gs == dd->K) mfma_from = 2;
    else if (dd->fmt == qp::Q6K) mfma_from = 4;
    // fp16-rounded weights add an error that grows like sqrt(K) against the
    // layer's element bound; past K = 16384 small M stays on the exact-code
    // qGEMV
    const bool exact_preferred = dd->K > 16384 && M <= 8 && gemv_fits;
    if (M >= mfma_from && M <= 16 && skinny_fits && !exact_preferred) *use = USE_SKINNY;
    else if (M <= 8 && gemv_fits) *use = USE_GEMV;
    else if (gemm_ok(*dd)) *use = USE_GEMM;
    else if (gemv_fits) *use = USE_GEMV;
    else return fail(QP_EUNSUPPORTED, "no kernel supports K=%lld for this format", (long long)dd->K);
  } else {
    *use = kernel == QP_KERNEL_GEMM ? USE_GEMM : kernel == QP_KERNEL_GEMV_MFMA ? USE_SKINNY : USE_GEMV;
  }
  return QP_OK;
}

}  // namespace

extern "C" {

qp_status qlinear_workspace_bytes(const qp_desc* d, int32_t x_dtype, int64_t M, int32_t kernel,
                                  size_t* bytes) {
  if (!bytes) return fail(QP_EINVAL, "bytes is NULL");
  *bytes = 0;
  qp::Desc dd;
  Use use;
  size_t nbytes[5];
  qp_status st = plan_forward(d, &dd, x_dtype, M, kernel, &use, nbytes);
  if (st != QP_OK) return st;
  if (use == USE_GEMM) *bytes = qp::gemm_workspace_bytes(dd, M);
  return ok();
}

qp_status qlinear_forward_ws(const qp_desc* d, const void* x, int32_t x_dtype, int64_t M,
                             const qp_weights* w, const void* bias, void* y, int32_t y_dtype,
                             int32_t kernel, void* workspace, size_t workspace_bytes,
                             void* stream) {
  qp::Desc dd;
  Use use;
  size_t nbytes[5];
  qp_status st = plan_forward(d, &dd, x_dtype, M, kernel, &use, nbytes);
  if (st != QP_OK) return st;
  if ((st = check_weights(dd, w, false)) != QP_OK) return st;
  if (y_dtype != QP_F16 && y_dtype != QP_BF16 && y_dtype != QP_F32)
    return fail(QP_EINVAL, "y_dtype must be QP_F16, QP_BF16 or QP_F32 (got %d)", y_dtype);
  if (!x) return fail(QP_EINVAL, "x is NULL");
  if (!y) return fail(QP_EINVAL, "y is NULL");
  if (!aligned16(x)) return fail(QP_EALIGN, "x is not 16-byte aligned");
  if (!aligned16(y)) return fail(QP_EALIGN, "y is not 16-byte aligned");
  if (bias && !aligned16(bias)) return fail(QP_EALIGN, "bias is not 16-byte aligned");
  if (workspace && !aligned16(workspace))
    return fail(QP_EALIGN, "workspace is not 16-byte aligned");
  void* ws = nullptr;
  if (use == USE_GEMM && workspace) {
    const size_t need = qp::gemm_workspace_bytes(dd, M);
    if (need > 0) {
      if (workspace_bytes < need)
        return fail(QP_EINVAL, "workspace too small: %zu bytes, this call needs %zu",
                    workspace_bytes, need);
      ws = workspace;
    }
  }
  (void)hipGetLastError();
  hipError_t e;
  const char* what;
  if (use == USE_GEMM) {
    e = qp::launch_gemm(dd, x, x_dtype, M, bufs_of(w), bias, y, y_dtype, ws, (hipStream_t)stream);
    what = "qGEMM launch";
  } else if (use == USE_SKINNY) {
    e = qp::launch_skinny(dd, x, x_dtype, M, bufs_of(w), bias, y, y_dtype, nbytes,
                          (hipStream_t)stream);
    what = "MFMA qGEMV launch";
  } else {
    e = qp::launch_gemv(dd, x, x_dtype, M, bufs_of(w), bias, y, y_dtype, nbytes,
                        (hipStream_t)stream);
    what = "qGEMV launch";
  }
  return hip_status(e, what);
}

qp_status qlinear_forward_kernel(const qp_desc* d, const void* x, int32_t x_dtype, int64_t M,
                                 const qp_weights* w, const void* bias, void* y, int32_t y_dtype,
                                 int32_t kernel, void* stream) {
  return qlinear_forward_ws(d, x, x_dtype, M, w, bias, y, y_dtype, kernel, nullptr, 0, stream);
}

qp_status qlinear_forward(const qp_desc* d, const void* x, int32_t x_dtype, int64_t M,
                          const qp_weights* w, const void* bias, void* y, int32_t y_dtype,
                          void* stream) {
  return qlinear_forward_kernel(d, x, x_dtype, M, w, bias, y, y_dtype, QP_KERNEL_AUTO, stream);
}

}  // extern "C"
