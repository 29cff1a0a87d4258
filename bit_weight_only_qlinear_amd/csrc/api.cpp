// C ABI of libqlinear: argument validation, error reporting and dispatch to
// the HIP kernels.  The contract of every entry point is documented in
// include/qlinear.h.  Shape rules follow the pages: K divisible by the group
// size and by whole packed words (the Metal export path filters out layers
// whose weights are not divisible by 8); for the nested superscale formats
// K % 256 == 0 and one step per 256-weight super-block, with detailed
// messages on failure (ExecuTorch PR #20571 review: kernel-side validation).
#include <cmath>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
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

// The qGEMM rounds each dequantized weight once to fp16 (relative error up
// to 2^-11).  That error grows like sqrt(K) against the layer's element
// bound 1e-2 * ||x|| * max|w| / sqrt(K); the kernel is held to the bound up
// to K = 8192 (the largest K of the workloads it is verified on), and longer
// rows take the exact-code MFMA kernel instead.
// fp16-rounded weights hold the output bound up to K = 8192; per-channel
// SYM4 runs on exact codes (K up to 2^20: 32-bit tile offsets)
constexpr int64_t kGemmMaxK = 8192;
bool gemm_ok(const qp::Desc& d) {
  const bool exact = d.fmt == qp::SYM4 && d.gs == d.K;
  return d.K % 64 == 0 && d.K <= (exact ? (int64_t(1) << 20) : kGemmMaxK);
}

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

qp_status qpack_quantize_hqq(const qp_desc* d, const float* W, const qp_weights* out,
                             int32_t iters, float lp_norm, float beta, float kappa,
                             void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if (dd.fmt != qp::AFFINE)
    return fail(QP_EUNSUPPORTED, "qpack_quantize_hqq takes the AFFINE format (got %d)", dd.fmt);
  if (iters < 0 || iters > 10000)
    return fail(QP_EINVAL, "iters must lie in [0, 10000] (got %d)", iters);
  if (!(lp_norm > 0.f && lp_norm <= 1.f))
    return fail(QP_EINVAL, "lp_norm must lie in (0, 1] (got %g)", (double)lp_norm);
  if (!(beta > 0.f && std::isfinite(beta)))
    return fail(QP_EINVAL, "beta must be positive and finite (got %g)", (double)beta);
  if (!(kappa > 0.f && std::isfinite(kappa)))
    return fail(QP_EINVAL, "kappa must be positive and finite (got %g)", (double)kappa);
  if (!W) return fail(QP_EINVAL, "W is NULL");
  if (!aligned16(W)) return fail(QP_EALIGN, "W is not 16-byte aligned");
  if ((st = check_weights(dd, out, false)) != QP_OK) return st;
  (void)hipGetLastError();
  return hip_status(qp::launch_quantize_hqq(dd, W, out->qweight, out->scales, out->zeros, iters,
                                            lp_norm, beta, kappa, (hipStream_t)stream),
                    "qpack_quantize_hqq launch");
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

qp_status qpack_encode_nested(const qp_desc* d, const float* s, const float* z,
                              const qp_weights* out, int32_t* bad, void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if (dd.fmt != qp::Q4K && dd.fmt != qp::Q6K)
    return fail(QP_EUNSUPPORTED, "qpack_encode_nested takes the Q4K or Q6K format (got %d)", dd.fmt);
  if (!out) return fail(QP_EINVAL, "out is NULL");
  if (!s) return fail(QP_EINVAL, "s is NULL");
  if (dd.fmt == qp::Q4K && !z) return fail(QP_EINVAL, "Q4K needs the zero points z");
  if (dd.fmt == qp::Q6K && z) return fail(QP_EINVAL, "Q6K has no zero points: z must be NULL");
  if (!aligned16(s) || (z && !aligned16(z)) || (bad && !aligned16(bad)))
    return fail(QP_EALIGN, "s, z and bad must be 16-byte aligned");
  const void* need[3] = {out->scales, dd.fmt == qp::Q4K ? out->zeros : out->scales, out->steps};
  for (int i = 0; i < 3; ++i) {
    if (!need[i]) return fail(QP_EINVAL, "out->scales, out->zeros (Q4K) and out->steps must be set");
    if (!aligned16(need[i])) return fail(QP_EALIGN, "metadata buffers must be 16-byte aligned");
  }
  (void)hipGetLastError();
  return hip_status(qp::launch_encode_nested(dd, s, z, out->scales, out->zeros, out->steps,
                                             reinterpret_cast<int*>(bad), (hipStream_t)stream),
                    "qpack_encode_nested launch");
}

qp_status qpack_concat_n(const qp_desc* d_out, int32_t parts, const qp_desc* d_in,
                         const qp_weights* w_in, const qp_weights* out, void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d_out, &dd);
  if (st != QP_OK) return st;
  if (parts < 1) return fail(QP_EINVAL, "parts must be >= 1 (got %d)", parts);
  if (!d_in || !w_in || !out) return fail(QP_EINVAL, "d_in, w_in and out must not be NULL");
  if ((st = check_weights(dd, out, false)) != QP_OK) return st;
  int64_t rows = 0;
  for (int32_t i = 0; i < parts; ++i) {
    qp::Desc di;
    if ((st = check_desc(&d_in[i], &di)) != QP_OK) return st;
    const qp_desc& a = d_in[i];
    if (a.fmt != d_out->fmt || a.bits != d_out->bits || a.group_size != d_out->group_size ||
        a.super_block != d_out->super_block || a.meta_dtype != d_out->meta_dtype ||
        a.K != d_out->K)
      return fail(QP_EINVAL, "part %d differs from d_out in format, bits, group size, "
                  "super-block, metadata dtype or K", i);
    if ((st = check_weights(di, &w_in[i], false)) != QP_OK) return st;
    rows += a.N;
  }
  if (rows != dd.N)
    return fail(QP_ESHAPE, "the parts' N add up to %lld, d_out has N=%lld", (long long)rows,
                (long long)dd.N);
  // every buffer is N-leading with a fixed byte count per row: each part's
  // buffer lands right after the previous part's
  size_t off[5] = {0, 0, 0, 0, 0};
  void* dst[5] = {out->qweight, out->qweight_hi, out->scales, out->zeros, out->steps};
  (void)hipGetLastError();
  for (int32_t i = 0; i < parts; ++i) {
    qp::Desc di;
    check_desc(&d_in[i], &di);
    size_t b[5];
    sizes_of(di, b);
    const void* src[5] = {w_in[i].qweight, w_in[i].qweight_hi, w_in[i].scales, w_in[i].zeros,
                          w_in[i].steps};
    for (int q = 0; q < 5; ++q) {
      if (!b[q]) continue;
      const hipError_t e = hipMemcpyAsync(static_cast<unsigned char*>(dst[q]) + off[q], src[q],
                                          b[q], hipMemcpyDeviceToDevice, (hipStream_t)stream);
      if (e != hipSuccess) return hip_status(e, "qpack_concat_n copy");
      off[q] += b[q];
    }
  }
  return ok();
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
    return fail(QP_EUNSUPPORTED,
                "the qGEMM kernel (fp16-rounded weights) needs K %% 64 == 0 and K <= %lld, "
                "where it meets the output bound (K=%lld; per-channel SYM4: exact codes, "
                "K <= 2^20); QP_KERNEL_AUTO and QP_KERNEL_GEMV_MFMA use exact codes at any K",
                (long long)kGemmMaxK, (long long)dd->K);
  sizes_of(*dd, nbytes);
  bool small_bufs = (size_t)M * (size_t)dd->K * 2 < (size_t(1) << 31);
  for (int i = 0; i < 5; ++i) small_bufs = small_bufs && nbytes[i] < (size_t(1) << 31);
  const bool gemv_fits = qp::gemv_supported(*dd) && small_bufs;
  const bool skinny_fits = qp::skinny_supported(*dd) && small_bufs;
  if (kernel == QP_KERNEL_GEMV && !gemv_fits)
    return fail(QP_EUNSUPPORTED,
                "the qGEMV kernel needs K <= its register plan (K=%lld) and every buffer < 2 GiB",
                (long long)dd->K);
  if (kernel == QP_KERNEL_GEMV_MFMA && !skinny_fits)
    return fail(QP_EUNSUPPORTED,
                "the MFMA qGEMV kernel needs K %% 128 == 0 and every buffer < 2 GiB (K=%lld)",
                (long long)dd->K);
  if (kernel == QP_KERNEL_AUTO) {
    // The MFMA qGEMV runs one set of MFMAs per 16 activation rows instead of
    // one dot product per row and code pair.  Where it takes over from the
    // streaming qGEMV (timed on the decode layers): 2 rows for per-channel
    // SYM4 and 4-bit affine codes (11.2 vs 12.5 us on 14336 x 4096), 3 for
    // Q6K (20.8 vs 22.3 us on 8192 x 8192), 5 for 8-bit affine codes (at 4
    // rows the qGEMV still wins: 19.1 vs 20.7 us), 3 for the others (Q4K at
    // 2 rows: 24.7 on the qGEMV vs 35.4 us).  Past 16 rows the qGEMM, up to
    // the K where its fp16 weights hold the output bound; beyond that the
    // exact MFMA qGEMV in tiles of 16 activation rows.
    int64_t mfma_from = 3;
    if (dd->fmt == qp::SYM4 && dd->gs == dd->K) mfma_from = 2;
    else if (dd->fmt == qp::AFFINE && dd->bits == 4) mfma_from = 2;
    else if (dd->fmt == qp::AFFINE && dd->bits == 8) mfma_from = 5;
    if (M >= mfma_from && M <= 16 && skinny_fits) *use = USE_SKINNY;
    else if (M <= 8 && gemv_fits) *use = USE_GEMV;
    else if (gemm_ok(*dd)) *use = USE_GEMM;
    else if (skinny_fits) *use = USE_SKINNY;
    else if (gemv_fits) *use = USE_GEMV;
    else return fail(QP_EUNSUPPORTED, "no kernel supports K=%lld for this format", (long long)dd->K);
  } else {
    *use = kernel == QP_KERNEL_GEMM ? USE_GEMM : kernel == QP_KERNEL_GEMV_MFMA ? USE_SKINNY : USE_GEMV;
  }
  return QP_OK;
}

}  // namespace

namespace {

// Memory pool of each device for qlinear_forward's stream-ordered
// workspace, created on first use with that device current; it keeps what
// it has served (release threshold at the maximum), so later calls reuse
// that memory.  Held until the process ends.
constexpr int kPoolDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kPoolDevices];

hipError_t forward_pool(hipMemPool_t* out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kPoolDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pool[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    e = hipMemPoolCreate(&p, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = ~uint64_t(0);
    e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(p);
      return e;
    }
    g_pool[dev] = p;
  }
  *out = g_pool[dev];
  return hipSuccess;
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

qp_status qlinear_forward_static(const qp_desc* d, const void* x, int32_t x_dtype, int64_t M,
                                 const qp_weights* w, const void* bias, void* y, int32_t y_dtype,
                                 int32_t kernel, void* stream) {
  qp::Desc dd;
  Use use;
  size_t nbytes[5];
  qp_status st = plan_forward(d, &dd, x_dtype, M, kernel, &use, nbytes);
  if (st != QP_OK) return st;
  void* ws = nullptr;
  size_t wsb = 0;
  if (use == USE_GEMM && qp::gemm_workspace_bytes(dd, M) > 0) {
    wsb = qp::gemm_workspace_bytes(dd, M);
    if (wsb > qp::static_scratch_bytes())
      return fail(QP_EUNSUPPORTED,
                  "qlinear_forward_static: this call stages %zu bytes of activations, more than "
                  "the library's static scratch (%zu bytes: ceil(M / 16) * 16 * (2 K + 4) "
                  "bytes at most); use qlinear_forward_ws with a workspace",
                  wsb, qp::static_scratch_bytes());
    (void)hipGetLastError();
    const hipError_t e = qp::static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "static scratch lookup");
  }
  return qlinear_forward_ws(d, x, x_dtype, M, w, bias, y, y_dtype, kernel, ws, wsb, stream);
}

qp_status qlinear_forward_kernel(const qp_desc* d, const void* x, int32_t x_dtype, int64_t M,
                                 const qp_weights* w, const void* bias, void* y, int32_t y_dtype,
                                 int32_t kernel, void* stream) {
  return qlinear_forward_ws(d, x, x_dtype, M, w, bias, y, y_dtype, kernel, nullptr, 0, stream);
}

qp_status qlinear_forward(const qp_desc* d, const void* x, int32_t x_dtype, int64_t M,
                          const qp_weights* w, const void* bias, void* y, int32_t y_dtype,
                          void* stream) {
  // Where the qGEMM's 224-row tiling wants staged activations, take the
  // workspace stream-ordered from the library's pool and give it back on the
  // same stream after the qGEMM (no other call, on any stream, can see it in
  // between).  Under stream capture, or if the pool cannot serve it, run the
  // workspace-free tiling (same result, slower).
  qp::Desc dd;
  Use use;
  size_t nbytes[5];
  qp_status st = plan_forward(d, &dd, x_dtype, M, QP_KERNEL_AUTO, &use, nbytes);
  if (st != QP_OK) return st;
  const size_t need = use == USE_GEMM ? qp::gemm_workspace_bytes(dd, M) : 0;
  if (need > 0) {
    const hipStream_t s = (hipStream_t)stream;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipMemPool_t pool = nullptr;
    void* ws = nullptr;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone &&
        forward_pool(&pool) == hipSuccess &&
        hipMallocFromPoolAsync(&ws, need, pool, s) == hipSuccess) {
      st = qlinear_forward_ws(d, x, x_dtype, M, w, bias, y, y_dtype, QP_KERNEL_AUTO, ws, need,
                              stream);
      const hipError_t e = hipFreeAsync(ws, s);
      if (st == QP_OK && e != hipSuccess) return hip_status(e, "workspace release");
      return st;
    }
    (void)hipGetLastError();
  }
  return qlinear_forward_kernel(d, x, x_dtype, M, w, bias, y, y_dtype, QP_KERNEL_AUTO, stream);
}

}  // extern "C"

extern "C" {

qp_status qpack_quantize_activations(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                     void* xq, float* xs, void* stream) {
  if (x_dtype != QP_F16 && x_dtype != QP_BF16)
    return fail(QP_EINVAL, "x_dtype must be QP_F16 or QP_BF16 (got %d)", x_dtype);
  if (M <= 0 || K <= 0)
    return fail(QP_ESHAPE, "M and K must be positive (M=%lld, K=%lld)", (long long)M, (long long)K);
  if (M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 24))
    return fail(QP_EUNSUPPORTED, "M must be < 2^31 and K <= 2^24 (M=%lld, K=%lld)", (long long)M,
                (long long)K);
  if (!x || !xq || !xs) return fail(QP_EINVAL, "x, xq and xs must not be NULL");
  if (!aligned16(x) || !aligned16(xq) || !aligned16(xs))
    return fail(QP_EALIGN, "x, xq and xs must be 16-byte aligned");
  (void)hipGetLastError();
  return hip_status(qp::launch_quant_act(x, x_dtype, M, K, xq, xs, (hipStream_t)stream),
                    "qpack_quantize_activations launch");
}

qp_status qlinear_forward_a8w4(const qp_desc* d, const void* xq, const float* xs, int64_t M,
                               const qp_weights* w, const float* bias, void* y, int32_t y_dtype,
                               void* stream) {
  qp::Desc dd;
  qp_status st = check_desc(d, &dd);
  if (st != QP_OK) return st;
  if (dd.fmt != qp::SYM4 || dd.gs != dd.K)
    return fail(QP_EUNSUPPORTED,
                "a8w4 takes the SYM4 format with one scale per output channel (group_size = K)");
  if (dd.K % 128)
    return fail(QP_ESHAPE, "a8w4 needs K %% 128 == 0 (K=%lld)", (long long)dd.K);
  if (M <= 0) return fail(QP_ESHAPE, "M must be positive (got %lld)", (long long)M);
  if ((uint64_t)M * (uint64_t)dd.K >= (uint64_t(1) << 31) ||
      (uint64_t)dd.N * (uint64_t)dd.K / 2 >= (uint64_t(1) << 31))
    return fail(QP_EUNSUPPORTED, "a8w4 needs the activations and the codes each < 2 GiB");
  if ((st = check_weights(dd, w, false)) != QP_OK) return st;
  if (y_dtype != QP_F16 && y_dtype != QP_BF16 && y_dtype != QP_F32)
    return fail(QP_EINVAL, "y_dtype must be QP_F16, QP_BF16 or QP_F32 (got %d)", y_dtype);
  if (!xq || !xs || !y) return fail(QP_EINVAL, "xq, xs and y must not be NULL");
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(y))
    return fail(QP_EALIGN, "xq, xs and y must be 16-byte aligned");
  if (bias && !aligned16(bias)) return fail(QP_EALIGN, "bias is not 16-byte aligned");
  (void)hipGetLastError();
  return hip_status(qp::launch_a8w4(dd, xq, xs, M, bufs_of(w), bias, y, y_dtype,
                                    (hipStream_t)stream),
                    "qlinear_forward_a8w4 launch");
}

}  // extern "C"
