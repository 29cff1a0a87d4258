// Internal declarations shared by the host API and the kernel translation
// units of libqlinear (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qp {

enum Fmt : int { AFFINE = 0, Q4K = 1, Q6K = 2, SYM4 = 3 };
enum DType : int { F16 = 0, BF16 = 1, F32 = 2 };

// Validated, host-side copy of the descriptor.
struct Desc {
  int fmt, bits, gs, sb, meta;
  int64_t N, K;
};

struct Bufs {
  const void* qweight;
  const void* qweight_hi;
  const void* scales;
  const void* zeros;
  const void* steps;
};

// Launchers (each returns the hipError_t of its launch).
hipError_t launch_quantize(const Desc& d, const float* W, void* qweight,
                           void* qweight_hi, void* scales, void* zeros,
                           void* steps, hipStream_t s);
hipError_t launch_quantize_hqq(const Desc& d, const float* W, void* qweight, void* scales,
                               void* zeros, int iters, float p, float beta, float kappa,
                               hipStream_t s);
hipError_t launch_unpack(const Desc& d, const Bufs& b, void* codes,
                         hipStream_t s);
hipError_t launch_pack(const Desc& d, const void* codes, void* qweight,
                       void* qweight_hi, hipStream_t s);
hipError_t launch_dequant(const Desc& d, const Bufs& b, void* out, int out_dt,
                          hipStream_t s);
// True when the qGEMV kernel's register plan covers this K (every lane's
// slice of the activations must fit in registers).
bool gemv_supported(const Desc& d);
// `bytes` are the five buffer sizes of the layout (each < 2 GiB, checked
// by the caller): the kernel addresses them through buffer resources.
hipError_t launch_gemv(const Desc& d, const void* x, int xdt, int64_t M,
                       const Bufs& b, const void* bias, void* y, int ydt,
                       const size_t bytes[5], hipStream_t s);
// Exact-code MFMA qGEMV, activation rows in tiles of 16 (any M): K must be
// a multiple of 128.
bool skinny_supported(const Desc& d);
hipError_t launch_skinny(const Desc& d, const void* x, int xdt, int64_t M,
                         const Bufs& b, const void* bias, void* y, int ydt,
                         const size_t bytes[5], hipStream_t s);
// Workspace bytes of the qGEMM with 224-row tiles and staged activations (M
// rounded up to 16 rows of K fp16); 0 where 256-row tiles are as good or
// the shape is past its 32-bit indexing.
size_t gemm_workspace_bytes(const Desc& d, int64_t M);
// ws: null (256-row tiles), or a device buffer of gemm_workspace_bytes(d, M)
// > 0 bytes (a staging kernel, then the 224-row-tile kernel, same stream).
hipError_t launch_gemm(const Desc& d, const void* x, int xdt, int64_t M,
                       const Bufs& b, const void* bias, void* y, int ydt,
                       void* ws, hipStream_t s);

// Plain per-group metadata (fp32 scales, Q4K zero points) into the nested
// Q4K / Q6K metadata buffers; *bad (optional, device) flags invalid inputs.
hipError_t launch_encode_nested(const Desc& d, const float* sv, const float* zv, void* scales,
                                void* zeros, void* steps, int* bad, hipStream_t st);
// Per-token symmetric int8 activations: q [M, K] int8, s [M] fp32.
hipError_t launch_quant_act(const void* x, int xdt, int64_t M, int64_t K, void* q, float* s,
                            hipStream_t st);
// a8w4 forward (SYM4 per output channel, K % 128 == 0, every buffer < 2 GiB).
hipError_t launch_a8w4(const Desc& d, const void* xq, const float* xs, int64_t M, const Bufs& b,
                       const float* bias, void* y, int ydt, hipStream_t s);

// Static device scratch of the allocation-free forward (noalloc.hip): its
// size, and its address on the current device (looked up once per device).
size_t static_scratch_bytes();
hipError_t static_scratch(void** out);

}  // namespace qp
