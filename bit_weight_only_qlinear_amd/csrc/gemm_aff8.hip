// qGEMM instantiations for 8-bit affine codes (kernels in gemm_kernels.hpp).
#include "gemm_kernels.hpp"

namespace qp {

hipError_t gemm_launch_aff8(const GemmArgs& a, const GemmPick& p, unsigned blocks,
                            hipStream_t s) {
  void (*fn)(GemmArgs) = nullptr;
  const bool g32 = a.gs == 32, g128 = a.gs == 128;
  // (kind, x dtype, metadata dtype, two groups per 64-column step)

#define QP_GEMM_FLAGS(KD, MB, G)                                                       \
  if (p.n224) fn = p.xb ? k_gemm224<KD, true, MB, G, 0> : k_gemm224<KD, false, MB, G, 0>;  \
  else fn = p.xb ? k_gemm<KD, true, MB, G> : k_gemm<KD, false, MB, G>;
#define QP_GEMM_FLAGS_CH(KD, MB, G, GSZ)                                               \
  if (p.n224 && p.mch) fn = p.xb ? k_gemm224<KD, true, MB, G, GSZ> : k_gemm224<KD, false, MB, G, GSZ>; \
  else { QP_GEMM_FLAGS(KD, MB, G) }

  if (p.mb) {
    if (g32) { QP_GEMM_FLAGS_CH(G_AFF8, true, true, 32) }
    else if (g128) { QP_GEMM_FLAGS_CH(G_AFF8, true, false, 128) }
    else { QP_GEMM_FLAGS_CH(G_AFF8, true, false, 64) }
  } else {
    if (g32) { QP_GEMM_FLAGS_CH(G_AFF8, false, true, 32) }
    else if (g128) { QP_GEMM_FLAGS_CH(G_AFF8, false, false, 128) }
    else { QP_GEMM_FLAGS_CH(G_AFF8, false, false, 64) }
  }
#undef QP_GEMM_FLAGS_CH
#undef QP_GEMM_FLAGS
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qp
