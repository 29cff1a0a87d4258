// qGEMM instantiations for the Q4K, Q6K and SYM4 formats (kernels in
// gemm_kernels.hpp).
#include "gemm_kernels.hpp"

namespace qp {

hipError_t gemm_launch_kq(int fmt, const GemmArgs& a, const GemmPick& p, unsigned blocks,
                          hipStream_t s) {
  void (*fn)(GemmArgs) = nullptr;
  const bool xb = p.xb, n224 = p.n224;
#define QP_GEMM_FLAGS(KD, MB, G)                                                 \
  if (n224) fn = xb ? k_gemm224<KD, true, MB, G, 0> : k_gemm224<KD, false, MB, G, 0>;  \
  else fn = xb ? k_gemm<KD, true, MB, G> : k_gemm<KD, false, MB, G>;
  if (fmt == Q4K) {
    if (n224 && a.K % 512 == 0)
      fn = xb ? k_gemm224<G_Q4K, true, false, false, 32> : k_gemm224<G_Q4K, false, false, false, 32>;
    else { QP_GEMM_FLAGS(G_Q4K, false, false) }
  } else if (fmt == Q6K) {
    if (n224)   // K % 256 == 0 always holds for Q6K
      fn = xb ? k_gemm224<G_Q6K, true, false, false, 16> : k_gemm224<G_Q6K, false, false, false, 16>;
    else { QP_GEMM_FLAGS(G_Q6K, false, false) }
  } else {
    if (a.gs == a.K) {   // per-channel scale: exact codes
      QP_GEMM_FLAGS(G_SYM4C, false, false)
    } else if (n224 && a.gs == 32 && a.K % 128 == 0)   // group-wise: 4 scales per chunk
      fn = xb ? k_gemm224<G_SYM4, true, false, true, 32> : k_gemm224<G_SYM4, false, false, true, 32>;
    else if (n224 && a.gs == 64 && a.K % 256 == 0)
      fn = xb ? k_gemm224<G_SYM4, true, false, false, 64> : k_gemm224<G_SYM4, false, false, false, 64>;
    else if (n224 && a.gs == 128 && a.K % 512 == 0)
      fn = xb ? k_gemm224<G_SYM4, true, false, false, 128> : k_gemm224<G_SYM4, false, false, false, 128>;
    else if (a.gs == 32) { QP_GEMM_FLAGS(G_SYM4, false, true) } else { QP_GEMM_FLAGS(G_SYM4, false, false) }
  }
#undef QP_GEMM_FLAGS
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qp
