// a8w4 forward: int8 activations x symmetric int4 weights on the int8 matrix
// cores (v_mfma_i32_16x16x64_i8), exact integer dot products.
//
//   y[m, n] = s_m * s_n * sum_k q[m, k] * qw[n, k]   (+ bias[n])
//
// q, s_m: per-token int8 activations and their fp32 scales (from
// qpack_quantize_activations); qw = u - 8 in [-7, 7]: the stored nibbles of
// the SYM4 format (ExecuTorch PR #16577, "Arm backend: Support a8w4 for
// convolution and linear": int4 weights in an int8 container, qmin = -7,
// qmax = 7), with one fp32 scale s_n per output channel.
//
// The A operand holds the nibbles u as int8 (0..15), B the int8
// activations; D = sum u q, and one more MFMA per step with A = 1 gives
// sum q, so sum qw q = D - 8 * sum q, exactly, in int32.  The sum over the
// block's K splits is taken in int64, then scaled in fp64 in the order
// ((sum * s_m) * s_n) + bias and rounded once to the output type.
//
// Work split as in the skinny MFMA qGEMV: a block owns 32 weight rows (two
// 16-row tiles) and 16 activation rows (blockIdx.y); its 8 waves take every
// 8th 128-column block of K with one block's loads in flight ahead; each
// lane streams 16 bytes of codes per tile and 32 activations per block.
// With one scale per output channel no per-group work is needed, so the
// k order inside an MFMA step is free: lane group g of step t takes columns
// 32 g + 16 t .. + 16 in both operands.
#include <utility>

#include "device_common.hpp"
#include "qp_internal.hpp"

namespace qp {
namespace {

constexpr int kA8Rows = 32;
constexpr int kA8Waves = 8;
constexpr int kA8Cols = 128;
constexpr uint32_t kOOB = 0x80000000u;

struct A8Args {
  const void* qw;        // SYM4 nibbles u = q + 8, [N, K/8] u32
  const float* ws;       // [N] channel scales
  const int8_t* xq;      // [M, K]
  const float* xs;       // [M]
  const float* bias;     // [N] or null
  void* y;
  int64_t M, N, K;
  int ydt;
  uint32_t qw_bytes, xq_bytes;
};

typedef int int4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 nibbles (two words, k order) -> 16 int8 in k order.
__device__ __forceinline__ int4_t nibbles_to_i8(uint32_t wa, uint32_t wb) {
  const uint32_t la = wa & 0x0F0F0F0Fu, ha = (wa >> 4) & 0x0F0F0F0Fu;   // even / odd codes
  const uint32_t lb = wb & 0x0F0F0F0Fu, hb = (wb >> 4) & 0x0F0F0F0Fu;
  return int4_t{(int)__builtin_amdgcn_perm(ha, la, 0x05010400u),   // codes 0..3
                (int)__builtin_amdgcn_perm(ha, la, 0x07030602u),   // codes 4..7
                (int)__builtin_amdgcn_perm(hb, lb, 0x05010400u),   // codes 8..11
                (int)__builtin_amdgcn_perm(hb, lb, 0x07030602u)};  // codes 12..15
}

struct A8Stage {
  uint4 w[2];     // codes of the lane's two rows, 32 columns each
  uint4 x[2];     // 16 activations per MFMA step
};

__device__ __forceinline__ void a8_load(const A8Args& a, int kb, int lane, int64_t n0, int64_t mrow,
                                        A8Stage& s) {
  const uint32_t c0 = (uint32_t)kb * kA8Cols;
  const int g = lane >> 4, r16 = lane & 15;
  const uint32_t K = (uint32_t)a.K;
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.xq, a.xq_bytes);
  const uint32_t xo = mrow < a.M ? (uint32_t)mrow * K + c0 + 32u * g : kOOB;
#pragma unroll
  for (int t = 0; t < 2; ++t)
    s.x[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rx, xo == kOOB ? kOOB : xo + 16u * t, 0, 0));
  const __amdgpu_buffer_rsrc_t rq = rsrc(a.qw, a.qw_bytes);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = n0 + 16 * i + r16;
    const uint32_t off = n < a.N ? (uint32_t)n * (K / 2u) + (c0 + 32u * g) / 2u : kOOB;
    s.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 2));
  }
}

template <typename F, int... I>
__device__ __forceinline__ void sfor_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>{});
}

__global__ void __launch_bounds__(64 * kA8Waves) k_a8w4(A8Args a) {
  __shared__ int s_part[kA8Waves][2][16][17];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * kA8Rows;
  const int64_t mrow = (int64_t)blockIdx.y * 16 + r16;
  const int KB = (int)(a.K / kA8Cols);
  const int4_t ONES = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  int4_t D[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  int4_t DX = {0, 0, 0, 0};

  auto compute = [&](const A8Stage& s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int4_t B = __builtin_bit_cast(int4_t, s.x[t]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t wa = t == 0 ? s.w[i].x : s.w[i].z, wb = t == 0 ? s.w[i].y : s.w[i].w;
        D[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(nibbles_to_i8(wa, wb), B, D[i], 0, 0, 0);
      }
      DX = __builtin_amdgcn_mfma_i32_16x16x64_i8(ONES, B, DX, 0, 0, 0);
    }
  };

  A8Stage st[2];
  const int J = wave < KB ? (KB - wave + kA8Waves - 1) / kA8Waves : 0;
  if (J > 0) a8_load(a, wave, lane, n0, mrow, st[0]);
  for (int j0 = 0; j0 < J; j0 += 2) {
    sfor<2>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const int j = j0 + q;
      if (j < J) {
        if (j + 1 < J) a8_load(a, wave + (j + 1) * kA8Waves, lane, n0, mrow, st[(q + 1) % 2]);
        compute(st[q]);
      }
    });
  }
  // sum qw q = sum u q - 8 sum q (per wave: |.| <= (K / 8) * 127 * 7, int32)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) s_part[wave][i][4 * g + v][r16] = D[i][v] - 8 * DX[v];
  __syncthreads();
  const int nl = tid >> 4, m = tid & 15;
  const int64_t n = n0 + nl;
  const int64_t mm = (int64_t)blockIdx.y * 16 + m;
  if (mm < a.M && n < a.N) {
    int64_t sum = 0;
#pragma unroll
    for (int w = 0; w < kA8Waves; ++w) sum += s_part[w][nl >> 4][nl & 15][m];
    double v = (double)sum * (double)a.xs[mm] * (double)a.ws[n];
    if (a.bias) v += (double)a.bias[n];
    const float f = (float)v;
    const int64_t idx = mm * a.N + n;
    if (a.ydt == F32) static_cast<float*>(a.y)[idx] = f;
    else static_cast<uint16_t*>(a.y)[idx] =
        (uint16_t)(a.ydt == BF16 ? f32_to_bf16_rne(f) : f32_to_f16_rne(f));
  }
}

}  // namespace

hipError_t launch_a8w4(const Desc& d, const void* xq, const float* xs, int64_t M, const Bufs& b,
                       const float* bias, void* y, int ydt, hipStream_t s) {
  A8Args a{};
  a.qw = b.qweight;
  a.ws = static_cast<const float*>(b.scales);
  a.xq = static_cast<const int8_t*>(xq);
  a.xs = xs;
  a.bias = bias;
  a.y = y;
  a.M = M;
  a.N = d.N;
  a.K = d.K;
  a.ydt = ydt;
  a.qw_bytes = (uint32_t)((uint64_t)d.N * d.K / 2);
  a.xq_bytes = (uint32_t)((uint64_t)M * d.K);
  const unsigned blocks = (unsigned)((d.N + kA8Rows - 1) / kA8Rows);
  const unsigned mtiles = (unsigned)((M + 15) / 16);
  hipLaunchKernelGGL(k_a8w4, dim3(blocks, mtiles), dim3(64 * kA8Waves), 0, s, a);
  return hipGetLastError();
}

}  // namespace qp
