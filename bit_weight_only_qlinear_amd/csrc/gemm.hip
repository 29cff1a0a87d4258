// qGEMM: prefill-shaped quantized linear, y = x W^T for large M, on gfx950
// fp16 MFMA (v_mfma_f32_32x32x16_f16), fp32 accumulation.
//
// The pages' prefill ran on dequantized bf16 "runtime weights" (superscale
// page, A100 take-aways); here the packed codes stay in HBM and each block
// dequantizes its weight tile on the way into LDS.  The tile is rounded once
// to fp16 rather than bf16: bf16 keeps 8 significant bits, which is not
// enough for the output tolerance of this layer, fp16 keeps 11, and gfx950
// runs fp16 and bf16 MFMA at the same rate.  Activations are converted from
// bf16 to fp16 in the same staging step (exact for magnitudes in
// [2^-17, 65504]).
//
// Every format dequantizes as w = fma(u, S, T) per group in fp32, with u the
// stored unsigned field and (S, T) derived from the group metadata:
//   AFFINE: S = scale, T = bias;  Q4K: S = sc*sstep, T = -S*zc*zstep;
//   Q6K: S = sc*step, T = -32*S;  SYM4: S = scale, T = -8*S.
#include "device_common.hpp"
#include "qp_internal.hpp"

namespace qp {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDA = BK + 8;  // padded LDS row (halves): 144 B, breaks bank aliasing

struct GemmArgs {
  const uint32_t* qw;
  const uint32_t* qh;
  const void* scales;
  const void* zeros;
  const void* steps;
  const uint16_t* x;
  const uint16_t* bias;
  void* y;
  int64_t M, N, K;
  int fmt, bits, gs, meta_bf16, xbf16, ydt;
  int tilesM, tilesN;
};

__device__ __forceinline__ float xval(uint32_t bits, int xbf16) {
  return xbf16 ? bf16_to_f32(bits) : f16_to_f32(bits);
}

// Per-group (S, T) of the weight row n at column k.
__device__ __forceinline__ void group_st(const GemmArgs& a, int64_t n, int64_t k, float& S,
                                         float& T) {
  if (a.fmt == AFFINE) {
    const int64_t g = n * (a.K / a.gs) + k / a.gs;
    S = meta_to_f32(static_cast<const uint16_t*>(a.scales)[g], a.meta_bf16);
    T = meta_to_f32(static_cast<const uint16_t*>(a.zeros)[g], a.meta_bf16);
  } else if (a.fmt == Q4K) {
    const int64_t g = n * (a.K / 32) + k / 32;
    const uint32_t st = static_cast<const uint32_t*>(a.steps)[n * (a.K / 256) + k / 256];
    S = (float)static_cast<const uint8_t*>(a.scales)[g] * f16_to_f32(st & 0xFFFFu);
    const float Z = (float)static_cast<const uint8_t*>(a.zeros)[g] * f16_to_f32(st >> 16);
    T = -S * Z;
  } else if (a.fmt == Q6K) {
    const int64_t g = n * (a.K / 16) + k / 16;
    const float step = f16_to_f32(static_cast<const uint16_t*>(a.steps)[n * (a.K / 256) + k / 256]);
    S = (float)static_cast<const int8_t*>(a.scales)[g] * step;
    T = -32.f * S;
  } else {
    S = static_cast<const float*>(a.scales)[n * (a.K / a.gs) + k / a.gs];
    T = -8.f * S;
  }
}

// 32 consecutive codes (row n, columns k..k+31) as unsigned fields.
struct Codes32 {
  uint32_t w[8];   // packed words (meaning depends on bits)
  uint32_t h[2];   // Q6K high plane
};

__device__ __forceinline__ void load_codes(const GemmArgs& a, int64_t n, int64_t k, bool ok,
                                           Codes32& c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c.w[i] = 0;
  c.h[0] = c.h[1] = 0;
  if (!ok) return;
  const int b = a.fmt == Q6K ? 4 : a.bits;
  const uint32_t* src = a.qw + (n * a.K + k) * b / 32;
  if (b == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(src);
    c.w[0] = v.x; c.w[1] = v.y;
  } else if (b == 4) {
    uint4 v = *reinterpret_cast<const uint4*>(src);
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  } else {
    uint4 v0 = reinterpret_cast<const uint4*>(src)[0];
    uint4 v1 = reinterpret_cast<const uint4*>(src)[1];
    c.w[0] = v0.x; c.w[1] = v0.y; c.w[2] = v0.z; c.w[3] = v0.w;
    c.w[4] = v1.x; c.w[5] = v1.y; c.w[6] = v1.z; c.w[7] = v1.w;
  }
  if (a.fmt == Q6K) {
    uint2 v = *reinterpret_cast<const uint2*>(a.qh + (n * a.K + k) / 16);
    c.h[0] = v.x; c.h[1] = v.y;
  }
}

__device__ __forceinline__ uint32_t field(const GemmArgs& a, const Codes32& c, int i) {
  if (a.fmt == Q6K)
    return ((c.w[i / 8] >> (4 * (i % 8))) & 15u) | (((c.h[i / 16] >> (2 * (i % 16))) & 3u) << 4);
  if (a.bits == 4) return (c.w[i / 8] >> (4 * (i % 8))) & 15u;
  if (a.bits == 2) return (c.w[i / 16] >> (2 * (i % 16))) & 3u;
  return (c.w[i / 4] >> (8 * (i % 4))) & 255u;
}

__global__ void __launch_bounds__(256) k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order: consecutive block ids land on different XCDs, so
  // give each XCD a contiguous run of tiles (m fastest) to share L2.
  const int T = a.tilesM * a.tilesN;
  const int bid = blockIdx.x;
  const int tile = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;  // a bijection
  const int tm = tile % a.tilesM, tn = tile / a.tilesM;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  // staging assignment: thread -> (row, 32-column half) of both tiles
  const int sr = tid >> 1;           // 0..127
  const int sk = (tid & 1) * 32;     // 0 or 32
  const int64_t xm = m0 + sr, wn_row = n0 + sr;
  const bool xok = xm < a.M, wok = wn_row < a.N;

  uint4 xr[4];
  Codes32 cr;
  float gS, gT;

  auto gload = [&](int64_t k0) {
    const uint16_t* xp = a.x + xm * a.K + k0 + sk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xr[i] = xok ? reinterpret_cast<const uint4*>(xp)[i] : make_uint4(0, 0, 0, 0);
    load_codes(a, wok ? wn_row : 0, k0 + sk, wok, cr);
    if (wok) group_st(a, wn_row, k0 + sk, gS, gT);
    else { gS = 0.f; gT = 0.f; }
  };

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (int)(a.K / BK);
  gload(0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
    // ---- stage activations (bf16|fp16 -> fp16) and weights (-> fp16)
    {
      _Float16* ad = As + sr * LDA + sk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
        half8_t h;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          h[t] = (_Float16)xval((u[t / 2] >> (16 * (t % 2))) & 0xFFFFu, a.xbf16);
        *reinterpret_cast<half8_t*>(ad + 8 * i) = h;
      }
      _Float16* bd = Bs + sr * LDA + sk;
      // groups of 16 (Q6K) may change inside the 32 columns
      float S1 = gS, T1 = gT;
      if (a.fmt == Q6K && wok) group_st(a, wn_row, (int64_t)kt * BK + sk + 16, S1, T1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half8_t h;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int e = 8 * i + t;
          const float S = e < 16 ? gS : S1, T = e < 16 ? gT : T1;
          h[t] = (_Float16)fmaf((float)field(a, cr, e), S, T);
        }
        *reinterpret_cast<half8_t*>(bd + 8 * i) = h;
      }
    }
    __syncthreads();
    if (kt + 1 < KT) gload((int64_t)(kt + 1) * BK);

    // ---- MFMA over the 4 K-slices of 16
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      half8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const half8_t*>(As + row * LDA + kk * 16 + 8 * (lane >> 5));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const half8_t*>(Bs + row * LDA + kk * 16 + 8 * (lane >> 5));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: D[i][j] of a 32x32 tile sits in lane (j + 32*((i/4)%2)),
  // register 4*(i/8) + i%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= a.N) continue;
      const float bv = a.bias ? xval(a.bias[n], a.xbf16) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (m >= a.M) continue;
        const float v = acc[i][j][r] + bv;
        const int64_t idx = m * a.N + n;
        if (a.ydt == F32) static_cast<float*>(a.y)[idx] = v;
        else if (a.ydt == BF16) static_cast<uint16_t*>(a.y)[idx] = (uint16_t)f32_to_bf16_rne(v);
        else static_cast<uint16_t*>(a.y)[idx] = (uint16_t)f32_to_f16_rne(v);
      }
    }
}

}  // namespace

hipError_t launch_gemm(const Desc& d, const void* x, int xdt, int64_t M, const Bufs& b,
                       const void* bias, void* y, int ydt, hipStream_t s) {
  GemmArgs a;
  a.qw = static_cast<const uint32_t*>(b.qweight);
  a.qh = static_cast<const uint32_t*>(b.qweight_hi);
  a.scales = b.scales;
  a.zeros = b.zeros;
  a.steps = b.steps;
  a.x = static_cast<const uint16_t*>(x);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = y;
  a.M = M;
  a.N = d.N;
  a.K = d.K;
  a.fmt = d.fmt;
  a.bits = d.bits;
  a.gs = d.gs;
  a.meta_bf16 = d.meta == BF16;
  a.xbf16 = xdt == BF16;
  a.ydt = ydt;
  a.tilesM = (int)((M + BM - 1) / BM);
  a.tilesN = (int)((d.N + BN - 1) / BN);
  const unsigned blocks = (unsigned)a.tilesM * (unsigned)a.tilesN;
  hipLaunchKernelGGL(k_gemm, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qp
