// qGEMM host side: activation staging (the bf16 prescale exponents and the
// fp16 fragments, into the workspace, for the 224-row tiles; the exponents
// alone, into y, for the 256-row tiles), the tiling choice and the dispatch to the
// per-format kernel instantiations.  The kernels and their design are in
// gemm_kernels.hpp.
#include "gemm_kernels.hpp"

namespace qp {
namespace {

// Staging for k_gemm224.  Every bf16 row gets a prescale exponent
// e = 14 - floor(log2 max|x|) (0 for an all-zero row or a padding row),
// which scales the row's peak into [2^14, 2^15) -- inside fp16's range --
// stored in xe[row] (rows up to the next multiple of 16), and x [M, K]
// (bf16 or fp16) goes to fp16 in the B-fragment order of
// v_mfma_f32_16x16x32_f16: 16-byte chunk c = (mb * K/32 + kq) * 64 + l
// holds row 16 mb + (l & 15), columns 32 kq + 8 (l >> 4) .. + 7 in the
// order (0,4,1,5,2,6,3,7), bf16 rows scaled by 2^e; rows from M up to the
// next multiple of 16 are zero.  k_xmax (one wave per row: the exponent)
// then k_xprep (the conversion) for any K; k_xstage and k_xstage8 do both
// in one pass over x where a wave can hold a whole row (at M = 2048,
// K = 4096: 8.96 us, against 10.46 for k_xstage and 4.8 + 6.7 for the two
// passes; a block that read each 16-row group twice took 14.7).
__global__ void __launch_bounds__(256) k_xmax(const uint16_t* __restrict__ x, int* __restrict__ xe,
                                              uint32_t M, uint32_t K, uint32_t Mpad) {
  const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6), l = threadIdx.x & 63u;
  if (row >= Mpad) return;   // whole waves: the row is uniform across the wave
  uint32_t mx = 0;           // |bf16| compares as its bit pattern with the sign cleared
  if (row < M) {
    const uint4* xw = reinterpret_cast<const uint4*>(x + (uint64_t)row * K);
#pragma unroll 8
    for (uint32_t c = l; c < K / 8u; c += 64u) {
      const uint4 u = xw[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) mx = max(mx, max(w[q] & 0x7FFFu, (w[q] >> 16) & 0x7FFFu));
    }
  }
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  const float f = bf16_to_f32(mx);
  if (l == 0) xe[row] = f == 0.f ? 0 : 14 - ilogbf(f);
}

template <bool XBF16>
__global__ void __launch_bounds__(256) k_xprep(const uint16_t* __restrict__ x, uint4* __restrict__ xf,
                                               const int* __restrict__ xe, uint32_t M, uint32_t K,
                                               uint32_t nchunks) {
  const uint32_t c = blockIdx.x * 256u + threadIdx.x;
  if (c >= nchunks) return;
  const uint32_t l = c & 63u, blk = c >> 6, kb = K / 32u;
  const uint32_t mb = blk / kb, kq = blk - mb * kb;
  const uint32_t row = 16u * mb + (l & 15u), col = 32u * kq + 8u * (l >> 4);
  uint4 u = make_uint4(0u, 0u, 0u, 0u);
  int e = 0;
  if (row < M) {
    u = *reinterpret_cast<const uint4*>(x + (uint64_t)row * K + col);
    if constexpr (XBF16) e = xe[row];
  }
  xf[c] = act_chunk<XBF16>(u, e);
}

// The two kernels above in one pass, for rows of up to NU * 512 columns:
// one wave per staged row holds the whole row in registers (NU 16-byte
// chunks per lane), takes its maximum, writes the exponent, converts and
// stores every chunk at its fragment position.  x is read once.  A 128-byte
// line of the fragments is written by 8 waves (rows), 16 bytes each, and
// completed in the L2.
template <bool XBF16, int NU>
__global__ void __launch_bounds__(256) k_xstage(const uint16_t* __restrict__ x, uint4* __restrict__ xf,
                                                int* __restrict__ xe, uint32_t M, uint32_t K,
                                                uint32_t Mpad) {
  const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6), l = threadIdx.x & 63u;
  if (row >= Mpad) return;   // whole waves: the row is uniform across the wave
  const uint32_t nq = K / 8u;   // 8-column chunks per row
  uint4 u[NU];
  uint32_t mx = 0;
  const uint4* xw = reinterpret_cast<const uint4*>(x + (uint64_t)row * K);
#pragma unroll
  for (int t = 0; t < NU; ++t) {
    const uint32_t q = l + 64u * t;
    u[t] = row < M && q < nq ? xw[q] : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (XBF16) {
      const uint32_t w[4] = {u[t].x, u[t].y, u[t].z, u[t].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) mx = max(mx, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
    }
  }
  int e = 0;
  if constexpr (XBF16) {
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    const float f = bf16_to_f32(mx);
    e = f == 0.f ? 0 : 14 - ilogbf(f);
    if (l == 0) xe[row] = e;
  }
  // chunk q of the row: fragment (row / 16, q / 4), lane (row % 16) + 16 (q % 4)
  const uint32_t base = (row / 16u) * (K / 32u) * 64u + (row % 16u);
#pragma unroll
  for (int t = 0; t < NU; ++t) {
    const uint32_t q = l + 64u * t;
    if (q < nq) xf[base + (q / 4u) * 64u + 16u * (q % 4u)] = act_chunk<XBF16>(u[t], e);
  }
}

// The same with 8 rows per block (K <= 4096): each wave converts its row as
// above, the block transposes the chunks through LDS, and every store
// instruction writes whole 128-byte lines (8 rows' chunks of one fragment
// column group).  LDS holds line L (fragment column group) position p at
// (8 L + p) * 16 with p = row ^ (L & 7), so that the 8 lanes of a write
// phase hit 8 different bank groups.
template <bool XBF16, int NU>
__global__ void __launch_bounds__(512) k_xstage8(const uint16_t* __restrict__ x, uint4* __restrict__ xf,
                                                 int* __restrict__ xe, uint32_t M, uint32_t K) {
  extern __shared__ __attribute__((aligned(16))) uint4 sx[];   // K / 8 lines' worth: K chunks
  const uint32_t w = threadIdx.x >> 6, l = threadIdx.x & 63u;
  const uint32_t row = blockIdx.x * 8u + w;
  const uint32_t nq = K / 8u;
  uint4 u[NU];
  uint32_t mx = 0;
  const uint4* xw = reinterpret_cast<const uint4*>(x + (uint64_t)row * K);
#pragma unroll
  for (int t = 0; t < NU; ++t) {
    const uint32_t q = l + 64u * t;
    u[t] = row < M && q < nq ? xw[q] : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (XBF16) {
      const uint32_t v[4] = {u[t].x, u[t].y, u[t].z, u[t].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) mx = max(mx, max(v[k] & 0x7FFFu, (v[k] >> 16) & 0x7FFFu));
    }
  }
  int e = 0;
  if constexpr (XBF16) {
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    const float f = bf16_to_f32(mx);
    e = f == 0.f ? 0 : 14 - ilogbf(f);
    if (l == 0) xe[row] = e;
  }
  // chunk q of this row belongs to line q (fragment q / 4, lanes 16 (q % 4) + ...)
#pragma unroll
  for (int t = 0; t < NU; ++t) {
    const uint32_t q = l + 64u * t;
    if (q < nq) sx[8u * q + (w ^ (q & 7u))] = act_chunk<XBF16>(u[t], e);
  }
  __syncthreads();
  // line L of the block: fragment L / 4, lanes 16 (L % 4) + r0 .. + 7
  const uint32_t r0 = (blockIdx.x * 8u) % 16u;
  const uint32_t base = (blockIdx.x * 8u / 16u) * (K / 32u) * 64u + r0;
#pragma unroll
  for (int t = 0; t < NU; ++t) {
    const uint32_t i = threadIdx.x + 512u * t;   // i < K: line i / 8, position i % 8
    if (i < K) {
      const uint32_t L = i / 8u, p = i % 8u;
      xf[base + (L / 4u) * 64u + 16u * (L % 4u) + (p ^ (L & 7u))] = sx[i];
    }
  }
}

// Prescale exponent of each bf16 activation row: e = 14 - floor(log2 of the
// row's largest magnitude) (0 for an all-zero row), so that every scaled row
// peaks in [2^14, 2^15) -- inside fp16's range, with fp16's full precision
// for everything within 2^-10 of the peak.  Written into y at the first
// column of every n-tile (tile width `colstep`), where the qGEMM block of
// that tile picks it up before it writes its outputs.  One block per row.
__global__ void __launch_bounds__(256) k_xexp(const uint16_t* __restrict__ x, int64_t K, void* y,
                                              int64_t N, int ydt, int colstep, int ntiles) {
  __shared__ float wm[4];
  const int64_t m = blockIdx.x;
  // K % 64 == 0 for the qGEMM: 16-byte loads of 8 bf16; |bf16| compares as
  // its bit pattern with the sign cleared
  const uint4* xr = reinterpret_cast<const uint4*>(x + m * K);
  uint32_t mb = 0;
  for (int64_t c = threadIdx.x; c < K / 8; c += 256) {
    const uint4 u = xr[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) mb = max(mb, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
  }
  float mx = bf16_to_f32(mb);
  mx = wave_max_all(mx);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  const int e = mx == 0.f ? 0 : 14 - ilogbf(mx);
  for (int t = threadIdx.x; t < ntiles; t += 256) {
    const int64_t i = m * N + (int64_t)t * colstep;
    if (ydt == F32) static_cast<int*>(y)[i] = e;
    else static_cast<int16_t*>(y)[i] = (int16_t)e;
  }
}

constexpr int64_t kCUs = 256;   // MI355X compute units

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 224-row tiles when they need less time than 256-row tiles counted in
// waves of blocks over the CUs (one block per CU at a time).
bool use_n224(const Desc& d, int64_t M) {
  const int64_t tm = cdiv(M, BM);
  return cdiv(tm * cdiv(d.N, BN7), kCUs) * BN7 < cdiv(tm * cdiv(d.N, BN), kCUs) * BN;
}

}  // namespace

// Staged activations (fp16 fragments), then one int32 prescale exponent per
// staged row.
static uint64_t staged_bytes(const Desc& d, int64_t M) {
  return (uint64_t)cdiv(M, 16) * 16u * (uint64_t)d.K * 2u;
}

size_t gemm_workspace_bytes(const Desc& d, int64_t M) {
  if (!use_n224(d, M)) return 0;
  const uint64_t bytes = staged_bytes(d, M);
  // 32-bit buffer offsets in k_gemm224
  if (bytes > (uint64_t(1) << 31)) return 0;
  return (size_t)(bytes + (uint64_t)cdiv(M, 16) * 16u * 4u);
}

hipError_t launch_gemm(const Desc& d, const void* x, int xdt, int64_t M, const Bufs& b,
                       const void* bias, void* y, int ydt, void* ws, hipStream_t s) {
  const size_t wsb = ws ? gemm_workspace_bytes(d, M) : 0;
  const bool n224 = wsb > 0;
  GemmArgs a;
  a.qw = b.qweight;
  a.qh = b.qweight_hi;
  a.scales = b.scales;
  a.zeros = b.zeros;
  a.steps = b.steps;
  a.x = x;
  a.xf = n224 ? ws : nullptr;
  a.xe = n224 ? reinterpret_cast<const int*>(static_cast<const unsigned char*>(ws) +
                                            staged_bytes(d, M))
              : nullptr;
  a.bias = bias;
  a.y = y;
  a.M = M;
  a.N = d.N;
  a.K = d.K;
  a.gs = d.gs;
  a.ydt = ydt;
  a.tilesM = (int)((M + BM - 1) / BM);
  a.tilesN = (int)cdiv(d.N, n224 ? BN7 : BN);
  if (n224) {   // staging (with the bf16 prescale exponents) into the workspace
    int* xe = const_cast<int*>(a.xe);
    const uint32_t mpad = (uint32_t)(cdiv(M, 16) * 16), nch = (uint32_t)(staged_bytes(d, M) / 16u);
    // bf16: one pass over x (8 rows per block up to K = 4096, one wave per
    // row up to 8192), else the exponent pass and the conversion pass
    const int64_t nu = cdiv(d.K, 512);   // 16-byte chunks per lane for one wave per row
    if (xdt == BF16 && d.K <= 4096) {
      auto fn = nu <= 1 ? k_xstage8<true, 1> : nu <= 2 ? k_xstage8<true, 2> : nu <= 4 ? k_xstage8<true, 4>
              : k_xstage8<true, 8>;
      hipLaunchKernelGGL(fn, dim3(mpad / 8), dim3(512), (unsigned)(d.K * 16), s,
                         static_cast<const uint16_t*>(x), static_cast<uint4*>(ws), xe, (uint32_t)M,
                         (uint32_t)d.K);
    } else if (xdt == BF16 && nu <= 16) {
      auto fn = nu <= 1 ? k_xstage<true, 1> : nu <= 2 ? k_xstage<true, 2> : nu <= 4 ? k_xstage<true, 4>
              : nu <= 8 ? k_xstage<true, 8> : k_xstage<true, 16>;
      hipLaunchKernelGGL(fn, dim3((mpad + 3) / 4), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                         static_cast<uint4*>(ws), xe, (uint32_t)M, (uint32_t)d.K, mpad);
    } else if (xdt == BF16) {
      hipLaunchKernelGGL(k_xmax, dim3((mpad + 3) / 4), dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), xe, (uint32_t)M, (uint32_t)d.K, mpad);
      hipLaunchKernelGGL(k_xprep<true>, dim3((nch + 255) / 256), dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), static_cast<uint4*>(ws), xe,
                         (uint32_t)M, (uint32_t)d.K, nch);
    } else {
      hipLaunchKernelGGL(k_xprep<false>, dim3((nch + 255) / 256), dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), static_cast<uint4*>(ws), xe,
                         (uint32_t)M, (uint32_t)d.K, nch);
    }
  } else if (xdt == BF16) {   // per-row prescale exponents into y (see k_xexp)
    hipLaunchKernelGGL(k_xexp, dim3((unsigned)M), dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       d.K, y, d.N, ydt, BN, a.tilesN);
  }
  const unsigned blocks = (unsigned)a.tilesM * (unsigned)a.tilesN;
  GemmPick p;
  p.n224 = n224;
  p.xb = xdt == BF16;
  p.mb = d.meta == BF16;
  // chunked affine metadata: whole 8-group chunks per row (16-byte aligned)
  p.mch = d.fmt == AFFINE && ((d.gs == 64 && d.K % 512 == 0) || (d.gs == 32 && d.K % 256 == 0) ||
                              (d.gs == 128 && d.K % 1024 == 0));
  if (d.fmt == AFFINE)
    return d.bits == 2 ? gemm_launch_aff2(a, p, blocks, s)
         : d.bits == 4 ? gemm_launch_aff4(a, p, blocks, s) : gemm_launch_aff8(a, p, blocks, s);
  return gemm_launch_kq(d.fmt, a, p, blocks, s);
}

}  // namespace qp
