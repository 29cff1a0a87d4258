// qGEMV: decode-shaped quantized linear, y[m, :] = x[m, :] W^T for M <= 8.
//
// Design (gfx950, wave64):
//  * The packed codes of a row are streamed in 16-byte chunks; lane l of a
//    wave always owns the chunks c = cbase + j*64 + l (j < CPL), so every
//    load instruction reads 1 KiB of contiguous codes and the lane's slice
//    of the activations is loaded once into registers and reused for every
//    row the wave visits.
//  * Codes are turned into bf16 (or fp16) pairs without a conversion
//    instruction: OR-ing a small integer q into the mantissa of 128.0 bf16
//    (1024.0 fp16) gives exactly 128 + q (1024 + q).  One v_dot2 per pair
//    accumulates sum (MAG + q) * x in fp32; the MAG * sum(x) part is removed
//    in the per-group epilogue, where the group's scale and offset are
//    applied once per chunk in fp32:
//        sum_k w_k x_k = S * sum (MAG + q) x - S * (MAG + Z) * sum x
//    (AFFINE: S = scale, S*Z = -bias; Q4K: S = sc*sstep, Z = zc*zstep;
//    Q6K: Z = 32, SYM4: Z = 8 from the stored code offsets).  8-bit codes use
//    byte-to-fp32 conversions and fp32 FMAs instead (128 + 255 is not exact
//    in bf16).
//  * Q4K / Q6K fp16 steps are shared by the 8 lanes that cover one
//    256-weight super-block: the first lane of each 8 loads the step word and
//    ds_swizzle (bit mode, and-mask 0x18) hands it to the other seven --
//    the superscale page's "one shuffle per super-block" on wave64.
//  * Partial sums of a row are reduced across the wave with DPP row
//    rotations and row broadcasts; when a row's K range is split over KW
//    waves of the block, the wave partials meet in LDS.
//
// Formats: see include/qlinear.h.  Sources: HF Transformers "Metal" page
// (uint32 codes, per-group scale/bias, bits 2/4/8); ExecuTorch PR #20571
// "Quant schema update" (Q4_K/Q6_K-style nested metadata; the int6 per-group
// int8 scale codes are loaded once per 16-byte code load); ExecuTorch PR
// #16577 (symmetric int4, qmin=-7..7).
#include "device_common.hpp"
#include "qp_internal.hpp"

namespace qp {
namespace {

enum Kind : int { K_AFF2 = 0, K_AFF4 = 1, K_AFF8 = 2, K_Q4K = 3, K_Q6K = 4, K_SYM4 = 5 };

template <int KIND>
struct KT;
template <>
struct KT<K_AFF2> { static constexpr int CC = 64, XW = 32, GP = 2; };
template <>
struct KT<K_AFF4> { static constexpr int CC = 32, XW = 16, GP = 1; };
template <>
struct KT<K_AFF8> { static constexpr int CC = 16, XW = 16, GP = 1; };
template <>
struct KT<K_Q4K> { static constexpr int CC = 32, XW = 16, GP = 1; };
template <>
struct KT<K_Q6K> { static constexpr int CC = 32, XW = 16, GP = 2; };
template <>
struct KT<K_SYM4> { static constexpr int CC = 32, XW = 16, GP = 1; };

struct GemvArgs {
  const uint32_t* qw;     // [N, C*4] u32 (16-byte chunks)
  const uint32_t* qh;     // Q6K high plane [N, K/16] u32
  const void* scales;
  const void* zeros;
  const void* steps;
  const uint16_t* x;      // [M, K] fp16|bf16 bits
  const uint16_t* bias;   // [N] or null, x dtype
  void* y;                // [M, N]
  int64_t N, K, M;
  int C;                  // 16-byte chunks per row
  int gs;
  int meta_bf16;
  int ydt;
  int KW;                 // waves splitting K per row team
  int RPT;                // rows per team
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <bool XBF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (XBF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                  __builtin_bit_cast(f16x2_t, b), c, false);
}

template <bool XBF16>
__device__ __forceinline__ float xval(uint32_t bits) {
  return XBF16 ? bf16_to_f32(bits) : f16_to_f32(bits);
}

__device__ __forceinline__ uint32_t bcast8(uint32_t v) {
  // every lane takes the value of the first lane of its group of 8
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x0018);
}

__device__ __forceinline__ void store_y(void* y, int64_t idx, float v, int ydt) {
  if (ydt == F32)
    static_cast<float*>(y)[idx] = v;
  else if (ydt == BF16)
    static_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
  else
    static_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_f16_rne(v);
}

template <int KIND, bool XBF16, int MT, int CPL>
__global__ void __launch_bounds__(256) k_gemv(GemvArgs a) {
  using T = KT<KIND>;
  constexpr int CC = T::CC, XW = T::XW, GP = T::GP;
  constexpr int RB0 = CPL >= 4 ? 1 : (CPL >= 2 ? 2 : 4);
  constexpr int RB = MT >= 4 ? (RB0 > 1 ? RB0 / 2 : 1) : RB0;
  constexpr uint32_t MAG = XBF16 ? 0x43004300u : 0x64006400u;
  constexpr float MAGF = XBF16 ? 128.f : 1024.f;

  __shared__ float red[4][RB][MT];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int KW = a.KW;
  const int kw = wave % KW;
  const int team = wave / KW;
  const int RW = 4 / KW;
  const int64_t row0 = ((int64_t)blockIdx.x * RW + team) * a.RPT;
  const int64_t rowEnd = min(row0 + a.RPT, a.N);
  const int mbase = blockIdx.y * MT;
  const int C = a.C;
  const int cbase = kw * CPL * 64;

  // ---- activations of this lane's chunks, as pairs matching the code pairs
  uint32_t xq[CPL][MT][XW];
  float xs[CPL][MT][GP];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = cbase + j * 64 + lane;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool ok = c < C && (mbase + m) < a.M;
      const uint16_t* xr = a.x + (int64_t)(mbase + m) * a.K + (int64_t)c * CC;
#pragma unroll
      for (int p = 0; p < GP; ++p) xs[j][m][p] = 0.f;
      if constexpr (KIND == K_AFF8) {
#pragma unroll
        for (int i = 0; i < 16; i += 8) {
          uint4 v = ok ? *reinterpret_cast<const uint4*>(xr + i) : make_uint4(0, 0, 0, 0);
          uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            uint32_t bits = (u[t / 2] >> (16 * (t % 2))) & 0xFFFFu;
            xq[j][m][i + t] = __float_as_uint(xval<XBF16>(bits));
            xs[j][m][0] += xval<XBF16>(bits);
          }
        }
      } else {
        constexpr int PW = (KIND == K_AFF2) ? 8 : 4;   // pairs per word
        constexpr int CW = 2 * PW;                      // codes per word
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t u[CW / 2];
#pragma unroll
          for (int t = 0; t < CW / 8; ++t) {
            uint4 v = ok ? *reinterpret_cast<const uint4*>(xr + w * CW + 8 * t)
                         : make_uint4(0, 0, 0, 0);
            u[4 * t] = v.x; u[4 * t + 1] = v.y; u[4 * t + 2] = v.z; u[4 * t + 3] = v.w;
          }
#pragma unroll
          for (int s = 0; s < PW; ++s) {
            // pair s = (code s, code s + PW) of the word
            uint32_t lo = (u[s / 2] >> (16 * (s % 2))) & 0xFFFFu;
            uint32_t hi = (u[(s + PW) / 2] >> (16 * ((s + PW) % 2))) & 0xFFFFu;
            xq[j][m][w * PW + s] = lo | (hi << 16);
            const int part = (GP == 2) ? (w / 2) : 0;
            xs[j][m][part] += xval<XBF16>(lo) + xval<XBF16>(hi);
          }
        }
      }
    }
  }

  const int64_t rowWords = (int64_t)C * 4;
  const int ng = (int)(a.K / a.gs);

  for (int64_t r = row0; r < row0 + a.RPT; r += RB) {
    if (r >= rowEnd && KW == 1) break;
    float yacc[RB][MT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int m = 0; m < MT; ++m) yacc[rb][m] = 0.f;

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t n = min(r + rb, a.N - 1);   // always a valid row index
      const bool rowok = (r + rb) < rowEnd;
      // ---- loads for this row
      uint4 cw[CPL];
      uint2 hw[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = cbase + j * 64 + lane;
        const bool ok = c < C && rowok;
        cw[j] = ok ? *reinterpret_cast<const uint4*>(a.qw + n * rowWords + (int64_t)c * 4)
                   : make_uint4(0, 0, 0, 0);
        if constexpr (KIND == K_Q6K)
          hw[j] = ok ? *reinterpret_cast<const uint2*>(a.qh + n * (a.K / 16) + (int64_t)c * 2)
                     : make_uint2(0, 0);
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = cbase + j * 64 + lane;
        const bool ok = c < C && rowok;
        const int cs = ok ? c : 0;
        float S[GP], Tt[GP];
        if constexpr (KIND == K_AFF2 || KIND == K_AFF4 || KIND == K_AFF8) {
#pragma unroll
          for (int p = 0; p < GP; ++p) {
            const int g = (cs * CC + p * (CC / GP)) / a.gs;
            const uint32_t sb = static_cast<const uint16_t*>(a.scales)[n * ng + g];
            const uint32_t bb = static_cast<const uint16_t*>(a.zeros)[n * ng + g];
            const float s = meta_to_f32(sb, a.meta_bf16), b = meta_to_f32(bb, a.meta_bf16);
            S[p] = s;
            Tt[p] = (KIND == K_AFF8) ? b : b - MAGF * s;
          }
        } else if constexpr (KIND == K_Q4K) {
          const uint32_t scb = static_cast<const uint8_t*>(a.scales)[n * (a.K / 32) + cs];
          const uint32_t zcb = static_cast<const uint8_t*>(a.zeros)[n * (a.K / 32) + cs];
          uint32_t st = 0;
          if ((lane & 7) == 0)
            st = static_cast<const uint32_t*>(a.steps)[n * (a.K / 256) + cs / 8];
          st = bcast8(st);
          const float Sv = (float)scb * f16_to_f32(st & 0xFFFFu);
          const float Z = (float)zcb * f16_to_f32(st >> 16);
          S[0] = Sv;
          Tt[0] = -Sv * (MAGF + Z);
        } else if constexpr (KIND == K_Q6K) {
          const uint32_t sc2 = static_cast<const uint16_t*>(a.scales)[n * (a.K / 32) + cs];
          uint32_t st = 0;
          if ((lane & 7) == 0)
            st = static_cast<const uint16_t*>(a.steps)[n * (a.K / 256) + cs / 8];
          st = bcast8(st);
          const float step = f16_to_f32(st);
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float Sv = (float)(int)(int8_t)(sc2 >> (8 * p)) * step;
            S[p] = Sv;
            Tt[p] = -Sv * (MAGF + 32.f);
          }
        } else {  // SYM4
          const float s = static_cast<const float*>(a.scales)[n * ng + (cs * CC) / a.gs];
          S[0] = s;
          Tt[0] = -s * (MAGF + 8.f);
        }

        // ---- dot products of this chunk
        float acc[MT][GP];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int p = 0; p < GP; ++p) acc[m][p] = 0.f;
        const uint32_t wv[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
        if constexpr (KIND == K_AFF8) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float q = (float)((wv[i] >> (8 * t)) & 0xFFu);
#pragma unroll
              for (int m = 0; m < MT; ++m)
                acc[m][0] = fmaf(q, __uint_as_float(xq[j][m][4 * i + t]), acc[m][0]);
            }
        } else if constexpr (KIND == K_AFF2) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const uint32_t pr = ((wv[i] >> (2 * s)) & 0x00030003u) | MAG;
#pragma unroll
              for (int m = 0; m < MT; ++m)
                acc[m][i / 2] = dot2<XBF16>(pr, xq[j][m][8 * i + s], acc[m][i / 2]);
            }
        } else if constexpr (KIND == K_Q6K) {
          const uint32_t h0 = __builtin_amdgcn_perm(hw[j].x, hw[j].x, 0x03010200u);
          const uint32_t h1 = __builtin_amdgcn_perm(hw[j].y, hw[j].y, 0x03010200u);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t hh = (i < 2 ? h0 : h1) >> (8 * (i % 2));
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const uint32_t pr = ((wv[i] >> (4 * s)) & 0x000F000Fu) |
                                  (((hh >> (2 * s)) & 0x00030003u) << 4) | MAG;
#pragma unroll
              for (int m = 0; m < MT; ++m)
                acc[m][i / 2] = dot2<XBF16>(pr, xq[j][m][4 * i + s], acc[m][i / 2]);
            }
          }
        } else {  // nibbles: AFF4, Q4K, SYM4
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const uint32_t pr = ((wv[i] >> (4 * s)) & 0x000F000Fu) | MAG;
#pragma unroll
              for (int m = 0; m < MT; ++m)
                acc[m][0] = dot2<XBF16>(pr, xq[j][m][4 * i + s], acc[m][0]);
            }
        }
        if (ok) {
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int p = 0; p < GP; ++p)
              yacc[rb][m] = fmaf(Tt[p], xs[j][m][p], fmaf(S[p], acc[m][p], yacc[rb][m]));
        }
      }
    }

    // ---- reduce across the wave (and across the KW waves of the team)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int m = 0; m < MT; ++m) yacc[rb][m] = wave_sum_lane63(yacc[rb][m]);

    if (KW == 1) {
      if (lane == 63) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int64_t n = r + rb;
          if (n >= rowEnd) break;
          const float bv = a.bias ? xval<XBF16>(a.bias[n]) : 0.f;
#pragma unroll
          for (int m = 0; m < MT; ++m)
            if (mbase + m < a.M)
              store_y(a.y, (int64_t)(mbase + m) * a.N + n, yacc[rb][m] + bv, a.ydt);
        }
      }
    } else {
      if (lane == 63) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int m = 0; m < MT; ++m) red[wave][rb][m] = yacc[rb][m];
      }
      __syncthreads();
      if (kw == 0 && lane < RB * MT) {
        const int rb = lane / MT, m = lane % MT;
        float v = 0.f;
        for (int q = 0; q < KW; ++q) v += red[wave + q][rb][m];
        const int64_t n = r + rb;
        if (n < rowEnd && mbase + m < a.M) {
          const float bv = a.bias ? xval<XBF16>(a.bias[n]) : 0.f;
          store_y(a.y, (int64_t)(mbase + m) * a.N + n, v + bv, a.ydt);
        }
      }
      __syncthreads();
    }
  }
}

typedef void (*GemvFn)(GemvArgs);

template <int KIND, bool XB, int MT>
GemvFn pick_cpl(int cpl) {
  switch (cpl) {
    case 1: return k_gemv<KIND, XB, MT, 1>;
    case 2: return MT <= 4 ? (GemvFn)k_gemv<KIND, XB, (MT <= 4 ? MT : 4), 2> : nullptr;
    case 3: return MT <= 2 ? (GemvFn)k_gemv<KIND, XB, (MT <= 2 ? MT : 2), 3> : nullptr;
    case 4: return MT <= 2 ? (GemvFn)k_gemv<KIND, XB, (MT <= 2 ? MT : 2), 4> : nullptr;
  }
  return nullptr;
}

template <int KIND, bool XB>
GemvFn pick_mt(int mt, int cpl) {
  switch (mt) {
    case 1: return pick_cpl<KIND, XB, 1>(cpl);
    case 2: return pick_cpl<KIND, XB, 2>(cpl);
    case 4: return pick_cpl<KIND, XB, 4>(cpl);
    case 8: return pick_cpl<KIND, XB, 8>(cpl);
  }
  return nullptr;
}

template <int KIND>
GemvFn pick_x(bool xb, int mt, int cpl) {
  return xb ? pick_mt<KIND, true>(mt, cpl) : pick_mt<KIND, false>(mt, cpl);
}

GemvFn pick(int kind, bool xb, int mt, int cpl) {
  switch (kind) {
    case K_AFF2: return pick_x<K_AFF2>(xb, mt, cpl);
    case K_AFF4: return pick_x<K_AFF4>(xb, mt, cpl);
    case K_AFF8: return pick_x<K_AFF8>(xb, mt, cpl);
    case K_Q4K: return pick_x<K_Q4K>(xb, mt, cpl);
    case K_Q6K: return pick_x<K_Q6K>(xb, mt, cpl);
    case K_SYM4: return pick_x<K_SYM4>(xb, mt, cpl);
  }
  return nullptr;
}

// Chooses the M tile, the K split and the chunks per lane so that the
// lane's activations fit the register budget (CPL * MT <= 8 u32 pairs
// blocks of 16; <= 4 for 2-bit codes).  Shrinks the M tile if needed.
bool gemv_plan(int kind, int C, int* mt, int* KW, int* cpl) {
  const int budget = kind == K_AFF2 ? 4 : 8;
  for (int m = *mt; m >= 1; m /= 2) {
    for (int kw = 1; kw <= 4; kw *= 2) {
      int c = (C + 64 * kw - 1) / (64 * kw);
      if (c * m <= budget && c <= 4) {
        *mt = m; *KW = kw; *cpl = c;
        return true;
      }
    }
  }
  return false;
}

#ifndef QP_GEMV_WAVES_PER_CU
#define QP_GEMV_WAVES_PER_CU 8
#endif
constexpr int kNumCU = 256;

}  // namespace

static int gemv_kind(const Desc& d) {
  if (d.fmt == AFFINE) return d.bits == 2 ? K_AFF2 : (d.bits == 4 ? K_AFF4 : K_AFF8);
  if (d.fmt == Q4K) return K_Q4K;
  if (d.fmt == Q6K) return K_Q6K;
  return K_SYM4;
}

static int gemv_chunks(const Desc& d, int kind) {
  const int CC = kind == K_AFF2 ? 64 : (kind == K_AFF8 ? 16 : 32);
  return (int)(d.K / CC);
}

bool gemv_supported(const Desc& d) {
  const int kind = gemv_kind(d);
  int mt = 1, kw = 0, cpl = 0;
  return gemv_plan(kind, gemv_chunks(d, kind), &mt, &kw, &cpl);
}

hipError_t launch_gemv(const Desc& d, const void* x, int xdt, int64_t M, const Bufs& b,
                       const void* bias, void* y, int ydt, hipStream_t s) {
  const int kind = gemv_kind(d);
  const int C = gemv_chunks(d, kind);
  int mt = M >= 8 ? 8 : (M >= 4 ? (M == 4 ? 4 : 8) : (M == 3 ? 4 : (int)M));
  int KW = 1, cpl = 0;
  if (!gemv_plan(kind, C, &mt, &KW, &cpl)) return hipErrorInvalidValue;
  GemvFn fn = pick(kind, xdt == BF16, mt, cpl);
  if (!fn) return hipErrorInvalidValue;
  const int RW = 4 / KW;
  const int64_t teamsTarget = (int64_t)kNumCU * QP_GEMV_WAVES_PER_CU / KW;
  const int64_t rpt = (d.N + teamsTarget - 1) / teamsTarget;
  const int64_t teams = (d.N + rpt - 1) / rpt;
  const int64_t blocks = (teams + RW - 1) / RW;
  GemvArgs a;
  a.qw = static_cast<const uint32_t*>(b.qweight);
  a.qh = static_cast<const uint32_t*>(b.qweight_hi);
  a.scales = b.scales;
  a.zeros = b.zeros;
  a.steps = b.steps;
  a.x = static_cast<const uint16_t*>(x);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = y;
  a.N = d.N;
  a.K = d.K;
  a.M = M;
  a.C = C;
  a.gs = d.gs;
  a.meta_bf16 = d.meta == BF16;
  a.ydt = ydt;
  a.KW = KW;
  a.RPT = (int)rpt;
  const unsigned mtiles = (unsigned)((M + mt - 1) / mt);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks, mtiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qp
