// Quantize, pack, unpack and dequantize kernels (bit-exact layout work).
//
// The quantization rules follow the HF Transformers "Metal" page (group
// affine codes with per-group scale/bias, uint32 packing), ExecuTorch PR
// #20571 "Quant schema update" (nested superscale Q4_K / Q6_K-style
// metadata: codes first, then the group scale/zero re-quantized to integer
// codes times one fp16 step per 256 weights, step = max/255 or max/127,
// rounding against the fp16-rounded step) and ExecuTorch PR #16577
// (symmetric int4, qmin=-7..qmax=7).  Every step is one IEEE fp32 operation
// (this file is compiled with -ffp-contract=off), quotients are correctly
// rounded, codes use rint (half to even).
//
// These kernels are off the decode/prefill hot path: they favour a simple
// one-thread-per-group structure over bandwidth tuning.
#include "device_common.hpp"
#include "qp_internal.hpp"

namespace qp {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
  return fminf(fmaxf(v, lo), hi);
}

__device__ __forceinline__ float meta_round(float v, int meta_bf16) {
  return meta_bf16 ? bf16_to_f32(f32_to_bf16_rne(v))
                   : f16_to_f32(f32_to_f16_rne(v));
}

// ---------------------------------------------------------------- AFFINE
// One thread per group: min/max, stored scale/bias, then codes.
template <int BITS>
__global__ void __launch_bounds__(kThreads)
k_quant_affine(const float* __restrict__ W, uint32_t* __restrict__ qw,
               uint16_t* __restrict__ scales, uint16_t* __restrict__ biases,
               int64_t N, int64_t K, int gs, int meta_bf16) {
  const int64_t ng = K / gs;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= N * ng) return;
  const int64_t n = g / ng, gi = g % ng;
  const float4* src = reinterpret_cast<const float4*>(W + n * K + gi * gs);
  float lo = INFINITY, hi = -INFINITY;
  for (int i = 0; i < gs / 4; ++i) {
    float4 v = src[i];
    lo = fminf(fminf(lo, v.x), fminf(v.y, fminf(v.z, v.w)));
    hi = fmaxf(fmaxf(hi, v.x), fmaxf(v.y, fmaxf(v.z, v.w)));
  }
  // signed zeros are canonical +0 in the metadata (x + 0 maps -0 to +0)
  lo = lo + 0.f;
  hi = hi + 0.f;
  constexpr float qmax = (float)((1 << BITS) - 1);
  const float s32 = div_rn(hi - lo, qmax);
  const uint32_t sb = meta_bf16 ? f32_to_bf16_rne(s32) : f32_to_f16_rne(s32);
  const uint32_t bb = meta_bf16 ? f32_to_bf16_rne(lo) : f32_to_f16_rne(lo);
  scales[g] = (uint16_t)sb;
  biases[g] = (uint16_t)bb;
  const float s = meta_to_f32(sb, meta_bf16), b = meta_to_f32(bb, meta_bf16);
  constexpr int per = 32 / BITS;
  const int wpg = gs / per;
  uint32_t* dst = qw + (n * K + gi * gs) / per;
  const float* wr = W + n * K + gi * gs;
  for (int wi = 0; wi < wpg; ++wi) {
    uint32_t word = 0;
    for (int j = 0; j < per; ++j) {
      float w = wr[wi * per + j];
      float q = (s == 0.f) ? 0.f : clampf(rintf(div_rn(w - b, s)), 0.f, qmax);
      word |= (uint32_t)q << (BITS * j);
    }
    dst[wi] = word;
  }
}

// ------------------------------------------------------------ AFFINE HQQ
// One thread per group: the min/max scale and bias of k_quant_affine, then
// the zero point chosen by Half-Quadratic Quantization (Badri and Shaji,
// 2023; the "hqq" quantization-parameter option that ExecuTorch PR #17235's
// review asks for on the Metal int4 affine weights).  The scale stays; the
// zero point z (code units, w ~ (q - z) s, starting at -bias / s) alternates
//   q = clamp(rint(w / s + z), 0, L),  e = w - (q - z) s,  err = sum |e|,
//   W_e = sign(e) max(|e| - |e|^(p-1) / beta, 0)   (generalised soft threshold),
//   z <- mean(q - (w - W_e) / s),  beta <- kappa beta,
// and keeps the iterate with the smallest err (a strictly smaller one
// replaces it; the start counts).  The kept z becomes the stored bias
// meta(-z s) and the codes are rounded against the stored scale and bias
// exactly as k_quant_affine does, so dequantization is unchanged.  Each step
// is one fp32 operation in that order (-ffp-contract=off), |e|^(p-1) is
// evaluated in fp64 and rounded once, the group sums run in ascending k.
template <int BITS>
__global__ void __launch_bounds__(kThreads)
k_quant_affine_hqq(const float* __restrict__ W, uint32_t* __restrict__ qw,
                   uint16_t* __restrict__ scales, uint16_t* __restrict__ biases,
                   int64_t N, int64_t K, int gs, int meta_bf16, int iters, float p,
                   float beta0, float kappa) {
  const int64_t ng = K / gs;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= N * ng) return;
  const int64_t n = g / ng, gi = g % ng;
  const float* wr = W + n * K + gi * gs;
  float lo = INFINITY, hi = -INFINITY;
  for (int k = 0; k < gs; ++k) {
    lo = fminf(lo, wr[k]);
    hi = fmaxf(hi, wr[k]);
  }
  lo = lo + 0.f;   // canonical +0
  hi = hi + 0.f;
  constexpr float qmax = (float)((1 << BITS) - 1);
  const uint32_t sb = meta_bf16 ? f32_to_bf16_rne(div_rn(hi - lo, qmax))
                                : f32_to_f16_rne(div_rn(hi - lo, qmax));
  uint32_t bb = meta_bf16 ? f32_to_bf16_rne(lo) : f32_to_f16_rne(lo);
  const float s = meta_to_f32(sb, meta_bf16);
  if (s != 0.f) {
    const double pm1 = (double)p - 1.0;
    float z = div_rn(-meta_to_f32(bb, meta_bf16), s);
    float best_z = z, best_err = INFINITY, beta = beta0;
    for (int t = 0; t <= iters; ++t) {
      const bool upd = t < iters;
      float err = 0.f, vsum = 0.f;
      for (int k = 0; k < gs; ++k) {
        const float w = wr[k];
        const float q = clampf(rintf(div_rn(w, s) + z), 0.f, qmax);
        const float e = w - (q - z) * s;
        const float a = fabsf(e);
        err = err + a;
        if (upd) {
          float we = 0.f;
          if (a > 0.f) {
            const float th = a - div_rn((float)pow((double)a, pm1), beta);
            if (th > 0.f) we = copysignf(th, e);
          }
          vsum = vsum + (q - div_rn(w - we, s));
        }
      }
      if (err < best_err) {
        best_err = err;
        best_z = z;
      }
      if (upd) {
        z = div_rn(vsum, (float)gs);
        beta = beta * kappa;
      }
    }
    const float bias = (-best_z) * s + 0.f;
    bb = meta_bf16 ? f32_to_bf16_rne(bias) : f32_to_f16_rne(bias);
  }
  scales[g] = (uint16_t)sb;
  biases[g] = (uint16_t)bb;
  const float b = meta_to_f32(bb, meta_bf16);
  constexpr int per = 32 / BITS;
  uint32_t* dst = qw + (n * K + gi * gs) / per;
  for (int wi = 0; wi < gs / per; ++wi) {
    uint32_t word = 0;
    for (int j = 0; j < per; ++j) {
      const float w = wr[wi * per + j];
      const float q = (s == 0.f) ? 0.f : clampf(rintf(div_rn(w - b, s)), 0.f, qmax);
      word |= (uint32_t)q << (BITS * j);
    }
    dst[wi] = word;
  }
}

// ------------------------------------------------------------------ Q4K
// One thread per super-block of 256 (8 groups of 32).
__global__ void __launch_bounds__(kThreads)
k_quant_q4k(const float* __restrict__ W, uint32_t* __restrict__ qw,
            uint8_t* __restrict__ sc, uint8_t* __restrict__ zc,
            uint32_t* __restrict__ steps, int64_t N, int64_t K) {
  const int64_t nsb = K / 256;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * nsb) return;
  const int64_t n = t / nsb, j = t % nsb;
  const float* wr = W + n * K + j * 256;
  float s[8], lo[8], z[8];
  float smax = 0.f, zmax = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const float4* src = reinterpret_cast<const float4*>(wr + g * 32);
    float mn = 0.f, mx = 0.f;  // range widened to contain 0
    for (int i = 0; i < 8; ++i) {
      float4 v = src[i];
      mn = fminf(fminf(mn, v.x), fminf(v.y, fminf(v.z, v.w)));
      mx = fmaxf(fmaxf(mx, v.x), fmaxf(v.y, fmaxf(v.z, v.w)));
    }
    mn = mn + 0.f;   // signed zeros are canonical +0
    mx = mx + 0.f;
    s[g] = div_rn(mx - mn, 15.f);
    lo[g] = mn;
    z[g] = (s[g] == 0.f) ? 0.f : div_rn(-mn, s[g]) + 0.f;
    smax = fmaxf(smax, s[g]);
    zmax = fmaxf(zmax, z[g]);
  }
  const uint32_t sbits = f32_to_f16_rne(div_rn(smax, 255.f));
  const uint32_t zbits = f32_to_f16_rne(div_rn(zmax, 255.f));
  const float sstep = f16_to_f32(sbits), zstep = f16_to_f32(zbits);
  steps[t] = sbits | (zbits << 16);
  uint8_t* scr = sc + n * (K / 32) + j * 8;
  uint8_t* zcr = zc + n * (K / 32) + j * 8;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    float a = (sstep == 0.f) ? 0.f : clampf(rintf(div_rn(s[g], sstep)), 0.f, 255.f);
    float b = (zstep == 0.f) ? 0.f : clampf(rintf(div_rn(z[g], zstep)), 0.f, 255.f);
    scr[g] = (uint8_t)a;
    zcr[g] = (uint8_t)b;
  }
  uint32_t* dst = qw + (n * K + j * 256) / 8;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    for (int wi = 0; wi < 4; ++wi) {
      uint32_t word = 0;
      for (int i = 0; i < 8; ++i) {
        float w = wr[g * 32 + wi * 8 + i];
        float q = (s[g] == 0.f) ? 0.f
                                : clampf(rintf(div_rn(w - lo[g], s[g])), 0.f, 15.f);
        word |= (uint32_t)q << (4 * i);
      }
      dst[g * 4 + wi] = word;
    }
  }
}

// ------------------------------------------------------------------ Q6K
// One thread per super-block of 256 (16 groups of 16).
__global__ void __launch_bounds__(kThreads)
k_quant_q6k(const float* __restrict__ W, uint32_t* __restrict__ ql,
            uint32_t* __restrict__ qh, int8_t* __restrict__ sc,
            uint16_t* __restrict__ steps, int64_t N, int64_t K) {
  const int64_t nsb = K / 256;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * nsb) return;
  const int64_t n = t / nsb, j = t % nsb;
  const float* wr = W + n * K + j * 256;
  float s[16];
  float smax = 0.f;
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    const float4* src = reinterpret_cast<const float4*>(wr + g * 16);
    float amax = 0.f;
    for (int i = 0; i < 4; ++i) {
      float4 v = src[i];
      amax = fmaxf(fmaxf(amax, fabsf(v.x)),
                   fmaxf(fabsf(v.y), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    s[g] = div_rn(amax, 31.f);
    smax = fmaxf(smax, s[g]);
  }
  const uint32_t stbits = f32_to_f16_rne(div_rn(smax, 127.f));
  const float step = f16_to_f32(stbits);
  steps[t] = (uint16_t)stbits;
  int8_t* scr = sc + n * (K / 16) + j * 16;
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    float a = (step == 0.f) ? 0.f : clampf(rintf(div_rn(s[g], step)), 0.f, 127.f);
    scr[g] = (int8_t)a;
  }
  uint32_t* lo_dst = ql + (n * K + j * 256) / 8;
  uint32_t* hi_dst = qh + (n * K + j * 256) / 16;
  for (int hw = 0; hw < 16; ++hw) {      // one qh word = 16 codes = 1 group
    uint32_t hword = 0, l0 = 0, l1 = 0;
    for (int i = 0; i < 16; ++i) {
      float w = wr[hw * 16 + i];
      float q = (s[hw] == 0.f) ? 0.f : clampf(rintf(div_rn(w, s[hw])), -32.f, 31.f);
      uint32_t u = (uint32_t)((int)q + 32);
      hword |= (u >> 4) << (2 * i);
      if (i < 8) l0 |= (u & 15u) << (4 * i);
      else l1 |= (u & 15u) << (4 * (i - 8));
    }
    hi_dst[hw] = hword;
    lo_dst[2 * hw] = l0;
    lo_dst[2 * hw + 1] = l1;
  }
}

// ----------------------------------------------------------------- SYM4
// Scale per group: one wave per group (groups may span a whole row).
__global__ void __launch_bounds__(kThreads)
k_sym4_scales(const float* __restrict__ W, float* __restrict__ scales,
              int64_t N, int64_t K, int64_t gs) {
  const int64_t ng = K / gs;
  const int64_t g = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x & 63;
  if (g >= N * ng) return;  // uniform per wave
  const int64_t n = g / ng, gi = g % ng;
  const float4* src = reinterpret_cast<const float4*>(W + n * K + gi * gs);
  float amax = 0.f;
  for (int64_t i = lane; i < gs / 4; i += 64) {
    float4 v = src[i];
    amax = fmaxf(fmaxf(amax, fabsf(v.x)),
                 fmaxf(fabsf(v.y), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = wave_max_all(amax);
  if (lane == 0) scales[g] = div_rn(amax, 7.f);
}

// Codes: one thread per packed word (8 codes).
__global__ void __launch_bounds__(kThreads)
k_sym4_codes(const float* __restrict__ W, const float* __restrict__ scales,
             uint32_t* __restrict__ qw, int64_t N, int64_t K, int64_t gs) {
  const int64_t nw = N * K / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nw) return;
  const int64_t n = (t * 8) / K, k0 = (t * 8) % K;
  const float s = scales[n * (K / gs) + k0 / gs];
  const float4* src = reinterpret_cast<const float4*>(W + n * K + k0);
  float4 a = src[0], b = src[1];
  float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = (s == 0.f) ? 0.f : clampf(rintf(div_rn(v[i], s)), -7.f, 7.f);
    word |= (uint32_t)((int)q + 8) << (4 * i);
  }
  qw[t] = word;
}

// --------------------------------------------------------------- unpack
// One thread per 8 codes along K (one int4 / int6-low word, two int2 or
// half... every format is walked in steps of 8 codes).
__global__ void __launch_bounds__(kThreads)
k_unpack(const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qh,
         uint8_t* __restrict__ codes, int64_t N, int64_t K, int fmt, int bits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * K / 8) return;
  const int64_t e0 = t * 8;  // flat element index (rows are contiguous)
  uint32_t out[2] = {0, 0};
  if (fmt == Q6K) {
    uint32_t lo = qw[t];
    uint32_t hw = qh[e0 / 16] >> (2 * (e0 % 16));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int u = (int)(((lo >> (4 * i)) & 15u) | (((hw >> (2 * i)) & 3u) << 4));
      out[i / 4] |= (uint32_t)(uint8_t)(int8_t)(u - 32) << (8 * (i % 4));
    }
  } else {
    const int per = 32 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t wi = e0 / per;
    const int sh0 = (int)(e0 % per) * bits;
    const int off = (fmt == SYM4) ? 8 : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // 8 consecutive codes never straddle words for bits in {2, 4};
      // bits = 8 spans two words.
      int64_t w = wi + (sh0 + i * bits) / 32;
      int sh = (sh0 + i * bits) % 32;
      int u = (int)((qw[w] >> sh) & mask) - off;
      out[i / 4] |= (uint32_t)(uint8_t)(int8_t)u << (8 * (i % 4));
    }
  }
  reinterpret_cast<uint2*>(codes)[t] = make_uint2(out[0], out[1]);
}

// ----------------------------------------------------------------- pack
__global__ void __launch_bounds__(kThreads)
k_pack(const uint8_t* __restrict__ codes, uint32_t* __restrict__ qw,
       uint32_t* __restrict__ qh, int64_t N, int64_t K, int fmt, int bits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (fmt == Q6K) {
    // one thread per 16 codes: one qh word and two ql words
    if (t >= N * K / 16) return;
    const uint4 c = reinterpret_cast<const uint4*>(codes)[t];
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t h = 0, l[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t u = (uint32_t)((int)(int8_t)(cw[i / 4] >> (8 * (i % 4))) + 32) & 63u;
      h |= (u >> 4) << (2 * i);
      l[i / 8] |= (u & 15u) << (4 * (i % 8));
    }
    qh[t] = h;
    qw[2 * t] = l[0];
    qw[2 * t + 1] = l[1];
    return;
  }
  // one thread per output word
  const int per = 32 / bits;
  if (t >= N * K / per) return;
  const uint32_t mask = (1u << bits) - 1u;
  const int off = (fmt == SYM4) ? 8 : 0;
  const uint8_t* src = codes + t * per;
  uint32_t word = 0;
  for (int i = 0; i < per; ++i) {
    int u = (fmt == SYM4 ? (int)(int8_t)src[i] : (int)src[i]) + off;
    word |= ((uint32_t)u & mask) << (bits * i);
  }
  qw[t] = word;
}

// -------------------------------------------------------------- dequant
// One thread per 8 consecutive weights.  Arithmetic order as documented in
// qlinear.h (AFFINE q*s + b with q*s exact; Q4K (q - zc*zstep)*(sc*sstep);
// Q6K q*(sc*step); SYM4 q*s).
__global__ void __launch_bounds__(kThreads)
k_dequant(const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qh,
          const void* __restrict__ scales, const void* __restrict__ zeros,
          const void* __restrict__ steps, void* __restrict__ out, int64_t N,
          int64_t K, int fmt, int bits, int gs, int meta_bf16, int out_dt) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * K / 8) return;
  const int64_t e0 = t * 8;
  const int64_t n = e0 / K, k0 = e0 % K;
  float w[8];
  if (fmt == Q6K) {
    const uint32_t lo = qw[t];
    const uint32_t hw = qh[e0 / 16] >> (2 * (e0 % 16));
    const float step = f16_to_f32(reinterpret_cast<const uint16_t*>(steps)[n * (K / 256) + k0 / 256]);
    const float S = (float)reinterpret_cast<const int8_t*>(scales)[n * (K / 16) + k0 / 16] * step;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int u = (int)(((lo >> (4 * i)) & 15u) | (((hw >> (2 * i)) & 3u) << 4));
      w[i] = (float)(u - 32) * S;
    }
  } else if (fmt == Q4K) {
    const uint32_t word = qw[t];
    const uint32_t st = reinterpret_cast<const uint32_t*>(steps)[n * (K / 256) + k0 / 256];
    const int64_t g = n * (K / 32) + k0 / 32;
    const float S = (float)reinterpret_cast<const uint8_t*>(scales)[g] * f16_to_f32(st & 0xFFFFu);
    const float Z = (float)reinterpret_cast<const uint8_t*>(zeros)[g] * f16_to_f32(st >> 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float d = (float)((word >> (4 * i)) & 15u) - Z;
      w[i] = d * S;
    }
  } else {
    const int per = 32 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t g = n * (K / gs) + k0 / gs;
    float s, b = 0.f;
    int off = 0;
    if (fmt == AFFINE) {
      s = meta_to_f32(reinterpret_cast<const uint16_t*>(scales)[g], meta_bf16);
      b = meta_to_f32(reinterpret_cast<const uint16_t*>(zeros)[g], meta_bf16);
    } else {
      s = reinterpret_cast<const float*>(scales)[g];
      off = 8;
    }
    const int64_t wi = e0 / per;
    const int sh0 = (int)(e0 % per) * bits;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t wv = wi + (sh0 + i * bits) / 32;
      int sh = (sh0 + i * bits) % 32;
      float q = (float)((int)((qw[wv] >> sh) & mask) - off);
      w[i] = q * s + b;
    }
  }
  if (out_dt == F32) {
    float4* o = reinterpret_cast<float4*>(out) + 2 * t;
    o[0] = make_float4(w[0], w[1], w[2], w[3]);
    o[1] = make_float4(w[4], w[5], w[6], w[7]);
  } else {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t a = out_dt == BF16 ? f32_to_bf16_rne(w[2 * i]) : f32_to_f16_rne(w[2 * i]);
      uint32_t c = out_dt == BF16 ? f32_to_bf16_rne(w[2 * i + 1]) : f32_to_f16_rne(w[2 * i + 1]);
      p[i] = a | (c << 16);
    }
    reinterpret_cast<uint4*>(out)[t] = make_uint4(p[0], p[1], p[2], p[3]);
  }
}

inline unsigned blocks_for(int64_t n) {
  return (unsigned)((n + kThreads - 1) / kThreads);
}

// ------------------------------------------------- nested re-encoding
// Plain per-group metadata into the nested superscale form (ExecuTorch PR
// #20571: the original int4 / int6 tensors are converted into Q4_K / Q6_K,
// codes unchanged, only the metadata re-quantized).  One thread per
// super-block of 256, the rule of the nested quantizers' second stage:
// step = fp16(fl32(max / levels)), code = step == 0 ? 0 :
// clamp(rint(fl32(v / step)), 0, code_max).  A negative or non-finite input
// sets *bad (when given) and is encoded as if it were 0.
__device__ __forceinline__ float plain_in(float v, int* bad) {
  if (!(v >= 0.f) || !(v <= 3.402823466e38f)) {
    if (bad) atomicOr(bad, 1);
    return 0.f;
  }
  return v;
}

template <int G, int LEVELS>
__device__ __forceinline__ uint32_t encode_super(const float* v, uint8_t* codes, int* bad) {
  float x[G];
  float mx = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    x[g] = plain_in(v[g], bad);
    mx = fmaxf(mx, x[g]);
  }
  const uint32_t bits = f32_to_f16_rne(div_rn(mx, (float)LEVELS));
  const float step = f16_to_f32(bits);
#pragma unroll
  for (int g = 0; g < G; ++g)
    codes[g] = (uint8_t)(step == 0.f ? 0.f : clampf(rintf(div_rn(x[g], step)), 0.f, (float)LEVELS));
  return bits;
}

__global__ void __launch_bounds__(kThreads)
k_encode_q4k(const float* __restrict__ s, const float* __restrict__ z, uint8_t* __restrict__ sc,
             uint8_t* __restrict__ zc, uint32_t* __restrict__ steps, int64_t nsb, int* bad) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nsb) return;   // super-block t: groups 8 t .. 8 t + 7 of the [N, K/32] arrays
  const uint32_t sb = encode_super<8, 255>(s + 8 * t, sc + 8 * t, bad);
  const uint32_t zb = encode_super<8, 255>(z + 8 * t, zc + 8 * t, bad);
  steps[t] = sb | (zb << 16);
}

__global__ void __launch_bounds__(kThreads)
k_encode_q6k(const float* __restrict__ s, int8_t* __restrict__ sc, uint16_t* __restrict__ steps,
             int64_t nsb, int* bad) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nsb) return;   // super-block t: groups 16 t .. 16 t + 15 of [N, K/16]
  steps[t] = (uint16_t)encode_super<16, 127>(s + 16 * t, reinterpret_cast<uint8_t*>(sc + 16 * t),
                                             bad);
}

// Per-token symmetric int8 activations (the "a8" of ExecuTorch PR #16577,
// "Arm backend: Support a8w4 for convolution and linear"; the page leaves
// the rule open, the one taken is per row m):
//   s_m = fl32(max_k |x[m, k]| / 127),
//   q[m, k] = s_m == 0 ? 0 : clamp(rint(fl32(x[m, k] / s_m)), -127, 127).
// One block of 1024 threads per row, 8 elements per thread and pass (16-byte
// loads, 8-byte stores) when K % 8 == 0, else one element; the second pass
// re-reads the row from cache.  Every step the single IEEE operation above.
constexpr int kActThreads = 1024;

template <bool XBF16>
__device__ __forceinline__ float act_val(uint32_t b) {
  return XBF16 ? bf16_to_f32(b) : f16_to_f32(b);
}

template <bool XBF16>
__device__ __forceinline__ int8_t act_code(float v, float sc) {
  return (int8_t)(int)(sc == 0.f ? 0.f : clampf(rintf(div_rn(v, sc)), -127.f, 127.f));
}

template <bool XBF16>
__global__ void __launch_bounds__(kActThreads)
k_quant_act(const uint16_t* __restrict__ x, int64_t K, int8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float wmax[kActThreads / 64];
  const int64_t m = blockIdx.x;
  const uint16_t* xr = x + m * K;
  int8_t* qr = q + m * K;
  const bool vec = (K & 7) == 0;
  float amax = 0.f;
  if (vec) {
    for (int64_t c = threadIdx.x; c < K / 8; c += kActThreads) {
      const uint4 u = reinterpret_cast<const uint4*>(xr)[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(act_val<XBF16>(w[e] & 0xFFFFu)),
                                 fabsf(act_val<XBF16>(w[e] >> 16))));
    }
  } else {
    for (int64_t k = threadIdx.x; k < K; k += kActThreads)
      amax = fmaxf(amax, fabsf(act_val<XBF16>(xr[k])));
  }
  amax = wave_max_all(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kActThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);
  const float sc = div_rn(amax, 127.f);
  if (threadIdx.x == 0) s[m] = sc;
  if (vec) {
    for (int64_t c = threadIdx.x; c < K / 8; c += kActThreads) {
      const uint4 u = reinterpret_cast<const uint4*>(xr)[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      uint32_t o[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (uint8_t)act_code<XBF16>(act_val<XBF16>(w[e] & 0xFFFFu), sc);
        const uint32_t hi = (uint8_t)act_code<XBF16>(act_val<XBF16>(w[e] >> 16), sc);
        o[e >> 1] |= (lo | (hi << 8)) << (16 * (e & 1));
      }
      reinterpret_cast<uint2*>(qr)[c] = make_uint2(o[0], o[1]);
    }
  } else {
    for (int64_t k = threadIdx.x; k < K; k += kActThreads)
      qr[k] = act_code<XBF16>(act_val<XBF16>(xr[k]), sc);
  }
}

}  // namespace

hipError_t launch_quantize(const Desc& d, const float* W, void* qweight,
                           void* qweight_hi, void* scales, void* zeros,
                           void* steps, hipStream_t s) {
  const int64_t N = d.N, K = d.K;
  if (d.fmt == AFFINE) {
    const int64_t ng = N * (K / d.gs);
    const int mb = d.meta == BF16;
    auto* qw = static_cast<uint32_t*>(qweight);
    auto* sc = static_cast<uint16_t*>(scales);
    auto* bi = static_cast<uint16_t*>(zeros);
    if (d.bits == 2)
      hipLaunchKernelGGL(k_quant_affine<2>, dim3(blocks_for(ng)), dim3(kThreads), 0, s, W, qw, sc, bi, N, K, d.gs, mb);
    else if (d.bits == 4)
      hipLaunchKernelGGL(k_quant_affine<4>, dim3(blocks_for(ng)), dim3(kThreads), 0, s, W, qw, sc, bi, N, K, d.gs, mb);
    else
      hipLaunchKernelGGL(k_quant_affine<8>, dim3(blocks_for(ng)), dim3(kThreads), 0, s, W, qw, sc, bi, N, K, d.gs, mb);
  } else if (d.fmt == Q4K) {
    hipLaunchKernelGGL(k_quant_q4k, dim3(blocks_for(N * (K / 256))), dim3(kThreads), 0, s, W,
                       static_cast<uint32_t*>(qweight), static_cast<uint8_t*>(scales),
                       static_cast<uint8_t*>(zeros), static_cast<uint32_t*>(steps), N, K);
  } else if (d.fmt == Q6K) {
    hipLaunchKernelGGL(k_quant_q6k, dim3(blocks_for(N * (K / 256))), dim3(kThreads), 0, s, W,
                       static_cast<uint32_t*>(qweight), static_cast<uint32_t*>(qweight_hi),
                       static_cast<int8_t*>(scales), static_cast<uint16_t*>(steps), N, K);
  } else {
    const int64_t ng = N * (K / d.gs);
    hipLaunchKernelGGL(k_sym4_scales, dim3(blocks_for(ng * 64)), dim3(kThreads), 0, s, W,
                       static_cast<float*>(scales), N, K, (int64_t)d.gs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sym4_codes, dim3(blocks_for(N * K / 8)), dim3(kThreads), 0, s, W,
                       static_cast<const float*>(scales), static_cast<uint32_t*>(qweight), N,
                       K, (int64_t)d.gs);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_hqq(const Desc& d, const float* W, void* qweight, void* scales,
                               void* zeros, int iters, float p, float beta, float kappa,
                               hipStream_t s) {
  const int64_t N = d.N, K = d.K;
  const int64_t ng = N * (K / d.gs);
  const int mb = d.meta == BF16;
  auto* qw = static_cast<uint32_t*>(qweight);
  auto* sc = static_cast<uint16_t*>(scales);
  auto* bi = static_cast<uint16_t*>(zeros);
  const dim3 grid(blocks_for(ng)), block(kThreads);
  if (d.bits == 2)
    hipLaunchKernelGGL(k_quant_affine_hqq<2>, grid, block, 0, s, W, qw, sc, bi, N, K, d.gs, mb,
                       iters, p, beta, kappa);
  else if (d.bits == 4)
    hipLaunchKernelGGL(k_quant_affine_hqq<4>, grid, block, 0, s, W, qw, sc, bi, N, K, d.gs, mb,
                       iters, p, beta, kappa);
  else
    hipLaunchKernelGGL(k_quant_affine_hqq<8>, grid, block, 0, s, W, qw, sc, bi, N, K, d.gs, mb,
                       iters, p, beta, kappa);
  return hipGetLastError();
}

hipError_t launch_unpack(const Desc& d, const Bufs& b, void* codes, hipStream_t s) {
  hipLaunchKernelGGL(k_unpack, dim3(blocks_for(d.N * d.K / 8)), dim3(kThreads), 0, s,
                     static_cast<const uint32_t*>(b.qweight),
                     static_cast<const uint32_t*>(b.qweight_hi), static_cast<uint8_t*>(codes),
                     d.N, d.K, d.fmt, d.bits);
  return hipGetLastError();
}

hipError_t launch_pack(const Desc& d, const void* codes, void* qweight, void* qweight_hi,
                       hipStream_t s) {
  const int64_t work = d.fmt == Q6K ? d.N * d.K / 16 : d.N * d.K / (32 / d.bits);
  hipLaunchKernelGGL(k_pack, dim3(blocks_for(work)), dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(codes), static_cast<uint32_t*>(qweight),
                     static_cast<uint32_t*>(qweight_hi), d.N, d.K, d.fmt, d.bits);
  return hipGetLastError();
}

hipError_t launch_dequant(const Desc& d, const Bufs& b, void* out, int out_dt, hipStream_t s) {
  hipLaunchKernelGGL(k_dequant, dim3(blocks_for(d.N * d.K / 8)), dim3(kThreads), 0, s,
                     static_cast<const uint32_t*>(b.qweight),
                     static_cast<const uint32_t*>(b.qweight_hi), b.scales, b.zeros, b.steps,
                     out, d.N, d.K, d.fmt, d.bits, d.gs, d.meta == BF16 ? 1 : 0, out_dt);
  return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, int xdt, int64_t M, int64_t K, void* q, float* s,
                            hipStream_t st) {
  if (xdt == BF16)
    hipLaunchKernelGGL(k_quant_act<true>, dim3((unsigned)M), dim3(kActThreads), 0, st,
                       static_cast<const uint16_t*>(x), K, static_cast<int8_t*>(q), s);
  else
    hipLaunchKernelGGL(k_quant_act<false>, dim3((unsigned)M), dim3(kActThreads), 0, st,
                       static_cast<const uint16_t*>(x), K, static_cast<int8_t*>(q), s);
  return hipGetLastError();
}

hipError_t launch_encode_nested(const Desc& d, const float* sv, const float* zv, void* scales,
                                void* zeros, void* steps, int* bad, hipStream_t st) {
  const int64_t nsb = d.N * (d.K / 256);   // super-blocks: one step word / step each
  if (d.fmt == Q4K)
    hipLaunchKernelGGL(k_encode_q4k, dim3(blocks_for(nsb)), dim3(kThreads), 0, st, sv, zv,
                       static_cast<uint8_t*>(scales), static_cast<uint8_t*>(zeros),
                       static_cast<uint32_t*>(steps), nsb, bad);
  else
    hipLaunchKernelGGL(k_encode_q6k, dim3(blocks_for(nsb)), dim3(kThreads), 0, st, sv,
                       static_cast<int8_t*>(scales), static_cast<uint16_t*>(steps), nsb, bad);
  return hipGetLastError();
}

}  // namespace qp
