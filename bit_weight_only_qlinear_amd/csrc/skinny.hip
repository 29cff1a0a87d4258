// Skinny MFMA qGEMV for small activation batches (up to 16 activation rows
// per block, any M in tiles of 16): y = x W^T on exact codes.
//
// v_mfma_f32_16x16x32_{bf16,f16} with the activation rows as the A operand
// (16 rows x 32 columns) and the *codes* of 16 weight rows as the B operand,
// each code held exactly as MAG + u (MAG = 128 in bf16 for 2-, 4- and 6-bit
// codes, 1024 in fp16; 8-bit codes with bf16 activations are held as u
// itself, MAG = 0), so every product code x activation is exact and the sums
// are fp32.  A lane's accumulators then hold 4 activation rows of ONE weight
// row, so the group's scale and offset are one register pair per lane,
// applied once per (weight row, group) in fp32 after the group's MFMAs (the
// superscale page's factorisation
//     sum_k w_k x_k = S * sum (MAG + u) x + T * sum x
// with AFFINE S = scale, T = bias - MAG * scale; Q4K S = sc*sstep,
// T = -S * (MAG + zc*zstep); Q6K S = sc*step, T = -S * (MAG + 32); SYM4
// S = scale, T = -S * (MAG + 8)).  sum x of the group comes from one more
// MFMA per step with B = 1.  Activations are used in their own type: bf16
// stays bf16, fp16 stays fp16 -- no range limit beyond the type's own.
//
// Group-pure MFMA steps.  A lane loads 16 contiguous bytes of a weight row
// (the 32 columns 32 g .. 32 g + 31 of a 128-column block, g = lane >> 4),
// but an MFMA step takes 8 columns from each of the four lane groups; with
// the loaded layout one step would mix four groups.  Four v_permlane swaps
// (gfx950: 32-lane and 16-lane half swaps) transpose the (lane group x word)
// 4 x 4 layout so that step t takes columns 32 t .. 32 t + 31 -- one group
// for group sizes >= 32.  For Q6K (group 16) each step holds two groups, and
// the activations are fed twice, masked to the lane groups of each.
//
// Work split: a block owns 32 weight rows (two 16-row tiles) and 16
// activation rows (blockIdx.y); its 8 waves take every 8th 128-column block
// of K, kSxStages - 1 blocks' loads in flight ahead of the one computed, and
// their partial sums meet in LDS.  The metadata of the block's 32 rows is
// one contiguous slab per array (rows are N-leading); the block first copies
// the slabs into LDS with 16-byte loads (when they fit in 64 KiB) and each
// lane then reads its rows' few bytes per column block from there.  Small
// per-lane loads straight from HBM, 16 rows per instruction, cost more than
// the codes themselves; they remain only for rows too long for LDS.
//
// Sources: HF Transformers "Metal" page (uint32 codes, per-group scale and
// bias, bits 2/4/8); ExecuTorch PR #20571 "Quant schema update" (Q4_K/Q6_K-
// style nested metadata); ExecuTorch PR #16577 (symmetric int4, stored as
// u = q + 8).
#include <utility>

#include "device_common.hpp"
#include "qp_internal.hpp"

namespace qp {
namespace {

enum SxKind : int { S_AFF2 = 0, S_AFF4 = 1, S_AFF8 = 2, S_Q4K = 3, S_Q6K = 4, S_SYM4 = 5 };

constexpr int kSxRows = 32;     // weight rows per block
#ifndef QP_SX_WAVES
#define QP_SX_WAVES 8
#endif
constexpr int kSxWaves = QP_SX_WAVES;   // K splits per block
static_assert(kSxWaves >= 8, "the final sum maps 512 threads to 32 x 16 outputs");
constexpr int kSxCols = 128;    // columns per block step
#ifndef QP_SX_STAGES
#define QP_SX_STAGES 2
#endif
constexpr int kSxStages = QP_SX_STAGES;   // register stages (kSxStages - 1 loads ahead)
constexpr uint32_t kOOB = 0x80000000u;

struct SxArgs {
  const void* qw;
  const void* qh;
  const void* meta[3];      // scales / scale codes, biases / zero codes, steps
  const void* x;
  const void* bias;
  void* y;
  int64_t M, N, K;
  int ydt;
  uint32_t qw_bytes, qh_bytes, x_bytes;
  uint32_t meta_bytes[3];   // allocated sizes (16-byte multiples)
  uint32_t meta_row[3];     // bytes per weight row of each metadata array
  uint32_t meta_lds[3];     // LDS offset of each array's slab (LDSM)
};

constexpr uint32_t kSxMetaLds = 64u << 10;   // LDS budget for the metadata slabs

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// D += A B with A the activations, B the codes.
template <bool XBF16>
__device__ __forceinline__ float4_t mfma(uint4 a, uint4 b, float4_t c) {
  if constexpr (XBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

template <typename F, int... I>
__device__ __forceinline__ void sfor_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>{});
}

// 4 x 4 transpose of (lane group g = lane >> 4, register t): afterwards
// register t of lane group g holds what register g of lane group t held.
__device__ __forceinline__ void transpose4(uint32_t (&w)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  w[0] = c[0]; w[1] = c[1]; w[2] = d[0]; w[3] = d[1];
}

// Code width in bits, per format.
constexpr int code_bits(int k) { return k == S_AFF2 ? 2 : k == S_AFF8 ? 8 : 4; }
// Magic offset held in every code element.
template <int KIND, bool XBF16>
constexpr float mag() { return KIND == S_AFF8 && XBF16 ? 0.f : (XBF16 ? 128.f : 1024.f); }
// Metadata words per lane and tile of one 128-column block.
template <int KIND, int GS>
constexpr int meta_words() {
  return KIND == S_Q4K || KIND == S_Q6K ? 2
       : KIND == S_SYM4 ? 128 / (GS > 0 ? GS : 128)
       : 4;   // AFFINE: scales in words 0-1, biases in words 2-3
}

// One lane's raw data of one 128-column block.
template <int KIND, int GS>
struct SxStage {
  // codes of the lane's row in each tile i = 0, 1, 32 columns each:
  // int2 2 words, int4 4, int8 8; Q6K 4 low-nibble words + 2 high-bit words
  uint32_t w[2][code_bits(KIND)];
  uint32_t h[2][KIND == S_Q6K ? 2 : 1];
  uint4 x[4];            // activations, 8 columns per MFMA step
  uint32_t m[2][meta_words<KIND, GS>()];
  uint32_t st[2];        // Q4K step word / Q6K fp16 step (per 256 columns)
};

// Metadata word(s) of `bytes` bytes (2, 4, 8 or 16) at byte `off` of array q
// for row n: from the LDS slab (row n - n0) or from HBM.
template <bool LDSM, int BYTES>
__device__ __forceinline__ void meta_ld(const SxArgs& a, const unsigned char* lds, int q,
                                        __amdgpu_buffer_rsrc_t r, bool ok, uint32_t row_local,
                                        uint32_t row_global, uint32_t off, uint32_t* dst) {
  if constexpr (LDSM) {
    const unsigned char* p = lds + a.meta_lds[q] + row_local * a.meta_row[q] + off;
    if constexpr (BYTES == 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    } else if constexpr (BYTES == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      dst[0] = v.x; dst[1] = v.y;
    } else if constexpr (BYTES == 4) {
      dst[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      dst[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  } else {
    const uint32_t o = ok ? row_global * a.meta_row[q] + off : kOOB;
    if constexpr (BYTES == 16) {
      const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    } else if constexpr (BYTES == 8) {
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0));
      dst[0] = v.x; dst[1] = v.y;
    } else if constexpr (BYTES == 4) {
      dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
    } else {
      dst[0] = __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, 0);
    }
  }
}

// PART: 3 = everything; 1 = the global loads only (codes, activations, and
// metadata when it is not staged); 2 = the staged metadata only (LDS reads).
template <int KIND, int GS, bool LDSM, int PART = 3>
__device__ __forceinline__ void sx_load(const SxArgs& a, const unsigned char* lds, int kb, int lane,
                                        int64_t n0, int64_t mrow, SxStage<KIND, GS>& s) {
  const uint32_t c0 = (uint32_t)kb * kSxCols;
  const int g = lane >> 4, r16 = lane & 15;
  constexpr bool GLOB = (PART & 1) != 0;
  constexpr bool META = LDSM ? (PART & 2) != 0 : GLOB;
  const uint32_t K = (uint32_t)a.K;
  // activations of row mrow: step t takes columns c0 + 32 t + 8 g .. + 8
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const uint32_t xo = mrow < a.M ? (uint32_t)mrow * K * 2u + 2u * (c0 + 8u * g) : kOOB;
  if constexpr (GLOB) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      s.x[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rx, xo == kOOB ? kOOB : xo + 64u * t, 0, 0));
  }
  constexpr uint32_t B = code_bits(KIND);
  const __amdgpu_buffer_rsrc_t rq = rsrc(a.qw, a.qw_bytes);
  const __amdgpu_buffer_rsrc_t r0 = rsrc(a.meta[0], a.meta_bytes[0]);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(a.meta[1], a.meta_bytes[1]);
  const __amdgpu_buffer_rsrc_t r2 = rsrc(a.meta[2], a.meta_bytes[2]);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // codes: row n0 + 16 i + r16, columns c0 + 32 g .. + 32
    const int64_t n = n0 + 16 * i + r16;
    const bool ok = n < a.N;
    const uint32_t off = ok ? (uint32_t)n * (K * B / 8u) + (c0 + 32u * g) * B / 8u : kOOB;
    if constexpr (!GLOB) {
    } else if constexpr (B == 2) {
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, 2));
      s.w[i][0] = v.x; s.w[i][1] = v.y;
    } else {
#pragma unroll
      for (int c = 0; c < (int)B / 4; ++c) {
        const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rq, off == kOOB ? kOOB : off + 16u * c, 0, 2));
        s.w[i][4 * c] = v.x; s.w[i][4 * c + 1] = v.y; s.w[i][4 * c + 2] = v.z; s.w[i][4 * c + 3] = v.w;
      }
    }
    if constexpr (KIND == S_Q6K && GLOB) {
      const __amdgpu_buffer_rsrc_t rh = rsrc(a.qh, a.qh_bytes);
      const uint32_t ho = ok ? (uint32_t)n * (K / 4u) + (c0 + 32u * g) / 4u : kOOB;
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rh, ho, 0, 2));
      s.h[i][0] = v.x; s.h[i][1] = v.y;
    }
    // metadata of row n for the block's groups (rows past N read 0)
    const uint32_t rl = (uint32_t)(16 * i + r16), rg = (uint32_t)n;
    if constexpr (!META) {
    } else if constexpr (KIND == S_AFF2 || KIND == S_AFF4 || KIND == S_AFF8) {
      // 128 / GS groups of 2 bytes: scales into m[0..1], biases into m[2..3]
      constexpr int MB = 256 / GS;
      s.m[i][1] = s.m[i][3] = 0;
      meta_ld<LDSM, MB>(a, lds, 0, r0, ok, rl, rg, (c0 / GS) * 2u, &s.m[i][0]);
      meta_ld<LDSM, MB>(a, lds, 1, r1, ok, rl, rg, (c0 / GS) * 2u, &s.m[i][2]);
    } else if constexpr (KIND == S_Q4K) {
      // 4 uint8 scale codes, 4 uint8 zero codes, the step word
      meta_ld<LDSM, 4>(a, lds, 0, r0, ok, rl, rg, c0 / 32u, &s.m[i][0]);
      meta_ld<LDSM, 4>(a, lds, 1, r1, ok, rl, rg, c0 / 32u, &s.m[i][1]);
      meta_ld<LDSM, 4>(a, lds, 2, r2, ok, rl, rg, (c0 / 256u) * 4u, &s.st[i]);
    } else if constexpr (KIND == S_Q6K) {
      // 8 int8 scale codes, the fp16 step
      meta_ld<LDSM, 8>(a, lds, 0, r0, ok, rl, rg, c0 / 16u, &s.m[i][0]);
      meta_ld<LDSM, 2>(a, lds, 2, r2, ok, rl, rg, (c0 / 256u) * 2u, &s.st[i]);
    } else if constexpr (GS > 0) {
      // SYM4 per group: 128 / GS fp32 scales
      meta_ld<LDSM, 512 / GS>(a, lds, 0, r0, ok, rl, rg, (c0 / GS) * 4u, &s.m[i][0]);
    }
  }
}

// 16-bit piece p of a 2-word, 2-bit code run (8 codes) as 8 codes in bytes
// 0 and 2: codes 0-3 in byte 0, codes 4-7 in byte 2 (2 bits each).
__device__ __forceinline__ uint32_t spread2(uint32_t p) { return (p & 0xFFu) | ((p & 0xFF00u) << 8); }

// B operand of one MFMA step: the lane's 8 codes in element order
// (0, 4, 1, 5, 2, 6, 3, 7), each MAG + u exactly.
template <int KIND, bool XBF16>
__device__ __forceinline__ uint4 code_frag(uint32_t w, uint32_t w2, uint32_t hq) {
  const uint32_t magic = XBF16 ? 0x43004300u : 0x64006400u;
  uint32_t p[4];
  if constexpr (KIND == S_AFF2) {
    const uint32_t q = spread2(w);
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = ((q >> (2 * e)) & 0x00030003u) | magic;
  } else if constexpr (KIND == S_AFF8) {
    // w: codes 0-3 (bytes), w2: codes 4-7
    if constexpr (XBF16) {
      // bf16 of a byte is the high half of its fp32 value (exact)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = (float)((w >> (8 * e)) & 0xFFu), hi = (float)((w2 >> (8 * e)) & 0xFFu);
        p[e] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p[e] = ((w >> (8 * e)) & 0xFFu) | (((w2 >> (8 * e)) & 0xFFu) << 16) | magic;
    }
  } else if constexpr (KIND == S_Q6K) {
    const uint32_t q = spread2(hq);   // high 2 bits of the 8 codes
#pragma unroll
    for (int e = 0; e < 4; ++e)
      p[e] = ((w >> (4 * e)) & 0x000F000Fu) | (((q >> (2 * e)) & 0x00030003u) << 4) | magic;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = ((w >> (4 * e)) & 0x000F000Fu) | magic;
  }
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// The same with per-lane byte selectors: (s0, s1) = (0x05040100,
// 0x07060302) give act_frag's element order, 0x0C0C0C0C gives zeros
// (v_perm_b32 selector byte 12 is the constant 0x00) -- the Q6K step's
// half-masked operands without a select per register.
__device__ __forceinline__ uint4 act_frag_sel(uint4 v, uint32_t s0, uint32_t s1) {
  return make_uint4(__builtin_amdgcn_perm(v.z, v.x, s0), __builtin_amdgcn_perm(v.z, v.x, s1),
                    __builtin_amdgcn_perm(v.w, v.y, s0), __builtin_amdgcn_perm(v.w, v.y, s1));
}

// A operand: 8 activations (two per word, column order) in the same element
// order as code_frag.
__device__ __forceinline__ uint4 act_frag(uint4 v) {
  return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),   // (x0, x4)
                    __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),   // (x1, x5)
                    __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),   // (x2, x6)
                    __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));  // (x3, x7)
}

__device__ __forceinline__ float meta_f(uint32_t bits, bool bf) {
  return bf ? bf16_to_f32(bits) : f16_to_f32(bits);
}

// (S, T) of group gg (a compile-time constant) of the block for the lane's
// row of tile i.
template <int KIND, int GS, bool MBF16>
__device__ __forceinline__ void group_st(const SxStage<KIND, GS>& s, int i, int gg, float mg,
                                         float& S, float& T) {
  if constexpr (KIND == S_AFF2 || KIND == S_AFF4 || KIND == S_AFF8) {
    const uint32_t sh = 16u * (uint32_t)(gg & 1);
    S = meta_f((s.m[i][gg >> 1] >> sh) & 0xFFFFu, MBF16);
    T = fmaf(-mg, S, meta_f((s.m[i][2 + (gg >> 1)] >> sh) & 0xFFFFu, MBF16));
  } else if constexpr (KIND == S_Q4K) {
    const float sc = (float)((s.m[i][0] >> (8 * gg)) & 0xFFu);
    const float zc = (float)((s.m[i][1] >> (8 * gg)) & 0xFFu);
    S = sc * f16_to_f32(s.st[i] & 0xFFFFu);
    T = -S * (mg + zc * f16_to_f32(s.st[i] >> 16));
  } else if constexpr (KIND == S_Q6K) {
    const float sc = (float)(int)(int8_t)((s.m[i][gg >> 2] >> (8 * (gg & 3))) & 0xFFu);
    S = sc * f16_to_f32(s.st[i] & 0xFFFFu);
    T = -S * (mg + 32.f);
  } else {
    S = __uint_as_float(s.m[i][gg]);
    T = -S * (mg + 8.f);
  }
}

// KIND / GS: format and group size (affine 32, 64, 128; Q4K 32; Q6K 16;
// SYM4 32, 64, 128, or 0 for one scale per output channel, applied once to
// the total).
template <int KIND, int GS, bool XBF16, bool MBF16, bool LDSM>
__global__ void __launch_bounds__(64 * kSxWaves) k_skinny(SxArgs a) {
  // partial sums [wave][tile][activation row][weight row]
  __shared__ float s_part[kSxWaves][2][16][17];
  extern __shared__ __attribute__((aligned(16))) unsigned char s_meta[];   // LDSM slabs

  constexpr float MAG = mag<KIND, XBF16>();
  constexpr bool PERCH = KIND == S_SYM4 && GS == 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * kSxRows;
  const int64_t mrow = (int64_t)blockIdx.y * 16 + r16;   // this lane's activation row (A row)
  const int KB = (int)(a.K / kSxCols);

  const uint32_t one = XBF16 ? 0x3F803F80u : 0x3C003C00u;
  // Q6K: v_perm selectors of the lane's half-masked activation operands
  const uint32_t selL0 = g < 2 ? 0x05040100u : 0x0C0C0C0Cu, selL1 = g < 2 ? 0x07060302u : 0x0C0C0C0Cu;
  const uint32_t selH0 = g < 2 ? 0x0C0C0C0Cu : 0x05040100u, selH1 = g < 2 ? 0x0C0C0C0Cu : 0x07060302u;
  const uint4 ONES = make_uint4(one, one, one, one);
  // acc[i][v]: activation row 4 g + v, weight row 16 i + r16
  float4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float4_t D[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float4_t DX = {0.f, 0.f, 0.f, 0.f};

  // Formats whose offset T = -S (MAG + c) has a constant c (Q6K: 32,
  // grouped SYM4: 8) subtract (MAG + c) sum x inside the accumulator with one
  // more MFMA against B = -(MAG + c) (exact in bf16 and fp16), so the group
  // sum is sum q x and the epilogue is one FMA per value: VALU work per
  // group traded for MFMA work, which has room.
  constexpr bool COFF = KIND == S_Q6K || (KIND == S_SYM4 && GS > 0);
  const uint32_t coff = XBF16 ? f32_to_bf16_rne(-(MAG + (KIND == S_Q6K ? 32.f : 8.f)))
                              : f32_to_f16_rne(-(MAG + (KIND == S_Q6K ? 32.f : 8.f)));
  const uint4 BC = make_uint4(coff | (coff << 16), coff | (coff << 16), coff | (coff << 16),
                              coff | (coff << 16));

  // group gg of the block is complete in Dd, DXd: apply its (S, T)
  auto epilogue = [&](const SxStage<KIND, GS>& s, int gg, const float4_t (&Dd)[2],
                      const float4_t& DXd) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float S, T;
      group_st<KIND, GS, MBF16>(s, i, gg, MAG, S, T);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        acc[i][v] = COFF ? fmaf(S, Dd[i][v], acc[i][v]) : fmaf(T, DXd[v], fmaf(S, Dd[i][v], acc[i][v]));
    }
  };

  auto compute = [&](const SxStage<KIND, GS>& s) __attribute__((always_inline)) {
    // code words of both tiles, transposed so that step t is columns
    // 32 t .. 32 t + 31 of the block (2-bit fields: 16 bits per 8 columns;
    // every index is a compile-time constant, so all stays in registers)
    uint32_t W[2][4], W2[2][4], H[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (KIND == S_AFF2) {
        uint32_t p[4] = {s.w[i][0] & 0xFFFFu, s.w[i][0] >> 16, s.w[i][1] & 0xFFFFu, s.w[i][1] >> 16};
        transpose4(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) W[i][t] = p[t];
      } else if constexpr (KIND == S_AFF8) {
        uint32_t p[4] = {s.w[i][0], s.w[i][2], s.w[i][4], s.w[i][6]};
        uint32_t q[4] = {s.w[i][1], s.w[i][3], s.w[i][5], s.w[i][7]};
        transpose4(p);
        transpose4(q);
#pragma unroll
        for (int t = 0; t < 4; ++t) { W[i][t] = p[t]; W2[i][t] = q[t]; }
      } else {
        uint32_t p[4] = {s.w[i][0], s.w[i][1], s.w[i][2], s.w[i][3]};
        transpose4(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) W[i][t] = p[t];
      }
      if constexpr (KIND == S_Q6K) {
        uint32_t p[4] = {s.h[i][0] & 0xFFFFu, s.h[i][0] >> 16, s.h[i][1] & 0xFFFFu, s.h[i][1] >> 16};
        transpose4(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) H[i][t] = p[t];
      }
    }
    sfor<4>([&](auto TT) {
      constexpr int t = decltype(TT)::value;
      if constexpr (KIND == S_Q6K) {
        // two groups per step: lane groups 0-1 (group 2 t), 2-3 (2 t + 1)
        const uint4 Al = act_frag_sel(s.x[t], selL0, selL1);
        const uint4 Ah = act_frag_sel(s.x[t], selH0, selH1);
        float4_t Dh[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 Bq = code_frag<KIND, XBF16>(W[i][t], 0u, H[i][t]);
          D[i] = mfma<XBF16>(Al, Bq, D[i]);
          D[i] = mfma<XBF16>(Al, BC, D[i]);
          Dh[i] = mfma<XBF16>(Ah, Bq, Dh[i]);
          Dh[i] = mfma<XBF16>(Ah, BC, Dh[i]);
        }
        epilogue(s, 2 * t, D, DX);
        epilogue(s, 2 * t + 1, Dh, DX);
        D[0] = D[1] = float4_t{0.f, 0.f, 0.f, 0.f};
      } else {
        const uint4 A = act_frag(s.x[t]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          D[i] = mfma<XBF16>(A, code_frag<KIND, XBF16>(W[i][t], KIND == S_AFF8 ? W2[i][t] : 0u, 0u),
                             D[i]);
          if constexpr (COFF) D[i] = mfma<XBF16>(A, BC, D[i]);
        }
        if constexpr (!COFF) DX = mfma<XBF16>(A, ONES, DX);
        if constexpr (!PERCH) {
          // a group ends every GS / 32 steps
          constexpr int spg = (GS > 0 ? GS : 128) / 32;
          if constexpr ((t + 1) % spg == 0) {
            epilogue(s, t / spg, D, DX);
            D[0] = D[1] = DX = float4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    });
  };

  // The block's metadata slabs (rows n0 .. n0 + 31, contiguous in each
  // array; rows past N read 0) go into LDS with direct buffer->LDS loads
  // (1 KiB per wave instruction, regions padded to whole KiB), issued before
  // the first code loads so that waiting for them does not wait for those.
  if constexpr (LDSM) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const uint32_t pieces = (32u * a.meta_row[q] + 1023u) / 1024u;
      const __amdgpu_buffer_rsrc_t r = rsrc(a.meta[q], a.meta_bytes[q]);
      const uint32_t base = (uint32_t)n0 * a.meta_row[q];
      for (uint32_t pc = (uint32_t)wave; pc < pieces; pc += kSxWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(s_meta + a.meta_lds[q] + 1024u * pc), 16,
            base + 1024u * pc + 16u * (uint32_t)lane, 0, 0, 0);
    }
  }

  // the wave's column blocks: wave, wave + 8, ...; kSxStages - 1 ahead
  SxStage<KIND, GS> st[kSxStages];
  const int J = wave < KB ? (KB - wave + kSxWaves - 1) / kSxWaves : 0;
  sfor<kSxStages - 1>([&](auto P) {
    constexpr int p = decltype(P)::value;
    if (p < J) sx_load<KIND, GS, LDSM, 1>(a, s_meta, wave + p * kSxWaves, lane, n0, mrow, st[p]);
  });

  if constexpr (LDSM) {
    // the slab copies are older than the code loads: wait for them only
    // (all loads where this wave has fewer blocks than stages ahead)
    constexpr int B = code_bits(KIND);
    constexpr int n = (kSxStages - 1) * (4 + 2 * (B == 2 ? 1 : B / 4) + (KIND == S_Q6K ? 2 : 0));
    static_assert(n < 64, "vmcnt range");
    if (J >= kSxStages - 1)
      __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
    __syncthreads();
  }

  if constexpr (LDSM) {
    sfor<kSxStages - 1>([&](auto P) {
      constexpr int p = decltype(P)::value;
      if (p < J) sx_load<KIND, GS, LDSM, 2>(a, s_meta, wave + p * kSxWaves, lane, n0, mrow, st[p]);
    });
  }
  for (int j0 = 0; j0 < J; j0 += kSxStages) {
    sfor<kSxStages>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const int j = j0 + q;
      if (j < J) {
        if (j + kSxStages - 1 < J)
          sx_load<KIND, GS, LDSM>(a, s_meta, wave + (j + kSxStages - 1) * kSxWaves, lane, n0,
                                  mrow, st[(q + kSxStages - 1) % kSxStages]);
        compute(st[q]);
      }
    });
  }
  if constexpr (PERCH) {
    // one group per row: sum (MAG + u) x - (MAG + 8) sum x = sum q x; the
    // channel scale multiplies the total below
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][v] = fmaf(-(MAG + 8.f), DX[v], D[i][v]);
  }

  // ---- partial sums of the 8 waves meet in LDS
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) s_part[wave][i][4 * g + v][r16] = acc[i][v];
  __syncthreads();
  // thread -> (weight row 0..31, activation row 0..15)
  const int nl = tid >> 4, m = tid & 15;
  const int64_t n = n0 + nl;
  const int64_t mm = (int64_t)blockIdx.y * 16 + m;
  if (tid < 512 && mm < a.M && n < a.N) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kSxWaves; ++w) sum += s_part[w][nl >> 4][m][nl & 15];
    if constexpr (PERCH) sum *= static_cast<const float*>(a.meta[0])[n];
    if (a.bias) {
      const uint32_t bb = static_cast<const uint16_t*>(a.bias)[n];
      sum += XBF16 ? bf16_to_f32(bb) : f16_to_f32(bb);
    }
    const int64_t idx = mm * a.N + n;
    if (a.ydt == F32) static_cast<float*>(a.y)[idx] = sum;
    else static_cast<uint16_t*>(a.y)[idx] =
        (uint16_t)(a.ydt == BF16 ? f32_to_bf16_rne(sum) : f32_to_f16_rne(sum));
  }
}

typedef void (*SxFn)(SxArgs);

template <int KIND, int GS, bool MB>
SxFn sx_pick(bool xb, bool lm) {
  if (lm) return xb ? k_skinny<KIND, GS, true, MB, true> : k_skinny<KIND, GS, false, MB, true>;
  return xb ? k_skinny<KIND, GS, true, MB, false> : k_skinny<KIND, GS, false, MB, false>;
}

template <int KIND>
SxFn sx_affine(int gs, bool mb, bool xb, bool lm) {
  if (gs == 32) return mb ? sx_pick<KIND, 32, true>(xb, lm) : sx_pick<KIND, 32, false>(xb, lm);
  if (gs == 64) return mb ? sx_pick<KIND, 64, true>(xb, lm) : sx_pick<KIND, 64, false>(xb, lm);
  return mb ? sx_pick<KIND, 128, true>(xb, lm) : sx_pick<KIND, 128, false>(xb, lm);
}

}  // namespace

bool skinny_supported(const Desc& d) { return d.K % kSxCols == 0; }

hipError_t launch_skinny(const Desc& d, const void* x, int xdt, int64_t M, const Bufs& b,
                         const void* bias, void* y, int ydt, const size_t bytes[5],
                         hipStream_t s) {
  if (M < 1 || !skinny_supported(d)) return hipErrorInvalidValue;
  SxArgs a{};
  a.qw = b.qweight;
  a.qh = b.qweight_hi;
  a.meta[0] = b.scales;
  a.meta[1] = b.zeros;
  a.meta[2] = b.steps;
  a.x = x;
  a.bias = bias;
  a.y = y;
  a.M = M;
  a.N = d.N;
  a.K = d.K;
  a.ydt = ydt;
  a.qw_bytes = (uint32_t)bytes[0];
  a.qh_bytes = (uint32_t)bytes[1];
  a.x_bytes = (uint32_t)((uint64_t)M * d.K * 2);
  uint32_t lds = 0;
  for (int q = 0; q < 3; ++q) {
    a.meta_bytes[q] = (uint32_t)((bytes[2 + q] + 15) & ~size_t(15));
    // bytes per row: sizes are N * per-row bytes for every metadata array
    a.meta_row[q] = (uint32_t)(bytes[2 + q] / (size_t)d.N);
    if (d.fmt == SYM4 && d.gs == d.K && q == 0) a.meta_row[q] = 0;   // scale applied at the end
    a.meta_lds[q] = lds;
    lds += (32u * a.meta_row[q] + 1023u) & ~1023u;   // whole KiB: the copies' unit
  }
  const bool lm = lds > 0 && lds <= kSxMetaLds;
  if (!lm) lds = 0;
  const bool xb = xdt == BF16, mb = d.meta == BF16;
  SxFn fn = nullptr;
  if (d.fmt == AFFINE) {
    fn = d.bits == 2 ? sx_affine<S_AFF2>(d.gs, mb, xb, lm)
       : d.bits == 4 ? sx_affine<S_AFF4>(d.gs, mb, xb, lm) : sx_affine<S_AFF8>(d.gs, mb, xb, lm);
  } else if (d.fmt == Q4K) {
    fn = sx_pick<S_Q4K, 32, false>(xb, lm);
  } else if (d.fmt == Q6K) {
    fn = sx_pick<S_Q6K, 16, false>(xb, lm);
  } else {
    fn = d.gs == d.K ? sx_pick<S_SYM4, 0, false>(xb, false)
       : d.gs == 32  ? sx_pick<S_SYM4, 32, false>(xb, lm)
       : d.gs == 64  ? sx_pick<S_SYM4, 64, false>(xb, lm) : sx_pick<S_SYM4, 128, false>(xb, lm);
  }
  const unsigned blocks = (unsigned)((d.N + kSxRows - 1) / kSxRows);
  const unsigned mtiles = (unsigned)((M + 15) / 16);
  hipLaunchKernelGGL(fn, dim3(blocks, mtiles), dim3(64 * kSxWaves), lds, s, a);
  return hipGetLastError();
}

}  // namespace qp
