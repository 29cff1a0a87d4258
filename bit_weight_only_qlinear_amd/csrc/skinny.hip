// Skinny MFMA qGEMV for small activation batches (M <= 16 per block row of
// activations, any M in tiles of 16): y = x W^T on exact codes.
//
// The activation rows ride in the 16 columns of v_mfma_f32_16x16x32_{bf16,
// f16}; the A operand is 16 weight rows x 32 columns of *codes*, each held
// exactly as MAG + u (MAG = 128 in bf16 for 2-, 4- and 6-bit codes, 1024 in
// fp16; 8-bit codes with bf16 activations are held as u itself, MAG = 0), so
// every product code x activation is exact and the sums are fp32.  The
// group's scale and offset are applied once per (weight row, group) in fp32
// after the group's MFMAs (the superscale page's factorisation
//     sum_k w_k x_k = S * sum (MAG + u) x + T * sum x
// with AFFINE S = scale, T = bias - MAG * scale; Q4K S = sc*sstep,
// T = -S * (MAG + zc*zstep); Q6K S = sc*step, T = -S * (MAG + 32); SYM4
// S = scale, T = -S * (MAG + 8)).  sum x of the group comes from one more
// MFMA per step with A = 1.  Activations are used in their own type: bf16
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
// of K, one block's loads in flight ahead of the one computed, and their
// partial sums meet in LDS.  Each wave turns its block's metadata into fp32
// (S, T) per (row, group) once, in its own LDS slice.
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
constexpr int kSxWaves = 8;     // K splits per block
constexpr int kSxCols = 128;    // columns per block step
constexpr uint32_t kOOB = 0x80000000u;

struct SxArgs {
  const void* qw;
  const void* qh;
  const void* meta[3];      // scales / scale codes, biases / zero codes, steps
  const void* x;
  const void* bias;
  void* y;
  int64_t M, N, K;
  int gs, ydt;
  uint32_t qw_bytes, qh_bytes, x_bytes;
  uint32_t meta_bytes[3];   // allocated sizes (16-byte multiples)
};

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

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

// One lane's raw data of one 128-column block.
template <int KIND>
struct SxStage {
  // codes of the lane's two rows (tiles i = 0, 1), 32 columns each:
  // int2 2 words, int4 4, int8 8; Q6K 4 low-nibble words + 2 high-bit words
  uint32_t w[2][code_bits(KIND) * 32 / 32];
  uint32_t h[2][KIND == S_Q6K ? 2 : 1];
  uint4 x[4];            // activations, 8 columns per MFMA step
  uint2 m;               // the lane's share of the block's metadata
  uint32_t st;           // Q4K / Q6K step (per 256 columns)
};

template <int KIND, bool PERCH>
__device__ __forceinline__ void sx_load(const SxArgs& a, int kb, int lane, int64_t n0,
                                        int64_t mrow, SxStage<KIND>& s) {
  const uint32_t c0 = (uint32_t)kb * kSxCols;
  const int g = lane >> 4, r16 = lane & 15;
  const uint32_t K = (uint32_t)a.K;
  // activations of row mrow: step t takes columns c0 + 32 t + 8 g .. + 8
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const uint32_t xo = mrow < a.M ? (uint32_t)mrow * K * 2u + 2u * (c0 + 8u * g) : kOOB;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    s.x[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rx, xo == kOOB ? kOOB : xo + 64u * t, 0, 0));
  // codes: row n0 + 16 i + r16, columns c0 + 32 g .. + 32
  const __amdgpu_buffer_rsrc_t rq = rsrc(a.qw, a.qw_bytes);
  constexpr uint32_t B = code_bits(KIND);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = n0 + 16 * i + r16;
    const bool ok = n < a.N;
    const uint32_t off = ok ? (uint32_t)n * (K * B / 8u) + (c0 + 32u * g) * B / 8u : kOOB;
    if constexpr (B == 2) {
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, 0));
      s.w[i][0] = v.x; s.w[i][1] = v.y;
    } else {
#pragma unroll
      for (int c = 0; c < (int)B / 4; ++c) {
        const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rq, off == kOOB ? kOOB : off + 16u * c, 0, 2));
        s.w[i][4 * c] = v.x; s.w[i][4 * c + 1] = v.y; s.w[i][4 * c + 2] = v.z; s.w[i][4 * c + 3] = v.w;
      }
    }
    if constexpr (KIND == S_Q6K) {
      const __amdgpu_buffer_rsrc_t rh = rsrc(a.qh, a.qh_bytes);
      const uint32_t ho = ok ? (uint32_t)n * (K / 4u) + (c0 + 32u * g) / 4u : kOOB;
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rh, ho, 0, 2));
      s.h[i][0] = v.x; s.h[i][1] = v.y;
    }
  }
  // metadata: lane -> block row rr = lane >> 1, half hh = lane & 1
  const int rr = lane >> 1, hh = lane & 1;
  const int64_t n = n0 + rr;
  s.m = make_uint2(0, 0);
  s.st = 0;
  if (n >= a.N) return;
  if constexpr (KIND == S_AFF2 || KIND == S_AFF4 || KIND == S_AFF8) {
    // hh = 0: scales, hh = 1: biases; 128 / gs groups of 2 bytes
    const uint32_t ng = 128u / (uint32_t)a.gs;
    const uint32_t off = (uint32_t)n * (K / (uint32_t)a.gs) * 2u + (c0 / (uint32_t)a.gs) * 2u;
    const __amdgpu_buffer_rsrc_t r = rsrc(a.meta[hh], a.meta_bytes[hh]);
    if (ng == 4)
      s.m = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    else if (ng == 2)
      s.m.x = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else
      s.m.x = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else if constexpr (KIND == S_Q4K) {
    // hh = 0: 4 scale codes, hh = 1: 4 zero codes; both: the step word
    const __amdgpu_buffer_rsrc_t r = rsrc(a.meta[hh], a.meta_bytes[hh]);
    s.m.x = __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)n * (K / 32u) + c0 / 32u, 0, 0);
    s.st = __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.meta[2], a.meta_bytes[2]),
                                                (uint32_t)n * (K / 256u) * 4u + (c0 / 256u) * 4u, 0, 0);
  } else if constexpr (KIND == S_Q6K) {
    // hh: 4 of the block's 8 int8 scale codes; both: the fp16 step
    s.m.x = __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.meta[0], a.meta_bytes[0]),
                                                 (uint32_t)n * (K / 16u) + c0 / 16u + 4u * hh, 0, 0);
    s.st = __builtin_amdgcn_raw_buffer_load_b16(rsrc(a.meta[2], a.meta_bytes[2]),
                                                (uint32_t)n * (K / 256u) * 2u + (c0 / 256u) * 2u, 0, 0);
  } else if constexpr (!PERCH) {
    // SYM4 per group: 128 / gs fp32 scales; hh takes half of them
    const uint32_t ng = 128u / (uint32_t)a.gs;
    const uint32_t off = (uint32_t)n * (K / (uint32_t)a.gs) * 4u + (c0 / (uint32_t)a.gs) * 4u;
    const __amdgpu_buffer_rsrc_t r = rsrc(a.meta[0], a.meta_bytes[0]);
    if (ng == 4)
      s.m = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 8u * hh, 0, 0));
    else if (ng == 2)
      s.m.x = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4u * hh, 0, 0);
    else if (hh == 0)
      s.m.x = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
}

// 16-bit piece p of a 2-word, 2-bit code run (8 codes) as 8 codes in bytes
// 0 and 2: codes 0-3 in byte 0, codes 4-7 in byte 2 (2 bits each).
__device__ __forceinline__ uint32_t spread2(uint32_t p) { return (p & 0xFFu) | ((p & 0xFF00u) << 8); }

// A operand of one MFMA step: the lane's 8 codes in element order
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

// B operand: 8 activations (two per word, column order) in the same element
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

template <int KIND, bool XBF16, bool MBF16, bool PERCH>
__global__ void __launch_bounds__(64 * kSxWaves) k_skinny(SxArgs a) {
  // per wave: S and T of the current block, [S/T][group in block][row]
  __shared__ __attribute__((aligned(16))) float s_st[kSxWaves][2][8][kSxRows];
  // partial sums [wave][tile][weight row][activation row]
  __shared__ float s_part[kSxWaves][2][16][17];

  constexpr float MAG = mag<KIND, XBF16>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * kSxRows;
  const int64_t mrow = (int64_t)blockIdx.y * 16 + r16;   // this lane's activation row (B column)
  const int KB = (int)(a.K / kSxCols);
  const int gs = KIND == S_Q6K ? 16 : (KIND == S_Q4K ? 32 : a.gs);

  const uint32_t one = XBF16 ? 0x3F803F80u : 0x3C003C00u;
  const uint4 ONES = make_uint4(one, one, one, one);
  float4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float4_t D[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float4_t DX = {0.f, 0.f, 0.f, 0.f};
  float4_t Dh[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // Q6K: second group of a step
  float4_t DXh = {0.f, 0.f, 0.f, 0.f};

  // the block's metadata of one 128-column block -> (S, T) in s_st[wave]
  auto stage_meta = [&](const SxStage<KIND>& s) {
    const int rr = lane >> 1, hh = lane & 1;
    if constexpr (KIND == S_AFF2 || KIND == S_AFF4 || KIND == S_AFF8) {
      const int ng = 128 / gs;
      // partner lane (hh ^ 1) holds the other array of the same row
      const uint32_t ox = (uint32_t)__builtin_amdgcn_mov_dpp((int)s.m.x, 0xB1, 0xF, 0xF, false);
      const uint32_t oy = (uint32_t)__builtin_amdgcn_mov_dpp((int)s.m.y, 0xB1, 0xF, 0xF, false);
      const uint32_t sw[2] = {hh ? ox : s.m.x, hh ? oy : s.m.y};   // scales
      const uint32_t bw[2] = {hh ? s.m.x : ox, hh ? s.m.y : oy};   // biases
      for (int gg = hh; gg < ng; gg += 2) {
        const uint32_t sb = (sw[gg >> 1] >> (16 * (gg & 1))) & 0xFFFFu;
        const uint32_t bb = (bw[gg >> 1] >> (16 * (gg & 1))) & 0xFFFFu;
        const float S = meta_f(sb, MBF16);
        s_st[wave][0][gg][rr] = S;
        s_st[wave][1][gg][rr] = fmaf(-MAG, S, meta_f(bb, MBF16));
      }
    } else if constexpr (KIND == S_Q4K) {
      const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)s.m.x, 0xB1, 0xF, 0xF, false);
      const uint32_t sc = hh ? o : s.m.x, zc = hh ? s.m.x : o;
      const float sstep = f16_to_f32(s.st & 0xFFFFu), zstep = f16_to_f32(s.st >> 16);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int gg = 2 * q + hh;
        const float S = (float)((sc >> (8 * gg)) & 0xFFu) * sstep;
        const float Z = (float)((zc >> (8 * gg)) & 0xFFu) * zstep;
        s_st[wave][0][gg][rr] = S;
        s_st[wave][1][gg][rr] = -S * (MAG + Z);
      }
    } else if constexpr (KIND == S_Q6K) {
      const float step = f16_to_f32(s.st & 0xFFFFu);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gg = 4 * hh + q;
        const float S = (float)(int)(int8_t)((s.m.x >> (8 * q)) & 0xFFu) * step;
        s_st[wave][0][gg][rr] = S;
        s_st[wave][1][gg][rr] = -S * (MAG + 32.f);
      }
    } else if constexpr (!PERCH) {
      const int ng = 128 / gs;
      for (int q = 0; q < 2; ++q) {
        const int gg = (ng == 4 ? 2 * hh : hh) + q;
        if (gg < ng && (ng == 4 || q == 0)) {
          const float S = __uint_as_float(q ? s.m.y : s.m.x);
          s_st[wave][0][gg][rr] = S;
          s_st[wave][1][gg][rr] = -S * (MAG + 8.f);
        }
      }
    }
  };

  // group gg of the current block is complete for D, DX: apply its (S, T)
  auto epilogue = [&](int gg, const float4_t (&Dd)[2], const float4_t& DXd) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float4_t S = *reinterpret_cast<const float4_t*>(&s_st[wave][0][gg][16 * i + 4 * g]);
      const float4_t T = *reinterpret_cast<const float4_t*>(&s_st[wave][1][gg][16 * i + 4 * g]);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][v] = fmaf(T[v], DXd[v], fmaf(S[v], Dd[i][v], acc[i][v]));
    }
  };

  auto compute = [&](SxStage<KIND>& s) {
    // code words of both tiles, transposed so that step t is columns
    // 32 t .. 32 t + 31 of the block
    uint32_t W[2][4], W2[2][4], H[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (KIND == S_AFF2 || KIND == S_Q6K) {
        const uint32_t* src = KIND == S_AFF2 ? s.w[i] : s.h[i];
        uint32_t p[4] = {src[0] & 0xFFFFu, src[0] >> 16, src[1] & 0xFFFFu, src[1] >> 16};
        transpose4(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) (KIND == S_AFF2 ? W : H)[i][t] = p[t];
      }
      if constexpr (KIND == S_AFF8) {
        uint32_t p[4] = {s.w[i][0], s.w[i][2], s.w[i][4], s.w[i][6]};
        uint32_t q[4] = {s.w[i][1], s.w[i][3], s.w[i][5], s.w[i][7]};
        transpose4(p);
        transpose4(q);
#pragma unroll
        for (int t = 0; t < 4; ++t) { W[i][t] = p[t]; W2[i][t] = q[t]; }
      } else if constexpr (KIND != S_AFF2) {
        uint32_t p[4] = {s.w[i][0], s.w[i][1], s.w[i][2], s.w[i][3]};
        transpose4(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) W[i][t] = p[t];
      }
    }
    if constexpr (!PERCH) {
      stage_meta(s);
      // the wave reads back other lanes' S, T: wait for the writes
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 B = act_frag(s.x[t]);
      if constexpr (KIND == S_Q6K) {
        // two groups per step: lane groups 0-1 (group 2 t), 2-3 (2 t + 1)
        const uint4 Z = make_uint4(0, 0, 0, 0);
        const uint4 Bl = g < 2 ? B : Z, Bh = g < 2 ? Z : B;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 A = code_frag<KIND, XBF16>(W[i][t], 0u, H[i][t]);
          D[i] = mfma<XBF16>(A, Bl, D[i]);
          Dh[i] = mfma<XBF16>(A, Bh, Dh[i]);
        }
        DX = mfma<XBF16>(ONES, Bl, DX);
        DXh = mfma<XBF16>(ONES, Bh, DXh);
        epilogue(2 * t, D, DX);
        epilogue(2 * t + 1, Dh, DXh);
        D[0] = D[1] = Dh[0] = Dh[1] = DX = DXh = float4_t{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          D[i] = mfma<XBF16>(code_frag<KIND, XBF16>(W[i][t], KIND == S_AFF8 ? W2[i][t] : 0u, 0u), B, D[i]);
        DX = mfma<XBF16>(ONES, B, DX);
        if constexpr (!PERCH) {
          // a group ends every gs / 32 steps
          const int spg = gs / 32;
          if ((t + 1) % spg == 0) {
            epilogue(t / spg, D, DX);
            D[0] = D[1] = DX = float4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
  };

  // the wave's column blocks: wave, wave + 8, ...; one block in flight ahead
  SxStage<KIND> st[2];
  const int J = wave < KB ? (KB - wave + kSxWaves - 1) / kSxWaves : 0;
  if (J > 0) sx_load<KIND, PERCH>(a, wave, lane, n0, mrow, st[0]);
  for (int j0 = 0; j0 < J; j0 += 2) {
    sfor<2>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const int j = j0 + q;
      if (j < J) {
        if (j + 1 < J) sx_load<KIND, PERCH>(a, wave + (j + 1) * kSxWaves, lane, n0, mrow, st[(q + 1) % 2]);
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
  if (mm < a.M && n < a.N) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kSxWaves; ++w) sum += s_part[w][nl >> 4][nl & 15][m];
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

template <int KIND, bool MB, bool PERCH>
SxFn sx_pick(bool xb) {
  return xb ? k_skinny<KIND, true, MB, PERCH> : k_skinny<KIND, false, MB, PERCH>;
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
  a.gs = d.gs;
  a.ydt = ydt;
  a.qw_bytes = (uint32_t)bytes[0];
  a.qh_bytes = (uint32_t)bytes[1];
  a.x_bytes = (uint32_t)((uint64_t)M * d.K * 2);
  for (int q = 0; q < 3; ++q) a.meta_bytes[q] = (uint32_t)((bytes[2 + q] + 15) & ~size_t(15));
  const bool xb = xdt == BF16, mb = d.meta == BF16;
  SxFn fn = nullptr;
  if (d.fmt == AFFINE) {
    if (d.bits == 2) fn = mb ? sx_pick<S_AFF2, true, false>(xb) : sx_pick<S_AFF2, false, false>(xb);
    else if (d.bits == 4) fn = mb ? sx_pick<S_AFF4, true, false>(xb) : sx_pick<S_AFF4, false, false>(xb);
    else fn = mb ? sx_pick<S_AFF8, true, false>(xb) : sx_pick<S_AFF8, false, false>(xb);
  } else if (d.fmt == Q4K) {
    fn = sx_pick<S_Q4K, false, false>(xb);
  } else if (d.fmt == Q6K) {
    fn = sx_pick<S_Q6K, false, false>(xb);
  } else {
    fn = d.gs == d.K ? sx_pick<S_SYM4, false, true>(xb) : sx_pick<S_SYM4, false, false>(xb);
  }
  const unsigned blocks = (unsigned)((d.N + kSxRows - 1) / kSxRows);
  const unsigned mtiles = (unsigned)((M + 15) / 16);
  hipLaunchKernelGGL(fn, dim3(blocks, mtiles), dim3(64 * kSxWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace qp
