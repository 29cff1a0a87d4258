// qGEMV: decode-shaped quantized linear, y[m, :] = x[m, :] W^T for M <= 8.
//
// Design (gfx950, wave64):
//  * Codes.  The packed codes of a row are streamed in 16-byte chunks; lane l
//    of a wave always owns the chunks c = cbase + j*64 + l (j < CPL), so each
//    load instruction reads 1 KiB of contiguous codes, the per-lane offsets
//    are fixed for the whole kernel and the row is added as the scalar offset
//    of a raw buffer load (non-temporal: the codes are read once).
//  * Metadata.  Scales, biases / zero codes, steps and the linear bias of all
//    the rows a block owns are contiguous in every array, so the block copies
//    each array's slice into LDS with direct 16-byte buffer->LDS loads before
//    it computes; lanes then read their group's metadata from LDS.  Small
//    per-lane metadata loads interleaved with the code stream cost more than
//    half of HBM bandwidth; the staged copy keeps the HBM traffic in long
//    contiguous runs.
//  * Activations.  With one activation row the block stages x in LDS next to
//    the metadata; each lane takes its slice from there (SYM4: the block
//    builds the pairs once), rearranged into the bf16 (fp16) pairs that
//    match the code pairs (one v_perm_b32 per pair) with their sums (v_dot2
//    against (1, 1)), and reuses it for every row.  With several rows (M
//    tile > 1) each lane loads its slices directly.
//  * Arithmetic.  Codes become bf16 (fp16) pairs without a conversion
//    instruction: v_perm_b32 places a code byte under the high byte of 128.0
//    bf16 (1024.0 fp16), which is exactly 128 + q (1024 + q).  One v_dot2
//    per pair accumulates sum (MAG + q) * x in fp32; the MAG * sum(x) part is
//    removed in the per-group epilogue, where the group's scale and offset
//    are applied once per chunk in fp32:
//        sum_k w_k x_k = S * sum (MAG + q) x - S * (MAG + Z) * sum x
//    (AFFINE: S = scale, S*Z = -bias; Q4K: S = sc*sstep, Z = zc*zstep;
//    Q6K: Z = 32, SYM4: Z = 8 from the stored code offsets).  8-bit codes use
//    byte-to-fp32 conversions and fp32 FMAs instead (128 + 255 is not exact
//    in bf16).
//  * Q4K / Q6K fp16 steps are shared by the 8 lanes that cover one
//    256-weight super-block: the first lane of each 8 reads the step word and
//    ds_swizzle (bit mode, and-mask 0x18) hands it to the other seven -- the
//    superscale page's "one shuffle per super-block" on wave64.
//  * Rows.  A wave owns a contiguous run of rows.  When they fit one batch
//    (M = 1) all of the wave's code loads go out at once; otherwise batches
//    of rows are double-buffered.  Partial sums of a row are reduced across
//    the wave with DPP row rotations and broadcasts; when a row's K range is
//    split over KW waves of the block, the wave partials meet in LDS.
//
// Formats: see include/qlinear.h.  Sources: HF Transformers "Metal" page
// (uint32 codes, per-group scale/bias, bits 2/4/8); ExecuTorch PR #20571
// "Quant schema update" (Q4_K/Q6_K-style nested metadata; the int6 per-group
// int8 scale codes are read once per 16-byte code load); ExecuTorch PR
// #16577 (symmetric int4, qmin=-7..7).
#include "device_common.hpp"
#include "qp_internal.hpp"

namespace qp {
namespace {

enum Kind : int {
  K_AFF2 = 0, K_AFF4 = 1, K_AFF8 = 2, K_Q4K = 3, K_Q6K = 4, K_SYM4 = 5,
  // affine codes with fp16 (instead of bf16) scales and biases
  K_AFF2H = 6, K_AFF4H = 7, K_AFF8H = 8
};
constexpr int base_kind(int k) { return k >= K_AFF2H ? k - K_AFF2H : k; }

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
template <>
struct KT<K_AFF2H> : KT<K_AFF2> {};
template <>
struct KT<K_AFF4H> : KT<K_AFF4> {};
template <>
struct KT<K_AFF8H> : KT<K_AFF8> {};

constexpr bool is_affine(int k) { return base_kind(k) <= K_AFF8; }
constexpr bool meta_is_bf16(int k) { return k < K_AFF2H; }
// With one activation row, SYM4 has the block build the activation pairs once
// in LDS; the other kinds are faster pairing in each wave (measured).
constexpr bool x_prep_in_lds(int k, int mt) { return mt == 1 && base_kind(k) == K_SYM4; }

// Metadata arrays staged in LDS: 0 = scales / scale codes, 1 = biases / zero
// codes, 2 = steps, 3 = linear bias.
constexpr int kMeta = 4;

struct GemvArgs {
  const uint32_t* qw;     // [N, C*4] u32 (16-byte chunks)
  const uint32_t* qh;     // Q6K high plane [N, K/16] u32
  const void* meta[kMeta];
  const uint16_t* x;      // [M, K] fp16|bf16 bits
  void* y;                // [M, N]
  int64_t N, K, M;
  int C;                  // 16-byte chunks per row
  int gs;
  int ydt;
  int KW;                 // waves splitting K per row team
  int RPT;                // rows per team
  // buffer sizes in bytes (bounds of the buffer resources)
  uint32_t qw_bytes, qh_bytes, x_bytes;
  uint32_t meta_bytes[kMeta];
  // metadata bytes per row, and LDS byte offset of each staged slice
  uint32_t meta_row[kMeta];
  uint32_t meta_lds[kMeta];
  uint32_t x_lds;         // LDS byte offset of the staged activation row (MT == 1)
  uint32_t x_prep;        // LDS byte offset of its pairs [C][XW] u32 and sums [C][GP] f32
};

// Raw buffer loads (gfx9 buffer resource, stride 0).  An offset at or beyond
// the resource's size reads 0 without touching memory, which is how lanes
// outside the problem are masked: no branches, and the loads of a batch
// stay independent of each other.
constexpr uint32_t kOOB = 0x80000000u;   // every buffer is < 2 GiB (host check)
// Cache policy of the streamed code loads: non-temporal (read once).
#ifndef QP_GEMV_CODE_AUX
#define QP_GEMV_CODE_AUX 2
#endif
constexpr int kNT = QP_GEMV_CODE_AUX;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

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

// v_perm_b32 pairs: S1 = the magic high byte replicated, S0 = code bytes.
// pair_bytes02 -> [code byte 0, magic, code byte 2, magic] (two halves of a
// bf16/fp16 pair); pair_bytes13 -> the same for bytes 1 and 3.
__device__ __forceinline__ uint32_t pair_bytes02(uint32_t codes, uint32_t magic) {
  return __builtin_amdgcn_perm(codes, magic, 0x00060004u);
}
__device__ __forceinline__ uint32_t pair_bytes13(uint32_t codes, uint32_t magic) {
  return __builtin_amdgcn_perm(codes, magic, 0x00070005u);
}

#ifndef QP_GEMV_LOADS_PER_BATCH
#define QP_GEMV_LOADS_PER_BATCH 4   // 16-byte code loads per lane, double-buffered mode
#endif
#ifndef QP_GEMV_MULTI_SUM
#define QP_GEMV_MULTI_SUM 1
#endif
// One activation row, one wave per row range: the batch's row sums by one
// transposed reduction (wave_sums8) instead of one DPP chain per row, and 8
// lanes store them.  It runs at the very end of every wave, where the last
// rows' data has just landed: timed on the decode layers, int4 affine
// 8.87 -> 8.10 us, int2 8.41 -> 7.40, SYM4 9.61 -> 9.49; Q4K, Q6K and int8
// were 0.5-2.5% slower with it and keep the per-row chains.
__host__ __device__ constexpr bool multi_sum(int k) {
  return QP_GEMV_MULTI_SUM &&
         (base_kind(k) == K_AFF4 || base_kind(k) == K_AFF2 || base_kind(k) == K_SYM4);
}
#ifndef QP_GEMV_MIN_WAVES_PER_EU
#define QP_GEMV_MIN_WAVES_PER_EU 2
#endif

// Single-batch mode, per format (timed on the decode layers): int4 affine
// and Q4K request up to 14 loads per lane (7 rows of two chunks at K = 4096)
// and all of them before the prologue wait; the other formats do best with
// 8 loads (int6, with its second code plane, 6), three rows of which go out
// before the wait.
__host__ __device__ constexpr bool wide_single(int k) {
  return base_kind(k) == K_AFF4 || base_kind(k) == K_Q4K;
}
__host__ __device__ constexpr int single_loads(int k) {
  return wide_single(k) ? 14 : (base_kind(k) == K_Q6K ? 6 : 8);
}
__host__ __device__ constexpr int early_rows(int k) { return wide_single(k) ? 8 : 3; }

// Rows per batch.  Double-buffered mode (NB = 2): enough 16-byte loads per
// lane in flight while the other batch is computed, fewer rows when the M
// tile multiplies the registers of every row.  Single-batch mode (NB = 1):
// a wave owns at most one batch and requests all of it at once.
__host__ __device__ constexpr int row_batch(int kind, int mt, int cpl, int nb) {
  const int loads = nb == 1 ? single_loads(kind) : QP_GEMV_LOADS_PER_BATCH;
  const int base = loads / cpl > 0 ? loads / cpl : 1;
  const int capped = base > 8 ? 8 : base;
  return mt >= 2 ? (capped > 2 ? 2 : capped) : capped;
}

// Raw code words of one batch of RB rows.
template <int KIND, int RB, int CPL>
struct Batch {
  uint4 cw[RB][CPL];
  uint2 hw[RB][CPL];          // Q6K high plane
};

template <int KIND, int RB, int CPL, int RLO = 0, int RHI = RB>
__device__ __forceinline__ void load_batch(const GemvArgs& a, __amdgpu_buffer_rsrc_t rqw,
                                           __amdgpu_buffer_rsrc_t rqh, const uint32_t (&lane_cw)[CPL],
                                           Batch<KIND, RB, CPL>& B, int r, int rowEnd) {
  const uint32_t C = (uint32_t)a.C;
#pragma unroll
  for (int rb = RLO; rb < RHI; ++rb) {
    // rows past the end of a partial batch re-read the last valid row
    // (already on its way to this wave's caches); their results are never
    // stored
    const uint32_t n = (uint32_t)max(min(r + rb, rowEnd - 1), 0);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      B.cw[rb][j] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rqw, lane_cw[j], n * C * 16u, kNT));
      if constexpr (base_kind(KIND) == K_Q6K)
        B.hw[rb][j] = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(rqh, lane_cw[j] == kOOB ? kOOB : lane_cw[j] / 2u,
                                                        n * (uint32_t)(a.K / 4), kNT));
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the loads in row order
  }
}

template <typename T>
__device__ __forceinline__ T lds_read(const uint8_t* smem, uint32_t byte) {
  return *reinterpret_cast<const T*>(smem + byte);
}

// Scale S and offset T of each part of one chunk (see the file comment):
// its contribution is S * (dot of codes and activations) + T * (sum of the
// activations).  m0..m2: LDS byte offsets of the row's staged scales,
// biases / zero codes and steps; meta: the lane's byte offset(s) in the
// row; step: the lane's step offset (kOOB for lanes that do not lead 8).
template <int KIND, bool XBF16, int GP>
__device__ __forceinline__ void chunk_meta(const uint8_t* smem, uint32_t m0, uint32_t m1,
                                           uint32_t m2, const uint32_t (&meta)[GP],
                                           uint32_t step, float (&S)[GP], float (&Tt)[GP]) {
  constexpr int BK = base_kind(KIND);
  constexpr float MAGF = XBF16 ? 128.f : 1024.f;
  if constexpr (is_affine(KIND)) {
#pragma unroll
    for (int p = 0; p < GP; ++p) {
      const uint32_t sb = lds_read<uint16_t>(smem, m0 + meta[p]);
      const uint32_t bb = lds_read<uint16_t>(smem, m1 + meta[p]);
      const float sv = meta_is_bf16(KIND) ? bf16_to_f32(sb) : f16_to_f32(sb);
      const float bv = meta_is_bf16(KIND) ? bf16_to_f32(bb) : f16_to_f32(bb);
      S[p] = sv;
      Tt[p] = (BK == K_AFF8) ? bv : fmaf(-MAGF, sv, bv);
    }
  } else if constexpr (BK == K_Q4K) {
    uint32_t st = 0;
    if (step != kOOB) st = lds_read<uint32_t>(smem, m2 + step);
    st = bcast8(st);
    const float Sv = (float)lds_read<uint8_t>(smem, m0 + meta[0]) * f16_to_f32(st & 0xFFFFu);
    const float Z = (float)lds_read<uint8_t>(smem, m1 + meta[0]) * f16_to_f32(st >> 16);
    S[0] = Sv;
    Tt[0] = -Sv * (MAGF + Z);
  } else if constexpr (BK == K_Q6K) {
    uint32_t st = 0;
    if (step != kOOB) st = lds_read<uint16_t>(smem, m2 + step);
    st = bcast8(st);
    const float stp = f16_to_f32(st & 0xFFFFu);
    const uint32_t sc2 = lds_read<uint16_t>(smem, m0 + meta[0]);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float Sv = (float)(int)(int8_t)(sc2 >> (8 * p)) * stp;
      S[p] = Sv;
      Tt[p] = -Sv * (MAGF + 32.f);
    }
  } else {  // SYM4
    const float sv = lds_read<float>(smem, m0 + meta[0]);
    S[0] = sv;
    Tt[0] = -sv * (MAGF + 8.f);
  }
}

// Dot products of one 16-byte code chunk (and for Q6K its high-plane bits)
// with the matching activation pairs: acc[m][part] = sum (MAG + q) * x
// (8-bit codes: sum q * x).  Codes only; no metadata.
template <int KIND, bool XBF16, int MT, int XW, int GP>
__device__ __forceinline__ void chunk_dots(const uint4 cw, const uint2 hw,
                                           const uint32_t (&xq)[MT][XW], float (&acc)[MT][GP]) {
  constexpr int BK = base_kind(KIND);
  // high byte of 128.0 bf16 (0x4300) or 1024.0 fp16 (0x6400), replicated
  const uint32_t magic = XBF16 ? 0x43434343u : 0x64646464u;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int p = 0; p < GP; ++p) acc[m][p] = 0.f;
  const uint32_t wv[4] = {cw.x, cw.y, cw.z, cw.w};
  if constexpr (BK == K_AFF8) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float q = (float)((wv[i] >> (8 * t)) & 0xFFu);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][0] = fmaf(q, __uint_as_float(xq[m][4 * i + t]), acc[m][0]);
      }
  } else if constexpr (BK == K_AFF2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // bytes of f = codes t, 4+t, 8+t, 12+t of the word
        const uint32_t f = (wv[i] >> (2 * t)) & 0x03030303u;
        const uint32_t pa = pair_bytes02(f, magic);   // pair t     = (t, 8+t)
        const uint32_t pb = pair_bytes13(f, magic);   // pair 4 + t = (4+t, 12+t)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[m][i / 2] = dot2<XBF16>(pa, xq[m][8 * i + t], acc[m][i / 2]);
          acc[m][i / 2] = dot2<XBF16>(pb, xq[m][8 * i + 4 + t], acc[m][i / 2]);
        }
      }
  } else if constexpr (BK == K_Q6K) {
    // high-plane bytes reordered [b0 b2 b1 b3] so that the two codes of
    // each pair find their 2-bit tops in the matching 16-bit halves
    const uint32_t h0 = __builtin_amdgcn_perm(hw.x, hw.x, 0x03010200u);
    const uint32_t h1 = __builtin_amdgcn_perm(hw.y, hw.y, 0x03010200u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t hh = (i < 2 ? h0 : h1) >> (8 * (i % 2));
      const uint32_t lo = wv[i] & 0x0F0F0F0Fu;
      const uint32_t hi = (wv[i] >> 4) & 0x0F0F0F0Fu;
      const uint32_t pl[4] = {pair_bytes02(lo, magic), pair_bytes02(hi, magic),
                              pair_bytes13(lo, magic), pair_bytes13(hi, magic)};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // top 2 bits of the pair's codes moved to bits 4-5 of each half
        const uint32_t top =
            (s == 0 ? (hh << 4) : s == 1 ? (hh << 2) : s == 2 ? hh : (hh >> 2)) & 0x00300030u;
        const uint32_t pr = pl[s] | top;
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][i / 2] = dot2<XBF16>(pr, xq[m][4 * i + s], acc[m][i / 2]);
      }
    }
  } else {  // nibbles: AFF4, Q4K, SYM4
    // even-position nibbles to bytes, odd-position nibbles to bytes, then
    // v_perm pairs byte b with byte b+2 under the magic high bytes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = wv[i] & 0x0F0F0F0Fu;          // codes 0 2 4 6
      const uint32_t hi = (wv[i] >> 4) & 0x0F0F0F0Fu;   // codes 1 3 5 7
      const uint32_t pr[4] = {pair_bytes02(lo, magic), pair_bytes02(hi, magic),
                              pair_bytes13(lo, magic), pair_bytes13(hi, magic)};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][0] = dot2<XBF16>(pr[s], xq[m][4 * i + s], acc[m][0]);
    }
  }
}

template <int KIND, bool XBF16, int MT, int CPL, int RB, int XW, int GP>
__device__ __forceinline__ void compute_batch(const GemvArgs& a, const uint8_t* smem,
                                              const Batch<KIND, RB, CPL>& B,
                                              const uint32_t (&lane_meta)[CPL][GP],
                                              const uint32_t (&lane_step)[CPL],
                                              const uint32_t (&row_base)[kMeta], int lrow0,
                                              int lrmax,
                                              const uint32_t (&xq)[CPL][MT][XW],
                                              const float (&xs)[CPL][MT][GP],
                                              float (&yacc)[RB][MT]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[rb][m] = 0.f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // LDS byte offsets of this row's metadata (wave-uniform); rows past the
    // end of a partial batch use the last valid row, like their code loads
    const uint32_t lr = (uint32_t)min(lrow0 + rb, lrmax);
    const uint32_t m0 = row_base[0] + lr * a.meta_row[0];
    const uint32_t m1 = row_base[1] + lr * a.meta_row[1];
    const uint32_t m2 = row_base[2] + lr * a.meta_row[2];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float S[GP], Tt[GP];
      chunk_meta<KIND, XBF16, GP>(smem, m0, m1, m2, lane_meta[j], lane_step[j], S, Tt);
      float acc[MT][GP];
      chunk_dots<KIND, XBF16, MT, XW, GP>(B.cw[rb][j], B.hw[rb][j], xq[j], acc);
      // masked chunks carry zero codes and zero activations: they add 0
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int p = 0; p < GP; ++p)
          yacc[rb][m] = fmaf(Tt[p], xs[j][m][p], fmaf(S[p], acc[m][p], yacc[rb][m]));
    }
  }
}

// The activations of one chunk (CC values, raw fp16/bf16 bits in u) as the
// pairs that match the code pairs of compute_batch, and their per-part sums.
template <int KIND, bool XBF16>
__device__ __forceinline__ void x_pairs(const uint32_t (&u)[KT<base_kind(KIND)>::CC / 2],
                                        uint32_t (&q)[KT<base_kind(KIND)>::XW],
                                        float (&sum)[KT<base_kind(KIND)>::GP]) {
  constexpr int GP = KT<base_kind(KIND)>::GP;
#pragma unroll
  for (int p = 0; p < GP; ++p) sum[p] = 0.f;
  if constexpr (base_kind(KIND) == K_AFF8) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t bits = (u[t / 2] >> (16 * (t % 2))) & 0xFFFFu;
      q[t] = __float_as_uint(xval<XBF16>(bits));
      sum[0] += xval<XBF16>(bits);
    }
  } else {
    // pair s of word w = (activation s, activation s + PW) of the word's
    // codes: the low halves of two raw words, or their high halves, joined
    // by one v_perm_b32 (S0 supplies the low half, S1 the high half)
    constexpr int PW = (base_kind(KIND) == K_AFF2) ? 8 : 4;   // pairs per word
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int sidx = 0; sidx < PW; ++sidx) {
        const uint32_t a = u[w * PW + sidx / 2];            // activations 2t, 2t+1
        const uint32_t b = u[w * PW + PW / 2 + sidx / 2];   // the same PW further on
        q[w * PW + sidx] = __builtin_amdgcn_perm(a, b, (sidx & 1) ? 0x03020706u : 0x01000504u);
      }
    // the part sums by v_dot2 against (1, 1): products exact, fp32 sums
    const uint32_t one2 = XBF16 ? 0x3F803F80u : 0x3C003C00u;
    constexpr int NU = KT<base_kind(KIND)>::CC / 2;
#pragma unroll
    for (int t = 0; t < NU; ++t) sum[GP == 2 ? t / (NU / 2) : 0] = dot2<XBF16>(u[t], one2, sum[GP == 2 ? t / (NU / 2) : 0]);
  }
}

// Copies bytes [row0 * rowBytes, (row0 + rows) * rowBytes) of a metadata
// array into LDS (from the 16-byte aligned address at or below the start;
// returns the start's offset inside the copy).  Wave w copies 1 KiB pieces
// w, w+4, ... with direct buffer->LDS loads; bytes past the array read 0.
__device__ __forceinline__ uint32_t stage_meta(uint8_t* smem, __amdgpu_buffer_rsrc_t r,
                                               uint32_t rowBytes, uint32_t row0, uint32_t rows,
                                               uint32_t ldsOff, int wave, int lane) {
  const uint32_t src0 = row0 * rowBytes;
  const uint32_t a0 = src0 & ~15u;
  const uint32_t nbytes = (src0 - a0) + rows * rowBytes;
  const uint32_t nch = (nbytes + 1023u) / 1024u;
  for (uint32_t ch = (uint32_t)wave; ch < nch; ch += 4) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(smem + ldsOff + ch * 1024u), 16,
        a0 + ch * 1024u + 16u * (uint32_t)lane, 0, 0, 0);
  }
  return src0 - a0;
}

template <int KIND, bool XBF16, int MT, int CPL, int NB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QP_GEMV_MIN_WAVES_PER_EU)))
k_gemv(GemvArgs a) {
  using T = KT<KIND>;
  constexpr int CC = T::CC, XW = T::XW, GP = T::GP;
  constexpr int RB = row_batch(KIND, MT, CPL, NB);
  constexpr int NV = CC / 8;   // 16-byte loads of x per chunk

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float red[4][RB][MT];

  const int lane = threadIdx.x & 63;
  // wave index: uniform across the wave, so row offsets stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KW = a.KW;
  const int kw = wave % KW;
  const int team = wave / KW;
  const int RW = 4 / KW;
  // row indices fit 32 bits: every buffer is < 2 GiB (host check)
  const int NR = (int)a.N;
  const int brow0 = (int)blockIdx.x * RW * a.RPT;   // first row of the block
  const int row0 = brow0 + team * a.RPT;
  const int rowEnd = min(row0 + a.RPT, NR);
  const int rowStop = row0 + a.RPT;   // same trip count for every team
  const int brows = min(RW * a.RPT, NR - brow0);
  const int mbase = blockIdx.y * MT;
  const int C = a.C;
  const int cbase = kw * CPL * 64;

  // ---- 1. the block's metadata slices, and (one activation row) x itself,
  // -> LDS with direct loads; the code stream is released only once this
  // small prologue has landed, so that it does not queue behind the codes
  // of the whole grid
  uint32_t row_base[kMeta];
#pragma unroll
  for (int i = 0; i < kMeta; ++i) {
    row_base[i] = a.meta_lds[i];
    if (a.meta_row[i])
      row_base[i] += stage_meta(smem, rsrc(a.meta[i], a.meta_bytes[i]), a.meta_row[i],
                                (uint32_t)brow0, (uint32_t)brows, a.meta_lds[i], wave, lane);
  }
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  if constexpr (MT == 1)
    stage_meta(smem, rx, (uint32_t)(2 * a.K), (uint32_t)mbase, 1u, a.x_lds, wave, lane);
  // other M tiles: this lane's activations straight into registers
  constexpr int NXR = MT == 1 ? 1 : MT;
  uint4 xv[CPL][NXR][NV];
  if constexpr (MT > 1) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = cbase + j * 64 + lane;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bool ok = c < C && (mbase + m) < a.M;
        const uint32_t base = (uint32_t)((mbase + m) * a.K + (int64_t)c * CC) * 2u;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          xv[j][m][v] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? base + 16u * v : kOOB, 0, 0));
      }
    }
  }
  // rows of the first batch requested before the wait (early_rows)
  const __amdgpu_buffer_rsrc_t rqw = rsrc(a.qw, a.qw_bytes);
  const __amdgpu_buffer_rsrc_t rqh = rsrc(a.qh, a.qh_bytes);
  uint32_t lane_cw[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = cbase + j * 64 + lane;
    lane_cw[j] = c < C ? (uint32_t)c * 16u : kOOB;
  }
  constexpr int EARLY = early_rows(KIND) < RB ? early_rows(KIND) : RB;
  Batch<KIND, RB, CPL> B0;
  if constexpr (EARLY > 0) {
    load_batch<KIND, RB, CPL, 0, EARLY>(a, rqw, rqh, lane_cw, B0, row0, rowEnd);
    constexpr int n = EARLY * CPL * (base_kind(KIND) == K_Q6K ? 2 : 1);
    constexpr int nn = n > 63 ? 63 : n;
    __builtin_amdgcn_s_waitcnt((nn & 0xF) | (0x7 << 4) | (0xF << 8) | ((nn >> 4) << 14));
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  constexpr bool PREP = x_prep_in_lds(KIND, MT);
  if constexpr (MT == 1 && !PREP) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = cbase + j * 64 + lane;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        xv[j][0][v] = c < C ? lds_read<uint4>(smem, a.x_lds + (uint32_t)c * (CC * 2) + 16u * v)
                            : make_uint4(0, 0, 0, 0);
    }
  }
  if constexpr (PREP) {
    // one activation row: the block turns it into pairs and sums once
    const uint32_t pq = a.x_prep, ps = a.x_prep + (uint32_t)C * XW * 4u;
    for (int c = threadIdx.x; c < C; c += 256) {
      uint32_t u[CC / 2], q[XW];
      float sm[GP];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint4 t = lds_read<uint4>(smem, a.x_lds + (uint32_t)c * (CC * 2) + 16u * v);
        u[4 * v] = t.x; u[4 * v + 1] = t.y; u[4 * v + 2] = t.z; u[4 * v + 3] = t.w;
      }
      x_pairs<KIND, XBF16>(u, q, sm);
#pragma unroll
      for (int v = 0; v < XW / 4; ++v)
        *reinterpret_cast<uint4*>(smem + pq + (uint32_t)c * XW * 4u + 16u * v) =
            make_uint4(q[4 * v], q[4 * v + 1], q[4 * v + 2], q[4 * v + 3]);
#pragma unroll
      for (int p = 0; p < GP; ++p)
        *reinterpret_cast<float*>(smem + ps + (uint32_t)(c * GP + p) * 4u) = sm[p];
    }
    __syncthreads();
  }

  // ---- 2. the rest of the first batch of code rows
  uint32_t lane_meta[CPL][GP], lane_step[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = cbase + j * 64 + lane;
    const bool ok = c < C;
    const uint32_t cu = ok ? (uint32_t)c : 0u;   // masked lanes read row metadata at 0
    lane_step[j] = kOOB;
#pragma unroll
    for (int p = 0; p < GP; ++p) lane_meta[j][p] = 0;
    if constexpr (is_affine(KIND)) {
#pragma unroll
      for (int p = 0; p < GP; ++p) lane_meta[j][p] = 2u * ((cu * CC + p * (CC / GP)) / (uint32_t)a.gs);
    } else if constexpr (base_kind(KIND) == K_Q4K) {
      lane_meta[j][0] = cu;
      if ((lane & 7) == 0) lane_step[j] = 4u * (cu / 8u);
    } else if constexpr (base_kind(KIND) == K_Q6K) {
      lane_meta[j][0] = 2u * cu;
      if ((lane & 7) == 0) lane_step[j] = 2u * (cu / 8u);
    } else {
      lane_meta[j][0] = 4u * ((cu * CC) / (uint32_t)a.gs);
    }
  }
  if constexpr (EARLY < RB) load_batch<KIND, RB, CPL, EARLY, RB>(a, rqw, rqh, lane_cw, B0, row0, rowEnd);

  // ---- 3. activations as pairs matching the code pairs, and their sums
  uint32_t xq[CPL][MT][XW];
  float xs[CPL][MT][GP];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = cbase + j * 64 + lane;
    if constexpr (PREP) {
      const bool ok = c < C;
      const uint32_t cc = ok ? (uint32_t)c : 0u;
#pragma unroll
      for (int v = 0; v < XW / 4; ++v) {
        const uint4 t = lds_read<uint4>(smem, a.x_prep + cc * XW * 4u + 16u * v);
        xq[j][0][4 * v] = ok ? t.x : 0u; xq[j][0][4 * v + 1] = ok ? t.y : 0u;
        xq[j][0][4 * v + 2] = ok ? t.z : 0u; xq[j][0][4 * v + 3] = ok ? t.w : 0u;
      }
#pragma unroll
      for (int p = 0; p < GP; ++p)
        xs[j][0][p] = ok ? lds_read<float>(smem, a.x_prep + (uint32_t)C * XW * 4u + (cc * GP + p) * 4u)
                         : 0.f;
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint32_t u[CC / 2];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          u[4 * v] = xv[j][m][v].x; u[4 * v + 1] = xv[j][m][v].y;
          u[4 * v + 2] = xv[j][m][v].z; u[4 * v + 3] = xv[j][m][v].w;
        }
        x_pairs<KIND, XBF16>(u, xq[j][m], xs[j][m]);
      }
    }
  }

  auto finish = [&](float (&yacc)[RB][MT], int r) {
    if constexpr (MT == 1 && multi_sum(KIND)) {
      if (KW == 1) {
        // all rows of the batch at once; 8 lanes store in parallel
        float v[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) v[rb] = yacc[rb][0];
        const float t = wave_sums8<RB>(v, lane);
        const int R = lane >> 4;
        const int rb = 4 * ((lane >> 3) & 1) + (((R & 1) << 1) | (R >> 1));
        const int n = r + rb;
        if ((lane & 7) == 0 && rb < RB && n < rowEnd && mbase < a.M) {
          const float bv =
              a.meta_row[3] ? xval<XBF16>(lds_read<uint16_t>(smem, row_base[3] + 2u * (uint32_t)(n - brow0)))
                            : 0.f;
          store_y(a.y, (int64_t)mbase * a.N + n, t + bv, a.ydt);
        }
        return;
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int m = 0; m < MT; ++m) yacc[rb][m] = wave_sum_lane63(yacc[rb][m]);
    if (KW == 1) {
      if (lane == 63) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int n = r + rb;
          if (n < rowEnd) {
            const float bv =
                a.meta_row[3] ? xval<XBF16>(lds_read<uint16_t>(smem, row_base[3] + 2u * (uint32_t)(n - brow0)))
                              : 0.f;
#pragma unroll
            for (int m = 0; m < MT; ++m)
              if (mbase + m < a.M)
                store_y(a.y, (int64_t)(mbase + m) * a.N + n, yacc[rb][m] + bv, a.ydt);
          }
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
        const int n = r + rb;
        if (n < rowEnd && mbase + m < a.M) {
          const float bv =
              a.meta_row[3] ? xval<XBF16>(lds_read<uint16_t>(smem, row_base[3] + 2u * (uint32_t)(n - brow0)))
                            : 0.f;
          store_y(a.y, (int64_t)(mbase + m) * a.N + n, v + bv, a.ydt);
        }
      }
      __syncthreads();
    }
  };

  float yacc[RB][MT];
  if constexpr (NB == 1) {
    // ---- one batch in flight at a time (normally a wave owns one batch)
    for (int r = row0; r < rowStop; r += RB) {
      if (KW == 1 && r >= rowEnd) break;
      if (r != row0 && r < rowEnd) load_batch<KIND, RB, CPL>(a, rqw, rqh, lane_cw, B0, r, rowEnd);
      compute_batch<KIND, XBF16, MT, CPL, RB, XW, GP>(a, smem, B0, lane_meta, lane_step, row_base,
                                                      r - brow0, rowEnd - 1 - brow0, xq, xs, yacc);
      finish(yacc, r);
    }
    return;
  }
  // ---- row loop, double-buffered: the next batch's loads are in flight
  // while the current one is computed
  Batch<KIND, RB, CPL> B1;
  for (int r = row0; r < rowStop; r += 2 * RB) {
    if (KW == 1 && r >= rowEnd) break;
    if (r + RB < rowEnd) load_batch<KIND, RB, CPL>(a, rqw, rqh, lane_cw, B1, r + RB, rowEnd);
    compute_batch<KIND, XBF16, MT, CPL, RB, XW, GP>(a, smem, B0, lane_meta, lane_step, row_base,
                                                    r - brow0, rowEnd - 1 - brow0, xq, xs, yacc);
    finish(yacc, r);
    if (r + RB >= rowStop || (KW == 1 && r + RB >= rowEnd)) break;
    if (r + 2 * RB < rowEnd) load_batch<KIND, RB, CPL>(a, rqw, rqh, lane_cw, B0, r + 2 * RB, rowEnd);
    compute_batch<KIND, XBF16, MT, CPL, RB, XW, GP>(a, smem, B1, lane_meta, lane_step, row_base,
                                                    r + RB - brow0, rowEnd - 1 - brow0, xq, xs, yacc);
    finish(yacc, r + RB);
  }
}

typedef void (*GemvFn)(GemvArgs);

template <int KIND, bool XB, int MT, int NB>
GemvFn pick_cpl(int cpl) {
  switch (cpl) {
    case 1: return k_gemv<KIND, XB, MT, 1, NB>;
    case 2: return MT <= 4 ? (GemvFn)k_gemv<KIND, XB, (MT <= 4 ? MT : 4), 2, NB> : nullptr;
    case 3: return MT <= 2 ? (GemvFn)k_gemv<KIND, XB, (MT <= 2 ? MT : 2), 3, NB> : nullptr;
    case 4: return MT <= 2 ? (GemvFn)k_gemv<KIND, XB, (MT <= 2 ? MT : 2), 4, NB> : nullptr;
  }
  return nullptr;
}

template <int KIND, bool XB>
GemvFn pick_mt(int mt, int cpl, int nb) {
  if (nb == 1) return mt == 1 ? pick_cpl<KIND, XB, 1, 1>(cpl) : nullptr;
  switch (mt) {
    case 1: return pick_cpl<KIND, XB, 1, 2>(cpl);
    case 2: return pick_cpl<KIND, XB, 2, 2>(cpl);
    case 4: return pick_cpl<KIND, XB, 4, 2>(cpl);
    case 8: return pick_cpl<KIND, XB, 8, 2>(cpl);
  }
  return nullptr;
}

template <int KIND>
GemvFn pick_x(bool xb, int mt, int cpl, int nb) {
  return xb ? pick_mt<KIND, true>(mt, cpl, nb) : pick_mt<KIND, false>(mt, cpl, nb);
}

GemvFn pick(int kind, bool xb, int mt, int cpl, int nb) {
  switch (kind) {
    case K_AFF2: return pick_x<K_AFF2>(xb, mt, cpl, nb);
    case K_AFF4: return pick_x<K_AFF4>(xb, mt, cpl, nb);
    case K_AFF8: return pick_x<K_AFF8>(xb, mt, cpl, nb);
    case K_Q4K: return pick_x<K_Q4K>(xb, mt, cpl, nb);
    case K_Q6K: return pick_x<K_Q6K>(xb, mt, cpl, nb);
    case K_SYM4: return pick_x<K_SYM4>(xb, mt, cpl, nb);
    case K_AFF2H: return pick_x<K_AFF2H>(xb, mt, cpl, nb);
    case K_AFF4H: return pick_x<K_AFF4H>(xb, mt, cpl, nb);
    case K_AFF8H: return pick_x<K_AFF8H>(xb, mt, cpl, nb);
  }
  return nullptr;
}

// Chooses the M tile, the K split and the chunks per lane so that the
// lane's activations fit its register budget (CPL * MT chunks of 16
// activation pairs; fewer for 2-bit codes, which have 32 pairs per chunk, and
// for int6, which carries a second code plane); one chunk per lane fits
// any M tile except for 2-bit codes, whose 32 activation pairs per chunk and
// row spill beyond an M tile of 4.  Shrinks the M tile if needed.
bool gemv_plan(int k, int C, int* mt, int* KW, int* cpl) {
  const int kind = base_kind(k);
  const int budget = kind == K_AFF2 ? 4 : (kind == K_Q6K ? 4 : (kind == K_AFF8 ? 8 : 6));
  const int mt_one_chunk = kind == K_AFF2 ? 4 : 8;
  for (int m = *mt; m >= 1; m /= 2) {
    for (int kw = 1; kw <= 4; kw *= 2) {
      int c = (C + 64 * kw - 1) / (64 * kw);
      if (c <= 4 && (c * m <= budget || (c == 1 && m <= mt_one_chunk))) {
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
#ifndef QP_GEMV_MAX_WAVES_PER_CU
#define QP_GEMV_MAX_WAVES_PER_CU 16
#endif
constexpr int kNumCU = 256;
constexpr uint32_t kMaxMetaLds = 48 * 1024;   // staged metadata per block

int gemv_kind(const Desc& d) {
  if (d.fmt == AFFINE)
    return (d.bits == 2 ? K_AFF2 : (d.bits == 4 ? K_AFF4 : K_AFF8)) + (d.meta == BF16 ? 0 : K_AFF2H);
  if (d.fmt == Q4K) return K_Q4K;
  if (d.fmt == Q6K) return K_Q6K;
  return K_SYM4;
}

int gemv_chunks(const Desc& d, int k) {
  const int kind = base_kind(k);
  const int CC = kind == K_AFF2 ? 64 : (kind == K_AFF8 ? 16 : 32);
  return (int)(d.K / CC);
}

// Metadata bytes per row of each staged array (0 = absent).
void meta_rows(const Desc& d, bool bias, uint32_t row[kMeta]) {
  const uint32_t K = (uint32_t)d.K, ng = (uint32_t)(d.K / d.gs);
  for (int i = 0; i < kMeta; ++i) row[i] = 0;
  if (d.fmt == AFFINE) { row[0] = 2 * ng; row[1] = 2 * ng; }
  else if (d.fmt == Q4K) { row[0] = K / 32; row[1] = K / 32; row[2] = 4 * (K / 256); }
  else if (d.fmt == Q6K) { row[0] = K / 16; row[2] = 2 * (K / 256); }
  else { row[0] = 4 * ng; }
  if (bias) row[3] = 2;
}

uint32_t meta_lds_bytes(const uint32_t row[kMeta], int64_t blockRows, uint32_t off[kMeta]) {
  uint32_t total = 0;
  for (int i = 0; i < kMeta; ++i) {
    off[i] = total;
    if (row[i]) total += ((15u + (uint32_t)blockRows * row[i] + 1023u) / 1024u) * 1024u;
  }
  return total;
}

}  // namespace

bool gemv_supported(const Desc& d) {
  const int kind = gemv_kind(d);
  int mt = 1, kw = 0, cpl = 0;
  if (!gemv_plan(kind, gemv_chunks(d, kind), &mt, &kw, &cpl)) return false;
  // one block's metadata rows and one activation row must fit LDS even for
  // a single row per wave
  uint32_t row[kMeta], off[kMeta];
  meta_rows(d, true, row);
  return meta_lds_bytes(row, 4 / kw, off) + 4 * d.K + 2048 + 34 * gemv_chunks(d, kind) * 4 <=
         kMaxMetaLds + 64 * 1024;
}

hipError_t launch_gemv(const Desc& d, const void* x, int xdt, int64_t M, const Bufs& b,
                       const void* bias, void* y, int ydt, const size_t bytes[5],
                       hipStream_t s) {
  const int kind = gemv_kind(d);
  const int C = gemv_chunks(d, kind);
  int mt = M >= 8 ? 8 : (M >= 4 ? (M == 4 ? 4 : 8) : (M == 3 ? 4 : (int)M));
  int KW = 1, cpl = 0;
  if (!gemv_plan(kind, C, &mt, &KW, &cpl)) return hipErrorInvalidValue;
  const int RW = 4 / KW;
  const int64_t teamsTarget = (int64_t)kNumCU * QP_GEMV_WAVES_PER_CU / KW;
  uint32_t row[kMeta];
  meta_rows(d, bias != nullptr, row);
  auto pad16 = [](uint64_t n) { return (uint32_t)((n + 15) & ~uint64_t(15)); };
  uint32_t rowMeta = 0;
  for (int i = 0; i < kMeta; ++i) rowMeta += row[i];
  // Single-batch mode when every team's rows fit one batch with at most
  // QP_GEMV_MAX_WAVES_PER_CU waves per CU: all of a wave's loads go out at
  // once.  Otherwise double-buffered batches.
  int nb = 2;
  int64_t rpt = (d.N + teamsTarget - 1) / teamsTarget;
  if (mt == 1) {
    const int rb1 = row_batch(kind, 1, cpl, 1);
    const int64_t teams1 = (d.N + rb1 - 1) / rb1;
    const int64_t teamsMax = (int64_t)kNumCU * QP_GEMV_MAX_WAVES_PER_CU / KW;
    if (teams1 <= teamsMax) {
      nb = 1;
      const int64_t teams = teams1 > teamsTarget ? teams1 : teamsTarget;
      rpt = (d.N + teams - 1) / teams;   // <= rb1
    }
  }
  // the block's staged metadata must fit LDS: fewer rows per team if not
  const int64_t rptMeta = (int64_t)((kMaxMetaLds / 2) / ((uint64_t)RW * (rowMeta + 1)));
  if (rpt > rptMeta) rpt = rptMeta > 0 ? rptMeta : 1;
  if (nb == 2) {
    const int rb = row_batch(kind, mt, cpl, 2);
    rpt = (rpt + rb - 1) / rb * rb;       // a whole number of batches
  }
  GemvFn fn = pick(kind, xdt == BF16, mt, cpl, nb);
  if (!fn) return hipErrorInvalidValue;
  const int64_t teams = (d.N + rpt - 1) / rpt;
  const int64_t blocks = (teams + RW - 1) / RW;
  GemvArgs a;
  a.qw = static_cast<const uint32_t*>(b.qweight);
  a.qh = static_cast<const uint32_t*>(b.qweight_hi);
  a.meta[0] = b.scales;
  a.meta[1] = b.zeros;
  a.meta[2] = b.steps;
  a.meta[3] = bias;
  a.x = static_cast<const uint16_t*>(x);
  a.y = y;
  a.N = d.N;
  a.K = d.K;
  a.M = M;
  a.C = C;
  a.gs = d.gs;
  a.ydt = ydt;
  a.KW = KW;
  a.RPT = (int)rpt;
  a.qw_bytes = (uint32_t)bytes[0];
  a.qh_bytes = (uint32_t)bytes[1];
  a.x_bytes = (uint32_t)(M * d.K * 2);
  // metadata is copied in 16-byte units: the buffers are readable up to
  // the next multiple of 16 bytes (part of the ABI contract)
  a.meta_bytes[0] = pad16(bytes[2]);
  a.meta_bytes[1] = pad16(bytes[3]);
  a.meta_bytes[2] = pad16(bytes[4]);
  a.meta_bytes[3] = bias ? pad16((uint64_t)d.N * 2) : 0u;
  for (int i = 0; i < kMeta; ++i) a.meta_row[i] = row[i];
  uint32_t lds = meta_lds_bytes(row, (int64_t)RW * rpt, a.meta_lds);
  a.x_lds = lds;
  a.x_prep = lds;
  if (mt == 1) lds += (uint32_t)(((15 + 2 * d.K) + 1023) / 1024 * 1024);
  a.x_prep = lds;
  if (x_prep_in_lds(kind, mt)) lds += ((uint32_t)C * (16 + 1) * 4u + 15u) & ~15u;
  const unsigned mtiles = (unsigned)((M + mt - 1) / mt);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks, mtiles), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace qp
