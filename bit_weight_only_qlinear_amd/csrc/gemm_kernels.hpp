// qGEMM kernels: prefill-shaped quantized linear, y = x W^T for large M, on gfx950
// fp16 MFMA (v_mfma_f32_32x32x16_f16), fp32 accumulation.
//
// The pages' prefill ran on dequantized bf16 "runtime weights" (superscale
// page, A100 take-aways); here the packed codes stay in HBM and each block
// dequantizes its weight tile on the way into LDS.  The tile is rounded once
// to fp16 rather than bf16: bf16 keeps 8 significant bits, which is not
// enough for the output tolerance of this layer, fp16 keeps 11, and gfx950
// runs fp16 and bf16 MFMA at the same rate.  bf16 activations are converted
// to fp16 in the same staging step after an exact power-of-two prescale per
// row (k_xexp) that puts the row's peak in [2^14, 2^15), so any finite bf16
// row fits fp16's range; the fp32 epilogue undoes the scale.
//
// Design:
//  * Block tile 256 (n) x 256 (m) x 64 (k), 8 waves in a 2 (n) x 4 (m)
//    grid, each wave owning 128 x 64 outputs (8 MFMA tiles of 32 x 32, 128
//    fp32 accumulators per lane), two waves per SIMD: while one wave waits on
//    LDS or converts, the other keeps the matrix core busy.  The weight tile
//    is the MFMA A operand, the activation tile the B operand, so each lane
//    ends with 4 consecutive output columns n per row m.
//  * LDS holds two stages of fp16 tiles (2 x (32 + 32) KiB); each 128-byte
//    tile row is split into 16-byte chunks stored at chunk ^ ((row >> 1) & 7).
//    gfx950 LDS has 64 banks (256 bytes per clock): two consecutive rows
//    share one bank line, and this swizzle gives the 16 lanes of every
//    ds_read_b128 / ds_write_b128 phase 16 different 16-byte bank groups
//    (a plain chunk ^ (row & 7) leaves every fragment read 2-way conflicted).
//  * Global loads are raw buffer loads (rows past M or N read 0) staged two
//    k-steps ahead in registers: while the MFMAs of step k run, the block
//    converts step k+1 (already in registers) into the other LDS stage and
//    the loads of step k+2 are in flight.  One barrier per k-step.
//  * Dequantization.  Within every 8-column chunk the columns are stored in
//    the order (0,4,1,5,2,6,3,7) in both tiles (a contraction does not care
//    about the order of k, as long as both operands agree), which is the
//    order in which a packed int4 word yields fp16 pairs: (w >> 4i) &
//    0x000F000F | 0x64006400 is the fp16 pair (1024 + q_i, 1024 + q_{i+4}).
//    Affine int4 then takes one packed subtract and one packed fma per pair:
//    w = fma(q, scale, bias) in fp16, a single rounding of the exact weight
//    when scale and bias are fp16-exact (any bf16 of magnitude >= 2^-14 is).
//    The other formats use w = fma(u, S, T) in fp32 with u the stored
//    unsigned field, rounded once to fp16:
//      AFFINE: S = scale, T = bias;  Q4K: S = sc*sstep, T = -S*zc*zstep;
//      Q6K: S = sc*step, T = -32*S;  SYM4: S = scale, T = -8*S.
//    SYM4 with one scale per output channel keeps the codes themselves
//    (S = 1, T = -8, exact in fp16) and scales the fp32 result per channel
//    in the epilogue: no weight rounding, so no limit on K.
//  * Tiles are handed out so that each XCD works on a contiguous run of
//    tiles (shared L2).
//
// The kernel templates live in this header; each format's instantiations are
// compiled in a translation unit of their own (gemm_aff2/4/8.hip,
// gemm_kq.hip) and the host side (activation staging, tiling choice,
// dispatch) in gemm.hip.
#pragma once
#include <utility>

#include "device_common.hpp"
#include "qp_internal.hpp"

namespace qp {

struct GemmArgs {
  const void* qw;
  const void* qh;
  const void* scales;
  const void* zeros;
  const void* steps;
  const void* x;
  const void* xf;   // activations staged for k_gemm224 (gemm.hip), else null
  const int* xe;    // their prescale exponents (bf16, k_gemm224), else null
  const void* bias;
  void* y;
  int64_t M, N, K;
  int gs, ydt, tilesM, tilesN;
};

// Launches the qGEMM kernel of one format family on `blocks` blocks: n224
// selects the 224-row tiles over staged activations, mch the chunked
// affine metadata, xb bf16 activations, mb bf16 metadata.
struct GemmPick {
  bool n224, mch, xb, mb;
};
hipError_t gemm_launch_aff2(const GemmArgs& a, const GemmPick& p, unsigned blocks, hipStream_t s);
hipError_t gemm_launch_aff4(const GemmArgs& a, const GemmPick& p, unsigned blocks, hipStream_t s);
hipError_t gemm_launch_aff8(const GemmArgs& a, const GemmPick& p, unsigned blocks, hipStream_t s);
hipError_t gemm_launch_kq(int fmt, const GemmArgs& a, const GemmPick& p, unsigned blocks,
                          hipStream_t s);

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 512;
#ifndef QP_GEMM_PIN_LOADS
#define QP_GEMM_PIN_LOADS 0
#endif
#ifndef QP_GEMM_ROLL
#define QP_GEMM_ROLL 1
#endif
#ifndef QP_GEMM_SGB
#define QP_GEMM_SGB 1
#endif
#ifndef QP_GEMM_SGB_VALU
#define QP_GEMM_SGB_VALU 4
#endif
#ifndef QP_GEMM_DSW_LATE
#define QP_GEMM_DSW_LATE 1
#endif
constexpr uint32_t kTileBytes = 256u * BK * 2u;   // one fp16 tile (32 KiB)
// LDS: weight tiles of stages 0 and 1, then activation tiles of stages 0, 1
// -- every address is a per-lane base plus an immediate below 64 KiB
constexpr uint32_t kXBase = 2u * kTileBytes;

// G_SYM4C: SYM4 with one scale per output channel, contracted on the exact
// codes q = u - 8 (fp16-exact); the channel scale multiplies the fp32 sum in
// the epilogue, so no weight is rounded.
enum GKind : int { G_AFF2 = 0, G_AFF4 = 1, G_AFF8 = 2, G_Q4K = 3, G_Q6K = 4, G_SYM4 = 5,
                   G_SYM4C = 6 };

// Packed code words per weight row per 64-column step (W), and Q6K high
// plane words (H).  Two threads share a weight row, each taking half.
template <int KIND> struct GT { static constexpr int W = 8, H = 0; };
template <> struct GT<G_AFF2> { static constexpr int W = 4, H = 0; };
template <> struct GT<G_AFF8> { static constexpr int W = 16, H = 0; };
template <> struct GT<G_Q6K> { static constexpr int W = 8, H = 4; };

// Prescale exponent of activation row m for the 256-row tiling, as the
// exponent kernel left it in y at (m, c): the first column of each n-tile of
// the row.  Only the block of that tile reads it, before it writes the tile.
__device__ __forceinline__ int read_exp(const GemmArgs& a, int64_t m, int64_t c) {
  const int64_t i = m * a.N + c;
  return a.ydt == F32 ? static_cast<const int*>(a.y)[i]
                      : (int)(int16_t) static_cast<const uint16_t*>(a.y)[i];
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at
// compile time (register arrays indexed by i stay in registers).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T>
__device__ __forceinline__ T lds_ld(const unsigned char* smem, uint32_t off) {
  return *reinterpret_cast<const T*>(smem + off);
}

// One k-step of one thread's global data, in registers: 4 activation
// chunks (rows (t >> 3) + 64 i, columns 8 (t & 7) ..), and half of weight row
// wrow_of(t) (columns 32 (t & 1) .. + 31) with its metadata.
template <int KIND>
struct Stage {
  uint4 x[4];                                     // raw activation bits
  uint32_t w[GT<KIND>::W / 2];                    // codes
  uint32_t h[GT<KIND>::H > 0 ? GT<KIND>::H / 2 : 1];
  uint32_t s0, s1, s2;                            // raw metadata (see load_stage)
};

// Buffer resources and per-thread offsets of one block.
struct Rsrc {
  __amdgpu_buffer_rsrc_t x, w, h, s, z, p;
  uint32_t xo;       // this thread's activation chunk in row (t >> 3)
  uint32_t xstride;  // 64 activation rows, bytes
  uint32_t wo, ho;   // this thread's half weight row: codes, Q6K high plane
  uint32_t so, zo, po;  // start of its row: scales, zeros, steps
  uint32_t half;     // t & 1
};

// Every offset is a per-lane (voffset) offset, so the buffer range check
// covers all of it: steps at or past K (the pipeline's two phantom steps)
// read either the next row's data or 0, never memory outside the buffers.
template <int KIND, bool GS32, bool LOADX = true, bool LOADMETA = true>
__device__ __forceinline__ void load_stage(const GemmArgs& a, const Rsrc& r, int kt,
                                           Stage<KIND>& st) {
  if constexpr (LOADX) {
    const uint32_t xk = (uint32_t)kt * (BK * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st.x[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(r.x, r.xo + (uint32_t)i * r.xstride + xk, 0, 0));
  }
  constexpr int W = GT<KIND>::W;
  const uint32_t wk = r.wo + (uint32_t)kt * (W * 4);
  if constexpr (W == 4) {
    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r.w, wk, 0, 0));
    st.w[0] = v.x; st.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < W / 8; ++i) {
      const uint4 v = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(r.w, wk + 16u * i, 0, 0));
      st.w[4 * i] = v.x; st.w[4 * i + 1] = v.y; st.w[4 * i + 2] = v.z; st.w[4 * i + 3] = v.w;
    }
  }
  st.s0 = st.s1 = st.s2 = 0;
  if constexpr (KIND == G_Q6K) {   // high code plane (codes, not metadata)
    const uint2 v = __builtin_bit_cast(
        uint2, __builtin_amdgcn_raw_buffer_load_b64(r.h, r.ho + (uint32_t)kt * 16u, 0, 0));
    st.h[0] = v.x; st.h[1] = v.y;
  }
  if constexpr (!LOADMETA) return;
  const uint32_t g2 = 2u * (uint32_t)kt + r.half;   // this half's group of 32
  if constexpr (KIND == G_AFF2 || KIND == G_AFF4 || KIND == G_AFF8) {
    const uint32_t g = GS32 ? g2 : (uint32_t)kt * BK / (uint32_t)a.gs;
    st.s0 = __builtin_amdgcn_raw_buffer_load_b16(r.s, r.so + g * 2u, 0, 0);
    st.s1 = __builtin_amdgcn_raw_buffer_load_b16(r.z, r.zo + g * 2u, 0, 0);
  } else if constexpr (KIND == G_Q4K) {
    // uint8 scale code, uint8 zero code, the super-block step word
    st.s0 = __builtin_amdgcn_raw_buffer_load_b8(r.s, r.so + g2, 0, 0);
    st.s1 = __builtin_amdgcn_raw_buffer_load_b8(r.z, r.zo + g2, 0, 0);
    st.s2 = __builtin_amdgcn_raw_buffer_load_b32(r.p, r.po + (uint32_t)(kt / 4) * 4u, 0, 0);
  } else if constexpr (KIND == G_Q6K) {
    // two int8 scale codes (groups of 16), the super-block fp16 step
    st.s0 = __builtin_amdgcn_raw_buffer_load_b16(r.s, r.so + 2u * g2, 0, 0);
    st.s2 = __builtin_amdgcn_raw_buffer_load_b16(r.p, r.po + (uint32_t)(kt / 4) * 2u, 0, 0);
  } else if constexpr (KIND == G_SYM4) {  // fp32 scale
    const uint32_t g = GS32 ? g2 : (uint32_t)kt * BK / (uint32_t)a.gs;
    st.s0 = __builtin_amdgcn_raw_buffer_load_b32(r.s, r.so + g * 4u, 0, 0);
  }
}

// (S, T) of group `grp` of a stage's half row (only Q6K has two groups).
template <int KIND, bool MBF16>
__device__ __forceinline__ void group_st(const Stage<KIND>& st, int grp, float& S, float& T) {
  if constexpr (KIND == G_AFF2 || KIND == G_AFF4 || KIND == G_AFF8) {
    const uint32_t sb = st.s0 & 0xFFFFu, tb = st.s1 & 0xFFFFu;
    S = MBF16 ? bf16_to_f32(sb) : f16_to_f32(sb);
    T = MBF16 ? bf16_to_f32(tb) : f16_to_f32(tb);
  } else if constexpr (KIND == G_Q4K) {
    const float sc = (float)(st.s0 & 0xFFu);
    const float zc = (float)(st.s1 & 0xFFu);
    S = sc * f16_to_f32(st.s2 & 0xFFFFu);
    T = -S * (zc * f16_to_f32(st.s2 >> 16));
  } else if constexpr (KIND == G_Q6K) {
    const float sc = (float)(int8_t)((st.s0 >> (8 * grp)) & 0xFFu);
    S = sc * f16_to_f32(st.s2 & 0xFFFFu);
    T = -32.f * S;
  } else if constexpr (KIND == G_SYM4) {
    S = __uint_as_float(st.s0);
    T = -8.f * S;
  } else {   // G_SYM4C: the code itself, u - 8
    S = 1.f;
    T = -8.f;
  }
}

// Unsigned field of element e (0..7) of 8-column chunk j (0..3) of a stage's
// half row.
template <int KIND>
__device__ __forceinline__ uint32_t field(const Stage<KIND>& st, int j, int e) {
  if constexpr (KIND == G_AFF2) return (st.w[j >> 1] >> (2 * (8 * (j & 1) + e))) & 3u;
  else if constexpr (KIND == G_AFF8) return (st.w[2 * j + (e >> 2)] >> (8 * (e & 3))) & 255u;
  else if constexpr (KIND == G_Q6K)
    return ((st.w[j] >> (4 * e)) & 15u) | (((st.h[j >> 1] >> (2 * (8 * (j & 1) + e))) & 3u) << 4);
  else return (st.w[j] >> (4 * e)) & 15u;
}

// (t & m) | c in one instruction; m comes from an SGPR, c from a VGPR (one
// VOP3 operand may be scalar).  Its result must pass through a compiler-
// visible VALU instruction before an MFMA reads it: the hazard recognizer
// does not see into inline asm.
__device__ __forceinline__ uint32_t and_or(uint32_t t, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(t), "s"(m), "v"(c));
  return r;
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  half2_t h;
  h.x = (_Float16)lo;
  h.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, h);
}

// Weight chunk j of the thread's row as 8 fp16 in the order (0,4,1,5,2,6,3,7).
template <int KIND, bool MBF16>
__device__ __forceinline__ uint4 weight_chunk(const Stage<KIND>& st, int j, uint32_t magic) {
  const int grp = KIND == G_Q6K ? (j >> 1) : 0;   // Q6K groups hold 16 columns
  float S, T;
  group_st<KIND, MBF16>(st, grp, S, T);
  uint32_t p[4];
  if constexpr (KIND == G_AFF4) {
    half2_t s2, t2;
    s2.x = s2.y = (_Float16)S;
    t2.x = t2.y = (_Float16)T;
    const half2_t mag = {(_Float16)1024.f, (_Float16)1024.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m = and_or(st.w[j] >> (4 * i), 0x000F000Fu, magic);
      const half2_t q = __builtin_bit_cast(half2_t, m) - mag;
      p[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, t2));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = pack_f16(fmaf((float)field<KIND>(st, j, i), S, T),
                      fmaf((float)field<KIND>(st, j, i + 4), S, T));
  }
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// 8 activations (raw bits) as fp16 in the order (0,4,1,5,2,6,3,7); bf16
// activations are first scaled by 2^e, the row's prescale exponent (exact),
// which brings the row's largest magnitude into [2^14, 2^15).
template <bool XBF16>
__device__ __forceinline__ uint4 act_chunk(const uint4 u, int e = 0) {
  if constexpr (XBF16) {
    // bf16 -> fp32 is a shift, the scaling exact; fp32 -> fp16 is exact for
    // magnitudes within 2^-10 .. 2^31 of the row's largest (everything a
    // bf16's 8 significant bits can hold there), smaller ones round
    auto lo = [e](uint32_t v) { return ldexpf(__uint_as_float(v << 16), e); };
    auto hi = [e](uint32_t v) { return ldexpf(__uint_as_float(v & 0xFFFF0000u), e); };
    return make_uint4(pack_f16(lo(u.x), lo(u.z)), pack_f16(hi(u.x), hi(u.z)),
                      pack_f16(lo(u.y), lo(u.w)), pack_f16(hi(u.y), hi(u.w)));
  } else {
    return make_uint4(__builtin_amdgcn_perm(u.z, u.x, 0x05040100u),
                      __builtin_amdgcn_perm(u.z, u.x, 0x07060302u),
                      __builtin_amdgcn_perm(u.w, u.y, 0x05040100u),
                      __builtin_amdgcn_perm(u.w, u.y, 0x07060302u));
  }
}

// Weight row staged by thread t (two threads per row, t & 1 = which half).
// LDS writes are serviced 8 lanes at a time over 32 banks; mapping the 8
// lanes of each phase to rows {0, 2, 4, 6} (+ 8k, then {1, 3, 5, 7}) gives
// them 4 different swizzles, i.e. 8 different bank groups.
__device__ __forceinline__ int wrow_of(int t) {
  return 8 * (t >> 4) + 2 * ((t >> 1) & 3) + ((t >> 3) & 1);
}

// Part p (0..3) of converting a stage into LDS stage buffer `buf`: the
// thread's activation chunk of row (t >> 3) + 64 p and weight chunk p of its
// half row.
template <int KIND, bool XBF16, bool MBF16>
__device__ __forceinline__ void convert_part(const Stage<KIND>& st, int p, unsigned char* smem,
                                             uint32_t buf, int tid, uint32_t magic, const int* xe) {
  // activation row (tid >> 3) + 64 p: (row >> 1) & 7 == (tid >> 4) & 7
  const uint32_t xb = kXBase + (uint32_t)(tid >> 3) * 128u +
                      (uint32_t)((tid & 7) ^ ((tid >> 4) & 7)) * 16u;
  *reinterpret_cast<uint4*>(smem + xb + (buf * kTileBytes + 8192u * p)) =
      act_chunk<XBF16>(st.x[p], XBF16 ? xe[(tid >> 3) + 64 * p] : 0);
  const int n = wrow_of(tid), j = 4 * (tid & 1) + p;
  const uint32_t wb = (uint32_t)n * 128u + (uint32_t)((j ^ ((n >> 1) & 7)) * 16);
  *reinterpret_cast<uint4*>(smem + wb + buf * kTileBytes) = weight_chunk<KIND, MBF16>(st, p, magic);
}

// Weight-side buffer resources and offsets of a block's rows n0 .. n0 +
// nrows - 1 (rows past them read 0); thread t stages half row wrow_of(t).
template <int KIND>
__device__ __forceinline__ void weight_rsrc(const GemmArgs& a, int64_t n0, int64_t nrows, int tid,
                                            Rsrc& r) {
  const int64_t K = a.K;
  const int64_t wrow = (KIND == G_AFF2 ? K / 4 : KIND == G_AFF8 ? K : K / 2);
  r.w = rsrc(static_cast<const unsigned char*>(a.qw) + n0 * wrow, (uint32_t)(nrows * wrow));
  r.half = (uint32_t)(tid & 1);
  const int64_t n = wrow_of(tid);
  r.wo = (uint32_t)(n * wrow) + r.half * (uint32_t)(GT<KIND>::W * 2);
  r.h = r.w;
  r.ho = 0;
  if constexpr (KIND == G_Q6K) {
    r.h = rsrc(static_cast<const unsigned char*>(a.qh) + n0 * (K / 4), (uint32_t)(nrows * (K / 4)));
    r.ho = (uint32_t)(n * (K / 4)) + r.half * 8u;
  }
  int64_t srow = 0, zrow = 0, prow = 0;   // bytes per weight row
  if constexpr (KIND == G_Q4K) { srow = K / 32; zrow = K / 32; prow = (K / 256) * 4; }
  else if constexpr (KIND == G_Q6K) { srow = K / 16; prow = (K / 256) * 2; }
  else if constexpr (KIND == G_SYM4 || KIND == G_SYM4C) { srow = (K / a.gs) * 4; }
  else { srow = (K / a.gs) * 2; zrow = srow; }
  r.s = rsrc(static_cast<const unsigned char*>(a.scales) + n0 * srow, (uint32_t)(nrows * srow));
  r.so = (uint32_t)(n * srow);
  r.z = r.s; r.zo = r.so;
  if (zrow) {
    r.z = rsrc(static_cast<const unsigned char*>(a.zeros) + n0 * zrow, (uint32_t)(nrows * zrow));
    r.zo = (uint32_t)(n * zrow);
  }
  r.p = r.s; r.po = 0;
  if (prow) {
    r.p = rsrc(static_cast<const unsigned char*>(a.steps) + n0 * prow, (uint32_t)(nrows * prow));
    r.po = (uint32_t)(n * prow);
  }
}

template <int KIND, bool XBF16, bool MBF16, bool GS32>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kTileBytes];
  __shared__ int s_xe[BM];   // prescale exponents of the block's activation rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 2, wj = wave & 3;   // n half, m quarter

  // XCD-aware tile order: consecutive block ids land on different XCDs, so
  // give each XCD a contiguous run of tiles (m fastest).
  const int T = a.tilesM * a.tilesN;
  const int bid = blockIdx.x;
  const int tile = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;  // a bijection
  const int tm = tile % a.tilesM, tn = tile / a.tilesM;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t mrows = a.M - m0 < BM ? a.M - m0 : BM;
  const int64_t nrows = a.N - n0 < BN ? a.N - n0 : BN;
  const int64_t K = a.K;

  // ---- buffer resources of this block's rows (rows past M / N read 0)
  Rsrc r;
  {
    const uint32_t xrow = (uint32_t)(K * 2);
    r.x = rsrc(static_cast<const unsigned char*>(a.x) + m0 * K * 2, (uint32_t)mrows * xrow);
    r.xo = (uint32_t)(tid >> 3) * xrow + (uint32_t)(tid & 7) * 16u;
    r.xstride = 64u * xrow;
    weight_rsrc<KIND>(a, n0, nrows, tid, r);
  }

  float16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment addresses: lane row (lane & 31), chunk 2s + (lane >> 5) stored
  // at chunk ^ ((row >> 1) & 7) with (row >> 1) & 7 == (lane >> 1) & 7
  uint32_t fa[4], fb[4];   // per k-slice bases: weight rows, activation rows of the wave
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t f = (uint32_t)(lane & 31) * 128u +
                       (uint32_t)(((2 * s + (lane >> 5)) ^ ((lane >> 1) & 7)) * 16);
    fa[s] = f + (uint32_t)wi * 128u * 128u;
    fb[s] = f + kXBase + (uint32_t)wj * 64u * 128u;
  }

  const int KT = (int)(K / BK);
  const uint32_t magic = 0x64006400u;   // fp16 pair (1024, 1024), kept in a VGPR

  auto rd_a = [&](uint32_t buf, int s, int i) {
    return *reinterpret_cast<const half8_t*>(smem + fa[s] + (buf * kTileBytes + 4096u * i));
  };
  auto rd_b = [&](uint32_t buf, int s, int j) {
    return *reinterpret_cast<const half8_t*>(smem + fb[s] + (buf * kTileBytes + 4096u * j));
  };

  // One k-step: MFMAs on stage kt (LDS buffer kt & 1), conversion of the
  // registers of step kt+1 (`nxt`) into the other buffer, loads of step kt+2
  // into `fre` (whose step kt was converted during the previous k-step).
  // The last two k-steps load and convert phantom steps KT and KT+1 into
  // the buffer nobody reads any more (see load_stage); no per-step branch.
  auto kstep = [&](int kt, Stage<KIND>& fre, Stage<KIND>& nxt) {
    const uint32_t cur = (uint32_t)(kt & 1);
    load_stage<KIND, GS32>(a, r, kt + 2, fre);
#if QP_GEMM_PIN_LOADS
    // keep the loads at the top of the step: a whole step to arrive
    __builtin_amdgcn_sched_barrier(0);
#endif
#if QP_GEMM_ROLL
    // Rolling fragment prefetch: the next k-slice's B fragments are read at
    // the start of a slice, and A fragment i is re-read for the next slice
    // as soon as its two MFMAs have issued, so LDS latency hides behind the
    // remaining MFMAs instead of stalling every slice.
    half8_t A[4], B[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) A[i] = rd_a(cur, 0, i);
#pragma unroll
    for (int j = 0; j < 2; ++j) B[j] = rd_b(cur, 0, j);
    static_for<4>([&](auto S) {
      constexpr int s = decltype(S)::value;
      half8_t Bn[2];
      if constexpr (s < 3) {
        Bn[0] = rd_b(cur, s + 1, 0);
        Bn[1] = rd_b(cur, s + 1, 1);
      }
      static_for<4>([&](auto I) {
        constexpr int i = decltype(I)::value;
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[0], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[1], acc[i][1], 0, 0, 0);
        if constexpr (s < 3) A[i] = rd_a(cur, s + 1, i);
      });
      if constexpr (s < 3) {
        B[0] = Bn[0];
        B[1] = Bn[1];
      }
      convert_part<KIND, XBF16, MBF16>(nxt, s, smem, cur ^ 1u, tid, magic, s_xe);
#if QP_GEMM_SGB
      // instruction order of the slice: B prefetch, then per A fragment two
      // MFMAs, its re-read and a share of the conversion
      if constexpr (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      static_for<4>([&](auto I) {
        constexpr int i = decltype(I)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if constexpr (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, QP_GEMM_SGB_VALU, 0);
#if QP_GEMM_DSW_LATE
        // LDS writes after the slice's last fragment read: lgkmcnt is in
        // order, so a write issued before a read would delay that read's wait
        if constexpr (i == 3) __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
#else
        if constexpr (i == 1 || i == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
#endif
      });
#endif
    });
#else
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = rd_a(cur, s, i);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = rd_b(cur, s, j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      convert_part<KIND, XBF16, MBF16>(nxt, s, smem, cur ^ 1u, tid, magic, s_xe);
    }
#endif
    __syncthreads();
  };

  Stage<KIND> st0, st1;
  load_stage<KIND, GS32>(a, r, 0, st0);
  load_stage<KIND, GS32>(a, r, 1, st1);
  if constexpr (XBF16) {
    if (tid < BM) s_xe[tid] = m0 + tid < a.M ? read_exp(a, m0 + tid, n0) : 0;
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) convert_part<KIND, XBF16, MBF16>(st0, p, smem, 0u, tid, magic, s_xe);
  __syncthreads();
  for (int kt = 0; kt < KT; kt += 2) {
    kstep(kt, st0, st1);
    if (kt + 1 < KT) kstep(kt + 1, st1, st0);
  }

  // ---- epilogue: lane holds rows n = 8g + 4*(lane >> 5) + q (q = 0..3) of
  // column m = lane & 31 of every 32 x 32 tile, in register 4g + q.
  // Expanded at compile time with predicated stores, so the accumulators
  // stay in registers.
  const bool vec4 = (a.N % 4) == 0;
  const int ydt = a.ydt;
  const uint16_t* bias = static_cast<const uint16_t*>(a.bias);
  // an opaque copy of the lane index keeps the epilogue's addresses and
  // bias loads from being hoisted above the main loop (register pressure)
  int el = lane;
  asm volatile("" : "+v"(el));
  static_for<4>([&](auto I) {
    constexpr int i = decltype(I)::value;
    static_for<4>([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int64_t n = n0 + wi * 128 + i * 32 + 8 * g + 4 * (el >> 5);
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias != nullptr) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t nn = n + q < a.N ? n + q : a.N - 1;
          const uint32_t bb = bias[nn];
          bv[q] = XBF16 ? bf16_to_f32(bb) : f16_to_f32(bb);   // bias has the x dtype
        }
      }
      float sv[4] = {1.f, 1.f, 1.f, 1.f};   // G_SYM4C: channel scales
      if constexpr (KIND == G_SYM4C) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sv[q] = static_cast<const float*>(a.scales)[n + q < a.N ? n + q : a.N - 1];
      }
      static_for<2>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int64_t m = m0 + wj * 64 + j * 32 + (el & 31);
        const int64_t idx = m * a.N + n;
        const int xe = XBF16 ? s_xe[wj * 64 + j * 32 + (el & 31)] : 0;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = KIND == G_SYM4C ? fmaf(ldexpf(acc[i][j][4 * g + q], -xe), sv[q], bv[q])
                                 : ldexpf(acc[i][j][4 * g + q], -xe) + bv[q];
        const bool mok = m < a.M;
        if (mok && vec4 && n < a.N) {
          if (ydt == F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.y) + idx) =
                make_float4(v[0], v[1], v[2], v[3]);
          } else {
            uint32_t h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              h[q] = ydt == BF16 ? f32_to_bf16_rne(v[q]) : f32_to_f16_rne(v[q]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + idx) =
                make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
          }
        } else if (mok && !vec4) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (n + q < a.N) {
              if (ydt == F32) static_cast<float*>(a.y)[idx + q] = v[q];
              else static_cast<uint16_t*>(a.y)[idx + q] =
                  (uint16_t)(ydt == BF16 ? f32_to_bf16_rne(v[q]) : f32_to_f16_rne(v[q]));
            }
          }
        }
      });
    });
  });
}

// ===========================================================================
// qGEMM with 224-row weight tiles and staged activations (k_gemm224).
//
// Where N is 7 * 2^k (14336 = 7 * 2048), 256 x 256 tiles leave the last
// wave of blocks partly empty: at M = 2048 they make 448 blocks, 1.75 waves
// on 256 CUs.  224 (n) x 256 (m) tiles make 512 blocks, two full waves of
// 7/8 the work each.  A wave then owns 112 weight rows, not a multiple of
// 32, so this kernel runs v_mfma_f32_16x16x32_f16: 7 x 4 tiles of 16 x 16
// per wave (wave grid 2 (n) x 4 (m) as in k_gemm).  The activations are
// staged once per call (gemm.hip) as fp16 in that MFMA's B-fragment order,
// and each wave loads its B fragments straight into registers, one step
// ahead; only the weight tile goes through LDS, staged, swizzled and
// dequantized as in k_gemm (rows 224..255 of the LDS tile are unused).
// ===========================================================================
constexpr int BN7 = 224;
typedef float float4_t __attribute__((ext_vector_type(4)));

// MCH = group size (affine, 128 with K % 1024 == 0, 64 with K % 512 == 0 or
// 32 with K % 256 == 0; else 0): the scales and biases come in 16-byte
// chunks of 8 groups (one chunk per 16, 8 or 4 steps) loaded a chunk ahead
// into a two-slot register ring (group size 128: current and next chunk)
// (per step, two 2-byte loads that touch 32 cache lines per wave cost more
// than the MFMAs can hide); the step loop is unrolled by 16 so that slot
// and element are compile-time constants (group size 32: the element also
// depends on the thread's half row).
template <int KIND, bool XBF16, bool MBF16, bool GS32, int MCH>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_gemm224(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kTileBytes];
  __shared__ int s_xe[BM];   // prescale exponents of the block's activation rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 2, wj = wave & 3;   // n half (112 rows), m quarter (64 rows)

  const int T = a.tilesM * a.tilesN;
  const int bid = blockIdx.x;
  const int tile = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;  // as in k_gemm
  const int tm = tile % a.tilesM, tn = tile / a.tilesM;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN7;
  const int64_t nrows = a.N - n0 < BN7 ? a.N - n0 : BN7;
  const int64_t K = a.K;

  Rsrc r;
  weight_rsrc<KIND>(a, n0, nrows, tid, r);
  // staged activations of rows m0 .. m0 + 255 (M rounded up to 16 is staged)
  const int64_t srows = (a.M + 15) / 16 * 16 - m0;
  const __amdgpu_buffer_rsrc_t xr = rsrc(static_cast<const unsigned char*>(a.xf) + m0 * K * 2,
                                         (uint32_t)((srows < BM ? srows : BM) * K * 2));
  const uint32_t xfj = (uint32_t)(K * 32);   // 16 rows
  const uint32_t xfo = (uint32_t)(4 * wj) * xfj + (uint32_t)lane * 16u;

  float4_t acc[7][4];
#pragma unroll
  for (int i = 0; i < 7; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  // A fragment (weight rows): lane row wi*112 + 16 i + (lane & 15), 16-byte
  // chunk 4 sub + (lane >> 4), stored at chunk ^ ((row >> 1) & 7), and
  // (row >> 1) & 7 == ((lane & 15) >> 1) since 112 and 16 are multiples of 16
  uint32_t fa[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
    fa[sub] = (uint32_t)(wi * 112 + (lane & 15)) * 128u +
              (uint32_t)(((4 * sub + (lane >> 4)) ^ ((lane & 15) >> 1)) * 16);
  auto rd_a = [&](uint32_t buf, int sub, int i) {
    return *reinterpret_cast<const half8_t*>(smem + fa[sub] + (buf * kTileBytes + 2048u * i));
  };
  // B fragment (j, sub) of step kt: one contiguous 1 KiB wave load
  auto ld_b = [&](int kt, int sub, int j) {
    return __builtin_bit_cast(
        half8_t, __builtin_amdgcn_raw_buffer_load_b128(
                     xr, xfo + (uint32_t)j * xfj + (uint32_t)(2 * kt + sub) * 1024u, 0, 0));
  };
  // weight chunk p of thread's half row into LDS stage buffer buf
  const int wn = wrow_of(tid);
  auto st_w = [&](uint32_t buf, int p, uint4 v) {
    const int j = 4 * (tid & 1) + p;
    const uint32_t wb = (uint32_t)wn * 128u + (uint32_t)((j ^ ((wn >> 1) & 7)) * 16);
    *reinterpret_cast<uint4*>(smem + wb + buf * kTileBytes) = v;
  };

  const int KT = (int)(K / BK);
  const uint32_t magic = 0x64006400u;
  half8_t Bf[2][4];

  // One k-step (two MFMA k-substeps of 32): MFMAs on LDS buffer kt & 1 and
  // the B fragments of step kt; dequantization of the registers of step
  // kt + 1 (`nxt`) into the other buffer; weight loads of step kt + 2 into
  // `fre` and B fragment loads of step kt + 1.  Phantom steps at the end
  // stay inside the buffers (range-checked offsets), as in k_gemm.
  // Instruction order is pinned with scheduling fences.
  // metadata chunks (MCH): [slot][scales, biases]; chunk c = groups 8c ..
  // 8c + 7 of the thread's row, in slot c & 1
  uint4 mc[2][2];
  auto ld_chunk = [&](int c, uint4 (&dst)[2]) {
    dst[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r.s, r.so + 16u * (uint32_t)c, 0, 0));
    if constexpr (KIND != G_Q6K && KIND != G_SYM4)   // one array only
      dst[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             r.z, r.zo + 16u * (uint32_t)c, 0, 0));
  };
  // Q4K: chunks of 16 uint8 scale and zero codes (8 steps), and the
  // super-block step word once per 4 steps into a two-slot ring.  Q6K:
  // chunks of 16 int8 scale codes (4 steps; two per half row and step), the
  // fp16 step once per 4 steps.
  uint32_t ms[2];
  auto ld_step = [&](int b, uint32_t& dst) {
    if constexpr (KIND == G_Q6K)
      dst = __builtin_amdgcn_raw_buffer_load_b16(r.p, r.po + 2u * (uint32_t)b, 0, 0);
    else
      dst = __builtin_amdgcn_raw_buffer_load_b32(r.p, r.po + 4u * (uint32_t)b, 0, 0);
  };
  constexpr bool STEPW = KIND == G_Q4K || KIND == G_Q6K;   // step words in ms
  // raw metadata of step t (t % 16 == tu) into a stage: group t (group size
  // 64) or 2t + half (group size 32, Q4K) of the thread's row
  // steps per chunk (group-wise SYM4: 4 fp32 scales per chunk)
  constexpr int MP = KIND == G_SYM4 ? (MCH >= 16 ? MCH / 16 : 1)
                     : ((MCH == 32 && KIND != G_Q4K) || KIND == G_Q6K) ? 4 : 8;
  const uint32_t msh = (KIND == G_Q4K ? 8u : 16u) * (uint32_t)(tid & 1);
  // group size 128: one chunk per 16 steps, i.e. per unrolled iteration;
  // mc[0] holds the current chunk, mc[1] the next (NEXT: step 16 it + 16,
  // converted in the iteration's last step)
  auto set_meta = [&](auto TU, Stage<KIND>& st, bool next = false) {
    constexpr int tu = decltype(TU)::value;
    constexpr int slot = (tu / MP) & 1;
    if constexpr (MCH == 128 && KIND != G_SYM4) {
      constexpr int e = tu >> 1;   // group of step tu within the chunk
      const uint4& c0 = next ? mc[1][0] : mc[0][0];
      const uint4& c1 = next ? mc[1][1] : mc[0][1];
      st.s0 = (c0[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      st.s1 = (c1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    } else if constexpr (KIND == G_SYM4) {
      if constexpr (MCH == 32) st.s0 = mc[slot][0][2 * (tu & 1) + (int)(tid & 1)];
      else if constexpr (MCH == 64) st.s0 = mc[slot][0][tu & 3];
      else st.s0 = mc[slot][0][(tu & 7) >> 1];
    } else if constexpr (KIND == G_Q6K) {
      st.s0 = (mc[slot][0][tu & 3] >> msh) & 0xFFFFu;
      st.s2 = ms[(tu >> 2) & 1];
    } else if constexpr (KIND == G_Q4K) {
      constexpr int w = (tu & 7) >> 1, sh = 16 * (tu & 1);
      st.s0 = (mc[slot][0][w] >> (msh + sh)) & 0xFFu;
      st.s1 = (mc[slot][1][w] >> (msh + sh)) & 0xFFu;
      st.s2 = ms[(tu >> 2) & 1];
    } else if constexpr (MCH == 32) {
      constexpr int w = tu & 3;
      st.s0 = (mc[slot][0][w] >> msh) & 0xFFFFu;
      st.s1 = (mc[slot][1][w] >> msh) & 0xFFFFu;
    } else {
      constexpr int e = tu & 7;
      st.s0 = (mc[slot][0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      st.s1 = (mc[slot][1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    }
  };

  // The last ND A groups of a step's second substep run after the barrier,
  // at the top of the next step, where both waves of a SIMD would otherwise
  // wait for their first LDS fragments (register operands only: the
  // fragments are kept in Ad, the substep's B fragments stay in Bf[1] and
  // are reloaded after them).  int8 and chunked Q4K / Q6K keep ND = 0 (register
  // budget).
  constexpr int ND = (KIND == G_AFF8 || ((KIND == G_Q4K || KIND == G_Q6K) && MCH)) ? 0 : 3;
  half8_t Ad[ND > 0 ? ND : 1];
  auto mfma_deferred = [&]() {
    static_for<ND>([&](auto I) {
      constexpr int i = decltype(I)::value;
      static_for<4>([&](auto J) {
        constexpr int j = decltype(J)::value;
        acc[7 - ND + i][j] =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(Ad[i], Bf[1][j], acc[7 - ND + i][j], 0, 0, 0);
      });
    });
  };

  // U: position of step kt in the unrolled loop (kt % 16 == U for MCH)
  auto kstep = [&](auto U, int kt, Stage<KIND>& fre, Stage<KIND>& nxt) {
    constexpr int u = decltype(U)::value;
    const uint32_t cur = (uint32_t)(kt & 1);
    load_stage<KIND, GS32, false, !MCH>(a, r, kt + 2, fre);
    if constexpr (MCH) {
      // where chunk c' starts (step MP c') load chunk c' + 1 into the slot
      // that chunk c' - 1 held: its last step was converted already
      if constexpr (MCH == 128 && KIND != G_SYM4) {
        if constexpr (u == 0) ld_chunk(kt / 16 + 1, mc[1]);
        set_meta(std::integral_constant<int, (u + 1) & 15>{}, nxt, u == 15);
      } else {
        if constexpr (u % MP == 0)
          ld_chunk(kt / MP + 1, mc[((u / MP) + 1) & 1]);
        // step words: super-block b' + 1 at step 4b' (same argument)
        if constexpr (STEPW && u % 4 == 0) ld_step(kt / 4 + 1, ms[((u >> 2) + 1) & 1]);
        set_meta(std::integral_constant<int, (u + 1) & 15>{}, nxt);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    half8_t A[7];
#pragma unroll
    for (int i = 0; i < 7; ++i) A[i] = rd_a(cur, 0, i);
    if constexpr (ND > 0) {
      __builtin_amdgcn_sched_barrier(0);
      if (kt > 0) mfma_deferred();
#pragma unroll
      for (int j = 0; j < 4; ++j) Bf[1][j] = ld_b(kt, 1, j);
    }
    static_for<2>([&](auto SUB) {
      constexpr int sub = decltype(SUB)::value;
      half8_t An[7];
      if constexpr (sub == 0) {
#pragma unroll
        for (int i = 0; i < 7; ++i) An[i] = rd_a(cur, 1, i);
      }
      __builtin_amdgcn_sched_barrier(0);
      uint4 w0 = weight_chunk<KIND, MBF16>(nxt, 2 * sub, magic);
      uint4 w1 = weight_chunk<KIND, MBF16>(nxt, 2 * sub + 1, magic);
      static_for<(sub == 1 ? 7 - ND : 7)>([&](auto I) {
        constexpr int i = decltype(I)::value;
        static_for<4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], Bf[sub][j], acc[i][j], 0, 0, 0);
        });
      });
      if constexpr (sub == 1 && ND > 0) {
#pragma unroll
        for (int i = 0; i < ND; ++i) Ad[i] = A[7 - ND + i];
      }
      // the dequantized chunks are complete here, so their VALU work stays
      // among the MFMAs (LLVM would otherwise sink it next to the LDS store,
      // after the last MFMA)
      asm volatile("" : "+v"(w0.x), "+v"(w0.y), "+v"(w0.z), "+v"(w0.w), "+v"(w1.x), "+v"(w1.y),
                   "+v"(w1.z), "+v"(w1.w));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (sub == 0 || ND == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) Bf[sub][j] = ld_b(kt + 1, sub, j);
      }
      st_w(cur ^ 1u, 2 * sub, w0);
      st_w(cur ^ 1u, 2 * sub + 1, w1);
      if constexpr (sub == 0) {
#pragma unroll
        for (int i = 0; i < 7; ++i) A[i] = An[i];
      }
    });
    __syncthreads();
  };

  Stage<KIND> st0, st1;
  load_stage<KIND, GS32, false, !MCH>(a, r, 0, st0);
  load_stage<KIND, GS32, false, !MCH>(a, r, 1, st1);
  if constexpr (MCH) {
    if constexpr (MCH == 128 && KIND != G_SYM4) {
      ld_chunk(0, mc[0]);   // mc[1] is loaded by the first step
    } else {
      ld_chunk(0, mc[0]);
      ld_chunk(1, mc[1]);
    }
    if constexpr (STEPW) {
      ld_step(0, ms[0]);
      ld_step(1, ms[1]);
    }
    set_meta(std::integral_constant<int, 0>{}, st0);
  }
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int j = 0; j < 4; ++j) Bf[sub][j] = ld_b(0, sub, j);
#pragma unroll
  for (int p = 0; p < 4; ++p) st_w(0u, p, weight_chunk<KIND, MBF16>(st0, p, magic));
  if constexpr (XBF16) {
    if (tid < BM) s_xe[tid] = m0 + tid < a.M ? a.xe[m0 + tid] : 0;
  }
  __syncthreads();
  if constexpr (MCH) {
    for (int kt = 0; kt < KT; kt += 16) {
      static_for<16>([&](auto U) {
        constexpr int u = decltype(U)::value;
        if (u == 0 || kt + u < KT) {
          if constexpr (u % 2 == 0) kstep(U, kt + u, st0, st1);
          else kstep(U, kt + u, st1, st0);
        }
      });
      if constexpr (MCH == 128 && KIND != G_SYM4) {   // the next chunk becomes the current one
        mc[0][0] = mc[1][0];
        mc[0][1] = mc[1][1];
      }
    }
  } else {
    for (int kt = 0; kt < KT; kt += 2) {
      kstep(std::integral_constant<int, 0>{}, kt, st0, st1);
      if (kt + 1 < KT) kstep(std::integral_constant<int, 1>{}, kt + 1, st1, st0);
    }
  }
  if constexpr (ND > 0) mfma_deferred();   // the last step's deferred groups

  // ---- epilogue: lane holds rows n = 16 i + 4 (lane >> 4) + v (v = 0..3)
  // of column m = 16 j + (lane & 15) of the wave's tiles.
  const bool vec4 = (a.N % 4) == 0;
  const int ydt = a.ydt;
  const uint16_t* bias = static_cast<const uint16_t*>(a.bias);
  int el = lane;
  asm volatile("" : "+v"(el));   // keeps the epilogue's addresses after the loop
  static_for<7>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int64_t n = n0 + wi * 112 + i * 16 + 4 * (el >> 4);
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias != nullptr) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t nn = n + v < a.N ? n + v : a.N - 1;
        const uint32_t bb = bias[nn];
        bv[v] = XBF16 ? bf16_to_f32(bb) : f16_to_f32(bb);   // bias has the x dtype
      }
    }
    float sv[4] = {1.f, 1.f, 1.f, 1.f};   // G_SYM4C: channel scales
    if constexpr (KIND == G_SYM4C) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        sv[v] = static_cast<const float*>(a.scales)[n + v < a.N ? n + v : a.N - 1];
    }
    static_for<4>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const int64_t m = m0 + wj * 64 + j * 16 + (el & 15);
      const int64_t idx = m * a.N + n;
      const int xe = XBF16 ? s_xe[wj * 64 + j * 16 + (el & 15)] : 0;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = KIND == G_SYM4C ? fmaf(ldexpf(acc[i][j][q], -xe), sv[q], bv[q])
                               : ldexpf(acc[i][j][q], -xe) + bv[q];
      const bool mok = m < a.M;
      if (mok && vec4 && n < a.N) {
        if (ydt == F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.y) + idx) =
              make_float4(v[0], v[1], v[2], v[3]);
        } else {
          uint32_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            h[q] = ydt == BF16 ? f32_to_bf16_rne(v[q]) : f32_to_f16_rne(v[q]);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + idx) =
              make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
      } else if (mok && !vec4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (n + q < a.N) {
            if (ydt == F32) static_cast<float*>(a.y)[idx + q] = v[q];
            else static_cast<uint16_t*>(a.y)[idx + q] =
                (uint16_t)(ydt == BF16 ? f32_to_bf16_rne(v[q]) : f32_to_f16_rne(v[q]));
          }
        }
      }
    });
  });
}

}  // namespace
}  // namespace qp
