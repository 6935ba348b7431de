// Internal definitions shared by the HIP kernels and the host ABI layer.
//
// Not part of the public interface (see include/nf4moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// The 16 NF4 levels, ascending, as fp32.  They are the 4-bit NormalFloat
// construction (normal quantiles at a 9-point grid from delta to 1/2 for the
// 8 positive levels and an 8-point grid for the 7 negative ones, an exact
// zero, normalised to [-1, 1], delta = ((1 - 1/32) + (1 - 1/30)) / 2), built
// in double precision and rounded once to fp32.  The pages fix only that
// training and serving use the same codebook (experts4bit-qlora 0.22.0
// README, "Inference").
#define NF4MOE_LEVELS_INIT                                                   \
  {-1.0f,          -0.6961928010f, -0.5250729322f, -0.3949174285f,           \
   -0.2844413221f, -0.1847734004f, -0.0910499766f, 0.0f,                     \
   0.0795803145f,  0.1609301418f,  0.2461122572f,  0.3379151225f,            \
   0.4407097399f,  0.5626168847f,  0.7229566574f,  1.0f}

// fp4 storage mode: the e2m1 element values {0, 0.5, 1, 1.5, 2, 3, 4, 6}
// over 6 (the block's absmax maps to the largest), indexed by code = sign
// bit << 3 | magnitude index; code 8 is -0.  Each value is the correctly
// rounded fp32 quotient.
#define NF4MOE_FP4_LEVELS_INIT                                                \
  {0.0f,         0.5f / 6.0f,  1.0f / 6.0f,  1.5f / 6.0f,                     \
   2.0f / 6.0f,  3.0f / 6.0f,  4.0f / 6.0f,  1.0f,                            \
   -0.0f,        -0.5f / 6.0f, -1.0f / 6.0f, -1.5f / 6.0f,                    \
   -2.0f / 6.0f, -3.0f / 6.0f, -4.0f / 6.0f, -1.0f}

// MXFP4 elements: the e2m1 values by code (sign bit 3), not normalised; the
// block's e8m0 byte carries the scale.
#define NF4MOE_E2M1_VALUES_INIT                                               \
  {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,                            \
   -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f}

namespace nf4moe {
constexpr int kQtNF4 = 0;
constexpr int kQtFP4 = 1;
constexpr int kQtMXFP4 = 2;  // e2m1 + e8m0 per 32, low nibble first (own entry points)
constexpr int kQtINT8 = 3;   // 8-bit codes: int8, value = code / 127 * absmax
constexpr int kQtFP8 = 4;    // 8-bit codes: fp8 e4m3, value = e4m3(code) / 448 * absmax
constexpr int kQtBF16 = 5;   // passthrough: the weights themselves as bf16, no absmax
constexpr int kQtF16 = 6;    // passthrough: the weights themselves as fp16, no absmax
}  // namespace nf4moe

namespace nf4moe {

constexpr int kBlock = 64;       // elements per absmax block
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;
constexpr int kMaxLoraR = 16;
constexpr int kRouteChunk = 32;  // tokens per routing chunk (one u32 mask bit each)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum DType { kF32 = 0, kBF16 = 1, kF16 = 2 };

// ---- small conversions (exact or round-to-nearest-even) ------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_half2(_Float16 lo, _Float16 hi) {
  f16x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f16x2 u32_as_half2(uint32_t u) {
  return __builtin_bit_cast(f16x2, u);
}

__device__ __forceinline__ uint32_t half2_as_u32(f16x2 v) {
  return __builtin_bit_cast(uint32_t, v);
}

// ---- the decode lookup table ---------------------------------------------
// One byte of packed codes holds two 4-bit codes (even element in the high
// nibble).  The LDS table maps the byte b to the packed fp16 pair
// (level[b >> 4], level[b & 15]) -- the first k element in the low half --
// so one lookup yields an MFMA/dot2-ready half2.  kLutCopies copies of the
// 256-entry table are interleaved word by word so that lane l always reads
// bank (l % kLutCopies): address(b, l) = b * (4 * kLutCopies) + 4 * (l %
// kLutCopies).  That keeps the random-index lookups free of bank conflicts.
template <int kLutCopies>
struct Lut {
  static constexpr int kBytes = 256 * 4 * kLutCopies;
  static constexpr int kShift = kLutCopies == 64 ? 8 : 7;  // log2(4*copies)
  static_assert(kLutCopies == 32 || kLutCopies == 64, "copies");
};

// Fill the LDS table from the fp32 levels (each half rounded to nearest-even
// fp16).  `stage` is a 16-entry LDS scratch array.  The fill ends with a
// barrier, so the table is ready to use on return.
// With low_first the byte holds the first element in its LOW nibble (the
// MXFP4 packing): the pair is (level[b & 15], level[b >> 4]).
template <int kLutCopies>
__device__ __forceinline__ void lut_fill(uint32_t* lut, uint16_t* stage,
                                         const float* levels, int tid,
                                         int nthreads, bool low_first = false) {
  if (tid < 16) stage[tid] = __builtin_bit_cast(uint16_t, (_Float16)levels[tid]);
  __syncthreads();
  for (int i = tid; i < 256 * kLutCopies; i += nthreads) {
    const int b = i / kLutCopies;
    const int first = low_first ? (b & 15) : (b >> 4);
    const int second = low_first ? (b >> 4) : (b & 15);
    lut[i] = (uint32_t)stage[first] | ((uint32_t)stage[second] << 16);
  }
  __syncthreads();
}

// e8m0 scale byte -> fp16 2^(s - 127): normal for s in [113, 142],
// subnormal down to s = 103, zero below, inf above, NaN for 255.
__device__ __forceinline__ _Float16 e8m0_to_half(uint32_t s) {
  uint32_t bits;
  if (s == 255u) bits = 0x7e00u;
  else if (s >= 143u) bits = 0x7c00u;
  else if (s >= 113u) bits = (s - 112u) << 10;
  else if (s >= 103u) bits = 1u << (s - 103u);
  else bits = 0u;
  return __builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Per-lane constant of the lookup address: 4 * (lane % copies).
template <int kLutCopies>
__device__ __forceinline__ uint32_t lut_lane_offset(int lane) {
  return (uint32_t)(lane % kLutCopies) * 4u;
}

// Byte j of q, placed at bits [kShift, kShift+8) of the table address, ORed
// with the lane's word offset, in one v_perm_b32.  For 64 copies the byte
// lands in address byte 1; for 32 copies the address needs a shift by 7, so
// a plain shift/mask is used instead.
template <int kLutCopies, int j>
__device__ __forceinline__ uint32_t lut_addr(uint32_t q, uint32_t lane_off) {
  if constexpr (kLutCopies == 64) {
    // D byte0 = lane_off.byte0 (sel 0: S1 byte 0), byte1 = q.byte j (sel 4+j),
    // bytes 2,3 = 0 (sel 12).
    constexpr uint32_t sel = 0x0c0c0000u | ((4u + j) << 8);
    return __builtin_amdgcn_perm(q, lane_off, sel);
  } else {
    return (((q >> (8 * j)) & 0xffu) << 7) | lane_off;
  }
}

__device__ __forceinline__ uint32_t lds_read_u32(const uint32_t* lut_base,
                                                 uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(
      reinterpret_cast<const char*>(lut_base) + byte_addr);
}

// Decode 8 codes (one little-endian u32 of packed bytes: k elements e0..e7)
// into 4 half2 words in k order, unscaled.
template <int kLutCopies>
__device__ __forceinline__ void decode8(const uint32_t* lut, uint32_t lane_off,
                                        uint32_t q, uint32_t out[4]) {
  out[0] = lds_read_u32(lut, lut_addr<kLutCopies, 0>(q, lane_off));
  out[1] = lds_read_u32(lut, lut_addr<kLutCopies, 1>(q, lane_off));
  out[2] = lds_read_u32(lut, lut_addr<kLutCopies, 2>(q, lane_off));
  out[3] = lds_read_u32(lut, lut_addr<kLutCopies, 3>(q, lane_off));
}

// ---- cross-lane reductions (wave64) ---------------------------------------
// Within a row of 16 lanes the butterfly runs on DPP lane moves (VALU
// latency): quad_perm [1,0,3,2] and [2,3,0,1] combine lanes i^1 and i^2,
// row_half_mirror (i <-> 7-i) and row_mirror (i <-> 15-i) then combine the
// already-uniform quads and half rows.  The four row results are combined
// through v_readlane into scalars, so every lane ends with the same value
// and no step goes through LDS (a ds_bpermute costs an LDS round trip).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, kCtrl, 0xf, 0xf, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<kCtrl>(__float_as_int(v)));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

// Wave-wide sum / max, returned (uniform) to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

}  // namespace nf4moe
