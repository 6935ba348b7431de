// Blockwise quantiser for fused expert stacks: NF4, and the fp4, int8 and
// fp8 storage modes.
//
// Experts4bit.from_float quantises the fused gate_up / down stacks to NF4
// with one absmax per 64 elements (experts4bit-qlora 0.22.0 README,
// "Quickstart" and "Which door?"); the blocks never cross an expert boundary
// (load_in_4bit solutions page, "Which project solves it").  A block here is
// 64 consecutive elements of one row of one expert, so it can cross neither.
//
// Layout: 16 lanes own one block, 4 consecutive elements each, so a wave64
// covers 4 blocks = 256 consecutive elements and every load is a coalesced
// 16-byte (fp32) or 8-byte (bf16) access.  HBM bound: 4 (or 2) bytes read and
// 0.5625 bytes written per element.

#include "common.h"
#include "launch.h"

namespace nf4moe {

// fp32 y with |y| <= 448 -> its nearest fp8 e4m3 code, ties to the even
// mantissa: below 2^-6 the subnormal steps of 2^-9 (a rint of y * 512, whose
// result 8 is the smallest normal), else the fp32 mantissa rounded to 3 bits
// (a carry moves into the exponent).  Zero of either sign gives code 0.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float ay = fabsf(y);
  uint32_t c;
  if (ay < 0.015625f) {
    c = (uint32_t)__builtin_rintf(ay * 512.0f);
  } else {
    const uint32_t u = __float_as_uint(ay);
    const uint32_t e = (u >> 23) - 120u;  // fp32 bias 127 -> e4m3 bias 7
    const uint32_t m = u & 0x7fffffu;
    c = (e << 3) + ((m + 0x7ffffu + ((m >> 20) & 1u)) >> 20);
  }
  return c == 0u ? 0u : (sign | c);
}

// kQ: 0 nf4, 1 fp4 (4-bit codes, two per byte), 2 int8, 3 fp8 e4m3 (one
// byte per element).
template <bool kBF16, int kQ>
__global__ __launch_bounds__(256) void quantize_kernel(
    const void* __restrict__ w, int64_t nblocks, uint8_t* __restrict__ packed,
    float* __restrict__ absmax, int32_t* __restrict__ nonfinite_flag,
    QuantThresholds thr) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15;   // position of this lane inside its block
  const int blk_in_wave = lane >> 4;
  const int64_t wave_global = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);

  float t[15];
#pragma unroll
  for (int j = 0; j < 15; ++j) t[j] = thr.t[j];

  // the fp16 multiplier the grouped GEMMs make of a block's absmax: absmax,
  // absmax / 127 (int8) or absmax / 448 (fp8)
  constexpr float kScaleDiv = kQ == 2 ? 127.0f : kQ == 3 ? 448.0f : 1.0f;
  bool bad = false;
  bool out_of_range = false;
  for (int64_t b0 = wave_global * 4; b0 < nblocks; b0 += nwaves * 4) {
    const int64_t blk = b0 + blk_in_wave;
    const bool live = blk < nblocks;
    const int64_t e0 = blk * kBlock + sub * 4;  // first element of this lane
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      if constexpr (kBF16) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(
            reinterpret_cast<const uint16_t*>(w) + e0);
        x[0] = bf16_bits_to_f32(v.x & 0xffffu);
        x[1] = bf16_bits_to_f32(v.x >> 16);
        x[2] = bf16_bits_to_f32(v.y & 0xffffu);
        x[3] = bf16_bits_to_f32(v.y >> 16);
      } else {
        const f32x4 v = *reinterpret_cast<const f32x4*>(
            reinterpret_cast<const float*>(w) + e0);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
      }
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bad |= !__builtin_isfinite(x[i]);
      a = fmaxf(a, fabsf(x[i]));
    }
    // max over the 16 lanes of the block (one DPP row: lanes differ only in
    // bits 0..3); max is exact, so the order of the butterfly is immaterial
    a = row16_max(a);
    {
      // outside fp16's normal range the multiplier overflows (|s| >= 65520
      // rounds to inf) or keeps fewer than 11 significant bits (s < 2^-14)
      const float sc = a / kScaleDiv;
      // (a non-finite block is reported by the first bit alone)
      out_of_range |= live && a != 0.f && __builtin_isfinite(a) &&
                      !(sc >= 0x1p-14f && sc < 65520.0f);
    }

    uint32_t codes[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t c = kQ == 0 ? 7u : 0u;  // all-zero block: the zero level / code 0
      if (a != 0.f) {
        const float xn = x[i] / a;  // IEEE fp32 division (no fast-math)
        c = 0u;
        if constexpr (kQ == 2) {
          c = (uint32_t)(int)__builtin_rintf(xn * 127.0f) & 0xffu;
        } else if constexpr (kQ == 3) {
          c = e4m3_code(xn * 448.0f);
        } else if constexpr (kQ == 1) {
          const float ax = fabsf(xn);
#pragma unroll
          for (int j = 0; j < 7; ++j) c += (ax > t[j]) ? 1u : 0u;
          c |= (xn < 0.f) ? 8u : 0u;
        } else {
#pragma unroll
          for (int j = 0; j < 15; ++j) c += (xn > t[j]) ? 1u : 0u;
        }
      }
      codes[i] = c;
    }
    if (live) {
      if constexpr (kQ >= 2) {
        *reinterpret_cast<uint32_t*>(packed + e0) =
            codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
      } else {
        const uint32_t b01 = (codes[0] << 4) | codes[1];
        const uint32_t b23 = (codes[2] << 4) | codes[3];
        *reinterpret_cast<uint16_t*>(packed + e0 / 2) = (uint16_t)(b01 | (b23 << 8));
      }
      if (sub == 0) absmax[blk] = a;
    }
  }
  if (nonfinite_flag != nullptr && (bad || out_of_range))
    atomicOr(nonfinite_flag, (bad ? 1 : 0) | (out_of_range ? 2 : 0));
}

// Flags of the fp16 conversion of n values (bf16 or fp32), OR-ed into *flags:
// 1 = a value fp16 cannot hold (|v| >= 65520 rounds to inf; NaN and inf
// included), 2 = a nonzero value fp16 flushes to zero (|v| <= 2^-25 rounds
// to 0), 4 = a nonzero value below fp16's normal range (|v| < 2^-14: fewer than
// 11 significant bits).  One atomic per wave that saw anything.
template <bool kBF16>
__global__ __launch_bounds__(256) void f16_range_kernel(const void* __restrict__ t, int64_t n,
                                                        int32_t* __restrict__ flags) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  uint32_t f = 0;
  for (int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i0 < n; i0 += stride) {
    float v[4];
    if (i0 + 4 <= n) {
      if constexpr (kBF16) {
        const u32x2 r = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(t) + i0);
        v[0] = bf16_bits_to_f32(r.x & 0xffffu);
        v[1] = bf16_bits_to_f32(r.x >> 16);
        v[2] = bf16_bits_to_f32(r.y & 0xffffu);
        v[3] = bf16_bits_to_f32(r.y >> 16);
      } else {
        const f32x4 r = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(t) + i0);
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = 0.f;
        if (i0 + j < n)
          v[j] = kBF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(t)[i0 + j])
                       : reinterpret_cast<const float*>(t)[i0 + j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = fabsf(v[j]);
      f |= !(a < 65520.0f) ? 1u : 0u;  // NaN compares false
      f |= (a != 0.f && a <= 0x1p-25f) ? 2u : 0u;
      f |= (a != 0.f && a < 0x1p-14f) ? 4u : 0u;
    }
  }
  // one OR per wave (the lanes' bits combined through ballots)
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 3; ++b) w |= __ballot((f >> b) & 1u) != 0ull ? (1u << b) : 0u;
  if ((threadIdx.x & 63) == 0 && w != 0u) atomicOr(flags, (int)w);
}

hipError_t launch_f16_range(const void* t, bool bf16, int64_t n, int32_t* flags, int num_cus,
                            hipStream_t stream) {
  int64_t grid = (n + 1023) / 1024;
  const int64_t cap = (int64_t)num_cus * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  if (bf16)
    hipLaunchKernelGGL(f16_range_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, t, n,
                       flags);
  else
    hipLaunchKernelGGL(f16_range_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, t, n,
                       flags);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* w, int w_dtype, int64_t nelem,
                           uint8_t* packed, float* absmax, int32_t* flag,
                           const QuantThresholds& thr, int num_cus,
                           hipStream_t stream) {
  const int64_t nblocks = nelem / kBlock;
  const int64_t waves_needed = (nblocks + 3) / 4;
  int64_t grid = (waves_needed + 3) / 4;
  const int64_t cap = (int64_t)num_cus * 16;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  const dim3 g((unsigned)grid);
  const bool bf = w_dtype == kBF16;
#define NF4MOE_QLAUNCH(B, Q) \
  hipLaunchKernelGGL((quantize_kernel<B, Q>), g, dim3(256), 0, stream, w, nblocks, packed, \
                     absmax, flag, thr)
  switch (thr.qtype) {
    case kQtFP4: if (bf) NF4MOE_QLAUNCH(true, 1); else NF4MOE_QLAUNCH(false, 1); break;
    case kQtINT8: if (bf) NF4MOE_QLAUNCH(true, 2); else NF4MOE_QLAUNCH(false, 2); break;
    case kQtFP8: if (bf) NF4MOE_QLAUNCH(true, 3); else NF4MOE_QLAUNCH(false, 3); break;
    default: if (bf) NF4MOE_QLAUNCH(true, 0); else NF4MOE_QLAUNCH(false, 0); break;
  }
#undef NF4MOE_QLAUNCH
  return hipGetLastError();
}

}  // namespace nf4moe
