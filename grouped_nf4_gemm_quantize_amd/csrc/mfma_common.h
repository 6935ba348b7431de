// Device helpers shared by the MFMA kernels (grouped GEMM, grouped dgrad):
// buffer resources, direct-to-LDS copies, counted waits, output staging.
#pragma once

#include "common.h"

namespace nf4moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

namespace {

// ---- buffer resources and the direct-to-LDS copies -------------------------

// Raw buffer resource over [base, base + bytes): stride 0, offset-addressed.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)p);
}

// Lane i copies 16 (resp. 4) bytes from rsrc + voff + soff to LDS address
// lds + 16 i (resp. 4 i).  M0 carries the LDS base; one wait state separates
// its write from the load.  The kernel uses M0 for nothing else.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are pending
// and its LDS operations are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- small helpers ---------------------------------------------------------

template <int kOut>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (kOut == kF32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if constexpr (kOut == kBF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
  }
}

// Four consecutive output values -> one 8-byte (16-byte for fp32) LDS write.
template <int kOut>
__device__ __forceinline__ void stage_out4(char* p, const float (&v)[4]) {
  if constexpr (kOut == kF32) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  } else if constexpr (kOut == kBF16) {
    *reinterpret_cast<u32x2*>(p) =
        u32x2{(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
              (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
  } else {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_half2((_Float16)v[0], (_Float16)v[1]),
                                         pack_half2((_Float16)v[2], (_Float16)v[3])};
  }
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 o;
  o.x = pack_half2((_Float16)bf16_bits_to_f32(v.x & 0xffffu), (_Float16)bf16_bits_to_f32(v.x >> 16));
  o.y = pack_half2((_Float16)bf16_bits_to_f32(v.y & 0xffffu), (_Float16)bf16_bits_to_f32(v.y >> 16));
  o.z = pack_half2((_Float16)bf16_bits_to_f32(v.z & 0xffffu), (_Float16)bf16_bits_to_f32(v.z >> 16));
  o.w = pack_half2((_Float16)bf16_bits_to_f32(v.w & 0xffffu), (_Float16)bf16_bits_to_f32(v.w >> 16));
  return o;
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

template <bool kBf16>
__device__ __forceinline__ void unpack8(const u32x4 w, float (&v)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kBf16) {
      v[2 * i] = bf16_bits_to_f32(ws[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(ws[i] >> 16);
    } else {
      const f16x2 h = u32_as_half2(ws[i]);
      v[2 * i] = (float)h.x;
      v[2 * i + 1] = (float)h.y;
    }
  }
}

template <int kOut>
__device__ __forceinline__ void store8(void* out, int64_t idx, const float (&v)[8]) {
  if constexpr (kOut == kF32) {
    float* p = reinterpret_cast<float*>(out) + idx;
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    u32x4 w;
    uint32_t* pw = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kOut == kBF16)
        pw[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) |
                ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
      else
        pw[i] = pack_half2((_Float16)v[2 * i], (_Float16)v[2 * i + 1]);
    }
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + idx) = w;
  }
}


// Per-expert M-tile table from the expert offsets: tiles[e] = number of
// BM-row tiles of experts 0..e-1, tiles[E] = the total.  Thread t owns
// experts kPer*t .. kPer*t + kPer - 1; a block-wide scan over the waves.
// Ends with a barrier.
template <int kThreads, int kBM>
__device__ __forceinline__ void build_tile_table(const int32_t* __restrict__ offsets, int E,
                                                 int32_t* tiles, int32_t* wsum, int tid) {
  constexpr int kPer = kMaxExperts / kThreads;
  const int lane = tid & 63, wave = tid >> 6;
  int32_t cnt[kPer];
  int32_t local = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int ex = tid * kPer + u;
    cnt[u] = 0;
    if (ex < E) cnt[u] = (offsets[ex + 1] - offsets[ex] + kBM - 1) / kBM;
    local += cnt[u];
  }
  int32_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int32_t run = incl - local;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int ex = tid * kPer + u;
    if (ex < E) tiles[ex] = run;
    run += cnt[u];
  }
  if (tid == kThreads - 1) tiles[E] = run;
  __syncthreads();
}

}  // namespace

}  // namespace nf4moe
