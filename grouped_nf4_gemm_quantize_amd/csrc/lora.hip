// Kernels of the QLoRA backward around the grouped dgrad: the SwiGLU of the
// recomputed pre-activation, the rank-r row projections onto an adapter, and
// the adapters' weight gradients.
//
// The adapters train while the packed stack stays frozen (solutions index,
// "How do I QLoRA-train the fused experts"): with delta = s * B (A x) on a
// projection whose input rows are x_i and whose output gradient rows are d_i
// (rows of expert e, s = alpha / r),
//   u_i = A_e x_i,  v_i = B_e^T d_i                     (rank-r projections)
//   dB_e = s * sum_i d_i u_i^T,  dA_e = s * sum_i v_i x_i^T
// and the input gradient gains s * A_e^T v_i (added inside the dgrad
// kernel's epilogue).  The sums over an expert's rows are taken in a fixed
// order: per 128-row tile (the tile table of the GEMMs) into a partial, then
// the partials of each expert in tile order, so results are deterministic.

#include "common.h"
#include "launch.h"
#include "mfma_common.h"

namespace nf4moe {

namespace {

constexpr int kLoraTile = 128;  // rows per partial (the GEMM M-tile)

template <bool kBf16>
__device__ __forceinline__ void ld8(const void* base, int64_t idx, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + idx);
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

// Expert of row i: the e with offsets[e] <= i < offsets[e + 1] (rows at or
// beyond offsets[E] return -1).
__device__ __forceinline__ int expert_of(const int32_t* __restrict__ offsets, int E, int64_t i) {
  if (i >= offsets[E]) return -1;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace

// h = silu(g[:, :I]) * g[:, I:], fp16 rows of the recomputed pre-activation.
__global__ __launch_bounds__(256) void swiglu_rows_kernel(const _Float16* __restrict__ g,
                                                          int64_t P, int I,
                                                          _Float16* __restrict__ h) {
  const int i8 = I / 8;
  const int64_t n = P * i8;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = q / i8;
    const int c = (int)(q - row * i8) * 8;
    float gate[8], up[8];
    ld8<false>(g, row * 2 * I + c, gate);
    ld8<false>(g, row * 2 * I + I + c, up);
    u32x4 o;
    uint32_t* po = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float a = gate[2 * t] * __builtin_amdgcn_rcpf(1.0f + __expf(-gate[2 * t])) * up[2 * t];
      const float b = gate[2 * t + 1] * __builtin_amdgcn_rcpf(1.0f + __expf(-gate[2 * t + 1])) *
                      up[2 * t + 1];
      po[t] = pack_half2((_Float16)a, (_Float16)b);
    }
    *reinterpret_cast<u32x4*>(h + row * I + c) = o;
  }
}

// bt[e, j, c] = b[e, c, j] (fp16), the adapter B stored rank-major.
__global__ __launch_bounds__(256) void lora_transpose_kernel(const uint16_t* __restrict__ b,
                                                             int b_bf16, int E, int C, int r,
                                                             _Float16* __restrict__ bt) {
  const int64_t n = (int64_t)E * C * r;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q / ((int64_t)C * r);
    const int64_t rem = q - e * C * r;
    const int j = (int)(rem / C), c = (int)(rem - (int64_t)j * C);
    const uint16_t raw = b[(e * C + c) * r + j];
    bt[q] = b_bf16 ? (_Float16)bf16_bits_to_f32(raw) : __builtin_bit_cast(_Float16, raw);
  }
}

// out[i, j] = sum_c m[src(i), c] * w[e(i), j, c] for the P rows that belong
// to an expert (src(i) = gather[i] / gather_div, else i; w [E, r, C]).  One
// wave per row; lane l covers columns 8 l + 512 t.
template <bool kMBf16, bool kWBf16>
__global__ __launch_bounds__(256) void lora_rowproj_kernel(LoraProjArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= a.P) return;
  const int e = expert_of(a.offsets, a.E, i);
  if (e < 0) return;
  const int64_t src = a.gather ? (int64_t)(a.gather[i] / a.gather_div) : i;
  float acc[kMaxLoraR];
#pragma unroll
  for (int j = 0; j < kMaxLoraR; ++j) acc[j] = 0.f;
  for (int c = lane * 8; c < a.C; c += 512) {
    float m[8];
    ld8<kMBf16>(a.m, src * a.C + c, m);
#pragma unroll
    for (int j = 0; j < kMaxLoraR; ++j) {
      if (j < a.r) {
        float w[8];
        ld8<kWBf16>(a.w, ((int64_t)e * a.r + j) * a.C + c, w);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[j] = fmaf(m[t], w[t], acc[j]);
      }
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxLoraR; ++j) {
    if (j < a.r) {
      const float s = wave_sum(acc[j]);
      if (lane == j) mine = s;
    }
  }
  if (lane < a.r) a.out[i * a.r + lane] = mine;
}

// Partial weight gradient of one 128-row tile and 512 columns:
//   part[tile, j, c] = sum_{rows i of the tile} rs(i) q[i, j] m[src(i), c]
// with rs(i) = rs[rs_idx ? rs_idx[i] : i] (1 when rs is null).  Four waves of
// 32 rows each; lane l holds columns 8 l .. 8 l + 7 for all r ranks; the
// waves' sums meet in LDS, four ranks at a time.
template <int kR, bool kMBf16>
__global__ __launch_bounds__(256) void lora_wgrad_partial_kernel(LoraGradArgs a, int n_chunks) {
  __shared__ int32_t tiles[kMaxExperts + 1];
  __shared__ int32_t wsum[4];
  __shared__ __attribute__((aligned(16))) float red[4][4][64 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  build_tile_table<256, kLoraTile>(a.offsets, a.E, tiles, wsum, tid);
  const int total = tiles[a.E];
  for (int u = blockIdx.x; u < total * n_chunks; u += gridDim.x) {
    const int tix = u / n_chunks, cc = u - tix * n_chunks;
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tiles[mid] <= tix) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int row0 = a.offsets[e] + (tix - tiles[e]) * kLoraTile;
    const int rows = min(kLoraTile, a.offsets[e + 1] - row0);
    const int c = cc * 512 + lane * 8;
    const bool live = c < a.C;
    float acc[kR][8];
#pragma unroll
    for (int j = 0; j < kR; ++j)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[j][t] = 0.f;
    const int rb = wave * 32, re = min(rows, rb + 32);
    for (int rr = rb; rr < re; ++rr) {
      const int64_t i = row0 + rr;
      const float rs = a.rs ? a.rs[a.rs_idx ? a.rs_idx[i] : i] : 1.0f;
      const int64_t src = a.gather ? (int64_t)(a.gather[i] / a.gather_div) : i;
      float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (live) ld8<kMBf16>(a.m, src * a.C + c, m);
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        const float qj = j < a.r ? a.q[i * a.r + j] * rs : 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[j][t] = fmaf(qj, m[t], acc[j][t]);
      }
    }
    float* part = a.part + (int64_t)tix * a.r * a.C;
#pragma unroll
    for (int j0 = 0; j0 < kR; j0 += 4) {
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int t = 0; t < 8; ++t) red[wave][jj][lane * 8 + t] = acc[j0 + jj][t];
      __syncthreads();
      const int j = j0 + wave;  // wave w sums rank j0 + w over the four waves
      if (j < a.r && live) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float s = (red[0][wave][lane * 8 + t] + red[1][wave][lane * 8 + t]) +
                          (red[2][wave][lane * 8 + t] + red[3][wave][lane * 8 + t]);
          part[(int64_t)j * a.C + c + t] = s;
        }
      }
    }
  }
}

// z[e] = scale * sum over expert e's tiles (in tile order) of part; stored
// [E, r, C] (kRankMajor) or [E, C, r].  Experts without rows get zeros.
__global__ __launch_bounds__(256) void lora_wgrad_reduce_kernel(LoraGradArgs a, int rank_major) {
  __shared__ int32_t tiles[kMaxExperts + 1];
  __shared__ int32_t wsum[4];
  build_tile_table<256, kLoraTile>(a.offsets, a.E, tiles, wsum, threadIdx.x);
  const int64_t n = (int64_t)a.E * a.r * a.C;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(q / ((int64_t)a.r * a.C));
    const int64_t rem = q - (int64_t)e * a.r * a.C;
    const int j = (int)(rem / a.C), c = (int)(rem - (int64_t)j * a.C);
    float s = 0.f;
    for (int t = tiles[e]; t < tiles[e + 1]; ++t) s += a.part[((int64_t)t * a.r + j) * a.C + c];
    s *= a.scale;
    if (rank_major) a.z[q] = s;
    else a.z[((int64_t)e * a.C + c) * a.r + j] = s;
  }
}

hipError_t launch_swiglu_rows(const _Float16* g, int64_t P, int I, _Float16* h, int num_cus,
                              hipStream_t s) {
  const int64_t n = P * (I / 8);
  int64_t grid = (n + 255) / 256;
  if (grid > (int64_t)num_cus * 16) grid = (int64_t)num_cus * 16;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(swiglu_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, g, P, I, h);
  return hipGetLastError();
}

hipError_t launch_lora_transpose(const void* b, int b_bf16, int E, int C, int r, _Float16* bt,
                                 int num_cus, hipStream_t s) {
  const int64_t n = (int64_t)E * C * r;
  int64_t grid = (n + 255) / 256;
  if (grid > (int64_t)num_cus * 16) grid = (int64_t)num_cus * 16;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(lora_transpose_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(b), b_bf16, E, C, r, bt);
  return hipGetLastError();
}

hipError_t launch_lora_rowproj(const LoraProjArgs& a, hipStream_t s) {
  if (a.P == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.P + 3) / 4));
  if (a.m_bf16) {
    if (a.w_bf16) hipLaunchKernelGGL((lora_rowproj_kernel<true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((lora_rowproj_kernel<true, false>), grid, dim3(256), 0, s, a);
  } else {
    if (a.w_bf16) hipLaunchKernelGGL((lora_rowproj_kernel<false, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((lora_rowproj_kernel<false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_lora_wgrad(const LoraGradArgs& a, int rank_major, int num_cus, hipStream_t s) {
  const int n_chunks = (a.C + 511) / 512;
  const int64_t max_units = ((a.P + kLoraTile - 1) / kLoraTile + a.E) * n_chunks;
  int64_t grid = max_units;
  if (grid > (int64_t)num_cus * 4) grid = (int64_t)num_cus * 4;
  if (grid < 1) grid = 1;
  const dim3 g((unsigned)grid);
  if (a.r <= 8) {
    if (a.m_bf16) hipLaunchKernelGGL((lora_wgrad_partial_kernel<8, true>), g, dim3(256), 0, s, a, n_chunks);
    else hipLaunchKernelGGL((lora_wgrad_partial_kernel<8, false>), g, dim3(256), 0, s, a, n_chunks);
  } else {
    if (a.m_bf16) hipLaunchKernelGGL((lora_wgrad_partial_kernel<16, true>), g, dim3(256), 0, s, a, n_chunks);
    else hipLaunchKernelGGL((lora_wgrad_partial_kernel<16, false>), g, dim3(256), 0, s, a, n_chunks);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n = (int64_t)a.E * a.r * a.C;
  int64_t rg = (n + 255) / 256;
  if (rg > (int64_t)num_cus * 16) rg = (int64_t)num_cus * 16;
  if (rg < 1) rg = 1;
  hipLaunchKernelGGL(lora_wgrad_reduce_kernel, dim3((unsigned)rg), dim3(256), 0, s, a, rank_major);
  return hipGetLastError();
}

}  // namespace nf4moe
