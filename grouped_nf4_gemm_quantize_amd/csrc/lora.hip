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
// order: per 64-row tile into a partial, then the partials of each expert in
// tile order, so results are deterministic.

#include "common.h"
#include "launch.h"
#include "mfma_common.h"

namespace nf4moe {

namespace {

constexpr int kLoraTile = 64;  // rows per tile (one expert's rows only)

}  // namespace

// bf16 -> fp16 rows (the output gradient, converted once so the dgrad's
// contraction loop reads fp16 operands); 8 elements per thread and step.
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ src,
                                                          int64_t n8, _Float16* __restrict__ dst) {
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n8;
       q += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + q * 8);
    *reinterpret_cast<u32x4*>(dst + q * 8) = bf16x8_to_f16x8(v);
  }
}

// bf16 adapter factors -> fp16 copies in their own layout (round to nearest
// even, as the GEMM's in-loop conversion of bf16 adapters): the layer
// forward converts once per call, so its k-loops read fp16 adapter rows.
// Up to four arrays in one launch; 8 elements per thread and step, read as
// one 16-byte vector where the source is 16-byte aligned.
__global__ __launch_bounds__(256) void half_copies_kernel(HalfCopies c) {
  int64_t total = 0;
  for (int i = 0; i < c.count; ++i) total += c.n8[i];
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    int seg = 0;
    int64_t local = q;
    while (seg + 1 < c.count && local >= c.n8[seg]) local -= c.n8[seg++];
    const uint16_t* src = c.src[seg] + local * 8;
    u32x4 v;
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
      v = *reinterpret_cast<const u32x4*>(src);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = (uint32_t)src[2 * t] | ((uint32_t)src[2 * t + 1] << 16);
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
    *reinterpret_cast<u32x4*>(c.dst[seg] + local * 8) = bf16x8_to_f16x8(v);
  }
}

// An adapter matrix as fp16 [E, r, C]: src is [E, r, C] (transpose = 0,
// the A factor) or [E, C, r] (transpose = 1, the B factor), bf16 or fp16.
__global__ __launch_bounds__(256) void lora_to_f16_kernel(const uint16_t* __restrict__ src,
                                                          int src_bf16, int transpose, int E,
                                                          int C, int r,
                                                          _Float16* __restrict__ dst) {
  const int64_t n = (int64_t)E * C * r;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q / ((int64_t)C * r);
    const int64_t rem = q - e * C * r;
    const int j = (int)(rem / C), c = (int)(rem - (int64_t)j * C);
    const uint16_t raw = transpose ? src[(e * C + c) * r + j] : src[q];
    dst[q] = src_bf16 ? (_Float16)bf16_bits_to_f32(raw) : __builtin_bit_cast(_Float16, raw);
  }
}

// One pass over the rows of a matrix m (rows of one expert per 64-row tile;
// src(i) = gather[i] / gather_div, else i), 64 columns at a time, on
// v_mfma_f32_16x16x32_f16:
//   kProj: out[i, j] = sum_c m[src(i), c] * w[e, j, c]      (w [E, r, C] fp16)
//   kGrad: part[tile, j, c] = sum_{i in tile} rs(i) q[i, j] m[src(i), c]
// Each 64x64 chunk of m is staged in LDS twice: row-major for the
// projection's A operand (8 columns of a row per lane) and column-major for
// the gradient's B operand (8 rows of a column per lane, the contraction of
// the sum over rows).  Wave w projects rows 16w..16w+15 and sums columns
// 16w..16w+15 of each chunk; ranks beyond r are zero.
constexpr int kPitch = 64 * 2 + 16;  // LDS row pitch of a staged chunk (bytes)
constexpr int kAhead = 4;            // chunks of m in flight per thread

template <bool kProj, bool kGrad, bool kMBf16>
__global__ __launch_bounds__(256) void lora_pass_kernel(LoraPassArgs a) {
  __shared__ int32_t tiles[kMaxExperts + 1];
  __shared__ int32_t wsum[4];
  __shared__ int32_t srcs[kLoraTile];
  __shared__ __attribute__((aligned(16))) char nat[kLoraTile * kPitch];  // [row][col]
  __shared__ __attribute__((aligned(16))) char tr[64 * kPitch];         // [col][row]
  __shared__ __attribute__((aligned(16))) _Float16 qt[16][kLoraTile + 8];  // [rank][row]
  __shared__ float qf[16][kLoraTile];  // the same in fp32, before scaling
  __shared__ float qexp[16][2];        // per rank: 2^-e applied, 2^e to undo
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  build_tile_table<256, kLoraTile>(a.offsets, a.E, tiles, wsum, tid);
  const int total = tiles[a.E];
  const int nchunk = a.C / 64;
  for (int tix = blockIdx.x; tix < total; tix += gridDim.x) {
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tiles[mid] <= tix) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int row0 = a.offsets[e] + (tix - tiles[e]) * kLoraTile;
    const int rows = min(kLoraTile, a.offsets[e + 1] - row0);
    __syncthreads();  // the previous tile is done with srcs / qt
    if (tid < kLoraTile) {
      const int i = row0 + (tid < rows ? tid : 0);
      srcs[tid] = a.gather ? a.gather[i] / a.gather_div : i;
    }
    if constexpr (kGrad) {
      // q^T of the tile with the row scale folded in.  Each rank's column is
      // scaled by a power of two that brings its largest magnitude into
      // [1/2, 1) before the fp16 conversion (undone on the fp32 result), so
      // small row scales (a tiny routing weight) stay out of fp16's
      // subnormal range
      for (int u = tid; u < 16 * kLoraTile; u += 256) {
        const int j = u / kLoraTile, rr = u % kLoraTile;
        float v = 0.f;
        if (j < a.r && rr < rows) {
          const int64_t i = row0 + rr;
          const float rs = a.rs ? a.rs[a.rs_idx ? a.rs_idx[i] : i] : 1.0f;
          v = a.q[i * a.r + j] * rs;
        }
        qf[j][rr] = v;
      }
      __syncthreads();
      if (tid < 16) {
        float m = 0.f;
        for (int rr = 0; rr < kLoraTile; ++rr) m = fmaxf(m, fabsf(qf[tid][rr]));
        int e = 0;
        if (m > 0.f) frexpf(m, &e);
        qexp[tid][0] = ldexpf(1.0f, -e);
        qexp[tid][1] = ldexpf(1.0f, e);
      }
      __syncthreads();
      for (int u = tid; u < 16 * kLoraTile; u += 256) {
        const int j = u / kLoraTile, rr = u % kLoraTile;
        qt[j][rr] = (_Float16)(qf[j][rr] * qexp[j][0]);
      }
    }
    __syncthreads();
    f32x4 accp = {0.f, 0.f, 0.f, 0.f};
    // this thread's two 16-byte pieces of a chunk: row tid % 64, columns
    // 8 g and 8 (g + 4) with g = tid / 64, so a wave's lanes are 64
    // consecutive rows of one 8-column group: its column-major writes are
    // 128 contiguous bytes each (no bank conflict).  kAhead chunks are in
    // flight (a register ring over the unrolled chunk loop): with one, each
    // chunk waited a full memory round trip.
    const int rr = tid & 63;
    u32x4 pre[kAhead][2];
    auto load_chunk = [&](int ch, u32x4 (&dst)[2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int lc = 8 * ((tid >> 6) + 4 * h);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (rr < rows) {
          v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.m) +
                                              (int64_t)srcs[rr] * a.C + ch * 64 + lc);
          if constexpr (kMBf16) v = bf16x8_to_f16x8(v);
        }
        dst[h] = v;
      }
    };
#pragma unroll
    for (int p = 0; p < kAhead; ++p)
      if (p < nchunk) load_chunk(p, pre[p]);
    // the projection's adapter fragments (w rows l16, from L2) one chunk
    // ahead, so no chunk waits on them
    u32x4 wnext[2];
    auto load_w = [&](int ch, u32x4 (&dst)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 bv = {0u, 0u, 0u, 0u};
        if (l16 < a.r)
          bv = *reinterpret_cast<const u32x4*>(a.w + ((int64_t)e * a.r + l16) * a.C + ch * 64 +
                                               32 * u + 8 * g4);
        dst[u] = bv;
      }
    };
    if constexpr (kProj) load_w(0, wnext);
    for (int ch0 = 0; ch0 < nchunk; ch0 += kAhead) {
#pragma unroll
      for (int p = 0; p < kAhead; ++p) {
        const int ch = ch0 + p;
        if (ch >= nchunk) break;
        __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int lc = 8 * ((tid >> 6) + 4 * h);
          if constexpr (kProj)
            *reinterpret_cast<u32x4*>(nat + rr * kPitch + lc * 2) = pre[p][h];
          if constexpr (kGrad) {
            const uint32_t w4[4] = {pre[p][h].x, pre[p][h].y, pre[p][h].z, pre[p][h].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              *reinterpret_cast<uint16_t*>(tr + (lc + 2 * t) * kPitch + rr * 2) =
                  (uint16_t)(w4[t] & 0xffffu);
              *reinterpret_cast<uint16_t*>(tr + (lc + 2 * t + 1) * kPitch + rr * 2) =
                  (uint16_t)(w4[t] >> 16);
            }
          }
        }
        __syncthreads();
        if (ch + kAhead < nchunk) load_chunk(ch + kAhead, pre[p]);
        if constexpr (kProj) {
          const u32x4 wcur[2] = {wnext[0], wnext[1]};
          if (ch + 1 < nchunk) load_w(ch + 1, wnext);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(nat + (16 * wave + l16) * kPitch +
                                                             (32 * u + 8 * g4) * 2);
            accp = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(av), as_f16x8(wcur[u]), accp,
                                                          0, 0, 0);
          }
        }
        if constexpr (kGrad) {
          f32x4 accg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const f16x8 qa = *reinterpret_cast<const f16x8*>(&qt[l16][32 * u + 8 * g4]);
            const u32x4 bv = *reinterpret_cast<const u32x4*>(tr + (16 * wave + l16) * kPitch +
                                                             (32 * u + 8 * g4) * 2);
            accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, as_f16x8(bv), accg, 0, 0, 0);
          }
          // lane holds ranks 4 g4 + t of column 16 wave + l16
          float* part = a.part + (int64_t)tix * a.r * a.C + ch * 64 + 16 * wave + l16;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int j = 4 * g4 + t;
            if (j < a.r) part[(int64_t)j * a.C] = accg[t] * qexp[j][1];
          }
        }
      }
    }
    if constexpr (kProj) {
      // lane holds rows 16 wave + 4 g4 + t, rank l16
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int rr = 16 * wave + 4 * g4 + t;
        if (rr < rows && l16 < a.r) a.out[(int64_t)(row0 + rr) * a.r + l16] = accp[t];
      }
    }
  }
}

// z[e] = scale * sum over expert e's tiles (in tile order) of part; stored
// [E, r, C] (kRankMajor) or [E, C, r].  Experts without rows get zeros.
__global__ __launch_bounds__(256) void lora_wgrad_reduce_kernel(LoraPassArgs a) {
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
    if (a.rank_major) a.z[q] = s;
    else a.z[((int64_t)e * a.C + c) * a.r + j] = s;
  }
}

hipError_t launch_bf16_to_f16(const void* src, int64_t n, _Float16* dst, int num_cus,
                              hipStream_t s) {
  const int64_t n8 = n / 8;
  int64_t grid = (n8 + 255) / 256;
  if (grid > (int64_t)num_cus * 16) grid = (int64_t)num_cus * 16;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(src), n8, dst);
  return hipGetLastError();
}

hipError_t launch_half_copies(const HalfCopies& c, int num_cus, hipStream_t s) {
  int64_t total = 0;
  for (int i = 0; i < c.count; ++i) total += c.n8[i];
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > (int64_t)num_cus * 8) grid = (int64_t)num_cus * 8;
  hipLaunchKernelGGL(half_copies_kernel, dim3((unsigned)grid), dim3(256), 0, s, c);
  return hipGetLastError();
}

hipError_t launch_lora_to_f16(const void* src, int src_bf16, int transpose, int E, int C,
                              int r, _Float16* dst, int num_cus, hipStream_t s) {
  const int64_t n = (int64_t)E * C * r;
  int64_t grid = (n + 255) / 256;
  if (grid > (int64_t)num_cus * 16) grid = (int64_t)num_cus * 16;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(lora_to_f16_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(src), src_bf16, transpose, E, C, r, dst);
  return hipGetLastError();
}

template <bool kProj, bool kGrad>
static void pass_m(const LoraPassArgs& a, dim3 g, hipStream_t s) {
  if (a.m_bf16) hipLaunchKernelGGL((lora_pass_kernel<kProj, kGrad, true>), g, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((lora_pass_kernel<kProj, kGrad, false>), g, dim3(256), 0, s, a);
}

hipError_t launch_lora_pass(const LoraPassArgs& a, int num_cus, hipStream_t s) {
  if (a.P == 0) return hipSuccess;
  int64_t grid = (a.P + kLoraTile - 1) / kLoraTile + a.E;
  if (grid > (int64_t)num_cus * 8) grid = (int64_t)num_cus * 8;
  const dim3 g((unsigned)grid);
  const bool proj = a.out != nullptr, grad = a.part != nullptr;
  if (proj && grad) pass_m<true, true>(a, g, s);
  else if (proj) pass_m<true, false>(a, g, s);
  else pass_m<false, true>(a, g, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !grad) return err;
  const int64_t n = (int64_t)a.E * a.r * a.C;
  int64_t rg = (n + 255) / 256;
  if (rg > (int64_t)num_cus * 16) rg = (int64_t)num_cus * 16;
  if (rg < 1) rg = 1;
  hipLaunchKernelGGL(lora_wgrad_reduce_kernel, dim3((unsigned)rg), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace nf4moe
