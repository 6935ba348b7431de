// Router top-k, token/expert pair permutation, and the per-token combine.
//
// The routed layer sorts token/expert pairs by expert and runs the groups
// (experts4bit-qlora 0.22.0 README, "Which training path?"), then sums each
// token's expert outputs back in group-sorted order.  Everything here runs on
// the device with no host synchronisation (the zero-host-sync contract of the
// README's "CUDA-graph decode capture" section).
//
// Pair id p = t*k + j.  Because a token's k experts are distinct, the rank of
// pair (t, j) inside its expert's group is the number of EARLIER TOKENS that
// picked the same expert.  Tokens are processed in chunks of 32: each chunk
// keeps, per expert, a 32-bit mask of the chunk tokens that picked it.  The
// rank is then  chunk_base[chunk][e] + popcount(mask & bits below t), a
// stable counting sort with no sequential pass over the pairs.
//
// Kernels (in launch order):
//   route_chunk_kernel  top-k + softmax weights per token (one wave per
//                       token), per-chunk expert masks; optionally converts
//                       the activation rows to fp16 for the GEMMs (spread
//                       over every workgroup of the launch, which has at
//                       least two per CU);
//   route_scan_kernel   per-expert totals -> offsets and per-chunk bases;
//   route_scatter_kernel  sorted_pair / pair_pos from the masks.
// When the masks are few (chunks x E <= kFuseMasks), one kernel replaces
// the last two: route_scan_scatter_kernel, in which every chunk's workgroup
// recomputes the expert totals and its own bases from all the masks (a few
// KB of L2 reads each) instead of waiting for a separate scan launch.

#include "common.h"
#include "launch.h"
#include "route_device.h"

namespace nf4moe {

// One workgroup of 8 waves per chunk of 32 tokens; wave w routes tokens
// w, w+8, w+16, w+24 of the chunk with all four logit rows loaded up front.
constexpr int kRouteWaves = 8;
constexpr int kTokPerWave = kRouteChunk / kRouteWaves;

template <int kRegs>
__global__ __launch_bounds__(512) void route_chunk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int renormalize,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    uint32_t* __restrict__ chunk_masks, const void* __restrict__ x_in,
    int x_bf16, _Float16* __restrict__ x16, int H) {
  __shared__ uint32_t mask[kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t chunk = blockIdx.x;
  const int64_t t0 = chunk * kRouteChunk;
  if (t0 < T) {  // workgroups past the last chunk only convert activations
  for (int e = tid; e < E; e += blockDim.x) mask[e] = 0u;

  float v[kTokPerWave][kRegs];
#pragma unroll
  for (int u = 0; u < kTokPerWave; ++u) {
    int64_t t = t0 + wave + kRouteWaves * u;
    if (t >= T) t = T - 1;  // clamp: routed again, never written
    route_load<kRegs>(logits + t * E, E, lane, v[u]);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kTokPerWave; ++u) {
    const int i = wave + kRouteWaves * u;
    const int64_t t = t0 + i;
    if (t >= T) break;
    int id;
    float w;
    route_select<kRegs>(v[u], E, k, renormalize, lane, &id, &w);
    if (lane < k) {
      topk_ids[t * k + lane] = id;
      topk_w[t * k + lane] = w;
      atomicOr(&mask[id], 1u << i);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) chunk_masks[chunk * E + e] = mask[e];
  }

  // Activation rows to fp16, 8 elements per 16-byte access, four accesses in
  // flight per thread, grid-strided over the whole [T, H] block -- by the
  // workgroups past the last chunk alone when there are at least as many of
  // them as chunks (the routing workgroups then finish with the routing).
  if (x16 != nullptr && x_bf16) {
    const int64_t nchunks = (T + kRouteChunk - 1) / kRouteChunk;
    const int64_t extra = (int64_t)gridDim.x - nchunks;
    const bool split = extra >= nchunks;
    if (split && chunk < nchunks) return;
    const int64_t wg = split ? chunk - nchunks : chunk;
    const int64_t nwg = split ? extra : (int64_t)gridDim.x;
    const int64_t n8 = T * H / 8;
    const int64_t stride = nwg * blockDim.x;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(x_in);
    _Float16* dst = x16;
    for (int64_t i0 = wg * blockDim.x + tid; i0 < n8; i0 += 4 * stride) {
      u32x4 v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * stride;
        if (i < n8) v4[u] = *reinterpret_cast<const u32x4*>(src + i * 8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * stride;
        if (i < n8) {
          const u32x4 a = v4[u];
          u32x4 o;
          o.x = pack_half2((_Float16)bf16_bits_to_f32(a.x & 0xffffu), (_Float16)bf16_bits_to_f32(a.x >> 16));
          o.y = pack_half2((_Float16)bf16_bits_to_f32(a.y & 0xffffu), (_Float16)bf16_bits_to_f32(a.y >> 16));
          o.z = pack_half2((_Float16)bf16_bits_to_f32(a.z & 0xffffu), (_Float16)bf16_bits_to_f32(a.z >> 16));
          o.w = pack_half2((_Float16)bf16_bits_to_f32(a.w & 0xffffu), (_Float16)bf16_bits_to_f32(a.w >> 16));
          *reinterpret_cast<u32x4*>(dst + i * 8) = o;
        }
      }
    }
  }
}

// Single workgroup of 1024 threads.  Thread t owns expert e = t % Ep (Ep =
// E rounded up to a power of two) and a contiguous group of chunks
// t / Ep; group partial counts meet in LDS for the expert totals, the
// exclusive scan over experts gives the offsets, and each thread then writes
// the running bases of its own chunks.
constexpr int kScanCache = 16;

__global__ __launch_bounds__(1024) void route_scan_kernel(
    const uint32_t* __restrict__ chunk_masks, int64_t nchunks, int E,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ chunk_base) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_cnt[kMaxExperts];
  const int t = threadIdx.x;
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int groups = 1024 / Ep;
  const int e = t % Ep;
  const int grp = t / Ep;
  const int64_t cpg = (nchunks + groups - 1) / groups;
  const int64_t c0 = (int64_t)grp * cpg;
  int64_t c1 = c0 + cpg;
  if (c1 > nchunks) c1 = nchunks;
  int32_t cached[kScanCache];
  int32_t part = 0;
  if (e < E) {
    if (cpg <= kScanCache) {
#pragma unroll
      for (int u = 0; u < kScanCache; ++u) {
        const int64_t c = c0 + u;
        cached[u] = (c < c1) ? __popc(chunk_masks[c * E + e]) : 0;
      }
#pragma unroll
      for (int u = 0; u < kScanCache; ++u) part += cached[u];
    } else {
      for (int64_t c = c0; c < c1; ++c) part += __popc(chunk_masks[c * E + e]);
    }
  }
  s_part[t] = part;
  __syncthreads();
  int32_t total = 0;
  if (t < E)
    for (int gi = 0; gi < groups; ++gi) total += s_part[gi * Ep + t];
  s_cnt[t] = (t < E) ? total : 0;
  __syncthreads();
  for (int off = 1; off < Ep; off <<= 1) {
    const int32_t a = (t >= off) ? s_cnt[t - off] : 0;
    __syncthreads();
    s_cnt[t] += a;
    __syncthreads();
  }
  if (t < E) {
    expert_offsets[t] = s_cnt[t] - total;
    if (t == E - 1) expert_offsets[E] = s_cnt[t];
  }
  if (e < E && chunk_base != nullptr) {
    int32_t run = (e == 0) ? 0 : s_cnt[e - 1];  // exclusive offset of expert e
    for (int gi = 0; gi < grp; ++gi) run += s_part[gi * Ep + e];
    if (cpg <= kScanCache) {
#pragma unroll
      for (int u = 0; u < kScanCache; ++u) {
        const int64_t c = c0 + u;
        if (c < c1) {
          chunk_base[c * E + e] = run;
          run += cached[u];
        }
      }
    } else {
      for (int64_t c = c0; c < c1; ++c) {
        chunk_base[c * E + e] = run;
        run += __popc(chunk_masks[c * E + e]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ topk_ids, const uint32_t* __restrict__ chunk_masks,
    const int32_t* __restrict__ chunk_base, int64_t T, int E, int k,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  const int64_t chunk = blockIdx.x;
  const int64_t t0 = chunk * kRouteChunk;
  int64_t t1 = t0 + kRouteChunk;
  if (t1 > T) t1 = T;
  for (int64_t p = t0 * k + threadIdx.x; p < t1 * k; p += blockDim.x) {
    const int64_t t = p / k;
    const int e = topk_ids[p];
    const uint32_t m = chunk_masks[chunk * E + e];
    const uint32_t below = (1u << (uint32_t)(t - t0)) - 1u;
    const int32_t rank = chunk_base[chunk * E + e] + __popc(m & below);
    sorted_pair[rank] = (int32_t)p;
    if (pair_pos != nullptr) pair_pos[p] = rank;
  }
}

// Fused scan + scatter (E <= kFuseThreads and chunks x E <= kFuseMasks).
// Workgroup c: thread t counts expert e = t % Ep over the chunks of its
// group t / Ep -- all of them for the expert's total, those before c for
// this chunk's base; the groups meet in LDS; an exclusive scan over the
// experts gives the offsets (workgroup 0 writes them); then the pairs of
// chunk c are placed as in route_scatter_kernel.
constexpr int kFuseThreads = 512;
constexpr int64_t kFuseMasks = 16384;
constexpr int kFuseBatch = 16;  // mask loads in flight per thread

__global__ __launch_bounds__(kFuseThreads) void route_scan_scatter_kernel(
    const int32_t* __restrict__ topk_ids, const uint32_t* __restrict__ chunk_masks,
    int64_t T, int E, int k, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  __shared__ int32_t s_tot[kFuseThreads];
  __shared__ int32_t s_pre[kFuseThreads];
  __shared__ int32_t s_base[kFuseThreads];
  __shared__ uint32_t s_mask[kFuseThreads];  // this chunk's mask per expert
  __shared__ int32_t s_wsum[kFuseThreads / 64];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t chunk = blockIdx.x;
  const int64_t nchunks = (T + kRouteChunk - 1) / kRouteChunk;
  const int64_t t0 = chunk * kRouteChunk;
  int64_t t1 = t0 + kRouteChunk;
  if (t1 > T) t1 = T;
  // this chunk's pair ids go out first (the scatter needs them after the
  // scan; at most kRouteChunk * k pairs, two per thread)
  constexpr int kPairsPerThread = kRouteChunk * kMaxTopK / kFuseThreads;
  static_assert(kPairsPerThread * kFuseThreads == kRouteChunk * kMaxTopK, "pair prefetch");
  int32_t ids_pre[kPairsPerThread];
#pragma unroll
  for (int u = 0; u < kPairsPerThread; ++u) {
    const int64_t p = t0 * k + t + (int64_t)u * kFuseThreads;
    ids_pre[u] = p < t1 * k ? topk_ids[p] : 0;
  }
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int groups = kFuseThreads / Ep;
  const int e = t % Ep, grp = t / Ep;
  const int64_t cpg = (nchunks + groups - 1) / groups;
  const int64_t c0 = (int64_t)grp * cpg;
  const int64_t c1 = c0 + cpg < nchunks ? c0 + cpg : nchunks;
  int32_t tot = 0, pre = 0;
  for (int64_t cb = c0; cb < c1; cb += kFuseBatch) {
    uint32_t mv[kFuseBatch];
#pragma unroll
    for (int u = 0; u < kFuseBatch; ++u) {
      const int64_t c = cb + u;
      mv[u] = (e < E && c < c1) ? chunk_masks[c * E + e] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kFuseBatch; ++u) {
      const int32_t n = __popc(mv[u]);
      tot += n;
      pre += (cb + u < chunk) ? n : 0;
      // the group holding this chunk: one thread per expert
      if (cb + u == chunk && cb + u < c1 && e < E) s_mask[e] = mv[u];
    }
  }
  s_tot[t] = tot;
  s_pre[t] = pre;
  __syncthreads();
  // expert t's total and prefix: the sum over the groups
  tot = 0;
  pre = 0;
  if (t < E) {
    for (int gi = 0; gi < groups; ++gi) {
      tot += s_tot[gi * Ep + t];
      pre += s_pre[gi * Ep + t];
    }
  }
  // exclusive scan of the totals over the experts
  int32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int32_t excl = incl - tot;
  for (int w = 0; w < wave; ++w) excl += s_wsum[w];
  if (t < E) {
    s_base[t] = excl + pre;
    if (chunk == 0) {
      expert_offsets[t] = excl;
      if (t == E - 1) expert_offsets[E] = excl + tot;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPairsPerThread; ++u) {
    const int64_t p = t0 * k + t + (int64_t)u * kFuseThreads;
    if (p < t1 * k) {
      const int64_t tk = p / k;
      const int ex = ids_pre[u];
      const uint32_t m = s_mask[ex];
      const uint32_t below = (1u << (uint32_t)(tk - t0)) - 1u;
      const int32_t rank = s_base[ex] + __popc(m & below);
      sorted_pair[rank] = (int32_t)p;
      if (pair_pos != nullptr) pair_pos[p] = rank;
    }
  }
}

// y[t] = sum_j w[t, j] * o[t*k + j]  (fp32, ascending j), per-slot rows o in
// pair order.  8 columns per thread and step.
template <int kOut>
__global__ __launch_bounds__(256) void combine_kernel(
    const _Float16* __restrict__ o, const float* __restrict__ w, int64_t T,
    int k, int H, void* __restrict__ y) {
  const int64_t n8 = (int64_t)T * H / 8;
  const int h8 = H / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / h8;
    const int64_t c = (i - t * h8) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const float wj = w ? w[t * k + j] : 1.0f;  // no weights: a plain sum
      const u32x4 v = *reinterpret_cast<const u32x4*>(o + (t * k + j) * H + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x2 hv = u32_as_half2(u[q]);
        acc[2 * q] = fmaf(wj, (float)hv.x, acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj, (float)hv.y, acc[2 * q + 1]);
      }
    }
    if constexpr (kOut == kF32) {
      float* dst = reinterpret_cast<float*>(y) + t * H + c;
      *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else if constexpr (kOut == kBF16) {
      u32x4 r;
      r.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
      r.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
      r.z = (uint32_t)f32_to_bf16_bits(acc[4]) | ((uint32_t)f32_to_bf16_bits(acc[5]) << 16);
      r.w = (uint32_t)f32_to_bf16_bits(acc[6]) | ((uint32_t)f32_to_bf16_bits(acc[7]) << 16);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + t * H + c) = r;
    } else {
      u32x4 r;
      r.x = pack_half2((_Float16)acc[0], (_Float16)acc[1]);
      r.y = pack_half2((_Float16)acc[2], (_Float16)acc[3]);
      r.z = pack_half2((_Float16)acc[4], (_Float16)acc[5]);
      r.w = pack_half2((_Float16)acc[6], (_Float16)acc[7]);
      *reinterpret_cast<u32x4*>(reinterpret_cast<_Float16*>(y) + t * H + c) = r;
    }
  }
}

// ------------------------------------------------------------ launchers

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int64_t nchunks = (a.T + kRouteChunk - 1) / kRouteChunk;
  const int regs = (a.E + 63) / 64;
  // with an activation conversion, at least two workgroups per CU share it
  int64_t g0 = nchunks;
  if (a.x16 != nullptr && a.x_bf16 && g0 < 2 * (int64_t)a.num_cus) g0 = 2 * (int64_t)a.num_cus;
  const dim3 grid((unsigned)g0), block(64 * kRouteWaves);
  const dim3 cgrid((unsigned)nchunks);
#define NF4MOE_ROUTE_CASE(R)                                                  \
  case R:                                                                     \
    hipLaunchKernelGGL(route_chunk_kernel<R>, grid, block, 0, stream,         \
                       a.logits, a.T, a.E, a.k, a.renormalize, a.topk_ids,    \
                       a.topk_w, a.chunk_masks, a.x_in, a.x_bf16, a.x16, a.H); \
    break;
  switch (regs) {
    NF4MOE_ROUTE_CASE(1)
    NF4MOE_ROUTE_CASE(2)
    NF4MOE_ROUTE_CASE(4)
    NF4MOE_ROUTE_CASE(8)
    NF4MOE_ROUTE_CASE(16)
    case 3:
      hipLaunchKernelGGL(route_chunk_kernel<4>, grid, block, 0, stream, a.logits,
                         a.T, a.E, a.k, a.renormalize, a.topk_ids, a.topk_w,
                         a.chunk_masks, a.x_in, a.x_bf16, a.x16, a.H);
      break;
    case 5: case 6: case 7:
      hipLaunchKernelGGL(route_chunk_kernel<8>, grid, block, 0, stream, a.logits,
                         a.T, a.E, a.k, a.renormalize, a.topk_ids, a.topk_w,
                         a.chunk_masks, a.x_in, a.x_bf16, a.x16, a.H);
      break;
    default:
      hipLaunchKernelGGL(route_chunk_kernel<16>, grid, block, 0, stream, a.logits,
                         a.T, a.E, a.k, a.renormalize, a.topk_ids, a.topk_w,
                         a.chunk_masks, a.x_in, a.x_bf16, a.x16, a.H);
      break;
  }
#undef NF4MOE_ROUTE_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.E <= kFuseThreads && nchunks * a.E <= kFuseMasks) {
    hipLaunchKernelGGL(route_scan_scatter_kernel, cgrid, dim3(kFuseThreads), 0, stream,
                       a.topk_ids, a.chunk_masks, a.T, a.E, a.k, a.expert_offsets,
                       a.sorted_pair, a.pair_pos);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream,
                     a.chunk_masks, nchunks, a.E, a.expert_offsets, a.chunk_base);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, cgrid, dim3(256), 0, stream, a.topk_ids,
                     a.chunk_masks, a.chunk_base, a.T, a.E, a.k, a.sorted_pair,
                     a.pair_pos);
  return hipGetLastError();
}

hipError_t launch_combine(const _Float16* o, const float* w, int64_t T, int k,
                          int H, void* y, int y_dtype, int num_cus,
                          hipStream_t stream) {
  const int64_t n8 = T * H / 8;
  int64_t grid = (n8 + 255) / 256;
  const int64_t cap = (int64_t)num_cus * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  if (y_dtype == kF32)
    hipLaunchKernelGGL(combine_kernel<kF32>, dim3((unsigned)grid), dim3(256), 0,
                       stream, o, w, T, k, H, y);
  else if (y_dtype == kBF16)
    hipLaunchKernelGGL(combine_kernel<kBF16>, dim3((unsigned)grid), dim3(256), 0,
                       stream, o, w, T, k, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<kF16>, dim3((unsigned)grid), dim3(256), 0,
                       stream, o, w, T, k, H, y);
  return hipGetLastError();
}

}  // namespace nf4moe
