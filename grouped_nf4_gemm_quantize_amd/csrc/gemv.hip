// Single-token (T = 1) decode path: split-K GEMVs over the routed experts.
//
// At batch 1 the expert projection is a matrix-vector product per routed
// expert that streams the packed bytes once (experts4bit-qlora 0.22.0 README,
// "Inference": the single-token decode fast path uses a fused 4-bit GEMV).  HBM
// bandwidth on the NF4 codes + absmax is the roofline, and with only ~21 MB
// per layer the time is set by the chain of dependent memory round trips, so
// each kernel issues its weight loads as early as their addresses are known
// and overlaps everything else (activation staging, the decode table) with
// them.
//
//   gemv_gate_up_kernel  every wave routes the token itself (a top-k over the
//     E logits costs a few hundred cycles -- cheaper than a barrier), then
//     owns up to kMaxItems (slot j, column i) items: the gate row i and the
//     up row I+i of expert ids[j], dotted with x; it writes
//     h[j, i] = w_j * silu(gate) * up  (fp16).
//   gemv_down_kernel  one wave per output row n: the K of the row is the
//     concatenation of the k routed experts' I inputs, so the combine over
//     the slots is part of the dot product; y[n] is written directly.
//
// Split-K inside a wave: lane l takes the 32-weight chunks l, l+64, ... of a
// row (16 packed bytes = one 16-byte load; a chunk is half of one 64-block so
// it needs one absmax -- or, for MXFP4 stacks, exactly one 32-block with its
// e8m0 scale, applied in fp32), decodes them through the LDS byte->half2 table
// (common.h) and multiplies with v_dot2_f32_f16 against fp16 activations held
// in LDS; the 64 partial sums are reduced across the wave.

#include "common.h"
#include "launch.h"
#include "route_device.h"

namespace nf4moe {

__constant__ float c_levels_gemv[16] = NF4MOE_LEVELS_INIT;
__constant__ float c_levels_gemv_fp4[16] = NF4MOE_FP4_LEVELS_INIT;
__constant__ float c_levels_gemv_mx[16] = NF4MOE_E2M1_VALUES_INIT;

namespace {
constexpr int kCopies = 32;
constexpr int kThreads = 512;          // 8 waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxItems = 4;           // gate/up items per wave and round
constexpr int kMaxChunksPerLane = 16;  // down: chunks of the concatenated K

__device__ __forceinline__ float dot_chunk(const uint32_t* lut, uint32_t lane_off,
                                           u32x4 q, const _Float16* act) {
  // act: 32 fp16 activations of this chunk (16-byte aligned, in LDS)
  const u32x4* a4 = reinterpret_cast<const u32x4*>(act);
  const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
  float p = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4 av = a4[w];
    const uint32_t aa[4] = {av.x, av.y, av.z, av.w};
    uint32_t d[4];
    decode8<kCopies>(lut, lane_off, qq[w], d);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      p = __builtin_amdgcn_fdot2(u32_as_half2(d[t]), u32_as_half2(aa[t]), p, false);
  }
  return p;
}

__device__ __forceinline__ float silu_g(float z) {
  return z / (1.0f + expf(-z));
}

template <int kOut>
__device__ __forceinline__ void store1(void* out, int64_t idx, float v) {
  if constexpr (kOut == kF32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if constexpr (kOut == kBF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
  }
}

// The scale of chunk c (32 weights) of a row: the fp32 absmax of its 64-block,
// or for MXFP4 stacks the e8m0 byte of its own 32-block as 2^(s - 127) in
// fp32 (exact over the whole e8m0 range; 255 is NaN).
__device__ __forceinline__ float chunk_scale(const float* absmax, int64_t row, int chunks,
                                             int c, bool mx) {
  if (mx) {
    const uint32_t b = reinterpret_cast<const uint8_t*>(absmax)[row * chunks + c];
    return b == 255u ? __builtin_nanf("") : ldexpf(1.0f, (int)b - 127);
  }
  return absmax[row * (chunks / 2) + (c >> 1)];
}

__device__ __forceinline__ void fill_table(uint32_t* lut, uint16_t* stage, int qtype, int tid) {
  if (qtype == kQtMXFP4)
    lut_fill<kCopies>(lut, stage, c_levels_gemv_mx, tid, kThreads, /*low_first=*/true);
  else
    lut_fill<kCopies>(lut, stage, qtype == kQtFP4 ? c_levels_gemv_fp4 : c_levels_gemv, tid,
                      kThreads);
}

// 16-bit activation -> fp16 (bf16 rounds to nearest even; fp16 passes through)
__device__ __forceinline__ _Float16 to_f16(uint16_t raw, bool bf16) {
  return bf16 ? (_Float16)bf16_bits_to_f32(raw) : __builtin_bit_cast(_Float16, raw);
}

}  // namespace

// kCpl = ceil(H / 2048) <= 4: 32-weight chunks of one row per lane.
template <int kRegs, int kCpl>
__global__ __launch_bounds__(kThreads) void gemv_gate_up_kernel(GemvArgs g) {
  __shared__ uint32_t s_lut[256 * kCopies];
  __shared__ uint16_t s_stage[16];
  extern __shared__ __attribute__((aligned(16))) _Float16 s_x[];  // [H]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = g.H, I = g.I, k = g.k;

  // activations: issued first, consumed after the weight loads are out
  constexpr int kXPer = 4;  // x elements per thread and pass
  uint2 xr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i0 = (p * kThreads + tid) * kXPer;
    xr[p] = i0 < H ? *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) + i0)
                   : make_uint2(0u, 0u);
  }

  // route in every wave: lane j < k holds slot j
  int id;
  float w;
  route_one_token<kRegs>(g.logits, g.E, k, g.renormalize, lane, &id, &w);
  if (blockIdx.x == 0 && wave == 0 && lane < k) {
    g.topk_ids[lane] = id;
    g.topk_w[lane] = w;
  }

  // this wave's items, every load issued before any arithmetic
  const int chunks = H / 32;
  const int64_t row_bytes = H / 2;
  const bool mx = g.qtype == kQtMXFP4;
  const int nw = gridDim.x * kWaves;
  const int items = k * I;
  const int q0 = blockIdx.x * kWaves + wave;
  u32x4 qg[kMaxItems][kCpl], qu[kMaxItems][kCpl];
  float sg[kMaxItems][kCpl], su[kMaxItems][kCpl];
#pragma unroll
  for (int it = 0; it < kMaxItems; ++it) {
    const int q = q0 + it * nw;
    const int qq = q < items ? q : (q0 < items ? q0 : 0);  // clamp: re-read a valid item
    const int j = qq / I;
    const int i = qq - j * I;
    const int e = __builtin_amdgcn_readlane(id, j);  // j is wave-uniform
    const int64_t rg = (int64_t)e * 2 * I + i;
    const int64_t ru = rg + I;
#pragma unroll
    for (int m = 0; m < kCpl; ++m) {
      int c = lane + 64 * m;
      if (c >= chunks) c = chunks - 1;
      qg[it][m] = *reinterpret_cast<const u32x4*>(g.gu_packed + rg * row_bytes + c * 16);
      qu[it][m] = *reinterpret_cast<const u32x4*>(g.gu_packed + ru * row_bytes + c * 16);
      sg[it][m] = chunk_scale(g.gu_absmax, rg, chunks, c, mx);
      su[it][m] = chunk_scale(g.gu_absmax, ru, chunks, c, mx);
    }
  }

  // stage x as fp16 and build the table while the weights are in flight
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i0 = (p * kThreads + tid) * kXPer;
    if (i0 < H) {
      s_x[i0 + 0] = to_f16(xr[p].x & 0xffffu, g.x_bf16);
      s_x[i0 + 1] = to_f16(xr[p].x >> 16, g.x_bf16);
      s_x[i0 + 2] = to_f16(xr[p].y & 0xffffu, g.x_bf16);
      s_x[i0 + 3] = to_f16(xr[p].y >> 16, g.x_bf16);
    }
  }
  fill_table(s_lut, s_stage, g.qtype, tid);  // ends with a barrier

  const uint32_t lane_off = lut_lane_offset<kCopies>(lane);
  _Float16* hout = reinterpret_cast<_Float16*>(g.hbuf);
#pragma unroll
  for (int it = 0; it < kMaxItems; ++it) {
    const int q = q0 + it * nw;
    float accg = 0.f, accu = 0.f;
#pragma unroll
    for (int m = 0; m < kCpl; ++m) {
      const int c = lane + 64 * m;
      if (c < chunks) {
        const _Float16* xs = s_x + c * 32;
        accg = fmaf(dot_chunk(s_lut, lane_off, qg[it][m], xs), sg[it][m], accg);
        accu = fmaf(dot_chunk(s_lut, lane_off, qu[it][m], xs), su[it][m], accu);
      }
    }
    accg = wave_sum(accg);
    accu = wave_sum(accu);
    const int j = q < items ? q / I : 0;
    const float wj = lane_f(w, j);
    if (lane == 0 && q < items) hout[q] = (_Float16)(silu_g(accg) * accu * wj);
  }
}

template <int kOut>
__global__ __launch_bounds__(kThreads) void gemv_down_kernel(GemvArgs g) {
  __shared__ uint32_t s_lut[256 * kCopies];
  __shared__ uint16_t s_stage[16];
  extern __shared__ __attribute__((aligned(16))) _Float16 s_h[];  // [k, I]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = g.H, I = g.I, k = g.k;

  // the routed experts (lane j < k holds slot j's id)
  const int id = lane < k ? g.topk_ids[lane] : 0;

  // this lane's chunks of the concatenated K (the same for every output row)
  const int cps = I / 32;  // chunks per slot
  const int total = k * cps;
  const bool mx = g.qtype == kQtMXFP4;
  int64_t pk_off[kMaxChunksPerLane];
  int64_t am_off[kMaxChunksPerLane];  // absmax element, or scale byte for MXFP4
  int h_off[kMaxChunksPerLane];
  int nc = 0;
#pragma unroll
  for (int m = 0; m < kMaxChunksPerLane; ++m) {
    const int cc = lane + 64 * m;
    const int j = cc < total ? cc / cps : 0;
    const int e = __shfl(id, j, 64);
    pk_off[m] = 0;
    am_off[m] = 0;
    h_off[m] = 0;
    if (cc < total) {
      const int c = cc - j * cps;
      pk_off[m] = (int64_t)e * H * (I / 2) + c * 16;
      am_off[m] = mx ? (int64_t)e * H * (I / 32) + c : (int64_t)e * H * (I / 64) + (c >> 1);
      h_off[m] = j * I + c * 32;
      nc = m + 1;
    }
  }
  // one output row per wave and round; the first row's loads go out before
  // h is staged and the table is built
  const int nw = gridDim.x * kWaves;
  int n = blockIdx.x * kWaves + wave;
  u32x4 q[kMaxChunksPerLane];
  float s[kMaxChunksPerLane];
  auto load_row = [&](int row) {
    const int64_t prow = (int64_t)row * (I / 2);
    const int64_t arow = (int64_t)row * (mx ? I / 32 : I / 64);
#pragma unroll
    for (int m = 0; m < kMaxChunksPerLane; ++m) {
      if (m < nc) {
        q[m] = *reinterpret_cast<const u32x4*>(g.dn_packed + pk_off[m] + prow);
        if (mx) {
          const uint32_t b = reinterpret_cast<const uint8_t*>(g.dn_absmax)[am_off[m] + arow];
          s[m] = b == 255u ? __builtin_nanf("") : ldexpf(1.0f, (int)b - 127);
        } else {
          s[m] = g.dn_absmax[am_off[m] + arow];
        }
      }
    }
  };
  if (n < H) load_row(n);

  // h (fp16, k*I values, a multiple of 8) -> LDS
  const _Float16* hin = reinterpret_cast<const _Float16*>(g.hbuf);
  for (int i = tid * 8; i < k * I; i += kThreads * 8)
    *reinterpret_cast<u32x4*>(s_h + i) = *reinterpret_cast<const u32x4*>(hin + i);
  fill_table(s_lut, s_stage, g.qtype, tid);  // ends with a barrier

  const uint32_t lane_off = lut_lane_offset<kCopies>(lane);
  for (; n < H; n += nw) {
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxChunksPerLane; ++m) {
      if (m < nc) acc = fmaf(dot_chunk(s_lut, lane_off, q[m], s_h + h_off[m]), s[m], acc);
    }
    if (n + nw < H) load_row(n + nw);
    acc = wave_sum(acc);
    if (lane == 0) store1<kOut>(g.y, n, acc);
  }
}

template <int kRegs>
static void launch_gate_up(const GemvArgs& g, int grid, size_t xs, hipStream_t stream) {
  const int cpl = (g.H + 2047) / 2048;
  if (cpl <= 1)
    hipLaunchKernelGGL((gemv_gate_up_kernel<kRegs, 1>), dim3(grid), dim3(kThreads), xs, stream, g);
  else if (cpl <= 2)
    hipLaunchKernelGGL((gemv_gate_up_kernel<kRegs, 2>), dim3(grid), dim3(kThreads), xs, stream, g);
  else
    hipLaunchKernelGGL((gemv_gate_up_kernel<kRegs, 4>), dim3(grid), dim3(kThreads), xs, stream, g);
}

hipError_t launch_decode(const GemvArgs& g, int num_cus, hipStream_t stream) {
  const int regs = (g.E + 63) / 64;
  const size_t xs = (size_t)g.H * sizeof(_Float16);
  // gate/up: enough waves that every item is loaded in one round
  const int items = g.k * g.I;
  int grid_gu = (items + kWaves * kMaxItems - 1) / (kWaves * kMaxItems);
  if (grid_gu < num_cus) grid_gu = (items + kWaves - 1) / kWaves < num_cus
                                       ? (items + kWaves - 1) / kWaves : num_cus;
  if (grid_gu < 1) grid_gu = 1;
  if (regs <= 1) launch_gate_up<1>(g, grid_gu, xs, stream);
  else if (regs <= 2) launch_gate_up<2>(g, grid_gu, xs, stream);
  else if (regs <= 4) launch_gate_up<4>(g, grid_gu, xs, stream);
  else if (regs <= 8) launch_gate_up<8>(g, grid_gu, xs, stream);
  else launch_gate_up<16>(g, grid_gu, xs, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int grid_dn = (g.H + kWaves - 1) / kWaves;
  if (grid_dn > num_cus * 2) grid_dn = num_cus * 2;
  const size_t hs = (size_t)g.k * g.I * sizeof(_Float16);
  if (g.y_dtype == kF32)
    hipLaunchKernelGGL(gemv_down_kernel<kF32>, dim3(grid_dn), dim3(kThreads), hs, stream, g);
  else if (g.y_dtype == kBF16)
    hipLaunchKernelGGL(gemv_down_kernel<kBF16>, dim3(grid_dn), dim3(kThreads), hs, stream, g);
  else
    hipLaunchKernelGGL(gemv_down_kernel<kF16>, dim3(grid_dn), dim3(kThreads), hs, stream, g);
  return hipGetLastError();
}

}  // namespace nf4moe
