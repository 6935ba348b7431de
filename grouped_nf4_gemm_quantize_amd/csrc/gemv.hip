// Single-token (T = 1) decode path: split-K GEMVs over the routed experts.
//
// At batch 1 the expert projection is a matrix-vector product per routed
// expert that streams the packed bytes once (experts4bit-qlora 0.22.0 README,
// "Inference": the single-token decode fast path uses a fused 4-bit GEMV).  HBM
// bandwidth on the NF4 codes + absmax is the roofline, and with only ~21 MB
// per layer the time is dominated by how early the loads are issued, so both
// kernels issue every weight load of a wave before doing any arithmetic.
//
//   gemv_gate_up_kernel  routes the token (every workgroup recomputes the
//     top-k of its E logits -- a few hundred cycles -- so no extra launch),
//     then one wave per (slot j, column i) item computes the gate row i and
//     the up row I+i of expert ids[j] against x and writes
//     h[j, i] = w_j * silu(gate) * up  (fp32).
//   gemv_down_kernel  one wave per output row n: the K of the row is the
//     concatenation of the k routed experts' I inputs, so the combine over
//     the slots is part of the dot product; y[n] is written directly.
//
// Split-K inside a wave: lane l takes the 32-weight chunks l, l+64, ... of a
// row (16 packed bytes = one 16-byte load; a chunk is half of one 64-block so
// it needs one absmax), decodes them through the LDS byte->half2 table
// (common.h) and multiplies with v_dot2_f32_f16 against fp16 activations held
// in LDS; the 64 partial sums are reduced across the wave.

#include "common.h"
#include "launch.h"
#include "route_device.h"

namespace nf4moe {

__constant__ float c_levels_gemv[16] = NF4MOE_LEVELS_INIT;

namespace {
constexpr int kCopies = 32;
constexpr int kMaxItems = 4;          // gate/up items preloaded per wave and round
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

}  // namespace

// kCpl = ceil(H / 2048) <= 4: 32-weight chunks of one row per lane.
template <int kRegs, int kCpl>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(GemvArgs g) {
  __shared__ uint32_t s_lut[256 * kCopies];
  __shared__ uint16_t s_stage[16];
  __shared__ int s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  extern __shared__ __attribute__((aligned(16))) _Float16 s_x[];  // [H]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = g.H, I = g.I, k = g.k;

  if (wave == 0) {
    int id;
    float w;
    route_one_token<kRegs>(g.logits, g.E, k, g.renormalize, lane, &id, &w);
    if (lane < k) {
      s_ids[lane] = id;
      s_w[lane] = w;
      if (blockIdx.x == 0) {
        g.topk_ids[lane] = id;
        g.topk_w[lane] = w;
      }
    }
  }
  for (int i = tid; i < H; i += 256) {
    const uint16_t raw = reinterpret_cast<const uint16_t*>(g.x)[i];
    s_x[i] = g.x_bf16 ? (_Float16)bf16_bits_to_f32(raw) : __builtin_bit_cast(_Float16, raw);
  }
  lut_fill<kCopies>(s_lut, s_stage, c_levels_gemv, tid, 256);  // ends with a barrier

  const uint32_t lane_off = lut_lane_offset<kCopies>(lane);
  const int chunks = H / 32;
  const int64_t row_bytes = H / 2;
  const int64_t row_blocks = H / 64;
  const int nw = gridDim.x * 4;
  const int items = k * I;
  for (int q0 = blockIdx.x * 4 + wave; q0 < items; q0 += nw * kMaxItems) {
    // issue every load of this round first
    u32x4 qg[kMaxItems][kCpl], qu[kMaxItems][kCpl];
    float sg[kMaxItems][kCpl], su[kMaxItems][kCpl];
#pragma unroll
    for (int it = 0; it < kMaxItems; ++it) {
      const int q = q0 + it * nw;
      const int qq = q < items ? q : q0;  // clamp: re-read a valid item
      const int j = qq / I;
      const int i = qq - j * I;
      const int e = s_ids[j];
      const int64_t rg = (int64_t)e * 2 * I + i;
      const int64_t ru = rg + I;
#pragma unroll
      for (int m = 0; m < kCpl; ++m) {
        int c = lane + 64 * m;
        if (c >= chunks) c = chunks - 1;
        qg[it][m] = *reinterpret_cast<const u32x4*>(g.gu_packed + rg * row_bytes + c * 16);
        qu[it][m] = *reinterpret_cast<const u32x4*>(g.gu_packed + ru * row_bytes + c * 16);
        sg[it][m] = g.gu_absmax[rg * row_blocks + (c >> 1)];
        su[it][m] = g.gu_absmax[ru * row_blocks + (c >> 1)];
      }
    }
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
      if (lane == 0 && q < items) {
        const int j = q / I;
        g.hbuf[q] = silu_g(accg) * accu * s_w[j];
      }
    }
  }
}

template <int kOut>
__global__ __launch_bounds__(256) void gemv_down_kernel(GemvArgs g) {
  __shared__ uint32_t s_lut[256 * kCopies];
  __shared__ uint16_t s_stage[16];
  extern __shared__ __attribute__((aligned(16))) _Float16 s_h[];  // [k, I]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = g.H, I = g.I, k = g.k;

  // this lane's chunks of the concatenated K (the same for every output row)
  const int cps = I / 32;  // chunks per slot
  const int total = k * cps;
  int64_t pk_off[kMaxChunksPerLane];
  int64_t am_off[kMaxChunksPerLane];
  int h_off[kMaxChunksPerLane];
  int nc = 0;
#pragma unroll
  for (int m = 0; m < kMaxChunksPerLane; ++m) {
    const int cc = lane + 64 * m;
    pk_off[m] = 0;
    am_off[m] = 0;
    h_off[m] = 0;
    if (cc < total) {
      const int j = cc / cps;
      const int c = cc - j * cps;
      const int e = g.topk_ids[j];
      pk_off[m] = (int64_t)e * H * (I / 2) + c * 16;
      am_off[m] = (int64_t)e * H * (I / 64) + (c >> 1);
      h_off[m] = j * I + c * 32;
      nc = m + 1;
    }
  }
  // one output row per wave and round; issue the row's loads before the
  // table fill so they are in flight meanwhile
  const int nw = gridDim.x * 4;
  int n = blockIdx.x * 4 + wave;
  u32x4 q[kMaxChunksPerLane];
  float s[kMaxChunksPerLane];
  auto load_row = [&](int row) {
    const int64_t prow = (int64_t)row * (I / 2);
    const int64_t arow = (int64_t)row * (I / 64);
#pragma unroll
    for (int m = 0; m < kMaxChunksPerLane; ++m) {
      if (m < nc) {
        q[m] = *reinterpret_cast<const u32x4*>(g.dn_packed + pk_off[m] + prow);
        s[m] = g.dn_absmax[am_off[m] + arow];
      }
    }
  };
  if (n < H) load_row(n);

  for (int i = tid; i < k * I; i += 256) s_h[i] = (_Float16)g.hbuf[i];
  lut_fill<kCopies>(s_lut, s_stage, c_levels_gemv, tid, 256);  // ends with a barrier

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
    hipLaunchKernelGGL((gemv_gate_up_kernel<kRegs, 1>), dim3(grid), dim3(256), xs, stream, g);
  else if (cpl <= 2)
    hipLaunchKernelGGL((gemv_gate_up_kernel<kRegs, 2>), dim3(grid), dim3(256), xs, stream, g);
  else
    hipLaunchKernelGGL((gemv_gate_up_kernel<kRegs, 4>), dim3(grid), dim3(256), xs, stream, g);
}

hipError_t launch_decode(const GemvArgs& g, int num_cus, hipStream_t stream) {
  const int regs = (g.E + 63) / 64;
  const size_t xs = (size_t)g.H * sizeof(_Float16);
  // gate/up: enough waves that every item is preloaded in one round
  const int items = g.k * g.I;
  int grid_gu = (items + 4 * kMaxItems - 1) / (4 * kMaxItems);
  if (grid_gu > num_cus * 2) grid_gu = num_cus * 2;
  if (grid_gu < 1) grid_gu = 1;
  if (regs <= 1) launch_gate_up<1>(g, grid_gu, xs, stream);
  else if (regs <= 2) launch_gate_up<2>(g, grid_gu, xs, stream);
  else if (regs <= 4) launch_gate_up<4>(g, grid_gu, xs, stream);
  else if (regs <= 8) launch_gate_up<8>(g, grid_gu, xs, stream);
  else launch_gate_up<16>(g, grid_gu, xs, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int grid_dn = (g.H + 3) / 4;
  if (grid_dn > num_cus * 2) grid_dn = num_cus * 2;
  const size_t hs = (size_t)g.k * g.I * sizeof(_Float16);
  if (g.y_dtype == kF32)
    hipLaunchKernelGGL(gemv_down_kernel<kF32>, dim3(grid_dn), dim3(256), hs, stream, g);
  else if (g.y_dtype == kBF16)
    hipLaunchKernelGGL(gemv_down_kernel<kBF16>, dim3(grid_dn), dim3(256), hs, stream, g);
  else
    hipLaunchKernelGGL(gemv_down_kernel<kF16>, dim3(grid_dn), dim3(256), hs, stream, g);
  return hipGetLastError();
}

}  // namespace nf4moe
