// Grouped NF4 GEMM on CDNA4 matrix cores (prefill / training shapes).
//
// One launch runs every expert's projection Y_e = X_e . dequant(W_e)^T, the
// single-launch grouped kernel with nibbles decoded in registers and fp32
// accumulation that replaces the dequantise-then-GEMM round trip
// (experts4bit-qlora 0.22.0 README, "The package family"; grouped-nf4-gemm
// solutions entry "How do I run a grouped GEMM directly on NF4 packed MoE
// expert weights").  The weights never exist in memory in decoded form.
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_f16):
//   workgroup = 4 waves = one M-tile of 128 rows of ONE expert x 512 weight
//   rows (N).  The waves split N only: wave w owns 128 weight rows (8 n-tiles
//   of 16) and all 128 rows (8 m-tiles), i.e. 256 fp32 accumulators per lane.
//   Every weight is therefore decoded exactly once per workgroup.
//   K advances 64 at a time (one absmax block): two MFMA k-substeps of 32.
//
// Operand paths:
//   A (activations, fp16) -- gathered rows staged through a double-buffered
//     LDS tile (128 rows x 64 k, 144-byte padded rows so the 16-byte
//     fragment reads are conflict-free) and shared by the 4 waves.
//   B (weights) -- each lane loads its 8 packed bytes (16 codes) of a weight
//     row straight from HBM into registers and decodes them through the LDS
//     byte->half2 table (common.h): one v_perm + one ds_read_b32 per two
//     weights, then one v_pk_mul_f16 by the block's absmax.
//   The MFMA k order inside an instruction only has to agree between A and B:
//   lane group g (= lane/16) supplies k in [16g, 16g+16) of the 64-block,
//   substep s takes [16g + 8s, 16g + 8s + 8).
//
// Epilogues: optional per-expert LoRA (u = X A_e^T accumulated as an extra
// 16-column MFMA tile, split over the waves by k-step and reduced in LDS,
// then G += scale * u B_e^T as one more MFMA step), SwiGLU (gate and up rows
// of the same output column sit in the same lane), row scale, scatter.
//
// Tile scheduling: every workgroup rebuilds the per-expert M-tile table from
// expert_offsets in LDS (one load and a scan, overlapped with filling the
// decode table), so no host synchronisation and no extra launch is needed;
// the grid is sized from the upper bound ceil(P/128) + E and surplus
// workgroups exit.  blockIdx is remapped
// so that the workgroups one XCD runs back to back share an M-tile (its A
// rows stay in that XCD's L2).

#include "common.h"
#include "launch.h"

namespace nf4moe {

__constant__ float c_levels_gemm[16] = NF4MOE_LEVELS_INIT;

namespace {

constexpr int BM = kGemmBM;            // 128 rows per M-tile
constexpr int BK = 64;                 // k per step (one absmax block)
constexpr int MT = BM / 16;            // 8 m-tiles of 16 rows
constexpr int NT = 8;                  // 8 n-tiles of 16 weight rows per wave
constexpr int NWAVES = 4;
constexpr int kLutCopies = 64;
constexpr int A_STRIDE = BK * 2 + 16;  // bytes per LDS A row (padded)
constexpr int A_BUF = BM * A_STRIDE;   // bytes per A buffer

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

// 8 bf16 (two u32x4 halves packed as u32x4) -> 8 fp16 packed as u32x4.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 o;
  o.x = pack_half2((_Float16)bf16_bits_to_f32(v.x & 0xffffu), (_Float16)bf16_bits_to_f32(v.x >> 16));
  o.y = pack_half2((_Float16)bf16_bits_to_f32(v.y & 0xffffu), (_Float16)bf16_bits_to_f32(v.y >> 16));
  o.z = pack_half2((_Float16)bf16_bits_to_f32(v.z & 0xffffu), (_Float16)bf16_bits_to_f32(v.z >> 16));
  o.w = pack_half2((_Float16)bf16_bits_to_f32(v.w & 0xffffu), (_Float16)bf16_bits_to_f32(v.w >> 16));
  return o;
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) {
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace

template <bool kSwiglu, bool kLora, bool kABf16, int kOut>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs g,
                                                              int n_tiles) {
  __shared__ uint32_t s_lut[256 * kLutCopies];
  __shared__ __attribute__((aligned(16))) char s_a[2 * A_BUF];
  __shared__ int32_t s_tiles[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;   // lane group: k sub-range
  const int c16 = lane & 15;  // row of an A fragment / column of a B fragment

  lut_fill<kLutCopies>(s_lut, c_levels_gemm, tid, 256);
  // M-tile table from the offsets: thread t owns experts 4t..4t+3; an
  // exclusive scan over the 256 thread sums gives each expert's first tile.
  {
    __shared__ int32_t s_wave_sum[NWAVES];
    int32_t cnt[4];
    int32_t local = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ex = tid * 4 + u;
      cnt[u] = 0;
      if (ex < g.E) {
        const int32_t rows = g.offsets[ex + 1] - g.offsets[ex];
        cnt[u] = (rows + BM - 1) / BM;
      }
      local += cnt[u];
    }
    int32_t incl = local;  // inclusive scan inside the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) s_wave_sum[wave] = incl;
    __syncthreads();
    int32_t base = 0;
    for (int w = 0; w < wave; ++w) base += s_wave_sum[w];
    int32_t run = base + incl - local;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ex = tid * 4 + u;
      if (ex < g.E) s_tiles[ex] = run;
      run += cnt[u];
    }
    if (tid == 255) s_tiles[g.E] = run;
  }
  __syncthreads();

  // ---- which (expert, M-tile, N-tile) this workgroup computes
  const int per_xcd = gridDim.x >> 3;  // grid is a multiple of 8
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int mt_global = logical / n_tiles;
  const int n_idx = logical - mt_global * n_tiles;
  if (mt_global >= s_tiles[g.E]) return;  // surplus workgroup (uniform exit)
  int lo = 0, hi = g.E;  // s_tiles[lo] <= mt_global < s_tiles[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tiles[mid] <= mt_global) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int m_local = mt_global - s_tiles[e];
  const int off_e = g.offsets[e];
  const int cnt_e = g.offsets[e + 1] - off_e;
  const int row0 = off_e + m_local * BM;
  const int rows_valid = min(BM, cnt_e - m_local * BM);
  const int mt_valid = (rows_valid + 15) >> 4;

  const int N = g.N;
  const int K = g.K;
  const int nk = K / BK;
  const int I = N >> 1;  // SwiGLU only

  // ---- A staging assignment: thread -> 4 (row, 16-byte chunk) slots
  const int a_chunk = tid & 7;
  int64_t a_off[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    a_ok[i] = r < rows_valid;
    int64_t src = 0;
    if (a_ok[i]) {
      const int idx = row0 + r;
      src = g.gather ? (int64_t)(g.gather[idx] / g.gather_div) : (int64_t)idx;
    }
    a_off[i] = src * K + a_chunk * 8;  // element offset at k = 0
  }

  // ---- B assignment: n-tile nt of this wave -> weight row of lane column
  const uint8_t* b_ptr[NT];
  const float* s_ptr[NT];
  bool n_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int nrow, base;
    if constexpr (kSwiglu) {
      base = n_idx * 256 + wave * 64 + (nt & 3) * 16;
      n_ok[nt] = base < I;
      nrow = (nt < 4 ? 0 : I) + base + c16;
    } else {
      base = n_idx * 512 + wave * 128 + nt * 16;
      n_ok[nt] = base < N;
      nrow = base + c16;
    }
    if (!n_ok[nt]) nrow = 0;
    const int64_t wrow = (int64_t)e * N + nrow;
    b_ptr[nt] = g.packed + wrow * (K / 2) + g4 * 8;
    s_ptr[nt] = g.absmax + wrow * (K / BK);
  }
  bool any_n = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) any_n |= n_ok[nt];

  const uint32_t lane_off = lut_lane_offset<kLutCopies>(lane);

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  f32x4 acc_u[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_u[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: A(0) -> LDS buffer 0, B(0) -> registers
  u32x4 a_reg[4];
  auto load_a = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (a_ok[i]) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint16_t*>(g.a) + a_off[i] + (int64_t)kb * BK);
        a_reg[i] = kABf16 ? bf16x8_to_f16x8(v) : v;
      } else {
        a_reg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4*>(s_a + buf * A_BUF + r * A_STRIDE + a_chunk * 16) = a_reg[i];
    }
  };
  u32x2 b_reg[NT];
  float s_reg[NT];
  auto load_b = [&](int kb) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (n_ok[nt]) {
        b_reg[nt] = *reinterpret_cast<const u32x2*>(b_ptr[nt] + (int64_t)kb * 32);
        s_reg[nt] = s_ptr[nt][kb];
      }
    }
  };

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();

  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    // decode this step's weights (registers loaded during the previous step)
    u32x4 bf[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (n_ok[nt]) {
        const _Float16 sh = (_Float16)s_reg[nt];
        const f16x2 sc = {sh, sh};
        uint32_t d0[4], d1[4];
        decode8<kLutCopies>(s_lut, lane_off, b_reg[nt].x, d0);
        decode8<kLutCopies>(s_lut, lane_off, b_reg[nt].y, d1);
        bf[nt][0] = u32x4{half2_as_u32(u32_as_half2(d0[0]) * sc), half2_as_u32(u32_as_half2(d0[1]) * sc),
                          half2_as_u32(u32_as_half2(d0[2]) * sc), half2_as_u32(u32_as_half2(d0[3]) * sc)};
        bf[nt][1] = u32x4{half2_as_u32(u32_as_half2(d1[0]) * sc), half2_as_u32(u32_as_half2(d1[1]) * sc),
                          half2_as_u32(u32_as_half2(d1[2]) * sc), half2_as_u32(u32_as_half2(d1[3]) * sc)};
      }
    }
    // LoRA A operand of this step (one wave per step, rotating)
    const bool lora_turn = kLora && ((kb & 3) == wave);
    u32x4 bl[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (lora_turn && c16 < g.lora_r) {
      const uint16_t* la = reinterpret_cast<const uint16_t*>(g.lora_a) +
                           ((int64_t)e * g.lora_r + c16) * K + (int64_t)kb * BK + g4 * 16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(la + 8 * s);
        bl[s] = g.lora_bf16 ? bf16x8_to_f16x8(v) : v;
      }
    }
    // prefetch the next step
    if (kb + 1 < nk) {
      load_a(kb + 1);
      load_b(kb + 1);
    }
    // MFMAs
    const char* abuf = s_a + buf * A_BUF;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < mt_valid && (any_n || lora_turn)) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(
              abuf + (mt * 16 + c16) * A_STRIDE + g4 * 32 + s * 16);
          const f16x8 af = as_f16x8(av);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (n_ok[nt])
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  af, as_f16x8(bf[nt][s]), acc[mt][nt], 0, 0, 0);
          }
          if (lora_turn)
            acc_u[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                af, as_f16x8(bl[s]), acc_u[mt], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nk) store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- LoRA: reduce u over the waves, then G += (scale * u) B_e^T
  if constexpr (kLora) {
    float* s_u = reinterpret_cast<float*>(s_a);  // [NWAVES][BM][16]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_u[(wave * BM + mt * 16 + g4 * 4 + i) * 16 + c16] = acc_u[mt][i];
    __syncthreads();
    u32x4 bl2[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint16_t v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = 0;
      const int rho0 = g4 * 8;
      if (n_ok[nt] && g4 < 2) {
        int nrow;
        if constexpr (kSwiglu) {
          nrow = (nt < 4 ? 0 : I) + n_idx * 256 + wave * 64 + (nt & 3) * 16 + c16;
        } else {
          nrow = n_idx * 512 + wave * 128 + nt * 16 + c16;
        }
        const uint16_t* lb = reinterpret_cast<const uint16_t*>(g.lora_b) +
                             ((int64_t)e * N + nrow) * g.lora_r;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (rho0 + t < g.lora_r) {
            const uint16_t raw = lb[rho0 + t];
            if (g.lora_bf16) {
              const _Float16 h = (_Float16)bf16_bits_to_f32(raw);
              v[t] = __builtin_bit_cast(uint16_t, h);
            } else {
              v[t] = raw;
            }
          }
        }
      }
      bl2[nt] = u32x4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                      (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_valid && any_n) {
        const int row = mt * 16 + c16;
        _Float16 u[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int rho = g4 * 8 + t;
          float sum = 0.f;
          if (g4 < 2 && rho < g.lora_r) {
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) sum += s_u[(w * BM + row) * 16 + rho];
          }
          u[t] = (_Float16)(sum * g.lora_scale);
        }
        const f16x8 af = {u[0], u[1], u[2], u[3], u[4], u[5], u[6], u[7]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          if (n_ok[nt])
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                af, as_f16x8(bl2[nt]), acc[mt][nt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: SwiGLU / row scale / scatter, convert and store
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= mt_valid) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + g4 * 4 + i;
      if (row >= rows_valid) continue;
      const int grow = row0 + row;
      const int64_t orow = g.scatter ? (int64_t)g.scatter[grow] : (int64_t)grow;
      const float rs = g.row_scale ? g.row_scale[grow] : 1.0f;
      if constexpr (kSwiglu) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (!n_ok[nt]) continue;
          const int col = n_idx * 256 + wave * 64 + nt * 16 + c16;
          const float h = silu_f(acc[mt][nt][i]) * acc[mt][nt + 4][i];
          store_out<kOut>(g.out, orow * I + col, h * rs);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (!n_ok[nt]) continue;
          const int col = n_idx * 512 + wave * 128 + nt * 16 + c16;
          store_out<kOut>(g.out, orow * N + col, acc[mt][nt][i] * rs);
        }
      }
    }
  }
}

template <bool kSwiglu, bool kLora, bool kABf16>
static void launch_out(const GemmArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  switch (g.out_dtype) {
    case kF32:
      hipLaunchKernelGGL((grouped_gemm_kernel<kSwiglu, kLora, kABf16, kF32>), grid,
                         dim3(256), 0, s, g, n_tiles);
      break;
    case kBF16:
      hipLaunchKernelGGL((grouped_gemm_kernel<kSwiglu, kLora, kABf16, kBF16>), grid,
                         dim3(256), 0, s, g, n_tiles);
      break;
    default:
      hipLaunchKernelGGL((grouped_gemm_kernel<kSwiglu, kLora, kABf16, kF16>), grid,
                         dim3(256), 0, s, g, n_tiles);
      break;
  }
}

template <bool kSwiglu, bool kLora>
static void launch_a(const GemmArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  if (g.a_bf16) launch_out<kSwiglu, kLora, true>(g, grid, n_tiles, s);
  else launch_out<kSwiglu, kLora, false>(g, grid, n_tiles, s);
}

hipError_t launch_grouped_gemm(const GemmArgs& g, int num_cus, hipStream_t stream) {
  (void)num_cus;
  const int n_tiles = g.swiglu ? (g.N / 2 + 255) / 256 : (g.N + 511) / 512;
  const int64_t max_mtiles = (g.P + BM - 1) / BM + g.E;
  int64_t grid = max_mtiles * n_tiles;
  grid = (grid + 7) / 8 * 8;
  const dim3 dg((unsigned)grid);
  const bool lora = g.lora_a != nullptr;
  if (g.swiglu) {
    if (lora) launch_a<true, true>(g, dg, n_tiles, stream);
    else launch_a<true, false>(g, dg, n_tiles, stream);
  } else {
    if (lora) launch_a<false, true>(g, dg, n_tiles, stream);
    else launch_a<false, false>(g, dg, n_tiles, stream);
  }
  return hipGetLastError();
}

}  // namespace nf4moe
