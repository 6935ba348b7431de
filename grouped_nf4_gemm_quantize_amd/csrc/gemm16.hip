// The grouped GEMM on a 16-bit passthrough stack (bf16 or fp16 weights, no
// quantisation): the bf16 / fp16 storage modes of ExpertsNbit (experts4bit-
// qlora README "Training + expert offload": QUANT_TYPE selects the frozen
// base's storage precision, bf16 and fp16 among the choices), with the
// grouped-GEMM contract of the packed kernels (gather, SwiGLU, row scale,
// scatter).  Nothing is decoded: both operands are copied straight into
// LDS.  A 16-bit weight row needs 128 bytes per 64-wide k-step, four times
// the 4-bit code bytes, so this kernel has its own, simpler tiling rather
// than a mode of the 4-bit one:
//
//   - tile: 256 rows of one expert x 256 weight rows (SwiGLU: the gate and
//     up rows of 128 output columns), 32-wide k-steps; 8 waves as 2 (M) x 4
//     (N), each 128 rows x 64 weight rows = 4 x 2 accumulator tiles of
//     v_mfma_f32_32x32x16_f16 with the weights as the first operand, so an
//     accumulator tile is the transposed output block (lane: output row
//     lane & 31; column 8 (j / 4) + 4 (lane / 32) + j % 4);
//   - staging: a 3-stage ring (activations 16 KB + weights 16 KB per
//     stage), batches copied up to three steps ahead straight to LDS; the
//     16-byte chunk c of a 64-byte row r sits at c ^ ((r >> 2) & 3), so the
//     16 lanes of a fragment read cover all 64 banks;
//   - operands: bf16 activations with bf16 weights go to bf16 MFMAs as
//     stored (exact products); otherwise fp16 MFMAs, bf16 weights or
//     activations converted to fp16 in registers (exact for magnitudes in
//     fp16's normal range; smaller ones round to fp16 subnormals): fp16
//     activations with bf16 weights need fp16 operands to keep fp16's
//     mantissa on the activations.
//
// An expert's 16-bit gate_up block (8 MB at olmoe size) does not fit an
// XCD's 4 MB L2, so each row tile reads its expert's weights again: 256-row
// tiles halve that traffic against 128-row ones.  Tiles are dealt to a
// persistent grid round-robin, expert-major, by XCD.

#include "common.h"
#include "launch.h"
#include "mfma_common.h"

namespace nf4moe {

namespace {

constexpr int BM = 256;                   // rows per tile
constexpr int BK = 32;                    // k per step (64 bytes of a row)
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int WN = 4;                     // waves along N (2 along M)
constexpr int MT = 4;                     // 32-row m-tiles per wave (128 rows)
constexpr int NT = 2;                     // 32-row n-tiles per wave
constexpr int BN = WN * NT * 32;          // 256 weight rows per tile
constexpr int A_BYTES = BM * BK * 2;      // 16 KB
constexpr int B_BYTES = BN * BK * 2;      // 16 KB
constexpr int STAGE = A_BYTES + B_BYTES;  // 32 KB
constexpr int kDma = 4;                   // copies per wave and step: 2 + 2

__shared__ __attribute__((aligned(16))) char s_ring[3 * STAGE];
__shared__ int32_t s_tiles[kMaxExperts + 1];
__shared__ int32_t s_wsum[NWAVES];
__shared__ int32_t s_orow[2][BM];    // output row of each tile row (by tile parity)
__shared__ float s_rscale[2][BM];    // row scale of each tile row

struct Src16 {
  i32x4 a_rsrc, b_rsrc;
  uint32_t a_off[2];  // activations: 2 x 16 B per lane and step
  uint32_t b_off[2];  // weights: 2 x 16 B per lane and step
};

// Batch kb (clamped by the caller) into the stage at LDS address st: wave
// instruction i covers LDS rows 16 (2 wave + i) .. +16 of the activations,
// and of the weights (64 lanes x 16 B = 16 rows of 64 B).
__device__ __forceinline__ void issue(const Src16& s, int kb, uint32_t st, int wave) {
  const uint32_t soff = (uint32_t)kb * (BK * 2);
#pragma unroll
  for (int i = 0; i < 2; ++i) dma16(s.a_rsrc, s.a_off[i], soff, st + (wave * 2 + i) * 1024);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    dma16(s.b_rsrc, s.b_off[i], soff, st + A_BYTES + (wave * 2 + i) * 1024);
}

template <bool kBf16>
__device__ __forceinline__ f16x8 frag(const char* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  if constexpr (kBf16) v = bf16x8_to_f16x8(v);
  return as_f16x8(v);
}

// bf16 activations with bf16 weights: bf16 MFMAs on the raw bits
template <bool kABf16, bool kWBf16>
constexpr bool kNativeBf16 = kABf16 && kWBf16;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// The fragments of substep s (k chunk 2 s + g2 of each row) from stage st
// (raw bits for the bf16 MFMAs, else fp16).
template <bool kABf16, bool kWBf16>
__device__ __forceinline__ void load_frags(const char* st, uint32_t ro, uint32_t a_base,
                                           uint32_t b_base, f16x8 (&af)[MT], f16x8 (&bf)[NT]) {
  constexpr bool kNat = kNativeBf16<kABf16, kWBf16>;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) af[mt] = frag<kABf16 && !kNat>(st + a_base + mt * 32 * 64 + ro);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    bf[nt] = frag<kWBf16 && !kNat>(st + A_BYTES + b_base + nt * 32 * 64 + ro);
}

// Substep S of a step: its MFMAs on af/bf while the next substep's
// fragments are read (for S = 1 those of the next step's substep 0, from
// the next stage).
template <int S, bool kABf16, bool kWBf16>
__device__ __forceinline__ void substep(const char* st, const char* nst, const uint32_t (&ro)[2],
                                        uint32_t a_base, uint32_t b_base, int mtv,
                                        f16x8 (&af)[MT], f16x8 (&bf)[NT],
                                        f32x16 (&acc)[MT][NT]) {
  f16x8 an[MT], bn[NT];
  if constexpr (S == 0) load_frags<kABf16, kWBf16>(st, ro[1], a_base, b_base, an, bn);
  else load_frags<kABf16, kWBf16>(nst, ro[0], a_base, b_base, an, bn);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < mtv) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (kNativeBf16<kABf16, kWBf16>)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, bf[nt]), __builtin_bit_cast(bf16x8_t, af[mt]),
              acc[mt][nt], 0, 0, 0);
        else
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[nt], af[mt], acc[mt][nt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) af[mt] = an[mt];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bf[nt] = bn[nt];
}

// The k-loop of one tile.  Batch kb goes into stage kb % 3; the prologue
// issues batches 0, 1, 2.  After the barrier of step kb (every wave has read
// its fragments of stage kb % 3: substep 0 read the last ones) the wave
// issues batch kb + 3 there.  Before that barrier step kb + 1 must have
// landed, while batch kb + 2 may be pending: the wait leaves kDma copies.
// Nothing past the last step is fetched (only the prologue repeats the last
// batch when there are fewer than three steps); in the last two steps batch
// kb + 2 does not exist, so they drain instead.
template <bool kABf16, bool kWBf16>
__device__ __forceinline__ void kloop(const Src16& src, int nk, const uint32_t (&ro)[2],
                                      uint32_t a_base, uint32_t b_base, int mtv, int wave,
                                      f32x16 (&acc)[MT][NT]) {
  const uint32_t ring = lds_addr(s_ring);
  const int last = nk - 1;
  issue(src, 0, ring, wave);
  issue(src, min(1, last), ring + STAGE, wave);
  issue(src, min(2, last), ring + 2 * STAGE, wave);
  wait_vm_barrier<2 * kDma>();  // batch 0 landed
  f16x8 af[MT], bf[NT];
  load_frags<kABf16, kWBf16>(s_ring, ro[0], a_base, b_base, af, bf);
  int sidx = 0;
  for (int kb = 0; kb < nk; ++kb) {
    const int nidx = sidx == 2 ? 0 : sidx + 1;
    const char* st = s_ring + sidx * STAGE;
    const char* nst = s_ring + nidx * STAGE;
    substep<0, kABf16, kWBf16>(st, nst, ro, a_base, b_base, mtv, af, bf, acc);
    if (kb >= last - 1) wait_vm_barrier<0>();
    else wait_vm_barrier<kDma>();
    if (kb + 3 <= last) issue(src, kb + 3, ring + sidx * STAGE, wave);
    substep<1, kABf16, kWBf16>(st, nst, ro, a_base, b_base, mtv, af, bf, acc);
    sidx = nidx;
  }
}

template <int kOut>
__device__ __forceinline__ void store4(void* out, int64_t idx, const float (&v)[4]) {
  if constexpr (kOut == kF32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) = f32x4{v[0], v[1], v[2], v[3]};
  } else if constexpr (kOut == kBF16) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) =
        u32x2{(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
              (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
  } else {
    *reinterpret_cast<u32x2*>(reinterpret_cast<_Float16*>(out) + idx) =
        u32x2{pack_half2((_Float16)v[0], (_Float16)v[1]), pack_half2((_Float16)v[2], (_Float16)v[3])};
  }
}

}  // namespace

template <bool kSwiglu, bool kABf16, bool kWBf16, int kOut>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_gemm16_kernel(GemmArgs g, int n_tiles) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int n32 = lane & 31, g2 = lane >> 5;

  build_tile_table<NTHREADS, BM>(g.offsets, g.E, s_tiles, s_wsum, tid);

  const int N = g.N, K = g.K, I = N >> 1;
  const int nk = K / BK;
  // fragment offsets: row n32 of a 32-row block, k chunk 2 s + g2
  uint32_t ro[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) ro[s] = n32 * 64 + (((2 * s + g2) ^ ((n32 >> 2) & 3)) << 4);
  const uint32_t a_base = (uint32_t)wm * 128 * 64;
  const uint32_t b_base = (uint32_t)wn * 64 * 64;

  // weight row of LDS B row l (0..255) of N-tile n_idx, clamped to a valid
  // row.  SwiGLU: wave column wn's n-tile 0 holds the gate rows and n-tile 1
  // the up rows of output columns n_idx * 128 + 32 wn + [0, 32).
  auto weight_row = [&](int l, int n_idx) -> int {
    if constexpr (kSwiglu) {
      const int w = l >> 6, nt = (l >> 5) & 1, n = l & 31;
      const int col = n_idx * 128 + w * 32 + n;
      return (col < I ? col : I - 1) + (nt ? I : 0);
    } else {
      const int col = n_idx * BN + l;
      return col < N ? col : N - 1;
    }
  };

  const i32x4 a_rsrc = make_rsrc(g.a, (uint32_t)(g.a_rows * (int64_t)K * 2));
  const uint32_t w_bytes = (uint32_t)N * (uint32_t)K * 2u;
  const int total = __builtin_amdgcn_readfirstlane(s_tiles[g.E]) * n_tiles;
  const int G = gridDim.x;  // a multiple of 8
  const int u = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  for (int r = 0;; ++r) {
    const int tix = r * G + u;
    if (tix >= total) break;
    const int mt_global = tix / n_tiles;
    const int n_idx = tix - mt_global * n_tiles;
    int lo = 0, hi = g.E;  // s_tiles[lo] <= mt_global < s_tiles[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tiles[mid] <= mt_global) lo = mid; else hi = mid;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int m_local = mt_global - __builtin_amdgcn_readfirstlane(s_tiles[e]);
    const int row0 = __builtin_amdgcn_readfirstlane(g.offsets[e]) + m_local * BM;
    const int rows_valid = min(BM, __builtin_amdgcn_readfirstlane(g.offsets[e + 1]) - row0);
    // this wave's valid 32-row m-tiles
    const int mtv = max(0, min(MT, (rows_valid - wm * 128 + 31) >> 5));

    Src16 src;
    src.a_rsrc = a_rsrc;
    src.b_rsrc = make_rsrc(reinterpret_cast<const char*>(g.packed) + (int64_t)e * w_bytes, w_bytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = (wave * 2 + i) * 64 + lane;
      const int row = c >> 2;
      const int gchunk = (c & 3) ^ ((row >> 2) & 3);
      const int rr = row < rows_valid ? row : 0;
      const int idx = row0 + rr;
      const uint32_t a_src = g.gather ? (uint32_t)(g.gather[idx] / g.gather_div) : (uint32_t)idx;
      src.a_off[i] = (a_src * (uint32_t)K + gchunk * 8) * 2;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = (wave * 2 + i) * 64 + lane;
      const int l = c >> 2;
      const int gchunk = (c & 3) ^ ((l >> 2) & 3);
      src.b_off[i] = ((uint32_t)weight_row(l, n_idx) * (uint32_t)K + gchunk * 8) * 2;
    }

    const int par = r & 1;
    if (tid < BM) {
      const int grow = row0 + (tid < rows_valid ? tid : 0);
      s_orow[par][tid] = g.scatter ? g.scatter[grow] : grow;
      s_rscale[par][tid] = g.row_scale ? g.row_scale[grow] : 1.0f;
    }

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.f;

    // every wave is done with the previous tile's ring and row tables
    lds_barrier();
    kloop<kABf16, kWBf16>(src, nk, ro, a_base, b_base, mtv, wave, acc);

    // epilogue straight from the accumulators: four consecutive output
    // columns per store, rows scattered to their output rows
    const int ncols = kSwiglu ? I : N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int trow = wm * 128 + mt * 32 + n32;
      if (mt >= mtv || trow >= rows_valid) continue;
      const int64_t orow = s_orow[par][trow];
      const float rs = s_rscale[par][trow];
      constexpr int NTO = kSwiglu ? 1 : NT;
#pragma unroll
      for (int nt = 0; nt < NTO; ++nt) {
        const int cb = kSwiglu ? n_idx * 128 + wn * 32 : n_idx * BN + wn * 64 + nt * 32;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int col = cb + 8 * jj + 4 * g2;
          if (col >= ncols) continue;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 4 * jj + i;
            if constexpr (kSwiglu)
              v[i] = silu_f(acc[mt][0][j]) * acc[mt][1][j] * rs;
            else
              v[i] = acc[mt][nt][j] * rs;
          }
          store4<kOut>(g.out, orow * ncols + col, v);
        }
      }
    }
  }
  // no memory operation of the wave is left in flight when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

namespace {

template <bool kSwiglu, bool kABf16, bool kWBf16>
void launch_out16(const GemmArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  switch (g.out_dtype) {
    case kF32:
      hipLaunchKernelGGL((grouped_gemm16_kernel<kSwiglu, kABf16, kWBf16, kF32>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
    case kBF16:
      hipLaunchKernelGGL((grouped_gemm16_kernel<kSwiglu, kABf16, kWBf16, kBF16>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
    default:
      hipLaunchKernelGGL((grouped_gemm16_kernel<kSwiglu, kABf16, kWBf16, kF16>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
  }
}

template <bool kSwiglu>
void launch_aw16(const GemmArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  const bool wb = g.qtype == kQtBF16;
  if (g.a_bf16) {
    if (wb) launch_out16<kSwiglu, true, true>(g, grid, n_tiles, s);
    else launch_out16<kSwiglu, true, false>(g, grid, n_tiles, s);
  } else {
    if (wb) launch_out16<kSwiglu, false, true>(g, grid, n_tiles, s);
    else launch_out16<kSwiglu, false, false>(g, grid, n_tiles, s);
  }
}

// fp32 or bf16 weights -> the 16-bit stack (round to nearest even), 8
// elements per thread and step.
template <bool kInBf16, bool kOutBf16>
__global__ __launch_bounds__(256) void to16_kernel(const void* __restrict__ w, int64_t n8,
                                                   uint16_t* __restrict__ out) {
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n8;
       q += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    if constexpr (kInBf16) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(w) + q * 8);
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(xs[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(xs[i] >> 16);
      }
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(w) + q * 8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(w) + q * 8 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kOutBf16)
        o[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
      else
        o[i] = pack_half2((_Float16)v[2 * i], (_Float16)v[2 * i + 1]);
    }
    *reinterpret_cast<u32x4*>(out + q * 8) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

}  // namespace

hipError_t launch_grouped_gemm16(const GemmArgs& g, int num_cus, hipStream_t stream) {
  const int n_tiles = g.swiglu ? (g.N / 2 + 127) / 128 : (g.N + BN - 1) / BN;
  int grid = (num_cus + 7) / 8 * 8;
  const int64_t max_tiles = ((g.P + BM - 1) / BM + g.E) * n_tiles;
  if ((int64_t)grid > max_tiles) grid = (int)((max_tiles + 7) / 8 * 8);
  if (grid < 8) grid = 8;
  const dim3 dg((unsigned)grid);
  if (g.swiglu) launch_aw16<true>(g, dg, n_tiles, stream);
  else launch_aw16<false>(g, dg, n_tiles, stream);
  return hipGetLastError();
}

hipError_t launch_to16(const void* w, bool w_bf16, int64_t n, bool out_bf16, uint16_t* out,
                       int num_cus, hipStream_t s) {
  const int64_t n8 = n / 8;
  int64_t grid = (n8 + 255) / 256;
  if (grid > (int64_t)num_cus * 16) grid = (int64_t)num_cus * 16;
  if (grid < 1) grid = 1;
  if (w_bf16) {
    if (out_bf16) hipLaunchKernelGGL((to16_kernel<true, true>), dim3(grid), dim3(256), 0, s, w, n8, out);
    else hipLaunchKernelGGL((to16_kernel<true, false>), dim3(grid), dim3(256), 0, s, w, n8, out);
  } else {
    if (out_bf16) hipLaunchKernelGGL((to16_kernel<false, true>), dim3(grid), dim3(256), 0, s, w, n8, out);
    else hipLaunchKernelGGL((to16_kernel<false, false>), dim3(grid), dim3(256), 0, s, w, n8, out);
  }
  return hipGetLastError();
}

}  // namespace nf4moe
