// Grouped NF4 GEMM on CDNA4 matrix cores (prefill / training shapes).
//
// One launch runs every expert's projection Y_e = X_e . dequant(W_e)^T, the
// single-launch grouped kernel with nibbles decoded in registers and fp32
// accumulation that replaces the dequantise-then-GEMM round trip
// (experts4bit-qlora 0.22.0 README, "The package family"; grouped-nf4-gemm
// solutions entry "How do I run a grouped GEMM directly on NF4 packed MoE
// expert weights").  Decoded weights never exist in memory.
//
// Work decomposition (gfx950, wave64, v_mfma_f32_32x32x16_f16):
//   A tile = 128 rows of ONE expert (an M-tile) x 512 weight rows (N).
//   Workgroup = 8 waves, two per SIMD; the waves split N only, so wave w
//   owns 64 weight rows (2 n-tiles of 32) against all 128 rows (4 m-tiles
//   of 32): 128 fp32 accumulators per lane, and every weight is decoded
//   exactly once per tile.  With two waves per SIMD, one wave's MFMAs run
//   while the other waits on LDS reads, copy issue or the step barrier (one
//   wave per SIMD leaves the matrix pipe idle through every such stall).
//   K advances 64 per step (one absmax block) in four MFMA substeps of 16.
//   Workgroups are persistent (one per CU): the decode table and the
//   per-expert tile table are built once, then tiles are taken in an order
//   that gives the 32 workgroups of one XCD consecutive tiles (tiles sharing
//   activation rows or weight rows meet in that XCD's L2).
//
// Operand staging: buffer loads that write LDS directly (no VGPR staging)
// copy the operands global -> LDS ahead of use:
//   activations (fp16) and the LoRA A rows of one step into a 2-stage ring,
//   one step ahead;
//   packed codes of a step PAIR (64 bytes of every weight row: half the
//   address-unit work of 32-byte rows, which cost as much per row as full
//   64-byte segments) into a 2-stage ring, two steps ahead;
//   absmax in groups of four steps (16 bytes per weight row) into a double
//   buffer, two steps ahead.
// The copies are issued from inline assembly, so the compiler does not
// track them: the kernel itself waits with a counted s_waitcnt on the
// vector-memory counter (copies complete in issue order; every wave issues
// the same copies, so one immediate per step phase holds for all of them)
// followed by s_barrier; see kloop for the schedule.
//   A stage: 128 rows x 128 B; the 16-byte chunk c of row r sits at chunk
//            c ^ ((r >> 1) & 7).  The LDS has 64 banks of 4 bytes and
//            serves a 16-byte read per lane in groups of 16 lanes: 16
//            fragment rows r..r+15 must cover all 64 banks, and two rows
//            2 apart (same bank half) must differ in the swizzled chunk.
//   pair stage: 512 rows x 64 B (steps 2p, 2p + 1: 64 codes each); the
//            16-byte chunk c of row l sits at c ^ ((l >> 2) & 3), so 16
//            consecutive rows cover all 64 banks.
//   L (after A in the A stage): 16 LoRA A rows x 128 B.
//   absmax group: 512 rows x 4 fp32.
// Buffer resources bound every copy: a source offset outside the tensor
// reads zeros instead of faulting.
// Decode: the lane's 8 codes for one MFMA operand (one u32) go through the
// LDS byte -> half2 table (common.h): per byte one address computation and
// one ds_read_b32, then one v_pk_mul_f16 by the block's absmax.
// MFMA k order: within a 64-block, lane group g = lane/32 takes k in
// [32g, 32g+32); substep s uses [32g + 8s, 32g + 8s + 8) for both operands.
//
// Epilogues: optional per-expert LoRA (u = X A_e^T on 16x16x32 MFMAs, each
// wave for its own 32 rows, exchanged through LDS in fp16 with the LoRA scale
// applied, then G += u B_e^T as one more 32x32x16 MFMA per accumulator tile),
// SwiGLU (gate and up columns of one output column share a lane), row scale,
// scatter, conversion to the output dtype.

#include "common.h"
#include "launch.h"
#include "mfma_common.h"

namespace nf4moe {

__constant__ float c_levels_gemm[16] = NF4MOE_LEVELS_INIT;
__constant__ float c_levels_gemm_fp4[16] = NF4MOE_FP4_LEVELS_INIT;
__constant__ float c_levels_gemm_mx[16] = NF4MOE_E2M1_VALUES_INIT;

namespace {

constexpr int BM = kGemmBM;       // 128 rows per M-tile
constexpr int BK = 64;            // k per step (one absmax block)
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int MT = BM / 32;       // 4 m-tiles of 32 rows
constexpr int NT = 2;             // 2 n-tiles of 32 weight rows per wave
constexpr int BNW = NT * 32;      // 64 weight rows per wave
constexpr int BN = NWAVES * BNW;  // 512 weight rows per workgroup
constexpr int kCopies = 32;
// Activation ring: 2 stages of one step (A 16384 B, then the LoRA A rows
// 2048 B).  Packed-code ring: 2 stages of one step PAIR (512 rows x 64 B).
constexpr int OFF_L = BM * BK * 2;                   // A: 16384 B
constexpr int ASTAGE = OFF_L + kMaxLoraR * BK * 2;   // + L: 2048 B -> 18432 B
constexpr int OFF_BR = 2 * ASTAGE;                   // packed-code ring
constexpr int BPAIR = BN * BK;                       // 512 rows x 64 B = 32768 B
constexpr int RING = OFF_BR + 2 * BPAIR;             // 102400 B
constexpr int kAbsGroup = 4;                   // steps of absmax per copy (16 B per row)
constexpr int kMxGroup = 8;                    // MXFP4: steps of scale bytes per copy (2 per step)
// weight formats (a template parameter of the kernel)
constexpr int kW4 = 0;   // 4-bit codes through the decode table, fp32 absmax per 64 (nf4, fp4)
constexpr int kWMx = 1;  // MXFP4: e2m1 codes through the table, e8m0 scale per 32
constexpr int kWI8 = 2;  // 8-bit int8 codes, fp32 absmax per 64
constexpr int kWF8 = 3;  // 8-bit fp8 e4m3 codes, fp32 absmax per 64
// Adapter storage, a compile-time choice so the k-loop carries no select
constexpr int kLoraNone = 0;
constexpr int kLoraF16 = 1;
constexpr int kLoraBF16 = 2;

}  // namespace

__shared__ __attribute__((aligned(16))) char g_ring[RING];
__shared__ uint32_t g_lut[256 * kCopies];
// absmax of kAbsGroup consecutive steps for the tile's 512 weight rows, two
// groups in flight: g_sabs[group & 1][row * kAbsGroup + step % kAbsGroup]
__shared__ __attribute__((aligned(16))) float g_sabs[2][BN * kAbsGroup];
__shared__ int32_t g_tiles[kMaxExperts + 1];
__shared__ uint16_t g_lstage[16];
__shared__ int32_t g_wsum[NWAVES];
__shared__ int32_t g_orow[2][BM];    // output row of each tile row (by tile parity)
__shared__ float g_rscale[2][BM];    // row scale of each tile row

namespace {

// LoRA u of the tile (fp16 [BM][16]) at the end of the ring, which is free
// once the k-loop has drained; the epilogue staging uses the ring's start.
constexpr int OFF_U = RING - BM * kMaxLoraR * 2;
__device__ __forceinline__ _Float16* u_buf() {
  return reinterpret_cast<_Float16*>(g_ring + OFF_U);
}

__device__ __forceinline__ uint32_t lut_read(uint32_t addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(g_lut) + addr);
}

// 8 codes -> 8 fp16 weights (x absmax), as an MFMA operand.
__device__ __forceinline__ f16x8 decode_scaled(uint32_t q, uint32_t lane_off, f16x2 sc) {
  const uint32_t d0 = lut_read(lut_addr<kCopies, 0>(q, lane_off));
  const uint32_t d1 = lut_read(lut_addr<kCopies, 1>(q, lane_off));
  const uint32_t d2 = lut_read(lut_addr<kCopies, 2>(q, lane_off));
  const uint32_t d3 = lut_read(lut_addr<kCopies, 3>(q, lane_off));
  const u32x4 v = {half2_as_u32(u32_as_half2(d0) * sc), half2_as_u32(u32_as_half2(d1) * sc),
                   half2_as_u32(u32_as_half2(d2) * sc), half2_as_u32(u32_as_half2(d3) * sc)};
  return as_f16x8(v);
}

// Copy sources of one tile: buffer resources (scalar) and per-lane byte
// offsets (fixed for the tile; the step adds a scalar offset).
struct Src {
  i32x4 a_rsrc, b_rsrc, s_rsrc, l_rsrc;
  uint32_t a_off[2];  // A: 2 x 16 B per lane (1 KB per wave instruction)
  uint32_t b_off[4];  // packed codes of a step pair: 4 x 16 B
  uint32_t s_off;     // absmax: 16 B (kAbsGroup steps of one row per lane)
  uint32_t l_off;     // LoRA A: 4 B
};

// Copies per wave: activations of one step (+ LoRA A), the packed codes of
// a step pair, an absmax group.
template <int kLora>
constexpr int kDmaA() { return kLora != kLoraNone ? 3 : 2; }
constexpr int kDmaB = 4;
constexpr int kDmaAbs = 1;

// Activations (and LoRA A rows) of step `kb` (clamped) into the A stage at
// LDS address `st`.
template <int kLora>
__device__ __forceinline__ void issue_a(const Src& s, int kb, uint32_t st, int wave) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    dma16(s.a_rsrc, s.a_off[i], (uint32_t)kb * (BK * 2), st + (wave * 2 + i) * 1024);
  if constexpr (kLora != kLoraNone)
    dma4(s.l_rsrc, s.l_off, (uint32_t)kb * (BK * 2), st + OFF_L + wave * 256);
}

// Packed codes of step pair `p` (clamped; steps 2p, 2p + 1: 64 bytes of
// every weight row) into the pair stage at LDS address `bst`.
__device__ __forceinline__ void issue_b(const Src& s, int p, uint32_t bst, int wave) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dma16(s.b_rsrc, s.b_off[i], (uint32_t)p * BK, bst + (wave * 4 + i) * 1024);
}

// Copies 2h and 2h + 1 of issue_b (h = 0, 1).
__device__ __forceinline__ void issue_b_half(const Src& s, int p, uint32_t bst, int wave, int h) {
#pragma unroll
  for (int i = 2 * h; i < 2 * h + 2; ++i)
    dma16(s.b_rsrc, s.b_off[i], (uint32_t)p * BK, bst + (wave * 4 + i) * 1024);
}

// The absmax of steps [4 grp, 4 grp + 4) into buffer `buf`.
__device__ __forceinline__ void issue_abs(const Src& s, int grp, int buf, int wave) {
  dma16(s.s_rsrc, s.s_off, (uint32_t)grp * (kAbsGroup * 4),
        lds_addr(&g_sabs[buf][0]) + wave * 1024);
}

// Per-lane LDS read offsets, fixed for the kernel.
struct Rd {
  uint32_t a[4];   // A fragment of substep s (m-tile 0; + 4096 per m-tile)
  uint32_t b[2];   // packed codes of n-tile 0 in a pair stage, by step parity (+ 2048 per n-tile)
  uint32_t b8[2];  // 8-bit codes: chunks 2 g2 and 2 g2 + 1 of a one-step stage (+ 2048 per n-tile)
  uint32_t s;      // absmax element of n-tile 0's row (+ 32 rows per n-tile)
  uint32_t ua[2];  // LoRA: A fragment (16x16x32) of this wave's 16 rows, [k half]
  uint32_t ul;     // LoRA: A_e fragment of this lane (k half 0; + 64 B for half 1)
  uint32_t lane_off;
};

// Registers of one step that come from the stage: this wave's packed
// weights (4 n-tiles x 16 B) and their absmax as an fp16 pair.
struct StepRegs {
  u32x4 bq[NT];
  u32x4 bq2[NT];  // 8-bit codes: the second 16 bytes of the lane's 32
  f16x2 sc[NT];
};

template <int kW>
__device__ __forceinline__ void load_step_regs(const char* bst, int step, const Rd& rd,
                                               StepRegs& r) {
  const uint32_t bo = (step & 1) ? rd.b[1] : rd.b[0];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    _Float16 sh;
    if constexpr (kW >= kWI8) {
      // 32 codes of the lane's k half; scale = absmax / 127 (int8) or / 448 (fp8)
      r.bq[nt] = *reinterpret_cast<const u32x4*>(bst + rd.b8[0] + nt * 2048);
      r.bq2[nt] = *reinterpret_cast<const u32x4*>(bst + rd.b8[1] + nt * 2048);
      const float a = g_sabs[(step / kAbsGroup) & 1][rd.s + nt * 32 * kAbsGroup + step % kAbsGroup];
      sh = (_Float16)(a / (kW == kWI8 ? 127.0f : 448.0f));
      r.sc[nt] = f16x2{sh, sh};
      continue;
    }
    r.bq[nt] = *reinterpret_cast<const u32x4*>(bst + bo + nt * 2048);
    if constexpr (kW == kWMx) {
      // the e8m0 byte of this lane's 32-element block (k half g2 of the step)
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(&g_sabs[(step / kMxGroup) & 1][0]);
      sh = e8m0_to_half(sb[rd.s + nt * 32 * 16 + (step % kMxGroup) * 2]);
    } else {
      sh = (_Float16)g_sabs[(step / kAbsGroup) & 1][rd.s + nt * 32 * kAbsGroup + step % kAbsGroup];
    }
    r.sc[nt] = f16x2{sh, sh};
  }
}

template <int MTV, bool kABf16>
__device__ __forceinline__ void load_a(const char* st, const Rd& rd, int s, f16x8 (&af)[MT]) {
#pragma unroll
  for (int mt = 0; mt < MTV; ++mt) {
    u32x4 v = *reinterpret_cast<const u32x4*>(st + rd.a[s] + mt * 4096);
    if constexpr (kABf16) v = bf16x8_to_f16x8(v);
    af[mt] = as_f16x8(v);
  }
}

__device__ __forceinline__ uint32_t q_of(const u32x4& v, int s) {
  return s == 0 ? v.x : (s == 1 ? v.y : (s == 2 ? v.z : v.w));
}

// Table lookups of substep s for all n-tiles (raw half2 pairs, unscaled).
__device__ __forceinline__ void lut_lookups(const StepRegs& r, int s, uint32_t lane_off,
                                            uint32_t (&d)[NT][4]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint32_t q = q_of(r.bq[nt], s);
    d[nt][0] = lut_read(lut_addr<kCopies, 0>(q, lane_off));
    d[nt][1] = lut_read(lut_addr<kCopies, 1>(q, lane_off));
    d[nt][2] = lut_read(lut_addr<kCopies, 2>(q, lane_off));
    d[nt][3] = lut_read(lut_addr<kCopies, 3>(q, lane_off));
  }
}

__device__ __forceinline__ void scale_b(const StepRegs& r, const uint32_t (&d)[NT][4],
                                        f16x8 (&bf)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const u32x4 v = {half2_as_u32(u32_as_half2(d[nt][0]) * r.sc[nt]),
                     half2_as_u32(u32_as_half2(d[nt][1]) * r.sc[nt]),
                     half2_as_u32(u32_as_half2(d[nt][2]) * r.sc[nt]),
                     half2_as_u32(u32_as_half2(d[nt][3]) * r.sc[nt])};
    bf[nt] = as_f16x8(v);
  }
}

// 8-bit codes of substep S (k = 32 g2 + 8 S .. + 8) -> scaled fp16 operands.
// int8: each byte b becomes the fp16 1024 + (b ^ 0x80) by placing it under
// the exponent byte 0x64 (one v_perm per two bytes), minus 1152 = b, exact;
// fp8 e4m3: the hardware fp8 -> fp16 conversion (exact at scale 1).
template <int kW, int S>
__device__ __forceinline__ void decode_b8(const StepRegs& r, f16x8 (&bf)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const u32x4 q = (S >> 1) ? r.bq2[nt] : r.bq[nt];
    const uint32_t w0 = (S & 1) ? q.z : q.x;
    const uint32_t w1 = (S & 1) ? q.w : q.y;
    f16x2 h[4];
    if constexpr (kW == kWI8) {
      const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
      const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
      h[0] = u32_as_half2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) - off;
      h[1] = u32_as_half2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) - off;
      h[2] = u32_as_half2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) - off;
      h[3] = u32_as_half2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) - off;
    } else {
      h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
      h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
      h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
      h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    }
    const u32x4 v = {half2_as_u32(h[0] * r.sc[nt]), half2_as_u32(h[1] * r.sc[nt]),
                     half2_as_u32(h[2] * r.sc[nt]), half2_as_u32(h[3] * r.sc[nt])};
    bf[nt] = as_f16x8(v);
  }
}

// Substep S of a step: its MFMAs, with A fragments `af` and its weights `bs`
// (table words already scaled by the block's absmax) in registers, while the
// A fragments and table words of the next substep are read -- for S = 3
// those of substep 0 of the next step, from the next stage `nst` (valid once
// the barrier before substep 3 has passed).  The next substep's weights are
// scaled at the end, behind the MFMAs.  (8-bit codes are decoded and scaled
// here, from the step's registers.)
template <int S, int MTV, int kLora, bool kABf16, int kW>
__device__ __forceinline__ void substep(const char* st, const char* nst, const char* nbst,
                                        int next_step, const Rd& rd,
                                        const StepRegs& cur, StepRegs& nxt, f16x8 (&af)[MT],
                                        f16x8 (&bs)[NT],
                                        f32x16 (&acc)[MT][NT], f32x4& acc_u) {
  f16x8 af_n[MT];
  uint32_t dn[NT][4];
  if constexpr (S < 3) {
    load_a<MTV, kABf16>(st, rd, S + 1, af_n);
    if constexpr (kW < kWI8) lut_lookups(cur, S + 1, rd.lane_off, dn);
  } else {
    load_step_regs<kW>(nbst, next_step, rd, nxt);
    load_a<MTV, kABf16>(nst, rd, 0, af_n);
    if constexpr (kW < kWI8) lut_lookups(nxt, 0, rd.lane_off, dn);
  }
  // LoRA: u[this wave's 16 rows][16 ranks] += X A_e^T, k half S - 1
  if constexpr (kLora != kLoraNone && (S == 1 || S == 2)) {
    constexpr int s2 = S - 1;
    u32x4 l = *reinterpret_cast<const u32x4*>(st + OFF_L + rd.ul + s2 * 64);
    if constexpr (kLora == kLoraBF16) l = bf16x8_to_f16x8(l);
    u32x4 v = *reinterpret_cast<const u32x4*>(st + rd.ua[s2]);
    if constexpr (kABf16) v = bf16x8_to_f16x8(v);
    acc_u = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(v), as_f16x8(l), acc_u, 0, 0, 0);
  }
  f16x8 bf[NT];
  if constexpr (kW >= kWI8) {
    decode_b8<kW, S>(cur, bf);
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bf[nt] = bs[nt];
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt)
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[nt], af[mt], acc[mt][nt], 0, 0, 0);
#pragma unroll
  for (int mt = 0; mt < MTV; ++mt) af[mt] = af_n[mt];
  // the next substep's weights scaled now, behind this substep's MFMAs, so
  // that its first MFMA does not wait on the multiplies
  if constexpr (kW < kWI8) {
    if constexpr (S < 3) scale_b(cur, dn, bs);
    else scale_b(nxt, dn, bs);
  }
}

// The k-loop of one tile.  Batch kb holds the copies that step kb issues,
// in this order:
//   activations of step kb + 2 into A stage kb % 2;
//   odd kb: codes of pair (kb + 3) / 2 into that pair stage;
//   kb % 4 == 1: absmax group (kb + 3) / 4 -- buffer ((kb + 3) / 4) & 1 last
//     served steps kb - 5 .. kb - 2, whose reads ended at the barrier of kb - 2.
// The activations go out right after the barrier of step kb (every wave is
// done reading step kb's activations).  For 4-bit codes the code and absmax
// copies of batch kb go out during step kb + 1 instead, two code copies
// after substep 0 and two (and the absmax) after substep 1, so that the
// eight waves do not all queue their copies at the barrier while their
// MFMAs wait behind them; their targets were last read before the barrier
// of step kb (pair stage) or kb - 2 (absmax), and they still complete in
// issue order before batch kb + 1.  The 8-bit and MXFP4 paths issue each
// batch whole after the barrier.
// Before substep 3 of step kb the activations of step kb + 1 (batch kb - 1,
// issued first in it) must have landed: at most the copies issued after them
// in batch kb - 1 may be pending -- 4 when kb - 1 is odd, +1 when it carried
// an absmax group; anything older (codes and absmax needed by step kb + 1,
// issued two or more steps earlier) has landed with them, since copies
// complete in order.  Pairs and activations are issued at least one full
// step before use, codes and absmax two.  Nothing past the last step, pair
// or group is fetched (only the prologue repeats the last ones, when K has
// one or two steps); batches from kb = last - 2 on may therefore carry
// fewer copies than the counts assume, so the last three steps drain all
// copies instead -- theirs were issued a step or more earlier.  The tile
// then ends with no copy in flight.
template <int MTV, int kLora, bool kABf16, int kW>
__device__ __forceinline__ void kloop(const Src& src, int nk, const Rd& rd, int wave, int lane,
                                      bool early, f32x16 (&acc)[MT][NT],
                                      f32x4& acc_u) {
  constexpr int NA = kDmaA<kLora>();
  const uint32_t ring = lds_addr(g_ring);
  const int last = nk - 1;
  const int last_pair = last >> 1;
  // prologue: absmax group 0, pair 0 (unless issued early, under the
  // previous tile's epilogue), activations of steps 0 and 1, pair 1 -- as if
  // batch -1 (odd, activations then a pair) were the last one issued
  if (!early) {
    issue_abs(src, 0, 0, wave);
    issue_b(src, 0, ring + OFF_BR, wave);
  }
  issue_a<kLora>(src, 0, ring, wave);
  issue_a<kLora>(src, min(1, last), ring + ASTAGE, wave);
  // 8-bit codes: one step per stage (64 bytes of a row), not a step pair
  issue_b(src, kW >= kWI8 ? min(1, last) : min(1, last_pair), ring + OFF_BR + BPAIR, wave);

  // absmax group 0, pair 0 and step 0's activations complete
  wait_vm_barrier<NA + kDmaB>();
  StepRegs cur, nxt;
  f16x8 af[MT];
  f16x8 bs[NT];
  load_step_regs<kW>(g_ring + OFF_BR, 0, rd, cur);
  load_a<MTV, kABf16>(g_ring, rd, 0, af);
  if constexpr (kW < kWI8) {
    uint32_t d[NT][4];
    lut_lookups(cur, 0, rd.lane_off, d);
    scale_b(cur, d, bs);
  }
  for (int kb = 0; kb < nk; ++kb) {
    const int a = kb & 1;
    const char* sp = g_ring + a * ASTAGE;              // step kb's activations
    const char* np = g_ring + (a ^ 1) * ASTAGE;        // step kb + 1's
    const char* nbp = g_ring + OFF_BR +
                      ((kW >= kWI8 ? (kb + 1) : ((kb + 1) >> 1)) & 1) * BPAIR;  // kb + 1's codes
    // 4-bit codes: the code and absmax copies of batch kb - 1
    const int pb = kb - 1;
    const int ppn = (pb + 3) >> 1;
    const bool defer_b = kW == kW4 && kb >= 1 && (pb & 1) && ppn <= last_pair;
    substep<0, MTV, kLora, kABf16, kW>(sp, np, nbp, kb + 1, rd, cur, nxt, af, bs, acc, acc_u);
    if (defer_b) issue_b_half(src, ppn, ring + OFF_BR + (ppn & 1) * BPAIR, wave, 0);
    substep<1, MTV, kLora, kABf16, kW>(sp, np, nbp, kb + 1, rd, cur, nxt, af, bs, acc, acc_u);
    if (defer_b) issue_b_half(src, ppn, ring + OFF_BR + (ppn & 1) * BPAIR, wave, 1);
    if constexpr (kW == kW4) {
      if (kb >= 1 && (pb & 3) == 1) {
        const int grp = (pb + 3) >> 2;
        if (grp <= (last >> 2)) issue_abs(src, grp, grp & 1, wave);
      }
    }
    substep<2, MTV, kLora, kABf16, kW>(sp, np, nbp, kb + 1, rd, cur, nxt, af, bs, acc, acc_u);
    if (kb >= last - 2) {
      // the batches of the last steps skip every copy past the end, so the
      // counts below no longer describe them: drain
      wait_vm_barrier<0>();
    } else if constexpr (kW >= kWI8) {
      // 8-bit codes: every batch carries the next step's codes and
      // activations, both needed now
      wait_vm_barrier<0>();
    } else if constexpr (kW == kWMx) {
      // MXFP4 scale groups cover 8 steps: batch kb - 1 carried one when it
      // was 5 mod 8
      if (kb & 1) wait_vm_barrier<0>();
      else if ((kb & 7) == 6) wait_vm_barrier<kDmaB + kDmaAbs>();
      else wait_vm_barrier<kDmaB>();
    } else {
      switch (kb & 3) {
        case 0: wait_vm_barrier<kDmaB>(); break;             // batch kb - 1 = 3 mod 4
        case 2: wait_vm_barrier<kDmaB + kDmaAbs>(); break;   // batch kb - 1 = 1 mod 4
        default: wait_vm_barrier<0>(); break;                // batch kb - 1 even
      }
    }
    // nothing past the last step, pair or group is fetched: the tile's
    // last wait then has no copy left in flight
    if (kb + 2 <= last) issue_a<kLora>(src, kb + 2, ring + a * ASTAGE, wave);
    if constexpr (kW >= kWI8) {
      if (kb + 2 <= last) issue_b(src, kb + 2, ring + OFF_BR + a * BPAIR, wave);
      if ((kb & 3) == 1) {
        const int grp = (kb + 3) >> 2;
        if (grp <= (last >> 2)) issue_abs(src, grp, grp & 1, wave);
      }
    } else if constexpr (kW == kWMx) {
      if (kb & 1) {
        const int pn = (kb + 3) >> 1;
        if (pn <= last_pair) issue_b(src, pn, ring + OFF_BR + (pn & 1) * BPAIR, wave);
        if ((kb & 7) == 5) {
          const int grp = (kb + 3) >> 3;
          if (grp <= (last >> 3)) issue_abs(src, grp, grp & 1, wave);
        }
      }
    }
    substep<3, MTV, kLora, kABf16, kW>(sp, np, nbp, kb + 1, rd, cur, nxt, af, bs, acc, acc_u);
    cur = nxt;
  }
}

}  // namespace

template <bool kSwiglu, int kLora, bool kABf16, int kOut, int kW, bool kBwd = false>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_gemm_kernel(GemmArgs g, int n_tiles) {
  static_assert(!kBwd || kSwiglu, "the SwiGLU backward pairs gate and up rows like SwiGLU");
  constexpr bool kMx = kW == kWMx;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;  // column of a B operand / row of an A operand
  const int g2 = lane >> 5;   // k half of the operands
  const int c16 = lane & 15, g4 = lane >> 4;  // 16x16x32 operand coordinates

  if constexpr (kMx)
    lut_fill<kCopies>(g_lut, g_lstage, c_levels_gemm_mx, tid, NTHREADS, /*low_first=*/true);
  else if constexpr (kW >= kWI8)
    __syncthreads();  // 8-bit codes decode without the table
  else
    lut_fill<kCopies>(g_lut, g_lstage, g.qtype == kQtFP4 ? c_levels_gemm_fp4 : c_levels_gemm,
                      tid, NTHREADS);

  build_tile_table<NTHREADS, BM>(g.offsets, g.E, g_tiles, g_wsum, tid);

  const int N = g.N;
  const int K = g.K;
  const int I = N >> 1;  // SwiGLU: output columns
  const int nk = K / BK;
  // adapter rows of B_e load as one 16-byte vector per 8 ranks
  const bool lora_vec = (g.lora_r & 7) == 0 && (reinterpret_cast<uintptr_t>(g.lora_b) & 15) == 0;

  Rd rd;
#pragma unroll
  for (int s = 0; s < 4; ++s) rd.a[s] = n32 * 128 + (((g2 * 4 + s) ^ ((n32 >> 1) & 7)) << 4);
  // pair stage: weight row l's 64 bytes hold steps 2p (chunks 0, 1) and
  // 2p + 1 (chunks 2, 3), 16-byte chunk c at c ^ ((l >> 2) & 3), so 16
  // consecutive rows cover all 64 banks
#pragma unroll
  for (int sp2 = 0; sp2 < 2; ++sp2)
    rd.b[sp2] = (wave * BNW + n32) * 64 + (((sp2 * 2 + g2) ^ ((n32 >> 2) & 3)) << 4);
  // 8-bit stage: weight row l's 64 bytes of one step, chunk c at c ^ ((l >> 2) & 3)
#pragma unroll
  for (int i = 0; i < 2; ++i)
    rd.b8[i] = (wave * BNW + n32) * 64 + (((2 * g2 + i) ^ ((n32 >> 2) & 3)) << 4);
  // absmax element (fp32 index) of n-tile 0's row; MXFP4: its scale byte of
  // k half g2 (16 bytes per row: 8 steps x 2 halves)
  rd.s = kMx ? (wave * BNW + n32) * 16 + g2 : (wave * BNW + n32) * kAbsGroup;
  // LoRA operands of 16x16x32: A row c16 of this wave's 16 rows and k chunk
  // 4*s2 + g4 (swizzled like the main fragments); A_e row c16, same k
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int row = wave * 16 + c16;
    rd.ua[s2] = row * 128 + (((4 * s2 + g4) ^ ((row >> 1) & 7)) << 4);
  }
  rd.ul = c16 * 128 + g4 * 16;
  rd.lane_off = (uint32_t)(lane & 31) * 4u;

  // weight row of LDS B row l (0..511) of N-tile n_idx, clamped to a valid
  // row.  SwiGLU: wave w's n-tile 0 holds the gate rows and n-tile 1 the up
  // rows of output columns n_idx*256 + 32w + [0, 32).
  auto weight_row = [&](int l, int n_idx) -> int {
    const int w = l / BNW, nt = (l >> 5) % NT, n = l & 31;
    int row;
    if constexpr (kSwiglu) {
      const int col = n_idx * 256 + w * 32 + n;
      row = (col < I ? col : I - 1) + (nt == 1 ? I : 0);
    } else {
      const int col = n_idx * 512 + w * BNW + nt * 32 + n;
      row = col < N ? col : N - 1;
    }
    return row;
  };

  const i32x4 a_rsrc = make_rsrc(g.a, (uint32_t)(g.a_rows * (int64_t)K * 2));
  const int total = __builtin_amdgcn_readfirstlane(g_tiles[g.E]) * n_tiles;
  const int G = gridDim.x;  // a multiple of 8
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  // A last, partial round of rem <= G/2 tiles would leave most workgroups
  // idle while the others finish: its tiles are split into two 64-row
  // halves (the same weights, half the rows each), one per workgroup.
  const int q = total / G, rem = total - q * G;
  const bool split_tail = rem > 0 && 2 * rem <= G;
  // Tile r of this workgroup: expert, N-tile, first row, valid rows.
  struct Tile {
    int e, n_idx, row0, rows_valid, mtv;
  };
  auto find_tile = [&](int r, Tile& t) -> bool {
    const int u = xcd * (G >> 3) + pos;  // position within the round
    int tix, half = -1;
    if (split_tail && r == q) {
      if (u >= 2 * rem) return false;
      tix = q * G + (u >> 1);
      half = u & 1;
    } else {
      tix = r * G + u;
      if (tix >= total) return false;
    }
    const int mt_global = tix / n_tiles;
    t.n_idx = tix - mt_global * n_tiles;
    int lo = 0, hi = g.E;  // g_tiles[lo] <= mt_global < g_tiles[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g_tiles[mid] <= mt_global) lo = mid; else hi = mid;
    }
    t.e = __builtin_amdgcn_readfirstlane(lo);
    const int m_local = mt_global - __builtin_amdgcn_readfirstlane(g_tiles[t.e]);
    t.row0 = __builtin_amdgcn_readfirstlane(g.offsets[t.e]) + m_local * BM;
    t.rows_valid = min(BM, __builtin_amdgcn_readfirstlane(g.offsets[t.e + 1]) - t.row0);
    if (half >= 0) {
      t.row0 += half * (BM / 2);
      t.rows_valid = min(BM / 2, t.rows_valid - half * (BM / 2));
      if (t.rows_valid <= 0) return false;  // the tile's rows fit its first half
    }
    t.mtv = (t.rows_valid + 31) >> 5;
    return true;
  };

  // The copy sources of a tile.
  auto make_src = [&](const Tile& t) -> Src {
    const int e = t.e, n_idx = t.n_idx, row0 = t.row0, rows_valid = t.rows_valid;
    Src src;
    src.a_rsrc = a_rsrc;
    const uint32_t brow = kW >= kWI8 ? (uint32_t)K : (uint32_t)(K / 2);  // code bytes per row
    const uint32_t b_bytes = (uint32_t)N * brow;
    const uint32_t s_bytes = kMx ? (uint32_t)N * (uint32_t)(K / 32) : (uint32_t)N * (uint32_t)nk * 4u;
    src.b_rsrc = make_rsrc(reinterpret_cast<const char*>(g.packed) + (int64_t)e * b_bytes, b_bytes);
    src.s_rsrc = make_rsrc(reinterpret_cast<const char*>(g.absmax) + (int64_t)e * s_bytes, s_bytes);
    // A: wave instruction i covers LDS chunks [64 j, 64 j + 64) = rows
    // 8j..8j+7, j = 2 wave + i
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = (wave * 2 + i) * 64 + lane;
      const int row = c >> 3;
      const int gchunk = (c & 7) ^ ((row >> 1) & 7);
      const int rr = row < rows_valid ? row : 0;
      const int idx = row0 + rr;
      const uint32_t a_src = g.gather ? (uint32_t)(g.gather[idx] / g.gather_div) : (uint32_t)idx;
      src.a_off[i] = (a_src * (uint32_t)K + gchunk * 8) * 2;
    }
    // packed codes of a step pair: wave instruction i covers pair-stage
    // rows [16 j, 16 j + 16), four 16-B chunks each, j = 4 wave + i; the
    // chunk at position q of row l is chunk q ^ ((l >> 2) & 3) of the row's
    // 64 bytes (steps 2p, 2p + 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int l = (wave * 4 + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((l >> 2) & 3);
      src.b_off[i] = (uint32_t)weight_row(l, n_idx) * brow + c * 16;
    }
    // absmax groups: the wave's instruction covers rows [64 wave, 64 wave +
    // 64), 16 bytes (kAbsGroup steps) per row
    src.s_off = (uint32_t)weight_row(wave * 64 + lane, n_idx) *
                (kMx ? (uint32_t)(K / 32) : (uint32_t)nk * 4u);
    if constexpr (kLora != kLoraNone) {
      const uint32_t l_bytes = (uint32_t)g.lora_r * (uint32_t)K * 2u;
      src.l_rsrc = make_rsrc(reinterpret_cast<const char*>(g.lora_a) + (int64_t)e * l_bytes, l_bytes);
      // LoRA A: 16 rows x 128 B per step; dword d of the block is row d / 32
      const int d = wave * 64 + lane;
      const int rho = d >> 5;
      const int rc = rho < g.lora_r ? rho : 0;
      src.l_off = (uint32_t)rc * (uint32_t)K * 2u + (uint32_t)(d & 31) * 4u;
    } else {
      src.l_rsrc = i32x4{0, 0, 0, 0};
      src.l_off = 0;
    }

    return src;
  };

  // The epilogue stages its output in the A stages only (for 16-bit
  // outputs, and 32-bit SwiGLU ones): the next tile's absmax group 0 and
  // code pair 0 are then copied in under the epilogue.
  // (The SwiGLU backward stages fp32 gate, then up, of its 32 columns.)
  constexpr int kStageBytes =
      kBwd ? NWAVES * 32 * (BNW / 2 * 4 + 16)
           : NWAVES * 32 * ((kSwiglu ? BNW / 2 : BNW) * (kOut == kF32 ? 4 : 2) + 16);
  constexpr bool kEarly = kStageBytes <= OFF_BR && kLora == kLoraNone;

  // (the found flags are made wave-uniform explicitly: the copy sources
  // below must stay in scalar registers)
  Tile tile;
  bool have = __builtin_amdgcn_readfirstlane((int)find_tile(0, tile)) != 0;
  bool early = false;  // this tile's absmax group 0 and pair 0 are issued
  for (int r = 0; have; ++r) {
    const int e = tile.e, n_idx = tile.n_idx, row0 = tile.row0, rows_valid = tile.rows_valid;
    const int mtv = tile.mtv;
    const Src src = make_src(tile);
    // output row and row scale of every tile row, for the epilogue
    const int par = r & 1;
    if (tid < BM) {
      const int grow = row0 + (tid < rows_valid ? tid : 0);
      g_orow[par][tid] = g.scatter ? g.scatter[grow] : grow;
      g_rscale[par][tid] = g.row_scale ? g.row_scale[grow] : 1.0f;
    }

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.f;
    f32x4 acc_u = f32x4{0.f, 0.f, 0.f, 0.f};

    // every wave is done with the previous tile's stages (and LoRA exchange)
    lds_barrier();
    switch (mtv) {
      case 1: kloop<1, kLora, kABf16, kW>(src, nk, rd, wave, lane, early, acc, acc_u); break;
      case 2: kloop<2, kLora, kABf16, kW>(src, nk, rd, wave, lane, early, acc, acc_u); break;
      case 3: kloop<3, kLora, kABf16, kW>(src, nk, rd, wave, lane, early, acc, acc_u); break;
      default: kloop<4, kLora, kABf16, kW>(src, nk, rd, wave, lane, early, acc, acc_u); break;
    }
    // SwiGLU backward: dh of every m-tile of the tile, two items of 8
    // columns per lane and m-tile (the epilogue's row layout), loaded before
    // the final wait so their latency is paid once per tile
    u32x4 dq[kBwd ? MT : 1][2];
    if constexpr (kBwd) {
      const _Float16* dh = reinterpret_cast<const _Float16*>(g.dh);
      const int cbase = n_idx * 256 + wave * (BNW / 2);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int idx = it * 64 + lane;
          const int row = mt * 32 + (idx >> 2);
          const int col = cbase + (idx & 3) * 8;
          dq[mt][it] = u32x4{0u, 0u, 0u, 0u};
          if (row < rows_valid && col < I)
            dq[mt][it] = *reinterpret_cast<const u32x4*>(dh + (int64_t)(row0 + row) * I + col);
        }
    }
    // LoRA B_e: ranks 8 g2 .. 8 g2 + 7 of this lane's weight row in each
    // n-tile (zero past r), loaded before the final wait so their latency
    // overlaps it; one 16-byte load when the rows are 16-byte aligned
    f16x8 bl2[NT];
    if constexpr (kLora != kLoraNone) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int l = wave * BNW + nt * 32 + n32;
        const uint16_t* lb = reinterpret_cast<const uint16_t*>(g.lora_b) +
                             ((int64_t)e * N + weight_row(l, n_idx)) * g.lora_r;
        if (lora_vec) {
          u32x4 raw = u32x4{0u, 0u, 0u, 0u};
          if (g2 * 8 < g.lora_r) raw = *reinterpret_cast<const u32x4*>(lb + g2 * 8);
          if constexpr (kLora == kLoraBF16) raw = bf16x8_to_f16x8(raw);
          bl2[nt] = as_f16x8(raw);
        } else {
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            const int rho = g2 * 8 + tt;
            _Float16 hv = (_Float16)0.f;
            if (rho < g.lora_r) {
              const uint16_t raw = lb[rho];
              if constexpr (kLora == kLoraBF16) hv = (_Float16)bf16_bits_to_f32(raw);
              else hv = __builtin_bit_cast(_Float16, raw);
            }
            bl2[nt][tt] = hv;
          }
        }
      }
    }
    // every copy has landed and every wave is done with the ring: the
    // epilogue stages its output there
    wait_vm_barrier<0>();

    // the next tile; its first absmax group and code pair go out now
    Tile next;
    const bool have_next = __builtin_amdgcn_readfirstlane((int)find_tile(r + 1, next)) != 0;
    early = kEarly && have_next;
    if (early) {
      const Src ns = make_src(next);
      issue_abs(ns, 0, 0, wave);
      issue_b(ns, 0, lds_addr(g_ring) + OFF_BR, wave);
    }

    // ---- LoRA: G += (scale * u) B_e^T, u exchanged between the waves in fp16
    if constexpr (kLora != kLoraNone) {
      // 16x16 accumulator layout: lane holds rank c16 of rows 4*g4 + i.
      // Ranks c16 >= r multiplied a stand-in row of A_e (the copies clamp
      // to row 0): they are stored as zero.
#pragma unroll
      for (int i = 0; i < 4; ++i)
        u_buf()[(wave * 16 + g4 * 4 + i) * kMaxLoraR + c16] =
            c16 < g.lora_r ? (_Float16)(acc_u[i] * g.lora_scale) : (_Float16)0.f;
      // training recompute: the projection u = X A_e^T itself (fp32, without
      // the scale) for the adapter's weight gradients, written once per
      // M-tile, by its first N-tile
      if constexpr (kBwd) {
        if (g.u_out != nullptr && n_idx == 0 && c16 < g.lora_r) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = wave * 16 + g4 * 4 + i;
            if (row < rows_valid) g.u_out[(int64_t)(row0 + row) * g.lora_r + c16] = acc_u[i];
          }
        }
      }
      lds_barrier();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f16x8 au = *reinterpret_cast<const f16x8*>(&u_buf()[(mt * 32 + n32) * kMaxLoraR + g2 * 8]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bl2[nt], au, acc[mt][nt], 0, 0, 0);
      }
    }

    // ---- SwiGLU backward (training): out = [dh*up*silu'(gate) | dh*silu(gate)]
    // for the gate and up pre-activations of this tile, with dh the
    // upstream gradient of h (fp16 [P, I], row i = tile row i), so the
    // pre-activations never leave the chip.  Each wave stages its m-tile's
    // gate values in fp32 in a private LDS region, reads them back as 8
    // consecutive columns of one row per item (two items per lane), then
    // does the same for up; dh was loaded in that row layout before the
    // tile's final wait.  No row scale applies.  Optionally h = silu(gate)
    // * up too (fp16 [P, I]), for the down adapter's gradients.
    if constexpr (kBwd) {
      constexpr int PITCH = BNW / 2 * 4 + 16;
      static_assert(NWAVES * 32 * PITCH == kStageBytes, "staging size as assumed");
      char* ws = g_ring + wave * 32 * PITCH;
      const int cbase = n_idx * 256 + wave * (BNW / 2);
      char* prow = ws + n32 * PITCH;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt >= mtv) continue;
        float gate[2][8], up[2][8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float v[4] = {acc[mt][half][4 * jj], acc[mt][half][4 * jj + 1],
                                acc[mt][half][4 * jj + 2], acc[mt][half][4 * jj + 3]};
            stage_out4<kF32>(prow + (8 * jj + 4 * g2) * 4, v);
          }
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const int idx = it * 64 + lane;
            const char* src = ws + (idx >> 2) * PITCH + (idx & 3) * 32;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
            float* dst = half == 0 ? gate[it] : up[it];
            dst[0] = lo.x; dst[1] = lo.y; dst[2] = lo.z; dst[3] = lo.w;
            dst[4] = hi.x; dst[5] = hi.y; dst[6] = hi.z; dst[7] = hi.w;
          }
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int idx = it * 64 + lane;
          const int row = mt * 32 + (idx >> 2);
          const int col = cbase + (idx & 3) * 8;
          if (row < rows_valid && col < I) {
            float d[8];
            unpack8<false>(dq[mt][it], d);
            float dg[8], du[8], hv[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const float z = gate[it][t];
              const float sg = sigmoid_f(z);
              const float si = z * sg;
              dg[t] = d[t] * up[it][t] * (sg * (1.0f + z * (1.0f - sg)));
              du[t] = d[t] * si;
              hv[t] = si * up[it][t];
            }
            const int64_t orow = g_orow[par][row];
            store8<kOut>(g.out, orow * 2 * I + col, dg);
            store8<kOut>(g.out, orow * 2 * I + I + col, du);
            if (g.h_out != nullptr) store8<kF16>(g.h_out, orow * I + col, hv);
          }
        }
      }
    } else
    // ---- epilogue: SwiGLU, row scale, conversion to the output dtype, then
    // coalesced stores.  Each wave stages its 32-row slices of the tile in a
    // private LDS region (rows of COLS values, padded by 16 bytes) and stores
    // them as 16-byte row chunks, scattered to their output rows.
    // The MFMAs take the weights as their first operand, so an accumulator
    // tile is the transposed output block: lane holds output row (lane & 31)
    // of the m-tile and, for j = 0..15, output column
    // 8*(j/4) + 4*(lane/32) + (j%4) of the n-tile -- four consecutive columns
    // per j/4, one 8-byte (16-byte for fp32) LDS write.
    {
      constexpr int ESZ = kOut == kF32 ? 4 : 2;
      constexpr int COLS = kSwiglu ? BNW / 2 : BNW;  // output columns of this wave
      constexpr int PITCH = COLS * ESZ + 16;
      constexpr int CPR = COLS * ESZ / 16;          // 16-byte chunks per row
      constexpr int EPC = 16 / ESZ;                 // elements per chunk
      static_assert(NWAVES * 32 * PITCH <= RING, "staging fits the ring");
      static_assert(NWAVES * 32 * PITCH == kStageBytes, "staging size as assumed");
      char* ws = g_ring + wave * 32 * PITCH;
      const int ncols = kSwiglu ? I : N;
      const int cbase = kSwiglu ? n_idx * 256 + wave * (BNW / 2) : n_idx * BN + wave * BNW;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt >= mtv) continue;
        const float rs = g_rscale[par][mt * 32 + n32];
        char* prow = ws + n32 * PITCH;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          constexpr int NTO = kSwiglu ? NT / 2 : NT;  // output n-tiles of this wave
#pragma unroll
          for (int nt = 0; nt < NTO; ++nt) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 4 * jj + i;
              if constexpr (kSwiglu)
                v[i] = silu_f(acc[mt][nt][j]) * acc[mt][nt + NTO][j] * rs;
              else
                v[i] = acc[mt][nt][j] * rs;
            }
            stage_out4<kOut>(prow + (nt * 32 + 8 * jj + 4 * g2) * ESZ, v);
          }
        }
#pragma unroll
        for (int it = 0; it < CPR / 2; ++it) {
          const int idx = it * 64 + lane;
          const int rr = idx / CPR, c = idx % CPR;
          const u32x4 v = *reinterpret_cast<const u32x4*>(ws + rr * PITCH + c * 16);
          const int row = mt * 32 + rr;
          const int col = cbase + c * EPC;
          if (row < rows_valid && col < ncols) {
            const int64_t orow = g_orow[par][row];
            *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(g.out) +
                                      (orow * ncols + col) * ESZ) = v;
          }
        }
      }
    }
    tile = next;
    have = have_next;
  }
  // no memory operation of the wave is left in flight when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool kSwiglu, int kLora, bool kABf16, int kW>
static void launch_out(const GemmArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  switch (g.out_dtype) {
    case kF32:
      hipLaunchKernelGGL((grouped_gemm_kernel<kSwiglu, kLora, kABf16, kF32, kW>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
    case kBF16:
      hipLaunchKernelGGL((grouped_gemm_kernel<kSwiglu, kLora, kABf16, kBF16, kW>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
    default:
      hipLaunchKernelGGL((grouped_gemm_kernel<kSwiglu, kLora, kABf16, kF16, kW>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
  }
}

// The layer backward's recompute with the SwiGLU backward in its epilogue:
// fp16 activations and fp16 output only.
template <int kLora>
static void launch_bwd(const GemmArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_kernel<true, kLora, false, kF16, kW4, true>), grid,
                     dim3(NTHREADS), 0, s, g, n_tiles);
}

template <bool kSwiglu, int kLora, int kW = kW4>
static void launch_a(const GemmArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  if (g.a_bf16) launch_out<kSwiglu, kLora, true, kW>(g, grid, n_tiles, s);
  else launch_out<kSwiglu, kLora, false, kW>(g, grid, n_tiles, s);
}

hipError_t launch_grouped_gemm(const GemmArgs& g, int num_cus, hipStream_t stream) {
  const int n_tiles = g.swiglu ? (g.N / 2 + 255) / 256 : (g.N + 511) / 512;
  // persistent: one workgroup per CU (a multiple of 8 for the XCD ordering)
  int grid = (num_cus + 7) / 8 * 8;
  const int64_t max_tiles = ((g.P + BM - 1) / BM + g.E) * n_tiles;
  if ((int64_t)grid > max_tiles) grid = (int)((max_tiles + 7) / 8 * 8);
  if (grid < 8) grid = 8;
  const dim3 dg((unsigned)grid);
  const bool lora = g.lora_a != nullptr;
  // no adapters on MXFP4 or 8-bit stacks (checked by the caller)
  if (g.qtype == kQtMXFP4) {
    if (g.swiglu) launch_a<true, kLoraNone, kWMx>(g, dg, n_tiles, stream);
    else launch_a<false, kLoraNone, kWMx>(g, dg, n_tiles, stream);
    return hipGetLastError();
  }
  if (g.qtype == kQtINT8 || g.qtype == kQtFP8) {
    if (g.qtype == kQtINT8) {
      if (g.swiglu) launch_a<true, kLoraNone, kWI8>(g, dg, n_tiles, stream);
      else launch_a<false, kLoraNone, kWI8>(g, dg, n_tiles, stream);
    } else {
      if (g.swiglu) launch_a<true, kLoraNone, kWF8>(g, dg, n_tiles, stream);
      else launch_a<false, kLoraNone, kWF8>(g, dg, n_tiles, stream);
    }
    return hipGetLastError();
  }
  const int kind = !lora ? kLoraNone : g.lora_bf16 ? kLoraBF16 : kLoraF16;
  if (g.dh != nullptr) {
    if (kind == kLoraBF16) launch_bwd<kLoraBF16>(g, dg, n_tiles, stream);
    else if (kind == kLoraF16) launch_bwd<kLoraF16>(g, dg, n_tiles, stream);
    else launch_bwd<kLoraNone>(g, dg, n_tiles, stream);
    return hipGetLastError();
  }
  if (g.swiglu) {
    if (kind == kLoraBF16) launch_a<true, kLoraBF16>(g, dg, n_tiles, stream);
    else if (kind == kLoraF16) launch_a<true, kLoraF16>(g, dg, n_tiles, stream);
    else launch_a<true, kLoraNone>(g, dg, n_tiles, stream);
  } else {
    if (kind == kLoraBF16) launch_a<false, kLoraBF16>(g, dg, n_tiles, stream);
    else if (kind == kLoraF16) launch_a<false, kLoraF16>(g, dg, n_tiles, stream);
    else launch_a<false, kLoraNone>(g, dg, n_tiles, stream);
  }
  return hipGetLastError();
}

}  // namespace nf4moe
