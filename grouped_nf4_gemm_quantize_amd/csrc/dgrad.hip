// Grouped NF4 dgrad on CDNA4 matrix cores: the backward of the grouped GEMM
// with respect to its input, through the frozen packed stack.
//
// One launch computes, for every expert e and each of its rows i,
//   out[i, :] = row_scale(i) * a[src(i), :] . W_e      (W_e = dequant [N, K])
// so it contracts over the N rows of the stack, along which the 64-element
// absmax blocks do NOT run; nothing dequantised is written to memory.  This
// is the single-launch dgrad of the fused training path (experts4bit-qlora
// 0.22.0 README, "Which training path?", dgrad=True), which replaced a
// per-expert decode loop and materialises no expert weights; the frozen
// projections are decoded again from the packed bytes inside backward
// (README "Training + expert offload").
//
// Work decomposition (gfx950, wave64, v_mfma_f32_32x32x16_f16):
//   A tile = 128 rows of ONE expert x 512 output columns (k).  Eight waves,
//   two per SIMD; wave w owns the 64 output columns of one absmax block
//   (2 n-tiles of 32) against all 128 rows (4 m-tiles), 128 fp32
//   accumulators per lane.  The contraction advances 64 stack rows (n) per
//   step, in four MFMA substeps of 16.
//
// The transposed decode.  An MFMA operand lane holds 8 consecutive
// contraction values of one output column: 8 nibbles from 8 different stack
// rows.  Eight lanes that need the same 8 rows and 8 adjacent columns each
// read the 32-bit code word of one of the rows (the 8 columns), and an 8x8
// nibble transpose across the 8 lanes -- three exchange stages on DPP lane
// moves (lanes 4, 2, 1 apart; 16-bit, 8-bit and 4-bit fields) with one bit
// select each -- leaves every lane with its own column's 8 codes, already in
// the byte order the decode table takes: byte m = (code of row 2m) << 4 |
// code of row 2m + 1.  Each byte then goes through the LDS byte -> half2
// table (one ds_read_b32) and one v_pk_mul_f16 by the pair of the two rows'
// absmax.  Because a wave's 64 columns are one absmax block, the wave needs
// one absmax per stack row and step; each lane converts one to fp16 and
// parks it in a per-wave LDS slot, from which a substep reads its 8 rows'
// scales in one 16-byte read.
//
// Operand staging: direct-to-LDS buffer loads into a 3-stage ring, up to
// three steps ahead, the same five copies per wave and step:
//   A (gradient rows, fp16/bf16): 128 rows x 128 B, 16-byte chunk c of row r
//     at chunk c ^ ((r >> 1) & 7) (as in the forward kernel);
//   B (codes): 64 stack rows x 256 B (the tile's 512 columns), 16-byte chunk
//     c of row n at c ^ f(n), f(n) = (n & 7) | 8 * ((n >> 5) & 1): the 64
//     lanes of one code-word read (16 rows, 4 words) hit 64 different banks;
//   S (absmax): [64 rows][the tile's 8 blocks] fp32, one 4-byte copy per
//     wave (8 rows x 32 contiguous bytes: 8 row segments per copy).
// The kernel waits with a counted s_waitcnt on the vector-memory counter
// (copies complete in issue order) and s_barrier, as the forward kernel.
//
// Epilogues: optional per-expert LoRA rank-r term out += scale * v_i . A_e
// (v = the rows' projections onto the adapter's B, one more MFMA per
// accumulator tile), row scale, and either a plain store (with an optional
// scatter of the rows) or the SwiGLU backward: with the forward's
// pre-activation g = [gate | up] of the same row, the output row is
// [dh * up * silu'(gate) | dh * silu(gate)] (2K columns).  v is either
// precomputed or, with the plain epilogue, computed in the k-loop from the
// rows this kernel reads anyway (a 16x16x32 MFMA per k half of a step on
// each wave's 16 rows and a sixth copy per wave and step, B^T's 16 ranks x
// 64 stack rows), exchanged between the waves through LDS and written out
// for the adapter's weight gradients.

#include "common.h"
#include "launch.h"
#include "mfma_common.h"

namespace nf4moe {

__constant__ float c_levels_dgrad[16] = NF4MOE_LEVELS_INIT;
__constant__ float c_levels_dgrad_fp4[16] = NF4MOE_FP4_LEVELS_INIT;

namespace {

constexpr int BM = kGemmBM;        // 128 rows per M-tile
constexpr int BK = 64;             // stack rows (contraction) per step
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int MT = BM / 32;        // 4 m-tiles
constexpr int NT = 2;              // 2 n-tiles of 32 output columns per wave
constexpr int BNW = NT * 32;       // 64 output columns per wave = one absmax block
constexpr int BN = NWAVES * BNW;   // 512 output columns per tile
constexpr int kCopies = 32;
constexpr int OFF_A = 0;                        // 128 rows x 128 B
constexpr int OFF_B = BM * BK * 2;              // 64 stack rows x 256 B
constexpr int OFF_S = OFF_B + BK * (BN / 2);    // [64 rows][8 blocks] fp32
constexpr int OFF_L = OFF_S + NWAVES * BK * 4;  // adapter B^T: [16 ranks][64 stack rows] fp16
constexpr int STAGE = OFF_L + kMaxLoraR * BK * 2;  // 36864 B
constexpr int NSTAGE = 3;
constexpr int RING = NSTAGE * STAGE;            // 110592 B
// copies per wave and step (one more with the in-loop adapter projection)
template <bool kVP>
constexpr int kDmaOf() { return kVP ? 6 : 5; }
// the in-loop projection v (fp16, scaled, [BM][16]) at the end of the ring,
// free once the k-loop has drained; the epilogue staging uses the start
constexpr int OFF_V = RING - BM * kMaxLoraR * 2;

}  // namespace

__shared__ __attribute__((aligned(16))) char d_ring[RING];
__shared__ uint32_t d_lut[256 * kCopies];
// fp16 absmax of the wave's block for the 64 stack rows of a step, by step
// parity: d_sc[step & 1][wave][row]
__shared__ __attribute__((aligned(16))) _Float16 d_sc[2][NWAVES][BK];
__shared__ int32_t d_tiles[kMaxExperts + 1];
__shared__ uint16_t d_lstage[16];
__shared__ int32_t d_wsum[NWAVES];
__shared__ int32_t d_orow[2][BM];
__shared__ float d_rscale[2][BM];

namespace {

__device__ __forceinline__ uint32_t dlut_read(uint32_t addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(d_lut) + addr);
}

struct DSrc {
  i32x4 a_rsrc, b_rsrc, s_rsrc, l_rsrc;
  uint32_t a_off[2];  // A: 2 x 16 B per lane
  uint32_t b_off[2];  // codes: 2 x 16 B per lane
  uint32_t s_off;     // absmax: 4 B per lane
  uint32_t l_off;     // adapter B^T rows: 4 B per lane
  uint32_t b_step;    // bytes of 64 stack rows of codes
  uint32_t s_step;    // bytes of 64 stack rows of absmax
};

// The copies of step `kb` (clamped by the caller) into the stage at `st`.
template <bool kVP>
__device__ __forceinline__ void issue_step(const DSrc& s, int kb, uint32_t st, int wave) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    dma16(s.a_rsrc, s.a_off[i], (uint32_t)kb * (BK * 2), st + OFF_A + (wave * 2 + i) * 1024);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    dma16(s.b_rsrc, s.b_off[i], (uint32_t)kb * s.b_step, st + OFF_B + (wave * 2 + i) * 1024);
  dma4(s.s_rsrc, s.s_off, (uint32_t)kb * s.s_step, st + OFF_S + wave * 256);
  if constexpr (kVP) dma4(s.l_rsrc, s.l_off, (uint32_t)kb * (BK * 2), st + OFF_L + wave * 256);
}

// Per-lane constants: LDS read offsets and the transpose's lane masks.
struct DRd {
  uint32_t a[4];      // A fragment of substep s (m-tile 0; + 4096 per m-tile)
  uint32_t b[NT];     // code word of n-tile nt, substep 0 (+ 2048 per substep)
  uint32_t sc;        // this lane's 8 scales of substep 0 in d_sc (+ 16 B per substep)
  uint32_t lane_off;  // decode-table word offset
  uint32_t s1, s2, k3, amt3;
};

// The 8x8 nibble transpose over the 8 lanes of a group (lanes 8j..8j+7):
// lane i enters with the code word of stack row i (8 columns) and leaves
// with the codes of column i for rows 0..7, byte m = row 2m << 4 | row 2m+1.
// Stage 1 exchanges 16-bit halves with the lane 4 away (row_shl:4 into the
// lower quad, row_shr:4 into the upper one), stage 2 bytes with the lane 2
// away -- in both, one byte permute of (partner, own) word keeps the lane's
// own field and moves the partner's into place -- and stage 3 nibbles with
// the neighbouring lane, rotating the word so the partner's field lands
// where it is kept.
__device__ __forceinline__ uint32_t transpose8(uint32_t x, const DRd& rd) {
  // the two masked moves of stage 1 together write every lane (banks 1, 3
  // from 4 lanes down, banks 0, 2 from 4 lanes up), so the first needs no
  // initialised destination
  int p = __builtin_amdgcn_mov_dpp((int)x, 0x114 /* row_shr:4 */, 0xf, 0xa, false);
  p = __builtin_amdgcn_update_dpp(p, (int)x, 0x104 /* row_shl:4 */, 0xf, 0x5, false);
  x = __builtin_amdgcn_perm((uint32_t)p, x, rd.s1);
  p = __builtin_amdgcn_mov_dpp((int)x, 0x4e /* quad_perm [2,3,0,1] */, 0xf, 0xf, false);
  x = __builtin_amdgcn_perm((uint32_t)p, x, rd.s2);
  const uint32_t y = __builtin_amdgcn_alignbit(x, x, rd.amt3);
  p = __builtin_amdgcn_mov_dpp((int)y, 0xb1 /* quad_perm [1,0,3,2] */, 0xf, 0xf, false);
  // (x & k3) | (p & ~k3) as one bit-field insert (the compiler otherwise
  // spends an AND and an AND-OR)
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(rd.k3), "v"(x), "v"(p));
  return r;
}

// Transpose and table lookups of one substep for both n-tiles.
__device__ __forceinline__ void lookups(const uint32_t (&cw)[NT], const DRd& rd,
                                        uint32_t (&d)[NT][4]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint32_t q = transpose8(cw[nt], rd);
    d[nt][0] = dlut_read(lut_addr<kCopies, 0>(q, rd.lane_off));
    d[nt][1] = dlut_read(lut_addr<kCopies, 1>(q, rd.lane_off));
    d[nt][2] = dlut_read(lut_addr<kCopies, 2>(q, rd.lane_off));
    d[nt][3] = dlut_read(lut_addr<kCopies, 3>(q, rd.lane_off));
  }
}

template <int MTV, bool kABf16>
__device__ __forceinline__ void load_a(const char* st, const DRd& rd, int s, f16x8 (&af)[MT]) {
#pragma unroll
  for (int mt = 0; mt < MTV; ++mt) {
    u32x4 v = *reinterpret_cast<const u32x4*>(st + OFF_A + rd.a[s] + mt * 4096);
    if constexpr (kABf16) v = bf16x8_to_f16x8(v);
    af[mt] = as_f16x8(v);
  }
}

// Code words of the 4 substeps x 2 n-tiles of the step in stage `st`.
__device__ __forceinline__ void load_codes(const char* st, const DRd& rd,
                                           uint32_t (&cw)[4][NT]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      cw[s][nt] = *reinterpret_cast<const uint32_t*>(st + rd.b[nt] + s * 2048);
}

__device__ __forceinline__ u32x4 load_sc(int par, const DRd& rd, int s) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&d_sc[par][0][0]) +
                                          rd.sc + s * 16);
}

// Decoded table words times the rows' absmax: the weight operands.
__device__ __forceinline__ void scale_b(const uint32_t (&d)[NT][4], const u32x4 sc,
                                        f16x8 (&bf)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const u32x4 v = {half2_as_u32(u32_as_half2(d[nt][0]) * u32_as_half2(sc.x)),
                     half2_as_u32(u32_as_half2(d[nt][1]) * u32_as_half2(sc.y)),
                     half2_as_u32(u32_as_half2(d[nt][2]) * u32_as_half2(sc.z)),
                     half2_as_u32(u32_as_half2(d[nt][3]) * u32_as_half2(sc.w))};
    bf[nt] = as_f16x8(v);
  }
}

// One substep: MFMAs of substep S with the operands prepared in registers,
// while the operands of the next substep are prepared -- for S = 3, substep
// 0 of the next step, from the next stage (valid once the barrier before
// substep 3 has passed), after converting that step's absmax.  The next
// weights are scaled after this substep's MFMAs are issued, so no MFMA
// waits on the multiplies.
template <int S, int MTV, bool kABf16, bool kVP>
__device__ __forceinline__ void substep(const char* st, const char* nst, int par, int wave,
                                        int lane, const DRd& rd, uint32_t (&cw)[4][NT],
                                        f16x8 (&af)[MT], f16x8 (&bf)[NT],
                                        f32x16 (&acc)[MT][NT], f32x4& acc_v) {
  f16x8 af_n[MT];
  uint32_t dn[NT][4];
  u32x4 sc_n;
  if constexpr (S < 3) {
    load_a<MTV, kABf16>(st, rd, S + 1, af_n);
    lookups(cw[S + 1], rd, dn);
    sc_n = load_sc(par, rd, S + 1);
  } else {
    const float sv = *reinterpret_cast<const float*>(nst + OFF_S + lane * 32 + wave * 4);
    d_sc[par ^ 1][wave][lane] = (_Float16)sv;
    load_codes(nst, rd, cw);
    load_a<MTV, kABf16>(nst, rd, 0, af_n);
    lookups(cw[0], rd, dn);
    sc_n = load_sc(par ^ 1, rd, 0);
  }
  // in-loop adapter projection: v[this wave's 16 rows][16 ranks] += a B_e,
  // stack-row half S - 1 of the step
  // (operand offsets recomputed here rather than held: the kernel is at its
  // register limit) -- A row c16 of this wave's 16 rows, k chunk 4 s2 + g4,
  // swizzled like the main fragments; B^T row (rank) c16, same k
  if constexpr (kVP && (S == 1 || S == 2)) {
    constexpr int s2 = S - 1;
    const int c16 = lane & 15, g4 = lane >> 4;
    const int row = wave * 16 + c16;
    const uint32_t ua = row * 128 + (((4 * s2 + g4) ^ ((row >> 1) & 7)) << 4);
    const u32x4 l = *reinterpret_cast<const u32x4*>(st + OFF_L + c16 * 128 + g4 * 16 + s2 * 64);
    u32x4 v = *reinterpret_cast<const u32x4*>(st + OFF_A + ua);
    if constexpr (kABf16) v = bf16x8_to_f16x8(v);
    acc_v = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(v), as_f16x8(l), acc_v, 0, 0, 0);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt)
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[nt], af[mt], acc[mt][nt], 0, 0, 0);
#pragma unroll
  for (int mt = 0; mt < MTV; ++mt) af[mt] = af_n[mt];
  scale_b(dn, sc_n, bf);
}

// The contraction loop of one tile.  Batch kb (the copies of step kb) goes
// into stage kb % 3.  The prologue issues batches 0, 1, 2; after the
// barrier of step kb (every wave is done reading stage kb % 3, whose last
// reads are substep 2's) the wave issues batch kb + 3 there.  Before that
// barrier step kb + 1 must have landed: batch kb + 2 may still be pending,
// so the wait leaves kDma copies outstanding.  Nothing past the last step is
// fetched (only the prologue repeats the last batch, when there are fewer
// than three steps); in the last two steps batch kb + 2 does not exist, so
// they drain all copies instead, and the tile ends with none in flight.
template <int MTV, bool kABf16, bool kVP>
__device__ __forceinline__ void kloop(const DSrc& src, int nk, const DRd& rd, int wave,
                                      int lane, f32x16 (&acc)[MT][NT], f32x4& acc_v) {
  constexpr int kDma = kDmaOf<kVP>();
  const uint32_t ring = lds_addr(d_ring);
  const int last = nk - 1;
  issue_step<kVP>(src, 0, ring, wave);
  issue_step<kVP>(src, min(1, last), ring + STAGE, wave);
  issue_step<kVP>(src, min(2, last), ring + 2 * STAGE, wave);
  wait_vm_barrier<2 * kDma>();  // batch 0 landed

  uint32_t cw[4][NT];
  f16x8 af[MT];
  f16x8 bf[NT];
  {
    const float sv = *reinterpret_cast<const float*>(d_ring + OFF_S + lane * 32 + wave * 4);
    d_sc[0][wave][lane] = (_Float16)sv;
  }
  load_codes(d_ring, rd, cw);
  load_a<MTV, kABf16>(d_ring, rd, 0, af);
  {
    uint32_t d[NT][4];
    lookups(cw[0], rd, d);
    scale_b(d, load_sc(0, rd, 0), bf);
  }
  int sidx = 0;  // kb % 3
  for (int kb = 0; kb < nk; ++kb) {
    const int nidx = sidx == 2 ? 0 : sidx + 1;
    const char* st = d_ring + sidx * STAGE;
    const char* nst = d_ring + nidx * STAGE;
    const int par = kb & 1;
    substep<0, MTV, kABf16, kVP>(st, nst, par, wave, lane, rd, cw, af, bf, acc, acc_v);
    substep<1, MTV, kABf16, kVP>(st, nst, par, wave, lane, rd, cw, af, bf, acc, acc_v);
    substep<2, MTV, kABf16, kVP>(st, nst, par, wave, lane, rd, cw, af, bf, acc, acc_v);
    if (kb >= last - 1) wait_vm_barrier<0>();
    else wait_vm_barrier<kDma>();
    if (kb + 3 <= last) issue_step<kVP>(src, kb + 3, ring + sidx * STAGE, wave);
    substep<3, MTV, kABf16, kVP>(st, nst, par, wave, lane, rd, cw, af, bf, acc, acc_v);
    sidx = nidx;
  }
}

}  // namespace

template <int kEpi, bool kLora, bool kABf16, int kOut, bool kVP>
__global__ __launch_bounds__(NTHREADS, 1) void grouped_dgrad_kernel(DgradArgs g, int n_tiles) {
  static_assert(!kVP || kLora, "the in-loop projection feeds the adapter term");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;
  const int g2 = lane >> 5;
  const int c16 = lane & 15, g4 = lane >> 4;  // 16x16x32 operand coordinates

  lut_fill<kCopies>(d_lut, d_lstage, g.qtype == kQtFP4 ? c_levels_dgrad_fp4 : c_levels_dgrad,
                    tid, NTHREADS);
  build_tile_table<NTHREADS, BM>(g.offsets, g.E, d_tiles, d_wsum, tid);

  const int N = g.N;  // contraction (stack rows)
  const int K = g.K;  // output columns
  const int KB = K / 64;
  const int nk = N / BK;

  DRd rd;
#pragma unroll
  for (int s = 0; s < 4; ++s) rd.a[s] = n32 * 128 + (((g2 * 4 + s) ^ ((n32 >> 1) & 7)) << 4);
  {
    // lane (g2, group gi, i) reads stack row 32 g2 + 8 s + i, word gi of the
    // 16-byte chunk 2 wave + nt, which sits at chunk (2 wave + nt) ^ f
    const int i = lane & 7, gi = (lane >> 3) & 3;
    const int f = i | (g2 << 3);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      rd.b[nt] = OFF_B + (32 * g2 + i) * 256 + (((2 * wave + nt) ^ f) << 4) + gi * 4;
  }
  rd.sc = (uint32_t)(wave * BK + 32 * g2) * 2u;
  rd.lane_off = (uint32_t)(lane & 31) * 4u;
  // byte selectors of (partner word : own word), own bytes 0-3, partner's
  // 4-7: stage 1 keeps the own low half and takes the partner's low half as
  // its high one (lanes 0-3 of a group) or keeps the own high half and takes
  // the partner's high half as its low one (lanes 4-7); stage 2 likewise
  // with bytes 0 and 2 (lanes with bit 1 clear) or 1 and 3
  rd.s1 = (lane & 4) ? 0x03020706u : 0x05040100u;
  rd.s2 = (lane & 2) ? 0x03070105u : 0x06020400u;
  rd.k3 = (lane & 1) ? 0x0f0f0f0fu : 0xf0f0f0f0u;
  rd.amt3 = (lane & 1) ? 4u : 28u;

  const i32x4 a_rsrc = make_rsrc(g.a, (uint32_t)(g.a_rows * (int64_t)N * 2));
  const int total = __builtin_amdgcn_readfirstlane(d_tiles[g.E]) * n_tiles;
  const int G = gridDim.x;  // a multiple of 8
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  const int q = total / G, rem = total - q * G;
  const bool split_tail = rem > 0 && 2 * rem <= G;
  for (int r = 0;; ++r) {
    const int u = xcd * (G >> 3) + pos;
    int tix, half = -1;
    if (split_tail && r == q) {
      if (u >= 2 * rem) break;
      tix = q * G + (u >> 1);
      half = u & 1;
    } else {
      tix = r * G + u;
      if (tix >= total) break;
    }
    const int mt_global = tix / n_tiles;
    const int n_idx = tix - mt_global * n_tiles;
    int lo = 0, hi = g.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (d_tiles[mid] <= mt_global) lo = mid; else hi = mid;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int m_local = mt_global - __builtin_amdgcn_readfirstlane(d_tiles[e]);
    int row0 = __builtin_amdgcn_readfirstlane(g.offsets[e]) + m_local * BM;
    int rows_valid = min(BM, __builtin_amdgcn_readfirstlane(g.offsets[e + 1]) - row0);
    if (half >= 0) {
      row0 += half * (BM / 2);
      rows_valid = min(BM / 2, rows_valid - half * (BM / 2));
      if (rows_valid <= 0) break;
    }
    const int mtv = (rows_valid + 31) >> 5;
    const int cbase = n_idx * BN;

    DSrc src;
    src.a_rsrc = a_rsrc;
    const uint32_t b_bytes = (uint32_t)N * (uint32_t)(K / 2);
    const uint32_t s_bytes = (uint32_t)N * (uint32_t)KB * 4u;
    src.b_rsrc = make_rsrc(reinterpret_cast<const char*>(g.packed) + (int64_t)e * b_bytes, b_bytes);
    src.s_rsrc = make_rsrc(reinterpret_cast<const char*>(g.absmax) + (int64_t)e * s_bytes, s_bytes);
    src.b_step = (uint32_t)BK * (uint32_t)(K / 2);
    src.s_step = (uint32_t)BK * (uint32_t)KB * 4u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = (wave * 2 + i) * 64 + lane;
      const int row = c >> 3;
      const int gchunk = (c & 7) ^ ((row >> 1) & 7);
      const int rr = row < rows_valid ? row : 0;
      const int idx = row0 + rr;
      const uint32_t a_src = g.gather ? (uint32_t)(g.gather[idx] / g.gather_div) : (uint32_t)idx;
      src.a_off[i] = (a_src * (uint32_t)N + gchunk * 8) * 2;
    }
    // codes: wave instruction j = 2 wave + i covers stack rows 4j..4j+3 of the
    // step, 16 chunks of 16 B each; LDS chunk p of row n holds chunk p ^ f(n)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (wave * 2 + i) * 4 + (lane >> 4);
      const int f = (row & 7) | ((row >> 2) & 8);
      const int c = (lane & 15) ^ f;
      src.b_off[i] = (uint32_t)row * (uint32_t)(K / 2) + (uint32_t)(cbase / 2 + c * 16);
    }
    // absmax: wave w copies stack rows 8w..8w+7 of the step, the tile's 8
    // blocks of each (32 contiguous bytes per row); blocks past KB (a partial
    // last tile) read values only waves with no live columns use
    src.s_off = ((uint32_t)(wave * 8 + (lane >> 3)) * (uint32_t)KB +
                 (uint32_t)(cbase / 64 + (lane & 7))) * 4u;
    if constexpr (kVP) {
      // adapter B^T [E, r, N] fp16: 16 ranks x 128 B per step; dword d of the
      // block is rank d / 32 (ranks past r read rank 0, zeroed afterwards)
      const uint32_t l_bytes = (uint32_t)g.lora_r * (uint32_t)N * 2u;
      src.l_rsrc = make_rsrc(reinterpret_cast<const char*>(g.lora_bt) + (int64_t)e * l_bytes,
                             l_bytes);
      const int d = wave * 64 + lane;
      const int rho = d >> 5;
      const int rc = rho < g.lora_r ? rho : 0;
      src.l_off = (uint32_t)rc * (uint32_t)N * 2u + (uint32_t)(d & 31) * 4u;
    } else {
      src.l_rsrc = i32x4{0, 0, 0, 0};
      src.l_off = 0;
    }

    const int par = r & 1;
    if (tid < BM) {
      const int grow = row0 + (tid < rows_valid ? tid : 0);
      d_orow[par][tid] = g.scatter ? g.scatter[grow] : grow;
      float rs = 1.0f;
      if (g.row_scale)
        rs = g.row_scale[g.rs_idx ? g.rs_idx[grow] : (g.gather ? g.gather[grow] : grow)];
      d_rscale[par][tid] = rs;
    }

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.f;
    f32x4 acc_v = f32x4{0.f, 0.f, 0.f, 0.f};

    lds_barrier();  // every wave is done with the previous tile's stages (and v)
    switch (mtv) {
      case 1: kloop<1, kABf16, kVP>(src, nk, rd, wave, lane, acc, acc_v); break;
      case 2: kloop<2, kABf16, kVP>(src, nk, rd, wave, lane, acc, acc_v); break;
      case 3: kloop<3, kABf16, kVP>(src, nk, rd, wave, lane, acc, acc_v); break;
      default: kloop<4, kABf16, kVP>(src, nk, rd, wave, lane, acc, acc_v); break;
    }
    wait_vm_barrier<0>();  // every copy landed; the ring is free for staging

    // ---- in-loop projection v = a . B_e: 16x16 accumulator layout, lane
    // holds rank c16 of rows 4 g4 + i of this wave's 16.  Written out once
    // per M-tile (by its first N-tile) in fp32 for the adapter's weight
    // gradients, and exchanged between the waves in fp16 with the scale
    // applied (ranks past r computed on a stand-in row, stored as zero).
    _Float16* v_buf = reinterpret_cast<_Float16*>(d_ring + OFF_V);
    if constexpr (kVP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave * 16 + g4 * 4 + i;
        v_buf[row * kMaxLoraR + c16] =
            c16 < g.lora_r ? (_Float16)(acc_v[i] * g.lora_scale) : (_Float16)0.f;
        if (g.lora_v_out != nullptr && n_idx == 0 && c16 < g.lora_r && row < rows_valid)
          g.lora_v_out[(int64_t)(row0 + row) * g.lora_r + c16] = acc_v[i];
      }
      lds_barrier();
    }

    const int col_w = cbase + wave * BNW;  // first output column of this wave
    const bool wave_live = col_w < K;

    // ---- LoRA: out += scale * v_i . A_e[:, col] as one more MFMA per tile
    if constexpr (kLora) {
      f16x8 bl[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = min(col_w + nt * 32 + n32, K - 1);
        const uint16_t* la = reinterpret_cast<const uint16_t*>(g.lora_a) +
                             (int64_t)e * g.lora_r * K + col;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int rho = g2 * 8 + t;
          _Float16 hv = (_Float16)0.f;
          if (rho < g.lora_r) {
            const uint16_t raw = la[(int64_t)rho * K];
            hv = g.lora_bf16 ? (_Float16)bf16_bits_to_f32(raw) : __builtin_bit_cast(_Float16, raw);
          }
          bl[nt][t] = hv;
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt >= mtv) continue;
        f16x8 au;
        if constexpr (kVP) {
          au = *reinterpret_cast<const f16x8*>(&v_buf[(mt * 32 + n32) * kMaxLoraR + g2 * 8]);
        } else {
          const int row = row0 + min(mt * 32 + n32, rows_valid - 1);
          const float* vr = g.lora_v + (int64_t)row * g.lora_r;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int rho = g2 * 8 + t;
            au[t] = (_Float16)(rho < g.lora_r ? vr[rho] * g.lora_scale : 0.f);
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bl[nt], au, acc[mt][nt], 0, 0, 0);
      }
    }

    // ---- epilogue.  Accumulator layout: lane holds tile row (lane & 31) of
    // the m-tile and, for j = 0..15, column 8*(j/4) + 4*(lane/32) + (j%4) of
    // the n-tile.  Each wave stages its 32-row slices (fp32 for the SwiGLU
    // backward, else the output dtype) in a private LDS region.
    if constexpr (kEpi == kDgradEpiSwigluBwd) {
      constexpr int PITCH = BNW * 4 + 16;
      static_assert(NWAVES * 32 * PITCH <= RING, "staging fits the ring");
      char* ws = d_ring + wave * 32 * PITCH;
      // lane item `it` of an m-tile: tile row mt*32 + (it*64 + lane)/8, 8
      // columns at col_w + 8*(lane % 8); the gate and up chunks of g (16 B
      // each) of all four items are loaded before the m-tile is staged, so
      // their latency overlaps the staging and is paid once per m-tile
      u32x4 gq[4][2];
      auto load_g = [&](int mt, u32x4 (&dst)[4][2]) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int row = mt * 32 + ((it * 64 + lane) >> 3);
          const int col = col_w + (lane & 7) * 8;
          dst[it][0] = u32x4{0u, 0u, 0u, 0u};
          dst[it][1] = u32x4{0u, 0u, 0u, 0u};
          if (wave_live && row < rows_valid) {
            const uint16_t* gp = reinterpret_cast<const uint16_t*>(g.g) +
                                 (int64_t)(row0 + row) * 2 * K + col;
            dst[it][0] = *reinterpret_cast<const u32x4*>(gp);
            dst[it][1] = *reinterpret_cast<const u32x4*>(gp + K);
          }
        }
      };
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt >= mtv) continue;
        load_g(mt, gq);
        const float rs = d_rscale[par][mt * 32 + n32];
        char* prow = ws + n32 * PITCH;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float v[4] = {acc[mt][nt][4 * jj] * rs, acc[mt][nt][4 * jj + 1] * rs,
                                acc[mt][nt][4 * jj + 2] * rs, acc[mt][nt][4 * jj + 3] * rs};
            stage_out4<kF32>(prow + (nt * 32 + 8 * jj + 4 * g2) * 4, v);
          }
        // 32 rows x 8 chunks of 8 columns: four passes of the 64 lanes
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int idx = it * 64 + lane;
          const int rr = idx >> 3, c8 = idx & 7;
          const int row = mt * 32 + rr;
          const int col = col_w + c8 * 8;
          if (wave_live && row < rows_valid) {
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(ws + rr * PITCH + c8 * 32);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(ws + rr * PITCH + c8 * 32 + 16);
            const float dh[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            float gate[8], up[8];
            if (g.g_bf16) {
              unpack8<true>(gq[it][0], gate);
              unpack8<true>(gq[it][1], up);
            } else {
              unpack8<false>(gq[it][0], gate);
              unpack8<false>(gq[it][1], up);
            }
            float dg[8], du[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const float sg = sigmoid_f(gate[t]);
              const float si = gate[t] * sg;
              dg[t] = dh[t] * up[t] * (sg * (1.0f + gate[t] * (1.0f - sg)));
              du[t] = dh[t] * si;
            }
            const int64_t orow = d_orow[par][row];
            store8<kOut>(g.out, orow * 2 * K + col, dg);
            store8<kOut>(g.out, orow * 2 * K + K + col, du);
          }
        }
      }
    } else {
      constexpr int ESZ = kOut == kF32 ? 4 : 2;
      constexpr int COLS = BNW;
      constexpr int PITCH = COLS * ESZ + 16;
      constexpr int CPR = COLS * ESZ / 16;
      constexpr int EPC = 16 / ESZ;
      static_assert(NWAVES * 32 * PITCH <= RING, "staging fits the ring");
      char* ws = d_ring + wave * 32 * PITCH;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt >= mtv) continue;
        const float rs = d_rscale[par][mt * 32 + n32];
        char* prow = ws + n32 * PITCH;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float v[4] = {acc[mt][nt][4 * jj] * rs, acc[mt][nt][4 * jj + 1] * rs,
                                acc[mt][nt][4 * jj + 2] * rs, acc[mt][nt][4 * jj + 3] * rs};
            stage_out4<kOut>(prow + (nt * 32 + 8 * jj + 4 * g2) * ESZ, v);
          }
#pragma unroll
        for (int it = 0; it < CPR / 2; ++it) {
          const int idx = it * 64 + lane;
          const int rr = idx / CPR, c = idx % CPR;
          const u32x4 v = *reinterpret_cast<const u32x4*>(ws + rr * PITCH + c * 16);
          const int row = mt * 32 + rr;
          const int col = col_w + c * EPC;
          if (row < rows_valid && col < K) {
            const int64_t orow = d_orow[par][row];
            *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(g.out) +
                                      (orow * K + col) * ESZ) = v;
          }
        }
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int kEpi, bool kLora, bool kABf16, bool kVP>
static void dgrad_out(const DgradArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  switch (g.out_dtype) {
    case kF32:
      hipLaunchKernelGGL((grouped_dgrad_kernel<kEpi, kLora, kABf16, kF32, kVP>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
    case kBF16:
      hipLaunchKernelGGL((grouped_dgrad_kernel<kEpi, kLora, kABf16, kBF16, kVP>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
    default:
      hipLaunchKernelGGL((grouped_dgrad_kernel<kEpi, kLora, kABf16, kF16, kVP>), grid,
                         dim3(NTHREADS), 0, s, g, n_tiles);
      break;
  }
}

template <int kEpi, bool kLora, bool kVP = false>
static void dgrad_a(const DgradArgs& g, dim3 grid, int n_tiles, hipStream_t s) {
  if (g.a_bf16) dgrad_out<kEpi, kLora, true, kVP>(g, grid, n_tiles, s);
  else dgrad_out<kEpi, kLora, false, kVP>(g, grid, n_tiles, s);
}

hipError_t launch_grouped_dgrad(const DgradArgs& g, int num_cus, hipStream_t stream) {
  const int n_tiles = (g.K + BN - 1) / BN;
  int grid = (num_cus + 7) / 8 * 8;
  const int64_t max_tiles = ((g.P + BM - 1) / BM + g.E) * n_tiles;
  if ((int64_t)grid > max_tiles) grid = (int)((max_tiles + 7) / 8 * 8);
  if (grid < 8) grid = 8;
  const dim3 dg((unsigned)grid);
  const bool lora = g.lora_v != nullptr;
  if (g.lora_bt != nullptr) {
    // the adapter's projection computed in the k-loop (plain epilogue only)
    if (g.epilogue != kDgradEpiNone) return hipErrorInvalidValue;
    dgrad_a<kDgradEpiNone, true, true>(g, dg, n_tiles, stream);
  } else if (g.epilogue == kDgradEpiSwigluBwd) {
    if (lora) dgrad_a<kDgradEpiSwigluBwd, true>(g, dg, n_tiles, stream);
    else dgrad_a<kDgradEpiSwigluBwd, false>(g, dg, n_tiles, stream);
  } else {
    if (lora) dgrad_a<kDgradEpiNone, true>(g, dg, n_tiles, stream);
    else dgrad_a<kDgradEpiNone, false>(g, dg, n_tiles, stream);
  }
  return hipGetLastError();
}

}  // namespace nf4moe
