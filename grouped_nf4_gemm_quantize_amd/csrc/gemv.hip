// Single-token (T = 1) decode path: one fused kernel over the routed experts.
//
// At batch 1 the expert projection is a matrix-vector product per routed
// expert that streams the packed bytes once (experts4bit-qlora 0.22.0 README,
// "Inference": the single-token decode fast path uses a fused 4-bit GEMV).  HBM
// bandwidth on the NF4 codes + absmax is the roofline, and with only ~21 MB
// per layer the time is set by the chain of dependent memory round trips:
// the router logits, then the weights.  So one kernel does the whole layer,
// and each of its waves:
//
//   1. loads the logits, x and the exchange's generation word, and (with its
//      workgroup) builds the decode table while they are in flight;
//   2. routes the token itself (a top-k over the E logits costs a few
//      hundred cycles, cheaper than any exchange);
//   3. issues the loads of its (slot j, column i) gate/up items -- the gate
//      row i and the up row I+i of expert ids[j] -- stages x as fp16 and
//      computes h[j, i] = w_j * silu(gate) * up (fp32, rounded once to fp16),
//      which it publishes;
//   4. issues the loads of its down output row n, whose K is the
//      concatenation of the k experts' I inputs (so the combine over the
//      slots is part of the dot product) -- after its h, so the gate/up bytes
//      the exchange waits for are not queued behind them;
//   5. takes part in a grid-wide exchange of h: every workgroup reads all
//      k*I values (a bounded wait), decoding its first down chunks while the
//      first reads are in flight, and finishes its down rows.
//
// Each h value travels as one 64-bit word: a 48-bit tag | the fp16 bits,
// stored and loaded whole at agent scope, so a word with this launch's tag
// holds this launch's value and no fence or flag is needed.  The tag is a
// hash of (generation + 1, workspace address); the generation word sits in
// the caller's workspace, every workgroup reads it before it publishes
// anything, and workgroup 0 advances it once every word was seen, so stale
// or uninitialised workspace bytes never match (the workspace needs no
// clearing).  The exchange needs every workgroup resident at once: the grid
// is at most one workgroup per compute unit, and each workgroup fits on one.
// A wait that exceeds its bound writes NaN to the workgroup's outputs and
// advances the generation, so a failure is loud and does not poison the next
// call.
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

namespace {
constexpr int kCopies = 32;
constexpr int kThreads = 512;          // 8 waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxChunksPerLane = 8;   // down: chunks of the concatenated K (k*I <= 16384)
constexpr int kDnFirst = 3;            // of which always loaded (k*I <= 6144 in one pass)

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

// The table words of one chunk (32 codes -> 16 half2, unscaled), decoded
// ahead of its activations; chunk_dot then matches dot_chunk exactly.
__device__ __forceinline__ void decode_chunk(const uint32_t* lut, uint32_t lane_off, u32x4 q,
                                             uint32_t (&d)[16]) {
  const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t dw[4];
    decode8<kCopies>(lut, lane_off, qq[w], dw);
#pragma unroll
    for (int t = 0; t < 4; ++t) d[4 * w + t] = dw[t];
  }
}

__device__ __forceinline__ float chunk_dot(const uint32_t (&d)[16], const _Float16* act) {
  const u32x4* a4 = reinterpret_cast<const u32x4*>(act);
  float p = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4 av = a4[w];
    const uint32_t aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      p = __builtin_amdgcn_fdot2(u32_as_half2(d[4 * w + t]), u32_as_half2(aa[t]), p, false);
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

// The scale of chunk c (32 weights) of a row, loaded as raw bits and turned
// into a value only where it is used (so no load waits at issue): the fp32
// absmax of its 64-block, or for MXFP4 stacks the e8m0 byte of its own
// 32-block, 2^(s - 127) in fp32 (exact over the whole e8m0 range; 255 is NaN).
__device__ __forceinline__ uint32_t chunk_scale_bits(const float* absmax, int64_t row,
                                                     int chunks, int c, bool mx) {
  if (mx) return reinterpret_cast<const uint8_t*>(absmax)[row * chunks + c];
  return reinterpret_cast<const uint32_t*>(absmax)[row * (chunks / 2) + (c >> 1)];
}

__device__ __forceinline__ float scale_value(uint32_t b, bool mx) {
  if (mx) return b == 255u ? __builtin_nanf("") : ldexpf(1.0f, (int)b - 127);
  return __uint_as_float(b);
}

// 16-bit activation -> fp16 (bf16 rounds to nearest even; fp16 passes through)
__device__ __forceinline__ _Float16 to_f16(uint16_t raw, bool bf16) {
  return bf16 ? (_Float16)bf16_bits_to_f32(raw) : __builtin_bit_cast(_Float16, raw);
}

}  // namespace

// splitmix64 finaliser: the tag of generation `g` for an exchange buffer at
// address `a` (a bijection of g for a fixed a); the top 48 bits are used.
__device__ __forceinline__ uint64_t exchange_tag(uint64_t g, uint64_t a) {
  uint64_t z = g * 0x9E3779B97F4A7C15ull ^ a;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (z ^ (z >> 31)) & ~0xffffull;
}

__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The routing views of a T = 1 forward (written by one wave; lane j < k
// holds slot j): ids, weights, the pairs p = j grouped by expert (the k ids are
// distinct, so a pair's position is the number of smaller ids) and the
// per-expert offsets (offsets[e] = number of selected ids below e).
__device__ __forceinline__ void write_routing(const GemvArgs& g, int lane, int id, float w) {
  const int k = g.k;
  if (lane < k) {
    g.topk_ids[lane] = id;
    g.topk_w[lane] = w;
  }
  int below = 0;
  for (int j = 0; j < k; ++j) below += __builtin_amdgcn_readlane(id, j) < id ? 1 : 0;
  if (lane < k) g.sorted_pair[below] = lane;
  for (int e = lane; e <= g.E; e += 64) {
    int c = 0;
    for (int j = 0; j < k; ++j) c += __builtin_amdgcn_readlane(id, j) < e ? 1 : 0;
    g.expert_offsets[e] = c;
  }
}

// The expert of slot j (lane-varying, lo <= j <= hi, wave-uniform bounds)
// from the ids held by lanes 0..k-1: one readlane per slot the wave spans.
__device__ __forceinline__ int slot_expert(int id, int j, int lo, int hi) {
  int e = 0;
  for (int jj = lo; jj <= hi; ++jj) {
    const int v = __builtin_amdgcn_readlane(id, jj);
    e = j == jj ? v : e;
  }
  return e;
}

// kCpl = ceil(H / 2048) <= 4: 32-weight chunks of one gate/up row per lane;
// kItems gate/up items per wave are loaded at once (3 of one chunk per lane
// -- the Qwen3-30B-A3B decode layer on 256 compute units has exactly 3 --, 2
// of two, 1 of four).
template <int kRegs, int kCpl, bool kMx>
__global__ __launch_bounds__(kThreads) void decode_layer_kernel(GemvArgs g) {
  constexpr int kItems = kCpl == 1 ? 3 : 4 / kCpl;
  constexpr int kHPer = 8;  // exchange words per thread and pass
  __shared__ uint32_t s_lut[256 * kCopies];
  __shared__ uint16_t s_stage[16];
  __shared__ int s_fail;
  extern __shared__ __attribute__((aligned(16))) _Float16 s_dyn[];  // x [H], then h [k*I]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = g.H, I = g.I, k = g.k;
  _Float16* s_x = s_dyn;
  _Float16* s_h = s_dyn + H;

  // the router logits first: they head the only dependent chain before the
  // weight loads (the other loads below are consumed much later)
  float lgv[kRegs];
  route_load<kRegs>(g.logits, g.E, lane, lgv);

  // activations: consumed while the weight loads are in flight
  constexpr int kXPer = 4;  // x elements per thread and pass
  uint2 xr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i0 = (p * kThreads + tid) * kXPer;
    // clamped: every thread loads (the staging below skips i0 >= H)
    xr[p] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) +
                                            (i0 < H ? i0 : H - kXPer));
  }

  // this launch's tag: the generation is read before this workgroup
  // publishes anything, and it is advanced only once every value is seen
  uint64_t* gen_p = g.barrier;
  uint64_t* hx = g.barrier + kDecodeFlagOffset;
  const uint64_t gen = load_agent(gen_p);

  // the decode table, built while the logits are in flight: the 16 levels
  // rounded to fp16 (immediates, no load), then entry b (two levels) is
  // written by two threads, 16 of its kCopies interleaved copies each
  static_assert(kThreads == 2 * 256 && kCopies == 32, "table fill layout");
  if (tid == 0) {
    s_fail = 0;
    constexpr float kNf4[16] = NF4MOE_LEVELS_INIT;
    constexpr float kFp4[16] = NF4MOE_FP4_LEVELS_INIT;
    constexpr float kE2m1[16] = NF4MOE_E2M1_VALUES_INIT;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float lv = g.qtype == kQtMXFP4 ? kE2m1[i] : g.qtype == kQtFP4 ? kFp4[i] : kNf4[i];
      s_stage[i] = __builtin_bit_cast(uint16_t, (_Float16)lv);
    }
  }
  __syncthreads();
  {
    const bool low_first = g.qtype == kQtMXFP4;
    const int b = tid >> 1;
    const int first = low_first ? (b & 15) : (b >> 4);
    const int second = low_first ? (b >> 4) : (b & 15);
    const uint32_t v = (uint32_t)s_stage[first] | ((uint32_t)s_stage[second] << 16);
    const u32x4 v4 = {v, v, v, v};
    u32x4* dst = reinterpret_cast<u32x4*>(s_lut + b * kCopies + (tid & 1) * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = v4;
  }

  // route in every wave: lane j < k holds slot j
  int id;
  float w;
  route_select<kRegs>(lgv, g.E, k, g.renormalize, lane, &id, &w);

  // x as fp16 in LDS (its loads went out with the logits'; converted by
  // every thread, so the wait for them is not inside a branch)
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i0 = (p * kThreads + tid) * kXPer;
    const uint2 hv = make_uint2(pack_half2(to_f16(xr[p].x & 0xffffu, g.x_bf16),
                                           to_f16(xr[p].x >> 16, g.x_bf16)),
                                pack_half2(to_f16(xr[p].y & 0xffffu, g.x_bf16),
                                           to_f16(xr[p].y >> 16, g.x_bf16)));
    if (i0 < H) *reinterpret_cast<uint2*>(s_x + i0) = hv;
  }
  __syncthreads();  // table and x complete

  const int chunks = H / 32;
  const int64_t row_bytes = H / 2;
  constexpr bool mx = kMx;
  const int nw = gridDim.x * kWaves;
  const int q0 = blockIdx.x * kWaves + wave;

  // ---- down rows of this wave: n = q0 + r * nw; this lane's chunks of the
  // concatenated K are cc = lane + 64 m, the same for every row.  The first
  // kDnFirst chunks are loaded for every lane (a lane past the end re-reads
  // the last chunk and contributes zero), the rest only where they exist.
  // Unconditional loads let the compiler count the loads in flight exactly,
  // so no later use waits for more of them than it needs.
  const int cps = I / 32;  // chunks per slot
  const int total = k * cps;
  // j = cc / cps through an fp32 reciprocal: with k*I <= 16384 there are at
  // most 512 chunks, so cps <= 512 and (cc + 1/2) / cps lies at least 2^-10
  // from an integer, while the rounded product is within 2^-15 of it: the
  // truncation is exact
  const float inv_cps = 1.0f / (float)cps;
  const uint32_t dn_stride = (uint32_t)H * (uint32_t)(I / 2);                 // bytes / expert
  const uint32_t am_stride = (uint32_t)H * (uint32_t)(mx ? I / 32 : I / 64);  // scales / expert
  uint64_t pk_off[kMaxChunksPerLane];
  uint64_t am_off[kMaxChunksPerLane];  // absmax element, or scale byte for MXFP4
  int h_off[kMaxChunksPerLane];
  bool dvalid[kMaxChunksPerLane];
#pragma unroll
  for (int m = 0; m < kMaxChunksPerLane; ++m) {
    const int cc0 = lane + 64 * m;
    dvalid[m] = cc0 < total;
    pk_off[m] = 0;
    am_off[m] = 0;
    h_off[m] = 0;
    if (m < kDnFirst || 64 * m < total) {  // compile-time or wave-uniform
      const int cc = dvalid[m] ? cc0 : total - 1;
      const int j = (int)(((float)cc + 0.5f) * inv_cps);
      const int lo = (int)(((float)(64 * m < total ? 64 * m : total - 1) + 0.5f) * inv_cps);
      const int hi = (int)(((float)(64 * m + 63 < total ? 64 * m + 63 : total - 1) + 0.5f) * inv_cps);
      const uint32_t e = (uint32_t)slot_expert(id, j, lo, hi);
      const uint32_t c = (uint32_t)(cc - j * cps);
      pk_off[m] = (uint64_t)e * dn_stride + c * 16u;
      am_off[m] = (uint64_t)e * am_stride + (mx ? c : c >> 1);
      h_off[m] = j * I + (int)c * 32;
    }
  }
  // ---- gate/up items of this wave: q = q0 + it * nw, it < n_items.  The
  // first kItems slots are loaded unconditionally (a slot past n_items
  // re-reads a valid item and publishes nothing).
  const int items = k * I;
  const int n_items = q0 < items ? (items - 1 - q0) / nw + 1 : 0;
  u32x4 qg[kItems][kCpl], qu[kItems][kCpl];
  uint32_t sg[kItems][kCpl], su[kItems][kCpl];
  auto load_item = [&](int t, int q) {
    const int j = q / I;  // wave-uniform: scalar arithmetic
    const int i = q - j * I;
    const int e = __builtin_amdgcn_readlane(id, j);
    const int64_t rg = (int64_t)e * 2 * I + i;
    const int64_t ru = rg + I;
#pragma unroll
    for (int m = 0; m < kCpl; ++m) {
      int c = lane + 64 * m;
      if (c >= chunks) c = chunks - 1;
      qg[t][m] = *reinterpret_cast<const u32x4*>(g.gu_packed + rg * row_bytes + c * 16);
      qu[t][m] = *reinterpret_cast<const u32x4*>(g.gu_packed + ru * row_bytes + c * 16);
      sg[t][m] = chunk_scale_bits(g.gu_absmax, rg, chunks, c, mx);
      su[t][m] = chunk_scale_bits(g.gu_absmax, ru, chunks, c, mx);
    }
  };
  auto item_q = [&](int it) {  // a valid item for every slot
    const int last = n_items > 0 ? n_items - 1 : 0;
    const int q = q0 + (it < last ? it : last) * nw;
    return q < items ? q : 0;
  };

  u32x4 qd[kMaxChunksPerLane];
  uint32_t sd[kMaxChunksPerLane];
  auto load_chunk = [&](int m, int row) {
    const int64_t prow = (int64_t)row * (I / 2);
    const int64_t arow = (int64_t)row * (mx ? I / 32 : I / 64);
    qd[m] = *reinterpret_cast<const u32x4*>(g.dn_packed + pk_off[m] + prow);
    sd[m] = mx ? reinterpret_cast<const uint8_t*>(g.dn_absmax)[am_off[m] + arow]
               : reinterpret_cast<const uint32_t*>(g.dn_absmax)[am_off[m] + arow];
  };
  auto load_row = [&](int row) {
#pragma unroll
    for (int m = 0; m < kMaxChunksPerLane; ++m)
      if (m < kDnFirst || 64 * m < total) load_chunk(m, row);
  };

  // the gate/up loads of the first round go out back to back (the address
  // arithmetic above is done, so no wait for an earlier load intervenes); the
  // down loads follow once this wave's h is computed, so the gate/up bytes
  // the exchange waits for are not queued behind them
#pragma unroll
  for (int t = 0; t < kItems; ++t) load_item(t, item_q(t));
  int n = q0;
  if (blockIdx.x == 0 && wave == 0) write_routing(g, lane, id, w);

  // ---- gate/up dots -> h (w_j * silu(gate) * up, rounded once to fp16),
  // published as one 64-bit word: this launch's tag | the fp16 bits
  const uint64_t tag = exchange_tag(gen + 1, (uint64_t)(uintptr_t)g.barrier);
  const uint32_t lane_off = lut_lane_offset<kCopies>(lane);
  auto item_dots = [&](int it0) {
#pragma unroll
    for (int t = 0; t < kItems; ++t) {
      if (it0 + t < n_items) {  // wave-uniform
        const int q = q0 + (it0 + t) * nw;
        float accg = 0.f, accu = 0.f;
#pragma unroll
        for (int m = 0; m < kCpl; ++m) {
          const int c = lane + 64 * m;
          if (c < chunks) {
            const _Float16* xs = s_x + c * 32;
            accg = fmaf(dot_chunk(s_lut, lane_off, qg[t][m], xs), scale_value(sg[t][m], mx), accg);
            accu = fmaf(dot_chunk(s_lut, lane_off, qu[t][m], xs), scale_value(su[t][m], mx), accu);
          }
        }
        accg = wave_sum(accg);
        accu = wave_sum(accu);
        const float wj = lane_f(w, q / I);
        const _Float16 hv = (_Float16)(silu_g(accg) * accu * wj);
        if (lane == 0) store_agent(hx + q, tag | __builtin_bit_cast(uint16_t, hv));
      }
    }
  };
  // the first round's loads went out before the table was built; later
  // rounds (more items than waves * kItems) load and compute in turn
  item_dots(0);
  {
    const int row = n < H ? n : H - 1;
#pragma unroll
    for (int m = 0; m < kDnFirst; ++m) load_chunk(m, row);
#pragma unroll
    for (int m = kDnFirst; m < kMaxChunksPerLane; ++m)
      if (64 * m < total) load_chunk(m, row);
  }
  for (int it0 = kItems; it0 < n_items; it0 += kItems) {
#pragma unroll
    for (int t = 0; t < kItems; ++t) load_item(t, item_q(it0 + t));
    item_dots(it0);
  }

  // ---- grid-wide exchange of h: every workgroup reads all k*I words until
  // each carries this launch's tag (a bounded wait), keeping the fp16 value
  // the first row's first kDnFirst chunks are decoded (table words, not yet
  // scaled) while the first polls are in flight: after the exchange only
  // their dot products with h remain
  uint32_t dd[kDnFirst][16];
  bool decoded = false;
  auto predecode = [&]() {
#pragma unroll
    for (int m = 0; m < kDnFirst; ++m) decode_chunk(s_lut, lane_off, qd[m], dd[m]);
    decoded = true;
  };
  bool ok = true;
  for (int i0 = tid; i0 < items; i0 += kThreads * kHPer) {
    uint64_t v[kHPer];
    uint32_t pending = 0;
#pragma unroll
    for (int t = 0; t < kHPer; ++t)
      if (i0 + t * kThreads < items) pending |= 1u << t;
    for (uint32_t spin = 0; pending != 0 && spin < g.spin_limit; ++spin) {
      if (spin > 0) __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int t = 0; t < kHPer; ++t)
        if (pending & (1u << t)) v[t] = load_agent(hx + i0 + t * kThreads);
      if (!decoded) predecode();
#pragma unroll
      for (int t = 0; t < kHPer; ++t) {
        if ((pending & (1u << t)) && (v[t] & ~0xffffull) == tag) {
          s_h[i0 + t * kThreads] = __builtin_bit_cast(_Float16, (uint16_t)(v[t] & 0xffffu));
          pending &= ~(1u << t);
        }
      }
    }
    ok = ok && pending == 0;
  }
  if (!decoded) predecode();  // a workgroup with no word to poll
  if (!ok) s_fail = 1;
  __syncthreads();
  const bool failed = s_fail != 0;
  // every workgroup published before it could finish its wait, so all of
  // them have read the generation: advance it (also after a failed wait, so
  // the next launch does not reuse this tag)
  if (tid == 0 && (blockIdx.x == 0 || failed)) store_agent(gen_p, gen + 1);

  // ---- down rows
  for (bool first = true; n < H; n += nw, first = false) {
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxChunksPerLane; ++m) {
      if (m < kDnFirst || 64 * m < total) {  // compile-time or wave-uniform
        const float dot = m < kDnFirst && first ? chunk_dot(dd[m], s_h + h_off[m])
                                                : dot_chunk(s_lut, lane_off, qd[m], s_h + h_off[m]);
        const float p = dot * scale_value(sd[m], mx);
        acc += dvalid[m] ? p : 0.f;
      }
    }
    if (n + nw < H) load_row(n + nw);
    acc = wave_sum(acc);
    if (failed) acc = __builtin_nanf("");
    if (lane == 0) {
      if (g.y_dtype == kF32) store1<kF32>(g.y, n, acc);
      else if (g.y_dtype == kBF16) store1<kBF16>(g.y, n, acc);
      else store1<kF16>(g.y, n, acc);
    }
  }
}

template <int kRegs, bool kMx>
static void launch_layer(const GemvArgs& g, int grid, size_t lds, hipStream_t stream) {
  const int cpl = (g.H + 2047) / 2048;
  if (cpl <= 1)
    hipLaunchKernelGGL((decode_layer_kernel<kRegs, 1, kMx>), dim3(grid), dim3(kThreads), lds,
                       stream, g);
  else if (cpl <= 2)
    hipLaunchKernelGGL((decode_layer_kernel<kRegs, 2, kMx>), dim3(grid), dim3(kThreads), lds,
                       stream, g);
  else
    hipLaunchKernelGGL((decode_layer_kernel<kRegs, 4, kMx>), dim3(grid), dim3(kThreads), lds,
                       stream, g);
}

template <bool kMx>
static void launch_regs(const GemvArgs& g, int grid, size_t lds, hipStream_t stream) {
  const int regs = (g.E + 63) / 64;
  if (regs <= 1) launch_layer<1, kMx>(g, grid, lds, stream);
  else if (regs <= 2) launch_layer<2, kMx>(g, grid, lds, stream);
  else if (regs <= 4) launch_layer<4, kMx>(g, grid, lds, stream);
  else if (regs <= 8) launch_layer<8, kMx>(g, grid, lds, stream);
  else launch_layer<16, kMx>(g, grid, lds, stream);
}

hipError_t launch_decode(const GemvArgs& g, int num_cus, hipStream_t stream) {
  // one workgroup per compute unit at most: the h exchange needs the whole
  // grid resident.  Every workgroup owns at least one h value (item q0 =
  // 8 * block), so each one has read the generation before the exchange can
  // complete anywhere.
  const int items = g.k * g.I;
  int grid = num_cus;
  if (grid > (items + kWaves - 1) / kWaves) grid = (items + kWaves - 1) / kWaves;
  if (grid < 1) grid = 1;
  const size_t lds = ((size_t)g.H + (size_t)g.k * g.I) * sizeof(_Float16);
  if (g.qtype == kQtMXFP4) launch_regs<true>(g, grid, lds, stream);
  else launch_regs<false>(g, grid, lds, stream);
  return hipGetLastError();
}

}  // namespace nf4moe
