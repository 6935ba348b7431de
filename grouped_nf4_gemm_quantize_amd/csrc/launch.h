// Internal launcher declarations (host side).  Each launcher enqueues its
// kernels on `stream` and returns the first HIP error, if any.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4moe {

// Records `fmt` as this thread's last-error message (nf4moe_last_error) and
// returns `status`.
int report_error(int status, const char* fmt, ...);

// fp32 thresholds of the quantiser: t[j] is the largest fp32 value that is
// <= the exact midpoint of levels j and j+1, so  xn > t[j]  <=>  xn lies
// strictly above that midpoint (a tie goes to the lower level).
// nf4: code = number of the 15 thresholds below x/absmax.  fp4: magnitude
// index = number of the first 7 thresholds below |x/absmax|, code = sign
// bit << 3 | index.
struct QuantThresholds {
  float t[15];
  int qtype;
};

hipError_t launch_quantize(const void* w, int w_dtype, int64_t nelem,
                           uint8_t* packed, float* absmax, int32_t* flag,
                           const QuantThresholds& thr, int num_cus,
                           hipStream_t stream);

// Scan of n bf16 or fp32 values for what an fp16 conversion loses (flag bits
// as documented at nf4moe_f16_range_check).
hipError_t launch_f16_range(const void* t, bool bf16, int64_t n, int32_t* flags, int num_cus,
                            hipStream_t stream);

struct RouteArgs {
  const float* logits;
  int64_t T;
  int E;
  int k;
  int renormalize;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* sorted_pair;
  int32_t* pair_pos;        // nullable
  int32_t* expert_offsets;  // [E+1]
  uint32_t* chunk_masks;    // [nchunks, E]
  int32_t* chunk_base;      // [nchunks, E]
  const void* x_in;         // optional activation rows to convert (bf16)
  int x_bf16;
  _Float16* x16;            // null: no conversion
  int H;
  int num_cus;              // sizes the conversion's grid
};

hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

hipError_t launch_combine(const _Float16* o, const float* w, int64_t T, int k,
                          int H, void* y, int y_dtype, int num_cus,
                          hipStream_t stream);

struct GemmArgs {
  const void* a;
  int64_t a_rows;  // rows of `a` (bounds the activation copies)
  int a_bf16;
  const int32_t* gather;  // nullable
  int gather_div;
  const uint8_t* packed;
  const float* absmax;
  const int32_t* offsets;     // [E+1]
  int E;
  int64_t P;
  int N;
  int K;
  const void* lora_a;  // nullable [E, r, K]
  const void* lora_b;  // [E, N, r]
  int lora_r;
  float lora_scale;
  int lora_bf16;
  int swiglu;
  // nullable: with swiglu, the SwiGLU backward instead of SwiGLU -- out =
  // [dh*up*silu'(gate) | dh*silu(gate)] ([P, N] fp16, row i = tile row i)
  // for dh the gradient of h ([P, N/2] fp16); fp16 a, fp16 out, nf4 / fp4
  // stacks, no row scale or scatter
  const void* dh;
  void* h_out;  // nullable (SwiGLU backward): h = silu(gate) * up, [P, N/2] fp16
  float* u_out;  // nullable (SwiGLU backward with an adapter): u = X A_e^T, [P, r] fp32
  const float* row_scale;  // nullable
  const int32_t* scatter;  // nullable
  void* out;
  int out_dtype;
  int qtype;               // storage mode (kQtNF4 / kQtFP4)
};

constexpr int kGemmBM = 128;  // rows of an M-tile (one expert's rows only)

hipError_t launch_grouped_gemm(const GemmArgs& g, int num_cus,
                               hipStream_t stream);
// The same contract on a 16-bit passthrough stack (qtype kQtBF16 / kQtF16:
// packed is the [E, N, K] weights, absmax unused, no adapters).
hipError_t launch_grouped_gemm16(const GemmArgs& g, int num_cus, hipStream_t stream);
// fp32 or bf16 weights -> bf16 or fp16 (round to nearest even); n % 8 == 0.
hipError_t launch_to16(const void* w, bool w_bf16, int64_t n, bool out_bf16, uint16_t* out,
                       int num_cus, hipStream_t s);

struct GemvArgs {
  const void* x;  // [H] bf16 or f16
  int x_bf16;
  const float* logits;  // [E]
  int E;
  int k;
  int renormalize;
  int H;
  int I;
  const uint8_t* gu_packed;
  const float* gu_absmax;
  const uint8_t* dn_packed;
  const float* dn_absmax;
  int32_t* topk_ids;        // [k]
  float* topk_w;            // [k]
  int32_t* sorted_pair;     // [k] the pairs grouped by expert
  int32_t* expert_offsets;  // [E+1]
  uint64_t* barrier;        // kDecodeBarrierBytes(k*I): generation word, then the h exchange
  uint32_t spin_limit;      // polls before the h exchange gives up (outputs NaN)
  void* y;                  // [H]
  int y_dtype;
  int qtype;                // storage mode of both stacks (kQtNF4 / kQtFP4 / kQtMXFP4)
};

// The decode kernel's grid-wide exchange of h: a generation word, then one
// 64-bit word per h value (a 48-bit tag of the launch | the fp16 bits).
constexpr int kDecodeFlagOffset = 32;  // words: the generation owns the first 256 bytes
constexpr size_t decode_exchange_bytes(int64_t kI) { return (kDecodeFlagOffset + kI) * 8; }
constexpr uint32_t kDecodeSpinLimit = 1u << 20;

hipError_t launch_decode(const GemvArgs& g, int num_cus, hipStream_t stream);

// Grouped dgrad: out[i, :K] = row_scale * (a[src(i), :N] . W_e [N, K]
// (+ lora_scale * v[i, :r] . A_e[:r, :K])), contracting over the stack rows.
constexpr int kDgradEpiNone = 0;
constexpr int kDgradEpiSwigluBwd = 1;  // out = [dh*up*silu'(gate) | dh*silu(gate)], 2K cols

struct DgradArgs {
  const void* a;           // [a_rows, N] f16/bf16
  int64_t a_rows;
  int a_bf16;
  const int32_t* gather;   // nullable: src(i) = gather[i] / gather_div
  int gather_div;
  const uint8_t* packed;   // [E, N, K/2]
  const float* absmax;     // [E, N, K/64]
  const int32_t* offsets;  // [E+1]
  int E;
  int64_t P;
  int N;                   // stack rows = contraction
  int K;                   // output columns
  const float* row_scale;  // nullable, row i scaled by row_scale[idx(i)], idx(i) =
                           // rs_idx[i] if rs_idx, else gather[i] if gather, else i
  const int32_t* rs_idx;   // nullable
  const int32_t* scatter;  // nullable: output row of row i
  int epilogue;
  const void* g;           // SwiGLU backward: pre-activation rows [P, 2K] (row i)
  int g_bf16;
  const float* lora_v;     // nullable [P, r] fp32 (row i)
  // nullable (plain epilogue only): v = a . B_e computed in the k-loop from
  // the adapter's B transposed, fp16 [E, r, N], instead of lora_v; written to
  // lora_v_out ([P, r] fp32, row i) when that is non-null
  const _Float16* lora_bt;
  float* lora_v_out;
  const void* lora_a;      // [E, r, K]
  int lora_r;
  float lora_scale;
  int lora_bf16;
  void* out;
  int out_dtype;
  int qtype;
};

hipError_t launch_grouped_dgrad(const DgradArgs& g, int num_cus, hipStream_t stream);

// One pass of the QLoRA backward over the rows of m (64-row tiles of one
// expert): a rank-r projection out[i, j] = sum_c m[src(i), c] w[e, j, c]
// and/or an adapter weight gradient z[e] = scale * sum_i rs(i) q[i, :] (x)
// m[src(i), :] (per-tile partials, then a fixed-order reduction per expert).
struct LoraPassArgs {
  const void* m;           // [rows, C] f16/bf16
  int m_bf16;
  const int32_t* gather;   // nullable: src(i) = gather[i] / gather_div
  int gather_div;
  const int32_t* offsets;  // [E+1]
  int E;
  int64_t P;
  int C;                   // a multiple of 64
  int r;
  const _Float16* w;       // projection weights [E, r, C]
  float* out;              // nullable: projection [P, r]
  const float* rs;         // nullable row scale rs[rs_idx ? rs_idx[i] : i]
  const int32_t* rs_idx;
  const float* q;          // [P, r]
  float* part;             // nullable: gradient partials [(P / 64 + E), r, C]
  float* z;                // gradient [E, r, C] (rank_major) or [E, C, r]
  float scale;
  int rank_major;
};

hipError_t launch_bf16_to_f16(const void* src, int64_t n, _Float16* dst, int num_cus,
                              hipStream_t s);
// Up to four bf16 arrays (each a multiple of 8 elements, dst 16-byte
// aligned) converted to fp16 in one launch.
struct HalfCopies {
  const uint16_t* src[4];
  _Float16* dst[4];
  int64_t n8[4];  // elements / 8
  int count;
};
hipError_t launch_half_copies(const HalfCopies& c, int num_cus, hipStream_t s);
hipError_t launch_lora_to_f16(const void* src, int src_bf16, int transpose, int E, int C,
                              int r, _Float16* dst, int num_cus, hipStream_t s);
hipError_t launch_lora_pass(const LoraPassArgs& a, int num_cus, hipStream_t s);

}  // namespace nf4moe
