// Internal launcher declarations (host side).  Each launcher enqueues its
// kernels on `stream` and returns the first HIP error, if any.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4moe {

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
  const float* row_scale;  // nullable
  const int32_t* scatter;  // nullable
  void* out;
  int out_dtype;
  int qtype;               // storage mode (kQtNF4 / kQtFP4)
};

constexpr int kGemmBM = 128;  // rows of an M-tile (one expert's rows only)

hipError_t launch_grouped_gemm(const GemmArgs& g, int num_cus,
                               hipStream_t stream);

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
  int32_t* topk_ids;  // [k]
  float* topk_w;      // [k]
  void* hbuf;         // [k, I] fp16 h, already scaled by the routing weight
  void* y;            // [H]
  int y_dtype;
  int qtype;          // storage mode of both stacks (kQtNF4 / kQtFP4)
};

hipError_t launch_decode(const GemvArgs& g, int num_cus, hipStream_t stream);

}  // namespace nf4moe
