// Host side of the C ABI declared in include/nf4moe.h: argument validation,
// workspace layout, and kernel launches on the caller's stream.
//
// Every check runs before anything is enqueued, and every failure returns a
// distinct status with a thread-local message (the pages' stance: refuse in
// the pre-flight rather than fail later, experts4bit-qlora 0.22.0 README
// "Which door?"; fail fast with a clear error, "Scope").

#include <hip/hip_runtime.h>

#include <atomic>
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/nf4moe.h"
#include "common.h"
#include "launch.h"

using namespace nf4moe;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return NF4MOE_OK;
}

}  // namespace

int nf4moe::report_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

namespace {

int hip_fail(hipError_t err, const char* what) {
  return fail(NF4MOE_EHIP, "%s: %s", what, hipGetErrorString(err));
}

const float kLevels[16] = NF4MOE_LEVELS_INIT;

// t[j] = the largest fp32 value <= the exact midpoint of levels j and j+1.
// The midpoint of two fp32 numbers is exact in double precision.
QuantThresholds make_thresholds() {
  QuantThresholds th;
  for (int j = 0; j < 15; ++j) {
    const double mid = ((double)kLevels[j] + (double)kLevels[j + 1]) * 0.5;
    float t = (float)mid;
    if ((double)t > mid) t = std::nextafter(t, -INFINITY);
    th.t[j] = t;
  }
  return th;
}

// fp4: thresholds between the 8 magnitude levels (codes 0..7); an exact tie
// (a midpoint that is an fp32 value) goes to the even magnitude index.
const float kLevelsFP4[16] = NF4MOE_FP4_LEVELS_INIT;

QuantThresholds make_thresholds_fp4() {
  QuantThresholds th;
  for (int j = 0; j < 15; ++j) th.t[j] = INFINITY;
  for (int j = 0; j < 7; ++j) {
    const double mid = ((double)kLevelsFP4[j] + (double)kLevelsFP4[j + 1]) * 0.5;
    float t = (float)mid;
    if ((double)t > mid) t = std::nextafter(t, -INFINITY);
    // x > t sends x to index j + 1; at an exact tie that must hold only when
    // j + 1 is even
    if ((double)t == mid && (j + 1) % 2 == 0) t = std::nextafter(t, -INFINITY);
    th.t[j] = t;
  }
  th.qtype = kQtFP4;
  return th;
}

const QuantThresholds& thresholds(int qt) {
  static const QuantThresholds nf4 = [] {
    QuantThresholds t = make_thresholds();
    t.qtype = kQtNF4;
    return t;
  }();
  static const QuantThresholds fp4 = make_thresholds_fp4();
  static const QuantThresholds int8 = [] {
    QuantThresholds t{};
    t.qtype = kQtINT8;
    return t;
  }();
  static const QuantThresholds fp8 = [] {
    QuantThresholds t{};
    t.qtype = kQtFP8;
    return t;
  }();
  if (qt == kQtINT8) return int8;
  if (qt == kQtFP8) return fp8;
  return qt == kQtFP4 ? fp4 : nf4;
}

bool valid_qtype(int qt) {
  return qt == kQtNF4 || qt == kQtFP4 || qt == kQtINT8 || qt == kQtFP8 || qt == kQtBF16 ||
         qt == kQtF16;
}
bool is_8bit(int qt) { return qt == kQtINT8 || qt == kQtFP8; }
bool is_16bit(int qt) { return qt == kQtBF16 || qt == kQtF16; }
// stack bytes of one [N, K] expert block per element, times 2
int64_t bytes_x2(int qt) { return is_16bit(qt) ? 4 : is_8bit(qt) ? 2 : 1; }

std::atomic<int> g_cu_cache[64];

int cu_count(int* out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    const int c = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return NF4MOE_OK;
    }
  }
  int n = 0;
  err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return hip_fail(err, "hipDeviceGetAttribute");
  if (n <= 0) n = 256;
  if (dev >= 0 && dev < 64) g_cu_cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return NF4MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_lora(const nf4moe_lora* l, const char* name) {
  if (l == nullptr) return NF4MOE_OK;
  if (l->A == nullptr || l->B == nullptr)
    return fail(NF4MOE_EINVAL, "%s: LoRA A and B must be non-null", name);
  if (l->r < 1 || l->r > NF4MOE_MAX_LORA_R)
    return fail(NF4MOE_EINVAL, "%s: LoRA rank r=%d outside [1, %d]", name, l->r,
                NF4MOE_MAX_LORA_R);
  if (l->dtype != NF4MOE_BF16 && l->dtype != NF4MOE_F16)
    return fail(NF4MOE_EDTYPE, "%s: LoRA dtype must be BF16 or F16", name);
  if (!std::isfinite(l->scale))
    return fail(NF4MOE_EINVAL, "%s: LoRA scale is not finite", name);
  if (!aligned(l->A, 16) || !aligned(l->B, 2))
    return fail(NF4MOE_EINVAL, "%s: LoRA A must be 16-byte aligned", name);
  return NF4MOE_OK;
}

int check_route_shape(int64_t T, int E, int k) {
  if (T < 1) return fail(NF4MOE_EINVAL, "T=%lld must be >= 1", (long long)T);
  if (E < 1) return fail(NF4MOE_EINVAL, "E=%d must be >= 1", E);
  if (E > NF4MOE_MAX_EXPERTS)
    return fail(NF4MOE_ESHAPE, "E=%d exceeds %d experts", E, NF4MOE_MAX_EXPERTS);
  if (k < 1 || k > E || k > NF4MOE_MAX_TOPK)
    return fail(NF4MOE_ETOPK, "k=%d must satisfy 1 <= k <= min(E=%d, %d)", k, E,
                NF4MOE_MAX_TOPK);
  if (T > (int64_t)INT32_MAX / k)
    return fail(NF4MOE_EOVERFLOW, "T*k = %lld pairs overflow int32 indexing",
                (long long)T * k);
  return NF4MOE_OK;
}

// ---- routing workspace layout
struct RouteLayout {
  size_t masks, base, total;
};

RouteLayout route_layout(int64_t T, int E) {
  const int64_t nchunks = (T + kRouteChunk - 1) / kRouteChunk;
  RouteLayout L;
  size_t o = 0;
  L.masks = o;
  o = align_up(o + (size_t)nchunks * E * 4, 256);
  L.base = o;
  o = align_up(o + (size_t)nchunks * E * 4, 256);
  L.total = o;
  return L;
}

// ---- forward workspace layout (the same regions for every path)
struct FwdLayout {
  size_t ids, w, sorted, pos, offsets, route, x16, h, o, bar;
  // fp16 copies of bf16 adapters (rank r; last, so the routing views above
  // do not depend on r): A_gu [E,r,H], B_gu [E,2I,r], A_dn [E,r,I], B_dn [E,H,r]
  size_t a_gu, b_gu, a_dn, b_dn;
  size_t total;
  RouteLayout r;
};

FwdLayout fwd_layout(int64_t T, int H, int I, int E, int k, int r = 0) {
  FwdLayout L;
  const size_t P = (size_t)T * k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.ids = take(P * 4);
  L.w = take(P * 4);
  L.sorted = take(P * 4);
  L.pos = take(P * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.r = route_layout(T, E);
  L.route = take(L.r.total);
  L.x16 = take((size_t)T * H * 2);
  L.h = take(P * (size_t)I * 2);
  L.o = take(P * (size_t)H * 2);
  L.bar = take(decode_exchange_bytes((int64_t)k * I));
  const size_t er = (size_t)E * r * 2;
  L.a_gu = take(er * H);
  L.b_gu = take(er * 2 * I);
  L.a_dn = take(er * I);
  L.b_dn = take(er * H);
  L.total = o;
  return L;
}

bool use_decode_path(int64_t T, int H, int I, int k, const nf4moe_lora* a,
                     const nf4moe_lora* b) {
  return T == 1 && a == nullptr && b == nullptr && H <= 8192 &&
         (int64_t)k * I <= 16384;
}

}  // namespace

extern "C" {

const char* nf4moe_strerror(int status) {
  switch (status) {
    case NF4MOE_OK: return "ok";
    case NF4MOE_EINVAL: return "invalid argument";
    case NF4MOE_ESHAPE: return "unsupported shape";
    case NF4MOE_EBLOCK: return "unsupported quantisation blocksize (must be 64)";
    case NF4MOE_ETOPK: return "invalid top-k";
    case NF4MOE_EDTYPE: return "unsupported dtype";
    case NF4MOE_EWORKSPACE: return "workspace too small";
    case NF4MOE_EOVERFLOW: return "size overflows 32-bit indexing";
    case NF4MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* nf4moe_last_error(void) { return g_last_error.c_str(); }

const char* nf4moe_version(void) { return "0.1.0"; }

int nf4moe_codebook(float* out16) {
  if (out16 == nullptr) return fail(NF4MOE_EINVAL, "out16 is NULL");
  std::memcpy(out16, kLevels, sizeof(kLevels));
  return ok();
}

int nbit_codebook(int quant_type, float* out16) {
  if (out16 == nullptr) return fail(NF4MOE_EINVAL, "out16 is NULL");
  if (!valid_qtype(quant_type) || is_8bit(quant_type) || is_16bit(quant_type))
    return fail(NF4MOE_EINVAL, "storage mode %d has no 16-level codebook", quant_type);
  std::memcpy(out16, quant_type == kQtFP4 ? kLevelsFP4 : kLevels, sizeof(kLevels));
  return ok();
}

int64_t nf4moe_packed_bytes(int64_t E, int64_t N, int64_t K) {
  if (E < 1 || N < 1 || K < 1) return fail(NF4MOE_EINVAL, "sizes must be positive");
  if (K % NF4MOE_BLOCKSIZE) return fail(NF4MOE_ESHAPE, "K=%lld is not a multiple of 64", (long long)K);
  const int64_t n = E * N * K;
  if (n / E / N != K) return fail(NF4MOE_EOVERFLOW, "E*N*K overflows");
  ok();
  return n / 2 + (n / NF4MOE_BLOCKSIZE) * 4;
}

static int quantize_impl(int qt, const void* w, int w_dtype, int64_t E, int64_t N,
                         int64_t K, int blocksize, uint8_t* packed,
                         float* absmax, int32_t* nonfinite_flag, void* stream) {
  if (w == nullptr || packed == nullptr || (absmax == nullptr && !is_16bit(qt)))
    return fail(NF4MOE_EINVAL, "w, packed and absmax must be non-null");
  if (E < 1 || N < 1 || K < 1)
    return fail(NF4MOE_EINVAL, "E, N, K must be positive (got %lld, %lld, %lld)",
                (long long)E, (long long)N, (long long)K);
  if (blocksize != NF4MOE_BLOCKSIZE)
    return fail(NF4MOE_EBLOCK, "blocksize=%d: only nf4/64 storage is supported", blocksize);
  if (K % NF4MOE_BLOCKSIZE)
    return fail(NF4MOE_ESHAPE, "K=%lld is not a multiple of 64", (long long)K);
  if (w_dtype != NF4MOE_F32 && w_dtype != NF4MOE_BF16)
    return fail(NF4MOE_EDTYPE, "w_dtype=%d: the quantiser takes F32 or BF16", w_dtype);
  const int64_t n = E * N * K;
  if (n / E / N != K || n > ((int64_t)1 << 50))
    return fail(NF4MOE_EOVERFLOW, "E*N*K is too large");
  if (!aligned(w, w_dtype == NF4MOE_F32 ? 16 : 8) || !aligned(packed, is_8bit(qt) ? 4 : 2) ||
      !aligned(absmax, 4) || !aligned(nonfinite_flag, 4))
    return fail(NF4MOE_EINVAL,
                "misaligned buffer (w needs 16 bytes for F32, 8 for BF16; packed 4 bytes for "
                "the 8-bit modes, 2 otherwise; absmax and nonfinite_flag 4)");
  if (is_16bit(qt) && (!aligned(w, 16) || !aligned(packed, 16)))
    return fail(NF4MOE_EINVAL, "passthrough storage needs w and packed 16-byte aligned");
  int cus = 0;
  int st = cu_count(&cus);
  if (st != NF4MOE_OK) return st;
  if (is_16bit(qt)) {
    // passthrough: the weights rounded to the storage type, nothing else
    hipError_t err = launch_to16(w, w_dtype == NF4MOE_BF16, n, qt == kQtBF16,
                                 reinterpret_cast<uint16_t*>(packed), cus, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "passthrough conversion launch");
    return ok();
  }
  hipError_t err = launch_quantize(w, w_dtype, n, packed, absmax, nonfinite_flag,
                                   thresholds(qt), cus, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "quantize launch");
  return ok();
}

int nf4_quantize_experts(const void* w, int w_dtype, int64_t E, int64_t N,
                         int64_t K, int blocksize, uint8_t* packed,
                         float* absmax, int32_t* nonfinite_flag, void* stream) {
  return quantize_impl(kQtNF4, w, w_dtype, E, N, K, blocksize, packed, absmax,
                       nonfinite_flag, stream);
}

int nbit_quantize_experts(int quant_type, const void* w, int w_dtype, int64_t E,
                          int64_t N, int64_t K, int blocksize, uint8_t* packed,
                          float* absmax, int32_t* nonfinite_flag, void* stream) {
  if (!valid_qtype(quant_type)) return fail(NF4MOE_EINVAL, "unknown storage mode %d", quant_type);
  return quantize_impl(quant_type, w, w_dtype, E, N, K, blocksize, packed, absmax,
                       nonfinite_flag, stream);
}

int nf4moe_f16_range_check(const void* t, int dtype, int64_t n, int32_t* flags, void* stream) {
  if (t == nullptr || flags == nullptr) return fail(NF4MOE_EINVAL, "t and flags must be non-null");
  if (n < 1) return fail(NF4MOE_EINVAL, "n=%lld must be positive", (long long)n);
  if (dtype != NF4MOE_BF16 && dtype != NF4MOE_F32)
    return fail(NF4MOE_EDTYPE, "dtype=%d: the range check takes BF16 or F32 values", dtype);
  if (!aligned(t, dtype == NF4MOE_F32 ? 16 : 8) || !aligned(flags, 4))
    return fail(NF4MOE_EINVAL, "misaligned buffer (t needs 16 bytes for F32, 8 for BF16; "
                               "flags 4)");
  int cus = 0;
  int st = cu_count(&cus);
  if (st != NF4MOE_OK) return st;
  hipError_t err = launch_f16_range(t, dtype == NF4MOE_BF16, n, flags, cus, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "range check launch");
  return ok();
}

size_t moe_route_permute_workspace(int64_t T, int E, int k) {
  (void)k;
  if (T < 1 || E < 1 || E > NF4MOE_MAX_EXPERTS) return 0;
  return route_layout(T, E).total;
}

int moe_route_permute(const float* logits, int64_t T, int E, int k,
                      int renormalize, int32_t* topk_ids, float* topk_w,
                      int32_t* sorted_pair, int32_t* pair_pos,
                      int32_t* expert_offsets, void* workspace,
                      size_t ws_bytes, void* stream) {
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr ||
      sorted_pair == nullptr || expert_offsets == nullptr)
    return fail(NF4MOE_EINVAL, "logits, topk_ids, topk_w, sorted_pair and expert_offsets must be non-null");
  int st = check_route_shape(T, E, k);
  if (st != NF4MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1)
    return fail(NF4MOE_EINVAL, "renormalize must be 0 or 1");
  const RouteLayout L = route_layout(T, E);
  if (workspace == nullptr || ws_bytes < L.total)
    return fail(NF4MOE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? ws_bytes : (size_t)0);
  char* ws = (char*)workspace;
  RouteArgs a{};
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.k = k;
  a.renormalize = renormalize;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.sorted_pair = sorted_pair;
  a.pair_pos = pair_pos;
  a.expert_offsets = expert_offsets;
  a.chunk_masks = (uint32_t*)(ws + L.masks);
  a.chunk_base = (int32_t*)(ws + L.base);
  a.x_in = nullptr;
  a.x16 = nullptr;
  hipError_t err = launch_route(a, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "route launch");
  return ok();
}

static int gemm_common(const void* a, int a_dtype, int64_t a_rows, const int32_t* gather,
                       int gather_div, const uint8_t* packed, const float* absmax,
                       const int32_t* expert_offsets, int E, int64_t P, int64_t N, int64_t K,
                       const nf4moe_lora* lora, int epilogue,
                       const float* row_scale, const int32_t* scatter, void* out,
                       int out_dtype, int qt, hipStream_t stream,
                       const void* swiglu_bwd_dh = nullptr, void* swiglu_bwd_h = nullptr,
                       float* swiglu_bwd_u = nullptr) {
  int cus = 0;
  int st = cu_count(&cus);
  if (st != NF4MOE_OK) return st;
  GemmArgs g{};
  g.a = a;
  g.a_rows = a_rows;
  g.a_bf16 = a_dtype == NF4MOE_BF16;
  g.gather = gather;
  g.gather_div = gather ? gather_div : 1;
  g.packed = packed;
  g.absmax = absmax;
  g.offsets = expert_offsets;
  g.E = E;
  g.P = P;
  g.N = (int)N;
  g.K = (int)K;
  if (lora) {
    g.lora_a = lora->A;
    g.lora_b = lora->B;
    g.lora_r = lora->r;
    g.lora_scale = lora->scale;
    g.lora_bf16 = lora->dtype == NF4MOE_BF16;
  }
  g.swiglu = epilogue == NF4MOE_EPI_SWIGLU || swiglu_bwd_dh != nullptr;
  g.dh = swiglu_bwd_dh;
  g.h_out = swiglu_bwd_h;
  g.u_out = swiglu_bwd_u;
  g.row_scale = row_scale;
  g.scatter = scatter;
  g.out = out;
  g.out_dtype = out_dtype;
  g.qtype = qt;
  hipError_t err =
      is_16bit(qt) ? launch_grouped_gemm16(g, cus, stream) : launch_grouped_gemm(g, cus, stream);
  if (err != hipSuccess) return hip_fail(err, "grouped GEMM launch");
  return NF4MOE_OK;
}

static int gemm_impl(int qt, const void* a, int a_dtype, int64_t a_rows,
                     const int32_t* gather, int gather_div,
                     const uint8_t* packed, const float* absmax,
                     const int32_t* expert_offsets, int E, int64_t P,
                     int64_t N, int64_t K, const nf4moe_lora* lora,
                     int epilogue, const float* row_scale,
                     const int32_t* scatter, void* out, int out_dtype,
                     void* stream) {
  if (a == nullptr || packed == nullptr || (absmax == nullptr && !is_16bit(qt)) ||
      expert_offsets == nullptr || out == nullptr)
    return fail(NF4MOE_EINVAL, "a, packed, absmax, expert_offsets and out must be non-null");
  if (E < 1 || E > NF4MOE_MAX_EXPERTS)
    return fail(E < 1 ? NF4MOE_EINVAL : NF4MOE_ESHAPE, "E=%d outside [1, %d]", E,
                NF4MOE_MAX_EXPERTS);
  if (P < 0 || a_rows < 0) return fail(NF4MOE_EINVAL, "P and a_rows must be >= 0");
  if (N < 16 || K < 64) return fail(NF4MOE_EINVAL, "N >= 16 and K >= 64 required");
  if (K % NF4MOE_BLOCKSIZE) return fail(NF4MOE_ESHAPE, "K=%lld is not a multiple of 64", (long long)K);
  if (N % 16) return fail(NF4MOE_ESHAPE, "N=%lld is not a multiple of 16", (long long)N);
  if (epilogue != NF4MOE_EPI_NONE && epilogue != NF4MOE_EPI_SWIGLU)
    return fail(NF4MOE_EINVAL, "unknown epilogue %d", epilogue);
  if (epilogue == NF4MOE_EPI_SWIGLU && N % 32)
    return fail(NF4MOE_ESHAPE, "SwiGLU needs N=2I with I a multiple of 16 (N=%lld)", (long long)N);
  if (a_dtype != NF4MOE_F16 && a_dtype != NF4MOE_BF16)
    return fail(NF4MOE_EDTYPE, "a_dtype=%d: activations must be F16 or BF16", a_dtype);
  if (out_dtype != NF4MOE_F16 && out_dtype != NF4MOE_BF16 && out_dtype != NF4MOE_F32)
    return fail(NF4MOE_EDTYPE, "out_dtype=%d unsupported", out_dtype);
  if (gather != nullptr && gather_div < 1)
    return fail(NF4MOE_EINVAL, "gather_div must be >= 1");
  if (P >= INT32_MAX || N > INT32_MAX / 2 || K > INT32_MAX / 2)
    return fail(NF4MOE_EOVERFLOW, "P, N or K too large for 32-bit row indexing");
  // the kernel addresses activations and one expert's weights with 32-bit
  // byte offsets
  if (a_rows * K * 2 > (int64_t)UINT32_MAX ||
      N * K * bytes_x2(qt) / 2 > (int64_t)UINT32_MAX)
    return fail(NF4MOE_EOVERFLOW, "activations or one expert's stack exceed 4 GiB");
  if (lora != nullptr && (is_8bit(qt) || is_16bit(qt) || qt == kQtMXFP4))
    return fail(NF4MOE_EINVAL, "adapters are supported on nf4 and fp4 stacks only");
  int st = check_lora(lora, "lora");
  if (st != NF4MOE_OK) return st;
  if (!aligned(a, 16) || !aligned(packed, 16) || !aligned(absmax, 4) ||
      !aligned(out, 16))
    return fail(NF4MOE_EINVAL, "misaligned buffer (a, packed and out need 16 bytes)");
  if (P == 0) return ok();
  st = gemm_common(a, a_dtype, a_rows, gather, gather_div, packed, absmax, expert_offsets,
                   E, P, N, K, lora, epilogue, row_scale, scatter, out, out_dtype, qt,
                   (hipStream_t)stream);
  if (st != NF4MOE_OK) return st;
  return ok();
}

int grouped_nf4_gemm(const void* a, int a_dtype, int64_t a_rows,
                     const int32_t* gather, int gather_div,
                     const uint8_t* packed, const float* absmax,
                     const int32_t* expert_offsets, int E, int64_t P,
                     int64_t N, int64_t K, const nf4moe_lora* lora,
                     int epilogue, const float* row_scale,
                     const int32_t* scatter, void* out, int out_dtype,
                     void* stream) {
  return gemm_impl(kQtNF4, a, a_dtype, a_rows, gather, gather_div, packed, absmax,
                   expert_offsets, E, P, N, K, lora, epilogue, row_scale, scatter, out,
                   out_dtype, stream);
}

int grouped_nbit_gemm(int quant_type, const void* a, int a_dtype, int64_t a_rows,
                      const int32_t* gather, int gather_div,
                      const uint8_t* packed, const float* absmax,
                      const int32_t* expert_offsets, int E, int64_t P,
                      int64_t N, int64_t K, const nf4moe_lora* lora,
                      int epilogue, const float* row_scale,
                      const int32_t* scatter, void* out, int out_dtype,
                      void* stream) {
  if (!valid_qtype(quant_type)) return fail(NF4MOE_EINVAL, "unknown storage mode %d", quant_type);
  return gemm_impl(quant_type, a, a_dtype, a_rows, gather, gather_div, packed, absmax,
                   expert_offsets, E, P, N, K, lora, epilogue, row_scale, scatter, out,
                   out_dtype, stream);
}

int grouped_nf4_gemm_swiglu_bwd(const void* a, int64_t a_rows, const int32_t* gather,
                                int gather_div, const uint8_t* packed, const float* absmax,
                                const int32_t* expert_offsets, int E, int64_t P, int64_t N,
                                int64_t K, const nf4moe_lora* lora, const void* dh, void* out,
                                void* h_out, void* stream) {
  if (dh == nullptr) return fail(NF4MOE_EINVAL, "dh must be non-null");
  if (!aligned(dh, 16) || !aligned(h_out, 16))
    return fail(NF4MOE_EINVAL, "misaligned buffer (dh and h_out need 16 bytes)");
  if (a == nullptr || packed == nullptr || absmax == nullptr || expert_offsets == nullptr ||
      out == nullptr)
    return fail(NF4MOE_EINVAL, "a, packed, absmax, expert_offsets and out must be non-null");
  // the shape, dtype, alignment and size checks of the SwiGLU GEMM
  int st = gemm_impl(kQtNF4, a, NF4MOE_F16, a_rows, gather, gather_div, packed, absmax,
                     expert_offsets, E, /*P=*/0, N, K, lora, NF4MOE_EPI_SWIGLU, nullptr,
                     nullptr, out, NF4MOE_F16, stream);
  if (st != NF4MOE_OK) return st;
  if (P < 0) return fail(NF4MOE_EINVAL, "P must be >= 0");
  if (P >= INT32_MAX) return fail(NF4MOE_EOVERFLOW, "P too large for 32-bit row indexing");
  if (P == 0) return ok();
  st = gemm_common(a, NF4MOE_F16, a_rows, gather, gather_div, packed, absmax, expert_offsets,
                   E, P, N, K, lora, NF4MOE_EPI_SWIGLU, nullptr, nullptr, out, NF4MOE_F16,
                   kQtNF4, (hipStream_t)stream, dh, h_out);
  if (st != NF4MOE_OK) return st;
  return ok();
}

size_t moe_expert_forward_workspace(int64_t T, int H, int I, int E, int k, int r) {
  if (T < 1 || H < 1 || I < 1 || E < 1 || E > NF4MOE_MAX_EXPERTS || k < 1) return 0;
  if (r < 0 || r > NF4MOE_MAX_LORA_R) return 0;
  return fwd_layout(T, H, I, E, k, r).total;
}

int moe_expert_forward_routing(void* workspace, int64_t T, int H, int I, int E,
                               int k, int32_t** topk_ids, float** topk_w,
                               int32_t** sorted_pair, int32_t** expert_offsets) {
  if (workspace == nullptr) return fail(NF4MOE_EINVAL, "workspace is NULL");
  int st = check_route_shape(T, E, k);
  if (st != NF4MOE_OK) return st;
  if (H < 1 || I < 1) return fail(NF4MOE_EINVAL, "H and I must be positive");
  const FwdLayout L = fwd_layout(T, H, I, E, k);
  char* ws = (char*)workspace;
  if (topk_ids) *topk_ids = (int32_t*)(ws + L.ids);
  if (topk_w) *topk_w = (float*)(ws + L.w);
  if (sorted_pair) *sorted_pair = (int32_t*)(ws + L.sorted);
  if (expert_offsets) *expert_offsets = (int32_t*)(ws + L.offsets);
  return ok();
}

static int forward_impl(int qt, const void* x, int x_dtype, const float* router_logits,
                       int64_t T, int H, int I, int E, int k, int renormalize,
                       const uint8_t* gu_packed, const float* gu_absmax,
                       const uint8_t* dn_packed, const float* dn_absmax,
                       const nf4moe_lora* gu_lora, const nf4moe_lora* dn_lora,
                       void* y, int y_dtype, void* workspace, size_t ws_bytes,
                       void* stream) {
  if (x == nullptr || router_logits == nullptr || gu_packed == nullptr ||
      dn_packed == nullptr || y == nullptr ||
      (!is_16bit(qt) && (gu_absmax == nullptr || dn_absmax == nullptr)))
    return fail(NF4MOE_EINVAL, "x, router_logits, the four stack buffers and y must be non-null");
  int st = check_route_shape(T, E, k);
  if (st != NF4MOE_OK) return st;
  if (H < 64 || I < 64) return fail(NF4MOE_EINVAL, "H and I must be >= 64");
  if (H % 64 || I % 64)
    return fail(NF4MOE_ESHAPE, "H=%d and I=%d must be multiples of 64", H, I);
  if (renormalize != 0 && renormalize != 1)
    return fail(NF4MOE_EINVAL, "renormalize must be 0 or 1");
  if (x_dtype != NF4MOE_BF16 && x_dtype != NF4MOE_F16)
    return fail(NF4MOE_EDTYPE, "x_dtype=%d: activations must be BF16 or F16", x_dtype);
  if (y_dtype != NF4MOE_BF16 && y_dtype != NF4MOE_F16 && y_dtype != NF4MOE_F32)
    return fail(NF4MOE_EDTYPE, "y_dtype=%d unsupported", y_dtype);
  st = check_lora(gu_lora, "gu_lora");
  if (st != NF4MOE_OK) return st;
  st = check_lora(dn_lora, "dn_lora");
  if (st != NF4MOE_OK) return st;
  const int64_t P = T * k;
  // the GEMMs address activations and one expert's weights with 32-bit byte
  // offsets
  if (T * H * 2 > (int64_t)UINT32_MAX || P * I * 2 > (int64_t)UINT32_MAX ||
      2 * (int64_t)I * H * bytes_x2(qt) / 2 > (int64_t)UINT32_MAX)
    return fail(NF4MOE_EOVERFLOW, "activations or one expert's stack exceed 4 GiB");
  if (!aligned(x, 16) || !aligned(gu_packed, 16) || !aligned(dn_packed, 16) ||
      !aligned(gu_absmax, 4) || !aligned(dn_absmax, 4) || !aligned(y, 16))
    return fail(NF4MOE_EINVAL, "misaligned buffer (x, y and packed stacks need 16 bytes)");
  const int r_ws = std::max(gu_lora ? gu_lora->r : 0, dn_lora ? dn_lora->r : 0);
  const FwdLayout L = fwd_layout(T, H, I, E, k, r_ws);
  if (workspace == nullptr || ws_bytes < L.total)
    return fail(NF4MOE_EWORKSPACE, "workspace of %zu bytes needed (adapter rank %d), %zu given",
                L.total, r_ws, workspace ? ws_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(NF4MOE_EINVAL, "workspace must be 256-byte aligned");
  int cus = 0;
  st = cu_count(&cus);
  if (st != NF4MOE_OK) return st;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  int32_t* ids = (int32_t*)(ws + L.ids);
  float* wts = (float*)(ws + L.w);

  if ((gu_lora != nullptr || dn_lora != nullptr) &&
      (is_8bit(qt) || is_16bit(qt) || qt == kQtMXFP4))
    return fail(NF4MOE_EINVAL, "adapters are supported on nf4 and fp4 stacks only");
  if (!is_8bit(qt) && !is_16bit(qt) && use_decode_path(T, H, I, k, gu_lora, dn_lora)) {
    GemvArgs g{};
    g.x = x;
    g.x_bf16 = x_dtype == NF4MOE_BF16;
    g.logits = router_logits;
    g.E = E;
    g.k = k;
    g.renormalize = renormalize;
    g.H = H;
    g.I = I;
    g.gu_packed = gu_packed;
    g.gu_absmax = gu_absmax;
    g.dn_packed = dn_packed;
    g.dn_absmax = dn_absmax;
    g.topk_ids = ids;
    g.topk_w = wts;
    g.sorted_pair = (int32_t*)(ws + L.sorted);
    g.expert_offsets = (int32_t*)(ws + L.offsets);
    g.barrier = (uint64_t*)(ws + L.bar);
    g.spin_limit = kDecodeSpinLimit;
    g.y = y;
    g.y_dtype = y_dtype;
    g.qtype = qt;
    hipError_t err = launch_decode(g, cus, s);
    if (err != hipSuccess) return hip_fail(err, "decode launch");
    return ok();
  }

  RouteArgs r{};
  r.logits = router_logits;
  r.T = T;
  r.E = E;
  r.k = k;
  r.renormalize = renormalize;
  r.topk_ids = ids;
  r.topk_w = wts;
  r.sorted_pair = (int32_t*)(ws + L.sorted);
  r.pair_pos = (int32_t*)(ws + L.pos);
  r.expert_offsets = (int32_t*)(ws + L.offsets);
  r.chunk_masks = (uint32_t*)(ws + L.route + L.r.masks);
  r.chunk_base = (int32_t*)(ws + L.route + L.r.base);
  // bf16 activations go to fp16 once for the GEMMs, except on a bf16
  // passthrough stack, whose gate_up multiplies bf16 by bf16 as stored
  const bool conv = x_dtype == NF4MOE_BF16 && qt != kQtBF16;
  r.x_in = x;
  r.x_bf16 = conv ? 1 : 0;
  r.x16 = conv ? (_Float16*)(ws + L.x16) : nullptr;
  r.H = H;
  r.num_cus = cus;
  hipError_t err = launch_route(r, s);
  if (err != hipSuccess) return hip_fail(err, "route launch");

  // bf16 adapters: fp16 copies, made once here, so the GEMMs' k-loops read
  // fp16 adapter rows (the same rounding as converting them in the loop)
  HalfCopies hc{};
  nf4moe_lora gu16{}, dn16{};
  auto to_f16 = [&](const nf4moe_lora* l, size_t a_off, size_t b_off, int kdim, int n,
                    nf4moe_lora* out) -> const nf4moe_lora* {
    if (l == nullptr || l->dtype != NF4MOE_BF16) return l;
    *out = *l;
    out->A = ws + a_off;
    out->B = ws + b_off;
    out->dtype = NF4MOE_F16;
    const int64_t na = (int64_t)E * l->r * kdim, nb = (int64_t)E * n * l->r;
    hc.src[hc.count] = (const uint16_t*)l->A;
    hc.dst[hc.count] = (_Float16*)(ws + a_off);
    hc.n8[hc.count++] = na / 8;
    hc.src[hc.count] = (const uint16_t*)l->B;
    hc.dst[hc.count] = (_Float16*)(ws + b_off);
    hc.n8[hc.count++] = nb / 8;
    return out;
  };
  const nf4moe_lora* gu_l = to_f16(gu_lora, L.a_gu, L.b_gu, H, 2 * I, &gu16);
  const nf4moe_lora* dn_l = to_f16(dn_lora, L.a_dn, L.b_dn, I, H, &dn16);
  if (hc.count > 0) {
    err = launch_half_copies(hc, cus, s);
    if (err != hipSuccess) return hip_fail(err, "adapter conversion launch");
  }

  const void* xa = conv ? (const void*)(ws + L.x16) : x;
  const int xa_dtype = conv ? NF4MOE_F16 : x_dtype;
  _Float16* h = (_Float16*)(ws + L.h);
  _Float16* o = (_Float16*)(ws + L.o);
  st = gemm_common(xa, xa_dtype, T, r.sorted_pair, k, gu_packed, gu_absmax,
                   r.expert_offsets, E, P, 2 * (int64_t)I, H, gu_l,
                   NF4MOE_EPI_SWIGLU, nullptr, nullptr, h, NF4MOE_F16, qt, s);
  if (st != NF4MOE_OK) return st;
  st = gemm_common(h, NF4MOE_F16, P, nullptr, 1, dn_packed, dn_absmax, r.expert_offsets,
                   E, P, H, I, dn_l, NF4MOE_EPI_NONE, nullptr,
                   r.sorted_pair, o, NF4MOE_F16, qt, s);
  if (st != NF4MOE_OK) return st;
  err = launch_combine(o, wts, T, k, H, y, y_dtype, cus, s);
  if (err != hipSuccess) return hip_fail(err, "combine launch");
  return ok();
}

int moe_expert_forward(const void* x, int x_dtype, const float* router_logits,
                       int64_t T, int H, int I, int E, int k, int renormalize,
                       const uint8_t* gu_packed, const float* gu_absmax,
                       const uint8_t* dn_packed, const float* dn_absmax,
                       const nf4moe_lora* gu_lora, const nf4moe_lora* dn_lora,
                       void* y, int y_dtype, void* workspace, size_t ws_bytes,
                       void* stream) {
  return forward_impl(kQtNF4, x, x_dtype, router_logits, T, H, I, E, k, renormalize,
                      gu_packed, gu_absmax, dn_packed, dn_absmax, gu_lora, dn_lora, y,
                      y_dtype, workspace, ws_bytes, stream);
}

int moe_expert_forward_nbit(int quant_type, const void* x, int x_dtype,
                            const float* router_logits, int64_t T, int H, int I, int E,
                            int k, int renormalize, const uint8_t* gu_packed,
                            const float* gu_absmax, const uint8_t* dn_packed,
                            const float* dn_absmax, const nf4moe_lora* gu_lora,
                            const nf4moe_lora* dn_lora, void* y, int y_dtype,
                            void* workspace, size_t ws_bytes, void* stream) {
  if (!valid_qtype(quant_type)) return fail(NF4MOE_EINVAL, "unknown storage mode %d", quant_type);
  return forward_impl(quant_type, x, x_dtype, router_logits, T, H, I, E, k, renormalize,
                      gu_packed, gu_absmax, dn_packed, dn_absmax, gu_lora, dn_lora, y,
                      y_dtype, workspace, ws_bytes, stream);
}

// ---- grouped dgrad ------------------------------------------------------

static int dgrad_common(const void* a, int a_dtype, int64_t a_rows, const int32_t* gather,
                        int gather_div, const uint8_t* packed, const float* absmax,
                        const int32_t* expert_offsets, int E, int64_t P, int64_t N, int64_t K,
                        int epilogue, const void* g_pre, int g_dtype, const float* row_scale,
                        const int32_t* rs_idx, const int32_t* scatter, const float* lora_v,
                        const nf4moe_lora* lora, void* out, int out_dtype, int qt,
                        hipStream_t stream, const _Float16* lora_bt = nullptr,
                        float* lora_v_out = nullptr) {
  int cus = 0;
  int st = cu_count(&cus);
  if (st != NF4MOE_OK) return st;
  DgradArgs d{};
  d.a = a;
  d.a_rows = a_rows;
  d.a_bf16 = a_dtype == NF4MOE_BF16;
  d.gather = gather;
  d.gather_div = gather ? gather_div : 1;
  d.packed = packed;
  d.absmax = absmax;
  d.offsets = expert_offsets;
  d.E = E;
  d.P = P;
  d.N = (int)N;
  d.K = (int)K;
  d.row_scale = row_scale;
  d.rs_idx = rs_idx;
  d.scatter = scatter;
  d.epilogue = epilogue == NF4MOE_EPI_SWIGLU_BWD ? kDgradEpiSwigluBwd : kDgradEpiNone;
  d.g = g_pre;
  d.g_bf16 = g_dtype == NF4MOE_BF16;
  if ((lora_v != nullptr || lora_bt != nullptr) && lora != nullptr) {
    d.lora_v = lora_v;
    d.lora_bt = lora_bt;
    d.lora_v_out = lora_v_out;
    d.lora_a = lora->A;
    d.lora_r = lora->r;
    d.lora_scale = lora->scale;
    d.lora_bf16 = lora->dtype == NF4MOE_BF16;
  }
  d.out = out;
  d.out_dtype = out_dtype;
  d.qtype = qt;
  hipError_t err = launch_grouped_dgrad(d, cus, stream);
  if (err != hipSuccess) return hip_fail(err, "grouped dgrad launch");
  return NF4MOE_OK;
}

static int dgrad_impl(int qt, const void* a, int a_dtype, int64_t a_rows,
                      const int32_t* gather, int gather_div, const uint8_t* packed,
                      const float* absmax, const int32_t* expert_offsets, int E, int64_t P,
                      int64_t N, int64_t K, int epilogue, const void* g_pre, int g_dtype,
                      const float* row_scale, const int32_t* scatter, void* out,
                      int out_dtype, void* stream) {
  if (a == nullptr || packed == nullptr || absmax == nullptr || expert_offsets == nullptr ||
      out == nullptr)
    return fail(NF4MOE_EINVAL, "a, packed, absmax, expert_offsets and out must be non-null");
  if (E < 1 || E > NF4MOE_MAX_EXPERTS)
    return fail(E < 1 ? NF4MOE_EINVAL : NF4MOE_ESHAPE, "E=%d outside [1, %d]", E,
                NF4MOE_MAX_EXPERTS);
  if (P < 0 || a_rows < 0) return fail(NF4MOE_EINVAL, "P and a_rows must be >= 0");
  if (N < 64 || K < 64) return fail(NF4MOE_EINVAL, "N >= 64 and K >= 64 required");
  if (N % 64 || K % 64)
    return fail(NF4MOE_ESHAPE, "N=%lld and K=%lld must be multiples of 64", (long long)N,
                (long long)K);
  if (epilogue != NF4MOE_EPI_NONE && epilogue != NF4MOE_EPI_SWIGLU_BWD)
    return fail(NF4MOE_EINVAL, "unknown dgrad epilogue %d", epilogue);
  if (epilogue == NF4MOE_EPI_SWIGLU_BWD) {
    if (g_pre == nullptr) return fail(NF4MOE_EINVAL, "the SwiGLU backward needs g_pre");
    if (g_dtype != NF4MOE_F16 && g_dtype != NF4MOE_BF16)
      return fail(NF4MOE_EDTYPE, "g_dtype=%d: the pre-activation must be F16 or BF16", g_dtype);
    if (!aligned(g_pre, 16)) return fail(NF4MOE_EINVAL, "g_pre must be 16-byte aligned");
  }
  if (a_dtype != NF4MOE_F16 && a_dtype != NF4MOE_BF16)
    return fail(NF4MOE_EDTYPE, "a_dtype=%d: gradient rows must be F16 or BF16", a_dtype);
  if (out_dtype != NF4MOE_F16 && out_dtype != NF4MOE_BF16 && out_dtype != NF4MOE_F32)
    return fail(NF4MOE_EDTYPE, "out_dtype=%d unsupported", out_dtype);
  if (gather != nullptr && gather_div < 1) return fail(NF4MOE_EINVAL, "gather_div must be >= 1");
  if (P >= INT32_MAX || N > INT32_MAX / 2 || K > INT32_MAX / 4)
    return fail(NF4MOE_EOVERFLOW, "P, N or K too large for 32-bit row indexing");
  if (a_rows * N * 2 > (int64_t)UINT32_MAX || N * K / 2 > (int64_t)UINT32_MAX)
    return fail(NF4MOE_EOVERFLOW, "gradient rows or one expert's stack exceed 4 GiB");
  if (!aligned(a, 16) || !aligned(packed, 16) || !aligned(absmax, 4) || !aligned(out, 16))
    return fail(NF4MOE_EINVAL, "misaligned buffer (a, packed and out need 16 bytes)");
  if (P == 0) return ok();
  int st = dgrad_common(a, a_dtype, a_rows, gather, gather_div, packed, absmax,
                        expert_offsets, E, P, N, K, epilogue, g_pre, g_dtype, row_scale,
                        nullptr, scatter, nullptr, nullptr, out, out_dtype, qt,
                        (hipStream_t)stream);
  if (st != NF4MOE_OK) return st;
  return ok();
}

int grouped_nf4_gemm_dgrad(const void* a, int a_dtype, int64_t a_rows, const int32_t* gather,
                           int gather_div, const uint8_t* packed, const float* absmax,
                           const int32_t* expert_offsets, int E, int64_t P, int64_t N,
                           int64_t K, int epilogue, const void* g_pre, int g_dtype,
                           const float* row_scale, const int32_t* scatter, void* out,
                           int out_dtype, void* stream) {
  return dgrad_impl(kQtNF4, a, a_dtype, a_rows, gather, gather_div, packed, absmax,
                    expert_offsets, E, P, N, K, epilogue, g_pre, g_dtype, row_scale, scatter,
                    out, out_dtype, stream);
}

int grouped_nbit_gemm_dgrad(int quant_type, const void* a, int a_dtype, int64_t a_rows,
                            const int32_t* gather, int gather_div, const uint8_t* packed,
                            const float* absmax, const int32_t* expert_offsets, int E,
                            int64_t P, int64_t N, int64_t K, int epilogue, const void* g_pre,
                            int g_dtype, const float* row_scale, const int32_t* scatter,
                            void* out, int out_dtype, void* stream) {
  if (quant_type != kQtNF4 && quant_type != kQtFP4)
    return fail(NF4MOE_EINVAL, "storage mode %d: the dgrad takes nf4 or fp4 stacks", quant_type);
  return dgrad_impl(quant_type, a, a_dtype, a_rows, gather, gather_div, packed, absmax,
                    expert_offsets, E, P, N, K, epilogue, g_pre, g_dtype, row_scale, scatter,
                    out, out_dtype, stream);
}

// ---- layer backward -----------------------------------------------------

struct BwdLayout {
  FwdLayout f;  // routing regions and x16 (h and o unused)
  size_t dy16, g, dg, dxp, h, u_gu, v_gu, u_dn, v_dn, a16_gu, bt_gu, a16_dn, bt_dn, b16_gu, part,
      total;
};

static BwdLayout bwd_layout(int64_t T, int H, int I, int E, int k, int r) {
  BwdLayout L;
  L.f = fwd_layout(T, H, I, E, k);
  const size_t P = (size_t)T * k;
  size_t o = L.f.total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.dy16 = take((size_t)T * H * 2);
  L.g = take(P * 2 * (size_t)I * 2);
  L.dg = take(P * 2 * (size_t)I * 2);
  L.dxp = take(P * (size_t)H * 2);
  const size_t rr = (size_t)(r > 0 ? r : 0);
  L.h = take(rr ? P * (size_t)I * 2 : 0);
  L.u_gu = take(P * rr * 4);
  L.v_gu = take(P * rr * 4);
  L.u_dn = take(P * rr * 4);
  L.v_dn = take(P * rr * 4);
  L.a16_gu = take((size_t)E * rr * H * 2);
  L.bt_gu = take((size_t)E * rr * 2 * I * 2);
  L.a16_dn = take((size_t)E * rr * I * 2);
  L.bt_dn = take((size_t)E * rr * H * 2);
  L.b16_gu = take((size_t)E * 2 * I * rr * 2);  // B_gu as fp16 [E, 2I, r] (recompute)
  const size_t cmax = (size_t)(H > 2 * I ? H : 2 * I);
  L.part = take(rr ? ((P + 63) / 64 + (size_t)E) * rr * cmax * 4 : 0);
  L.total = o;
  return L;
}

size_t moe_expert_backward_workspace(int64_t T, int H, int I, int E, int k, int r) {
  if (T < 1 || H < 1 || I < 1 || E < 1 || E > NF4MOE_MAX_EXPERTS || k < 1 || r < 0 ||
      r > NF4MOE_MAX_LORA_R)
    return 0;
  return bwd_layout(T, H, I, E, k, r).total;
}

// One LoRA pass over the rows of m: the projection onto w (out non-null)
// and/or the weight gradient from q (z non-null; part is scratch).
static int lora_pass(const void* m, int m_bf16, const int32_t* gather, int gather_div,
                     const int32_t* offsets, int E, int64_t P, int C, int r,
                     const _Float16* w, float* out, const float* rs, const int32_t* rs_idx,
                     const float* q, float* part, float* z, float scale, int rank_major,
                     int cus, hipStream_t s) {
  LoraPassArgs a{};
  a.m = m;
  a.m_bf16 = m_bf16;
  a.gather = gather;
  a.gather_div = gather ? gather_div : 1;
  a.offsets = offsets;
  a.E = E;
  a.P = P;
  a.C = C;
  a.r = r;
  a.w = w;
  a.out = out;
  a.rs = rs;
  a.rs_idx = rs_idx;
  a.q = q;
  a.part = z ? part : nullptr;
  a.z = z;
  a.scale = scale;
  a.rank_major = rank_major;
  hipError_t err = launch_lora_pass(a, cus, s);
  if (err != hipSuccess) return hip_fail(err, "LoRA pass launch");
  return NF4MOE_OK;
}

static int backward_impl(int qt, const void* x, int x_dtype, const float* router_logits,
                         const void* dy, int dy_dtype, int64_t T, int H, int I, int E, int k,
                         int renormalize, const uint8_t* gu_packed, const float* gu_absmax,
                         const uint8_t* dn_packed, const float* dn_absmax,
                         const nf4moe_lora* gu_lora, const nf4moe_lora* dn_lora, void* dx,
                         int dx_dtype, float* d_gu_A, float* d_gu_B, float* d_dn_A,
                         float* d_dn_B, void* workspace, size_t ws_bytes, void* stream) {
  if (x == nullptr || router_logits == nullptr || dy == nullptr || gu_packed == nullptr ||
      gu_absmax == nullptr || dn_packed == nullptr || dn_absmax == nullptr || dx == nullptr)
    return fail(NF4MOE_EINVAL, "x, router_logits, dy, the four stack buffers and dx must be non-null");
  int st = check_route_shape(T, E, k);
  if (st != NF4MOE_OK) return st;
  if (H < 64 || I < 64) return fail(NF4MOE_EINVAL, "H and I must be >= 64");
  if (H % 64 || I % 64)
    return fail(NF4MOE_ESHAPE, "H=%d and I=%d must be multiples of 64", H, I);
  if (renormalize != 0 && renormalize != 1)
    return fail(NF4MOE_EINVAL, "renormalize must be 0 or 1");
  if (x_dtype != NF4MOE_BF16 && x_dtype != NF4MOE_F16)
    return fail(NF4MOE_EDTYPE, "x_dtype=%d: activations must be BF16 or F16", x_dtype);
  if (dy_dtype != NF4MOE_BF16 && dy_dtype != NF4MOE_F16)
    return fail(NF4MOE_EDTYPE, "dy_dtype=%d: the output gradient must be BF16 or F16", dy_dtype);
  if (dx_dtype != NF4MOE_BF16 && dx_dtype != NF4MOE_F16 && dx_dtype != NF4MOE_F32)
    return fail(NF4MOE_EDTYPE, "dx_dtype=%d unsupported", dx_dtype);
  st = check_lora(gu_lora, "gu_lora");
  if (st != NF4MOE_OK) return st;
  st = check_lora(dn_lora, "dn_lora");
  if (st != NF4MOE_OK) return st;
  if (gu_lora && (d_gu_A == nullptr || d_gu_B == nullptr))
    return fail(NF4MOE_EINVAL, "gu_lora given: d_gu_A and d_gu_B must be non-null");
  if (dn_lora && (d_dn_A == nullptr || d_dn_B == nullptr))
    return fail(NF4MOE_EINVAL, "dn_lora given: d_dn_A and d_dn_B must be non-null");
  if (gu_lora && dn_lora && gu_lora->r != dn_lora->r)
    return fail(NF4MOE_EINVAL, "gu_lora and dn_lora must have the same rank");
  const int r = gu_lora ? gu_lora->r : (dn_lora ? dn_lora->r : 0);
  const int64_t P = T * k;
  if (T * H * 2 > (int64_t)UINT32_MAX || P * 2 * (int64_t)I * 2 > (int64_t)UINT32_MAX ||
      2 * (int64_t)I * H / 2 > (int64_t)UINT32_MAX)
    return fail(NF4MOE_EOVERFLOW, "activations or one expert's stack exceed 4 GiB");
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(gu_packed, 16) ||
      !aligned(dn_packed, 16) || !aligned(gu_absmax, 4) || !aligned(dn_absmax, 4) ||
      !aligned(dx, 16))
    return fail(NF4MOE_EINVAL, "misaligned buffer (x, dy, dx and packed stacks need 16 bytes)");
  const BwdLayout L = bwd_layout(T, H, I, E, k, r);
  if (workspace == nullptr || ws_bytes < L.total)
    return fail(NF4MOE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(NF4MOE_EINVAL, "workspace must be 256-byte aligned");
  int cus = 0;
  st = cu_count(&cus);
  if (st != NF4MOE_OK) return st;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;

  // 1. routing (recomputed from the same logits), x in fp16
  RouteArgs ra{};
  ra.logits = router_logits;
  ra.T = T;
  ra.E = E;
  ra.k = k;
  ra.renormalize = renormalize;
  ra.topk_ids = (int32_t*)(ws + L.f.ids);
  ra.topk_w = (float*)(ws + L.f.w);
  ra.sorted_pair = (int32_t*)(ws + L.f.sorted);
  ra.pair_pos = (int32_t*)(ws + L.f.pos);
  ra.expert_offsets = (int32_t*)(ws + L.f.offsets);
  ra.chunk_masks = (uint32_t*)(ws + L.f.route + L.f.r.masks);
  ra.chunk_base = (int32_t*)(ws + L.f.route + L.f.r.base);
  const bool conv = x_dtype == NF4MOE_BF16;
  ra.x_in = x;
  ra.x_bf16 = conv ? 1 : 0;
  ra.x16 = conv ? (_Float16*)(ws + L.f.x16) : nullptr;
  ra.H = H;
  ra.num_cus = cus;
  hipError_t err = launch_route(ra, s);
  if (err != hipSuccess) return hip_fail(err, "route launch");
  const void* xa = conv ? (const void*)(ws + L.f.x16) : x;
  const int32_t* sorted = ra.sorted_pair;
  const int32_t* offs = ra.expert_offsets;
  const float* wts = ra.topk_w;
  _Float16* G = (_Float16*)(ws + L.g);
  _Float16* dG = (_Float16*)(ws + L.dg);
  _Float16* dXp = (_Float16*)(ws + L.dxp);
  _Float16* hbuf = (_Float16*)(ws + L.h);
  float* u_gu = (float*)(ws + L.u_gu);
  float* v_gu = (float*)(ws + L.v_gu);
  float* u_dn = (float*)(ws + L.u_dn);
  float* v_dn = (float*)(ws + L.v_dn);
  _Float16* a16_gu = (_Float16*)(ws + L.a16_gu);
  _Float16* bt_gu = (_Float16*)(ws + L.bt_gu);
  _Float16* a16_dn = (_Float16*)(ws + L.a16_dn);
  _Float16* bt_dn = (_Float16*)(ws + L.bt_dn);
  float* part = (float*)(ws + L.part);
  // the output gradient in fp16 (the dgrad and LoRA passes read fp16 rows)
  const void* dyh = dy;
  if (dy_dtype == NF4MOE_BF16) {
    err = launch_bf16_to_f16(dy, T * H, (_Float16*)(ws + L.dy16), cus, s);
    if (err != hipSuccess) return hip_fail(err, "conversion launch");
    dyh = ws + L.dy16;
  }

  // 2. the gate_up adapter of the recompute: bf16 adapters go to fp16 once
  //    here (A_gu and B_gu), so the recompute's k-loop reads fp16 adapter
  //    rows (the same rounding the GEMM would apply)
  nf4moe_lora gu16{};
  const nf4moe_lora* gu_rc = gu_lora;
  if (gu_lora) {
    const int bf = gu_lora->dtype == NF4MOE_BF16;
    if (bf) {
      err = launch_lora_to_f16(gu_lora->A, bf, 0, E, H, r, a16_gu, cus, s);
      if (err != hipSuccess) return hip_fail(err, "LoRA conversion launch");
      HalfCopies hc{};
      hc.src[0] = (const uint16_t*)gu_lora->B;
      hc.dst[0] = (_Float16*)(ws + L.b16_gu);
      hc.n8[0] = (int64_t)E * 2 * I * r / 8;
      hc.count = 1;
      err = launch_half_copies(hc, cus, s);
      if (err != hipSuccess) return hip_fail(err, "LoRA conversion launch");
      gu16 = *gu_lora;
      gu16.A = a16_gu;
      gu16.B = ws + L.b16_gu;
      gu16.dtype = NF4MOE_F16;
      gu_rc = &gu16;
    }
  }

  // 3. with a down adapter: A_dn and B_dn to fp16 (B_dn transposed)
  if (dn_lora) {
    const int bf = dn_lora->dtype == NF4MOE_BF16;
    err = launch_lora_to_f16(dn_lora->A, bf, 0, E, I, r, a16_dn, cus, s);
    if (err == hipSuccess) err = launch_lora_to_f16(dn_lora->B, bf, 1, E, H, r, bt_dn, cus, s);
    if (err != hipSuccess) return hip_fail(err, "LoRA conversion launch");
  }

  // 4. dH = dy_t W_dn (+ s v' A_dn) for a unit routing weight, fp16 (in
  //    G's space: G itself never goes to memory).  Everything downstream is
  //    linear in w, so w is applied later as a row scale: stored fp16
  //    gradients then keep their precision however small a pair's weight is.
  //    With a down adapter the dgrad's k-loop, which reads the dy rows
  //    anyway, also computes v' = dy B_dn (without the routing weight) and
  //    writes it out for dA_dn
  _Float16* dH = G;
  st = dgrad_common(dyh, NF4MOE_F16, T, sorted, k, dn_packed, dn_absmax, offs, E, P, H, I,
                    NF4MOE_EPI_NONE, nullptr, NF4MOE_F16, nullptr, nullptr, nullptr, nullptr,
                    dn_lora, dH, NF4MOE_F16, qt, s, dn_lora ? bt_dn : nullptr,
                    dn_lora ? v_dn : nullptr);
  if (st != NF4MOE_OK) return st;

  // 5. G = x W_gu^T (+ LoRA) recomputed with the SwiGLU backward in its
  //    epilogue: dG1 = [dh * up * silu'(gate) | dh * silu(gate)] in fp16,
  //    h = silu(gate) * up as well when the down adapter needs it, and the
  //    gate_up adapter's u = x A_gu^T (fp32), which its k-loop computes anyway
  st = gemm_common(xa, NF4MOE_F16, T, sorted, k, gu_packed, gu_absmax, offs, E, P,
                   2 * (int64_t)I, H, gu_rc, NF4MOE_EPI_SWIGLU, nullptr, nullptr, dG,
                   NF4MOE_F16, qt, s, dH, dn_lora ? hbuf : nullptr, gu_lora ? u_gu : nullptr);
  if (st != NF4MOE_OK) return st;

  // 6. the down adapter's gradients: one pass over h for u = h A_dn^T and
  //    dA_dn = s sum w v' h^T, one over dy for dB_dn = s sum w dy u^T
  if (dn_lora) {
    st = lora_pass(hbuf, 0, nullptr, 1, offs, E, P, I, r, a16_dn, u_dn, wts, sorted, v_dn,
                   part, d_dn_A, dn_lora->scale, 1, cus, s);
    if (st != NF4MOE_OK) return st;
    st = lora_pass(dyh, 0, sorted, k, offs, E, P, H, r, nullptr, nullptr, wts, sorted, u_dn,
                   part, d_dn_B, dn_lora->scale, 0, cus, s);
    if (st != NF4MOE_OK) return st;
  }

  // 7. gate_up adapter (u = x A_gu^T came from the recompute): one pass
  //    over dG1 for v1 = dG1 B_gu and dB_gu = s sum w dG1 u^T
  if (gu_lora) {
    const int bf = gu_lora->dtype == NF4MOE_BF16;
    err = launch_lora_to_f16(gu_lora->B, bf, 1, E, 2 * I, r, bt_gu, cus, s);
    if (err != hipSuccess) return hip_fail(err, "LoRA conversion launch");
    st = lora_pass(dG, 0, nullptr, 1, offs, E, P, 2 * I, r, bt_gu, v_gu, wts, sorted, u_gu,
                   part, d_gu_B, gu_lora->scale, 0, cus, s);
    if (st != NF4MOE_OK) return st;
  }

  // 8. per-pair input gradients dG W_gu (+ LoRA) in pair order, then the sum
  //    over each token's k pairs
  // (the routing weight w of each pair applied here as the row scale)
  st = dgrad_common(dG, NF4MOE_F16, P, nullptr, 1, gu_packed, gu_absmax, offs, E, P,
                    2 * (int64_t)I, H, NF4MOE_EPI_NONE, nullptr, 0, wts, sorted, sorted,
                    gu_lora ? v_gu : nullptr, gu_lora, dXp, NF4MOE_F16, qt, s);
  if (st != NF4MOE_OK) return st;
  err = launch_combine(dXp, nullptr, T, k, H, dx, dx_dtype, cus, s);
  if (err != hipSuccess) return hip_fail(err, "combine launch");

  // 9. dA_gu = s sum w v1 x^T
  if (gu_lora) {
    st = lora_pass(xa, 0, sorted, k, offs, E, P, H, r, nullptr, nullptr, wts, sorted, v_gu,
                   part, d_gu_A, gu_lora->scale, 1, cus, s);
    if (st != NF4MOE_OK) return st;
  }
  return ok();
}

int moe_expert_backward(const void* x, int x_dtype, const float* router_logits, const void* dy,
                        int dy_dtype, int64_t T, int H, int I, int E, int k, int renormalize,
                        const uint8_t* gu_packed, const float* gu_absmax,
                        const uint8_t* dn_packed, const float* dn_absmax,
                        const nf4moe_lora* gu_lora, const nf4moe_lora* dn_lora, void* dx,
                        int dx_dtype, float* d_gu_A, float* d_gu_B, float* d_dn_A,
                        float* d_dn_B, void* workspace, size_t ws_bytes, void* stream) {
  return backward_impl(kQtNF4, x, x_dtype, router_logits, dy, dy_dtype, T, H, I, E, k,
                       renormalize, gu_packed, gu_absmax, dn_packed, dn_absmax, gu_lora,
                       dn_lora, dx, dx_dtype, d_gu_A, d_gu_B, d_dn_A, d_dn_B, workspace,
                       ws_bytes, stream);
}

int moe_expert_backward_nbit(int quant_type, const void* x, int x_dtype,
                             const float* router_logits, const void* dy, int dy_dtype,
                             int64_t T, int H, int I, int E, int k, int renormalize,
                             const uint8_t* gu_packed, const float* gu_absmax,
                             const uint8_t* dn_packed, const float* dn_absmax,
                             const nf4moe_lora* gu_lora, const nf4moe_lora* dn_lora, void* dx,
                             int dx_dtype, float* d_gu_A, float* d_gu_B, float* d_dn_A,
                             float* d_dn_B, void* workspace, size_t ws_bytes, void* stream) {
  if (quant_type != kQtNF4 && quant_type != kQtFP4)
    return fail(NF4MOE_EINVAL, "storage mode %d: the backward takes nf4 or fp4 stacks", quant_type);
  return backward_impl(quant_type, x, x_dtype, router_logits, dy, dy_dtype, T, H, I, E, k,
                       renormalize, gu_packed, gu_absmax, dn_packed, dn_absmax, gu_lora,
                       dn_lora, dx, dx_dtype, d_gu_A, d_gu_B, d_dn_A, d_dn_B, workspace,
                       ws_bytes, stream);
}

// ---- MXFP4 stacks (e2m1 + e8m0 per 32) ----------------------------------

static int mx_shape_check(int64_t N, int64_t K) {
  if (K % 128)
    return fail(NF4MOE_ESHAPE, "MXFP4: K=%lld must be a multiple of 128", (long long)K);
  (void)N;
  return NF4MOE_OK;
}

int grouped_mxfp4_gemm(const void* a, int a_dtype, int64_t a_rows, const int32_t* gather,
                       int gather_div, const uint8_t* blocks, const uint8_t* scales,
                       const int32_t* expert_offsets, int E, int64_t P, int64_t N, int64_t K,
                       int epilogue, const float* row_scale, const int32_t* scatter,
                       void* out, int out_dtype, void* stream) {
  int st = mx_shape_check(N, K);
  if (st != NF4MOE_OK) return st;
  return gemm_impl(kQtMXFP4, a, a_dtype, a_rows, gather, gather_div, blocks,
                   reinterpret_cast<const float*>(scales), expert_offsets, E, P, N, K, nullptr,
                   epilogue, row_scale, scatter, out, out_dtype, stream);
}

int moe_expert_forward_mxfp4(const void* x, int x_dtype, const float* router_logits, int64_t T,
                             int H, int I, int E, int k, int renormalize,
                             const uint8_t* gu_blocks, const uint8_t* gu_scales,
                             const uint8_t* dn_blocks, const uint8_t* dn_scales, void* y,
                             int y_dtype, void* workspace, size_t ws_bytes, void* stream) {
  int st = mx_shape_check(2 * (int64_t)I, H);
  if (st == NF4MOE_OK) st = mx_shape_check(H, I);
  if (st != NF4MOE_OK) return st;
  return forward_impl(kQtMXFP4, x, x_dtype, router_logits, T, H, I, E, k, renormalize,
                      gu_blocks, reinterpret_cast<const float*>(gu_scales), dn_blocks,
                      reinterpret_cast<const float*>(dn_scales), nullptr, nullptr, y, y_dtype,
                      workspace, ws_bytes, stream);
}

}  // extern "C"
