/*
 * nf4moe.h -- C ABI of the MI355X (gfx950) grouped NF4 MoE expert library.
 *
 * The library runs the routed Mixture-of-Experts expert projections directly
 * on a frozen, fused, NF4-packed expert stack:
 *
 *   gate_up_proj [E, 2I, H] and down_proj [E, H, I]  (rows are [out, in]),
 *
 * as described on the experts4bit-qlora pages ("The problem", "Quickstart"
 * of the 0.22.0 README) and the grouped-nf4-gemm solutions entry ("How do I
 * run a grouped GEMM directly on NF4 packed MoE expert weights, without
 * dequantizing to bf16 first?").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns all
 *    memory; the library never allocates device memory.  Entry points that
 *    need scratch take a caller-provided workspace and expose a size query.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *    default stream).  No call synchronises the host with the device, so the
 *    calls can be captured in a HIP graph.
 *  - Every call returns an int status: NF4MOE_OK (0) or a negative error.
 *    Argument errors are found on the host BEFORE anything is enqueued;
 *    nf4moe_last_error() then returns a thread-local description.  A failed
 *    kernel launch returns NF4MOE_EHIP.  There is no fallback path.
 *  - Storage format (pinned by the byte totals the pages print: 16.31 GB for
 *    the 48-layer Qwen3-30B-A3B stack, "Training + expert offload" of the
 *    0.22.0 README, and 12,846,366,720 bytes per cell in the 2026 narrative's
 *    "What these numbers do not say"): for a stack [E, N, K],
 *      packed [E, N, K/2] uint8, two 4-bit codes per byte, the even element
 *             in the HIGH nibble: byte = (code[2i] << 4) | code[2i+1];
 *      absmax [E, N, K/64] fp32, one scale per 64 consecutive elements of a
 *             row (blocks never cross a row or an expert: "Which project
 *             solves it" on the load_in_4bit solutions page);
 *      weight = fp32(level[code] * absmax), level = the 16-entry NF4
 *             codebook returned by nf4moe_codebook().
 *  - Compute precision: fp32 accumulation ("NF4 decoded in-register inside
 *    the GEMM, fp32 accumulation", 0.22.0 README "Which door?").  Weights
 *    are decoded to fp16 MFMA operands (level and absmax rounded to fp16,
 *    product rounded to fp16); activations enter the MFMA as fp16.  Values
 *    must therefore lie in fp16 range (|v| < 65504); values below 2^-14 lose
 *    precision gradually (fp16 subnormals).  Both are observable without a
 *    host sync: the quantiser flags a stack whose absmax leaves the range
 *    (nonfinite_flag bit 2), nf4moe_f16_range_check flags activations or
 *    gradients, and values past 65504 inside the layer become +-inf in y.
 */
#ifndef NF4MOE_H
#define NF4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define NF4MOE_OK          0
#define NF4MOE_EINVAL     -1  /* null required pointer, non-positive size     */
#define NF4MOE_ESHAPE     -2  /* a dimension is not a multiple it must be     */
#define NF4MOE_EBLOCK     -3  /* blocksize other than 64                      */
#define NF4MOE_ETOPK      -4  /* k < 1, k > E or k > NF4MOE_MAX_TOPK          */
#define NF4MOE_EDTYPE     -5  /* unsupported dtype for this argument          */
#define NF4MOE_EWORKSPACE -6  /* workspace smaller than the size query        */
#define NF4MOE_EOVERFLOW  -7  /* a size overflows the 32-bit row indexing     */
#define NF4MOE_EHIP       -8  /* a HIP runtime call or kernel launch failed   */

#define NF4MOE_BLOCKSIZE   64
#define NF4MOE_MAX_TOPK    32
#define NF4MOE_MAX_EXPERTS 1024
#define NF4MOE_MAX_LORA_R  16

typedef enum {
  NF4MOE_F32 = 0,
  NF4MOE_BF16 = 1,
  NF4MOE_F16 = 2
} nf4moe_dtype;

/* Epilogues of grouped_nf4_gemm. */
#define NF4MOE_EPI_NONE   0
#define NF4MOE_EPI_SWIGLU 1 /* N = 2I outputs -> I outputs: silu(first I) * next I */
#define NF4MOE_EPI_SWIGLU_BWD 2 /* dgrad only: see grouped_nf4_gemm_dgrad */

/* Static description of the status code (never NULL). */
const char* nf4moe_strerror(int status);
/* Thread-local detail of the last error returned on this thread ("" if none). */
const char* nf4moe_last_error(void);
/* Library version string, e.g. "0.1.0". */
const char* nf4moe_version(void);

/* [host] Writes the 16 fp32 NF4 levels, ascending, to out16.
 * The levels are the 4-bit NormalFloat construction (normal quantiles with an
 * exact zero, 8 positive and 7 negative levels, normalised to [-1, 1]); the
 * pages fix only that training and serving share one codebook (0.22.0
 * README, "Inference").  Returns NF4MOE_EINVAL if out16 is NULL. */
int nf4moe_codebook(float* out16);

/* Bytes of one packed stack [E, N, K]: E*N*K/2 + (E*N*K/64)*4.
 * Returns a negative status if a size is non-positive or K % 64 != 0. */
int64_t nf4moe_packed_bytes(int64_t E, int64_t N, int64_t K);

/* ---- NF4 blockwise quantiser ---------------------------------------------
 * Quantises an expert stack w [E, N, K] (row-major, fp32 or bf16) with
 * blocks of 64 consecutive elements along K, as Experts4bit.from_float does
 * for the fused stacks (0.22.0 README "Quickstart"; blocks never cross an
 * expert: load_in_4bit solutions page, "Which project solves it").
 *   absmax = max |x| over the block (exact);
 *   xn     = x / absmax (IEEE fp32 division);
 *   code   = index of the nearest level to xn (exact comparison; a tie goes
 *            to the lower index); an all-zero block stores absmax 0, code 7.
 * Output bytes are identical on every run and device.
 *   w_dtype        NF4MOE_F32 or NF4MOE_BF16 (else EDTYPE)
 *   blocksize      must be 64 (else EBLOCK)
 *   K              must be a positive multiple of 64 (else ESHAPE)
 *   packed, absmax outputs as described in the conventions above
 *   nonfinite_flag nullable device int32, 4-byte aligned; bits OR-ed in,
 *                  never cleared: 1 if any input element is NaN or +-Inf
 *                  (codes of such blocks are unspecified); 2 if a block's
 *                  absmax, as the fp16 multiplier the grouped GEMMs make of
 *                  it (absmax; absmax/127 for int8, absmax/448 for fp8), is
 *                  outside fp16's normal range [2^-14, 65504] (all-zero
 *                  and non-finite blocks excepted): such a block's weights lose precision in
 *                  the GEMMs (below) or become infinite (above).
 * Alignment (else EINVAL): w 16 bytes (F32) or 8 (BF16), packed 2 bytes (4
 * for the 8-bit modes of nbit_quantize_experts), absmax 4.
 */
int nf4_quantize_experts(const void* w, int w_dtype, int64_t E, int64_t N,
                         int64_t K, int blocksize, uint8_t* packed,
                         float* absmax, int32_t* nonfinite_flag, void* stream);

/* ---- fp16 range check ----------------------------------------------------
 * The grouped GEMMs multiply in fp16 (activations converted from bf16, see the
 * conventions above); this reports on the device, without a host sync, what
 * that conversion would lose for n values t (BF16 or F32; x before a forward,
 * dL/dy before a backward).  Bits OR-ed into *flags (never cleared):
 *   1  a value fp16 cannot hold: |v| >= 65520 rounds to +-inf (NaN and inf
 *      included) -- the layer's output then carries non-finite values;
 *   2  a nonzero value fp16 flushes to zero (|v| <= 2^-25);
 *   4  a nonzero value below fp16's normal range (|v| < 2^-14): fewer than 11
 *      significant bits (an absolute error below 2^-25; N(0,1) activations
 *      have a few such values per hundred thousand, harmless in a dot
 *      product).
 * Alignment: t 16 bytes (F32) or 8 (BF16), flags 4 (else EINVAL); other
 * dtypes -> EDTYPE.  The absmax of a stack is checked by the quantiser
 * (nonfinite_flag bit 2). */
int nf4moe_f16_range_check(const void* t, int dtype, int64_t n, int32_t* flags, void* stream);

/* ---- router top-k and pair permutation -----------------------------------
 * For T tokens with fp32 router logits [T, E] (E <= NF4MOE_MAX_EXPERTS):
 *   topk_ids [T, k] int32  the k largest logits per token, descending; equal
 *                          logits go to the lower expert id;
 *   topk_w   [T, k] fp32   renormalize=1: softmax over the k selected logits
 *                          (sums to 1); renormalize=0: the full-softmax
 *                          probabilities of the selected experts;
 *   sorted_pair [T*k]      pair ids p = t*k + j grouped by expert, ascending
 *                          expert and ascending p inside an expert ("sort
 *                          token/expert pairs, run the groups", 0.22.0 README
 *                          "Which training path?");
 *   pair_pos [T*k]         nullable; inverse permutation (pair_pos[p] = i
 *                          iff sorted_pair[i] = p);
 *   expert_offsets [E+1]   exclusive prefix sum of the per-expert pair counts;
 *                          expert_offsets[E] = T*k.
 * Logits must be finite (non-finite logits give unspecified ids).
 * workspace: moe_route_permute_workspace(T, E, k) bytes (may be NULL if 0).
 */
size_t moe_route_permute_workspace(int64_t T, int E, int k);
int moe_route_permute(const float* logits, int64_t T, int E, int k,
                      int renormalize, int32_t* topk_ids, float* topk_w,
                      int32_t* sorted_pair, int32_t* pair_pos,
                      int32_t* expert_offsets, void* workspace,
                      size_t ws_bytes, void* stream);

/* ---- per-expert LoRA adapter ---------------------------------------------
 * delta = scale * (a A_e^T) B_e^T with A [E, r, K] and B [E, N, r] (the
 * trainable per-expert low-rank delta of ExpertsLoRA, solutions index "How do
 * I QLoRA-train the fused experts"; r=8, alpha=16 in the 0.22.0 Quickstart,
 * so scale = alpha / r).  1 <= r <= NF4MOE_MAX_LORA_R; dtype BF16 or F16.
 * Pass a NULL pointer to the struct for "no adapter".
 */
typedef struct {
  const void* A;
  const void* B;
  int r;
  float scale;
  int dtype;
} nf4moe_lora;

/* ---- grouped NF4 GEMM ----------------------------------------------------
 * out_row(i) = a[src(i)] . W_e^T  (+ LoRA delta)  for rows
 * expert_offsets[e] <= i < expert_offsets[e+1], with W_e = dequant(packed[e],
 * absmax[e]) [N, K], decoded in registers (never written to memory) and fp32
 * accumulation: the single-launch grouped kernel of grouped-nf4-gemm ("How do
 * I run a grouped GEMM directly on NF4 packed MoE expert weights").
 *   a [a_rows, K]   activations, F16 or BF16 (else EDTYPE);
 *   gather          nullable int32 [P]; src(i) = gather[i] / gather_div,
 *                   else src(i) = i.  Indices are not checked on the device:
 *                   src(i) must be < a_rows;
 *   packed, absmax  the stack [E, N, K] (K % 64 == 0, N % 16 == 0);
 *   expert_offsets  device int32 [E+1], non-decreasing, offsets[0] = 0 and
 *                   offsets[E] <= P (rows at and beyond offsets[E] are not
 *                   written);
 *   P               host-side upper bound of the row count (sizes the grid);
 *   lora            [host] nullable adapter on this projection (added before
 *                   the epilogue);
 *   epilogue        NF4MOE_EPI_NONE, or NF4MOE_EPI_SWIGLU (N = 2I must be a
 *                   multiple of 32; the output has N/2 columns);
 *   row_scale       nullable fp32 [P], multiplies output row i;
 *   scatter         nullable int32 [P]; output row i is written to row
 *                   scatter[i] of out, else to row i;
 *   out             F32, F16 or BF16 rows of N (or N/2) elements, 16-byte
 *                   aligned (rows are written as 16-byte chunks).
 * Buffers: a and packed 16-byte aligned, absmax 4-byte aligned, else EINVAL.
 * One kernel launch; no workspace (the per-expert tile table is rebuilt from
 * expert_offsets inside the kernel).
 */
int grouped_nf4_gemm(const void* a, int a_dtype, int64_t a_rows,
                     const int32_t* gather, int gather_div,
                     const uint8_t* packed, const float* absmax,
                     const int32_t* expert_offsets, int E, int64_t P,
                     int64_t N, int64_t K, const nf4moe_lora* lora,
                     int epilogue, const float* row_scale,
                     const int32_t* scatter, void* out, int out_dtype,
                     void* stream);

/* ---- full routed-expert layer --------------------------------------------
 * y [T, H] = sum_j w_tj * down_e(silu(gate_e(x_t)) * up_e(x_t)) over the k
 * experts the router picks for token t: route + permute, gate_up (+LoRA),
 * SwiGLU, down (+LoRA), combine over the slots in ascending slot order
 * (experts summed per token in group-sorted pair order, 0.22.0 README
 * "Which training path?").  T == 1 without adapters (and H <= 8192,
 * k*I <= 16384) runs one fused split-K decode kernel (the single-token fast
 * path, 0.22.0 README "Inference"); otherwise the grouped MFMA kernels.  Same
 * contract either way.  The decode kernel exchanges h between its
 * workgroups inside one launch: it needs its grid (at most one workgroup per
 * compute unit) resident at once, and keeps a generation word and the
 * exchanged values in the workspace, tagged per launch, so the workspace
 * needs no clearing between calls; two calls must not share a workspace
 * while both run (as for every path).  Should that exchange ever wait past
 * its bound, y is written as NaN (a loud failure, never a stale value).
 *   x [T, H]        BF16 or F16 activations;
 *   router_logits   fp32 [T, E];
 *   H, I            multiples of 64; E <= NF4MOE_MAX_EXPERTS; k <= min(E, 32);
 *   gu_*            gate_up stack [E, 2I, H]; dn_* down stack [E, H, I];
 *   gu_lora/dn_lora [host] nullable adapters; BF16 adapters are copied to
 *                   fp16 in the workspace once per call (the same rounding
 *                   the GEMM applies to bf16 adapters itself);
 *   y               [T, H] in y_dtype (BF16, F16 or F32);
 *   workspace       moe_expert_forward_workspace(T, H, I, E, k, r) bytes,
 *                   256-byte aligned, r = the larger adapter rank (0 without
 *                   adapters); too small -> EWORKSPACE, naming the size.
 * moe_expert_forward_workspace returns 0 for invalid sizes (r outside
 * [0, NF4MOE_MAX_LORA_R] included).
 */
size_t moe_expert_forward_workspace(int64_t T, int H, int I, int E, int k, int r);
int moe_expert_forward(const void* x, int x_dtype, const float* router_logits,
                       int64_t T, int H, int I, int E, int k, int renormalize,
                       const uint8_t* gu_packed, const float* gu_absmax,
                       const uint8_t* dn_packed, const float* dn_absmax,
                       const nf4moe_lora* gu_lora, const nf4moe_lora* dn_lora,
                       void* y, int y_dtype, void* workspace, size_t ws_bytes,
                       void* stream);

/* ---- grouped NF4 dgrad (backward through the frozen stack) ---------------
 * out_row(i) = row_scale(i) * a[src(i)] . W_e  for rows
 * expert_offsets[e] <= i < expert_offsets[e+1], W_e = dequant(packed[e],
 * absmax[e]) [N, K]: the input gradient of the grouped GEMM above, which
 * contracts over the N stack rows (across the absmax blocks).  Nibbles are
 * decoded in registers, nothing dequantised is written, fp32 accumulation:
 * the single-launch dgrad kernel of the fused training path (0.22.0 README
 * "Which training path?", dgrad=True; the frozen projections re-dequantise
 * from the packed bytes inside backward, README "Training + expert
 * offload").
 *   a [a_rows, N]   gradient rows, F16 or BF16 (else EDTYPE);
 *   gather          nullable int32 [P]: src(i) = gather[i] / gather_div, else
 *                   i (not checked on the device: src(i) < a_rows);
 *   packed, absmax  the stack [E, N, K]; N and K multiples of 64 (ESHAPE);
 *   expert_offsets  device int32 [E+1] as for grouped_nf4_gemm;
 *   epilogue        NF4MOE_EPI_NONE: out has K columns;
 *                   NF4MOE_EPI_SWIGLU_BWD: the backward of the SwiGLU that
 *                   followed the forward GEMM whose pre-activation row i is
 *                   g_pre[i] = [gate | up] (2K columns, F16 or BF16): with
 *                   dh = the dgrad row, out row i = [dh * up * silu'(gate) |
 *                   dh * silu(gate)] (2K columns);
 *   row_scale       nullable fp32; row i is scaled by row_scale[gather[i]]
 *                   when gather is given (a per-pair weight), else
 *                   row_scale[i]; applied before the SwiGLU backward;
 *   scatter         nullable int32 [P]: output row i goes to row scatter[i];
 *   out             F32, F16 or BF16, 16-byte aligned.
 * One kernel launch, no workspace.  Errors as for grouped_nf4_gemm. */
int grouped_nf4_gemm_dgrad(const void* a, int a_dtype, int64_t a_rows,
                           const int32_t* gather, int gather_div,
                           const uint8_t* packed, const float* absmax,
                           const int32_t* expert_offsets, int E, int64_t P,
                           int64_t N, int64_t K, int epilogue, const void* g_pre,
                           int g_dtype, const float* row_scale,
                           const int32_t* scatter, void* out, int out_dtype,
                           void* stream);

/* ---- recompute-and-differentiate SwiGLU (training) -----------------------
 * The gate_up GEMM of grouped_nf4_gemm recomputed inside backward, with the
 * SwiGLU backward as its epilogue: for rows expert_offsets[e] <= i <
 * expert_offsets[e+1], the pre-activation G_i = a[src(i)] . dequant(W_e)^T
 * ([gate | up], N = 2I columns, fp32 in registers) is never written; the
 * output is
 *   out row i = [dh_i * up * silu'(gate) | dh_i * silu(gate)]  (2I columns)
 * for dh the upstream gradient of h = silu(gate) * up, and optionally h
 * itself.  The frozen projection is decoded again from the packed bytes
 * inside backward (README "Training + expert offload"; the dgrad=True
 * training path of the 0.22.0 README "Which training path?").
 *   a [a_rows, K]   F16 rows; gather / gather_div as for grouped_nf4_gemm;
 *   packed, absmax  the gate_up stack [E, N, K]; N = 2I with I a multiple of
 *                   16, K a multiple of 64 (ESHAPE);
 *   lora            [host] nullable adapter on the gate_up projection;
 *   dh              F16 [P, I] (row i), 16-byte aligned;
 *   out             F16 [P, 2I], 16-byte aligned;
 *   h_out           nullable F16 [P, I], 16-byte aligned.
 * No row scale or scatter.  One kernel launch, no workspace; other
 * arguments and errors as for grouped_nf4_gemm. */
int grouped_nf4_gemm_swiglu_bwd(const void* a, int64_t a_rows, const int32_t* gather,
                                int gather_div, const uint8_t* packed, const float* absmax,
                                const int32_t* expert_offsets, int E, int64_t P, int64_t N,
                                int64_t K, const nf4moe_lora* lora, const void* dh, void* out,
                                void* h_out, void* stream);

/* ---- routed-expert layer backward (QLoRA) --------------------------------
 * Given dL/dy for y = moe_expert_forward(x, ...), returns dL/dx through the
 * frozen stacks and, per adapter, dL/dA and dL/dB; the stacks get no
 * gradient (only the adapters train: solutions entry "How do I QLoRA-train
 * the fused experts").  Nothing from the forward is kept: routing and the
 * gate_up pre-activation are recomputed from x and the logits, and both
 * projections are decoded again from the packed bytes (README "Training +
 * expert offload").  The router logits are an input, so no gradient flows
 * through the routing.  Steps: route; dh = dy . W_dn (+ LoRA), one dgrad
 * launch; G = gate_up(x) (+LoRA) recomputed with the SwiGLU backward as its
 * epilogue, dG = [dh * up * silu'(gate) | dh * silu(gate)] (and h for the
 * down adapter, u = x A_gu^T for the gate_up one), one grouped GEMM launch;
 * per-pair dX = w * dG . W_gu (+ LoRA), one dgrad launch; dx_t = sum of its
 * k pairs; the adapters' gradients as per-64-row partial sums reduced per
 * expert in a fixed order (deterministic).
 *   x [T, H]        BF16 or F16; dy [T, H] BF16 or F16 (dy_dtype);
 *   dx [T, H]       BF16, F16 or F32 (dx_dtype);
 *   d_gu_A [E, r, H], d_gu_B [E, 2I, r], d_dn_A [E, r, I], d_dn_B [E, H, r]
 *                   fp32, required when the matching adapter is given
 *                   (experts that no token picked get zeros); both adapters
 *                   must share r;
 *   workspace       moe_expert_backward_workspace(T, H, I, E, k, r) bytes,
 *                   256-byte aligned (r = 0 without adapters).
 * Other arguments and errors as for moe_expert_forward. */
size_t moe_expert_backward_workspace(int64_t T, int H, int I, int E, int k, int r);
int moe_expert_backward(const void* x, int x_dtype, const float* router_logits,
                        const void* dy, int dy_dtype, int64_t T, int H, int I,
                        int E, int k, int renormalize, const uint8_t* gu_packed,
                        const float* gu_absmax, const uint8_t* dn_packed,
                        const float* dn_absmax, const nf4moe_lora* gu_lora,
                        const nf4moe_lora* dn_lora, void* dx, int dx_dtype,
                        float* d_gu_A, float* d_gu_B, float* d_dn_A, float* d_dn_B,
                        void* workspace, size_t ws_bytes, void* stream);

/* ---- other 4-bit storage modes ---------------------------------------------
 * ExpertsNbit stores the same fused stack at selectable precision; nf4 and
 * fp4 are its two 4-bit packed modes, and nf4 reconstructs with less error
 * than fp4 (0.22.0 README, "The problem").  These entry points take the mode
 * first and are otherwise identical to the nf4 ones above (same packing, same
 * absmax blocks, same kernels; only the 16 levels differ).
 *   NF4MOE_QT_NF4  the NF4 levels of nf4moe_codebook;
 *   NF4MOE_QT_FP4  e2m1 element values {0, .5, 1, 1.5, 2, 3, 4, 6} / 6 (the
 *                  block's absmax maps to the largest), code = sign << 3 |
 *                  magnitude index, code 8 = -0; quantiser: sign of
 *                  x/absmax, nearest magnitude level (an exact tie goes to
 *                  the even index), an all-zero block stores code 0.  The
 *                  pages print no fp4 values; this is the OCP e2m1 format.
 *   NF4MOE_QT_INT8 8-bit blockwise: one byte per element (packed is
 *                  [E, N, K]), code = round-half-even(x/absmax * 127) as
 *                  int8, value = code / 127 * absmax;
 *   NF4MOE_QT_FP8  8-bit blockwise: one byte per element, code = the
 *                  nearest OCP fp8 e4m3 value of x/absmax * 448 (ties to the
 *                  even mantissa; zero of either sign is code 0), value =
 *                  e4m3(code) / 448 * absmax.
 *   NF4MOE_QT_BF16 passthrough: packed is the weights themselves, [E, N, K]
 *   NF4MOE_QT_F16  bf16 (resp. fp16) values, 2 bytes per element, rounded
 *                  to nearest even from the input by nbit_quantize_experts
 *                  (fp32 beyond fp16's range becomes +-inf); absmax is
 *                  neither written nor read and may be NULL; the
 *                  nonfinite flag is not set.  The GEMM multiplies in fp16
 *                  (bf16 weights converted in registers: exact in fp16's
 *                  normal range, smaller magnitudes rounded to fp16
 *                  subnormals) with fp32 accumulation.
 * The 8-bit and 16-bit modes have no 16-level codebook (nbit_codebook
 * returns NF4MOE_EINVAL), run the grouped kernels for every T, and take no
 * adapters; the dgrad and the backward take nf4 and fp4 only.  The pages
 * name int8, fp8, bf16 and fp16 modes of ExpertsNbit (README "Training +
 * expert offload", QUANT_TYPE) but not the 8-bit maps; these are the plain
 * absmax-scaled readings.  An unknown mode returns NF4MOE_EINVAL. */
#define NF4MOE_QT_NF4 0
#define NF4MOE_QT_FP4 1
#define NF4MOE_QT_INT8 3
#define NF4MOE_QT_FP8 4
#define NF4MOE_QT_BF16 5
#define NF4MOE_QT_F16 6
int nbit_codebook(int quant_type, float* out16);  /* [host] levels by code */
int nbit_quantize_experts(int quant_type, const void* w, int w_dtype, int64_t E,
                          int64_t N, int64_t K, int blocksize, uint8_t* packed,
                          float* absmax, int32_t* nonfinite_flag, void* stream);
int grouped_nbit_gemm(int quant_type, const void* a, int a_dtype, int64_t a_rows,
                      const int32_t* gather, int gather_div,
                      const uint8_t* packed, const float* absmax,
                      const int32_t* expert_offsets, int E, int64_t P,
                      int64_t N, int64_t K, const nf4moe_lora* lora,
                      int epilogue, const float* row_scale,
                      const int32_t* scatter, void* out, int out_dtype,
                      void* stream);
int moe_expert_forward_nbit(int quant_type, const void* x, int x_dtype,
                            const float* router_logits, int64_t T, int H, int I, int E,
                            int k, int renormalize, const uint8_t* gu_packed,
                            const float* gu_absmax, const uint8_t* dn_packed,
                            const float* dn_absmax, const nf4moe_lora* gu_lora,
                            const nf4moe_lora* dn_lora, void* y, int y_dtype,
                            void* workspace, size_t ws_bytes, void* stream);
int grouped_nbit_gemm_dgrad(int quant_type, const void* a, int a_dtype,
                            int64_t a_rows, const int32_t* gather, int gather_div,
                            const uint8_t* packed, const float* absmax,
                            const int32_t* expert_offsets, int E, int64_t P,
                            int64_t N, int64_t K, int epilogue, const void* g_pre,
                            int g_dtype, const float* row_scale,
                            const int32_t* scatter, void* out, int out_dtype,
                            void* stream);
int moe_expert_backward_nbit(int quant_type, const void* x, int x_dtype,
                             const float* router_logits, const void* dy,
                             int dy_dtype, int64_t T, int H, int I, int E, int k,
                             int renormalize, const uint8_t* gu_packed,
                             const float* gu_absmax, const uint8_t* dn_packed,
                             const float* dn_absmax, const nf4moe_lora* gu_lora,
                             const nf4moe_lora* dn_lora, void* dx, int dx_dtype,
                             float* d_gu_A, float* d_gu_B, float* d_dn_A,
                             float* d_dn_B, void* workspace, size_t ws_bytes,
                             void* stream);

/* ---- MXFP4 stacks (released e2m1 blocks + e8m0 scales) --------------------
 * The grouped GEMM and the layer forward on expert stacks released in MXFP4,
 * multiplied on their own bytes with no requantisation to NF4 and no bf16
 * copy (grouped-nf4-gemm solutions entry "How do I run MoE expert inference
 * natively on MXFP4 (e2m1 + e8m0) weights, straight from the released
 * checkpoint bytes?").  Format (OCP microscaling):
 *   blocks [E, N, K/2] uint8: two e2m1 codes per byte, element 2i in the LOW
 *          nibble (the released packing; the NF4 stacks put it high);
 *   scales [E, N, K/32] uint8: e8m0, weight = e2m1 value * 2^(s - 127).
 * The elements are decoded in registers to fp16 (value x scale, exact while
 * 2^(s-127) is within fp16's range, 2^-24 .. 2^15; s = 255 decodes as NaN);
 * fp32 accumulation.  K must be a multiple of 128 (ESHAPE).  No adapters.
 * Other arguments, layouts and errors as for grouped_nf4_gemm and
 * moe_expert_forward; the T == 1 case runs the fused split-K decode kernel,
 * which applies each 32-block's scale in fp32 (the weights have no fp16 range limit
 * there; h between the projections is fp16). */
int grouped_mxfp4_gemm(const void* a, int a_dtype, int64_t a_rows,
                       const int32_t* gather, int gather_div,
                       const uint8_t* blocks, const uint8_t* scales,
                       const int32_t* expert_offsets, int E, int64_t P,
                       int64_t N, int64_t K, int epilogue, const float* row_scale,
                       const int32_t* scatter, void* out, int out_dtype,
                       void* stream);
int moe_expert_forward_mxfp4(const void* x, int x_dtype, const float* router_logits,
                             int64_t T, int H, int I, int E, int k,
                             int renormalize, const uint8_t* gu_blocks,
                             const uint8_t* gu_scales, const uint8_t* dn_blocks,
                             const uint8_t* dn_scales, void* y, int y_dtype,
                             void* workspace, size_t ws_bytes, void* stream);

/* ---- allocation-free layer forward ----------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The same
 * computation, kernels and arguments as moe_expert_forward, without the
 * workspace: the library keeps NF4MOE_NOALLOC_SCRATCH_BYTES (32 MiB) of device
 * memory per device in its code object, held until the process ends, and this
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Sizes whose workspace (moe_expert_forward_workspace) exceeds it
 * are refused with NF4MOE_EWORKSPACE before anything is launched (the
 * Qwen3-30B-A3B layer fits up to about 670 tokens without adapters, 410 with
 * rank-8 adapters on both projections); other
 * argument errors as for moe_expert_forward.  Every call on one device shares
 * that memory: calls that overlap in time on one device (other streams,
 * other threads) race and must be serialised by the caller. */
#define NF4MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_expert_forward_noalloc(const void* x, int x_dtype, const float* router_logits,
                               int64_t T, int H, int I, int E, int k, int renormalize,
                               const uint8_t* gu_packed, const float* gu_absmax,
                               const uint8_t* dn_packed, const float* dn_absmax,
                               const nf4moe_lora* gu_lora, const nf4moe_lora* dn_lora,
                               void* y, int y_dtype, void* stream);

/* Device-pointer views into a moe_expert_forward workspace (for inspection of
 * the routing a forward used; valid after the forward completes on its
 * stream, the T == 1 decode path included: it writes ids, weights, the k
 * pairs grouped by expert and the offsets as well).  Any out-pointer may be
 * NULL.  Returns a negative status on bad sizes. */
int moe_expert_forward_routing(void* workspace, int64_t T, int H, int I,
                               int E, int k, int32_t** topk_ids,
                               float** topk_w, int32_t** sorted_pair,
                               int32_t** expert_offsets);

#ifdef __cplusplus
}
#endif

#endif /* NF4MOE_H */
