// Device-side top-k routing of one token by one wave (shared by the routing
// kernel and the decode GEMV kernel).
#pragma once

#include "common.h"

namespace nf4moe {

// One wave routes one token at a time.  Logit e of the token lives in lane
// e % 64, register e / 64 (route_load); route_select then picks the top k.
template <int kRegs>
__device__ __forceinline__ void route_load(const float* __restrict__ lg_row, int E,
                                           int lane, float v[kRegs]) {
#pragma unroll
  for (int r = 0; r < kRegs; ++r) {
    const int e = lane + 64 * r;
    v[r] = lg_row[e < E ? e : E - 1];  // clamped: no branch around the load
  }
#pragma unroll
  for (int r = 0; r < kRegs; ++r) v[r] = (lane + 64 * r < E) ? v[r] : -__builtin_inff();
}

// Order-preserving 32-bit key of a logit: larger key = larger logit.  -0.0
// is folded onto +0.0 (they compare equal), NaN ranks with -inf.
__device__ __forceinline__ uint32_t logit_key(float x) {
  const uint32_t u = (x == 0.0f) ? 0u : __float_as_uint(x);
  if (x != x) return 0x007fffffu;  // the key of -inf
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Lane j < k receives slot j: the expert id and its routing weight.  The
// selection is a radix select over the 32-bit logit keys:
//   1. the k-th largest key t is the largest value with #{key >= t} >= k,
//      found bit by bit from the top with wave ballots (32 rounds of one
//      compare per register, a popcount and a scalar select);
//   2. every key above t is selected, and among the keys equal to t the
//      lowest expert ids (ties go to the lower id);
//   3. each of the k winners is ranked with the same ballots (its slot is
//      the number of keys above it), so lane j ends with the (j+1)-th
//      largest logit; then the softmax weights.
template <int kRegs>
__device__ __forceinline__ void route_select(const float v[kRegs], int E, int k,
                                             int renormalize, int lane, int* out_id,
                                             float* out_w) {
  // keys computed for every lane, then masked (branch-free: the first use of
  // the loaded logits is then a wait in uniform control flow)
  uint32_t hk[kRegs];
#pragma unroll
  for (int r = 0; r < kRegs; ++r)
    hk[r] = logit_key(v[r]) & (lane + 64 * r < E ? 0xffffffffu : 0u);

  // 1. the k-th largest key (padding keys are 0, below every real key)
  uint32_t t = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < kRegs; ++r) cnt += __popcll(__ballot(hk[r] >= c));
    if (cnt >= k) t = c;
  }

  // 2. above t, plus the lowest-id ties at t (ids grow with (register, lane))
  const uint64_t below = (1ull << lane) - 1ull;
  int above = 0;
#pragma unroll
  for (int r = 0; r < kRegs; ++r) above += __popcll(__ballot(hk[r] > t));
  const int need = k - above;
  bool sel[kRegs];
  int ties = 0;
#pragma unroll
  for (int r = 0; r < kRegs; ++r) {
    const uint64_t tm = __ballot(hk[r] == t);
    sel[r] = hk[r] > t || (hk[r] == t && ties + __popcll(tm & below) < need);
    ties += __popcll(tm);
  }

  // 3. visit the k winners in (register, lane) order: a winner's slot is the
  //    number of keys above it plus the equal keys with a lower id (all of
  //    which are winners too); lane `slot` keeps it
  uint32_t my_key = 0u;
  int my_id = 0;
#pragma unroll
  for (int r = 0; r < kRegs; ++r) {
    uint64_t m = __ballot(sel[r]);
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1ull;
      const uint32_t kk = (uint32_t)__builtin_amdgcn_readlane((int)hk[r], l);
      int slot = 0;
#pragma unroll
      for (int r2 = 0; r2 < kRegs; ++r2) {
        slot += __popcll(__ballot(hk[r2] > kk));
        if (r2 < r) slot += __popcll(__ballot(hk[r2] == kk));
        if (r2 == r) slot += __popcll(__ballot(hk[r2] == kk) & ((1ull << l) - 1ull));
      }
      if (lane == slot) {
        my_key = kk;
        my_id = 64 * r + l;
      }
    }
  }
  const float my_v = key_logit(my_key);
  const float top = lane_f(my_v, 0);
  const float ej = (lane < k) ? expf(my_v - top) : 0.f;
  float s;
  if (renormalize) {
    s = wave_sum(ej);
  } else {
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
      const int e = lane + 64 * r;
      if (e < E) part += expf(v[r] - top);
    }
    s = wave_sum(part);
  }
  *out_id = my_id;
  *out_w = ej / s;
}

template <int kRegs>
__device__ __forceinline__ void route_one_token(const float* __restrict__ lg_row, int E,
                                                int k, int renormalize, int lane,
                                                int* out_id, float* out_w) {
  float v[kRegs];
  route_load<kRegs>(lg_row, E, lane, v);
  route_select<kRegs>(v, E, k, renormalize, lane, out_id, out_w);
}

}  // namespace nf4moe
