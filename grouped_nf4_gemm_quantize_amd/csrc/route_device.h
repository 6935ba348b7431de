// Device-side top-k routing of one token by one wave (shared by the routing
// kernels and the fused decode kernel).
#pragma once

#include "common.h"

namespace nf4moe {

namespace route_detail {

// true if b ranks before a: larger logit, or equal logit and lower id.
__device__ __forceinline__ bool better(float bv, int bid, float av, int aid) {
  return bv > av || (bv == av && bid < aid);
}

template <int kCtrl>
__device__ __forceinline__ void best_step(float& v, int& id) {
  const float ov = dpp_f<kCtrl>(v);
  const int oid = dpp_i<kCtrl>(id);
  if (better(ov, oid, v, id)) {
    v = ov;
    id = oid;
  }
}

// Wave-wide best (largest value, ties to the lower id), uniform in every
// lane: DPP butterfly inside each row of 16 lanes, then the four row
// winners compared as scalars.
__device__ __forceinline__ void wave_best(float& v, int& id) {
  best_step<kDppXor1>(v, id);
  best_step<kDppXor2>(v, id);
  best_step<kDppHalfMirror>(v, id);
  best_step<kDppMirror>(v, id);
  float bv = lane_f(v, 0);
  int bid = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = lane_f(v, 16 * r);
    const int rid = __builtin_amdgcn_readlane(id, 16 * r);
    if (better(rv, rid, bv, bid)) {
      bv = rv;
      bid = rid;
    }
  }
  v = bv;
  id = bid;
}

}  // namespace route_detail

// One wave routes one token at a time.  Logit e of the token lives in lane
// e % 64, register e / 64 (route_load); route_select then picks the top k.
template <int kRegs>
__device__ __forceinline__ void route_load(const float* __restrict__ lg_row, int E,
                                           int lane, float v[kRegs]) {
#pragma unroll
  for (int r = 0; r < kRegs; ++r) {
    const int e = lane + 64 * r;
    v[r] = (e < E) ? lg_row[e] : -__builtin_inff();
  }
}

// Lane j < k receives slot j: the expert id and its routing weight.
template <int kRegs>
__device__ __forceinline__ void route_select(const float v[kRegs], int E, int k,
                                             int renormalize, int lane, int* out_id,
                                             float* out_w) {
  uint32_t taken = 0u;
  float my_v = 0.f;
  int my_id = 0;
  float top = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bid = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
      const int e = lane + 64 * r;
      if (e < E && !((taken >> r) & 1u) && route_detail::better(v[r], e, bv, bid)) {
        bv = v[r];
        bid = e;
      }
    }
    route_detail::wave_best(bv, bid);
    // every lane now holds the winner of round j
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
    if (lane == j) {
      my_v = bv;
      my_id = bid;
    }
    if (j == 0) top = bv;
  }
  float s;
  const float ej = (lane < k) ? expf(my_v - top) : 0.f;
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
