// Device side of the routing, shared by the routing kernels and the
// small-batch expert kernel that routes for itself: the top-k keys and their
// wave-wide maximum, scans, the top-k of one token and the fold of z.  The
// routing follows the release cards' top-k gating (35B-A3B card, "Model
// Overview": top-8; FlashNext card, "Model Overview": top-10 routed + 1 shared)
// with the readings of include/moe_ternary.h (ties to the lower expert index,
// softmax over the k selected logits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"
#include "wave_ops.h"

namespace moe {

// Top-k candidates as 64-bit keys whose unsigned order is the selection
// order.  High word: the fp32 logit mapped to an order-preserving integer
// (-0.0 taken as +0.0; logits are finite); low word: the complemented expert
// index, so of two equal logits the lower expert ranks first.  Key 0 lies
// below every candidate and marks a used or absent one.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// x from another lane (DPP pattern CTRL) in the rows of ROWS; other rows keep x.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
  const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false);
  const uint32_t h = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false);
  return ((uint64_t)h << 32) | l;
}

constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Wave-wide maximum key, returned in every lane, with compares and selects
// only: four exchanges inside each row of 16 lanes; then lane 15 of rows 0 and
// 2 folds into rows 1 and 3, and lane 31 (rows 0-1) into rows 2 and 3, which
// leaves the maximum in lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t x) {
  x = umax64(x, dpp_u64<kDppXor1, 0xF>(x));
  x = umax64(x, dpp_u64<kDppXor2, 0xF>(x));
  x = umax64(x, dpp_u64<kDppHalfMirror, 0xF>(x));
  x = umax64(x, dpp_u64<kDppMirror, 0xF>(x));
  x = umax64(x, dpp_u64<kDppRowBcast15, 0xA>(x));
  x = umax64(x, dpp_u64<kDppRowBcast31, 0xC>(x));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Wave-wide sum: every lane returns the same value (rows summed in row order).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return ((readlane_f32(v, 0) + readlane_f32(v, 16)) + readlane_f32(v, 32)) + readlane_f32(v, 48);
}

// Inclusive prefix sum over the lanes of a wave: shifts by 1, 2, 4, 8 inside
// each row (lanes shifted in from outside the row read 0), then each row adds
// the totals of the rows before it.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppShr1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppShr2, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppShr4, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppShr8, 0xF, 0xF, true);
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Inclusive prefix sum over the 1024 threads of a block; *total receives the
// block's sum.  wsum: 16 ints of shared memory.  Every thread must call it.
__device__ __forceinline__ int block_inclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_inclusive_scan(v, lane);
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int s = wsum[w];
    before += w < wave ? s : 0;
    all += s;
  }
  *total = all;
  return v + before;
}

// Wave-wide maximum of a 32-bit value, returned in every lane (the same
// exchange pattern as wave_max_key, one max instruction per step).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppXor1, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppXor2, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppHalfMirror, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppMirror, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppRowBcast15, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Logit of token t, expert e: the x-projection partials added in slice order.
__device__ __forceinline__ float fold_logit(const RouteArgs& a, int64_t t, int e) {
  const int64_t stride = a.T * (int64_t)a.lN;
  const float* p = a.lpart + t * a.lN + e;
  float v = 0.f;
  for (int s0 = 0; s0 < a.lsplits; s0 += 8) {
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = p[min(s0 + j, a.lsplits - 1) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < a.lsplits) v += pv[j];
  }
  return v;
}

// One wave selects the top k of token t: k rounds of a wave-wide maximum over
// the candidate keys (lane l holds experts l, l + 64, ...), each round taking
// the winner out of its lane's list.  Lane i % 64 keeps the i-th selected key
// for the softmax and the coalesced stores at the end.  The logits come from
// slog (shared memory, [T x E]) when it is given, else from the x-projection
// partials when a.lpart is set (stored to a.logits with `store`), else from
// a.logits.  sidx: NULL, or LDS that also receives the indices; `store`: write
// a.idx and a.w (and the logits summed here).
template <int PER>  // keys per lane: E <= 64 * PER
__device__ __forceinline__ void topk_token(const RouteArgs& a, int64_t t, int lane, int* sidx, bool store = true,
                                           const float* slog = nullptr) {
  const int E = a.E, k = a.k;
  float lv[PER];  // every load unconditional (clamped index) so all are in flight together
  if (slog) {
#pragma unroll
    for (int c = 0; c < PER; ++c) lv[c] = slog[t * E + min(lane + 64 * c, E - 1)];
  } else if (a.lpart) {
    // the logits: the x-projection partials added in slice order, SU slices' loads at a time
    constexpr int SU = PER >= 16 ? 4 : 8;
    const int64_t stride = a.T * (int64_t)a.lN;
    const float* base = a.lpart + t * a.lN;
#pragma unroll
    for (int c = 0; c < PER; ++c) lv[c] = 0.f;
    for (int s0 = 0; s0 < a.lsplits; s0 += SU) {
      float pv[SU][PER];
#pragma unroll
      for (int j = 0; j < SU; ++j)
#pragma unroll
        for (int c = 0; c < PER; ++c)
          pv[j][c] = base[min(s0 + j, a.lsplits - 1) * stride + min(lane + 64 * c, E - 1)];
#pragma unroll
      for (int j = 0; j < SU; ++j)
#pragma unroll
        for (int c = 0; c < PER; ++c)
          if (s0 + j < a.lsplits) lv[c] += pv[j][c];
    }
#pragma unroll
    for (int c = 0; c < PER; ++c)
      if (store && lane + 64 * c < E) a.logits[t * E + lane + 64 * c] = lv[c];
  } else {
#pragma unroll
    for (int c = 0; c < PER; ++c) lv[c] = a.logits[t * E + min(lane + 64 * c, E - 1)];
  }
  uint64_t key[PER], sel[PER];  // sel[c] in lane l: the (64 c + l)-th selected key (k <= E)
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int e = lane + 64 * c;
    key[c] = e < E ? route_key(lv[c], e) : 0ull;
    sel[c] = 0ull;
  }
  // each lane sorts its keys once (descending; odd-even transposition), so a
  // round is the wave-wide maximum of the lanes' first keys and the winning
  // lane (keys are distinct: the low word is the expert) moves its list up
#pragma unroll
  for (int pass = 0; pass < PER; ++pass)
#pragma unroll
    for (int c = pass & 1; c + 1 < PER; c += 2) {
      const bool gt = key[c] > key[c + 1];
      const uint64_t hi = gt ? key[c] : key[c + 1], lo = gt ? key[c + 1] : key[c];
      key[c] = hi;
      key[c + 1] = lo;
    }
  float m = 0.f;
  for (int i = 0; i < k; ++i) {
    // the largest value word first; equal values (rare) then the largest low
    // word, i.e. the lowest expert, among the lanes that hold that value
    const uint32_t hv = (uint32_t)(key[0] >> 32);
    const uint32_t mx = wave_max_u32(hv);
    const uint64_t cand = __ballot(hv == mx);
    uint32_t wlo;
    if (__popcll(cand) == 1)
      wlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[0], __ffsll((long long)cand) - 1);
    else
      wlo = wave_max_u32(hv == mx ? (uint32_t)key[0] : 0u);
    const uint64_t w = ((uint64_t)mx << 32) | wlo;
    if (i == 0) m = key_value(w);
    const bool won = key[0] == w;
#pragma unroll
    for (int c = 0; c + 1 < PER; ++c) key[c] = won ? key[c + 1] : key[c];
    key[PER - 1] = won ? 0ull : key[PER - 1];
#pragma unroll
    for (int c = 0; c < PER; ++c)
      if ((i >> 6) == c) sel[c] = (i & 63) == lane ? w : sel[c];
  }
  // softmax over the selected logits
  float ev[PER], part = 0.f;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    ev[c] = 64 * c + lane < k ? __expf(key_value(sel[c]) - m) : 0.f;
    part += ev[c];
  }
  const float inv = 1.f / wave_sum(part);
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int i = 64 * c + lane;
    if (i < k) {
      const int e = key_expert(sel[c]);
      if (sidx) sidx[t * k + i] = e;
      if (store) {
        a.idx[t * k + i] = e;
        a.w[t * k + i] = ev[c] * inv;
      }
    }
  }
}

// z = bf16 of the x-projection partials' columns E .. E + zr - 1, added in
// slice order.  Fold block b of nb takes elements b * blockDim + thread, then
// every nb * blockDim-th.
__device__ __forceinline__ void fold_z(const RouteArgs& a, int b, int nb) {
  const int n = (int)a.T * a.zr;
  const int64_t stride = a.T * (int64_t)a.lN;
  for (int i = b * (int)blockDim.x + (int)threadIdx.x; i < n; i += nb * (int)blockDim.x) {
    const int t = i / a.zr, c = i - t * a.zr;
    const float* p = a.lpart + (int64_t)t * a.lN + a.E + c;
    float v = 0.f;
    for (int s0 = 0; s0 < a.lsplits; s0 += 8) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = p[min(s0 + j, a.lsplits - 1) * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < a.lsplits) v += pv[j];
    }
    a.z[i] = (uint16_t)f32_to_bf16(v);
  }
}

// Blocks of the first routing launch beyond its routing blocks: fold z.
inline int fold_blocks(const RouteArgs& a, int threads) {
  if (!a.z || !a.lpart || a.zr <= 0) return 0;
  return (int)std::min<int64_t>(256, (a.T * a.zr + threads - 1) / threads);
}


}  // namespace moe
