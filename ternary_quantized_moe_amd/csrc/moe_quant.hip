// Ternary quantizer for gfx950: bfloat16 weights -> PQ2_0 or PTQ1_0 containers.
//
// A group of 128 weights becomes ternary codes t and one scale s (project
// README, "What the experiments established": the deployed ternary Lloyd
// quantizer over groups of 128 beats one-shot absmean; Scion-35B-A3B discussion
// thread, its list of findings; container layouts from the 35B-A3B card and the
// FlashNext card, "Weight Representation").  Two rules:
//   absmean  s = mean |w|;  t = sign(w) where 2|w| > s, else 0
//   Lloyd    from the absmean codes, alternate  s = mean |w| over the weights
//            with t != 0  and  t = sign(w) where 2|w| > s, until the codes
//            repeat (at most 32 rounds); the stored scale belongs to the final
//            codes.
// Every decision is taken in fp32 and every group sum is a balanced tree over
// adjacent pairs (weights 2m and 2m+1 first), so the containers are fixed bit
// for bit.  The scale is rounded to binary16 (nearest even), saturating at the
// largest finite value; a group of zeros gets scale 0.
//
// Layout: a row of LPG lanes (16 or 8) holds one group, lane i weights
// E i .. E i + E - 1 with E = 128 / LPG (one or two 16-byte loads), so a wave
// takes 64 / LPG consecutive groups.  A sum takes log2 E levels inside the lane
// and log2 LPG DPP exchanges inside the row, after which every lane of the row
// holds it.  The Lloyd loop runs until no group of the
// wave changes: a group that has converged is a fixed point of the iteration,
// so the rounds it runs after that leave it as it is.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "moe_internal.h"
#include "moe_ternary.h"
#include "wave_ops.h"

namespace moe {

namespace {

constexpr int kQuantThreads = 256;
// Lanes per 128-weight group: 16 lanes of 8 weights (four groups per wave) for
// absmean, 8 lanes of 16 weights (eight per wave) for Lloyd, whose rounds then
// spend fewer exchanges and divisions per group (measured on 604 M weights:
// Lloyd 737 us with 8 lanes against 862 with 16; absmean 231 us with 16
// against 249 with 8).
constexpr int kQuantLanesAbsmean = 16, kQuantLanesLloyd = 8;
constexpr int kQuantMinGroupsPerBlock = kQuantThreads / 16;
constexpr int kQuantMaxRounds = 32;
constexpr uint32_t kF16MaxFinite = 0x7BFFu;

// Sum over the LPG lanes of each group's row (8: lanes 1, 2 and 4 apart;
// 16: also 8 apart), returned to every lane of the row.
template <int LPG>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_row_f32<kDppXor1>(v);
  v += dpp_row_f32<kDppXor2>(v);
  v += dpp_row_f32<kDppHalfMirror>(v);
  if (LPG == 16) v += dpp_row_f32<kDppMirror>(v);
  return v;
}
template <int LPG>
__device__ __forceinline__ int row_sum_i32(int v) {
  v += dpp_row_i32<kDppXor1>(v);
  v += dpp_row_i32<kDppXor2>(v);
  v += dpp_row_i32<kDppHalfMirror>(v);
  if (LPG == 16) v += dpp_row_i32<kDppMirror>(v);
  return v;
}

// Adjacent-pair tree over a lane's E values.
template <int E>
__device__ __forceinline__ float tree_sum(const float (&v)[E]) {
  float t[E];
#pragma unroll
  for (int j = 0; j < E; ++j) t[j] = v[j];
#pragma unroll
  for (int w = E; w > 1; w /= 2)
#pragma unroll
    for (int j = 0; j < w / 2; ++j) t[j] = t[2 * j] + t[2 * j + 1];
  return t[0];
}

// The codes for scale s: bit j of the mask set where 2 a_j > s.  The sum of
// the selected a_j (adjacent-pair tree) and their number over the group come
// back in *total and *count.
template <int E, int LPG>
__device__ __forceinline__ uint32_t select_codes(const float (&a)[E], const float (&a2)[E], float s, float* total,
                                                 int* count) {
  uint32_t m = 0;
  int n = 0;
  float v[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const bool on = a2[j] > s;
    v[j] = on ? a[j] : 0.0f;
    n += on ? 1 : 0;
    m |= (on ? 1u : 0u) << j;
  }
  *total = row_sum<LPG>(tree_sum<E>(v));
  *count = row_sum_i32<LPG>(n);
  return m;
}

__device__ __forceinline__ float mean_or_zero(float total, int count) {
  const float q = total / (float)max(count, 1);
  return count > 0 ? q : 0.0f;
}

// E bits -> the even bits of a 2E-bit word (bit j -> bit 2j), E = 8 or 16.
__device__ __forceinline__ uint32_t spread_bits(uint32_t x) {
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  x = (x | (x << 1)) & 0x55555555u;
  return x;
}

// Five (or four) 2-bit base-3 digits, least significant first -> sum d_i 3^i.
__device__ __forceinline__ uint32_t base3_byte(uint64_t digits, int n) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 4; i >= 0; --i)
    if (i < n) v = v * 3u + (uint32_t)((digits >> (2 * i)) & 3u);
  return v;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src_lane) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

// Quantize the group g of this lane's row of LPG lanes; v holds lane i's
// E = 128 / LPG weights of it (weights E i .. E i + E - 1).  Rows past the last
// group (valid false) compute on zeros and store nothing.
template <int FMT, int METHOD, int LPG>
__device__ __forceinline__ void quantize_group(const u32x4 (&v)[128 / LPG / 8], int64_t g, bool valid, int i,
                                               int row0, uint8_t* __restrict__ dst, uint8_t* __restrict__ rounds) {
  constexpr int E = 128 / LPG;
  // |w| in fp32 (and 2|w|, exact) and the sign bits, weight E i + j in slot j
  float a[E], a2[E];
  uint32_t neg = 0;
#pragma unroll
  for (int c = 0; c < E / 8; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 8 * c + 2 * k;
      a[j] = fabsf(__uint_as_float(v[c][k] << 16));
      a[j + 1] = fabsf(__uint_as_float(v[c][k] & 0xFFFF0000u));
      neg |= ((v[c][k] >> 15) & 1u) << j;
      neg |= (v[c][k] >> 31) << (j + 1);
    }
#pragma unroll
  for (int j = 0; j < E; ++j) a2[j] = 2.0f * a[j];

  float s = row_sum<LPG>(tree_sum<E>(a)) / 128.0f;
  float total;
  int count;
  uint32_t nz = select_codes<E, LPG>(a, a2, s, &total, &count);
  if (METHOD == MOE_QUANT_LLOYD) {
    // The codes are the weights above a threshold, so two code sets of one
    // group are nested and equal exactly when their sizes are: a round that
    // keeps the count keeps the codes.  Each round's scale is the mean of the
    // current codes; the loop ends with s the mean of the final codes.
    // taken: the rounds this group needs, the one that repeats its codes
    // included (kQuantMaxRounds if none does)
    int taken = kQuantMaxRounds;
    for (int r = 0; r < kQuantMaxRounds; ++r) {
      s = mean_or_zero(total, count);
      int next_count;
      nz = select_codes<E, LPG>(a, a2, s, &total, &next_count);
      if (next_count == count) taken = min(taken, r + 1);
      const bool changed = __ballot(next_count != count) != 0;  // wave-uniform
      count = next_count;
      if (!changed) break;
    }
    s = mean_or_zero(total, count);
    if (rounds && valid && i == 0) rounds[g] = (uint8_t)taken;
  } else {
    if (rounds && valid && i == 0) rounds[g] = 0;
  }

  uint32_t sbits = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s);
  if (sbits == 0x7C00u) sbits = kF16MaxFinite;  // s >= 0: +Inf is the only overflow

  if (FMT == kPQ2) {
    // 2-bit codes: 01 = +1, 11 = -1; lane i writes bytes E/4 i .. E/4 i + E/4 - 1
    // as 2-byte stores (a block starts at 2-byte alignment)
    const uint32_t codes = spread_bits(nz) | (spread_bits(nz & neg) << 1);
    if (valid) {
      uint8_t* blk = dst + g * 34;
#pragma unroll
      for (int h = 0; h < E / 8; ++h) *(uint16_t*)(blk + (E / 4) * i + 2 * h) = (uint16_t)(codes >> (16 * h));
      if (i == 0) *(uint16_t*)(blk + 32) = (uint16_t)sbits;
    }
  } else {
    // base-3 digits d = t mod 3 as 2-bit fields: 1 -> 01, -1 -> 10
    const uint32_t digits = spread_bits(nz & ~neg) | (spread_bits(nz & neg) << 1);
    // Lane i < 6 writes bytes 4i..4i+3 = weights 20i..20i+19, which start at
    // slot o = 20i mod E of lane L = 20i / E and end in lane L + 2 (E = 8) or
    // L + 1 (E = 16).  Lane 6 writes the two tail bytes (weights 120..127, in
    // the row's last lane) and the scale.
    const int L = i < 6 ? (20 * i) / E : (120 / E);
    const int o = i < 6 ? (20 * i) % E : 120 % E;
    const uint64_t d0 = lane_value(digits, row0 + L);
    const uint64_t d1 = lane_value(digits, row0 + min(L + 1, LPG - 1));
    uint64_t d;
    if (E == 8) {
      const uint64_t d2 = lane_value(digits, row0 + min(L + 2, LPG - 1));
      d = (d0 | (d1 << 16) | (d2 << 32)) >> (2 * o);
    } else {
      d = (d0 | (d1 << 32)) >> (2 * o);
    }
    uint32_t word;
    if (i < 6) {
      word = base3_byte(d, 5) | (base3_byte(d >> 10, 5) << 8) | (base3_byte(d >> 20, 5) << 16) |
             (base3_byte(d >> 30, 5) << 24);
    } else {
      word = base3_byte(d, 4) | (base3_byte(d >> 8, 4) << 8) | (sbits << 16);
    }
    if (valid && i < 7) *(uint32_t*)(dst + g * 28 + 4 * i) = word;
  }
}

// A wave takes 64 / LPG consecutive groups U times over, a block 256 U / LPG
// groups; the loads of all U are issued first.  U = 2 for absmean (HBM-bound:
// 232 us against 250 with U = 1 and 248 with U = 4 on 604 M weights), 1 for
// Lloyd (VALU-bound).  A grid-stride loop with the next groups loaded ahead
// measured slower at every grid size tried (4 to 32 blocks per CU).
template <int FMT, int METHOD, int U, int LPG>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const u32x4* __restrict__ w, int64_t groups,
                                                                 uint8_t* __restrict__ dst, uint8_t* __restrict__ rounds) {
  constexpr int C = 128 / LPG / 8;  // 16-byte loads per lane
  constexpr int per_block = kQuantThreads / LPG;
  const int lane = threadIdx.x & 63, i = lane & (LPG - 1), row0 = lane & (64 - LPG);
  u32x4 v[U][C];
  int64_t g[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    g[u] = ((int64_t)blockIdx.x * U + u) * per_block + threadIdx.x / LPG;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      v[u][c] = u32x4{0u, 0u, 0u, 0u};
      if (g[u] < groups) v[u][c] = w[g[u] * 16 + i * C + c];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) quantize_group<FMT, METHOD, LPG>(v[u], g[u], g[u] < groups, i, row0, dst, rounds);
}

template <int FMT>
hipError_t launch_quantize_fmt(int method, const u32x4* w, int64_t groups, uint8_t* dst, uint8_t* rounds,
                               hipStream_t stream) {
  if (method == MOE_QUANT_LLOYD) {
    constexpr int64_t per_block = kQuantThreads / kQuantLanesLloyd;
    quantize_kernel<FMT, MOE_QUANT_LLOYD, 1, kQuantLanesLloyd>
        <<<(unsigned)((groups + per_block - 1) / per_block), kQuantThreads, 0, stream>>>(w, groups, dst, rounds);
  } else {
    constexpr int64_t per_block = 2 * kQuantThreads / kQuantLanesAbsmean;
    quantize_kernel<FMT, MOE_QUANT_ABSMEAN, 2, kQuantLanesAbsmean>
        <<<(unsigned)((groups + per_block - 1) / per_block), kQuantThreads, 0, stream>>>(w, groups, dst, rounds);
  }
  return hipGetLastError();
}

}  // namespace

int64_t quantize_max_groups() { return (int64_t)0x7FFFFFFF * kQuantMinGroupsPerBlock; }

hipError_t launch_quantize(int fmt, int method, const uint16_t* w, int64_t groups, uint8_t* dst,
                           uint8_t* rounds, hipStream_t stream) {
  const u32x4* wv = (const u32x4*)w;
  return fmt == MOE_PQ2_0 ? launch_quantize_fmt<kPQ2>(method, wv, groups, dst, rounds, stream)
                          : launch_quantize_fmt<kPTQ1>(method, wv, groups, dst, rounds, stream);
}

}  // namespace moe
