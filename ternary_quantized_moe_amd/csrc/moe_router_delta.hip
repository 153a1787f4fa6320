// U (V x) for the factorised router delta, on the vector units.  A block
// takes TB tokens and folds their V x slices (in slice order) into shared
// memory, with every slice's loads in flight together (V x comes as columns of
// the router's own partials up to 256 tokens, as an fp32 matrix beyond); each wave then
// walks groups of router rows, RB rows for each 16-lane row of the wave.  Lane
// c of a row takes the 8-wide chunks c, c + 16, ... of the rd inputs, so its
// loads of U and its shared-memory reads of V x are contiguous across the
// row's lanes, and each V x read feeds RB rows.  A token's partial dot products
// meet in four DPP exchanges inside the row; lane c writes token c.  The work
// is small next to the x-projection (E x rd weights against (E + r) x d), so it
// is not put on matrix cores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "router_delta.h"
#include "wave_ops.h"

namespace moe {

namespace {

constexpr int kDeltaThreads = 256;
constexpr int kDeltaWaves = kDeltaThreads / 64;
constexpr int kDeltaMaxSlices = 8;

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_row_f32<kDppXor1>(v);
  v += dpp_row_f32<kDppXor2>(v);
  v += dpp_row_f32<kDppHalfMirror>(v);
  v += dpp_row_f32<kDppMirror>(v);
  return v;
}

template <int TB, int RB, bool ADD>
__global__ __launch_bounds__(kDeltaThreads) void router_delta_kernel(const float* __restrict__ vpart, int vsplits,
                                                                     int ldv, int64_t T, int rd,
                                                                     const uint16_t* __restrict__ U, int E,
                                                                     float* __restrict__ dst, int ldd) {
  static_assert(TB <= 16, "one token per lane of a 16-lane row");
  extern __shared__ __align__(16) float vs[];  // [TB][rd]
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int nt = (int)min<int64_t>(TB, T - t0);
  if (ldv % 4 == 0 && (uintptr_t)vpart % 16 == 0) {  // 16-byte pieces
    const int nv = TB * rd / 4;
    const int64_t slice = T * ldv / 4;
    for (int i0 = threadIdx.x; i0 < nv; i0 += 4 * kDeltaThreads) {
      f32x4 part[4][kDeltaMaxSlices];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kDeltaThreads;
        const int tl = 4 * i / rd;
        const bool live = i < nv && tl < nt;
        const f32x4* src = (const f32x4*)vpart + (t0 + tl) * (ldv / 4) + (i - tl * (rd / 4));
#pragma unroll
        for (int s = 0; s < kDeltaMaxSlices; ++s)
          part[u][s] = (live && s < vsplits) ? src[s * slice] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kDeltaThreads;
        f32x4 v = part[u][0];
#pragma unroll
        for (int s = 1; s < kDeltaMaxSlices; ++s)
          if (s < vsplits) v += part[u][s];
        if (i < nv) ((f32x4*)vs)[i] = v;
      }
    }
  } else {  // single values (a partial row whose V x columns are not 16-byte aligned)
    const int nv = TB * rd;
    const int64_t slice = T * (int64_t)ldv;
    for (int i0 = threadIdx.x; i0 < nv; i0 += 4 * kDeltaThreads) {
      float part[4][kDeltaMaxSlices];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kDeltaThreads;
        const int tl = i / rd;
        const bool live = i < nv && tl < nt;
        const float* src = vpart + (t0 + tl) * ldv + (i - tl * rd);
#pragma unroll
        for (int s = 0; s < kDeltaMaxSlices; ++s) part[u][s] = (live && s < vsplits) ? src[s * slice] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kDeltaThreads;
        float v = part[u][0];
#pragma unroll
        for (int s = 1; s < kDeltaMaxSlices; ++s)
          if (s < vsplits) v += part[u][s];
        if (i < nv) vs[i] = v;
      }
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane >> 4, c16 = lane & 15;
  const int groups = (E + 4 * RB - 1) / (4 * RB);
  for (int g = blockIdx.y * kDeltaWaves + wave; g < groups; g += kDeltaWaves * gridDim.y) {
    const int e0 = (4 * g + r16) * RB;
    float acc[TB][RB];
#pragma unroll
    for (int tl = 0; tl < TB; ++tl)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[tl][rb] = 0.f;
    // KB chunks per batch, their U loads in flight together
    constexpr int KB = kDeltaMaxRank / 128 / RB;
    for (int k0 = 8 * c16; k0 < rd; k0 += 128 * KB) {
      u32x4 ub[KB][RB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int k = k0 + 128 * kb;
          ub[kb][rb] = (k < rd && e0 + rb < E) ? *(const u32x4*)(U + (int64_t)(e0 + rb) * rd + k)
                                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k = k0 + 128 * kb;
        if (k >= rd) break;
        float uf[RB][8];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uf[rb][2 * j] = f16_to_f32(ub[kb][rb][j] & 0xFFFFu);
            uf[rb][2 * j + 1] = f16_to_f32(ub[kb][rb][j] >> 16);
          }
#pragma unroll
        for (int tl = 0; tl < TB; ++tl) {
          const f32x4 v0 = *(const f32x4*)(vs + tl * rd + k);
          const f32x4 v1 = *(const f32x4*)(vs + tl * rd + k + 4);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[tl][rb] += uf[rb][j] * v0[j];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[tl][rb] += uf[rb][4 + j] * v1[j];
          }
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mine = 0.f;
#pragma unroll
      for (int tl = 0; tl < TB; ++tl) {
        const float s = row16_sum(acc[tl][rb]);
        if (c16 == tl) mine = s;
      }
      if (e0 + rb < E && c16 < nt) {
        float* o = dst + (t0 + c16) * (int64_t)ldd + e0 + rb;
        *o = ADD ? *o + mine : mine;
      }
    }
  }
  if (!ADD && blockIdx.y == 0) {
    const int zc = ldd - E;
    for (int i = threadIdx.x; i < nt * zc; i += kDeltaThreads) {
      const int tl = i / zc;
      dst[(t0 + tl) * (int64_t)ldd + E + (i - tl * zc)] = 0.f;
    }
  }
}

template <int TB, int RB>
hipError_t launch_tb(const float* vpart, int vsplits, int ldv, int64_t T, int rd, const uint16_t* U, int E, float* dst,
                     int ldd, bool add, int64_t target_blocks, hipStream_t stream) {
  const int64_t bx = (T + TB - 1) / TB;
  if (bx > 0x7FFFFFFF) return hipErrorInvalidValue;
  // row-group slices: enough blocks to spread U over the chip at few tokens;
  // fewer as token groups multiply (each block folds all its tokens' inputs)
  const int64_t per_wave = (E + 4 * RB * kDeltaWaves - 1) / (4 * RB * kDeltaWaves);
  const unsigned by = (unsigned)std::min<int64_t>(per_wave, std::max<int64_t>(1, target_blocks / bx));
  const size_t lds = (size_t)TB * rd * sizeof(float);
  const dim3 grid((unsigned)bx, by);
  if (add)
    router_delta_kernel<TB, RB, true><<<grid, kDeltaThreads, lds, stream>>>(vpart, vsplits, ldv, T, rd, U, E, dst,
                                                                                     ldd);
  else
    router_delta_kernel<TB, RB, false><<<grid, kDeltaThreads, lds, stream>>>(vpart, vsplits, ldv, T, rd, U, E, dst,
                                                                                     ldd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_delta(const float* vpart, int vsplits, int ldv, int64_t T, int rd, const uint16_t* U,
                               int E, float* dst, int ldd, bool add, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (rd <= 0 || rd % 8 || rd > kDeltaMaxRank || E <= 0 || ldd < E || ldv < rd || vsplits < 1 ||
      vsplits > kDeltaMaxSlices)
    return hipErrorInvalidValue;
  // few tokens: 8 per block, one row per lane row, many row slices; many
  // tokens (one fp32 V x): 16 per block and 4 rows per lane row, so each read
  // of V x feeds four rows, about four blocks per compute unit
  if (T <= 256) return launch_tb<8, 1>(vpart, vsplits, ldv, T, rd, U, E, dst, ldd, add, 256, stream);
  return launch_tb<16, 4>(vpart, vsplits, ldv, T, rd, U, E, dst, ldd, add, 1024, stream);
}

}  // namespace moe
