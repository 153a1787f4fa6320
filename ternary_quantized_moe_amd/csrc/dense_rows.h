// Weight rows of the x-projection and the combine held as ternary PQ2_0
// containers: the 35B-A3B release stores its trained corrections and router
// deltas in the PQ2_0 byte layout (Scion-35B-A3B card, "Weight
// Representation").  A code times its fp16 group scale is itself an fp16 value
// (s, -s or 0), so the dense kernels expand the codes into exactly the fp16
// operands they read from an fp16 matrix and everything after the load is
// shared: a ternary-coded matrix gives bit for bit the result of its fp16
// expansion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

constexpr int kPq2BlockBytes = 34;

// Bytes of one row of K weights (K % 128 == 0) in row-major PQ2_0 groups.
__host__ __device__ __forceinline__ int64_t pq2_row_bytes(int K) { return (int64_t)(K / 128) * kPq2BlockBytes; }

// Weights k..k+7 (k % 8 == 0) of a PQ2_0 row as four packed fp16 pairs:
// code 01 -> s, 11 -> -s (the sign bit flipped), 00 -> +0.
__device__ __forceinline__ u32x4 pq2_row_f16x8(const uint8_t* row, int k) {
  const uint8_t* blk = row + (k >> 7) * kPq2BlockBytes;
  const uint32_t codes = *(const uint16_t*)(blk + ((k & 127) >> 2));
  const uint32_t s = *(const uint16_t*)(blk + 32);
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t c0 = (codes >> (4 * e)) & 3u, c1 = (codes >> (4 * e + 2)) & 3u;
    const uint32_t h0 = (s ^ ((c0 >> 1) << 15)) & (0u - (c0 & 1u));
    const uint32_t h1 = (s ^ ((c1 >> 1) << 15)) & (0u - (c1 & 1u));
    out[e] = (h0 & 0xFFFFu) | ((h1 & 0xFFFFu) << 16);
  }
  return out;
}

}  // namespace moe
