// Gather and decode rows of a Q4_0 table for gfx950: the FlashNext n-gram table
// (Scion-FlashNext-176B-A6B card, "Model Overview": 320,001,536 rows of 160
// values; "Weight Representation": one Q4_0 tensor, groups of 32 along each
// row, decoded per row).
//
// Q4_0 block (ggml's layout, which the card's format name refers to): a
// binary16 scale d, then 16 code bytes; value j < 16 is the low nibble of byte
// j, value 16 + j its high nibble; value = d (q - 8).  Rows are back to back,
// 18 bytes per 32 values.  Every d (q - 8) is exact in fp32, so the output is
// the exact decoded value.
//
// Layout: four threads per 32-value block.  Thread k reads the scale and code
// bytes 4k..4k+3, decodes values 4k..4k+3 and 16+4k..16+4k+3 and writes them
// as two 16-byte stores; consecutive threads walk the blocks of one row, then
// the next row, so the output is written in order, 128 contiguous bytes per
// block.  An index outside [0, rows) gives a row of quiet NaN and reads nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kPleThreads = 256;
constexpr int kQ4Block = 32;
constexpr int kQ4BlockBytes = 18;

__global__ __launch_bounds__(kPleThreads) void ple_gather_kernel(const uint8_t* __restrict__ table, int64_t n_rows,
                                                                 uint32_t row_blocks, const int64_t* __restrict__ idx,
                                                                 uint32_t n_idx, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * kPleThreads + threadIdx.x;
  const uint32_t per_row = row_blocks * 4;
  const uint32_t i = t / per_row;
  if (i >= n_idx) return;
  const uint32_t rem = t - i * per_row, b = rem >> 2, k = rem & 3;
  const int64_t r = idx[i];
  f32x4 lo, hi;
  if (r >= 0 && r < n_rows) {
    const uint8_t* blk = table + r * (int64_t)(row_blocks * kQ4BlockBytes) + b * kQ4BlockBytes;
    const float d = f16_to_f32(*(const uint16_t*)blk);
    const uint32_t q = *(const uint16_t*)(blk + 2 + 4 * k) | ((uint32_t)*(const uint16_t*)(blk + 4 + 4 * k) << 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = d * (float)((int)((q >> (8 * e)) & 15u) - 8);
      hi[e] = d * (float)((int)((q >> (8 * e + 4)) & 15u) - 8);
    }
  } else {
    const float nan = __builtin_nanf("");
    lo = f32x4{nan, nan, nan, nan};
    hi = lo;
  }
  float* o = out + (int64_t)i * (row_blocks * kQ4Block) + b * kQ4Block + 4 * k;
  *(f32x4*)o = lo;
  *(f32x4*)(o + 16) = hi;
}

}  // namespace

hipError_t launch_ple_gather(const uint8_t* table, int64_t n_rows, int row_len, const int64_t* idx, int64_t n_idx,
                             float* out, hipStream_t stream) {
  const uint32_t row_blocks = (uint32_t)(row_len / kQ4Block), per_row = row_blocks * 4;
  // each launch covers at most 2^31 threads, so thread and row numbers fit 32 bits
  const int64_t rows_per_launch = std::max<int64_t>(1, ((int64_t)1 << 31) / per_row);
  for (int64_t i0 = 0; i0 < n_idx; i0 += rows_per_launch) {
    const uint32_t n = (uint32_t)std::min<int64_t>(rows_per_launch, n_idx - i0);
    const uint32_t blocks = (uint32_t)(((int64_t)n * per_row + kPleThreads - 1) / kPleThreads);
    ple_gather_kernel<<<blocks, kPleThreads, 0, stream>>>(table, n_rows, row_blocks, idx + i0, n,
                                                          out + i0 * row_len);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
