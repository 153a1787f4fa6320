// Dense projections of large batches on the matrix cores:
//   x-projection  logits = (W_r + dW_r) x (fp32) and z = A x (bf16)
//   combine       y = B z + the token's expert slots (bf16)
// Scion README "The idea" and "Serving notes" (router delta and the low-rank
// correction branch on the block output).
//
// The fp16 weight rows are first split once per call into exact bf16 hi/lo
// operand pairs (device_common.h), stored tile by tile in matrix-core operand
// order, so a wave reads each operand of a 16-row tile as one contiguous 1 KB.
// A unit of work is (64 tokens, 128 weight rows); a block of 8 waves stages the
// tokens' activations one 128-wide group at a time into a double-buffered LDS
// tile and each wave multiplies them with its 16-row tile, whose split operands
// it streams from the workspace one group ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.h"
#include "dense_rows.h"
#include "moe_internal.h"

namespace moe {

// Blocks of 8 waves, one 16-row tile each, run two to a CU (four waves per
// SIMD at up to 128 registers), so one block's barrier and load waits overlap
// the other's matrix work even where the units are few (a 4096 x 512 product
// has 256 units, one per CU).
constexpr int kDenseWaves = 8;
constexpr int kDenseRT = 1;                             // row tiles per wave
constexpr int kDenseRows = kDenseWaves * 16 * kDenseRT;  // weight rows per unit
constexpr int kDenseTok = 64;                     // tokens per unit (4 MFMA M tiles)
constexpr int kDenseRow = 256 + 32;               // staged bytes per token row and group (32 bytes of padding: 16 left a third of the LDS cycles bank conflicts)
constexpr int kDenseBuf = kDenseTok * kDenseRow;  // one staged group
constexpr int kOutStride = kDenseRows + 4;        // floats per token row of the combine tile
constexpr size_t kDenseLds = std::max<size_t>(2 * (size_t)kDenseBuf, (size_t)kDenseTok * kOutStride * 4);
constexpr int kDenseP = kDenseTok * 16 / (64 * kDenseWaves);  // staged 16-byte chunks per thread and group

int dense_kpad(int K) { return (K + kGroup - 1) / kGroup * kGroup; }

int64_t dense_split_bytes(int N, int K) { return (int64_t)(N + 15) / 16 * 16 * dense_kpad(K) * 4; }

// ------------------------------------------------------------------ split
// Split weights: 16-row tile, group g, MFMA m, hi/lo, quarter q, row i16 ->
// 16 bytes (8 bf16 of elements g*128 + 32m + 8q .. +7 of row 16 tile + i16) at
// ((((tile * G + g) * 4 + m) * 2 + hl) * 64 + 16 q + i16) * 16.  Elements past K
// and rows past N are zero.  Block (tile, g) reads its 16 rows x 128 elements
// with 256-byte row pieces and writes its 8 KB of hi/lo operands as one run
// after rearranging them in shared memory.
__global__ __launch_bounds__(256) void split_kernel(DenseArgs a, int N, int Kp, u32x4* __restrict__ out) {
  __shared__ u32x4 tile_ops[512];
  const int G = Kp / kGroup;
  const int tile = blockIdx.x / G, g = blockIdx.x % G;
  const int t = threadIdx.x;
  const int i16 = t >> 4, c = t & 15;  // row of the tile, 8-element chunk of the group
  const int n = tile * 16 + i16, k = g * kGroup + 8 * c;
  u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
  if (k < a.K && n < N) {
    const int64_t rb = pq2_row_bytes(a.K);
    if (n < a.N0) {
      const u32x4 w = a.q0 ? pq2_row_f16x8(a.q0 + n * rb, k) : *(const u32x4_a4*)(a.w0 + (int64_t)n * a.K + k);
      if (a.q0b)
        split_sum_f16x8(w, pq2_row_f16x8(a.q0b + n * rb, k), hi, lo);
      else if (a.w0b)
        split_sum_f16x8(w, *(const u32x4_a4*)(a.w0b + (int64_t)n * a.K + k), hi, lo);
      else
        split_f16x8(w, hi, lo);
    } else {
      split_f16x8(a.q1 ? pq2_row_f16x8(a.q1 + (n - a.N0) * rb, k)
                       : *(const u32x4_a4*)(a.w1 + (int64_t)(n - a.N0) * a.K + k), hi, lo);
    }
  }
  const int m = c >> 2, q = c & 3;
  tile_ops[(m * 2) * 64 + 16 * q + i16] = hi;
  tile_ops[(m * 2 + 1) * 64 + 16 * q + i16] = lo;
  __syncthreads();
  u32x4* dst = out + (int64_t)blockIdx.x * 512;
  dst[t] = tile_ops[t];
  dst[t + 256] = tile_ops[t + 256];
}

// ------------------------------------------------------------------ GEMM
template <int EPI, int NTT>
__device__ __forceinline__ void dense_unit(const DenseArgs& a, const u32x4* __restrict__ w2, int N, int Kp,
                                           int64_t t0, int rb, char* smem) {
  // the wave index through readfirstlane: the compiler then knows it (and
  // `active`) to be uniform, so the branch on it is scalar and does not break
  // the counting of loads in flight
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, q = lane >> 4;
  const int G = Kp / kGroup;
  const int row0 = rb * kDenseRows + wave * 16 * kDenseRT;
  const bool active = row0 < N;

  // the wave's row tiles (a tile past the last one repeats it; rows past N
  // are zero and not stored); operand (g, m, hl) at + (g * 8 + m * 2 + hl) * 64
  const u32x4* wp[kDenseRT];
#pragma unroll
  for (int rt = 0; rt < kDenseRT; ++rt) {
    const int tile = min(row0 / 16 + rt, (N - 1) / 16);
    wp[rt] = w2 + (int64_t)tile * G * 512 + lane;
  }

  // staging roles: token row si, 16-byte chunk sc (elements 8 sc .. 8 sc + 7 of
  // the group = MFMA sc / 4, quarter sc % 4); a wave reads 4 rows x 256 bytes
  int si[kDenseP], sc[kDenseP];
  const uint16_t* srow[kDenseP];
#pragma unroll
  for (int pp = 0; pp < kDenseP; ++pp) {
    const int u = threadIdx.x + pp * 64 * kDenseWaves;
    si[pp] = u >> 4;
    sc[pp] = u & 15;
    srow[pp] = a.act + std::min<int64_t>(t0 + si[pp], a.T - 1) * a.lda;
  }
  // Every lane stages (rows past the unit's tokens repeat the last token and
  // are not read), with no branch: loads under a lane condition would make the
  // compiler wait for every load in flight, the next group's weights included,
  // before each staging store.  K is a multiple of 8 (of 128 but for the
  // combine's K = r, whose tail past K is zero-filled by the compare).
  auto stage_load = [&](int g, u32x4 (&raw)[kDenseP]) {
#pragma unroll
    for (int pp = 0; pp < kDenseP; ++pp) {
      const int k = g * kGroup + 8 * sc[pp];
      const u32x4 v = *(const u32x4*)(srow[pp] + min(k, a.K - 8));
      raw[pp] = k < a.K ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_store = [&](const u32x4 (&raw)[kDenseP], char* buf) {
#pragma unroll
    for (int pp = 0; pp < kDenseP; ++pp) *(u32x4*)(buf + si[pp] * kDenseRow + sc[pp] * 16) = raw[pp];
  };

  u32x4 B[kDenseRT][4][2];  // [row tile][m][hi, lo] of the next group
  if (active && G > 0) {
#pragma unroll
    for (int rt = 0; rt < kDenseRT; ++rt)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) B[rt][m][hl] = wp[rt][(m * 2 + hl) * 64];
  }
  u32x4 s0[kDenseP], s1[kDenseP];  // staged loads of the next two groups
  __syncthreads();  // the previous unit is done with the shared memory
  if (G > 0) {      // (K = 0: a combine without correction, the slots alone)
    stage_load(0, s0);
    stage_store(s0, smem);
    stage_load(min(1, G - 1), s1);
  }
  __syncthreads();

  f32x4 acc[NTT][kDenseRT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int rt = 0; rt < kDenseRT; ++rt) acc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // step g: issue the loads of group g + 2, multiply group g, store group g + 1
  // (loaded one step earlier), load the weights of group g + 1; the last steps
  // refetch the last group (unused).  The A operands are read from shared
  // memory one MFMA slice m at a time.
  auto step = [&](int g, u32x4 (&issue)[kDenseP], const u32x4 (&ready)[kDenseP]) {
    const int gn = min(g + 1, G - 1);
    stage_load(min(g + 2, G - 1), issue);
    if (active) {
      const char* ab = smem + (g & 1) * kDenseBuf + i16 * kDenseRow + q * 16;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4 A[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) A[tt] = *(const u32x4*)(ab + tt * 16 * kDenseRow + m * 64);
#pragma unroll
        for (int rt = 0; rt < kDenseRT; ++rt)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) acc[tt][rt] = mfma16(A[tt], B[rt][m][hl], acc[tt][rt]);
      }
#pragma unroll
      for (int rt = 0; rt < kDenseRT; ++rt)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) B[rt][m][hl] = wp[rt][(gn * 8 + m * 2 + hl) * 64];
    }
    stage_store(ready, smem + ((g + 1) & 1) * kDenseBuf);
    __syncthreads();
  };
  for (int g = 0; g < G; g += 2) {
    step(g, s0, s1);
    if (g + 1 < G) step(g + 1, s1, s0);
  }

  if (EPI == EPI_XPROJ) {
    if (!active) return;
    // lane holds tokens t0 + 16 tt + 4q + j, rows row0 + 16 rt + i16
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = t0 + 16 * tt + 4 * q + j;
        if (t >= a.T) continue;
#pragma unroll
        for (int rt = 0; rt < kDenseRT; ++rt) {
          const int r = row0 + 16 * rt + i16;
          if (r < a.N0)
            a.logits[t * a.N0 + r] = acc[tt][rt][j];
          else if (r < N)
            a.z[t * a.N1 + (r - a.N0)] = (uint16_t)f32_to_bf16(acc[tt][rt][j]);
        }
      }
  } else {
    // through shared memory, so each thread sums 8 consecutive rows of a token
    // with 16-byte slot reads
    float* tile = (float*)smem;
    if (active) {
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int rt = 0; rt < kDenseRT; ++rt)
            tile[(16 * tt + 4 * q + j) * kOutStride + row0 - rb * kDenseRows + 16 * rt + i16] = acc[tt][rt][j];
    }
    __syncthreads();
    const int d = a.N0;
    const int64_t Tk = a.T * a.top_k;
    // a thread takes two items (a token's 8 consecutive rows) at a time and reads
    // their slots (routed in rank order, then shared) in batches of 8 per item,
    // 16 loads in flight, added in slot order.  Loads past the last slot, and
    // those of an item past the tile, re-read a valid row and are not used.
    constexpr int kItems = NTT * 16 * (kDenseRows / 8), kStep = 64 * kDenseWaves;
    const int ns = a.top_k + a.n_shared;
    for (int item = threadIdx.x; item < kItems; item += 2 * kStep) {
      bool ok[2];
      int64_t t[2];
      int n0[2];
      const uint16_t* rbase[2];  // routed slot i of the token: rbase + i d
      const uint16_t* sbase[2];  // shared slot s: sbase + s T d
      float v[2][8];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int ip = item + p * kStep;
        const int tl = ip / (kDenseRows / 8), c = ip % (kDenseRows / 8);
        t[p] = t0 + tl;
        n0[p] = rb * kDenseRows + 8 * c;
        ok[p] = ip < kItems && t[p] < a.T && n0[p] < d;
        const int64_t tc = ok[p] ? t[p] : t0;
        const int nc = ok[p] ? n0[p] : rb * kDenseRows;
        rbase[p] = a.slots + tc * a.top_k * d + nc;
        sbase[p] = a.slots + (Tk + tc) * d + nc;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[p][e] = ok[p] ? tile[(ok[p] ? tl : 0) * kOutStride + 8 * (ok[p] ? c : 0) + e] : 0.f;
      }
      for (int i0 = 0; i0 < ns; i0 += 8) {
        u32x4 sv[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = min(i0 + u, ns - 1);
          const int64_t off = i < a.top_k ? (int64_t)i * d : (int64_t)(i - a.top_k) * a.T * d;
#pragma unroll
          for (int p = 0; p < 2; ++p) sv[u][p] = *(const u32x4*)((i < a.top_k ? rbase[p] : sbase[p]) + off);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (i0 + u >= ns) break;
#pragma unroll
          for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[p][2 * e] += bf16_to_f32(sv[u][p][e] & 0xFFFFu);
              v[p][2 * e + 1] += bf16_to_f32(sv[u][p][e] >> 16);
            }
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (!ok[p]) continue;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f32x2_to_bf16x2(v[p][2 * e], v[p][2 * e + 1]);
        *(u32x4_a4*)(a.y + t[p] * d + n0[p]) = o;
      }
    }
  }
}

// Persistent blocks over units l = (row block l / TB, token tile l % TB); the
// blocks of one XCD (block index mod 8) take a contiguous range of units, so
// they share one row block's split weights in their L2.  (32-token units, which
// give small products a second block per CU, measured slower.)
template <int EPI>
__global__ __launch_bounds__(64 * kDenseWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void dense_gemm_kernel(DenseArgs a, const u32x4* w2, int N, int Kp) {
  extern __shared__ __align__(16) char smem[];
  const int64_t TB = (a.T + kDenseTok - 1) / kDenseTok;
  const int64_t U = TB * ((N + kDenseRows - 1) / kDenseRows);
  const int64_t per = (U + 7) / 8;
  for (int64_t u = blockIdx.x; u < 8 * per; u += gridDim.x) {
    const int64_t l = (u & 7) * per + (u >> 3);
    if (l >= U) continue;
    const int rb = (int)(l / TB);
    const int64_t t0 = (l % TB) * kDenseTok;
    switch ((int)std::min<int64_t>(4, (a.T - t0 + 15) / 16)) {
      case 1: dense_unit<EPI, 1>(a, w2, N, Kp, t0, rb, smem); break;
      case 2: dense_unit<EPI, 2>(a, w2, N, Kp, t0, rb, smem); break;
      case 3: dense_unit<EPI, 3>(a, w2, N, Kp, t0, rb, smem); break;
      default: dense_unit<EPI, 4>(a, w2, N, Kp, t0, rb, smem); break;
    }
  }
}

template <int EPI>
hipError_t launch_dense_gemm(const DenseArgs& a, int N, hipStream_t stream) {
  const int Kp = dense_kpad(a.K);
  u32x4* w2 = (u32x4*)a.wsplit;
  const int64_t blocks = (int64_t)(N + 15) / 16 * (Kp / kGroup);  // (tile, group) pairs
  if (blocks > 0) {
    split_kernel<<<(unsigned)blocks, 256, 0, stream>>>(a, N, Kp, w2);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  auto kern = dense_gemm_kernel<EPI>;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kDenseWaves, kDenseLds);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t U = ((a.T + kDenseTok - 1) / kDenseTok) * ((N + kDenseRows - 1) / kDenseRows);
  const int64_t grid = std::min<int64_t>((int64_t)cu_count() * per_cu, U);
  kern<<<dim3((unsigned)grid), 64 * kDenseWaves, kDenseLds, stream>>>(a, w2, N, Kp);
  return hipGetLastError();
}

template hipError_t launch_dense_gemm<EPI_XPROJ>(const DenseArgs&, int, hipStream_t);
template hipError_t launch_dense_gemm<EPI_COMBINE>(const DenseArgs&, int, hipStream_t);

}  // namespace moe
