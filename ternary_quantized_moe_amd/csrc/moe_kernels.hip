// HIP kernels of the ternary-expert MoE block for gfx950 (CDNA4).
//
// Pipeline of one forward pass (all on one stream, no host synchronisation):
//   xproj     router logits (W_r + dW_r) x  and  z = A x          matrix cores
//   topk      per token: top-k with lower-index ties, softmax over the k
//   rank      per 256-token block: rank of each slot among the block's slots of
//             the same expert (LDS ballot masks), block histograms
//   scan      per expert: offsets, per-block bases, expert work items
//   scatter   perm[base + rank] = slot id        (counting sort, no atomics)
//   experts   grouped gate/up + SwiGLU, then grouped down + gate weight
//   combine   y = sum of the token's slots + B z                  matrix cores
//
// The forward pass follows the release cards (Scion project README, "The idea"
// and "Serving notes"; FlashNext card, "Model Overview"; container layouts from
// the 35B-A3B card "Weight Representation" and the FlashNext card "Weight
// Representation").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.h"
#include "dense_rows.h"
#include "moe_internal.h"
#include "route_device.h"
#include "wave_ops.h"

namespace moe {

// ============================================================ container decode
// One wave decodes 16 groups: lane l takes quarter q = l/16 of group l%16 with
// the same decoder the expert kernels inline, then writes trits back in
// natural order.
template <int FMT>
__global__ __launch_bounds__(64) void unpack_device_kernel(const uint8_t* __restrict__ src,
                                                          int64_t n_blocks,
                                                          int8_t* __restrict__ trits,
                                                          uint16_t* __restrict__ scales) {
  __shared__ u32x2 lut[FMT == kPTQ1 ? 256 * kLutCopies : 1];
  const int lane = threadIdx.x;
  if (FMT == kPTQ1) {
    ptq1_lut_fill(lut, lane, 64);
    __syncthreads();
  }
  const int r = lane & 15, q = lane >> 4;
  const int64_t b = (int64_t)blockIdx.x * 16 + min<int64_t>(r, n_blocks - 1 - (int64_t)blockIdx.x * 16);
  const uint8_t* blk = src + b * block_bytes_c<FMT>();
  const uint8_t* end = src + n_blocks * block_bytes_c<FMT>();
  // the same 12-byte read the expert kernels make, byte by byte where it would
  // pass the end of the container (this entry point promises no slack)
  const uint8_t* p = blk + (FMT == kPQ2 ? 8 : 6) * q;
  u32x3 v;
  if (p + 12 <= end) {
    v = load_block_x3<FMT>(blk, q);
  } else {
    uint32_t w[3] = {0u, 0u, 0u};
    for (int i = 0; i < 12; ++i)
      if (p + i < end) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
    v = u32x3{w[0], w[1], w[2]};
  }
  u32x4 W[4];
  (void)decode_block_x3<FMT>(v, lut, lane, W);  // all lanes take part in the cross-lane read
  if ((int64_t)blockIdx.x * 16 + r >= n_blocks) return;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t bits = (W[m][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const int8_t t = bits == 0x4000u ? 1 : (bits == 0xC000u ? -1 : 0);
      const int wi = FMT == kPQ2 ? kslot_pq2(m, q, j) : kslot_ptq1(m, q, j);
      trits[b * 128 + wi] = t;
    }
  }
  if (q == 0) scales[b] = *(const uint16_t*)(blk + (FMT == kPQ2 ? 32 : 26));
}

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

hipError_t launch_unpack_device(int fmt, const uint8_t* src, int64_t n_weights, int8_t* trits,
                                uint16_t* scales, hipStream_t stream) {
  const int64_t nb = n_weights / kGroup;
  if (nb == 0) return hipSuccess;
  dim3 grid((unsigned)((nb + 15) / 16));
  if (fmt == kPQ2)
    unpack_device_kernel<kPQ2><<<grid, 64, 0, stream>>>(src, nb, trits, scales);
  else
    unpack_device_kernel<kPTQ1><<<grid, 64, 0, stream>>>(src, nb, trits, scales);
  return hipGetLastError();
}

// ============================================================ dense projections
// out[t][n] = sum_k act[t][k] W[n][k] with fp16 weight rows split exactly into
// two bfloat16 terms (hi + lo) so bf16 matrix cores give fp32-accurate products.
// Block: KS waves splitting K; one 16-token x 16-row tile per block.

// Block = one 16-row tile x up to MT*16 tokens; its KS waves split K in
// 32-wide steps and reduce through LDS.  Each weight k-step is split into bf16
// hi/lo once and reused for all MT token tiles.
template <int EPI, int KS, int MT>
__global__ __launch_bounds__(64 * KS) void dense_kernel(DenseArgs a) {
  __shared__ f32x4 red[KS > 1 ? KS - 1 : 1][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.y * 16 * MT;
  const int n0 = blockIdx.x * 16;
  const int N = a.N0 + a.N1;
  const int n = n0 + i16;

  const int nsteps = (a.K + 31) / 32;
  const int spw = (nsteps + KS - 1) / KS;
  const int s_begin = wave * spw, s_end = min(nsteps, s_begin + spw);

  const uint16_t* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = t0 + 16 * m + i16;
    arow[m] = t < a.T ? a.act + t * a.lda : nullptr;
  }
  const uint16_t* wrow = nullptr;
  const uint16_t* wrowb = nullptr;
  if (n < a.N0) {
    wrow = a.w0 + (int64_t)n * a.K;
    if (a.w0b) wrowb = a.w0b + (int64_t)n * a.K;
  } else if (n < N) {
    wrow = a.w1 + (int64_t)(n - a.N0) * a.K;
  }
  const bool summed = a.w0b != nullptr && n < a.N0;

  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the wave's k-steps in batches of SB, every load of a batch issued before
  // the first multiply (one memory round trip per batch)
  constexpr int SB = 4;
  for (int s0 = s_begin; s0 < s_end; s0 += SB) {
    u32x4 wv[SB], wb[SB], av[SB][MT];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const int kb = 32 * (s0 + j) + 8 * q;
      const bool kin = s0 + j < s_end && kb < a.K;
      wv[j] = (wrow && kin) ? *(const u32x4_a4*)(wrow + kb) : u32x4{0u, 0u, 0u, 0u};
      wb[j] = (summed && kin) ? *(const u32x4_a4*)(wrowb + kb) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < MT; ++m)
        av[j][m] = (arow[m] && kin) ? *(const u32x4*)(arow[m] + kb) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      u32x4 hi, lo;
      if (summed)
        split_sum_f16x8(wv[j], wb[j], hi, lo);
      else
        split_f16x8(wv[j], hi, lo);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        acc[m] = mfma16(av[j][m], hi, acc[m]);
        acc[m] = mfma16(av[j][m], lo, acc[m]);
      }
    }
  }

  if (KS > 1) {
    if (wave > 0)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wave - 1][m][lane] = acc[m];
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] += red[w][m][lane];
  }
  if (n >= N) return;

  // lane holds tokens t0 + 16m + 4q + j, row n
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t tt = t0 + 16 * m + 4 * q + j;
      if (tt >= a.T) continue;
      if (EPI == EPI_XPROJ) {
        if (n < a.N0)
          a.logits[tt * a.N0 + n] = acc[m][j];
        else
          a.z[tt * a.N1 + (n - a.N0)] = (uint16_t)f32_to_bf16(acc[m][j]);
      } else {
        const int d = a.N0;
        float v = acc[m][j];
        const int64_t Tk = a.T * a.top_k;
        const int ns = a.top_k + a.n_shared;
        // the token's slots in batches of 8 loads in flight, summed in slot order
        for (int i0 = 0; i0 < ns; i0 += 8) {
          uint16_t sv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u;
            const int64_t slot = i < a.top_k ? tt * a.top_k + i : Tk + (int64_t)(i - a.top_k) * a.T + tt;
            sv[u] = i < ns ? a.slots[slot * d + n] : (uint16_t)0;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (i0 + u < ns) v += bf16_to_f32(sv[u]);
        }
        a.y[tt * d + n] = (uint16_t)f32_to_bf16(v);
      }
    }
  }
}

// Small-batch x-projection with K split across blocks (xproj_split): block
// (row tile, K slice, group of up to 64 tokens) has 4 waves, each taking kpw
// 32-wide steps of the slice for all MT token tiles with every load of a batch
// of steps in flight at once.  The waves' sums meet in shared memory in wave
// order and the block stores one fp32 partial; the partials are added in slice
// order by their consumers, so no block waits for another and the weight bytes
// spread over the whole chip.
constexpr int kXprojWideRows = 2048;  // output rows from which 33+ tokens take xproj_wide_kernel

// TQ: some rows come from ternary PQ2_0 containers (a.q0b, a.q1).  RT: row
// tiles per block; each activation load then feeds RT tiles (worth it where the
// activations of many tokens would otherwise be re-read once per 16 rows).
template <int MT, int RT, bool TQ>
__global__ __launch_bounds__(256) void xproj_split_kernel(DenseArgs a, int kpw) {
  __shared__ f32x4 red[3][RT][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int N = a.N0 + a.N1 + a.N2;
  const int64_t t0 = (int64_t)blockIdx.z * 64;
  const int nsteps = (a.K + 31) / 32;
  const int s_begin = (blockIdx.y * 4 + wave) * kpw, s_end = min(nsteps, s_begin + kpw);

  const uint16_t* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t t = t0 + 16 * m + i16;
    arow[m] = t < a.T ? a.act + t * a.lda : nullptr;
  }
  const uint16_t* wrow[RT];
  const uint16_t* wrowb[RT];
  const uint8_t* qrow[RT];
  const uint8_t* qrowb[RT];
  bool summed[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int n = (blockIdx.x * RT + r) * 16 + i16;
    wrow[r] = wrowb[r] = nullptr;
    qrow[r] = qrowb[r] = nullptr;
    if (n < a.N0) {
      wrow[r] = a.w0 + (int64_t)n * a.K;
      if (TQ && a.q0b) qrowb[r] = a.q0b + n * pq2_row_bytes(a.K);
      else if (a.w0b) wrowb[r] = a.w0b + (int64_t)n * a.K;
    } else if (n < a.N0 + a.N1) {
      if (TQ && a.q1) qrow[r] = a.q1 + (n - a.N0) * pq2_row_bytes(a.K);
      else wrow[r] = a.w1 + (int64_t)(n - a.N0) * a.K;
    } else if (n < N) {
      wrow[r] = a.w2 + (int64_t)(n - a.N0 - a.N1) * a.K;
    }
    summed[r] = wrowb[r] != nullptr || qrowb[r] != nullptr;
  }

  f32x4 acc[RT][MT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int SB = RT > 1 ? 2 : 4;  // steps whose loads are in flight together
  for (int s0 = s_begin; s0 < s_end; s0 += SB) {
    u32x4 wv[SB][RT], wb[SB][RT], av[SB][MT];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const int kb = 32 * (s0 + j) + 8 * q;
      const bool kin = s0 + j < s_end && kb < a.K;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        wv[j][r] = (wrow[r] && kin) ? *(const u32x4_a4*)(wrow[r] + kb) : u32x4{0u, 0u, 0u, 0u};
        wb[j][r] = (wrowb[r] && kin) ? *(const u32x4_a4*)(wrowb[r] + kb) : u32x4{0u, 0u, 0u, 0u};
        if (TQ) {
          if (qrow[r] && kin) wv[j][r] = pq2_row_f16x8(qrow[r], kb);
          if (qrowb[r] && kin) wb[j][r] = pq2_row_f16x8(qrowb[r], kb);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
        av[j][m] = (arow[m] && kin) ? *(const u32x4*)(arow[m] + kb) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      if (s0 + j >= s_end) break;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        u32x4 hi, lo;
        if (summed[r])
          split_sum_f16x8(wv[j][r], wb[j][r], hi, lo);
        else
          split_f16x8(wv[j][r], hi, lo);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[r][m] = mfma16(av[j][m], hi, acc[r][m]);
          acc[r][m] = mfma16(av[j][m], lo, acc[r][m]);
        }
      }
    }
  }
  if (wave > 0)
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wave - 1][r][m][lane] = acc[r][m];
  __syncthreads();
  if (wave > 0) return;
  float* out = a.part + (int64_t)blockIdx.y * a.T * N;
  // lane holds tokens t0 + 16m + 4q + j, row n of each tile
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int n = (blockIdx.x * RT + r) * 16 + i16;
    if (n >= N) continue;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const f32x4 v = ((acc[r][m] + red[0][r][m][lane]) + red[1][r][m][lane]) + red[2][r][m][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = t0 + 16 * m + 4 * q + j;
        if (t < a.T) out[t * N + n] = v[j];
      }
    }
  }
}

// Combine of a small batch: a block covers RTB 16-row tiles of the model rows
// x 16 tokens with 4 RTB waves = RTB row tiles x 4 slices of K.  The slices'
// partial sums meet in shared memory and are added in slice order; then each
// of 32 RTB threads adds one token's slots to 8 consecutive rows with 16-byte
// reads, in slot order.
// TQ: B comes from a ternary PQ2_0 container (a.q0).
template <int RTB, bool TQ>
__global__ __launch_bounds__(256 * RTB) void combine_small_kernel(DenseArgs a) {
  constexpr int R = 16 * RTB;  // model rows per block
  __shared__ float part[4][16][R + 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int rt = wave % RTB, ks = wave / RTB;
  const int d = a.N0, K = a.K;
  const int n = blockIdx.x * R + rt * 16 + i16;  // d is a multiple of 128
  const int64_t t0 = (int64_t)blockIdx.y * 16;
  const uint16_t* zrow = a.act + std::min<int64_t>(t0 + i16, a.T - 1) * a.lda;
  const uint16_t* wrow = !(TQ && a.q0) && a.w0 ? a.w0 + (int64_t)n * K : nullptr;
  const uint8_t* qrow = TQ && a.q0 ? a.q0 + n * pq2_row_bytes(K) : nullptr;
  const int nsteps = (K + 31) / 32, spw = (nsteps + 3) / 4;
  const int s_begin = ks * spw, s_end = min(nsteps, s_begin + spw);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int SB = 4;  // k-steps whose loads are in flight together
  for (int s0 = s_begin; s0 < s_end; s0 += SB) {
    u32x4 wv[SB], zv[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const int kb = 32 * (s0 + j) + 8 * q;
      const bool kin = (wrow || qrow) && s0 + j < s_end && kb < K;
      if (TQ && qrow)
        wv[j] = kin ? pq2_row_f16x8(qrow, kb) : u32x4{0u, 0u, 0u, 0u};
      else
        wv[j] = kin ? *(const u32x4_a4*)(wrow + kb) : u32x4{0u, 0u, 0u, 0u};
      zv[j] = kin ? *(const u32x4*)(zrow + kb) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      u32x4 hi, lo;
      split_f16x8(wv[j], hi, lo);
      acc = mfma16(zv[j], hi, acc);
      acc = mfma16(zv[j], lo, acc);
    }
  }
  // lane holds tokens 4q + j of the tile, row rt * 16 + i16 of the block
#pragma unroll
  for (int j = 0; j < 4; ++j) part[ks][4 * q + j][rt * 16 + i16] = acc[j];
  __syncthreads();
  constexpr int CPT = R / 8;  // 8-row groups per token
  if (threadIdx.x >= 16 * CPT) return;
  const int tl = threadIdx.x / CPT, c = threadIdx.x % CPT;
  const int64_t t = t0 + tl;
  if (t >= a.T) return;
  const int n0 = blockIdx.x * R + 8 * c;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    v[e] = ((part[0][tl][8 * c + e] + part[1][tl][8 * c + e]) + part[2][tl][8 * c + e]) + part[3][tl][8 * c + e];
  const int64_t Tk = a.T * a.top_k;
  const int ns = a.top_k + a.n_shared;
  for (int i0 = 0; i0 < ns; i0 += 8) {  // slots in order, eight reads in flight
    u32x4 sv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u;
      const int64_t slot = i < a.top_k ? t * a.top_k + i : Tk + (int64_t)(i - a.top_k) * a.T + t;
      sv[u] = i < ns ? *(const u32x4*)(a.slots + slot * d + n0) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u >= ns) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] += bf16_to_f32(sv[u][e] & 0xFFFFu);
        v[2 * e + 1] += bf16_to_f32(sv[u][e] >> 16);
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = f32x2_to_bf16x2(v[2 * e], v[2 * e + 1]);
  *(u32x4_a4*)(a.y + t * d + n0) = o;
}

template <int EPI, int MT>
static void launch_dense_mt(const DenseArgs& a, int N, hipStream_t stream) {
  dim3 grid((unsigned)((N + 15) / 16), (unsigned)((a.T + 16 * MT - 1) / (16 * MT)));
  const int steps = (a.K + 31) / 32;
  // about 4 k-steps (128 inputs) per wave, at most 16 waves (8 with 4 token tiles)
  const int ks = std::max(1, std::min(MT >= 4 ? 8 : 16, (steps + 3) / 4));
  if (ks <= 1) dense_kernel<EPI, 1, MT><<<grid, 64, 0, stream>>>(a);
  else if (ks <= 2) dense_kernel<EPI, 2, MT><<<grid, 128, 0, stream>>>(a);
  else if (ks <= 4) dense_kernel<EPI, 4, MT><<<grid, 256, 0, stream>>>(a);
  else if (ks <= 8 || MT >= 4) dense_kernel<EPI, 8, MT><<<grid, 512, 0, stream>>>(a);
  else dense_kernel<EPI, MT >= 4 ? 8 : 16, MT><<<grid, 1024, 0, stream>>>(a);
}

// Small batches want many blocks (the projections read far more weight bytes
// than activations), so one 16-token tile per block up to 256 tokens; larger
// batches reuse each split weight step for four token tiles.
template <int EPI>
static hipError_t launch_dense(const DenseArgs& a, int N, hipStream_t stream) {
  if (a.T <= 256)
    launch_dense_mt<EPI, 1>(a, N, stream);
  else
    launch_dense_mt<EPI, 4>(a, N, stream);
  return hipGetLastError();
}

// Small-batch x-projection of many rows for 33-256 tokens (fp16 weights): the
// same K slices and fp32 partials as xproj_split_kernel, but a block stages its
// 64 tokens' activations for the slice in LDS, one 128-wide group at a time
// (double-buffered), and each of its four row waves takes RW 16-row tiles over
// the slice (KS wave groups splitting each group's k-steps), so the
// activations are read from L2 once per 64 RW rows instead of once per 16.
constexpr int kWideRowBytes = 256 + 16;  // one token's staged group, padded

template <int MT, int RW, int KS>
__global__ __launch_bounds__(256 * KS) void xproj_wide_kernel(DenseArgs a, int kpw) {
  // KS: wave groups that split each staged group's four k-steps between them
  // (more waves per block where blocks are few), adding up at the end
  constexpr int JS = 4 / KS;           // k-steps per wave and group
  constexpr int NP = 4 / KS;           // staged pieces per thread and group
  __shared__ __align__(16) char stage[2][64 * kWideRowBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wt = wave & 3, ks = wave >> 2;
  const int i16 = lane & 15, q = lane >> 4;
  const int N = a.N0 + a.N1;
  const int64_t t0 = (int64_t)blockIdx.z * 64;
  const int nsteps = (a.K + 31) / 32;
  const int s_begin = blockIdx.y * 4 * kpw, s_end = min(nsteps, s_begin + 4 * kpw);
  const int g_begin = s_begin / 4, g_end = (s_end + 3) / 4;  // 128-wide groups of the slice

  // rows [0, N0) of w0, then [N0, N) of w1 (no summed delta, no third segment)
  const uint16_t* wrow[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int n = blockIdx.x * (64 * RW) + (wt * RW + r) * 16 + i16;
    wrow[r] = n < a.N0 ? a.w0 + (int64_t)n * a.K : n < N ? a.w1 + (int64_t)(n - a.N0) * a.K : nullptr;
  }

  // staging roles: piece u = threadIdx.x + 256 KS p is token row u / 16,
  // 16-byte chunk u % 16 of the group
  const uint16_t* srow[NP];
  int soff[NP], schunk[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int u = threadIdx.x + 256 * KS * p;
    const int64_t t = t0 + (u >> 4);
    schunk[p] = u & 15;
    srow[p] = t < a.T ? a.act + t * a.lda + 8 * schunk[p] : nullptr;
    soff[p] = (u >> 4) * kWideRowBytes + schunk[p] * 16;
  }
  auto stage_load = [&](int g, u32x4 (&raw)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int k = g * 128 + 8 * schunk[p];
      raw[p] = (srow[p] && g < g_end && k < a.K) ? *(const u32x4*)(srow[p] + g * 128) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_store = [&](const u32x4 (&raw)[NP], char* buf) {
#pragma unroll
    for (int p = 0; p < NP; ++p) *(u32x4*)(buf + soff[p]) = raw[p];
  };

  f32x4 acc[RW][MT];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 raw[NP];
  stage_load(g_begin, raw);
  stage_store(raw, stage[0]);
  stage_load(g_begin + 1, raw);
  __syncthreads();
  for (int g = g_begin; g < g_end; ++g) {
    // the wave's steps of the group, their weight loads in flight together
    u32x4 wv[JS][RW];
#pragma unroll
    for (int jj = 0; jj < JS; ++jj) {
      const int st = 4 * g + ks * JS + jj;
      const int kb = 32 * st + 8 * q;
      const bool kin = st < s_end && kb < a.K;
#pragma unroll
      for (int r = 0; r < RW; ++r)
        wv[jj][r] = (wrow[r] && kin) ? *(const u32x4_a4*)(wrow[r] + kb) : u32x4{0u, 0u, 0u, 0u};
    }
    const char* buf = stage[(g - g_begin) & 1];
#pragma unroll
    for (int jj = 0; jj < JS; ++jj) {
      const int j = ks * JS + jj;
      if (4 * g + j >= s_end) break;
      u32x4 av[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) av[m] = *(const u32x4*)(buf + (16 * m + i16) * kWideRowBytes + (4 * j + q) * 16);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        u32x4 hi, lo;
        split_f16x8(wv[jj][r], hi, lo);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[r][m] = mfma16(av[m], hi, acc[r][m]);
          acc[r][m] = mfma16(av[m], lo, acc[r][m]);
        }
      }
    }
    if (g + 1 < g_end) {
      stage_store(raw, stage[(g + 1 - g_begin) & 1]);
      stage_load(g + 2, raw);
    }
    __syncthreads();
  }
  // the other wave groups' sums meet the first's in shared memory, in group order
  f32x4* red = (f32x4*)stage[0];  // [4 row waves][RW][MT][64 lanes]
  for (int kk = 1; kk < KS; ++kk) {
    if (ks == kk)
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) red[((wt * RW + r) * MT + m) * 64 + lane] = acc[r][m];
    __syncthreads();
    if (ks == 0)
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] += red[((wt * RW + r) * MT + m) * 64 + lane];
    __syncthreads();
  }
  if (ks > 0) return;
  float* out = a.part + (int64_t)blockIdx.y * a.T * N;
  // lane holds tokens t0 + 16m + 4q + j, row n of each tile
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int n = blockIdx.x * (64 * RW) + (wt * RW + r) * 16 + i16;
    if (n >= N) continue;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = t0 + 16 * m + 4 * q + j;
        if (t < a.T) out[t * N + n] = acc[r][m][j];
      }
  }
}

// Large batches take the LDS-tiled matrix-core kernels (moe_dense.hip).
hipError_t launch_xproj(const DenseArgs& a, hipStream_t stream) {
  if (a.N2 && !(a.T <= kGroupMaxT && a.part)) return hipErrorInvalidValue;  // w2 rows: split path only
  const int N = a.N0 + a.N1 + a.N2;
  if (a.T > kGroupMaxT && a.wsplit) return launch_dense_gemm<EPI_XPROJ>(a, N, stream);
  if (a.T <= kGroupMaxT && a.part) {
    const XprojSplit sp = xproj_split(a.K);
    const dim3 grid((unsigned)((N + 15) / 16), (unsigned)sp.splits, (unsigned)((a.T + 63) / 64));
    const int mt = (int)std::min<int64_t>(4, (a.T + 15) / 16);
    // where many tokens meet many fp16 rows (the draft head's 2048-4096 rows
    // at 33-256 tokens) the LDS-staged kernel; one 16-row tile per block elsewhere
    const bool tq = a.q0b || a.q1;
    const dim3 g((unsigned)((N + 15) / 16), grid.y, grid.z);
    if (a.staged && !tq && !a.w0b && !a.N2 && mt >= 3 && N >= kXprojWideRows) {
      // 64 rows per block, and eight waves (two per 16-row tile, splitting the
      // k-steps) where that leaves fewer than four blocks per compute unit.
      // Measured on the draft head at 64 tokens (fc1 4096 rows, 512 blocks):
      // 128 rows and four waves per block 22.2 us, 64 rows and four waves
      // 17.8, 64 rows and eight waves 17.0, sixteen waves 20.8
      const dim3 gw((unsigned)((N + 63) / 64), grid.y, grid.z);
      const bool ks2 = (int64_t)gw.x * gw.y * gw.z < 1024;
      if (ks2) {
        if (mt == 3) xproj_wide_kernel<3, 1, 2><<<gw, 512, 0, stream>>>(a, sp.kpw);
        else xproj_wide_kernel<4, 1, 2><<<gw, 512, 0, stream>>>(a, sp.kpw);
      } else {
        if (mt == 3) xproj_wide_kernel<3, 1, 1><<<gw, 256, 0, stream>>>(a, sp.kpw);
        else xproj_wide_kernel<4, 1, 1><<<gw, 256, 0, stream>>>(a, sp.kpw);
      }
    } else if (tq) {
      if (mt == 1) xproj_split_kernel<1, 1, true><<<g, 256, 0, stream>>>(a, sp.kpw);
      else if (mt == 2) xproj_split_kernel<2, 1, true><<<g, 256, 0, stream>>>(a, sp.kpw);
      else if (mt == 3) xproj_split_kernel<3, 1, true><<<g, 256, 0, stream>>>(a, sp.kpw);
      else xproj_split_kernel<4, 1, true><<<g, 256, 0, stream>>>(a, sp.kpw);
    } else {
      if (mt == 1) xproj_split_kernel<1, 1, false><<<g, 256, 0, stream>>>(a, sp.kpw);
      else if (mt == 2) xproj_split_kernel<2, 1, false><<<g, 256, 0, stream>>>(a, sp.kpw);
      else if (mt == 3) xproj_split_kernel<3, 1, false><<<g, 256, 0, stream>>>(a, sp.kpw);
      else xproj_split_kernel<4, 1, false><<<g, 256, 0, stream>>>(a, sp.kpw);
    }
    return hipGetLastError();
  }
  if (a.q0b || a.q1) return hipErrorInvalidValue;  // ternary rows need the split or the tiled path
  return launch_dense<EPI_XPROJ>(a, N, stream);
}

hipError_t launch_combine(const DenseArgs& a, hipStream_t stream) {
  if (a.T > kGroupMaxT && a.wsplit) return launch_dense_gemm<EPI_COMBINE>(a, a.N0, stream);
  // blocks of 16 rows up to 32 tokens, of 32 rows beyond (measured: fewer
  // weight bytes per CU win until the token tiles multiply the blocks)
  const unsigned tt = (unsigned)((a.T + 15) / 16);
  if (a.q0) {
    if (a.T <= 32)
      combine_small_kernel<1, true><<<dim3((unsigned)(a.N0 / 16), tt), 256, 0, stream>>>(a);
    else
      combine_small_kernel<2, true><<<dim3((unsigned)(a.N0 / 32), tt), 512, 0, stream>>>(a);
  } else {
    if (a.T <= 32)
      combine_small_kernel<1, false><<<dim3((unsigned)(a.N0 / 16), tt), 256, 0, stream>>>(a);
    else
      combine_small_kernel<2, false><<<dim3((unsigned)(a.N0 / 32), tt), 512, 0, stream>>>(a);
  }
  return hipGetLastError();
}

// ============================================================ routing
// One wave per token: k rounds of a wave-wide argmax over the E logits (larger
// value first, equal values to the lower expert index; -0.0 equals +0.0), then
// the softmax over the selected logits.

// One wave per token: k rounds of a wave-wide argmax over the E logits (larger
// value first, equal values to the lower expert index; -0.0 equals +0.0), then
// the softmax over the selected logits.
template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntk = (int)((a.T + 3) / 4);
  if ((int)blockIdx.x >= ntk) {
    fold_z(a, (int)blockIdx.x - ntk, (int)gridDim.x - ntk);
    return;
  }
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t < a.T) topk_token<PER>(a, t, lane, nullptr);
}

// Lane = token.  Each wave of the 256-token block sets bit `lane` of
// mask[wave][e] for each expert e the token selected; a slot's rank inside the
// block is the number of earlier tokens (lower waves, then lower lanes) that
// selected the same expert.
__global__ __launch_bounds__(256) void rank_kernel(RouteArgs a) {
  extern __shared__ unsigned long long mask[];  // [4][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.E, k = a.k;
  for (int i = threadIdx.x; i < 4 * E; i += 256) mask[i] = 0ull;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kRouteBlock + threadIdx.x;
  const bool valid = t < a.T;
  if (valid)
    for (int i = 0; i < k; ++i) atomicOr(&mask[wave * E + a.idx[t * k + i]], 1ull << lane);
  __syncthreads();
  if (valid) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i = 0; i < k; ++i) {
      const int e = a.idx[t * k + i];
      int r = __popcll(mask[wave * E + e] & below);
      for (int w = 0; w < wave; ++w) r += __popcll(mask[w * E + e]);
      a.slot_rank[t * k + i] = r;
    }
  }
  for (int e = threadIdx.x; e < E; e += 256) {
    int c = 0;
    for (int w = 0; w < 4; ++w) c += __popcll(mask[w * E + e]);
    a.block_cnt[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Work items of C positions over the experts' runs of the permutation (thread
// e of the 1024: expert e with `total` slots from off_e), then the shared
// experts' tokens in runs of C.  Every thread of the block calls it.
__device__ __forceinline__ void emit_items(const RouteArgs& a, int e, int total, int off_e, int C, Item* items,
                                           int32_t* n_items, int* wsum) {
  const int E = a.E;
  const int chunks = e < E ? (total + C - 1) / C : 0;
  int routed_items;
  const int istart = block_inclusive_scan(chunks, wsum, &routed_items) - chunks;
  for (int c = 0; c < chunks; ++c) {
    Item it;
    it.bank = e;
    it.pos = off_e + c * C;
    it.n = min(C, total - c * C);
    it.pad = 0;
    items[istart + c] = it;
  }
  const int per_shared = (int)((a.T + C - 1) / C);
  const int64_t Tk = a.T * a.k;
  for (int idx = e; idx < a.S * per_shared; idx += 1024) {
    const int s = idx / per_shared, c = idx % per_shared;
    Item it;
    it.bank = E + s;
    it.pos = (int)(Tk + (int64_t)s * a.T + (int64_t)c * C);
    it.n = (int)min((int64_t)C, a.T - (int64_t)c * C);
    it.pad = 0;
    items[routed_items + idx] = it;
  }
  if (e == 0) *n_items = routed_items + a.S * per_shared;
}

// One block of 1024 threads, thread = expert.
__global__ __launch_bounds__(1024) void scan_kernel(RouteArgs a, int nb) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  const int E = a.E;
  // the expert's per-block counts are read in batches of 32 with every load
  // of a batch in flight (two passes: the total, then the bases), so a batch
  // costs one memory round trip
  constexpr int NBB = 32;
  int total = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nb; b0 += NBB) {
      int c[NBB];
#pragma unroll
      for (int j = 0; j < NBB; ++j) c[j] = b0 + j < nb ? a.block_cnt[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < NBB; ++j) total += c[j];
    }
  }
  // exclusive scan of totals
  int unused;
  const int off_e = block_inclusive_scan(total, wsum, &unused) - total;
  if (e < E) {
    a.counts[e] = total;
    a.offsets[e] = off_e;
    int run = off_e;
    for (int b0 = 0; b0 < nb; b0 += NBB) {
      int c[NBB];
#pragma unroll
      for (int j = 0; j < NBB; ++j) c[j] = b0 + j < nb ? a.block_cnt[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < NBB; ++j) {
        if (b0 + j < nb) a.block_base[(int64_t)(b0 + j) * E + e] = run;
        run += c[j];
      }
    }
  }
  if (e == 0) a.offsets[E] = (int)(a.T * a.k);
  // work items: ceil(count / chunk) per routed expert, then the shared experts;
  // a second list of the same form for the down projection when it is asked for
  emit_items(a, e, total, off_e, a.chunk, a.items, a.n_items, wsum);
  if (a.items2) emit_items(a, e, total, off_e, a.chunk2, a.items2, a.n_items2, wsum);
}

__global__ __launch_bounds__(256) void scatter_kernel(RouteArgs a) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= a.T * a.k) return;
  const int64_t t = s / a.k;
  const int e = a.idx[s];
  const int64_t b = t / kRouteBlock;
  a.perm[a.block_base[b * a.E + e] + a.slot_rank[s]] = (int)s;
}

// Grouping of a small batch (T <= kGroupMaxT) in one block: per-expert counts,
// offsets, ranks (ballot masks per 64-token chunk, the same order rule as the
// multi-block path), permutation and work items of a.chunk tokens (and of
// a.chunk2 for the down projection when a.items2 is set).  PER = 0: after topk_kernel.  PER > 0 (T <= kFusedMaxT
// and T k <= kFusedMaxSlots): the block's 16 waves first select the top k of
// the tokens themselves, keeping the indices in LDS, which saves a launch.
constexpr int kFusedMaxT = 16;  // one token per wave: beyond that one CU does too much of the top-k
constexpr int kFusedMaxSlots = 4096;

template <int PER>
__global__ __launch_bounds__(1024) void group_small_kernel(RouteArgs a) {
  __shared__ unsigned long long mask[kGroupMaxT / 64][kMaxExperts];
  __shared__ int scan_buf[1024];
  __shared__ int wsum[16];
  __shared__ int sidx[PER > 0 ? kFusedMaxSlots : 1];
  if (blockIdx.x > 0) {  // fused launch: fold blocks
    fold_z(a, (int)blockIdx.x - 1, (int)gridDim.x - 1);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.E, k = a.k;
  const int T = (int)a.T;
  const int nchunks = (T + 63) / 64;
  constexpr int P1 = PER > 0 ? PER : 1;
  if (PER > 0)
    for (int t = wave; t < T; t += 16) topk_token<P1>(a, t, lane, sidx);
  const int* ix = PER > 0 ? sidx : a.idx;
  for (int i = threadIdx.x; i < nchunks * kMaxExperts; i += 1024) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  if (wave < nchunks) {
    const int t = 64 * wave + lane;
    if (t < T)
      for (int i = 0; i < k; ++i) atomicOr(&mask[wave][ix[t * k + i]], 1ull << lane);
  }
  __syncthreads();

  const int e = threadIdx.x;
  int total = 0;
  if (e < E)
    for (int c = 0; c < nchunks; ++c) total += __popcll(mask[c][e]);
  int unused;
  const int off_e = block_inclusive_scan(total, wsum, &unused) - total;
  if (e < E) {
    a.counts[e] = total;
    a.offsets[e] = off_e;
  }
  if (e == 0) a.offsets[E] = T * k;
  // work items of a.chunk tokens, and (when asked for) the down projection's
  // of a.chunk2
  emit_items(a, e, total, off_e, a.chunk, a.items, a.n_items, wsum);
  if (a.items2) emit_items(a, e, total, off_e, a.chunk2, a.items2, a.n_items2, wsum);
  __syncthreads();
  scan_buf[e] = off_e;
  __syncthreads();
  for (int sl = threadIdx.x; sl < T * k; sl += 1024) {
    const int t = sl / k;
    const int ex = ix[sl];
    const int c = t >> 6, ln = t & 63;
    int r = __popcll(mask[c][ex] & (ln == 0 ? 0ull : (~0ull >> (64 - ln))));
    for (int cc = 0; cc < c; ++cc) r += __popcll(mask[cc][ex]);
    a.perm[scan_buf[ex] + r] = sl;
  }
}

hipError_t launch_route(const RouteArgs& a, int64_t max_items, hipStream_t stream) {
  (void)max_items;
  const int nb = (int)((a.T + kRouteBlock - 1) / kRouteBlock);
  // (E > 512 would need more registers than a 1024-thread block's waves have)
  if (a.T <= kFusedMaxT && a.T * a.k <= kFusedMaxSlots && a.E <= 512) {
    const unsigned g = 1u + (unsigned)fold_blocks(a, 1024);
    if (a.E <= 64) group_small_kernel<1><<<g, 1024, 0, stream>>>(a);
    else if (a.E <= 128) group_small_kernel<2><<<g, 1024, 0, stream>>>(a);
    else if (a.E <= 256) group_small_kernel<4><<<g, 1024, 0, stream>>>(a);
    else group_small_kernel<8><<<g, 1024, 0, stream>>>(a);
    return hipGetLastError();
  }
  const dim3 tg((unsigned)((a.T + 3) / 4 + fold_blocks(a, 256)));
  if (a.E <= 64) topk_kernel<1><<<tg, 256, 0, stream>>>(a);
  else if (a.E <= 128) topk_kernel<2><<<tg, 256, 0, stream>>>(a);
  else if (a.E <= 256) topk_kernel<4><<<tg, 256, 0, stream>>>(a);
  else if (a.E <= 512) topk_kernel<8><<<tg, 256, 0, stream>>>(a);
  else topk_kernel<16><<<tg, 256, 0, stream>>>(a);
  if (a.T <= kGroupMaxT) {
    group_small_kernel<0><<<1, 1024, 0, stream>>>(a);
  } else {
    rank_kernel<<<nb, 256, 4 * a.E * sizeof(unsigned long long), stream>>>(a);
    scan_kernel<<<1, 1024, 0, stream>>>(a, nb);
    scatter_kernel<<<(unsigned)((a.T * a.k + 255) / 256), 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
