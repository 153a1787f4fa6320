// Grouped ternary expert kernels (gate/up + SwiGLU, down + gate weight).
//
// Containers are tile-major on the device (include/moe_ternary.h): the 16
// blocks of one group of a 16-row tile are contiguous, so the block of row
// tile_row0 + i16, group g sits at tile base + (16 g + i16) * block bytes, and
// one load instruction of a wave (16 rows x 4 quarters) reads 16 consecutive
// blocks.
//
// Work item = (bank, up to 16 consecutive positions of the (expert, token)
// order).  A unit of work is (item, block tile): the block stages the item's
// activation rows in LDS once (coalesced, already in matrix-core operand order)
// and its waves take 16-row tiles of the bank's containers and stream them
// along K with a register prefetch ring.
// Every 128-weight block is decoded in registers into bf16 B operands (+-2
// encoding, see device_common.h), multiplied with v_mfma_f32_16x16x32_bf16
// (tokens are the M dimension, rows the N dimension), and the group scale is
// applied to the fp32 accumulator.  With KS > 1 the waves of a tile split K and
// reduce through LDS.  Blocks are persistent: each loops over units, so the
// PTQ1_0 byte table is filled once per block.
// Expert FFN: Scion README "Serving notes" (per-expert mul_mat_id); SwiGLU
// reading and container layouts: include/moe_ternary.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "dense_rows.h"
#include "device_common.h"
#include "moe_internal.h"
#include "route_device.h"

namespace moe {

constexpr int MODE_GATEUP = 0;
constexpr int MODE_DOWN = 1;

// Stage the item's activation rows (n tokens x K) into LDS as matrix-core A
// operands in the container format's k-slot order: row i, group g, MFMA m,
// quarter q -> 16 bytes at i * stride + ((g * 4 + m) * 4 + q) * 16.  The
// rows are padded by 32 bytes (a row stride of 8 mod 64 dwords): with 16 bytes
// the operand reads of lanes 16 apart (quarters q and q + 1) met on the same
// banks, and the LDS counted a third of its cycles as bank conflicts.
__host__ __device__ constexpr int stage_stride(int K) { return 2 * K + 32; }

// Per-item table of the down projection, after the staged rows: each token
// row's slot and half its gate weight (the operands encode 2t).  It is filled
// with the staging, so a tile epilogue reads shared memory instead of making
// two dependent global loads (position -> slot -> gate weight) per tile.
__host__ __device__ constexpr int slot_table_bytes(int nmax) { return (8 * nmax + 15) / 16 * 16; }

__device__ __forceinline__ void stage_slots(const ExpertArgs& a, const Item& it, int* slot_of, float* wgt_of) {
  const int i = threadIdx.x;
  if (i < it.n) {
    const int64_t p = it.pos + i;
    const bool routed = p < a.Tk;
    const int slot = routed ? a.perm[p] : (int)p;
    slot_of[i] = slot;
    wgt_of[i] = 0.5f * (routed ? a.topk_w[slot] : 1.f);
  }
}

template <int FMT, int MODE>
__device__ __forceinline__ void stage_rows(const ExpertArgs& a, const Item& it, char* xs, int K) {
  const int G = K / kGroup;
  const int units = it.n * G * 4;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int i = u / (G * 4), rem = u % (G * 4), g = rem >> 2, q = rem & 3;
    const int64_t p = it.pos + i;
    const uint16_t* row;
    if (MODE == MODE_GATEUP) {
      const int64_t tok = p < a.Tk ? a.perm[p] / a.k : (p - a.Tk) % a.T;
      row = a.x + tok * a.d;
    } else {
      row = a.h + p * a.f;
    }
    u32x4 out[4];
    act_operands<FMT>(load_act_raw<FMT>(row, g, q), out);
    char* dst = xs + i * stage_stride(K) + (g * 16 + q) * 16;
#pragma unroll
    for (int m = 0; m < 4; ++m) *(u32x4*)(dst + m * 64) = out[m];
  }
}

// One (item, tile block) unit.  GW > 0: each wave covers exactly GW groups
// (K = GW * KS * 128, a compile-time shape), fully unrolled so the prefetch
// ring, the load offsets and the LDS offsets are static.  GW = 0: any K.
template <int FMT, int MODE, int WPB, int KS, int RT, int D, int GW>
__device__ __forceinline__ void expert_unit(const ExpertArgs& a, const Item& it, int tblock, const u32x2* lut,
                                            char* xs, f32x4* red, int* slot_of, float* wgt_of,
                                            const uint8_t* bank_in = nullptr) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar rows
  const int i16 = lane & 15, q = lane >> 4;
  const int K = MODE == MODE_GATEUP ? a.d : a.f;
  const int G = K / kGroup;
  constexpr int BB = block_bytes_c<FMT>();
  const int64_t row_bytes = (int64_t)G * BB;
  const uint8_t* bank = bank_in ? bank_in : a.banks + a.offsets[it.bank];  // (the caller's, if given)
  const int64_t gu_bytes = (int64_t)a.f * (a.d / kGroup) * BB;

  constexpr int TPB = WPB / KS;  // tiles per block
  const int tile = tblock * TPB + wave / KS;
  const int ks = wave % KS;
  const int n_tiles = MODE == MODE_GATEUP ? a.f / 16 : a.d / (16 * RT);
  const bool active = tile < n_tiles;
  const int gpk = GW > 0 ? GW : (G + KS - 1) / KS;
  const int gb = ks * gpk, ge = min(G, gb + gpk);

  // rows of the RT tiles, already advanced to the wave's first group
  const uint8_t* rows[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int64_t off;
    if (MODE == MODE_GATEUP)  // r even: gate rows, r odd: up rows, of features tile*16 .. +16 (RT == 2)
      off = (r & 1) * gu_bytes + (int64_t)tile * 16 * row_bytes;
    else
      off = 2 * gu_bytes + ((int64_t)tile * RT + r) * 16 * row_bytes;
    rows[r] = bank + off + i16 * BB + (int64_t)gb * 16 * BB;
  }

  auto fetch = [&](const uint8_t* blk) -> u32x3 {
    return FMT == kPQ2 ? load_block_x3_a4<FMT>(blk, q) : load_block_x3<FMT>(blk, q);
  };
  // weight prefetch starts before the activations are staged
  u32x3 ring[D][RT];
  if (active) {
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (GW > 0 ? j < GW : gb + j < ge)
#pragma unroll
        for (int r = 0; r < RT; ++r) ring[j][r] = fetch(rows[r] + j * 16 * BB);
  }

  __syncthreads();  // the previous unit is done with the staging buffer
  stage_rows<FMT, MODE>(a, it, xs, K);
  if (MODE == MODE_DOWN) stage_slots(a, it, slot_of, wgt_of);
  __syncthreads();

  f32x4 acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // rows past the item's tokens read its last row; their results are dropped
  const char* arow = xs + min(i16, it.n - 1) * stage_stride(K) + q * 16 + gb * 256;

  auto step = [&](int i, u32x3 (&cur)[RT]) {
    u32x4 A[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = *(const u32x4*)(arow + i * 256 + m * 64);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      u32x4 W[4];
      const float s = decode_block_x3<FMT>(cur[r], lut, lane, W);
      f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) tmp = mfma16(A[m], W[m], tmp);
      acc[r] += s * tmp;
    }
  };

  if (active) {
    if (GW > 0) {
#pragma unroll
      for (int i = 0; i < (GW > 0 ? GW : 1); ++i) {
        u32x3 cur[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) cur[r] = ring[i % D][r];
        if (i + D < GW)
#pragma unroll
          for (int r = 0; r < RT; ++r) ring[i % D][r] = fetch(rows[r] + (i + D) * 16 * BB);
        step(i, cur);
      }
    } else {
      const int n = ge - gb;
      for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
          const int i = i0 + j;
          if (i >= n) break;
          // the slot is used before it is refilled: in this rolled loop a refill
          // while the old value is live would move the ring through copies at
          // every turn, each waiting for all loads in flight
          step(i, ring[j]);
          if (i + D < n)
#pragma unroll
            for (int r = 0; r < RT; ++r) ring[j][r] = fetch(rows[r] + (int64_t)(i + D) * 16 * BB);
        }
      }
    }
  }

  if (KS > 1) {
    const int tl = wave / KS;
    if (ks > 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) red[((tl * (KS - 1) + ks - 1) * RT + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int w = 1; w < KS; ++w)
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] += red[((tl * (KS - 1) + w - 1) * RT + r) * 64 + lane];
    }
    __syncthreads();  // red is reused by the block's next unit
    if (ks > 0) return;
  }
  if (!active) return;

  // lane holds positions it.pos + 4q + j, column i16 of each tile; the
  // operands encode 2t, hence the 0.5
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ti = 4 * q + j;
    if (ti >= it.n) continue;
    const int64_t p = it.pos + ti;
    if (MODE == MODE_GATEUP) {
      const float g = 0.5f * acc[0][j], u = 0.5f * acc[1][j];
      const float hv = silu_mul(g, u);
      a.h[p * a.f + (int64_t)tile * 16 + i16] = (uint16_t)f32_to_bf16(hv);
    } else {
      const int64_t slot = slot_of[ti];
      const float wgt = wgt_of[ti];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int64_t row = ((int64_t)tile * RT + r) * 16 + i16;
        a.slots[slot * a.d + row] = (uint16_t)f32_to_bf16(wgt * acc[r][j]);
      }
    }
  }
}

// Epilogue of one tile: lane holds positions it.pos + 4q + j, column i16 of
// each of the RT row tiles; the operands encode 2t, hence the 0.5.
template <int MODE, int RT>
__device__ __forceinline__ void tile_epilogue(const ExpertArgs& a, const Item& it, int tile, int lane,
                                              const f32x4 (&acc)[RT], const int* slot_of, const float* wgt_of) {
  const int i16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ti = 4 * q + j;
    if (ti >= it.n) continue;
    const int64_t p = it.pos + ti;
    if (MODE == MODE_GATEUP) {
      const float g = 0.5f * acc[0][j], u = 0.5f * acc[1][j];
      const float hv = silu_mul(g, u);
      a.h[p * a.f + (int64_t)tile * 16 + i16] = (uint16_t)f32_to_bf16(hv);
    } else {
      const int64_t slot = slot_of[ti];
      const float wgt = wgt_of[ti];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int64_t row = ((int64_t)tile * RT + r) * 16 + i16;
        a.slots[slot * a.d + row] = (uint16_t)f32_to_bf16(wgt * acc[r][j]);
      }
    }
  }
}

// Streaming unit: the item's tiles [tile0, tile_end); wave w takes tiles
// tile0 + w, tile0 + w + WPB, ...  and streams them back to back through one
// prefetch ring of D groups (D divides the compile-time group count G), so the
// loads for the next tile are in flight while the current one finishes.
// PIPE: each step adds the previous step's product to the accumulators, so
// the add does not wait for the MFMAs just issued (5 more registers per row
// tile: the kernels built for two waves per SIMD have them, the others not).
template <int FMT, int MODE, int WPB, int RT, int D, int G, bool PIPE>
__device__ __forceinline__ void expert_stream_unit(const ExpertArgs& a, const Item& it, int tile0, int tile_end,
                                                   const u32x2* lut, char* xs, char* scratch, int* slot_of,
                                                   float* wgt_of) {
  static_assert(G % D == 0 && D <= G, "the ring depth must divide the group count");
  // the wave index through readfirstlane, so the wave's row bases are known to
  // be uniform (scalar registers, scalar branches)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, q = lane >> 4;
  constexpr int K = G * kGroup;
  constexpr int BB = block_bytes_c<FMT>();
  constexpr int64_t row_bytes = (int64_t)G * BB;
  const uint8_t* bank = a.banks + a.offsets[it.bank];
  const int64_t gu_bytes = (int64_t)a.f * (a.d / kGroup) * BB;
  constexpr int rows_per_tile = MODE == MODE_GATEUP ? 16 : 16 * RT;
  constexpr int64_t tile_stride = (int64_t)rows_per_tile * row_bytes * WPB;  // to the wave's next tile

  const int first = tile0 + wave;
  const int ntw = first < tile_end ? (tile_end - first + WPB - 1) / WPB : 0;

  const uint8_t* rows[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int64_t off;
    if (MODE == MODE_GATEUP)  // r even: gate rows, r odd: up rows (RT == 2)
      off = (r & 1) * gu_bytes + (int64_t)first * 16 * row_bytes;
    else
      off = 2 * gu_bytes + ((int64_t)first * RT + r) * 16 * row_bytes;
    rows[r] = bank + off;  // the tile's base: chunk of group g at + g * 16 * BB
  }

  // PQ2_0 streams aligned chunks and rearranges them through LDS; PTQ1_0, whose
  // decoder already leans on LDS for its byte table, loads its windows directly
  constexpr bool CH = FMT == kPQ2;
  auto fetch = [&](const uint8_t* chunk) -> u32x4 {
    if (CH) return load_chunk<FMT>(chunk, lane);
    const u32x3 v = load_block_x3<FMT>(chunk + i16 * BB, q);
    return u32x4{v.x, v.y, v.z, 0u};
  };
  u32x4 ring[D][RT];
  if (ntw > 0) {
#pragma unroll
    for (int j = 0; j < D; ++j)
#pragma unroll
      for (int r = 0; r < RT; ++r) ring[j][r] = fetch(rows[r] + j * 16 * BB);
  }

  __syncthreads();  // the previous unit is done with the staging buffer
  stage_rows<FMT, MODE>(a, it, xs, K);
  if (MODE == MODE_DOWN) stage_slots(a, it, slot_of, wgt_of);
  __syncthreads();

  const char* arow = xs + min(i16, it.n - 1) * stage_stride(K) + q * 16;
  // PQ2_0 with a ring of two or more slots: the realigned window of the next
  // group is taken from the ring one step ahead, so its shared-memory round trip
  // overlaps this step's decode and products (ring slot j + 1 holds the next
  // group; after the last slot, slot 0, refilled first, holds it).  A one-slot
  // ring holds the next group only after this step's refill.
  constexpr bool PF = CH && D > 1;
  u32x3 win[RT];
  if (PF && ntw > 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r) win[r] = chunk_window<FMT>(ring[0][r], scratch, lane);
  }
  for (int t = 0; t < ntw; ++t) {
    const bool more = t + 1 < ntw;
    f32x4 acc[RT], ptmp[RT];
    float ps[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      ptmp[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      ps[r] = 0.f;
    }
#pragma unroll 1
    for (int g0 = 0; g0 < G; g0 += D) {
      // the next D groups: the rest of this tile, else the start of the next
      // one; after the wave's last tile, the groups of this step again (in
      // bounds and unused; just read, so they come from the caches, not HBM).
      // The refills are unconditional so the compiler can wait for each ring
      // slot alone instead of for every load in flight.
      const int64_t nxt = g0 + D < G ? (int64_t)(g0 + D) * 16 * BB : (more ? tile_stride : (int64_t)g0 * 16 * BB);
#pragma unroll
      for (int j = 0; j < D; ++j) {
        u32x4 A[4];
        const char* ap = arow + (g0 + j) * 256;
#pragma unroll
        for (int m = 0; m < 4; ++m) A[m] = *(const u32x4*)(ap + m * 64);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          u32x4 W[4];
          u32x3 v;
          if (PF) {
            v = win[r];
            win[r] = chunk_window<FMT>(ring[(j + 1) % D][r], scratch, lane);
          } else if (CH) {
            v = chunk_window<FMT>(ring[j][r], scratch, lane);
          } else {
            v = u32x3{ring[j][r].x, ring[j][r].y, ring[j][r].z};
          }
          float s;
          if (CH) {
            ring[j][r] = fetch(rows[r] + nxt + j * 16 * BB);
            s = decode_block_x3<FMT>(v, lut, lane, W);
          } else {
            // PTQ1_0 decodes the slot before refilling it: with the old value
            // dead at the refill, the load lands in the slot's own registers and
            // the ring needs no copies (and no wait for every load) at its turn
            s = decode_block_x3<FMT>(v, lut, lane, W);
            __builtin_amdgcn_sched_barrier(0);
            ring[j][r] = fetch(rows[r] + nxt + j * 16 * BB);
          }
          f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
          // the wave issues its products at a raised priority, so a wave of the
          // SIMD that is ready to multiply goes ahead of the others' decode work
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int m = 0; m < 4; ++m) tmp = mfma16(A[m], W[m], tmp);
          __builtin_amdgcn_s_setprio(0);
          if (PIPE) {
            acc[r] += ps[r] * ptmp[r];
            ptmp[r] = tmp;
            ps[r] = s;
          } else {
            acc[r] += s * tmp;
          }
        }
        // keep each step's loads and decode in place: hoisting the ring's
        // refills would double the registers the ring needs
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (PIPE)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r] += ps[r] * ptmp[r];
    tile_epilogue<MODE, RT>(a, it, first + WPB * t, lane, acc, slot_of, wgt_of);
#pragma unroll
    for (int r = 0; r < RT; ++r) rows[r] += tile_stride;
  }
}

// FS: container formats the kernel handles (1: PQ2_0, 2: PTQ1_0, 3: both), so a
// single-format layer does not pay for the other decoder's registers.
template <int MODE, int WPB, int RT, int D, int G, int FS, int WPE>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void expert_stream_kernel(ExpertArgs a, int tiles_per_unit, int units_per_item) {
  extern __shared__ __align__(16) char smem[];
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  char* xs = smem + lut_bytes;
  if (a.fmt_mask & 2) ptq1_lut_fill(lut, threadIdx.x, blockDim.x);  // visible after the unit's first sync
  // one chunk scratch per wave: its LDS operations complete in order, so row tile
  // r + 1 writes only after tile r's window has been read
  int* slot_of = (int*)(xs + a.nmax * stage_stride(G * kGroup));
  float* wgt_of = (float*)(slot_of + a.nmax);
  char* scratch = xs + a.nmax * stage_stride(G * kGroup) + slot_table_bytes(a.nmax) + (threadIdx.x >> 6) * kChunkScratch;
  const int n_tiles = MODE == MODE_GATEUP ? a.f / 16 : a.d / (16 * RT);
  const int64_t units = (int64_t)(*a.n_items) * units_per_item;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const Item it = a.items[u / units_per_item];
    const int tile0 = (int)(u % units_per_item) * tiles_per_unit;
    const int tile_end = min(n_tiles, tile0 + tiles_per_unit);
    if (FS == 2 || (FS == 3 && a.formats[it.bank] == kPTQ1))
      expert_stream_unit<kPTQ1, MODE, WPB, RT, D, G, (WPE <= 2)>(a, it, tile0, tile_end, lut, xs, scratch, slot_of, wgt_of);
    else
      expert_stream_unit<kPQ2, MODE, WPB, RT, D, G, (WPE <= 2)>(a, it, tile0, tile_end, lut, xs, scratch, slot_of, wgt_of);
  }
}

// Persistent blocks over units (item, tile block).
// Dynamic LDS: [PTQ1_0 byte table if the layer has PTQ1_0 banks][staged rows][slot table][KS reduction]
template <int MODE, int WPB, int KS, int RT, int D, int GW>
__global__ __launch_bounds__(64 * WPB) void expert_dec_kernel(ExpertArgs a, int tblocks_per_item) {
  extern __shared__ __align__(16) char smem[];
  const int K = MODE == MODE_GATEUP ? a.d : a.f;
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  char* xs = smem + lut_bytes;
  int* slot_of = (int*)(xs + a.nmax * stage_stride(K));
  float* wgt_of = (float*)(slot_of + a.nmax);
  f32x4* red = (f32x4*)(xs + a.nmax * stage_stride(K) + slot_table_bytes(a.nmax));
  if (a.fmt_mask & 2) ptq1_lut_fill(lut, threadIdx.x, blockDim.x);  // visible after the unit's first sync
  const int64_t units = (int64_t)(*a.n_items) * tblocks_per_item;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const Item it = a.items[u / tblocks_per_item];
    const int tb = (int)(u % tblocks_per_item);
    if (a.formats[it.bank] == kPTQ1)
      expert_unit<kPTQ1, MODE, WPB, KS, RT, D, GW>(a, it, tb, lut, xs, red, slot_of, wgt_of);
    else
      expert_unit<kPQ2, MODE, WPB, KS, RT, D, GW>(a, it, tb, lut, xs, red, slot_of, wgt_of);
  }
}

// ============================================================ batches of at most 4 tokens
// The block takes three launches instead of five: the x-projection; the
// gate/up kernel below, whose blocks each route the batch themselves; and one
// kernel for the down projection and the combine.
//
// Routing in the gate/up kernel: every block adds up the logit partials of the
// T tokens and selects their top k with the routing kernels' own topk_token
// (the same summation order, so the choice equals the one moe_route exports),
// then groups the slots in shared memory: a bit mask of the tokens per expert,
// exclusive scans over the experts for the offsets and the work items, and the
// permutation in canonical (expert, token) order.  Block 0 also stores the
// logits, indices, gate weights, counts, offsets, permutation and work items
// for the down kernel.  Blocks past route_blocks fold z from the partials.

// Shared-memory bytes of the routing area for T tokens, top k, E experts, S shared.
__host__ __device__ constexpr int tiny_route_bytes(int T, int k, int E, int S) {
  return (T * E + 2 * T * k + 4) * 4 + (std::min(E, T * k) + S) * (int)sizeof(Item);
}

// The byte offsets and container formats of the layer's nb = E + S banks,
// copied into LDS at the start of the small-batch kernels, where reading them
// after the routing (or the work item) would add one dependent memory round
// trip before the first weight load.  [offsets: nb int64][formats: nb bytes,
// padded to 8]
__host__ __device__ constexpr int bank_table_bytes(int nb) { return nb * 8 + ((nb + 7) & ~7); }
__host__ __device__ constexpr int align8(int b) { return (b + 7) & ~7; }

// The batch's top k per token (waves 0 .. T-1, one token each), then the
// grouping by one wave with one slot per lane (T k <= 64): slot s of token
// t = s / k and expert e sorts by the key 4 e + t, so its position in the
// canonical (expert, token) order is the number of smaller keys; the slot with
// an expert's smallest key starts that expert's work item.
template <int PER>
__device__ void tiny_route(const RouteArgs& r, char* area, bool store, const int*& perm_out, const Item*& items_out,
                           int& n_items_out) {
  const int T = (int)r.T, k = r.k, E = r.E, S = r.S, Tk = T * k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = (int)blockDim.x >> 6;
  float* slog = (float*)area;
  int* sidx = (int*)(slog + T * E);
  int* perm = sidx + Tk;
  int* nitems = perm + Tk;
  Item* items = (Item*)(nitems + 4);
  // the logits: every wave folds 64 experts of one token at a time
  const int nch = (E + 63) / 64;
  for (int c = wave; c < T * nch; c += nw) {
    const int t = c / nch, e = (c % nch) * 64 + lane;
    if (e < E) {
      const float v = fold_logit(r, t, e);
      slog[t * E + e] = v;
      if (store) r.logits[(int64_t)t * E + e] = v;
    }
  }
  __syncthreads();
  if (wave < T) topk_token<PER>(r, wave, lane, sidx, store, slog);
  __syncthreads();
  if (wave == 0) {
    const bool valid = lane < Tk;
    const int e = valid ? sidx[lane] : 0x7FFFFFF;
    const int key = valid ? 4 * e + lane / k : 0x7FFFFFFF;
    int pos = 0, cnt = 0, before = 0;
    for (int j = 0; j < Tk; ++j) {  // j is uniform: the loop runs the same count in every lane
      const int kj = __builtin_amdgcn_readlane(key, j);
      pos += kj < key ? 1 : 0;
      cnt += (kj >> 2) == e ? 1 : 0;
      before += ((kj >> 2) == e && kj < key) ? 1 : 0;
    }
    const bool first = valid && before == 0;
    const uint64_t firsts = __ballot(first);
    int iidx = 0;
    for (int j = 0; j < Tk; ++j) {
      const int kj = __builtin_amdgcn_readlane(key, j);
      iidx += (((firsts >> j) & 1ull) && kj < key) ? 1 : 0;
    }
    const int n_routed = __popcll(firsts);
    if (valid) {
      perm[pos] = lane;
      if (store) r.perm[pos] = lane;
    }
    if (first) items[iidx] = Item{e, pos, cnt, 0};
    if (lane < S) items[n_routed + lane] = Item{E + lane, Tk + lane * T, T, 0};
    if (lane == 0) *nitems = n_routed + S;
  }
  __syncthreads();
  const int n_items = *nitems;
  if (store) {
    for (int i = tid; i < n_items; i += blockDim.x) r.items[i] = items[i];
    if (tid == 0) *r.n_items = n_items;
  }
  perm_out = perm;
  items_out = items;
  n_items_out = n_items;
}

// Dynamic LDS: [PTQ1_0 byte table][staged rows][slot table][KS reduction][routing area]
template <int WPB, int KS, int RT, int D, int GW, int PER>
__global__ __launch_bounds__(64 * WPB) void expert_route_dec_kernel(ExpertArgs a, RouteArgs r, int tblocks_per_item,
                                                                    int route_blocks) {
  extern __shared__ __align__(16) char smem[];
  if ((int)blockIdx.x >= route_blocks) {  // the fold of z
    fold_z(r, (int)blockIdx.x - route_blocks, (int)gridDim.x - route_blocks);
    return;
  }
  const int K = a.d;
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  char* xs = smem + lut_bytes;
  int* slot_of = (int*)(xs + a.nmax * stage_stride(K));
  float* wgt_of = (float*)(slot_of + a.nmax);
  f32x4* red = (f32x4*)(xs + a.nmax * stage_stride(K) + slot_table_bytes(a.nmax));
  char* area = (char*)red + (KS > 1 ? (WPB / KS) * (KS - 1) * RT * 64 * 16 : 0);
  const int nbk = a.E + a.S;
  int64_t* soff = (int64_t*)(area + align8(tiny_route_bytes((int)a.T, a.k, a.E, a.S)));
  uint8_t* sfmt = (uint8_t*)(soff + nbk);
  // the bank table's loads go out with the routing's own (visible after its syncs)
  for (int i = threadIdx.x; i < nbk; i += blockDim.x) {
    soff[i] = a.offsets[i];
    sfmt[i] = a.formats[i];
  }
  if (a.fmt_mask & 2) ptq1_lut_fill(lut, threadIdx.x, blockDim.x);  // visible after the routing's syncs
  const int* perm;
  const Item* items;
  int n_items;
  tiny_route<PER>(r, area, blockIdx.x == 0, perm, items, n_items);
  ExpertArgs la = a;
  la.perm = perm;  // this block's own permutation (block 0's global copy is not yet visible to the others)
  const int64_t units = (int64_t)n_items * tblocks_per_item;
  for (int64_t u = blockIdx.x; u < units; u += route_blocks) {
    const Item it = items[u / tblocks_per_item];
    const int tb = (int)(u % tblocks_per_item);
    const uint8_t* bank = a.banks + soff[it.bank];
    if (sfmt[it.bank] == kPTQ1)
      expert_unit<kPTQ1, MODE_GATEUP, WPB, KS, RT, D, GW>(la, it, tb, lut, xs, red, slot_of, wgt_of, bank);
    else
      expert_unit<kPQ2, MODE_GATEUP, WPB, KS, RT, D, GW>(la, it, tb, lut, xs, red, slot_of, wgt_of, bank);
  }
}

// Down projection and combine of a batch of at most 4 tokens.  Block = one
// 16-row tile of the model dimension for every token.  Its sixteen waves take
// pieces: piece i < n_items is item i (an expert and the positions routed to
// it, or a shared expert), which multiplies the tile's down rows with the
// item's h rows and leaves each slot's o * gate weight in shared memory; the
// pieces after them are 128-wide slices of the correction's inner dimension,
// each the tile's B rows times z.  The block then adds, per token and row, B z
// (slices in order) and the slots in slot order (routed in rank order, then
// shared) in fp32, and rounds once to bf16.
constexpr int kTinyDownWaves = 16;
constexpr int kTinyGroups = 8;   // groups of the down rows whose loads are in flight together

// soff: the bank offsets, sperm / swgt: the batch's permutation and gate weights
// (T k entries), all in LDS.
template <int FMT>
__device__ __forceinline__ void tiny_down_piece(const ExpertArgs& a, const Item& it, int tile, const u32x2* lut,
                                                float* part, int lane, const int64_t* soff, const int* sperm,
                                                const float* swgt) {
  const int i16 = lane & 15, q = lane >> 4;
  const int G = a.f / kGroup;
  constexpr int BB = block_bytes_c<FMT>();
  const int64_t row_bytes = (int64_t)G * BB;
  const uint8_t* bank = a.banks + soff[it.bank];
  const int64_t gu_bytes = (int64_t)a.f * (a.d / kGroup) * BB;
  const uint8_t* wrow = bank + 2 * gu_bytes + (int64_t)tile * 16 * row_bytes + i16 * BB;
  const uint16_t* hrow = a.h + (int64_t)(it.pos + min(i16, it.n - 1)) * a.f;  // rows past the item repeat its last
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < G; g0 += kTinyGroups) {
    u32x3 wv[kTinyGroups];
    ActRaw av[kTinyGroups];
#pragma unroll
    for (int j = 0; j < kTinyGroups; ++j) {  // every load of the chunk issued first (clamped, in bounds)
      const int g = min(g0 + j, G - 1);
      wv[j] = load_block_x3<FMT>(wrow + (int64_t)g * 16 * BB, q);
      av[j] = load_act_raw<FMT>(hrow, g, q);
    }
#pragma unroll
    for (int j = 0; j < kTinyGroups; ++j) {
      if (g0 + j >= G) break;
      u32x4 A[4], W[4];
      act_operands<FMT>(av[j], A);
      const float sc = decode_block_x3<FMT>(wv[j], lut, lane, W);
      f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) tmp = mfma16(A[m], W[m], tmp);
      acc += sc * tmp;
    }
  }
  // lane holds positions it.pos + 4q + j, row i16; the operands encode 2t, hence the 0.5
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ti = 4 * q + j;
    if (ti >= it.n) continue;
    const int64_t p = it.pos + ti;
    const bool routed = p < a.Tk;
    const int64_t slot = routed ? sperm[p] : p;
    const float w = routed ? swgt[slot] : 1.f;
    part[slot * 16 + i16] = 0.5f * w * acc[j];
  }
}

template <int FS>
__global__ __launch_bounds__(64 * kTinyDownWaves) void down_combine_kernel(ExpertArgs a, DenseArgs c) {
  extern __shared__ __align__(16) char smem[];
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  const int T = (int)a.T, d = a.d, r = c.K;
  const int n_slots = (int)a.Tk + a.S * T;
  float* part = (float*)(smem + lut_bytes);        // [slot][16 rows]
  float* partb = part + n_slots * 16;               // [B slice][token][16 rows]
  const bool has_b = c.w0 || c.q0;
  const int nbs = has_b ? (r + 127) / 128 : 0;
  const int nbk = a.E + a.S, Tk = (int)a.Tk;
  int64_t* soff = (int64_t*)(partb + nbs * kTinyMaxT * 16);  // [bank offsets][formats][perm][gate weights]
  uint8_t* sfmt = (uint8_t*)(soff + nbk);
  int* sperm = (int*)((char*)soff + bank_table_bytes(nbk));
  float* swgt = (float*)(sperm + Tk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // every read the pieces depend on goes out at once, before the first barrier:
  // the item count, each wave's first item (the workspace rounds the item list
  // up to 256 bytes, so it holds at least kTinyDownWaves items; an entry past
  // the count is not used), the bank table, the permutation and gate weights
  const int n_items = *a.n_items;
  const Item first = a.items[wave];
  for (int i = threadIdx.x; i < nbk; i += blockDim.x) {
    soff[i] = a.offsets[i];
    sfmt[i] = a.formats[i];
  }
  for (int i = threadIdx.x; i < Tk; i += blockDim.x) {
    sperm[i] = a.perm[i];
    swgt[i] = a.topk_w[i];
  }
  if (a.fmt_mask & 2) ptq1_lut_fill(lut, threadIdx.x, blockDim.x);
  __syncthreads();
  const int i16 = lane & 15, q = lane >> 4;
  const int tile = blockIdx.x, n0 = tile * 16;
  for (int pc = wave; pc < n_items + nbs; pc += kTinyDownWaves) {
    if (pc < n_items) {
      const Item it = pc == wave ? first : a.items[pc];
      if (FS == 2 || (FS == 3 && sfmt[it.bank] == kPTQ1))
        tiny_down_piece<kPTQ1>(a, it, tile, lut, part, lane, soff, sperm, swgt);
      else if (FS != 2)
        tiny_down_piece<kPQ2>(a, it, tile, lut, part, lane, soff, sperm, swgt);
    } else {
      const int bs = pc - n_items;  // k-steps 4 bs .. 4 bs + 3 of B z
      const uint16_t* zrow = c.act + (int64_t)min(i16, T - 1) * c.lda;
      const uint16_t* brow = c.q0 ? nullptr : c.w0 + (int64_t)(n0 + i16) * r;
      const uint8_t* qrow = c.q0 ? c.q0 + (n0 + i16) * pq2_row_bytes(r) : nullptr;
      u32x4 wv[4], zv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = 128 * bs + 32 * j + 8 * q;
        const bool kin = kb < r;
        if (qrow)
          wv[j] = kin ? pq2_row_f16x8(qrow, kb) : u32x4{0u, 0u, 0u, 0u};
        else
          wv[j] = kin ? *(const u32x4_a4*)(brow + kb) : u32x4{0u, 0u, 0u, 0u};
        zv[j] = kin ? *(const u32x4*)(zrow + kb) : u32x4{0u, 0u, 0u, 0u};
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 hi, lo;
        split_f16x8(wv[j], hi, lo);
        acc = mfma16(zv[j], hi, acc);
        acc = mfma16(zv[j], lo, acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * q + j < T) partb[(bs * kTinyMaxT + 4 * q + j) * 16 + i16] = acc[j];
    }
  }
  __syncthreads();
  if ((int)threadIdx.x >= T * 16) return;
  const int t = threadIdx.x >> 4, row = threadIdx.x & 15;
  float v = 0.f;
  for (int bs = 0; bs < nbs; ++bs) v = bs == 0 ? partb[(t) * 16 + row] : v + partb[(bs * kTinyMaxT + t) * 16 + row];
  for (int i = 0; i < a.k; ++i) v += part[(t * a.k + i) * 16 + row];
  for (int sh = 0; sh < a.S; ++sh) v += part[((int)a.Tk + sh * T + t) * 16 + row];
  c.y[(int64_t)t * d + n0 + row] = (uint16_t)f32_to_bf16(v);
}

// ============================================================ large batches
// Work unit = (item of up to 128 positions of one bank, row block).  A block of
// WAVES waves stages the item's activations one 128-wide group at a time into a
// double-buffered LDS tile while its waves multiply the previous group.  Each
// wave owns 4 row tiles (gate/up: 32 features, their gate and up rows; down:
// 64 model rows).  Per group it decodes its 4 row tiles once into operands,
// then walks the item's token tiles: the 4 LDS reads of a token tile's
// activations feed 16 MFMAs (4 row tiles x 4 k-steps), and each row tile's
// group scale is applied to the token tile's fp32 partial sums.  One decoded
// weight feeds up to 8 token tiles.  Blocks of 8 waves run one to a CU.
constexpr int kGemmWaves = 8;
constexpr int kGemmRow = 256 + 32;                // staged bytes per token row and group (padded as stage_stride)
constexpr int kGemmBuf = kGemmChunk * kGemmRow;   // one staged group
constexpr int gemm_rows(int mode, int waves) { return waves * (mode == 0 ? 32 : 64); }  // per unit

// Half of one activation quarter: elements of row `row`, group g, quarter q
// feeding MFMAs m = 2h and 2h + 1 (PQ2_0: elements 32q + 16h .. +15; PTQ1_0: the
// raw operands 2h, 2h + 1 of load_act_raw).
template <int FMT>
__device__ __forceinline__ void act_half_load(const uint16_t* row, int g, int q, int h, u32x4 (&raw)[2]) {
  if (FMT == kPQ2) {
    const u32x4* p = (const u32x4*)(row + g * 128 + 32 * q + 16 * h);
    raw[0] = p[0];
    raw[1] = p[1];
  } else {
    // the same three loads in every lane (a lane-dependent branch here would
    // make the compiler wait for every load in flight before the staging
    // stores): elements 30q + 16h .. + 15 of the group, and the quarter's tail
    // pair (elements 120 + 2q, + 1), which half 1 takes in place of its last two
    // (past the quarter's 30: up to element 121 of the group's 128)
    const uint16_t* p = row + g * 128 + 30 * q + 16 * h;  // 4-byte aligned
    raw[0] = *(const u32x4_a4*)p;
    const u32x4 v = *(const u32x4_a4*)(p + 8);
    const uint32_t t = *(const uint32_t*)(row + g * 128 + 120 + 2 * q);
    raw[1] = u32x4{v.x, v.y, v.z, h ? t : v.w};
  }
}

// MFMA operands 2h, 2h + 1 from a half quarter, stored at their staged places
// (the same pair order as act_operands).
template <int FMT>
__device__ __forceinline__ void act_half_store(const u32x4 (&raw)[2], char* dst_row, int q, int h) {
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    u32x4 o;
    if (FMT == kPQ2) {
      const uint32_t x[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dl = 2 * mm + (i >> 1);
        o[i] = perm_b32(x[dl + 4], x[dl], (i & 1) ? 0x07060302u : 0x05040100u);
      }
    } else {
      o = raw[mm];
    }
    *(u32x4*)(dst_row + ((2 * h + mm) * 4 + q) * 16) = o;
  }
}

// NTT: token tiles of the item (a compile-time count keeps the multiply free of
// branches).  The activations of group g + 1 are loaded while group g is
// multiplied and staged after it.
//
// MF: the wave's phase within a group step.  A wave with MF = false decodes
// group g and then multiplies it; a wave with MF = true multiplies group g
// (decoded in the previous step) and then decodes group g + 1.  The block
// barrier of each step keeps all waves in step, so with one wave of each kind
// on a SIMD one of them issues matrix instructions while the other runs its
// decode on the vector ALU, instead of both decoding and then both multiplying.
template <int FMT, int MODE, int NTT, int WAVES, bool PIPE_A, bool MF>
__device__ __forceinline__ void gemm_unit(const ExpertArgs& a, const Item& it, int rb, const u32x2* lut,
                                          char* bufs, char* scratch) {
  // the wave index through readfirstlane, so branches on it are scalar (a
  // lane-divergent branch makes the compiler wait for every load in flight)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, q = lane >> 4;
  const int K = MODE == MODE_GATEUP ? a.d : a.f;
  const int G = K / kGroup;
  constexpr int BB = block_bytes_c<FMT>();
  const int64_t row_bytes = (int64_t)G * BB;
  const uint8_t* bank = a.banks + a.offsets[it.bank];
  const int64_t gu_bytes = (int64_t)a.f * (a.d / kGroup) * BB;

  // the wave's row tiles; gate/up: rt 0, 1 gate rows of features row0 + 16 rt,
  // rt 2, 3 the up rows of the same features
  const int row0 = rb * gemm_rows(MODE, WAVES) + wave * (MODE == MODE_GATEUP ? 32 : 64);
  const bool active = row0 < (MODE == MODE_GATEUP ? a.f : a.d);
  const uint8_t* wrow[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    int64_t off;
    if (MODE == MODE_GATEUP)
      off = (rt >> 1) * gu_bytes + (int64_t)(row0 + 16 * (rt & 1)) * row_bytes;
    else
      off = 2 * gu_bytes + (int64_t)(row0 + 16 * rt) * row_bytes;
    wrow[rt] = bank + (active ? off + i16 * BB : 0);  // the lane's row; group g at + g * 16 * BB
  }
  // the lane's 12-byte window directly: here the LDS is busy with the
  // activation operands, and rearranging aligned chunks through it measured no
  // faster (the down projection below does use them)
  constexpr bool CH = false;
  static_assert(!CH, "the gate/up kernel reads 12-byte windows");
  (void)scratch;
  using RingT = u32x3;
  auto fetch = [&](const uint8_t* p) -> RingT { return load_block_x3<FMT>(p, q); };

  // staging roles of the thread: token row si, quarter sq, half sh of the
  // kGemmChunk x 8 half quarters of a group.  Every thread stages, with no
  // branch (a lane condition would make every staging store wait for all loads
  // in flight, the next group's weights included): rows past the item repeat
  // its last row, and threads past the buffer's last row repeat that row's
  // work (the same values to the same place); rows past NTT tiles are not read.
  constexpr int P = (kGemmChunk * 8 + 64 * WAVES - 1) / (64 * WAVES);
  int si[P], sq[P], sh[P];
  const uint16_t* srow[P];
#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    const int u = threadIdx.x + pp * 64 * WAVES;
    si[pp] = min(u >> 3, kGemmChunk - 1);
    sq[pp] = (u >> 1) & 3;
    sh[pp] = u & 1;
    const int64_t p = it.pos + min(si[pp], it.n - 1);  // rows past the item repeat its last row
    if (MODE == MODE_GATEUP) {
      const int64_t tok = p < a.Tk ? a.perm[p] / a.k : (p - a.Tk) % a.T;
      srow[pp] = a.x + tok * a.d;
    } else {
      srow[pp] = a.h + p * a.f;
    }
  }

  // weights of the next group in flight (a group step is long enough to cover
  // the load latency)
  RingT ring[4];
  if (active) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) ring[rt] = fetch(wrow[rt]);
  }
  u32x4 s0[P][2];  // staged loads in flight
  __syncthreads();  // the previous unit is done with the staging buffers
#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    act_half_load<FMT>(srow[pp], 0, sq[pp], sh[pp], s0[pp]);
    act_half_store<FMT>(s0[pp], bufs + si[pp] * kGemmRow, sq[pp], sh[pp]);
  }
  __syncthreads();

  f32x4 acc[NTT][4];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the group's 4 row tiles, decoded once (the byte table is visible after
  // the first barrier above); then the weights of a later group, fetched in
  // every wave (an idle wave's rows are the bank's first, in bounds), so the
  // waits before the staging stores count them exactly
  u32x4 W[4][4];
  float sc[4];
  auto decode_fetch = [&](int gf) {
    if (active) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) sc[rt] = decode_block_x3<FMT, kLutCopiesWide>(ring[rt], lut, lane, W[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) ring[rt] = fetch(wrow[rt] + (int64_t)gf * 16 * BB);
  };
  if (MF) decode_fetch(min(1, G - 1));  // group 0 decoded, group 1 in flight

  // The last step fetches the last group again (in bounds, unused) and
  // restages it into the idle buffer, so the loop body has no branch on g.
  for (int g = 0; g < G; ++g) {
    const int gn = min(g + 1, G - 1);
#pragma unroll
    for (int pp = 0; pp < P; ++pp) act_half_load<FMT>(srow[pp], gn, sq[pp], sh[pp], s0[pp]);
    if (!MF) decode_fetch(gn);  // group g decoded, group g + 1 in flight
    if (active) {
      // the products at a raised wave priority, so the SIMD's other wave
      // decodes in the gaps between them
      __builtin_amdgcn_s_setprio(1);
      const char* ab = bufs + (g & 1) * kGemmBuf + i16 * kGemmRow + q * 16;
      if constexpr (PIPE_A) {
        // A operands (token tile tt, slice m) in order i = 4 tt + m through a
        // three-slot ring, each read two slices before its products, so the
        // shared-memory latency overlaps the matrix work instead of preceding
        // it.  Only the PQ2_0-only kernel: with the byte-table reads of
        // PTQ1_0 (sharing the LDS and the registers) and in the kernel that
        // holds both decoders it measured slower.
        constexpr int NA = NTT * 4;
        auto a_at = [&](int i) { return *(const u32x4*)(ab + (i >> 2) * 16 * kGemmRow + (i & 3) * 64); };
        u32x4 Ar[3];
        Ar[0] = a_at(0);
        if (NA > 1) Ar[1] = a_at(1);
        f32x4 tmp[4];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          if (i + 2 < NA) Ar[(i + 2) % 3] = a_at(i + 2);
          const int tt = i >> 2, m = i & 3;
          if (m == 0) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) tmp[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) tmp[rt] = mfma16(Ar[i % 3], W[rt][m], tmp[rt]);
          if (m == 3) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[tt][rt] += sc[rt] * tmp[rt];
          }
        }
      } else {
        // one slice ahead (two slots): the byte-table reads leave no room for more
        constexpr int NA = NTT * 4;
        auto a_at = [&](int i) { return *(const u32x4*)(ab + (i >> 2) * 16 * kGemmRow + (i & 3) * 64); };
        u32x4 Ar[2];
        Ar[0] = a_at(0);
        f32x4 tmp[4];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          if (i + 1 < NA) Ar[(i + 1) & 1] = a_at(i + 1);
          const int tt = i >> 2, m = i & 3;
          if (m == 0) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) tmp[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) tmp[rt] = mfma16(Ar[i & 1], W[rt][m], tmp[rt]);
          if (m == 3) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[tt][rt] += sc[rt] * tmp[rt];
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (MF) decode_fetch(min(g + 2, G - 1));  // group g + 1 decoded, group g + 2 in flight
#pragma unroll
    for (int pp = 0; pp < P; ++pp)
      act_half_store<FMT>(s0[pp], bufs + ((g + 1) & 1) * kGemmBuf + si[pp] * kGemmRow, sq[pp], sh[pp]);
    __syncthreads();
  }
  if (!active) return;

  // lane holds positions it.pos + 16 tt + 4q + j, column i16 of each row tile;
  // the operands encode 2t, hence the 0.5
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ti = 16 * tt + 4 * q + j;
      if (ti >= it.n) continue;
      const int64_t p = it.pos + ti;
      if (MODE == MODE_GATEUP) {
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) {
          const float gv = 0.5f * acc[tt][ft][j], uv = 0.5f * acc[tt][2 + ft][j];
          const float hv = silu_mul(gv, uv);
          a.h[p * a.f + row0 + 16 * ft + i16] = (uint16_t)f32_to_bf16(hv);
        }
      } else {
        int64_t slot;
        float wgt;
        if (p < a.Tk) {
          slot = a.perm[p];
          wgt = a.topk_w[slot];
        } else {
          slot = p;
          wgt = 1.f;
        }
        wgt *= 0.5f;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          a.slots[slot * a.d + row0 + 16 * rt + i16] = (uint16_t)f32_to_bf16(wgt * acc[tt][rt][j]);
      }
    }
  }
}

template <int MODE, int FS, int NTT, int WAVES>
__device__ __forceinline__ void gemm_dispatch(const ExpertArgs& a, const Item& it, int rb, const u32x2* lut,
                                              char* bufs, bool ptq1, bool mf) {
  if (FS != 1 && ptq1) {
    // (PTQ1_0: the two phases measured no faster, the byte-table reads of the
    // decode sharing the LDS with the other wave's operand reads)
    gemm_unit<kPTQ1, MODE, NTT, WAVES, false, false>(a, it, rb, lut, bufs, nullptr);
  } else if (FS != 2) {
    if (mf)
      gemm_unit<kPQ2, MODE, NTT, WAVES, FS == 1, true>(a, it, rb, lut, bufs, nullptr);
    else
      gemm_unit<kPQ2, MODE, NTT, WAVES, FS == 1, false>(a, it, rb, lut, bufs, nullptr);
  }
}

// Persistent blocks over units.  Unit l = (item l / row_blocks, row block
// l % row_blocks); the blocks of one XCD (block index mod 8, the order in which
// workgroups are spread over the XCDs) take a contiguous range of units, so the
// items of one expert and the row blocks of one item meet in the same L2.
// Dynamic LDS: [PTQ1_0 byte table if the layer has PTQ1_0 banks][2 staged groups]
template <int MODE, int FS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void expert_gemm_kernel(ExpertArgs a, int row_blocks) {
  extern __shared__ __align__(16) char smem[];
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * kLutCopiesWide * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  char* bufs = smem + lut_bytes;
  if (a.fmt_mask & 2) ptq1_lut_fill<kLutCopiesWide>(lut, threadIdx.x, blockDim.x);  // visible after the unit's first sync
  // The wave's phase (see gemm_unit): the first wave of the block to arrive on
  // a SIMD multiplies first, the next one decodes first.  The SIMD comes from
  // the hardware-ID register, the order of arrival from a counter per SIMD in
  // shared memory (an initialisation only: any outcome is a correct result).
  __shared__ int simd_waves[4];
  if (threadIdx.x < 4) simd_waves[threadIdx.x] = 0;
  __syncthreads();
  bool mf;
  {
    const int simd = (int)((__builtin_amdgcn_s_getreg(kHwIdSimd) >> 0) & 3);
    int arrived = 0;
    if ((threadIdx.x & 63) == 0) arrived = atomicAdd(&simd_waves[simd], 1);
    mf = (__builtin_amdgcn_readfirstlane(arrived) & 1) == 0;
  }
  const int64_t U = (int64_t)(*a.n_items) * row_blocks;
  const int64_t per = (U + 7) / 8;
  for (int64_t u = blockIdx.x; u < 8 * per; u += gridDim.x) {
    const int64_t l = (u & 7) * per + (u >> 3);
    if (l >= U) continue;
    const Item it = a.items[l / row_blocks];
    const int rb = (int)(l % row_blocks);
    const bool ptq1 = FS == 2 || (FS == 3 && a.formats[it.bank] == kPTQ1);
    switch ((it.n + 15) / 16) {
      case 1: gemm_dispatch<MODE, FS, 1, WAVES>(a, it, rb, lut, bufs, ptq1, mf); break;
      case 2: gemm_dispatch<MODE, FS, 2, WAVES>(a, it, rb, lut, bufs, ptq1, mf); break;
      case 3: gemm_dispatch<MODE, FS, 3, WAVES>(a, it, rb, lut, bufs, ptq1, mf); break;
      case 4: gemm_dispatch<MODE, FS, 4, WAVES>(a, it, rb, lut, bufs, ptq1, mf); break;
      case 5: gemm_dispatch<MODE, FS, 5, WAVES>(a, it, rb, lut, bufs, ptq1, mf); break;
      default: gemm_dispatch<MODE, FS, kGemmChunk / 16, WAVES>(a, it, rb, lut, bufs, ptq1, mf); break;
    }
  }
}

// ------------------------------------------------------------ large batches: down
// Work unit = one item.  The block stages the item's h rows (all f inputs, in
// the container format's k-slot order) in LDS once; each wave then takes
// 64-row quads of the d output rows (quad w, w + WAVES, ...) and streams their
// weights group after group through a ring that runs on from one quad into the
// next, so after the staging the block waits on no barrier and no empty ring.
constexpr int kDownWaves = 8;

// The thread index as a value the compiler treats as new at each use, so index
// arithmetic derived from it stays inside the persistent loop instead of being
// hoisted to kernel entry, where it would hold registers for the whole kernel.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

template <int FMT, int NTT, int G, bool CHK, int NC, int CAP>
__device__ __forceinline__ void down_unit(const ExpertArgs& a, const Item& it, const u32x2* lut, char* xs,
                                          char* scratch) {
  const int tid = opaque_tid();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, q = lane >> 4;
  constexpr int K = G * kGroup;
  constexpr int stride = stage_stride(K);
  constexpr int BB = block_bytes_c<FMT>();
  constexpr int64_t row_bytes = (int64_t)G * BB;
  constexpr int D = 1;  // groups in flight (two spill at four token tiles)
  const uint8_t* bank = a.banks + a.offsets[it.bank];
  const int64_t gu_bytes = (int64_t)a.f * (a.d / kGroup) * BB;
  const int nquads = a.d / 64;
  const int nqw = wave < nquads ? (nquads - wave + kDownWaves - 1) / kDownWaves : 0;
  constexpr int64_t quad_stride = (int64_t)64 * kDownWaves * row_bytes;

  // the tiles' bases are wave-uniform (scalar registers); the window path adds
  // the lane's row at each load
  const uint8_t* rows[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) rows[rt] = bank + 2 * gu_bytes + (int64_t)(wave * 64 + 16 * rt) * row_bytes;
  const uint32_t lane_row = CHK && FMT == kPQ2 ? 0u : (uint32_t)(i16 * BB);
  // CHK (kernels for PQ2_0-only layers): aligned chunk pieces rearranged
  // through the wave's LDS scratch; otherwise the lane's 12-byte window directly
  // (the PTQ1_0 decoder already leans on LDS, and the mixed kernel has no
  // registers to spare)
  constexpr bool CH = CHK && FMT == kPQ2;
  using RingT = std::conditional_t<CH, u32x4, u32x3>;
  auto fetch = [&](const uint8_t* chunk) -> RingT {
    if constexpr (CH)
      return load_chunk<FMT>(chunk, lane);
    else
      return load_block_x3<FMT>(chunk + lane_row, q);
  };
  auto window = [&](const RingT& r) -> u32x3 {
    if constexpr (CH)
      return chunk_window<FMT>(r, scratch, lane);
    else
      return r;
  };
  RingT ring0[4], ring1[4];
  if (nqw > 0) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      ring0[rt] = fetch(rows[rt]);
      if (D == 2) ring1[rt] = fetch(rows[rt] + 16 * BB);
    }
  }

  // per token row: its slot and half its gate weight (the operands encode 2t),
  // read back through volatile pointers so the quad loop does not hold them
  int* slot_of = (int*)(xs + CAP * stride);
  float* wgt_of = (float*)(slot_of + CAP);
  __syncthreads();  // the previous unit is done with the staged rows
  if (tid < NTT * 16) {
    const int64_t p = it.pos + min(tid, it.n - 1);
    const bool routed = p < a.Tk;
    const int slot = routed ? a.perm[p] : (int)p;
    slot_of[tid] = slot;
    wgt_of[tid] = 0.5f * (routed ? a.topk_w[slot] : 1.f);
  }
  {
    // the thread's share in batches of 4, all loads of a batch in flight
    // before its first store
    constexpr int total = NTT * 16 * G * 8, PER = (total + 64 * kDownWaves - 1) / (64 * kDownWaves);
    constexpr int NB = PER < 4 ? PER : 4;
#pragma unroll
    for (int k0 = 0; k0 < PER; k0 += NB) {
      u32x4 raw[NB][2];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int u = tid + (k0 + k) * 64 * kDownWaves;
        if (k0 + k < PER && u < total) {
          const int i = u / (G * 8), rem = u % (G * 8);
          const uint16_t* row = a.h + (int64_t)(it.pos + min(i, it.n - 1)) * a.f;  // rows past the item repeat its last
          act_half_load<FMT>(row, rem >> 3, (rem >> 1) & 3, rem & 1, raw[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int u = tid + (k0 + k) * 64 * kDownWaves;
        if (k0 + k < PER && u < total) {
          const int i = u / (G * 8), rem = u % (G * 8);
          act_half_store<FMT>(raw[k], xs + i * stride + (rem >> 3) * 256, (rem >> 1) & 3, rem & 1);
        }
      }
    }
  }
  __syncthreads();

  const char* ab = xs + i16 * stride + q * 16;
  for (int t = 0; t < nqw; ++t) {
    const bool more = t + 1 < nqw;
    f32x4 acc[NTT][4];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // refill with group g + D of this quad, else of the next quad (the last
    // quad refetches its own groups: in bounds, unused)
    auto next_off = [&](int g) -> int64_t {
      return g + D < G ? (int64_t)(g + D) * 16 * BB : (more ? quad_stride : 0) + (int64_t)(g + D - G) * 16 * BB;
    };
    // up to four token tiles: the step's A operands stay in registers while
    // each row tile is decoded and multiplied
    auto step = [&](int g, RingT (&ring)[4]) {
      u32x4 A[NTT][4];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int m = 0; m < 4; ++m) A[tt][m] = *(const u32x4*)(ab + tt * 16 * stride + g * 256 + m * 64);
      const int64_t nxt = next_off(g);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        u32x4 W[4];
        float sc;
        if constexpr (CH) {
          const u32x3 v = window(ring[rt]);
          ring[rt] = fetch(rows[rt] + nxt);
          sc = decode_block_x3<FMT, NC>(v, lut, lane, W);
        } else {
          sc = decode_block_x3<FMT, NC>(ring[rt], lut, lane, W);
          ring[rt] = fetch(rows[rt] + nxt);
        }
        f32x4 tmp[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) tmp[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // products at a raised wave priority, as in the streaming decode (the
        // waves here run without a block barrier, so they drift out of phase)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) tmp[tt] = mfma16(A[tt][m], W[m], tmp[tt]);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[tt][rt] += sc * tmp[tt];
      }
    };
    // five or six token tiles: the step's four row tiles are decoded once and
    // stay in registers while the token tiles are walked, the four shared-memory
    // reads of each feeding 16 MFMAs (the same products, summed in the same order)
    auto step_walk = [&](int g, RingT (&ring)[4]) {
      u32x4 W[4][4];
      float sc[4];
      const int64_t nxt = next_off(g);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if constexpr (CH) {
          const u32x3 v = window(ring[rt]);
          ring[rt] = fetch(rows[rt] + nxt);
          sc[rt] = decode_block_x3<FMT, NC>(v, lut, lane, W[rt]);
        } else {
          sc[rt] = decode_block_x3<FMT, NC>(ring[rt], lut, lane, W[rt]);
          ring[rt] = fetch(rows[rt] + nxt);
        }
      }
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        u32x4 A[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) A[m] = *(const u32x4*)(ab + tt * 16 * stride + g * 256 + m * 64);
        f32x4 tmp[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) tmp[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) tmp[rt] = mfma16(A[m], W[rt][m], tmp[rt]);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[tt][rt] += sc[rt] * tmp[rt];
      }
    };
#pragma unroll 1
    for (int g = 0; g < G; g += D) {
      if constexpr (NTT > 4) {
        step_walk(g, ring0);
        if (D == 2) step_walk(g + 1, ring1);
      } else {
        step(g, ring0);
        if (D == 2) step(g + 1, ring1);
      }
    }
    // lane holds positions it.pos + 16 tt + 4q + j, column i16 of each row tile
    const int row0 = (wave + t * kDownWaves) * 64;
    // (LDS-qualified: through generic pointers these reads become flat loads,
    // whose waits also wait for every weight load in flight)
    typedef const volatile int __attribute__((address_space(3))) lds_int;
    typedef const volatile float __attribute__((address_space(3))) lds_float;
    lds_int* vslot = (lds_int*)slot_of;
    lds_float* vwgt = (lds_float*)wgt_of;
    // the lane's indices taken anew here, so the per-token tests and table
    // addresses are not hoisted out of the quad loop, where they would hold
    // registers (a pair per token) for the whole unit
    const int el = opaque_tid() & 63, eq = el >> 4, ei = el & 15;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      // the token tile's four slots and weights read together (positions past
      // the item read its last one, unused), so their shared-memory round trips
      // overlap instead of one per token before its stores
      int slot[4];
      float wgt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ti = min(16 * tt + 4 * eq + j, it.n - 1);
        slot[j] = vslot[ti];
        wgt[j] = vwgt[ti];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (16 * tt + 4 * eq + j >= it.n) continue;
        uint16_t* dst = a.slots + (int64_t)slot[j] * a.d + row0 + ei;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dst[16 * rt] = (uint16_t)f32_to_bf16(wgt[j] * acc[tt][rt][j]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) rows[rt] += quad_stride;
  }
}

template <int FS, int NTT, int G, int NC, int CAP>
__device__ __forceinline__ void down_dispatch(const ExpertArgs& a, const Item& it, const u32x2* lut, char* xs,
                                              bool ptq1) {
  char* scratch = xs + CAP * (stage_stride(G * kGroup) + 8) + (threadIdx.x >> 6) * kChunkScratch;
  if (FS != 1 && ptq1)
    down_unit<kPTQ1, NTT, G, false, NC, CAP>(a, it, lut, xs, scratch);
  else if (FS != 2)
    down_unit<kPQ2, NTT, G, FS == 1, NC, CAP>(a, it, lut, xs, scratch);
}

// Persistent blocks over items, the blocks of one XCD taking a contiguous range
// (so the items of one expert share its down weights in one L2).
// CAP: staged rows, the most positions of a unit (64, or 96 where the items
// hold up to six token tiles).
// Dynamic LDS: [PTQ1_0 byte table if the layer has PTQ1_0 banks][CAP staged rows][CAP slots][CAP weights]
// [per-wave chunk scratch]
template <int FS, int G, int NC, int CAP>
__global__ __launch_bounds__(64 * kDownWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void down_resident_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * NC * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  char* xs = smem + lut_bytes;
  if (a.fmt_mask & 2) ptq1_lut_fill<NC>(lut, threadIdx.x, blockDim.x);  // visible after the unit's first sync
  const int64_t U = *a.down_n_items;
  const int64_t per = (U + 7) / 8;
  for (int64_t u = blockIdx.x; u < 8 * per; u += gridDim.x) {
    const int64_t l = (u & 7) * per + (u >> 3);
    if (l >= U) continue;
    const Item item = a.down_items[l];
    const bool ptq1 = FS == 2 || (FS == 3 && a.formats[item.bank] == kPTQ1);
    for (int h0 = 0; h0 < item.n; h0 += CAP) {  // (the items hold at most CAP positions)
      const Item it{item.bank, item.pos + h0, min(CAP, item.n - h0), 0};
      switch ((it.n + 15) / 16) {
        case 1: down_dispatch<FS, 1, G, NC, CAP>(a, it, lut, xs, ptq1); break;
        case 2: down_dispatch<FS, 2, G, NC, CAP>(a, it, lut, xs, ptq1); break;
        case 3: down_dispatch<FS, 3, G, NC, CAP>(a, it, lut, xs, ptq1); break;
        case 4: down_dispatch<FS, 4, G, NC, CAP>(a, it, lut, xs, ptq1); break;
        case 5: if constexpr (CAP > 64) down_dispatch<FS, 5, G, NC, CAP>(a, it, lut, xs, ptq1); break;
        default: if constexpr (CAP > 64) down_dispatch<FS, 6, G, NC, CAP>(a, it, lut, xs, ptq1); break;
      }
    }
  }
}

template <int MODE, int WPB, int KS, int RT, int D, int GW>
static hipError_t launch_dec(const ExpertArgs& a, int64_t max_items, hipStream_t stream) {
  const int K = MODE == MODE_GATEUP ? a.d : a.f;
  const int n_tiles = MODE == MODE_GATEUP ? a.f / 16 : a.d / (16 * RT);
  constexpr int TPB = WPB / KS;
  const int tbpi = (n_tiles + TPB - 1) / TPB;
  const size_t lds = ((a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0) + (size_t)a.nmax * stage_stride(K) +
                     slot_table_bytes(a.nmax) + (KS > 1 ? (size_t)TPB * (KS - 1) * RT * 64 * 16 : 0);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = expert_dec_kernel<MODE, WPB, KS, RT, D, GW>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * WPB, lds);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t grid = std::min<int64_t>((int64_t)cu_count() * per_cu, max_items * tbpi);
  kern<<<dim3((unsigned)grid), 64 * WPB, lds, stream>>>(a, tbpi);
  return hipGetLastError();
}

// Expected number of work items (the exact count is only known on the device):
// touched routed experts plus extra 16-token chunks, plus the shared experts.
// (A low estimate: splitting work too finely costs less than idle blocks.)
constexpr double kCoResidentGain = 1.4;  // streaming blocks sharing a CU, measured

static double expected_items(const ExpertArgs& a) {
  const double slots = (double)a.T * a.k;
  const double touched = a.E * (1.0 - std::exp(-slots / a.E));
  return std::max(touched, slots / a.chunk) + (double)a.S * ((a.T + a.chunk - 1) / a.chunk);
}

template <int MODE, int WPB, int RT, int D, int G, int FS, int WPE>
static hipError_t launch_stream_fs(const ExpertArgs& a, int64_t max_items, hipStream_t stream) {
  constexpr int K = G * kGroup;
  const int n_tiles = MODE == MODE_GATEUP ? a.f / 16 : a.d / (16 * RT);
  const size_t lds = ((a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0) + (size_t)a.nmax * stage_stride(K) +
                     slot_table_bytes(a.nmax) + (size_t)WPB * kChunkScratch;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = expert_stream_kernel<MODE, WPB, RT, D, G, FS, WPE>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * WPB, lds);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  const int cus = cu_count();
  const int64_t blocks = (int64_t)cus * per_cu;
  // tiles per wave per unit: the busiest CU takes ceil(units / CUs) units of
  // (tpw + 1) tile-times each (one for the unit's staging bubble); units that
  // share a CU overlap each other's bubbles and load waits, measured as 1.4x
  // the throughput of one block alone
  const double items = std::min<double>((double)max_items, expected_items(a));
  const int max_tpw = (n_tiles + WPB - 1) / WPB;
  int best_tpw = 1;
  double best = 1e30;
  for (int tpw = 1; tpw <= max_tpw; ++tpw) {
    const int tpu = tpw * WPB;
    const double units = items * ((n_tiles + tpu - 1) / tpu);
    const double on_cu = std::ceil(units / cus);
    const double cost = on_cu * (tpw + 1) / (per_cu >= 2 && on_cu >= 2 ? kCoResidentGain : 1.0);
    if (cost < best) {
      best = cost;
      best_tpw = tpw;
    }
  }
  const int tpu = best_tpw * WPB;
  const int upi = (n_tiles + tpu - 1) / tpu;
  const int64_t grid = std::min<int64_t>(blocks, max_items * upi);
  kern<<<dim3((unsigned)grid), 64 * WPB, lds, stream>>>(a, tpu, upi);
  return hipGetLastError();
}

// WPE: waves per SIMD the kernel is built for (1: up to 512 registers per
// wave, so the prefetch ring can hold a whole tile of loads).
template <int MODE, int WPB, int RT, int D, int G, int WPE = 2>
static hipError_t launch_stream(const ExpertArgs& a, int64_t max_items, hipStream_t stream) {
  if (a.fmt_mask == 1) return launch_stream_fs<MODE, WPB, RT, D, G, 1, WPE>(a, max_items, stream);
  if (a.fmt_mask == 2) return launch_stream_fs<MODE, WPB, RT, D, G, 2, WPE>(a, max_items, stream);
  return launch_stream_fs<MODE, WPB, RT, D, G, 3, WPE>(a, max_items, stream);
}

template <int MODE, int FS, int WAVES>
static hipError_t launch_gemm_fs(const ExpertArgs& a, int64_t max_items, hipStream_t stream) {
  const int N = MODE == MODE_GATEUP ? a.f : a.d;
  const int row_blocks = (N + gemm_rows(MODE, WAVES) - 1) / gemm_rows(MODE, WAVES);
  const size_t lds = ((a.fmt_mask & 2) ? 256 * kLutCopiesWide * 8 : 0) + 2 * (size_t)kGemmBuf;
  auto kern = expert_gemm_kernel<MODE, FS, WAVES>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * WAVES, lds);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t grid = std::min<int64_t>((int64_t)cu_count() * per_cu, max_items * row_blocks);
  kern<<<dim3((unsigned)grid), 64 * WAVES, lds, stream>>>(a, row_blocks);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gemm(const ExpertArgs& a, int64_t max_items, hipStream_t stream) {
  if (a.fmt_mask == 1) return launch_gemm_fs<MODE, 1, kGemmWaves>(a, max_items, stream);
  if (a.fmt_mask == 2) return launch_gemm_fs<MODE, 2, kGemmWaves>(a, max_items, stream);
  return launch_gemm_fs<MODE, 3, kGemmWaves>(a, max_items, stream);
}

template <int FS, int G, int NC, int CAP>
static hipError_t launch_down_resident_fs(const ExpertArgs& a, int64_t max_items, size_t lds, hipStream_t stream) {
  auto kern = down_resident_kernel<FS, G, NC, CAP>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kDownWaves, lds);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t grid = std::min<int64_t>((int64_t)cu_count() * per_cu, max_items);
  kern<<<dim3((unsigned)grid), 64 * kDownWaves, lds, stream>>>(a);
  return hipGetLastError();
}

// wide: the byte table in kLutCopiesWide copies (layers with PTQ1_0 banks
// whose staged rows leave room for it)
template <int G, int CAP>
static hipError_t launch_down_resident(const ExpertArgs& a, int64_t max_items, size_t lds, bool wide,
                                       hipStream_t stream) {
  if (a.fmt_mask == 1) return launch_down_resident_fs<1, G, kLutCopies, CAP>(a, max_items, lds, stream);
  if (wide) {
    if (a.fmt_mask == 2) return launch_down_resident_fs<2, G, kLutCopiesWide, CAP>(a, max_items, lds, stream);
    return launch_down_resident_fs<3, G, kLutCopiesWide, CAP>(a, max_items, lds, stream);
  }
  if (a.fmt_mask == 2) return launch_down_resident_fs<2, G, kLutCopies, CAP>(a, max_items, lds, stream);
  return launch_down_resident_fs<3, G, kLutCopies, CAP>(a, max_items, lds, stream);
}

template <int CAP>
static hipError_t launch_down_cap(const ExpertArgs& a, int64_t mi, hipStream_t s) {
  const size_t rows = (size_t)CAP * (stage_stride(a.f) + 8) + (size_t)kDownWaves * kChunkScratch;
  const bool wide = (a.fmt_mask & 2) && 256 * kLutCopiesWide * 8 + rows <= 160 * 1024;
  const size_t lds = ((a.fmt_mask & 2) ? 256 * (wide ? kLutCopiesWide : kLutCopies) * 8 : 0) + rows;
  if (lds > 160 * 1024) return hipErrorNotSupported;
  switch (a.f / kGroup) {
    case 8: return launch_down_resident<8, CAP>(a, mi, lds, wide, s);
    case 6: return launch_down_resident<6, CAP>(a, mi, lds, wide, s);
    case 4: return launch_down_resident<4, CAP>(a, mi, lds, wide, s);
    case 1: return launch_down_resident<1, CAP>(a, mi, lds, wide, s);
    default: return hipErrorNotSupported;
  }
}

// Down projection of a large batch: LDS-resident h rows where the shape is
// compiled in and the rows fit, else the group-staged kernel.  The resident
// kernel takes the gate/up items (up to 96 positions) where their rows fit in
// shared memory: each weight group decoded then feeds up to six token tiles, and
// an expert whose load is one such item streams its down weights once (measured
// faster than 64-position units at every prefill shape here, skewed routing
// included); else the down projection's own 64-position items.
static hipError_t launch_down_large(const ExpertArgs& a, int64_t mi, int64_t mi_gateup, hipStream_t s) {
  {
    ExpertArgs g = a;
    g.down_items = a.items;
    g.down_n_items = a.n_items;
    const hipError_t e = launch_down_cap<kGemmChunk>(g, mi_gateup, s);
    if (e != hipErrorNotSupported) return e;
  }
  const hipError_t e = launch_down_cap<kDownChunk>(a, mi, s);
  if (e != hipErrorNotSupported) return e;
  return launch_gemm<MODE_DOWN>(a, mi, s);
}

// Shapes with a compile-time group count stream; others take the generic loop.
//   gate/up: K = d;  down: K = f.  Few tokens: K split over KS waves per tile.
static hipError_t launch_gateup(const ExpertArgs& a, int64_t mi, bool small, hipStream_t s) {
  const int G = a.d / kGroup;
  if (small) {
    switch (G) {
      case 24: return launch_dec<MODE_GATEUP, 8, 4, 2, 6, 6>(a, mi, s);
      case 16: return launch_dec<MODE_GATEUP, 8, 4, 2, 4, 4>(a, mi, s);
      case 2: return launch_dec<MODE_GATEUP, 8, 2, 2, 1, 1>(a, mi, s);
      default: return launch_dec<MODE_GATEUP, 8, 4, 2, 4, 0>(a, mi, s);
    }
  }
  switch (G) {
    case 24:  // up to 4 tokens per item: two blocks per CU fit beside the byte table
      if (a.nmax <= kSmallChunkMin) return launch_stream<MODE_GATEUP, 8, 2, 4, 24, 4>(a, mi, s);
      return launch_stream<MODE_GATEUP, 8, 2, 8, 24>(a, mi, s);
    case 16:  // PQ2_0-only layers: two blocks per CU at 128 registers (no byte table)
      if (a.fmt_mask == 1) return launch_stream_fs<MODE_GATEUP, 8, 2, 4, 16, 1, 4>(a, mi, s);
      return launch_stream<MODE_GATEUP, 8, 2, 8, 16>(a, mi, s);
    case 2: return launch_stream<MODE_GATEUP, 8, 2, 2, 2>(a, mi, s);
    default: return launch_dec<MODE_GATEUP, 8, 1, 2, 8, 0>(a, mi, s);
  }
}

static hipError_t launch_down(const ExpertArgs& a, int64_t mi, bool small, hipStream_t s) {
  const int G = a.f / kGroup;
  if (small) {
    switch (G) {
      case 8: return launch_dec<MODE_DOWN, 8, 2, 2, 4, 4>(a, mi, s);
      case 6: return launch_dec<MODE_DOWN, 8, 2, 2, 3, 3>(a, mi, s);
      case 4: return launch_dec<MODE_DOWN, 8, 2, 2, 2, 2>(a, mi, s);
      case 1: return launch_dec<MODE_DOWN, 8, 1, 2, 1, 1>(a, mi, s);
      default: return launch_dec<MODE_DOWN, 8, 2, 2, 4, 0>(a, mi, s);
    }
  }
  switch (G) {
    case 8:  // PQ2_0-only layers: two row tiles per wave, two blocks per CU
      if (a.fmt_mask == 1) return launch_stream_fs<MODE_DOWN, 8, 2, 4, 8, 1, 4>(a, mi, s);
      return launch_stream<MODE_DOWN, 8, 4, 4, 8>(a, mi, s);
    case 6:
      if (a.fmt_mask == 1) return launch_stream_fs<MODE_DOWN, 8, 2, 3, 6, 1, 4>(a, mi, s);
      return launch_stream<MODE_DOWN, 8, 4, 3, 6>(a, mi, s);
    case 4: return launch_stream<MODE_DOWN, 8, 2, 4, 4, 4>(a, mi, s);  // two blocks per CU beside the byte table
    case 1: return launch_stream<MODE_DOWN, 8, 4, 1, 1>(a, mi, s);
    default: return launch_dec<MODE_DOWN, 8, 1, 4, 4, 0>(a, mi, s);
  }
}

template <int KS, int RT, int D, int GW, int PER>
static hipError_t launch_route_dec(const ExpertArgs& a, const RouteArgs& r, int64_t max_items, hipStream_t stream) {
  constexpr int WPB = 8;
  const int K = a.d;
  const int n_tiles = a.f / 16;
  constexpr int TPB = WPB / KS;
  const int tbpi = (n_tiles + TPB - 1) / TPB;
  const size_t lds = ((a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0) + (size_t)a.nmax * stage_stride(K) +
                     slot_table_bytes(a.nmax) + (KS > 1 ? (size_t)TPB * (KS - 1) * RT * 64 * 16 : 0) +
                     (size_t)align8(tiny_route_bytes((int)a.T, a.k, a.E, a.S)) + (size_t)bank_table_bytes(a.E + a.S);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = expert_route_dec_kernel<WPB, KS, RT, D, GW, PER>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * WPB, lds);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  const int route_blocks = (int)std::min<int64_t>((int64_t)cu_count() * per_cu, max_items * tbpi);
  const int fold = fold_blocks(r, 64 * WPB);
  kern<<<dim3((unsigned)(route_blocks + fold)), 64 * WPB, lds, stream>>>(a, r, tbpi, route_blocks);
  return hipGetLastError();
}

template <int PER>
static hipError_t launch_route_gateup(const ExpertArgs& a, const RouteArgs& r, int64_t mi, hipStream_t s) {
  switch (a.d / kGroup) {
    case 24: return launch_route_dec<4, 2, 6, 6, PER>(a, r, mi, s);
    case 16: return launch_route_dec<4, 2, 4, 4, PER>(a, r, mi, s);
    case 2: return launch_route_dec<2, 2, 1, 1, PER>(a, r, mi, s);
    default: return launch_route_dec<4, 2, 4, 0, PER>(a, r, mi, s);
  }
}

bool tiny_path_fits(int64_t T, int E, int k, int S, int d, int f) {
  (void)d;
  (void)f;
  return T >= 1 && T <= kTinyMaxT && E <= 512 && T * (int64_t)k <= 64 && T * (int64_t)(k + S) <= kTinyMaxSlots;
}

hipError_t launch_tiny(const ExpertArgs& a, const RouteArgs& r, const DenseArgs& c, int64_t max_items,
                       hipStream_t stream, void** ev) {
  auto mark = [&](int i) { return (ev && ev[i]) ? hipEventRecord((hipEvent_t)ev[i], stream) : hipSuccess; };
  hipError_t e = mark(4);
  if (e == hipSuccess) e = a.E <= 128 ? launch_route_gateup<2>(a, r, max_items, stream)
                                      : launch_route_gateup<8>(a, r, max_items, stream);
  if (e == hipSuccess) e = mark(5);
  if (e == hipSuccess) e = mark(6);
  if (e == hipSuccess) {
    const int nbs = (c.w0 || c.q0) ? (c.K + 127) / 128 : 0;
    const size_t lds = ((a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0) +
                       (size_t)(a.Tk + (int64_t)a.S * a.T) * 16 * 4 + (size_t)nbs * kTinyMaxT * 16 * 4 +
                       (size_t)bank_table_bytes(a.E + a.S) + (size_t)a.Tk * 8;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.d / 16));
    if (a.fmt_mask == 1) down_combine_kernel<1><<<grid, 64 * kTinyDownWaves, lds, stream>>>(a, c);
    else if (a.fmt_mask == 2) down_combine_kernel<2><<<grid, 64 * kTinyDownWaves, lds, stream>>>(a, c);
    else down_combine_kernel<3><<<grid, 64 * kTinyDownWaves, lds, stream>>>(a, c);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark(7);
  return e;
}

hipError_t launch_experts(const ExpertArgs& a, int64_t max_items, int64_t max_down_items, hipStream_t stream,
                          void** ev) {
  if (max_items <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  const bool small = a.T <= 4;
  const bool gemm = a.chunk == kGemmChunk;
  auto mark = [&](int i) { return (ev && ev[i]) ? hipEventRecord((hipEvent_t)ev[i], stream) : hipSuccess; };
  e = mark(4);
  if (e == hipSuccess)
    e = gemm ? launch_gemm<MODE_GATEUP>(a, max_items, stream) : launch_gateup(a, max_items, small, stream);
  if (e == hipSuccess) e = mark(5);
  if (e == hipSuccess) e = mark(6);
  if (e == hipSuccess) {
    if (gemm) {
      e = launch_down_large(a, max_down_items, max_items, stream);
    } else {
      // the down projection's own items (16 tokens) where gate/up takes smaller ones
      ExpertArgs d = a;
      d.items = a.down_items;
      d.n_items = a.down_n_items;
      d.chunk = kChunk;
      d.nmax = (int)std::min<int64_t>(a.T, kChunk);
      e = launch_down(d, max_down_items, small, stream);
    }
  }
  if (e == hipSuccess) e = mark(7);
  return e;
}

}  // namespace moe
