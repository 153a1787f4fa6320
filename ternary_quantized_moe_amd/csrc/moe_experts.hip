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

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int MODE_GATEUP = 0;
constexpr int MODE_DOWN = 1;

// Stage the item's activation rows (n tokens x K) into LDS as matrix-core A
// operands in the container format's k-slot order: row i, group g, MFMA m,
// quarter q -> 16 bytes at i * stride + ((g * 4 + m) * 4 + q) * 16.  The
// 16-byte row padding puts the 16 token rows of one operand read on different
// LDS banks.
__host__ __device__ constexpr int stage_stride(int K) { return 2 * K + 16; }

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
                                            char* xs, f32x4* red, int* slot_of, float* wgt_of) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int K = MODE == MODE_GATEUP ? a.d : a.f;
  const int G = K / kGroup;
  constexpr int BB = block_bytes_c<FMT>();
  const int64_t row_bytes = (int64_t)G * BB;
  const uint8_t* bank = a.banks + a.offsets[it.bank];
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
          u32x3 cur[RT];
#pragma unroll
          for (int r = 0; r < RT; ++r) cur[r] = ring[j][r];
          if (i + D < n)
#pragma unroll
            for (int r = 0; r < RT; ++r) ring[j][r] = fetch(rows[r] + (int64_t)(i + D) * 16 * BB);
          step(i, cur);
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
      const float hv = g / (1.f + __expf(-g)) * u;
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
      const float hv = g / (1.f + __expf(-g)) * u;
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
          const u32x3 v = CH ? chunk_window<FMT>(ring[j][r], scratch, lane)
                             : u32x3{ring[j][r].x, ring[j][r].y, ring[j][r].z};
          ring[j][r] = fetch(rows[r] + nxt + j * 16 * BB);
          const float s = decode_block_x3<FMT>(v, lut, lane, W);
          f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m) tmp = mfma16(A[m], W[m], tmp);
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

// ============================================================ large batches
// Work unit = (item of up to 64 positions of one bank, row block).  A block of
// WAVES waves stages the item's activations one 128-wide group at a time into a
// double-buffered LDS tile while its waves multiply the previous group.  Each
// wave owns 4 row tiles (gate/up: 32 features, their gate and up rows; down:
// 64 model rows), decodes the 4 row tiles of a group once and multiplies them
// with every token tile of the item, so one decoded weight feeds up to 4 MFMAs.
// Blocks of 4 waves run two to a CU, so one block's barrier and load waits
// overlap the other's matrix work.
constexpr int kGemmWaves = 4;
constexpr int kGemmRow = 256 + 16;                // staged bytes per token row and group
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
    const uint16_t* p = row + g * 128 + 30 * q + 16 * h;  // 4-byte aligned
    raw[0] = *(const u32x4_a4*)p;
    if (h == 0) {
      raw[1] = *(const u32x4_a4*)(p + 8);
    } else {
      const u32x2 w = *(const u32x2_a4*)(p + 8);
      const uint32_t w2 = *(const uint32_t*)(p + 12);
      const uint32_t t = *(const uint32_t*)(row + g * 128 + 120 + 2 * q);
      raw[1] = u32x4{w.x, w.y, w2, t};
    }
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
// branches, so the independent MFMA chains of the token tiles interleave).
// SD: groups of activations in flight (1: loaded in the step before they are
// staged; 2: two steps before, so a load has two group steps to land, which
// only the PQ2_0-only gate/up kernel has the registers for).
template <int FMT, int MODE, int NTT, int WAVES, int SD>
__device__ __forceinline__ void gemm_unit(const ExpertArgs& a, const Item& it, int rb, const u32x2* lut,
                                          char* bufs, char* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
  // 64 x 8 half quarters of a group
  constexpr int P = 512 / (64 * WAVES);
  int si[P], sq[P], sh[P];
  bool stage_on[P];
  const uint16_t* srow[P];
#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    const int u = threadIdx.x + pp * 64 * WAVES;
    si[pp] = u >> 3;
    sq[pp] = (u >> 1) & 3;
    sh[pp] = u & 1;
    stage_on[pp] = si[pp] < NTT * 16;
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
  u32x4 s0[P][2], s1[P][SD == 2 ? 2 : 1];  // staged loads in flight (SD = 1: s0 only)
  __syncthreads();  // the previous unit is done with the staging buffers
#pragma unroll
  for (int pp = 0; pp < P; ++pp)
    if (stage_on[pp]) {
      act_half_load<FMT>(srow[pp], 0, sq[pp], sh[pp], s0[pp]);
      act_half_store<FMT>(s0[pp], bufs + si[pp] * kGemmRow, sq[pp], sh[pp]);
      if constexpr (SD == 2) act_half_load<FMT>(srow[pp], min(1, G - 1), sq[pp], sh[pp], s1[pp]);
    }
  __syncthreads();

  f32x4 acc[NTT][4];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the item's activation operands of group g, then one row tile at a time:
  // decode it, refill its ring slot with group gn, multiply it with every token tile
  auto multiply = [&](int g, int gn) {
    if (!active) return;
    const char* ab = bufs + (g & 1) * kGemmBuf + i16 * kGemmRow + q * 16;
    u32x4 A[NTT][4];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int m = 0; m < 4; ++m) A[tt][m] = *(const u32x4*)(ab + tt * 16 * kGemmRow + m * 64);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      u32x4 W[4];
      const float sc = decode_block_x3<FMT>(ring[rt], lut, lane, W);
      ring[rt] = fetch(wrow[rt] + (int64_t)gn * 16 * BB);
      f32x4 tmp[NTT];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) tmp[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) tmp[tt] = mfma16(A[tt][m], W[m], tmp[tt]);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) acc[tt][rt] += sc * tmp[tt];
    }
  };
  auto load = [&](int g, u32x4 (&raw)[P][2]) {
#pragma unroll
    for (int pp = 0; pp < P; ++pp)
      if (stage_on[pp]) act_half_load<FMT>(srow[pp], g, sq[pp], sh[pp], raw[pp]);
  };
  auto store = [&](int g, const u32x4 (&raw)[P][2]) {  // into the buffer of group g
#pragma unroll
    for (int pp = 0; pp < P; ++pp)
      if (stage_on[pp]) act_half_store<FMT>(raw[pp], bufs + (g & 1) * kGemmBuf + si[pp] * kGemmRow, sq[pp], sh[pp]);
  };
  // The last steps fetch the last group again (in bounds, unused) and restage
  // it into the idle buffer, so the loop bodies have no branch on g.
  if constexpr (SD == 2) {
    // step g: issue group g + 2, multiply group g, stage group g + 1 (issued a step ago)
    for (int g = 0; g < G; g += 2) {
      load(min(g + 2, G - 1), s0);
      multiply(g, min(g + 1, G - 1));
      store(g + 1, s1);
      __syncthreads();
      if (g + 1 < G) {
        load(min(g + 3, G - 1), s1);
        multiply(g + 1, min(g + 2, G - 1));
        store(g + 2, s0);
        __syncthreads();
      }
    }
  } else {
    for (int g = 0; g < G; ++g) {
      const int gn = min(g + 1, G - 1);
#pragma unroll
      for (int pp = 0; pp < P; ++pp)
        if (stage_on[pp]) act_half_load<FMT>(srow[pp], gn, sq[pp], sh[pp], s0[pp]);
      if (active) {  // the multiply written out (as a lambda call it spills here)
        const char* ab = bufs + (g & 1) * kGemmBuf + i16 * kGemmRow + q * 16;
        u32x4 A[NTT][4];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int m = 0; m < 4; ++m) A[tt][m] = *(const u32x4*)(ab + tt * 16 * kGemmRow + m * 64);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          u32x4 W[4];
          const float sc = decode_block_x3<FMT>(ring[rt], lut, lane, W);
          ring[rt] = fetch(wrow[rt] + (int64_t)gn * 16 * BB);
          f32x4 tmp[NTT];
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) tmp[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) tmp[tt] = mfma16(A[tt][m], W[m], tmp[tt]);
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) acc[tt][rt] += sc * tmp[tt];
        }
      }
#pragma unroll
      for (int pp = 0; pp < P; ++pp)
        if (stage_on[pp])
          act_half_store<FMT>(s0[pp], bufs + ((g + 1) & 1) * kGemmBuf + si[pp] * kGemmRow, sq[pp], sh[pp]);
      __syncthreads();
    }
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
          const float hv = gv / (1.f + __expf(-gv)) * uv;
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
                                              char* bufs, bool ptq1) {
  if (FS != 1 && ptq1)
    gemm_unit<kPTQ1, MODE, NTT, WAVES, 1>(a, it, rb, lut, bufs, nullptr);
  else if (FS != 2)
    gemm_unit<kPQ2, MODE, NTT, WAVES, (FS == 1 && MODE == MODE_GATEUP) ? 2 : 1>(a, it, rb, lut, bufs, nullptr);
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
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  char* bufs = smem + lut_bytes;
  if (a.fmt_mask & 2) ptq1_lut_fill(lut, threadIdx.x, blockDim.x);  // visible after the unit's first sync
  const int64_t U = (int64_t)(*a.n_items) * row_blocks;
  const int64_t per = (U + 7) / 8;
  for (int64_t u = blockIdx.x; u < 8 * per; u += gridDim.x) {
    const int64_t l = (u & 7) * per + (u >> 3);
    if (l >= U) continue;
    const Item it = a.items[l / row_blocks];
    const int rb = (int)(l % row_blocks);
    const bool ptq1 = FS == 2 || (FS == 3 && a.formats[it.bank] == kPTQ1);
    switch ((it.n + 15) / 16) {
      case 1: gemm_dispatch<MODE, FS, 1, WAVES>(a, it, rb, lut, bufs, ptq1); break;
      case 2: gemm_dispatch<MODE, FS, 2, WAVES>(a, it, rb, lut, bufs, ptq1); break;
      case 3: gemm_dispatch<MODE, FS, 3, WAVES>(a, it, rb, lut, bufs, ptq1); break;
      default: gemm_dispatch<MODE, FS, 4, WAVES>(a, it, rb, lut, bufs, ptq1); break;
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

template <int FMT, int NTT, int G, bool CHK>
__device__ __forceinline__ void down_unit(const ExpertArgs& a, const Item& it, const u32x2* lut, char* xs,
                                          char* scratch) {
  const int tid = opaque_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  constexpr int K = G * kGroup;
  constexpr int stride = stage_stride(K);
  constexpr int BB = block_bytes_c<FMT>();
  constexpr int64_t row_bytes = (int64_t)G * BB;
  constexpr int D = 1;  // groups in flight (D = 2 takes 12 more registers than the wave has)
  const uint8_t* bank = a.banks + a.offsets[it.bank];
  const int64_t gu_bytes = (int64_t)a.f * (a.d / kGroup) * BB;
  const int nquads = a.d / 64;
  const int nqw = wave < nquads ? (nquads - wave + kDownWaves - 1) / kDownWaves : 0;
  constexpr int64_t quad_stride = (int64_t)64 * kDownWaves * row_bytes;

  const uint8_t* rows[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)  // chunk path: the tile's base; window path: the lane's row
    rows[rt] = bank + 2 * gu_bytes + (int64_t)(wave * 64 + 16 * rt) * row_bytes + (CHK && FMT == kPQ2 ? 0 : i16 * BB);
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
      return load_block_x3<FMT>(chunk, q);
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
  int* slot_of = (int*)(xs + kGemmChunk * stride);
  float* wgt_of = (float*)(slot_of + kGemmChunk);
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
    auto step = [&](int g, RingT (&ring)[4]) {
      u32x4 A[NTT][4];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int m = 0; m < 4; ++m) A[tt][m] = *(const u32x4*)(ab + tt * 16 * stride + g * 256 + m * 64);
      // refill with group g + D of this quad, else of the next quad (the last
      // quad refetches its own groups: in bounds, unused)
      const int64_t nxt = g + D < G ? (int64_t)(g + D) * 16 * BB : (more ? quad_stride : 0) + (int64_t)(g + D - G) * 16 * BB;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        u32x4 W[4];
        float sc;
        if constexpr (CH) {
          const u32x3 v = window(ring[rt]);
          ring[rt] = fetch(rows[rt] + nxt);
          sc = decode_block_x3<FMT>(v, lut, lane, W);
        } else {
          sc = decode_block_x3<FMT>(ring[rt], lut, lane, W);
          ring[rt] = fetch(rows[rt] + nxt);
        }
        f32x4 tmp[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) tmp[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) tmp[tt] = mfma16(A[tt][m], W[m], tmp[tt]);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[tt][rt] += sc * tmp[tt];
      }
    };
#pragma unroll 1
    for (int g = 0; g < G; g += D) {
      step(g, ring0);
      if (D == 2) step(g + 1, ring1);
    }
    // lane holds positions it.pos + 16 tt + 4q + j, column i16 of each row tile
    const int row0 = (wave + t * kDownWaves) * 64;
    // (LDS-qualified: through generic pointers these reads become flat loads,
    // whose waits also wait for every weight load in flight)
    typedef const volatile int __attribute__((address_space(3))) lds_int;
    typedef const volatile float __attribute__((address_space(3))) lds_float;
    lds_int* vslot = (lds_int*)slot_of;
    lds_float* vwgt = (lds_float*)wgt_of;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ti = 16 * tt + 4 * q + j;
        if (ti >= it.n) continue;
        const int64_t slot = vslot[ti];
        const float wgt = vwgt[ti];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          a.slots[slot * a.d + row0 + 16 * rt + i16] = (uint16_t)f32_to_bf16(wgt * acc[tt][rt][j]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) rows[rt] += quad_stride;
  }
}

template <int FS, int NTT, int G>
__device__ __forceinline__ void down_dispatch(const ExpertArgs& a, const Item& it, const u32x2* lut, char* xs,
                                              bool ptq1) {
  char* scratch = xs + kGemmChunk * (stage_stride(G * kGroup) + 8) + (threadIdx.x >> 6) * kChunkScratch;
  if (FS != 1 && ptq1)
    down_unit<kPTQ1, NTT, G, false>(a, it, lut, xs, scratch);
  else if (FS != 2)
    down_unit<kPQ2, NTT, G, FS == 1>(a, it, lut, xs, scratch);
}

// Persistent blocks over items, the blocks of one XCD taking a contiguous range
// (so the items of one expert share its down weights in one L2).
// Dynamic LDS: [PTQ1_0 byte table if the layer has PTQ1_0 banks][64 staged rows][64 slots][64 weights]
// [per-wave chunk scratch]
template <int FS, int G>
__global__ __launch_bounds__(64 * kDownWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void down_resident_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int lut_bytes = (a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0;
  u32x2* lut = (u32x2*)smem;
  char* xs = smem + lut_bytes;
  if (a.fmt_mask & 2) ptq1_lut_fill(lut, threadIdx.x, blockDim.x);  // visible after the unit's first sync
  const int64_t U = *a.n_items;
  const int64_t per = (U + 7) / 8;
  for (int64_t u = blockIdx.x; u < 8 * per; u += gridDim.x) {
    const int64_t l = (u & 7) * per + (u >> 3);
    if (l >= U) continue;
    const Item it = a.items[l];
    const bool ptq1 = FS == 2 || (FS == 3 && a.formats[it.bank] == kPTQ1);
    switch ((it.n + 15) / 16) {
      case 1: down_dispatch<FS, 1, G>(a, it, lut, xs, ptq1); break;
      case 2: down_dispatch<FS, 2, G>(a, it, lut, xs, ptq1); break;
      case 3: down_dispatch<FS, 3, G>(a, it, lut, xs, ptq1); break;
      default: down_dispatch<FS, 4, G>(a, it, lut, xs, ptq1); break;
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
  return std::max(touched, slots / kChunk) + (double)a.S * ((a.T + kChunk - 1) / kChunk);
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
  const size_t lds = ((a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0) + 2 * (size_t)kGemmBuf;
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

template <int FS, int G>
static hipError_t launch_down_resident_fs(const ExpertArgs& a, int64_t max_items, size_t lds, hipStream_t stream) {
  auto kern = down_resident_kernel<FS, G>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kDownWaves, lds);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t grid = std::min<int64_t>((int64_t)cu_count() * per_cu, max_items);
  kern<<<dim3((unsigned)grid), 64 * kDownWaves, lds, stream>>>(a);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_down_resident(const ExpertArgs& a, int64_t max_items, size_t lds, hipStream_t stream) {
  if (a.fmt_mask == 1) return launch_down_resident_fs<1, G>(a, max_items, lds, stream);
  if (a.fmt_mask == 2) return launch_down_resident_fs<2, G>(a, max_items, lds, stream);
  return launch_down_resident_fs<3, G>(a, max_items, lds, stream);
}

// Down projection of a large batch: LDS-resident h rows where the shape is
// compiled in and the rows fit, else the group-staged kernel.
static hipError_t launch_down_large(const ExpertArgs& a, int64_t mi, hipStream_t s) {
  const size_t lds = ((a.fmt_mask & 2) ? 256 * kLutCopies * 8 : 0) + (size_t)kGemmChunk * (stage_stride(a.f) + 8) +
                     (size_t)kDownWaves * kChunkScratch;
  if (lds <= 160 * 1024) {
    switch (a.f / kGroup) {
      case 8: return launch_down_resident<8>(a, mi, lds, s);
      case 6: return launch_down_resident<6>(a, mi, lds, s);
      case 4: return launch_down_resident<4>(a, mi, lds, s);
      case 1: return launch_down_resident<1>(a, mi, lds, s);
      default: break;
    }
  }
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
    case 24: return launch_stream<MODE_GATEUP, 8, 2, 8, 24>(a, mi, s);
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
    case 4: return launch_stream<MODE_DOWN, 8, 4, 4, 4>(a, mi, s);
    case 1: return launch_stream<MODE_DOWN, 8, 4, 1, 1>(a, mi, s);
    default: return launch_dec<MODE_DOWN, 8, 1, 4, 4, 0>(a, mi, s);
  }
}

hipError_t launch_experts(const ExpertArgs& a, int64_t max_items, hipStream_t stream, void** ev) {
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
  if (e == hipSuccess)
    e = gemm ? launch_down_large(a, max_items, stream) : launch_down(a, max_items, small, stream);
  if (e == hipSuccess) e = mark(7);
  return e;
}

}  // namespace moe
