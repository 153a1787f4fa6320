// Device helpers shared by the kernels: matrix-core wrappers, bf16 rounding and
// the in-register container decoders.
//
// Both decoders turn one lane's quarter of a 128-weight group into matrix-core
// B operands for v_mfma_f32_16x16x32_bf16.  A weight t in {-1, 0, +1} becomes
// the bfloat16 value 2t, whose bit pattern is the 2-bit two's-complement code
// shifted to bits 14..15 (00 -> 0x0000, 01 -> 0x4000 = +2, 11 -> 0xC000 = -2);
// the factor 2 is folded into the group scale.  Inside a group the order of the
// K dimension is free as long as the activation operand uses the same order, so
// each decoder fixes the order that is cheapest to produce (kslot_* below) and
// the activation loaders follow it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef uint32_t __attribute__((aligned(2))) u32_a2;
typedef u32x2 __attribute__((aligned(2))) u32x2_a2;
typedef u32x2 __attribute__((aligned(4))) u32x2_a4;
typedef u32x4 __attribute__((aligned(4))) u32x4_a4;

constexpr int kPQ2 = 142;
constexpr int kPTQ1 = 143;
constexpr int kLutCopies = 16;   // PTQ1_0 byte table copies (one per LDS bank pair)
// Kernels with shared memory to spare keep 32 copies: a ds_read_b64 serves 32
// lanes per cycle, and with lane % 32 as the copy no two of them share a bank
// pair (with 16 copies lanes l and l + 16 collide when their bytes differ).
constexpr int kLutCopiesWide = 32;

// D = A(16x32) * B(32x16) + C, fp32 accumulate.  Lane l supplies row l%16 of A
// and column l%16 of B for its k-slot quarter; D lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// SwiGLU's silu(g) * u (Shazeer 2020, "GLU Variants Improve Transformer"),
// with the hardware reciprocal (within 1 ulp) in place of an IEEE division: a
// very negative g gives exp(-g) = inf, a reciprocal of 0 and a zero result, as
// the division does.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// s_getreg operand reading the SIMD field (bits 5:4) of the hardware-ID
// register (id 4): size - 1 in bits 15:11, bit offset in 10:6, id in 5:0
constexpr int kHwIdSimd = (1 << 11) | (4 << 6) | 4;

// fp32 -> bf16, rounded to nearest even (NaN stays a quiet NaN): CDNA4 converts
// in one instruction, two values at a time in the packed form
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// the pair (lo, hi) as one packed word, lo in the low half
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// ---------------------------------------------------------------- PQ2_0
// Lane quarter q of a group covers weights 32q .. 32q+31: code dwords w0, w1 at
// block bytes 8q .. 8q+7.  MFMA m takes code word m>>1 and the four pairs
// jj = 4(m&1) .. 4(m&1)+3, each pair being weights (jj, jj+8) of that word.
//   k-slot (m, q, j) -> weight 32q + 16(m>>1) + 4(m&1) + (j>>1) + 8(j&1)
__device__ __forceinline__ int kslot_pq2(int m, int q, int j) {
  return 32 * q + 16 * (m >> 1) + 4 * (m & 1) + (j >> 1) + 8 * (j & 1);
}

__device__ __forceinline__ void decode_pq2(uint32_t w0, uint32_t w1, u32x4 out[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t w = (m >> 1) ? w1 : w0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jj = 4 * (m & 1) + i;
      out[m][i] = (w << (14 - 2 * jj)) & 0xC000C000u;
    }
  }
}

// ---------------------------------------------------------------- PTQ1_0
// Byte table: entry v (0..242) holds the five digits of v as bytes c<<6 with
// c the 2-bit code of the digit's trit (0 -> 0x00, 1 -> 0x40, 2 -> 0xC0):
// lo = digits 0..3, hi = digit 4.  A tail byte (< 81) reads the same table.
// Lane quarter q covers data bytes 6q .. 6q+5 (weights 30q .. 30q+29) and the
// tail digits 2(q&1), 2(q&1)+1 of tail byte 24 + (q>>1) (weights 120+2q, 121+2q).
// Pairs P = 0..15 (MFMA m = P/4) are consecutive weights:
//   k-slot (m, q, j) -> weight 30q + 8m + j for 8m + j < 30, else 120 + 2q + (j&1)
__device__ __forceinline__ int kslot_ptq1(int m, int q, int j) {
  const int r = 8 * m + j;
  return r < 30 ? 30 * q + r : 120 + 2 * q + (j & 1);
}

// The byte table as a compile-time constant in the code object (2 KB).
struct Ptq1Table {
  uint32_t lo[256];
  uint32_t hi[256];
};
__host__ __device__ constexpr uint32_t ptq1_code_byte(int v, int i) {
  int r = v;
  for (int j = 0; j < i; ++j) r /= 3;
  return r % 3 == 0 ? 0u : (r % 3 == 1 ? 0x40u : 0xC0u);
}
__host__ __device__ constexpr Ptq1Table make_ptq1_table() {
  Ptq1Table t{};
  for (int v = 0; v < 256; ++v) {
    t.lo[v] = ptq1_code_byte(v, 0) | (ptq1_code_byte(v, 1) << 8) | (ptq1_code_byte(v, 2) << 16) |
              (ptq1_code_byte(v, 3) << 24);
    t.hi[v] = ptq1_code_byte(v, 4);
  }
  return t;
}
__device__ constexpr Ptq1Table kPtq1Table = make_ptq1_table();

// Fill the LDS byte table of NC copies (all threads of the block take part;
// caller syncs).
template <int NC = kLutCopies>
__device__ __forceinline__ void ptq1_lut_fill(u32x2* lut, int tid, int nthreads) {
  for (int idx = tid; idx < 256 * NC; idx += nthreads) {
    const int v = idx / NC;
    lut[idx] = u32x2{kPtq1Table.lo[v], kPtq1Table.hi[v]};
  }
}

template <int NC = kLutCopies>
__device__ __forceinline__ u32x2 lut_get(const u32x2* lut, uint32_t v, int copy) {
  return lut[v * NC + copy];
}

// sel for perm_b32 building a bf16 pair from two table bytes: byte `a` of
// {s0:s1} to bits 8..15 and byte `b` to bits 24..31, low bytes zero.
__host__ __device__ constexpr uint32_t pair_sel(uint32_t a, uint32_t b) {
  return 0x0Cu | (a << 8) | (0x0Cu << 16) | (b << 24);
}

// d0, d1: block bytes 6q .. 6q+7; tail: block bytes 24 .. 27.
template <int NC = kLutCopies>
__device__ __forceinline__ void decode_ptq1(const u32x2* lut, int copy, uint32_t d0, uint32_t d1,
                                            uint32_t tail, int q, u32x4 out[4]) {
  u32x2 L[6];
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint32_t src = b < 4 ? d0 : d1;
    L[b] = lut_get<NC>(lut, (src >> (8 * (b & 3))) & 0xFFu, copy);
  }
  const u32x2 Lt = lut_get<NC>(lut, (tail >> (8 * (q >> 1))) & 0xFFu, copy);
  uint32_t P[16];
#pragma unroll
  for (int bp = 0; bp < 3; ++bp) {
    const u32x2 A = L[2 * bp], B = L[2 * bp + 1];
    P[5 * bp + 0] = perm_b32(0u, A.x, pair_sel(0, 1));
    P[5 * bp + 1] = perm_b32(0u, A.x, pair_sel(2, 3));
    P[5 * bp + 2] = perm_b32(B.x, A.y, pair_sel(0, 4));
    P[5 * bp + 3] = perm_b32(0u, B.x, pair_sel(1, 2));
    P[5 * bp + 4] = perm_b32(B.y, B.x, pair_sel(3, 4));
  }
  const uint32_t ts = (q & 1) ? pair_sel(2, 3) : pair_sel(0, 1);
  P[15] = perm_b32(0u, Lt.x, ts);
#pragma unroll
  for (int m = 0; m < 4; ++m) out[m] = u32x4{P[4 * m], P[4 * m + 1], P[4 * m + 2], P[4 * m + 3]};
}

// One load per lane per block: three dwords from byte 8q (PQ2_0) or 6q
// (PTQ1_0) of the block.  The first two are the lane's code dwords (PQ2_0:
// bytes 8q .. 8q+7; PTQ1_0: bytes 6q .. 6q+7); quarter 3's load also covers the
// bytes after the data (PQ2_0: the scale at 32..33; PTQ1_0: tail bytes 24..25
// and the scale at 26..27) and runs 2 bytes past the block, which is why
// expert banks carry 16 bytes of readable slack after their last block.  The
// row's four lanes are l%16 + 16q, so quarter 3's bytes reach the others with
// one cross-lane read.
typedef __attribute__((ext_vector_type(3))) uint32_t u32x3;
typedef u32x3 __attribute__((aligned(2))) u32x3_a2;

template <int FMT>
__device__ __forceinline__ u32x3 load_block_x3(const uint8_t* blk, int q) {
  return *(const u32x3_a2*)(blk + (FMT == kPQ2 ? 8 : 6) * q);
}

// The same window from one 12-byte load at 4-byte alignment (windows start
// 2-byte aligned): when the window starts at 2 mod 4 the load begins 2 bytes
// early and the window's last 2 bytes, which no decoder uses, are dropped.
// Such loads stream about 1.4x faster than the 2-byte-aligned ones; the small-
// batch PQ2_0 reads take them (elsewhere the per-load address arithmetic cost
// more than it saved).
typedef u32x3 __attribute__((aligned(4))) u32x3_a4;
template <int FMT>
__device__ __forceinline__ u32x3 load_block_x3_a4(const uint8_t* blk, int q) {
  const uint8_t* p = blk + (FMT == kPQ2 ? 8 : 6) * q;
  const int mis = (int)((uintptr_t)p & 2);  // pointer arithmetic keeps the global address space
  const u32x3 v = *(const u32x3_a4*)(p - mis);
  const uint32_t sh = (uint32_t)mis * 8;
  return u32x3{__builtin_amdgcn_alignbit(v.y, v.x, sh), __builtin_amdgcn_alignbit(v.z, v.y, sh), v.z >> sh};
}

// Decode one lane's quarter of a block fetched with load_block_x3 into the
// B operands; returns the group scale.  The operands encode 2t, so results
// carry a factor 2 that the caller removes once.
template <int FMT, int NC = kLutCopies>
__device__ __forceinline__ float decode_block_x3(u32x3 v, const u32x2* lut, int lane, u32x4 out[4]) {
  const int q = lane >> 4;
  // PQ2_0: quarter 3's third dword holds bytes 32..35 (scale low half);
  // PTQ1_0: bytes 24..27 (tail bytes low half, scale high half).
  const uint32_t mine = FMT == kPQ2 ? v.z : __builtin_amdgcn_alignbit(v.z, v.y, 16);
  const uint32_t shared = __shfl(mine, (lane & 15) + 48, 64);
  if (FMT == kPQ2) {
    decode_pq2(v.x, v.y, out);
    return f16_to_f32(shared & 0xFFFFu);
  } else {
    decode_ptq1<NC>(lut, lane % NC, v.x, v.y, shared, q, out);
    return f16_to_f32(shared >> 16);
  }
}

template <int FMT>
__host__ __device__ constexpr int block_bytes_c() {
  return FMT == kPQ2 ? 34 : 28;
}

// ---------------------------------------------------------------- aligned chunks
// On the device the 16 blocks of one group of a 16-row tile are contiguous
// (16 * BB bytes, 16-byte aligned).  Aligned 16-byte loads stream about 1.5x
// faster than the 2-byte-aligned 12-byte window of load_block_x3, so a wave
// reads the chunk as BB pieces of 16 bytes (lanes past BB - 1 repeat the last
// piece) and rearranges it through a per-wave LDS scratch into the same
// per-lane window.
constexpr int kChunkScratch = 64 * 16;  // bytes of scratch per chunk: one 16-byte piece per lane

template <int FMT>
__device__ __forceinline__ u32x4 load_chunk(const uint8_t* chunk, int lane) {
  constexpr int NL = block_bytes_c<FMT>();  // 16 * BB / 16 pieces
  return *(const u32x4*)(chunk + 16 * min(lane, NL - 1));
}

template <int FMT>
__device__ __forceinline__ u32x3 chunk_window(u32x4 piece, char* scratch, int lane) {
  constexpr int BB = block_bytes_c<FMT>();
  // every lane writes (lanes past BB - 1 a repeat of the last piece, past the
  // chunk), so no branch splits the caller's loop body
  *(u32x4*)(scratch + 16 * lane) = piece;
  // the wave's LDS operations complete in order; the fences keep the compiler
  // from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int o = (lane & 15) * BB + (FMT == kPQ2 ? 8 : 6) * (lane >> 4);
  const u32x4 d = *(const u32x4_a4*)(scratch + (o & ~3));
  const uint32_t sh = (uint32_t)(o & 3) * 8;
  const u32x3 v = u32x3{__builtin_amdgcn_alignbit(d.y, d.x, sh), __builtin_amdgcn_alignbit(d.z, d.y, sh),
                        __builtin_amdgcn_alignbit(d.w, d.z, sh)};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return v;
}

// ---------------------------------------------------------------- dense fp16 weights
// Dense fp16 weight rows feed bf16 matrix cores as two bf16 terms (hi + lo).
// fp16 x8 (4 dwords) -> exact bf16 hi/lo operand pairs (truncated hi).
__device__ __forceinline__ void split_f16x8(u32x4 w, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = f16_to_f32(w[i] & 0xFFFFu), b = f16_to_f32(w[i] >> 16);
    const uint32_t ha = __float_as_uint(a) & 0xFFFF0000u, hb = __float_as_uint(b) & 0xFFFF0000u;
    const uint32_t la = __float_as_uint(a - __uint_as_float(ha)), lb = __float_as_uint(b - __uint_as_float(hb));
    hi[i] = perm_b32(hb, ha, 0x07060302u);
    lo[i] = perm_b32(lb, la, 0x07060302u);
  }
}

// fp16 x8 from two sources summed in fp32 -> bf16 hi (round to nearest even) +
// bf16 lo (round to nearest even); |error| <= 2^-18 |a + b|.
__device__ __forceinline__ void split_sum_f16x8(u32x4 w, u32x4 v, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = f16_to_f32(w[i] & 0xFFFFu) + f16_to_f32(v[i] & 0xFFFFu);
    const float b = f16_to_f32(w[i] >> 16) + f16_to_f32(v[i] >> 16);
    const uint32_t h = f32x2_to_bf16x2(a, b);
    hi[i] = h;
    lo[i] = f32x2_to_bf16x2(a - bf16_to_f32(h & 0xFFFFu), b - bf16_to_f32(h >> 16));
  }
}

// ---------------------------------------------------------------- activations
// Matrix-core A operands (bf16) for one row of activations and one group, in the
// k-slot order of the container format.  The raw loads and the reordering are
// separate so a prefetch ring can hold the raw dwords.
//   PQ2_0: raw = elements 32q .. 32q+31 of the group (16 dwords);
//   PTQ1_0: raw = elements 30q .. 30q+29 and the tail pair 120+2q, 121+2q.
struct ActRaw {
  u32x4 v[4];
};

template <int FMT>
__device__ __forceinline__ ActRaw load_act_raw(const uint16_t* row, int g, int q) {
  ActRaw r;
  if (FMT == kPQ2) {
    const u32x4* p = (const u32x4*)(row + g * 128 + 32 * q);
    r.v[0] = p[0];
    r.v[1] = p[1];
    r.v[2] = p[2];
    r.v[3] = p[3];
  } else {
    const uint16_t* p = row + g * 128 + 30 * q;  // 4-byte aligned
    r.v[0] = *(const u32x4_a4*)(p + 0);
    r.v[1] = *(const u32x4_a4*)(p + 8);
    r.v[2] = *(const u32x4_a4*)(p + 16);
    const u32x2 w = *(const u32x2_a4*)(p + 24);
    const uint32_t w2 = *(const uint32_t*)(p + 28);
    const uint32_t t = *(const uint32_t*)(row + g * 128 + 120 + 2 * q);
    r.v[3] = u32x4{w.x, w.y, w2, t};
  }
  return r;
}

template <int FMT>
__device__ __forceinline__ void act_operands(const ActRaw& r, u32x4 out[4]) {
  if (FMT == kPQ2) {
    uint32_t x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[4 * i + 0] = r.v[i].x;
      x[4 * i + 1] = r.v[i].y;
      x[4 * i + 2] = r.v[i].z;
      x[4 * i + 3] = r.v[i].w;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d1 = 8 * (m >> 1) + 2 * (m & 1) + (i >> 1);
        out[m][i] = perm_b32(x[d1 + 4], x[d1], (i & 1) ? 0x07060302u : 0x05040100u);
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) out[m] = r.v[m];
  }
}

}  // namespace moe
