// Internal interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

constexpr int kGroup = 128;     // weights per container group
constexpr int kChunk = 16;      // tokens per expert work item of a small batch (one MFMA M tile)
constexpr int kGemmChunk = 96;  // tokens per expert work item of a large batch (six M tiles)
constexpr int kRouteBlock = 256;  // tokens per ranking block
constexpr int kGroupMaxT = 256;   // largest batch grouped by one block
constexpr int kMaxExperts = 1024;

// Small batches stream each touched expert's weights once per 16 tokens; large
// batches multiply each decoded weight group with up to 96 tokens.
__host__ __device__ inline int item_chunk(int64_t T) { return T > kGroupMaxT ? kGemmChunk : kChunk; }
// The down projection of a large batch stages 64 positions at a time and takes
// work items of that size.
constexpr int kDownChunk = 64;
__host__ __device__ inline int down_chunk(int64_t T) { return T > kGroupMaxT ? kDownChunk : kChunk; }
// Small batches take 4-token work items where a streaming block with 16 staged
// token rows (2 d + 32 bytes each) and the PTQ1_0 byte table would fill more
// than half of a CU's 160 KB of LDS, but four rows leave room for two blocks,
// and the batch puts at most two tokens per expert on average (so few items
// split: mostly the shared experts' tokens).  The workspace is sized for this
// smallest chunk, so its size does not depend on the bank formats.
constexpr int kSmallChunkMin = 4;
inline int small_chunk(int64_t T, int d, int E, int k, bool ptq1) {
  const int64_t lut = ptq1 ? 256 * 16 * 8 : 0, rest = 8 * 1024 + 256;  // byte table; chunk scratch, slot table
  const int64_t row = 2 * (int64_t)d + 32;
  if (16 * row + lut + rest <= 80 * 1024) return kChunk;
  if (4 * row + lut + rest <= 80 * 1024 && T * k <= 2 * (int64_t)E) return kSmallChunkMin;
  return kChunk;
}

// Work item of the grouped expert kernels: bank, first position in the
// (expert, token)-ordered slot space, number of tokens (<= item_chunk(T)).
struct Item {
  int32_t bank;
  int32_t pos;
  int32_t n;
  int32_t pad;
};

struct DenseArgs {
  const uint16_t* act;  // bf16 [T x K], row stride lda (elements)
  int64_t lda;
  int64_t T;
  int K;
  // weight rows [0, N0) = w0 (+ w0b, summed in fp32), rows [N0, N0+N1) = w1; fp16, row stride K.
  // q0, q0b, q1: the same operands as ternary PQ2_0 rows (row-major groups,
  // K % 128 == 0), used in place of w0, w0b, w1 when not NULL
  const uint16_t* w0;
  const uint16_t* w0b;
  int N0;
  const uint16_t* w1;
  int N1;
  const uint8_t* q0;
  const uint8_t* q0b;
  const uint8_t* q1;
  // small-batch x-projection only: rows [N0 + N1, N0 + N1 + N2) = w2 (fp16),
  // which reach the fp32 partials and nothing else
  const uint16_t* w2;
  int N2;
  // the caller accepts xproj_wide_kernel for 33-256 tokens and 2048+ fp16 rows
  // (w0 without w0b, or w1): its K-step order differs from the split kernel's,
  // so a row's sums are no longer the same for every batch size
  bool staged;
  // xproj epilogue
  float* logits;   // fp32 [T x N0]
  uint16_t* z;     // bf16 [T x N1]
  // combine epilogue: y = acc + sum of the token's slots
  const uint16_t* slots;  // bf16 [(T*k + S*T) x N0]
  int top_k;
  int n_shared;
  uint16_t* y;     // bf16 [T x N0]
  // large batches: workspace for the split weights, dense_split_bytes(N0 + N1, K)
  void* wsplit;
  // small batches (T <= kGroupMaxT): fp32 partial products [splits][T][N0 + N1]
  // over the K slices of xproj_split(), added up by their consumers
  float* part;
};

// Small-batch x-projection split: each block covers one 16-row tile, one group
// of up to 64 tokens and one slice of 128 * kpw inputs (kpw 32-wide steps per
// wave); at most eight slices.  The slicing depends on K alone, so a token's
// logits come out the same whatever the batch and whether the correction rows
// share the launch.
struct XprojSplit {
  int kpw, splits;
};
inline XprojSplit xproj_split(int K) {
  const int steps = (K + 31) / 32;
  XprojSplit s;
  s.kpw = std::max(1, (steps + 31) / 32);
  s.splits = (steps + 4 * s.kpw - 1) / (4 * s.kpw);
  return s;
}

constexpr int EPI_XPROJ = 0;
constexpr int EPI_COMBINE = 1;

struct RouteArgs {
  float* logits;        // [T x E]
  int64_t T;
  int E;
  int k;
  int S;
  int32_t* idx;         // [T x k]
  float* w;             // [T x k]
  int32_t* slot_rank;   // [T x k]
  int32_t* block_cnt;   // [nb x E]
  int32_t* block_base;  // [nb x E]
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  int32_t* perm;        // [T x k]
  Item* items;          // [max_items]
  int32_t* n_items;     // [1]
  int chunk;            // tokens per work item (item_chunk(T), or small_chunk for small batches)
  // NULL, or a second list of work items of chunk2 positions (the down
  // projection's, for large batches)
  Item* items2;
  int32_t* n_items2;
  int chunk2;
  // NULL, or the x-projection partials [lsplits][T][lN] whose first E columns
  // sum (in slice order) to the logits; the top-k then also stores the sums
  // into logits
  const float* lpart;
  int lsplits, lN;
  // NULL, or z (bf16 [T x zr]) to receive the sums of the same partials'
  // columns E .. E + zr - 1: blocks beyond the routing blocks of the first
  // routing launch add them up while the routing runs
  uint16_t* z;
  int zr;
};

struct ExpertArgs {
  const uint8_t* banks;
  const int64_t* offsets;
  const uint8_t* formats;
  int d, f, E, S, k;
  int64_t T, Tk;
  const Item* items;
  const int32_t* n_items;
  const Item* down_items;      // the down projection's work items (== items for small batches)
  const int32_t* down_n_items;
  const int32_t* perm;
  const float* topk_w;
  const uint16_t* x;   // bf16 [T x d]
  uint16_t* h;         // bf16 [(Tk + S*T) x f]
  uint16_t* slots;     // bf16 [(Tk + S*T) x d]
  int nmax;            // most tokens any work item holds (<= chunk)
  int chunk;           // tokens per work item (item_chunk(T), or small_chunk for small batches)
  int fmt_mask;        // 1: some bank is PQ2_0, 2: some bank is PTQ1_0
};

hipError_t launch_unpack_device(int fmt, const uint8_t* src, int64_t n_weights, int8_t* trits,
                                uint16_t* scales, hipStream_t stream);
// Q4_0 row gather: rows idx[0..n_idx) of a table of n_rows rows of row_len
// values (row_len % 32 == 0; table 2-byte, out 16-byte aligned) -> fp32 rows.
hipError_t launch_ple_gather(const uint8_t* table, int64_t n_rows, int row_len, const int64_t* idx, int64_t n_idx,
                             float* out, hipStream_t stream);
// The k=1 draft head: y = W2 gelu(W1 [hidden ; emb] + b1) + b2 (bf16 in and out,
// fp16 weights W1 [m x 2h], W2 [h x m], biases optional).
struct HeadArgs {
  const uint16_t* hidden;
  const uint16_t* emb;
  int64_t T;
  int h, m;
  const uint16_t* w1;
  const uint16_t* b1;
  const uint16_t* w2;
  const uint16_t* b2;
  uint16_t* y;
};
// Workspace regions of the draft head (byte offsets, 256-byte aligned).
struct HeadPlan {
  int64_t xc, g, part, wsplit, total;
  bool large;
};
HeadPlan head_plan(int64_t T, int h, int m);
// stage_events: NULL or the caller's events; [0..1] bracket fc1's product, [2..3] fc2's.
hipError_t launch_head(const HeadArgs& a, char* ws, hipStream_t stream, void** stage_events);
// out[t, n] = bf16 of the sum, in slice order, of fp32 partials part[s][t][n].
hipError_t launch_fold_bf16(const float* part, int splits, int64_t T, int N, uint16_t* out, hipStream_t stream);
// Compute units of the current device (256 if the query fails).
int cu_count();
// Quantizer: groups of 128 bfloat16 weights (w 16-byte aligned, dst 4-byte
// aligned) -> container blocks, and the Lloyd rounds per group if rounds is not
// NULL; groups <= quantize_max_groups().
int64_t quantize_max_groups();
hipError_t launch_quantize(int fmt, int method, const uint16_t* w, int64_t groups, uint8_t* dst,
                           uint8_t* rounds, hipStream_t stream);
int64_t dense_split_bytes(int N, int K);
template <int EPI>
hipError_t launch_dense_gemm(const DenseArgs& a, int N, hipStream_t stream);
hipError_t launch_xproj(const DenseArgs& a, hipStream_t stream);
hipError_t launch_combine(const DenseArgs& a, hipStream_t stream);
hipError_t launch_route(const RouteArgs& a, int64_t max_items, hipStream_t stream);
// Batches of at most kTinyMaxT tokens with E <= 512, T k <= 64 and T (k + S) <= kTinyMaxSlots
// run in three launches: the x-projection, then launch_tiny: the gate/up
// kernel whose blocks route the batch themselves (and fold z), and the down
// projection fused with the combine (c: the combine's DenseArgs).
constexpr int kTinyMaxT = 4;
constexpr int kTinyMaxSlots = 256;
bool tiny_path_fits(int64_t T, int E, int k, int S, int d, int f);
hipError_t launch_tiny(const ExpertArgs& a, const RouteArgs& r, const DenseArgs& c, int64_t max_items,
                       hipStream_t stream, void** stage_events);
// stage_events: NULL or the caller's events; [4..7] bracket gate/up and down.
hipError_t launch_experts(const ExpertArgs& a, int64_t max_items, int64_t max_down_items, hipStream_t stream,
                          void** stage_events);

}  // namespace moe
