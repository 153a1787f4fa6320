// Host side of the C ABI: the container codec, argument validation, workspace
// carving and the launch sequence of one forward pass.  Container layouts:
// Scion-35B-A3B card, "Weight Representation" (PQ2_0) and Scion-FlashNext card,
// "Weight Representation" (PTQ1_0); see include/moe_ternary.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "moe_ternary.h"
#include "host_error.h"
#include "moe_internal.h"
#include "router_delta.h"

namespace {

thread_local void** g_stage_events = nullptr;

// Record the stage's start (end=false) or end event if measurement is on.
hipError_t stage_mark(int stage, bool end, hipStream_t st) {
  if (!g_stage_events) return hipSuccess;
  hipEvent_t ev = (hipEvent_t)g_stage_events[2 * stage + (end ? 1 : 0)];
  return ev ? hipEventRecord(ev, st) : hipSuccess;
}

using moe::bad_fmt;
using moe::fail;
using moe::known_fmt;
using moe::ok;

int32_t device_fail(hipError_t e, const char* what) {
  return fail(MOE_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// --------------------------------------------------------------- workspace plan
constexpr int64_t kAlign = 256;
int64_t up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int64_t T, Tk, n_pos, nb, max_items, max_items2;
  int64_t logits, z, idx, w, rank, bcnt, bbase, counts, offsets, perm, items, nitems, items2, nitems2, wsplit, xpart,
      vpart, h, slots;
  int rd;  // rank of a factorised router delta, 0 for none
  int chunk, chunk2;  // tokens per gate/up and per down work item (set_chunk for small batches)
  bool large;
  int64_t route_end, total;
};

Plan make_plan(int64_t T, int d, int E, int S, int f, int k, int r, int rd = 0) {
  Plan p{};
  p.T = T;
  p.rd = rd;
  p.Tk = T * k;
  p.n_pos = p.Tk + (int64_t)S * T;
  p.nb = (T + moe::kRouteBlock - 1) / moe::kRouteBlock;
  p.chunk = moe::item_chunk(T);
  p.chunk2 = moe::down_chunk(T);
  // small batches: room for the smallest chunk set_chunk can choose
  const int64_t C = T > moe::kGroupMaxT ? p.chunk : moe::kSmallChunkMin, C2 = p.chunk2;
  p.max_items = p.Tk / C + std::min<int64_t>(E, p.Tk) + (int64_t)S * ((T + C - 1) / C);
  p.max_items2 = p.Tk / C2 + std::min<int64_t>(E, p.Tk) + (int64_t)S * ((T + C2 - 1) / C2);
  int64_t o = 0;
  p.logits = o; o += up(T * E * 4);
  p.idx = o; o += up(p.Tk * 4);
  p.w = o; o += up(p.Tk * 4);
  p.rank = o; o += up(p.Tk * 4);
  p.bcnt = o; o += up(p.nb * E * 4);
  p.bbase = o; o += up(p.nb * E * 4);
  p.counts = o; o += up((int64_t)E * 4);
  p.offsets = o; o += up((int64_t)(E + 1) * 4);
  p.perm = o; o += up(p.Tk * 4);
  p.items = o; o += up(std::max<int64_t>(p.max_items, 1) * (int64_t)sizeof(moe::Item));
  p.nitems = o; o += up(4);
  // the down projection's own work items (when its chunk differs from gate/up's)
  p.items2 = o;
  p.nitems2 = o;
  {
    o += up(std::max<int64_t>(p.max_items2, 1) * (int64_t)sizeof(moe::Item));
    p.nitems2 = o;
    o += up(4);
  }
  // large batches: split dense weights of the x-projection, later of the combine
  p.large = T > moe::kGroupMaxT;
  p.wsplit = o;
  if (p.large)
    o += up(std::max({moe::dense_split_bytes(E + r, d), moe::dense_split_bytes(d, r),
                      rd ? moe::dense_split_bytes(rd, d) : (int64_t)0}));
  // small batches: fp32 x-projection partials over the K slices; a factorised
  // router delta adds its V rows to the projection and one more slice, its
  // U (V x) and zeros
  const int splits = moe::xproj_split(d).splits;
  p.xpart = o;
  if (!p.large && T > 0) o += up((int64_t)(splits + (rd ? 1 : 0)) * T * (E + r + rd) * 4);
  // large batches: V x of a factorised delta as fp32 rows
  p.vpart = o;
  if (rd && p.large) o += up(T * (int64_t)rd * 4);
  p.route_end = o;
  p.z = o; o += up(T * (int64_t)r * 2);
  p.h = o; o += up(p.n_pos * f * 2);
  p.slots = o; o += up(p.n_pos * d * 2);
  p.total = o;
  return p;
}

// The work-item sizes of a small batch for this layer: gate/up small_chunk,
// the down projection (whose staged rows are short) 16 tokens.  Up to four
// tokens the items hold at most four tokens either way: one list.
void set_chunk(Plan& p, int d, int E, int k, bool ptq1) {
  if (p.large) return;
  p.chunk = p.T <= moe::kTinyMaxT ? moe::kChunk : moe::small_chunk(p.T, d, E, k, ptq1);
  p.chunk2 = moe::kChunk;
}

template <class T>
T* at(void* ws, int64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int32_t check_dims(int64_t T, int d, int E, int k) {
  if (T < 0) return fail(MOE_E_ARG, "n_tokens must be >= 0 (got %lld)", (long long)T);
  if (d <= 0 || d % 128) return fail(MOE_E_SHAPE, "d_model must be a positive multiple of 128 (got %d)", d);
  if (d > 8192) return fail(MOE_E_SHAPE, "d_model above 8192 is not supported (got %d)", d);
  if (E < 1 || E > moe::kMaxExperts)
    return fail(MOE_E_SHAPE, "n_experts must be in [1, %d] (got %d)", moe::kMaxExperts, E);
  if (k < 1 || k > E) return fail(MOE_E_SHAPE, "top_k must be in [1, n_experts=%d] (got %d)", E, k);
  if (T * (int64_t)k > (int64_t)1 << 30)
    return fail(MOE_E_SHAPE, "n_tokens * top_k above 2^30 is not supported");
  return MOE_OK;
}

int32_t check_banks(const moe_expert_banks* b) {
  if (!b) return fail(MOE_E_ARG, "expert_banks is NULL");
  if (b->d_model <= 0 || b->d_model % 128)
    return fail(MOE_E_SHAPE, "d_model must be a positive multiple of 128 (got %d)", b->d_model);
  if (b->d_ff <= 0 || b->d_ff % 128)
    return fail(MOE_E_SHAPE, "d_ff must be a positive multiple of 128 (got %d)", b->d_ff);
  if (b->d_ff > 8192) return fail(MOE_E_SHAPE, "d_ff above 8192 is not supported (got %d)", b->d_ff);
  if (b->n_shared < 0 || b->n_shared > 8)
    return fail(MOE_E_SHAPE, "n_shared must be in [0, 8] (got %d)", b->n_shared);
  if (b->n_experts < 1 || b->n_experts > moe::kMaxExperts)
    return fail(MOE_E_SHAPE, "n_experts must be in [1, %d] (got %d)", moe::kMaxExperts, b->n_experts);
  if (!b->banks || !b->offsets || !b->formats || !b->formats_host || !b->offsets_host)
    return fail(MOE_E_ARG, "expert_banks has a NULL pointer");
  if (b->layout == MOE_BANKS_ROW_MAJOR)
    return fail(MOE_E_ARG,
                "expert_banks.layout is MOE_BANKS_ROW_MAJOR (moe_pack's block order); reorder each container "
                "with moe_tile_container and set layout = MOE_BANKS_TILE_MAJOR");
  if (b->layout != MOE_BANKS_TILE_MAJOR)
    return fail(MOE_E_ARG, "expert_banks.layout is %d; it must be MOE_BANKS_TILE_MAJOR (%d), the block order of "
                "moe_tile_container", (int)b->layout, (int)MOE_BANKS_TILE_MAJOR);
  const int nb = b->n_experts + b->n_shared;
  const int64_t nblocks = 3 * (int64_t)b->d_ff * b->d_model / 128;
  for (int e = 0; e < nb; ++e) {
    const int fmt = b->formats_host[e];
    if (!known_fmt(fmt))
      return fail(MOE_E_FORMAT, "bank %d: unknown container id %d; valid ids are 142 (PQ2_0) and 143 (PTQ1_0)",
                  e, fmt);
    const int64_t off = b->offsets_host[e];
    const int64_t bytes = nblocks * moe_block_bytes(fmt);
    if (off < 0 || off % 16)
      return fail(MOE_E_ARG, "bank %d: offset %lld is not a non-negative multiple of 16", e, (long long)off);
    if (off + bytes + MOE_BANK_SLACK > b->banks_bytes)
      return fail(MOE_E_SPACE, "bank %d: bytes [%lld, %lld) plus %d bytes of slack exceed banks_bytes %lld", e,
                  (long long)off, (long long)(off + bytes), (int)MOE_BANK_SLACK, (long long)b->banks_bytes);
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_set_stage_events(void** events, int32_t n_events) {
  if (events == nullptr || n_events == 0) {
    g_stage_events = nullptr;
    return ok();
  }
  if (n_events < 2 * MOE_N_STAGES)
    return fail(MOE_E_ARG, "need %d events, got %d", 2 * MOE_N_STAGES, (int)n_events);
  g_stage_events = events;
  return ok();
}

int32_t moe_unpack_device(int32_t fmt, const uint8_t* d_src, int64_t n, int8_t* d_trits, uint16_t* d_scales,
                          void* stream) {
  if (!known_fmt(fmt)) return bad_fmt(fmt);
  if (n < 0 || n % 128) return fail(MOE_E_SHAPE, "weight count %lld is not a multiple of 128", (long long)n);
  if (n == 0) return ok();
  if (!d_src || !d_trits || !d_scales) return fail(MOE_E_ARG, "NULL pointer");
  if ((uintptr_t)d_src % 4) return fail(MOE_E_ARG, "d_src must be 4-byte aligned");
  hipError_t e = moe::launch_unpack_device(fmt, d_src, n, d_trits, d_scales, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "moe_unpack_device launch");
  return ok();
}

int32_t moe_quantize_device(int32_t fmt, int32_t method, const uint16_t* d_w, int64_t n, uint8_t* d_dst,
                            uint8_t* d_rounds, void* stream) {
  if (!known_fmt(fmt)) return bad_fmt(fmt);
  if (method != MOE_QUANT_ABSMEAN && method != MOE_QUANT_LLOYD)
    return fail(MOE_E_ARG, "unknown quantizer method %d; valid are 0 (absmean) and 1 (Lloyd)", (int)method);
  if (n < 0 || n % 128) return fail(MOE_E_SHAPE, "weight count %lld is not a multiple of 128", (long long)n);
  if (n / 128 > moe::quantize_max_groups())
    return fail(MOE_E_SHAPE, "weight count %lld exceeds one launch", (long long)n);
  if (n == 0) return ok();
  if (!d_w || !d_dst) return fail(MOE_E_ARG, "NULL pointer");
  if ((uintptr_t)d_w % 16) return fail(MOE_E_ARG, "d_w must be 16-byte aligned");
  if ((uintptr_t)d_dst % 4) return fail(MOE_E_ARG, "d_dst must be 4-byte aligned");
  const uintptr_t w0 = (uintptr_t)d_w, w1 = w0 + (uintptr_t)n * 2;
  const uintptr_t d0 = (uintptr_t)d_dst, d1 = d0 + (uintptr_t)(n / 128 * (fmt == MOE_PQ2_0 ? 34 : 28));
  if (w0 < d1 && d0 < w1) return fail(MOE_E_ARG, "d_w and d_dst overlap");
  if (d_rounds) {
    const uintptr_t r0 = (uintptr_t)d_rounds, r1 = r0 + (uintptr_t)(n / 128);
    if ((r0 < w1 && w0 < r1) || (r0 < d1 && d0 < r1)) return fail(MOE_E_ARG, "d_rounds overlaps d_w or d_dst");
  }
  hipError_t e = moe::launch_quantize(fmt, method, d_w, n / 128, d_dst, d_rounds, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "moe_quantize_device launch");
  return ok();
}

int32_t moe_ple_gather_q4_0(const uint8_t* d_table, int64_t n_rows, int32_t row_len, const int64_t* d_idx,
                            int64_t n_idx, float* d_out, void* stream) {
  if (row_len <= 0 || row_len % 32)
    return fail(MOE_E_SHAPE, "row length %d is not a positive multiple of 32", (int)row_len);
  if (n_rows < 0 || n_idx < 0)
    return fail(MOE_E_SHAPE, "negative count (rows %lld, indices %lld)", (long long)n_rows, (long long)n_idx);
  if (n_idx == 0) return ok();
  if (!d_idx || !d_out || (!d_table && n_rows > 0)) return fail(MOE_E_ARG, "NULL pointer");
  if ((uintptr_t)d_table % 2) return fail(MOE_E_ARG, "d_table must be 2-byte aligned");
  if ((uintptr_t)d_idx % 8) return fail(MOE_E_ARG, "d_idx must be 8-byte aligned");
  if ((uintptr_t)d_out % 16) return fail(MOE_E_ARG, "d_out must be 16-byte aligned");
  hipError_t e = moe::launch_ple_gather(d_table, n_rows, row_len, d_idx, n_idx, d_out, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "moe_ple_gather_q4_0 launch");
  return ok();
}

// ------------------------------------------------------------ low-rank branch
struct LowrankPlan {
  int64_t z, part, wsplit, total;
  bool large;
};

static LowrankPlan lowrank_plan(int64_t T, int d, int r) {
  LowrankPlan p{};
  p.large = T > moe::kGroupMaxT;
  int64_t o = 0;
  p.z = o; o += up(T * (int64_t)r * 2);
  p.part = o;
  if (!p.large) o += up((int64_t)moe::xproj_split(d).splits * T * r * 4);
  p.wsplit = o;
  if (p.large) o += up(std::max(moe::dense_split_bytes(r, d), moe::dense_split_bytes(d, r)));
  p.total = o;
  return p;
}

int64_t moe_lowrank_workspace_bytes(int64_t n_tokens, int32_t d, int32_t r) {
  if (n_tokens < 0 || d <= 0 || r <= 0) return -1;
  return lowrank_plan(n_tokens, d, r).total;
}

int32_t moe_lowrank_apply(const uint16_t* x, const uint16_t* y_in, int64_t T, int32_t d, const uint16_t* A,
                          const uint8_t* A_q, const uint16_t* B, const uint8_t* B_q, int32_t r, uint16_t* y,
                          void* ws, int64_t ws_bytes, void* stream) {
  try {
    if (T < 0) return fail(MOE_E_SHAPE, "negative token count %lld", (long long)T);
    if (d <= 0 || d % 128) return fail(MOE_E_SHAPE, "d_model %d is not a positive multiple of 128", (int)d);
    if (r <= 0 || r % 8 || r > 4096)
      return fail(MOE_E_SHAPE, "rank %d must be a positive multiple of 8, at most 4096", (int)r);
    if (B_q && r % 128) return fail(MOE_E_SHAPE, "a ternary B needs a rank that is a multiple of 128 (got %d)", (int)r);
    if ((A == nullptr) == (A_q == nullptr) || (B == nullptr) == (B_q == nullptr))
      return fail(MOE_E_ARG, "give exactly one of A, A_q and one of B, B_q");
    if (T == 0) return ok();
    if (!x || !y || !ws) return fail(MOE_E_ARG, "NULL pointer");
    if (x == y) return fail(MOE_E_ARG, "y must not alias x");
    if ((uintptr_t)ws % kAlign) return fail(MOE_E_ARG, "workspace must be 256-byte aligned");
    if ((uintptr_t)x % 16 || (uintptr_t)y % 16 || (uintptr_t)y_in % 16)
      return fail(MOE_E_ARG, "x, y and y_in must be 16-byte aligned");
    if ((uintptr_t)A % 4 || (uintptr_t)B % 4 || (uintptr_t)A_q % 2 || (uintptr_t)B_q % 2)
      return fail(MOE_E_ARG, "A, B must be 4-byte and ternary containers 2-byte aligned");
    const LowrankPlan p = lowrank_plan(T, d, r);
    if (ws_bytes < p.total)
      return fail(MOE_E_SPACE, "workspace holds %lld bytes, %lld needed", (long long)ws_bytes, (long long)p.total);
    const hipStream_t st = (hipStream_t)stream;
    uint16_t* z = at<uint16_t>(ws, p.z);
    moe::DenseArgs xa{};
    xa.act = x;
    xa.lda = d;
    xa.T = T;
    xa.K = d;
    xa.N0 = 0;
    xa.w1 = A;
    xa.q1 = A_q;
    xa.N1 = r;
    xa.z = z;
    xa.part = p.large ? nullptr : at<float>(ws, p.part);
    xa.staged = true;
    xa.wsplit = p.large ? at<void>(ws, p.wsplit) : nullptr;
    hipError_t e = stage_mark(0, false, st);
    if (e == hipSuccess) e = moe::launch_xproj(xa, st);
    if (e == hipSuccess) e = stage_mark(0, true, st);
    if (e == hipSuccess && !p.large) e = moe::launch_fold_bf16(xa.part, moe::xproj_split(d).splits, T, r, z, st);
    if (e != hipSuccess) return device_fail(e, "low-rank projection launch");
    moe::DenseArgs ca{};
    ca.act = z;
    ca.lda = r;
    ca.T = T;
    ca.K = r;
    ca.w0 = B;
    ca.q0 = B_q;
    ca.N0 = d;
    ca.slots = y_in;           // y_in enters as the one "shared" slot of each token
    ca.top_k = 0;
    ca.n_shared = y_in ? 1 : 0;
    ca.y = y;
    ca.wsplit = p.large ? at<void>(ws, p.wsplit) : nullptr;
    e = stage_mark(1, false, st);
    if (e == hipSuccess) e = moe::launch_combine(ca, st);
    if (e == hipSuccess) e = stage_mark(1, true, st);
    if (e != hipSuccess) return device_fail(e, "low-rank combine launch");
    return ok();
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_lowrank_apply");
  }
}

int64_t moe_draft_head_workspace_bytes(int64_t n_tokens, int32_t hidden, int32_t inner) {
  if (n_tokens < 0 || hidden <= 0 || inner <= 0) return -1;
  return moe::head_plan(n_tokens, hidden, inner).total;
}

int32_t moe_draft_head(const uint16_t* hidden, const uint16_t* emb, int64_t T, int32_t h, int32_t m,
                       const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, const uint16_t* b2, uint16_t* y,
                       void* ws, int64_t ws_bytes, void* stream) {
  if (T < 0) return fail(MOE_E_SHAPE, "negative token count %lld", (long long)T);
  if (h <= 0 || m <= 0 || h % 128 || m % 128)
    return fail(MOE_E_SHAPE, "hidden %d and inner %d must be positive multiples of 128", (int)h, (int)m);
  if (T == 0) return ok();
  if (!hidden || !emb || !w1 || !w2 || !y || !ws) return fail(MOE_E_ARG, "NULL pointer");
  if ((uintptr_t)ws % kAlign) return fail(MOE_E_ARG, "workspace must be 256-byte aligned");
  if ((uintptr_t)w1 % 4 || (uintptr_t)w2 % 4 || (uintptr_t)hidden % 16 || (uintptr_t)emb % 16 ||
      (uintptr_t)y % 2 || (uintptr_t)b1 % 2 || (uintptr_t)b2 % 2)
    return fail(MOE_E_ARG, "hidden and emb must be 16-byte, weights 4-byte and y, biases 2-byte aligned");
  const int64_t need = moe::head_plan(T, h, m).total;
  if (ws_bytes < need)
    return fail(MOE_E_SPACE, "workspace holds %lld bytes, %lld needed", (long long)ws_bytes, (long long)need);
  moe::HeadArgs a{hidden, emb, T, h, m, w1, b1, w2, b2, y};
  hipError_t e = moe::launch_head(a, (char*)ws, (hipStream_t)stream, g_stage_events);
  if (e != hipSuccess) return device_fail(e, "moe_draft_head launch");
  return ok();
}

int64_t moe_route_workspace_bytes(int64_t n_tokens, int32_t d_model, int32_t n_experts, int32_t top_k) {
  if (n_tokens < 0 || n_experts < 1 || top_k < 1) return -1;
  return make_plan(n_tokens, d_model, n_experts, 0, 128, top_k, 0).route_end;
}

int64_t moe_workspace_bytes(const moe_expert_banks* banks, int64_t n_tokens, int32_t top_k, int32_t corr_rank) {
  if (!banks || n_tokens < 0 || top_k < 1 || corr_rank < 0) return -1;
  return make_plan(n_tokens, banks->d_model, banks->n_experts, banks->n_shared, banks->d_ff, top_k, corr_rank).total;
}

// delta_q, corr_A_q: the router delta and A as ternary PQ2_0 containers (in
// place of delta, corr_A), or NULL.
// delta_U, delta_V: the router delta as factors U [E x p.rd], V [p.rd x d]
// (p.rd > 0), in place of delta / delta_q.
static int32_t route_impl(const uint16_t* x, int64_t T, int d, int E, int S, const uint16_t* router,
                          const uint16_t* delta, const uint8_t* delta_q, const uint16_t* corr_A,
                          const uint8_t* corr_A_q, int r, int k, const Plan& p, void* ws, hipStream_t stream,
                          float* logits, int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                          int32_t* perm, const uint16_t* delta_U = nullptr, const uint16_t* delta_V = nullptr,
                          moe::RouteArgs* route_out = nullptr) {
  const int splits = moe::xproj_split(d).splits;
  hipError_t e = stage_mark(0, false, stream);
  if (p.rd && p.large && e == hipSuccess) {  // V x first, a tiled product of its own with fp32 outputs
    moe::DenseArgs va{};
    va.act = x;
    va.lda = d;
    va.T = T;
    va.K = d;
    va.w0 = delta_V;
    va.N0 = p.rd;
    va.logits = at<float>(ws, p.vpart);
    va.wsplit = at<void>(ws, p.wsplit);
    e = moe::launch_xproj(va, stream);
  }
  if (e != hipSuccess) return device_fail(e, "router delta V x launch");
  moe::DenseArgs da{};
  da.act = x;
  da.lda = d;
  da.T = T;
  da.K = d;
  da.w0 = router;
  da.w0b = delta;
  da.q0b = delta_q;
  da.N0 = E;
  da.w1 = corr_A;
  da.q1 = corr_A_q;
  da.N1 = (corr_A || corr_A_q) ? r : 0;
  da.logits = logits;
  da.z = at<uint16_t>(ws, p.z);
  da.wsplit = p.large ? at<void>(ws, p.wsplit) : nullptr;
  da.part = p.large ? nullptr : at<float>(ws, p.xpart);
  if (p.rd && !p.large) {  // V's rows join the projection, after the router's and A's
    da.w2 = delta_V;
    da.N2 = p.rd;
  }
  const int lN = da.N0 + da.N1 + da.N2;
  e = moe::launch_xproj(da, stream);
  if (e == hipSuccess && p.rd) {
    // U (V x): added to the logits (large batches), or written as one more
    // partial slice that the routing adds last (small batches)
    if (p.large)
      e = moe::launch_router_delta(at<float>(ws, p.vpart), 1, p.rd, T, p.rd, delta_U, E, logits, E, true, stream);
    else
      e = moe::launch_router_delta(da.part + da.N0 + da.N1, splits, lN, T, p.rd, delta_U, E,
                                   da.part + (int64_t)splits * T * lN, lN, false, stream);
  }
  if (e == hipSuccess) e = stage_mark(0, true, stream);
  if (e != hipSuccess) return device_fail(e, "xproj launch");

  moe::RouteArgs ra{};
  ra.logits = logits;
  ra.T = T;
  ra.E = E;
  ra.k = k;
  ra.S = S;
  ra.idx = idx;
  ra.w = w;
  ra.slot_rank = at<int32_t>(ws, p.rank);
  ra.block_cnt = at<int32_t>(ws, p.bcnt);
  ra.block_base = at<int32_t>(ws, p.bbase);
  ra.counts = counts;
  ra.offsets = offsets;
  ra.perm = perm;
  ra.items = at<moe::Item>(ws, p.items);
  ra.n_items = at<int32_t>(ws, p.nitems);
  ra.chunk = p.chunk;
  if (p.chunk2 != p.chunk) {
    ra.items2 = at<moe::Item>(ws, p.items2);
    ra.n_items2 = at<int32_t>(ws, p.nitems2);
    ra.chunk2 = p.chunk2;
  }
  if (!p.large) {  // the routing adds up the partials: the logits, and z for the combine
    ra.lpart = da.part;
    ra.lsplits = splits + (p.rd ? 1 : 0);
    ra.lN = lN;
    ra.z = da.N1 > 0 ? da.z : nullptr;
    ra.zr = da.N1;
  }
  e = stage_mark(1, false, stream);
  // route_out: the caller's expert kernel routes the batch itself (stage 1 stays empty)
  if (e == hipSuccess && !route_out) e = moe::launch_route(ra, p.max_items, stream);
  if (e == hipSuccess) e = stage_mark(1, true, stream);
  if (e != hipSuccess) return device_fail(e, "routing launch");
  if (route_out) *route_out = ra;
  return MOE_OK;
}

int32_t moe_route(const uint16_t* x, int64_t T, int32_t d, int32_t E, const uint16_t* router,
                  const uint16_t* delta, int32_t k, float* logits, int32_t* idx, float* w, int32_t* counts,
                  int32_t* offsets, int32_t* perm, void* ws, int64_t ws_bytes, void* stream) {
  try {
    int32_t rc = check_dims(T, d, E, k);
    if (rc) return rc;
    if (T == 0) return ok();
    if (!x || !router || !logits || !idx || !w || !counts || !offsets || !perm || !ws)
      return fail(MOE_E_ARG, "NULL pointer");
    if ((uintptr_t)ws % kAlign || (uintptr_t)x % 16) return fail(MOE_E_ARG, "workspace must be 256-byte and x 16-byte aligned");
    const Plan p = make_plan(T, d, E, 0, 128, k, 0);
    if (ws_bytes < p.route_end)
      return fail(MOE_E_SPACE, "workspace holds %lld bytes, %lld needed", (long long)ws_bytes, (long long)p.route_end);
    rc = route_impl(x, T, d, E, 0, router, delta, nullptr, nullptr, nullptr, 0, k, p, ws, (hipStream_t)stream,
                    logits, idx, w, counts, offsets, perm);
    if (rc) return rc;
    return ok();
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_route");
  }
}

int64_t moe_route_workspace_bytes_factored(int64_t n_tokens, int32_t d_model, int32_t n_experts, int32_t top_k,
                                           int32_t delta_rank) {
  if (n_tokens < 0 || n_experts < 1 || top_k < 1 || delta_rank < 1) return -1;
  return make_plan(n_tokens, d_model, n_experts, 0, 128, top_k, 0, delta_rank).route_end;
}

int32_t moe_route_factored(const uint16_t* x, int64_t T, int32_t d, int32_t E, const uint16_t* router,
                           const uint16_t* delta_U, const uint16_t* delta_V, int32_t rd, int32_t k, float* logits,
                           int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* perm, void* ws,
                           int64_t ws_bytes, void* stream) {
  try {
    int32_t rc = check_dims(T, d, E, k);
    if (rc) return rc;
    if (rd <= 0 || rd % 8 || rd > moe::kDeltaMaxRank)
      return fail(MOE_E_SHAPE, "delta_rank must be a positive multiple of 8, at most %d (got %d)",
                  moe::kDeltaMaxRank, (int)rd);
    if (T == 0) return ok();
    if (!x || !router || !delta_U || !delta_V || !logits || !idx || !w || !counts || !offsets || !perm || !ws)
      return fail(MOE_E_ARG, "NULL pointer");
    if ((uintptr_t)ws % kAlign || (uintptr_t)x % 16) return fail(MOE_E_ARG, "workspace must be 256-byte and x 16-byte aligned");
    if ((uintptr_t)delta_U % 16 || (uintptr_t)delta_V % 4)
      return fail(MOE_E_ARG, "delta_U must be 16-byte and delta_V 4-byte aligned");
    const Plan p = make_plan(T, d, E, 0, 128, k, 0, rd);
    if (ws_bytes < p.route_end)
      return fail(MOE_E_SPACE, "workspace holds %lld bytes, %lld needed", (long long)ws_bytes, (long long)p.route_end);
    rc = route_impl(x, T, d, E, 0, router, nullptr, nullptr, nullptr, nullptr, 0, k, p, ws, (hipStream_t)stream,
                    logits, idx, w, counts, offsets, perm, delta_U, delta_V);
    if (rc) return rc;
    return ok();
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_route_factored");
  }
}

// The forward pass with the router delta and the correction either dense fp16
// (delta, corr_A, corr_B) or ternary PQ2_0 containers (delta_q, corr_A_q,
// corr_B_q); the caller passes one form of each.
static int32_t forward_impl(const uint16_t* x, int64_t T, const uint16_t* router, const uint16_t* delta,
                            const uint8_t* delta_q, const moe_expert_banks* banks, const uint16_t* corr_A,
                            const uint8_t* corr_A_q, const uint16_t* corr_B, const uint8_t* corr_B_q, int32_t r,
                            int32_t k, uint16_t* y, void* ws, int64_t ws_bytes, void* stream,
                            const uint16_t* delta_U = nullptr, const uint16_t* delta_V = nullptr, int rd = 0) {
  {
    int32_t rc = check_banks(banks);
    if (rc) return rc;
    const int d = banks->d_model, f = banks->d_ff, E = banks->n_experts, S = banks->n_shared;
    rc = check_dims(T, d, E, k);
    if (rc) return rc;
    if (r < 0) return fail(MOE_E_ARG, "corr_rank must be >= 0 (got %d)", r);
    const bool has_A = corr_A || corr_A_q, has_B = corr_B || corr_B_q;
    if (has_A != has_B) return fail(MOE_E_ARG, "corr_A and corr_B must both be given or both be NULL");
    if (has_A && r == 0) return fail(MOE_E_ARG, "corr_rank is 0 but corr_A/corr_B are given");
    if (!has_A) r = 0;
    if (corr_A_q && r % 128)
      return fail(MOE_E_SHAPE, "a ternary corr_B needs corr_rank to be a multiple of 128 (got %d)", r);
    if ((uintptr_t)delta_q % 2 || (uintptr_t)corr_A_q % 2 || (uintptr_t)corr_B_q % 2)
      return fail(MOE_E_ARG, "ternary containers must be 2-byte aligned");
    if (r % 8) return fail(MOE_E_SHAPE, "corr_rank must be a multiple of 8 (got %d)", r);
    if (r > 4096) return fail(MOE_E_SHAPE, "corr_rank above 4096 is not supported (got %d)", r);
    if (rd) {
      if (rd < 0 || rd % 8 || rd > moe::kDeltaMaxRank)
        return fail(MOE_E_SHAPE, "delta_rank must be a positive multiple of 8, at most %d (got %d)",
                    moe::kDeltaMaxRank, rd);
      if (delta || delta_q) return fail(MOE_E_ARG, "give the router delta dense or as factors, not both");
    }
    if (T == 0) return ok();
    if (!x || !router || !y || !ws) return fail(MOE_E_ARG, "NULL pointer");
    if (rd && (!delta_U || !delta_V)) return fail(MOE_E_ARG, "NULL delta factor");
    if ((uintptr_t)delta_U % 16 || (uintptr_t)delta_V % 4)
      return fail(MOE_E_ARG, "delta_U must be 16-byte and delta_V 4-byte aligned");
    if (x == y) return fail(MOE_E_ARG, "y must not alias x");
    if ((uintptr_t)ws % kAlign) return fail(MOE_E_ARG, "workspace must be 256-byte aligned");
    if ((uintptr_t)x % 16 || (uintptr_t)y % 4) return fail(MOE_E_ARG, "x must be 16-byte and y 4-byte aligned");
    Plan p = make_plan(T, d, E, S, f, k, r, rd);
    if (ws_bytes < p.total)
      return fail(MOE_E_SPACE, "workspace holds %lld bytes, %lld needed", (long long)ws_bytes, (long long)p.total);
    bool any_ptq1 = false;
    for (int e = 0; e < E + S; ++e) any_ptq1 |= banks->formats_host[e] != MOE_PQ2_0;
    set_chunk(p, d, E, k, any_ptq1);
    const hipStream_t st = (hipStream_t)stream;
    // up to four tokens: the gate/up kernel routes the batch itself and the
    // down projection carries the combine (three launches instead of five)
    const bool tiny = !p.large && moe::tiny_path_fits(T, E, k, S, d, f);
    moe::RouteArgs ra{};

    rc = route_impl(x, T, d, E, S, router, delta, delta_q, corr_A, corr_A_q, r, k, p, ws, st,
                    at<float>(ws, p.logits), at<int32_t>(ws, p.idx), at<float>(ws, p.w),
                    at<int32_t>(ws, p.counts), at<int32_t>(ws, p.offsets), at<int32_t>(ws, p.perm), delta_U,
                    delta_V, tiny ? &ra : nullptr);
    if (rc) return rc;

    moe::ExpertArgs ea{};
    ea.banks = banks->banks;
    ea.offsets = banks->offsets;
    ea.formats = banks->formats;
    ea.d = d;
    ea.f = f;
    ea.E = E;
    ea.S = S;
    ea.k = k;
    ea.T = T;
    ea.Tk = T * k;
    ea.items = at<moe::Item>(ws, p.items);
    ea.n_items = at<int32_t>(ws, p.nitems);
    const bool two_lists = p.chunk2 != p.chunk;
    ea.down_items = two_lists ? at<moe::Item>(ws, p.items2) : ea.items;
    ea.down_n_items = two_lists ? at<int32_t>(ws, p.nitems2) : ea.n_items;
    ea.perm = at<int32_t>(ws, p.perm);
    ea.topk_w = at<float>(ws, p.w);
    ea.x = x;
    ea.h = at<uint16_t>(ws, p.h);
    ea.slots = at<uint16_t>(ws, p.slots);
    ea.chunk = p.chunk;
    ea.nmax = (int)std::min<int64_t>(T, ea.chunk);
    ea.fmt_mask = 0;
    for (int e = 0; e < E + S; ++e) ea.fmt_mask |= banks->formats_host[e] == MOE_PQ2_0 ? 1 : 2;

    moe::DenseArgs ca{};
    ca.act = at<uint16_t>(ws, p.z);
    ca.lda = r;
    ca.T = T;
    ca.K = r;
    ca.w0 = corr_B;
    ca.q0 = corr_B_q;
    ca.N0 = d;
    ca.slots = at<uint16_t>(ws, p.slots);
    ca.top_k = k;
    ca.n_shared = S;
    ca.y = y;
    ca.wsplit = p.large ? at<void>(ws, p.wsplit) : nullptr;
    if (tiny) {
      hipError_t e = moe::launch_tiny(ea, ra, ca, p.max_items, st, g_stage_events);
      if (e == hipSuccess) e = stage_mark(4, false, st);  // the combine is part of the down launch
      if (e == hipSuccess) e = stage_mark(4, true, st);
      if (e != hipSuccess) return device_fail(e, "expert launch");
      return ok();
    }
    hipError_t e = moe::launch_experts(ea, p.max_items, p.max_items2, st, g_stage_events);
    if (e != hipSuccess) return device_fail(e, "expert launch");
    e = stage_mark(4, false, st);
    if (e == hipSuccess) e = moe::launch_combine(ca, st);
    if (e == hipSuccess) e = stage_mark(4, true, st);
    if (e != hipSuccess) return device_fail(e, "combine launch");
    return ok();
  }
}

int32_t moe_ternary_forward(const uint16_t* x, int64_t T, const uint16_t* router, const uint16_t* delta,
                            const moe_expert_banks* banks, const uint16_t* corr_A, const uint16_t* corr_B,
                            int32_t r, int32_t k, uint16_t* y, void* ws, int64_t ws_bytes, void* stream) {
  try {
    return forward_impl(x, T, router, delta, nullptr, banks, corr_A, nullptr, corr_B, nullptr, r, k, y, ws,
                        ws_bytes, stream);
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_ternary_forward");
  }
}

int64_t moe_workspace_bytes_factored(const moe_expert_banks* banks, int64_t n_tokens, int32_t top_k,
                                     int32_t corr_rank, int32_t delta_rank) {
  if (!banks || n_tokens < 0 || top_k < 1 || corr_rank < 0 || delta_rank < 1) return -1;
  return make_plan(n_tokens, banks->d_model, banks->n_experts, banks->n_shared, banks->d_ff, top_k, corr_rank,
                   delta_rank)
      .total;
}

int32_t moe_ternary_forward_factored(const uint16_t* x, int64_t T, const uint16_t* router, const uint16_t* delta_U,
                                     const uint16_t* delta_V, int32_t delta_rank, const moe_expert_banks* banks,
                                     const uint16_t* corr_A, const uint16_t* corr_B, int32_t r, int32_t k, uint16_t* y,
                                     void* ws, int64_t ws_bytes, void* stream) {
  try {
    if (delta_rank <= 0) return fail(MOE_E_SHAPE, "delta_rank must be positive (got %d)", (int)delta_rank);
    return forward_impl(x, T, router, nullptr, nullptr, banks, corr_A, nullptr, corr_B, nullptr, r, k, y, ws,
                        ws_bytes, stream, delta_U, delta_V, delta_rank);
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_ternary_forward_factored");
  }
}

int32_t moe_ternary_forward_q(const uint16_t* x, int64_t T, const uint16_t* router, const uint8_t* delta_q,
                              const moe_expert_banks* banks, const uint8_t* corr_A_q, const uint8_t* corr_B_q,
                              int32_t r, int32_t k, uint16_t* y, void* ws, int64_t ws_bytes, void* stream) {
  try {
    return forward_impl(x, T, router, nullptr, delta_q, banks, nullptr, corr_A_q, nullptr, corr_B_q, r, k, y, ws,
                        ws_bytes, stream);
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_ternary_forward_q");
  }
}

// ------------------------------------------------------- no-allocation forward
// The workspace of moe_ternary_forward_noalloc: one array per device, loaded
// with the library's code object and held until the process ends.  In host
// code the name `scratch` is only a stand-in for the symbol: its device address
// comes from hipGetSymbolAddress, taken once per device on the first call made
// with that device current, and only that address reaches a kernel.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or NULL after setting the error.
void* device_scratch() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    device_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(MOE_E_DEVICE, "device %d is beyond the %d devices the scratch table covers", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      device_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

int32_t moe_ternary_forward_noalloc(const uint16_t* x, int64_t T, const uint16_t* router, const uint16_t* delta,
                                    const moe_expert_banks* banks, const uint16_t* corr_A, const uint16_t* corr_B,
                                    int32_t r, int32_t k, uint16_t* y, void* stream) {
  try {
    int32_t rc = check_banks(banks);
    if (rc) return rc;
    rc = check_dims(T, banks->d_model, banks->n_experts, k);
    if (rc) return rc;
    if (r < 0) return fail(MOE_E_ARG, "corr_rank must be >= 0 (got %d)", r);
    const int64_t need = make_plan(T, banks->d_model, banks->n_experts, banks->n_shared, banks->d_ff, k,
                                   (corr_A || corr_B) ? r : 0)
                             .total;
    if (need > (int64_t)MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_E_SPACE,
                  "%lld tokens need %lld bytes of workspace; the library's scratch holds %lld "
                  "(moe_ternary_forward takes a caller workspace of any size)",
                  (long long)T, (long long)need, (long long)MOE_NOALLOC_SCRATCH_BYTES);
    if (T == 0) return ok();
    void* ws = device_scratch();
    if (!ws) return MOE_E_DEVICE;
    return forward_impl(x, T, router, delta, nullptr, banks, corr_A, nullptr, corr_B, nullptr, r, k, y, ws,
                        (int64_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_ternary_forward_noalloc");
  }
}

}  // extern "C"
