// The k=1 draft head that ships beside the 35B-A3B release: fc1, gelu, fc2 in
// fp16 over the model's hidden state and the next token's embedding
// (Scion-35B-A3B card, "Shipped Components": a 50 MB fp16 head; "Highlights":
// it drafts the next token from the model's own hidden state).
//
//   x = [hidden ; embedding]        (hidden first)
//   g = gelu(W1 x + b1)             rounded to bf16, gelu(v) = v (1 + erf(v / sqrt 2)) / 2
//   y = W2 g + b2                   rounded to bf16
//
// Both products are the x-projection's dense kernels: up to 256 tokens the
// split kernel (fp32 partials over at most eight K slices, every weight row
// streamed once and spread over the chip), beyond that the tiled matrix-core
// GEMM.  A small kernel then adds the slices in order, the bias and the gelu;
// another one first concatenates the two inputs into the workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kFinishThreads = 256;

// out[t, n] = act(sum over slices s of part[s][t][n] + bias[n]) in bf16, the
// slices added in order.  part: fp32 [splits][T][N].
template <bool GELU>
__global__ __launch_bounds__(kFinishThreads) void head_finish_kernel(const float* __restrict__ part, int splits,
                                                                     int64_t T, int N,
                                                                     const uint16_t* __restrict__ bias,
                                                                     uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kFinishThreads + threadIdx.x;
  if (i >= T * N) return;
  const int n = (int)(i % N);
  float v = part[i];
  for (int s = 1; s < splits; ++s) v += part[(int64_t)s * T * N + i];
  if (bias) v += f16_to_f32(bias[n]);
  if (GELU) v = 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
  out[i] = (uint16_t)f32_to_bf16(v);
}

// x = [hidden ; emb]: 16-byte pieces, T rows of 2h values (h % 8 == 0).
__global__ __launch_bounds__(kFinishThreads) void head_concat_kernel(const u32x4* __restrict__ hidden,
                                                                     const u32x4* __restrict__ emb, int64_t T,
                                                                     int h8, u32x4* __restrict__ xc) {
  const int64_t i = (int64_t)blockIdx.x * kFinishThreads + threadIdx.x;
  if (i >= T * 2 * h8) return;
  const int64_t t = i / (2 * h8);
  const int c = (int)(i - t * 2 * h8);
  xc[i] = c < h8 ? hidden[t * h8 + c] : emb[t * h8 + c - h8];
}

template <bool GELU>
hipError_t launch_finish(const float* part, int splits, int64_t T, int N, const uint16_t* bias, uint16_t* out,
                         hipStream_t stream) {
  const int64_t n = T * N;
  head_finish_kernel<GELU><<<(unsigned)((n + kFinishThreads - 1) / kFinishThreads), kFinishThreads, 0, stream>>>(
      part, splits, T, N, bias, out);
  return hipGetLastError();
}

int64_t up256(int64_t v) { return (v + 255) / 256 * 256; }

}  // namespace

hipError_t launch_fold_bf16(const float* part, int splits, int64_t T, int N, uint16_t* out, hipStream_t stream) {
  return launch_finish<false>(part, splits, T, N, nullptr, out, stream);
}

HeadPlan head_plan(int64_t T, int h, int m) {
  HeadPlan p{};
  p.large = T > kGroupMaxT;
  int64_t o = 0;
  p.xc = o; o += up256(T * 2 * h * 2);
  p.g = o; o += up256(T * (int64_t)m * 2);
  const int s1 = p.large ? 1 : xproj_split(2 * h).splits, s2 = p.large ? 1 : xproj_split(m).splits;
  p.part = o; o += up256(std::max((int64_t)s1 * T * m, (int64_t)s2 * T * h) * 4);
  p.wsplit = o;
  if (p.large) o += up256(std::max(dense_split_bytes(m, 2 * h), dense_split_bytes(h, m)));
  p.total = o;
  return p;
}

hipError_t launch_head(const HeadArgs& a, char* ws, hipStream_t stream, void** stage_events) {
  const HeadPlan p = head_plan(a.T, a.h, a.m);
  const int64_t T = a.T;
  const int h = a.h, m = a.m;
  uint16_t* xc = (uint16_t*)(ws + p.xc);
  uint16_t* g = (uint16_t*)(ws + p.g);
  float* part = (float*)(ws + p.part);
  auto mark = [&](int i) -> hipError_t {
    return stage_events && stage_events[i] ? hipEventRecord((hipEvent_t)stage_events[i], stream) : hipSuccess;
  };
  // x = [hidden ; embedding], rows of 2h
  const int64_t pieces = T * 2 * (h / 8);
  head_concat_kernel<<<(unsigned)((pieces + kFinishThreads - 1) / kFinishThreads), kFinishThreads, 0, stream>>>(
      (const u32x4*)a.hidden, (const u32x4*)a.emb, T, h / 8, (u32x4*)xc);
  hipError_t e = hipGetLastError();
  for (int layer = 0; layer < 2 && e == hipSuccess; ++layer) {
    DenseArgs d{};
    d.act = layer == 0 ? xc : g;
    d.lda = layer == 0 ? 2 * h : m;
    d.T = T;
    d.K = layer == 0 ? 2 * h : m;
    d.w0 = layer == 0 ? a.w1 : a.w2;
    d.N0 = layer == 0 ? m : h;
    d.logits = part;  // the tiled path writes the whole fp32 product here
    d.wsplit = p.large ? ws + p.wsplit : nullptr;
    d.part = p.large ? nullptr : part;
    d.staged = true;
    e = mark(2 * layer);
    if (e == hipSuccess) e = launch_xproj(d, stream);
    if (e == hipSuccess) e = mark(2 * layer + 1);
    const int splits = p.large ? 1 : xproj_split(d.K).splits;
    if (e == hipSuccess)
      e = layer == 0 ? launch_finish<true>(part, splits, T, m, a.b1, g, stream)
                     : launch_finish<false>(part, splits, T, h, a.b2, a.y, stream);
  }
  return e;
}

}  // namespace moe
