// The router delta given as two low-rank factors (FlashNext card, "Weight
// Representation": the router deltas ship as rank-512 F16 factors U [E x rd]
// and V [rd x d]): the logits gain U (V x).  V x is an x-projection of its own;
// this kernel adds up its fp32 slices and applies U.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kDeltaMaxRank = 1024;  // rd bound: a block keeps 8 tokens' V x in shared memory

// dst[t * ldd + e] for e < E: (dst +) sum_c U[e, c] v[t, c], where v[t, c] is the
// sum in slice order of the fp32 slices vpart[s * T * ldv + t * ldv + c],
// s < vsplits <= 8 (ldv >= rd: V x may be columns of a wider partial row).
// add == false: also writes 0 to columns E .. ldd - 1 of each row (an extra
// partial slice, whose other columns must add nothing).
// Requires rd % 8 == 0, 1 <= rd <= kDeltaMaxRank, U 16-byte aligned.
hipError_t launch_router_delta(const float* vpart, int vsplits, int ldv, int64_t T, int rd, const uint16_t* U,
                               int E, float* dst, int ldd, bool add, hipStream_t stream);

}  // namespace moe
