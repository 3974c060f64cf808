// Internal launch interface between the C ABI (mea_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "mea_common.h"

namespace mea {

// Prefill: workgroups of 4 waves; a wave owns 32 consecutive query rows of one
// head, so a workgroup covers 32 * (4 / heads_per_wg) tokens of heads_per_wg
// query heads that share one key/value head.
constexpr int kPfWaves = 4;
constexpr int kPfBN = 64;          // keys per LDS tile
// Decode: workgroups of 4 waves, each streaming its own 32-key blocks of a chunk.
constexpr int kDcBN = 128;        // chunk granularity: 4 waves x 32-key blocks
constexpr int kDcHeadsPerWg = 16;  // query heads of one group served per workgroup

hipError_t launch_prefill(const FwdArgs& a, int D, bool bf16, bool causal, bool alibi,
                          int max_seqlen_k, hipStream_t stream);
hipError_t launch_decode(const FwdArgs& a, int D, bool bf16, bool alibi, hipStream_t stream);

}  // namespace mea
