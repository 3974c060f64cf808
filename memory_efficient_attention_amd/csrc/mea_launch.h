// Internal launch interface between the C ABI (mea_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "mea_common.h"

namespace mea {

// Prefill: workgroups of two groups of 4 waves; a wave owns 32 consecutive
// query rows of one head, so a group covers 32 * (4 / heads_per_wg) tokens of
// heads_per_wg query heads that share one key/value head, and the second
// group the next as many tokens.
constexpr int kPfGroupWaves = 4;
constexpr int kPfGroups = 2;
constexpr int kPfWaves = kPfGroupWaves * kPfGroups;
constexpr int kPfBN = 64;          // keys per LDS tile
// Decode: workgroups of 8 waves (one per CU); nh = gcd(Hkv, 4) key/value heads
// per workgroup (gcd(Hkv, 8) for fp8 K/V when the default pieces are at least
// kDcFp8WidePiece keys), the 8 / nh waves of a head each streaming every
// (8 / nh)-th block of that head's part of a piece of the concatenated key axis.
constexpr int kDcWaves = 8;         // decode workgroup: 8 waves, one workgroup per CU
constexpr int kDcKvPerWgMax = 4;      // key/value heads per decode workgroup: gcd(Hkv, 4)
constexpr int kDcKvPerWgMaxFp8 = 8;   // fp8 K/V on long pieces: gcd(Hkv, 8)
constexpr int kDcFp8WidePiece = 2048; // shortest default piece on which fp8 takes gcd(Hkv, 8)
constexpr int kDcPieceAlign = 32;    // piece lengths are multiples of one wave block
constexpr int kDcMinPiece = 128;     // shortest default piece
constexpr int kDcTargetWgs = 256;    // default: one round of one workgroup per CU on 256 CUs
constexpr int kDcHeadsPerWg = 16;    // query heads of one group served per workgroup

// Backward: workgroups of 8 waves (two groups of 4).  dK/dV: a wave owns 32
// keys of one key/value head (128 keys per workgroup, each owned by one wave
// of each group) and its group takes one 32-row half of every 64-row query
// tile; dQ: a wave owns 32 query rows of one head and walks 64-key tiles.
constexpr int kBwWaves = 8;
constexpr int kBwGroupWaves = 4;
constexpr int kBwKeys = 32 * kBwGroupWaves;  // keys per dK/dV workgroup
constexpr int kBwRows = 64;                  // query rows per dK/dV stage
constexpr int kBwKeyTile = 64;               // keys per dQ stage

hipError_t launch_prefill(const FwdArgs& a, int D, bool bf16, bool causal, bool alibi,
                          int max_seqlen_k, hipStream_t stream);
hipError_t launch_prefill_fp8(const FwdArgs& a, bool out_bf16, bool causal, bool alibi, int max_seqlen_k,
                              hipStream_t stream);
hipError_t launch_decode(const FwdArgs& a, int D, bool bf16, bool alibi, hipStream_t stream);
hipError_t launch_decode_fp8(const FwdArgs& a, bool out_bf16, bool alibi, hipStream_t stream);
hipError_t launch_backward(const BwdArgs& a, int D, bool bf16, bool causal, bool alibi, hipStream_t stream);
hipError_t launch_swiglu_ffn(const void* x, const void* w_gate, const void* w_up, const void* w_down, void* hidden,
                             void* out, int tokens, int d_model, int d_ff, bool bf16, hipStream_t stream);

}  // namespace mea
