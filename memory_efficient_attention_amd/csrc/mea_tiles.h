// Staging of key/value tiles from HBM into LDS.
//
// A tile is BN consecutive keys of one sequence and one key/value head.
//   K is stored row-major [BN][D + 8] (16-bit elements; the 8-element pad
//     makes the 16-byte fragment reads of the Q.K^T product bank-conflict free);
//   V is stored transposed, V^T [D][BN + 8], because the P.V product needs 8
//     consecutive keys of one feature per lane.  The transpose happens in
//     registers: each thread loads 4 consecutive keys x 8 features (four
//     16-byte loads) and writes 8 runs of 4 keys (8-byte LDS writes).
// Keys at or past the end of the sequence are zero-filled, so a tile never
// reads outside its sequence's rows.
#pragma once

#include "mea_common.h"

namespace mea {

template <int D, int BN>
struct TileLayout {
  static constexpr int kStride = D + 8;         // elements per K row in LDS
  static constexpr int vStride = BN + 8;        // elements per V^T row in LDS
  static constexpr int kElems = BN * kStride;
  static constexpr int vElems = D * vStride;
  static constexpr int bufElems = kElems + vElems;
  static constexpr int bufBytes = bufElems * 2;
};

// Per-thread registers holding one tile in flight between HBM and LDS.
template <int D, int BN, int NT, bool CVT_V>
struct TileStager {
  static constexpr int CH = D / 8;                          // 16-byte chunks per row
  static constexpr int K_JOBS = BN * CH;                    // 16-byte K pieces per tile
  static constexpr int K_LOADS = (K_JOBS + NT - 1) / NT;
  static constexpr int QUADS = BN / 4;                      // runs of 4 keys
  static constexpr int V_JOBS = QUADS * CH;                 // (4 keys x 8 features) pieces
  static constexpr int V_PASSES = (V_JOBS + NT - 1) / NT;
  using L = TileLayout<D, BN>;

  u32x4 kr[K_LOADS];
  u32x4 vr[V_PASSES][4];

  // Issue the global loads of the tile starting at key j0 of a sequence whose
  // keys begin at row `row0` of the packed k/v tensors and number `len`.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                       int row0, int len, int j0, int head, int Hkv, int tid) {
    const size_t rs = (size_t)Hkv * D;                      // elements between key rows
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int job = tid + i * NT;
      const int c = job % CH, r = job / CH;
      const int j = j0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if ((K_JOBS % NT == 0 || job < K_JOBS) && j < len)
        x = *(const u32x4*)(k + (size_t)(row0 + j) * rs + (size_t)head * D + c * 8);
      kr[i] = x;
    }
#pragma unroll
    for (int p = 0; p < V_PASSES; ++p) {
      const int job = tid + p * NT;
      const int kq = job % QUADS, c = job / QUADS;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * kq + i;
        u32x4 x = {0u, 0u, 0u, 0u};
        if ((V_JOBS % NT == 0 || job < V_JOBS) && j < len)
          x = *(const u32x4*)(v + (size_t)(row0 + j) * rs + (size_t)head * D + c * 8);
        vr[p][i] = x;
      }
    }
  }

  // Write the registers into one LDS buffer (K row-major, V transposed and,
  // for bfloat16 inputs, re-encoded as IEEE half).
  __device__ __forceinline__ void store(uint16_t* __restrict__ buf, int tid) const {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int job = tid + i * NT;
      if (K_JOBS % NT == 0 || job < K_JOBS) {
        const int c = job % CH, r = job / CH;
        *(u32x4*)(buf + r * L::kStride + c * 8) = kr[i];
      }
    }
    uint16_t* vt = buf + L::kElems;
#pragma unroll
    for (int p = 0; p < V_PASSES; ++p) {
      const int job = tid + p * NT;
      if (V_JOBS % NT == 0 || job < V_JOBS) {
        const int kq = job % QUADS, c = job / QUADS;
        u32x4 a0 = vr[p][0], a1 = vr[p][1], a2 = vr[p][2], a3 = vr[p][3];
        if constexpr (CVT_V) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            a0[w] = bf16x2_to_f16x2(a0[w]);
            a1[w] = bf16x2_to_f16x2(a1[w]);
            a2[w] = bf16x2_to_f16x2(a2[w]);
            a3[w] = bf16x2_to_f16x2(a3[w]);
          }
        }
        // word w of a_i holds features 2w (low) and 2w+1 (high) of key i
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          u32x2 even, odd;
          even[0] = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);
          even[1] = __builtin_amdgcn_perm(a3[w], a2[w], 0x05040100u);
          odd[0] = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);
          odd[1] = __builtin_amdgcn_perm(a3[w], a2[w], 0x07060302u);
          *(u32x2*)(vt + (8 * c + 2 * w) * L::vStride + 4 * kq) = even;
          *(u32x2*)(vt + (8 * c + 2 * w + 1) * L::vStride + 4 * kq) = odd;
        }
      }
    }
  }
};

}  // namespace mea
