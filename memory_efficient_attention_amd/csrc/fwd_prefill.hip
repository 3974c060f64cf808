// Fused attention forward for packed sequences with more than one query per
// sequence (the prefill case), on the gfx950 matrix cores.
//
// Work decomposition: a workgroup takes one sequence, one key/value head g and
// one tile of query tokens, and serves every query head of g's group that it
// covers (grouped-query attention: the K/V tile staged in LDS is read by all
// of them).  Each wave owns 32 query rows (32 consecutive tokens of one head):
//   S^T = K Q^T      32 keys x 32 queries per 32x32x16 product, Q kept in registers
//   online softmax   per query row = per lane, in float32, in log2 units
//   O^T += V^T P^T   32 features x 32 queries per product, P re-used from S^T's
//                    registers without any data movement
// The causal mask and the end of a sequence only cost element tests on the
// tiles that straddle them; tiles entirely above the diagonal are never
// loaded, and a wave whose rows are all finished skips its products.
#include "mea_common.h"
#include "mea_launch.h"
#include "mea_tiles.h"

namespace mea {

template <int D, bool BF16, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(256) void fwd_prefill_kernel(FwdArgs a) {
  using L = TileLayout<D, kPfBN>;
  using Stager = TileStager<D, kPfBN, 256, BF16>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::bufElems];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;

  const int b = blockIdx.y;
  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  const int sk0 = a.seqstart_k[b], Lk = a.seqstart_k[b + 1] - sk0;
  const int tc = kPfWaves / a.heads_per_wg;  // 32-token chunks per workgroup
  const int BT = 32 * tc;
  const int ntiles = (Lq + BT - 1) / BT;
  if ((int)blockIdx.z >= ntiles) return;
  const int t0 = (ntiles - 1 - (int)blockIdx.z) * BT;  // longest causal tiles launch first
  const int off = Lk - Lq;                              // query row r sits at key position r + off

  const int g = blockIdx.x / a.head_slices;
  const int hs = blockIdx.x % a.head_slices;
  const int hw = wave % a.heads_per_wg, tw = wave / a.heads_per_wg;
  const int head = g * a.group + hs * a.heads_per_wg + hw;
  const int tok0 = t0 + 32 * tw;  // first query row of this wave
  const int my_tok = tok0 + l32;  // this lane's query row
  const bool row_valid = my_tok < Lq;

  int kv_end = Lk, wave_kv_end = Lk;
  if constexpr (CAUSAL) {
    kv_end = min(Lk, min(t0 + BT, Lq) + off);
    wave_kv_end = min(Lk, min(tok0 + 32, Lq) + off);
  }
  if (tok0 >= Lq) wave_kv_end = 0;
  const int nkt = kv_end > 0 ? (kv_end + kPfBN - 1) / kPfBN : 0;

  // Q^T operand: lane holds features 16*s + 8*hi .. +7 of its row, s = 0 .. D/16-1
  u32x4 qf[D / 16];
  {
    const uint16_t* qrow = a.q + ((size_t)(sq0 + my_tok) * a.Hq + head) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_valid) x = *(const u32x4*)(qrow + 16 * s);
      qf[s] = x;
    }
  }
  const float c = a.scale_log2;
  float slope2 = 0.f;
  if constexpr (ALIBI) slope2 = a.slopes[head] * kLog2e;

  f32x16 o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) o[d] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  Stager st;
  if (nkt > 0) {
    st.load(a.k, a.v, sk0, Lk, 0, g, a.Hkv, tid);
    st.store(smem, tid);
    if (nkt > 1) st.load(a.k, a.v, sk0, Lk, kPfBN, g, a.Hkv, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int j0 = kt * kPfBN;
    const uint16_t* Kb = smem + (kt & 1) * L::bufElems;
    const uint16_t* Vt = Kb + L::kElems;
    if (j0 < wave_kv_end) {
      // ---- S^T = K Q^T (two 32-key blocks)
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* kp = Kb + (32 * kb + key_of_row(l32)) * L::kStride + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
          s[kb] = mfma_32x32x16<BF16>(*(const u32x4*)(kp + 16 * ks), qf[ks], s[kb]);
      }
      // ---- scale, ALiBi, masks (log2 units)
      const bool need_mask = (j0 + kPfBN > Lk) || (CAUSAL && j0 + kPfBN - 1 > tok0 + off);
      const int jlane = j0 + 8 * hi;         // key of register 0 in block 0
      const int qpos = my_tok + off;         // key position of this query row
      const float base = (float)(jlane - qpos);
      const float sb = slope2 * base;
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = 32 * kb + key_of_reg(r, 0);
          float x;
          if constexpr (ALIBI) {
            if constexpr (CAUSAL) {
              x = __builtin_fmaf(s[kb][r], c, __builtin_fmaf(slope2, (float)jl, sb));
            } else {
              x = __builtin_fmaf(s[kb][r], c, -slope2 * __builtin_fabsf(base + (float)jl));
            }
          } else {
            x = s[kb][r] * c;
          }
          if (need_mask) {
            const int j = jlane + jl;
            if (j >= Lk || (CAUSAL && j > qpos)) x = kNegInf;
          }
          s[kb][r] = x;
          mx = __builtin_fmaxf(mx, x);
        }
      }
      // ---- online softmax
      mx = halfwave_max(mx);
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float lsum = 0.f;
      u32x4 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(s[kb][r] - m_use);
          const float p1 = fast_exp2(s[kb][r + 1] - m_use);
          lsum += p0 + p1;
          pf[2 * kb + r / 8][(r % 8) / 2] = pack_f16x2(p0, p1);
        }
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < D / 32; ++d) o[d] *= alpha;
      // ---- O^T += V^T P^T (four 16-key chunks)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
          const u32x4 vf = *(const u32x4*)(Vt + (32 * d + l32) * L::vStride + 16 * ch + 8 * hi);
          o[d] = mfma_32x32x16<false>(vf, pf[ch], o[d]);
        }
      }
    }
    if (kt + 1 < nkt) {
      st.store(smem + ((kt + 1) & 1) * L::bufElems, tid);
      if (kt + 2 < nkt) st.load(a.k, a.v, sk0, Lk, (kt + 2) * kPfBN, g, a.Hkv, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, round, store out and lse
  const float l_tot = halfwave_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_valid) {
    uint16_t* orow = a.out + ((size_t)(sq0 + my_tok) * a.Hq + head) * D + 4 * hi;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_out_x2<BF16>(o[d][4 * r4] * inv, o[d][4 * r4 + 1] * inv);
        w[1] = pack_out_x2<BF16>(o[d][4 * r4 + 2] * inv, o[d][4 * r4 + 3] * inv);
        *(u32x2*)(orow + 32 * d + 8 * r4) = w;
      }
    }
    if (a.lse != nullptr && hi == 0)
      a.lse[(size_t)head * a.total_q + sq0 + my_tok] =
          l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

template <int D, bool BF16>
static hipError_t launch_prefill_d(const FwdArgs& a, bool causal, bool alibi, dim3 grid,
                                   hipStream_t stream) {
  const dim3 block(256);
  if (causal) {
    if (alibi) hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, true, false>), grid, block, 0, stream, a);
  } else {
    if (alibi) hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const FwdArgs& a, int D, bool bf16, bool causal, bool alibi,
                          int max_seqlen_q, hipStream_t stream) {
  const int bt = 32 * (kPfWaves / a.heads_per_wg);
  const dim3 grid(a.Hkv * a.head_slices, a.num_seqs, (max_seqlen_q + bt - 1) / bt);
  if (D == 64) {
    return bf16 ? launch_prefill_d<64, true>(a, causal, alibi, grid, stream)
                : launch_prefill_d<64, false>(a, causal, alibi, grid, stream);
  }
  return bf16 ? launch_prefill_d<128, true>(a, causal, alibi, grid, stream)
              : launch_prefill_d<128, false>(a, causal, alibi, grid, stream);
}

}  // namespace mea
