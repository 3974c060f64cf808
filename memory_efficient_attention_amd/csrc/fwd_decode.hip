// Split-KV attention forward for one query per sequence (the decode case).
//
// Partial kernel: a workgroup takes one sequence, one key/value head g (and up
// to 32 of its query heads) and one chunk of the sequence's keys.  It streams
// that chunk's K/V from HBM exactly once, in 128-key tiles staged through LDS,
// and serves all query heads of the group from each tile: the heads are the
// 32 columns of the matrix-core products, so GQA's sharing turns directly
// into fewer HBM bytes.  Each of the 4 waves takes one 32-key block of a tile
// with its own online-softmax state; the waves merge in LDS at the end and
// write one normalised float32 partial output and its log-sum-exp per head.
//
// Combine kernel: per (sequence, query head) the chunk partials are merged
// by their log-sum-exps: lse = log sum_c exp(lse_c), out = sum_c exp(lse_c -
// lse) o_c, then rounded to the output dtype.
#include "mea_common.h"
#include "mea_launch.h"
#include "mea_tiles.h"

namespace mea {

template <int D, bool BF16, bool ALIBI>
__global__ __launch_bounds__(256) void fwd_decode_partial_kernel(FwdArgs a) {
  using L = TileLayout<D, kDcBN>;
  using Stager = TileStager<D, kDcBN, 256, BF16>;
  constexpr int kRedStride = D + 1;  // floats per query row in the merge buffer
  static_assert(4 * 32 * kRedStride * 4 + 2 * 4 * 32 * 4 <= L::bufBytes, "merge buffer");
  __shared__ __attribute__((aligned(16))) uint16_t smem[L::bufElems];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int g = blockIdx.z / a.head_slices, hs = blockIdx.z % a.head_slices;

  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  const int sk0 = a.seqstart_k[b], Lk = a.seqstart_k[b + 1] - sk0;
  const int c0 = chunk * a.chunk_keys;
  if (Lq == 0 || c0 >= Lk) return;
  const int c1 = min(Lk, c0 + a.chunk_keys);
  const int qpos = Lk - 1;  // the single query is the sequence's last position

  const int hl = hs * kDcHeadsPerWg + l32;  // query head within the group (= MFMA column)
  const bool col_valid = hl < a.group;
  const int head = g * a.group + hl;

  u32x4 qf[D / 16];
  {
    const uint16_t* qrow = a.q + ((size_t)sq0 * a.Hq + head) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (col_valid) x = *(const u32x4*)(qrow + 16 * s);
      qf[s] = x;
    }
  }
  const float c = a.scale_log2;
  float slope2 = 0.f;
  if constexpr (ALIBI) slope2 = col_valid ? a.slopes[head] * kLog2e : 0.f;

  f32x16 o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) o[d] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  Stager st;
  st.load(a.k, a.v, sk0, c1, c0, g, a.Hkv, tid);
  for (int j0 = c0; j0 < c1; j0 += kDcBN) {
    __syncthreads();
    st.store(smem, tid);
    __syncthreads();
    if (j0 + kDcBN < c1) st.load(a.k, a.v, sk0, c1, j0 + kDcBN, g, a.Hkv, tid);

    const int jw = j0 + 32 * wave;  // first key of this wave's block
    if (jw < c1) {
      f32x16 s = f32x16{};
      const uint16_t* kp = smem + (32 * wave + key_of_row(l32)) * L::kStride + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) s = mfma_32x32x16<BF16>(*(const u32x4*)(kp + 16 * ks), qf[ks], s);

      const bool need_mask = jw + 32 > c1;
      const int jlane = jw + 8 * hi;
      const float sb = slope2 * (float)(jlane - qpos);
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = key_of_reg(r, 0);
        float x;
        if constexpr (ALIBI) x = __builtin_fmaf(s[r], c, __builtin_fmaf(slope2, (float)jl, sb));
        else x = s[r] * c;
        if (need_mask && jlane + jl >= c1) x = kNegInf;
        s[r] = x;
        mx = __builtin_fmaxf(mx, x);
      }
      mx = halfwave_max(mx);
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float lsum = 0.f;
      u32x4 pf[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(s[r] - m_use);
        const float p1 = fast_exp2(s[r + 1] - m_use);
        lsum += p0 + p1;
        pf[r / 8][(r % 8) / 2] = pack_f16x2(p0, p1);
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < D / 32; ++d) o[d] *= alpha;
      const uint16_t* Vt = smem + L::kElems;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
          const u32x4 vf = *(const u32x4*)(Vt + (32 * d + l32) * L::vStride + 32 * wave + 16 * ch + 8 * hi);
          o[d] = mfma_32x32x16<false>(vf, pf[ch], o[d]);
        }
      }
    }
  }

  // ---- merge the 4 waves' partial states in LDS
  const float l_tot = halfwave_sum(l_run);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [4][32][kRedStride]
  float* mred = red + 4 * 32 * kRedStride;       // [4][32]
  float* lred = mred + 4 * 32;                   // [4][32]
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 32 + l32) * kRedStride + 32 * d + acc_row(r, hi)] = o[d][r];
  if (hi == 0) {
    mred[wave * 32 + l32] = m_run;
    lred[wave * 32 + l32] = l_tot;
  }
  __syncthreads();

  const int q = tid >> 3, part = tid & 7;  // 32 columns x 8 parts of D/8 features
  if (hs * kDcHeadsPerWg + q >= a.group) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = __builtin_fmaxf(M, mred[w * 32 + q]);
  float wgt[4], Ls = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = mred[w * 32 + q];
    wgt[w] = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
    Ls += wgt[w] * lred[w * 32 + q];
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  const int hq = g * a.group + hs * kDcHeadsPerWg + q;
  const size_t prow = ((size_t)b * a.max_chunks + chunk) * a.Hq + hq;
  float* dst = a.ws_o + prow * D + part * (D / 8);
#pragma unroll
  for (int e = 0; e < D / 8; ++e) {
    const int d = part * (D / 8) + e;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += wgt[w] * red[(w * 32 + q) * kRedStride + d];
    dst[e] = acc * inv;
  }
  if (part == 0) a.ws_lse[prow] = Ls > 0.f ? M + fast_log2(Ls) : kNegInf;
}

template <int D, bool BF16>
__global__ __launch_bounds__(D) void fwd_decode_combine_kernel(FwdArgs a) {
  const int b = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  if (Lq == 0) return;
  const int Lk = a.seqstart_k[b + 1] - a.seqstart_k[b];
  const int nch = (Lk + a.chunk_keys - 1) / a.chunk_keys;
  const size_t row0 = (size_t)b * a.max_chunks * a.Hq + h;  // partial row of chunk 0
  float M = kNegInf;
  for (int ch = 0; ch < nch; ++ch) M = __builtin_fmaxf(M, a.ws_lse[row0 + (size_t)ch * a.Hq]);
  float S = 0.f, acc = 0.f;
  if (M != kNegInf) {
    for (int ch = 0; ch < nch; ++ch) {
      const float lc = a.ws_lse[row0 + (size_t)ch * a.Hq];
      const float w = (lc == kNegInf) ? 0.f : fast_exp2(lc - M);
      S += w;
      acc += w * a.ws_o[(row0 + (size_t)ch * a.Hq) * D + d];
    }
  }
  const float val = S > 0.f ? acc / S : 0.f;
  uint16_t bits;
  if constexpr (BF16) bits = __builtin_bit_cast(uint16_t, (__bf16)val);
  else bits = __builtin_bit_cast(uint16_t, (_Float16)val);
  a.out[((size_t)sq0 * a.Hq + h) * D + d] = bits;
  if (d == 0 && a.lse != nullptr)
    a.lse[(size_t)h * a.total_q + sq0] = S > 0.f ? (M + fast_log2(S)) * kLn2 : kNegInf;
}

template <int D, bool BF16>
static hipError_t launch_decode_d(const FwdArgs& a, bool alibi, hipStream_t stream) {
  if (a.max_chunks > 0) {
    const dim3 grid(a.max_chunks, a.num_seqs, a.Hkv * a.head_slices);
    if (alibi) hipLaunchKernelGGL((fwd_decode_partial_kernel<D, BF16, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((fwd_decode_partial_kernel<D, BF16, false>), grid, dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((fwd_decode_combine_kernel<D, BF16>), dim3(a.num_seqs, a.Hq), dim3(D), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const FwdArgs& a, int D, bool bf16, bool alibi, hipStream_t stream) {
  if (D == 64) return bf16 ? launch_decode_d<64, true>(a, alibi, stream) : launch_decode_d<64, false>(a, alibi, stream);
  return bf16 ? launch_decode_d<128, true>(a, alibi, stream) : launch_decode_d<128, false>(a, alibi, stream);
}

}  // namespace mea
