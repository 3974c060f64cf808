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
// Key tiles run from the causal diagonal backwards, so the largest scores (and,
// with ALiBi, the smallest distance penalties) come first and the running
// maximum rarely has to move; O is rescaled only when some row's maximum
// grows by more than 2^8.  The causal mask and the end of a sequence cost
// element tests only on the tiles that straddle them; tiles entirely above
// the diagonal are never loaded.
//
// Staging: K tiles go HBM -> LDS directly (buffer loads with the LDS
// destination, no registers); V tiles go through registers, where they are
// transposed (and, for bfloat16 inputs, re-encoded as IEEE half) on the way
// into LDS.  Both use buffer resources bounded by the sequence's rows, so a
// tile that runs past the sequence's end reads zeros instead of neighbours.
//
// Grid: one linear index, remapped so that the 8 XCDs each take a contiguous
// run of (head slice, sequence, tile) work items: the workgroups working on
// one sequence's K/V at the same time share one XCD's L2.
#include "mea_common.h"
#include "mea_launch.h"

namespace mea {

namespace {

constexpr int kThreads = 256;
constexpr float kRescaleThreshold = 8.f;  // log2 units: p may reach 2^8 before O is rescaled

template <int D>
struct PfLayout {
  static constexpr int BN = kPfBN;                    // keys per tile
  static constexpr int kBytes = BN * D * 2;           // K rows, 16-byte chunks XOR-swizzled
  static constexpr int vStride = BN + 8;              // elements per V^T row (padded)
  static constexpr int vBytes = D * vStride * 2;
  static constexpr int bufBytes = kBytes + vBytes;
  static constexpr int chunks = D / 8;                // 16-byte chunks per K row
  static constexpr int rowsPerKB = 1024 / (D * 2);    // K rows per 1 KB direct-load block
  static constexpr int kLoads = kBytes / (kThreads * 16);
};

// Position of 16-byte chunk c of K row r inside the row: rows that 16 lanes
// read together land on 16 different bank groups.
template <int D>
__device__ __forceinline__ int k_pos(int r, int c) {
  if constexpr (D == 128) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace

template <int D, bool BF16, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(kThreads, 2) void fwd_prefill_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses buffer-resource types that exist only for the GPU target
  using L = PfLayout<D>;
  constexpr int BN = L::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * L::bufBytes];

  // ---- work item: XCD-aware remap of the linear workgroup index
  const int per_xcd = (int)gridDim.x >> 3;
  const int w = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
  if (w >= a.pf_items) return;
  const int t_rev = w % a.pf_max_tiles;
  const int rest = w / a.pf_max_tiles;
  const int b = rest % a.num_seqs;
  const int hslice = rest / a.num_seqs;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  const int sk0 = a.seqstart_k[b], Lk = a.seqstart_k[b + 1] - sk0;
  const int tc = kPfWaves / a.heads_per_wg;   // 32-token chunks per workgroup
  const int BT = 32 * tc;
  const int ntiles = (Lq + BT - 1) / BT;
  if (t_rev >= ntiles) return;
  const int t0 = (ntiles - 1 - t_rev) * BT;    // longest causal tiles launch first
  const int off = Lk - Lq;                     // query row r sits at key position r + off

  const int g = hslice / a.head_slices;
  const int hs = hslice % a.head_slices;
  const int hw = wave % a.heads_per_wg, tw = wave / a.heads_per_wg;
  const int head = g * a.group + hs * a.heads_per_wg + hw;
  const int tok0 = t0 + 32 * tw;  // first query row of this wave
  const int my_tok = tok0 + l32;  // this lane's query row
  const bool row_valid = my_tok < Lq;
  const int qpos = my_tok + off;  // key position of this query row

  int kv_end = Lk, wave_kv_end = Lk;
  if constexpr (CAUSAL) {
    kv_end = min(Lk, min(t0 + BT, Lq) + off);
    wave_kv_end = min(Lk, min(tok0 + 32, Lq) + off);
  }
  if (tok0 >= Lq) wave_kv_end = 0;
  const int nkt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

  // ---- Q^T operand: lane holds features 16*s + 8*hi .. +7 of its row
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

  // ---- staging setup: buffer resources over this sequence's rows of head g
  const uint32_t rs_bytes = (uint32_t)a.Hkv * D * 2;   // bytes between key rows
  const uint32_t seq_bytes = Lk > 0 ? (uint32_t)(Lk - 1) * rs_bytes + D * 2 : 0u;
  const size_t head_off = ((size_t)sk0 * a.Hkv + g) * D;
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc(a.k + head_off, seq_bytes);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(a.v + head_off, seq_bytes);
  // K: direct loads, block q = i * 4 + wave of 1 KB (rowsPerKB rows) per instruction
  uint32_t k_voff[L::kLoads];
#pragma unroll
  for (int i = 0; i < L::kLoads; ++i) {
    const int q = i * 4 + wave;
    const int r = q * L::rowsPerKB + lane / L::chunks;
    const int pos = lane % L::chunks;
    k_voff[i] = (uint32_t)r * rs_bytes + (uint32_t)k_pos<D>(r, pos) * 16u;
  }
  // V: thread (kq, cv) holds keys 4kq..4kq+3 x features 8cv..8cv+7
  constexpr int V_JOBS = (BN / 4) * L::chunks;
  const bool v_job = V_JOBS >= kThreads || tid < V_JOBS;
  const int kq = tid % (BN / 4), cv = tid / (BN / 4);
  const uint32_t v_voff = (uint32_t)(4 * kq) * rs_bytes + (uint32_t)cv * 16u;
  u32x4 vr[4];

  auto issue_loads = [&](int ti, int buf) {
    const int soff = ti * BN * (int)rs_bytes;
    uint8_t* kdst = smem + buf * L::bufBytes;
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(kdst + (i * 4 + wave) * 1024),
                                               16, k_voff[i], soff, 0, 0);
    if (v_job) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, v_voff + i * rs_bytes, soff, 0));
    }
  };
  auto store_v = [&](int buf) {
    if (!v_job) return;
    uint16_t* vt = reinterpret_cast<uint16_t*>(smem + buf * L::bufBytes + L::kBytes);
    u32x4 a0 = vr[0], a1 = vr[1], a2 = vr[2], a3 = vr[3];
    if constexpr (BF16) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a0[x] = bf16x2_to_f16x2(a0[x]);
        a1[x] = bf16x2_to_f16x2(a1[x]);
        a2[x] = bf16x2_to_f16x2(a2[x]);
        a3[x] = bf16x2_to_f16x2(a3[x]);
      }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      u32x2 even, odd;
      even[0] = __builtin_amdgcn_perm(a1[x], a0[x], 0x05040100u);
      even[1] = __builtin_amdgcn_perm(a3[x], a2[x], 0x05040100u);
      odd[0] = __builtin_amdgcn_perm(a1[x], a0[x], 0x07060302u);
      odd[1] = __builtin_amdgcn_perm(a3[x], a2[x], 0x07060302u);
      *(u32x2*)(vt + (8 * cv + 2 * x) * L::vStride + 4 * kq) = even;
      *(u32x2*)(vt + (8 * cv + 2 * x + 1) * L::vStride + 4 * kq) = odd;
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) o[d] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  // One 64-key tile: S^T = K Q^T, softmax update, O^T += V^T P^T.
  auto tile_step = [&](const uint8_t* buf, int j0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint8_t* Kb = buf;
    const uint16_t* Vt = reinterpret_cast<const uint16_t*>(buf + L::kBytes);
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int r = 32 * kb + key_of_row(l32);
      const uint8_t* krow = Kb + r * (D * 2);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 kf = *(const u32x4*)(krow + k_pos<D>(r, 2 * ks + hi) * 16);
        s[kb] = mfma_32x32x16<BF16>(kf, qf[ks], s[kb]);
      }
    }
    const int jlane = j0 + 8 * hi;  // key of register 0 in block 0
    float mx = kNegInf;
    if constexpr (ALIBI) {
      const float sb = slope2 * (float)(jlane - qpos);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = 32 * kb + key_of_reg(r, 0);
          float x;
          if constexpr (CAUSAL) x = __builtin_fmaf(s[kb][r], c, __builtin_fmaf(slope2, (float)jl, sb));
          else x = __builtin_fmaf(s[kb][r], c, -slope2 * __builtin_fabsf((float)(jlane + jl - qpos)));
          if constexpr (MASK) {
            const int j = jlane + jl;
            if (j >= Lk || (CAUSAL && j > qpos)) x = kNegInf;
          }
          s[kb][r] = x;
          mx = __builtin_fmaxf(mx, x);
        }
    } else {
      // scores stay unscaled here; the scale (> 0) is folded into the exponent
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (MASK) {
            const int j = jlane + 32 * kb + key_of_reg(r, 0);
            if (j >= Lk || (CAUSAL && j > qpos)) s[kb][r] = kNegInf;
          }
          mx = __builtin_fmaxf(mx, s[kb][r]);
        }
      mx *= c;
    }
    mx = halfwave_max(mx);
    if (__any(mx > m_run + kRescaleThreshold)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < D / 32; ++d) o[d] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float lsum = 0.f;
    u32x4 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0, p1;
        if constexpr (ALIBI) {
          p0 = fast_exp2(s[kb][r] - m_use);
          p1 = fast_exp2(s[kb][r + 1] - m_use);
        } else {
          p0 = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
          p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c, -m_use));
        }
        lsum += p0 + p1;
        pf[2 * kb + r / 8][(r % 8) / 2] = pack_f16x2(p0, p1);
      }
    l_run += lsum;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const u32x4 vf = *(const u32x4*)(Vt + (32 * d + l32) * L::vStride + 16 * ch + 8 * hi);
        o[d] = mfma_32x32x16<false>(vf, pf[ch], o[d]);
      }
  };

  if (nkt > 0) {
    issue_loads(nkt - 1, 0);
    __builtin_amdgcn_s_waitcnt(0);
    store_v(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int ti = nkt - 1 - kt;  // diagonal tile first
    const int j0 = ti * BN;
    const int cur = kt & 1;
    if (kt + 1 < nkt) issue_loads(ti - 1, cur ^ 1);
    if (j0 < wave_kv_end) {
      const bool need_mask = (j0 + BN > Lk) || (CAUSAL && j0 + BN - 1 > tok0 + off);
      if (need_mask) tile_step(smem + cur * L::bufBytes, j0, std::true_type{});
      else tile_step(smem + cur * L::bufBytes, j0, std::false_type{});
    }
    if (kt + 1 < nkt) {
      __builtin_amdgcn_s_waitcnt(0);
      store_v(cur ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, round, stage the wave's 32 x D tile through LDS
  // so that every global store writes whole 16-byte runs of a row.
  const float l_tot = halfwave_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* ot = reinterpret_cast<uint16_t*>(smem) + wave * 32 * (D + 8);  // [32][D + 8]
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 wv;
      wv[0] = pack_out_x2<BF16>(o[d][4 * r4] * inv, o[d][4 * r4 + 1] * inv);
      wv[1] = pack_out_x2<BF16>(o[d][4 * r4 + 2] * inv, o[d][4 * r4 + 3] * inv);
      *(u32x2*)(ot + l32 * (D + 8) + 32 * d + 8 * r4 + 4 * hi) = wv;
    }
  if (a.lse != nullptr && hi == 0 && row_valid)
    a.lse[(size_t)head * a.total_q + sq0 + my_tok] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  constexpr int RPI = 64 / L::chunks;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + lane / L::chunks, ch = lane % L::chunks;
    if (tok0 + row < Lq) {
      const u32x4 val = *(const u32x4*)(ot + row * (D + 8) + ch * 8);
      *(u32x4*)(a.out + ((size_t)(sq0 + tok0 + row) * a.Hq + head) * D + ch * 8) = val;
    }
  }
#endif
}

template <int D, bool BF16>
static hipError_t launch_prefill_d(const FwdArgs& a, bool causal, bool alibi, dim3 grid,
                                   hipStream_t stream) {
  const dim3 block(kThreads);
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
                          int /*max_seqlen_q*/, hipStream_t stream) {
  const dim3 grid((unsigned)(((long long)a.pf_items + 7) / 8 * 8));
  if (D == 64) {
    return bf16 ? launch_prefill_d<64, true>(a, causal, alibi, grid, stream)
                : launch_prefill_d<64, false>(a, causal, alibi, grid, stream);
  }
  return bf16 ? launch_prefill_d<128, true>(a, causal, alibi, grid, stream)
              : launch_prefill_d<128, false>(a, causal, alibi, grid, stream);
}

}  // namespace mea
