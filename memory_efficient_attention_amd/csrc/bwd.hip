// Backward of the fused attention over packed sequences (dQ, dK, dV), on the
// gfx950 matrix cores.
//
// For every sequence and query head h, with g the key/value head of h's group
// and P the forward's softmax weights, recomputed tile by tile from the
// forward's log-sum-exp:
//   dV_g += P^T dO_h
//   dP    = dO_h V_g^T
//   dS    = P * (dP - Dsum),  Dsum = rowsum(dO_h * O_h)  (= rowsum(P * dP))
//   dQ_h  = scale dS K_g
//   dK_g += scale dS^T Q_h
// The score matrix, P and dS never reach HBM.
//
// Launches, in stream order:
//   prep     per (query row, head): Dsum from O and dO in float32, and the
//            log-sum-exp in log2 units (+inf for a row with no allowed key,
//            so that its weights come out as 0);
//   dK/dV    a workgroup of 8 waves owns 128 keys of one key/value head: K
//            and V rows sit in LDS for the whole walk, each wave accumulates
//            dK^T and dV^T of 32 keys in registers, and the two groups of 4
//            waves take the two 32-row halves of every 64-row query tile of
//            every query head of the group that can see the keys (causal:
//            rows from the key tile's diagonal on).  Per tile, with the Q and
//            dO rows staged in LDS:
//              S = Q K^T, dP = dO V^T        query rows fed in key_of_row
//                                            order, so a lane's registers hold
//                                            two runs of 8 consecutive rows
//              P, dS                         float32, per element
//              dV^T += dO^T P, dK^T += Q^T dS  P and dS taken straight from
//                                            the registers as the k-operand,
//                                            dO^T and Q^T read from the same
//                                            row tiles by LDS transpose loads;
//            the two groups' partial sums meet in LDS at the end; no atomics;
//   dQ       a workgroup of 8 waves owns 32-row chunks of one or more query
//            heads of a group (as in the forward), Q and dO in registers, and
//            walks 64-key tiles of K and V rows staged in LDS:
//              S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T
//            with K^T read from the K rows by transpose loads.
// Products run in the input precision (P and dS are rounded to it) with
// float32 accumulation.
#include "mea_common.h"
#include "mea_launch.h"
#include "mea_tiles.h"

namespace mea {

namespace {

constexpr int kThreads = 64 * kBwWaves;
constexpr int kAuxThreads = 256;  // prep kernel

template <int D>
struct DkvLayout {
  static constexpr int kvBytes = kBwKeys * D * 2;           // K or V rows [128][D], kt_pos swizzle
  static constexpr int rowBytes = kBwRows * D * 2;          // Q or dO rows [64][D], kt_pos swizzle
  static constexpr int offK = 0;
  static constexpr int offV = kvBytes;
  static constexpr int offStage = 2 * kvBytes;
  static constexpr int offQ = 0;                            // within a stage buffer
  static constexpr int offDO = rowBytes;
  static constexpr int offL = 2 * rowBytes;                 // lse2[64], then Dsum[64] (float32)
  static constexpr int stageBytes = offL + 2 * kBwRows * 4;
  static constexpr int slots = 2;                           // stage buffers
  static constexpr int bytes = offStage + slots * stageBytes;
  static constexpr int chunks = D / 8;                      // 16-byte chunks per row
  static constexpr int rowsPerKB = 1024 / (D * 2);          // rows per 1 KB direct-load block
  static constexpr int kvLoads = kvBytes / (kThreads * 16); // 1 KB blocks per wave for K (and for V)
  static constexpr int loads = rowBytes / (kThreads * 16);  // 1 KB blocks per wave for Q (and for dO)
};

template <int D>
struct DqLayout {
  static constexpr int rowBytes = kBwKeyTile * D * 2;       // K or V rows [64][D], kt_pos swizzle
  static constexpr int offK = 0;
  static constexpr int offV = rowBytes;
  static constexpr int bufBytes = 2 * rowBytes;
  static constexpr int slots = 3;                           // ring of stage buffers
  static constexpr int chunks = D / 8;
  static constexpr int rowsPerKB = 1024 / (D * 2);
  static constexpr int loads = rowBytes / (kThreads * 16);
};

// Writes a wave's 32 x D float32 accumulator tile (rows = the lane's
// column l32, features 32 d + acc_row(r, hi)) times `mul` as rows of the
// output dtype into an LDS staging tile [32][D + 8].
template <int D, bool BF16>
__device__ __forceinline__ void stage_rows(uint16_t* tile, const f32x16 (&acc)[D / 32], float mul, int l32, int hi) {
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2 wv;
      wv[0] = pack_out_x2<BF16>(acc[d][4 * r4] * mul, acc[d][4 * r4 + 1] * mul);
      wv[1] = pack_out_x2<BF16>(acc[d][4 * r4 + 2] * mul, acc[d][4 * r4 + 3] * mul);
      *(u32x2*)(tile + l32 * (D + 8) + 32 * d + 8 * r4 + 4 * hi) = wv;
    }
}

// Copies rows row < nrows of a staged [32][D + 8] tile to dst + row * stride
// (elements), whole 16-byte runs per lane.
template <int D>
__device__ __forceinline__ void store_rows(const uint16_t* tile, uint16_t* dst, size_t stride, int nrows, int lane) {
  constexpr int chunks = D / 8;
  constexpr int RPI = 64 / chunks;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + lane / chunks, ch = lane % chunks;
    if (row < nrows)
      __builtin_nontemporal_store(*(const u32x4*)(tile + row * (D + 8) + ch * 8), (u32x4*)(dst + (size_t)row * stride + ch * 8));
  }
}

}  // namespace

// ---------------------------------------------------------------------------- prep
// Dsum[h, t] = sum_d dO[t, h, d] O[t, h, d] (float32) and lse2[h, t] = lse[h, t]
// * log2(e), +inf where lse is -inf.  D / 8 threads per (row, head).
template <int D, bool BF16>
__global__ __launch_bounds__(kAuxThreads) void bwd_prep_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;
  const long long row = (long long)blockIdx.x * (kAuxThreads / TPR) + threadIdx.x / TPR;  // t * Hq + h
  if (row >= (long long)a.total_q * a.Hq) return;
  const int j = threadIdx.x % TPR;
  const u32x4 o = *(const u32x4*)(a.out + row * D + 8 * j);
  const u32x4 d = *(const u32x4*)(a.dout + row * D + 8 * j);
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // words copied out first: a bit cast of a vector element in place reads element 0
    const uint32_t ow = o[w], dw = d[w];
    float o0, o1, d0, d1;
    if constexpr (BF16) {
      o0 = __builtin_bit_cast(float, ow << 16);
      o1 = __builtin_bit_cast(float, ow & 0xffff0000u);
      d0 = __builtin_bit_cast(float, dw << 16);
      d1 = __builtin_bit_cast(float, dw & 0xffff0000u);
    } else {
      const f16x2 oh = __builtin_bit_cast(f16x2, ow), dh = __builtin_bit_cast(f16x2, dw);
      o0 = (float)oh[0];
      o1 = (float)oh[1];
      d0 = (float)dh[0];
      d1 = (float)dh[1];
    }
    acc = __builtin_fmaf(o0, d0, acc);
    acc = __builtin_fmaf(o1, d1, acc);
  }
#pragma unroll
  for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
  if (j == 0) {
    const int t = (int)(row / a.Hq), h = (int)(row % a.Hq);
    const size_t idx = (size_t)h * a.total_q + t;
    a.ws_dsum[idx] = acc;
    const float l = a.lse[idx];
    a.ws_lse2[idx] = (l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------- dK, dV
template <int D, bool BF16, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = DkvLayout<D>;
  constexpr int KS = D / 16;  // k-steps of S = Q K^T
  constexpr int ND = D / 32;  // 32-feature blocks of dK^T, dV^T
  constexpr int kPartBytes = kBwWaves * 32 * D * 4;      // one fp32 accumulator set per wave
  constexpr int kStageOut = kBwWaves * 32 * (D + 8) * 2;  // one [32][D + 8] output tile per wave
  static_assert(kPartBytes <= L::bytes && kStageOut <= L::bytes, "LDS reuse");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::bytes];

  // ---- work item (XCD-aware remap): key tile kt of sequence b, key/value head g
  const int per_xcd = (int)gridDim.x >> 3;
  const int w = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
  if (w >= a.kv_items) return;
  const int kt = w % a.kv_tiles;
  const int rest = w / a.kv_tiles;
  const int b = rest % a.num_seqs;
  const int g = rest / a.num_seqs;
  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  const int sk0 = a.seqstart_k[b], Lk = a.seqstart_k[b + 1] - sk0;
  const int kt0 = kt * kBwKeys;
  if (kt0 >= Lk) return;
  const int off = Lk - Lq;  // query row r sits at key position r + off

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kBwGroupWaves;  // which 32-row half of each query tile
  const int wk = wave % kBwGroupWaves;   // which 32-key block
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wkey0 = kt0 + 32 * wk;  // first key of this wave
  const int my_key = wkey0 + l32;

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }

  // query tiles that see any of the keys: causal, row r sees key j when j <= r + off
  const int q_first = CAUSAL ? max(0, kt0 - off) : 0;
  const int qb0 = q_first / kBwRows;
  const int nqt = Lq > q_first ? (Lq + kBwRows - 1) / kBwRows - qb0 : 0;
  const int nst = nqt * a.group;  // stages: (query tile, query head of the group)
  // Query tiles run from the sequence's last down to the key tile's diagonal,
  // so that the workgroups of one sequence (consecutive work items, one XCD)
  // start on the same tile and read the same Q and dO rows at about the same
  // time: one fetch from HBM serves them all from the XCD's L2.
  const int qb_last = qb0 + nqt - 1;

  // ---- staging: K and V rows of the 128 keys once; Q and dO rows of the
  // sequence (all heads) per stage; rows past a sequence's end read zeros
  const uint32_t rs_k = (uint32_t)a.Hkv * D * 2;
  const uint32_t kv_bytes = (uint32_t)(Lk - kt0 - 1) * rs_k + D * 2;
  const size_t kv_first = ((size_t)(sk0 + kt0) * a.Hkv + g) * D;
  const __amdgpu_buffer_rsrc_t krs = buf_rsrc(a.k + kv_first, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(a.v + kv_first, kv_bytes);
  const uint32_t rs_q = (uint32_t)a.Hq * D * 2;
  const __amdgpu_buffer_rsrc_t qrs = buf_rsrc(a.q + (size_t)sq0 * a.Hq * D, (uint32_t)Lq * rs_q);
  const __amdgpu_buffer_rsrc_t dors = buf_rsrc(a.dout + (size_t)sq0 * a.Hq * D, (uint32_t)Lq * rs_q);
  auto row_voff = [&](int blk, uint32_t rs) {
    const int r = blk * L::rowsPerKB + lane / L::chunks;
    return (uint32_t)r * rs + (uint32_t)kt_pos<D>(r, lane % L::chunks) * 16u;
  };
  if (nst > 0) {
#pragma unroll
    for (int i = 0; i < L::kvLoads; ++i) {
      const int blk = i * kBwWaves + wave;
      load_lds16(krs, smem + L::offK + blk * 1024, row_voff(blk, rs_k), 0);
      load_lds16(vrs, smem + L::offV + blk * 1024, row_voff(blk, rs_k), 0);
    }
  }

  auto stage_buf = [&](int st) { return smem + L::offStage + (st % L::slots) * L::stageBytes; };
  auto issue = [&](int st, uint8_t* buf) {
    const int hh = st % a.group, qb = qb_last - st / a.group;
    const int h = g * a.group + hh;
    if (wave < 2) {
      const float* src = (wave == 0 ? a.ws_lse2 : a.ws_dsum) + (size_t)h * a.total_q + sq0;
      load_lds4(buf_rsrc(src, (uint32_t)Lq * 4), buf + L::offL + wave * (kBwRows * 4), (uint32_t)lane * 4,
                qb * kBwRows * 4);
    }
    const int rsoff = qb * kBwRows * (int)rs_q + h * D * 2;
#pragma unroll
    for (int i = 0; i < L::loads; ++i) {
      const int blk = i * kBwWaves + wave;
      load_lds16(qrs, buf + L::offQ + blk * 1024, row_voff(blk, rs_q), rsoff);
      load_lds16(dors, buf + L::offDO + blk * 1024, row_voff(blk, rs_q), rsoff);
    }
  };

  const float c = a.scale_log2;
  const int sb = grp;  // this wave's 32-row half of every stage
  auto compute = [&](int st, const uint8_t* buf) {
    const int hh = st % a.group, qb = qb_last - st / a.group;
    const int h = g * a.group + hh;
    float slope2 = 0.f;
    if constexpr (ALIBI) slope2 = a.slopes[h] * kLog2e;
    const int kd0 = my_key - (qb * kBwRows + off);  // key position minus the stage's first query position
    const bool need_mask = CAUSAL && (wkey0 + 31 > qb * kBwRows + 32 * sb + off);
    f32x16 s = f32x16{}, dp = f32x16{};
    const int rr = 32 * sb + key_of_row(l32);  // query row fed to A-row l32
    const int kr = 32 * wk + l32;              // key row of this lane's K and V operands
    // fragments of k-step ks: Q, K, dO, V; those of ks + 1 are read while the
    // products of ks run (two register sets, the order fixed below)
    auto frags = [&](int ks, u32x4 (&f)[4]) {
      const int at = rr * (D * 2) + kt_pos<D>(rr, 2 * ks + hi) * 16;
      const int kat = kr * (D * 2) + kt_pos<D>(kr, 2 * ks + hi) * 16;
      f[0] = *(const u32x4*)(buf + L::offQ + at);
      f[1] = *(const u32x4*)(smem + L::offK + kat);
      f[2] = *(const u32x4*)(buf + L::offDO + at);
      f[3] = *(const u32x4*)(smem + L::offV + kat);
    };
    u32x4 fr[2][4];
    frags(0, fr[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) frags(ks + 1, fr[(ks + 1) & 1]);
      s = mfma_32x32x16<BF16>(fr[ks & 1][0], fr[ks & 1][1], s);
      dp = mfma_32x32x16<BF16>(fr[ks & 1][2], fr[ks & 1][3], dp);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // reads of k-step 0
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // reads of ks + 1
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // products of ks
    }
    // register r holds stage row 32 sb + key_of_reg(r, hi); key position minus
    // query position of register r: kd0 - 32 sb - 8 hi - ro(r)
    if constexpr (CAUSAL) {
      if (need_mask) {  // scores of keys after the query row -> -inf, so their weights are 0
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kd0 - (32 * sb + 8 * hi + 16 * (r / 8) + r % 8) > 0) s[r] = kNegInf;
      }
    }
    const float* lrow = reinterpret_cast<const float*>(buf + L::offL) + 32 * sb + 8 * hi;
    const float* drow = lrow + kBwRows;
    u32x4 pf[2], dsf[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p[2], ds[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int ro = 16 * ((r + e) / 8) + (r + e) % 8;  // key_of_reg(r + e, hi) - 8 hi
        float x = __builtin_fmaf(s[r + e], c, -lrow[ro]);
        if constexpr (ALIBI) x = __builtin_fmaf(-slope2, __builtin_fabsf((float)(kd0 - (32 * sb + 8 * hi + ro))), x);
        const float pe = fast_exp2(x);
        p[e] = pe;
        ds[e] = pe * (dp[r + e] - drow[ro]);
      }
      pf[r / 8][(r % 8) / 2] = pack_out_x2<BF16>(p[0], p[1]);
      dsf[r / 8][(r % 8) / 2] = pack_out_x2<BF16>(ds[0], ds[1]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const u32x4 oa = read_rows_transposed<D>(buf + L::offDO, 32 * sb + 16 * kk, 32 * d, lane);
        const u32x4 qa = read_rows_transposed<D>(buf + L::offQ, 32 * sb + 16 * kk, 32 * d, lane);
        dv[d] = mfma_32x32x16<BF16>(oa, pf[kk], dv[d]);
        dk[d] = mfma_32x32x16<BF16>(qa, dsf[kk], dk[d]);
      }
  };

  // ---- two stage buffers, one barrier per stage.  In iteration st: wait for
  // this wave's share of tile st, barrier (every wave has its share of tile
  // st and is done with tile st - 1, whose buffer tile st + 1 takes), request
  // tile st + 1, compute st.
  if (nst > 0) {
    // the stage being read and the one being filled as restrict pointers:
    // the compiler then knows that the transposed LDS reads of stage st do
    // not touch the DMA of stage st + 1 in flight, and does not wait for it
    // before them
    auto step = [&](int st, uint8_t* __restrict__ next, const uint8_t* __restrict__ cur) {
      if (st + 1 < nst) issue(st + 1, next);
      compute(st, cur);
    };
    issue(0, stage_buf(0));
    for (int st = 0; st < nst; ++st) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      step(st, stage_buf(st + 1), stage_buf(st));
    }
    __syncthreads();  // every wave is done with the buffers before the epilogue reuses LDS
  }

  // ---- epilogue: the two groups' partial sums meet in LDS.  Group 0 hands
  // its dV^T to group 1 and finishes dK; group 1 hands its dK^T to group 0 and
  // finishes dV.  Partials are laid out [wave][block d][register r][lane].
  float* part = reinterpret_cast<float*>(smem);
  {
    const f32x16* mine = grp == 0 ? dv : dk;
    float* dst = part + (size_t)(grp * kBwGroupWaves + wk) * (ND * 16 * 64);
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(d * 16 + r) * 64 + lane] = mine[d][r];
  }
  __syncthreads();
  {
    f32x16* acc = grp == 0 ? dk : dv;
    const float* src = part + (size_t)((1 - grp) * kBwGroupWaves + wk) * (ND * 16 * 64);
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] += src[(d * 16 + r) * 64 + lane];
  }
  __syncthreads();
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem) + wave * 32 * (D + 8);
  if (grp == 0) stage_rows<D, BF16>(tile, dk, a.scale, l32, hi);
  else stage_rows<D, BF16>(tile, dv, 1.f, l32, hi);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const size_t first = ((size_t)(sk0 + wkey0) * a.Hkv + g) * D;
  store_rows<D>(tile, (grp == 0 ? a.dk : a.dv) + first, (size_t)a.Hkv * D, Lk - wkey0, lane);
#endif
}

// ---------------------------------------------------------------------------- dQ
template <int D, bool BF16, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = DqLayout<D>;
  constexpr int KS = D / 16;
  constexpr int ND = D / 32;
  constexpr int kStageBytes = kBwWaves * 32 * (D + 8) * 2;
  constexpr int kSmemBytes = L::slots * L::bufBytes > kStageBytes ? L::slots * L::bufBytes : kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];

  // ---- work item (XCD-aware remap): query tile of sequence b, head slice
  const int per_xcd = (int)gridDim.x >> 3;
  const int w = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
  if (w >= a.q_items) return;
  const int t_rev = w % a.q_tiles;
  const int rest = w / a.q_tiles;
  const int b = rest % a.num_seqs;
  const int hslice = rest / a.num_seqs;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  const int sk0 = a.seqstart_k[b], Lk = a.seqstart_k[b + 1] - sk0;
  const int tc = kBwWaves / a.heads_per_wg;  // 32-row chunks per head
  const int BT = 32 * tc;                    // query rows per workgroup
  const int ntiles = (Lq + BT - 1) / BT;
  if (t_rev >= ntiles) return;
  const int t0 = (ntiles - 1 - t_rev) * BT;  // longest causal tiles launch first
  const int off = Lk - Lq;

  const int g = hslice / a.head_slices;
  const int hs = hslice % a.head_slices;
  const int hw = wave % a.heads_per_wg, tw = wave / a.heads_per_wg;
  const int head = g * a.group + hs * a.heads_per_wg + hw;
  const int tok0 = t0 + 32 * tw;  // first query row of this wave
  const int my_tok = tok0 + l32;
  const bool row_valid = my_tok < Lq;
  const int qpos = my_tok + off;

  // Q and dO as the k-operands of S^T = K Q^T and dP^T = V dO^T
  u32x4 qf[KS], of[KS];
  {
    const size_t base = ((size_t)(sq0 + my_tok) * a.Hq + head) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (row_valid) {
        x = *(const u32x4*)(a.q + base + 16 * s);
        y = *(const u32x4*)(a.dout + base + 16 * s);
      }
      qf[s] = x;
      of[s] = y;
    }
  }
  float lse2 = 0.f, dsum = 0.f;
  if (row_valid) {
    lse2 = a.ws_lse2[(size_t)head * a.total_q + sq0 + my_tok];
    dsum = a.ws_dsum[(size_t)head * a.total_q + sq0 + my_tok];
  }
  float slope2 = 0.f;
  if constexpr (ALIBI) slope2 = a.slopes[head] * kLog2e;
  const float c = a.scale_log2;

  int kv_end = Lk;
  if constexpr (CAUSAL) kv_end = min(Lk, min(t0 + BT, Lq) + off);
  const int nkt = kv_end > 0 ? (kv_end + kBwKeyTile - 1) / kBwKeyTile : 0;

  // ---- staging: K and V rows of head g (rows past the end read zeros)
  const uint32_t rs_k = (uint32_t)a.Hkv * D * 2;
  const uint32_t seq_bytes = Lk > 0 ? (uint32_t)(Lk - 1) * rs_k + D * 2 : 0u;
  const size_t head_off = ((size_t)sk0 * a.Hkv + g) * D;
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc(a.k + head_off, seq_bytes);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(a.v + head_off, seq_bytes);
  uint32_t row_voff[L::loads];
#pragma unroll
  for (int i = 0; i < L::loads; ++i) {
    const int blk = i * kBwWaves + wave;
    const int r = blk * L::rowsPerKB + lane / L::chunks;
    row_voff[i] = (uint32_t)r * rs_k + (uint32_t)kt_pos<D>(r, lane % L::chunks) * 16u;
  }

  auto ring_buf = [&](int t) { return smem + (t % L::slots) * L::bufBytes; };
  auto issue = [&](int t, uint8_t* buf) {
    const int rsoff = t * kBwKeyTile * (int)rs_k;
#pragma unroll
    for (int i = 0; i < L::loads; ++i) {
      const int blk = i * kBwWaves + wave;
      load_lds16(krs, buf + L::offK + blk * 1024, row_voff[i], rsoff);
      load_lds16(vrs, buf + L::offV + blk * 1024, row_voff[i], rsoff);
    }
  };

  f32x16 dq[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dq[d] = f32x16{};

  auto compute = [&](int t, const uint8_t* buf) {
    const int j0 = t * kBwKeyTile;
    const int jlane = j0 + 8 * hi;  // key of register 0 in block 0
    const bool need_mask = (j0 + kBwKeyTile > Lk) || (CAUSAL && j0 + kBwKeyTile - 1 > tok0 + off);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const int rr = 32 * kb + key_of_row(l32);
      // K and V fragments of k-step ks + 1 are read while the products of ks run
      auto frags = [&](int ks, u32x4 (&f)[2]) {
        const int at = rr * (D * 2) + kt_pos<D>(rr, 2 * ks + hi) * 16;
        f[0] = *(const u32x4*)(buf + L::offK + at);
        f[1] = *(const u32x4*)(buf + L::offV + at);
      };
      u32x4 fr[2][2];
      frags(0, fr[0]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) frags(ks + 1, fr[(ks + 1) & 1]);
        s = mfma_32x32x16<BF16>(fr[ks & 1][0], qf[ks], s);
        dp = mfma_32x32x16<BF16>(fr[ks & 1][1], of[ks], dp);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // reads of k-step 0
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // reads of ks + 1
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // products of ks
      }
      if (need_mask) {  // keys past the end, or after the query row -> -inf, so their weights are 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jlane + 32 * kb + key_of_reg(r, 0);
          if (j >= Lk || (CAUSAL && j > qpos)) s[r] = kNegInf;
        }
      }
      u32x4 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float x = __builtin_fmaf(s[r + e], c, -lse2);
          if constexpr (ALIBI) {
            const int j = jlane + 32 * kb + key_of_reg(r + e, 0);
            x = __builtin_fmaf(-slope2, __builtin_fabsf((float)(qpos - j)), x);
          }
          const float pe = fast_exp2(x);
          ds[e] = pe * (dp[r + e] - dsum);
        }
        dsf[r / 8][(r % 8) / 2] = pack_out_x2<BF16>(ds[0], ds[1]);
      }
      // dQ^T += K^T dS^T over this block's 32 keys (two k-steps of 16)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const u32x4 ka = read_rows_transposed<D>(buf + L::offK, 32 * kb + 16 * kk, 32 * d, lane);
          dq[d] = mfma_32x32x16<BF16>(ka, dsf[kk], dq[d]);
        }
    }
  };

  // ---- a ring of 3 tile buffers, tiles requested two ahead, one barrier per
  // tile (as in the dK/dV kernel)
  constexpr int kWaitNextLds = (2 * L::loads) | (7 << 4);  // vmcnt(2 loads), lgkmcnt(0)
  if (nkt > 0) {
    // restrict pointers, as in the dK/dV kernel: no wait for the DMA of tile
    // t + 2 before the transposed reads of tile t
    // the three ring slots as restrict pointers, and the loop unrolled by
    // three so that each step's slots are fixed: the compiler then knows that
    // the transposed reads of tile t touch neither the DMA of tile t + 1 nor
    // that of tile t + 2 in flight
    auto ring = [&](uint8_t* __restrict__ b0, uint8_t* __restrict__ b1, uint8_t* __restrict__ b2) {
      auto step = [&](int t, uint8_t* next, const uint8_t* cur) {
        // tile t landed (tile t + 1 may stay in flight across the barrier:
        // __syncthreads would wait for it) and this wave's reads of tile
        // t - 1, whose slot tile t + 2 takes, are done
        if (t + 1 < nkt) __builtin_amdgcn_s_waitcnt(kWaitNextLds);
        else __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (t + 2 < nkt) issue(t + 2, next);
        compute(t, cur);
      };
      issue(0, b0);
      if (nkt > 1) issue(1, b1);
      for (int t = 0; t < nkt; t += 3) {
        step(t, b2, b0);
        if (t + 1 < nkt) step(t + 1, b0, b1);
        if (t + 2 < nkt) step(t + 2, b1, b2);
      }
    };
    ring(ring_buf(0), ring_buf(1), ring_buf(2));
    __syncthreads();  // every wave is done with the ring before the epilogue reuses LDS
  }

  // ---- epilogue: dQ = scale dS K, staged through LDS as rows
  uint16_t* tq = reinterpret_cast<uint16_t*>(smem) + wave * 32 * (D + 8);
  stage_rows<D, BF16>(tq, dq, a.scale, l32, hi);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  store_rows<D>(tq, a.dq + ((size_t)(sq0 + tok0) * a.Hq + head) * D, (size_t)a.Hq * D, Lq - tok0, lane);
#endif
}

// ---------------------------------------------------------------------------- launch
namespace {

template <int D, bool BF16, bool CAUSAL, bool ALIBI>
hipError_t launch_main(const BwdArgs& a, hipStream_t stream) {
  if (a.kv_items > 0) {
    const dim3 grid((unsigned)(((long long)a.kv_items + 7) / 8 * 8));
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BF16, CAUSAL, ALIBI>), grid, dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.q_items > 0) {
    const dim3 grid((unsigned)(((long long)a.q_items + 7) / 8 * 8));
    hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, CAUSAL, ALIBI>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_backward_d(const BwdArgs& a, bool causal, bool alibi, hipStream_t stream) {
  if (a.total_q > 0) {
    constexpr int rows_per_block = kAuxThreads / (D / 8);
    const long long rows = (long long)a.total_q * a.Hq;
    hipLaunchKernelGGL((bwd_prep_kernel<D, BF16>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                       dim3(kAuxThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (causal) {
    return alibi ? launch_main<D, BF16, true, true>(a, stream) : launch_main<D, BF16, true, false>(a, stream);
  }
  return alibi ? launch_main<D, BF16, false, true>(a, stream) : launch_main<D, BF16, false, false>(a, stream);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, int D, bool bf16, bool causal, bool alibi, hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_backward_d<64, true>(a, causal, alibi, stream)
                : launch_backward_d<64, false>(a, causal, alibi, stream);
  }
  return bf16 ? launch_backward_d<128, true>(a, causal, alibi, stream)
              : launch_backward_d<128, false>(a, causal, alibi, stream);
}

}  // namespace mea
