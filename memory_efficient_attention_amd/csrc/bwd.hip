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
//   images   transposed [D][64] tile images of Q, dO (per 64-row tile of a
//            sequence and query head) and of K (per 64-key tile and
//            key/value head), in the LDS layout, so that operands that enter
//            a product along their row axis load as 16-byte rows;
//   dK/dV    a workgroup owns 128 keys of one key/value head (32 per wave,
//            with their dK^T and dV^T accumulators and the K and V operands in
//            registers) and walks the 64-row query tiles of every query head
//            of the group that can see them (causal: rows from the key tile's
//            diagonal on).  Per tile, with Q and dO rows and their images
//            staged in LDS:
//              S = Q K^T, dP = dO V^T        query rows fed in key_of_row
//                                            order, so a lane's registers hold
//                                            two runs of 8 consecutive rows
//              P, dS                         float32, per element
//              dV^T += dO^T P, dK^T += Q^T dS  P and dS taken straight from
//                                            the registers as the k-operand;
//            no atomics: the group's query heads are summed in registers;
//   dQ       a workgroup owns 32-row chunks of one or more query heads of a
//            group (as in the forward), Q and dO in registers, and walks
//            64-key tiles staged in LDS (K rows, V rows, K^T image):
//              S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
// Products run in the input precision (P and dS are rounded to it) with
// float32 accumulation.
#include "mea_common.h"
#include "mea_launch.h"
#include "mea_tiles.h"

namespace mea {

namespace {

constexpr int kThreads = 64 * kBwWaves;
constexpr int kAuxThreads = 256;  // prep and image kernels

template <int D>
struct DkvLayout {
  static constexpr int rowBytes = kBwRows * D * 2;          // Q or dO rows [64][D], k_pos swizzle
  static constexpr int imgBytes = D * kBwImg * 2;           // Q^T or dO^T image [D][64]
  static constexpr int offQ = 0;
  static constexpr int offDO = rowBytes;
  static constexpr int offQT = 2 * rowBytes;
  static constexpr int offDOT = 2 * rowBytes + imgBytes;
  static constexpr int offL = 2 * rowBytes + 2 * imgBytes;  // lse2[64], then Dsum[64] (float32)
  static constexpr int bufBytes = offL + 2 * kBwRows * 4;
  static constexpr int chunks = D / 8;                      // 16-byte chunks per row
  static constexpr int rowsPerKB = 1024 / (D * 2);          // rows per 1 KB direct-load block
  static constexpr int loads = rowBytes / (kThreads * 16);  // 1 KB blocks per wave for each tile
};

template <int D>
struct DqLayout {
  static constexpr int rowBytes = kBwKeyTile * D * 2;       // K or V rows [64][D], k_pos swizzle
  static constexpr int imgBytes = D * kBwImg * 2;           // K^T image [D][64]
  static constexpr int offK = 0;
  static constexpr int offV = rowBytes;
  static constexpr int offKT = 2 * rowBytes;
  static constexpr int bufBytes = 2 * rowBytes + imgBytes;
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
    if (row < nrows) *(u32x4*)(dst + (size_t)row * stride + ch * 8) = *(const u32x4*)(tile + row * (D + 8) + ch * 8);
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

// ---------------------------------------------------------------------------- images
// Rows 64 i .. 64 i + 63 of sequence b, head h of src [T, H, D] become the
// [D][64] image at slot (seqstart[b] / 64 + b + i) * H + h of dst (rows past
// the sequence's end are zero).
template <int D>
__global__ __launch_bounds__(kAuxThreads) void bwd_images_kernel(const uint16_t* src, uint16_t* dst,
                                                                 const int32_t* seqstart, int H) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int h = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int s0 = seqstart[b], L = seqstart[b + 1] - s0;
  if (i * kBwImg >= L) return;
  const int tid = threadIdx.x;
  const int kq = tid % (kBwImg / 4), cv = tid / (kBwImg / 4);
  if (cv >= D / 8) return;
  const uint32_t rs_bytes = (uint32_t)H * D * 2;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(src + ((size_t)s0 * H + h) * D, (uint32_t)(L - 1) * rs_bytes + D * 2);
  uint8_t* img = reinterpret_cast<uint8_t*>(dst + ((size_t)(s0 / kBwImg + b + i) * H + h) * (D * kBwImg));
  write_tile_image<D, false>(rs, (uint32_t)(i * kBwImg), rs_bytes, img, kq, cv);
#endif
}

// ---------------------------------------------------------------------------- dK, dV
template <int D, bool BF16, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = DkvLayout<D>;
  constexpr int KS = D / 16;  // k-steps of S = Q K^T
  constexpr int ND = D / 32;  // 32-feature blocks of dK^T, dV^T
  constexpr int kStageBytes = kBwWaves * 2 * 32 * (D + 8) * 2;
  constexpr int kSmemBytes = 2 * L::bufBytes > kStageBytes ? 2 * L::bufBytes : kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];

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
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wkey0 = kt0 + 32 * wave;  // first key of this wave
  const int my_key = wkey0 + l32;

  // K and V as the k-operands of S = Q K^T and dP = dO V^T: lane holds key
  // my_key, features 16 s + 8 hi .. + 7 (zero past the sequence's end)
  u32x4 kf[KS], vf[KS];
  {
    const bool valid = my_key < Lk;
    const size_t base = ((size_t)(sk0 + my_key) * a.Hkv + g) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (valid) {
        x = *(const u32x4*)(a.k + base + 16 * s);
        y = *(const u32x4*)(a.v + base + 16 * s);
      }
      kf[s] = x;
      vf[s] = y;
    }
  }
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

  // ---- staging: Q, dO rows of the sequence (all heads; rows past the end read
  // zeros) and the images of the sequence's tiles
  const uint32_t rs_q = (uint32_t)a.Hq * D * 2;
  const __amdgpu_buffer_rsrc_t qrs = buf_rsrc(a.q + (size_t)sq0 * a.Hq * D, (uint32_t)Lq * rs_q);
  const __amdgpu_buffer_rsrc_t dors = buf_rsrc(a.dout + (size_t)sq0 * a.Hq * D, (uint32_t)Lq * rs_q);
  const int ntq = (Lq + kBwImg - 1) / kBwImg;
  const size_t img0 = ((size_t)(sq0 / kBwImg) + b) * a.Hq * (D * kBwImg);
  const uint32_t img_bytes = (uint32_t)ntq * a.Hq * L::imgBytes;
  const __amdgpu_buffer_rsrc_t qtrs = buf_rsrc(a.ws_qt + img0, img_bytes);
  const __amdgpu_buffer_rsrc_t dotrs = buf_rsrc(a.ws_dot + img0, img_bytes);
  uint32_t row_voff[L::loads];
#pragma unroll
  for (int i = 0; i < L::loads; ++i) {
    const int blk = i * kBwWaves + wave;
    const int r = blk * L::rowsPerKB + lane / L::chunks;
    row_voff[i] = (uint32_t)r * rs_q + (uint32_t)k_pos<D>(r, lane % L::chunks) * 16u;
  }

  auto issue = [&](int st) {
    const int hh = st % a.group, qb = qb0 + st / a.group;
    const int h = g * a.group + hh;
    uint8_t* buf = smem + (st & 1) * L::bufBytes;
    if (wave < 2) {  // issued first: the count-based wait below may only over-wait for it
      const float* src = (wave == 0 ? a.ws_lse2 : a.ws_dsum) + (size_t)h * a.total_q + sq0;
      load_lds4(buf_rsrc(src, (uint32_t)Lq * 4), buf + L::offL + wave * (kBwRows * 4), (uint32_t)lane * 4,
                qb * kBwRows * 4);
    }
    const int rsoff = qb * kBwRows * (int)rs_q + h * D * 2;
    const int isoff = (qb * a.Hq + h) * L::imgBytes;
#pragma unroll
    for (int i = 0; i < L::loads; ++i) {
      const int blk = i * kBwWaves + wave;
      load_lds16(qrs, buf + L::offQ + blk * 1024, row_voff[i], rsoff);
      load_lds16(dors, buf + L::offDO + blk * 1024, row_voff[i], rsoff);
      load_lds16(qtrs, buf + L::offQT + blk * 1024, (uint32_t)(blk * 1024 + lane * 16), isoff);
      load_lds16(dotrs, buf + L::offDOT + blk * 1024, (uint32_t)(blk * 1024 + lane * 16), isoff);
    }
  };

  const float c = a.scale_log2;
  auto compute = [&](int st) {
    const int hh = st % a.group, qb = qb0 + st / a.group;
    const int h = g * a.group + hh;
    const uint8_t* buf = smem + (st & 1) * L::bufBytes;
    float slope2 = 0.f;
    if constexpr (ALIBI) slope2 = a.slopes[h] * kLog2e;
    const int kd0 = my_key - (qb * kBwRows + off);  // key position minus the stage's first query position
    const bool need_mask = CAUSAL && (wkey0 + 31 > qb * kBwRows + off);
#pragma unroll
    for (int sb = 0; sb < kBwRows / 32; ++sb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const int rr = 32 * sb + key_of_row(l32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int at = rr * (D * 2) + k_pos<D>(rr, 2 * ks + hi) * 16;
        const u32x4 qa = *(const u32x4*)(buf + L::offQ + at);
        const u32x4 da = *(const u32x4*)(buf + L::offDO + at);
        s = mfma_32x32x16<BF16>(qa, kf[ks], s);
        dp = mfma_32x32x16<BF16>(da, vf[ks], dp);
      }
      // register r holds stage row 32 sb + key_of_reg(r, hi)
      const float* lrow = reinterpret_cast<const float*>(buf + L::offL) + 32 * sb + 8 * hi;
      const float* drow = lrow + kBwRows;
      u32x4 pf[2], dsf[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p[2], ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ro = 16 * ((r + e) / 8) + (r + e) % 8;  // key_of_reg(r + e, hi) - 8 hi
          const int dist = kd0 - (32 * sb + 8 * hi + ro);     // key position - query position
          float x = __builtin_fmaf(s[r + e], c, -lrow[ro]);
          if constexpr (ALIBI) x = __builtin_fmaf(-slope2, __builtin_fabsf((float)dist), x);
          float pe = fast_exp2(x);
          if constexpr (CAUSAL) {
            if (need_mask && dist > 0) pe = 0.f;
          }
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
          const int at = vt_off(32 * d + l32, 4 * sb + 2 * kk + hi);
          const u32x4 oa = *(const u32x4*)(buf + L::offDOT + at);
          const u32x4 qa = *(const u32x4*)(buf + L::offQT + at);
          dv[d] = mfma_32x32x16<BF16>(oa, pf[kk], dv[d]);
          dk[d] = mfma_32x32x16<BF16>(qa, dsf[kk], dk[d]);
        }
    }
  };

  // ---- double-buffered stages: tile st + 1 loads while tile st is computed
  constexpr int kWaitNext = vmcnt_at_most(4 * L::loads);
  if (nst > 0) {
    issue(0);
    for (int st = 0; st < nst; ++st) {
      if (st + 1 < nst) {
        issue(st + 1);
        __builtin_amdgcn_s_waitcnt(kWaitNext);  // this wave's share of tile st landed
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();
      compute(st);
      __syncthreads();  // everyone is done with buffer st & 1 before tile st + 2 refills it
    }
  }

  // ---- epilogue: dK = scale dS^T Q and dV, staged through LDS as rows
  uint16_t* tk = reinterpret_cast<uint16_t*>(smem) + wave * 2 * 32 * (D + 8);
  uint16_t* tv = tk + 32 * (D + 8);
  stage_rows<D, BF16>(tk, dk, a.scale, l32, hi);
  stage_rows<D, BF16>(tv, dv, 1.f, l32, hi);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const size_t first = ((size_t)(sk0 + wkey0) * a.Hkv + g) * D;
  const size_t stride = (size_t)a.Hkv * D;
  store_rows<D>(tk, a.dk + first, stride, Lk - wkey0, lane);
  store_rows<D>(tv, a.dv + first, stride, Lk - wkey0, lane);
#endif
}

// ---------------------------------------------------------------------------- dQ
template <int D, bool BF16, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = DqLayout<D>;
  constexpr int KS = D / 16;
  constexpr int ND = D / 32;
  constexpr int kStageBytes = kBwWaves * 32 * (D + 8) * 2;
  constexpr int kSmemBytes = 2 * L::bufBytes > kStageBytes ? 2 * L::bufBytes : kStageBytes;
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

  // ---- staging: K and V rows of head g (rows past the end read zeros), K^T images
  const uint32_t rs_k = (uint32_t)a.Hkv * D * 2;
  const uint32_t seq_bytes = Lk > 0 ? (uint32_t)(Lk - 1) * rs_k + D * 2 : 0u;
  const size_t head_off = ((size_t)sk0 * a.Hkv + g) * D;
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc(a.k + head_off, seq_bytes);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(a.v + head_off, seq_bytes);
  const int ntk = (Lk + kBwImg - 1) / kBwImg;
  const __amdgpu_buffer_rsrc_t ktrs =
      buf_rsrc(a.ws_kt + ((size_t)(sk0 / kBwImg) + b) * a.Hkv * (D * kBwImg), (uint32_t)ntk * a.Hkv * L::imgBytes);
  uint32_t row_voff[L::loads];
#pragma unroll
  for (int i = 0; i < L::loads; ++i) {
    const int blk = i * kBwWaves + wave;
    const int r = blk * L::rowsPerKB + lane / L::chunks;
    row_voff[i] = (uint32_t)r * rs_k + (uint32_t)k_pos<D>(r, lane % L::chunks) * 16u;
  }

  auto issue = [&](int t) {
    uint8_t* buf = smem + (t & 1) * L::bufBytes;
    const int rsoff = t * kBwKeyTile * (int)rs_k;
    const int isoff = (t * a.Hkv + g) * L::imgBytes;
#pragma unroll
    for (int i = 0; i < L::loads; ++i) {
      const int blk = i * kBwWaves + wave;
      load_lds16(krs, buf + L::offK + blk * 1024, row_voff[i], rsoff);
      load_lds16(vrs, buf + L::offV + blk * 1024, row_voff[i], rsoff);
      load_lds16(ktrs, buf + L::offKT + blk * 1024, (uint32_t)(blk * 1024 + lane * 16), isoff);
    }
  };

  f32x16 dq[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dq[d] = f32x16{};

  auto compute = [&](int t) {
    const uint8_t* buf = smem + (t & 1) * L::bufBytes;
    const int j0 = t * kBwKeyTile;
    const int jlane = j0 + 8 * hi;  // key of register 0 in block 0
    const bool need_mask = (j0 + kBwKeyTile > Lk) || (CAUSAL && j0 + kBwKeyTile - 1 > tok0 + off);
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int rr = 32 * kb + key_of_row(l32);
        const int at = rr * (D * 2) + k_pos<D>(rr, 2 * ks + hi) * 16;
        const u32x4 ka = *(const u32x4*)(buf + L::offK + at);
        const u32x4 va = *(const u32x4*)(buf + L::offV + at);
        s[kb] = mfma_32x32x16<BF16>(ka, qf[ks], s[kb]);
        dp[kb] = mfma_32x32x16<BF16>(va, of[ks], dp[kb]);
      }
    u32x4 dsf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = jlane + 32 * kb + key_of_reg(r + e, 0);
          float x = __builtin_fmaf(s[kb][r + e], c, -lse2);
          if constexpr (ALIBI) x = __builtin_fmaf(-slope2, __builtin_fabsf((float)(qpos - j)), x);
          float pe = fast_exp2(x);
          if (need_mask && (j >= Lk || (CAUSAL && j > qpos))) pe = 0.f;
          ds[e] = pe * (dp[kb][r + e] - dsum);
        }
        dsf[2 * kb + r / 8][(r % 8) / 2] = pack_out_x2<BF16>(ds[0], ds[1]);
      }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const u32x4 ka = *(const u32x4*)(buf + L::offKT + vt_off(32 * d + l32, 2 * ch + hi));
        dq[d] = mfma_32x32x16<BF16>(ka, dsf[ch], dq[d]);
      }
  };

  constexpr int kWaitNext = vmcnt_at_most(3 * L::loads);
  if (nkt > 0) {
    issue(0);
    for (int t = 0; t < nkt; ++t) {
      if (t + 1 < nkt) {
        issue(t + 1);
        __builtin_amdgcn_s_waitcnt(kWaitNext);
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();
      compute(t);
      __syncthreads();
    }
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
hipError_t launch_backward_d(const BwdArgs& a, bool causal, bool alibi, int max_seqlen_q, int max_seqlen_k,
                             hipStream_t stream) {
  if (a.total_q > 0) {
    constexpr int rows_per_block = kAuxThreads / (D / 8);
    const long long rows = (long long)a.total_q * a.Hq;
    hipLaunchKernelGGL((bwd_prep_kernel<D, BF16>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                       dim3(kAuxThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 qgrid(a.Hq, (max_seqlen_q + kBwImg - 1) / kBwImg, a.num_seqs);
    hipLaunchKernelGGL((bwd_images_kernel<D>), qgrid, dim3(kAuxThreads), 0, stream, a.q, a.ws_qt, a.seqstart_q, a.Hq);
    hipLaunchKernelGGL((bwd_images_kernel<D>), qgrid, dim3(kAuxThreads), 0, stream, a.dout, a.ws_dot, a.seqstart_q,
                       a.Hq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.total_k > 0 && max_seqlen_k > 0 && a.q_items > 0) {
    const dim3 kgrid(a.Hkv, (max_seqlen_k + kBwImg - 1) / kBwImg, a.num_seqs);
    hipLaunchKernelGGL((bwd_images_kernel<D>), kgrid, dim3(kAuxThreads), 0, stream, a.k, a.ws_kt, a.seqstart_k, a.Hkv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (causal) {
    return alibi ? launch_main<D, BF16, true, true>(a, stream) : launch_main<D, BF16, true, false>(a, stream);
  }
  return alibi ? launch_main<D, BF16, false, true>(a, stream) : launch_main<D, BF16, false, false>(a, stream);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, int D, bool bf16, bool causal, bool alibi, int max_seqlen_q,
                           int max_seqlen_k, hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_backward_d<64, true>(a, causal, alibi, max_seqlen_q, max_seqlen_k, stream)
                : launch_backward_d<64, false>(a, causal, alibi, max_seqlen_q, max_seqlen_k, stream);
  }
  return bf16 ? launch_backward_d<128, true>(a, causal, alibi, max_seqlen_q, max_seqlen_k, stream)
              : launch_backward_d<128, false>(a, causal, alibi, max_seqlen_q, max_seqlen_k, stream);
}

}  // namespace mea
