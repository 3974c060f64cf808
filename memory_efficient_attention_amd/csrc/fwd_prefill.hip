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
//
// Ping-pong: a workgroup is two groups of 4 waves (one workgroup per CU, two
// waves per SIMD, the two waves of a SIMD in different groups).  Barriers cut
// the work into phases, and the groups run one phase apart, so that on every
// SIMD one wave issues matrix products (P V of the previous tile, then Q K of
// this tile) while the other turns its scores into probabilities on the
// vector ALU.  Both groups walk the same key tiles, so each staged K/V tile
// serves 8 waves.
//
// Key tiles run from the causal diagonal backwards, so the largest scores (and,
// with ALiBi, the smallest distance penalties) come first and the running
// maximum rarely has to move; O is rescaled only when some row's maximum grows
// by more than 2^8.  The causal mask and the end of a sequence cost element
// tests only on the tiles that straddle them; tiles entirely above the
// diagonal of the whole workgroup are never loaded.
//
// Staging: both tiles go HBM -> LDS directly (buffer loads with the LDS
// destination, no registers, no vector ALU work), into rings of 3 K and 3 V
// buffers; each wave issues its share of a tile's requests during one of its
// own vector phases, two phases before the tile is needed.  K is read from
// the packed input with a buffer resource bounded by the sequence's rows, so a
// tile that runs past the sequence's end reads zeros instead of its
// neighbours.  V is
// read from V^T tile images that a small pre-pass kernel writes into the
// workspace: each (key/value head, 64-key tile of a sequence) becomes one
// D x 64 image of IEEE halves (bfloat16 V is re-encoded), laid out exactly as
// the LDS tile, so the transposition and conversion happen once per tile
// instead of once per workgroup that reads it.
//
// Grid: the 8 XCDs each take a contiguous run of the (head slice, sequence,
// tile) work items, so the workgroups working on one sequence's K/V at the
// same time share one XCD's L2.  Large batches (at least 32 items per compute
// unit) run persistent workgroups, one per compute unit, that draw the items
// of their XCD's run from a counter; smaller ones one workgroup per item.
#include "mea_common.h"
#include "mea_launch.h"
#include "mea_tiles.h"

namespace mea {

namespace {

constexpr int kThreads = 64 * kPfWaves;  // main kernel: two groups of 4 waves
constexpr int kVtThreads = 256;           // V pre-pass
constexpr int kBufs = 3;                  // LDS buffers of K tiles and of V tiles (a ring of 3 each)
constexpr float kRescaleThreshold = 8.f;  // log2 units: p may reach 2^8 before O is rescaled

template <int D, int ESZ = 2>
struct PfLayout {
  static constexpr int BN = kPfBN;                    // keys per tile
  static constexpr int kBytes = BN * D * ESZ;         // K rows [BN][D] of ESZ-byte values, 16-byte chunks XOR-swizzled
  static constexpr int vBytes = D * BN * 2;           // V^T rows [D][BN] of halves, 16-byte chunks XOR-swizzled
  static constexpr int bufBytes = kBytes + vBytes;
  static constexpr int chunks = D * ESZ / 16;         // 16-byte chunks per K row
  static constexpr int rowsPerKB = 1024 / (D * ESZ);  // K rows per 1 KB direct-load block
  static constexpr int kLoads = kBytes / (kThreads * 16);
  static constexpr int vLoads = vBytes / (kThreads * 16);
};

}  // namespace

// FP8: q, k and v hold OCP e4m3 values (one byte each) and BF16 names the
// output dtype; Q K^T runs on the fp8 matrix cores, V enters P V as halves
// (the pre-pass widens it exactly), and the output is scaled by out_scale.
//
// VBF: bfloat16 V outside the range where IEEE halves are exact.  The
// pre-pass keeps such V^T tiles in bfloat16 and flags them; the normal
// launch (VBF false) runs every work item as usual, and its result for an
// item that reads a flagged tile is wrong.  A second launch with VBF true,
// one workgroup per (sequence, key/value head), computes exactly those items
// again with P V in bfloat16 (V and weights), overwriting their rows: all its
// threads read the sequence's flags at once, so a sequence with none (the
// normal case) costs that one read; otherwise the workgroup runs the items
// of its sequence and head whose key tiles reach the first flagged one, in
// turn.
//
// PERSIST: one workgroup per compute unit that draws work items from the
// per-XCD counters in a.pf_tickets (which must be set) until they run out;
// otherwise one workgroup per item.
template <int D, bool BF16, bool CAUSAL, bool ALIBI, bool PAGED, bool FP8 = false, bool VBF = false,
          bool PERSIST = false>
__global__ __launch_bounds__(kThreads, 1) void fwd_prefill_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses buffer-resource types that exist only for the GPU target
  constexpr int ESZ = FP8 ? 1 : 2;        // bytes per q/k element
  using L = PfLayout<D, ESZ>;
  constexpr int BN = L::BN;
  constexpr int KS = D / 16;             // k-steps of the Q K^T product
  constexpr int NV = 4 * (D / 32);       // products of P V per tile
  constexpr int kStageBytes = kThreads / 64 * 32 * (D + 8) * 2;  // epilogue: a [32][D + 8] tile per wave
  constexpr int kSmemBytes = kBufs * L::bufBytes > kStageBytes ? kBufs * L::bufBytes : kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];

  // VBF: the sequence vb and key/value head vg of this workgroup, the first
  // flagged key tile vfirst of them, and the number of candidate items
  int vb = 0, vg = 0, vfirst = 0, vcand = 0;
  if constexpr (VBF) {
    __shared__ int first_flagged;
    vb = (int)blockIdx.x / a.Hkv;
    vg = (int)blockIdx.x % a.Hkv;
    const int sk = load_const(a.seqstart_k, vb), lk = load_const(a.seqstart_k, vb + 1) - sk;
    const int lq = load_const(a.seqstart_q, vb + 1) - load_const(a.seqstart_q, vb);
    const int ntk = (lk + BN - 1) / BN;
    if (threadIdx.x == 0) first_flagged = ntk;
    __syncthreads();
    const int32_t* fl = a.ws_vflag + ((size_t)(sk / BN) + vb) * a.Hkv + vg;
    for (int t = (int)threadIdx.x; t < ntk; t += kThreads)
      if (fl[(size_t)t * a.Hkv] != 0) atomicMin(&first_flagged, t);
    __syncthreads();
    vfirst = first_flagged;
    if (vfirst >= ntk || lq == 0) return;  // uniform over the workgroup
    const int bt = kPfGroups * 32 * (kPfGroupWaves / a.heads_per_wg);
    vcand = a.head_slices * ((lq + bt - 1) / bt);
  }
  // Persistent workgroups (PERSIST): the work items of XCD x =
  // blockIdx mod 8 are x * per_xcd .. + per_xcd - 1; its n workgroups start
  // with items 0 .. n - 1 of that run and then draw tickets n, n + 1, ...
  // from the XCD's counter, the next ticket fetched while an item runs.
  // Otherwise one item per workgroup, by the XCD-aware remap of blockIdx.
  constexpr bool persistent = PERSIST && !VBF;
  const int xcd = (int)blockIdx.x & 7;
  const int per_xcd = persistent ? (a.pf_items + 7) / 8 : (int)gridDim.x >> 3;
  int ticket = (int)blockIdx.x >> 3;
  __shared__ int next_ticket;
  // the next ticket, before the offset of the first round (lane 0 of wave 0;
  // declared outside the item loop so that no reset of it at the top of the
  // loop has to wait for the previous atomic, or for the stores in flight)
  int ticket_raw = 0;
  for (int vi = 0;; ++vi) {  // VBF: candidate vi; persistent: item vi of this workgroup; otherwise one pass
  // ---- work item (VBF: candidate vi of (vb, vg), or -1 when it reads no
  // flagged tile)
  int w = xcd * per_xcd + ticket;
  if (persistent) {
    if (ticket >= per_xcd) return;  // uniform over the workgroup
    if (threadIdx.x == 0) {
      // lane 0 alone; the lane-dependent offset (0 there) keeps the compiler
      // from aggregating the atomic over the wave, whose result it would
      // broadcast at once: the returned ticket stays in flight while the item
      // runs and is waited for where it is used
      const int lane_zero = (int)__builtin_amdgcn_mbcnt_lo(~0u, 0u);
      ticket_raw = atomicAdd(a.pf_tickets + xcd + lane_zero, 1);
    }
  }
  if constexpr (VBF) {
    if (vi >= vcand) return;
    const int lq = load_const(a.seqstart_q, vb + 1) - load_const(a.seqstart_q, vb);
    const int lk = load_const(a.seqstart_k, vb + 1) - load_const(a.seqstart_k, vb);
    const int bt = kPfGroups * 32 * (kPfGroupWaves / a.heads_per_wg);
    const int nt = (lq + bt - 1) / bt;
    const int t_r = vi % nt, h_s = vi / nt;
    const int first_tok = (nt - 1 - t_r) * bt;
    const int end = CAUSAL ? min(lk, min(first_tok + bt, lq) + lk - lq) : lk;
    const int tiles = end > 0 ? (end + BN - 1) / BN : 0;
    w = tiles > vfirst ? ((vg * a.head_slices + h_s) * a.num_seqs + vb) * a.pf_max_tiles + t_r : -1;
    if (w < 0) continue;
  }
  if (w >= a.pf_items) return;
  const int t_rev = w % a.pf_max_tiles;
  const int rest = w / a.pf_max_tiles;
  const int b = rest % a.num_seqs;
  const int hslice = rest / a.num_seqs;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int grp = wave >> 2;                 // 0 leads, 1 trails by one phase
  const int wq = wave & 3;                   // wave within its group
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int sq0 = load_const(a.seqstart_q, b), Lq = load_const(a.seqstart_q, b + 1) - sq0;
  const int sk0 = load_const(a.seqstart_k, b), Lk = load_const(a.seqstart_k, b + 1) - sk0;
  const int tc = kPfGroupWaves / a.heads_per_wg;  // 32-token chunks per group
  const int BT = kPfGroups * 32 * tc;             // tokens per workgroup
  const int ntiles = (Lq + BT - 1) / BT;
  if (t_rev >= ntiles) {  // uniform over the workgroup: an empty item
    if (!persistent) return;
    if (threadIdx.x == 0) next_ticket = ticket_raw + ((int)gridDim.x >> 3);
    __syncthreads();
    ticket = next_ticket;
    __syncthreads();
    continue;
  }
  const int t0 = (ntiles - 1 - t_rev) * BT;    // longest causal tiles launch first
  const int off = Lk - Lq;                     // query row r sits at key position r + off

  const int g = hslice / a.head_slices;
  const int hs = hslice % a.head_slices;
  const int hw = wq % a.heads_per_wg, tw = wq / a.heads_per_wg;
  const int head = g * a.group + hs * a.heads_per_wg + hw;
  const int tok0 = t0 + 32 * (grp * tc + tw);  // first query row of this wave
  const int my_tok = tok0 + l32;               // this lane's query row
  const bool row_valid = my_tok < Lq;
  const int qpos = my_tok + off;               // key position of this query row

  // key tiles of the whole workgroup (both groups walk the same tiles)
  int kv_end = Lk;
  if constexpr (CAUSAL) kv_end = min(Lk, min(t0 + BT, Lq) + off);
  const int nkt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

  // ---- Q^T operand: lane holds features 16*s + 8*hi .. +7 of its row
  // (fp8: chunk s holds features 64 (s / 2) + 32 hi + 16 (s % 2) .. + 15)
  constexpr int QC = FP8 ? D / 32 : KS;  // 16-byte chunks of Q per lane
  u32x4 qf[QC];
  if constexpr (FP8) {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)(sq0 + my_tok) * a.Hq + head) * D + 32 * hi;
#pragma unroll
    for (int s = 0; s < QC; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_valid) x = *(const u32x4*)(qrow + 64 * (s / 2) + 16 * (s % 2));
      qf[s] = x;
    }
  } else {
    const uint16_t* qrow = a.q + ((size_t)(sq0 + my_tok) * a.Hq + head) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row_valid) x = *(const u32x4*)(qrow + 16 * s);
      qf[s] = x;
    }
  }
  const float c = a.scale_log2;
  float slope2 = 0.f;
  if constexpr (ALIBI) slope2 = a.slopes[head] * kLog2e;

  // ---- staging setup: buffer resources over this sequence's rows of head g
  const uint32_t rs_bytes = (uint32_t)a.Hkv * D * ESZ;   // bytes between key rows
  const uint32_t seq_bytes = Lk > 0 ? (uint32_t)(Lk - 1) * rs_bytes + D * ESZ : 0u;
  const size_t head_off = ((size_t)sk0 * a.Hkv + g) * D;
  const __amdgpu_buffer_rsrc_t krs =
      buf_rsrc(reinterpret_cast<const uint8_t*>(a.k) + head_off * ESZ, seq_bytes);
  // K: direct loads, 1 KB block q = i * 8 + wave (rowsPerKB rows) per instruction
  uint32_t k_voff[L::kLoads];
#pragma unroll
  for (int i = 0; i < L::kLoads; ++i) {
    const int q = i * kPfWaves + wave;
    const int r = q * L::rowsPerKB + lane / L::chunks;
    const int pos = lane % L::chunks;
    k_voff[i] = (uint32_t)r * rs_bytes + (uint32_t)k_pos<D * ESZ / 2>(r, pos) * 16u;
  }
  // V: V^T images of this sequence and head in the workspace (tile ti at
  // ti * Hkv images from the first), loaded 1 KB per instruction per wave
  constexpr int kImgBytes = L::vBytes;
  const int ntk = (Lk + BN - 1) / BN;  // key tiles of the sequence
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(
      a.ws_vt + ((size_t)((sk0 / BN) + b) * a.Hkv + g) * (kImgBytes / 2),
      (uint32_t)ntk * a.Hkv * kImgBytes);

  // tile index of pipeline step t (diagonal tile first) and its LDS buffers
  auto tile_of = [&](int t) { return nkt - 1 - t; };
  auto kbuf = [&](int t) { return smem + (t % kBufs) * L::kBytes; };
  auto vbuf = [&](int t) { return smem + kBufs * L::kBytes + (t % kBufs) * L::vBytes; };

  // K tile of step t.  Paged: the 64-key tile lies in one page (page_size
  // is a multiple of 64); its resource is bounded by the rows of that page
  // the sequence uses, so rows past the sequence's end read zeros.  A block
  // past the table's row or a page index outside [0, num_pages) gets a
  // zero-byte resource: its rows read zeros and no memory is touched.
  auto issue_k = [&](int t) {
    const int kt = tile_of(t) * BN;
    int soff = kt * (int)rs_bytes;
    __amdgpu_buffer_rsrc_t kr = krs;
    if constexpr (PAGED) {
      const int pb = kt / a.page_size;
      const int page = pb < a.max_blocks ? a.block_table[(size_t)b * a.max_blocks + pb] : -1;
      const bool ok = (uint32_t)page < (uint32_t)a.num_pages;
      const uint32_t rows = (uint32_t)min(a.page_size, Lk - pb * a.page_size);
      kr = buf_rsrc(reinterpret_cast<const uint8_t*>(a.k) + ((size_t)(ok ? page : 0) * a.page_size * a.Hkv + g) * D * ESZ,
                    ok ? (rows - 1) * rs_bytes + D * ESZ : 0u);
      soff = (kt - pb * a.page_size) * (int)rs_bytes;
    }
    uint8_t* dst = kbuf(t);
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          kr, (__attribute__((address_space(3))) void*)(dst + (i * kPfWaves + wave) * 1024), 16, k_voff[i], soff, 0, 0);
  };
  auto issue_v = [&](int t) {
    const int vsoff = tile_of(t) * a.Hkv * kImgBytes;
    uint8_t* dst = vbuf(t);
#pragma unroll
    for (int i = 0; i < L::vLoads; ++i) {
      const int blk = i * kPfWaves + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, (__attribute__((address_space(3))) void*)(dst + blk * 1024), 16, (uint32_t)(blk * 1024 + lane * 16), vsoff, 0, 0);
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) o[d] = f32x16{};
  float m_run = kNegInf;
  // Row sums of P.  Where the vector phase is the longer one (ALiBi adds a
  // bias to every score; fp8 halves the Q K^T products), they run on the
  // matrix cores, as a
  // 16x16x32 product of a selector with each 16-key chunk of the P operand.
  // Lane n + 16 u of the P operand holds 8 weights of query n + 16 (u % 2);
  // selector row 0 takes the lanes of query n (u = 0, 2), row 1 those of
  // query n + 16 (u = 1, 3), so lane n < 16 accumulates the row sum of query
  // n in register 0 and of query n + 16 in register 1: the sum of the weights
  // P V used, in float32 (within 2^-11 of the sum of the unrounded ones).
  // bfloat16 weights (VBF) would leave the sum within only 2^-9, too coarse
  // for the log-sum-exp.  Otherwise each lane adds its float32 weights
  // (l_run), which keeps the matrix phase of bf16/fp16 without ALiBi at its
  // 32 products (4 more measured 3 % slower there; 2-3 % faster with ALiBi or fp8).
  constexpr bool kRowSumMfma = (ALIBI || FP8) && !VBF;
  f32x4 lacc = {};
  float l_run = 0.f;
  u32x4 sel = {0u, 0u, 0u, 0u};
  if (((lane & 15) == 0 && (lane & 16) == 0) || ((lane & 15) == 1 && (lane & 16) != 0))
    sel = u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};  // halves 1.0
  auto rowsums = [&](const u32x4 (&pf)[4]) {
    if constexpr (kRowSumMfma) {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) lacc = mfma_16x16x32<false>(sel, pf[ch], lacc);
    }
  };

  // S^T = K Q^T for tile t, K fragments straight from LDS
  auto qk = [&](int t, f32x16 (&s)[2]) {
    const uint8_t* Kb = kbuf(t);
    s[0] = f32x16{};
    s[1] = f32x16{};
    if constexpr (FP8) {
      // K fragment of k-step ks: row r, bytes 64 ks + 32 hi .. + 31 (chunks 4 ks + 2 hi, + 1)
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r = 32 * kb + key_of_row(l32);
          const u32x4 k0 = *(const u32x4*)(Kb + r * D + k_pos<D / 2>(r, 4 * ks + 2 * hi) * 16);
          const u32x4 k1 = *(const u32x4*)(Kb + r * D + k_pos<D / 2>(r, 4 * ks + 2 * hi + 1) * 16);
          s[kb] = mfma_32x32x64_fp8(k0, k1, qf[2 * ks], qf[2 * ks + 1], s[kb]);
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 kf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r = 32 * kb + key_of_row(l32);
          kf[kb] = *(const u32x4*)(Kb + r * (D * 2) + k_pos<D>(r, 2 * ks + hi) * 16);
        }
        s[0] = mfma_32x32x16<BF16>(kf[0], qf[ks], s[0]);
        s[1] = mfma_32x32x16<BF16>(kf[1], qf[ks], s[1]);
      }
      interleave_reads_and_products<2 * KS>();
    }
  };

  // Scores of tile t -> log2 units with bias and masks, row maximum, and the
  // (rare) rescale of O.
  auto prepare = [&](int t, f32x16 (&s)[2]) {
    const int j0 = tile_of(t) * BN;
    const int jlane = j0 + 8 * hi;  // key of register 0 in block 0
    const bool need_mask = (j0 + BN > Lk) || (CAUSAL && j0 + BN - 1 > tok0 + off);
    float mx = kNegInf;
    if constexpr (ALIBI) {
      const float sb = slope2 * (float)(jlane - qpos);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = 32 * kb + key_of_reg(r, 0);
          if constexpr (CAUSAL) s[kb][r] = __builtin_fmaf(s[kb][r], c, __builtin_fmaf(slope2, (float)jl, sb));
          else s[kb][r] = __builtin_fmaf(s[kb][r], c, -slope2 * __builtin_fabsf((float)(jlane + jl - qpos)));
        }
    }
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jlane + 32 * kb + key_of_reg(r, 0);
          if (j >= Lk || (CAUSAL && j > qpos)) s[kb][r] = kNegInf;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
    if constexpr (!ALIBI) mx *= c;  // unscaled scores: the scale (> 0) is folded into the exponent
    mx = halfwave_max(mx);
    if (__any(mx > m_run + kRescaleThreshold)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      if constexpr (!kRowSumMfma) {
        l_run *= alpha;
      } else {  // lane n < 16 holds the sums of queries n and n + 16 (lanes n and n + 16)
        lacc[0] *= alpha;
        lacc[1] *= __shfl(alpha, (lane & 15) + 16);
      }
#pragma unroll
      for (int d = 0; d < D / 32; ++d) o[d] *= alpha;
      m_run = m_new;
    }
  };

  // Probabilities of the prepared scores, packed as the P operand.
  auto probs = [&](f32x16 (&s)[2], u32x4 (&pf)[4], float& lsum) {
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
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
        if constexpr (!kRowSumMfma) lsum += p0 + p1;
        pf[2 * kb + r / 8][(r % 8) / 2] = VBF ? pack_out_x2<true>(p0, p1) : pack_f16x2(p0, p1);
      }
  };

  // O^T += V^T P^T for tile t: V^T fragment of 16-key chunk ch, feature block d
  auto pv = [&](int t, const u32x4 (&pf)[4]) {
    const uint8_t* Vt = vbuf(t);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int ch = i / (D / 32), d = i % (D / 32);
      const u32x4 vf = *(const u32x4*)(Vt + vt_off(32 * d + l32, 2 * ch + hi));
      o[d] = mfma_32x32x16<VBF>(vf, pf[ch], o[d]);
    }
    interleave_reads_and_products<NV>();
  };

  // ---- the ping-pong schedule.  The two waves on each SIMD belong to
  // different groups (waves w and w + 4 share a SIMD).  Phase k is one step
  // between two barriers; a group alternates
  //   matrix phase   M(j): O += V(j-1) P(j-1), then S(j) = K(j) Q^T
  //   vector phase   V(j): softmax update of S(j) -> P(j)
  // and group 1 runs one phase behind group 0, so in every phase one wave of
  // a SIMD feeds the matrix pipe while the other works on the vector ALU:
  // group 0 runs M(j) in phase 2j and V(j) in phase 2j+1, group 1 runs M(j)
  // in phase 2j+1 and V(j-1) in phase 2j.
  //
  // Staging: request R(j) = {K(j+1), V(j)} is split over all 8 waves; each
  // wave issues its share during one of its own vector phases (group 0 in
  // phase 2j-1, group 1 in phase 2j), so the issue cost never lengthens a
  // matrix phase, and every wave waits for its share of R(j) at the end of
  // phase 2j+1.  R(j) lands in the ring slots of K(j-2) and V(j-3), which the
  // last reader (group 1) finished with in phase 2j-3.  Each group runs its
  // own loop, so that within a loop the phase kinds are fixed and the scores
  // and P are never both carried around it.  Both loops pass the same
  // barriers: two per tile and two at the end.
  auto softmax = [&](int t, f32x16 (&s)[2], u32x4 (&pf)[4]) {
    prepare(t, s);
    float lsum = 0.f;
    probs(s, pf, lsum);
    l_run += lsum;
    rowsums(pf);
  };
  auto request = [&](int j) {
    if (j + 1 < nkt) issue_k(j + 1);
    if (j < nkt) issue_v(j);
  };
  // s_waitcnt immediate: at most n vector-memory loads outstanding (other counters unchecked)
  constexpr int kWaitNone = 0;
  constexpr int kWaitV = 0xF70 | L::vLoads;
  constexpr int kWaitKV = 0xF70 | (L::kLoads + L::vLoads);
  static_assert(L::kLoads + L::vLoads < 16, "vmcnt immediate");
  if (nkt > 0) {
    issue_k(0);
    if (grp == 0) request(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 s[2];
    u32x4 pf[4];
    if (grp == 0) {
      for (int j = 0; j < nkt; ++j) {
        if (j >= 1) pv(j - 1, pf);       // phase 2j: M(j)
        qk(j, s);
        __syncthreads();
        request(j + 1);                  // phase 2j+1: V(j), and this wave's share of R(j+1)
        softmax(j, s, pf);
        // this wave's share of R(j) landed; R(j+1) may stay in flight
        if (j + 2 < nkt) __builtin_amdgcn_s_waitcnt(kWaitKV);
        else if (j + 1 < nkt) __builtin_amdgcn_s_waitcnt(kWaitV);
        else __builtin_amdgcn_s_waitcnt(kWaitNone);
        __syncthreads();
      }
      pv(nkt - 1, pf);                   // phase 2 nkt: M(nkt)
      __syncthreads();
      __syncthreads();                   // phase 2 nkt + 1
    } else {
      for (int j = 0; j < nkt; ++j) {
        request(j);                      // phase 2j: V(j-1), and this wave's share of R(j)
        if (j >= 1) softmax(j - 1, s, pf);
        __syncthreads();
        if (j >= 1) pv(j - 1, pf);       // phase 2j+1: M(j)
        qk(j, s);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's share of R(j) landed
        __syncthreads();
      }
      softmax(nkt - 1, s, pf);           // phase 2 nkt: V(nkt-1)
      __syncthreads();
      pv(nkt - 1, pf);                   // phase 2 nkt + 1: M(nkt)
      __syncthreads();
    }
  }

  // ---- epilogue: normalise, round, stage the wave's 32 x D tile through LDS
  // so that every global store writes whole 16-byte runs of a row.
  // the row sum of this lane's query l32 sits in lane l32 % 16, register l32 / 16
  float l_tot;
  if constexpr (!kRowSumMfma) {
    l_tot = halfwave_sum(l_run);
  } else {
    const float ls0 = __shfl(lacc[0], l32 & 15), ls1 = __shfl(lacc[1], l32 & 15);
    l_tot = l32 < 16 ? ls0 : ls1;
  }
  float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if constexpr (FP8) inv *= a.out_scale;
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
  constexpr int kOutChunks = D / 8;     // 16-byte chunks per output row (16-bit values)
  constexpr int RPI = 64 / kOutChunks;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + lane / kOutChunks, ch = lane % kOutChunks;
    if (tok0 + row < Lq) {
      const u32x4 val = *(const u32x4*)(ot + row * (D + 8) + ch * 8);
      __builtin_nontemporal_store(val, (u32x4*)(a.out + ((size_t)(sq0 + tok0 + row) * a.Hq + head) * D + ch * 8));
    }
  }
  if (!VBF && !persistent) break;
  if (persistent && threadIdx.x == 0) next_ticket = ticket_raw + ((int)gridDim.x >> 3);
  __syncthreads();  // the next item reuses the LDS
  if (persistent) {
    ticket = next_ticket;
    __syncthreads();  // every wave has read next_ticket before it is written again
  }
  }
#endif
}

// V pre-pass: the 64 keys of tile i of sequence b and key/value head g become
// one V^T image [D][64] at slot (seqstart_k[b] / 64 + b + i) * Hkv + g of the
// workspace (the slots of consecutive sequences never overlap, since a
// sequence of L keys has at most L / 64 + 1 tiles).  Keys past the
// sequence's end are zero.  Thread (kq, cv) transposes 4 keys x 8 features in
// registers.  The image holds IEEE halves (fp16 V as is, fp8 V widened,
// bfloat16 V re-encoded); a bfloat16 tile whose values the re-encoding would
// not keep (v_needs_bf16) stays bfloat16, and the slot's flag in ws_vflag
// says which (bfloat16 inputs only).
template <int D, bool BF16, bool PAGED, bool FP8 = false>
__global__ __launch_bounds__(kVtThreads) void vt_images_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BN = kPfBN;
  const int g = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  if (a.pf_tickets != nullptr && g == 0 && i == 0 && b == 0 && threadIdx.x < 8) a.pf_tickets[threadIdx.x] = 0;
  const int sk0 = a.seqstart_k[b], Lk = a.seqstart_k[b + 1] - sk0;
  if (i * BN >= Lk) return;  // uniform over the workgroup
  const int tid = threadIdx.x;
  const int kq = tid % (BN / 4), cv = tid / (BN / 4);
  const bool active = cv < D / 8;  // D = 64: half the threads hold no part of the tile
  constexpr int ESZ = FP8 ? 1 : 2;  // bytes per v element
  const uint32_t rs_bytes = (uint32_t)a.Hkv * D * ESZ;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v);
  // the tile's rows, bounded so that rows past the sequence's end read zeros
  // (paged: the tile lies in one page, bounded by the rows the sequence uses)
  __amdgpu_buffer_rsrc_t vrs;
  uint32_t row0;
  if constexpr (PAGED) {
    // a block past the table's row or a page outside [0, num_pages) reads zeros
    const int pb = (i * BN) / a.page_size;
    const int page = pb < a.max_blocks ? a.block_table[(size_t)b * a.max_blocks + pb] : -1;
    const bool ok = (uint32_t)page < (uint32_t)a.num_pages;
    const uint32_t rows = (uint32_t)min(a.page_size, Lk - pb * a.page_size);
    vrs = buf_rsrc(vbase + ((size_t)(ok ? page : 0) * a.page_size * a.Hkv + g) * D * ESZ,
                   ok ? (rows - 1) * rs_bytes + D * ESZ : 0u);
    row0 = (uint32_t)(i * BN - pb * a.page_size);
  } else {
    vrs = buf_rsrc(vbase + ((size_t)sk0 * a.Hkv + g) * D * ESZ, (uint32_t)(Lk - 1) * rs_bytes + D * ESZ);
    row0 = (uint32_t)(i * BN);
  }
  const size_t slot = ((size_t)(sk0 / BN) + b + i) * a.Hkv + g;
  uint8_t* img = reinterpret_cast<uint8_t*>(a.ws_vt + slot * (D * BN));
  if constexpr (FP8) {
    if (active) write_tile_image_fp8(vrs, row0, rs_bytes, img, kq, cv);
  } else {
    u32x4 r[4] = {};
    if (active) load_tile_part(vrs, row0, rs_bytes, kq, cv, r);
    if constexpr (BF16) {
      const bool keep_bf16 = __syncthreads_or(active && v_needs_bf16(tile_part_absmax_bf16(r))) != 0;
      if (!keep_bf16) tile_part_to_f16(r);
      if (tid == 0) a.ws_vflag[slot] = keep_bf16 ? 1 : 0;
    }
    if (active) store_tile_image(r, img, kq, cv);
  }
#endif
}

template <int D, bool BF16, bool PAGED, bool FP8, bool PERSIST>
static hipError_t launch_prefill_d(const FwdArgs& a, bool causal, bool alibi, dim3 grid,
                                   hipStream_t stream) {
  const dim3 block(kThreads);
  if (causal) {
    if (alibi) hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, true, true, PAGED, FP8, false, PERSIST>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, true, false, PAGED, FP8, false, PERSIST>), grid, block, 0, stream, a);
  } else {
    if (alibi) hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, false, true, PAGED, FP8, false, PERSIST>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_prefill_kernel<D, BF16, false, false, PAGED, FP8, false, PERSIST>), grid, block, 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (BF16 && !FP8) {
    // items that read a V^T tile kept in bfloat16, again (one workgroup per
    // sequence and key/value head; almost all of them exit at once)
    const dim3 fgrid((unsigned)a.num_seqs * (unsigned)a.Hkv);
    if (causal) {
      if (alibi) hipLaunchKernelGGL((fwd_prefill_kernel<D, true, true, true, PAGED, false, true>), fgrid, block, 0, stream, a);
      else hipLaunchKernelGGL((fwd_prefill_kernel<D, true, true, false, PAGED, false, true>), fgrid, block, 0, stream, a);
    } else {
      if (alibi) hipLaunchKernelGGL((fwd_prefill_kernel<D, true, false, true, PAGED, false, true>), fgrid, block, 0, stream, a);
      else hipLaunchKernelGGL((fwd_prefill_kernel<D, true, false, false, PAGED, false, true>), fgrid, block, 0, stream, a);
    }
    e = hipGetLastError();
  }
  return e;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int D, bool BF16, bool PAGED, bool FP8 = false>
static hipError_t launch_prefill_dp(const FwdArgs& a, bool causal, bool alibi, int max_seqlen_k,
                                    hipStream_t stream) {
  if (max_seqlen_k > 0 || a.pf_tickets != nullptr) {
    // (with no keys at all the pre-pass only zeroes the tickets)
    const dim3 vgrid(a.Hkv, max(1, (max_seqlen_k + kPfBN - 1) / kPfBN), a.num_seqs);
    hipLaunchKernelGGL((vt_images_kernel<D, BF16, PAGED, FP8>), vgrid, dim3(kVtThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // persistent: one workgroup per compute unit (8 XCDs; the grid is a
  // multiple of 8, at least 8) when there are at least kPersistItemsPerCu
  // items per unit; otherwise one workgroup per item.
  // (64 sequences of U[128, 4096] tokens, 128 items per unit: persistent 1.4 %
  // faster; 4 x 2048 tokens, 4 items per unit: one per item 11 % faster.)
  constexpr long long kPersistItemsPerCu = 32;
  const long long per_item = ((long long)a.pf_items + 7) / 8 * 8;
  const long long cus = (long long)device_cus() / 8 * 8;
  if (a.pf_tickets != nullptr && cus >= 8 && per_item >= kPersistItemsPerCu * cus)
    return launch_prefill_d<D, BF16, PAGED, FP8, true>(a, causal, alibi, dim3((unsigned)cus), stream);
  return launch_prefill_d<D, BF16, PAGED, FP8, false>(a, causal, alibi, dim3((unsigned)per_item), stream);
}

template <int D, bool BF16>
static hipError_t launch_prefill_db(const FwdArgs& a, bool causal, bool alibi, int max_seqlen_k,
                                    hipStream_t stream) {
  return a.block_table != nullptr ? launch_prefill_dp<D, BF16, true>(a, causal, alibi, max_seqlen_k, stream)
                                  : launch_prefill_dp<D, BF16, false>(a, causal, alibi, max_seqlen_k, stream);
}

hipError_t launch_prefill(const FwdArgs& a, int D, bool bf16, bool causal, bool alibi,
                          int max_seqlen_k, hipStream_t stream) {
  if (D == 64) {
    return bf16 ? launch_prefill_db<64, true>(a, causal, alibi, max_seqlen_k, stream)
                : launch_prefill_db<64, false>(a, causal, alibi, max_seqlen_k, stream);
  }
  return bf16 ? launch_prefill_db<128, true>(a, causal, alibi, max_seqlen_k, stream)
              : launch_prefill_db<128, false>(a, causal, alibi, max_seqlen_k, stream);
}

// fp8 (OCP e4m3) q, k, v; D = 128; out_bf16 picks the output dtype; K/V packed
// or in a paged cache (a.block_table).
hipError_t launch_prefill_fp8(const FwdArgs& a, bool out_bf16, bool causal, bool alibi, int max_seqlen_k,
                              hipStream_t stream) {
  if (a.block_table != nullptr)
    return out_bf16 ? launch_prefill_dp<128, true, true, true>(a, causal, alibi, max_seqlen_k, stream)
                    : launch_prefill_dp<128, false, true, true>(a, causal, alibi, max_seqlen_k, stream);
  return out_bf16 ? launch_prefill_dp<128, true, false, true>(a, causal, alibi, max_seqlen_k, stream)
                  : launch_prefill_dp<128, false, false, true>(a, causal, alibi, max_seqlen_k, stream);
}

}  // namespace mea
