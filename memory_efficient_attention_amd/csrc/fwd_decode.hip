// Split-KV attention forward for one query per sequence (the decode case).
//
// This path is bound by HBM bandwidth: every K/V byte of a sequence is read
// once, so the kernels are built to keep as many bytes in flight per CU as
// possible and to spend little else.
//
// Work split: the concatenated key axis [0, total_k) of all sequences (from
// dc_key_base = seqstart_k[dc_seq_base] when only the sequences from
// dc_seq_base on are served: the decode part of a mixed batch) is cut
// into pieces of W keys, W chosen so that the launch is one round of
// equal-sized workgroups on the chip (equal pieces leave no long tail, unlike
// per-sequence chunks of unequal length).  A piece that spans the end of one
// sequence and the start of the next produces one partial result per
// sequence it touches.
//
// Partial kernel: a workgroup of 8 waves (one per CU) takes one piece and
// nh neighbouring key/value heads (with up to 16 query heads of each head's
// group): gcd(Hkv, 4), or gcd(Hkv, 8) for fp8 K/V on long pieces.  The nh heads of a key are adjacent in memory, so a
// workgroup reads runs of nh * D * 2 contiguous bytes per key rather than one
// head's D * 2 bytes out of each token row.  Wave w serves head w % nh, and
// the 8 / nh waves of a head take every (8 / nh)-th 32-key block of the
// piece's part of a sequence, each with its own online-softmax state and no
// workgroup barrier until the end of that part.  Per block, a wave computes
//   S^T = K Q^T   16x16x32 products; the query heads of the group are the 16
//                 columns, so one K/V read serves every head of the group
//                 (GQA's saving becomes fewer HBM bytes);
//   O^T += V^T P^T  with V transposed through a per-wave LDS slot.
// K goes from HBM straight into the product's operand registers; the loads of
// the wave's next block are in flight while a block is computed.  At the end
// of each sequence part the waves of a head merge in LDS and write one
// normalised float32 partial output and its log-sum-exp (log2 units) per
// query head.
//
// Combine kernel: per (sequence, query head) the piece partials are merged
// by their log-sum-exps: lse = log sum_c exp(lse_c), out = sum_c exp(lse_c -
// lse) o_c, then rounded to the output dtype.
#include "mea_common.h"
#include "mea_launch.h"

namespace mea {

namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache policy of the K/V stream loads: non-temporal (the nt bit).  Every K/V
// byte is read once, and with each workgroup reading 1 KB runs of the token
// rows the hint measured ~7% faster than the default policy.
constexpr int kStreamPolicy = 2;

constexpr int kWaves = kDcWaves;
constexpr int kBlk = 32;                  // keys per wave block
constexpr int kVtStride = kBlk + 8;       // elements per V^T row in a wave's LDS slot

}  // namespace

// FP8: q, k and v hold OCP e4m3 values (one byte each) and BF16 names the
// output dtype.  Q K^T runs on the 16x16x128 fp8 products; V is widened to
// IEEE halves (exactly) on its way into the LDS transpose, so P V is the
// 16-bit path's product.  A wave block is then two 32-key sub-blocks, which
// keeps the bytes in flight per wave those of the 16-bit kernel.
template <int D, bool BF16, bool ALIBI, bool PAGED, bool FP8 = false>
__global__ __launch_bounds__(64 * kWaves, 8 / kWaves) void fwd_decode_partial_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses buffer-resource types that exist only for the GPU target
  constexpr int ESZ = FP8 ? 1 : 2;        // bytes per q/k/v element
  constexpr int KS = D / 32;              // k-steps of the 16x16x32 Q K^T product
  constexpr int KR = FP8 ? D / 64 : KS;   // 16-byte K chunks per lane and 16-key half of a sub-block
  constexpr int QR = FP8 ? D / 64 : KS;   // 16-byte Q chunks per lane
  constexpr int NSB = FP8 ? 2 : 1;        // 32-key sub-blocks per wave block
  constexpr int NBUF = 2;                 // register buffers: NBUF - 1 blocks in flight
  constexpr int kBlkKeys = kBlk * NSB;    // keys per wave block
  constexpr int DB = D / 16;              // 16-feature blocks of O^T
  constexpr int VCH = D * ESZ / 128;      // 16-byte V chunks per lane per key
  constexpr int kSlotElems = D * kVtStride;
  constexpr int kRedStride = D + 1;       // floats per query column in the merge buffer
  constexpr int kSmemBytes = kWaves * kSlotElems * 2 > kWaves * 16 * kRedStride * 4 + 2 * kWaves * 16 * 4
                                 ? kWaves * kSlotElems * 2
                                 : kWaves * 16 * kRedStride * 4 + 2 * kWaves * 16 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q = lane & 15, g4 = lane >> 4;
  // grid: one work item per (piece, head group), item = piece * groups +
  // group, so the head groups of one piece are read together and share DRAM
  // pages.  A head group is nh neighbouring key/value heads and one slice of
  // 16 query heads of each head's group.  With more than one slice, the
  // slices of a head read the same key/value rows: items are then remapped so
  // that each XCD (blockIdx mod 8) takes a contiguous run of them and the
  // slices of one piece share that XCD's L2 (measured +7-12 % with 32 query
  // heads on one key/value head; without slices the remap cost ~1.5 %).
  const int nh = a.kv_per_wg, stripes = kWaves / nh;
  const int hh = wave % nh;
  const int groups = (a.Hkv / nh) * a.head_slices;
  int item = (int)blockIdx.x;
  if (a.head_slices > 1) item = ((int)blockIdx.x & 7) * ((int)gridDim.x >> 3) + ((int)blockIdx.x >> 3);
  if (item >= a.dc_pieces * groups) return;
  const int piece = item / groups, gi = item - piece * groups;
  const int g = (gi / a.head_slices) * nh + hh, hs = gi % a.head_slices;
  const int g0 = (gi / a.head_slices) * nh;  // first head of the group

  // the piece: keys [k0, k1) of the concatenated key axis
  const int W = a.chunk_keys;
  const int k0 = a.dc_key_base + piece * W, k1 = min(a.total_k, k0 + W);
  // first sequence that owns a key >= k0: smallest b with seqstart_k[b + 1] > k0
  int b = a.dc_seq_base;
  {
    int hi = a.num_seqs - 1;
    while (b < hi) {
      const int mid = (b + hi) >> 1;
      if (a.seqstart_k[mid + 1] > k0) hi = mid;
      else b = mid + 1;
    }
  }
  for (; b < a.num_seqs; ++b) {
  const int sk0 = a.seqstart_k[b], sk1 = a.seqstart_k[b + 1];
  if (sk0 >= k1) break;
  const int Lk = sk1 - sk0;
  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  if (Lq == 0 || Lk == 0) continue;
  // this segment: keys [c0, c1) of sequence b; its partial goes to slot
  // `slot` of the sequence (slot 0 = the piece holding the sequence's first key)
  const int c0 = max(k0, sk0) - sk0, c1 = min(k1, sk1) - sk0;
  const int slot = piece - (sk0 - a.dc_key_base) / W;
  const int qpos = Lk - 1;  // the single query is the sequence's last position

  const int hl = hs * 16 + q;  // query head within the group (= product column)
  const bool col_valid = hl < a.group;
  const int head = g * a.group + hl;

  // Q^T operand: lane (q, g4) holds 16-byte feature chunk 4*ks + g4 at k-step
  // ks (the K operand uses the same chunks, so a K load instruction reads 64
  // contiguous bytes of each of its 16 rows).  fp8: lane (q, g4) holds bytes
  // 32*g4 .. +31 of the row for the single 16x16x128 product, K the same.
  u32x4 qf[QR];
  {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)sq0 * a.Hq + head) * D * ESZ;
#pragma unroll
    for (int ks = 0; ks < QR; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (col_valid) x = *(const u32x4*)(qrow + (FP8 ? 32 * g4 + 16 * ks : 16 * g4 + 64 * ks));
      qf[ks] = x;
    }
  }
  const float c = a.scale_log2;
  float slope2 = 0.f;
  if constexpr (ALIBI) slope2 = col_valid ? a.slopes[head] * kLog2e : 0.f;

  // K/V rows of this sequence and head, bounded: rows past the end read zeros.
  // With a block table the rows live in pages instead (see load below).
  const uint32_t rs_bytes = (uint32_t)a.Hkv * D * ESZ;
  const uint32_t seq_bytes = (uint32_t)(Lk - 1) * rs_bytes + D * ESZ;
  const size_t head_off = ((size_t)sk0 * a.Hkv + g) * D * ESZ;
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc(reinterpret_cast<const uint8_t*>(a.k) + head_off, seq_bytes);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(reinterpret_cast<const uint8_t*>(a.v) + head_off, seq_bytes);
  // K operand rows: half bb row r = lane & 15 holds key 8*(r/4) + 4*bb + r%4,
  // so that a lane's 8 scores are 8 consecutive keys (the P operand layout)
  uint32_t k_off[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb)
    k_off[bb] = (uint32_t)(8 * (q >> 2) + 4 * bb + (q & 3)) * rs_bytes + (uint32_t)g4 * (FP8 ? 32u : 16u);
  // V staging: lane (kq, cv) loads keys 4kq..4kq+3 x feature chunks cv + 8*x
  const int kq = lane & 7, cv = lane >> 3;
  const uint32_t v_off = (uint32_t)(4 * kq) * rs_bytes + (uint32_t)cv * 16u;
  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * kSlotElems;  // this wave's V^T [D][kVtStride]

  struct Regs {
    u32x4 k[NSB][2][KR];
    u32x4 v[NSB][VCH][4];
  };
  // Block j0 of the sequence.  Paged: the block lies in one page (on the
  // sequence's grid of kBlkKeys = 32 or 64 keys, page_size a multiple of 64);
  // its resource is bounded by the rows of that page the sequence uses, so
  // rows past the sequence's end read zeros whatever the page holds there.
  //
  // Every call issues the same loads: a block past the end of the wave's
  // blocks (valid false), or a sub-block wholly past the segment's end, reads
  // through a resource of zero bytes, so its loads return zeros without a
  // memory access.  Loads behind a branch would leave the compiler's wait
  // counts unable to tell the paths apart, and its merged count would wait
  // for the loads just issued as well as for the block about to be computed.
  const __amdgpu_buffer_rsrc_t none = rows_rsrc(a.k, 0u);
  struct Src {
    __amdgpu_buffer_rsrc_t k, v;
    int soff;
  };
  auto src_of = [&](int j0, bool valid) -> Src {
    Src r{krs, vrs, valid ? j0 * (int)rs_bytes : 0};
    if constexpr (PAGED) {
      if (valid) {
        // a block past the table's row or a page outside [0, num_pages)
        // reads zeros through a zero-byte resource
        const int pb = j0 / a.page_size;
        const int page = pb < a.max_blocks ? a.block_table[(size_t)b * a.max_blocks + pb] : -1;
        const bool ok = (uint32_t)page < (uint32_t)a.num_pages;
        const uint32_t rows = (uint32_t)min(a.page_size, Lk - pb * a.page_size);
        const uint32_t bytes = ok ? (rows - 1) * rs_bytes + D * ESZ : 0u;
        const size_t off = ((size_t)(ok ? page : 0) * a.page_size * a.Hkv + g) * D * ESZ;
        r.k = rows_rsrc(reinterpret_cast<const uint8_t*>(a.k) + off, bytes);
        r.v = rows_rsrc(reinterpret_cast<const uint8_t*>(a.v) + off, bytes);
        r.soff = (j0 - pb * a.page_size) * (int)rs_bytes;
      }
    }
    return r;
  };
  auto load = [&](Regs& R, int j0, bool valid) {
    const Src sr = src_of(j0, valid);
    const int soff = sr.soff;
    const __amdgpu_buffer_rsrc_t kr = sr.k, vr = sr.v;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const bool live = valid && (sb == 0 || j0 + kBlk * sb < c1);
      const __amdgpu_buffer_rsrc_t ks_r = live ? kr : none, vs_r = live ? vr : none;
      const int so = live ? soff + kBlk * sb * (int)rs_bytes : 0;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int ks = 0; ks < KR; ++ks)
          R.k[sb][bb][ks] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(ks_r, k_off[bb] + (FP8 ? 16 : 64) * ks, so, kStreamPolicy));
#pragma unroll
      for (int x = 0; x < VCH; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          R.v[sb][x][i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(vs_r, v_off + i * rs_bytes + x * 128, so, kStreamPolicy));
    }
  };

  f32x4 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  bool redo = false;  // a block of this wave was left to the second walk

  // One 32-key sub-block sb of a block at key j0.  bfloat16 V normally
  // enters P V as IEEE halves.  A block that holds a value outside the range
  // where that is exact (v_needs_bf16 of its largest |v|, decided per wave)
  // is skipped by the main walk (REDO false), which only notes that there is
  // one, and computed in a second walk over the wave's blocks (REDO true)
  // that takes just such blocks, with V and P in bfloat16.  Keeping the rare
  // case out of the main walk keeps that walk within the register budget.
  auto compute_sub = [&](auto redo_c, Regs& R, int sb, int j0) {
    constexpr bool REDO = decltype(redo_c)::value;
    // V block -> LDS, transposed (and re-encoded as IEEE half for bfloat16)
    if constexpr (FP8) {
      // lane (kq, cv) holds features 16 cv .. + 15 of keys 4 kq .. + 3; word
      // w of key i widens to the half pairs (4w, 4w + 1) and (4w + 2, 4w + 3)
      const u32x4 a0 = R.v[sb][0][0], a1 = R.v[sb][0][1], a2 = R.v[sb][0][2], a3 = R.v[sb][0][3];
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int hsel = 0; hsel < 2; ++hsel) {
          const uint32_t h0 = fp8x2_to_f16x2(a0[w], hsel), h1 = fp8x2_to_f16x2(a1[w], hsel);
          const uint32_t h2 = fp8x2_to_f16x2(a2[w], hsel), h3 = fp8x2_to_f16x2(a3[w], hsel);
          const int d = 16 * cv + 4 * w + 2 * hsel;
          u32x2 even, odd;
          even[0] = __builtin_amdgcn_perm(h1, h0, 0x05040100u);
          even[1] = __builtin_amdgcn_perm(h3, h2, 0x05040100u);
          odd[0] = __builtin_amdgcn_perm(h1, h0, 0x07060302u);
          odd[1] = __builtin_amdgcn_perm(h3, h2, 0x07060302u);
          *(u32x2*)(vt + d * kVtStride + 4 * kq) = even;
          *(u32x2*)(vt + (d + 1) * kVtStride + 4 * kq) = odd;
        }
    } else {
    // transposed store of lane (kq, cv)'s 4 keys x 8 features of chunk x
    auto store_vt = [&](const u32x4& a0, const u32x4& a1, const u32x4& a2, const u32x4& a3, int x) {
      const int d0 = 8 * (cv + 8 * x);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2 even, odd;
        even[0] = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);
        even[1] = __builtin_amdgcn_perm(a3[w], a2[w], 0x05040100u);
        odd[0] = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);
        odd[1] = __builtin_amdgcn_perm(a3[w], a2[w], 0x07060302u);
        *(u32x2*)(vt + (d0 + 2 * w) * kVtStride + 4 * kq) = even;
        *(u32x2*)(vt + (d0 + 2 * w + 1) * kVtStride + 4 * kq) = odd;
      }
    };
    float vmax = 0.f;  // bfloat16: the block's largest |v|
    if constexpr (REDO) {
#pragma unroll
      for (int x = 0; x < VCH; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int w = 0; w < 4; ++w) vmax = bf16x2_absmax(vmax, R.v[sb][x][i][w]);
      if (!__any(v_needs_bf16(vmax))) return;  // done in the main walk
#pragma unroll
      for (int x = 0; x < VCH; ++x) store_vt(R.v[sb][x][0], R.v[sb][x][1], R.v[sb][x][2], R.v[sb][x][3], x);
    } else {
#pragma unroll
      for (int x = 0; x < VCH; ++x) {
        u32x4 a0 = R.v[sb][x][0], a1 = R.v[sb][x][1], a2 = R.v[sb][x][2], a3 = R.v[sb][x][3];
        if constexpr (BF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            vmax = bf16x2_absmax(bf16x2_absmax(vmax, a0[w]), a1[w]);
            vmax = bf16x2_absmax(bf16x2_absmax(vmax, a2[w]), a3[w]);
            a0[w] = bf16x2_to_f16x2(a0[w]);
            a1[w] = bf16x2_to_f16x2(a1[w]);
            a2[w] = bf16x2_to_f16x2(a2[w]);
            a3[w] = bf16x2_to_f16x2(a3[w]);
          }
        }
        store_vt(a0, a1, a2, a3, x);
      }
      if constexpr (BF16) {
        if (__any(v_needs_bf16(vmax))) {  // left to the second walk
          redo = true;
          return;
        }
      }
    }
    }
    // scores: lane (q, g4) gets keys j0 + 8*g4 + 0..7 of column q
    f32x4 s[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      s[bb] = f32x4{};
      if constexpr (FP8) {
        s[bb] = mfma_16x16x128_fp8(R.k[sb][bb][0], R.k[sb][bb][1], qf[0], qf[1], s[bb]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[bb] = mfma_16x16x32<BF16>(R.k[sb][bb][ks], qf[ks], s[bb]);
      }
    }
    const int jlane = j0 + 8 * g4;
    float x[8];
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sc = s[e / 4][e % 4];
      if constexpr (ALIBI) x[e] = __builtin_fmaf(sc, c, slope2 * (float)(jlane + e - qpos));
      else x[e] = sc * c;
    }
    // element tests only on a segment's last block (and, paged, its first):
    // a wave-uniform branch
    if (j0 + kBlk > c1 || (PAGED && j0 < c0)) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (jlane + e >= c1 || (PAGED && jlane + e < c0)) x[e] = kNegInf;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = __builtin_fmaxf(mx, x[e]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run + 8.f)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    u32x4 pf;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = fast_exp2(x[e] - m_use), p1 = fast_exp2(x[e + 1] - m_use);
      l_run += p0 + p1;
      pf[e / 2] = REDO ? pack_out_x2<true>(p0, p1) : pack_f16x2(p0, p1);
    }
    // O^T += V^T P^T: V^T fragment of feature block d is row 16d + q, keys 8*g4..+7
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const u32x4 vf = *(const u32x4*)(vt + (16 * d + q) * kVtStride + 8 * g4);
      o[d] = mfma_16x16x32<REDO>(vf, pf, o[d]);
    }
  };
  auto compute = [&](Regs& R, int j0) {
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      if (sb > 0 && j0 + kBlk * sb >= c1) break;
      compute_sub(std::false_type{}, R, sb, j0 + kBlk * sb);
    }
  };

  // Blocks of kBlkKeys keys from cb (paged: on the sequence's kBlkKeys-key
  // grid so that none crosses a page, keys before c0 masked in the first
  // block; packed: from c0).  The `stripes` waves of a head take every stripes-th
  // block, wave w from block w / nh on: a fixed split, so that the result is
  // the same from run to run (blocks claimed from a shared LDS counter measured
  // no faster).
  const int cb = PAGED ? (c0 & ~(kBlkKeys - 1)) : c0;
  const int nblk = (c1 - cb + kBlkKeys - 1) / kBlkKeys;
  int next_own = wave / nh;
  auto next_block = [&]() -> int {
    const int v = next_own;
    next_own += stripes;
    return v;
  };
  // A ring of NBUF register buffers: buffer u holds block jb[u]; the load of
  // the block NBUF - 1 places ahead is issued before each compute, so NBUF -
  // 1 blocks stay in flight.  A wave's blocks only grow, so the first block
  // past the end ends its walk.
  Regs rg[NBUF];
  int jb[NBUF];
#pragma unroll
  for (int u = 0; u + 1 < NBUF; ++u) {
    jb[u] = next_block();
    load(rg[u], cb + kBlkKeys * jb[u], jb[u] < nblk);
  }
  for (bool more = true; more;) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      if (jb[u] >= nblk) {
        more = false;
        break;
      }
      const int un = (u + NBUF - 1) % NBUF;
      jb[un] = next_block();
      load(rg[un], cb + kBlkKeys * jb[un], jb[un] < nblk);
      compute(rg[u], cb + kBlkKeys * jb[u]);
    }
  }

  // The second walk (bfloat16 only, rare): the wave's blocks again, those
  // that need bfloat16 V computed.  redo is wave-uniform.
  if constexpr (BF16 && !FP8) {
    if (redo) {
      for (int jw = wave / nh; jw < nblk; jw += stripes) {
        load(rg[0], cb + kBlkKeys * jw, true);
        compute_sub(std::true_type{}, rg[0], 0, cb + kBlkKeys * jw);
      }
    }
  }

  // ---- merge the partial states of the waves that share a head, in LDS
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [4][16][kRedStride]
  float* mred = red + kWaves * 16 * kRedStride;  // [4][16]
  float* lred = mred + kWaves * 16;              // [4][16]
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 16 + q) * kRedStride + 16 * d + 4 * g4 + r] = o[d][r];
  if (g4 == 0) {
    mred[wave * 16 + q] = m_run;
    lred[wave * 16 + q] = l_run;
  }
  __syncthreads();

  // thread (qc, part): query column qc, features part*FP..+FP-1, for each of
  // the nh heads in turn; the waves of head h2 are h2, h2 + nh, ...
  constexpr int kParts = 4 * kWaves, FP = D / kParts;
  const int qc = tid / kParts, part = tid % kParts;
  for (int h2 = 0; h2 < nh && hs * 16 + qc < a.group; ++h2) {
    float M = kNegInf;
#pragma unroll
    for (int s2 = 0; s2 < kWaves; ++s2)
      if (s2 < stripes) M = __builtin_fmaxf(M, mred[(s2 * nh + h2) * 16 + qc]);
    float wgt[kWaves], Ls = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kWaves; ++s2) {
      wgt[s2] = 0.f;
      if (s2 < stripes) {
        const float mw = mred[(s2 * nh + h2) * 16 + qc];
        wgt[s2] = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
        Ls += wgt[s2] * lred[(s2 * nh + h2) * 16 + qc];
      }
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    const int hq = (g0 + h2) * a.group + hs * 16 + qc;
    const size_t prow = ((size_t)(b - a.dc_seq_base) * a.max_chunks + slot) * a.Hq + hq;
    float* dst = a.ws_o + prow * D + part * FP;
#pragma unroll
    for (int e = 0; e < FP; ++e) {
      const int d = part * FP + e;
      float acc = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < kWaves; ++s2)
        if (s2 < stripes) acc += wgt[s2] * red[((s2 * nh + h2) * 16 + qc) * kRedStride + d];
      dst[e] = acc * inv;
    }
    if (part == 0) a.ws_lse[prow] = Ls > 0.f ? M + fast_log2(Ls) : kNegInf;
  }
  __syncthreads();  // the merge buffer is reused by the next segment
  }
#endif
}

// One wave per (sequence, query head).  The wave reads D/8 lanes to a partial
// row (8 features, 32 bytes a lane), 512/D rows side by side and four such
// loads in flight, so that a sequence split into hundreds of pieces is
// combined with 16 (D 128) or 32 (D 64) rows in flight instead of a row at a
// time.  The chunk log-sum-exps are reduced across the wave first; the lane
// groups' sums are added with cross-lane shuffles at the end.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fwd_decode_combine_kernel(FwdArgs a) {
  constexpr int LPR = D / 8;    // lanes per partial row
  constexpr int RPL = 64 / LPR;  // partial rows per wave-wide load
  constexpr int U = 4;           // wave-wide loads in flight
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPR, f0 = (lane % LPR) * 8;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = a.dc_seq_base + (int)blockIdx.y;
  if (h >= a.Hq) return;
  const int sq0 = a.seqstart_q[b], Lq = a.seqstart_q[b + 1] - sq0;
  if (Lq == 0) return;
  const int sk0 = a.seqstart_k[b] - a.dc_key_base, sk1 = a.seqstart_k[b + 1] - a.dc_key_base;
  // partial slots of sequence b: one per piece of the key axis its keys touch
  const int nch = sk1 > sk0 ? (sk1 - 1) / a.chunk_keys - sk0 / a.chunk_keys + 1 : 0;
  const size_t row0 = (size_t)(b - a.dc_seq_base) * a.max_chunks * a.Hq + h;  // partial row of chunk 0
  const float* lse_p = a.ws_lse + row0;                        // chunk c at [c * Hq]
  float M = kNegInf;
  for (int ch = lane; ch < nch; ch += 64) M = __builtin_fmaxf(M, lse_p[(size_t)ch * a.Hq]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = __builtin_fmaxf(M, __shfl_xor(M, m));
  float S = 0.f;
  float acc[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) acc[f] = 0.f;
  if (M != kNegInf) {
    const float* o_p = a.ws_o + row0 * D + f0;  // chunk c at [c * Hq * D]
    const size_t ostride = (size_t)a.Hq * D;
    auto add = [&](float lc, const float4& x0, const float4& x1) {
      const float w = (lc == kNegInf) ? 0.f : fast_exp2(lc - M);
      S += w;
      acc[0] += w * x0.x; acc[1] += w * x0.y; acc[2] += w * x0.z; acc[3] += w * x0.w;
      acc[4] += w * x1.x; acc[5] += w * x1.y; acc[6] += w * x1.z; acc[7] += w * x1.w;
    };
    int ch = grp;
    for (; ch + (U - 1) * RPL < nch; ch += U * RPL) {
      float lc[U];
      float4 x[U][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t c = (size_t)(ch + u * RPL);
        lc[u] = lse_p[c * a.Hq];
        x[u][0] = *(const float4*)(o_p + c * ostride);
        x[u][1] = *(const float4*)(o_p + c * ostride + 4);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) add(lc[u], x[u][0], x[u][1]);
    }
    for (; ch < nch; ch += RPL)
      add(lse_p[(size_t)ch * a.Hq], *(const float4*)(o_p + (size_t)ch * ostride),
          *(const float4*)(o_p + (size_t)ch * ostride + 4));
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) {
    S += __shfl_xor(S, m);
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[f] += __shfl_xor(acc[f], m);
  }
  const float inv = (S > 0.f ? 1.f / S : 0.f) * a.out_scale;  // out_scale: 1, or the fp8 V scale
  if (grp == 0) {
    uint4 o;
    o.x = pack_out_x2<BF16>(acc[0] * inv, acc[1] * inv);
    o.y = pack_out_x2<BF16>(acc[2] * inv, acc[3] * inv);
    o.z = pack_out_x2<BF16>(acc[4] * inv, acc[5] * inv);
    o.w = pack_out_x2<BF16>(acc[6] * inv, acc[7] * inv);
    *(uint4*)(a.out + ((size_t)sq0 * a.Hq + h) * D + f0) = o;
  }
  if (lane == 0 && a.lse != nullptr)
    a.lse[(size_t)h * a.total_q + sq0] = S > 0.f ? (M + fast_log2(S)) * kLn2 : kNegInf;
}

template <int D, bool BF16>
static hipError_t launch_decode_d(const FwdArgs& a, bool alibi, hipStream_t stream) {
  if (a.dc_pieces > 0) {
    const dim3 grid((unsigned)(((long long)a.dc_pieces * ((a.Hkv / a.kv_per_wg) * a.head_slices) + 7) / 8 * 8));
    const dim3 block(64 * kWaves);
    if (a.block_table != nullptr) {
      if (alibi) hipLaunchKernelGGL((fwd_decode_partial_kernel<D, BF16, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((fwd_decode_partial_kernel<D, BF16, false, true>), grid, block, 0, stream, a);
    } else {
      if (alibi) hipLaunchKernelGGL((fwd_decode_partial_kernel<D, BF16, true, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((fwd_decode_partial_kernel<D, BF16, false, false>), grid, block, 0, stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((fwd_decode_combine_kernel<D, BF16>), dim3((a.Hq + 3) / 4, a.num_seqs - a.dc_seq_base), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// fp8 (OCP e4m3) q, k, v; D = 128; out_bf16 picks the output dtype; K/V packed
// or in a paged cache (a.block_table).
template <bool OUT_BF16, bool PAGED>
static void launch_decode_fp8_partial(const FwdArgs& a, bool alibi, dim3 grid, dim3 block, hipStream_t stream) {
  if (alibi) hipLaunchKernelGGL((fwd_decode_partial_kernel<128, OUT_BF16, true, PAGED, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((fwd_decode_partial_kernel<128, OUT_BF16, false, PAGED, true>), grid, block, 0, stream, a);
}

hipError_t launch_decode_fp8(const FwdArgs& a, bool out_bf16, bool alibi, hipStream_t stream) {
  if (a.dc_pieces > 0) {
    const dim3 grid((unsigned)(((long long)a.dc_pieces * ((a.Hkv / a.kv_per_wg) * a.head_slices) + 7) / 8 * 8));
    const dim3 block(64 * kWaves);
    const bool paged = a.block_table != nullptr;
    if (out_bf16) {
      if (paged) launch_decode_fp8_partial<true, true>(a, alibi, grid, block, stream);
      else launch_decode_fp8_partial<true, false>(a, alibi, grid, block, stream);
    } else {
      if (paged) launch_decode_fp8_partial<false, true>(a, alibi, grid, block, stream);
      else launch_decode_fp8_partial<false, false>(a, alibi, grid, block, stream);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (out_bf16) hipLaunchKernelGGL((fwd_decode_combine_kernel<128, true>), dim3((a.Hq + 3) / 4, a.num_seqs - a.dc_seq_base), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((fwd_decode_combine_kernel<128, false>), dim3((a.Hq + 3) / 4, a.num_seqs - a.dc_seq_base), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const FwdArgs& a, int D, bool bf16, bool alibi, hipStream_t stream) {
  if (D == 64) return bf16 ? launch_decode_d<64, true>(a, alibi, stream) : launch_decode_d<64, false>(a, alibi, stream);
  return bf16 ? launch_decode_d<128, true>(a, alibi, stream) : launch_decode_d<128, false>(a, alibi, stream);
}

}  // namespace mea
