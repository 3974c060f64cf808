// SwiGLU feed-forward layer on the gfx950 matrix cores:
//   hidden = SiLU(x W_gate^T) * (x W_up^T)     [tokens, d_ff]
//   out    = hidden W_down^T                   [tokens, d_model]
// with SiLU(z) = z sigmoid(z).  Weights are in the out_features x in_features
// layout, so both operands of every product run along k in memory: a lane's
// MFMA fragment is one 16-byte row chunk of each, and no operand is ever
// transposed.
//
// One kernel template serves both products.  A workgroup of 8 waves (4 along
// M x 2 along N) computes a 256 x 256 output tile over k-steps of 64:
//   GATED   the tile is 256 rows x 128 columns of both the gate and the up
//           product (each wave 64 x 64 of each), and the epilogue writes
//           SiLU(gate) * up;
//   plain   256 x 256 of one product (each wave 64 x 128).
// Either way a wave keeps 128 float32 accumulators and issues 32 MFMAs per
// k-step.  Operand tiles go HBM -> LDS by buffer loads with an LDS
// destination into two stage buffers (a request one k-step ahead, one barrier
// per k-step, placed before the k-step's last 8 products so that they run
// while the next stage's first fragments are read); rows of 64 values are 128
// bytes with their 16-byte chunks XOR-swizzled so that the 16 rows a fragment
// read touches hit 16 different bank groups.  Rows past `rows` read zeros and
// are never stored.
//
// Work order: groups of 4 row tiles walk every column tile before the next
// group starts, remapped so that each XCD takes a contiguous run of
// (column tile, row tile) items: the 32 workgroups an XCD runs at once share
// 4 row tiles and 8 column tiles, a weight column tile is read from HBM once
// per group and then served from L2, and the row tiles of a group stay in the
// infinity cache (groups of 4 measured 1.2-1.5 % faster than 8 and 3-20 %
// faster than 1, 16 or 32).
#include "mea_common.h"
#include "mea_launch.h"
#include "mea_tiles.h"

namespace mea {

namespace {

constexpr int kFfThreads = 512;
constexpr int kBM = 256;   // output rows per workgroup
constexpr int kBK = 64;    // k per stage
constexpr int kRowBytes = kBK * 2;                 // one 64-value row of a stage tile
constexpr int kTileBytes = kBM * kRowBytes;        // 256 rows = 32 KB
constexpr int kStageBytes = 2 * kTileBytes;        // A tile + B tile(s)
constexpr int kGroupRows = 4;                      // row tiles per group of the work order

// position of 16-byte chunk c of row r in a 128-byte-row tile
__device__ __forceinline__ int ff_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ float silu(float z) {
  return z / (1.f + fast_exp2(-z * kLog2e));
}

}  // namespace

struct FfnArgs {
  const uint16_t* a;     // [rows, K]
  const uint16_t* b0;    // [N0, K]  (GATED: W_gate)
  const uint16_t* b1;    // [N0, K]  (GATED: W_up; else unused)
  uint16_t* c;           // [rows, N]
  int32_t rows;          // M
  int32_t n;             // columns of the output
  int32_t k;             // a multiple of 64
  int32_t row_tiles;     // ceil(rows / 256)
  int32_t col_tiles;     // n / (GATED ? 128 : 256)
};

template <bool BF16, bool GATED>
__global__ __launch_bounds__(kFfThreads) void ffn_gemm_kernel(FfnArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BN = GATED ? 128 : 256;       // output columns per workgroup
  constexpr int NB = GATED ? 2 : 4;           // 32-column blocks per wave and product
  constexpr int kOutPitch = (GATED ? 64 : 128) + 8;  // staged output row (elements)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];

  // ---- work item: XCD-aware remap, then groups of 4 row tiles x all column tiles
  const int items = p.row_tiles * p.col_tiles;
  const int per_xcd = (int)gridDim.x >> 3;
  const int w = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
  if (w >= items) return;
  const int group = w / (kGroupRows * p.col_tiles);
  const int first_row_tile = group * kGroupRows;
  const int rows_in_group = min(kGroupRows, p.row_tiles - first_row_tile);
  const int in_group = w - group * kGroupRows * p.col_tiles;
  const int mt = first_row_tile + in_group % rows_in_group;
  const int nt = in_group / rows_in_group;
  const int m0 = mt * kBM, n0 = nt * BN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;   // 4 waves along M, 2 along N

  // ---- staging: A rows m0.., B rows n0.. (GATED: gate rows in the first 128
  // tile rows, up rows in the last 128), 64 values of k per stage
  const uint32_t row_stride = (uint32_t)p.k * 2;
  const int a_rows = min(kBM, p.rows - m0);
  const __amdgpu_buffer_rsrc_t ars = buf_rsrc(p.a + (size_t)m0 * p.k, (uint32_t)a_rows * row_stride);
  const __amdgpu_buffer_rsrc_t b0rs = buf_rsrc(p.b0 + (size_t)n0 * p.k, (uint32_t)BN * row_stride);
  const __amdgpu_buffer_rsrc_t b1rs = GATED ? buf_rsrc(p.b1 + (size_t)n0 * p.k, (uint32_t)BN * row_stride) : b0rs;
  // 1 KB direct-load block blk = i * 8 + wave covers rows 8 blk .. 8 blk + 7
  constexpr int kLoads = kTileBytes / (kFfThreads * 16);  // 4 per tile
  uint32_t voff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = (i * 8 + wave) * 8 + lane / 8;
    voff[i] = (uint32_t)(r % 128) * row_stride + (uint32_t)ff_pos(r, lane % 8) * 16u;
  }
  auto issue = [&](int ks) {
    uint8_t* buf = smem + (ks & 1) * kStageBytes;
    const int soff = ks * kRowBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int blk = i * 8 + wave;
      // A: rows 0..255 of the tile; voff carries r % 128, the upper half adds 128 rows
      load_lds16(ars, buf + blk * 1024, voff[i] + (blk >= 16 ? 128u * row_stride : 0u), soff);
      if constexpr (GATED) {
        load_lds16(blk < 16 ? b0rs : b1rs, buf + kTileBytes + blk * 1024, voff[i], soff);
      } else {
        load_lds16(b0rs, buf + kTileBytes + blk * 1024, voff[i] + (blk >= 16 ? 128u * row_stride : 0u), soff);
      }
    }
  };

  f32x16 acc[2][2 * NB / (GATED ? 1 : 2)];   // [m block][n block] (GATED: gate blocks 0..1, up blocks 2..3)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2 * NB / (GATED ? 1 : 2); ++j) acc[i][j] = f32x16{};

  // Fragments of sub-step kk + 1 are read into the other half of a register
  // double buffer while the products of sub-step kk run.  The barrier that
  // publishes stage ks + 1 sits before the last sub-step's products of stage
  // ks, whose fragments are then in registers: after it those products keep
  // the matrix pipe busy while the first fragments of stage ks + 1 arrive.
  constexpr int NJ = 2 * NB / (GATED ? 1 : 2);  // B fragments per sub-step
  constexpr int KK = kBK / 16;                  // sub-steps per k-step
  constexpr int NR = 2 + NJ;                    // fragment reads per sub-step
  constexpr int NP = 2 * NJ;                    // products per sub-step
  static_assert(NR <= NP, "reads interleave with products");
  u32x4 af[2][2], bf[2][NJ];
  auto read_frags = [&](const uint8_t* A, const uint8_t* B, int kk, int slot) {
    const int c = 2 * kk + hi;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r = 64 * wm + 32 * mb + l32;
      af[slot][mb] = *(const u32x4*)(A + r * kRowBytes + ff_pos(r, c) * 16);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      // GATED: j < 2 gate columns 64 wn + 32 j, j >= 2 up columns 128 + 64 wn + 32 (j - 2)
      const int r = GATED ? (j < 2 ? 64 * wn + 32 * j : 128 + 64 * wn + 32 * (j - 2)) + l32
                          : 128 * wn + 32 * j + l32;
      bf[slot][j] = *(const u32x4*)(B + r * kRowBytes + ff_pos(r, c) * 16);
    }
  };
  auto products = [&](int slot) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[mb][j] = mfma_32x32x16<BF16>(af[slot][mb], bf[slot][j], acc[mb][j]);
  };
  // one product, one read in turn, then the remaining products
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NP - NR, 0);
  };

  const int nks = p.k / kBK;
  issue(0);
  if (nks > 1) {
    issue(1);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(2 * kLoads));  // stage 0 landed, stage 1 may be in flight
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  read_frags(smem, smem + kTileBytes, 0, 0);
  for (int ks = 0; ks < nks; ++ks) {
    const uint8_t* A = smem + (ks & 1) * kStageBytes;
    const uint8_t* B = A + kTileBytes;
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) {
      read_frags(A, B, kk + 1, (kk + 1) & 1);
      products(kk & 1);
    }
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) interleave();
    // the last sub-step's fragments are in registers and this wave's share of
    // stage ks + 1 has landed; after the barrier nobody reads stage ks again
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ks + 2 < nks) issue(ks + 2);
    const uint8_t* An = smem + ((ks + 1) & 1) * kStageBytes;
    read_frags(An, An + kTileBytes, 0, 0);  // past the last stage: unused LDS reads
    products((KK - 1) & 1);
    interleave();
  }
  __syncthreads();

  // ---- epilogue: rows 64 wm + 32 mb + acc_row(r, hi), column l32 of block j.
  // Each 32-row block is staged per wave as [32][cols + 8] (at most 68 KB for
  // 8 waves) so that the stores are 16-byte row runs.
  constexpr int kOutCols = GATED ? 64 : 128;
  constexpr int kChunks = kOutCols / 8;         // 16-byte chunks per staged row
  constexpr int kRowsPerStore = 64 / kChunks;
  static_assert(8 * 32 * kOutPitch * 2 <= 2 * kStageBytes, "epilogue staging fits the stage buffers");
  uint16_t* st = reinterpret_cast<uint16_t*>(smem) + wave * 32 * kOutPitch;
  const int col0 = n0 + kOutCols * wn;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int j = 0; j < kOutCols / 32; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = acc[mb][j][r];
        if constexpr (GATED) v = silu(v) * acc[mb][j + 2][r];
        st[acc_row(r, hi) * kOutPitch + 32 * j + l32] = (uint16_t)(pack_out_x2<BF16>(v, 0.f) & 0xffffu);
      }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 32 / kRowsPerStore; ++i) {
      const int row = i * kRowsPerStore + lane / kChunks, ch = lane % kChunks;
      const int grow = m0 + 64 * wm + 32 * mb + row;
      if (grow < p.rows)
        __builtin_nontemporal_store(*(const u32x4*)(st + row * kOutPitch + ch * 8), (u32x4*)(p.c + (size_t)grow * p.n + col0 + ch * 8));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
#endif
}

namespace {

template <bool BF16>
hipError_t launch_ffn_d(const uint16_t* x, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, uint16_t* h,
                        uint16_t* y, int tokens, int d_model, int d_ff, hipStream_t stream) {
  const int row_tiles = (tokens + kBM - 1) / kBM;
  FfnArgs up{x, wg, wu, h, tokens, d_ff, d_model, row_tiles, d_ff / 128};
  const long long up_items = (long long)row_tiles * up.col_tiles;
  hipLaunchKernelGGL((ffn_gemm_kernel<BF16, true>), dim3((unsigned)((up_items + 7) / 8 * 8)), dim3(kFfThreads), 0,
                     stream, up);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FfnArgs down{h, wd, nullptr, y, tokens, d_model, d_ff, row_tiles, d_model / 256};
  const long long down_items = (long long)row_tiles * down.col_tiles;
  hipLaunchKernelGGL((ffn_gemm_kernel<BF16, false>), dim3((unsigned)((down_items + 7) / 8 * 8)), dim3(kFfThreads),
                     0, stream, down);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swiglu_ffn(const void* x, const void* w_gate, const void* w_up, const void* w_down, void* hidden,
                             void* out, int tokens, int d_model, int d_ff, bool bf16, hipStream_t stream) {
  auto u = [](const void* q) { return static_cast<const uint16_t*>(q); };
  if (bf16)
    return launch_ffn_d<true>(u(x), u(w_gate), u(w_up), u(w_down), static_cast<uint16_t*>(hidden),
                              static_cast<uint16_t*>(out), tokens, d_model, d_ff, stream);
  return launch_ffn_d<false>(u(x), u(w_gate), u(w_up), u(w_down), static_cast<uint16_t*>(hidden),
                             static_cast<uint16_t*>(out), tokens, d_model, d_ff, stream);
}

}  // namespace mea
