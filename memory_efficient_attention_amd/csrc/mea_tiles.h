// LDS tile layouts and staging helpers shared by the prefill forward and the
// backward kernels (gfx950 / CDNA4 only).
#pragma once

#include "mea_common.h"

namespace mea {

// Position of 16-byte chunk c of row r inside a row-major [rows][D] LDS tile
// (rows of D half-precision values): the rows that 16 lanes read together
// land on 16 different bank groups.  An involution in c for every r, so the
// same function maps a position to its chunk and a chunk to its position.
template <int D>
__device__ __forceinline__ int k_pos(int r, int c) {
  if constexpr (D == 128) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

// Position of 16-byte chunk c of row r in a row-major [rows][D] LDS tile that
// is read both by rows (16 lanes: 16 consecutive rows, one chunk) and by the
// transpose loads below (32 lanes: 4 consecutive rows x 4 consecutive chunks).
// The chunk is XORed with a bit permutation of the row that is a bijection on
// any 16 consecutive rows (rows) and puts the row's low two bits (D = 128: 16
// chunks per 256-byte bank line) or bit 1 (D = 64: two rows per line) on chunk
// bit 2 and up (transpose loads), so both patterns touch every bank once.
// An involution in c for every r.
template <int D>
__device__ __forceinline__ int kt_pos(int r, int c) {
  if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  else return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset of columns 8c..8c+7 of row r in a transposed [D][64] tile image
// (rows of 64 half-precision values = 128 bytes; two rows share a 256-byte
// bank line).  The same layout is used in HBM and in LDS.
__device__ __forceinline__ int vt_off(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

// A raw buffer resource over `bytes` bytes from `base`: loads past the end
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, uint32_t bytes) {
  return buf_rsrc(base, bytes);
}

// Direct HBM -> LDS loads: lane l's 16 (or 4) bytes land at lds + l * 16 (or 4).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt immediate: at most n vector-memory loads outstanding, the other
// counters unchecked (vmcnt is split over bits 3:0 and 15:14).
__device__ __forceinline__ constexpr int vmcnt_at_most(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

// Instruction order for a block of N LDS fragment reads feeding N matrix
// products: three reads ahead, then one product and one read in turn, so a
// product's operand has had three products' time to arrive and only a few
// fragments are live at once.
template <int N>
__device__ __forceinline__ void interleave_reads_and_products() {
  constexpr int kAhead = 3;
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The k-operand of a product whose k axis runs along the rows of a row-major
// [rows][D] LDS tile (kt_pos layout), read transposed by the gfx950 LDS
// transpose loads: lane l receives column f0 + l % 32 of rows
// r0 + 8 (l / 32) .. + 7 (f0 a multiple of 32, r0 a multiple of 16).
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane j of a group reads 4
// consecutive 16-bit values, and lane i of the group receives value i % 4 of
// lanes 4c + i / 4 for c = 0..3.  Lane j here reads columns
// f + 4 (j % 4) .. + 3 of row r + j / 4, so lane i receives column f + i of
// rows r .. r + 3; two such reads give the 8 rows.
template <int D>
__device__ __forceinline__ u32x4 read_rows_transposed(const uint8_t* tile, int r0, int f0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int f = f0 + 16 * (g & 1) + 4 * (j & 3);
  u32x4 res;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + 8 * (g >> 1) + 4 * h + (j >> 2);
    const int at = r * (D * 2) + kt_pos<D>(r, f >> 3) * 16 + (f & 7) * 2;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(tile + at));
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    res[2 * h] = w[0];
    res[2 * h + 1] = w[1];
  }
  return res;
}

// One thread's share of writing a transposed tile image: r[k] holds columns
// 8cv .. 8cv + 7 of row 4kq + k (kq < 16) of a 64-row tile as packed 16-bit
// values (word w: columns 2w low, 2w + 1 high); they land in the [D][64] image
// at `img` (vt_off layout).
__device__ __forceinline__ void store_tile_image(const u32x4 (&r)[4], uint8_t* img, int kq, int cv) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    u32x2 even, odd;
    even[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x05040100u);
    even[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x05040100u);
    odd[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x07060302u);
    odd[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x07060302u);
    const int row = 8 * cv + 2 * w;
    *(u32x2*)(img + vt_off(row, kq / 2) + 8 * (kq % 2)) = even;
    *(u32x2*)(img + vt_off(row + 1, kq / 2) + 8 * (kq % 2)) = odd;
  }
}

// Rows row0 + 4kq .. + 3 and columns 8cv .. 8cv + 7 of a 64-row tile of 16-bit
// values, read through `rs` (row stride rs_bytes; rows past the resource's end
// read zeros), as store_tile_image takes them.
__device__ __forceinline__ void load_tile_part(__amdgpu_buffer_rsrc_t rs, uint32_t row0, uint32_t rs_bytes,
                                               int kq, int cv, u32x4 (&r)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rs, (row0 + 4 * kq + k) * rs_bytes + cv * 16u, 0, 0));
}

// Largest magnitude among the 32 bfloat16 values of a load_tile_part share.
__device__ __forceinline__ float tile_part_absmax_bf16(const u32x4 (&r)[4]) {
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int w = 0; w < 4; ++w) m = bf16x2_absmax(m, r[k][w]);
  return m;
}

// The share's bfloat16 values re-encoded as IEEE halves.
__device__ __forceinline__ void tile_part_to_f16(u32x4 (&r)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int w = 0; w < 4; ++w) r[k][w] = bf16x2_to_f16x2(r[k][w]);
}

// The same for a tile of OCP e4m3 (fp8) values, re-encoded as IEEE halves
// (exact: every e4m3 value is a half).
__device__ __forceinline__ void write_tile_image_fp8(__amdgpu_buffer_rsrc_t rs, uint32_t row0, uint32_t rs_bytes,
                                                     uint8_t* img, int kq, int cv) {
  u32x4 r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  rs, (row0 + 4 * kq + k) * rs_bytes + cv * 8u, 0, 0));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = b[h];
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
      r[k][2 * h] = pack_f16x2(lo[0], lo[1]);
      r[k][2 * h + 1] = pack_f16x2(hi[0], hi[1]);
    }
  }
  store_tile_image(r, img, kq, cv);
}

}  // namespace mea
