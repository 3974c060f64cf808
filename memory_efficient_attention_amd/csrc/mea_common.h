// Shared device helpers for the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mea {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Everything a launch needs; passed by value as the kernel argument.
struct FwdArgs {
  const uint16_t* q;         // [total_q, Hq, D]
  const uint16_t* k;         // [total_k, Hkv, D]
  const uint16_t* v;         // [total_k, Hkv, D]
  uint16_t* out;             // [total_q, Hq, D]
  float* lse;                // [Hq, total_q] or nullptr
  const int32_t* seqstart_q; // [num_seqs + 1]
  const int32_t* seqstart_k; // [num_seqs + 1]
  const float* slopes;       // [Hq] or nullptr
  float* ws_o;               // decode: [num_seqs, max_chunks, Hq, D] float32 partials
  float* ws_lse;             // decode: [num_seqs, max_chunks, Hq] float32 (log2 units)
  uint16_t* ws_vt;           // prefill: transposed half-precision V tile images (see fwd_prefill.hip)
  int32_t* ws_vflag;         // prefill, bfloat16: per V^T image, 1 if it was kept in bfloat16
  const int32_t* block_table;  // paged K/V: [num_seqs, max_blocks] page of each page_size-key block, or nullptr
  int32_t page_size;         // paged K/V: keys per page (a multiple of 64)
  int32_t max_blocks;        // paged K/V: row length of block_table
  int32_t num_pages;         // paged K/V: pages in the cache; entries outside [0, num_pages) read as zeros
  float scale_log2;          // scale * log2(e)
  int32_t num_seqs;
  int32_t total_q;
  int32_t total_k;
  int32_t Hq;
  int32_t Hkv;
  int32_t group;             // Hq / Hkv
  int32_t heads_per_wg;      // prefill: query heads of one group served per workgroup
  int32_t head_slices;       // prefill: group / heads_per_wg; decode: ceil(group / 16)
  int32_t kv_per_wg;         // decode: key/value heads per workgroup (one wave per head and key stripe)
  int32_t chunk_keys;        // decode: keys per piece of the concatenated key axis
  int32_t max_chunks;        // decode: partial slots per sequence, ceil(max_seqlen_k / chunk_keys) + 1
  int32_t dc_pieces;         // decode: ceil(total_k / chunk_keys)
  int32_t pf_max_tiles;      // prefill: query tiles of the longest sequence
  int32_t pf_items;          // prefill: head slices * num_seqs * pf_max_tiles
  float out_scale;           // fp8 inputs: the V scale, applied to the output (else 1)
  int32_t dc_seq_base;       // decode: first sequence served (a mixed batch's decode part: the sequences after its prefills)
  int32_t dc_key_base;       // decode: seqstart_k[dc_seq_base], where the split key axis starts
  int32_t* pf_tickets;       // prefill: 8 work counters (one per XCD), zeroed by the V pre-pass; nullptr: one item per workgroup
};

// Everything a backward launch needs; passed by value as the kernel argument.
struct BwdArgs {
  const uint16_t* q;         // [total_q, Hq, D]
  const uint16_t* k;         // [total_k, Hkv, D]
  const uint16_t* v;         // [total_k, Hkv, D]
  const uint16_t* out;       // [total_q, Hq, D] forward output
  const float* lse;          // [Hq, total_q] forward log-sum-exp (natural log)
  const uint16_t* dout;      // [total_q, Hq, D] gradient of the output
  uint16_t* dq;              // [total_q, Hq, D]
  uint16_t* dk;              // [total_k, Hkv, D]
  uint16_t* dv;              // [total_k, Hkv, D]
  const int32_t* seqstart_q; // [num_seqs + 1]
  const int32_t* seqstart_k; // [num_seqs + 1]
  const float* slopes;       // [Hq] or nullptr
  float* ws_lse2;            // [Hq, total_q] lse * log2(e); +inf for a row with no key
  float* ws_dsum;            // [Hq, total_q] rowsum(dO * O)
  float scale;
  float scale_log2;          // scale * log2(e)
  int32_t num_seqs;
  int32_t total_q;
  int32_t total_k;
  int32_t Hq;
  int32_t Hkv;
  int32_t group;             // Hq / Hkv
  int32_t kv_tiles;          // dK/dV: key tiles of the longest sequence
  int32_t kv_items;          // dK/dV: Hkv * num_seqs * kv_tiles
  int32_t heads_per_wg;      // dQ: query heads of one group served per workgroup
  int32_t head_slices;       // dQ: group / heads_per_wg
  int32_t q_tiles;           // dQ: query tiles of the longest sequence
  int32_t q_items;           // dQ: Hkv * head_slices * num_seqs * q_tiles
};

// 32x32x16 matrix-core products, float32 accumulate.  Lane l holds row (or
// column) l % 32 of a 32 x 16 operand and the 8 consecutive k-values 8*(l/32)..+7;
// the accumulator register r of lane l is element (8*(r/4) + 4*(l/32) + r%4, l%32).
template <bool BF16>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// 16x16x32 matrix-core products, float32 accumulate.  Lane l holds row (or
// column) l % 16 of a 16 x 32 operand and 8 k-values of group l / 16 (both
// operands share the assignment); accumulator register r of lane l is element
// (4*(l/16) + r, l%16).
template <bool BF16>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32x64 products of OCP e4m3 (fp8) operands, float32 accumulate.  Lane l
// holds row (or column) l % 32 and 32 k-values, 16 bytes in each of lo and hi;
// the output layout is that of mfma_32x32x16.  Any assignment of k-values to
// lanes and bytes gives the same product as long as both operands share it.
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(u32x4 alo, u32x4 ahi, u32x4 blo, u32x4 bhi, f32x16 c) {
  const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7));
  // format 0 (e4m3) for both operands; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x128 products of OCP e4m3 operands, float32 accumulate.  Lane l holds
// row (or column) l % 16 and 32 k-values, 16 bytes in each of lo and hi, with
// the same freedom of k-assignment; the output layout is that of the 16x16x32
// 16-bit products (lane l: column l % 16, rows 4 (l / 16) .. + 3).
__device__ __forceinline__ f32x4 mfma_16x16x128_fp8(u32x4 alo, u32x4 ahi, u32x4 blo, u32x4 bhi, f32x4 c) {
  const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// p[i] read through the constant address space: with a wave-uniform i it
// becomes a scalar load (scalar cache and counter, so it neither waits for
// nor holds up the vector-memory operations in flight).  Only for arrays that
// no kernel of the launch writes.
__device__ __forceinline__ int32_t load_const(const int32_t* p, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// The other half-wave's value of x (lane l <-> lane l ^ 32), combined.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]),
                         __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two float32 values to a packed pair of IEEE halves, round to nearest even
// (one v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two float32 values to the output dtype, packed, round to nearest even (one
// v_cvt_pk_bf16_f32 or v_cvt_pk_f16_f32).
template <bool BF16>
__device__ __forceinline__ uint32_t pack_out_x2(float lo, float hi) {
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  } else {
    return pack_f16x2(lo, hi);
  }
}

// A packed pair of bfloat16 values re-encoded as a packed pair of IEEE halves.
// Exact for magnitudes in [2^-14, 65504]; larger ones saturate (round toward 0).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  float lo = __builtin_bit_cast(float, w << 16);
  float hi = __builtin_bit_cast(float, w & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// A packed pair of IEEE halves re-encoded as a packed pair of bfloat16
// values, round to nearest even.
__device__ __forceinline__ uint32_t f16x2_to_bf16x2(uint32_t w) {
  const f16x2 h = __builtin_bit_cast(f16x2, w);
  return pack_out_x2<true>((float)h[0], (float)h[1]);
}

// Running maximum magnitude of the two bfloat16 values packed in w.
__device__ __forceinline__ float bf16x2_absmax(float m, uint32_t w) {
  const float lo = __builtin_bit_cast(float, w << 16);
  const float hi = __builtin_bit_cast(float, w & 0xffff0000u);
  return __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(lo), __builtin_fabsf(hi)));
}

// Whether a block of bfloat16 V values whose largest magnitude is m must stay
// in bfloat16 for P V.  bf16x2_to_f16x2 is exact for every bfloat16 value
// with 2^-14 <= |v| <= 65504 and errs by less than 2^-24 below that, i.e. by
// less than 2^-10 of the block's largest magnitude whenever that is at least
// 2^-14.  Blocks with a larger magnitude (which would saturate) or with only
// smaller ones (which would lose their precision) keep bfloat16 and use
// bfloat16 weights instead.  (A NaN converts to a NaN either way.)
__device__ __forceinline__ bool v_needs_bf16(float m) {
  return !(m <= 65504.f) || (m > 0.f && m < 0x1p-14f);
}

// Bytes 2 hi and 2 hi + 1 of w, two OCP e4m3 values, widened to a packed pair
// of IEEE halves (low half from the lower byte).  Exact: every e4m3 value,
// subnormals included, is a half.
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w, bool hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// MFMA accumulator row of register r in half-wave `hi` (32x32 layout).
__device__ __forceinline__ constexpr int acc_row(int r, int hi) { return 8 * (r / 4) + 4 * hi + (r % 4); }

// Key rows are fed to the Q.K^T product in a permuted order so that the 16
// accumulator registers of a lane hold two runs of 8 consecutive keys, which
// is exactly the k-operand layout of the following P.V product.  Row rho of
// a 32-key block holds key swap_bits_2_3(rho).
__device__ __forceinline__ constexpr int key_of_row(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}
// Tile-local key (within a 32-key block) held by accumulator register r of half-wave hi.
__device__ __forceinline__ constexpr int key_of_reg(int r, int hi) { return 16 * (r / 8) + 8 * hi + (r % 8); }

}  // namespace mea
