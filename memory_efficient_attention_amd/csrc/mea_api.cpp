// C ABI of the attention forward and backward: argument validation, path choice, launch.
// The contract (layouts, ownership, errors) is documented in include/mea.h.
#include "mea.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <mutex>

#include "mea_launch.h"

// Scratch of mea_fwd_noalloc: one fixed array per device, in the library's
// device code (it exists on every GPU the library runs on, for the life of the
// process).  Host code never passes `scratch` itself to a kernel: in host
// code that name is a stand-in, not a device address.  The device address is
// taken once per device with hipGetSymbolAddress, that device current, and
// kept in g_scratch_ptr (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[MEA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

mea_status_t fail(mea_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int gcd_int(int x, int y) {
  while (y != 0) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
}

// Decode head groups: nh = kv neighbouring key/value heads (kDcWaves / nh
// waves serve each) times the slices of 16 query heads of each head's group.
int32_t decode_head_groups(int32_t Hq, int32_t Hkv, int32_t kv) {
  const int32_t group = Hq / Hkv;
  return (Hkv / kv) * ((group + mea::kDcHeadsPerWg - 1) / mea::kDcHeadsPerWg);
}

int32_t default_chunk(int32_t total_k, int32_t Hq, int32_t Hkv, int32_t kv) {
  // Piece length W of the concatenated key axis: about kDcTargetWgs
  // equal-sized (piece, head group) workgroups in all, i.e. one full round of
  // one workgroup per CU on 256 CUs: every workgroup starts at once and
  // none is left over for a tail (measured: one round beats two or four,
  // which pay each workgroup's start-up again).  Never below kDcMinPiece keys,
  // so that partial results stay a small fraction of the K/V bytes.
  const long long work = (long long)total_k * (long long)decode_head_groups(Hq, Hkv, kv);
  long long w = (work + mea::kDcTargetWgs - 1) / mea::kDcTargetWgs;
  w = (w + mea::kDcPieceAlign - 1) / mea::kDcPieceAlign * mea::kDcPieceAlign;
  if (w < mea::kDcMinPiece) w = mea::kDcMinPiece;
  if (w > (1ll << 30)) w = 1ll << 30;
  return (int32_t)w;
}

// Key/value heads per decode head group and the default piece length.  16-bit
// K/V: gcd(Hkv, 4) heads, runs of up to 1 KiB of each 2 KiB token row (8 heads
// of D 128).  fp8 K/V: the token row of 8 heads is 1 KiB, and groups of 4
// heads read its halves at unequal rates (measured: the workgroups on the
// first half of the rows took ~13 % longer); gcd(Hkv, 8) heads read whole
// rows, 5-7 % faster, as long as the pieces stay long (>= kDcFp8WidePiece
// keys).  On
// short pieces (one long sequence: the default splits it into pieces of a
// few hundred keys) the wide groups' halved piece length costs more than they
// save, so fp8 keeps gcd(Hkv, 4) there.
struct DecodeSplit {
  int32_t kv_per_wg, chunk;
};

DecodeSplit decode_split(int32_t total_k, int32_t Hq, int32_t Hkv, bool fp8) {
  const int32_t kv4 = gcd_int(Hkv, mea::kDcKvPerWgMax);
  if (fp8) {
    const int32_t kv8 = gcd_int(Hkv, mea::kDcKvPerWgMaxFp8);
    const int32_t w = default_chunk(total_k, Hq, Hkv, kv8);
    if (kv8 > kv4 && w >= mea::kDcFp8WidePiece) return {kv8, w};
  }
  return {kv4, default_chunk(total_k, Hq, Hkv, kv4)};
}

// Partial slots per sequence: the pieces a sequence of L keys touches are at
// most ceil(L / W) + 1.
int32_t decode_slots(int32_t max_seqlen_k, int32_t w) { return (int32_t)((max_seqlen_k + (long long)w - 1) / w) + 1; }

size_t decode_ws_bytes(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_k, int32_t Hq, int32_t D, int32_t w) {
  if (total_k == 0 || max_seqlen_k == 0) return 0;
  return (size_t)num_seqs * (size_t)decode_slots(max_seqlen_k, w) * (size_t)Hq * (size_t)(D + 1) * sizeof(float);
}

// Prefill: one 16-bit V^T image of D x 64 keys per key/value head and key
// tile, then one int32 flag per image (1: the image stayed bfloat16), then
// the work counters of the persistent prefill workgroups;
// sequence b's tiles start at slot seqstart_k[b] / 64 + b, so total_k / 64 +
// num_seqs slots per head cover every sequence.  Each part is 256-byte
// aligned.
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// The prefill's work counters (8 int32, one per XCD) after the flags.
constexpr size_t kPfTicketBytes = 256;

size_t prefill_slots(int32_t num_seqs, int32_t total_k, int32_t Hkv) {
  return ((size_t)total_k / mea::kPfBN + (size_t)num_seqs) * (size_t)Hkv;
}

size_t prefill_ws_bytes(int32_t num_seqs, int32_t total_k, int32_t Hkv, int32_t D) {
  if (total_k == 0) return 0;
  const size_t slots = prefill_slots(num_seqs, total_k, Hkv);
  return align256(slots * (size_t)D * mea::kPfBN * 2) + align256(slots * sizeof(int32_t)) + kPfTicketBytes;
}

// Paged K/V cache: block_table[b * max_blocks + i] is the page holding keys
// [i * page_size, (i + 1) * page_size) of sequence b.
struct PagedKv {
  const int32_t* block_table;
  int32_t page_size, num_pages, max_blocks;
};

// fp8 (OCP e4m3) q, k, v with per-tensor scales: the values are q_scale * q8
// etc.  q_scale * k_scale folds into the score scale, v_scale into the output.
struct Fp8Scales {
  float q, k, v;
};

// A mixed batch: sequences [0, n_pre) are prefills (any query count) and
// sequences [n_pre, num_seqs) decode steps of exactly one query each;
// pre_q = seqstart_q[n_pre], pre_k = seqstart_k[n_pre]; dec_max_k bounds the
// key count of the decode sequences.
struct MixedSplit {
  int32_t n_pre, pre_q, pre_k, dec_max_k;
};

// How one forward call is carried out: a prefill part (sequences [0, n) on the
// prefill kernels) and a decode part (sequences [seq_base, num_seqs), keys
// [key_base, total_k), on the split-KV kernels), each with its workspace
// region.
struct FwdPlan {
  bool pre = false, dec = false;
  int32_t pre_n = 0, pre_k = 0;
  int32_t dec_base = 0, dec_key_base = 0, dec_n = 0, dec_keys = 0, dec_max_k = 0;
  DecodeSplit split{0, 0};
  size_t pre_bytes = 0, dec_bytes = 0, dec_off = 0, total = 0;
};

FwdPlan fwd_plan(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                 int32_t Hkv, int32_t D, int32_t chunk_keys, bool forced_split, bool fp8, const MixedSplit* mixed) {
  FwdPlan p;
  if (mixed != nullptr) {
    p.pre = mixed->n_pre > 0;
    p.pre_n = mixed->n_pre;
    p.pre_k = mixed->pre_k;
    p.dec = mixed->n_pre < num_seqs;
    p.dec_base = mixed->n_pre;
    p.dec_key_base = mixed->pre_k;
    p.dec_n = num_seqs - mixed->n_pre;
    p.dec_keys = total_k - mixed->pre_k;
    p.dec_max_k = mixed->dec_max_k;
  } else if (max_seqlen_q == 1) {
    p.dec = true;
    p.dec_n = num_seqs;
    p.dec_keys = total_k;
    p.dec_max_k = max_seqlen_k;
  } else {
    p.pre = true;
    p.pre_n = num_seqs;
    p.pre_k = total_k;
  }
  if (p.pre) p.pre_bytes = prefill_ws_bytes(p.pre_n, p.pre_k, Hkv, D);
  if (p.dec) {
    p.split = forced_split ? DecodeSplit{gcd_int(Hkv, mea::kDcKvPerWgMax), chunk_keys}
                           : decode_split(p.dec_keys, Hq, Hkv, fp8);
    p.dec_bytes = decode_ws_bytes(p.dec_n, p.dec_keys, p.dec_max_k, Hq, D, p.split.chunk);
  }
  p.dec_off = p.pre_bytes > 0 && p.dec_bytes > 0 ? align256(p.pre_bytes) : 0;
  p.total = p.dec_bytes > 0 ? p.dec_off + p.dec_bytes : p.pre_bytes;
  return p;
}

size_t fwd_ws_size(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                   int32_t Hkv, int32_t D, int32_t chunk_keys, bool fp8) {
  if (num_seqs <= 0 || total_k < 0 || max_seqlen_q <= 0 || max_seqlen_k < 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv != 0 || (D != 64 && D != 128) || chunk_keys < 0 ||
      (chunk_keys > 0 && chunk_keys % mea::kDcPieceAlign != 0))
    return 0;
  return fwd_plan(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, chunk_keys, chunk_keys > 0, fp8,
                  nullptr).total;
}

mea_status_t fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse,
                      const int32_t* seqstart_q, const int32_t* seqstart_k, int32_t num_seqs,
                      int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                      int32_t Hkv, int32_t D, mea_dtype_t dtype, int32_t causal,
                      const float* alibi_slopes, float scale, void* workspace,
                      size_t workspace_bytes, void* stream, int32_t chunk_keys, bool forced_split,
                      const PagedKv* paged = nullptr, const Fp8Scales* fp8 = nullptr,
                      const MixedSplit* mixed = nullptr) {
  g_last_error[0] = '\0';
  // q and out are read/written only when total_q > 0, k and v only when total_k > 0
  if (((q == nullptr || out == nullptr) && total_q > 0) || ((k == nullptr || v == nullptr) && total_k > 0))
    return fail(MEA_ERR_INVALID, "q, k, v and out must be non-NULL device pointers (k and v may be NULL when "
                "total_k == 0, q and out when total_q == 0)");
  if (seqstart_q == nullptr || seqstart_k == nullptr)
    return fail(MEA_ERR_INVALID, "seqstart_q and seqstart_k must be non-NULL device pointers");
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(MEA_ERR_INVALID, "negative size (num_seqs=%d total_q=%d total_k=%d max_seqlen_q=%d max_seqlen_k=%d)",
                num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(MEA_ERR_INVALID, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0 (Hq=%d Hkv=%d)", Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(MEA_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
  if (total_q > 0 && max_seqlen_q == 0)
    return fail(MEA_ERR_INVALID, "total_q=%d > 0 but max_seqlen_q == 0", total_q);
  if (forced_split) {
    if (max_seqlen_q != 1) return fail(MEA_ERR_INVALID, "mea_fwd_splitkv needs max_seqlen_q == 1 (got %d)", max_seqlen_q);
    if (chunk_keys <= 0 || chunk_keys % mea::kDcPieceAlign != 0)
      return fail(MEA_ERR_INVALID, "chunk_keys must be a positive multiple of %d (got %d)", mea::kDcPieceAlign, chunk_keys);
  }
  if (D != 64 && D != 128) return fail(MEA_ERR_UNSUPPORTED, "head dimension D=%d is not 64 or 128", D);
  if (fp8 != nullptr) {
    if (D != 128) return fail(MEA_ERR_UNSUPPORTED, "fp8 inputs need D=128 (got %d)", D);
    if (!std::isfinite(fp8->q) || !(fp8->q > 0.f) || !std::isfinite(fp8->k) || !(fp8->k > 0.f) ||
        !std::isfinite(fp8->v) || !(fp8->v > 0.f))
      return fail(MEA_ERR_UNSUPPORTED, "fp8 scales must be finite and > 0 (got %g, %g, %g)", (double)fp8->q,
                  (double)fp8->k, (double)fp8->v);
  }
  if (dtype != MEA_F16 && dtype != MEA_BF16) return fail(MEA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(MEA_ERR_UNSUPPORTED, "scale must be finite and > 0 (got %g)", (double)scale);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(MEA_ERR_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
  if ((lse != nullptr && !aligned(lse, 4)) || (alibi_slopes != nullptr && !aligned(alibi_slopes, 4)) ||
      !aligned(seqstart_q, 4) || !aligned(seqstart_k, 4))
    return fail(MEA_ERR_UNSUPPORTED, "lse, alibi_slopes and seqstart arrays must be 4-byte aligned");
  if (num_seqs > 65535) return fail(MEA_ERR_UNSUPPORTED, "num_seqs=%d exceeds 65535", num_seqs);
  if (paged != nullptr) {
    if (paged->block_table == nullptr) return fail(MEA_ERR_INVALID, "block_table must be a non-NULL device pointer");
    if (!aligned(paged->block_table, 4)) return fail(MEA_ERR_UNSUPPORTED, "block_table must be 4-byte aligned");
    if (paged->page_size <= 0 || paged->num_pages <= 0 || paged->max_blocks <= 0)
      return fail(MEA_ERR_INVALID, "need page_size > 0, num_pages > 0 and max_blocks > 0 (got %d, %d, %d)",
                  paged->page_size, paged->num_pages, paged->max_blocks);
    if (paged->page_size % 64 != 0)
      return fail(MEA_ERR_UNSUPPORTED, "page_size=%d is not a multiple of 64", paged->page_size);
    if ((long long)paged->max_blocks * paged->page_size < max_seqlen_k)
      return fail(MEA_ERR_INVALID, "max_blocks * page_size = %lld keys < max_seqlen_k = %d",
                  (long long)paged->max_blocks * paged->page_size, max_seqlen_k);
    if ((long long)paged->page_size * Hkv * D * 2 >= (1ll << 31))
      return fail(MEA_ERR_UNSUPPORTED, "page_size * Hkv * D * 2 bytes must stay below 2^31");
  }
  // key/value rows of one sequence are addressed with 32-bit byte offsets
  if ((long long)max_seqlen_k * Hkv * D * 2 >= (1ll << 31))
    return fail(MEA_ERR_UNSUPPORTED, "max_seqlen_k * Hkv * D * 2 bytes must stay below 2^31");
  if (mixed != nullptr) {
    const int32_t n_dec = num_seqs - mixed->n_pre;
    if (mixed->n_pre < 0 || n_dec < 0 || mixed->pre_q < 0 || mixed->pre_q > total_q || mixed->pre_k < 0 ||
        mixed->pre_k > total_k || mixed->dec_max_k < 0 || mixed->dec_max_k > max_seqlen_k)
      return fail(MEA_ERR_INVALID, "mixed batch: need 0 <= num_prefill_seqs <= num_seqs, 0 <= prefill_total_q <= "
                  "total_q, 0 <= prefill_total_k <= total_k and 0 <= decode_max_seqlen_k <= max_seqlen_k (got %d, %d, "
                  "%d, %d)", mixed->n_pre, mixed->pre_q, mixed->pre_k, mixed->dec_max_k);
    if (total_q - mixed->pre_q != n_dec)
      return fail(MEA_ERR_INVALID, "mixed batch: the %d decode sequences must hold one query each, but total_q - "
                  "prefill_total_q = %d", n_dec, total_q - mixed->pre_q);
    if (mixed->pre_q > 0 && max_seqlen_q == 0)
      return fail(MEA_ERR_INVALID, "mixed batch: prefill_total_q=%d > 0 but max_seqlen_q == 0", mixed->pre_q);
  }
  if (num_seqs == 0 || total_q == 0) return MEA_OK;

  mea::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.seqstart_q = seqstart_q;
  a.seqstart_k = seqstart_k;
  a.slopes = alibi_slopes;
  a.scale_log2 = scale * mea::kLog2e;
  a.out_scale = 1.f;
  if (fp8 != nullptr) {
    a.scale_log2 = (float)((double)scale * fp8->q * fp8->k * (double)mea::kLog2e);
    a.out_scale = fp8->v;
  }
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.total_k = total_k;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  if (paged != nullptr) {
    a.block_table = paged->block_table;
    a.page_size = paged->page_size;
    a.max_blocks = paged->max_blocks;
    a.num_pages = paged->num_pages;
  }
  const bool bf16 = dtype == MEA_BF16;
  const bool alibi = alibi_slopes != nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);

  const FwdPlan plan = fwd_plan(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, chunk_keys, forced_split,
                                fp8 != nullptr, mixed);
  if (plan.total > 0 && (workspace == nullptr || workspace_bytes < plan.total))
    return fail(MEA_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu bytes required", workspace_bytes,
                plan.total);
  if (plan.total > 0 && !aligned(workspace, 256)) return fail(MEA_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  mea::FwdArgs ap = a, ad = a;  // the prefill part's and the decode part's arguments
  if (plan.dec) {
    const int32_t chunk = plan.split.chunk;
    ad.chunk_keys = chunk;
    ad.dc_pieces = plan.dec_bytes > 0 ? (int32_t)(((long long)plan.dec_keys + chunk - 1) / chunk) : 0;
    ad.max_chunks = plan.dec_bytes > 0 ? decode_slots(plan.dec_max_k, chunk) : 0;
    ad.head_slices = (a.group + mea::kDcHeadsPerWg - 1) / mea::kDcHeadsPerWg;
    ad.heads_per_wg = mea::kDcHeadsPerWg;
    ad.kv_per_wg = plan.split.kv_per_wg;
    ad.dc_seq_base = plan.dec_base;
    ad.dc_key_base = plan.dec_key_base;
    ad.ws_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + plan.dec_off);
    ad.ws_lse = ad.ws_o + (size_t)plan.dec_n * ad.max_chunks * Hq * D;
    if ((long long)ad.dc_pieces * decode_head_groups(Hq, Hkv, plan.split.kv_per_wg) > 0x7ffffff8ll)  // padded to 8
      return fail(MEA_ERR_UNSUPPORTED, "too many decode workgroups (%d pieces of %d keys)", ad.dc_pieces, chunk);
  }
  if (plan.pre) {
    if ((long long)max_seqlen_k / mea::kPfBN + 1 > 65535)
      return fail(MEA_ERR_UNSUPPORTED, "max_seqlen_k=%d needs more than 65535 key tiles", max_seqlen_k);
    ap.num_seqs = plan.pre_n;
    ap.ws_vt = static_cast<uint16_t*>(workspace);
    if (plan.pre_bytes > 0) {
      const size_t slots = prefill_slots(plan.pre_n, plan.pre_k, Hkv);
      uint8_t* ws = static_cast<uint8_t*>(workspace);
      ap.ws_vflag = reinterpret_cast<int32_t*>(ws + align256(slots * (size_t)D * mea::kPfBN * 2));
      ap.pf_tickets = reinterpret_cast<int32_t*>(ws + align256(slots * (size_t)D * mea::kPfBN * 2) +
                                                 align256(slots * sizeof(int32_t)));
    }
    ap.heads_per_wg = gcd_int(a.group, mea::kPfGroupWaves);
    ap.head_slices = a.group / ap.heads_per_wg;
    const int bt = mea::kPfGroups * 32 * (mea::kPfGroupWaves / ap.heads_per_wg);
    const long long tiles = (max_seqlen_q + bt - 1) / bt;
    const long long items = (long long)Hkv * ap.head_slices * plan.pre_n * tiles;
    if (items > (1ll << 31) - 8)
      return fail(MEA_ERR_UNSUPPORTED, "%lld prefill work items exceed the grid limit", items);
    ap.pf_max_tiles = (int32_t)tiles;
    ap.pf_items = (int32_t)items;
  }
  hipError_t err = hipSuccess;
  if (plan.pre && !(mixed != nullptr && mixed->pre_q == 0))
    err = fp8 != nullptr ? mea::launch_prefill_fp8(ap, bf16, causal != 0, alibi, max_seqlen_k, s)
                         : mea::launch_prefill(ap, D, bf16, causal != 0, alibi, max_seqlen_k, s);
  if (err == hipSuccess && plan.dec)
    err = fp8 != nullptr ? mea::launch_decode_fp8(ad, bf16, alibi, s) : mea::launch_decode(ad, D, bf16, alibi, s);
  if (err != hipSuccess) return fail(MEA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return MEA_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the device of `stream`, which must be
// the current device.
mea_status_t noalloc_scratch(void* stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(MEA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  hipDevice_t sdev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return fail(MEA_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
  }
  if (sdev != cur)
    return fail(MEA_ERR_INVALID, "the stream belongs to device %d but device %d is current", (int)sdev, cur);
  if (cur < 0 || cur >= kMaxDevices) return fail(MEA_ERR_UNSUPPORTED, "device %d: at most %d devices", cur, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[cur] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MEA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
    g_scratch_ptr[cur] = p;
  }
  *out = g_scratch_ptr[cur];
  return MEA_OK;
}

// Backward workspace: lse2 and Dsum [Hq, total_q] float32, each part
// 256-byte aligned.

struct BwdWs {
  size_t lse2, dsum, total;
};

BwdWs bwd_ws_layout(int32_t total_q, int32_t Hq) {
  BwdWs w{};
  const size_t rows = total_q > 0 ? align256((size_t)Hq * (size_t)total_q * sizeof(float)) : 0;
  w.lse2 = 0;
  w.dsum = rows;
  w.total = 2 * rows;
  return w;
}

mea_status_t bwd_impl(const void* q, const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, const int32_t* seqstart_q,
                      const int32_t* seqstart_k, int32_t num_seqs, int32_t total_q, int32_t total_k,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                      mea_dtype_t dtype, int32_t causal, const float* alibi_slopes, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  // the query-side arrays are used only when total_q > 0, the key-side ones only when total_k > 0
  if ((q == nullptr || out == nullptr || lse == nullptr || dout == nullptr) && total_q > 0)
    return fail(MEA_ERR_INVALID, "q, k, v, out, lse and dout must be non-NULL device pointers (the query-side "
                "ones may be NULL when total_q == 0)");
  if ((k == nullptr || v == nullptr) && total_k > 0)
    return fail(MEA_ERR_INVALID, "q, k, v, out, lse and dout must be non-NULL device pointers (k and v may be "
                "NULL when total_k == 0)");
  if ((dq == nullptr && total_q > 0) || ((dk == nullptr || dv == nullptr) && total_k > 0))
    return fail(MEA_ERR_INVALID, "dq, dk and dv must be non-NULL device pointers (dq may be NULL when "
                "total_q == 0, dk and dv when total_k == 0)");
  if (seqstart_q == nullptr || seqstart_k == nullptr)
    return fail(MEA_ERR_INVALID, "seqstart_q and seqstart_k must be non-NULL device pointers");
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(MEA_ERR_INVALID, "negative size (num_seqs=%d total_q=%d total_k=%d max_seqlen_q=%d max_seqlen_k=%d)",
                num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(MEA_ERR_INVALID, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0 (Hq=%d Hkv=%d)", Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(MEA_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
  if (total_q > 0 && max_seqlen_q == 0)
    return fail(MEA_ERR_INVALID, "total_q=%d > 0 but max_seqlen_q == 0", total_q);
  if (total_k > 0 && max_seqlen_k == 0)
    return fail(MEA_ERR_INVALID, "total_k=%d > 0 but max_seqlen_k == 0", total_k);
  if (D != 64 && D != 128) return fail(MEA_ERR_UNSUPPORTED, "head dimension D=%d is not 64 or 128", D);
  if (dtype != MEA_F16 && dtype != MEA_BF16) return fail(MEA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(MEA_ERR_UNSUPPORTED, "scale must be finite and > 0 (got %g)", (double)scale);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(MEA_ERR_UNSUPPORTED, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(lse, 4) || (alibi_slopes != nullptr && !aligned(alibi_slopes, 4)) || !aligned(seqstart_q, 4) ||
      !aligned(seqstart_k, 4))
    return fail(MEA_ERR_UNSUPPORTED, "lse, alibi_slopes and seqstart arrays must be 4-byte aligned");
  if (num_seqs > 65535) return fail(MEA_ERR_UNSUPPORTED, "num_seqs=%d exceeds 65535", num_seqs);
  // one sequence's rows are addressed with 32-bit byte offsets
  if ((long long)max_seqlen_k * Hkv * D * 2 >= (1ll << 31))
    return fail(MEA_ERR_UNSUPPORTED, "max_seqlen_k * Hkv * D * 2 bytes must stay below 2^31");
  if ((long long)max_seqlen_q * Hq * D * 2 >= (1ll << 31))
    return fail(MEA_ERR_UNSUPPORTED, "max_seqlen_q * Hq * D * 2 bytes must stay below 2^31");
  if (num_seqs == 0 || (total_q == 0 && total_k == 0)) return MEA_OK;

  const BwdWs lay = bwd_ws_layout(total_q, Hq);
  if (lay.total > 0 && (workspace == nullptr || workspace_bytes < lay.total))
    return fail(MEA_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu bytes required", workspace_bytes,
                lay.total);
  if (lay.total > 0 && !aligned(workspace, 256)) return fail(MEA_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");

  mea::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<const uint16_t*>(out);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.seqstart_q = seqstart_q;
  a.seqstart_k = seqstart_k;
  a.slopes = alibi_slopes;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.ws_lse2 = reinterpret_cast<float*>(ws + lay.lse2);
  a.ws_dsum = reinterpret_cast<float*>(ws + lay.dsum);
  a.scale = scale;
  a.scale_log2 = scale * mea::kLog2e;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.total_k = total_k;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  const long long kv_tiles = ((long long)max_seqlen_k + mea::kBwKeys - 1) / mea::kBwKeys;
  const long long kv_items = (long long)Hkv * num_seqs * kv_tiles;
  a.heads_per_wg = gcd_int(a.group, mea::kBwWaves);
  a.head_slices = a.group / a.heads_per_wg;
  const int bt = 32 * (mea::kBwWaves / a.heads_per_wg);
  const long long q_tiles = ((long long)max_seqlen_q + bt - 1) / bt;
  const long long q_items = (long long)Hkv * a.head_slices * num_seqs * q_tiles;
  if (kv_items > (1ll << 31) - 8 || q_items > (1ll << 31) - 8)
    return fail(MEA_ERR_UNSUPPORTED, "backward work items exceed the grid limit");
  a.kv_tiles = (int32_t)kv_tiles;
  a.kv_items = (int32_t)kv_items;
  a.q_tiles = (int32_t)q_tiles;
  a.q_items = (int32_t)q_items;
  const hipError_t err = mea::launch_backward(a, D, dtype == MEA_BF16, causal != 0, alibi_slopes != nullptr,
                                              static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(MEA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return MEA_OK;
}

}  // namespace

extern "C" {

mea_status_t mea_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     const int32_t* seqstart_q, const int32_t* seqstart_k, int32_t num_seqs,
                     int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                     int32_t Hkv, int32_t D, mea_dtype_t dtype, int32_t causal,
                     const float* alibi_slopes, float scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace,
                  workspace_bytes, stream, 0, false);
}

mea_status_t mea_fwd_mixed(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* seqstart_q, const int32_t* seqstart_k, int32_t num_seqs, int32_t total_q,
                           int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_prefill_seqs,
                           int32_t prefill_total_q, int32_t prefill_total_k, int32_t decode_max_seqlen_k, int32_t Hq,
                           int32_t Hkv, int32_t D, mea_dtype_t dtype, int32_t causal, const float* alibi_slopes,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const MixedSplit mixed{num_prefill_seqs, prefill_total_q, prefill_total_k, decode_max_seqlen_k};
  return fwd_impl(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace, workspace_bytes, stream, 0,
                  false, nullptr, nullptr, &mixed);
}

size_t mea_fwd_mixed_workspace_size(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_prefill_seqs, int32_t prefill_total_k, int32_t decode_max_seqlen_k,
                                    int32_t Hq, int32_t Hkv, int32_t D) {
  if (num_seqs <= 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv != 0 || (D != 64 && D != 128) || num_prefill_seqs < 0 || num_prefill_seqs > num_seqs ||
      prefill_total_k < 0 || prefill_total_k > total_k || decode_max_seqlen_k < 0)
    return 0;
  const MixedSplit mixed{num_prefill_seqs, 0, prefill_total_k, decode_max_seqlen_k};
  return fwd_plan(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, 0, false, false, &mixed).total;
}

mea_status_t mea_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* seqstart_q, const int32_t* seqstart_k, int32_t num_seqs,
                             int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t Hq, int32_t Hkv, int32_t D, mea_dtype_t dtype, int32_t causal,
                             const float* alibi_slopes, float scale, void* stream) {
  g_last_error[0] = '\0';
  const size_t need = fwd_ws_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, 0, false);
  if (need > (size_t)MEA_NOALLOC_SCRATCH_BYTES)
    return fail(MEA_ERR_UNSUPPORTED, "this call needs %zu bytes of scratch, more than the %zu bytes mea_fwd_noalloc "
                "holds per device (use mea_fwd with a workspace)", need, (size_t)MEA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    const mea_status_t st = noalloc_scratch(stream, &ws);
    if (st != MEA_OK) return st;
  }
  return fwd_impl(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, ws,
                  need > 0 ? (size_t)MEA_NOALLOC_SCRATCH_BYTES : 0, stream, 0, false);
}

mea_status_t mea_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                             const int32_t* seqstart_q, const int32_t* seqstart_k,
                             int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                             int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                             mea_dtype_t dtype, int32_t causal, const float* alibi_slopes,
                             float scale, void* workspace, size_t workspace_bytes, void* stream,
                             int32_t chunk_keys) {
  return fwd_impl(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace,
                  workspace_bytes, stream, chunk_keys, true);
}

mea_status_t mea_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                           const int32_t* seqstart_q, const int32_t* seqstart_k, const int32_t* block_table,
                           int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                           int32_t max_seqlen_k, int32_t page_size, int32_t num_pages, int32_t max_blocks,
                           int32_t Hq, int32_t Hkv, int32_t D, mea_dtype_t dtype, int32_t causal,
                           const float* alibi_slopes, float scale, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const PagedKv paged{block_table, page_size, num_pages, max_blocks};
  return fwd_impl(q, k_cache, v_cache, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace,
                  workspace_bytes, stream, 0, false, &paged);
}

mea_status_t mea_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, const int32_t* seqstart_q,
                     const int32_t* seqstart_k, int32_t num_seqs, int32_t total_q, int32_t total_k,
                     int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                     mea_dtype_t dtype, int32_t causal, const float* alibi_slopes, float scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, out, lse, dout, dq, dk, dv, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, Hq, Hkv, D, dtype, causal, alibi_slopes, scale, workspace,
                  workspace_bytes, stream);
}

size_t mea_bwd_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t Hq, int32_t Hkv,
                              int32_t D) {
  if (num_seqs <= 0 || total_q < 0 || total_k < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
      (D != 64 && D != 128))
    return 0;
  return bwd_ws_layout(total_q, Hq).total;
}

mea_status_t mea_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale,
                         void* out, float* lse, const int32_t* seqstart_q, const int32_t* seqstart_k,
                         int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D, mea_dtype_t out_dtype,
                         int32_t causal, const float* alibi_slopes, float scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const Fp8Scales sc{q_scale, k_scale, v_scale};
  return fwd_impl(q, k, v, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, Hq, Hkv, D, out_dtype, causal, alibi_slopes, scale, workspace, workspace_bytes,
                  stream, 0, false, nullptr, &sc);
}

mea_status_t mea_fwd_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float q_scale,
                               float k_scale, float v_scale, void* out, float* lse, const int32_t* seqstart_q,
                               const int32_t* seqstart_k, const int32_t* block_table, int32_t num_seqs,
                               int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t page_size, int32_t num_pages, int32_t max_blocks, int32_t Hq, int32_t Hkv,
                               int32_t D, mea_dtype_t out_dtype, int32_t causal, const float* alibi_slopes,
                               float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const PagedKv paged{block_table, page_size, num_pages, max_blocks};
  const Fp8Scales sc{q_scale, k_scale, v_scale};
  return fwd_impl(q, k_cache, v_cache, out, lse, seqstart_q, seqstart_k, num_seqs, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, Hq, Hkv, D, out_dtype, causal, alibi_slopes, scale, workspace,
                  workspace_bytes, stream, 0, false, &paged, &sc);
}

size_t mea_fwd_fp8_workspace_size(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  int32_t Hq, int32_t Hkv, int32_t D) {
  if (D != 128) return 0;
  return fwd_ws_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, 0, true);
}

mea_status_t mea_swiglu_ffn(const void* x, const void* w_gate, const void* w_up, const void* w_down, void* hidden,
                            void* out, int32_t tokens, int32_t d_model, int32_t d_ff, mea_dtype_t dtype,
                            void* stream) {
  g_last_error[0] = '\0';
  if (x == nullptr || w_gate == nullptr || w_up == nullptr || w_down == nullptr || hidden == nullptr ||
      out == nullptr)
    return fail(MEA_ERR_INVALID, "x, w_gate, w_up, w_down, hidden and out must be non-NULL device pointers");
  if (tokens < 0) return fail(MEA_ERR_INVALID, "negative tokens (%d)", tokens);
  if (d_model <= 0 || d_ff <= 0) return fail(MEA_ERR_INVALID, "need d_model > 0 and d_ff > 0 (got %d, %d)", d_model, d_ff);
  if (dtype != MEA_F16 && dtype != MEA_BF16) return fail(MEA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (d_model % 256 != 0 || d_ff % 128 != 0 || d_model > 65536 || d_ff > 65536)
    return fail(MEA_ERR_UNSUPPORTED, "need d_model a multiple of 256 and d_ff a multiple of 128, both <= 65536 "
                "(got %d, %d)", d_model, d_ff);
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(hidden, 16) ||
      !aligned(out, 16))
    return fail(MEA_ERR_UNSUPPORTED, "all pointers must be 16-byte aligned");
  if (tokens == 0) return MEA_OK;
  const hipError_t err = mea::launch_swiglu_ffn(x, w_gate, w_up, w_down, hidden, out, tokens, d_model, d_ff,
                                                dtype == MEA_BF16, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(MEA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return MEA_OK;
}

size_t mea_fwd_workspace_size(int32_t num_seqs, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t Hq, int32_t Hkv, int32_t D, int32_t chunk_keys) {
  return fwd_ws_size(num_seqs, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, chunk_keys, false);
}

int32_t mea_default_chunk_keys(int32_t total_k, int32_t Hq, int32_t Hkv) {
  if (Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return mea::kDcMinPiece;
  return decode_split(total_k < 0 ? 0 : total_k, Hq, Hkv, false).chunk;
}

const char* mea_status_string(mea_status_t status) {
  switch (status) {
    case MEA_OK: return "MEA_OK";
    case MEA_ERR_INVALID: return "MEA_ERR_INVALID: malformed argument";
    case MEA_ERR_UNSUPPORTED: return "MEA_ERR_UNSUPPORTED: outside what the kernels implement";
    case MEA_ERR_HIP: return "MEA_ERR_HIP: the HIP runtime refused a launch";
  }
  return "unknown mea_status_t";
}

const char* mea_last_error(void) { return g_last_error; }

int32_t mea_abi_version(void) { return MEA_ABI_VERSION; }

}  // extern "C"
