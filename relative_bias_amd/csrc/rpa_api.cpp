// C-ABI host layer of librpa.so: argument validation, the split planner and
// kernel launches.  Every check here runs before any HIP call, so error
// paths are testable on a machine without a GPU.
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "rpa.h"
#include "rpa_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte offset of the partial-LSE array inside the workspace.
size_t part_lse_offset(int64_t S, int64_t T, int64_t H, int64_t D) {
  return round_up((size_t)S * (size_t)T * (size_t)H * (size_t)D * sizeof(float), kAlign);
}

}  // namespace

extern "C" {

const char *rpa_status_string(int status) {
  switch (status) {
    case RPA_OK: return "ok";
    case RPA_ERR_NULL: return "a required pointer is NULL";
    case RPA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case RPA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size or bf16 rel_logits layout";
    case RPA_ERR_WORKSPACE: return "workspace missing or too small for num_splits";
    case RPA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t rpa_workspace_bytes(int32_t num_splits, int32_t num_tokens, int32_t num_heads, int32_t head_dim) {
  if (num_splits < 0 || num_splits == 1 || num_tokens < 0 || num_heads < 0 || head_dim < 0) return 0;
  if (num_splits == 0) return round_up(rpa::bal_desc_bytes() + rpa::bal_part_bytes(head_dim), kAlign);
  const size_t n = (size_t)num_splits * (size_t)num_tokens * (size_t)num_heads;
  return round_up(part_lse_offset(num_splits, num_tokens, num_heads, head_dim) + n * sizeof(float), kAlign);
}

// Planner: work items are (request, q-tile, kv head).  A decode batch gets
// 0, the balanced decode, which cuts the batch's KV into equal shares per
// CU whatever the length mix.  Otherwise the split count is raised until
// the grid offers about two workgroups per CU, never below 512 keys per
// split and never above RPA_MAX_SPLITS.  A window bounds the keys a row
// sees, so local attention is not split, as in the walkthrough's
// inkling_fa4_num_splits.
int rpa_choose_splits(int32_t batch, int32_t max_seqlen_q, int32_t num_heads, int32_t num_kv_heads,
                      int64_t max_seqlen_k, int is_local, int32_t num_cus) {
  if (batch < 0 || max_seqlen_q < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_seqlen_k < 0 ||
      num_heads % num_kv_heads != 0)
    return RPA_ERR_SHAPE;
  if (num_cus <= 0) num_cus = 256;
  if (batch == 0 || max_seqlen_q == 0 || max_seqlen_k == 0 || is_local) return 1;
  const int64_t G = num_heads / num_kv_heads;
  const int64_t items = rpa::items_for_request(max_seqlen_q, G);
  const bool decode = G <= rpa::kDecCols && (int64_t)max_seqlen_q * G <= rpa::kDecCols;
  const int64_t base = (int64_t)batch * num_kv_heads * items;
  if (decode && batch <= rpa::kBalMaxBatch) return 0;
  const int64_t target = (decode ? 4 : 2) * (int64_t)num_cus;
  int64_t s = (target + base - 1) / base;
  const int64_t by_len = max_seqlen_k / 512;
  if (s > by_len) s = by_len;
  if (s > RPA_MAX_SPLITS) s = RPA_MAX_SPLITS;
  if (s < 1) s = 1;
  return (int)s;
}

int rpa_split_combine(const float *partial_out, const float *partial_lse, int32_t num_splits,
                      int32_t num_tokens, int32_t num_heads, int32_t head_dim, void *out, float *lse,
                      void *stream) {
  if (num_splits < 1 || num_splits > RPA_MAX_SPLITS || num_tokens < 0 || num_heads <= 0 ||
      head_dim <= 0)
    return RPA_ERR_SHAPE;
  if (head_dim % 64 != 0 || head_dim > 256) return RPA_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens * num_heads > INT32_MAX) return RPA_ERR_SHAPE;
  if (num_tokens == 0) return RPA_OK;
  if (!partial_out || !partial_lse || !out) return RPA_ERR_NULL;
  rpa::CombineParams p;
  p.part_out = partial_out;
  p.part_lse = partial_lse;
  p.out = static_cast<uint16_t *>(out);
  p.lse = lse;
  p.S = num_splits;
  p.rows = num_tokens * num_heads;
  p.D = head_dim;
  if (rpa::launch_combine(p, static_cast<hipStream_t>(stream)) != hipSuccess) return RPA_ERR_HIP;
  return RPA_OK;
}

}  // extern "C"

namespace {

// Workspace of the balanced decode with `wgs` workgroups: the per-workgroup
// records (sized for kBalMaxWGs), then two partial slots per workgroup.
size_t bal_workspace_bytes(int wgs, int head_dim) {
  return round_up(rpa::bal_desc_bytes() + rpa::bal_part_bytes(head_dim, wgs), kAlign);
}

// Every attention entry point: kv8 selects E4M3 caches with their scales.
// use_scratch (rpa_attn_varlen_noalloc): the workspace is the current
// device's static scratch array, looked up after every argument check and
// only when the call needs a workspace; its size is checked against what
// the call needs on this device.
int attn_impl(const void *q, const void *key_cache, const void *value_cache, bool kv8, float k_scale,
              float v_scale, const int32_t *block_table, int32_t max_pages_per_seq,
              const int32_t *cache_seqlens, const int32_t *cu_seqlens_q, int32_t batch, int32_t num_tokens,
              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
              int32_t max_seqlen_q, float softmax_scale, int causal, int32_t window_left, int32_t window_right,
              int32_t rel_extent, const float *rel_logits, bool rel_bf16, const float *alibi_slopes,
              int32_t num_splits, void *workspace, size_t workspace_bytes, void *out, float *lse, void *stream,
              bool use_scratch = false) {
  if (kv8 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return RPA_ERR_SHAPE;
  // Sizes.
  if (batch < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_blocks < 0 || block_size <= 0 || max_pages_per_seq < 0 || max_seqlen_q < 0 ||
      rel_extent < 0 || window_left < -1 || window_right < -1)
    return RPA_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0) return RPA_ERR_SHAPE;
  // Key positions, row offsets (qa = i + Lk - Lq, with Lk at most
  // max_pages_per_seq * block_size) and the band's lower end qa - R + 1 are
  // 32-bit on the device.
  if ((int64_t)max_pages_per_seq * block_size + max_seqlen_q + rel_extent + rpa::kTileRows >= ((int64_t)1 << 31))
    return RPA_ERR_SHAPE;
  // A window side that reaches past every key leaves that side unbounded:
  // no key lies more than max_pages_per_seq * block_size - 1 to the left of
  // a row, nor more than max_seqlen_q - 1 to its right.  Taken as -1 here,
  // so that the device never adds a window near 2^31 to a position.
  if (window_left >= 0 && (int64_t)window_left >= (int64_t)max_pages_per_seq * block_size) window_left = -1;
  if (window_right >= 0 && window_right >= max_seqlen_q) window_right = -1;
  if (num_splits < 0 || num_splits > RPA_MAX_SPLITS) return RPA_ERR_SHAPE;
  if (!std::isfinite(softmax_scale)) return RPA_ERR_SHAPE;
  if (batch == 0 && num_tokens > 0) return RPA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return RPA_ERR_UNSUPPORTED;
  if (block_size % 16 != 0) return RPA_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens * num_heads * head_dim > ((int64_t)1 << 40)) return RPA_ERR_SHAPE;
  // bf16 rel_logits in prefill tiles: one buffer resource spans the rows of a
  // 128-row tile (up to 128 / G + 2 tokens of every head), below 2 GiB.
  if (rel_bf16 && rel_extent > 0) {
    // bf16 rel_logits are read as dwords: the array must start on one.
    if (rel_logits && (reinterpret_cast<uintptr_t>(rel_logits) & 3) != 0) return RPA_ERR_UNSUPPORTED;
    const int64_t g_ = num_heads / num_kv_heads;
    const bool has_prefill = (int64_t)max_seqlen_q * g_ > rpa::kDecCols || g_ > rpa::kDecCols;
    if (has_prefill && ((int64_t)rpa::kTileRows / g_ + 2) * num_heads * rel_extent * 2 + 64 >= ((int64_t)1 << 31))
      return RPA_ERR_UNSUPPORTED;
  }
  if (num_tokens == 0) return RPA_OK;
  // Pointers.
  if (!q || !key_cache || !value_cache || !block_table || !cache_seqlens || !cu_seqlens_q || !out)
    return RPA_ERR_NULL;
  if (rel_extent > 0 && !rel_logits) return RPA_ERR_NULL;
  // Workspace for split partials (a caller-given buffer: the size that
  // rpa_workspace_bytes states, whatever the device).
  if (num_splits != 1 && !use_scratch) {
    if (!workspace) return RPA_ERR_WORKSPACE;
    if (workspace_bytes < rpa_workspace_bytes(num_splits, num_tokens, num_heads, head_dim))
      return RPA_ERR_WORKSPACE;
  }
  // Grid: an upper bound on the work items.  Each request gives at most
  // ceil(Lq*G/128) + 1 items and at most items_for_request(max_seqlen_q).
  const int64_t G = num_heads / num_kv_heads;
  const int64_t ub_tokens = (int64_t)batch + ((int64_t)num_tokens * G + rpa::kTileRows - 1) / rpa::kTileRows;
  const int64_t ub_maxq = (int64_t)batch * rpa::items_for_request(max_seqlen_q, G);
  const int64_t n_items_ub = ub_tokens < ub_maxq ? ub_tokens : ub_maxq;
  const bool decode_only = G <= rpa::kDecCols && (int64_t)max_seqlen_q * G <= rpa::kDecCols;
  // num_splits = 0: the balanced decode where it applies, else one split.
  const bool balanced = num_splits == 0 && decode_only && batch <= rpa::kBalMaxBatch &&
                        (int64_t)num_tokens * num_heads * rel_extent * 4 < ((int64_t)1 << 31);
  if (num_splits == 0 && !balanced) num_splits = 1;
  if (n_items_ub * num_kv_heads * (int64_t)num_splits > INT32_MAX) return RPA_ERR_SHAPE;
  int32_t bal_wgs = 0;
  if (balanced) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return RPA_ERR_HIP;
    bal_wgs = cus < rpa::kBalMaxWGs ? cus : rpa::kBalMaxWGs;
  }
  if (use_scratch) {
    const size_t need = balanced ? bal_workspace_bytes(bal_wgs, head_dim)
                        : num_splits > 1 ? rpa_workspace_bytes(num_splits, num_tokens, num_heads, head_dim)
                                         : 0;
    if (need > rpa::kScratchBytes) return RPA_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      if (rpa::scratch_device_ptr(&workspace) != hipSuccess) return RPA_ERR_HIP;
      workspace_bytes = rpa::kScratchBytes;
    }
  }

  rpa::AttnParams p;
  p.q = static_cast<const uint16_t *>(q);
  p.k = static_cast<const uint16_t *>(key_cache);
  p.v = static_cast<const uint16_t *>(value_cache);
  p.block_table = block_table;
  p.cache_seqlens = cache_seqlens;
  p.cu_seqlens_q = cu_seqlens_q;
  p.rel_logits = rel_extent > 0 ? rel_logits : nullptr;
  p.out = static_cast<uint16_t *>(out);
  p.lse = lse;
  p.part_out = nullptr;
  p.part_lse = nullptr;
  p.bal_part = nullptr;
  p.bal_desc = nullptr;
  p.bal_wgs = bal_wgs;
  if (balanced) {
    p.bal_desc = static_cast<int32_t *>(workspace);
    p.bal_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + rpa::bal_desc_bytes());
  }
  if (num_splits > 1) {
    p.part_out = static_cast<float *>(workspace);
    p.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                           part_lse_offset(num_splits, num_tokens, num_heads, head_dim));
  }
  p.batch = batch;
  p.num_tokens = num_tokens;
  p.H = num_heads;
  p.Hkv = num_kv_heads;
  p.G = (int32_t)G;
  p.BS = block_size;
  p.R = rel_extent;
  p.S = num_splits;
  p.P = max_pages_per_seq;
  p.left = window_left;
  p.right = window_right;
  p.causal = causal ? 1 : 0;
  p.bs_shift = -1;
  for (int sh = 4; sh < 31; ++sh)
    if ((1 << sh) == block_size) p.bs_shift = sh;
  // An E4M3 cache's k_scale multiplies <q, k> alone, so it joins the softmax
  // scale; v_scale multiplies the normalised output.
  const double qk_scale = (double)softmax_scale * (kv8 ? (double)k_scale : 1.0);
  p.scale = (float)qk_scale;
  p.scale_log2 = (float)(qk_scale * 1.4426950408889634);
  p.v_scale = kv8 ? v_scale : 1.f;
  p.kv8 = kv8 ? 1 : 0;
  p.alibi = alibi_slopes;
  p.rel_bf16 = rel_bf16 ? 1 : 0;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (balanced) return rpa::launch_balanced_decode(p, head_dim, st) == hipSuccess ? RPA_OK : RPA_ERR_HIP;
  if (rpa::launch_attention(p, head_dim, n_items_ub, decode_only, st) != hipSuccess) return RPA_ERR_HIP;
  if (num_splits > 1) {
    rpa::CombineParams c;
    c.part_out = p.part_out;
    c.part_lse = p.part_lse;
    c.out = p.out;
    c.lse = lse;
    c.S = num_splits;
    c.rows = num_tokens * num_heads;
    c.D = head_dim;
    if (rpa::launch_combine(c, st) != hipSuccess) return RPA_ERR_HIP;
  }
  return RPA_OK;
}

}  // namespace

extern "C" {

int rpa_attn_varlen(const void *q, const void *key_cache, const void *value_cache,
                    const int32_t *block_table, int32_t max_pages_per_seq,
                    const int32_t *cache_seqlens, const int32_t *cu_seqlens_q, int32_t batch,
                    int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t num_blocks, int32_t block_size, int32_t max_seqlen_q, float softmax_scale,
                    int causal, int32_t window_left, int32_t window_right, int32_t rel_extent,
                    const float *rel_logits, int32_t num_splits, void *workspace,
                    size_t workspace_bytes, void *out, float *lse, void *stream) {
  return attn_impl(q, key_cache, value_cache, false, 1.f, 1.f, block_table, max_pages_per_seq, cache_seqlens,
                   cu_seqlens_q, batch, num_tokens, num_heads, num_kv_heads, head_dim, num_blocks, block_size,
                   max_seqlen_q, softmax_scale, causal, window_left, window_right, rel_extent, rel_logits, false,
                   nullptr, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int rpa_attn_varlen_fp8(const void *q, const void *key_cache, const void *value_cache, float k_scale,
                        float v_scale, const int32_t *block_table, int32_t max_pages_per_seq,
                        const int32_t *cache_seqlens, const int32_t *cu_seqlens_q, int32_t batch,
                        int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t num_blocks, int32_t block_size, int32_t max_seqlen_q, float softmax_scale,
                        int causal, int32_t window_left, int32_t window_right, int32_t rel_extent,
                        const float *rel_logits, int32_t num_splits, void *workspace,
                        size_t workspace_bytes, void *out, float *lse, void *stream) {
  return attn_impl(q, key_cache, value_cache, true, k_scale, v_scale, block_table, max_pages_per_seq,
                   cache_seqlens, cu_seqlens_q, batch, num_tokens, num_heads, num_kv_heads, head_dim, num_blocks,
                   block_size, max_seqlen_q, softmax_scale, causal, window_left, window_right, rel_extent,
                   rel_logits, false, nullptr, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int rpa_attn_varlen_ex(const void *q, const void *key_cache, const void *value_cache, int kv_e4m3, float k_scale,
                       float v_scale, const int32_t *block_table, int32_t max_pages_per_seq,
                       const int32_t *cache_seqlens, const int32_t *cu_seqlens_q, int32_t batch,
                       int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t num_blocks, int32_t block_size, int32_t max_seqlen_q, float softmax_scale,
                       int causal, int32_t window_left, int32_t window_right, int32_t rel_extent,
                       const void *rel_logits, int rel_logits_bf16, const float *alibi_slopes, int32_t num_splits,
                       void *workspace, size_t workspace_bytes, void *out, float *lse, void *stream) {
  return attn_impl(q, key_cache, value_cache, kv_e4m3 != 0, k_scale, v_scale, block_table, max_pages_per_seq,
                   cache_seqlens, cu_seqlens_q, batch, num_tokens, num_heads, num_kv_heads, head_dim, num_blocks,
                   block_size, max_seqlen_q, softmax_scale, causal, window_left, window_right, rel_extent,
                   static_cast<const float *>(rel_logits), rel_logits_bf16 != 0, alibi_slopes, num_splits, workspace,
                   workspace_bytes, out, lse, stream);
}

int rpa_attn_varlen_noalloc(const void *q, const void *key_cache, const void *value_cache, int kv_e4m3,
                            float k_scale, float v_scale, const int32_t *block_table, int32_t max_pages_per_seq,
                            const int32_t *cache_seqlens, const int32_t *cu_seqlens_q, int32_t batch,
                            int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t num_blocks, int32_t block_size, int32_t max_seqlen_q, float softmax_scale,
                            int causal, int32_t window_left, int32_t window_right, int32_t rel_extent,
                            const void *rel_logits, int rel_logits_bf16, const float *alibi_slopes,
                            int32_t num_splits, void *out, float *lse, void *stream) {
  return attn_impl(q, key_cache, value_cache, kv_e4m3 != 0, k_scale, v_scale, block_table, max_pages_per_seq,
                   cache_seqlens, cu_seqlens_q, batch, num_tokens, num_heads, num_kv_heads, head_dim, num_blocks,
                   block_size, max_seqlen_q, softmax_scale, causal, window_left, window_right, rel_extent,
                   static_cast<const float *>(rel_logits), rel_logits_bf16 != 0, alibi_slopes, num_splits, nullptr, 0,
                   out, lse, stream, true);
}

int rpa_slot_mapping(const int32_t *block_table, int32_t max_pages_per_seq, const int32_t *cache_seqlens,
                     const int32_t *cu_seqlens_q, int32_t batch, int32_t num_tokens, int32_t block_size,
                     int64_t *slot_mapping, void *stream) {
  if (batch < 0 || num_tokens < 0 || block_size <= 0 || max_pages_per_seq < 0) return RPA_ERR_SHAPE;
  if (batch == 0 && num_tokens > 0) return RPA_ERR_SHAPE;
  if (num_tokens == 0) return RPA_OK;
  if (!block_table || !cache_seqlens || !cu_seqlens_q || !slot_mapping) return RPA_ERR_NULL;
  rpa::SlotParams p;
  p.block_table = block_table;
  p.cache_seqlens = cache_seqlens;
  p.cu_seqlens_q = cu_seqlens_q;
  p.slots = slot_mapping;
  p.batch = batch;
  p.num_tokens = num_tokens;
  p.P = max_pages_per_seq;
  p.BS = block_size;
  return rpa::launch_slot_mapping(p, static_cast<hipStream_t>(stream)) == hipSuccess ? RPA_OK : RPA_ERR_HIP;
}

int rpa_kv_cache_write(const void *key, const void *value, const int64_t *slot_mapping, int32_t num_tokens,
                       int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                       void *key_cache, void *value_cache, void *stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0 || block_size <= 0)
    return RPA_ERR_SHAPE;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row % 8 != 0) return RPA_ERR_UNSUPPORTED;
  if (row / 8 > INT32_MAX) return RPA_ERR_SHAPE;
  if (num_tokens == 0) return RPA_OK;
  if (!key || !value || !slot_mapping || !key_cache || !value_cache) return RPA_ERR_NULL;
  rpa::KvWriteParams p;
  p.key = static_cast<const uint16_t *>(key);
  p.value = static_cast<const uint16_t *>(value);
  p.slots = slot_mapping;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.capacity = (int64_t)num_blocks * block_size;
  p.num_tokens = num_tokens;
  p.row_units = (int32_t)(row / 8);
  p.k_scale = 1.f;
  p.v_scale = 1.f;
  return rpa::launch_kv_write(p, static_cast<hipStream_t>(stream)) == hipSuccess ? RPA_OK : RPA_ERR_HIP;
}

int rpa_kv_cache_write_fp8(const void *key, const void *value, const int64_t *slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                           float k_scale, float v_scale, void *key_cache, void *value_cache, void *stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0 || block_size <= 0)
    return RPA_ERR_SHAPE;
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return RPA_ERR_SHAPE;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row % 8 != 0) return RPA_ERR_UNSUPPORTED;
  if (row / 8 > INT32_MAX) return RPA_ERR_SHAPE;
  if (num_tokens == 0) return RPA_OK;
  if (!key || !value || !slot_mapping || !key_cache || !value_cache) return RPA_ERR_NULL;
  rpa::KvWriteParams p;
  p.key = static_cast<const uint16_t *>(key);
  p.value = static_cast<const uint16_t *>(value);
  p.slots = slot_mapping;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.capacity = (int64_t)num_blocks * block_size;
  p.num_tokens = num_tokens;
  p.row_units = (int32_t)(row / 8);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  return rpa::launch_kv_write_fp8(p, static_cast<hipStream_t>(stream)) == hipSuccess ? RPA_OK : RPA_ERR_HIP;
}

}  // extern "C"
