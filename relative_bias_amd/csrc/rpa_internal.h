// Internal interface between the C-ABI host layer (rpa_api.cpp) and the HIP
// kernels (rpa_kernels.hip).  Not installed; include/rpa.h is the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa.h"

namespace rpa {

// Work decomposition shared by host and device.
constexpr int kThreads = 256;      // 4 wave64 per workgroup
constexpr int kTileRows = 128;     // prefill q-tile: (token, head) rows of one kv head
constexpr int kTileKeys = 64;      // prefill KV tile
constexpr int kDecCols = 16;       // decode item: up to 16 (token, head) columns
constexpr int kDecWaveKeys = 32;   // keys per wave per decode iteration

// Balanced decode (num_splits = 0 on a decode-only batch).
constexpr int kBalWaves = 8;        // waves per workgroup (one workgroup per CU)
constexpr int kBalMaxBatch = 2048;  // requests (their unit prefix sums live in LDS)
constexpr int kBalMaxWGs = 512;     // workgroups at most
constexpr int kBalDescInts = 8;     // per-workgroup combine record
constexpr int kBalHeads = 8;        // kv heads streamed side by side (one per wave)
// Workspace of the balanced decode: kBalMaxWGs records, then two partial
// slots per workgroup, each with kBalHeads entries of kDecCols *
// (head_dim + 1) fp32 (outputs, then LSEs).  The one-head-per-workgroup
// form uses the first entry of each slot.
__host__ __device__ inline size_t bal_desc_bytes() { return (size_t)kBalMaxWGs * kBalDescInts * 4; }
__host__ __device__ inline size_t bal_part_bytes(int head_dim, int wgs = kBalMaxWGs) {
  return (size_t)2 * wgs * kBalHeads * kDecCols * (size_t)(head_dim + 1) * 4;
}

// Scratch of rpa_attn_varlen_noalloc: a static device array of this many
// bytes on every GPU the library runs on (enough for the balanced decode of
// head_dim 128 on up to 300 compute units, or for split partials of that
// size).
constexpr size_t kScratchBytes = RPA_NOALLOC_SCRATCH_BYTES;
// Device address of the current GPU's scratch array, looked up once per
// device (hipGetSymbolAddress) and cached.
hipError_t scratch_device_ptr(void **ptr);

struct AttnParams {
  const uint16_t *q;            // bf16 [T, H, D]
  const uint16_t *k;            // bf16 [NB, BS, Hkv, D]
  const uint16_t *v;            // bf16 [NB, BS, Hkv, D]
  const int32_t *block_table;   // [B, P]
  const int32_t *cache_seqlens; // [B]
  const int32_t *cu_seqlens_q;  // [B+1]
  const float *rel_logits;      // [T, H, R] or null
  uint16_t *out;                // bf16 [T, H, D]
  float *lse;                   // [T, H] or null
  float *part_out;              // [S, T, H, D] when S > 1
  float *part_lse;              // [S, T, H]   when S > 1
  int32_t batch, num_tokens, H, Hkv, G, BS, R, S, P;
  int32_t left, right, causal;
  int32_t bs_shift;             // log2(BS) when BS is a power of two, else -1
  float *bal_part;              // balanced decode: partial slots
  int32_t *bal_desc;            // balanced decode: per-workgroup combine records
  int32_t bal_wgs;              // balanced decode: workgroups
  float scale;                  // softmax_scale (times k_scale for E4M3 caches)
  float scale_log2;             // scale * log2(e)
  float v_scale;                // E4M3 caches: the value cache's scale (1 for bf16 caches)
  int32_t kv8;                  // 1: k / v are E4M3 codes (uint8) instead of bf16
  const float *alibi;           // [H] ALiBi slopes, or null
  int32_t rel_bf16;             // 1: rel_logits holds bf16 values (uint16) instead of fp32
};

struct CombineParams {
  const float *part_out;        // [S, T, H, D]
  const float *part_lse;        // [S, T, H], natural log
  uint16_t *out;                // bf16 [T, H, D]
  float *lse;                   // [T, H] or null
  int32_t S, rows, D;           // rows = T * H
  int32_t wr;                   // waves per row (set by launch_combine)
};

struct SlotParams {
  const int32_t *block_table;   // [B, P]
  const int32_t *cache_seqlens; // [B]
  const int32_t *cu_seqlens_q;  // [B+1]
  int64_t *slots;               // [T]
  int32_t batch, num_tokens, P, BS;
};

struct KvWriteParams {
  const uint16_t *key;          // bf16 [T, Hkv, D]
  const uint16_t *value;        // bf16 [T, Hkv, D]
  const int64_t *slots;         // [T]
  void *key_cache;              // bf16 (or E4M3 codes) [NB, BS, Hkv, D]
  void *value_cache;            // bf16 (or E4M3 codes) [NB, BS, Hkv, D]
  int64_t capacity;             // NB * BS slots
  int32_t num_tokens, row_units;  // row_units: 16-byte bf16 units per token row (Hkv * D / 8)
  float k_scale, v_scale;       // E4M3 caches: quantisation scales
};

// Number of work items a request with lq query tokens contributes.
__host__ __device__ inline int64_t items_for_request(int64_t lq, int64_t G) {
  if (lq <= 0) return 0;
  if (G <= kDecCols && lq * G <= kDecCols) return 1;  // decode item
  return (lq * G + kTileRows - 1) / kTileRows;        // prefill q-tiles
}

// decode_only: every request has Lq * G <= kDecCols (the prefill path is
// then left out of the launched kernel).
hipError_t launch_attention(const AttnParams &p, int head_dim, int64_t n_items_ub, bool decode_only,
                            hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, hipStream_t stream);
hipError_t launch_slot_mapping(const SlotParams &p, hipStream_t stream);
hipError_t launch_kv_write(const KvWriteParams &p, hipStream_t stream);
hipError_t launch_kv_write_fp8(const KvWriteParams &p, hipStream_t stream);
// Balanced decode: the attention kernel on p.bal_wgs workgroups, then the
// combine of the pairs cut between workgroups.
hipError_t launch_balanced_decode(const AttnParams &p, int head_dim, hipStream_t stream);

}  // namespace rpa
