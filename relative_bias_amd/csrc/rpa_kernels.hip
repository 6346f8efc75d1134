// HIP kernels for paged, varlen, causal attention with an additive relative
// position bias, written for gfx950 (MI355X, CDNA4, wave64).
//
// Method: the Inkling FA4 relative-attention walkthrough
// ("vllm中提取Inkling FA4 Relative Attention算子基础的base优化版本",
// nxmr.cn/news/19446): the FA4 inner loop scales Q·Kᵀ by softmax_scale,
// applies the score_mod that adds rel_logits[token, head, q_abs - kv_pos]
// when that distance lies in [0, rel_extent), runs an online softmax and
// accumulates P·V; split-KV partials are merged by a log-sum-exp combine
// ("paged_attention_v2_pytorch.py — BI-V100 PagedAttention V2", phase 2).
//
// One launch serves a whole mixed batch.  Workgroup id = (item, kv head,
// split); each workgroup finds its request by scanning cu_seqlens_q on the
// device, so no host-side metadata and no device->host copy is needed.
//   * prefill item: 128 (token, q-head) rows of one kv head.  Four waves,
//     32 rows each.  S^T = K·Q^T and O^T = V^T·P^T on 32x32x16 bf16 MFMA so
//     that each lane owns one query row: softmax statistics stay lane-local
//     except one exchange with the partner lane 32 away.
//   * decode item: up to 16 (token, q-head) columns of one kv head (the GQA
//     group shares every K/V row it reads).  Four waves stream disjoint
//     32-key blocks straight from HBM into 16x16x32 MFMA operands and merge
//     their softmax states through LDS at the end.
// K rows feed MFMA A operands directly (16-byte loads).  V is transposed to
// V^T in LDS (register 8x8 / 4x8 transposes) so that each lane reads eight
// consecutive keys of one head_dim column.  The key order inside each 16/32
// key chunk is permuted so that the softmax output already sits in the P^T
// operand layout; K/V operands follow the same permutation.
#include "rpa_internal.h"

namespace rpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack8_bf16(const float *x) {
  u32x4 u = {pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]), pack2_bf16(x[4], x[5]),
             pack2_bf16(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Element e (0..7) of two 8 x bf16 rows, packed as (a_e, b_e).
__device__ __forceinline__ uint32_t pair_elem(u32x4 a, u32x4 b, int e) {
  const uint32_t x = a[e >> 1], y = b[e >> 1];
  return (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
}

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Orders this wave's LDS writes before its later LDS reads (and vice versa).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

struct Item {
  int b;     // request
  int tile;  // q-tile within the request (prefill)
  int kind;  // 0 none, 1 prefill, 2 decode
};

// Maps a linear work-item index to (request, tile).  Items are numbered in
// request order; request b contributes items_for_request(Lq_b, G) of them.
// Every wave scans independently (the reads hit cache), so no barrier.
__device__ Item resolve_item(const AttnParams &p, int item) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c = 0; c < p.batch; c += 64) {
    const int b = c + lane;
    int n = 0, lq = 0;
    if (b < p.batch) {
      lq = p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
      n = (int)items_for_request(lq, p.G);
    }
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int excl = incl - n;
    const bool hit = item >= base + excl && item < base + incl;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll((long long)mask) - 1;
      const int e = __shfl(excl, src);
      const int lqs = __shfl(lq, src);
      const bool dec = (int64_t)lqs * p.G <= kDecCols && p.G <= kDecCols;
      return Item{c + src, item - base - e, dec ? 2 : 1};
    }
    base += __shfl(incl, 63);
  }
  return Item{-1, 0, 0};
}

// Key range [lo, hi) visible to rows with absolute positions in
// [qa_min, qa_max] (window / causal / length), before splitting.
struct Range {
  int lo, hi;
};
__device__ __forceinline__ Range visible_range(const AttnParams &p, int lk, int qa_min, int qa_max) {
  int hi = lk;
  if (p.causal) hi = min(hi, qa_max + 1);
  if (p.right >= 0) hi = min(hi, qa_max + p.right + 1);
  int lo = 0;
  if (p.left >= 0) lo = max(0, qa_min - p.left);
  return Range{lo, hi};
}

// Contiguous cut s of S over [lo aligned down to 16, hi), chunks rounded to
// `align` keys.  Empty when t0 >= t1.
__device__ __forceinline__ Range split_range(Range r, int S, int s, int align) {
  const int lo_a = r.lo & ~15;
  const int span = r.hi - lo_a;
  if (span <= 0) return Range{0, 0};
  int chunk = (span + S - 1) / S;
  chunk = (chunk + align - 1) / align * align;
  const int t0 = lo_a + s * chunk;
  return Range{t0, min(r.hi, t0 + chunk)};
}

// ---------------------------------------------------------------- prefill

template <int D>
struct PrefillLds {
  static constexpr int KS = D + 8;          // K tile row stride (bf16): +16 B pad
  static constexpr int VS = kTileKeys + 8;  // V^T row stride (bf16): +16 B pad
  static constexpr int kBytes = kTileKeys * KS * 2;
  static constexpr int vBytes = D * VS * 2;
  static constexpr int bytes = kBytes + vBytes;
};

// Position of key kl (0..63) of a prefill KV tile inside a V^T row.  Within
// each 16-key chunk c, slot 8h + i (h = half-wave, i = operand element)
// holds key 16c + 8(i/4) + 4h + i%4: the keys that lane (row, h) of the
// 32x32 S^T accumulator holds for that chunk.
__device__ __forceinline__ int prefill_vpos(int kl) {
  return 16 * (kl >> 4) + 8 * ((kl >> 2) & 1) + 4 * ((kl >> 3) & 1) + (kl & 3);
}

template <int D, bool MASK, bool BIAS>
__device__ __forceinline__ void prefill_tile_step(const uint16_t *Ks, const uint16_t *Vt,
                                                  const bf16x8 *qf, f32x16 *oacc, float &m_run,
                                                  float &l_run, int kb, int lo_r, int hi_r, int qa,
                                                  const float *rel_row, int R, float scale_log2,
                                                  int l32, int hf) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KS = PrefillLds<D>::KS;
  constexpr int VS = PrefillLds<D>::VS;
  f32x16 sacc[2];
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    sacc[kb2] = f32x16{};
    const uint16_t *kp = Ks + (32 * kb2 + l32) * KS + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) sacc[kb2] = mfma32(as_bf16x8(ld16(kp + 16 * ks)), qf[ks], sacc[kb2]);
  }
  // Lane (l32, hf) holds S[row l32][key kb + 32 kb2 + 8 (j/4) + 4 hf + j%4].
  float x[2][16];
  float mx = neg_inf();
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = kb + 32 * kb2 + 8 * (j >> 2) + 4 * hf + (j & 3);
      float v = sacc[kb2][j] * scale_log2;
      if (BIAS) {
        const int d = qa - t;
        if ((unsigned)d < (unsigned)R) v = __builtin_fmaf(rel_row[d], kLog2e, v);
      }
      if (MASK) {
        if (t < lo_r || t > hi_r) v = neg_inf();
      }
      x[kb2][j] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float m_use = m_new == neg_inf() ? 0.f : m_new;
  const float alpha = exp2_fast(m_run - m_use);
  m_run = m_new;
  float psum = 0.f;
  bf16x8 pb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float pe[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pe[i] = exp2_fast(x[c >> 1][8 * (c & 1) + i] - m_use);
      psum += pe[i];
    }
    pb[c] = pack8_bf16(pe);
  }
  l_run = l_run * alpha + psum;
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = as_bf16x8(ld16(Vt + (32 * db + l32) * VS + 16 * c + 8 * hf));
      oacc[db] = mfma32(a, pb[c], oacc[db]);
    }
  }
}

template <int D>
__device__ void prefill_item(const AttnParams &p, int b, int tile, int g, int s, char *smem) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CH = D / 8;                          // 16-byte chunks per K/V row
  constexpr int KPT = kTileKeys * CH / kThreads;     // staged keys per thread (4 or 2)
  constexpr int NKG = kTileKeys / KPT;               // key groups per tile
  constexpr int KS = PrefillLds<D>::KS;
  constexpr int VS = PrefillLds<D>::VS;
  static_assert(KPT == 4 || KPT == 2, "staging layout");
  uint16_t *Ks = reinterpret_cast<uint16_t *>(smem);
  uint16_t *Vt = reinterpret_cast<uint16_t *>(smem + PrefillLds<D>::kBytes);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int tok0 = p.cu_seqlens_q[b];
  const int lq = p.cu_seqlens_q[b + 1] - tok0;
  const int lk = p.cache_seqlens[b];
  const int G = p.G;
  const int nrows = lq * G;
  const int row0 = tile * kTileRows;
  const int row_last = min(row0 + kTileRows, nrows) - 1;
  int r = row0 + 32 * w + l32;
  const bool row_valid = r <= row_last;
  if (!row_valid) r = row_last;  // idle lanes shadow the last row; never stored
  const int qi = r / G;
  const int head = g * G + (r - qi * G);
  const int tok = tok0 + qi;
  const int qa = qi + lk - lq;
  const int qa_min = row0 / G + lk - lq;
  const int qa_max = row_last / G + lk - lq;

  const Range sr = split_range(visible_range(p, lk, qa_min, qa_max), p.S, s, kTileKeys);
  const int t0 = sr.lo, t1 = sr.hi;
  // This lane's visible keys inside the split: [lo_r, hi_r].
  int lo_r = t0, hi_r = min(lk, t1) - 1;
  if (p.left >= 0) lo_r = max(lo_r, qa - p.left);
  if (p.causal) hi_r = min(hi_r, qa);
  if (p.right >= 0) hi_r = min(hi_r, qa + p.right);
  // Keys in [in_lo, in_hi] are visible to every row of the tile.
  int in_lo = t0, in_hi = min(lk, t1) - 1;
  if (p.left >= 0) in_lo = max(in_lo, qa_max - p.left);
  if (p.causal) in_hi = min(in_hi, qa_min);
  if (p.right >= 0) in_hi = min(in_hi, qa_min + p.right);
  const int band_lo = qa_min - p.R + 1, band_hi = qa_max;
  const float *rel_row = p.R > 0 ? p.rel_logits + ((int64_t)tok * p.H + head) * p.R : nullptr;

  bf16x8 qf[KSTEPS];
  {
    const uint16_t *qp = p.q + ((int64_t)tok * p.H + head) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = as_bf16x8(ld16(qp + 16 * ks));
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = neg_inf(), l_run = 0.f;

  const int64_t tok_stride = (int64_t)p.Hkv * D;     // elements between consecutive slots
  const int32_t *bt = p.block_table + (int64_t)b * p.P;
  // K staging: 16-byte chunk dck of keys kgk*KPT .. +KPT-1 (chunk index fastest).
  const int dck = tid % CH, kgk = tid / CH;
  // V staging: key group fastest, so the transposed LDS writes spread over banks.
  const int kgv = tid % NKG, dcv = tid / NKG;
  u32x4 kreg[KPT], vreg[KPT];

  auto load_rows = [&](const uint16_t *base, int key0, int dc, u32x4 *regs) {
    if (key0 < lk) {
      const int page = bt[key0 / p.BS];
      const int64_t off = (((int64_t)page * p.BS + key0 % p.BS) * p.Hkv + g) * D + dc * 8;
#pragma unroll
      for (int rr = 0; rr < KPT; ++rr) regs[rr] = (key0 + rr < lk) ? ld16(base + off + rr * tok_stride) : zero16();
    } else {
#pragma unroll
      for (int rr = 0; rr < KPT; ++rr) regs[rr] = zero16();
    }
  };
  auto stage_load = [&](int kb) {
    load_rows(p.k, kb + kgk * KPT, dck, kreg);
    load_rows(p.v, kb + kgv * KPT, dcv, vreg);
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int rr = 0; rr < KPT; ++rr)
      *reinterpret_cast<u32x4 *>(Ks + (kgk * KPT + rr) * KS + dck * 8) = kreg[rr];
    const int pos = prefill_vpos(kgv * KPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t *dst = Vt + (dcv * 8 + e) * VS + pos;
      if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pair_elem(vreg[0], vreg[1], e), pair_elem(vreg[2], vreg[3], e)};
      } else {
        *reinterpret_cast<uint32_t *>(dst) = pair_elem(vreg[0], vreg[1], e);
      }
    }
  };

  if (t0 < t1) {
    stage_load(t0);
    for (int kb = t0; kb < t1; kb += kTileKeys) {
      __syncthreads();
      stage_store();
      __syncthreads();
      if (kb + kTileKeys < t1) stage_load(kb + kTileKeys);
      const bool interior = kb >= in_lo && kb + kTileKeys - 1 <= in_hi;
      const bool bias = p.R > 0 && kb <= band_hi && kb + kTileKeys - 1 >= band_lo;
      if (interior) {
        if (bias)
          prefill_tile_step<D, false, true>(Ks, Vt, qf, oacc, m_run, l_run, kb, lo_r, hi_r, qa, rel_row, p.R, p.scale_log2, l32, hf);
        else
          prefill_tile_step<D, false, false>(Ks, Vt, qf, oacc, m_run, l_run, kb, lo_r, hi_r, qa, rel_row, p.R, p.scale_log2, l32, hf);
      } else {
        if (bias)
          prefill_tile_step<D, true, true>(Ks, Vt, qf, oacc, m_run, l_run, kb, lo_r, hi_r, qa, rel_row, p.R, p.scale_log2, l32, hf);
        else
          prefill_tile_step<D, true, false>(Ks, Vt, qf, oacc, m_run, l_run, kb, lo_r, hi_r, qa, rel_row, p.R, p.scale_log2, l32, hf);
      }
    }
  }

  // Epilogue: lane (l32, hf) holds O^T[d = 32 db + 8 (j/4) + 4 hf + j%4][row l32].
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : neg_inf();
  if (!row_valid) return;
  if (p.S == 1) {
    uint16_t *op = p.out + ((int64_t)tok * p.H + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = 32 * db + 8 * jg + 4 * hf;
        *reinterpret_cast<u32x2 *>(op + d0) =
            u32x2{pack2_bf16(oacc[db][4 * jg] * inv, oacc[db][4 * jg + 1] * inv),
                  pack2_bf16(oacc[db][4 * jg + 2] * inv, oacc[db][4 * jg + 3] * inv)};
      }
    }
    if (hf == 0 && p.lse) p.lse[(int64_t)tok * p.H + head] = lse_v;
  } else {
    float *pp = p.part_out + (((int64_t)s * p.num_tokens + tok) * p.H + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = 32 * db + 8 * jg + 4 * hf;
        *reinterpret_cast<f32x4 *>(pp + d0) =
            f32x4{oacc[db][4 * jg] * inv, oacc[db][4 * jg + 1] * inv, oacc[db][4 * jg + 2] * inv,
                  oacc[db][4 * jg + 3] * inv};
      }
    }
    if (hf == 0) p.part_lse[((int64_t)s * p.num_tokens + tok) * p.H + head] = lse_v;
  }
}

// ----------------------------------------------------------------- decode

template <int D>
struct DecodeLds {
  static constexpr int VS = kDecWaveKeys + 8;              // V^T row stride (bf16): 80 B
  static constexpr int vtBytes = 4 * D * VS * 2;           // one V^T tile per wave
  static constexpr int redOBytes = 4 * D * kDecCols * 4;   // per-wave O^T partials
  static constexpr int redMLBytes = 2 * 4 * kDecCols * 4;  // per-wave m and l
  static constexpr int bytes = (vtBytes > redOBytes ? vtBytes : redOBytes) + redMLBytes;
};

// Key (0..31, relative to the wave's block) held at V^T slot p: slot 8q + i
// holds key 4q + i for i < 4 and 16 + 4q + i - 4 otherwise, matching the
// two 16x16 S^T accumulators of lane group q.
__device__ __forceinline__ int decode_key_of_slot(int p) {
  return 4 * (p >> 3) + (p & 7) + ((p & 4) ? 12 : 0);
}

template <int D>
struct DecodeRegs {
  u32x4 k[2][D / 32];
  u32x4 v[D / 16];
};

template <int D>
__device__ void decode_item(const AttnParams &p, int b, int g, int s, char *smem) {
  constexpr int QK = D / 32;       // 16x16x32 k-steps over head_dim
  constexpr int DB = D / 16;       // 16-row blocks of O^T
  constexpr int DQ = D / 4;        // head_dim span of one lane group in K operands
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int NG = 64 / CH;      // lane groups per chunk in V staging
  constexpr int KPL = kDecWaveKeys / NG;  // V keys per lane (8 or 4)
  constexpr int VS = DecodeLds<D>::VS;
  static_assert(KPL == 8 || KPL == 4, "staging layout");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, q = lane >> 4;
  uint16_t *Vt = reinterpret_cast<uint16_t *>(smem) + w * D * VS;

  const int tok0 = p.cu_seqlens_q[b];
  const int lq = p.cu_seqlens_q[b + 1] - tok0;
  const int lk = p.cache_seqlens[b];
  const int G = p.G;
  const int ncols = lq * G;
  const int col = c16 < ncols ? c16 : ncols - 1;  // idle columns shadow the last one
  const int qi = col / G;
  const int head = g * G + (col - qi * G);
  const int tok = tok0 + qi;
  const int qa = qi + lk - lq;
  const int qa_min = lk - lq;
  const int qa_max = (ncols - 1) / G + lk - lq;
  const Range sr = split_range(visible_range(p, lk, qa_min, qa_max), p.S, s, kDecStep);
  const int t0 = sr.lo, t1 = sr.hi;
  int lo_c = t0, hi_c = min(lk, t1) - 1;
  if (p.left >= 0) lo_c = max(lo_c, qa - p.left);
  if (p.causal) hi_c = min(hi_c, qa);
  if (p.right >= 0) hi_c = min(hi_c, qa + p.right);
  int in_lo = t0, in_hi = min(lk, t1) - 1;
  if (p.left >= 0) in_lo = max(in_lo, qa_max - p.left);
  if (p.causal) in_hi = min(in_hi, qa_min);
  if (p.right >= 0) in_hi = min(in_hi, qa_min + p.right);
  const int band_lo = qa_min - p.R + 1, band_hi = qa_max;
  const float *rel_row = p.R > 0 ? p.rel_logits + ((int64_t)tok * p.H + head) * p.R : nullptr;

  bf16x8 qf[QK];
  {
    const uint16_t *qp = p.q + ((int64_t)tok * p.H + head) * D + q * DQ;
#pragma unroll
    for (int ks = 0; ks < QK; ++ks) qf[ks] = as_bf16x8(ld16(qp + 8 * ks));
  }
  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};
  float m_run = neg_inf(), l_run = 0.f;

  const int64_t tok_stride = (int64_t)p.Hkv * D;
  const int32_t *bt = p.block_table + (int64_t)b * p.P;
  const int vg = lane % NG, vdc = lane / NG;

  auto issue = [&](DecodeRegs<D> &Rg, int base) {
    int64_t row0[2];  // element offset of slot 0 of each 16-key block
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kb = base + 16 * blk;
      int page = 0, slot0 = 0;
      if (kb < lk) {
        page = bt[kb / p.BS];
        slot0 = kb % p.BS;
      }
      row0[blk] = (((int64_t)page * p.BS + slot0) * p.Hkv + g) * D;
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = base + 16 * blk + c16;
      const uint16_t *src = p.k + row0[blk] + c16 * tok_stride + q * DQ;
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) Rg.k[blk][ks] = key < lk ? ld16(src + 8 * ks) : zero16();
    }
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) {
      const int kr = decode_key_of_slot(vg * KPL + rr);
      const int blk = kr >> 4;
      const int key = base + kr;
      Rg.v[rr] = key < lk ? ld16(p.v + row0[blk] + (kr & 15) * tok_stride + vdc * 8) : zero16();
    }
  };

  auto compute = [&](DecodeRegs<D> &Rg, int base, auto mask_tag, auto bias_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool BIAS = decltype(bias_tag)::value;
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t *dst = Vt + (vdc * 8 + e) * VS + vg * KPL;
      if constexpr (KPL == 8) {
        *reinterpret_cast<u32x4 *>(dst) =
            u32x4{pair_elem(Rg.v[0], Rg.v[1], e), pair_elem(Rg.v[2], Rg.v[3], e),
                  pair_elem(Rg.v[4], Rg.v[5], e), pair_elem(Rg.v[6], Rg.v[7], e)};
      } else {
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pair_elem(Rg.v[0], Rg.v[1], e), pair_elem(Rg.v[2], Rg.v[3], e)};
      }
    }
    f32x4 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sacc[blk] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) sacc[blk] = mfma16(as_bf16x8(Rg.k[blk][ks]), qf[ks], sacc[blk]);
    }
    // Lane (c16, q) holds S[col c16][key base + 16 blk + 4 q + j].
    float x[2][4];
    float mx = neg_inf();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = base + 16 * blk + 4 * q + j;
        float v = sacc[blk][j] * p.scale_log2;
        if (BIAS) {
          const int d = qa - t;
          if ((unsigned)d < (unsigned)p.R) v = __builtin_fmaf(rel_row[d], kLog2e, v);
        }
        if (MASK) {
          if (t < lo_c || t > hi_c) v = neg_inf();
        }
        x[blk][j] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == neg_inf() ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    float pe[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pe[i] = exp2_fast(x[i >> 2][i & 3] - m_use);
      psum += pe[i];
    }
    l_run = l_run * alpha + psum;
    const bf16x8 pf = pack8_bf16(pe);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    wave_lds_sync();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = as_bf16x8(ld16(Vt + (16 * db + c16) * VS + 8 * q));
      oacc[db] = mfma16(a, pf, oacc[db]);
    }
  };

  auto step = [&](DecodeRegs<D> &Rg, int base) {
    const bool interior = base >= in_lo && base + kDecWaveKeys - 1 <= in_hi;
    const bool bias = p.R > 0 && base <= band_hi && base + kDecWaveKeys - 1 >= band_lo;
    if (interior) {
      if (bias) compute(Rg, base, BoolTag<false>{}, BoolTag<true>{});
      else compute(Rg, base, BoolTag<false>{}, BoolTag<false>{});
    } else {
      if (bias) compute(Rg, base, BoolTag<true>{}, BoolTag<true>{});
      else compute(Rg, base, BoolTag<true>{}, BoolTag<false>{});
    }
  };

  // Wave w takes 32-key blocks w, w + 4, w + 8, ... of the split; loads for
  // the next block are in flight while the current one is computed.
  const int nblk = t1 > t0 ? (t1 - t0 + kDecWaveKeys - 1) / kDecWaveKeys : 0;
  const int my_n = nblk > w ? (nblk - w + 3) / 4 : 0;
  DecodeRegs<D> RA, RB;
  if (my_n > 0) issue(RA, t0 + kDecWaveKeys * w);
  for (int it = 0; it < my_n; it += 2) {
    if (it + 1 < my_n) issue(RB, t0 + kDecWaveKeys * (w + 4 * (it + 1)));
    step(RA, t0 + kDecWaveKeys * (w + 4 * it));
    if (it + 1 >= my_n) break;
    if (it + 2 < my_n) issue(RA, t0 + kDecWaveKeys * (w + 4 * (it + 2)));
    step(RB, t0 + kDecWaveKeys * (w + 4 * (it + 1)));
  }

  // Merge the four waves' (m, l, O^T) through LDS.
  float l_col = l_run + __shfl_xor(l_run, 16);
  l_col += __shfl_xor(l_col, 32);
  __syncthreads();
  float *red_o = reinterpret_cast<float *>(smem);  // [4][D][16]
  float *red_m = reinterpret_cast<float *>(smem + (DecodeLds<D>::bytes - DecodeLds<D>::redMLBytes));
  float *red_l = red_m + 4 * kDecCols;
  if (q == 0) {
    red_m[w * kDecCols + c16] = m_run;
    red_l[w * kDecCols + c16] = l_col;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red_o[(w * D + 16 * db + 4 * q + j) * kDecCols + c16] = oacc[db][j];
  }
  __syncthreads();
  constexpr int DPG = D / 16;  // head_dim values per thread in the merge
  const int fc = tid & 15, fg = tid >> 4;
  if (fc >= ncols) return;
  float mw[4], sc[4];
  float M = neg_inf();
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    mw[ww] = red_m[ww * kDecCols + fc];
    M = fmaxf(M, mw[ww]);
  }
  float L = 0.f;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    sc[ww] = mw[ww] == neg_inf() ? 0.f : exp2_fast(mw[ww] - M);
    L += sc[ww] * red_l[ww * kDecCols + fc];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float lse_v = L > 0.f ? (M + log2_fast(L)) * kLn2 : neg_inf();
  float o[DPG];
#pragma unroll
  for (int e = 0; e < DPG; ++e) {
    const int d = fg * DPG + e;
    float acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) acc += sc[ww] * red_o[(ww * D + d) * kDecCols + fc];
    o[e] = acc * inv;
  }
  const int fqi = fc / G;
  const int fhead = g * G + (fc - fqi * G);
  const int ftok = tok0 + fqi;
  if (p.S == 1) {
    uint16_t *op = p.out + ((int64_t)ftok * p.H + fhead) * D + fg * DPG;
    if constexpr (DPG == 8) {
      *reinterpret_cast<u32x4 *>(op) = u32x4{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]),
                                             pack2_bf16(o[4], o[5]), pack2_bf16(o[6], o[7])};
    } else {
      *reinterpret_cast<u32x2 *>(op) = u32x2{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
    }
    if (fg == 0 && p.lse) p.lse[(int64_t)ftok * p.H + fhead] = lse_v;
  } else {
    float *pp = p.part_out + (((int64_t)s * p.num_tokens + ftok) * p.H + fhead) * D + fg * DPG;
#pragma unroll
    for (int e = 0; e < DPG; e += 4) *reinterpret_cast<f32x4 *>(pp + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
    if (fg == 0) p.part_lse[((int64_t)s * p.num_tokens + ftok) * p.H + fhead] = lse_v;
  }
}

template <int D>
constexpr int attn_lds_bytes() {
  return PrefillLds<D>::bytes > DecodeLds<D>::bytes ? PrefillLds<D>::bytes : DecodeLds<D>::bytes;
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[attn_lds_bytes<D>()];
  const int bid = blockIdx.x;
  const int s = bid % p.S;
  const int rest = bid / p.S;
  const int g = rest % p.Hkv;
  const int item = rest / p.Hkv;
  const Item it = resolve_item(p, item);
  if (it.kind == 1) {
    prefill_item<D>(p, it.b, it.tile, g, s, smem);
  } else if (it.kind == 2) {
    decode_item<D>(p, it.b, g, s, smem);
  }
}

// ---------------------------------------------------------------- combine

// One wave per (token, head) row: weights exp(lse_s - LSE) over the splits,
// then a weighted sum of the normalised partials.
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  __shared__ float wts[4][128];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= p.rows) return;
  const float l0 = lane < p.S ? p.part_lse[(int64_t)lane * p.rows + row] : neg_inf();
  const float l1 = lane + 64 < p.S ? p.part_lse[(int64_t)(lane + 64) * p.rows + row] : neg_inf();
  float M = fmaxf(l0, l1);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  uint16_t *op = p.out + (int64_t)row * p.D;
  if (M == neg_inf()) {
    for (int d = lane; d < p.D; d += 64) op[d] = 0;
    if (lane == 0 && p.lse) p.lse[row] = neg_inf();
    return;
  }
  const float e0 = l0 == neg_inf() ? 0.f : exp2_fast((l0 - M) * kLog2e);
  const float e1 = l1 == neg_inf() ? 0.f : exp2_fast((l1 - M) * kLog2e);
  float W = e0 + e1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
  const float invW = 1.f / W;
  wts[w][lane] = e0 * invW;
  wts[w][lane + 64] = e1 * invW;
  wave_lds_sync();
  for (int d = lane; d < p.D; d += 64) {
    float acc = 0.f;
    for (int s = 0; s < p.S; ++s) acc += wts[w][s] * p.part_out[((int64_t)s * p.rows + row) * p.D + d];
    op[d] = __builtin_bit_cast(uint16_t, (__bf16)acc);
  }
  if (lane == 0 && p.lse) p.lse[row] = M + log2_fast(W) * kLn2;
}

}  // namespace

hipError_t launch_attention(const AttnParams &p, int head_dim, int64_t n_items_ub, hipStream_t stream) {
  const int64_t blocks = n_items_ub * p.Hkv * p.S;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (head_dim == 128) {
    hipLaunchKernelGGL(attn_kernel<128>, grid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL(attn_kernel<64>, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.rows + 3) / 4)), block(kThreads);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace rpa
