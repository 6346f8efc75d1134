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
// split); each workgroup finds its item by scanning cu_seqlens_q on the
// device (no host metadata, no device->host copy).  Decode items are
// numbered first, then prefill q-tiles, heaviest tile of each request first.
//   * prefill item: 128 (token, q-head) rows of one kv head.  Four waves,
//     32 rows each.  S^T = K·Q^T and O^T = V^T·P^T on 32x32x16 bf16 MFMA so
//     that each lane owns one query row: softmax statistics stay lane-local
//     except one exchange with the partner lane 32 away.  K and V^T tiles of
//     64 keys are double-buffered in LDS (one barrier per tile); the global
//     loads of tile i+1 and the block-table reads of tile i+2 are in flight
//     while tile i is computed.
//   * decode item (Lq*G <= 16): up to 16 (token, q-head) columns of one kv
//     head; the GQA group shares every K/V row it reads.  The split's page
//     ids are staged in LDS; four waves stream disjoint 32-key blocks from
//     HBM (K straight into 16x16x32 MFMA operands, V through a per-wave LDS
//     transpose), loads of the next block in flight, and merge their
//     softmax states through LDS at the end.
// The key order inside each 16/32-key chunk is permuted so that the softmax
// output already sits in the P^T operand layout; V^T follows the same
// permutation.  The running max is only raised when a row's new maximum
// exceeds it by more than kTau (log2 units), so the O rescale is skipped on
// most tiles; exp2 arguments then stay <= kTau, and the final normalisation
// uses the same running max, so the result is unchanged.
#include <type_traits>

#include <mutex>

#include "rpa_internal.h"

namespace rpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kTau = 8.0f;      // lazy-rescale threshold (log2 units)
constexpr int kPageCache = 512;   // decode: block-table entries staged in LDS

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

// Raw buffer resource over `bytes` bytes at `base` (gfx9 layout, stride 0):
// loads at offsets past the range return zeros without touching memory.
// Both arguments must be wave-uniform; they are passed through readfirstlane
// so that the descriptor is built in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void *ub = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read_b128_asm(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ u32x2 lds_read_b64_asm(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void lgkm_wait_n(u32x2 (&r)[2]) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r[0]), "+v"(r[1]) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_n(u32x4 (&r)[2]) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r[0]), "+v"(r[1]) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_n(u32x4 (&r)[1]) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r[0]) : "n"(N));
}
// Two or four 16-byte LDS writes, complete when the asm ends.
__device__ __forceinline__ void lds_write_b128x2_now(uint32_t a0, uint32_t a1, u32x4 v0, u32x4 v1) {
  asm volatile("ds_write_b128 %0, %2\n\tds_write_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               :
               : "v"(a0), "v"(a1), "v"(v0), "v"(v1)
               : "memory");
}
__device__ __forceinline__ void lds_write_b128x4_now(const uint32_t (&a)[4], const u32x4 (&v)[4]) {
  asm volatile(
      "ds_write_b128 %0, %4\n\tds_write_b128 %1, %5\n\tds_write_b128 %2, %6\n\tds_write_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3])
      : "memory");
}

// E4M3 (OCP) codes to bf16: v_cvt_scalef32_pk_bf16_fp8 turns the two codes
// of one 16-bit half of a dword into a bf16 pair (first code in the low
// half), here with scale 1.  The conversion is exact: an E4M3 value has at
// most four significant bits and an exponent inside bf16's range.  Four
// codes of one dword become two dwords of bf16 pairs in element order.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t x) {
  typedef __bf16 bf16x2_ __attribute__((ext_vector_type(2)));
  const bf16x2_ lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  const bf16x2_ hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t x0, uint32_t x1) {
  const u32x2 lo = e4m3x4_to_bf16(x0), hi = e4m3x4_to_bf16(x1);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}


__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Cross-lane exchanges.  permlane32_swap with both operands = v leaves, in
// every lane, v of lane l%32 in one result and v of lane l%32 + 32 in the
// other; permlane16_swap does the same for lanes l and l ^ 16.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier without the fences of __syncthreads(): those make the
// compiler wait for every outstanding global load (vmcnt(0)) first, which
// would also wait for loads meant to stay in flight across the barrier.
// Callers wait explicitly for what the barrier publishes (the LDS writes of
// direct loads: vmcnt; ds_write: lgkmcnt).  The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_raw() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
template <int I>
struct IntTag {
  static constexpr int value = I;
};
// Calls f(IntTag<I>{}) for I = B .. E-1 (compile-time unrolled).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(IntTag<B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ bool is_decode(int lq, int G) { return lq > 0 && G <= kDecCols && lq * G <= kDecCols; }
__device__ __forceinline__ int prefill_tiles(int lq, int G, int rows) {
  return (lq <= 0 || is_decode(lq, G)) ? 0 : (int)(((int64_t)lq * G + rows - 1) / rows);
}

struct Item {
  int b;     // request
  int tile;  // q-tile within the request (prefill)
  int kind;  // 0 none, 1 prefill, 2 decode
  int kmax;  // longest cache_seqlens in the batch (sets the split chunk)
};

// Maps a linear work-item index to (request, tile).  Items [0, ND) are the
// decode items in request order, items [ND, ND + NP) the prefill q-tiles,
// request by request, the heaviest (last) tile of a request first.  Decode
// items go first so that their streaming overlaps the prefill tiles'
// compute (about 1 % on a mixed batch) instead of running in the tail.
// With at most 64 requests the prefill requests are taken longest first:
// by the key count of their heaviest q-tile (the whole KV length, or the
// window's span), ties in request order; a request's q-tiles stay
// together, so its tiles still read the same K/V tiles at about the same
// time, and the short requests end the grid instead of a long request's
// tiles.  Every wave scans independently (the reads hit cache), so no
// barrier is needed.
__device__ Item resolve_item(const AttnParams &p, int item, bool decode_only, int rows) {
  const int lane = threadIdx.x & 63;
  int kmax = 0, nd = 0;
  for (int c = 0; c < p.batch; c += 64) {
    const int b = c + lane;
    if (b < p.batch) {
      kmax = max(kmax, p.cache_seqlens[b]);
      const int lqb = p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
      nd += is_decode(lqb, p.G) ? 1 : 0;
    }
  }
  kmax = wave_max_i(kmax);
  // Wave-uniform: readfirstlane lets the compiler see it, so that the
  // branch on it stays scalar.
  nd = __builtin_amdgcn_readfirstlane(wave_sum_i(nd));
  const bool pre = item >= nd;
  const int target = pre ? item - nd : item;
  if (pre && p.batch <= 64) {
    // Rank key of request lane: its heaviest tile's key count, then the
    // request index (lower first), in one integer; -1 without prefill tiles.
    const int b = lane;
    int n = 0, key = -1;
    if (b < p.batch) {
      const int lq = p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
      n = prefill_tiles(lq, p.G, rows);
      int span = p.cache_seqlens[b];
      if (p.left >= 0) span = min(span, p.left + rows / p.G);
      if (n > 0) key = (min(max(span, 0), 1 << 24) << 6) | (63 - b);
    }
    // Tiles of the requests ranked before this one.
    int excl = 0;
    for (int i = 0; i < p.batch; ++i) {
      const int ki = __builtin_amdgcn_readlane(key, i);
      const int ni = __builtin_amdgcn_readlane(n, i);
      excl += ki > key ? ni : 0;
    }
    const unsigned long long mask = __ballot(n > 0 && target >= excl && target < excl + n);
    if (mask) {
      const int src = __ffsll((long long)mask) - 1;
      const int k = target - __shfl(excl, src);
      return Item{__builtin_amdgcn_readfirstlane(src), __builtin_amdgcn_readfirstlane(__shfl(n, src) - 1 - k), 1,
                  __builtin_amdgcn_readfirstlane(kmax)};
    }
    return Item{-1, 0, 0, kmax};
  }
  int base = 0;
  for (int c = 0; c < p.batch; c += 64) {
    const int b = c + lane;
    int n = 0;
    if (b < p.batch) {
      const int lq = p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
      n = pre ? prefill_tiles(lq, p.G, rows) : (is_decode(lq, p.G) ? 1 : 0);
    }
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int excl = incl - n;
    const unsigned long long mask = __ballot(target >= base + excl && target < base + incl);
    if (mask) {
      const int src = __ffsll((long long)mask) - 1;
      const int e = __shfl(excl, src);
      const int nb = __shfl(n, src);
      const int k = target - base - e;
      // Wave-uniform by construction; readfirstlane lets the compiler keep
      // everything derived from the item in scalar registers.
      return Item{__builtin_amdgcn_readfirstlane(c + src), __builtin_amdgcn_readfirstlane(pre ? nb - 1 - k : 0),
                  pre ? 1 : 2, __builtin_amdgcn_readfirstlane(kmax)};
    }
    base += __shfl(incl, 63);
  }
  return Item{-1, 0, 0, kmax};
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

// Split s of S: the range starts at lo aligned down to 16 and is cut into
// chunks of ceil(kmax / S) keys rounded up to `align`, the same chunk size
// for every item of the batch (so split workgroups carry equal work); an
// item shorter than kmax leaves its last splits empty.
__device__ __forceinline__ Range split_range(Range r, int kmax, int S, int s, int align) {
  const int lo_a = r.lo & ~15;
  if (r.hi <= lo_a) return Range{0, 0};
  int chunk = (kmax + S - 1) / S;
  chunk = (chunk + align - 1) / align * align;
  const int t0 = lo_a + s * chunk;
  return Range{t0, min(r.hi, t0 + chunk)};
}

// ---------------------------------------------------------------- prefill

template <int D, bool KV8 = false>
struct PrefillLds {
  static constexpr int UNITS = D / 8;                 // 16-byte units per key row
  static constexpr int ROWB = D * 2;                  // bytes per key row (unpadded)
  static constexpr int tileBytes = kTileKeys * ROWB;  // 16 KB for head_dim 128
  static constexpr int NK = 2, NV = 2;                // double-buffered K and V tiles
  static constexpr int kOff(int i) { return i * tileBytes; }
  static constexpr int vOff(int i) { return (NK + i) * tileBytes; }  // bf16 caches
  // E4M3 caches: the V tiles stay raw (rows of D codes, read transposed and
  // decoded in registers), and the raw K rows of a tile land in one of two
  // areas, from which each wave decodes its own rows into a bf16 K slot.
  static constexpr int rawBytes = kTileKeys * D;
  static constexpr int v8Off(int i) { return NK * tileBytes + i * rawBytes; }
  static constexpr int landK(int i) { return NK * tileBytes + (2 + i) * rawBytes; }
  static constexpr int bytes = KV8 ? NK * tileBytes + 4 * rawBytes : (NK + NV) * tileBytes;
};

// K and V tiles are stored row-major (one key per row) with the 16-byte
// units of each row XOR-swizzled, instead of padded, so that they can be
// filled by direct buffer->LDS loads.  K: unit u of row r sits at
// u ^ swz_k(r), which spreads the 16 consecutive rows one MFMA operand read
// touches over all banks.  V: unit u sits at u ^ swz_v(r), which does the
// same for the transposing reads of four consecutive keys.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return (4 * (r & 3)) & (D / 8 - 1); }
// Raw E4M3 V rows (D codes, D / 16 units): unit u of row r sits at
// u ^ swz_v8(r).  An 8-bit transposing read takes, per half-wave, the same
// two units of the eight rows {0..3, 8..11} + 4 hf (+ 16 c4); the swizzle
// moves them onto distinct banks.
template <int D>
__device__ __forceinline__ int swz_v8(int r) {
  return D == 128 ? ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2)) : (((r >> 3) & 1) << 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// ds_read_b64_tr_b16 (lds_read_tr_asm below): within each 16-lane group,
// lane j receives 16-bit element j%4 of the 8-byte rows addressed by lanes
// j/4, 4 + j/4, 8 + j/4 and 12 + j/4 of the group.

// Key offset, within a tile, of accumulator element (kb2, j) of a lane with
// hf = 0 (lanes with hf = 1 hold keys 4 further on).  K and V rows are staged
// with the keys of every group of four in reverse order (row r holds key
// rev4(r)), so element j%4 = m of a group holds key 3 - m of it.
__device__ __forceinline__ constexpr int rev4(int r) { return (r & ~3) + 3 - (r & 3); }
__device__ __forceinline__ constexpr int key_of(int kb2, int j) { return 32 * kb2 + 8 * (j >> 2) + 3 - (j & 3); }

// Raw bias values of a 64-key tile for this lane's row, in the S^T
// accumulator layout: rel_row[qa - t] for the lane's keys t.  Band
// membership is applied later by tile_init, so nothing waits on these loads
// here.
//
// Fast form: the lane's keys come in eight groups of four consecutive keys,
// i.e. four consecutive logits, fetched by one 16-byte load each through a
// buffer resource over the tile's rel_logits rows plus a margin of 4 values
// on either side.  A group that runs past its row's band picks up values of
// the neighbouring row (or zeros past the resource) that the band select
// discards.  lane_base is the byte offset of this lane's logit at distance
// qa - 4 hf - 3, the lowest distance of its first group when kb = 0; offsets
// below the resource wrap and read as zeros.  With the reversed key order of
// a group, memory order is element order, so the loads land in place and
// nothing waits on them here.
__device__ __forceinline__ void tile_bias_load4(f32x16 *sacc, __amdgpu_buffer_rsrc_t rs, uint32_t lane_base, int kb) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const uint32_t voff = lane_base - 4u * (uint32_t)(kb + 32 * kb2 + 8 * g4);
      const u32x4 v = bload16(rs, voff);
#pragma unroll
      for (int m = 0; m < 4; ++m) sacc[kb2][4 * g4 + m] = __uint_as_float(v[m]);
    }
  }
}

// Slow form, for tiles whose rows sit at either end of rel_logits (where the
// margin of the fast form does not exist): clamped per-value loads.
__device__ __forceinline__ void tile_bias_load(f32x16 *sacc, int kb, int qa, const float *rel_row, int R, int hf) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int d = qa - (kb + key_of(kb2, j) + 4 * hf);
      sacc[kb2][j] = rel_row[min(max(d, 0), R - 1)];
    }
  }
}
// bf16 rel_logits, fast form: the four logits of a group (8 bytes at a
// 2-byte boundary, lowest distance first) come from one 12-byte load of the
// three dwords around them, through a buffer resource over the tile's rows
// with an 8-value margin on either side; el_base is the element offset of
// this lane's logit at distance qa - 4 hf - 3 (the lowest distance of its
// first group when kb = 0).  The three raw dwords land in the group's first
// three elements; tile_bf16_widen4 shifts the pairs into place and widens.
__device__ __forceinline__ void tile_bias_load4_bf16(f32x16 *sacc, __amdgpu_buffer_rsrc_t rs, int el_base, int kb) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = el_base - (kb + 32 * kb2 + 8 * g4);
      // The dword holding element d; a negative d wraps far past the
      // resource, so it reads as zeros.
      const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs, 4 * (d >> 1), 0, 0);
#pragma unroll
      for (int m = 0; m < 3; ++m) sacc[kb2][4 * g4 + m] = __uint_as_float(v[m]);
    }
  }
}
// Per-value form of the above for tiles whose rows sit at either end of the
// array (no margin there): each logit by its own 2-byte load through the
// same resource, clipped to the array (a load outside it reads zero; every
// value of the band lies inside it).  The loads are awaited here and the
// pairs packed into the layout of the fast form with its groups starting at
// an even element (sh = 0 for tile_bf16_widen4); these tiles are rare.
__device__ __forceinline__ void tile_bias_load1_bf16(f32x16 *sacc, __amdgpu_buffer_rsrc_t rs, int el_base, int kb) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int off = 2 * (el_base - (kb + 32 * kb2 + 8 * g4));
      uint32_t e[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) e[m] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off + 2 * m, 0, 0);
      sacc[kb2][4 * g4] = __uint_as_float(e[0] | (e[1] << 16));
      sacc[kb2][4 * g4 + 1] = __uint_as_float(e[2] | (e[3] << 16));
    }
  }
}
// sh: 16 when the groups of the tile start at an odd element (the same for
// every group of a tile), else 0.
__device__ __forceinline__ void tile_bf16_widen4(f32x16 *sacc, uint32_t sh) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const uint32_t w0 = __float_as_uint(sacc[kb2][4 * g4]), w1 = __float_as_uint(sacc[kb2][4 * g4 + 1]);
      const uint32_t w2 = __float_as_uint(sacc[kb2][4 * g4 + 2]);
      const uint32_t x0 = __builtin_amdgcn_alignbit(w1, w0, sh), x1 = __builtin_amdgcn_alignbit(w2, w1, sh);
      float e0 = __uint_as_float(x0 << 16), e1 = __uint_as_float(x0 & 0xFFFF0000u);
      float e2 = __uint_as_float(x1 << 16), e3 = __uint_as_float(x1 & 0xFFFF0000u);
      // One group at a time: otherwise the compiler forms every group's
      // shifted pairs first and holds them all.
      asm volatile("" : "+v"(e0), "+v"(e1), "+v"(e2), "+v"(e3));
      sacc[kb2][4 * g4] = e0;
      sacc[kb2][4 * g4 + 1] = e1;
      sacc[kb2][4 * g4 + 2] = e2;
      sacc[kb2][4 * g4 + 3] = e3;
    }
  }
}


// Per-lane bounds of one tile, relative to the lane's first key kb + 4 hf:
// element keys k in [vis_lo, vis_hi] are visible, keys in [band_lo, band_hi]
// get the bias.
struct TileBounds {
  int vis_lo, vis_hi, band_lo, band_hi;
};

// Initial value of the score accumulator of a general tile (a mask edge or
// the bias band), so that the MFMA chain yields s + bias/scale directly:
// bias/scale inside the band (sacc holds the raw loaded values when BAND),
// 0 outside it, and masked (an infinity that the scaled exp2 sends to 0)
// where the row may not see the key.
// Number of a lane's 32 accumulator elements, counted in the order of their
// key offsets, whose offset (without the 4 hf shift) is below x.  Element
// (kb2, j) holds offset 32 kb2 + 8 (j/4) + 3 - j%4, so sorted by offset the
// elements run (kb2, 4 g + 3), (kb2, 4 g + 2), ...
__device__ __forceinline__ int elems_below(int x) {
  x = min(max(x, 0), 64);
  return 16 * (x >> 5) + 4 * ((x >> 3) & 3) + min(x & 7, 4);
}
// Bitmap over that order: bit i set iff the i-th element's offset is in [lo, hi].
__device__ __forceinline__ uint32_t range_bits(int lo, int hi) {
  const int a = elems_below(lo), b = elems_below(min(hi, 64) + 1);
  return b > a ? (uint32_t)((1ull << b) - (1ull << a)) : 0u;
}
// Bit position, in that order, of element (kb2, j).
__device__ __forceinline__ constexpr int order_of(int kb2, int j) { return 16 * kb2 + (j & ~3) + 3 - (j & 3); }
// All-ones if bit pos of bits is set, else 0 (v_bfe_i32), and the bitwise
// select (m & a) | (~m & b) (v_bfi_b32); as asm so they stay single
// instructions instead of per-element compares.
__device__ __forceinline__ uint32_t bit_mask(uint32_t bits, int pos) {
  uint32_t r;
  asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(r) : "v"(bits), "i"(pos));
  return r;
}
__device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

// Accumulator start of a general tile, by what the tile needs:
//   kInitEdge: no bias; 0 where visible, masked elsewhere;
//   kInitBand: bias/scale where in the band and visible, 0 where visible
//              only, masked elsewhere;
//   kInitFull: every key of the tile visible to, and in the band of, every
//              row: bias/scale.
// sacc holds the raw loaded bias values for the band modes.  (Tiles that
// need only one of the two masks measured no faster with a form of their
// own, which costs registers.)
enum { kInitEdge, kInitBand, kInitFull };
// Key offset (without the 4 hf shift) of accumulator element (kb2, j).
__device__ __forceinline__ constexpr int offset_of(int kb2, int j) { return 32 * kb2 + 8 * (j >> 2) + 3 - (j & 3); }
template <int MODE>
__device__ __forceinline__ void tile_init(f32x16 *sacc, TileBounds tb, float inv_scale, float masked) {
  if constexpr (MODE == kInitFull) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) sacc[kb2] *= inv_scale;
    return;
  }
  constexpr bool USE_VIS = true;
  constexpr bool USE_BAND = MODE == kInitBand;
  const uint32_t vis = USE_VIS ? range_bits(tb.vis_lo, tb.vis_hi) : 0u;
  const uint32_t band = USE_BAND ? range_bits(tb.band_lo, tb.band_hi) : 0u;
  const uint32_t mbits = __float_as_uint(masked);
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int pos = order_of(kb2, j);
      uint32_t v = 0u;
      if constexpr (MODE != kInitEdge) v = __float_as_uint(sacc[kb2][j] * inv_scale);
      if constexpr (USE_BAND) v &= bit_mask(band, pos);
      if constexpr (USE_VIS) v = bit_select(bit_mask(vis, pos), v, mbits);
      sacc[kb2][j] = __uint_as_float(v);
    }
  }
}

// ALiBi inside a tile: slope * (t - qa) = al_s * offset_of(kb2, j), the
// same for every tile, plus al_s * (kb + 4 hf - qa), a per-row constant of
// the tile (al_s: the slope in raw score units).  The first part is added
// to the scores once the QK is done (an fma with a constant per element, so
// that nothing per element is held across the tile loop), the second joins
// the exp's subtrahend and the tile's row max.
__device__ __forceinline__ float alibi_ramp_add(float al_s, int kb2, int j, float s) {
  return __builtin_fmaf(al_s, (float)offset_of(kb2, j), s);
}
__device__ __forceinline__ void tile_alibi_ramp(f32x16 *sacc, float al_s) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[kb2][j] = alibi_ramp_add(al_s, kb2, j, sacc[kb2][j]);
}

// Row max of a tile in raw score units (the scale is positive).
__device__ __forceinline__ float tile_rowmax(const f32x16 *sacc) {
  float mx = neg_inf();
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb2][j]);
  return mx;
}

// S^T = K·Q^T (+ the initial sacc when INIT) for a 64-key tile: lane
// (l32, hf) gets S[row l32][key 32 kb2 + 8 (j/4) + 4 hf + j%4] in
// sacc[kb2][j].  The two 32-key halves are independent accumulation chains,
// issued alternately.  Unit 2 ks + hf of row r sits at (2 ks + hf) ^ sw(r),
// i.e. at byte offset off0 ^ 32 ks.
template <int D, bool INIT>
__device__ __forceinline__ void qk_mfma(const char *Kb, const bf16x8 *qf, f32x16 *sacc, int l32, int hf) {
  constexpr int KSTEPS = D / 16;
  constexpr int ROWB = PrefillLds<D>::ROWB;
  const char *row = Kb + l32 * ROWB;  // row l32 + 32 shares the swizzle of row l32
  const int off0 = (hf ^ swz_k<D>(l32)) << 4;
  if constexpr (!INIT) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
  }
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int off = off0 ^ (ks << 5);
    const u32x4 a0 = *reinterpret_cast<const u32x4 *>(row + off);
    const u32x4 a1 = *reinterpret_cast<const u32x4 *>(row + 32 * ROWB + off);
    sacc[0] = mfma32(as_bf16x8(a0), qf[ks], sacc[0]);
    sacc[1] = mfma32(as_bf16x8(a1), qf[ks], sacc[1]);
  }
}

// The two overlapped phases of a pipeline iteration.  Each is written out
// in the order it should issue, in groups of one MFMA (32 cycles on the
// matrix pipe), the LDS read of the operand needed a few MFMAs later, and a
// slice of the other phase's VALU work; sched_barrier keeps the groups in
// that order, so the wave issues VALU instructions while its MFMAs run.
// Values that are only consumed after the phase (partial sums, partial
// maxima, zeroed registers) are pinned inside their group: otherwise the
// compiler sinks their arithmetic to the point of use, after the MFMAs.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

// Phase A: S^T(next) = K·Q^T on the MFMA pipe, starting from the initial
// sacc, or from zero when zc (a plain tile: the first MFMA of each chain
// takes a zero accumulator), and P = exp2(c*s - m) of the current tile as
// bf16 PV operands (pb[c] covers keys 16c .. 16c+15 in V^T slot order);
// returns this lane's part of the row sum (of the fp32 P).
template <int D>
__device__ __forceinline__ float phase_a(const char *Kb, const bf16x8 *qf, f32x16 *sn, const f32x16 *sc,
                                         float c, float m_use, bf16x8 *pb, int l32, int hf, bool zc) {
  constexpr int KSTEPS = D / 16;
  constexpr int NM = 2 * KSTEPS;     // MFMAs
  constexpr int EPM = 32 / NM;       // exp elements per MFMA group
  constexpr int AHEAD = 3;           // operand reads in flight
  constexpr int ROWB = PrefillLds<D>::ROWB;
  const char *row = Kb + l32 * ROWB;  // row l32 + 32 shares the swizzle of row l32
  const int off0 = (hf ^ swz_k<D>(l32)) << 4;
  u32x4 a[NM];
  auto rd = [&](int i) __attribute__((always_inline)) {
    a[i] = *reinterpret_cast<const u32x4 *>(row + (i & 1) * 32 * ROWB + (off0 ^ ((i >> 1) << 5)));
  };
  // The exp work is skewed over the groups so that no instruction waits on
  // the one just before it: group i scales the elements of group i+2, takes
  // exp2 of those of group i+1 and sums and packs those of group i (two
  // partial sums).
  float pe[32];
  float psum[2] = {0.f, 0.f};
  auto fma_g = [&](int gi) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < EPM; ++e) {
      const int x = gi * EPM + e;
      pe[x] = __builtin_fmaf(sc[x >> 4][x & 15], c, -m_use);
    }
  };
  auto exp_g = [&](int gi) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < EPM; ++e) pe[gi * EPM + e] = exp2_fast(pe[gi * EPM + e]);
  };
  auto sum_g = [&](int gi) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < EPM; ++e) psum[e & 1] += pe[gi * EPM + e];
    pin(psum[0]);
    if (EPM > 1) pin(psum[1]);
    if (((gi + 1) * EPM) % 8 == 0) {
      const int c4 = (gi + 1) * EPM / 8 - 1;
      pb[c4] = pack8_bf16(&pe[8 * c4]);
    }
  };
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) rd(i);
  fma_g(0);
  fma_g(1);
  exp_g(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i < 2) {
      if (zc) sn[i & 1] = mfma32(as_bf16x8(a[i]), qf[i >> 1], f32x16{});
      else sn[i & 1] = mfma32(as_bf16x8(a[i]), qf[i >> 1], sn[i & 1]);
    } else {
      sn[i & 1] = mfma32(as_bf16x8(a[i]), qf[i >> 1], sn[i & 1]);
    }
    if (i + AHEAD < NM) rd(i + AHEAD);
    if (i + 2 < NM) fma_g(i + 2);
    if (i + 1 < NM) exp_g(i + 1);
    sum_g(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  return psum[0] + psum[1];
}

// Phase B: O^T += V^T·P^T on the MFMA pipe (the V^T operand of row
// d = lane%32 and eight slot-order keys comes from two transposing reads of
// the row-major V tile), and the row max (raw units) of the next tile on the
// VALU, after adding the ALiBi ramp of slope al_s to its scores when ALIBI.
//
// The transposing reads are issued as inline asm: the compiler cannot tell
// them apart from the direct loads in flight into the other V slot and would
// wait for those (vmcnt(0)) before the first read.  Their completion is
// awaited explicitly: each wait names the operand it guards, and LDS reads
// complete in order, so lgkmcnt(n) with n = reads issued after the operand's
// two is sufficient (other LGKM traffic only makes it stricter).
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr_asm(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void lgkm_wait_for(u32x4 &a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_for(u32x2 &a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
// ds_read_b64_tr_b8: within each 16-lane group, lane j receives byte j % 8
// of the 8-byte rows addressed by lanes j/8, j/8 + 2, ..., j/8 + 14 of the
// group, in that order.
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr8_asm(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128_off(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
  return v;
}
// One 16-byte LDS write, issued and not awaited (its source registers are
// read at issue).
template <int OFF>
__device__ __forceinline__ void lds_write_b128_off(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "n"(OFF) : "memory");
}
// s_waitcnt operand that waits until at most n vector-memory loads are in flight.
constexpr int vmcnt_enc(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// Cache policy of a buffer load (its aux operand): nt, for data read once.
// The balanced decodes' K/V streams take it; a streaming read probe reads
// HBM about 10 % faster with it than with the default policy.
constexpr int kNonTemporal = 2;

template <int D, int VOFF, bool ALIBI, bool LANE_PIN>
__device__ __forceinline__ float phase_b(const char *smem, const bf16x8 *pb, f32x16 *oacc, int lane, f32x16 *sn,
                                         float al_s) {
  constexpr int DB = D / 32;
  constexpr int NM = 4 * DB;
  constexpr int EPM = 32 / NM;
  constexpr int AHEAD = 3;
  constexpr int ROWB = PrefillLds<D>::ROWB;
  // LANE_PIN: the addresses are formed from an opaque copy of the lane id at
  // each call, so that the compiler does not hoist them out of the tile loop
  // and hold DB registers there (worth it only where registers are short: the
  // E4M3 kernel with ALiBi spills without it, while the others run about 1 %
  // slower with it).
  int ln = lane;
  if constexpr (LANE_PIN) asm volatile("" : "+v"(ln));
  const int grp = ln >> 4, h = grp >> 1, dh = grp & 1;
  const int k = (ln >> 2) & 3, q = ln & 3;
  const int key_lo = 4 * h + k;           // + 16 c4 (+ 8 for slots 4..7)
  const int sw = swz_v<D>(key_lo);       // same for key_lo + 16 c4 + 8
  // Per-lane address of head_dim block db; the slot, the 16-key chunk c4 and
  // the +8 keys of the second read are immediate offsets.
  uint32_t base[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int d0 = 32 * db + 16 * dh + 4 * q;
    base[db] = (uint32_t)(uintptr_t)smem + key_lo * ROWB + ((((d0 >> 3) ^ sw) << 4) + ((d0 & 7) << 1));
  }
  u32x4 a[NM];
  auto rd = [&](auto i_tag) __attribute__((always_inline)) {
    constexpr int i = decltype(i_tag)::value;
    constexpr int c4 = i / DB, db = i % DB;
    const u32x2 lo = lds_read_tr_asm<VOFF + 16 * c4 * ROWB>(base[db]);
    const u32x2 hi = lds_read_tr_asm<VOFF + (16 * c4 + 8) * ROWB>(base[db]);
    a[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // Four partial maxima keep the max chain from serialising the groups.
  float mx[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
  static_for<0, AHEAD>([&](auto i_tag) __attribute__((always_inline)) { rd(i_tag); });
  static_for<0, NM>([&](auto i_tag) __attribute__((always_inline)) {
    constexpr int i = decltype(i_tag)::value;
    constexpr int newer = 2 * (NM - 1 - i < AHEAD - 1 ? NM - 1 - i : AHEAD - 1);
    lgkm_wait_for<newer>(a[i]);
    oacc[i % DB] = mfma32(as_bf16x8(a[i]), pb[i / DB], oacc[i % DB]);
    if constexpr (i + AHEAD < NM) rd(IntTag<i + AHEAD>{});
#pragma unroll
    for (int e = 0; e < EPM; ++e) {
      const int x = i * EPM + e;
      if constexpr (ALIBI) sn[x >> 4][x & 15] = alibi_ramp_add(al_s, x >> 4, x & 15, sn[x >> 4][x & 15]);
      mx[i & 3] = fmaxf(mx[i & 3], sn[x >> 4][x & 15]);
    }
    pin(mx[i & 3]);
    __builtin_amdgcn_sched_barrier(0);
  });
  return fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
}

// Phase B with E4M3 caches.  The V tile stays raw in LDS: the V^T operand
// of row d and eight slot-order keys is one 8-bit transposing read (lanes of
// a 16-lane group address the rows 4 hf + {0..3, 8..11} of the 16-key chunk,
// the lane pairs the two 8-byte halves of one 16-code unit), decoded in
// registers.  Beside the PV MFMAs and the row max, the wave decodes its own
// 16 raw K rows of tile j+2, which landed an iteration earlier, into K slot
// KOFF: after kwait (how many vector-memory loads issued after them may stay
// in flight: this iteration's V and K direct loads, plus 0, 8 or 32 bias loads),
// their reads go out before the first V read, and one decoded 16-byte unit is
// written per group from group 1 on.  LDS reads and writes complete in
// order, so each operand's lgkmcnt counts the LDS operations issued after it.
template <int D, int V8OFF, int LANDOFF, int KOFF, bool ALIBI, bool LANE_PIN>
__device__ __forceinline__ float phase_b8(const char *smem, const bf16x8 *pb, f32x16 *oacc, int lane, f32x16 *sn,
                                          float al_s, int kwait, uint32_t kraw, uint32_t krow, uint32_t kuk) {
  constexpr int DB = D / 32;
  constexpr int NM = 4 * DB;
  constexpr int EPM = 32 / NM;
  constexpr int AHEAD = 3;
  constexpr int U8 = D / 16, RPI8 = 64 / U8, NI8 = 16 / RPI8;
  constexpr int NKW = 2 * NI8;  // decoded K units per lane
  constexpr int ROWB = PrefillLds<D>::ROWB;
  static_assert(NKW + 1 <= NM, "K writes fit the groups");
  int ln = lane;
  if constexpr (LANE_PIN) asm volatile("" : "+v"(ln));
  const int grp = ln >> 4, i16 = ln & 15, hfl = ln >> 5;
  // Slot row of this lane's address inside each 16-key chunk; its swizzle
  // does not depend on the chunk.
  const int r = 4 * hfl + ((i16 >> 1) & 3) + 8 * (i16 >> 3);
  const int f2 = swz_v8<D>(r) >> 1;
  uint32_t base[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    base[db] = (uint32_t)(uintptr_t)smem + (uint32_t)(r * D + ((2 * (db ^ f2) + (grp & 1)) << 4) + 8 * (i16 & 1));
  u32x2 a[NM];
  auto rd = [&](auto i_tag) __attribute__((always_inline)) {
    constexpr int i = decltype(i_tag)::value;
    constexpr int c4 = i / DB, db = i % DB;
    a[i] = lds_read_tr8_asm<V8OFF + 16 * c4 * D>(base[db]);
  };
  if (kwait == 0) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * NI8));
  else if (kwait == 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * NI8 + 8));
  else __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * NI8 + 32));
  u32x4 kr[NI8];
  static_for<0, NI8>([&](auto n_tag) __attribute__((always_inline)) {
    constexpr int n = decltype(n_tag)::value;
    kr[n] = lds_read_b128_off<LANDOFF + RPI8 * n * D>(kraw);
  });
  float mx[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
  static_for<0, AHEAD>([&](auto i_tag) __attribute__((always_inline)) { rd(i_tag); });
  static_for<0, NM>([&](auto i_tag) __attribute__((always_inline)) {
    constexpr int i = decltype(i_tag)::value;
    // LDS operations issued after V read i: the V reads of operands i+1 ..
    // (at most AHEAD - 1 of them) and the K writes of groups m in
    // [max(1, i - AHEAD), i - 1] (group m writes after its V read m + AHEAD).
    constexpr int vnew = NM - 1 - i < AHEAD - 1 ? NM - 1 - i : AHEAD - 1;
    constexpr int mlo = i - AHEAD > 1 ? i - AHEAD : 1;
    constexpr int mhi = i - 1 < NKW ? i - 1 : NKW;
    constexpr int knew = mhi >= mlo ? mhi - mlo + 1 : 0;
    lgkm_wait_for<vnew + knew>(a[i]);
    const u32x4 v = e4m3x8_to_bf16(a[i][0], a[i][1]);
    oacc[i % DB] = mfma32(as_bf16x8(v), pb[i / DB], oacc[i % DB]);
    if constexpr (i + AHEAD < NM) rd(IntTag<i + AHEAD>{});
    if constexpr (i >= 1 && i <= NKW) {
      constexpr int m = i - 1, n = m >> 1, e = m & 1;
      if constexpr (m == 0) {
        // The K reads are older than every V read, and V read 0 has landed.
#pragma unroll
        for (int nn = 0; nn < NI8; ++nn) asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kr[nn]) : "n"(AHEAD + 1));
      }
      const uint32_t flip = (uint32_t)((((D == 128) ? 8 * n : 0) ^ e) << 4);
      lds_write_b128_off<KOFF + RPI8 * n * ROWB>(krow + (kuk ^ flip),
                                                  e4m3x8_to_bf16(kr[n][2 * e], kr[n][2 * e + 1]));
    }
#pragma unroll
    for (int e = 0; e < EPM; ++e) {
      const int x = i * EPM + e;
      if constexpr (ALIBI) sn[x >> 4][x & 15] = alibi_ramp_add(al_s, x >> 4, x & 15, sn[x >> 4][x & 15]);
      mx[i & 3] = fmaxf(mx[i & 3], sn[x >> 4][x & 15]);
    }
    pin(mx[i & 3]);
    __builtin_amdgcn_sched_barrier(0);
  });
  // The decoded K rows are complete before the barrier that publishes them.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  return fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
}

// Prefill variants (compile-time, so that calls without them run the plain
// kernel): bit 0 ALiBi slopes, bit 1 bf16 rel_logits.
constexpr int kFeatAlibi = 1, kFeatRelBf16 = 2;

template <int D, bool KV8, int FEAT>
__device__ void prefill_item(const AttnParams &p, const Item &it, int g, int s, char *smem) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int ROWS = kTileRows;
  using L = PrefillLds<D, KV8>;

  const int b = it.b;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  // Per-request scalars (uniform: kept in SGPRs so the range arithmetic runs
  // on the scalar unit).
  const int tok0 = __builtin_amdgcn_readfirstlane(p.cu_seqlens_q[b]);
  const int lq = __builtin_amdgcn_readfirstlane(p.cu_seqlens_q[b + 1]) - tok0;
  const int lk = __builtin_amdgcn_readfirstlane(p.cache_seqlens[b]);
  const int G = p.G;
  const int nrows = lq * G;
  const int row0 = it.tile * ROWS;
  const int row_last = min(row0 + ROWS, nrows) - 1;
  int r = row0 + 32 * w + l32;
  const bool row_valid = r <= row_last;
  if (!row_valid) r = row_last;  // idle lanes shadow the last row; never stored
  const int qi = r / G;
  const int head = g * G + (r - qi * G);
  const int tok = tok0 + qi;
  const int qa = qi + lk - lq;
  const int qa_min = row0 / G + lk - lq;
  const int qa_max = row_last / G + lk - lq;

  const Range sr = split_range(visible_range(p, lk, qa_min, qa_max), it.kmax, p.S, s, kTileKeys);
  const int t0 = __builtin_amdgcn_readfirstlane(sr.lo), t1 = __builtin_amdgcn_readfirstlane(sr.hi);
  const int kend = min(lk, t1);  // keys at or past this are neither loaded nor visible
  // This lane's visible keys inside the split: [lo_r, hi_r].
  int lo_r = t0, hi_r = kend - 1;
  if (p.left >= 0) lo_r = max(lo_r, qa - p.left);
  if (p.causal) hi_r = min(hi_r, qa);
  if (p.right >= 0) hi_r = min(hi_r, qa + p.right);
  // Keys in [in_lo, in_hi] are visible to every row of the tile.
  int in_lo = t0, in_hi = kend - 1;
  if (p.left >= 0) in_lo = max(in_lo, qa_max - p.left);
  if (p.causal) in_hi = min(in_hi, qa_min);
  if (p.right >= 0) in_hi = min(in_hi, qa_min + p.right);
  in_lo = __builtin_amdgcn_readfirstlane(in_lo);
  in_hi = __builtin_amdgcn_readfirstlane(in_hi);
  const int band_lo = __builtin_amdgcn_readfirstlane(qa_min - p.R + 1);
  const int band_hi = __builtin_amdgcn_readfirstlane(qa_max);
  // Fast bias loads: resource over rel_logits rows first .. last of this
  // tile (row index tok * H + head) with a 4-value margin on either side.
  const int64_t first_row = (int64_t)(tok0 + row0 / G) * p.H + g * G + row0 % G;
  const int64_t last_row = (int64_t)(tok0 + row_last / G) * p.H + g * G + row_last % G;
  constexpr bool rel_bf16 = (FEAT & kFeatRelBf16) != 0;
  // bf16 rel_logits: the same with an 8-value margin (a group's 12-byte
  // load starts up to one value below it and ends up to two above it); where
  // the margin runs past either end of the array, the resource is clipped to
  // the array and each value is loaded on its own (a 12-byte load that
  // straddles an end would lose the values inside).  The host refuses calls
  // whose tiles could span 2 GiB of bf16 rel_logits.
  const int64_t bmargin = rel_bf16 ? 8 : 4, ebytes = rel_bf16 ? 2 : 4;
  const int64_t total_e = (int64_t)p.num_tokens * p.H * p.R;
  int64_t bias_lo_e = first_row * p.R - bmargin, bias_hi_e = (last_row + 1) * p.R + bmargin;
  // bf16: an even start keeps the resource base on a dword (the array starts
  // on one), so that the dword loads see the pairs of the array.
  if constexpr (rel_bf16) bias_lo_e &= ~(int64_t)1;
  const bool bias_in = bias_lo_e >= 0 && bias_hi_e <= total_e;
  if constexpr (rel_bf16) {
    bias_lo_e = max(bias_lo_e, (int64_t)0);
    bias_hi_e = min(bias_hi_e, total_e);
  }
  const bool bias_fast = p.R > 0 && bias_in && (bias_hi_e - bias_lo_e) * ebytes < ((int64_t)1 << 31);
  // Bias loads a band tile leaves in flight until the end of its iteration:
  // 0 none (the bf16 per-value form waits for its own), 1: 8 per lane (the
  // fast forms), 2: 32 (the fp32 per-value form).
  const int band_wait = bias_fast ? 1 : rel_bf16 ? 0 : 2;
  __amdgpu_buffer_rsrc_t bias_rs = make_rsrc(p.rel_logits, 0);
  uint32_t bias_lane_base = 0;
  int bias_el_base = 0;
  if (bias_fast || (rel_bf16 && p.R > 0 && (bias_hi_e - bias_lo_e) * ebytes < ((int64_t)1 << 31))) {
    bias_rs = make_rsrc(reinterpret_cast<const char *>(p.rel_logits) + bias_lo_e * ebytes,
                        (uint32_t)((bias_hi_e - bias_lo_e) * ebytes));
    const int64_t row_rel = ((int64_t)tok * p.H + head) * p.R - bias_lo_e;
    bias_lane_base = (uint32_t)(4 * (row_rel + qa - 4 * hf - 3));
    bias_el_base = (int)(row_rel + qa - 4 * hf - 3);
  }
  // The bias enters the score accumulator as bias/scale, and the scale is
  // made positive: a negative scale negates Q instead (exact in bf16), and a
  // scale below 2^-100 in magnitude is treated as 0 (its q·k term then
  // changes no fp32 logit), which zeroes Q and leaves the bias alone.
  const bool zero_scale = fabsf(p.scale) < 0x1p-100f;
  const bool neg_scale = !zero_scale && p.scale < 0.f;
  const float c = zero_scale ? kLog2e : fabsf(p.scale_log2);
  const float inv_scale = zero_scale ? 1.f : 1.f / fabsf(p.scale);
  const float masked = neg_inf();
  // ALiBi joins the scores in raw units, like the bias: slope * (t - qa) /
  // scale, as a ramp added after each tile's QK plus a per-row constant.
  constexpr bool alibi = (FEAT & kFeatAlibi) != 0;
  const float al_s = alibi ? p.alibi[head] * inv_scale : 0.f;
  // The per-row ALiBi constant of the tile at kb, in log2 units: it joins the
  // exp's subtrahend and the tile's row max (the scores hold only the
  // tile-invariant ramp).  kb - qa is formed in integers, so the product is
  // exact to one rounding however long the sequence.
  const float al_c = al_s * c;
  auto crow = [&](int kb) { return al_c * (float)(kb + 4 * hf - qa); };
  // The exp's subtrahend and the row max of the tile at kb (without ALiBi
  // these are the running max and the max as they are).
  auto m_at = [&](float m, int kb) {
    if constexpr (alibi) return m - crow(kb);
    else return m;
  };
  auto mx_at = [&](float mx, int kb) {
    if constexpr (alibi) return mx + crow(kb);
    else return mx;
  };

  bf16x8 qf[KSTEPS];
  {
    const uint16_t *qp = p.q + ((int64_t)tok * p.H + head) * D + 8 * hf;
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 v = ld16(qp + 16 * ks);
      qf[ks] = zero_scale ? bf16x8{} : as_bf16x8(u32x4{v[0] ^ flip, v[1] ^ flip, v[2] ^ flip, v[3] ^ flip});
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = neg_inf(), l_run = 0.f;

  const int64_t tok_stride = (int64_t)p.Hkv * D;     // elements between consecutive slots
  constexpr int EB = KV8 ? 1 : 2;                     // bytes per cache element
  const uint32_t slot_bytes = (uint32_t)(tok_stride * EB);
  const uint64_t page_bytes = (uint64_t)p.BS * slot_bytes;
  const int32_t *bt = p.block_table + (int64_t)b * p.P;
  auto pidx = [&](int key) { return p.bs_shift >= 0 ? key >> p.bs_shift : key / p.BS; };
  auto pslot = [&](int key) { return p.bs_shift >= 0 ? key & (p.BS - 1) : key % p.BS; };
  // Staging: wave w fills rows 16w .. 16w+15 of each K and V tile (one
  // 16-key block, hence one page) with direct buffer->LDS loads through a
  // scalar buffer resource over the block's keys below kend; keys past it
  // arrive as zeros.  Each load instruction writes 1 KB of LDS in lane order,
  // RPI rows of UNITS 16-byte units; lane l brings the unit that the swizzle
  // places at its position.
  constexpr int UNITS = L::UNITS;
  constexpr int ROWB = L::ROWB;
  constexpr int RPI = 64 / UNITS;      // rows per load instruction
  constexpr int NI = 16 / RPI;         // load instructions per wave per operand
  const int kbw = 16 * w;
  // Lane l of load n brings row rr = RPI n + l / UNITS of the wave's block,
  // unit (l % UNITS) ^ swz(kbw + rr), from key slot rev4(rr) of the page.
  // RPI is a multiple of 4, so rev4(rr) = RPI n + rev4(l / UNITS); the V
  // swizzle does not depend on n, and the K swizzle of load n is that of
  // load 0 XOR 4 n.  Three registers per lane give every load's offset.
  const int lx = lane / UNITS, pu = lane % UNITS;
  const uint32_t vrow = (uint32_t)rev4(lx) * slot_bytes;
  const uint32_t uk16 = (uint32_t)((pu ^ swz_k<D>(kbw + lx)) << 4);
  const uint32_t vrow_v = vrow + (uint32_t)((pu ^ swz_v<D>(kbw + lx)) << 4);
  // Tiles are visited from the bottom of the range up: tile jt starts at key
  // tile_kb(jt).  The bias band sits just under the diagonal, so its tiles
  // come last and each item starts with plain tiles (measured 5 % faster on
  // the chunked prefill batch than visiting the band first).
  const int nt = t0 < t1 ? (t1 - t0 + kTileKeys - 1) / kTileKeys : 0;
  auto tile_kb = [&](int jt) { return t0 + jt * kTileKeys; };
  // Page ids of this wave's 16-key block for a window of 64 tiles, one per
  // lane, read back with readlane (no memory access in the loop); the next
  // window is loaded 64 tiles ahead.
  auto load_pages = [&](int jt0) {
    const int jt = jt0 + lane;
    const int key = tile_kb(jt) + kbw;
    return jt < nt && key < kend ? bt[pidx(key)] : 0;
  };
  int pc_base = 0;
  int pc = load_pages(0);
  int pc_next = load_pages(64);
  auto page_t = [&](int jt) { return __builtin_amdgcn_readlane(pc, jt - pc_base); };
  const char *kcache = reinterpret_cast<const char *>(p.k) + (uint64_t)g * D * EB;
  const char *vcache = reinterpret_cast<const char *>(p.v) + (uint64_t)g * D * EB;
  // Direct loads of tile jt (zeros past the last tile) into the K (IS_K) or
  // V slot at lds_off.  The offsets are formed at each call from the three
  // lane registers (pinned there, so that the compiler does not hoist NI
  // offsets per operand out of the tile loop and hold them throughout).
  auto dma = [&](auto is_k_tag, const char *cache, int jt, int page, int lds_off) __attribute__((always_inline)) {
    constexpr bool IS_K = decltype(is_k_tag)::value;
    const bool live = jt < nt;
    const int key = (live ? tile_kb(jt) : t0) + kbw;
    const int nvalid = live ? min(max(kend - key, 0), 16) : 0;
    const char *src = cache + (uint64_t)(uint32_t)page * page_bytes + (uint64_t)(uint32_t)pslot(key) * slot_bytes;
    const auto rs = make_rsrc(src, (uint32_t)nvalid * slot_bytes);
    uint32_t vb = IS_K ? vrow : vrow_v;
    uint32_t u = uk16;
    asm volatile("" : "+v"(vb), "+v"(u));
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const uint32_t rows = (uint32_t)(RPI * n) * slot_bytes;
      const uint32_t voff = IS_K ? vb + (u ^ (uint32_t)(64 * n)) + rows : vb + rows;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(smem + lds_off + (kbw + RPI * n) * ROWB), 16, voff, 0, 0, 0);
    }
  };
  // E4M3 caches: the direct loads bring the raw K rows of a tile (key order,
  // D bytes a row) to one of two landing areas, wave w its own 16 keys, and
  // the wave decodes its rows into the tile's bf16 K slot at the places the
  // bf16 loads would have filled (in the prologue, and for later tiles in
  // the phase B before their QK), so phase A is unchanged.  V rows stay raw
  // (dma8v, phase_b8).
  constexpr int U8 = D / 16, RPI8 = 64 / U8, NI8 = 16 / RPI8;
  // Block n of a wave's raw K rows: lane l loads raw unit l % U8 of landing
  // row RPI8 n + l / U8.  The decode then reads back raw unit pc8 = l % U8
  // of landing row RPI8 n + xd and writes it as the two bf16 units 2 pc8 + e
  // of K row kbw + rev4(RPI8 n + xd), at the places the swizzle gives them.
  // LDS writes go eight lanes at a time over 32 banks, and the eight lanes of
  // one row would write only four distinct 16-byte bank groups (2 pc8 + e is
  // even or odd with e), so with head_dim 128 the lanes of a write group take
  // eight different rows, xd = (l / U8 + pc8) mod 8: their swizzles then put
  // the eight units on distinct banks, and the raw reads stay conflict-free.
  // RPI8 is a multiple of 4, so rev4 keeps RPI8 n as it is, and the K
  // swizzle of block n is that of block 0 XOR 8 n (head_dim 128; 64 has one
  // block).  Three lane registers give every address.
  const int x8 = lane / U8, pc8 = lane % U8;
  const int xd = D == 128 ? (x8 + pc8) % RPI8 : x8;
  const int r8 = kbw + rev4(xd);
  const uint32_t row8 = (uint32_t)(r8 * ROWB);
  const uint32_t uk8 = (uint32_t)(((2 * pc8) ^ swz_k<D>(r8)) << 4);
  const uint32_t vb8 = (uint32_t)x8 * slot_bytes + (uint32_t)(pc8 << 4);
  // Landing offset (inside a block) of the raw unit this lane decodes.
  auto raw_at = [&]() { return (uint32_t)(16 * (xd * U8 + pc8)); };
  // K-slot byte offset of unit e of block n, from pinned copies of the lane
  // registers so that the compiler forms them where they are used instead
  // of holding 2 NI8 offsets across the tile loop.
  auto dst8 = [&](int n, int e, uint32_t row, uint32_t u) {
    const uint32_t flip = (uint32_t)((((D == 128) ? 8 * n : 0) ^ e) << 4);
    return row + (uint32_t)(RPI8 * n * ROWB) + (u ^ flip);
  };
  auto dma8 = [&](const char *cache, int jt, int page, int land_off) __attribute__((always_inline)) {
    const bool live = jt < nt;
    const int key = (live ? tile_kb(jt) : t0) + kbw;
    const int nvalid = live ? min(max(kend - key, 0), 16) : 0;
    const char *src = cache + (uint64_t)(uint32_t)page * page_bytes + (uint64_t)(uint32_t)pslot(key) * slot_bytes;
    const auto rs = make_rsrc(src, (uint32_t)nvalid * slot_bytes);
    uint32_t vb = vb8;
    asm volatile("" : "+v"(vb));
#pragma unroll
    for (int n = 0; n < NI8; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(smem + land_off + (kbw + RPI8 * n) * D), 16,
          vb + (uint32_t)(RPI8 * n) * slot_bytes, 0, 0, 0);
  };
  // Raw E4M3 V rows of tile jt into the V slot at off: row kbw + rr of the
  // slot holds key slot rev4(rr) of the wave's block (the order the bf16
  // tiles use), its units swizzled by swz_v8.  With RPI8 a multiple of 4 the
  // key slot is RPI8 n + rev4(l / U8), and the swizzle of block n is that of
  // block 0 XOR 4 n (head_dim 128; 64 has one block).
  const uint32_t vrow8 = (uint32_t)rev4(x8) * slot_bytes;
  const uint32_t u8v = (uint32_t)((pc8 ^ swz_v8<D>(kbw + x8)) << 4);
  auto dma8v = [&](const char *cache, int jt, int page, int off) __attribute__((always_inline)) {
    const bool live = jt < nt;
    const int key = (live ? tile_kb(jt) : t0) + kbw;
    const int nvalid = live ? min(max(kend - key, 0), 16) : 0;
    const char *src = cache + (uint64_t)(uint32_t)page * page_bytes + (uint64_t)(uint32_t)pslot(key) * slot_bytes;
    const auto rs = make_rsrc(src, (uint32_t)nvalid * slot_bytes);
    uint32_t vb = vrow8, u = u8v;
    asm volatile("" : "+v"(vb), "+v"(u));
#pragma unroll
    for (int n = 0; n < NI8; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(smem + off + (kbw + RPI8 * n) * D), 16,
          vb + (uint32_t)(RPI8 * n) * slot_bytes + (u ^ (uint32_t)(((D == 128) ? 4 * n : 0) << 4)), 0, 0, 0);
  };
  const uint32_t smem_u = (uint32_t)(uintptr_t)smem;
  // Prologue form of the K decode (later tiles are decoded inside phase_b8).
  auto decode8 = [&](int land_off, int slot_off) __attribute__((always_inline)) {
    u32x4 raw[NI8];
#pragma unroll
    for (int n = 0; n < NI8; ++n) raw[n] = lds_read_b128_asm(smem_u + land_off + (kbw + RPI8 * n) * D + raw_at());
    lgkm_wait_n<0>(raw);
    uint32_t row = smem_u + slot_off + row8, u = uk8;
    asm volatile("" : "+v"(row), "+v"(u));
    uint32_t dst[4];
#pragma unroll
    for (int i = 0; i < 2 * NI8; ++i) dst[i] = dst8(i >> 1, i & 1, row, u);
    if constexpr (NI8 == 2) {
      const uint32_t a[4] = {dst[0], dst[1], dst[2], dst[3]};
      const u32x4 vv[4] = {e4m3x8_to_bf16(raw[0][0], raw[0][1]), e4m3x8_to_bf16(raw[0][2], raw[0][3]),
                           e4m3x8_to_bf16(raw[1][0], raw[1][1]), e4m3x8_to_bf16(raw[1][2], raw[1][3])};
      lds_write_b128x4_now(a, vv);
    } else {
      lds_write_b128x2_now(dst[0], dst[1], e4m3x8_to_bf16(raw[0][0], raw[0][1]),
                           e4m3x8_to_bf16(raw[0][2], raw[0][3]));
    }
  };
  // The LDS writes of direct loads are tracked by vmcnt only: wait for them
  // before the barrier that publishes a tile.  When the 8 or 32 bias loads
  // of a later tile were issued after them, those may stay in flight.
  auto wait_vm0 = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)
  auto wait_vm8 = [&]() { __builtin_amdgcn_s_waitcnt(0x0F78); };   // vmcnt(8)
  auto wait_vm32 = [&]() { __builtin_amdgcn_s_waitcnt(0x8F70); };  // vmcnt(32)
  auto load_bias = [&](f32x16 *sacc, int kb) __attribute__((always_inline)) {
    if constexpr (rel_bf16) {
      if (bias_fast) tile_bias_load4_bf16(sacc, bias_rs, bias_el_base, kb);
      else tile_bias_load1_bf16(sacc, bias_rs, bias_el_base, kb);
    } else if (bias_fast) {
      tile_bias_load4(sacc, bias_rs, bias_lane_base, kb);
    } else {
      // Rows at either end of rel_logits: the lane's row pointer is formed
      // here from an opaque copy of the lane id, so that nothing of this
      // rare path is held across the tile loop.
      int ln = l32;
      asm volatile("" : "+v"(ln));
      const int rs_ = min(row0 + 32 * w + ln, row_last);
      const int qs_ = rs_ / G;
      const int64_t row_b = ((int64_t)(tok0 + qs_) * p.H + g * G + (rs_ - qs_ * G)) * p.R;
      tile_bias_load(sacc, kb, qa, p.rel_logits + row_b, p.R, hf);
    }
  };

  auto is_band = [&](int kb) { return p.R > 0 && kb <= band_hi && kb + kTileKeys - 1 >= band_lo; };
  // Plain: every key visible to every row, outside the band (the ALiBi ramp
  // is added after the QK, so it does not make a tile general).
  auto is_plain = [&](int kb) { return kb >= in_lo && kb + kTileKeys - 1 <= in_hi && !is_band(kb); };
  // Every key of the tile visible to, and in the band of, every row.
  const int full_lo = __builtin_amdgcn_readfirstlane(max(in_lo, qa_max - p.R + 1));
  const int full_hi = __builtin_amdgcn_readfirstlane(min(in_hi, qa_min));
  auto is_full_band = [&](int kb) { return kb >= full_lo && kb + kTileKeys - 1 <= full_hi; };
  auto bounds = [&](int kb) {
    const int off = kb + 4 * hf;
    return TileBounds{lo_r - off, hi_r - off, qa - p.R + 1 - off, qa - off};
  };
  // Lazy max update after the row max mx of a tile: O and l are rescaled
  // only when some row's max grew by more than kTau.
  auto update_max = [&](float mx) __attribute__((always_inline)) {
    if (__any(mx > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == neg_inf() ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
  };

  // Accumulator start of tile kb in set sacc, in two steps: begin() right
  // after the set is released (raw bias loads for a band tile, the masks
  // of an edge tile; a plain tile's set is zeroed first), finish() once
  // those loads have landed (band tiles only).
  auto start_general = [&](f32x16 *sacc, int kb) __attribute__((always_inline)) {
    tile_init<kInitEdge>(sacc, bounds(kb), inv_scale, masked);
  };
  auto begin = [&](f32x16 *sacc, int kb) __attribute__((always_inline)) {
    if (is_band(kb)) load_bias(sacc, kb);
    else if (!is_plain(kb)) start_general(sacc, kb);
  };
  auto finish = [&](f32x16 *sacc, int kb) __attribute__((always_inline)) {
    if (is_band(kb)) {
      if constexpr (rel_bf16) tile_bf16_widen4(sacc, bias_fast ? (uint32_t)((bias_el_base - kb) & 1) << 4 : 0u);
      if (is_full_band(kb)) tile_init<kInitFull>(sacc, bounds(kb), inv_scale, masked);
      else tile_init<kInitBand>(sacc, bounds(kb), inv_scale, masked);
    }
  };
  auto zero = [&](f32x16 *sacc) __attribute__((always_inline)) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
  };

  if (nt > 0) {
    // Software pipeline over 64-key tiles.  Tile j's K sits in K slot j%2,
    // its V in V slot j%2, its scores in register set j%2 (sa or sb).  While
    // tile j is in flight:
    //   phase A: exp of tile j on the VALU, QK of tile j+1 on the MFMA pipe;
    //   phase B: PV of tile j on the MFMA pipe, row max of tile j+1 on the
    //            VALU;
    // the direct loads of K(j+2) and V(j+1) and the raw bias of tile j+2
    // (into the register set tile j just freed) are in flight, and one
    // barrier ends the iteration.  A general tile's bias and masks are put
    // into its accumulator before its QK, so every tile's softmax is the same.
    f32x16 sa[2], sb[2];
    bf16x8 pb[4];
    // Page ids: pg_v of tile j+1 and pg_k of tile j+2 at the top of iteration j.
    int pg_v = page_t(1);
    int pg_k = page_t(2);
    {
      const int pg0 = page_t(0);
      if constexpr (KV8) {
        dma8(kcache, 0, pg0, L::landK(0));
        dma8(kcache, 1, pg_v, L::landK(1));
        dma8v(vcache, 0, pg0, L::v8Off(0));
        wait_vm0();
        decode8(L::landK(0), L::kOff(0));
        decode8(L::landK(1), L::kOff(1));
      } else {
        dma(BoolTag<true>{}, kcache, 0, pg0, L::kOff(0));
        dma(BoolTag<false>{}, vcache, 0, pg0, L::vOff(0));
        dma(BoolTag<true>{}, kcache, 1, pg_v, L::kOff(1));
      }
      zero(sa);
      begin(sa, tile_kb(0));
      wait_vm0();
      __syncthreads();
      // E4M3: the raw K(2), decoded in iteration 0's phase B (this wave's
      // rows of landing 0 were read by its own decode above).
      if constexpr (KV8) dma8(kcache, 2, pg_k, L::landK(0));
      finish(sa, tile_kb(0));
      qk_mfma<D, true>(smem + L::kOff(0), qf, sa, l32, hf);
      if constexpr (alibi) tile_alibi_ramp(sa, al_s);
      update_max(xor32_max(mx_at(tile_rowmax(sa) * c, tile_kb(0))));
      zero(sb);
      if (nt > 1) begin(sb, tile_kb(1));
      // Iteration 0 refills K slot 0: every wave must be done reading K(0)
      // (its reads completed before the QK used them; E4M3: a raw barrier, so
      // that the raw K(2) may stay in flight).
      if constexpr (KV8) barrier_raw();
      else __syncthreads();
    }

    // One pipeline iteration; PAR = j % 2 selects slots and register sets.
    // Both phases are branch-free; on the last tile the QK (of a K slot the
    // direct loads zero-filled) and the row max are computed and dropped.
    // The direct loads are issued on every iteration (past the split they
    // fill slots already consumed with zeros), so the number of loads in
    // flight is the same on every path.
    //
    // A plain tile's set is never set up: its QK starts from a zero
    // accumulator.  A general tile's set was started one iteration earlier
    // and is finished here before the direct loads are issued (the raw bias
    // of a band tile, loaded into it while the previous PV ran, has landed by
    // then); the raw bias of a band tile j+2 is loaded into the set tile j
    // releases between the two phases, so it has phase B and the barrier to
    // arrive.
    auto iteration = [&](auto par_tag, int j, f32x16 *cur, f32x16 *nxt) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_tag)::value ? 1 : 0;
      // The wave issues at raised priority from here to the end of phase A,
      // so that the other wave on its SIMD yields while this one is in the
      // VALU-heavy phase (measured 2-3 % faster on uniform shapes and the
      // continuous batch, no change on the chunked prefill).
      __builtin_amdgcn_s_setprio(1);
      const bool has_next = j + 1 < nt;
      const bool zc = !has_next || is_plain(tile_kb(j + 1));
      if (!zc) finish(nxt, tile_kb(j + 1));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (KV8) {
        // Direct loads: raw V(j+1) into V slot 1-PAR, then the raw K(j+3)
        // into landing 1-PAR (K(j+1) was decoded from it in the last phase
        // B), so that the waits can leave K in flight for an iteration.
        if (j + 3 - pc_base == 64) {
          pc = pc_next;
          pc_base += 64;
          pc_next = load_pages(pc_base + 64);
        }
        const int pg3 = page_t(j + 3);
        dma8v(vcache, j + 1, pg_v, L::v8Off(1 - PAR));
        dma8(kcache, j + 3, pg3, L::landK(1 - PAR));
        pg_v = pg_k;
        pg_k = pg3;
      } else {
        // Direct loads: K(j+2) into K slot PAR (K(j) was consumed before the
        // last barrier), V(j+1) into V slot 1-PAR.
        dma(BoolTag<true>{}, kcache, j + 2, pg_k, L::kOff(PAR));
        dma(BoolTag<false>{}, vcache, j + 1, pg_v, L::vOff(1 - PAR));
        if (j + 3 - pc_base == 64) {
          pc = pc_next;
          pc_base += 64;
          pc_next = load_pages(pc_base + 64);
        }
        pg_v = pg_k;
        pg_k = page_t(j + 3);
      }
      const float m_use = m_run == neg_inf() ? 0.f : m_run;
      __builtin_amdgcn_sched_barrier(0);
      // Phase A: QK of tile j+1 (MFMA) || exp of tile j (VALU).
      l_run += phase_a<D>(smem + L::kOff(1 - PAR), qf, nxt, cur, c, m_at(m_use, tile_kb(j)), pb, l32, hf, zc);
      __builtin_amdgcn_s_setprio(0);
      const bool band2 = j + 2 < nt && is_band(tile_kb(j + 2));
      if (band2) load_bias(cur, tile_kb(j + 2));
      __builtin_amdgcn_sched_barrier(0);
      // Phase B: PV of tile j (MFMA) || row max of tile j+1 (VALU); E4M3:
      // also the decode of this wave's rows of the raw K(j+2) into K slot PAR.
      float mx_raw;
      if constexpr (KV8) {
        uint32_t krow = smem_u + row8, kuk = uk8, kraw = smem_u + (uint32_t)(kbw * D) + raw_at();
        asm volatile("" : "+v"(krow), "+v"(kuk), "+v"(kraw));
        mx_raw = phase_b8<D, L::v8Off(PAR), L::landK(PAR), L::kOff(PAR), alibi, alibi>(
            smem, pb, oacc, lane, nxt, al_s, !band2 ? 0 : band_wait, kraw, krow, kuk);
      } else {
        mx_raw = phase_b<D, L::vOff(PAR), alibi, false>(smem, pb, oacc, lane, nxt, al_s);
      }
      const float mx = mx_at(mx_raw * c, tile_kb(j + 1));
      // Masks of an edge tile j+2 in the released set, then the barrier that
      // publishes K(j+2) and V(j+1).  Raw bias loads (and with E4M3 caches
      // the raw K(j+3)) may stay in flight.
      if (!band2 && j + 2 < nt && !is_plain(tile_kb(j + 2))) start_general(cur, tile_kb(j + 2));
      __builtin_amdgcn_sched_barrier(0);
      const int bw = band2 ? band_wait : 0;
      if constexpr (KV8) {
        if (bw == 0) __builtin_amdgcn_s_waitcnt(vmcnt_enc(NI8));
        else if (bw == 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(NI8 + 8));
        else __builtin_amdgcn_s_waitcnt(vmcnt_enc(NI8 + 32));
      } else {
        if (bw == 0) wait_vm0();
        else if (bw == 1) wait_vm8();
        else wait_vm32();
      }
      barrier_raw();
      if (has_next) update_max(xor32_max(mx));
    };

    for (int j = 0; j < nt; j += 2) {
      iteration(BoolTag<false>{}, j, sa, sb);
      if (j + 1 < nt) iteration(BoolTag<true>{}, j + 1, sb, sa);
    }
    if constexpr (KV8) wait_vm0();  // the raw K loads past the last tile
  }

  // Epilogue: lane (l32, hf) holds O^T[d = 32 db + 8 (j/4) + 4 hf + j%4][row l32].
  const float l_tot = xor32_sum(l_run);
  const float inv = l_tot > 0.f ? (KV8 ? p.v_scale / l_tot : 1.f / l_tot) : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : neg_inf();
  if (!row_valid) return;
  // The lane's token and head once more, from an opaque copy of the lane id:
  // the compiler would otherwise keep the output offsets from before the
  // tile loop, in registers spilled across it.
  int lane_e = l32;
  asm volatile("" : "+v"(lane_e));
  const int r_e = row0 + 32 * w + lane_e;
  const int qi_e = r_e / G;
  const int64_t row_out = (int64_t)(tok0 + qi_e) * p.H + g * G + (r_e - qi_e * G);
  if (p.S == 1) {
    uint16_t *op = p.out + row_out * D;
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
    if (hf == 0 && p.lse) p.lse[row_out] = lse_v;
  } else {
    const int64_t part_row = (int64_t)s * p.num_tokens * p.H + row_out;
    float *pp = p.part_out + part_row * D;
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
    if (hf == 0) p.part_lse[part_row] = lse_v;
  }
}

// ----------------------------------------------------------------- decode

// NW waves per decode workgroup.
template <int D, int NW>
struct DecodeLds {
  static constexpr int VS = kDecWaveKeys + 8;              // V^T row stride (bf16): 80 B
  static constexpr int vtBytes = NW * D * VS * 2;          // one V^T tile per wave
  static constexpr int redOBytes = NW * D * kDecCols * 4;  // per-wave O^T partials
  static constexpr int mainBytes = vtBytes > redOBytes ? vtBytes : redOBytes;
  static constexpr int redMLBytes = 2 * NW * kDecCols * 4; // per-wave m and l
  static constexpr int pageBytes = kPageCache * 4;
  static constexpr int bytes = mainBytes + redMLBytes + pageBytes;
};

// Key (0..31, relative to the wave's block) held at V^T slot p: slot 8q + i
// holds key 4q + i for i < 4 and 16 + 4q + i - 4 otherwise, matching the
// two 16x16 S^T accumulators of lane group q.
__device__ __forceinline__ int decode_key_of_slot(int p) {
  return 4 * (p >> 3) + (p & 7) + ((p & 4) ? 12 : 0);
}

template <int D, bool KV8>
struct DecodeRegs {
  // bf16: 16-byte loads; E4M3 caches: 8-byte loads of the same elements.
  using R = typename std::conditional<KV8, u32x2, u32x4>::type;
  R k[2][D / 32];
  R v[D / 16];
};

// NSET register sets form a ring: while block i is computed, the loads of
// blocks i+1 .. i+NSET-1 (and, once block i's registers are consumed, of
// block i+NSET) are in flight.
template <int D, int NSET, int NW, bool KV8>
__device__ void decode_item(const AttnParams &p, const Item &it, int g, int s, char *smem) {
  using DL = DecodeLds<D, NW>;
  constexpr int STEP = NW * kDecWaveKeys;  // keys per workgroup per iteration
  constexpr int QK = D / 32;       // 16x16x32 k-steps over head_dim
  constexpr int DB = D / 16;       // 16-row blocks of O^T
  constexpr int DQ = D / 4;        // head_dim span of one lane group in K operands
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int NG = 64 / CH;      // lane groups per chunk in V staging
  constexpr int KPL = kDecWaveKeys / NG;  // V keys per lane (8 or 4)
  constexpr int VS = DL::VS;
  static_assert(KPL == 8 || KPL == 4, "staging layout");

  const int b = it.b;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q = lane >> 4;
  uint16_t *Vt = reinterpret_cast<uint16_t *>(smem) + w * D * VS;
  int32_t *pcache = reinterpret_cast<int32_t *>(smem + DL::mainBytes + DL::redMLBytes);

  // Per-request scalars (uniform: kept in SGPRs so the range arithmetic runs
  // on the scalar unit).
  const int tok0 = __builtin_amdgcn_readfirstlane(p.cu_seqlens_q[b]);
  const int lq = __builtin_amdgcn_readfirstlane(p.cu_seqlens_q[b + 1]) - tok0;
  const int lk = __builtin_amdgcn_readfirstlane(p.cache_seqlens[b]);
  const int G = p.G;
  const int ncols = lq * G;
  const int col = c16 < ncols ? c16 : ncols - 1;  // idle columns shadow the last one
  const int qi = col / G;
  const int head = g * G + (col - qi * G);
  const int tok = tok0 + qi;
  const int qa = qi + lk - lq;
  const int qa_min = lk - lq;
  const int qa_max = (ncols - 1) / G + lk - lq;
  const Range sr = split_range(visible_range(p, lk, qa_min, qa_max), it.kmax, p.S, s, STEP);
  const int t0 = sr.lo, t1 = sr.hi;
  const int kend = min(lk, t1);
  int lo_c = t0, hi_c = kend - 1;
  if (p.left >= 0) lo_c = max(lo_c, qa - p.left);
  if (p.causal) hi_c = min(hi_c, qa);
  if (p.right >= 0) hi_c = min(hi_c, qa + p.right);
  int in_lo = t0, in_hi = kend - 1;
  if (p.left >= 0) in_lo = max(in_lo, qa_max - p.left);
  if (p.causal) in_hi = min(in_hi, qa_min);
  if (p.right >= 0) in_hi = min(in_hi, qa_min + p.right);
  const int band_lo = qa_min - p.R + 1, band_hi = qa_max;
  const float *rel_row = p.R > 0 ? p.rel_logits + ((int64_t)tok * p.H + head) * p.R : nullptr;
  const float c = p.scale_log2;
  const bool pos_scale = c > 0.f;
  const bool alibi = p.alibi != nullptr;
  const float al = alibi ? p.alibi[head] * kLog2e : 0.f;
  // bf16 rel_logits: the same row in 16-bit elements.
  const uint16_t *rel_row16 =
      p.R > 0 ? reinterpret_cast<const uint16_t *>(p.rel_logits) + ((int64_t)tok * p.H + head) * p.R : nullptr;

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
  int pfirst = 0;  // block-table index of pcache[0]

  // Buffer resources over the two 16-key blocks at `base`, one per cache:
  // the page id is wave-uniform, so the address arithmetic runs on the
  // scalar unit, and each resource covers only the block's keys below kend,
  // so the hardware returns zeros for the rest.
  struct BlockRsrc {
    __amdgpu_buffer_rsrc_t k[2], v[2];
  };
  constexpr int EB = KV8 ? 1 : 2;  // bytes per cache element
  const uint32_t slot_bytes = (uint32_t)(tok_stride * EB);
  auto rows_of = [&](int base, BlockRsrc &br) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kb = __builtin_amdgcn_readfirstlane(base + 16 * blk);
      const int nvalid = __builtin_amdgcn_readfirstlane(min(max(kend - kb, 0), 16));
      int page = 0, slot0 = 0;
      if (nvalid > 0) {
        const int pidx = p.bs_shift >= 0 ? (kb >> p.bs_shift) : kb / p.BS;
        slot0 = p.bs_shift >= 0 ? (kb & (p.BS - 1)) : kb % p.BS;
        page = __builtin_amdgcn_readfirstlane(pcache[pidx - pfirst]);
      }
      const int64_t off = (((int64_t)page * p.BS + slot0) * p.Hkv + g) * D;
      br.k[blk] = make_rsrc(reinterpret_cast<const char *>(p.k) + off * EB, (uint32_t)nvalid * slot_bytes);
      br.v[blk] = make_rsrc(reinterpret_cast<const char *>(p.v) + off * EB, (uint32_t)nvalid * slot_bytes);
    }
  };
  // Per-lane byte offsets inside a block (fixed for the whole loop).
  uint32_t koff[QK], voff[KPL];
#pragma unroll
  for (int ks = 0; ks < QK; ++ks) koff[ks] = c16 * slot_bytes + (uint32_t)(q * DQ + 8 * ks) * EB;
#pragma unroll
  for (int rr = 0; rr < KPL; ++rr) {
    const int kr = decode_key_of_slot(vg * KPL + rr);
    voff[rr] = (kr & 15) * slot_bytes + (uint32_t)vdc * 8 * EB;
  }
  auto ld = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (KV8) return bload8(r, off);
    else return bload16(r, off);
  };
  // Eight elements as bf16 (E4M3 codes are decoded exactly).
  auto as_bf = [&](const typename DecodeRegs<D, KV8>::R &x) {
    if constexpr (KV8) return e4m3x8_to_bf16(x[0], x[1]);
    else return x;
  };
  auto issue_k = [&](DecodeRegs<D, KV8> &Rg, const BlockRsrc &br) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) Rg.k[blk][ks] = ld(br.k[blk], koff[ks]);
  };
  auto issue_v = [&](DecodeRegs<D, KV8> &Rg, const BlockRsrc &br) {
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) {
      const int kr = decode_key_of_slot(vg * KPL + rr);
      Rg.v[rr] = ld(br.v[kr >> 4], voff[rr]);
    }
  };

  // One 32-key block.  A single register set carries the block: V is moved
  // to LDS first and its registers immediately receive the next block's V;
  // once the QK MFMAs have read K, the next block's K loads land there too.
  auto compute = [&](DecodeRegs<D, KV8> &Rg, int base, int nbase, bool has_next, auto mask_tag, auto bias_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool BIAS = decltype(bias_tag)::value;
    constexpr bool PLAIN = !MASK && !BIAS;
    BlockRsrc nbr;
    if (has_next) rows_of(nbase, nbr);
    wave_lds_sync();
    u32x4 vb[KPL];
#pragma unroll
    for (int rr = 0; rr < KPL; ++rr) vb[rr] = as_bf(Rg.v[rr]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t *dst = Vt + (vdc * 8 + e) * VS + vg * KPL;
      if constexpr (KPL == 8) {
        *reinterpret_cast<u32x4 *>(dst) =
            u32x4{pair_elem(vb[0], vb[1], e), pair_elem(vb[2], vb[3], e),
                  pair_elem(vb[4], vb[5], e), pair_elem(vb[6], vb[7], e)};
      } else {
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pair_elem(vb[0], vb[1], e), pair_elem(vb[2], vb[3], e)};
      }
    }
    if (has_next) issue_v(Rg, nbr);
    f32x4 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sacc[blk] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) sacc[blk] = mfma16(as_bf16x8(as_bf(Rg.k[blk][ks])), qf[ks], sacc[blk]);
    }
    if (has_next) issue_k(Rg, nbr);
    // Lane (c16, q) holds S[col c16][key base + 16 blk + 4 q + j].
    float mx = neg_inf();
    if constexpr (PLAIN) {
      if (pos_scale) {
        float ms = neg_inf();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int j = 0; j < 4; ++j) ms = fmaxf(ms, sacc[blk][j]);
        mx = ms * c;
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sacc[blk][j] * c);
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = base + 16 * blk + 4 * q + j;
          float v = sacc[blk][j] * c;
          if constexpr (BIAS) {
            const int d = qa - t;
            float rb = 0.f;
            if ((unsigned)d < (unsigned)p.R)
              rb = p.rel_bf16 ? __uint_as_float((uint32_t)rel_row16[d] << 16) : rel_row[d];
            v = __builtin_fmaf(rb, kLog2e, v);
            if (alibi) v = __builtin_fmaf(al, (float)(t - qa), v);
          }
          if constexpr (MASK) {
            if (t < lo_c || t > hi_c) v = neg_inf();
          }
          sacc[blk][j] = v;
          mx = fmaxf(mx, v);
        }
      }
    }
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    if (__any(mx > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == neg_inf() ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float m_use = m_run == neg_inf() ? 0.f : m_run;
    float pe[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sv = sacc[i >> 2][i & 3];
      pe[i] = exp2_fast(PLAIN ? __builtin_fmaf(sv, c, -m_use) : sv - m_use);
      psum += pe[i];
    }
    l_run += psum;
    const bf16x8 pf = pack8_bf16(pe);
    wave_lds_sync();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = as_bf16x8(ld16(Vt + (16 * db + c16) * VS + 8 * q));
      oacc[db] = mfma16(a, pf, oacc[db]);
    }
  };

  auto step = [&](DecodeRegs<D, KV8> &Rg, int base, int nbase, bool has_next) {
    const bool interior = base >= in_lo && base + kDecWaveKeys - 1 <= in_hi;
    const bool bias = (p.R > 0 && base <= band_hi && base + kDecWaveKeys - 1 >= band_lo) || alibi;
    if (interior && !bias) compute(Rg, base, nbase, has_next, BoolTag<false>{}, BoolTag<false>{});
    else compute(Rg, base, nbase, has_next, BoolTag<true>{}, BoolTag<true>{});
  };

  // The split is walked in segments whose block-table entries fit the LDS
  // page cache.  Inside a segment, wave w takes 32-key blocks w, w + NW, ...
  // with the loads of its next block in flight while the current one is
  // computed.
  const int seg_keys = ((kPageCache - 2) * p.BS) / STEP * STEP;
  for (int sg0 = t0; sg0 < t1; sg0 += seg_keys) {
    const int sg1 = min(t1, sg0 + seg_keys);
    __syncthreads();  // every wave is done with the previous segment's pages
    if (sg0 < kend) {
      pfirst = sg0 / p.BS;
      const int np = (min(sg1, kend) - 1) / p.BS - pfirst + 1;
      for (int i = tid; i < np; i += 64 * NW) pcache[i] = bt[pfirst + i];
    }
    __syncthreads();
    const int nblk = (sg1 - sg0 + kDecWaveKeys - 1) / kDecWaveKeys;
    const int my_n = nblk > w ? (nblk - w + NW - 1) / NW : 0;
    DecodeRegs<D, KV8> Rg[NSET];
#pragma unroll
    for (int j = 0; j < NSET; ++j) {
      if (j < my_n) {
        BlockRsrc br;
        rows_of(sg0 + kDecWaveKeys * (w + NW * j), br);
        issue_k(Rg[j], br);
        issue_v(Rg[j], br);
      }
    }
    for (int i = 0; i < my_n; i += NSET) {
#pragma unroll
      for (int j = 0; j < NSET; ++j) {
        if (i + j < my_n) {
          const int base = sg0 + kDecWaveKeys * (w + NW * (i + j));
          step(Rg[j], base, base + NSET * STEP, i + j + NSET < my_n);
        }
      }
    }
  }

  // Merge the NW waves' (m, l, O^T) through LDS.
  const float l_col = xor32_sum(xor16_sum(l_run));
  __syncthreads();
  float *red_o = reinterpret_cast<float *>(smem);  // [NW][D][16]
  float *red_m = reinterpret_cast<float *>(smem + DL::mainBytes);
  float *red_l = red_m + NW * kDecCols;
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
  constexpr int DPG = D / (4 * NW);  // head_dim values per thread in the merge
  const int fc = tid & 15, fg = tid >> 4;
  if (fc >= ncols) return;
  float mw[NW], sc[NW];
  float M = neg_inf();
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    mw[ww] = red_m[ww * kDecCols + fc];
    M = fmaxf(M, mw[ww]);
  }
  float L = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    sc[ww] = mw[ww] == neg_inf() ? 0.f : exp2_fast(mw[ww] - M);
    L += sc[ww] * red_l[ww * kDecCols + fc];
  }
  const float inv = L > 0.f ? (KV8 ? p.v_scale / L : 1.f / L) : 0.f;
  const float lse_v = L > 0.f ? (M + log2_fast(L)) * kLn2 : neg_inf();
  float o[DPG];
#pragma unroll
  for (int e = 0; e < DPG; ++e) {
    const int d = fg * DPG + e;
    float acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) acc += sc[ww] * red_o[(ww * D + d) * kDecCols + fc];
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
    } else if constexpr (DPG == 4) {
      *reinterpret_cast<u32x2 *>(op) = u32x2{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
    } else {
      *reinterpret_cast<uint32_t *>(op) = pack2_bf16(o[0], o[1]);
    }
    if (fg == 0 && p.lse) p.lse[(int64_t)ftok * p.H + fhead] = lse_v;
  } else {
    float *pp = p.part_out + (((int64_t)s * p.num_tokens + ftok) * p.H + fhead) * D + fg * DPG;
    if constexpr (DPG >= 4) {
#pragma unroll
      for (int e = 0; e < DPG; e += 4) *reinterpret_cast<f32x4 *>(pp + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
    } else {
      *reinterpret_cast<f32x2 *>(pp) = f32x2{o[0], o[1]};
    }
    if (fg == 0) p.part_lse[((int64_t)s * p.num_tokens + ftok) * p.H + fhead] = lse_v;
  }
}

// Waves per workgroup (four for both variants: a decode workgroup of eight
// waves, one per CU, streamed no faster than two of four, since a CU's
// outstanding misses, not its waves, bound its KV rate).
template <bool DECODE_ONLY>
constexpr int attn_waves() { return 4; }

template <int D, bool DECODE_ONLY, bool KV8>
constexpr int attn_lds_bytes() {
  using DL = DecodeLds<D, attn_waves<DECODE_ONLY>()>;
  using PL = PrefillLds<D, KV8>;
  return (DECODE_ONLY || PL::bytes < DL::bytes) ? DL::bytes : PL::bytes;
}

// DECODE_ONLY: every request of the batch has Lq*G <= 16 (known on the host
// from max_seqlen_q), so the prefill path is not compiled in.  Both variants
// hold two workgroups, i.e. two waves per SIMD, per CU.
// FEAT: the prefill variant (ALiBi: the ramp is added to each tile's scores
// after its QK; bf16 rel_logits: band tiles load 16-bit values); the decode
// items test p.alibi and p.rel_bf16 at run time.  Register pressure decides
// where the ALiBi ramp goes: an accumulator initialised before the QK and
// held across the barrier needs about 20 more VGPRs than the 256 a wave has
// at two waves per SIMD, and the scratch reloads that the spills put in the
// tile loop wait for every direct load in flight.
template <int D, bool DECODE_ONLY, bool KV8, int FEAT>
__global__ __launch_bounds__(64 * attn_waves<DECODE_ONLY>(), 2) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[attn_lds_bytes<D, DECODE_ONLY, KV8>()];
  const int bid = blockIdx.x;
  const int s = bid % p.S;
  const int rest = bid / p.S;
  const int g = rest % p.Hkv;
  const int item = rest / p.Hkv;
  const Item it = resolve_item(p, item, DECODE_ONLY, kTileRows);
  const int kind = __builtin_amdgcn_readfirstlane(it.kind);
  if (kind == 2) {
    decode_item<D, 1, attn_waves<DECODE_ONLY>(), KV8>(p, it, g, s, smem);
  } else if constexpr (!DECODE_ONLY) {
    if (kind == 1) prefill_item<D, KV8, FEAT>(p, it, g, s, smem);
  }
}

// ------------------------------------------------------ balanced decode
//
// Decode-only batches with num_splits = 0.  The work of the batch is the
// sequence of 16-key units of every (request, kv head) pair, pairs in
// (request, kv head) order and units in key order; workgroup w of W takes
// units [w*TU/W, (w+1)*TU/W), so every CU streams the same number of KV
// bytes whatever the length mix.  A workgroup walks its range piece by piece
// (a piece is the part of one pair inside the range); its waves take the
// piece's units round-robin, each with the next unit's loads in flight, and
// merge their softmax states through LDS at the end of the piece.  A piece
// that is a whole pair writes the output; a piece of a pair cut between
// workgroups writes a normalised partial to its slot, and the workgroup that
// holds the pair's first unit records the pair for the combine.
//
// K and V rows reach LDS by direct loads in which 16 lanes cover one key's
// 256-byte head slice (a load instruction reads whole 128-byte lines), with
// the 16-byte units of each row XOR-swizzled.  S^T = K·Q^T runs on 16x16x32
// MFMA (K rows from LDS, Q^T in registers); O^T = V^T·P^T on 16x16x16 MFMA,
// V^T read with ds_read_b64_tr_b16 and P^T taken straight from the S^T
// accumulator (lane (col, q) holds keys 4q..4q+3 of its column, which is
// the B operand layout of the 16x16x16 product).

constexpr int kBalStages = 2;  // 16-key units in flight or in use per wave

template <int D>
struct BalLds {
  static constexpr int ROWB = D * 2;           // bytes per key row
  static constexpr int UNITS = D / 8;          // 16-byte units per row
  static constexpr int RPI = 64 / UNITS;       // rows per direct-load instruction
  static constexpr int NI = 16 / RPI;          // instructions per 16-key unit (K or V)
  static constexpr int halfBytes = 16 * ROWB;  // K (or V) of one unit
  static constexpr int stageBytes = 2 * halfBytes;
  static constexpr int NST = kBalStages;       // stages per wave
  static constexpr int biasOff = kBalWaves * NST * stageBytes;  // per wave and stage: 4 x 64 fp32
  static constexpr int mlOff = biasOff + kBalWaves * NST * 1024;     // merge: m, then l [waves][16]
  static constexpr int slotOff = mlOff + 2 * kBalWaves * kDecCols * 4;  // merge: each wave's stage
  static constexpr int prefixOff = slotOff + 64;
  static constexpr int bytes = prefixOff + (kBalMaxBatch + 1) * 4;
  // A wave's O^T partial (D x 16 fp32) fits in one of its stages.
  static_assert(D * kDecCols * 4 <= stageBytes, "merge buffer");
};

// V rows: unit u sits at u ^ swz_vt(r).  A transposing read touches two
// adjacent units of 16 consecutive rows; the swizzle moves them in pairs so
// that each half-wave's eight rows cover all banks.  Its low bit (head_dim
// 128) only swaps the two units of a pair, which leaves the reads' banks as
// they are; it lets the E4M3 decode's writes below reach odd and even bank
// groups from one instruction.
template <int D>
__device__ __forceinline__ int swz_vt(int r) {
  return D == 128 ? (2 * (r & 7)) | (((r >> 2) & 1) ^ 1) : 2 * ((r >> 1) & 3);
}
// E4M3 V (head_dim 128): which of the eight raw rows of a block lane l
// decodes (its raw unit is l % 8).  LDS reads and writes of 16 bytes go eight
// lanes at a time over 32 banks; with this choice the eight lanes of each
// group read eight distinct units of their 128-byte raw rows and write eight
// distinct bank groups of the bf16 rows (four rows whose swizzle has the low
// bit set, four without), so neither side has bank conflicts.
__device__ __forceinline__ int v8_row_of(int l) {
  const int g = l >> 3;
  return (g >> 1) + 4 * ((g & 1) ^ ((l & 7) >> 2));
}

// s_waitcnt lgkmcnt(N) that the listed registers wait for (their values
// arrive by inline-asm LDS reads the compiler does not track).
template <int N>
__device__ __forceinline__ void lgkm_wait_n(u32x4 (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_n(u32x2 (&r)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
               : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_n(u32x2 (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_n(float (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(N));
}

// s_waitcnt vmcnt(N): at most N vector-memory instructions of this wave
// still outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Load through the scalar cache (the data must not be written by the
// running kernel: the block table).
__device__ __forceinline__ int scalar_load_i32(const int32_t *p) {
  return *(const __attribute__((address_space(4))) int32_t *)p;
}
__device__ __forceinline__ float lds_read_f32_asm(uint32_t addr) {
  float v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ int lds_read_i32_now(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// LDS writes in inline asm complete before the asm ends: the compiler's
// hazard checks do not see inside asm, and the data registers may be
// overwritten by the next instruction.
__device__ __forceinline__ void lds_write_b32_now(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write4_b128_now(const uint32_t (&a)[4], const f32x4 (&v)[4]) {
  asm volatile(
      "ds_write_b128 %0, %4\n\tds_write_b128 %1, %5\n\tds_write_b128 %2, %6\n\tds_write_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3])
      : "memory");
}
__device__ __forceinline__ void lgkm_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }
// Eight LDS reads in flight together, then one wait that the results depend on.
__device__ __forceinline__ void lds_read8_b32(uint32_t a0, uint32_t stride, uint32_t (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("ds_read_b32 %0, %1" : "=v"(v[i]) : "v"(a0 + i * stride) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}
__device__ __forceinline__ void lds_read8_b128(const uint32_t (&a)[8], u32x4 (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("ds_read_b128 %0, %1" : "=v"(v[i]) : "v"(a[i]) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}
__device__ __forceinline__ void lds_read8_b64(const uint32_t (&a)[8], u32x2 (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("ds_read_b64 %0, %1" : "=v"(v[i]) : "v"(a[i]) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}
__device__ __forceinline__ u32x2 lds_read_tr_at(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}

// 16-key units of request b's (request, kv head) pair: the visible range of
// its rows from its start rounded down to 16; at least one unit, so that a
// request without visible keys still writes its rows.
__device__ __forceinline__ int bal_units(const AttnParams &p, int b) {
  const int lq = p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
  if (lq <= 0) return 0;
  const int lk = p.cache_seqlens[b];
  const Range r = visible_range(p, lk, lk - lq, lk - 1);
  const int lo_a = r.lo & ~15;
  return r.hi > lo_a ? max((r.hi - lo_a + 15) >> 4, 1) : 1;
}

// prefix[b] = mult * (units of requests before b); prefix[batch] = all.
__device__ void bal_prefix(const AttnParams &p, int32_t *prefix, int32_t *tmp, int mult) {
  constexpr int NT = 64 * kBalWaves;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int B = p.batch;
  const int per = (B + NT - 1) / NT;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += bal_units(p, b);
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  int base = 0;
  for (int ww = 0; ww < w; ++ww) base += tmp[ww];
  int run = (base + incl - local) * mult;
  for (int b = b0; b < b1; ++b) {
    prefix[b] = run;
    run += bal_units(p, b) * mult;
  }
  if (b0 < b1 && b1 == B) prefix[B] = run;
  __syncthreads();
}

__device__ __forceinline__ int bal_unit_at(int TU, int x, int nwg) { return (int)((int64_t)TU * x / nwg); }

template <int D, bool BIAS, bool KV8>
__device__ void decode_balanced(const AttnParams &p, char *smem) {
  using L = BalLds<D>;
  constexpr int NW = kBalWaves;
  constexpr int QK = D / 32, DB = D / 16, NI = L::NI, RPI = L::RPI, UNITS = L::UNITS, ROWB = L::ROWB;
  static_assert(L::NST == 2, "two stages per wave: one computed, one in flight");
  // E4M3 caches (as in decode_heads): two raw stages, then the bf16 V stage,
  // which the merge also uses for the wave's O^T (it holds no load).
  constexpr int U8 = D / 16, RPI8 = 64 / U8, NI8 = 16 / RPI8;
  constexpr uint32_t LAND = 32 * D;
  static_assert(!KV8 || 2 * LAND + D * kDecCols * 4 <= 2 * L::stageBytes, "fp8 stages and merge fit");
  constexpr int NLD = KV8 ? NI8 : NI;
  constexpr int NPER = 2 * NLD + (BIAS ? 4 : 0);  // vector-memory instructions per unit
  int32_t *prefix = reinterpret_cast<int32_t *>(smem + L::prefixOff);
  bal_prefix(p, prefix, reinterpret_cast<int32_t *>(smem + L::mlOff), p.Hkv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q = lane >> 4;
  const int B = p.batch, Hkv = p.Hkv, G = p.G;
  const int nwg = p.bal_wgs, wg = blockIdx.x;
  const int TU = __builtin_amdgcn_readfirstlane(prefix[B]);
  const int u0 = bal_unit_at(TU, wg, nwg), u1 = bal_unit_at(TU, wg + 1, nwg);
  int b_it = 0;
  {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= u0) lo = mid;
      else hi = mid - 1;
    }
    b_it = __builtin_amdgcn_readfirstlane(lo);
  }

  const uint32_t slot_bytes = (uint32_t)Hkv * D * (KV8 ? 1 : 2);
  uint32_t gk[NLD], gv[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    if constexpr (KV8) {
      const int r = RPI8 * n + lane / U8, pu = lane % U8;
      gk[n] = r * slot_bytes + ((pu ^ (r & (U8 - 1))) << 4);
      gv[n] = r * slot_bytes + (pu << 4);
    } else {
      const int r = RPI * n + lane / UNITS, pu = lane % UNITS;
      gk[n] = r * slot_bytes + ((pu ^ swz_k<D>(r)) << 4);
      gv[n] = r * slot_bytes + ((pu ^ swz_vt<D>(r)) << 4);
    }
  }
  uint32_t lk_off[QK], lv_off[DB];
#pragma unroll
  for (int ks = 0; ks < QK; ++ks) {
    if constexpr (KV8)
      lk_off[ks] = c16 * D + (((2 * ks + (q >> 1)) ^ (c16 & (U8 - 1))) << 4) + 8 * (q & 1);
    else
      lk_off[ks] = c16 * ROWB + (((4 * ks + q) ^ swz_k<D>(c16)) << 4);
  }
  uint32_t v8_dst[KV8 ? 2 * NI8 : 1];
  // E4M3: offset, inside a raw block, of the raw V unit this lane decodes.
  const uint32_t v8_src = (uint32_t)(16 * (D == 128 ? U8 * v8_row_of(lane) + lane % U8 : lane));
  if constexpr (KV8) {
#pragma unroll
    for (int n = 0; n < NI8; ++n) {
      const int r = RPI8 * n + (D == 128 ? v8_row_of(lane) : lane / U8), pu = lane % U8;
#pragma unroll
      for (int e = 0; e < 2; ++e) v8_dst[2 * n + e] = r * ROWB + (((2 * pu + e) ^ swz_vt<D>(r)) << 4);
    }
  }
  {
    const int i = (lane & 15) >> 2, t = lane & 3, row = 4 * q + i;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      lv_off[db] = L::halfBytes + row * ROWB + ((((2 * db + (t >> 1)) ^ swz_vt<D>(row)) << 4)) + 8 * (t & 1);
  }
  const uint32_t smem_u = (uint32_t)(uintptr_t)smem;
  const uint32_t lds_wave = smem_u + (uint32_t)(w * 2 * L::stageBytes);
  const uint32_t lds_bias = smem_u + (uint32_t)(L::biasOff + w * 2 * 1024 + 4 * lane);
  const uint32_t lds_m = smem_u + L::mlOff, lds_l = lds_m + NW * kDecCols * 4;
  const uint32_t lds_slot = smem_u + L::slotOff;
  const uint32_t lds_prefix = smem_u + L::prefixOff;
  const float c = p.scale_log2;
  const bool pos_scale = c > 0.f;
  // bf16 rel_logits: each lane loads the dword holding its element (the
  // range rounded up to whole dwords; a page never ends inside one) and
  // compute() keeps the element's half.
  const bool rel_bf16 = p.rel_bf16 != 0;
  const uint32_t bias_bytes =
      BIAS ? (rel_bf16 ? ((uint32_t)p.num_tokens * (uint32_t)p.H * (uint32_t)p.R * 2u + 3u) & ~3u
                       : (uint32_t)p.num_tokens * (uint32_t)p.H * (uint32_t)p.R * 4u)
           : 0u;
  const float v_scale = KV8 ? p.v_scale : 1.f;
  const bool alibi = p.alibi != nullptr;

  // A piece: units [j0, j1) of pair (b, g) inside this workgroup's range,
  // with what its rows need (uniform fields, then the lane's column).
  struct Piece {
    int b, g, j0, j1, nu, which, pair_start;
    int tok0, lq, ncols, lo_a, kend, in_lo, in_hi, band_lo, band_hi, my_n;
    int qa, lo_c, hi_c, tok, head;
    uint32_t rel_base;
    float al;  // ALiBi slope of the lane's head times log2(e), or 0
  };
  // LDS reads while direct loads are in flight go through inline asm (the
  // compiler would wait for the loads first).
  auto prefix_at = [&](int i) { return __builtin_amdgcn_readfirstlane(lds_read_i32_now(lds_prefix + 4u * i)); };
  auto make_piece = [&](int cur) __attribute__((always_inline)) {
    Piece P;
    while (prefix_at(b_it + 1) <= cur) ++b_it;
    P.b = b_it;
    const int pb = prefix_at(b_it);
    P.nu = (prefix_at(b_it + 1) - pb) / Hkv;
    const int off = cur - pb;
    P.g = off / P.nu;
    P.j0 = off - P.g * P.nu;
    P.j1 = min(P.nu, P.j0 + (u1 - cur));
    P.which = cur == u0 ? 0 : 1;
    P.pair_start = pb + P.g * P.nu;
    P.tok0 = scalar_load_i32(p.cu_seqlens_q + P.b);
    P.lq = scalar_load_i32(p.cu_seqlens_q + P.b + 1) - P.tok0;
    const int lk = scalar_load_i32(p.cache_seqlens + P.b);
    P.ncols = P.lq * G;
    const int col = c16 < P.ncols ? c16 : P.ncols - 1;
    const int qi = col / G;
    P.head = P.g * G + (col - qi * G);
    P.tok = P.tok0 + qi;
    P.qa = qi + lk - P.lq;
    const int qa_min = lk - P.lq, qa_max = lk - 1;
    const Range vr = visible_range(p, lk, qa_min, qa_max);
    P.lo_a = vr.lo & ~15;
    P.kend = min(lk, vr.hi);
    P.lo_c = P.lo_a;
    P.hi_c = P.kend - 1;
    if (p.left >= 0) P.lo_c = max(P.lo_c, P.qa - p.left);
    if (p.causal) P.hi_c = min(P.hi_c, P.qa);
    if (p.right >= 0) P.hi_c = min(P.hi_c, P.qa + p.right);
    P.in_lo = P.lo_a;
    P.in_hi = P.kend - 1;
    if (p.left >= 0) P.in_lo = max(P.in_lo, qa_max - p.left);
    if (p.causal) P.in_hi = min(P.in_hi, qa_min);
    if (p.right >= 0) P.in_hi = min(P.in_hi, qa_min + p.right);
    P.band_lo = qa_min - p.R + 1;
    P.band_hi = qa_max;
    P.rel_base = BIAS ? (uint32_t)((P.tok * p.H + P.head) * p.R) : 0u;
    P.al = alibi ? p.alibi[P.head] * kLog2e : 0.f;
    const int n_units = P.j1 - P.j0;
    P.my_n = n_units > w ? (n_units - w + NW - 1) / NW : 0;
    return P;
  };
  auto key_of = [&](const Piece &P, int k) { return P.lo_a + 16 * (P.j0 + w + NW * k); };
  auto in_band = [&](const Piece &P, int key0) { return BIAS && key0 <= P.band_hi && key0 + 15 >= P.band_lo; };
  // Page ids come from scalar loads one unit ahead of their use.
  auto page_of = [&](const Piece &P, int k) -> int {
    const int key = key_of(P, k);
    if (k >= P.my_n || key >= P.kend) return 0;
    return scalar_load_i32(p.block_table + (int64_t)P.b * p.P + (p.bs_shift >= 0 ? (key >> p.bs_shift) : key / p.BS));
  };
  auto load_q = [&](const Piece &P, bf16x8 (&qf)[QK]) __attribute__((always_inline)) {
    const uint16_t *qp = p.q + ((int64_t)P.tok * p.H + P.head) * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < QK; ++ks) qf[ks] = as_bf16x8(ld16(qp + 32 * ks));
  };

  auto issue = [&](const Piece &P, int k, int page, int slot) __attribute__((always_inline)) {
    const int key0 = __builtin_amdgcn_readfirstlane(key_of(P, k));
    const int nvalid = __builtin_amdgcn_readfirstlane(min(max(P.kend - key0, 0), 16));
    const int slot0 = p.bs_shift >= 0 ? (key0 & (p.BS - 1)) : key0 % p.BS;
    const int64_t eoff = (((int64_t)page * p.BS + slot0) * Hkv + P.g) * D;
    const auto rk = make_rsrc(reinterpret_cast<const char *>(p.k) + eoff * (KV8 ? 1 : 2), (uint32_t)nvalid * slot_bytes);
    const auto rv = make_rsrc(reinterpret_cast<const char *>(p.v) + eoff * (KV8 ? 1 : 2), (uint32_t)nvalid * slot_bytes);
    if constexpr (BIAS) {
      // Raw logits of the lane's four keys (distance clamped into the row;
      // the band test in compute() discards what lies outside it), through
      // an empty resource outside the band, so that every unit counts the
      // same vector-memory instructions.
      const auto brs = make_rsrc(p.rel_logits, in_band(P, key0) ? bias_bytes : 0u);
      char *bst = smem + L::biasOff + (w * 2 + slot) * 1024;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = min(max(P.qa - (key0 + 4 * q + j), 0), p.R - 1);
        const uint32_t boff = rel_bf16 ? ((P.rel_base + (uint32_t)d) * 2u) & ~3u : (P.rel_base + (uint32_t)d) * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (__attribute__((address_space(3))) void *)(bst + 256 * j), 4,
                                                 boff, 0, 0, 0);
      }
    }
    char *st = KV8 ? smem + w * 2 * L::stageBytes + slot * LAND : smem + (w * 2 + slot) * L::stageBytes;
    constexpr int VHALF = KV8 ? 16 * D : L::halfBytes;
#pragma unroll
    for (int n = 0; n < NLD; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void *)(st + n * 1024), 16,
                                               gk[n], 0, 0, kNonTemporal);
#pragma unroll
    for (int n = 0; n < NLD; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void *)(st + VHALF + n * 1024), 16, gv[n], 0, 0, kNonTemporal);
  };

  f32x4 oacc[DB];
  float m_run, l_run;
  auto compute = [&](const Piece &P, int k, int slot, const bf16x8 (&qf)[QK]) __attribute__((always_inline)) {
    const int key0 = __builtin_amdgcn_readfirstlane(key_of(P, k));
    u32x4 kf[QK];
    u32x2 va[DB];
    if constexpr (KV8) {
      const uint32_t land = lds_wave + slot * LAND;
      const uint32_t vst = lds_wave + 2 * LAND;
      u32x2 k8[QK];
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) k8[ks] = lds_read_b64_asm(land + lk_off[ks]);
      u32x4 v8[NI8];
#pragma unroll
      for (int n = 0; n < NI8; ++n) v8[n] = lds_read_b128_asm(land + 16 * D + n * 1024 + v8_src);
      lgkm_wait_n<0>(v8);
      lgkm_wait_n<0>(k8);
      if constexpr (NI8 == 2) {
        const uint32_t a[4] = {vst + v8_dst[0], vst + v8_dst[1], vst + v8_dst[2], vst + v8_dst[3]};
        const u32x4 vv[4] = {e4m3x8_to_bf16(v8[0][0], v8[0][1]), e4m3x8_to_bf16(v8[0][2], v8[0][3]),
                             e4m3x8_to_bf16(v8[1][0], v8[1][1]), e4m3x8_to_bf16(v8[1][2], v8[1][3])};
        lds_write_b128x4_now(a, vv);
      } else {
        lds_write_b128x2_now(vst + v8_dst[0], vst + v8_dst[1], e4m3x8_to_bf16(v8[0][0], v8[0][1]),
                             e4m3x8_to_bf16(v8[0][2], v8[0][3]));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = lds_read_tr_at(vst - L::halfBytes + lv_off[db]);
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) kf[ks] = e4m3x8_to_bf16(k8[ks][0], k8[ks][1]);
    } else {
      const uint32_t st = lds_wave + slot * L::stageBytes;
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) kf[ks] = lds_read_b128_asm(st + lk_off[ks]);
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = lds_read_tr_at(st + lv_off[db]);
      // LDS reads complete in order: the K operands are in once at most the
      // DB V reads issued after them are outstanding.
      lgkm_wait_n<DB>(kf);
    }
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < QK; ++ks) sacc = mfma16(as_bf16x8(kf[ks]), qf[ks], sacc);
    // Lane (c16, q) holds S[col c16][key key0 + 4q + j].
    const bool interior = key0 >= P.in_lo && key0 + 15 <= P.in_hi;
    const bool band = in_band(P, key0);
    const bool plain = interior && !band && !alibi;
    float mx = neg_inf();
    if (plain) {
      if (pos_scale) {
        mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3])) * c;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sacc[j] * c);
      }
    } else {
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if (band) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bias[j] = lds_read_f32_asm(lds_bias + slot * 1024 + 256 * j);
        lgkm_wait_n<0>(bias);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = key0 + 4 * q + j;
        float v = sacc[j] * c;
        if (band && (unsigned)(P.qa - t) < (unsigned)p.R) {
          float bv = bias[j];
          if (rel_bf16) {
            const uint32_t bits = __float_as_uint(bv);
            bv = __uint_as_float(((P.rel_base + (uint32_t)(P.qa - t)) & 1u) ? (bits & 0xffff0000u) : (bits << 16));
          }
          v = __builtin_fmaf(bv, kLog2e, v);
        }
        if (alibi) v = __builtin_fmaf(P.al, (float)(t - P.qa), v);
        if (t < P.lo_c || t > P.hi_c) v = neg_inf();
        sacc[j] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    if (__any(mx > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == neg_inf() ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float m_use = m_run == neg_inf() ? 0.f : m_run;
    float pe[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pe[j] = exp2_fast(plain ? __builtin_fmaf(sacc[j], c, -m_use) : sacc[j] - m_use);
    l_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
    const u32x2 pf = u32x2{pack2_bf16(pe[0], pe[1]), pack2_bf16(pe[2], pe[3])};
    lgkm_wait_n<0>(va);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = mfma16k16(va[db], pf, oacc[db]);
  };

  int own_b = -1, own_g = 0, own_last = 0, own_which = 0;
  int cur = u0;
  if (cur < u1) {
    Piece P = make_piece(cur);
    bf16x8 qf[QK];
    // The first unit's loads go out before Q's, so that the two latencies
    // overlap; the wait before the first unit is computed covers both.
    int slot0 = 0;        // stage of this wave's first unit of P
    if (P.my_n > 0) issue(P, 0, page_of(P, 0), 0);
    load_q(P, qf);
    while (true) {
      const int cur_next = cur + (P.j1 - P.j0);
      const bool has_next = cur_next < u1;
      Piece N;
      int page_n0 = 0;
      if (has_next) {
        N = make_piece(cur_next);
        page_n0 = page_of(N, 0);
      }
      const bool pre_n = has_next && N.my_n > 0;  // this wave prefetches N's first unit
      int page_nx = page_of(P, 1);
      bf16x8 qn[QK];
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};
      m_run = neg_inf();
      l_run = 0.f;
      // The direct loads write LDS behind the compiler's back: their
      // completion is awaited explicitly (vmcnt counts this wave's
      // vector-memory instructions in issue order).  While unit k is
      // computed the next unit of this wave's stream is in flight: unit
      // k+1 of P or, after P's last, unit 0 of the next piece.
      int pslot = -1;  // stage holding the next piece's first unit
      for (int k = 0; k < P.my_n; ++k) {
        const int sk = (slot0 + k) & 1;
        if (k + 1 < P.my_n) {
          issue(P, k + 1, page_nx, sk ^ 1);
          page_nx = page_of(P, k + 2);
          wait_vm<NPER>();
        } else if (pre_n) {
          load_q(N, qn);
          issue(N, 0, page_n0, sk ^ 1);
          pslot = sk ^ 1;
          wait_vm<NPER>();
        } else {
          wait_vm<0>();
        }
        compute(P, k, sk, qf);
      }
      if (P.my_n == 0 && pre_n) {
        load_q(N, qn);
        issue(N, 0, page_n0, 0);
        pslot = 0;
      }

      // Merge the waves' (m, l, O^T) through LDS: each wave's O^T goes to
      // its stage that holds no load in flight.  Raw barriers (no memory
      // fence) keep the next piece's loads in flight across the merge.
      const float l_col = xor32_sum(xor16_sum(l_run));
      const int rs = pslot == 0 ? 1 : 0;
      {
        const uint32_t red = KV8 ? lds_wave + 2 * LAND : lds_wave + rs * L::stageBytes;
#pragma unroll
        for (int d4 = 0; d4 < DB; d4 += 4) {
          uint32_t a[4];
          f32x4 v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = red + ((4 * (d4 + i) + q) * kDecCols + c16) * 16;
            v[i] = oacc[d4 + i];
          }
          lds_write4_b128_now(a, v);
        }
        if (q == 0) {
          lds_write_b32_now(lds_m + (w * kDecCols + c16) * 4, __builtin_bit_cast(uint32_t, m_run));
          lds_write_b32_now(lds_l + (w * kDecCols + c16) * 4, __builtin_bit_cast(uint32_t, l_col));
        }
        if (lane == 0) lds_write_b32_now(lds_slot + 4 * w, (uint32_t)rs);
      }
      lgkm_wait_all();
      __builtin_amdgcn_s_barrier();
      {
        constexpr int DPG = D * kDecCols / (64 * NW);
        const int fc = tid & 15, fg = tid >> 4;
        if (fc < P.ncols) {
          uint32_t sl[NW], mw[NW], lw[NW];
          lds_read8_b32(lds_slot, 4, sl);
          lds_read8_b32(lds_m + fc * 4, kDecCols * 4, mw);
          lds_read8_b32(lds_l + fc * 4, kDecCols * 4, lw);
          float M = neg_inf();
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, __builtin_bit_cast(float, mw[ww]));
          float sc[NW];
          float Lsum = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) {
            const float m_w = __builtin_bit_cast(float, mw[ww]);
            sc[ww] = m_w == neg_inf() ? 0.f : exp2_fast(m_w - M);
            Lsum += sc[ww] * __builtin_bit_cast(float, lw[ww]);
          }
          const float inv = Lsum > 0.f ? (KV8 ? v_scale / Lsum : 1.f / Lsum) : 0.f;
          const float lse_v = Lsum > 0.f ? (M + log2_fast(Lsum)) * kLn2 : neg_inf();
          // O^T of wave ww, head_dim d, column fc sits at float
          // ((d / 4) * 16 + fc) * 4 + d % 4 of its merge stage.
          uint32_t oaddr[NW];
#pragma unroll
          for (int ww = 0; ww < NW; ++ww)
            oaddr[ww] = smem_u +
                        (KV8 ? (uint32_t)(ww * 2 * L::stageBytes) + 2 * LAND
                             : (uint32_t)((ww * 2 + (int)sl[ww]) * L::stageBytes)) +
                        ((((fg * DPG) >> 2) * kDecCols + fc) * 4 + ((fg * DPG) & 3)) * 4;
          float o[DPG];
          if constexpr (DPG == 4) {
            u32x4 part[NW];
            lds_read8_b128(oaddr, part);
            // Whole vectors are bit-cast: a bit_cast of one ext-vector
            // element is not reliable with this compiler.
            f32x4 acc = f32x4{};
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) acc += sc[ww] * __builtin_bit_cast(f32x4, part[ww]);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[e] * inv;
          } else {
            u32x2 part[NW];
            lds_read8_b64(oaddr, part);
            f32x2 acc = f32x2{};
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) acc += sc[ww] * __builtin_bit_cast(f32x2, part[ww]);
#pragma unroll
            for (int e = 0; e < 2; ++e) o[e] = acc[e] * inv;
          }
          const int fqi = fc / G;
          const int fhead = P.g * G + (fc - fqi * G);
          const int ftok = P.tok0 + fqi;
          if (P.j0 == 0 && P.j1 == P.nu) {
            uint16_t *op = p.out + ((int64_t)ftok * p.H + fhead) * D + fg * DPG;
            if constexpr (DPG == 4) {
              *reinterpret_cast<u32x2 *>(op) = u32x2{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
            } else {
              *reinterpret_cast<uint32_t *>(op) = pack2_bf16(o[0], o[1]);
            }
            if (fg == 0 && p.lse) p.lse[(int64_t)ftok * p.H + fhead] = lse_v;
          } else {
            float *slot = p.bal_part + (size_t)(2 * wg + P.which) * (kDecCols * (D + 1));
            float *pp = slot + fc * D + fg * DPG;
            if constexpr (DPG == 4) {
              *reinterpret_cast<f32x4 *>(pp) = f32x4{o[0], o[1], o[2], o[3]};
            } else {
              *reinterpret_cast<f32x2 *>(pp) = f32x2{o[0], o[1]};
            }
            if (fg == 0) slot[kDecCols * D + fc] = lse_v;
          }
        }
      }
      lgkm_wait_all();
      __builtin_amdgcn_s_barrier();  // merge stages and m / l / slot entries are free again

      if (!has_next && P.j0 == 0 && P.j1 < P.nu) {
        // This workgroup holds the first unit of a pair that continues into
        // later workgroups: the combine of that pair is its job.
        const int last_unit = P.pair_start + P.nu - 1;
        int wl = (int)(((int64_t)last_unit * nwg) / TU);
        while (wl + 1 < nwg && bal_unit_at(TU, wl + 1, nwg) <= last_unit) ++wl;
        while (wl > 0 && bal_unit_at(TU, wl, nwg) > last_unit) --wl;
        own_b = P.b;
        own_g = P.g;
        own_last = wl;
        own_which = P.which;
      }
      if (!has_next) break;
      cur = cur_next;
      P = N;
      if (pre_n) {
#pragma unroll
        for (int ks = 0; ks < QK; ++ks) qf[ks] = qn[ks];
      }
      slot0 = pslot < 0 ? 0 : pslot;
    }
  }
  if (u0 == u1 && tid < kDecCols) {
    // Empty range: a pair cut around it finds an empty piece in its slot.
    p.bal_part[(size_t)(2 * wg) * (kDecCols * (D + 1)) + kDecCols * D + tid] = neg_inf();
  }
  if (tid == 0) {
    int32_t *dsc = p.bal_desc + wg * kBalDescInts;
    dsc[0] = own_b;
    dsc[1] = own_g;
    dsc[2] = own_last;
    dsc[3] = own_which;
    dsc[4] = TU;
  }
}

template <int D, bool BIAS, bool KV8>
__global__ __launch_bounds__(64 * kBalWaves, 1) void decode_balanced_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[BalLds<D>::bytes];
  decode_balanced<D, BIAS, KV8>(p, smem);
}

// Merges the pieces of the pair recorded by decode workgroup blockIdx.x /
// kBalCombineParts: its own piece, then the first piece of every later
// workgroup up to the one holding the pair's last unit (a workgroup with an
// empty range marks its slot empty).  The pair's outputs are shared by
// kBalCombineParts workgroups, one output per thread; the pieces' weights
// are gathered in LDS first, then each thread has the loads of 16 pieces in
// flight together.  Sums run in piece order, so the result is repeatable.
constexpr int kBalCombineParts = 4;
template <int D>
__global__ __launch_bounds__(kThreads) void combine_balanced_kernel(AttnParams p) {
  __shared__ float wts[kBalMaxWGs][kDecCols];
  __shared__ float red[2][kThreads / 64][kDecCols];
  __shared__ float colM[kDecCols], colW[kDecCols];
  const int wg = blockIdx.x / kBalCombineParts, part = blockIdx.x % kBalCombineParts;
  const int32_t *dsc = p.bal_desc + wg * kBalDescInts;
  const int b = dsc[0];
  if (b < 0) return;
  const int g = dsc[1], w_last = dsc[2], which = dsc[3];
  const int np = w_last - wg + 1;
  const int G = p.G;
  const int tok0 = p.cu_seqlens_q[b];
  const int ncols = (p.cu_seqlens_q[b + 1] - tok0) * G;
  constexpr int SLOT = kDecCols * (D + 1);
  auto slot_of = [&](int i) { return (size_t)(i == 0 ? 2 * wg + which : 2 * (wg + i)) * SLOT; };
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int x = tid; x < np * kDecCols; x += kThreads)
    wts[x / kDecCols][x % kDecCols] = p.bal_part[slot_of(x / kDecCols) + kDecCols * D + x % kDecCols];
  __syncthreads();
  // Column c = tid % 16 is reduced by the 16 threads tid / 16.
  const int c = tid & 15, sub = tid >> 4;
  float M = neg_inf();
  for (int i = sub; i < np; i += kThreads / kDecCols) M = fmaxf(M, wts[i][c]);
  M = fmaxf(M, __shfl_xor(M, 16));
  M = fmaxf(M, __shfl_xor(M, 32));
  if (lane < 16) red[0][wv][c] = M;
  __syncthreads();
#pragma unroll
  for (int ww = 0; ww < kThreads / 64; ++ww) M = fmaxf(M, red[0][ww][c]);
  float W = 0.f;
  if (M != neg_inf()) {
    for (int i = sub; i < np; i += kThreads / kDecCols) {
      const float ls = wts[i][c];
      W += ls == neg_inf() ? 0.f : exp2_fast((ls - M) * kLog2e);
    }
  }
  W += __shfl_xor(W, 16);
  W += __shfl_xor(W, 32);
  if (lane < 16) red[1][wv][c] = W;
  __syncthreads();
  W = 0.f;
#pragma unroll
  for (int ww = 0; ww < kThreads / 64; ++ww) W += red[1][ww][c];
  const float invW = W > 0.f ? 1.f / W : 0.f;
  for (int i = sub; i < np; i += kThreads / kDecCols) {
    const float ls = wts[i][c];
    wts[i][c] = ls == neg_inf() ? 0.f : exp2_fast((ls - M) * kLog2e) * invW;
  }
  if (sub == 0) {
    colM[c] = M;
    colW[c] = W;
  }
  __syncthreads();
  // Outputs of this part: one (column, d) per thread.
  const int n_out = ncols * D;
  const int per = (n_out + kBalCombineParts - 1) / kBalCombineParts;
  for (int oi = part * per + tid; oi < min(n_out, (part + 1) * per); oi += kThreads) {
    const int cc = oi / D, d = oi - cc * D;
    float acc = 0.f;
    for (int i0 = 0; i0 < np; i0 += 16) {
      float v[16], wt[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = min(i0 + u, np - 1);
        wt[u] = i0 + u < np ? wts[i][cc] : 0.f;
        v[u] = p.bal_part[slot_of(i) + cc * D + d];
      }
      // An empty piece has weight 0 and may hold anything: select, not scale.
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += wt[u] != 0.f ? wt[u] * v[u] : 0.f;
    }
    const int fqi = cc / G;
    const int fhead = g * G + (cc - fqi * G);
    const int ftok = tok0 + fqi;
    p.out[((int64_t)ftok * p.H + fhead) * D + d] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    if (d == 0 && p.lse) {
      const float Mc = colM[cc], Wc = colW[cc];
      p.lse[(int64_t)ftok * p.H + fhead] = Mc == neg_inf() ? neg_inf() : Mc + log2_fast(Wc) * kLn2;
    }
  }
}

// ------------------------------------- balanced decode, kv heads in parallel
//
// The same balance for batches with eight kv heads, but a unit is a 16-key
// block of a request over all eight heads: units run in (request, key)
// order, workgroup x of W takes units [x*TU/W, (x+1)*TU/W), and wave w
// streams kv head w over them.  The waves of a workgroup read the same
// tokens, so together they fetch whole token rows of the cache (all heads,
// 2 KB for head_dim 128) instead of one head's 256-byte slice.  Waves never
// merge: each finishes its head of a piece (the part of one request inside
// the range) on its own, with the output when the piece is the whole
// request, else with a normalised partial in its head's entry of the
// piece's slot; the workgroup holding a cut request's first unit records it
// for combine_heads_kernel.  Per unit and wave the loads, LDS layout and
// arithmetic are those of decode_balanced.

template <int D, bool BIAS, bool KV8>
__device__ void decode_heads(const AttnParams &p, char *smem) {
  using L = BalLds<D>;
  constexpr int QK = D / 32, DB = D / 16, NI = L::NI, RPI = L::RPI, UNITS = L::UNITS, ROWB = L::ROWB;
  static_assert(L::NST == 2, "two stages per wave: one computed, one in flight");
  static_assert(kBalWaves == kBalHeads, "one wave per kv head");
  // E4M3 caches: a stage is the unit's raw rows (K then V, D bytes a row);
  // K operands are decoded from it, V is decoded into one bf16 V stage per
  // wave that the transposing reads use.
  constexpr int U8 = D / 16, RPI8 = 64 / U8, NI8 = 16 / RPI8;
  constexpr uint32_t LAND = 32 * D;
  static_assert(!KV8 || 2 * LAND + L::halfBytes <= 2 * L::stageBytes, "fp8 stages fit the wave's region");
  constexpr int NLD = KV8 ? NI8 : NI;
  constexpr int NPER = 2 * NLD + (BIAS ? 4 : 0);  // vector-memory instructions per unit
  constexpr int SLOT = kDecCols * (D + 1);
  int32_t *prefix = reinterpret_cast<int32_t *>(smem + L::prefixOff);
  bal_prefix(p, prefix, reinterpret_cast<int32_t *>(smem + L::mlOff), 1);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = w;  // this wave's kv head
  const int c16 = lane & 15, q = lane >> 4;
  const int B = p.batch, G = p.G;
  const int nwg = p.bal_wgs, wg = blockIdx.x;
  const int TU = __builtin_amdgcn_readfirstlane(prefix[B]);
  const int u0 = bal_unit_at(TU, wg, nwg), u1 = bal_unit_at(TU, wg + 1, nwg);
  int b_it = 0;
  {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= u0) lo = mid;
      else hi = mid - 1;
    }
    b_it = __builtin_amdgcn_readfirstlane(lo);
  }

  const uint32_t slot_bytes = (uint32_t)kBalHeads * D * (KV8 ? 1 : 2);
  uint32_t gk[NLD], gv[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    if constexpr (KV8) {
      // Raw K rows: piece pu of row r lands at (pu ^ (r % U8)) so that the
      // 16 rows of an operand read spread over the banks.
      const int r = RPI8 * n + lane / U8, pu = lane % U8;
      gk[n] = r * slot_bytes + ((pu ^ (r & (U8 - 1))) << 4);
      gv[n] = r * slot_bytes + (pu << 4);
    } else {
      const int r = RPI * n + lane / UNITS, pu = lane % UNITS;
      gk[n] = r * slot_bytes + ((pu ^ swz_k<D>(r)) << 4);
      gv[n] = r * slot_bytes + ((pu ^ swz_vt<D>(r)) << 4);
    }
  }
  uint32_t lk_off[QK], lv_off[DB];
#pragma unroll
  for (int ks = 0; ks < QK; ++ks) {
    if constexpr (KV8)
      lk_off[ks] = c16 * D + (((2 * ks + (q >> 1)) ^ (c16 & (U8 - 1))) << 4) + 8 * (q & 1);
    else
      lk_off[ks] = c16 * ROWB + (((4 * ks + q) ^ swz_k<D>(c16)) << 4);
  }
  // fp8: where this lane's decoded V pieces go in the bf16 V stage.
  uint32_t v8_dst[KV8 ? 2 * NI8 : 1];
  // E4M3: offset, inside a raw block, of the raw V unit this lane decodes.
  const uint32_t v8_src = (uint32_t)(16 * (D == 128 ? U8 * v8_row_of(lane) + lane % U8 : lane));
  if constexpr (KV8) {
#pragma unroll
    for (int n = 0; n < NI8; ++n) {
      const int r = RPI8 * n + (D == 128 ? v8_row_of(lane) : lane / U8), pu = lane % U8;
#pragma unroll
      for (int e = 0; e < 2; ++e) v8_dst[2 * n + e] = r * ROWB + (((2 * pu + e) ^ swz_vt<D>(r)) << 4);
    }
  }
  {
    const int i = (lane & 15) >> 2, t = lane & 3, row = 4 * q + i;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      lv_off[db] = L::halfBytes + row * ROWB + ((((2 * db + (t >> 1)) ^ swz_vt<D>(row)) << 4)) + 8 * (t & 1);
  }
  const uint32_t smem_u = (uint32_t)(uintptr_t)smem;
  const uint32_t lds_wave = smem_u + (uint32_t)(w * 2 * L::stageBytes);
  const uint32_t lds_bias = smem_u + (uint32_t)(L::biasOff + w * 2 * 1024 + 4 * lane);
  const uint32_t lds_prefix = smem_u + L::prefixOff;
  const float c = p.scale_log2;
  const bool pos_scale = c > 0.f;
  // bf16 rel_logits: each lane loads the dword holding its element (the
  // range rounded up to whole dwords; a page never ends inside one) and
  // compute() keeps the element's half.
  const bool rel_bf16 = p.rel_bf16 != 0;
  const uint32_t bias_bytes =
      BIAS ? (rel_bf16 ? ((uint32_t)p.num_tokens * (uint32_t)p.H * (uint32_t)p.R * 2u + 3u) & ~3u
                       : (uint32_t)p.num_tokens * (uint32_t)p.H * (uint32_t)p.R * 4u)
           : 0u;
  const float v_scale = KV8 ? p.v_scale : 1.f;
  const bool alibi = p.alibi != nullptr;

  // A piece: units [j0, j1) of request b inside this workgroup's range,
  // with what its rows need (uniform fields, then the lane's column).
  struct Piece {
    int b, j0, j1, nu, which, pair_start;
    int tok0, lq, ncols, lo_a, kend, in_lo, in_hi, band_lo, band_hi, n;
    int qa, lo_c, hi_c, tok, head;
    uint32_t rel_base;
    float al;  // ALiBi slope of the lane's head times log2(e), or 0
  };
  auto prefix_at = [&](int i) { return __builtin_amdgcn_readfirstlane(lds_read_i32_now(lds_prefix + 4u * i)); };
  auto make_piece = [&](int cur) __attribute__((always_inline)) {
    Piece P;
    while (prefix_at(b_it + 1) <= cur) ++b_it;
    P.b = b_it;
    P.pair_start = prefix_at(b_it);
    P.nu = prefix_at(b_it + 1) - P.pair_start;
    P.j0 = cur - P.pair_start;
    P.j1 = min(P.nu, P.j0 + (u1 - cur));
    P.n = P.j1 - P.j0;
    P.which = cur == u0 ? 0 : 1;
    P.tok0 = scalar_load_i32(p.cu_seqlens_q + P.b);
    P.lq = scalar_load_i32(p.cu_seqlens_q + P.b + 1) - P.tok0;
    const int lk = scalar_load_i32(p.cache_seqlens + P.b);
    P.ncols = P.lq * G;
    const int col = c16 < P.ncols ? c16 : P.ncols - 1;
    const int qi = col / G;
    P.head = g * G + (col - qi * G);
    P.tok = P.tok0 + qi;
    P.qa = qi + lk - P.lq;
    const int qa_min = lk - P.lq, qa_max = lk - 1;
    const Range vr = visible_range(p, lk, qa_min, qa_max);
    P.lo_a = vr.lo & ~15;
    P.kend = min(lk, vr.hi);
    P.lo_c = P.lo_a;
    P.hi_c = P.kend - 1;
    if (p.left >= 0) P.lo_c = max(P.lo_c, P.qa - p.left);
    if (p.causal) P.hi_c = min(P.hi_c, P.qa);
    if (p.right >= 0) P.hi_c = min(P.hi_c, P.qa + p.right);
    P.in_lo = P.lo_a;
    P.in_hi = P.kend - 1;
    if (p.left >= 0) P.in_lo = max(P.in_lo, qa_max - p.left);
    if (p.causal) P.in_hi = min(P.in_hi, qa_min);
    if (p.right >= 0) P.in_hi = min(P.in_hi, qa_min + p.right);
    P.band_lo = qa_min - p.R + 1;
    P.band_hi = qa_max;
    P.rel_base = BIAS ? (uint32_t)((P.tok * p.H + P.head) * p.R) : 0u;
    P.al = alibi ? p.alibi[P.head] * kLog2e : 0.f;
    return P;
  };
  auto key_of = [&](const Piece &P, int k) { return P.lo_a + 16 * (P.j0 + k); };
  auto in_band = [&](const Piece &P, int key0) { return BIAS && key0 <= P.band_hi && key0 + 15 >= P.band_lo; };
  auto page_of = [&](const Piece &P, int k) -> int {
    const int key = key_of(P, k);
    if (k >= P.n || key >= P.kend) return 0;
    return scalar_load_i32(p.block_table + (int64_t)P.b * p.P + (p.bs_shift >= 0 ? (key >> p.bs_shift) : key / p.BS));
  };
  auto load_q = [&](const Piece &P, bf16x8 (&qf)[QK]) __attribute__((always_inline)) {
    const uint16_t *qp = p.q + ((int64_t)P.tok * p.H + P.head) * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < QK; ++ks) qf[ks] = as_bf16x8(ld16(qp + 32 * ks));
  };
  auto issue = [&](const Piece &P, int k, int page, int slot) __attribute__((always_inline)) {
    const int key0 = __builtin_amdgcn_readfirstlane(key_of(P, k));
    const int nvalid = __builtin_amdgcn_readfirstlane(min(max(P.kend - key0, 0), 16));
    const int slot0 = p.bs_shift >= 0 ? (key0 & (p.BS - 1)) : key0 % p.BS;
    const int64_t eoff = (((int64_t)page * p.BS + slot0) * kBalHeads + g) * D;
    const auto rk = make_rsrc(reinterpret_cast<const char *>(p.k) + eoff * (KV8 ? 1 : 2), (uint32_t)nvalid * slot_bytes);
    const auto rv = make_rsrc(reinterpret_cast<const char *>(p.v) + eoff * (KV8 ? 1 : 2), (uint32_t)nvalid * slot_bytes);
    if constexpr (BIAS) {
      const auto brs = make_rsrc(p.rel_logits, in_band(P, key0) ? bias_bytes : 0u);
      char *bst = smem + L::biasOff + (w * 2 + slot) * 1024;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = min(max(P.qa - (key0 + 4 * q + j), 0), p.R - 1);
        const uint32_t boff = rel_bf16 ? ((P.rel_base + (uint32_t)d) * 2u) & ~3u : (P.rel_base + (uint32_t)d) * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (__attribute__((address_space(3))) void *)(bst + 256 * j), 4,
                                                 boff, 0, 0, 0);
      }
    }
    char *st = KV8 ? smem + w * 2 * L::stageBytes + slot * LAND : smem + (w * 2 + slot) * L::stageBytes;
    constexpr int VHALF = KV8 ? 16 * D : L::halfBytes;
#pragma unroll
    for (int n = 0; n < NLD; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void *)(st + n * 1024), 16,
                                               gk[n], 0, 0, kNonTemporal);
#pragma unroll
    for (int n = 0; n < NLD; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void *)(st + VHALF + n * 1024), 16, gv[n], 0, 0, kNonTemporal);
  };

  f32x4 oacc[DB];
  float m_run, l_run;
  auto compute = [&](const Piece &P, int k, int slot, const bf16x8 (&qf)[QK]) __attribute__((always_inline)) {
    const int key0 = __builtin_amdgcn_readfirstlane(key_of(P, k));
    u32x4 kf[QK];
    u32x2 va[DB];
    if constexpr (KV8) {
      // Raw rows of the unit: K operands decoded in registers; this lane's
      // V pieces decoded into the bf16 V stage, then read transposed.
      const uint32_t land = lds_wave + slot * LAND;
      const uint32_t vst = lds_wave + 2 * LAND;
      u32x2 k8[QK];
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) k8[ks] = lds_read_b64_asm(land + lk_off[ks]);
      u32x4 v8[NI8];
#pragma unroll
      for (int n = 0; n < NI8; ++n) v8[n] = lds_read_b128_asm(land + 16 * D + n * 1024 + v8_src);
      lgkm_wait_n<0>(v8);
      lgkm_wait_n<0>(k8);
      if constexpr (NI8 == 2) {
        const uint32_t a[4] = {vst + v8_dst[0], vst + v8_dst[1], vst + v8_dst[2], vst + v8_dst[3]};
        const u32x4 vv[4] = {e4m3x8_to_bf16(v8[0][0], v8[0][1]), e4m3x8_to_bf16(v8[0][2], v8[0][3]),
                             e4m3x8_to_bf16(v8[1][0], v8[1][1]), e4m3x8_to_bf16(v8[1][2], v8[1][3])};
        lds_write_b128x4_now(a, vv);
      } else {
        lds_write_b128x2_now(vst + v8_dst[0], vst + v8_dst[1], e4m3x8_to_bf16(v8[0][0], v8[0][1]),
                             e4m3x8_to_bf16(v8[0][2], v8[0][3]));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = lds_read_tr_at(vst - L::halfBytes + lv_off[db]);
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) kf[ks] = e4m3x8_to_bf16(k8[ks][0], k8[ks][1]);
    } else {
      const uint32_t st = lds_wave + slot * L::stageBytes;
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) kf[ks] = lds_read_b128_asm(st + lk_off[ks]);
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = lds_read_tr_at(st + lv_off[db]);
      lgkm_wait_n<DB>(kf);
    }
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < QK; ++ks) sacc = mfma16(as_bf16x8(kf[ks]), qf[ks], sacc);
    const bool interior = key0 >= P.in_lo && key0 + 15 <= P.in_hi;
    const bool band = in_band(P, key0);
    const bool plain = interior && !band && !alibi;
    float mx = neg_inf();
    if (plain) {
      if (pos_scale) {
        mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3])) * c;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sacc[j] * c);
      }
    } else {
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if (band) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bias[j] = lds_read_f32_asm(lds_bias + slot * 1024 + 256 * j);
        lgkm_wait_n<0>(bias);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = key0 + 4 * q + j;
        float v = sacc[j] * c;
        if (band && (unsigned)(P.qa - t) < (unsigned)p.R) {
          float bv = bias[j];
          if (rel_bf16) {
            const uint32_t bits = __float_as_uint(bv);
            bv = __uint_as_float(((P.rel_base + (uint32_t)(P.qa - t)) & 1u) ? (bits & 0xffff0000u) : (bits << 16));
          }
          v = __builtin_fmaf(bv, kLog2e, v);
        }
        if (alibi) v = __builtin_fmaf(P.al, (float)(t - P.qa), v);
        if (t < P.lo_c || t > P.hi_c) v = neg_inf();
        sacc[j] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    if (__any(mx > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == neg_inf() ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float m_use = m_run == neg_inf() ? 0.f : m_run;
    float pe[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pe[j] = exp2_fast(plain ? __builtin_fmaf(sacc[j], c, -m_use) : sacc[j] - m_use);
    l_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
    const u32x2 pf = u32x2{pack2_bf16(pe[0], pe[1]), pack2_bf16(pe[2], pe[3])};
    lgkm_wait_n<0>(va);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = mfma16k16(va[db], pf, oacc[db]);
  };
  // Lane (c16, q) holds O^T[16 db + 4 q + e][column c16] in oacc[db][e];
  // the column's l is spread over its four q lanes.
  auto finish_piece = [&](const Piece &P) __attribute__((always_inline)) {
    const float l_col = xor32_sum(xor16_sum(l_run));
    const float inv = l_col > 0.f ? (KV8 ? v_scale / l_col : 1.f / l_col) : 0.f;
    const float lse_v = l_col > 0.f ? (m_run + log2_fast(l_col)) * kLn2 : neg_inf();
    if (c16 >= P.ncols) return;
    if (P.j0 == 0 && P.j1 == P.nu) {
      uint16_t *op = p.out + ((int64_t)P.tok * p.H + P.head) * D + 4 * q;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<u32x2 *>(op + 16 * db) =
            u32x2{pack2_bf16(oacc[db][0] * inv, oacc[db][1] * inv), pack2_bf16(oacc[db][2] * inv, oacc[db][3] * inv)};
      if (q == 0 && p.lse) p.lse[(int64_t)P.tok * p.H + P.head] = lse_v;
    } else {
      float *slot = p.bal_part + ((size_t)(2 * wg + P.which) * kBalHeads + g) * SLOT;
      float *pp = slot + c16 * D + 4 * q;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4 *>(pp + 16 * db) = oacc[db] * inv;
      if (q == 0) slot[kDecCols * D + c16] = lse_v;
    }
  };

  int own_b = -1, own_ncols = 0, own_last = 0, own_which = 0;
  int cur = u0;
  if (cur < u1) {
    Piece P = make_piece(cur);
    bf16x8 qf[QK];
    // The first unit's loads go out before Q's, so that the two latencies
    // overlap; the wait before the first unit is computed covers both.
    int slot = 0;  // stage of the next unit to compute
    issue(P, 0, page_of(P, 0), 0);
    load_q(P, qf);
    while (true) {
      const int cur_next = cur + P.n;
      const bool has_next = cur_next < u1;
      Piece N;
      int page_n0 = 0;
      if (has_next) {
        N = make_piece(cur_next);
        page_n0 = page_of(N, 0);
      }
      int page_nx = page_of(P, 1);
      bf16x8 qn[QK];
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};
      m_run = neg_inf();
      l_run = 0.f;
      // While unit k is computed the next unit of the wave's stream is in
      // flight: unit k+1 of P or, after P's last, unit 0 of the next piece
      // (this wave's head of the next request).
      for (int k = 0; k < P.n; ++k) {
        if (k + 1 < P.n) {
          issue(P, k + 1, page_nx, slot ^ 1);
          page_nx = page_of(P, k + 2);
          wait_vm<NPER>();
        } else if (has_next) {
          load_q(N, qn);
          issue(N, 0, page_n0, slot ^ 1);
          wait_vm<NPER>();
        } else {
          wait_vm<0>();
        }
        compute(P, k, slot, qf);
        slot ^= 1;
      }
      finish_piece(P);
      if (!has_next && P.j0 == 0 && P.j1 < P.nu) {
        // This workgroup holds the first unit of a request that continues
        // into later workgroups: the combine of its heads is its job.
        const int last_unit = P.pair_start + P.nu - 1;
        int wl = (int)(((int64_t)last_unit * nwg) / TU);
        while (wl + 1 < nwg && bal_unit_at(TU, wl + 1, nwg) <= last_unit) ++wl;
        while (wl > 0 && bal_unit_at(TU, wl, nwg) > last_unit) --wl;
        own_b = P.b;
        own_ncols = P.ncols;
        own_last = wl;
        own_which = P.which;
      }
      if (!has_next) break;
      cur = cur_next;
      P = N;
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) qf[ks] = qn[ks];
    }
  }
  if (u0 == u1 && tid < kBalHeads * kDecCols) {
    // Empty range: a request cut around it finds empty pieces in its slot.
    p.bal_part[((size_t)(2 * wg) * kBalHeads + tid / kDecCols) * SLOT + kDecCols * D + tid % kDecCols] = neg_inf();
  }
  if (tid == 0) {
    int32_t *dsc = p.bal_desc + wg * kBalDescInts;
    dsc[0] = own_b;
    dsc[1] = own_ncols;
    dsc[2] = own_last;
    dsc[3] = own_which;
    dsc[4] = TU;
  }
}

template <int D, bool BIAS, bool KV8>
__global__ __launch_bounds__(64 * kBalWaves, 1) void decode_heads_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[BalLds<D>::bytes];
  decode_heads<D, BIAS, KV8>(p, smem);
}

// Combine of the requests cut by decode_heads.  A task is (recording
// workgroup x, kv head, column, block of head_dim values) and takes one
// wave: the pieces' LSEs and the first 16 pieces of each lane's group are
// loaded together, the weights exp(lse_i - LSE) go to LDS, and lane
// (piece group, d) sums every PG-th piece for one d; the piece groups are
// added by shuffles.  PG grows with the piece count (1 up to 16 pieces,
// then up to 16 groups) so that long requests spread over many waves.
// Tasks are numbered over the recording workgroups in order; every
// workgroup scans the records (request, column count, last workgroup).
template <int D>
__global__ __launch_bounds__(kThreads) void combine_heads_kernel(AttnParams p) {
  constexpr int SLOT = kDecCols * (D + 1);
  constexpr int NWV = kThreads / 64;
  __shared__ int tpre[kBalMaxWGs + 1];
  __shared__ int wpart[NWV];
  __shared__ float wts[NWV][kBalMaxWGs];
  const int nwg = p.bal_wgs, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // Piece groups of a record: log2 PG with PG = pow2ceil(np / 16) in [1, 16].
  auto lg_pg = [&](int np) {
    int lg = 0;
    while (lg < 4 && (16 << lg) < np) ++lg;
    return lg;
  };
  auto tasks_of = [&](int x) {
    if (x >= nwg) return 0;
    const int32_t *dsc = p.bal_desc + x * kBalDescInts;
    if (dsc[0] < 0) return 0;
    const int dl_bits = 6 - lg_pg(dsc[2] - x + 1);
    return kBalHeads * dsc[1] * max(D >> dl_bits, 1);
  };
  // Exclusive prefix of the task counts over records (two per thread).
  const int n0 = tasks_of(2 * tid), n1 = tasks_of(2 * tid + 1);
  int incl = n0 + n1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wpart[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int ww = 0; ww < wv; ++ww) base += wpart[ww];
  const int ex = base + incl - n0 - n1;
  if (2 * tid < kBalMaxWGs) tpre[2 * tid] = ex;
  if (2 * tid + 1 < kBalMaxWGs) tpre[2 * tid + 1] = ex + n0;
  if (tid == kThreads - 1) tpre[kBalMaxWGs] = ex + n0 + n1;
  __syncthreads();
  const int total = tpre[kBalMaxWGs];
  for (int task = blockIdx.x * NWV + wv; task < total; task += gridDim.x * NWV) {
    int lo = 0, hi = kBalMaxWGs - 1;  // the last record x with tpre[x] <= task
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tpre[mid] <= task) lo = mid;
      else hi = mid - 1;
    }
    const int x = __builtin_amdgcn_readfirstlane(lo);
    const int32_t *dsc = p.bal_desc + x * kBalDescInts;
    const int b = dsc[0], ncols = dsc[1], w_last = dsc[2], which = dsc[3];
    const int np = w_last - x + 1;
    const int tok0 = p.cu_seqlens_q[b];
    const int lg = lg_pg(np), dl_bits = 6 - lg;
    const int nch = max(D >> dl_bits, 1);
    const int rem = task - tpre[x];
    const int g = rem / (ncols * nch);
    const int rem2 = rem - g * ncols * nch;
    const int cc = rem2 / nch, ch = rem2 - cc * nch;
    auto slot_of = [&](int i) {
      return ((size_t)(i == 0 ? 2 * x + which : 2 * (x + i)) * kBalHeads + g) * SLOT;
    };
    const int pg = lane >> dl_bits, dl = lane & ((1 << dl_bits) - 1);
    const int d = (ch << dl_bits) + dl;
    const int PG = 1 << lg;
    // The pieces' LSEs (lane i holds pieces i, i + 64, ...) and the first
    // 16 pieces of this lane's group are loaded together.
    float ls[kBalMaxWGs / 64], v[16];
#pragma unroll
    for (int u = 0; u < kBalMaxWGs / 64; ++u) {
      const int i = lane + 64 * u;
      ls[u] = i < np ? p.bal_part[slot_of(i) + kDecCols * D + cc] : neg_inf();
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = pg + u * PG;
      v[u] = i < np && d < D ? p.bal_part[slot_of(i) + cc * D + d] : 0.f;
    }
    float M = neg_inf();
#pragma unroll
    for (int u = 0; u < kBalMaxWGs / 64; ++u) M = fmaxf(M, ls[u]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float W = 0.f;
#pragma unroll
    for (int u = 0; u < kBalMaxWGs / 64; ++u) {
      const int i = lane + 64 * u;
      const float e = (M == neg_inf() || ls[u] == neg_inf()) ? 0.f : exp2_fast((ls[u] - M) * kLog2e);
      if (i < np) wts[wv][i] = e;
      W += e;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
    wave_lds_sync();
    // An empty piece has weight 0 and may hold anything: select, not scale.
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = pg + u * PG;
      const float wt = i < np ? wts[wv][i] : 0.f;
      acc += wt != 0.f ? wt * v[u] : 0.f;
    }
    if (d < D) {
      for (int i0 = pg + 16 * PG; i0 < np; i0 += 8 * PG) {
        float wt[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * PG;
          wt[u] = i < np ? wts[wv][i] : 0.f;
          v[u] = i < np ? p.bal_part[slot_of(i) + cc * D + d] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += wt[u] != 0.f ? wt[u] * v[u] : 0.f;
      }
    }
    for (int bit = dl_bits; bit < 6; ++bit) acc += __shfl_xor(acc, 1 << bit);
    wave_lds_sync();  // wts[wv] is rewritten by the next task
    if (pg == 0 && d < D) {
      const int fqi = cc / p.G;
      const int fhead = g * p.G + (cc - fqi * p.G);
      const int ftok = tok0 + fqi;
      const float invW = W > 0.f ? 1.f / W : 0.f;
      p.out[((int64_t)ftok * p.H + fhead) * D + d] = __builtin_bit_cast(uint16_t, (__bf16)(acc * invW));
      if (d == 0 && p.lse) p.lse[(int64_t)ftok * p.H + fhead] = M == neg_inf() ? neg_inf() : M + log2_fast(W) * kLn2;
    }
  }
}

// ---------------------------------------------------------------- combine

// One row (token, head) per p.wr waves of a workgroup (one, two or four:
// more when there are many splits, so that few rows with many partials
// still spread over many waves).  Every wave of a row reduces all S LSEs to
// the weights exp(lse_s - LSE); wave `sub` of the row sums the normalised
// partials of its slice of the splits, and the slices are added through LDS.
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  __shared__ float wts[4][128];
  __shared__ float part[4][256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int WR = p.wr, sub = w % WR;
  const int row = blockIdx.x * (4 / WR) + w / WR;
  const bool live = row < p.rows;
  const int S = p.S, D = p.D;
  const float l0 = live && lane < S ? p.part_lse[(int64_t)lane * p.rows + row] : neg_inf();
  const float l1 = live && lane + 64 < S ? p.part_lse[(int64_t)(lane + 64) * p.rows + row] : neg_inf();
  float M = fmaxf(l0, l1);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float e0 = l0 == neg_inf() ? 0.f : exp2_fast((l0 - M) * kLog2e);
  const float e1 = l1 == neg_inf() ? 0.f : exp2_fast((l1 - M) * kLog2e);
  float W = e0 + e1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) W += __shfl_xor(W, o);
  const float invW = W > 0.f ? 1.f / W : 0.f;
  wts[w][lane] = e0 * invW;
  wts[w][lane + 64] = e1 * invW;
  wave_lds_sync();
  // A split with weight 0 (an empty chunk, lse = -inf, or one whose weight
  // underflows) is skipped, not multiplied: its partial may hold anything,
  // NaN included, without reaching the output.
  const int s0 = sub * S / WR, s1 = (sub + 1) * S / WR;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (live && M != neg_inf()) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = lane + 64 * k;
      if (d >= D) break;
      const float *src = p.part_out + (int64_t)row * D + d;
#pragma unroll 8
      for (int s = s0; s < s1; ++s) {
        const float wt = wts[w][s];
        const float v = src[(int64_t)s * p.rows * D];
        acc[k] += wt != 0.f ? wt * v : 0.f;
      }
    }
  }
  if (WR > 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (lane + 64 * k < D) part[w][lane + 64 * k] = acc[k];
    __syncthreads();
    if (sub == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        for (int ww = 1; ww < WR; ++ww)
          if (lane + 64 * k < D) acc[k] += part[w + ww][lane + 64 * k];
    }
  }
  if (!live || sub != 0) return;
  uint16_t *op = p.out + (int64_t)row * D;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (lane + 64 * k < D) op[lane + 64 * k] = __builtin_bit_cast(uint16_t, (__bf16)acc[k]);
  if (lane == 0 && p.lse) p.lse[row] = M == neg_inf() ? neg_inf() : M + log2_fast(W) * kLn2;
}

// ------------------------------------------------------- paged KV write
//
// The step before attention ("vLLM V1 Attention — Part 2", 附录O.1 Step 2
// and 6.5 step 2): each new token's cache slot, and the copy of its key
// and value rows into the pages.

// One thread per token: its request is the last b with cu_seqlens_q[b] <=
// token (empty requests share their start with the next one).
__global__ __launch_bounds__(kThreads) void slot_mapping_kernel(SlotParams p) {
  const int tok = blockIdx.x * kThreads + threadIdx.x;
  if (tok >= p.num_tokens) return;
  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu_seqlens_q[mid] <= tok) lo = mid;
    else hi = mid - 1;
  }
  const int c0 = p.cu_seqlens_q[lo];
  const int lq = p.cu_seqlens_q[lo + 1] - c0;
  const int pos = p.cache_seqlens[lo] - lq + (tok - c0);
  int64_t slot = -1;
  if (pos >= 0) slot = (int64_t)p.block_table[(int64_t)lo * p.P + pos / p.BS] * p.BS + pos % p.BS;
  p.slots[tok] = slot;
}

// One wave per token at a time: the token's key and value rows (row_units
// 16-byte units each) are copied to row `slot` of the caches, which is
// contiguous in the [blocks, block_size, kv heads, head_dim] layout.  Every
// lane has its units of both rows in flight before any store.
__global__ __launch_bounds__(kThreads) void kv_write_kernel(KvWriteParams p) {
  const int lane = threadIdx.x & 63;
  const int nwave = gridDim.x * (kThreads / 64);
  const int n = p.row_units;
  for (int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); t < p.num_tokens; t += nwave) {
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.capacity) continue;
    const u32x4 *sk = reinterpret_cast<const u32x4 *>(p.key) + (int64_t)t * n;
    const u32x4 *sv = reinterpret_cast<const u32x4 *>(p.value) + (int64_t)t * n;
    u32x4 *dk = reinterpret_cast<u32x4 *>(p.key_cache) + slot * n;
    u32x4 *dv = reinterpret_cast<u32x4 *>(p.value_cache) + slot * n;
    int c = lane;
    for (; c + 64 < n; c += 128) {
      const u32x4 k0 = sk[c], k1 = sk[c + 64], v0 = sv[c], v1 = sv[c + 64];
      dk[c] = k0;
      dk[c + 64] = k1;
      dv[c] = v0;
      dv[c + 64] = v1;
    }
    if (c < n) {
      const u32x4 k0 = sk[c], v0 = sv[c];
      dk[c] = k0;
      dv[c] = v0;
    }
  }
}

// E4M3 (OCP) code of an fp32 value: nearest value, ties to the even code;
// magnitudes of 448 and above (infinity included) saturate to 448; NaN
// gives a NaN code with the value's sign.  Normal results round the fp32
// mantissa to 3 bits (the carry may raise the exponent); below 2^-6 the
// code is |y| * 2^9 rounded to an integer (0..8, where 8 is 2^-6).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;
  if (a >= 0x3c800000u) {
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    return sign | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
  }
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

// Eight bf16 values (one 16-byte unit) to eight E4M3 codes of x / scale.
__device__ __forceinline__ u32x2 quant8_e4m3(u32x4 x, float scale) {
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = e4m3_code(__fdiv_rn(__uint_as_float(x[i] << 16), scale));
    c[2 * i + 1] = e4m3_code(__fdiv_rn(__uint_as_float(x[i] & 0xffff0000u), scale));
  }
  return u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
}

// kv_write_kernel for E4M3 caches: each 16-byte unit of a bf16 row becomes
// 8 bytes of codes at the same element offsets of the slot's row.
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(KvWriteParams p) {
  const int lane = threadIdx.x & 63;
  const int nwave = gridDim.x * (kThreads / 64);
  const int n = p.row_units;
  for (int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); t < p.num_tokens; t += nwave) {
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.capacity) continue;
    const u32x4 *sk = reinterpret_cast<const u32x4 *>(p.key) + (int64_t)t * n;
    const u32x4 *sv = reinterpret_cast<const u32x4 *>(p.value) + (int64_t)t * n;
    u32x2 *dk = reinterpret_cast<u32x2 *>(p.key_cache) + slot * n;
    u32x2 *dv = reinterpret_cast<u32x2 *>(p.value_cache) + slot * n;
    for (int c = lane; c < n; c += 64) {
      const u32x4 k0 = sk[c], v0 = sv[c];
      dk[c] = quant8_e4m3(k0, p.k_scale);
      dv[c] = quant8_e4m3(v0, p.v_scale);
    }
  }
}

}  // namespace

hipError_t launch_kv_write_fp8(const KvWriteParams &p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  const int64_t wgs = ((int64_t)p.num_tokens + kThreads / 64 - 1) / (kThreads / 64);
  const dim3 grid((unsigned)(wgs < 2048 ? wgs : 2048)), block(kThreads);
  hipLaunchKernelGGL(kv_write_fp8_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const SlotParams &p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.num_tokens + kThreads - 1) / kThreads)), block(kThreads);
  hipLaunchKernelGGL(slot_mapping_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteParams &p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  // One wave per token up to 2048 workgroups (8 per CU); beyond that the
  // waves loop over the tokens.
  const int64_t wgs = ((int64_t)p.num_tokens + kThreads / 64 - 1) / (kThreads / 64);
  const dim3 grid((unsigned)(wgs < 2048 ? wgs : 2048)), block(kThreads);
  hipLaunchKernelGGL(kv_write_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams &p, int head_dim, int64_t n_items_ub, bool decode_only,
                            hipStream_t stream) {
  const int64_t blocks = n_items_ub * p.Hkv * p.S;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  auto go = [&](auto d_tag, auto dec_tag, auto k_tag, auto f_tag) {
    const dim3 block(64 * attn_waves<decltype(dec_tag)::value>());
    hipLaunchKernelGGL((attn_kernel<decltype(d_tag)::value, decltype(dec_tag)::value, decltype(k_tag)::value,
                                    decltype(f_tag)::value>),
                       grid, block, 0, stream, p);
  };
  auto go_k = [&](auto d_tag, auto k_tag) {
    using T_ = std::true_type;
    using F_ = std::false_type;
    using I = std::integral_constant<int, 0>;
    if (decode_only) return go(d_tag, T_{}, k_tag, I{});
    const int feat = (p.alibi ? kFeatAlibi : 0) | (p.rel_bf16 ? kFeatRelBf16 : 0);
    switch (feat) {
      case 0: go(d_tag, F_{}, k_tag, std::integral_constant<int, 0>{}); break;
      case 1: go(d_tag, F_{}, k_tag, std::integral_constant<int, 1>{}); break;
      case 2: go(d_tag, F_{}, k_tag, std::integral_constant<int, 2>{}); break;
      default: go(d_tag, F_{}, k_tag, std::integral_constant<int, 3>{}); break;
    }
  };
  auto go_d = [&](auto d_tag) {
    if (p.kv8) go_k(d_tag, std::true_type{});
    else go_k(d_tag, std::false_type{});
  };
  if (head_dim == 128) go_d(std::integral_constant<int, 128>{});
  else go_d(std::integral_constant<int, 64>{});
  return hipGetLastError();
}

hipError_t launch_balanced_decode(const AttnParams &p, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)p.bal_wgs), block(64 * kBalWaves), cgrid((unsigned)(p.bal_wgs * kBalCombineParts)),
      cblock(kThreads);
  const bool bias = p.R > 0;
  if (p.Hkv == kBalHeads) {
    const dim3 hgrid((unsigned)(p.bal_wgs * 2));
    auto heads = [&](auto d_tag, auto b_tag, auto k_tag) {
      hipLaunchKernelGGL((decode_heads_kernel<decltype(d_tag)::value, decltype(b_tag)::value,
                                              decltype(k_tag)::value>),
                         grid, block, 0, stream, p);
    };
    using D128 = std::integral_constant<int, 128>;
    using D64 = std::integral_constant<int, 64>;
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (head_dim == 128) {
      if (p.kv8) bias ? heads(D128{}, T_{}, T_{}) : heads(D128{}, F_{}, T_{});
      else bias ? heads(D128{}, T_{}, F_{}) : heads(D128{}, F_{}, F_{});
      hipLaunchKernelGGL((combine_heads_kernel<128>), hgrid, cblock, 0, stream, p);
    } else {
      if (p.kv8) bias ? heads(D64{}, T_{}, T_{}) : heads(D64{}, F_{}, T_{});
      else bias ? heads(D64{}, T_{}, F_{}) : heads(D64{}, F_{}, F_{});
      hipLaunchKernelGGL((combine_heads_kernel<64>), hgrid, cblock, 0, stream, p);
    }
    return hipGetLastError();
  }
  auto pairs = [&](auto d_tag, auto b_tag, auto k_tag) {
    hipLaunchKernelGGL((decode_balanced_kernel<decltype(d_tag)::value, decltype(b_tag)::value,
                                               decltype(k_tag)::value>),
                       grid, block, 0, stream, p);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (head_dim == 128) {
    if (p.kv8) bias ? pairs(D128{}, T_{}, T_{}) : pairs(D128{}, F_{}, T_{});
    else bias ? pairs(D128{}, T_{}, F_{}) : pairs(D128{}, F_{}, F_{});
    hipLaunchKernelGGL((combine_balanced_kernel<128>), cgrid, cblock, 0, stream, p);
  } else {
    if (p.kv8) bias ? pairs(D64{}, T_{}, T_{}) : pairs(D64{}, F_{}, T_{});
    else bias ? pairs(D64{}, T_{}, F_{}) : pairs(D64{}, F_{}, F_{});
    hipLaunchKernelGGL((combine_balanced_kernel<64>), cgrid, cblock, 0, stream, p);
  }
  return hipGetLastError();
}

// ----------------------------------------------------- no-alloc scratch
//
// The workspace of rpa_attn_varlen_noalloc.  Each GPU that loads the library
// holds one copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: the kernels only ever receive the
// device address that hipGetSymbolAddress returns for the current device.

static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_device_ptr(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_combine(const CombineParams &p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  CombineParams q = p;
  q.wr = p.S > 64 ? 4 : p.S > 16 ? 2 : 1;  // waves per row
  const int rows_per_wg = 4 / q.wr;
  const dim3 grid((unsigned)((p.rows + rows_per_wg - 1) / rows_per_wg)), block(kThreads);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, q);
  return hipGetLastError();
}

}  // namespace rpa
