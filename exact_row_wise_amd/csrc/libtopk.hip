// libtopk.hip -- exact per-row top-k of BF16 logits for MI355X (gfx950).
//
// Definition of the result: vLLM API page "vllm.models.deepseek_v41.nvidia.
// specialized_decode.attention.decode_topk_cute", module docstring,
// paragraph "What this module computes"; the 16-bit order-preserving key:
// sglang PR #39305, section "What is kept from DeepSelect"; the block-table
// transform and the short-row bypass: vLLM kimi_k3 indexer page,
// IndexerSelect.emit and IndexerSelect.kernel.
//
// Shape of the hot path (same page, paragraphs "How." and the two ways to
// the answer), re-planned for CDNA4:
//   * every logit is read from HBM once, with 16-byte vector loads, into
//     VGPRs, and turned into packed 16-bit keys there;
//   * a cutoff is taken from a sample of the row (the q-th largest sample,
//     q chosen so that at least k keys lie at or above it with
//     overwhelming probability), found with two 8-bit radix passes over
//     the samples in LDS;
//   * survivors (keys above the cutoff; keys equal to it up to k) are
//     compacted with wave64 ballots and lane-mask counts -- per-wave
//     regions in LDS, so the compaction costs no atomic per key;
//   * the exact k-th key over the survivors again takes two 8-bit LDS radix
//     passes, then the indices are written (with the page transform);
//   * if the sample misjudged the row (fewer than k keys at or above the
//     cutoff, or more survivors than the buffers hold) the row takes the
//     direct path: two whole-row 8-bit radix histograms with 8 replicated
//     copies per bin (lane mod 8), then a write pass;
//   * rows wider than one workgroup's registers are split over a team of
//     workgroups with equal blockIdx % 8 (one XCD, one L2).  Every member
//     derives the same cutoff from the same samples, so members never wait
//     for each other: each reserves its survivor range in the row's global
//     scratch with one 64-bit atomic, and the last member to arrive
//     finishes the row.  No barrier spans workgroups, so no residency
//     assumption is needed.
// There is no MFMA: this is a memory-bound selection, and all selection
// arithmetic is on integer keys.

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "libtopk.h"

namespace {

constexpr int kNT = 256;                 // threads per workgroup (4 wave64)
constexpr int kWaves = kNT / 64;
constexpr int kCopies = 8;               // replicated bins of whole-row histograms
constexpr int kTokenVPT = 8;             // 16-byte vectors per thread, token rows
constexpr int kBlockVPT = 16;            // 16-byte vectors per thread, block rows
constexpr int kTokenSV = 2;              // sample vectors per thread, token teams
constexpr int kBlockSV = 4;              // sample vectors per thread, block teams
constexpr int kTeamLCW = 1024;           // per-wave survivor slots in a team member
constexpr int kTeamBatch = 1024;         // rows per team launch (scratch bound)

constexpr uint32_t kKeyNegInf = 0x007Fu; // key(-inf)
constexpr uint32_t kKeyPosInf = 0xFF80u; // key(+inf): the pinned newest block
constexpr uint32_t kKeyNaN = 0xFFFFu;    // key of the canonical positive NaN
constexpr uint32_t kNone = 0xFFFFFFFFu;  // empty sample slot

// LDS map (32-bit words)
constexpr int kHist = 0;                           // 256 bins x kCopies
constexpr int kSums = kHist + 256 * kCopies;       // 256 words
constexpr int kBc = kSums + 256;                   // 32 words: broadcast + counters
constexpr int kLists = kBc + 32;                   // per-wave lists, then the tie list
enum {
  BC_B1 = 0, BC_A1 = 1, BC_B2 = 2, BC_A2 = 3,   // radix results
  BC_C1 = 4, BC_C2 = 5,                         // emit counters (above T, equal T)
  BC_EQ = 6,                                    // keys equal to the cutoff
  BC_FLAG = 7, BC_GTB = 8, BC_EQB = 9,          // team: last-arriver flag, bases
  BC_GT = 10, BC_EQT = 11, BC_OVF = 12,         // team: row totals, overflow
  BC_TMP = 16,                                  // kWaves words for reductions
  BC_GTW = 24                                   // kWaves per-wave survivor counts
};

struct RowCtl {
  unsigned long long counts;  // (keys above cutoff << 32) | keys equal to it
  unsigned int arrive;        // members done
  unsigned int flags;         // bit 0: a member's survivors overflowed
};

struct Params {
  const uint16_t* logits;
  int64_t row_stride;
  const int32_t* valid_len;
  int32_t rows;        // rows of this launch
  int32_t row0;        // first row of this launch
  int32_t width;
  int32_t k;
  const int32_t* pages;
  int64_t pages_stride;
  int32_t page_shift;
  int32_t* out;
  int32_t* path;
  int32_t force_direct;
  int32_t lcw;         // per-wave survivor slots
  // teams
  int32_t G;
  int32_t xcd_map;
  RowCtl* ctl;
  unsigned long long* gt_list;   // [rows][capg]: (key << 32) | index
  uint32_t* eq_list;             // [rows][TOPK_MAX_K]
  int32_t capg;
};

// ------------------------------------------------------------------ keys
// Two BF16 patterns in one word -> their two keys in the same halves:
// a half with the sign bit set is inverted entirely, any other half only
// its sign bit (sglang PR #39305, "What is kept from DeepSelect").
__device__ __forceinline__ uint32_t key2(uint32_t w) {
  const uint32_t neg = w & 0x80008000u;
  const uint32_t flip = neg - (neg >> 15);  // 0x7FFF in each negative half
  return w ^ flip ^ 0x80008000u;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Key of the NaN-propagating maximum of the 8 logits of one 16-byte vector
// (decode_topk_cute, block_key / max_nan_bf16x2): a NaN of either sign
// anywhere gives the canonical positive NaN; otherwise the largest key.
// In key space a NaN is a key above key(+inf) or below key(-inf).
__device__ __forceinline__ uint32_t block_key4(uint4 v) {
  const uint32_t a = key2(v.x), b = key2(v.y), c = key2(v.z), d = key2(v.w);
  const uint32_t mx = pk_max(pk_max(a, b), pk_max(c, d));
  const uint32_t mn = pk_min(pk_min(a, b), pk_min(c, d));
  const uint32_t hi = max(mx & 0xFFFFu, mx >> 16);
  const uint32_t lo = min(mn & 0xFFFFu, mn >> 16);
  return (hi > kKeyPosInf || lo < kKeyNegInf) ? kKeyNaN : hi;
}

__device__ __forceinline__ uint32_t half_of(uint32_t w, int h) {
  return h ? (w >> 16) : (w & 0xFFFFu);
}

// ----------------------------------------------------------- wave tools
__device__ __forceinline__ uint32_t mbcnt(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(x, d, 64);
    if (lane >= d) x += t;
  }
  return x;
}

// One wave over a 256-bin histogram: the bin b where counts summed from the
// top bin down first reach `need`, and the count strictly above b
// (decode_topk_cute, select_bin).  res[0] = b, res[1] = count above.
__device__ void find_bin(const uint32_t* hist, uint32_t need, uint32_t* res) {
  const int lane = __lane_id();
  const int b0 = 255 - 4 * lane;
  const uint32_t h0 = hist[b0], h1 = hist[b0 - 1], h2 = hist[b0 - 2], h3 = hist[b0 - 3];
  const uint32_t s = h0 + h1 + h2 + h3;
  const uint32_t incl = wave_incl_scan(s);
  const unsigned long long m = __ballot(incl >= need);
  const int L = m ? (__ffsll((unsigned long long)m) - 1) : 63;
  if (lane == L) {
    uint32_t acc = incl - s;
    int bin;
    if (acc + h0 >= need) {
      bin = b0;
    } else {
      acc += h0;
      if (acc + h1 >= need) {
        bin = b0 - 1;
      } else {
        acc += h1;
        if (acc + h2 >= need) {
          bin = b0 - 2;
        } else {
          acc += h2;
          bin = b0 - 3;
        }
      }
    }
    res[0] = (uint32_t)bin;
    res[1] = acc;
  }
}

// Sum over the workgroup (every thread gets the total).
__device__ uint32_t block_sum(uint32_t x, uint32_t* tmp) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  if (__lane_id() == 0) tmp[threadIdx.x >> 6] = x;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += tmp[w];
  __syncthreads();
  return t;
}

// A slot per predicated lane from one LDS counter: one atomic per wave.
__device__ __forceinline__ uint32_t wave_slot(bool pred, uint32_t* ctr) {
  const unsigned long long m = __ballot(pred);
  uint32_t slot = 0;
  if (m) {
    const int leader = __ffsll(m) - 1;
    uint32_t base = 0;
    if (__lane_id() == leader) base = atomicAdd(ctr, (uint32_t)__popcll(m));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
    slot = base + mbcnt(m);
  }
  return slot;
}

// ----------------------------------------------------------------- output
struct Out {
  int32_t* out;          // this row's k outputs
  const int32_t* pages;  // this row's block-table entries, or null
  int32_t shift;         // log2 of the page size
  uint32_t k;            // slots of the row (writes past them are dropped)
  bool block;

  // Element index idx with key `key` into output slot pos: -1 for a -inf
  // block; otherwise the index, through the block table when there is one
  // (vLLM kimi_k3 indexer, IndexerSelect.emit).
  __device__ __forceinline__ void put(uint32_t pos, uint32_t idx, uint32_t key) const {
    if (pos >= k) return;
    int32_t val;
    if (block && key == kKeyNegInf) {
      val = -1;
    } else if (pages) {
      val = pages[idx >> shift] * (1 << shift) + (int32_t)(idx & ((1u << shift) - 1u));
    } else {
      val = (int32_t)idx;
    }
    out[pos] = val;
  }
  __device__ __forceinline__ int32_t plain(uint32_t idx) const {
    if (pages) return pages[idx >> shift] * (1 << shift) + (int32_t)(idx & ((1u << shift) - 1u));
    return (int32_t)idx;
  }
};

__device__ __forceinline__ Out row_out(const Params& p, int row, bool block) {
  Out o;
  o.out = p.out + (int64_t)row * p.k;
  o.pages = p.pages ? p.pages + (int64_t)row * p.pages_stride : nullptr;
  o.shift = p.page_shift;
  o.k = (uint32_t)p.k;
  o.block = block;
  return o;
}

__device__ __forceinline__ int clamp_len(int v, int width) {
  return v < 0 ? 0 : (v > width ? width : v);
}

__device__ __forceinline__ void set_path(const Params& p, int row, int code) {
  if (p.path && threadIdx.x == 0) p.path[row] = code;
}

// Token rows with n <= k: 0..n-1 then -1, no logits read
// (decode_topk_cute result definition; kimi_k3 IndexerSelect bypass).
__device__ void write_short_token(const Out& o, int n, int k) {
  for (int e = threadIdx.x; e < k; e += kNT) o.out[e] = e < n ? o.plain((uint32_t)e) : -1;
}

// Block rows with n <= k: every block in order, -1 for -inf blocks, the
// newest pinned at +inf, then -1 padding.
__device__ void write_short_block(const Out& o, const uint4* src, int n, int k) {
  for (int b = threadIdx.x; b < k; b += kNT) {
    if (b < n) {
      const uint32_t key = (b == n - 1) ? kKeyPosInf : block_key4(src[b]);
      o.put((uint32_t)b, (uint32_t)b, key);
    } else {
      o.out[b] = -1;
    }
  }
}

// Emit one candidate against the exact threshold: keys above T take slots
// [0, cgt), keys equal to T the first `take` slots after cgt.
__device__ __forceinline__ void emit_one(bool has, uint32_t key, uint32_t idx, uint32_t T,
                                         uint32_t cgt, uint32_t take, uint32_t* bc,
                                         const Out& o) {
  const bool gt = has && key > T;
  const bool eq = has && key == T;
  const uint32_t s1 = wave_slot(gt, &bc[BC_C1]);
  if (gt) o.put(s1, idx, key);
  const uint32_t s2 = wave_slot(eq, &bc[BC_C2]);
  if (eq && s2 < take) o.put(cgt + s2, idx, key);
}

// ------------------------------------------------------------ direct path
// The exact k-th key from two whole-row 8-bit radix histograms, every
// histogram atomic spread over kCopies replicated bins (lane mod 8), then
// one pass writing the selected indices (decode_topk_cute "Direct" path and
// its note on replicated copies).  Reads the row from global memory; used
// when the sampled cutoff misjudged the row, or on request.  n > k.
template <int MODE>
__device__ void direct_select(const uint4* src, int v, int n, int k, const Out& o,
                              uint32_t* smem) {
  const int tid = threadIdx.x;
  const int copy = __lane_id() & (kCopies - 1);
  const int nvec = (MODE == TOPK_MODE_BLOCK) ? n : (v + 7) >> 3;
  uint32_t* hist = smem + kHist;
  uint32_t* sums = smem + kSums;
  uint32_t* bc = smem + kBc;
  uint32_t b1 = 0, a1 = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = tid; i < 256 * kCopies; i += kNT) hist[i] = 0;
    if (tid == 0) {
      bc[BC_C1] = 0;
      bc[BC_C2] = 0;
    }
    __syncthreads();
    for (int vid = tid; vid < nvec; vid += kNT) {
      const uint4 raw = src[vid];
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        const uint32_t key = (vid == n - 1) ? kKeyPosInf : block_key4(raw);
        if (pass == 0) {
          atomicAdd(&hist[(key >> 8) * kCopies + copy], 1u);
        } else if ((key >> 8) == b1) {
          atomicAdd(&hist[(key & 255u) * kCopies + copy], 1u);
        }
      } else {
        const uint32_t w[4] = {key2(raw.x), key2(raw.y), key2(raw.z), key2(raw.w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t key = half_of(w[e >> 1], e & 1);
          if (vid * 8 + e < v) {
            if (pass == 0) {
              atomicAdd(&hist[(key >> 8) * kCopies + copy], 1u);
            } else if ((key >> 8) == b1) {
              atomicAdd(&hist[(key & 255u) * kCopies + copy], 1u);
            }
          }
        }
      }
    }
    __syncthreads();
    {
      uint32_t s = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) s += hist[tid * kCopies + c];
      sums[tid] = s;
    }
    __syncthreads();
    if (tid < 64) find_bin(sums, pass == 0 ? (uint32_t)k : (uint32_t)k - a1, bc + 2 * pass);
    __syncthreads();
    if (pass == 0) {
      b1 = bc[BC_B1];
      a1 = bc[BC_A1];
    }
  }
  const uint32_t T = (b1 << 8) | bc[BC_B2];
  const uint32_t cgt = a1 + bc[BC_A2];
  const uint32_t take = (uint32_t)k - cgt;
  for (int vid = tid; vid < nvec; vid += kNT) {
    const uint4 raw = src[vid];
    if constexpr (MODE == TOPK_MODE_BLOCK) {
      const uint32_t key = (vid == n - 1) ? kKeyPosInf : block_key4(raw);
      emit_one(true, key, (uint32_t)vid, T, cgt, take, bc, o);
    } else {
      const uint32_t w[4] = {key2(raw.x), key2(raw.y), key2(raw.z), key2(raw.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t idx = (uint32_t)(vid * 8 + e);
        emit_one((int)idx < v, half_of(w[e >> 1], e & 1), idx, T, cgt, take, bc, o);
      }
    }
  }
}

// --------------------------------------------------------- sampled path
// Rank of the cutoff among S samples of an n-element row: k scaled to the
// sample plus a margin of ~4.5 standard deviations and a constant, so that
// fewer than k keys at or above the cutoff is a rare event (then the row
// falls back to the direct path; exactness never depends on this choice).
__device__ __forceinline__ uint32_t isqrt32(uint32_t x) {
  uint32_t r = 0;
  for (uint32_t b = 1u << 15; b; b >>= 1) {
    const uint32_t t = r | b;
    if (t * t <= x) r = t;
  }
  return r;
}

__device__ __forceinline__ uint32_t sample_rank(uint32_t k, uint32_t n, uint32_t S) {
  if (S >= n) return k;  // every element sampled: the cutoff is the k-th key
  const uint32_t q0 = (uint32_t)(((uint64_t)k * S) / n);
  const uint32_t q = q0 + (9u * isqrt32(q0) + 1u) / 2u + 8u;
  return q < S ? q : S;
}

// The q-th largest of the samples (kNone marks an empty slot): two 8-bit
// radix passes, one histogram each (decode_topk_cute, radix_select).
template <int NSK>
__device__ uint32_t sample_cutoff(const uint32_t (&sk)[NSK], uint32_t q, uint32_t* smem) {
  uint32_t* hist = smem + kHist;
  uint32_t* bc = smem + kBc;
  for (int i = threadIdx.x; i < 512; i += kNT) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NSK; ++i)
    if (sk[i] != kNone) atomicAdd(&hist[sk[i] >> 8], 1u);
  __syncthreads();
  if (threadIdx.x < 64) find_bin(hist, q, bc + BC_B1);
  __syncthreads();
  const uint32_t b1 = bc[BC_B1], a1 = bc[BC_A1];
#pragma unroll
  for (int i = 0; i < NSK; ++i)
    if (sk[i] != kNone && (sk[i] >> 8) == b1) atomicAdd(&hist[256 + (sk[i] & 255u)], 1u);
  __syncthreads();
  if (threadIdx.x < 64) find_bin(hist + 256, q - a1, bc + BC_B2);
  __syncthreads();
  return (b1 << 8) | bc[BC_B2];
}

// Survivor compaction of one key against the cutoff c, one wave at a time:
// keys above c go to this wave's region at its running count (ballot +
// lane-mask count, no atomic); keys equal to c go to the shared tie list,
// at most k of them, one LDS atomic per wave that has any.
__device__ __forceinline__ void compact_one(uint32_t key, uint32_t idx, uint32_t c,
                                            uint32_t* glist, uint32_t lcw, uint32_t& gcount,
                                            uint16_t* elist, uint32_t* eqctr, uint32_t k) {
  const unsigned long long mge = __ballot(key >= c);
  if (mge) {
    const unsigned long long mgt = __ballot(key > c);
    if (mgt) {
      const uint32_t pos = gcount + mbcnt(mgt);
      if (key > c && pos < lcw) glist[pos] = (key << 16) | idx;
      gcount += (uint32_t)__popcll(mgt);
    }
    const unsigned long long meq = mge & ~mgt;
    if (meq) {
      const int leader = __ffsll(meq) - 1;
      uint32_t base = 0;
      if (__lane_id() == leader) base = atomicAdd(eqctr, (uint32_t)__popcll(meq));
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
      const uint32_t pos = base + mbcnt(meq);
      if (key == c && pos < k) elist[pos] = (uint16_t)idx;
    }
  }
}

// Exact k-th key over the LDS survivor lists (keys above the cutoff only,
// count >= k): two 8-bit radix passes, then the write pass.
__device__ void select_lds_lists(const uint32_t* lists, uint32_t lcw, const uint32_t* cnt,
                                 uint32_t k, uint32_t* smem, const Out& o) {
  const int tid = threadIdx.x;
  uint32_t* hist = smem + kHist;
  uint32_t* bc = smem + kBc;
  for (int i = tid; i < 512; i += kNT) hist[i] = 0;
  __syncthreads();
  for (int w = 0; w < kWaves; ++w)
    for (uint32_t i = tid; i < cnt[w]; i += kNT) atomicAdd(&hist[lists[w * lcw + i] >> 24], 1u);
  __syncthreads();
  if (tid < 64) find_bin(hist, k, bc + BC_B1);
  __syncthreads();
  const uint32_t b1 = bc[BC_B1], a1 = bc[BC_A1];
  for (int w = 0; w < kWaves; ++w)
    for (uint32_t i = tid; i < cnt[w]; i += kNT) {
      const uint32_t e = lists[w * lcw + i];
      if ((e >> 24) == b1) atomicAdd(&hist[256 + ((e >> 16) & 255u)], 1u);
    }
  __syncthreads();
  if (tid < 64) find_bin(hist + 256, k - a1, bc + BC_B2);
  __syncthreads();
  const uint32_t T = (b1 << 8) | bc[BC_B2];
  const uint32_t cgt = a1 + bc[BC_A2];
  const uint32_t take = k - cgt;
  for (int w = 0; w < kWaves; ++w)
    for (uint32_t i = tid; i < cnt[w]; i += kNT) {
      const uint32_t e = lists[w * lcw + i];
      emit_one(true, e >> 16, e & 0xFFFFu, T, cgt, take, bc, o);
    }
}

// Zero the keys of elements r..7 of one staged vector (r valid elements,
// 0..8).  Only a row's (or chunk's) last occupied vector slot needs it.
__device__ __forceinline__ void mask_tail(uint32_t (&w)[4], int r) {
  w[0] &= r >= 2 ? 0xFFFFFFFFu : (r == 1 ? 0x0000FFFFu : 0u);
  w[1] &= r >= 4 ? 0xFFFFFFFFu : (r == 3 ? 0x0000FFFFu : 0u);
  w[2] &= r >= 6 ? 0xFFFFFFFFu : (r == 5 ? 0x0000FFFFu : 0u);
  w[3] &= r >= 8 ? 0xFFFFFFFFu : (r == 7 ? 0x0000FFFFu : 0u);
}

__device__ __forceinline__ int clamp8(int x) { return x < 0 ? 0 : (x > 8 ? 8 : x); }

// ============================================ one workgroup per row
// Rows whose valid vectors fit kNT * VPT: the whole row sits in VGPRs.
template <int MODE, int VPT>
__global__ __launch_bounds__(kNT) void topk_rows_wg(Params p) {
  extern __shared__ uint32_t smem[];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int k = p.k;
  const int v = clamp_len(p.valid_len[row], p.width);
  const int n = (MODE == TOPK_MODE_BLOCK) ? (v + 7) >> 3 : v;
  const Out o = row_out(p, row, MODE == TOPK_MODE_BLOCK);
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
  uint32_t* bc = smem + kBc;

  if (n <= k) {
    if constexpr (MODE == TOPK_MODE_BLOCK) write_short_block(o, src, n, k);
    else write_short_token(o, n, k);
    set_path(p, row, TOPK_PATH_SHORT);
    return;
  }
  bool direct = p.force_direct != 0;
  int code = TOPK_PATH_DIRECT_FORCED;
  if (!direct) {
    const int nvec = (v + 7) >> 3;
    const int jt = (nvec - 1) / kNT;  // last vector slot holding row data

    // -- stage the row: 16-byte loads into VGPRs, keys computed in place
    uint4 raw[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vid = j * kNT + tid;
      raw[j] = vid < nvec ? src[vid] : make_uint4(0u, 0u, 0u, 0u);
    }
    constexpr int kSampleEvery = VPT / 8;  // sampled slots: j % kSampleEvery == 0
    uint32_t sk[8];
    uint32_t my_samples = 0;
    uint32_t kw[MODE == TOPK_MODE_BLOCK ? 1 : VPT][4];
    uint32_t kb[MODE == TOPK_MODE_BLOCK ? VPT : 1];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vid = j * kNT + tid;
      uint32_t s = kNone;
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        kb[j] = vid < n ? (vid == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
        s = kb[j];
      } else {
        uint32_t w[4] = {key2(raw[j].x), key2(raw[j].y), key2(raw[j].z), key2(raw[j].w)};
        if (j == jt) mask_tail(w, clamp8(v - 8 * vid));
#pragma unroll
        for (int i = 0; i < 4; ++i) kw[j][i] = w[i];
        // sample: element (j & 7) of the vector, element 0 if that is past v
        const int e = (j / kSampleEvery) & 7;
        s = (vid * 8 + e < v) ? half_of(w[e >> 1], e & 1) : (w[0] & 0xFFFFu);
      }
      if (j % kSampleEvery == 0) {
        sk[j / kSampleEvery] = vid < nvec ? s : kNone;
        my_samples += vid < nvec ? 1u : 0u;
      }
    }

    if (tid == 0) bc[BC_EQ] = 0;
    const uint32_t S = block_sum(my_samples, bc + BC_TMP);
    const uint32_t q = sample_rank((uint32_t)k, (uint32_t)n, S);
    const uint32_t c = sample_cutoff(sk, q, smem);

    if (MODE == TOPK_MODE_TOKEN && c == 0u) {
      // a zero cutoff would admit the zero keys of slots past the length
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    } else {
      // -- filter + compaction of survivors
      const uint32_t lcw = (uint32_t)p.lcw;
      uint32_t* glist = smem + kLists + wave * lcw;
      uint16_t* elist = reinterpret_cast<uint16_t*>(smem + kLists + kWaves * lcw);
      uint32_t gcount = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j <= jt) {
          const uint32_t vid = (uint32_t)(j * kNT + tid);
          if constexpr (MODE == TOPK_MODE_BLOCK) {
            compact_one(kb[j], vid, c, glist, lcw, gcount, elist, &bc[BC_EQ], (uint32_t)k);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              compact_one(half_of(kw[j][e >> 1], e & 1), (vid << 3) | (uint32_t)e, c, glist,
                          lcw, gcount, elist, &bc[BC_EQ], (uint32_t)k);
          }
        }
      }
      if (__lane_id() == 0) bc[BC_GTW + wave] = gcount;
      if (tid == 0) {
        bc[BC_C1] = 0;
        bc[BC_C2] = 0;
      }
      __syncthreads();
      uint32_t cnt[kWaves];
      uint32_t gt_total = 0;
      bool ovf = false;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        cnt[w] = bc[BC_GTW + w];
        gt_total += cnt[w];
        ovf |= cnt[w] > lcw;
      }
      const uint32_t eq_total = bc[BC_EQ];
      if (ovf) {
        direct = true;
        code = TOPK_PATH_DIRECT_OVERFLOW;
      } else if (gt_total + eq_total < (uint32_t)k) {
        direct = true;
        code = TOPK_PATH_DIRECT_MISJUDGED;
      } else if (gt_total >= (uint32_t)k) {
        // the k-th key lies above the cutoff: exact select over the survivors
        select_lds_lists(smem + kLists, lcw, cnt, (uint32_t)k, smem, o);
        code = TOPK_PATH_SAMPLED;
      } else {
        // the k-th key is the cutoff: every survivor above it, then ties
        const uint32_t take = (uint32_t)k - gt_total;
        for (int w = 0; w < kWaves; ++w)
          for (uint32_t i = tid; i < cnt[w]; i += kNT) {
            const uint32_t e = smem[kLists + w * lcw + i];
            const uint32_t s1 = wave_slot(true, &bc[BC_C1]);
            o.put(s1, e & 0xFFFFu, e >> 16);
          }
        for (uint32_t i = tid; i < take; i += kNT) o.put(gt_total + i, elist[i], c);
        code = TOPK_PATH_SAMPLED_TIES;
      }
    }
  }
  if (direct) {
    __syncthreads();
    direct_select<MODE>(src, v, n, k, o, smem);
  }
  set_path(p, row, code);
}
// ============================================ team of workgroups per row
// Exact k-th key over the row's global survivor list (count >= k).
__device__ void select_global_list(const unsigned long long* gl, uint32_t m, uint32_t k,
                                   uint32_t* smem, const Out& o) {
  const int tid = threadIdx.x;
  uint32_t* hist = smem + kHist;
  uint32_t* bc = smem + kBc;
  for (int i = tid; i < 512; i += kNT) hist[i] = 0;
  if (tid == 0) {
    bc[BC_C1] = 0;
    bc[BC_C2] = 0;
  }
  __syncthreads();
  for (uint32_t i = tid; i < m; i += kNT) atomicAdd(&hist[(uint32_t)(gl[i] >> 40)], 1u);
  __syncthreads();
  if (tid < 64) find_bin(hist, k, bc + BC_B1);
  __syncthreads();
  const uint32_t b1 = bc[BC_B1], a1 = bc[BC_A1];
  for (uint32_t i = tid; i < m; i += kNT) {
    const uint32_t key = (uint32_t)(gl[i] >> 32);
    if ((key >> 8) == b1) atomicAdd(&hist[256 + (key & 255u)], 1u);
  }
  __syncthreads();
  if (tid < 64) find_bin(hist + 256, k - a1, bc + BC_B2);
  __syncthreads();
  const uint32_t T = (b1 << 8) | bc[BC_B2];
  const uint32_t cgt = a1 + bc[BC_A2];
  const uint32_t take = k - cgt;
  for (uint32_t i = tid; i < m; i += kNT) {
    const unsigned long long e = gl[i];
    emit_one(true, (uint32_t)(e >> 32), (uint32_t)e, T, cgt, take, bc, o);
  }
}

template <int MODE, int VPT, int SV>
__global__ __launch_bounds__(kNT) void topk_rows_team(Params p) {
  extern __shared__ uint32_t smem[];
  const int G = p.G;
  int lrow, member;
  if (p.xcd_map) {
    // members of a row share blockIdx % 8, i.e. the same XCD and L2
    const int b = blockIdx.x, x = b & 7, y = b >> 3;
    lrow = (y / G) * 8 + x;
    member = y % G;
  } else {
    lrow = blockIdx.x / G;
    member = blockIdx.x % G;
  }
  if (lrow >= p.rows) return;
  const int row = p.row0 + lrow;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int k = p.k;
  const int v = clamp_len(p.valid_len[row], p.width);
  const int n = (MODE == TOPK_MODE_BLOCK) ? (v + 7) >> 3 : v;
  const Out o = row_out(p, row, MODE == TOPK_MODE_BLOCK);
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
  uint32_t* bc = smem + kBc;

  if (n <= k) {
    if (member == 0) {
      if constexpr (MODE == TOPK_MODE_BLOCK) write_short_block(o, src, n, k);
      else write_short_token(o, n, k);
      set_path(p, row, TOPK_PATH_SHORT);
    }
    return;
  }
  bool direct = false;
  int code = TOPK_PATH_DIRECT_FORCED;
  if (p.force_direct) {
    if (member != 0) return;
    direct = true;
  } else {
    const int nvec = (v + 7) >> 3;
    const int per = (nvec + G - 1) / G;
    const int vb = min(member * per, nvec);
    const int ve = min(vb + per, nvec);
    const int jt = ve > vb ? (ve - vb - 1) / kNT : -1;  // last occupied slot

    // -- chunk loads and sample loads, all issued before any use
    uint4 raw[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vid = vb + j * kNT + tid;
      raw[j] = vid < ve ? src[vid] : make_uint4(0u, 0u, 0u, 0u);
    }
    const int ns = min(SV * kNT, nvec);  // sample vectors, spread over the row
    uint4 sraw[SV];
    int spos[SV];
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      const int s = j * kNT + tid;
      spos[j] = s < ns ? (int)(((int64_t)(2 * s + 1) * nvec) / (2 * (int64_t)ns)) : -1;
      sraw[j] = spos[j] >= 0 ? src[spos[j]] : make_uint4(0u, 0u, 0u, 0u);
    }

    // -- sample keys and the cutoff (identical in every member)
    constexpr int NSK = (MODE == TOPK_MODE_BLOCK) ? SV : SV * 8;
    uint32_t sk[NSK];
    uint32_t my_samples = 0;
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      const int vid = spos[j];
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        sk[j] = vid < 0 ? kNone : (vid == n - 1 ? kKeyPosInf : block_key4(sraw[j]));
        my_samples += vid >= 0 ? 1u : 0u;
      } else {
        const uint32_t w[4] = {key2(sraw[j].x), key2(sraw[j].y), key2(sraw[j].z),
                               key2(sraw[j].w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = vid >= 0 && vid * 8 + e < v;
          sk[j * 8 + e] = ok ? half_of(w[e >> 1], e & 1) : kNone;
          my_samples += ok ? 1u : 0u;
        }
      }
    }
    if (tid == 0) bc[BC_EQ] = 0;
    const uint32_t S = block_sum(my_samples, bc + BC_TMP);
    const uint32_t q = sample_rank((uint32_t)k, (uint32_t)n, S);
    const uint32_t c = sample_cutoff(sk, q, smem);

    if (MODE == TOPK_MODE_TOKEN && c == 0u) {
      // every member sees the same cutoff: member 0 alone takes the row
      if (member != 0) return;
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    } else {
      // -- keys of the chunk, filter + compaction into LDS
      const uint32_t lcw = (uint32_t)p.lcw;
      uint32_t* glist = smem + kLists + wave * lcw;
      uint16_t* elist = reinterpret_cast<uint16_t*>(smem + kLists + kWaves * lcw);
      uint32_t gcount = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j > jt) continue;
        const int lvid = j * kNT + tid;
        const int vid = vb + lvid;
        if constexpr (MODE == TOPK_MODE_BLOCK) {
          const uint32_t key = vid < ve ? (vid == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
          compact_one(key, (uint32_t)lvid, c, glist, lcw, gcount, elist, &bc[BC_EQ],
                      (uint32_t)k);
        } else {
          uint32_t w[4] = {key2(raw[j].x), key2(raw[j].y), key2(raw[j].z), key2(raw[j].w)};
          if (j == jt) mask_tail(w, vid < ve ? clamp8(v - 8 * vid) : 0);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            compact_one(half_of(w[e >> 1], e & 1), ((uint32_t)lvid << 3) | (uint32_t)e, c,
                        glist, lcw, gcount, elist, &bc[BC_EQ], (uint32_t)k);
        }
      }
      if (__lane_id() == 0) bc[BC_GTW + wave] = gcount;
      __syncthreads();
      uint32_t cnt[kWaves], pre[kWaves];
      uint32_t g_gt = 0;
      bool ovf = false;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        cnt[w] = bc[BC_GTW + w];
        pre[w] = g_gt;
        g_gt += cnt[w];
        ovf |= cnt[w] > lcw;
      }
      const uint32_t g_eq = bc[BC_EQ];
      RowCtl* ctl = p.ctl + lrow;
      unsigned long long* gl = p.gt_list + (int64_t)lrow * p.capg;
      uint32_t* el = p.eq_list + (int64_t)lrow * TOPK_MAX_K;

      // -- one 64-bit atomic reserves this member's ranges in the row's lists
      if (tid == 0) {
        const unsigned long long old = __hip_atomic_fetch_add(
            &ctl->counts, ((unsigned long long)g_gt << 32) | g_eq, __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT);
        if (ovf)
          __hip_atomic_fetch_or(&ctl->flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bc[BC_GTB] = (uint32_t)(old >> 32);
        bc[BC_EQB] = (uint32_t)old;
      }
      __syncthreads();
      const uint32_t gbase = bc[BC_GTB], ebase = bc[BC_EQB];
      const uint32_t ebias = (MODE == TOPK_MODE_BLOCK) ? (uint32_t)vb : (uint32_t)vb * 8u;
      if (!ovf) {
        for (int w = 0; w < kWaves; ++w)
          for (uint32_t i = tid; i < cnt[w]; i += kNT) {
            const uint32_t pos = gbase + pre[w] + i;
            const uint32_t e = smem[kLists + w * lcw + i];
            if (pos < (uint32_t)p.capg)
              gl[pos] = ((unsigned long long)(e >> 16) << 32) | ((e & 0xFFFFu) + ebias);
          }
      }
      const uint32_t neq = min(g_eq, (uint32_t)k);
      for (uint32_t i = tid; i < neq; i += kNT) {
        const uint32_t pos = ebase + i;
        if (pos < (uint32_t)k) el[pos] = (uint32_t)elist[i] + ebias;
      }

      // -- arrive; the last member of the row finishes it
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) {
        const unsigned int prev =
            __hip_atomic_fetch_add(&ctl->arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        bc[BC_FLAG] = (prev == (unsigned int)(G - 1)) ? 1u : 0u;
      }
      __syncthreads();
      if (!bc[BC_FLAG]) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (tid == 0) {
        const unsigned long long tot =
            __hip_atomic_load(&ctl->counts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned int fl =
            __hip_atomic_load(&ctl->flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bc[BC_GT] = (uint32_t)(tot >> 32);
        bc[BC_EQT] = (uint32_t)tot;
        bc[BC_OVF] = fl;
        // leave the row's control words zeroed for the next launch
        __hip_atomic_store(&ctl->counts, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl->flags, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      const uint32_t gt_total = bc[BC_GT], eq_total = bc[BC_EQT];
      const bool row_ovf = bc[BC_OVF] != 0u || gt_total > (uint32_t)p.capg;
      if (row_ovf) {
        direct = true;
        code = TOPK_PATH_DIRECT_OVERFLOW;
      } else if (gt_total + eq_total < (uint32_t)k) {
        direct = true;
        code = TOPK_PATH_DIRECT_MISJUDGED;
      } else if (gt_total >= (uint32_t)k) {
        select_global_list(gl, gt_total, (uint32_t)k, smem, o);
        code = TOPK_PATH_SAMPLED;
      } else {
        const uint32_t take = (uint32_t)k - gt_total;
        for (uint32_t i = tid; i < gt_total; i += kNT) {
          const unsigned long long e = gl[i];
          o.put(i, (uint32_t)e, (uint32_t)(e >> 32));
        }
        for (uint32_t i = tid; i < take; i += kNT) o.put(gt_total + i, el[i], c);
        code = TOPK_PATH_SAMPLED_TIES;
      }
    }
  }
  if (direct) {
    __syncthreads();
    direct_select<MODE>(src, v, n, k, o, smem);
  }
  set_path(p, row, code);
}
// ================================================================= host
thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

struct Scratch {
  void* base = nullptr;
  size_t bytes = 0;
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

// Team scratch: the control words of kTeamBatch rows first, at a fixed
// place whatever the call (each launch leaves them zeroed for the next, so
// they must never move or share bytes with a previous call's lists), then
// the survivor lists of `rows` rows.
size_t team_ctl_bytes() { return (size_t)kTeamBatch * sizeof(RowCtl); }

size_t team_scratch_bytes(int rows, int capg) {
  return team_ctl_bytes() + (size_t)rows * ((size_t)capg * 8 + (size_t)TOPK_MAX_K * 4);
}

int get_scratch(hipStream_t stream, size_t need, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& sc = g_scratch[std::make_pair(dev, stream)];
  if (sc.bytes < need) {
    if (sc.base) {
      e = hipStreamSynchronize(stream);
      if (e == hipSuccess) e = hipFree(sc.base);
      sc.base = nullptr;
      sc.bytes = 0;
      if (e != hipSuccess) return fail(TOPK_ERR_HIP, "scratch release: %s", hipGetErrorString(e));
    }
    e = hipMalloc(&sc.base, need);
    if (e != hipSuccess) {
      sc.base = nullptr;
      return fail(TOPK_ERR_HIP, "scratch hipMalloc(%zu): %s", need, hipGetErrorString(e));
    }
    e = hipMemsetAsync(sc.base, 0, need, stream);
    if (e != hipSuccess) return fail(TOPK_ERR_HIP, "scratch memset: %s", hipGetErrorString(e));
    sc.bytes = need;
  }
  *out = sc.base;
  return TOPK_OK;
}

size_t lds_bytes(int lcw, int k) {
  return (size_t)(kLists + kWaves * lcw) * 4 + (((size_t)k * 2 + 15) & ~(size_t)15);
}

int row_lcw(int k) {
  int l = k / 2 + 256;
  return l < 512 ? 512 : (l > 2048 ? 2048 : l);
}

template <class K>
int launch(K kernel, int grid, size_t lds, hipStream_t stream, const Params& p) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kNT), lds, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return TOPK_OK;
}

int run(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len, int32_t rows,
        int32_t width, int32_t k, int32_t mode, const topk_block_table_t* bt, int32_t* out,
        const topk_options_t* opt, void* stream_ptr) {
  g_err[0] = '\0';
  if (rows < 0) return fail(TOPK_ERR_INVALID_ARG, "rows < 0");
  if (k < 1 || k > TOPK_MAX_K) return fail(TOPK_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, TOPK_MAX_K);
  if (mode != TOPK_MODE_TOKEN && mode != TOPK_MODE_BLOCK)
    return fail(TOPK_ERR_INVALID_ARG, "mode = %d", mode);
  if (width < 0 || width > TOPK_MAX_WIDTH)
    return fail(TOPK_ERR_INVALID_ARG, "width = %d outside [0, %d]", width, TOPK_MAX_WIDTH);
  if (row_stride < width) return fail(TOPK_ERR_INVALID_ARG, "row_stride < width");
  if (row_stride % 8 != 0) return fail(TOPK_ERR_MISALIGNED, "row_stride not a multiple of 8");
  if (rows == 0) return TOPK_OK;
  if (!logits || !valid_len || !out) return fail(TOPK_ERR_INVALID_ARG, "null pointer");
  if (((uintptr_t)logits & 15u) != 0) return fail(TOPK_ERR_MISALIGNED, "logits not 16-byte aligned");
  if (((uintptr_t)out & 3u) != 0 || ((uintptr_t)valid_len & 3u) != 0)
    return fail(TOPK_ERR_MISALIGNED, "out or valid_len not 4-byte aligned");
  int page_shift = 0;
  if (bt) {
    if (!bt->pages) return fail(TOPK_ERR_INVALID_ARG, "block table without pages");
    const int P = bt->page_size;
    if (P < 1 || (P & (P - 1)) != 0)
      return fail(TOPK_ERR_INVALID_ARG, "page_size %d is not a power of two", P);
    while ((1 << page_shift) < P) ++page_shift;
    const int64_t need = ((int64_t)width + P - 1) / P;
    if (bt->row_stride < need) return fail(TOPK_ERR_INVALID_ARG, "block table rows too short");
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);

  Params p;
  memset(&p, 0, sizeof(p));
  p.logits = logits;
  p.row_stride = row_stride;
  p.valid_len = valid_len;
  p.width = width;
  p.k = k;
  p.pages = bt ? bt->pages : nullptr;
  p.pages_stride = bt ? bt->row_stride : 0;
  p.page_shift = page_shift;
  p.out = out;
  p.path = opt ? opt->path_codes : nullptr;
  p.force_direct = opt ? (opt->force_direct != 0) : 0;

  const int nvec_max = (width + 7) / 8;
  const int cap_wg = kNT * (mode == TOPK_MODE_BLOCK ? kBlockVPT : kTokenVPT);
  if (nvec_max <= cap_wg) {
    p.rows = rows;
    p.row0 = 0;
    p.lcw = row_lcw(k);
    const size_t lds = lds_bytes(p.lcw, k);
    if (mode == TOPK_MODE_BLOCK)
      return launch(topk_rows_wg<TOPK_MODE_BLOCK, kBlockVPT>, rows, lds, stream, p);
    return launch(topk_rows_wg<TOPK_MODE_TOKEN, kTokenVPT>, rows, lds, stream, p);
  }

  // team path
  const int G = (nvec_max + cap_wg - 1) / cap_wg;
  const int capg = 8 * k + 8192;
  const int batch = rows < kTeamBatch ? rows : kTeamBatch;
  void* scratch = nullptr;
  int rc = get_scratch(stream, team_scratch_bytes(batch, capg), &scratch);
  if (rc != TOPK_OK) return rc;
  char* sp = static_cast<char*>(scratch);
  p.G = G;
  p.lcw = kTeamLCW;
  p.capg = capg;
  p.ctl = reinterpret_cast<RowCtl*>(sp);
  p.gt_list = reinterpret_cast<unsigned long long*>(sp + team_ctl_bytes());
  p.eq_list = reinterpret_cast<uint32_t*>(sp + team_ctl_bytes() + (size_t)capg * 8 * batch);
  const size_t lds = lds_bytes(kTeamLCW, k);
  for (int r0 = 0; r0 < rows; r0 += batch) {
    const int nr = (rows - r0) < batch ? (rows - r0) : batch;
    p.row0 = r0;
    p.rows = nr;
    p.xcd_map = nr >= 8 ? 1 : 0;
    const int grid = p.xcd_map ? ((nr + 7) / 8) * 8 * G : nr * G;
    if (mode == TOPK_MODE_BLOCK)
      rc = launch(topk_rows_team<TOPK_MODE_BLOCK, kBlockVPT, kBlockSV>, grid, lds, stream, p);
    else
      rc = launch(topk_rows_team<TOPK_MODE_TOKEN, kTokenVPT, kTokenSV>, grid, lds, stream, p);
    if (rc != TOPK_OK) return rc;
  }
  return TOPK_OK;
}

}  // namespace

extern "C" {

int topk_bf16_rows(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len,
                   int32_t rows, int32_t width, int32_t k, int32_t mode,
                   const topk_block_table_t* block_table, int32_t* out, void* stream) {
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, nullptr,
             stream);
}

int topk_bf16_rows_ex(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len,
                      int32_t rows, int32_t width, int32_t k, int32_t mode,
                      const topk_block_table_t* block_table, int32_t* out,
                      const topk_options_t* options, void* stream) {
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, options,
             stream);
}

const char* topk_status_string(int status) {
  switch (status) {
    case TOPK_OK: return "ok";
    case TOPK_ERR_INVALID_ARG: return "invalid argument";
    case TOPK_ERR_MISALIGNED: return "misaligned logits or row stride";
    case TOPK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* topk_last_error(void) { return g_err; }

int topk_release_scratch(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int rc = TOPK_OK;
  for (auto& kv : g_scratch) {
    if (kv.second.base) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(kv.first.first);
      hipError_t e = hipStreamSynchronize(kv.first.second);
      if (e == hipSuccess) e = hipFree(kv.second.base);
      if (e != hipSuccess) rc = fail(TOPK_ERR_HIP, "release: %s", hipGetErrorString(e));
      (void)hipSetDevice(cur);
    }
  }
  g_scratch.clear();
  return rc;
}

}  // extern "C"
