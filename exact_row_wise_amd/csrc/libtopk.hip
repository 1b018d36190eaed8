// libtopk.hip -- exact per-row top-k of BF16 logits for MI355X (gfx950).
//
// Definition of the result: vLLM API page "vllm.models.deepseek_v41.nvidia.
// specialized_decode.attention.decode_topk_cute", module docstring,
// paragraph "What this module computes"; the 16-bit order-preserving key:
// sglang PR #39305, section "What is kept from DeepSelect"; the block-table
// transform and the short-row bypass: vLLM kimi_k3 indexer page,
// IndexerSelect.emit and IndexerSelect.kernel.
//
// Shape of the hot path (decode_topk_cute docstring, paragraph "How." and
// its sampled and direct ways to the answer), re-planned for CDNA4:
//   * every logit is read from HBM once, with 16-byte vector loads, into
//     VGPRs, and turned into packed 16-bit keys there;
//   * a cutoff c is taken from a sample of the row: the q-th largest
//     sample, q scaled from k with a margin so that at least k keys lie at
//     or above c with overwhelming probability; two 8-bit LDS radix passes
//     over the samples find it, and every wave reads the bins itself;
//   * keys above c are compacted with one wave64 ballot and a lane-mask
//     count per key into the wave's own region, so no key costs an atomic;
//   * the exact k-th key T over the survivors takes one pass of a
//     1024-bin LDS histogram of (key - c), which resolves T to the exact
//     key whenever T - c <= 1024 (else two 8-bit passes); the indices are
//     then written from per-wave counts, again without atomics;
//   * rows whose k-th key equals the cutoff take the tie pass: every key
//     above c, then the first keys equal to c;
//   * a misjudged sample (fewer than k keys at or above c) or a survivor
//     overflow sends the row to the direct path: two whole-row 8-bit radix
//     histograms, every atomic spread over 8 replicated bins (lane mod 8);
//   * rows wider than one workgroup's registers are split over a team of
//     workgroups that share blockIdx % 8 (one XCD, one L2).  Every member
//     derives the same cutoff from the same samples and writes its
//     survivors to its own slice of global scratch; a second kernel, one
//     workgroup per row, reads them after the kernel boundary and finishes
//     the row.  No workgroup ever waits for another, no atomic or fence
//     crosses workgroups, and the scratch needs no reset.
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
constexpr int kTeamLCW = 1024;           // survivor slots per wave of a team member
constexpr int kTeamBatch = 1024;         // rows per team launch at most
constexpr size_t kTeamScratchMax = size_t(256) << 20;
constexpr int kRelBins = 1024;           // histogram bins of (key - cutoff)
constexpr int kSelectMax = 8192;         // survivors the select kernel stages in LDS
constexpr int kDirectWords = 256 * 8 + 256;   // direct path LDS words

constexpr uint32_t kKeyNegInf = 0x007Fu; // key(-inf)
constexpr uint32_t kKeyPosInf = 0xFF80u; // key(+inf): the pinned newest block
constexpr uint32_t kKeyNaN = 0xFFFFu;    // key of the canonical positive NaN
constexpr uint32_t kNone = 0xFFFFFFFFu;  // empty sample slot

// LDS of the one-workgroup kernel and of the select kernel (32-bit words)
constexpr int kSampHist = 0;                    // 2 x 256 bins, descending keys
constexpr int kRelHist = kSampHist + 512;       // kRelBins bins / u16 tie list
constexpr int kBc = kRelHist + kRelBins;        // 64 words
constexpr int kLists = kBc + 64;                // survivor segments / direct path
enum {
  BC_CNT = 0,    // 4: survivors per wave
  BC_CGT = 4,    // 4: keys above T per wave
  BC_CEQ = 8,    // 4: keys equal to T (or to c) per wave
  BC_EQ = 12,    // tie-list counter
  BC_C1 = 13, BC_C2 = 14,   // direct-path write counters
  BC_TMP = 16,   // 4: reductions
  BC_X = 20      // 4: reductions
};

// One team member's slice of global scratch (32-bit words):
//   [0, 4) survivors of each wave, [4] keys equal to the cutoff, [5] the
//   cutoff, [6] flags, [7] unused; [8, 8 + 4 kTeamLCW) the waves' survivor
//   segments (key << 16 | chunk-local index); then up to k chunk-local
//   indices (u16) of keys equal to the cutoff.
constexpr int kMemberHdr = 8;
constexpr int kMemberWords = kMemberHdr + 4 * kTeamLCW + TOPK_MAX_K / 2;
constexpr uint32_t kFlagDirect = 1u;

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
  int32_t lcw;         // per-wave survivor slots (one-workgroup kernel)
  int32_t G;           // team members per row
  int32_t xcd_map;
  uint32_t* team;      // team scratch: [rows][G][kMemberWords]
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

// Zero the keys of elements r..7 of one staged vector (r valid elements,
// 0..8).  Only a row's (or chunk's) last occupied vector slot needs it.
__device__ __forceinline__ void mask_tail(uint32_t (&w)[4], int r) {
  w[0] &= r >= 2 ? 0xFFFFFFFFu : (r == 1 ? 0x0000FFFFu : 0u);
  w[1] &= r >= 4 ? 0xFFFFFFFFu : (r == 3 ? 0x0000FFFFu : 0u);
  w[2] &= r >= 6 ? 0xFFFFFFFFu : (r == 5 ? 0x0000FFFFu : 0u);
  w[3] &= r >= 8 ? 0xFFFFFFFFu : (r == 7 ? 0x0000FFFFu : 0u);
}

__device__ __forceinline__ int clamp8(int x) { return x < 0 ? 0 : (x > 8 ? 8 : x); }

__device__ __forceinline__ int clamp_len(int v, int width) {
  return v < 0 ? 0 : (v > width ? width : v);
}

// The vector a thread stages in slot j of a run of `count` vectors, or -1.
// Full slots hold 256 consecutive vectors, lane-ordered within each wave
// (coalesced 1 KB per wave load).  The last occupied slot jt, holding
// rem = count - 256 jt vectors, gives each wave an equal consecutive share,
// so that every wave sees about the same number of keys whatever the
// length: the per-wave survivor regions stay balanced on short rows.
__device__ __forceinline__ int slot_vid(int j, int jt, int rem) {
  if (j < jt) return j * kNT + (int)threadIdx.x;
  if (j > jt) return -1;
  const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
  const int per_w = (rem + kWaves - 1) / kWaves;
  const int x = wave * per_w + lane;
  return (lane < per_w && x < rem) ? jt * kNT + x : -1;
}

// ----------------------------------------------------------- wave tools
__device__ __forceinline__ uint32_t mbcnt(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

#define TOPK_DPP(x, ctrl, rmask) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x), (ctrl), (rmask), 0xF, false))

// Inclusive sum over the 64 lanes with DPP row shifts and row broadcasts
// (all lanes active).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += TOPK_DPP(x, 0x111, 0xF);  // row_shr:1
  x += TOPK_DPP(x, 0x112, 0xF);  // row_shr:2
  x += TOPK_DPP(x, 0x114, 0xF);  // row_shr:4
  x += TOPK_DPP(x, 0x118, 0xF);  // row_shr:8
  x += TOPK_DPP(x, 0x142, 0xA);  // row_bcast:15
  x += TOPK_DPP(x, 0x143, 0xC);  // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t readlane(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// One wave over a histogram of 64*B bins whose index 0 holds the largest
// keys: the first bin where the running count reaches `need`, and the count
// before it (decode_topk_cute, select_bin).  Every lane gets the answer.
template <int B>
__device__ __forceinline__ void find_desc(const uint32_t* hist, uint32_t need, uint32_t& bin,
                                          uint32_t& above) {
  const int lane = __lane_id();
  uint32_t h[B];
  uint32_t s = 0;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    h[b] = hist[lane * B + b];
    s += h[b];
  }
  const uint32_t incl = wave_incl_scan(s);
  const unsigned long long m = __ballot(incl >= need);
  const int L = m ? (__ffsll(m) - 1) : 63;
  uint32_t acc = incl - s, pos = B - 1;
  bool found = false;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const bool hit = !found && acc + h[b] >= need;
    pos = hit ? (uint32_t)b : pos;
    found = found || hit;
    acc += found ? 0u : h[b];
  }
  bin = readlane((uint32_t)lane * B + pos, L);
  above = readlane(acc, L);
}

// Sum over the workgroup (every thread gets the total).
__device__ uint32_t block_sum(uint32_t x, uint32_t* tmp) {
  const uint32_t incl = wave_incl_scan(x);
  if (__lane_id() == 63) tmp[threadIdx.x >> 6] = incl;
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
    slot = readlane(base, leader) + mbcnt(m);
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

// ------------------------------------------------------------ direct path
// The exact k-th key from two whole-row 8-bit radix histograms, every
// histogram atomic spread over kCopies replicated bins (lane mod 8), then
// one pass writing the selected indices (decode_topk_cute "Direct" path and
// its note on replicated copies).  Reads the row from global memory; taken
// when the sampled cutoff misjudged the row, or on request.  n > k.
// `region` holds kDirectWords words of LDS.
template <int MODE>
__device__ void direct_select(const uint4* src, int v, int n, int k, const Out& o,
                              uint32_t* region, uint32_t* bc) {
  const int tid = threadIdx.x;
  const int copy = __lane_id() & (kCopies - 1);
  const int nvec = (MODE == TOPK_MODE_BLOCK) ? n : (v + 7) >> 3;
  uint32_t* hist = region;
  uint32_t* sums = region + 256 * kCopies;
  uint32_t b1 = 0, a1 = 0, b2 = 0, a2 = 0;
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
      sums[255 - tid] = s;  // descending key order
    }
    __syncthreads();
    uint32_t bin, above;
    find_desc<4>(sums, pass == 0 ? (uint32_t)k : (uint32_t)k - a1, bin, above);
    if (pass == 0) {
      b1 = 255u - bin;
      a1 = above;
    } else {
      b2 = 255u - bin;
      a2 = above;
    }
    __syncthreads();
  }
  const uint32_t T = (b1 << 8) | b2;
  const uint32_t cgt = a1 + a2;
  const uint32_t take = (uint32_t)k - cgt;
  for (int vid = tid; vid < nvec; vid += kNT) {
    const uint4 raw = src[vid];
    if constexpr (MODE == TOPK_MODE_BLOCK) {
      const uint32_t key = (vid == n - 1) ? kKeyPosInf : block_key4(raw);
      const bool gt = key > T, eq = key == T;
      const uint32_t s1 = wave_slot(gt, &bc[BC_C1]);
      if (gt) o.put(s1, (uint32_t)vid, key);
      const uint32_t s2 = wave_slot(eq, &bc[BC_C2]);
      if (eq && s2 < take) o.put(cgt + s2, (uint32_t)vid, key);
    } else {
      const uint32_t w[4] = {key2(raw.x), key2(raw.y), key2(raw.z), key2(raw.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t idx = (uint32_t)(vid * 8 + e);
        const uint32_t key = half_of(w[e >> 1], e & 1);
        const bool ok = (int)idx < v;
        const bool gt = ok && key > T, eq = ok && key == T;
        const uint32_t s1 = wave_slot(gt, &bc[BC_C1]);
        if (gt) o.put(s1, idx, key);
        const uint32_t s2 = wave_slot(eq, &bc[BC_C2]);
        if (eq && s2 < take) o.put(cgt + s2, idx, key);
      }
    }
  }
}

// --------------------------------------------------------- sampled path
// Rank of the cutoff among S samples of an n-element row: k scaled to the
// sample plus a margin of ~4.5 standard deviations and a constant, so that
// fewer than k keys at or above the cutoff is a rare event (the row then
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
// radix passes over one zeroed 2 x 256-bin histogram, each wave finding
// the bins itself (decode_topk_cute, radix_select over the samples).
template <int NSK>
__device__ uint32_t sample_cutoff(const uint32_t (&sk)[NSK], uint32_t q, uint32_t* sh) {
#pragma unroll
  for (int i = 0; i < NSK; ++i)
    if (sk[i] != kNone) atomicAdd(&sh[255u - (sk[i] >> 8)], 1u);
  __syncthreads();
  uint32_t i1, a1;
  find_desc<4>(sh, q, i1, a1);
  const uint32_t b1 = 255u - i1;
#pragma unroll
  for (int i = 0; i < NSK; ++i)
    if (sk[i] != kNone && (sk[i] >> 8) == b1) atomicAdd(&sh[256 + 255u - (sk[i] & 255u)], 1u);
  __syncthreads();
  uint32_t i2, a2;
  find_desc<4>(sh + 256, q - a1, i2, a2);
  return (b1 << 8) | (255u - i2);
}

// Survivor compaction of one key: a key above the cutoff goes to this
// wave's segment at the wave's running count plus its rank among the
// lanes (ballot + lane-mask count); no atomic.  `cnt` is wave-uniform.
__device__ __forceinline__ void keep_above(uint32_t key, uint32_t idx, uint32_t c, uint32_t* seg,
                                           uint32_t lcw, uint32_t& cnt) {
  const bool gt = key > c;
  const unsigned long long m = __ballot(gt);
  const uint32_t pos = cnt + mbcnt(m);
  if (gt && pos < lcw) seg[pos] = (key << 16) | idx;
  cnt += (uint32_t)__popcll(m);
}

// Tie collection of one key equal to the cutoff (the rare second pass).
__device__ __forceinline__ void keep_equal(uint32_t key, uint32_t idx, uint32_t c,
                                           uint16_t* list, uint32_t cap, uint32_t* ctr) {
  const bool eq = key == c;
  const uint32_t slot = wave_slot(eq, ctr);
  if (eq && slot < cap) list[slot] = (uint16_t)idx;
}

// Exact k-th key T over survivors spread over the waves (all keys above
// the cutoff c, at least k of them), then the write.  Wave w sees `cnt`
// entries get(i) = (key, index); `rel` is a zeroed kRelBins histogram and
// `sh` 512 free words.  The 1024 bins of (key - c - 1), largest first,
// resolve T exactly unless T - c > 1024 (then two 8-bit passes over the
// keys above c + 1024).  The write gives keys above T the slots
// [0, cgt) and the first keys equal to T the slots after, from per-wave
// counts (one barrier, no atomics).
template <class Get>
__device__ void select_and_write(Get get, uint32_t cnt, uint32_t c, uint32_t k, uint32_t* rel,
                                 uint32_t* sh, uint32_t* bc, const Out& o) {
  const int lane = __lane_id();
  const int wave = threadIdx.x >> 6;
  for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
    const uint32_t i = b0 + lane;
    if (i < cnt) {
      const uint32_t d = get.key(i) - c - 1u;
      atomicAdd(&rel[(kRelBins - 1) - min(d, (uint32_t)(kRelBins - 1))], 1u);
    }
  }
  __syncthreads();
  uint32_t ri, above;
  find_desc<kRelBins / 64>(rel, k, ri, above);
  uint32_t T, cgt;
  if (ri != 0) {
    T = c + (uint32_t)kRelBins - ri;
    cgt = above;
  } else {
    // the k-th key is at least c + kRelBins: 8-bit passes over those keys
    const uint32_t floor = c + (uint32_t)kRelBins;
    for (int i = threadIdx.x; i < 512; i += kNT) sh[i] = 0;
    __syncthreads();
    for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
      const uint32_t i = b0 + lane;
      if (i < cnt) {
        const uint32_t key = get.key(i);
        if (key >= floor) atomicAdd(&sh[255u - (key >> 8)], 1u);
      }
    }
    __syncthreads();
    uint32_t i1, a1, i2, a2;
    find_desc<4>(sh, k, i1, a1);
    const uint32_t b1 = 255u - i1;
    for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
      const uint32_t i = b0 + lane;
      if (i < cnt) {
        const uint32_t key = get.key(i);
        if (key >= floor && (key >> 8) == b1) atomicAdd(&sh[256 + 255u - (key & 255u)], 1u);
      }
    }
    __syncthreads();
    find_desc<4>(sh + 256, k - a1, i2, a2);
    T = (b1 << 8) | (255u - i2);
    cgt = a1 + a2;
  }
  const uint32_t take = k - cgt;
  uint32_t ngt = 0, neq = 0;
  for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
    const uint32_t i = b0 + lane;
    const uint32_t key = i < cnt ? get.key(i) : 0u;
    ngt += (uint32_t)__popcll(__ballot(i < cnt && key > T));
    neq += (uint32_t)__popcll(__ballot(i < cnt && key == T));
  }
  if (lane == 0) {
    bc[BC_CGT + wave] = ngt;
    bc[BC_CEQ + wave] = neq;
  }
  __syncthreads();
  uint32_t bgt = 0, beq = 0;
  for (int w = 0; w < wave; ++w) {
    bgt += bc[BC_CGT + w];
    beq += bc[BC_CEQ + w];
  }
  for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
    const uint32_t i = b0 + lane;
    const bool ok = i < cnt;
    const uint32_t key = ok ? get.key(i) : 0u;
    const bool gt = ok && key > T, eq = ok && key == T;
    const unsigned long long mg = __ballot(gt);
    const unsigned long long me = __ballot(eq);
    if (gt) o.put(bgt + mbcnt(mg), get.idx(i), key);
    const uint32_t r = beq + mbcnt(me);
    if (eq && r < take) o.put(cgt + r, get.idx(i), key);
    bgt += (uint32_t)__popcll(mg);
    beq += (uint32_t)__popcll(me);
  }
}

// A wave's survivor segment in LDS: entries key << 16 | index.
struct SegView {
  const uint32_t* seg;
  __device__ __forceinline__ uint32_t key(uint32_t i) const { return seg[i] >> 16; }
  __device__ __forceinline__ uint32_t idx(uint32_t i) const { return seg[i] & 0xFFFFu; }
};

// ============================================ one workgroup per row
// Rows whose valid vectors fit kNT * VPT: the whole row sits in VGPRs.
template <int MODE, int VPT>
__global__ __launch_bounds__(kNT) void topk_rows_wg(Params p) {
  extern __shared__ uint32_t smem[];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = tid >> 6;
  const int k = p.k;
  const int v = clamp_len(p.valid_len[row], p.width);
  const int n = (MODE == TOPK_MODE_BLOCK) ? (v + 7) >> 3 : v;
  const Out o = row_out(p, row, MODE == TOPK_MODE_BLOCK);
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
  uint32_t* sh = smem + kSampHist;
  uint32_t* rel = smem + kRelHist;
  uint32_t* bc = smem + kBc;
  uint32_t* lists = smem + kLists;

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
    const int rem = nvec - jt * kNT;  // vectors in it
    for (int i = tid; i < 512 + kRelBins; i += kNT) smem[i] = 0;  // sample + relative hists
    if (tid == 0) bc[BC_EQ] = 0;

    // -- stage the row: 16-byte loads into VGPRs, keys computed in place
    uint4 raw[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vid = slot_vid(j, jt, rem);
      raw[j] = vid >= 0 ? src[vid] : make_uint4(0u, 0u, 0u, 0u);
    }
    constexpr int kSampleEvery = VPT / 8;  // sampled slots: j % kSampleEvery == 0
    uint32_t sk[8];
    uint32_t kw[MODE == TOPK_MODE_BLOCK ? 1 : VPT][4];
    uint32_t kb[MODE == TOPK_MODE_BLOCK ? VPT : 1];
    uint32_t S = 0;  // samples taken over the workgroup
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vid = slot_vid(j, jt, rem);
      uint32_t s = kNone;
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        kb[j] = vid >= 0 ? (vid == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
        s = kb[j];
      } else {
        uint32_t w[4] = {key2(raw[j].x), key2(raw[j].y), key2(raw[j].z), key2(raw[j].w)};
        if (j == jt) mask_tail(w, vid >= 0 ? clamp8(v - 8 * vid) : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) kw[j][i] = w[i];
        // sample: element (j & 7) of the vector, element 0 if that is past v
        const int e = (j / kSampleEvery) & 7;
        s = (vid * 8 + e < v) ? half_of(w[e >> 1], e & 1) : (w[0] & 0xFFFFu);
      }
      if (j % kSampleEvery == 0) {
        sk[j / kSampleEvery] = vid >= 0 ? s : kNone;
        S += (uint32_t)(j < jt ? kNT : (j == jt ? rem : 0));
      }
    }
    const uint32_t q = sample_rank((uint32_t)k, (uint32_t)n, S);
    __syncthreads();  // histograms zeroed
    const uint32_t c = sample_cutoff(sk, q, sh);

    if (MODE == TOPK_MODE_TOKEN && c == 0u) {
      // a zero cutoff would admit the zero keys of slots past the length
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    } else {
      // -- filter + compaction of the keys above the cutoff
      const uint32_t lcw = (uint32_t)p.lcw;
      uint32_t* seg = lists + wave * lcw;
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j <= jt) {
          const uint32_t vid = (uint32_t)slot_vid(j, jt, rem);  // keys of -1 slots are 0
          if constexpr (MODE == TOPK_MODE_BLOCK) {
            keep_above(kb[j], vid, c, seg, lcw, cnt);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              keep_above(half_of(kw[j][e >> 1], e & 1), (vid << 3) | (uint32_t)e, c, seg, lcw,
                         cnt);
          }
        }
      }
      if (lane == 0) bc[BC_CNT + wave] = cnt;
      __syncthreads();
      uint32_t gt_total = 0, before = 0;
      bool ovf = false;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint32_t cw = bc[BC_CNT + w];
        before += w < wave ? cw : 0u;
        gt_total += cw;
        ovf |= cw > lcw;
      }
      if (ovf) {
        direct = true;
        code = TOPK_PATH_DIRECT_OVERFLOW;
      } else if (gt_total >= (uint32_t)k) {
        // the k-th key lies above the cutoff: exact select over the survivors
        select_and_write(SegView{seg}, cnt, c, (uint32_t)k, rel, sh, bc, o);
        code = TOPK_PATH_SAMPLED;
      } else {
        // the k-th key can only be the cutoff: collect keys equal to it
        uint16_t* ties = reinterpret_cast<uint16_t*>(rel);  // room for 2 kRelBins >= k
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          if (j <= jt) {
            const uint32_t vid = (uint32_t)slot_vid(j, jt, rem);
            if constexpr (MODE == TOPK_MODE_BLOCK) {
              keep_equal(kb[j], vid, c, ties, (uint32_t)k, &bc[BC_EQ]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                keep_equal(half_of(kw[j][e >> 1], e & 1), (vid << 3) | (uint32_t)e, c, ties,
                           (uint32_t)k, &bc[BC_EQ]);
            }
          }
        }
        __syncthreads();
        const uint32_t eq_total = bc[BC_EQ];
        if (gt_total + eq_total < (uint32_t)k) {
          direct = true;
          code = TOPK_PATH_DIRECT_MISJUDGED;
        } else {
          for (uint32_t i = lane; i < cnt; i += 64) o.put(before + i, seg[i] & 0xFFFFu, seg[i] >> 16);
          const uint32_t take = (uint32_t)k - gt_total;
          for (uint32_t i = tid; i < take; i += kNT) o.put(gt_total + i, ties[i], c);
          code = TOPK_PATH_SAMPLED_TIES;
        }
      }
    }
  }
  if (direct) {
    __syncthreads();
    direct_select<MODE>(src, v, n, k, o, lists, bc);
  }
  set_path(p, row, code);
}

// ============================================ team of workgroups per row
// Stage 1: every member of a row's team stages its chunk of the row (the
// chunks split the valid length), derives the row's cutoff from samples
// spread over the whole row (the same in every member), and writes the
// keys above it, and if any, the keys equal to it, to its scratch slice.
template <int MODE, int VPT, int SV>
__global__ __launch_bounds__(kNT) void topk_team_filter(Params p) {
  __shared__ uint32_t sh[512];
  __shared__ uint32_t bc[64];
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
  const int lane = __lane_id();
  const int wave = tid >> 6;
  const int k = p.k;
  const int v = clamp_len(p.valid_len[row], p.width);
  const int n = (MODE == TOPK_MODE_BLOCK) ? (v + 7) >> 3 : v;
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);

  if (n <= k) {
    if (member == 0) {
      const Out o = row_out(p, row, MODE == TOPK_MODE_BLOCK);
      if constexpr (MODE == TOPK_MODE_BLOCK) write_short_block(o, src, n, k);
      else write_short_token(o, n, k);
      set_path(p, row, TOPK_PATH_SHORT);
    }
    return;
  }
  if (p.force_direct) return;  // the select stage takes the whole row
  uint32_t* slice = p.team + ((size_t)lrow * G + member) * kMemberWords;
  const int nvec = (v + 7) >> 3;
  const int per = (nvec + G - 1) / G;
  const int vb = min(member * per, nvec);
  const int ve = min(vb + per, nvec);
  const int jt = ve > vb ? (ve - vb - 1) / kNT : -1;  // last occupied slot
  const int rem = (ve - vb) - jt * kNT;               // vectors in it
  for (int i = tid; i < 512; i += kNT) sh[i] = 0;
  if (tid == 0) bc[BC_EQ] = 0;

  // -- chunk loads and sample loads, all issued before any use
  uint4 raw[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int lvid = slot_vid(j, jt, rem);
    raw[j] = lvid >= 0 ? src[vb + lvid] : make_uint4(0u, 0u, 0u, 0u);
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
  // block keys right away, so the raw vectors die early
  uint32_t kb[MODE == TOPK_MODE_BLOCK ? VPT : 1];
  if constexpr (MODE == TOPK_MODE_BLOCK) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int lvid = slot_vid(j, jt, rem);
      kb[j] = lvid >= 0 ? (vb + lvid == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
    }
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
  const uint32_t S = block_sum(my_samples, bc + BC_TMP);  // also publishes the zeroed hists
  const uint32_t q = sample_rank((uint32_t)k, (uint32_t)n, S);
  const uint32_t c = sample_cutoff(sk, q, sh);
  if (MODE == TOPK_MODE_TOKEN && c == 0u) {
    // a zero cutoff would admit the zero keys of slots past the length:
    // every member sees the same cutoff and flags the row for the direct path
    if (tid == 0) {
      slice[5] = c;
      slice[6] = kFlagDirect;
    }
    return;
  }

  // -- keys of the chunk; the ones above the cutoff go straight to scratch
  uint32_t* seg = slice + kMemberHdr + wave * kTeamLCW;
  uint32_t cnt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    if (j <= jt) {
      const int lvid = slot_vid(j, jt, rem);
      const int vid = vb + lvid;
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        keep_above(kb[j], (uint32_t)lvid, c, seg, kTeamLCW, cnt);
        neq += (uint32_t)__popcll(__ballot(kb[j] == c));
      } else {
        uint32_t w[4] = {key2(raw[j].x), key2(raw[j].y), key2(raw[j].z), key2(raw[j].w)};
        if (j == jt) mask_tail(w, lvid >= 0 ? clamp8(v - 8 * vid) : 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t key = half_of(w[e >> 1], e & 1);
          keep_above(key, ((uint32_t)lvid << 3) | (uint32_t)e, c, seg, kTeamLCW, cnt);
          neq += (uint32_t)__popcll(__ballot(key == c));
        }
      }
    }
  }
  if (lane == 0) {
    slice[wave] = cnt;
    bc[BC_CEQ + wave] = neq;
  }
  __syncthreads();
  const uint32_t eq_total = bc[BC_CEQ] + bc[BC_CEQ + 1] + bc[BC_CEQ + 2] + bc[BC_CEQ + 3];
  if (eq_total) {
    // second pass: up to k chunk-local indices of keys equal to the cutoff
    uint16_t* ties = reinterpret_cast<uint16_t*>(slice + kMemberHdr + 4 * kTeamLCW);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      if (j <= jt) {
        const int lvid = slot_vid(j, jt, rem);
        const int vid = vb + lvid;
        if constexpr (MODE == TOPK_MODE_BLOCK) {
          keep_equal(kb[j], (uint32_t)lvid, c, ties, (uint32_t)k, &bc[BC_EQ]);
        } else {
          uint32_t w[4] = {key2(raw[j].x), key2(raw[j].y), key2(raw[j].z), key2(raw[j].w)};
          if (j == jt) mask_tail(w, lvid >= 0 ? clamp8(v - 8 * vid) : 0);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            keep_equal(half_of(w[e >> 1], e & 1), ((uint32_t)lvid << 3) | (uint32_t)e, c, ties,
                       (uint32_t)k, &bc[BC_EQ]);
        }
      }
    }
  }
  if (tid == 0) {
    slice[4] = eq_total;
    slice[5] = c;
    slice[6] = 0u;
  }
}

// Survivors staged in LDS by the select kernel.
struct StageView {
  const uint16_t* keys;
  const uint32_t* idxs;
  __device__ __forceinline__ uint32_t key(uint32_t i) const { return keys[i]; }
  __device__ __forceinline__ uint32_t idx(uint32_t i) const { return idxs[i]; }
};

// LDS of the select kernel (words), after the shared first kLists words
constexpr int kSelPrefix = kLists;                     // 4 G + 1 segment starts, G + 1 tie starts
constexpr int kSelStage = kSelPrefix + 512;            // u16 keys, then u32 indices
constexpr int kSelWords = kSelStage + kSelectMax / 2 + kSelectMax;

// Index of the segment holding flattened entry i: the last s with
// start[s] <= i (start[0] = 0, nseg + 1 entries).
__device__ __forceinline__ int find_segment(const uint32_t* start, int nseg, uint32_t i) {
  int lo = 0, hi = nseg;  // start[lo] <= i < start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (start[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Stage 2: one workgroup per row reads the team's slices (written by the
// previous kernel, so plain loads see them), checks the cutoff held, and
// writes the row: exact select over the survivors, the tie pass, or the
// direct path.
template <int MODE>
__global__ __launch_bounds__(kNT) void topk_team_select(Params p) {
  extern __shared__ uint32_t smem[];
  const int lrow = blockIdx.x;
  const int row = p.row0 + lrow;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = tid >> 6;
  const int k = p.k;
  const int G = p.G;
  const int v = clamp_len(p.valid_len[row], p.width);
  const int n = (MODE == TOPK_MODE_BLOCK) ? (v + 7) >> 3 : v;
  if (n <= k) return;  // written by the filter stage
  const Out o = row_out(p, row, MODE == TOPK_MODE_BLOCK);
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
  uint32_t* sh = smem + kSampHist;
  uint32_t* rel = smem + kRelHist;
  uint32_t* bc = smem + kBc;
  uint32_t* start = smem + kSelPrefix;          // 4G + 1 segment starts
  uint32_t* tstart = start + 4 * G + 1;         // G + 1 tie-list starts
  uint16_t* skeys = reinterpret_cast<uint16_t*>(smem + kSelStage);
  uint32_t* sidx = smem + kSelStage + kSelectMax / 2;
  bool direct = p.force_direct != 0;
  int code = TOPK_PATH_DIRECT_FORCED;
  if (!direct) {
    const uint32_t* slices = p.team + (size_t)lrow * G * kMemberWords;
    const int nvec = (v + 7) >> 3;
    const int per = (nvec + G - 1) / G;
    const uint32_t scale = (MODE == TOPK_MODE_BLOCK) ? 1u : 8u;
    for (int i = tid; i < 512 + kRelBins; i += kNT) smem[i] = 0;
    // segment sizes -> starts (block-wide inclusive scan; 4 G <= kNT)
    uint32_t sz = 0, bad = 0;
    if (tid < 4 * G) {
      sz = slices[(size_t)(tid >> 2) * kMemberWords + (tid & 3)];
      bad = sz > (uint32_t)kTeamLCW ? 1u : 0u;
    }
    uint32_t tz = 0, ties = 0;
    if (tid < G) {
      ties = slices[(size_t)tid * kMemberWords + 4];
      tz = min(ties, (uint32_t)k);
      bad |= slices[(size_t)tid * kMemberWords + 6] ? 2u : 0u;
    }
    const uint32_t incl = wave_incl_scan(sz);
    const uint32_t tincl = wave_incl_scan(tz);
    const uint32_t eqsum = wave_incl_scan(ties);
    const unsigned long long anybad = __ballot((bad & 1u) != 0);
    const unsigned long long anyflag = __ballot((bad & 2u) != 0);
    if (lane == 63) {
      bc[BC_TMP + wave] = incl;
      bc[BC_X + wave] = eqsum;
    }
    if (lane == 0) {
      bc[BC_CGT + wave] = anybad ? 1u : 0u;
      bc[BC_CEQ + wave] = anyflag ? 1u : 0u;
    }
    __syncthreads();
    uint32_t off = 0, gt_total = 0, eq_total = 0, flagged = 0, broken = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      off += w < wave ? bc[BC_TMP + w] : 0u;
      gt_total += bc[BC_TMP + w];
      eq_total += bc[BC_X + w];
      broken |= bc[BC_CGT + w];
      flagged |= bc[BC_CEQ + w];
    }
    if (tid < 4 * G) start[tid + 1] = off + incl;
    if (tid == 0) start[0] = 0;
    if (tid < G) tstart[tid + 1] = tincl;  // G <= 64: the first wave holds them all
    if (tid == 0) tstart[0] = 0;
    const uint32_t c = slices[5];
    __syncthreads();
    if (flagged) {
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    } else if (broken) {
      direct = true;
      code = TOPK_PATH_DIRECT_OVERFLOW;
    } else if (gt_total + eq_total < (uint32_t)k) {
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    } else if (gt_total >= (uint32_t)k) {
      if (gt_total > (uint32_t)kSelectMax) {
        direct = true;
        code = TOPK_PATH_DIRECT_OVERFLOW;
      } else {
        // stage every survivor in LDS: key, row index
#pragma unroll 8
        for (uint32_t i = tid; i < gt_total; i += kNT) {
          const int s = find_segment(start, 4 * G, i);
          const int g = s >> 2;
          const uint32_t e =
              slices[(size_t)g * kMemberWords + kMemberHdr + (s & 3) * kTeamLCW + (i - start[s])];
          skeys[i] = (uint16_t)(e >> 16);
          sidx[i] = (uint32_t)(g * per) * scale + (e & 0xFFFFu);
        }
        __syncthreads();
        const uint32_t quarter = (gt_total + kWaves - 1) / kWaves;
        const uint32_t lo = min((uint32_t)wave * quarter, gt_total);
        const uint32_t hi = min(lo + quarter, gt_total);
        select_and_write(StageView{skeys + lo, sidx + lo}, hi - lo, c, (uint32_t)k, rel, sh, bc, o);
        code = TOPK_PATH_SAMPLED;
      }
    } else {
      // the k-th key is the cutoff: every survivor above it, then ties
#pragma unroll 8
      for (uint32_t i = tid; i < gt_total; i += kNT) {
        const int s = find_segment(start, 4 * G, i);
        const int g = s >> 2;
        const uint32_t e =
            slices[(size_t)g * kMemberWords + kMemberHdr + (s & 3) * kTeamLCW + (i - start[s])];
        o.put(i, (uint32_t)(g * per) * scale + (e & 0xFFFFu), e >> 16);
      }
      const uint32_t take = (uint32_t)k - gt_total;
      for (uint32_t j = tid; j < take; j += kNT) {
        const int g = find_segment(tstart, G, j);
        const uint16_t* tl =
            reinterpret_cast<const uint16_t*>(slices + (size_t)g * kMemberWords + kMemberHdr +
                                              4 * kTeamLCW);
        o.put(gt_total + j, (uint32_t)(g * per) * scale + tl[j - tstart[g]], c);
      }
      code = TOPK_PATH_SAMPLED_TIES;
    }
  }
  if (direct) {
    __syncthreads();
    direct_select<MODE>(src, v, n, k, o, smem + kLists, bc);
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

// Team scratch: one slice of kMemberWords words per (row, member) of a
// launch.  Every word the select kernel reads is written by the filter
// kernel of the same call, so nothing needs zeroing between calls.
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
    sc.bytes = need;
  }
  *out = sc.base;
  return TOPK_OK;
}

// Survivor slots per wave of the one-workgroup kernel: about 1.3 times the
// expected survivors of a 16384-logit row plus a margin, capped so that the
// kernel's LDS stays at 20 KB (eight rows in flight per CU).
int row_lcw(int k) {
  const int l = k / 2 + 96;
  return l > 880 ? 880 : l;
}

size_t row_lds_bytes(int lcw) {
  const int lists = 4 * lcw > kDirectWords ? 4 * lcw : kDirectWords;
  return (size_t)(kLists + lists) * 4;
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
    const size_t lds = row_lds_bytes(p.lcw);
    if (mode == TOPK_MODE_BLOCK)
      return launch(topk_rows_wg<TOPK_MODE_BLOCK, kBlockVPT>, rows, lds, stream, p);
    return launch(topk_rows_wg<TOPK_MODE_TOKEN, kTokenVPT>, rows, lds, stream, p);
  }

  // team path: a filter kernel (G members a row), then a select kernel
  const int G = (nvec_max + cap_wg - 1) / cap_wg;  // <= 64, so 4 G <= kNT
  const size_t row_bytes = (size_t)G * kMemberWords * 4;
  int batch = rows < kTeamBatch ? rows : kTeamBatch;
  if ((size_t)batch * row_bytes > kTeamScratchMax) batch = (int)(kTeamScratchMax / row_bytes);
  if (batch < 1) batch = 1;
  void* scratch = nullptr;
  int rc = get_scratch(stream, (size_t)batch * row_bytes, &scratch);
  if (rc != TOPK_OK) return rc;
  p.G = G;
  p.team = static_cast<uint32_t*>(scratch);
  const size_t sel_lds = (size_t)kSelWords * 4;
  for (int r0 = 0; r0 < rows; r0 += batch) {
    const int nr = (rows - r0) < batch ? (rows - r0) : batch;
    p.row0 = r0;
    p.rows = nr;
    p.xcd_map = nr >= 8 ? 1 : 0;
    const int grid = p.xcd_map ? ((nr + 7) / 8) * 8 * G : nr * G;
    if (mode == TOPK_MODE_BLOCK) {
      rc = launch(topk_team_filter<TOPK_MODE_BLOCK, kBlockVPT, kBlockSV>, grid, 0, stream, p);
      if (rc == TOPK_OK) rc = launch(topk_team_select<TOPK_MODE_BLOCK>, nr, sel_lds, stream, p);
    } else {
      rc = launch(topk_team_filter<TOPK_MODE_TOKEN, kTokenVPT, kTokenSV>, grid, 0, stream, p);
      if (rc == TOPK_OK) rc = launch(topk_team_select<TOPK_MODE_TOKEN>, nr, sel_lds, stream, p);
    }
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
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_scratch) {
    if (kv.second.base) {
      (void)hipSetDevice(kv.first.first);
      hipError_t e = hipStreamSynchronize(kv.first.second);
      if (e == hipSuccess) e = hipFree(kv.second.base);
      if (e != hipSuccess) rc = fail(TOPK_ERR_HIP, "release: %s", hipGetErrorString(e));
    }
  }
  (void)hipSetDevice(cur);
  g_scratch.clear();
  return rc;
}

}  // extern "C"
