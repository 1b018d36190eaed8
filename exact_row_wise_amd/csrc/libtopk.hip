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
//     VGPRs, and stays there as raw BF16 words;
//   * a cutoff c is taken from a sample of the row: the q-th largest
//     sample, q scaled from k with a margin so that at least k keys lie at
//     or above c with overwhelming probability; two 8-bit LDS radix passes
//     over the sampled keys find it, and every wave reads the bins itself;
//   * words holding a key above c are compacted, two logits per wave64
//     ballot step, into the wave's own LDS region (ballot + lane-mask
//     count, no atomic).  Survivor words hold signed keys (key - 0x8000 in
//     each half); when c is the key of a non-negative value the raw word
//     already serves, so the key transform never touches the whole row;
//   * the exact k-th key T over the survivors takes one pass of a 256-bin
//     LDS histogram of (key - c), kept in 4 copies (lane mod 4) so that the
//     many equal keys near c seldom meet on one word, which gives T itself
//     whenever T - c < 256 (else two 8-bit passes); the write pass takes
//     output slots from one LDS counter pair, one atomic per wave and 64
//     entries, and writes each index straight to the row's output through
//     the block table (an LDS copy of the row's entries where it fits);
//   * rows whose k-th key equals the cutoff take the tie pass: every key
//     above c, then the first keys equal to c;
//   * a misjudged sample (fewer than k keys at or above c) or a survivor
//     overflow sends the row to the direct path: two whole-row 8-bit radix
//     histograms, every atomic spread over 8 replicated bins (lane mod 8);
//   * rows wider than one workgroup's registers are split over a team of
//     workgroups.  Every member derives the same cutoff from the same
//     samples, then loads its chunk and writes its survivors, with a
//     histogram of their keys relative to the cutoff, to its own slice of
//     global scratch; a second kernel, one 1024-thread workgroup per row,
//     takes the k-th key from the summed histograms after the kernel
//     boundary and writes the row from the members' lists.  No workgroup
//     ever waits for another, no atomic or fence crosses workgroups, and the
//     scratch needs no reset.
// There is no MFMA: this is a memory-bound selection, and all selection
// arithmetic is on integer keys.

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <tuple>
#include <mutex>
#include <utility>

#include "libtopk.h"

namespace {

constexpr int kCopies = 8;               // replicated bins of whole-row histograms
constexpr int kCopyStride = 260;         // words between the copies of a replicated sample bin
constexpr int kSampBins = kCopies * kCopyStride;  // words of the replicated sample bins
constexpr int kTeamNT = 256;             // filter workgroup size
constexpr int kSelNT = 1024;             // select workgroup size
constexpr int kRowNT = 512;              // one-workgroup-per-row size
constexpr int kRowTokenVPT = 4;          // 16-byte vectors per thread, one-workgroup token rows
constexpr int kRowBlockVPT = 8;          // 16-byte vectors per thread, one-workgroup block rows
constexpr int kWideNT = 1024;            // one-workgroup token rows when all are resident
constexpr int kWideTokenVPT = 2;         // 16-byte vectors per thread at that size
constexpr int kTeamBlockVPT = 12;        // 16-byte vectors per thread of a block work item
constexpr int kTokenSV = 1;              // sample vectors per thread, token cutoff kernel
constexpr int kBlockSV = 4;              // sample vectors per thread, block cutoff kernel
constexpr int kMaxMembers = 64;          // members of a row at most (4 segments each <= 256)
constexpr int kSpare = 64;               // region entries past the cap (one ballot step)
constexpr int kTieLCW = TOPK_MAX_K / 4 + 128;     // tie entries per wave region of a member
constexpr int kTeamBatch = 1024;         // rows per team launch at most
constexpr size_t kTeamScratchMax = size_t(256) << 20;
constexpr int kRelBins = 256;            // histogram bins of (key - cutoff): 4 per lane
constexpr int kRelCopies = 4;            // copies of those bins (lane mod 4)
constexpr int kRelStride = 276;          // words per copy: the bins, then per-lane spill words
constexpr int kRelWords = kRelCopies * kRelStride;
constexpr int kRowLoCopies = 2;           // copies of the low-byte sample bins, one-workgroup kernel
constexpr int kDirectWords = 256 * kCopies + 256;   // direct path LDS words
constexpr int kPageLdsMax = 1024;        // block-table entries a one-workgroup row copies to LDS
constexpr int kAllSampled = 512;         // token rows of at most this many vectors: every logit sampled

constexpr uint32_t kKeyNegInf = 0x007Fu; // key(-inf)
constexpr uint32_t kKeyPosInf = 0xFF80u; // key(+inf): the pinned newest block
constexpr uint32_t kKeyNaN = 0xFFFFu;    // key of the canonical positive NaN
constexpr uint32_t kNone = 0xFFFFFFFFu;  // empty sample slot
constexpr int32_t kSNegInf = (int32_t)kKeyNegInf - 0x8000;  // signed key of -inf
constexpr uint32_t kDeadPair = 0x80008000u;  // two signed keys at the very bottom

// LDS (32-bit words), shared by the one-workgroup and the select kernels
constexpr int kBc = 0;                          // 128 words of counters and per-wave fields
constexpr int kHists = 128;                     // histograms:
constexpr int kSampHist = kHists;               //   low-byte sample bins / 2 x 256 fallback bins
constexpr int kRelHist = kHists + 552;          //   kRelWords of relative bins / u16 ties
static_assert(kRowLoCopies * kRelStride <= kRelHist - kSampHist && kRelHist - kSampHist >= 512,
              "low-byte sample bins, fallback bins");
constexpr int kLists = kRelHist + kRelWords;    // survivor entries / direct path
static_assert(kLists % 4 == 0, "16-byte aligned lists");
static_assert(kRelBins + 16 <= kRelStride && (kRelStride * 4) % 16 == 0, "relative bin copies");
static_assert(2 * kRelWords >= TOPK_MAX_K, "the u16 tie list fits the relative bins");
enum {
  BC_CNT = 0,     // 16: entries per wave
  BC_ECNT = 16,   // 16: survivor keys per wave
  BC_EQ = 64,     // tie-list counter
  BC_C1 = 65, BC_C2 = 66,   // direct-path write counters
  BC_SLOT = 68,   // 2 (8-byte aligned): output slots taken above T | equal to T
  BC_TMP = 96     // 32: reductions, a team row's totals, the select's bin search
};

// One team member's slice of global scratch (32-bit words):
//   [0, 32)                 header (MH_* fields)
//   [32, 160)               256-bin histogram of its survivors' keys relative
//                           to the cutoff, two 16-bit bins to a word
//   [160, 160 + 2 kMemberCap)  its survivor entries, one list (2 words each)
//   then the waves' tie entries (kTieLCW each, 2 words each)
constexpr int kFiltStage = (kSampBins + 256 + kRelWords - 128) / 8;  // LDS entries a filter wave holds
constexpr int kFiltCap = kFiltStage - 64;                             // kept before the overflow
constexpr int kMemberCap = 4 * kFiltCap;
constexpr int kMemberHistOfs = 32;
constexpr int kMemberList = kMemberHistOfs + kRelBins / 2;
constexpr int kMemberTies = kMemberList + 2 * kMemberCap;
constexpr int kMemberWords = kMemberTies + 4 * 2 * kTieLCW;
constexpr int MH_E = 0, MH_TKEPT = 2, MH_NEQ = 3, MH_TW = 4, MH_CUT = 8, MH_FLAGS = 9,
              MH_TDROP = 12;
constexpr uint32_t kFlagDirect = 1u;    // a zero token cutoff: the direct path
constexpr uint32_t kFlagOverflow = 2u;  // a wave kept more entries than its region holds
constexpr uint32_t kFlagTies = 4u;      // the keys equal to the cutoff were kept
static_assert(kMemberList % 4 == 0 && kMemberTies % 2 == 0, "aligned lists");
static_assert((TOPK_MAX_WIDTH / 8 + kTeamNT * 8 - 1) / (kTeamNT * 8) <= kMaxMembers,
              "too many token members per row");
static_assert((TOPK_MAX_WIDTH / 8 + kTeamNT * kTeamBlockVPT - 1) / (kTeamNT * kTeamBlockVPT) <=
                  kMaxMembers, "too many block members per row");
static_assert(4 * kMaxMembers <= 1024, "the select's segment arrays hold every segment");

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
  int32_t lcw;         // survivor entries per wave before the cap (one-workgroup kernel)
  int32_t page_lds;    // LDS word offset of a row's block-table copy (one-workgroup kernel), or 0
  // team path (rows wider than one workgroup), all in one scratch buffer:
  int32_t G;             // team members per row (for the widest row)
  int32_t team_cv;       // 16-byte vectors of one member
  uint32_t* team_slices; // [rows][G][kMemberWords]
  int32_t sel_bw;        // ordered results: bitmap words over one member's elements
  int32_t sel_parts;     // ordered results: select workgroups per row (members 16 each)
  // ordered results (ascending element index, lowest-index ties):
  int32_t ord;           // 1: ordered results, with counts and logical ids
  int32_t* valid;        // [rows] counts, or null
  int32_t* ids;          // [rows][k] logical element indices, or null
  // vector-max bound: the producer's maxima of every 8 logits, and the LDS
  // word offset of the per-wave hot-vector lists
  const uint16_t* tops;  // [rows][tops_stride], or null
  int64_t tops_stride;
  int32_t hot_lds;
  int32_t tops_lo;       // LDS word offset of the bound's low-byte bins
};

// Row of workgroup b of a one-workgroup-per-row launch.  Workgroups go to
// the XCDs round robin (b mod 8), so with b itself as the row, row r would
// always run on XCD r mod 8, and rows whose cost follows a period of the
// row index that shares a factor with 8 (every tenth row costly: all of
// them odd) would load some XCDs more than others, which then finish last.
// Each group of 8 consecutive rows still goes to the 8 XCDs, one row each,
// but rotated by the top 3 bits of a Fibonacci hash of the group index, so
// that every XCD draws its rows from all residues of any period; a last
// group of fewer than 8 rows keeps b.
__device__ __forceinline__ int spread_row(const Params& p, int b) {
  const int g = b & ~7;
  if (g + 8 > p.rows) return b;
  const uint32_t h = ((uint32_t)(b >> 3) * 2654435761u) >> 29;
  return g + (int)(((uint32_t)b + h) & 7u);
}

// ------------------------------------------------------------------ keys
// Two BF16 patterns in one word -> their two keys in the same halves:
// a half with the sign bit set is inverted entirely, any other half only
// its sign bit (sglang PR #39305, "What is kept from DeepSelect").
__device__ __forceinline__ uint32_t key2(uint32_t w) {
  const uint32_t neg = w & 0x80008000u;
  const uint32_t flip = neg - (neg >> 15);  // 0x7FFF in each negative half
  return w ^ flip ^ 0x80008000u;
}

__device__ __forceinline__ uint32_t key1(uint32_t x) {
  return (x & 0x8000u) ? (x ^ 0xFFFFu) : (x ^ 0x8000u);
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Signed keys: key - 0x8000 as a signed 16-bit number, same order as the
// key.  For a word of two BF16 patterns that is the word with the low 15
// bits of each negative half inverted (a non-negative half is its own
// signed key).
__device__ __forceinline__ uint32_t skey2(uint32_t w) {
  const s16x2 sm = __builtin_bit_cast(s16x2, w) >> (s16x2){15, 15};
  return w ^ (__builtin_bit_cast(uint32_t, sm) & 0x7FFF7FFFu);
}

__device__ __forceinline__ int32_t lo16s(uint32_t x) { return (int32_t)(int16_t)(x & 0xFFFFu); }
__device__ __forceinline__ int32_t hi16s(uint32_t x) { return (int32_t)x >> 16; }

__device__ __forceinline__ uint32_t pk_max_s(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, a),
                                                                __builtin_bit_cast(s16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_s(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2, a),
                                                                __builtin_bit_cast(s16x2, b)));
}

// Key of the NaN-propagating maximum of the 8 logits of one 16-byte vector
// (decode_topk_cute, block_key / max_nan_bf16x2): a NaN of either sign
// anywhere gives the canonical positive NaN; otherwise the largest key.
// Taken over signed keys with packed 16-bit max/min: a NaN is a signed key
// above that of +inf or below that of -inf.
__device__ __forceinline__ uint32_t block_key4(uint4 v) {
  const uint32_t a = skey2(v.x), b = skey2(v.y), c = skey2(v.z), d = skey2(v.w);
  const uint32_t mx = pk_max_s(pk_max_s(a, b), pk_max_s(c, d));
  const uint32_t mn = pk_min_s(pk_min_s(a, b), pk_min_s(c, d));
  const int32_t hi = max(lo16s(mx), hi16s(mx));
  const int32_t lo = min(lo16s(mn), hi16s(mn));
  return (hi > (int32_t)kKeyPosInf - 0x8000 || lo < kSNegInf) ? kKeyNaN : (uint32_t)(hi + 0x8000);
}

// Vector i of a row (a 32-bit byte offset from the row's base: one scalar
// base and one vector register per load)
__device__ __forceinline__ uint4 ld_vec(const uint4* row, uint32_t i) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(row) + (i << 4));
}

__device__ __forceinline__ uint32_t half_of(uint32_t w, int h) {
  return h ? (w >> 16) : (w & 0xFFFFu);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Overwrite elements r..7 of one staged vector (r valid elements, 0..8)
// with 0xFFFF, whose key is 0 and whose signed value is -1: such an element
// is never above a cutoff.  Only the last occupied vector slot needs it.
// The first r of the 8 halves of v kept, the rest zeroed.
__device__ __forceinline__ void keep_first(uint4& v, int r) {
  v.x &= r >= 2 ? 0xFFFFFFFFu : (r == 1 ? 0x0000FFFFu : 0u);
  v.y &= r >= 4 ? 0xFFFFFFFFu : (r == 3 ? 0x0000FFFFu : 0u);
  v.z &= r >= 6 ? 0xFFFFFFFFu : (r == 5 ? 0x0000FFFFu : 0u);
  v.w &= r >= 8 ? 0xFFFFFFFFu : (r == 7 ? 0x0000FFFFu : 0u);
}

__device__ __forceinline__ void poison_tail(uint4& v, int r) {
  v.x |= r >= 2 ? 0u : (r == 1 ? 0xFFFF0000u : 0xFFFFFFFFu);
  v.y |= r >= 4 ? 0u : (r == 3 ? 0xFFFF0000u : 0xFFFFFFFFu);
  v.z |= r >= 6 ? 0u : (r == 5 ? 0xFFFF0000u : 0xFFFFFFFFu);
  v.w |= r >= 8 ? 0u : (r == 7 ? 0xFFFF0000u : 0xFFFFFFFFu);
}

// a - b, or 0 when b >= a.  A guarded subtraction written as a comparison
// and a difference can be hoisted out of its guard with a no-wrap flag
// kept, from which the optimizer then wrongly concludes a >= b for every
// other use of the pair (it folded min(b, a) into b); the saturating
// builtin carries no such flag.
__device__ __forceinline__ uint32_t sat_sub(uint32_t a, uint32_t b) {
  return __builtin_elementwise_sub_sat(a, b);
}

__device__ __forceinline__ int clamp8(int x) { return x < 0 ? 0 : (x > 8 ? 8 : x); }

__device__ __forceinline__ int clamp_len(int v, int width) {
  return v < 0 ? 0 : (v > width ? width : v);
}

// The vector a thread stages in slot j of a run of vectors whose last
// occupied slot is jt (holding rem vectors), or -1.  Full slots hold NT
// consecutive vectors, lane-ordered within each wave (coalesced 1 KB per
// wave load).  Slot jt gives each wave an equal consecutive share, so that
// every wave sees about the same number of keys whatever the length: the
// per-wave survivor regions stay balanced on short rows.
template <int NT>
__device__ __forceinline__ int slot_vid(int j, int jt, int rem, int tid = (int)threadIdx.x) {
  constexpr int NW = NT / 64;
  if (j < jt) return j * NT + tid;
  if (j > jt) return -1;
  const int lane = tid & 63, wave = tid >> 6;
  const int per_w = (rem + NW - 1) / NW;
  const int x = wave * per_w + lane;
  return (lane < per_w && x < rem) ? jt * NT + x : -1;
}

// ----------------------------------------------------------- wave tools
// Byte address in LDS of a pointer into shared memory (the low half of its
// generic address), computed once into a scalar register (left alone, the
// compiler recomputes the conversion's null test at every use).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(p);
  asm("" : "+s"(a));
  return a;
}
// Lanes of m take a, the others b: one vector select (the compiler would
// otherwise turn some of these into exec-mask branches).
__device__ __forceinline__ uint32_t pick(unsigned long long m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(m));
  return r;
}
// Store of the pair (lo, hi) at LDS byte address a (a plain 32-bit
// address, so that address arithmetic stays in single vector ops).
__device__ __forceinline__ void lds_store2(uint32_t a, uint32_t lo, uint32_t hi) {
  *reinterpret_cast<__attribute__((address_space(3))) unsigned long long*>(a) =
      ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t mbcnt(unsigned long long m, uint32_t add = 0u) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, add));
}

__device__ __forceinline__ uint32_t popc(unsigned long long m) {
  return (uint32_t)__popcll(m);
}

// True in exactly the lanes whose bit is set in the wave-uniform mask m:
// lets a ballot taken earlier serve as the branch mask itself.
__device__ __forceinline__ bool in_mask(unsigned long long m) {
  return __builtin_amdgcn_inverse_ballot_w64(m);
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

__device__ __forceinline__ uint32_t readfirst(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

// One wave over a 256-bin histogram (16-byte aligned) whose index 0 holds
// the largest keys: the first bin where the running count reaches `need`,
// and the count before it (decode_topk_cute, select_bin).  A lane holds 4
// bins; the lane that crosses `need` is found with one ballot, and the bin
// inside it with scalar code.  Every lane gets the answer.
__device__ __forceinline__ void find_desc(const uint32_t* hist, uint32_t need, uint32_t& bin,
                                          uint32_t& above, int tid = (int)threadIdx.x) {
  const int lane = (tid & 63);
  const uint4 h = *reinterpret_cast<const uint4*>(hist + lane * 4);
  const uint32_t s = h.x + h.y + h.z + h.w;
  const uint32_t incl = wave_incl_scan(s);
  const unsigned long long m = __ballot(incl >= need);
  const int L = m ? (__ffsll(m) - 1) : 63;
  uint32_t acc = readlane(incl - s, L);
  const uint32_t h0 = readlane(h.x, L), h1 = readlane(h.y, L), h2 = readlane(h.z, L);
  uint32_t pos = 3;
  if (acc + h0 >= need) {
    pos = 0;
  } else if (acc + h0 + h1 >= need) {
    pos = 1;
    acc += h0;
  } else if (acc + h0 + h1 + h2 >= need) {
    pos = 2;
    acc += h0 + h1;
  } else {
    acc += h0 + h1 + h2;
  }
  bin = (uint32_t)L * 4u + pos;
  above = acc;
}

// One wave over C copies of a 256-bin histogram (copy c at hist + c STRIDE,
// 16-byte aligned), index 0 holding the largest keys: as find_desc over the
// summed copies, with `total` the count of all bins.
template <int C, int STRIDE>
__device__ __forceinline__ void find_copies(const uint32_t* hist, uint32_t need, uint32_t& bin,
                                            uint32_t& above, uint32_t& total,
                                            uint32_t* count = nullptr, int tid = (int)threadIdx.x) {
  const int lane = (tid & 63);
  uint4 h = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const uint4 u = *reinterpret_cast<const uint4*>(hist + c * STRIDE + lane * 4);
    h.x += u.x;
    h.y += u.y;
    h.z += u.z;
    h.w += u.w;
  }
  const uint32_t s = h.x + h.y + h.z + h.w;
  const uint32_t incl = wave_incl_scan(s);
  total = readlane(incl, 63);
  const unsigned long long m = __ballot(incl >= need);
  const int L = m ? (__ffsll(m) - 1) : 63;
  uint32_t acc = readlane(incl - s, L);
  const uint32_t h0 = readlane(h.x, L), h1 = readlane(h.y, L), h2 = readlane(h.z, L);
  uint32_t pos = 3;
  if (acc + h0 >= need) {
    pos = 0;
  } else if (acc + h0 + h1 >= need) {
    pos = 1;
    acc += h0;
  } else if (acc + h0 + h1 + h2 >= need) {
    pos = 2;
    acc += h0 + h1;
  } else {
    acc += h0 + h1 + h2;
  }
  bin = (uint32_t)L * 4u + pos;
  above = acc;
  if (count) *count = pos == 0 ? h0 : (pos == 1 ? h1 : (pos == 2 ? h2 : readlane(h.w, L)));
}

// Sum over the workgroup (every thread gets the total).
template <int NT>
__device__ uint32_t block_sum(uint32_t x, uint32_t* tmp, int tid = (int)threadIdx.x) {
  const uint32_t incl = wave_incl_scan(x);
  if ((tid & 63) == 63) tmp[tid >> 6] = incl;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += tmp[w];
  __syncthreads();
  return t;
}

// A slot per predicated lane from one LDS counter: one atomic per wave.
__device__ __forceinline__ uint32_t wave_slot(bool pred, uint32_t* ctr,
                                              int tid = (int)threadIdx.x) {
  const unsigned long long m = __ballot(pred);
  uint32_t slot = 0;
  if (m) {
    const int leader = __ffsll(m) - 1;
    uint32_t base = 0;
    if ((tid & 63) == leader) base = atomicAdd(ctr, popc(m));
    slot = mbcnt(m, readlane(base, leader));
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

  // An element index (or -1) as written: through the block table when
  // there is one (vLLM kimi_k3 indexer, IndexerSelect.emit), -1 kept.
  __device__ __forceinline__ int32_t map(int32_t x) const {
    if (!pages) return x;
    const int32_t i = x < 0 ? 0 : x;
    const int32_t pg = pages[i >> shift];
    return x < 0 ? -1 : (pg << shift) | (i & ((1 << shift) - 1));
  }
  // Element index idx with key `key` into output slot pos: -1 for a -inf
  // block, otherwise map(idx).
  __device__ __forceinline__ void put(uint32_t pos, uint32_t idx, uint32_t key) const {
    if (pos >= k) return;
    out[pos] = (block && key == kKeyNegInf) ? -1 : map((int32_t)idx);
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

// An element index (or -1) as written, through the block table: the row's
// copy in LDS when `lpages` is given, else the table in global memory.
__device__ __forceinline__ int32_t map_out(const Out& o, const int32_t* lpages, int32_t x) {
  if (!lpages) return o.map(x);
  const int32_t i = x < 0 ? 0 : x;
  return x < 0 ? -1 : (lpages[i >> o.shift] << o.shift) | (i & ((1 << o.shift) - 1));
}

__device__ __forceinline__ void set_path(const Params& p, int row, int code,
                                         int tid = (int)threadIdx.x) {
  if (p.path && tid == 0) p.path[row] = code;
}

// Token rows with n <= k: 0..n-1 then -1, no logits read
// (decode_topk_cute result definition; kimi_k3 IndexerSelect bypass).
template <int NT>
__device__ void write_short_token(const Out o, int n, int k, int tid = (int)threadIdx.x) {
  for (int e = tid; e < k; e += NT) o.out[e] = o.map(e < n ? e : -1);
}

// Block rows with n <= k: every block in order, -1 for -inf blocks, the
// newest pinned at +inf, then -1 padding.
template <int NT>
__device__ void write_short_block(const Out o, const uint4* src, int n, int k,
                                  int tid = (int)threadIdx.x) {
  for (int b = tid; b < k; b += NT) {
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
// `region` holds kDirectWords words of LDS.  Returns the k-th key and the
// count of keys above it; with `ordered` nothing is written (the caller's
// ordered pass writes).
template <int MODE, int NT>
__device__ uint2 direct_select(const uint4* src, int v, int n, int k, const Out o,
                               uint32_t* region, uint32_t* bc, bool ordered = false,
                               int tid = (int)threadIdx.x) {
  const int copy = (tid & 63) & (kCopies - 1);
  const int nvec = (MODE == TOPK_MODE_BLOCK) ? n : (v + 7) >> 3;
  uint32_t* hist = region;
  uint32_t* sums = region + 256 * kCopies;
  uint32_t b1 = 0, a1 = 0, b2 = 0, a2 = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = tid; i < 256 * kCopies; i += NT) hist[i] = 0;
    if (tid == 0) {
      bc[BC_C1] = 0;
      bc[BC_C2] = 0;
    }
    __syncthreads();
    for (int vid = tid; vid < nvec; vid += NT) {
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
    if (tid < 256) {
      uint32_t s = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) s += hist[tid * kCopies + c];
      sums[255 - tid] = s;  // descending key order
    }
    __syncthreads();
    uint32_t bin, above;
    find_desc(sums, pass == 0 ? (uint32_t)k : (uint32_t)k - a1, bin, above, tid);
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
  if (ordered) return make_uint2(T, cgt);  // ordered results: the caller writes
  for (int vid = tid; vid < nvec; vid += NT) {
    const uint4 raw = src[vid];
    if constexpr (MODE == TOPK_MODE_BLOCK) {
      const uint32_t key = (vid == n - 1) ? kKeyPosInf : block_key4(raw);
      const bool gt = key > T, eq = key == T;
      const uint32_t s1 = wave_slot(gt, &bc[BC_C1], tid);
      if (gt) o.put(s1, (uint32_t)vid, key);
      const uint32_t s2 = wave_slot(eq, &bc[BC_C2], tid);
      if (eq && s2 < take) o.put(cgt + s2, (uint32_t)vid, key);
    } else {
      const uint32_t w[4] = {key2(raw.x), key2(raw.y), key2(raw.z), key2(raw.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t idx = (uint32_t)(vid * 8 + e);
        const uint32_t key = half_of(w[e >> 1], e & 1);
        const bool ok = (int)idx < v;
        const bool gt = ok && key > T, eq = ok && key == T;
        const uint32_t s1 = wave_slot(gt, &bc[BC_C1], tid);
        if (gt) o.put(s1, idx, key);
        const uint32_t s2 = wave_slot(eq, &bc[BC_C2], tid);
        if (eq && s2 < take) o.put(cgt + s2, idx, key);
      }
    }
  }
  return make_uint2(T, cgt);
}

// --------------------------------------------------------- sampled path
// Rank of the cutoff among S samples of an n-element row: k scaled to the
// sample plus a margin of ~4.5 standard deviations and a constant, so that
// fewer than k keys at or above the cutoff is a rare event (the row then
// falls back to the direct path; exactness never depends on this choice).
__device__ __forceinline__ uint32_t sample_rank(uint32_t k, uint32_t n, uint32_t S) {
  if (S >= n) return k;  // every element sampled: the cutoff is the k-th key
  // k S / n and the margin's square root in single precision with the
  // hardware's approximate reciprocal and root: they size the work only
  const float f0 = (float)(k * S) * __builtin_amdgcn_rcpf((float)n);
  const uint32_t q = (uint32_t)(f0 + 4.5f * __builtin_amdgcn_sqrtf(f0)) + 9u;
  return q < S ? q : S;
}

// Whether a cutoff with `above` of S samples strictly above it almost surely
// has at least k of the row's n keys above it: `above` at least the
// expected count at rank k plus 3 standard deviations and 3.
__device__ __forceinline__ bool tie_unlikely(uint32_t k, uint32_t n, uint32_t S, uint32_t above) {
  if (S >= n) return above >= k;  // every element sampled: exact
  const float f0 = (float)(k * S) * __builtin_amdgcn_rcpf((float)n);
  return (float)above >= f0 + 3.0f * __builtin_amdgcn_sqrtf(f0) + 3.0f;
}

// The q-th largest of the samples (kNone marks an empty slot; the first
// `lead` samples are known not to be empty): two 8-bit radix passes
// (decode_topk_cute, radix_select over the samples).  The high-byte pass
// counts into kCopies replicated bins (lane mod 8) at h8 (256 kCopies
// words, zeroed), since sampled keys of smooth data crowd a few high bytes
// and same-word LDS atomics serialize (copy c of bin b at word
// c kCopyStride + b: the copies of a bin lie in distinct banks); 256
// threads then sum the copies into h8 + kSampBins (256 words; h8 holds
// kSampBins + 256 words, zeroed but for the sums).  The low-byte pass
// counts into LC copies (lane mod LC) at lo8, each kRelStride words, laid
// out as the relative histogram (LC kRelStride words, zeroed; a sample
// outside the chosen high byte counts into a spill word of its lane).
// Every wave finds the bins itself.  `above` and `equal`, when given,
// receive the numbers of samples strictly above and equal to the returned
// key.
template <int NSK, int NT, int LC>
__device__ uint32_t sample_cutoff(const uint32_t (&sk)[NSK], int lead, uint32_t q, uint32_t* h8,
                                  uint32_t* lo8, uint32_t* above = nullptr,
                                  uint32_t* equal = nullptr, int tid = (int)threadIdx.x) {
  static_assert(NT >= 256, "one thread per high-byte bin");
  const uint32_t copy = (tid & 63) & (kCopies - 1);
#pragma unroll
  for (int i = 0; i < NSK; ++i) {
    if (i < lead || sk[i] != kNone) atomicAdd(&h8[copy * kCopyStride + 255u - (sk[i] >> 8)], 1u);
  }
  __syncthreads();
  uint32_t* sums = h8 + kSampBins;
  if (tid < 256) {
    uint32_t t = 0;
#pragma unroll
    for (int c = 0; c < kCopies; ++c) t += h8[c * kCopyStride + tid];
    sums[tid] = t;
  }
  __syncthreads();
  uint32_t i1, a1;
  find_desc(sums, q, i1, a1, tid);
  const uint32_t b1 = 255u - i1;
  uint32_t* const loc = lo8 + ((tid & 63) % LC) * kRelStride;
  const uint32_t spill = 256u + (((tid & 63) / LC) & 15);
#pragma unroll
  for (int i = 0; i < NSK; ++i) {
    const uint32_t x = sk[i];  // an empty slot's high byte is never b1
    atomicAdd(&loc[pick(__ballot((x >> 8) == b1), 255u - (x & 255u), spill)], 1u);
  }
  __syncthreads();
  uint32_t i2, a2, t2;
  find_copies<LC, kRelStride>(lo8, q - a1, i2, a2, t2, equal, tid);  // equal: samples at the cutoff
  if (above) *above = a1 + a2;  // samples strictly above the cutoff
  return (b1 << 8) | (255u - i2);
}

// Survivor entries: two words each, a word x of two signed keys and the
// element index of its low half.  Token entries are two neighbouring
// logits; a block entry holds its block's signed key in the low half and
// the bottom key in the high half.
//
// Compaction of one entry into LDS, without touching the exec mask: if
// either half of x is above the signed cutoff cs, (x, eidx) goes to this
// wave's region at the wave's running count plus the lane's rank among the
// kept lanes (ballot + lane-mask count, no atomic); a lane without a key
// above cs stores into its own slot of a dummy area (LDS byte address
// `dummy`).  One test per entry on the larger of its two keys.  at is the
// LDS byte address of the wave's next entry (wave-uniform); stores stop
// advancing at lim, so a region needs 64 entries past lim, and a final at
// above lim means the row overflowed.
__device__ __forceinline__ void keep_word_lds(uint32_t x, uint32_t eidx, int32_t cs, uint32_t lim,
                                              uint32_t dummy, uint32_t& at) {
  const unsigned long long m = __ballot(max(lo16s(x), hi16s(x)) > cs);
  // lane rank * 8 + the first free entry's address in one shift-add (left
  // to itself the compiler adds first and shifts after the select)
  uint32_t a;
  asm("v_lshl_add_u32 %0, %1, 3, %2" : "=v"(a) : "v"(mbcnt(m)), "s"(min(at, lim)));
  lds_store2(pick(m, a, dummy), x, eidx);
  asm("s_lshl3_add_u32 %0, %1, %2" : "=s"(at) : "s"(popc(m)), "s"(at));  // at += 8 * kept
}

// Block entries: signed key in the low half, the bottom key above it.
__device__ __forceinline__ uint32_t block_entry(uint32_t key) { return key ^ kDeadPair; }

// x clamped to [0, hi] (hi >= 0) in one vector op.
__device__ __forceinline__ int32_t clamp0(int32_t x, int32_t hi) {
  int32_t r;
  asm("v_med3_i32 %0, %1, 0, %2" : "=v"(r) : "v"(x), "v"(hi));
  return r;
}

// Entry lists handed to the passes below are padded: the entries from cnt
// up to the next multiple of 64 exist and hold dead pairs (both keys at
// the bottom), so a pass reads whole 64-entry chunks with no bounds test.
//
// Output slots of the keys above a threshold Ts and of the keys equal to
// it, from the entries at e: per 64 entries a wave takes its slots with one
// 64-bit LDS atomic on `slot` (keys above in the low word, equal in the
// high word).  Keys above take output slot `slot`, keys equal slot
// cgt + `slot` while that is below `take`; each is written straight to the
// row's output (through the block table, `lpages` its LDS copy or null).
// Block entries of -inf blocks write -1.
// Output slot i of a row (a 32-bit byte offset from the row's base: one
// scalar base and one vector register per store)
__device__ __forceinline__ void st_slot(int32_t* out, uint32_t i, int32_t v) {
  *reinterpret_cast<int32_t*>(reinterpret_cast<char*>(out) + (i << 2)) = v;
}

template <int MODE, bool GT, bool EQ>
__device__ void emit_entries(const uint32_t* e, uint32_t cnt, int32_t Ts, uint32_t cgt,
                             uint32_t take, unsigned long long* slot, const Out o,
                             const int32_t* lpages, int tid = (int)threadIdx.x) {
  const int lane = (tid & 63);
  int32_t* const out = o.out;
  for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
    const uint2 en = *reinterpret_cast<const uint2*>(e + 2 * (b0 + lane));
    const int32_t s0 = lo16s(en.x), s1 = hi16s(en.x);
    const unsigned long long g0 = GT ? __ballot(s0 > Ts) : 0ull;
    const unsigned long long g1 = GT ? __ballot(s1 > Ts) : 0ull;
    const unsigned long long q0 = EQ ? __ballot(s0 == Ts) : 0ull;
    const unsigned long long q1 = EQ ? __ballot(s1 == Ts) : 0ull;
    const uint32_t ng0 = popc(g0), nq0 = popc(q0);
    const uint32_t ng = ng0 + popc(g1), nq = nq0 + popc(q1);
    unsigned long long base = 0;
    if (lane == 0) base = atomicAdd(slot, (unsigned long long)ng | ((unsigned long long)nq << 32));
    const uint32_t bg = readfirst((uint32_t)base), bq = readfirst((uint32_t)(base >> 32));
    int32_t v0 = (int32_t)en.y;
    int32_t v1 = (int32_t)en.y + 1;
    if constexpr (MODE == TOPK_MODE_BLOCK) v0 = s0 == kSNegInf ? -1 : v0;
    if (o.pages) {
      v0 = map_out(o, lpages, v0);
      v1 = map_out(o, lpages, v1);
    }
    if (GT) {
      if (in_mask(g0)) st_slot(out, bg + mbcnt(g0), v0);
      if (in_mask(g1)) st_slot(out, (bg + ng0) + mbcnt(g1), v1);
    }
    if (EQ && nq) {  // keys equal to Ts are few: most chunks skip this
      // slots cgt + bq + rank while bq + rank < take (room: what is left)
      const uint32_t b1 = bq + nq0;
      const uint32_t room0 = sat_sub(take, bq), room1 = sat_sub(take, b1);
      const uint32_t r0 = mbcnt(q0), r1 = mbcnt(q1);
      if (in_mask(q0) && r0 < room0) st_slot(out, (cgt + bq) + r0, v0);
      if (in_mask(q1) && r1 < room1) st_slot(out, (cgt + b1) + r1, v1);
    }
  }
}

enum { SEL_DONE = 0, SEL_TIES = 1, SEL_OVERFLOW = 2 };

// Exact k-th key T over the survivor entries spread over the waves, then
// the write of the row's k outputs (o, through the block table, `lpages`
// its LDS copy or null).  Wave w sees `cnt` entries at e; `rel`
// is kRelWords zeroed words (kRelCopies copies of a kRelBins histogram,
// the copy chosen by lane mod 4 so that lanes with equal keys rarely hit
// one word, each copy followed by the spill words of its lanes), `sh` 512
// free words, bc[BC_SLOT..+1] zero.  The bins of (key - cs - 1), largest
// first, give T exactly unless T >= cs + kRelBins (then two 8-bit passes
// over the keys above that).  The
// keys above T take the slots [0, cgt) and the first keys equal to T the
// slots [cgt, k).
// Returns SEL_OVERFLOW when a wave's published entry count bc[BC_CNT + w]
// passed `cap` (checked after the histogram barrier), SEL_TIES when fewer
// than k keys lie above cs (nothing written then), else SEL_DONE.
template <int MODE, int NW, bool ONE = false>
__device__ int select_and_write(const uint32_t* __restrict__ e, uint32_t cnt, int32_t cs,
                                uint32_t k, uint32_t* __restrict__ rel, uint32_t* sh,
                                uint32_t* bc, uint32_t cap, const Out o,
                                const int32_t* lpages, bool ordered = false,
                                uint2* tsel = nullptr, int tid = (int)threadIdx.x) {
  const int lane = (tid & 63);
  const int32_t top = cs + kRelBins;  // signed keys at or above top share bin 0
  // keys at or below cs (top - s >= kRelBins) count into the lane's own
  // spill word after its copy's bins, or into one of the 15 below it
  uint32_t* const relc = rel + (lane & (kRelCopies - 1)) * kRelStride;
  const int32_t spill = kRelBins + (lane >> 2);
  for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
    const uint32_t x = e[2 * (b0 + lane)];
    atomicAdd(&relc[clamp0(top - lo16s(x), spill)], 1u);
    atomicAdd(&relc[clamp0(top - hi16s(x), spill)], 1u);
  }
  __syncthreads();
  if (__ballot(lane < NW && bc[BC_CNT + lane] > cap)) return SEL_OVERFLOW;
  uint32_t ri, above, total;
  if constexpr (ONE) {
    // wave 0 alone searches the bins and publishes the result (with many
    // waves per SIMD the others would only repeat it; with few, the extra
    // barrier costs more than the repeats)
    if ((tid >> 6) == 0) {
      find_copies<kRelCopies, kRelStride>(rel, k, ri, above, total, nullptr, tid);
      if (lane == 0) {
        bc[BC_TMP + 8] = ri;
        bc[BC_TMP + 9] = above;
        bc[BC_TMP + 10] = total;
      }
    }
    __syncthreads();
    ri = bc[BC_TMP + 8];
    above = bc[BC_TMP + 9];
    total = bc[BC_TMP + 10];
  } else {
    find_copies<kRelCopies, kRelStride>(rel, k, ri, above, total, nullptr, tid);
  }
  if (total < k) return SEL_TIES;
  int32_t Ts;
  uint32_t cgt;
  if (ri != 0) {
    Ts = top - (int32_t)ri;
    cgt = above;
  } else {
    // the k-th key lies at or above top: 8-bit passes over those keys
    for (int i = tid; i < 512; i += 64 * NW) sh[i] = 0;
    __syncthreads();
    for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
      const uint32_t i = b0 + lane;
      if (i < cnt) {
        const uint32_t x = e[2 * i];
        const int32_t s0 = lo16s(x), s1 = hi16s(x);
        if (s0 >= top) atomicAdd(&sh[255 - ((s0 + 0x8000) >> 8)], 1u);
        if (s1 >= top) atomicAdd(&sh[255 - ((s1 + 0x8000) >> 8)], 1u);
      }
    }
    __syncthreads();
    uint32_t i1, a1, i2, a2;
    find_desc(sh, k, i1, a1, tid);
    const int32_t b1 = 255 - (int32_t)i1;
    for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
      const uint32_t i = b0 + lane;
      if (i < cnt) {
        const uint32_t x = e[2 * i];
        const int32_t s0 = lo16s(x) + 0x8000, s1 = hi16s(x) + 0x8000;
        if (s0 >= top + 0x8000 && (s0 >> 8) == b1) atomicAdd(&sh[256 + 255 - (s0 & 255)], 1u);
        if (s1 >= top + 0x8000 && (s1 >> 8) == b1) atomicAdd(&sh[256 + 255 - (s1 & 255)], 1u);
      }
    }
    __syncthreads();
    find_desc(sh + 256, k - a1, i2, a2, tid);
    Ts = ((b1 << 8) | (255 - (int32_t)i2)) - 0x8000;
    cgt = a1 + a2;
  }
  if (ordered) {  // ordered results: the caller writes
    *tsel = make_uint2((uint32_t)(Ts + 0x8000), cgt);
    return SEL_DONE;
  }
  emit_entries<MODE, true, true>(e, cnt, Ts, cgt, k - cgt,
                                 reinterpret_cast<unsigned long long*>(bc + BC_SLOT), o, lpages,
                                 tid);
  return SEL_DONE;
}

// Keys above cs in the entries at e (wave-uniform count).
__device__ __forceinline__ uint32_t count_above(const uint32_t* e, uint32_t cnt, int32_t cs,
                                                 int tid = (int)threadIdx.x) {
  uint32_t c = 0;
  for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
    const uint32_t i = b0 + (tid & 63);
    const uint32_t x = i < cnt ? e[2 * i] : kDeadPair;
    c += popc(__ballot(lo16s(x) > cs)) + popc(__ballot(hi16s(x) > cs));
  }
  return c;
}

// Every survivor key above cs of the entries at e, in order, straight out
// to the slots from `base` on: the one-workgroup tie pass's first part.
template <int MODE>
__device__ void write_above(const uint32_t* e, uint32_t cnt, int32_t cs, uint32_t base,
                            const Out o, int tid = (int)threadIdx.x) {
  const int lane = (tid & 63);
  for (uint32_t b0 = 0; b0 < cnt; b0 += 64) {
    const uint32_t i = b0 + lane;
    uint32_t x = kDeadPair, id = 0;
    if (i < cnt) {
      x = e[2 * i];
      id = e[2 * i + 1];
    }
    const int32_t s0 = lo16s(x), s1 = hi16s(x);
    const unsigned long long g0 = __ballot(s0 > cs), g1 = __ballot(s1 > cs);
    const uint32_t p0 = mbcnt(g0, base), p1 = mbcnt(g1, base + popc(g0));
    if (in_mask(g0)) o.put(p0, id, (uint32_t)(s0 + 0x8000));
    if (in_mask(g1)) o.put(p1, id + 1, (uint32_t)(s1 + 0x8000));
    base += popc(g0) + popc(g1);
  }
}

// Tie collection of one key equal to the cutoff into a list shared by the
// workgroup, one LDS atomic per wave (the rare pass of the one-workgroup
// kernel).
__device__ __forceinline__ void keep_equal_slot(bool eq, uint32_t idx, uint16_t* list,
                                                uint32_t cap, uint32_t* ctr,
                                                int tid = (int)threadIdx.x) {
  const uint32_t slot = wave_slot(eq, ctr, tid);
  if (eq && slot < cap) list[slot] = (uint16_t)idx;
}

// Entries whose key pair holds a key equal to cs go to this wave's tie
// region the same way (compaction at tbase + tcnt), until tcnt passes
// tcap.  tw counts the entries written, tkept the equal keys in them, neq
// every equal key; tdrop is the smallest element index of an equal key
// that was not kept (every equal key below it was).
__device__ __forceinline__ void keep_ties(uint32_t x, uint32_t eidx, int32_t cs, uint32_t* tl,
                                          uint32_t tbase, uint32_t tcap, uint32_t& tcnt,
                                          uint32_t& tw, uint32_t& tkept, uint32_t& neq,
                                          uint32_t& tdrop) {
  const bool lo_eq = lo16s(x) == cs;
  const unsigned long long elo = __ballot(lo_eq), ehi = __ballot(hi16s(x) == cs);
  const unsigned long long me = elo | ehi;
  if (me) {
    const uint32_t ne = popc(elo) + popc(ehi);
    if (tcnt <= tcap) {
      if (in_mask(me)) {
        const uint32_t pos = mbcnt(me) + (tbase + tcnt);
        *reinterpret_cast<uint2*>(tl + 2 * pos) = make_uint2(x, eidx);
      }
      tw += popc(me);
      tkept += ne;
    } else {
      // lanes hold ascending element indices: the first lane is the smallest
      const uint32_t e = readlane(eidx + (lo_eq ? 0u : 1u), __ffsll(me) - 1);
      tdrop = min(tdrop, e);
    }
    tcnt += popc(me);
    neq += ne;
  }
}

// Tie entries each wave of a team member keeps before it stops: enough for
// its share of k.
__device__ __forceinline__ uint32_t tie_cap(int k) { return (uint32_t)k / 4u + 64u; }

// ============================================ one workgroup per row
// Rows whose valid vectors fit NT * VPT: the whole row sits in VGPRs.

// ------------------------------------------------------- ordered results
// The ordered write pass (vLLM kimi_k3 indexer, IndexerSelect: the selected
// keys in key order, that is by element index, with the ties at the
// threshold going to the lowest indices; -1 past the count; the logical
// indices alongside).  Given the k-th key T, the count cgt of keys above it
// and take = k - cgt, an element is selected when its key is above T, or
// equal to T with fewer than `take` equal keys before it; its output slot
// is the number of selected elements before it.

// A thread's selected elements take consecutive slots: with pa keys above
// T and pt keys equal to T before its first element, its first slot is
// pa + min(pt, take), and it keeps its keys above T and its first
// take - pt keys equal to T (ga, te: bit e for element e).  Returns that
// mask; `first` receives the first slot.
__device__ __forceinline__ uint32_t ordered_mask(uint32_t ga, uint32_t te, uint32_t pa,
                                                 uint32_t pt, uint32_t take, uint32_t& first) {
  const uint32_t room = sat_sub(take, pt);
  first = pa + (take - room);  // pa + min(pt, take)
  uint32_t tk = te;
  for (uint32_t c = (uint32_t)__builtin_popcount(te); c > room; --c)
    tk &= ~(1u << (31 - __builtin_clz(tk)));  // drop the last tie
  return ga | tk;
}

// The ordered write pass over a run of vectors staged in registers: vector
// vofs + slot_vid(j) in slot j of a thread (slots in order, and within a
// slot waves and lanes in order, follow the element order).  Per slot the
// counts of keys above and equal to T (packed 16 | 16 bits) are scanned
// over the wave, and the waves' totals, published before one barrier, give
// every thread its counts before it.  The run's selected elements take the
// output slots from na + min(nt, take) on (na, nt: keys above and equal to
// T before the run), staged in LDS and then written as one contiguous
// piece.  kb: block keys
// (block mode).  tmp: VPT NT/64 LDS words, stage: as many words as the run
// takes slots (at most k), both free when called.  Returns the run's counts
// of keys above and equal to T (16 | 16 bits).
template <int MODE, int NT, int VPT, int KB>
__device__ uint32_t ordered_regs(const uint4 (&raw)[VPT], const uint32_t (&kb)[KB], int jt, int rem,
                             int vofs, int v, uint32_t T, uint32_t cgt, uint32_t na,
                             uint32_t nt, const Out o, const int32_t* lpages, int32_t* ids,
                             uint32_t* tmp, uint32_t* stage, int tid = (int)threadIdx.x) {
  constexpr int NW = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t take = o.k - cgt;
  const uint32_t lo = na + min(nt, take);  // the run's first slot
  uint32_t ga[VPT], te[VPT], ex[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int lv = slot_vid<NT>(j, jt, rem, tid);
    const int vid = vofs + lv;
    ga[j] = 0;
    te[j] = 0;
    if (lv >= 0) {
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        ga[j] = kb[j] > T;
        te[j] = kb[j] == T;
      } else {
        if (T >= 0x8000u) {
          // a non-negative k-th key: the raw halves, as signed 16-bit
          // numbers, order non-negative values as their keys do, and every
          // negative value is below it, so no key is formed
          const int32_t Ts = (int32_t)T - 0x8000;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = word_of(raw[j], e >> 1);
            const int32_t h = (e & 1) ? hi16s(w) : lo16s(w);
            ga[j] |= (uint32_t)(h > Ts) << e;
            te[j] |= (uint32_t)(h == Ts) << e;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t key = key1(half_of(word_of(raw[j], e >> 1), e & 1));
            ga[j] |= (uint32_t)(key > T) << e;
            te[j] |= (uint32_t)(key == T) << e;
          }
        }
        // elements past the row's length (the last vector only)
        const int r = v - vid * 8;
        if (r < 8) {
          const uint32_t okm = r > 0 ? (1u << r) - 1u : 0u;
          ga[j] &= okm;
          te[j] &= okm;
        }
      }
    }
    // a run holds at most 2^15 elements: 16-bit counts
    const uint32_t c = ((uint32_t)__builtin_popcount(ga[j]) << 16) |
                       (uint32_t)__builtin_popcount(te[j]);
    const uint32_t incl = wave_incl_scan(c);
    ex[j] = incl - c;
    if (lane == 63) tmp[j * NW + wave] = incl;
  }
  __syncthreads();
  uint32_t base = 0;  // counts of the slots before j
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    uint32_t before = base + ex[j], tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = tmp[j * NW + w];
      before += w < wave ? x : 0u;
      tot += x;
    }
    base += tot;
    if (ga[j] | te[j]) {
      // the slots' element indices (bit 31: a -inf block) go to LDS first
      const int vid = vofs + slot_vid<NT>(j, jt, rem, tid);
      const uint32_t neg =
          (MODE == TOPK_MODE_BLOCK && kb[MODE == TOPK_MODE_BLOCK ? j : 0] == kKeyNegInf)
              ? 0x80000000u
              : 0u;
      uint32_t pos;
      uint32_t m = ordered_mask(ga[j], te[j], na + (before >> 16), nt + (before & 0xFFFFu), take,
                                pos);
      for (; m && pos < o.k; m &= m - 1, ++pos)
        stage[pos - lo] = (uint32_t)(MODE == TOPK_MODE_BLOCK ? vid : vid * 8 + __builtin_ctz(m)) | neg;
    }
  }
  // then the run's slots as one piece (every slot in [lo, hi) is taken; an
  // index past the row's elements, which would mean a slot left untaken,
  // is never mapped)
  const uint32_t hi = min(na + (base >> 16) + min(nt + (base & 0xFFFFu), take), o.k);
  __syncthreads();
  const int n = MODE == TOPK_MODE_BLOCK ? (v + 7) >> 3 : v;
  for (uint32_t i = lo + tid; i < hi; i += NT) {
    const uint32_t x = stage[i - lo];
    const int32_t idx = (int32_t)(x & 0x7FFFFFFFu);
    o.out[i] = ((x >> 31) || idx >= n) ? -1 : map_out(o, lpages, idx);
    if (ids) ids[i] = idx;
  }
  return base;
}

// Ordered results of a row with n <= k: the logical ids 0..n-1, then -1,
// and the count (the output itself is written by write_short_*).
template <int NT>
__device__ void short_ids(const Params& p, int row, int n, int tid = (int)threadIdx.x) {
  if (p.ids)
    for (int e = tid; e < p.k; e += NT) p.ids[(int64_t)row * p.k + e] = e < n ? e : -1;
  if (p.valid && tid == 0) p.valid[row] = n;
}

// One row of the one-workgroup kernel.
template <int MODE, int NT, int VPT, bool ONE, bool ORD>
__device__ __forceinline__ void rows_wg_body(const Params& p, const int row) {
  constexpr int NW = NT / 64;
  extern __shared__ uint32_t smem[];
  const uint32_t lds0 = lds_addr(smem);
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
  // the LDS copy of the row's block-table entries (made by the sampled
  // path, so not when the direct path is forced)
  int32_t* lpages = (p.page_lds && o.pages && !p.force_direct)
                        ? reinterpret_cast<int32_t*>(smem + p.page_lds)
                        : nullptr;

  if (n <= k) {
    if constexpr (MODE == TOPK_MODE_BLOCK) write_short_block<NT>(o, src, n, k);
    else write_short_token<NT>(o, n, k);
    if constexpr (ORD) short_ids<NT>(p, row, n);
    set_path(p, row, TOPK_PATH_SHORT);
    return;
  }
  bool direct = p.force_direct != 0;
  int code = TOPK_PATH_DIRECT_FORCED;
  uint2 tc = make_uint2(0u, 0u);  // ordered results: the k-th key, the count above it
  const int nvec = (v + 7) >> 3;
  const int jt = (nvec - 1) / NT;   // last vector slot holding row data
  const int rem = nvec - jt * NT;   // vectors in it
  uint4 raw[VPT];                   // the staged row
  uint32_t kb[MODE == TOPK_MODE_BLOCK ? VPT : 1];  // its block keys (block mode)
  if (!direct) {
    // zero the sample and relative histograms and the replicated sample bins
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = tid; i < (kRelHist - kSampHist + kRelWords) / 4; i += NT)
      reinterpret_cast<uint4*>(sh)[i] = z4;
#pragma unroll
    for (int i = tid; i < kSampBins / 4; i += NT) reinterpret_cast<uint4*>(lists)[i] = z4;
    if (tid == 0) {
      bc[BC_EQ] = 0;
      bc[BC_SLOT] = 0;
      bc[BC_SLOT + 1] = 0;
    }
    // -- stage the row: 16-byte loads into VGPRs.  Every lane loads (a lane
    // without a vector in slot jt reads vector 0 and poisons it below; the
    // slots past jt are never used), so that no load sits under a branch.
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      raw[j] = ld_vec(src, (uint32_t)max(slot_vid<NT>(j, jt, rem), 0));
    // the row's block-table entries ride along, for an LDS copy
    constexpr int PPT = kPageLdsMax / NT;
    int32_t pgv[PPT];
    const int npg = lpages ? (v + (1 << p.page_shift) - 1) >> p.page_shift : 0;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int i = j * NT + tid;
      pgv[j] = i < npg ? o.pages[i] : 0;
    }
    // sampled slots: every slot in token mode (one logit of every vector),
    // every SE-th slot in block mode (at most 2048 block keys)
    constexpr int SE = (MODE == TOPK_MODE_TOKEN || VPT * NT <= 2048) ? 1 : VPT * NT / 2048;
    constexpr int NSK = VPT / SE;  // one sample a sampled slot
    uint32_t sk[NSK];
    uint32_t S = 0;  // samples over the workgroup
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vid = slot_vid<NT>(j, jt, rem);
      uint32_t s = kNone;
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        kb[j] = vid >= 0 ? (vid == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
        s = vid >= 0 ? kb[j] : kNone;
      } else {
        // sample: logit (vid / 512) mod 8 of the vector, whatever the
        // workgroup size (with 512 threads, logit j mod 8 of slot j).
        // Slots before jt hold whole vectors; in slot jt, with a length
        // that is not a multiple of 8, the row's last vector is cut: its
        // logits past the length become the bottom key, and its sample is
        // logit 0 when its sampled logit is past the length.
        const int es = NT == 512 ? (j & 7) : ((vid >> 9) & 7);
        const uint32_t se = key1(half_of(word_of(raw[j], es >> 1), es & 1));
        if (j < jt) {
          s = se;
        } else if (j == jt) {
          poison_tail(raw[j], vid >= 0 ? clamp8(v - 8 * vid) : 0);
          if (v & 7) {
            const uint32_t s0 = key1(raw[j].x & 0xFFFFu);
            s = vid >= 0 ? ((vid * 8 + es < v) ? se : s0) : kNone;
          } else {
            s = vid >= 0 ? se : kNone;
          }
        }
      }
      if (j % SE == 0) {
        sk[j / SE] = s;
        S += (uint32_t)(j < jt ? NT : (j == jt ? rem : 0));
      }
    }
    // token rows of at most kAllSampled vectors: with one sample a vector
    // the sampled rank's margin spans most of such a row, and its k-th key
    // lies near zero, where keys spread over many exponents, so the cutoff
    // would fall 256 keys or more below it and the exact select would need
    // two more passes.  Every logit is a sample there instead (a thread's
    // one vector gives 8), which gives the k-th key itself.  Only while
    // every row is resident, where the slowest row is the call's time (the
    // throughput variant's code for the other rows is then left as it was:
    // the extra branch cost it 1.4 % on full rows).
    const bool all = MODE == TOPK_MODE_TOKEN && !ONE && jt == 0 && rem <= kAllSampled;
    if (all) S = (uint32_t)v;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int i = j * NT + tid;
      if (i < npg) lpages[i] = pgv[j];
    }
    const uint32_t q = sample_rank((uint32_t)k, (uint32_t)n, S);
    __syncthreads();  // histograms zeroed, block-table copy complete
    uint32_t c, sa = 0, se = 0;
    if (MODE == TOPK_MODE_TOKEN && all) {
      const int vid = slot_vid<NT>(0, 0, rem);
      uint32_t s8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        s8[e] = (vid >= 0 && vid * 8 + e < v) ? key1(half_of(word_of(raw[0], e >> 1), e & 1))
                                              : kNone;
      c = sample_cutoff<8, NT, kRowLoCopies>(s8, 0, q, lists, sh, &sa, &se);
    } else {
      c = sample_cutoff<NSK, NT, kRowLoCopies>(sk, (jt + SE - 1) / SE, q, lists, sh);
    }
    // every element sampled: c is the k-th key itself.  The cutoff moves to
    // the key below it, so that the keys equal to it survive and the exact
    // select finds it one bin above the cutoff (no tie pass).  Block rows of
    // one slot: every wave's whole share (ceil(rem / NW) entries) fits its
    // survivor region.  Token rows: when the keys at or above the k-th
    // (exact counts, sa + se) fill at most half of the waves' regions (a
    // wave that still overflows sends the row to the direct path).
    // Otherwise the keys equal to it take the tie pass.
    if (S >= (uint32_t)n && c > 0u && jt == 0 &&
        (MODE == TOPK_MODE_BLOCK
             ? (uint32_t)((rem + NW - 1) / NW) <= (uint32_t)p.lcw
             : all && sa + se <= (uint32_t)(NW * p.lcw / 2)))
      c -= 1u;

    if (MODE == TOPK_MODE_TOKEN && c == 0u) {
      // a zero cutoff would make the zero keys of slots past the length ties
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    } else {
      // -- filter + compaction of the entries holding a key above the cutoff
      const int32_t cs = (int32_t)c - 0x8000;
      const uint32_t cap = (uint32_t)p.lcw;
      const uint32_t wbase = readfirst((uint32_t)wave) * (cap + kSpare);
      uint32_t* seg = lists + 2 * wbase;
      // LDS byte addresses: the wave's next entry, its cap, the lane's dummy
      const uint32_t first = lds0 + 4u * (kLists + 2u * wbase);
      const uint32_t lim = first + cap * 8u;
      uint32_t at = first;
      const uint32_t dummy = lds0 + 4u * (kLists + 2u * (NW * (cap + kSpare) + lane));
      if constexpr (MODE == TOPK_MODE_BLOCK) {
#pragma unroll
        for (int j = 0; j < VPT; ++j)
          if (j <= jt)
            keep_word_lds(block_entry(kb[j]), (uint32_t)slot_vid<NT>(j, jt, rem), cs, lim, dummy,
                          at);
      } else if (cs >= 0) {
        // non-negative cutoff: the raw words serve as signed keys
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          if (j <= jt) {
            const uint32_t e8 = (uint32_t)slot_vid<NT>(j, jt, rem) * 8u;
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2)
              keep_word_lds(word_of(raw[j], q2), e8 + 2 * q2, cs, lim, dummy, at);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          if (j <= jt) {
            const uint32_t e8 = (uint32_t)slot_vid<NT>(j, jt, rem) * 8u;
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2)
              keep_word_lds(skey2(word_of(raw[j], q2)), e8 + 2 * q2, cs, lim, dummy, at);
          }
        }
      }
      const uint32_t wcnt = (at - first) / 8u;
      if (lane == 0) bc[BC_CNT + wave] = wcnt;
      // dead entries after the wave's last (the passes read whole chunks)
      lds_store2(min(at, lim) + 8u * lane, kDeadPair, 0u);
      // exact select over the survivors; its histogram barrier also publishes
      // the entry counts (overflow) and the count of keys above the cutoff
      const int st = select_and_write<MODE, NW, ONE>(seg, min(wcnt, cap), cs, (uint32_t)k, rel,
                                                     sh, bc, cap, o, lpages,
                                                     ORD, ORD ? &tc : nullptr);
      if (st == SEL_OVERFLOW) {
        direct = true;
        code = TOPK_PATH_DIRECT_OVERFLOW;
      } else if (st == SEL_DONE) {
        code = TOPK_PATH_SAMPLED;
      } else {
        // fewer than k keys above the cutoff: per-wave counts for the slots
        const uint32_t ew = count_above(seg, wcnt, cs);  // every lane takes part
        if (lane == 0) bc[BC_ECNT + wave] = ew;
        __syncthreads();
        uint32_t gt_total = 0, before = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t ew = bc[BC_ECNT + w];
          before += w < wave ? ew : 0u;
          gt_total += ew;
        }
        // the k-th key can only be the cutoff: collect keys equal to it
        uint16_t* ties = reinterpret_cast<uint16_t*>(rel);  // room for 2 kRelWords >= k
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          if (j <= jt) {
            const int vid = slot_vid<NT>(j, jt, rem);
            if constexpr (MODE == TOPK_MODE_BLOCK) {
              keep_equal_slot(vid >= 0 && kb[j] == c, (uint32_t)vid, ties, (uint32_t)k,
                              &bc[BC_EQ]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t key = key1(half_of(word_of(raw[j], e >> 1), e & 1));
                keep_equal_slot(key == c, (uint32_t)(vid * 8 + e), ties, (uint32_t)k, &bc[BC_EQ]);
              }
            }
          }
        }
        __syncthreads();
        const uint32_t eq_total = bc[BC_EQ];
        if (gt_total + eq_total < (uint32_t)k) {
          direct = true;
          code = TOPK_PATH_DIRECT_MISJUDGED;
        } else {
          if constexpr (ORD) {
            tc = make_uint2(c, gt_total);
          } else {
            write_above<MODE>(seg, wcnt, cs, before, o);
            const uint32_t take = (uint32_t)k - gt_total;
            for (uint32_t i = tid; i < take; i += NT) o.put(gt_total + i, ties[i], c);
          }
          code = TOPK_PATH_SAMPLED_TIES;
        }
      }
    }
  }
  if (direct) {
    __syncthreads();
    const uint2 dt = direct_select<MODE, NT>(src, v, n, k, o, lists, bc, ORD);
    if constexpr (ORD) tc = dt;
  }
  if constexpr (ORD) {
    if (p.force_direct) {  // the sampled path did not stage the row
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int vid = slot_vid<NT>(j, jt, rem);
        raw[j] = ld_vec(src, (uint32_t)max(vid, 0));
        if constexpr (MODE == TOPK_MODE_BLOCK)
          kb[j] = vid >= 0 ? (vid == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
      }
    }
    __syncthreads();  // the pass's LDS words are free
    ordered_regs<MODE, NT, VPT>(raw, kb, jt, rem, 0, v, tc.x, tc.y, 0u, 0u, o, lpages,
                                p.ids ? p.ids + (int64_t)row * k : nullptr, sh, lists);
    if (p.valid && tid == 0) p.valid[row] = k;
  }
  set_path(p, row, code);
}

template <int MODE, int NT, int VPT, bool ONE, bool ORD>
__global__ __launch_bounds__(NT) void topk_rows_wg(Params p) {
  // the throughput variant runs its rows in several waves of workgroups,
  // spread over the XCDs; with every row resident at once the order of
  // rows on the XCDs changes nothing but which rows share a unit
  rows_wg_body<MODE, NT, VPT, ONE, ORD>(p, ONE ? spread_row(p, blockIdx.x) : (int)blockIdx.x);
}



// ============================================ the vector-max bound
// A producer's side array of the largest key of every aligned group of 8
// logits (vLLM kimi_k3 indexer page, IndexerScore epilogue: each 8 logits'
// largest key, a side array 1/8 of the row) bounds the k-th key from below:
// the k-th largest of those maxima, `low`, is the largest key of k distinct
// groups, so at least k keys lie at or above it (the same page,
// IndexerSelect passes 1 and 2).  Every key at or above low lies in a group
// whose maximum reaches low ("hot" vectors, about k of them on smooth data),
// so those groups alone are loaded; the survivors are their keys at or above
// low, and the exact select runs over them as on the sampled path.

constexpr int kHotWave = 256;  // hot vectors one wave gathers at most (4 per lane)
constexpr int kTopsTPT = 8;    // 16-byte words of maxima per thread at most
constexpr int kTopsLC = 8;     // copies of the bound's low-byte bins (lane mod 8)
// Copies of the bound's high-byte bins (lane mod HC): 8 for rows of one
// word of maxima per thread (at most 2048 maxima, 4 atomics a lane), 32 for
// wider rows; a copy's stride puts the copies of one bin in distinct banks
// (260 = 4 mod 32 for 8 copies, 289 = 1 mod 32 for 32), with spare words
// past the bins.
template <int TPT> struct TopsBins {
  static constexpr int HC = TPT == 1 ? 8 : 32;
  static constexpr int STRIDE = TPT == 1 ? 260 : 289;
  static constexpr int WORDS = HC * STRIDE + 256;  // the copies, then their sums
};


// The q-th largest of a row's vector maxima, held 8 to a 16-byte word (word
// wi[j] in slot j, -1 for none, not counted; maxima of no vector are 0): the
// two 8-bit radix passes of sample_cutoff over every maximum, with more
// copies of the bins, since every maximum costs an atomic and the maxima of
// crowded rows share a few bins: TopsBins<TPT> copies of the high-byte bins
// at h8 (TopsBins<TPT>::WORDS zeroed words; the sums go after the copies)
// and kTopsLC copies of the low-byte bins at lo8 (kTopsLC kRelStride zeroed
// words).
template <int NT, int TPT>
__device__ uint32_t tops_cutoff(const uint4 (&tw)[TPT], const int (&wi)[TPT], int jt,
                                uint32_t q, uint32_t* h8, uint32_t* lo8, int tid) {
  constexpr int HC = TopsBins<TPT>::HC, STRIDE = TopsBins<TPT>::STRIDE;
  const int lane = tid & 63;
  const uint32_t copy = (uint32_t)lane & (HC - 1);
  // every lane adds every slot (no branch around the atomics): a slot past
  // the row counts into one of its copy's 4 spare words past the bins
  uint32_t* const hc = h8 + copy * STRIDE;
  const uint32_t hspill = 256u + (((uint32_t)lane / HC) & 3u);
  static_assert(STRIDE >= 260, "four spare words per copy of the high-byte bins");
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    if (j > jt) break;  // (uniform: the slots past jt hold no word)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t t = half_of(word_of(tw[j], e >> 1), e & 1);
      atomicAdd(&hc[wi[j] >= 0 ? 255u - (t >> 8) : hspill], 1u);
    }
  }
  __syncthreads();
  uint32_t* sums = h8 + HC * STRIDE;
  if (tid < 256) {
    uint32_t t = 0;
#pragma unroll
    for (int c = 0; c < HC; ++c) t += h8[c * STRIDE + tid];
    sums[tid] = t;
  }
  __syncthreads();
  uint32_t i1, a1;
  find_desc(sums, q, i1, a1, tid);
  const uint32_t b1 = 255u - i1;
  uint32_t* const loc = lo8 + (lane % kTopsLC) * kRelStride;
  const uint32_t spill = 256u + (((uint32_t)lane / kTopsLC) & 15u);
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    if (j > jt) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t t = half_of(word_of(tw[j], e >> 1), e & 1);
      atomicAdd(&loc[wi[j] >= 0 && (t >> 8) == b1 ? 255u - (t & 255u) : spill], 1u);
    }
  }
  __syncthreads();
  uint32_t i2, a2, t2;
  find_copies<kTopsLC, kRelStride>(lo8, q - a1, i2, a2, t2, nullptr, tid);
  return (b1 << 8) | (255u - i2);
}

// One token row (v > k, at least 2k vectors) on the vector-max bound: the
// maxima are staged, low is found, each wave lists its hot vectors in its
// LDS region and loads them (up to kHotWave), keeps their keys at or above
// low in its survivor region, and the exact select writes the row.  A wave
// with more hot vectors than it holds, or survivors beyond the regions, or a
// bound of 0 (the keys past the length are 0) sends the row to the direct
// path.  A workgroup of NT threads holds NT TPT 16-byte words of maxima.
template <int NT, int TPT, bool ONE>
__device__ __forceinline__ void tops_body(const Params& p, const int row, const int v,
                                          const Out o) {
  constexpr int NW = NT / 64, GPL = kHotWave / 64;
  extern __shared__ uint32_t smem[];
  const uint32_t lds0 = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = p.k;
  const int nvec = (v + 7) >> 3, ntw = (nvec + 7) >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
  const uint4* tsrc = reinterpret_cast<const uint4*>(p.tops + (int64_t)row * p.tops_stride);
  uint32_t* sh = smem + kSampHist;
  uint32_t* rel = smem + kRelHist;
  uint32_t* bc = smem + kBc;
  uint32_t* lists = smem + kLists;
  int32_t* lpages = (p.page_lds && o.pages) ? reinterpret_cast<int32_t*>(smem + p.page_lds)
                                            : nullptr;
  // the bound's bins: TopsBins words at the start of the survivor area, the
  // low-byte copies at p.tops_lo, past the survivor regions (which fill as
  // soon as a wave has the bound, while others may still read those copies)
  uint32_t* lo8 = smem + p.tops_lo;
  // zero the relative histogram and the bound's bins
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  for (int i = tid; i < (kRelHist - kSampHist + kRelWords) / 4; i += NT)
    reinterpret_cast<uint4*>(sh)[i] = z4;
  for (int i = tid; i < TopsBins<TPT>::WORDS / 4; i += NT) reinterpret_cast<uint4*>(lists)[i] = z4;
  for (int i = tid; i < kTopsLC * kRelStride / 4; i += NT) reinterpret_cast<uint4*>(lo8)[i] = z4;
  if (tid == 0) {
    bc[BC_SLOT] = 0;
    bc[BC_SLOT + 1] = 0;
  }
  // -- the maxima, in the slots of the sampled path's vectors (the last
  // occupied slot shared out evenly over the waves, so that every wave lists
  // about as many hot vectors); a lane without a word in a slot reads word 0
  // and counts none of it
  const int jt = (ntw - 1) / NT, rem = ntw - jt * NT;
  uint4 tw[TPT];
  int wi[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    wi[j] = slot_vid<NT>(j, jt, rem, tid);
    tw[j] = ld_vec(tsrc, (uint32_t)max(wi[j], 0));
  }
  // maxima of no vector of the row (past nvec, or a slot without a word)
  // become 0: they then fall in the bottom bin of the bound's histogram,
  // below the k-th largest of the row's own 2k or more maxima unless that
  // is 0 too (the row then takes the direct path), and are never hot
#pragma unroll
  for (int j = 0; j < TPT; ++j) keep_first(tw[j], wi[j] >= 0 ? clamp8(nvec - 8 * wi[j]) : 0);
  // the row's block-table entries ride along, for an LDS copy
  constexpr int PPT = kPageLdsMax / NT;
  int32_t pgv[PPT];
  const int npg = lpages ? (v + (1 << p.page_shift) - 1) >> p.page_shift : 0;
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int i = j * NT + tid;
    pgv[j] = i < npg ? o.pages[i] : 0;
  }
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int i = j * NT + tid;
    if (i < npg) lpages[i] = pgv[j];
  }
  __syncthreads();  // histograms zeroed, block-table copy complete
  const uint32_t low = tops_cutoff<NT, TPT>(tw, wi, jt, (uint32_t)k, lists, lo8, tid);

  int code = TOPK_PATH_TOPS;
  bool direct = false;
  if (low == 0u) {
    direct = true;
    code = TOPK_PATH_DIRECT_MISJUDGED;
  } else {
    // -- this wave's hot vectors, listed in its LDS region: each lane
    // counts its own, one wave scan gives its offset, then every lane
    // stores every slot, a cold one (or one past the region) into a word of
    // its own after the wave's kHotWave entries
    uint32_t* hot = smem + p.hot_lds + wave * (kHotWave + 64);
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      if (j > jt) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t t = half_of(word_of(tw[j], e >> 1), e & 1);
        mine += t >= low ? 1u : 0u;
      }
    }
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t hc = readlane(incl, 63);  // wave-uniform
    uint32_t pos = incl - mine;
    const uint32_t cold = (uint32_t)kHotWave + (uint32_t)lane;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      if (j > jt) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t t = half_of(word_of(tw[j], e >> 1), e & 1);
        const bool h = t >= low;
        hot[h && pos < (uint32_t)kHotWave ? pos : cold] = (uint32_t)(wi[j] * 8 + e);
        pos += h ? 1u : 0u;
      }
    }
    const uint32_t hn = min(hc, (uint32_t)kHotWave);
    // -- load them: lane l takes entries l, l + 64, ... of the list
    int gv[GPL];
    uint4 g[GPL];
#pragma unroll
    for (int u = 0; u < GPL; ++u) {
      const uint32_t i = (uint32_t)(u * 64 + lane);
      gv[u] = i < hn ? (int)hot[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < GPL; ++u)
      if ((uint32_t)(u * 64) < hn) g[u] = ld_vec(src, (uint32_t)max(gv[u], 0));
    // -- their keys at or above low (above cs = low - 1), compacted as on
    // the sampled path; a lane without a listed vector keeps nothing
    const int32_t cs = (int32_t)low - 1 - 0x8000;
    const uint32_t cap = (uint32_t)p.lcw;
    const uint32_t wbase = readfirst((uint32_t)wave) * (cap + kSpare);
    uint32_t* seg = lists + 2 * wbase;
    const uint32_t first = lds0 + 4u * (kLists + 2u * wbase);
    const uint32_t lim = first + cap * 8u;
    uint32_t at = first;
    const uint32_t dummy = lds0 + 4u * (kLists + 2u * (NW * (cap + kSpare) + lane));
#pragma unroll
    for (int u = 0; u < GPL; ++u) {
      if ((uint32_t)(u * 64) < hn) {
        uint4 x = g[u];
        poison_tail(x, gv[u] >= 0 ? clamp8(v - 8 * gv[u]) : 0);
        const uint32_t e8 = (uint32_t)max(gv[u], 0) * 8u;
        if (cs >= 0) {
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) keep_word_lds(word_of(x, q2), e8 + 2 * q2, cs, lim, dummy, at);
        } else {
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2)
            keep_word_lds(skey2(word_of(x, q2)), e8 + 2 * q2, cs, lim, dummy, at);
        }
      }
    }
    const uint32_t wcnt = (at - first) / 8u;
    // a wave with hot vectors it could not list reports a count past the
    // cap: the select then routes the row to the direct path
    if (lane == 0) bc[BC_CNT + wave] = hc > (uint32_t)kHotWave ? cap + 1u : wcnt;
    lds_store2(min(at, lim) + 8u * lane, kDeadPair, 0u);
    const int st = select_and_write<TOPK_MODE_TOKEN, NW, ONE>(seg, min(wcnt, cap), cs, (uint32_t)k,
                                                              rel, sh, bc, cap, o, lpages, false,
                                                              nullptr, tid);
    if (st != SEL_DONE) {
      // (fewer than k keys at or above low: maxima that break their
      // definition)
      direct = true;
      code = st == SEL_OVERFLOW ? TOPK_PATH_DIRECT_OVERFLOW : TOPK_PATH_DIRECT_MISJUDGED;
    }
  }
  if (direct) {
    __syncthreads();
    direct_select<TOPK_MODE_TOKEN, NT>(src, v, v, k, o, lists, bc, false, tid);
  }
  set_path(p, row, code, tid);
}

// Token rows with their vector maxima, one workgroup per row: n <= k rows
// as always; rows with fewer than 2k vectors (where the k-th largest
// maximum bounds loosely) on the sampled path when they fit its registers
// (16384 logits), else on the direct path; the rest on the bound.
template <int TPT, bool ONE>
__global__ __launch_bounds__(kRowNT) void topk_rows_tops(Params p) {
  const int row = ONE ? spread_row(p, blockIdx.x) : (int)blockIdx.x;
  const int v = clamp_len(p.valid_len[row], p.width);
  const int k = p.k;
  const Out o = row_out(p, row, false);
  if (v <= k) {
    write_short_token<kRowNT>(o, v, k);
    set_path(p, row, TOPK_PATH_SHORT);
    return;
  }
  if ((v + 7) >> 3 < 2 * k) {
    if (v <= kRowNT * kRowTokenVPT * 8) {
      rows_wg_body<TOPK_MODE_TOKEN, kRowNT, kRowTokenVPT, ONE, false>(p, row);
    } else {
      extern __shared__ uint32_t smem[];
      const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
      direct_select<TOPK_MODE_TOKEN, kRowNT>(src, v, v, k, o, smem + kLists, smem + kBc);
      set_path(p, row, TOPK_PATH_DIRECT_DENSE);
    }
    return;
  }
  tops_body<kRowNT, TPT, ONE>(p, row, v, o);
}

// The producer's side array, for callers whose scorer does not write it:
// tops[r][j] = the largest key among logits 8j .. 8j+7 of row r below its
// valid length, 0 where none is, for every j < ceil(width / 8) (and the
// rest of the 16-byte word holding the last one).  One thread per 16-byte
// word of maxima (8 vectors of 8 logits).
struct MaxParams {
  const uint16_t* logits;
  int64_t row_stride;
  const int32_t* valid_len;
  int32_t width;
  uint16_t* tops;
  int64_t tops_stride;
};

__global__ __launch_bounds__(256) void topk_vector_maxima(MaxParams q, int rows) {
  const int w = blockIdx.x * 256 + threadIdx.x;  // word of maxima
  const int nvw = (q.width + 7) >> 3;            // vectors of the width
  if (w * 8 >= nvw) return;
  for (int row = blockIdx.y; row < rows; row += gridDim.y) {
  const int v = clamp_len(q.valid_len[row], q.width);
  const int nvec = (v + 7) >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(q.logits + (int64_t)row * q.row_stride);
  uint4 x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int vid = w * 8 + e;
    x[e] = vid < nvec ? ld_vec(src, (uint32_t)vid) : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int vid = w * 8 + e;
    uint32_t m = 0;
    if (vid < nvec) {
      poison_tail(x[e], clamp8(v - 8 * vid));  // logits past the length: key 0
#pragma unroll
      for (int h = 0; h < 8; ++h) m = max(m, key1(half_of(word_of(x[e], h >> 1), h & 1)));
    }
    t[e] = m;
  }
  *reinterpret_cast<uint4*>(q.tops + (int64_t)row * q.tops_stride + (int64_t)w * 8) =
      make_uint4(t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16),
                 t[6] | (t[7] << 16));
  }
}

// ============================================ team of workgroups per row
// A row wider than one workgroup is split over member workgroups of fixed
// chunks of its valid length (G per row in the grid, for the widest row); a
// second kernel, one workgroup per row, finishes it after the kernel
// boundary.

// Stage 1: every member loads the row's samples (spread over the whole row,
// the same in every member) and waits for them before its chunk loads go
// out, so that the samples do not queue behind the chunks of every other
// member; then it loads its chunk of NT * VPT vectors (members past the
// row's valid length exit at once), derives the row's cutoff while the
// chunk streams in, compacts the entries holding a key above the cutoff in
// LDS and writes them to its scratch slice as one list, with a 256-bin
// histogram of their keys relative to the cutoff; when the cutoff may be
// tied, it also keeps the entries holding a key equal to it (chunk-local
// indices).  Short rows and rows sent straight to the direct path are left
// to stage 2.  Every load is issued unconditionally (a lane past the row's
// end reads vector 0 and masks it), so that the compiler counts the loads
// exactly and each wait covers only what it needs.
template <int MODE, int VPT, int SV>
__global__ __launch_bounds__(kTeamNT) void topk_team_filter(Params p) {
  constexpr int NT = kTeamNT;
  __shared__ __align__(16) uint32_t h8[kSampBins + 256 + kRelWords];
  __shared__ __align__(16) uint32_t mh[kRelWords];
  __shared__ uint32_t bc[128];
  const int G = p.G;
  // groups of 8 rows: member m of row r of a group runs on XCD (r + m) % 8
  // (blockIdx % 8), which spreads the rows' members evenly over the XCDs
  // whatever the rows' lengths
  const int b = blockIdx.x, xg = b & 7, yg = b >> 3;
  const int member = yg % G;
  const int lrow = (yg / G) * 8 + ((xg - member) & 7);
  if (lrow >= p.rows) return;
  const int row = p.row0 + lrow;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = tid >> 6;
  const int k = p.k;
  const int v = clamp_len(p.valid_len[row], p.width);
  const int n = (MODE == TOPK_MODE_BLOCK) ? (v + 7) >> 3 : v;
  if (n <= k || p.force_direct) return;
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
  // members take NT * VPT vectors each; those past the row's length exit
  const int nvec = (v + 7) >> 3;
  const int vb = member * NT * VPT;
  if (vb >= nvec) return;
  const int ve = min(vb + NT * VPT, nvec);
  const int jt = (ve - vb - 1) / NT;   // last occupied slot
  const int rem = (ve - vb) - jt * NT; // vectors in it
  for (int i = tid; i < kSampBins + 256 + kRelWords; i += NT) h8[i] = 0;
  for (int i = tid; i < kRelWords; i += NT) mh[i] = 0;

  // -- samples: the same in every member of the row: every vector of a
  // short row; otherwise SV * NT / 8 runs of 8 consecutive vectors (one
  // 128-byte line each), run r starting at line floor((2 r + 1) lines / (2
  // runs)) (a 32.32 step), so that the row's members share few lines
  const int ns = min(SV * NT, nvec);
  const int nl = nvec >> 3, runs = SV * NT / 8;
  const uint64_t step = nvec > SV * NT ? ((uint64_t)nl << 32) / (uint64_t)(2 * runs) : 0;
  uint4 sraw[SV];
  int spos[SV];
#pragma unroll
  for (int j = 0; j < SV; ++j) {
    const int si = j * NT + tid;
    if (nvec <= SV * NT) {
      spos[j] = si < ns ? si : -1;
    } else {
      const int r = si >> 3;
      spos[j] = (int)((((uint64_t)(2 * r + 1) * step) >> 32) << 3) + (si & 7);
    }
    sraw[j] = ld_vec(src, (uint32_t)max(spos[j], 0));
  }
  constexpr int NSK = (MODE == TOPK_MODE_BLOCK) ? SV : SV * 8;
  uint32_t sk[NSK];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < SV; ++j) {
    const int vid = spos[j];
    if constexpr (MODE == TOPK_MODE_BLOCK) {
      sk[j] = vid < 0 ? kNone : (vid == n - 1 ? kKeyPosInf : block_key4(sraw[j]));
      mine += vid >= 0 ? 1u : 0u;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = vid >= 0 && vid * 8 + e < v;
        sk[j * 8 + e] = ok ? key1(half_of(word_of(sraw[j], e >> 1), e & 1)) : kNone;
        mine += ok ? 1u : 0u;
      }
    }
  }
  // -- the cutoff, identical in every member, before the chunk loads go
  // out: issued behind every member's chunk, the samples would arrive late,
  // and a wave issuing into the full memory queues stalls there; with the
  // cutoff known, the filter takes each vector as it arrives
  const uint32_t S = block_sum<NT>(mine, bc + BC_TMP);  // also publishes the zeroed hists
  uint32_t sa, se;
  uint32_t c =
      sample_cutoff<NSK, NT, kRelCopies>(sk, 0, sample_rank((uint32_t)k, (uint32_t)n, S), h8,
                                         h8 + kSampBins + 256, &sa, &se);
  // keys equal to the cutoff are only needed when fewer than k keys lie
  // above it; when the samples above it exceed their expected count at
  // rank k by 3 standard deviations that is a rare event, and the members
  // skip collecting ties (a row that needs them after all finds no ties
  // and takes the direct path, so exactness is kept)
  bool ties = !tie_unlikely((uint32_t)k, (uint32_t)n, S, sa);
  // Otherwise, when the keys at or above c are few enough for the members'
  // regions, the cutoff moves to the key below c: the keys equal to c become
  // survivors and no ties are collected (at least q of the samples lie at or
  // above c, so k keys almost surely do; a row where they do not takes the
  // direct path as above).  Every member takes the same decision from the
  // same samples.
  if (ties && c >= 2u) {
    constexpr float kKeysPerWave = 64.0f * VPT * (MODE == TOPK_MODE_BLOCK ? 1 : 8);
    const float f = (float)(sa + se) * __builtin_amdgcn_rcpf((float)S);
    if (1.25f * f * kKeysPerWave + 48.0f <= (float)kFiltCap) {
      c -= 1u;
      ties = false;
    }
  }
  uint32_t* slice = p.team_slices + ((size_t)lrow * G + member) * kMemberWords;
  if (MODE == TOPK_MODE_TOKEN && c == 0u) {
    // a zero cutoff would make the zero keys of slots past the length ties:
    // every member sees the same cutoff and flags the row for the direct path
    if (tid == 0) {
      slice[MH_CUT] = c;
      slice[MH_FLAGS] = kFlagDirect;
    }
    return;
  }
  // -- the chunk
  asm volatile("" ::: "memory");
  uint4 raw[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j)
    raw[j] = ld_vec(src, (uint32_t)(vb + max(slot_vid<NT>(j, jt, rem), 0)));

  // -- entries above the cutoff: compacted into this wave's region of the
  // sample-bin area (free once every wave has its cutoff).  Entries holding
  // a key equal to the cutoff (when collected at all) go straight to their
  // global regions.
  const int32_t cs = (int32_t)c - 0x8000;
  uint32_t* tl = slice + kMemberTies;
  const uint32_t wv = readfirst((uint32_t)wave);
  const uint32_t tbase = wv * kTieLCW;
  const uint32_t tcap = tie_cap(k);
  // LDS: 64 dummy entries, then 4 wave regions of kFiltStage entries
  // (kFiltCap kept, the rest for the stores past the cap)
  static_assert(NT == 256 && 128 + 8 * kFiltStage <= kSampBins + 256 + kRelWords,
                "four wave regions in the sample-bin area");
  const uint32_t lds_h8 = lds_addr(h8);
  const uint32_t first = lds_h8 + 4u * (128u + 2u * wv * kFiltStage);
  const uint32_t lim = first + (uint32_t)kFiltCap * 8u;
  const uint32_t dummy = lds_h8 + 8u * (uint32_t)lane;
  uint32_t at = first;
  uint32_t tcnt = 0, tw = 0, tkept = 0, neq = 0, tdrop = 0xFFFFFFFFu;
  __syncthreads();  // every wave is done with the sample bins (and the samples were waited for)
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    if (j <= jt) {
      const int lvid = slot_vid<NT>(j, jt, rem);
      if constexpr (MODE == TOPK_MODE_BLOCK) {
        const uint32_t key =
            lvid >= 0 ? (vb + lvid == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
        const uint32_t x = block_entry(key);
        keep_word_lds(x, (uint32_t)lvid, cs, lim, dummy, at);
        if (ties) keep_ties(x, (uint32_t)lvid, cs, tl, tbase, tcap, tcnt, tw, tkept, neq, tdrop);
      } else {
        // slot jt: the row's last vector is cut at the length, and lanes
        // without a vector there hold vector 0: both become bottom keys
        if (j == jt) poison_tail(raw[j], lvid >= 0 ? clamp8(v - 8 * (vb + lvid)) : 0);
        const uint32_t e8 = (uint32_t)lvid * 8u;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t w = word_of(raw[j], q2);
          const uint32_t x = cs >= 0 ? w : skey2(w);  // raw words serve when cs >= 0
          keep_word_lds(x, e8 + 2 * q2, cs, lim, dummy, at);
          if (ties)
            keep_ties(x, e8 + 2 * q2, cs, tl, tbase, tcap, tcnt, tw, tkept, neq, tdrop);
        }
      }
    }
  }
  // -- the histogram of this wave's entries, relative to the cutoff (bin 0:
  // keys at or above cs + 256; bin i: key cs + 256 - i; keys at or below cs
  // into a spill word of the lane), in 4 lane-replicated copies
  const uint32_t wcnt = (at - first) / 8u;
  const uint32_t nw = min(wcnt, (uint32_t)kFiltCap);
  const uint32_t* stg = h8 + 128 + 2 * wv * kFiltStage;
  {
    const int32_t top = cs + kRelBins;
    uint32_t* const mhc = mh + (lane & (kRelCopies - 1)) * kRelStride;
    const int32_t spill = kRelBins + (lane >> 2);
    for (uint32_t i = (uint32_t)lane; i < nw; i += 64) {
      const uint32_t x = stg[2 * i];
      atomicAdd(&mhc[clamp0(top - lo16s(x), spill)], 1u);
      if constexpr (MODE == TOPK_MODE_TOKEN) atomicAdd(&mhc[clamp0(top - hi16s(x), spill)], 1u);
    }
  }
  if (lane == 0) {
    bc[BC_CNT + wave] = wcnt;
    bc[BC_ECNT + wave] = tkept;
    bc[BC_ECNT + 4 + wave] = neq;
    bc[BC_ECNT + 8 + wave] = tw;
    bc[BC_ECNT + 12 + wave] = tdrop;
  }
  __syncthreads();
  uint32_t off = 0, E = 0, tk = 0, nq = 0;
  bool ovf = false;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t cw = bc[BC_CNT + w];
    off += w < wave ? cw : 0u;
    E += cw;
    ovf |= cw > (uint32_t)kFiltCap;
    tk += bc[BC_ECNT + w];
    nq += bc[BC_ECNT + 4 + w];
  }
  // the list: this wave's entries after the earlier waves'
  uint32_t* list = slice + kMemberList;
  if (!ovf)
    for (uint32_t i = (uint32_t)lane; i < nw; i += 64)
      *reinterpret_cast<uint2*>(list + 2 * (off + i)) =
          *reinterpret_cast<const uint2*>(stg + 2 * i);
  // the histogram, two 16-bit bins to a word (a chunk holds at most 2^14
  // keys)
  if (tid < kRelBins / 2) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int c4 = 0; c4 < kRelCopies; ++c4) {
      lo += mh[c4 * kRelStride + 2 * tid];
      hi += mh[c4 * kRelStride + 2 * tid + 1];
    }
    slice[kMemberHistOfs + tid] = lo | (hi << 16);
  }
  if (tid < 4) {
    slice[MH_TW + tid] = bc[BC_ECNT + 8 + tid];
    slice[MH_TDROP + tid] = bc[BC_ECNT + 12 + tid];
  }
  if (tid == 0) {
    slice[MH_E] = E;
    slice[MH_TKEPT] = tk;
    slice[MH_NEQ] = nq;
    slice[MH_CUT] = c;
    slice[MH_FLAGS] = (ovf ? kFlagOverflow : 0u) | (ties ? kFlagTies : 0u);
  }
}

// One chunk of 64 survivor entries (en: this lane's; a dead pair past the
// list) of element offset g: keys above Ts to output slots from the low word
// of `slot`, keys equal to Ts (when EQ) to slots cgt + the high word while
// below take; one 64-bit LDS atomic per chunk, each index written straight
// to the row's output through the block table (block entries of -inf blocks
// write -1).
template <int MODE, bool GT, bool EQ>
__device__ __forceinline__ void emit_chunk(uint2 en, uint32_t g, int32_t Ts, uint32_t cgt,
                                           uint32_t take, unsigned long long* slot,
                                           const Out& o) {
  const int lane = __lane_id();
  const int32_t s0 = lo16s(en.x), s1 = hi16s(en.x);
  const unsigned long long g0 = GT ? __ballot(s0 > Ts) : 0ull;
  const unsigned long long g1 = GT ? __ballot(s1 > Ts) : 0ull;
  const unsigned long long q0 = EQ ? __ballot(s0 == Ts) : 0ull;
  const unsigned long long q1 = EQ ? __ballot(s1 == Ts) : 0ull;
  const uint32_t ng0 = popc(g0), nq0 = popc(q0);
  const uint32_t ng = ng0 + popc(g1), nq = nq0 + popc(q1);
  if (!(ng | nq)) return;
  unsigned long long base = 0;
  if (lane == 0) base = atomicAdd(slot, (unsigned long long)ng | ((unsigned long long)nq << 32));
  const uint32_t bg = readfirst((uint32_t)base), bq = readfirst((uint32_t)(base >> 32));
  int32_t v0 = (int32_t)(en.y + g);
  int32_t v1 = v0 + 1;
  if constexpr (MODE == TOPK_MODE_BLOCK) v0 = s0 == kSNegInf ? -1 : v0;
  if (o.pages) {
    v0 = o.map(v0);
    v1 = o.map(v1);
  }
  int32_t* const out = o.out;
  if (GT) {
    if (in_mask(g0)) st_slot(out, bg + mbcnt(g0), v0);
    if (in_mask(g1)) st_slot(out, (bg + ng0) + mbcnt(g1), v1);
  }
  if (EQ && nq) {
    const uint32_t b1 = bq + nq0;
    const uint32_t room0 = sat_sub(take, bq), room1 = sat_sub(take, b1);
    const uint32_t r0 = mbcnt(q0), r1 = mbcnt(q1);
    if (in_mask(q0) && r0 < room0) st_slot(out, (cgt + bq) + r0, v0);
    if (in_mask(q1) && r1 < room1) st_slot(out, (cgt + b1) + r1, v1);
  }
}

// Survivor entry i of a member's list (i clamped into the list's region, so
// that speculative loads past the list's end stay inside the slice).
__device__ __forceinline__ uint2 ld_entry(const uint32_t* list, uint32_t i) {
  return *reinterpret_cast<const uint2*>(list + 2 * min(i, (uint32_t)kMemberCap - 1u));
}

// Exclusive prefix of the set bits over the bitmap words bm[0, nw) of one
// wave (nw a multiple of 64 or below it), into pre[0, nw).
__device__ __forceinline__ void bitmap_prefix(const uint32_t* bm, uint32_t* pre, int nw) {
  const int lane = __lane_id();
  uint32_t carry = 0;
  for (int w0 = 0; w0 < nw; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t c = w < nw ? (uint32_t)__builtin_popcount(bm[w]) : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (w < nw) pre[w] = carry + incl - c;
    carry += readlane(incl, 63);
  }
}

// Set bits in the wave's bitmap bm for the keys of entries that pass
// `pick` (chunk-local element indices; token entries hold two keys).
template <int MODE, class Pick>
__device__ __forceinline__ void bitmap_mark(uint2 en, uint32_t* bm, Pick pick) {
  const int32_t s0 = lo16s(en.x), s1 = hi16s(en.x);
  if (pick(s0)) atomicOr(&bm[en.y >> 5], 1u << (en.y & 31));
  if (MODE == TOPK_MODE_TOKEN && pick(s1))
    atomicOr(&bm[(en.y + 1) >> 5], 1u << ((en.y + 1) & 31));
}

// The selected keys of one entry (bit set in the wave's bitmap sel, key at
// or above Ts) to their ordered slots base + (selected elements before them
// in the member's chunk); pre: the exclusive prefix of sel.
template <int MODE>
__device__ __forceinline__ void bitmap_write(uint2 en, uint32_t g, int32_t Ts, uint32_t base,
                                             const uint32_t* sel, const uint32_t* pre,
                                             const Out& o, int32_t* ids) {
#pragma unroll
  for (int h = 0; h < (MODE == TOPK_MODE_TOKEN ? 2 : 1); ++h) {
    const int32_t s = h ? hi16s(en.x) : lo16s(en.x);
    const uint32_t e = en.y + (uint32_t)h;
    if (s >= Ts) {
      const uint32_t w = sel[e >> 5], bit = 1u << (e & 31);
      if (w & bit) {
        const uint32_t pos = base + pre[e >> 5] + (uint32_t)__builtin_popcount(w & (bit - 1u));
        const int32_t idx = (int32_t)(g + e);
        if (pos < o.k) {
          o.out[pos] = (MODE == TOPK_MODE_BLOCK && s == kSNegInf) ? -1 : o.map(idx);
          if (ids) ids[pos] = idx;
        }
      }
    }
  }
}

// LDS of the select kernel (32-bit words): control words, the row's summed
// histogram, a table of 16 words per member, the members' own histograms
// (ordered results), then the waves' work areas (ordered bitmaps) or the
// direct path's bins.
constexpr int kSelHist = 128;
constexpr int kSelMem = kSelHist + 272;
constexpr int kSelMhist = kSelMem + 16 * kMaxMembers;
constexpr int kSelWave = kSelMhist + (kRelBins / 2) * kMaxMembers;
enum { MT_E = 0, MT_TK = 1, MT_NQ = 2, MT_CUT = 3, MT_TW = 4, MT_GT = 8, MT_EQ = 9, MT_BASE = 10,
       MT_QUOTA = 11, MT_X = 12 };
constexpr int kListBatch = 8;  // 64-entry chunks of a member's list loaded together
constexpr int kListPre = 3;    // of them, loaded with the headers
constexpr int kItemBatch = 4;  // chunks past those a wave loads together (unordered writes)

// Stage 2: one 1024-thread workgroup per row.  Short rows are written
// directly.  Otherwise the members' headers, histograms and first entries
// are loaded together (before the row's length is known); the summed
// histogram gives the k-th key T and the count above it exactly (the keys
// above the cutoff are all in the members' lists), and the entries are
// written straight from the lists: unordered through LDS slot counters, or
// in element order through per-member bitmaps (the members' counts above
// and at T, scanned over the members, give each member its first slot and
// its share of the ties).  A cutoff tied with the k-th key takes the tie
// pass (the ties kept beside the lists); a misjudged cutoff, an overflow
// of a member's list, or a k-th key 256 or more above the cutoff sends the
// row to the direct path.
// (one 1024-thread workgroup: 4 waves a SIMD, so each may hold 128 VGPRs)
template <int MODE, bool ORD>
__global__ __launch_bounds__(kSelNT) __attribute__((amdgpu_waves_per_eu(4, 4))) void
topk_team_select(Params p) {
  constexpr int NT = kSelNT, NW = NT / 64;
  extern __shared__ uint32_t smem[];
  // ordered results: S workgroups per row, part s writing members 16 s ..
  // 16 s + 15, 16 (S + s) .., each finding T and the members' slots itself;
  // part 0 alone takes the short, direct and tie-check outcomes' writes
  const int S = ORD ? p.sel_parts : 1;
  const int lrow = blockIdx.x / S, part = blockIdx.x % S;
  const int row = p.row0 + lrow;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = tid >> 6;
  const int k = p.k;
  const int G = p.G;
  const uint32_t* slices = p.team_slices + (size_t)lrow * G * kMemberWords;
  // -- loads that need not wait for the row's length: the headers (lane m
  // of wave 0: member m), the histograms (thread t: word t % 128 of
  // members t / 128, + 8, ...) and the first kListPre 64-entry chunks of the
  // members this wave writes (wave + (part + u S) NW for u = 0, 1, ...); the
  // words of members past the row's end are stale, and dropped once the
  // length is known
  uint4 h0 = make_uint4(0u, 0u, 0u, 0u), h1 = h0, h2 = h0, h3 = h0;
  if (wave == 0 && lane < G) {
    const uint4* h4 = reinterpret_cast<const uint4*>(slices + (size_t)lane * kMemberWords);
    h0 = h4[0];
    h1 = h4[1];
    h2 = h4[2];
    if (ORD) h3 = h4[3];
  }
  constexpr int kHPer = kMaxMembers * (kRelBins / 2) / NT;
  uint32_t hw[kHPer];
#pragma unroll
  for (int i = 0; i < kHPer; ++i) {
    const int m = (tid >> 7) + (NT >> 7) * i;
    hw[i] = m < G ? slices[(size_t)m * kMemberWords + kMemberHistOfs + (tid & 127)] : 0u;
  }
  constexpr int kPreM = kMaxMembers / NW;
  uint2 pre[kPreM][kListPre];
#pragma unroll
  for (int u = 0; u < kPreM; ++u) {
    const int m = wave + (part + u * S) * NW;
#pragma unroll
    for (int c = 0; c < kListPre; ++c)
      pre[u][c] = m < G ? ld_entry(slices + (size_t)m * kMemberWords + kMemberList,
                                   (uint32_t)c * 64u + (uint32_t)lane)
                        : make_uint2(kDeadPair, 0u);
  }
  const int v = clamp_len(p.valid_len[row], p.width);
  const int n = (MODE == TOPK_MODE_BLOCK) ? (v + 7) >> 3 : v;
  const Out o = row_out(p, row, MODE == TOPK_MODE_BLOCK);
  const uint4* src = reinterpret_cast<const uint4*>(p.logits + (int64_t)row * p.row_stride);
  int32_t* const ids = (ORD && p.ids) ? p.ids + (int64_t)row * k : nullptr;
  if (n <= k) {
    if (part != 0) return;
    if constexpr (MODE == TOPK_MODE_BLOCK) write_short_block<NT>(o, src, n, k);
    else write_short_token<NT>(o, n, k);
    if constexpr (ORD) short_ids<NT>(p, row, n);
    set_path(p, row, TOPK_PATH_SHORT);
    return;
  }
  uint32_t* bc = smem;
  uint32_t* hs = smem + kSelHist;
  uint32_t* mt = smem + kSelMem;
  uint32_t* mhist = smem + kSelMhist;
  bool direct = p.force_direct != 0;
  int code = TOPK_PATH_DIRECT_FORCED;
  uint2 tc = make_uint2(0u, 0u);  // ordered results: the k-th key, the count above it
  if (!direct) {
    const int nvec = (v + 7) >> 3;
    const int gr = (nvec + p.team_cv - 1) / p.team_cv;  // members of this row
    const uint32_t chunk = (uint32_t)p.team_cv * (MODE == TOPK_MODE_BLOCK ? 1u : 8u);
    for (int i = tid; i < kRelBins; i += NT) hs[i] = 0;
    if (tid == 0) {
      bc[BC_SLOT] = 0;
      bc[BC_SLOT + 1] = 0;
    }
    // the member table and the row's totals (wave 0, lane m: member m)
    if (wave == 0) {
      const bool live = lane < gr;
      const uint32_t tk = live ? h0.z : 0u, nq = live ? h0.w : 0u;
      const uint32_t fl = live ? h2.y : 0u;
      if (lane < kMaxMembers) {
        uint32_t* e = mt + lane * 16;
        // the member's tie cut: every key equal to the cutoff below this
        // chunk-local element index was kept
        const uint32_t cut = min(min(h3.x, h3.y), min(h3.z, h3.w));
        *reinterpret_cast<uint4*>(e) = make_uint4(live ? h0.x : 0u, tk, nq, cut);
        *reinterpret_cast<uint4*>(e + MT_TW) = live ? h1 : make_uint4(0u, 0u, 0u, 0u);
      }
      // the chunks past the first kListPre of every member's list, numbered
      // over the row (member m's from e[MT_X] on), shared by all the waves
      const uint32_t xm = live ? sat_sub((h0.x + 63u) >> 6, (uint32_t)kListPre) : 0u;
      const uint32_t ix = wave_incl_scan(xm);
      if (lane < kMaxMembers) mt[lane * 16 + MT_X] = live ? ix - xm : 0xFFFFFFFFu;
      if (lane == 63) bc[BC_TMP + 5] = ix;
      const uint32_t itk = wave_incl_scan(tk), inq = wave_incl_scan(nq);
      const unsigned long long fd = __ballot(fl & kFlagDirect), fo = __ballot(fl & kFlagOverflow);
      const unsigned long long ft = __ballot(fl & kFlagTies);
      if (lane == 63) {
        bc[BC_TMP + 0] = (fd ? 1u : 0u) | (fo ? 2u : 0u) | (ft ? 4u : 0u);
        bc[BC_TMP + 1] = itk;  // tie keys kept
        bc[BC_TMP + 2] = inq;  // keys equal to the cutoff
      }
      if (lane == 0) bc[BC_TMP + 3] = h2.x;  // the cutoff (the same in every member)
    }
    __syncthreads();
    // the row's histogram, and (ordered results) the members' own
#pragma unroll
    for (int i = 0; i < kHPer; ++i) {
      const int m = (tid >> 7) + (NT >> 7) * i;
      const uint32_t w = hw[i];
      if (m < gr) {
        if (w) {
          atomicAdd(&hs[2 * (tid & 127)], w & 0xFFFFu);
          atomicAdd(&hs[2 * (tid & 127) + 1], w >> 16);
        }
        if (ORD) mhist[m * (kRelBins / 2) + (tid & 127)] = w;
      }
    }
    __syncthreads();
    const uint32_t fl = bc[BC_TMP + 0], avail = bc[BC_TMP + 1], eq_total = bc[BC_TMP + 2];
    const uint32_t c = bc[BC_TMP + 3];
    const int32_t cs = (int32_t)c - 0x8000;
    uint32_t ri, above, total;
    find_copies<1, kRelStride>(hs, (uint32_t)k, ri, above, total);
    bool tie_pass = false;
    int32_t Ts = 0;
    uint32_t cgt = 0;
    if (fl & 1u) {
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    } else if (fl & 2u) {
      direct = true;
      code = TOPK_PATH_DIRECT_OVERFLOW;
    } else if (total >= (uint32_t)k) {
      if (ri == 0) {  // the k-th key lies 256 or more above the cutoff
        direct = true;
        code = TOPK_PATH_DIRECT_OVERFLOW;
      } else {
        Ts = cs + kRelBins - (int32_t)ri;
        cgt = above;
        code = TOPK_PATH_SAMPLED;
      }
    } else if ((fl & 4u) && total + eq_total >= (uint32_t)k && avail >= (uint32_t)k - total) {
      tie_pass = true;  // the k-th key is the cutoff
      Ts = cs;
      cgt = total;
      code = TOPK_PATH_SAMPLED_TIES;
    } else {
      direct = true;
      code = TOPK_PATH_DIRECT_MISJUDGED;
    }
    const uint32_t take = (uint32_t)k - cgt;
    if (!direct && !ORD) {
      // -- unordered: every wave writes the first chunks of its members'
      // lists; the rest of the lists is shared by all the waves.
      unsigned long long* slot = reinterpret_cast<unsigned long long*>(bc + BC_SLOT);
      // the first kListPre chunks of this wave's members, loaded with the
      // headers
#pragma unroll
      for (int u = 0; u < kPreM; ++u) {
        const int m = wave + u * NW;
        if (m < gr) {
          const uint32_t g = (uint32_t)m * chunk;
          const uint32_t E = mt[m * 16 + MT_E];
#pragma unroll
          for (int c = 0; c < kListPre; ++c) {
            const uint32_t b0 = (uint32_t)c * 64u;
            if (b0 < E) {
              const uint2 e = b0 + lane < E ? pre[u][c] : make_uint2(kDeadPair, 0u);
              if (tie_pass) emit_chunk<MODE, true, false>(e, g, Ts, cgt, take, slot, o);
              else emit_chunk<MODE, true, true>(e, g, Ts, cgt, take, slot, o);
            }
          }
        }
      }
      // the chunks past those, over all the waves: item i is chunk
      // kListPre + i - X of the member m with X = e[MT_X] <= i (the last
      // such), kItemBatch of a wave's items loaded together
      const uint32_t nx = bc[BC_TMP + 5];
      const uint32_t xl = lane < gr ? mt[lane * 16 + MT_X] : 0xFFFFFFFFu;
      for (uint32_t i0 = (uint32_t)wave; i0 < nx; i0 += NW * kItemBatch) {
        uint2 en[kItemBatch];
        uint32_t im[kItemBatch], ib[kItemBatch], iE[kItemBatch];
#pragma unroll
        for (int t = 0; t < kItemBatch; ++t) {
          const uint32_t i = i0 + (uint32_t)t * NW;
          im[t] = 0;
          ib[t] = 0;
          iE[t] = 0;
          if (i < nx) {
            const int m = popc(__ballot(xl <= i)) - 1;
            const uint32_t b0 = (kListPre + i - readlane(xl, m)) * 64u;
            im[t] = (uint32_t)m;
            ib[t] = b0;
            iE[t] = mt[m * 16 + MT_E];
            en[t] = ld_entry(slices + (size_t)m * kMemberWords + kMemberList, b0 + lane);
          }
        }
#pragma unroll
        for (int t = 0; t < kItemBatch; ++t) {
          if (i0 + (uint32_t)t * NW < nx) {
            const uint2 e = ib[t] + lane < iE[t] ? en[t] : make_uint2(kDeadPair, 0u);
            const uint32_t g = im[t] * chunk;
            if (tie_pass) emit_chunk<MODE, true, false>(e, g, Ts, cgt, take, slot, o);
            else emit_chunk<MODE, true, true>(e, g, Ts, cgt, take, slot, o);
          }
        }
      }
      if (tie_pass) {
        // the first keys equal to the cutoff, from the tie regions
#pragma unroll
        for (int u = 0; u < kPreM; ++u) {
          const int m = wave + u * NW;
          if (m < gr) {
            const uint32_t g = (uint32_t)m * chunk;
            const uint32_t* tl = slices + (size_t)m * kMemberWords + kMemberTies;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t tw = mt[m * 16 + MT_TW + w];
              for (uint32_t b0 = 0; b0 < tw; b0 += 64) {
                uint2 e = b0 + lane < tw ? *reinterpret_cast<const uint2*>(
                                               tl + 2 * (w * kTieLCW + b0 + lane))
                                         : make_uint2(kDeadPair, 0u);
                emit_chunk<MODE, false, true>(e, g, Ts, cgt, take, slot, o);
              }
            }
          }
        }
      }
    } else if (!direct) {
      // -- ordered: each member's keys above and at T, scanned over the
      // members (wave w: members w, w + NW, ...; lane l: bins 4l .. 4l + 3)
#pragma unroll
      for (int u = 0; u < kPreM; ++u) {
        const int m = wave + u * NW;
        if (m < gr) {
          uint32_t gt = 0, eq = 0;
          if (tie_pass) {
            const uint2 w2 = *reinterpret_cast<const uint2*>(mhist + m * (kRelBins / 2) + 2 * lane);
            gt = (w2.x & 0xFFFFu) + (w2.x >> 16) + (w2.y & 0xFFFFu) + (w2.y >> 16);
          } else {
            const uint2 w2 = *reinterpret_cast<const uint2*>(mhist + m * (kRelBins / 2) + 2 * lane);
            const uint32_t b4[4] = {w2.x & 0xFFFFu, w2.x >> 16, w2.y & 0xFFFFu, w2.y >> 16};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t bin = 4u * (uint32_t)lane + q;
              gt += bin < ri ? b4[q] : 0u;
              eq += bin == ri ? b4[q] : 0u;
            }
          }
          gt = readlane(wave_incl_scan(gt), 63);
          eq = tie_pass ? mt[m * 16 + MT_NQ] : readlane(wave_incl_scan(eq), 63);
          if (lane == 0) {
            mt[m * 16 + MT_GT] = gt;
            mt[m * 16 + MT_EQ] = eq;
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        const bool live = lane < gr;
        const uint32_t gt = live ? mt[lane * 16 + MT_GT] : 0u;
        const uint32_t eq = live ? mt[lane * 16 + MT_EQ] : 0u;
        const uint32_t gb = wave_incl_scan(gt) - gt, eb = wave_incl_scan(eq) - eq;
        const uint32_t room = sat_sub(take, eb);  // ties left for this member and after
        const uint32_t quota = min(room, eq);
        // the tie pass needs each member's first `quota` ties by element
        // index: all of them when it takes every tie (none dropped), else
        // (the one member that takes some) enough kept below its cut
        const uint32_t cut = live ? mt[lane * 16 + MT_CUT] : 0xFFFFFFFFu;
        const bool all_short = live && tie_pass && quota > 0 && quota >= eq && cut != 0xFFFFFFFFu;
        const bool some = live && tie_pass && quota > 0 && quota < eq && cut != 0xFFFFFFFFu;
        if (live) {
          mt[lane * 16 + MT_BASE] = gb + (take - room);  // gb + min(eb, take)
          mt[lane * 16 + MT_QUOTA] = quota;
        }
        const unsigned long long bad = __ballot(all_short);
        const unsigned long long chk = __ballot(some);
        uint32_t fail_ties = bad ? 1u : 0u;
        if (chk) {
          // that member's kept ties below its cut, counted in wave 0's area
          const int m = __ffsll(chk) - 1;
          const uint32_t cm = readlane(cut, m), qm = readlane(quota, m);
          uint32_t* wb = smem + kSelWave;
          const int bw = p.sel_bw;
          for (int i = lane; i < bw; i += 64) wb[i] = 0;
          const uint32_t* tl = slices + (size_t)m * kMemberWords + kMemberTies;
          for (int w = 0; w < 4; ++w) {
            const uint32_t tw = mt[m * 16 + MT_TW + w];
            for (uint32_t b0 = 0; b0 < tw; b0 += 64) {
              const uint2 en = b0 + lane < tw ? *reinterpret_cast<const uint2*>(
                                                    tl + 2 * (w * kTieLCW + b0 + lane))
                                              : make_uint2(kDeadPair, 0u);
              bitmap_mark<MODE>(en, wb, [&](int32_t s) { return s == Ts; });
            }
          }
          uint32_t below = 0;
          for (int i = lane; i < bw; i += 64) {
            const uint32_t lo = (uint32_t)i * 32u;
            const uint32_t keep = cm >= lo + 32u ? 0xFFFFFFFFu
                                                 : (cm > lo ? (1u << (cm - lo)) - 1u : 0u);
            below += (uint32_t)__builtin_popcount(wb[i] & keep);
          }
          below = readlane(wave_incl_scan(below), 63);
          if (below < qm) fail_ties = 1u;
        }
        if (lane == 0) bc[BC_TMP + 4] = fail_ties;
      }
      __syncthreads();
      if (bc[BC_TMP + 4]) {
        direct = true;
        code = TOPK_PATH_DIRECT_OVERFLOW;
      } else {
        // per member: the selected keys' bitmap over its chunk (keys above
        // T, and its first `quota` keys at T by element index), its prefix,
        // then every selected key to base + its rank
        const int bw = p.sel_bw;
        uint32_t* sel = smem + kSelWave + wave * 3 * bw;
        uint32_t* wk = sel + bw;
        uint32_t* pf = wk + bw;
#pragma unroll 1
        for (int u = 0; u < kPreM; ++u) {
          const int m = wave + (part + u * S) * NW;
          if (m >= gr) break;
          const uint32_t Em = mt[m * 16 + MT_E], eqm = mt[m * 16 + MT_EQ];
          const uint32_t quota = mt[m * 16 + MT_QUOTA], base = mt[m * 16 + MT_BASE];
          const uint32_t* list = slices + (size_t)m * kMemberWords + kMemberList;
          const uint32_t* tl = slices + (size_t)m * kMemberWords + kMemberTies;
          const uint32_t g = (uint32_t)m * chunk;
          for (int i = lane; i < bw; i += 64) {
            sel[i] = 0;
            wk[i] = 0;
          }
          // the list's first kListBatch chunks in registers, for every pass
          // below (the first kListPre of them loaded with the headers); the
          // rest (long lists) read again per pass
          uint2 en[kListBatch];
#pragma unroll
          for (int c = 0; c < kListBatch; ++c) {
            if (c < kListPre) {
              en[c] = pre[0][c];
#pragma unroll
              for (int w = 1; w < kPreM; ++w) en[c] = u == w ? pre[w][c] : en[c];
            } else if ((uint32_t)c * 64u < Em) {
              en[c] = ld_entry(list, (uint32_t)c * 64u + (uint32_t)lane);
            }
          }
          auto for_list = [&](auto&& f) {
#pragma unroll
            for (int c = 0; c < kListBatch; ++c) {
              const uint32_t b0 = (uint32_t)c * 64u;
              if (b0 < Em) f(b0 + lane < Em ? en[c] : make_uint2(kDeadPair, 0u));
            }
            for (uint32_t b0 = kListBatch * 64u; b0 < Em; b0 += 64) {
              const uint2 e = b0 + lane < Em
                                  ? *reinterpret_cast<const uint2*>(list + 2 * (b0 + lane))
                                  : make_uint2(kDeadPair, 0u);
              f(e);
            }
          };
          auto for_ties = [&](auto&& f) {
            if (!tie_pass) {
              for_list(f);
            } else {
              for (int w = 0; w < 4; ++w) {
                const uint32_t tw = mt[m * 16 + MT_TW + w];
                for (uint32_t b0 = 0; b0 < tw; b0 += 64) {
                  const uint2 en = b0 + lane < tw ? *reinterpret_cast<const uint2*>(
                                                        tl + 2 * (w * kTieLCW + b0 + lane))
                                                  : make_uint2(kDeadPair, 0u);
                  f(en);
                }
              }
            }
          };
          for_list([&](uint2 en) { bitmap_mark<MODE>(en, sel, [&](int32_t s) { return s > Ts; }); });
          if (quota > 0) {
            if (quota >= eqm) {
              for_ties([&](uint2 en) {
                bitmap_mark<MODE>(en, sel, [&](int32_t s) { return s == Ts; });
              });
            } else {
              // the member's first `quota` keys at T: ranks from their own
              // bitmap's prefix
              for_ties([&](uint2 en) {
                bitmap_mark<MODE>(en, wk, [&](int32_t s) { return s == Ts; });
              });
              bitmap_prefix(wk, pf, bw);
              for_ties([&](uint2 en) {
#pragma unroll
                for (int h = 0; h < (MODE == TOPK_MODE_TOKEN ? 2 : 1); ++h) {
                  const int32_t s = h ? hi16s(en.x) : lo16s(en.x);
                  const uint32_t e = en.y + (uint32_t)h;
                  if (s == Ts) {
                    const uint32_t r = pf[e >> 5] +
                        (uint32_t)__builtin_popcount(wk[e >> 5] & ((1u << (e & 31)) - 1u));
                    if (r < quota) atomicOr(&sel[e >> 5], 1u << (e & 31));
                  }
                }
              });
            }
          }
          bitmap_prefix(sel, pf, bw);
          for_list([&](uint2 en) { bitmap_write<MODE>(en, g, Ts, base, sel, pf, o, ids); });
          if (tie_pass && quota > 0)
            for_ties([&](uint2 en) { bitmap_write<MODE>(en, g, Ts, base, sel, pf, o, ids); });
        }
        if (tid == 0 && part == 0 && p.valid) p.valid[row] = k;
      }
    }
    tc = make_uint2((uint32_t)(Ts + 0x8000), cgt);
  }
  if (part != 0) return;  // the direct path and the path code: part 0
  if (direct) {
    __syncthreads();
    const uint2 dt = direct_select<MODE, NT>(src, v, n, k, o, smem + kSelWave, bc, ORD);
    if constexpr (ORD) tc = dt;
    if constexpr (ORD) {
      // the ordered write pass over the row, in spans of NT * 2 vectors
      constexpr int VPT = 2;
      uint32_t* tmp = smem + kSelWave;
      uint32_t* stage = tmp + VPT * NW;
      const int nvec = (v + 7) >> 3;
      uint32_t na = 0, nt = 0;
      const uint32_t take = (uint32_t)k - tc.y;
#pragma unroll 1
      for (int vb = 0; vb < nvec && (na < tc.y || nt < take); vb += NT * VPT) {
        const int ve = min(vb + NT * VPT, nvec);
        const int jt = (ve - vb - 1) / NT, rem = (ve - vb) - jt * NT;
        uint4 raw[VPT];
        uint32_t kb[MODE == TOPK_MODE_BLOCK ? VPT : 1];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          const int lv = slot_vid<NT>(j, jt, rem, tid);
          raw[j] = ld_vec(src, (uint32_t)(vb + max(lv, 0)));
          if constexpr (MODE == TOPK_MODE_BLOCK)
            kb[j] = lv >= 0 ? (vb + lv == n - 1 ? kKeyPosInf : block_key4(raw[j])) : 0u;
        }
        __syncthreads();  // the previous span's LDS words are free
        const uint32_t tot = ordered_regs<MODE, NT, VPT>(raw, kb, jt, rem, vb, v, tc.x, tc.y, na,
                                                         nt, o, nullptr, ids, tmp, stage);
        na += tot >> 16;
        nt += tot & 0xFFFFu;
      }
      if (tid == 0 && p.valid) p.valid[row] = k;
    }
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
  bool reserved = false;  // sized by topk_reserve_scratch: calls never replace it
  bool captured = false;  // used under graph capture: nothing replaces it
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

// Team scratch, one buffer per (device, stream).  Every word a team kernel
// reads was written by an earlier kernel of the same call, so nothing needs
// zeroing between calls.  A call that needs more than the buffer holds
// replaces it (after synchronizing the stream) unless the buffer was
// reserved, or used by a call under graph capture (a captured graph keeps
// its address); the call then fails and names the reason.
int get_scratch(hipStream_t stream, size_t need, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& sc = g_scratch[std::make_pair(dev, stream)];
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  const bool capturing =
      hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone;
  if (sc.bytes < need) {
    if (capturing)
      return fail(TOPK_ERR_UNSUPPORTED, "the stream's team scratch (%zu bytes) must be set up "
                  "outside graph capture, by an earlier call or topk_reserve_scratch", need);
    if (sc.reserved || sc.captured)
      return fail(TOPK_ERR_UNSUPPORTED, "this call needs %zu bytes of team scratch on its "
                  "stream, more than the %zu %s; reserve more before capturing", need, sc.bytes,
                  sc.captured ? "held by a captured graph" : "reserved");
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
  if (capturing) sc.captured = true;
  *out = sc.base;
  return TOPK_OK;
}

// Geometry of the team path (rows wider than one workgroup): G members of
// cv vectors per row, row_bytes of scratch per row, batch rows per launch:
// all of them, unless the scratch cap (or a caller's fixed scratch) or
// kTeamBatch bounds a launch; a capped batch of 8 rows or more holds whole
// groups of 8 (one per XCD), and every launch's grid is padded to whole
// groups of 8 anyway.  False when one row needs more than cap_bytes.
struct TeamGeom {
  int vpt, cv, G, batch;
  size_t row_bytes;
};
bool team_geom(int32_t rows, int32_t width, int32_t mode, size_t cap_bytes, TeamGeom& t) {
  const int nvec_max = (width + 7) / 8;
  t.vpt = mode == TOPK_MODE_BLOCK ? kTeamBlockVPT
                                  : (nvec_max <= kMaxMembers * kTeamNT * 4 ? 4 : 8);
  t.cv = kTeamNT * t.vpt;
  t.G = (nvec_max + t.cv - 1) / t.cv;  // <= kMaxMembers
  t.row_bytes = (size_t)t.G * kMemberWords * 4;
  if (t.row_bytes > cap_bytes) return false;
  t.batch = rows < kTeamBatch ? rows : kTeamBatch;
  if ((size_t)t.batch * t.row_bytes > cap_bytes) {
    t.batch = (int)(cap_bytes / t.row_bytes);
    t.batch = t.batch < 8 ? t.batch : t.batch / 8 * 8;
  }
  return true;
}

// Whether rows of this width take the team path.
bool team_rows(int32_t width, int32_t mode) {
  const int cap_wg = kRowNT * (mode == TOPK_MODE_BLOCK ? kRowBlockVPT : kRowTokenVPT);
  return (width + 7) / 8 > cap_wg;
}

// The scratch of topk_bf16_rows_noalloc: one array per device, part of the
// code object (no allocation call creates it).  In host code its name is a
// host-side stand-in, never a device address: only the address that
// hipGetSymbolAddress returns for the current device is passed to kernels.
constexpr size_t kNoAllocBytes = size_t(16) << 20;
static __device__ __align__(256) uint32_t scratch[kNoAllocBytes / 4];

std::mutex g_noalloc_mu;
void* g_noalloc_ptr[64] = {};  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device.
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TOPK_ERR_UNSUPPORTED, "device %d beyond 64", dev);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(TOPK_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_noalloc_ptr[dev] = ptr;
  }
  *out = g_noalloc_ptr[dev];
  return TOPK_OK;
}

// Survivor entries per wave of the one-workgroup kernel before a wave
// stops writing (its region holds kSpare more).  A 16384-logit row with
// the cutoff rank of sample_rank keeps about 1.2 k + 400 entries holding a
// key above the cutoff; the workgroup takes k + k/4 + 512 of them, spread
// evenly over its waves, plus 32 per wave for imbalance.
int row_lcw(int k, int nw) { return (k + k / 4 + 512) / nw + 32; }

size_t row_lds_bytes(int lcw, int nw) {
  const int lists = nw * (lcw + kSpare) * 2 + 2 * 64;  // regions, then the dummy area
  int words = lists > kDirectWords ? lists : kDirectWords;
  if (words < kSampBins + 256) words = kSampBins + 256;  // the sample bins and their sums
  return (size_t)(kLists + words) * 4;
}

// Dynamic LDS a workgroup may take on this device (cached per device).
int device_lds_limit(int dev) {
  static int cached[64] = {0};
  if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
  int v = 65536;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    v = 65536;
  if (dev >= 0 && dev < 64) cached[dev] = v;
  return v;
}

// Raise a kernel's dynamic LDS limit to `lds` bytes once per device (not at
// every call, so that calls also work under stream capture).
int allow_lds(const void* kernel, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> g(mu);
  size_t& have = done[{dev, kernel}];
  if (have >= lds) return TOPK_OK;
  const hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "LDS of %zu bytes: %s", lds, hipGetErrorString(e));
  have = lds;
  return TOPK_OK;
}

// Workgroups of `kernel` (nt threads, lds bytes) resident on the device at
// once, cached per device, kernel and size; 0 when the runtime cannot say.
int resident_grid(const void* kernel, int nt, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = done.find({dev, kernel, lds});
    if (it != done.end()) return it->second;
  }
  if (lds > 65536 && allow_lds(kernel, lds) != TOPK_OK) return 0;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  std::lock_guard<std::mutex> g(mu);
  return done[{dev, kernel, lds}] = per_cu * cus;
}

template <class K>
int launch(K kernel, int grid, int nt, size_t lds, hipStream_t stream, const Params& p) {
  if (lds > 65536) {
    const int rc = allow_lds(reinterpret_cast<const void*>(kernel), lds);
    if (rc != TOPK_OK) return rc;
  }
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(nt), lds, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return TOPK_OK;
}

// One workgroup per row: the latency variant while every row's workgroup
// is resident at once, else the throughput variant.
template <bool ORD>
int launch_rows(int mode, int rows, size_t lds, hipStream_t stream, const Params& p) {
  if (mode == TOPK_MODE_BLOCK) {
    auto lat = topk_rows_wg<TOPK_MODE_BLOCK, kRowNT, kRowBlockVPT, false, ORD>;
    if (rows <= resident_grid(reinterpret_cast<const void*>(lat), kRowNT, lds))
      return launch(lat, rows, kRowNT, lds, stream, p);
    return launch(topk_rows_wg<TOPK_MODE_BLOCK, kRowNT, kRowBlockVPT, true, ORD>, rows, kRowNT,
                  lds, stream, p);
  }
  auto lat = topk_rows_wg<TOPK_MODE_TOKEN, kRowNT, kRowTokenVPT, false, ORD>;
  if (rows <= resident_grid(reinterpret_cast<const void*>(lat), kRowNT, lds))
    return launch(lat, rows, kRowNT, lds, stream, p);
  return launch(topk_rows_wg<TOPK_MODE_TOKEN, kRowNT, kRowTokenVPT, true, ORD>, rows, kRowNT,
                lds, stream, p);
}

// Compute units of the current device (cached per device; 0 when the
// runtime cannot say).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> g(mu);
  auto it = done.find(dev);
  if (it != done.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  return done[dev] = cus;
}

// Token rows at 1024 threads a row (2 vectors a thread), when there are no
// more rows than compute units (a row's workgroup then has its unit to
// itself; two of them on one unit, barriers of 16 waves and 16 waves' fixed
// costs outweigh the shorter serial work); kNotLaunched otherwise.
constexpr int kNotLaunched = 1;
template <bool ORD>
int launch_wide(int rows, size_t lds, hipStream_t stream, const Params& p) {
  auto wide = topk_rows_wg<TOPK_MODE_TOKEN, kWideNT, kWideTokenVPT, false, ORD>;
  if (rows > device_cus() ||
      rows > resident_grid(reinterpret_cast<const void*>(wide), kWideNT, lds))
    return kNotLaunched;
  return launch(wide, rows, kWideNT, lds, stream, p);
}

// Rows on the vector-max bound: for one word of maxima per thread, the
// latency variant while every row's workgroup is resident, else the
// throughput variant; wider rows are few.
int launch_tops(int tpt, int rows, size_t lds, hipStream_t stream, const Params& p) {
  if (tpt == 1) {
    auto lat = topk_rows_tops<1, false>;
    if (rows <= resident_grid(reinterpret_cast<const void*>(lat), kRowNT, lds))
      return launch(lat, rows, kRowNT, lds, stream, p);
    return launch(topk_rows_tops<1, true>, rows, kRowNT, lds, stream, p);
  }
  if (tpt == 2) return launch(topk_rows_tops<2, false>, rows, kRowNT, lds, stream, p);
  if (tpt == 4) return launch(topk_rows_tops<4, false>, rows, kRowNT, lds, stream, p);
  return launch(topk_rows_tops<8, false>, rows, kRowNT, lds, stream, p);
}

// Validation of a side array of vector maxima: 16-byte aligned rows of at
// least ceil(width / 8) entries.
int check_tops(const uint16_t* tops, int64_t tops_stride, int32_t width) {
  if (!tops) return fail(TOPK_ERR_INVALID_ARG, "null vector maxima");
  if (((uintptr_t)tops & 15u) != 0 || tops_stride % 8 != 0)
    return fail(TOPK_ERR_MISALIGNED, "vector maxima rows not 16-byte aligned");
  if (tops_stride < ((int64_t)width + 7) / 8)
    return fail(TOPK_ERR_INVALID_ARG, "vector maxima rows shorter than ceil(width / 8)");
  return TOPK_OK;
}

int run(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len, int32_t rows,
        int32_t width, int32_t k, int32_t mode, const topk_block_table_t* bt, int32_t* out,
        const topk_options_t* opt, int ord, int32_t* valid, int32_t* ids, void* stream_ptr,
        bool noalloc = false, const uint16_t* tops = nullptr,
        int64_t tops_stride = 0) {
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
  if (((uintptr_t)out & 3u) != 0 || ((uintptr_t)valid_len & 3u) != 0 ||
      ((uintptr_t)valid & 3u) != 0 || ((uintptr_t)ids & 3u) != 0)
    return fail(TOPK_ERR_MISALIGNED, "out, valid_len, valid or ids not 4-byte aligned");
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
  p.ord = ord;
  p.valid = ord ? valid : nullptr;
  p.ids = ord ? ids : nullptr;

  const int nvec_max = (width + 7) / 8;
  // the vector maxima, when given, serve token rows (unordered results) of
  // at least 2k vectors and at most kTopsTPT words of maxima per thread:
  // one workgroup per row, whatever the width
  if (tops && mode == TOPK_MODE_TOKEN && !ord && !p.force_direct && nvec_max >= 2 * k &&
      nvec_max <= kRowNT * 8 * kTopsTPT) {
    p.tops = tops;
    p.tops_stride = tops_stride;
    p.rows = rows;
    p.row0 = 0;
    p.lcw = row_lcw(k, kRowNT / 64);
    const int ntw = (nvec_max + 7) / 8;
    const int tpt = ntw <= kRowNT ? 1 : ntw <= 2 * kRowNT ? 2 : ntw <= 4 * kRowNT ? 4 : 8;
    // the survivor area holds the bound's high-byte bins first; its
    // low-byte bins lie past both those and the survivor regions
    const int regions = (kRowNT / 64) * (p.lcw + kSpare) * 2 + 2 * 64;
    const int h8 = tpt == 1 ? TopsBins<1>::WORDS : TopsBins<2>::WORDS;
    const int lo = kLists + ((regions > h8 ? regions : h8) + 3) / 4 * 4;
    p.tops_lo = lo;
    size_t lds = row_lds_bytes(p.lcw, kRowNT / 64);
    const size_t lo_end = (size_t)(lo + kTopsLC * kRelStride) * 4;
    if (lds < lo_end) lds = lo_end;
    p.hot_lds = (int32_t)(lds / 4);
    lds += (size_t)(kRowNT / 64) * (kHotWave + 64) * 4;
    if (bt && ((int64_t)width + bt->page_size - 1) / bt->page_size <= kPageLdsMax) {
      p.page_lds = (int32_t)(lds / 4);
      lds += (size_t)kPageLdsMax * 4;
    }
    return launch_tops(tpt, rows, lds, stream, p);
  }
  // one workgroup of 512 threads per row while the row fits its
  // registers: 2048 vectors (token) or 4096 (block)
  if (!team_rows(width, mode)) {
    p.rows = rows;
    p.row0 = 0;
    p.lcw = row_lcw(k, kRowNT / 64);
    size_t lds = row_lds_bytes(p.lcw, kRowNT / 64);
    if (bt && ((int64_t)width + bt->page_size - 1) / bt->page_size <= kPageLdsMax) {
      // the rows' block-table entries get an LDS copy after everything else
      p.page_lds = (int32_t)(lds / 4);
      lds += (size_t)kPageLdsMax * 4;
    }
    // few token rows: 1024 threads each, 2 vectors a thread, which halves
    // every thread's serial work on a row's path
    if (mode == TOPK_MODE_TOKEN) {
      Params pw = p;
      pw.lcw = row_lcw(k, kWideNT / 64);
      size_t ldw = row_lds_bytes(pw.lcw, kWideNT / 64);
      if (p.page_lds) {
        pw.page_lds = (int32_t)(ldw / 4);
        ldw += (size_t)kPageLdsMax * 4;
      }
      const int rc = ord ? launch_wide<true>(rows, ldw, stream, pw)
                         : launch_wide<false>(rows, ldw, stream, pw);
      if (rc != kNotLaunched) return rc;
    }
    // more rows than resident workgroups: the throughput variant, whose
    // exact select searches its bins with one wave (the other waves' copies
    // of that search cost issue slots that other rows' waves could use);
    // otherwise every wave searches for itself, one barrier fewer on the
    // row's path
    if (ord) return launch_rows<true>(mode, rows, lds, stream, p);
    return launch_rows<false>(mode, rows, lds, stream, p);
  }

  // team path: G members per row (filter kernel), then one workgroup per
  // row (select kernel).  Scratch: one slice per member of a launch's rows.
  const size_t cap_bytes = noalloc ? kNoAllocBytes : kTeamScratchMax;
  TeamGeom tg;
  if (!team_geom(rows, width, mode, cap_bytes, tg))
    return fail(TOPK_ERR_UNSUPPORTED, "one row of width %d needs %zu bytes of team scratch, "
                "more than the %zu available", width, tg.row_bytes, cap_bytes);
  const int vpt = tg.vpt, cv = tg.cv, G = tg.G, batch = tg.batch;
  const size_t row_bytes = tg.row_bytes;
  // (the entry point that allocates nothing: the fixed per-device array,
  // looked up only now, after every argument check)
  void* team_buf = nullptr;
  {
    const int rc = noalloc ? noalloc_scratch(&team_buf)
                           : get_scratch(stream, (size_t)batch * row_bytes, &team_buf);
    if (rc != TOPK_OK) return rc;
  }
  int rc = TOPK_OK;
  p.G = G;
  p.team_cv = cv;
  p.team_slices = static_cast<uint32_t*>(team_buf);
  // select kernel LDS: its tables, then the direct path's bins or (ordered
  // results) three bitmaps over one member's elements per wave
  p.sel_bw = (cv * (mode == TOPK_MODE_BLOCK ? 1 : 8) + 31) / 32;
  // ordered results: two select workgroups per row of more than 16 members
  // (one member a wave, or two); more parts only repeat the headers' loads
  // (43 members in 3 parts: 36.6 us against 35.9 on 1M-block rows)
  p.sel_parts = ord ? (G > kSelNT / 64 ? 2 : 1) : 1;
  size_t sel_words = kDirectWords;
  if (ord) {
    const size_t bm = (size_t)3 * (kSelNT / 64) * p.sel_bw;
    const size_t od = (size_t)2 * (kSelNT / 64) + TOPK_MAX_K;  // the ordered direct pass
    sel_words = bm > sel_words ? bm : sel_words;
    sel_words = od > sel_words ? od : sel_words;
  }
  const size_t sel_lds = (kSelWave + sel_words) * 4;
  for (int r0 = 0; r0 < rows; r0 += batch) {
    const int nr = (rows - r0) < batch ? (rows - r0) : batch;
    p.row0 = r0;
    p.rows = nr;
    const int grid = (nr + 7) / 8 * 8 * G;
    if (mode == TOPK_MODE_BLOCK)
      rc = launch(topk_team_filter<TOPK_MODE_BLOCK, kTeamBlockVPT, kBlockSV>, grid, kTeamNT, 0,
                  stream, p);
    else if (vpt == 4)
      rc = launch(topk_team_filter<TOPK_MODE_TOKEN, 4, kTokenSV>, grid, kTeamNT, 0, stream, p);
    else
      rc = launch(topk_team_filter<TOPK_MODE_TOKEN, 8, kTokenSV>, grid, kTeamNT, 0, stream, p);
    if (rc == TOPK_OK) {
      const int sg = nr * p.sel_parts;
      if (mode == TOPK_MODE_BLOCK)
        rc = ord ? launch(topk_team_select<TOPK_MODE_BLOCK, true>, sg, kSelNT, sel_lds, stream, p)
                 : launch(topk_team_select<TOPK_MODE_BLOCK, false>, sg, kSelNT, sel_lds, stream, p);
      else
        rc = ord ? launch(topk_team_select<TOPK_MODE_TOKEN, true>, sg, kSelNT, sel_lds, stream, p)
                 : launch(topk_team_select<TOPK_MODE_TOKEN, false>, sg, kSelNT, sel_lds, stream, p);
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
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, nullptr, 0,
             nullptr, nullptr, stream);
}

int topk_bf16_rows_ex(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len,
                      int32_t rows, int32_t width, int32_t k, int32_t mode,
                      const topk_block_table_t* block_table, int32_t* out,
                      const topk_options_t* options, void* stream) {
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, options, 0,
             nullptr, nullptr, stream);
}

int topk_bf16_rows_noalloc(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len,
                           int32_t rows, int32_t width, int32_t k, int32_t mode,
                           const topk_block_table_t* block_table, int32_t* out, void* stream) {
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, nullptr, 0,
             nullptr, nullptr, stream, true);
}

int topk_bf16_rows_tops(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len,
                        int32_t rows, int32_t width, int32_t k, int32_t mode,
                        const uint16_t* tops, int64_t tops_stride,
                        const topk_block_table_t* block_table, int32_t* out,
                        const topk_options_t* options, void* stream) {
  g_err[0] = '\0';
  if (mode == TOPK_MODE_TOKEN && rows > 0) {
    const int rc = check_tops(tops, tops_stride, width);
    if (rc != TOPK_OK) return rc;
  }
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, options, 0,
             nullptr, nullptr, stream, false, mode == TOPK_MODE_TOKEN ? tops : nullptr,
             tops_stride);
}

int topk_bf16_vector_maxima(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len,
                            int32_t rows, int32_t width, uint16_t* tops, int64_t tops_stride,
                            void* stream) {
  g_err[0] = '\0';
  if (rows < 0) return fail(TOPK_ERR_INVALID_ARG, "rows < 0");
  if (width < 0 || width > TOPK_MAX_WIDTH)
    return fail(TOPK_ERR_INVALID_ARG, "width = %d outside [0, %d]", width, TOPK_MAX_WIDTH);
  if (row_stride < width) return fail(TOPK_ERR_INVALID_ARG, "row_stride < width");
  if (row_stride % 8 != 0) return fail(TOPK_ERR_MISALIGNED, "row_stride not a multiple of 8");
  if (rows == 0 || width == 0) return TOPK_OK;
  if (!logits || !valid_len) return fail(TOPK_ERR_INVALID_ARG, "null pointer");
  if (((uintptr_t)logits & 15u) != 0) return fail(TOPK_ERR_MISALIGNED, "logits not 16-byte aligned");
  if (((uintptr_t)valid_len & 3u) != 0)
    return fail(TOPK_ERR_MISALIGNED, "valid_len not 4-byte aligned");
  const int rc = check_tops(tops, tops_stride, width);
  if (rc != TOPK_OK) return rc;
  MaxParams q;
  q.logits = logits;
  q.row_stride = row_stride;
  q.valid_len = valid_len;
  q.width = width;
  q.tops = tops;
  q.tops_stride = tops_stride;
  const int words = ((width + 7) / 8 + 7) / 8;
  const dim3 grid((unsigned)((words + 255) / 256), (unsigned)(rows < 65535 ? rows : 65535));
  hipLaunchKernelGGL(topk_vector_maxima, grid, dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), q, rows);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return TOPK_OK;
}

int topk_bf16_rows_ordered(const uint16_t* logits, int64_t row_stride, const int32_t* valid_len,
                           int32_t rows, int32_t width, int32_t k, int32_t mode,
                           const topk_block_table_t* block_table, int32_t* out, int32_t* valid,
                           int32_t* ids, void* stream) {
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, nullptr, 1,
             valid, ids, stream);
}

int topk_bf16_rows_ordered_ex(const uint16_t* logits, int64_t row_stride,
                              const int32_t* valid_len, int32_t rows, int32_t width, int32_t k,
                              int32_t mode, const topk_block_table_t* block_table, int32_t* out,
                              int32_t* valid, int32_t* ids, const topk_options_t* options,
                              void* stream) {
  return run(logits, row_stride, valid_len, rows, width, k, mode, block_table, out, options, 1,
             valid, ids, stream);
}

const char* topk_status_string(int status) {
  switch (status) {
    case TOPK_OK: return "ok";
    case TOPK_ERR_INVALID_ARG: return "invalid argument";
    case TOPK_ERR_MISALIGNED: return "misaligned logits or row stride";
    case TOPK_ERR_HIP: return "HIP runtime error";
    case TOPK_ERR_UNSUPPORTED: return "unsupported call";
    default: return "unknown status";
  }
}

const char* topk_last_error(void) { return g_err; }

}  // extern "C"

// The status of a call made in another source file of the library, its
// text kept for topk_last_error.
__attribute__((visibility("hidden"))) int topk_report(int status, const char* text) {
  return fail(status, "%s", text);
}

extern "C" {

int topk_reserve_scratch(int32_t rows, int32_t width, int32_t k, int32_t mode, int32_t ordered,
                         void* stream_ptr) {
  g_err[0] = '\0';
  (void)ordered;  // the ordered results take no more scratch
  if (rows < 0) return fail(TOPK_ERR_INVALID_ARG, "rows < 0");
  if (k < 1 || k > TOPK_MAX_K) return fail(TOPK_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, TOPK_MAX_K);
  if (mode != TOPK_MODE_TOKEN && mode != TOPK_MODE_BLOCK)
    return fail(TOPK_ERR_INVALID_ARG, "mode = %d", mode);
  if (width < 0 || width > TOPK_MAX_WIDTH)
    return fail(TOPK_ERR_INVALID_ARG, "width = %d outside [0, %d]", width, TOPK_MAX_WIDTH);
  if (rows == 0 || !team_rows(width, mode)) return TOPK_OK;  // every row fits one workgroup
  TeamGeom tg;
  if (!team_geom(rows, width, mode, kTeamScratchMax, tg))
    return fail(TOPK_ERR_UNSUPPORTED, "one row of width %d needs more than %zu bytes of team "
                "scratch", width, kTeamScratchMax);
  const int64_t need = (int64_t)tg.batch * (int64_t)tg.row_bytes;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TOPK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& sc = g_scratch[std::make_pair(dev, stream)];
  if (sc.bytes < (size_t)need) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone)
      return fail(TOPK_ERR_UNSUPPORTED, "scratch cannot be reserved under graph capture");
    if (sc.captured)
      return fail(TOPK_ERR_UNSUPPORTED, "the stream's team scratch (%zu bytes) is held by a "
                  "captured graph; growing it to %lld bytes would free memory the graph uses "
                  "(reserve before capturing)", sc.bytes, (long long)need);
    if (sc.base) {
      e = hipStreamSynchronize(stream);
      if (e == hipSuccess) e = hipFree(sc.base);
      sc.base = nullptr;
      sc.bytes = 0;
      if (e != hipSuccess) return fail(TOPK_ERR_HIP, "scratch release: %s", hipGetErrorString(e));
    }
    e = hipMalloc(&sc.base, (size_t)need);
    if (e != hipSuccess) {
      sc.base = nullptr;
      return fail(TOPK_ERR_HIP, "scratch hipMalloc(%lld): %s", (long long)need,
                  hipGetErrorString(e));
    }
    sc.bytes = (size_t)need;
  }
  sc.reserved = true;
  return TOPK_OK;
}

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
