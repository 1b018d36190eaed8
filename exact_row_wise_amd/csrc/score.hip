// FP8 and MXFP4 MQA indexer logits for the exact top-k: the scorer of the
// decode indexer (vLLM API page "vllm.models.kimi_k3.nvidia.specialized_
// decode.cutedsl.dsa.indexer", module docstring and IndexerScore).  For
// query row t of request r = t / qpr and key i of that request:
//   FP8:   logit[t][i] = bf16(2^(s_i - 127) * sum_h bf16(relu(q[t][h] . key[i])) * w[t][h])
//   MXFP4: logit[t][i] = sum_h bf16(relu(q[t][h] . key[i])) * w[t][h], where the
//          dot product scales each 32-dim block by its query and key UE8M0 bytes
// at the page's precision: each head's FP32 dot product rounded to BF16
// after relu, the heads weighted by BF16 FMAs into four accumulators (heads
// j, j + 4, ..., j + 28), summed (a0 + a2) + (a1 + a3); for FP8 then scaled
// by the key's UE8M0 exponent (MXFP4: the scales are in the dot products,
// and a -0 logit is written +0); and each 8 keys' largest order-preserving
// key into a side array (the vector maxima topk_bf16_rows_tops takes).
//
// MI355X design.  Keys are the only large stream (FP8: 128 + 1 bytes a key;
// MXFP4: 64 + 4), so the kernel is HBM-bound: a workgroup of 4 waves takes
// 256 consecutive keys of one request and reads each key once for all the
// request's rows.  Per wave and row, 8 FP8 MFMAs (16 heads x 16 keys x 128
// dims each) give the 32 heads of 64 keys (MXFP4: the block-scaled form of
// the same MFMA, each lane's scale byte covering its 32-dim block); an LDS
// transpose hands every lane one key's 32 heads, and the lane runs the BF16
// chain in FP32 FMAs, each result rounded to BF16 by the hardware
// conversion (to nearest, ties to even).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "libtopk.h"

// error text of the library (libtopk.hip)
int topk_report(int status, const char* text);

namespace {

constexpr int kHeads = 32;
constexpr int kDim = 128;
constexpr int kScoreNT = 256;           // 4 waves
constexpr int kWaveKeys = 64;           // keys a wave scores (4 MFMA columns of 16)
constexpr int kTileKeys = kScoreNT;     // keys a workgroup scores
constexpr int kRowBytes = 72;           // LDS bytes per key of the transpose (64 + 8: fewer bank conflicts)
constexpr int kMaxQ = 8;                // query rows a request at most

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct ScoreParams {
  const uint8_t* q;         // FP8: [rows, 32, 128] E4M3; MXFP4: [rows, 32, 64] E2M1
  const uint8_t* q_scales;  // MXFP4: [rows, 32, 4] UE8M0 (one per 32 dims of a head)
  const uint16_t* w;        // [rows, 32] BF16
  const uint8_t* keys;      // FP8: [requests, key_stride, 128] E4M3; MXFP4: [.., 64] E2M1
  const uint8_t* scales;    // FP8: [requests, key_stride] UE8M0; MXFP4: [.., 4]
  int64_t key_stride;       // keys a request's slot holds
  const int32_t* valid_len; // [rows]
  int32_t rows, qpr, width;
  uint16_t* logits;
  int64_t logits_stride;
  uint16_t* tops;
  int64_t tops_stride;
};

// Two FP32 values rounded to BF16 (to nearest, ties to even), packed.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_f(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_f(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// relu of a head's FP32 dot product (NaN counts as 0).  E2M1 inputs hold
// no NaN, so there the sign bit alone decides: one integer maximum of the
// bits (negatives and -0 become +0).
template <bool FP4>
__device__ __forceinline__ float relu(float x) {
  if constexpr (FP4) return __int_as_float(max(__float_as_int(x), 0));
  return x > 0.f ? x : 0.f;
}

// The order-preserving 16-bit key of a BF16 pattern.
__device__ __forceinline__ uint32_t order16(uint32_t b) {
  return b ^ ((b & 0x8000u) ? 0xFFFFu : 0x8000u);
}

__device__ __forceinline__ int32_t clamp_len(int32_t v, int32_t width) {
  return v < 0 ? 0 : (v > width ? width : v);
}

// 32 bytes of E4M3 at p (16-byte aligned) as one MFMA operand.
__device__ __forceinline__ v8i ld32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

// 16 bytes of E2M1 at p (16-byte aligned, 32 dims) as one MFMA operand (the
// FP4 form reads the first four registers).
__device__ __forceinline__ v8i ld16(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  // operand formats 0, 0: FP8 E4M3 both; scales 0: unscaled
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// The block-scaled FP4 form: formats 4, 4 (E2M1 both); each lane's UE8M0
// byte scales its 32-dim block of A (sa) and of B (sb).
__device__ __forceinline__ v4f mfma_fp4(v8i a, v8i b, int sa, int sb) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 0, sa, 0, sb);
}

// Workgroup: keys [tile * 256, tile * 256 + 256) of request blockIdx.y, for
// each of its rows; wave w: keys +64 w.  Operand layouts of the 16x16x128
// MFMA: lane l holds row (l % 16) of A and column (l % 16) of B over dims
// 32 (l / 16) .. +32 (and, block-scaled, those dims' scale bytes), and D's
// rows 4 (l / 16) .. +4 at column l % 16.
template <bool FP4>
__global__ __launch_bounds__(kScoreNT) void topk_mqa_score(ScoreParams p) {
  __shared__ __align__(16) uint8_t tr[kScoreNT / 64][kWaveKeys * kRowBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int req = blockIdx.y;
  const int t0 = req * p.qpr;
  int vmax = 0;
  for (int u = 0; u < p.qpr; ++u) vmax = max(vmax, clamp_len(p.valid_len[t0 + u], p.width));
  const int kb = blockIdx.x * kTileKeys + wave * kWaveKeys;  // this wave's first key
  if (kb >= vmax) return;
  const int64_t kbase = (int64_t)req * p.key_stride;
  const int lc = lane & 15, lg = lane >> 4;
  // the wave's 64 keys: column c holds keys kb + 16 c + (l % 16); a key
  // past the slot reads the slot's last key (its logit is never written)
  v8i kop[4];
  int ksc[4];  // MXFP4: column c's key scale byte of this lane's block
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t i = min((int64_t)(kb + 16 * c + lc), p.key_stride - 1);
    if constexpr (FP4) {
      kop[c] = ld16(p.keys + (kbase + i) * (kDim / 2) + 16 * lg);
      ksc[c] = p.scales[(kbase + i) * 4 + lg];
    } else {
      kop[c] = ld32(p.keys + (kbase + i) * kDim + 32 * lg);
    }
  }
  const int64_t si = min((int64_t)(kb + lane), p.key_stride - 1);
  const uint32_t sbyte = FP4 ? 0u : p.scales[kbase + si];
  uint8_t* const lt = tr[wave];
  for (int u = 0; u < p.qpr; ++u) {
    const int t = t0 + u;
    const int v = clamp_len(p.valid_len[t], p.width);
    if (kb >= v) continue;
    v8i qa, qb;  // heads 0..15, 16..31
    int sqa = 0, sqb = 0;
    if constexpr (FP4) {
      const uint8_t* qt = p.q + (int64_t)t * kHeads * (kDim / 2);
      qa = ld16(qt + (int64_t)lc * (kDim / 2) + 16 * lg);
      qb = ld16(qt + (int64_t)(16 + lc) * (kDim / 2) + 16 * lg);
      const uint8_t* st = p.q_scales + (int64_t)t * kHeads * 4;
      sqa = st[lc * 4 + lg];
      sqb = st[(16 + lc) * 4 + lg];
    } else {
      const uint8_t* qt = p.q + (int64_t)t * kHeads * kDim;
      qa = ld32(qt + (int64_t)lc * kDim + 32 * lg);
      qb = ld32(qt + (int64_t)(16 + lc) * kDim + 32 * lg);
    }
    // the head weights as FP32 (the same in every lane: scalar registers)
    const uint32_t* wt = reinterpret_cast<const uint32_t*>(p.w + (int64_t)t * kHeads);
    float wf[kHeads];
#pragma unroll
    for (int i = 0; i < kHeads / 2; ++i) {
      const uint32_t x = wt[i];
      wf[2 * i] = lo_f(x);
      wf[2 * i + 1] = hi_f(x);
    }
    // heads x keys, relu, BF16, into the wave's transpose area: key row
    // 16 c + l % 16, heads 4 (l / 16) .. +4 (and 16 more)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v4f da = FP4 ? mfma_fp4(qa, kop[c], sqa, ksc[c]) : mfma_fp8(qa, kop[c]);
      const v4f db = FP4 ? mfma_fp4(qb, kop[c], sqb, ksc[c]) : mfma_fp8(qb, kop[c]);
      uint8_t* row = lt + (16 * c + lc) * kRowBytes;
      const uint2 pa = make_uint2(pack_bf16(relu<FP4>(da[0]), relu<FP4>(da[1])),
                                  pack_bf16(relu<FP4>(da[2]), relu<FP4>(da[3])));
      const uint2 pb = make_uint2(pack_bf16(relu<FP4>(db[0]), relu<FP4>(db[1])),
                                  pack_bf16(relu<FP4>(db[2]), relu<FP4>(db[3])));
      *reinterpret_cast<uint2*>(row + 8 * lg) = pa;
      *reinterpret_cast<uint2*>(row + 32 + 8 * lg) = pb;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane l: key kb + l, its 32 heads as 16 BF16 pairs
    uint32_t r[16];
    const uint8_t* row = lt + lane * kRowBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint2 x = *reinterpret_cast<const uint2*>(row + 8 * i);
      r[2 * i] = x.x;
      r[2 * i + 1] = x.y;
    }
    // accumulators j = 0..3 over heads j, j + 4, ...: pairs (0, 1), (2, 3)
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t r01 = r[2 * i], r23 = r[2 * i + 1];
      const uint32_t s01 = pack_bf16(fmaf(lo_f(r01), wf[4 * i], a0), fmaf(hi_f(r01), wf[4 * i + 1], a1));
      const uint32_t s23 = pack_bf16(fmaf(lo_f(r23), wf[4 * i + 2], a2), fmaf(hi_f(r23), wf[4 * i + 3], a3));
      a0 = lo_f(s01);
      a1 = hi_f(s01);
      a2 = lo_f(s23);
      a3 = hi_f(s23);
    }
    const uint32_t pr = pack_bf16(a0 + a2, a1 + a3);
    const float total = lo_f(pack_bf16(lo_f(pr) + hi_f(pr), 0.f));
    uint32_t bits;
    if constexpr (FP4) {
      bits = pack_bf16(total, 0.f) & 0xFFFFu;  // exact: total is a BF16 value
      if (bits == 0x8000u) bits = 0u;
    } else {
      bits = pack_bf16(ldexpf(total, (int)sbyte - 127), 0.f) & 0xFFFFu;
    }
    const int key = kb + lane;
    if (key < v) p.logits[(int64_t)t * p.logits_stride + key] = (uint16_t)bits;
    // each 8 keys' largest key (keys past the row's length count as 0)
    uint32_t top = key < v ? order16(bits) : 0u;
    top = max(top, (uint32_t)__shfl_xor((int)top, 1));
    top = max(top, (uint32_t)__shfl_xor((int)top, 2));
    top = max(top, (uint32_t)__shfl_xor((int)top, 4));
    if ((lane & 7) == 0 && key < v) p.tops[(int64_t)t * p.tops_stride + key / 8] = (uint16_t)top;
    __builtin_amdgcn_wave_barrier();  // the next row's transpose reuses the area
  }
}

int report(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int report(int status, const char* fmt, ...) {
  char text[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(text, sizeof(text), fmt, ap);
  va_end(ap);
  return topk_report(status, text);
}

}  // namespace

namespace {

int score_call(bool fp4, const uint8_t* q, const uint8_t* q_scale, const uint16_t* w,
               const uint8_t* keys, const uint8_t* key_scale, int64_t key_stride,
               const int32_t* valid_len, int32_t rows, int32_t qpr, int32_t width,
               uint16_t* logits, int64_t logits_stride, uint16_t* tops, int64_t tops_stride,
               void* stream) {
  if (rows < 0) return report(TOPK_ERR_INVALID_ARG, "rows %d < 0", rows);
  if (qpr < 1 || qpr > kMaxQ)
    return report(TOPK_ERR_INVALID_ARG, "rows per request %d not in [1, %d]", qpr, kMaxQ);
  if (rows % qpr) return report(TOPK_ERR_INVALID_ARG, "rows %d not a multiple of %d", rows, qpr);
  if (width < 0 || width > TOPK_MAX_WIDTH)
    return report(TOPK_ERR_INVALID_ARG, "width %d not in [0, %d]", width, TOPK_MAX_WIDTH);
  if (rows == 0 || width == 0) return report(TOPK_OK, "");
  if (!q || !w || !keys || !key_scale || !valid_len || !logits || !tops || (fp4 && !q_scale))
    return report(TOPK_ERR_INVALID_ARG, "a null pointer");
  if (key_stride < width)
    return report(TOPK_ERR_INVALID_ARG, "key stride %lld < width %d", (long long)key_stride, width);
  if (logits_stride < width)
    return report(TOPK_ERR_INVALID_ARG, "logits stride %lld < width %d", (long long)logits_stride,
                  width);
  if (tops_stride < (width + 7) / 8)
    return report(TOPK_ERR_INVALID_ARG, "tops stride %lld < %d", (long long)tops_stride,
                  (width + 7) / 8);
  if (((uintptr_t)q | (uintptr_t)keys) & 15)
    return report(TOPK_ERR_MISALIGNED, "q and keys must be 16-byte aligned");
  if (((uintptr_t)w | (uintptr_t)logits | (uintptr_t)tops) & 1)
    return report(TOPK_ERR_MISALIGNED, "w, logits and tops must be 2-byte aligned");
  if ((uintptr_t)w & 3) return report(TOPK_ERR_MISALIGNED, "w must be 4-byte aligned");
  ScoreParams p;
  p.q = q;
  p.q_scales = q_scale;
  p.w = w;
  p.keys = keys;
  p.scales = key_scale;
  p.key_stride = key_stride;
  p.valid_len = valid_len;
  p.rows = rows;
  p.qpr = qpr;
  p.width = width;
  p.logits = logits;
  p.logits_stride = logits_stride;
  p.tops = tops;
  p.tops_stride = tops_stride;
  const dim3 grid((width + kTileKeys - 1) / kTileKeys, rows / qpr);
  if (fp4)
    hipLaunchKernelGGL(topk_mqa_score<true>, grid, dim3(kScoreNT), 0,
                       static_cast<hipStream_t>(stream), p);
  else
    hipLaunchKernelGGL(topk_mqa_score<false>, grid, dim3(kScoreNT), 0,
                       static_cast<hipStream_t>(stream), p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return report(TOPK_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return report(TOPK_OK, "");
}

}  // namespace

extern "C" int topk_fp8_mqa_logits(const uint8_t* q, const uint16_t* w, const uint8_t* keys,
                                   const uint8_t* key_scale, int64_t key_stride,
                                   const int32_t* valid_len, int32_t rows, int32_t qpr,
                                   int32_t width, uint16_t* logits, int64_t logits_stride,
                                   uint16_t* tops, int64_t tops_stride, void* stream) {
  return score_call(false, q, nullptr, w, keys, key_scale, key_stride, valid_len, rows, qpr,
                    width, logits, logits_stride, tops, tops_stride, stream);
}

extern "C" int topk_mxfp4_mqa_logits(const uint8_t* q, const uint8_t* q_scale, const uint16_t* w,
                                     const uint8_t* keys, const uint8_t* key_scale,
                                     int64_t key_stride, const int32_t* valid_len, int32_t rows,
                                     int32_t qpr, int32_t width, uint16_t* logits,
                                     int64_t logits_stride, uint16_t* tops, int64_t tops_stride,
                                     void* stream) {
  return score_call(true, q, q_scale, w, keys, key_scale, key_stride, valid_len, rows, qpr,
                    width, logits, logits_stride, tops, tops_stride, stream);
}
