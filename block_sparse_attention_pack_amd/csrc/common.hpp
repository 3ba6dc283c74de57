// Shared device and host helpers of the gfx950 sparse decode-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/bsa.h"

namespace bsa {

constexpr int kHeadDim = 128;
constexpr int kBlock = 128;       // tokens per selectable block (Jet-QSparse abstract)
constexpr int kCodeRecord = 8192; // bytes of E2M1 codes per (unit, block)
constexpr int kScaleRecord = 1024;// bytes of E4M3 scales per (unit, block)
constexpr int kWave = 64;
constexpr int kMaxGroup = 16;     // query heads per KV head held by one MFMA row set

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

// The block scan's query side of one unit, staged in LDS by its work-group:
// with an NVFP4 query, e2m1 * e4m3 of head n, channels 8 c .. 8 c + 7 at
// q[16 n + c] and the head's FP32 scale at s_q[n]; for every query, the head's
// q . c (times s_q) at qc[n].
struct ScanQueryLds {
  half8 q[kMaxGroup * 16];
  float s_q[kMaxGroup];
  float qc[kMaxGroup];
};

// Token selection's first radix digit: the top 12 bits of a score's key
// (score_key), counted per unit in a 4096-bin histogram.
constexpr int kTokHistShift = 20;
constexpr int kTokHistBins = 4096;

// --- number formats --------------------------------------------------------

// OCP E4M3FN byte -> float (exact). 0x7F / 0xFF (NaN) never occur in a packed
// scale: the packer saturates at 0x7E.
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e ? __builtin_ldexpf(float(8u + m), int(e) - 10)  // 2^(e-7) (1 + m/8)
                      : __builtin_ldexpf(float(m), -9);               // m 2^-9
  return (b & 0x80u) ? -mag : mag;
}

// Nearest E4M3FN code of r >= 0, ties to the even code, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_from_float(float r) {
  if (!(r > 0.0f)) return 0u;
  if (r >= 448.0f) return 0x7Eu;
  const int e = int((__float_as_uint(r) >> 23) & 0xFFu) - 127;  // r is a normal float here
  uint32_t code;
  if (e < -6) {
    // subnormal range: value = m * 2^-9, m in 0..8 (m = 8 is the smallest normal)
    code = uint32_t(__builtin_rintf(__builtin_ldexpf(r, 9)));
  } else {
    // r = 2^e * (1 + f), mantissa 3 bits: m = rne((r / 2^e - 1) * 8), may carry to 8
    const float frac = __builtin_ldexpf(r, 3 - e) - 8.0f;  // exact
    const uint32_t m = uint32_t(__builtin_rintf(frac));
    code = (uint32_t(e + 7) << 3) + m;
  }
  return code > 0x7Eu ? 0x7Eu : code;
}

// Nearest E2M1 code of x (ties to the even code, saturating at 6), sign from x.
__device__ __forceinline__ uint32_t e2m1_from_float(float x) {
  const float a = __builtin_fabsf(x);
  uint32_t c;
  if (a <= 0.25f) c = 0;        // 0   (0.25 ties to code 0)
  else if (a < 0.75f) c = 1;    // 0.5
  else if (a <= 1.25f) c = 2;   // 1   (0.75 and 1.25 tie to code 2)
  else if (a < 1.75f) c = 3;    // 1.5
  else if (a <= 2.5f) c = 4;    // 2   (1.75 and 2.5 tie to code 4)
  else if (a < 3.5f) c = 5;     // 3
  else if (a <= 5.0f) c = 6;    // 4   (3.5 and 5 tie to code 6)
  else c = 7;                   // 6   (saturation)
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Value of an E2M1 code (sign in bit 3): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_to_float(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e ? __builtin_ldexpf(float(2u + m), int(e) - 2) : 0.5f * float(m);
  return (c & 8u) ? -mag : mag;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t bits) {
  union { uint16_t u; _Float16 h; } cv;
  cv.u = bits;
  return float(cv.h);
}

// Order-preserving map of a float score to an unsigned key: larger score ->
// larger key; -0 and +0 share a key; NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 0u;
  if (s == 0.0f) s = 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// --- wave reductions (64 lanes) --------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// DPP row rotation (within each 16-lane row) of a float.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, false));
}

// Maximum over the 16 lanes of a row (lanes 16r .. 16r+15), in every lane of it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}

// Sum over the 16 lanes of a row; every lane gets a sum (the summation order
// differs between lanes, so only one lane's value should be kept).
__device__ __forceinline__ float row16_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  return v + row_ror<1>(v);
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Maximum over the wave, as a wave-uniform value: DPP within the 16-lane rows,
// then the four row results. Every lane of the wave must be active.
__device__ __forceinline__ float wave_max_uniform(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// Sum over the wave, as a wave-uniform value, in a fixed order (rows as
// row16_sum's lane 16r sums them, then (r0 + r1) + (r2 + r3)). Every lane of
// the wave must be active.
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Orders a wave's LDS writes before its later LDS reads (of other lanes' data).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// --- device-wide hand-off between work-groups of one launch -----------------
// The attention kernel's merge passes the split partials from every
// work-group of a unit to the unit's last one. Those values are stored and
// loaded as device-scope atomics, which reach the memory-side coherence point
// past each XCD's L2, so no L2 write-back fence is needed: a writer waits for
// its stores to complete before it counts itself in the unit's counter.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wave-wide scans and reductions with DPP moves (ALU lane exchanges, no LDS
// round trip): four row shifts combine the lanes of each 16-lane row, then
// lane 15 of rows 0 and 2 is broadcast into rows 1 and 3, and lane 31 into
// rows 2 and 3. A lane whose source lies outside its row keeps `old`.
constexpr int kDppRowShr = 0x110;      // + n: lane i takes lane i - n of its row
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of a row into the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 into rows 2 and 3

template <int CTRL, int ROWS>
using DppStep = std::integral_constant<int, CTRL | ROWS << 16>;  // a step: control, rows written
template <class Step>
__device__ __forceinline__ int dpp_move(int old, int x, Step) {
  return __builtin_amdgcn_update_dpp(old, x, Step::value & 0xFFFF, Step::value >> 16, 0xF, false);
}
template <class Op>
__device__ __forceinline__ void wave_dpp_steps(Op&& op) {
  op(DppStep<kDppRowShr + 1, 0xF>{});
  op(DppStep<kDppRowShr + 2, 0xF>{});
  op(DppStep<kDppRowShr + 4, 0xF>{});
  op(DppStep<kDppRowShr + 8, 0xF>{});
  op(DppStep<kDppRowBcast15, 0xA>{});
  op(DppStep<kDppRowBcast31, 0xC>{});
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ int wave_scan_dpp(int x) {
  wave_dpp_steps([&](auto step) { x += dpp_move(0, x, step); });
  return x;
}

// The wave's minimum and maximum (the same in every lane).
__device__ __forceinline__ void wave_minmax_dpp(uint32_t& lo, uint32_t& hi) {
  wave_dpp_steps([&](auto step) {
    const uint32_t l = uint32_t(dpp_move(int(lo), int(lo), step));
    const uint32_t h = uint32_t(dpp_move(int(hi), int(hi), step));
    lo = l < lo ? l : lo;
    hi = h > hi ? h : hi;
  });
  lo = uint32_t(__builtin_amdgcn_readlane(int(lo), kWave - 1));
  hi = uint32_t(__builtin_amdgcn_readlane(int(hi), kWave - 1));
}

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Counts the calling work-group in counters[unit]; true in exactly one group,
// the last of `groups` to arrive, which also returns the counter to zero.
// Call from every thread after the group's hand-off stores (all threads must
// reach it: it synchronises the group).
__device__ __forceinline__ bool last_group_of_unit(uint32_t* counters, int unit, uint32_t groups,
                                                  int* lds_flag) {
  wait_all_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(&counters[unit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = before == groups - 1;
    if (last) __hip_atomic_store(&counters[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag != 0;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int clamp_len(int L, int tmax) { return L < 0 ? 0 : (L > tmax ? tmax : L); }

}  // namespace bsa

// --- host launchers (defined in the kernel files, called by api.hip) -------

namespace bsa {

struct UnitGeom {
  int B, Hkv, Hq, G, Tmax, NBmax;
  int64_t sb, sh, st;  // K/V strides in elements
  int dtype;
  bool vq;  // V is the 4-bit value store (BSA_VALUE_NVFP4)
};

// The 4-bit value store in one buffer: E2M1 codes [B][Hkv][Tmax][64], then
// E4M3 scales [B][Hkv][Tmax][8], then the FP32 scale per KV head.
constexpr int kValueCodeRow = 64;
constexpr int kValueScaleRow = 8;
struct ValueStore {
  uint8_t* codes;
  uint8_t* scales;
  float* s_v;
};
inline size_t value_store_bytes(const UnitGeom& g) {
  const size_t rows = size_t(g.B) * size_t(g.Hkv) * size_t(g.Tmax);
  return rows * (kValueCodeRow + kValueScaleRow) + sizeof(float) * size_t(g.Hkv);
}
inline ValueStore value_store(const UnitGeom& g, const void* base) {
  uint8_t* p = static_cast<uint8_t*>(const_cast<void*>(base));
  const size_t rows = size_t(g.B) * size_t(g.Hkv) * size_t(g.Tmax);
  return ValueStore{p, p + rows * kValueCodeRow,
                    reinterpret_cast<float*>(p + rows * (kValueCodeRow + kValueScaleRow))};
}

hipError_t launch_pack_block(const UnitGeom& g, const void* k, const float* center,
                             const float* gscale, int blk0, int blk1, uint8_t* codes,
                             uint8_t* scales, hipStream_t s);
hipError_t launch_pack_values(const UnitGeom& g, const void* v, const float* vscale, int blk0,
                              int blk1, void* store, hipStream_t s);
hipError_t launch_pack_proj(const UnitGeom& g, const void* k, const float* proj, int rank,
                            bool fp8, int blk0, int blk1, void* kproj, hipStream_t s);
hipError_t launch_append(const UnitGeom& g, int n_tail, int rank, bool fp8, const void* k_new,
                         const void* v_new, const int32_t* seq_lens, void* k, void* v,
                         const float* center, const float* gscale, uint8_t* codes,
                         uint8_t* scales, const float* proj, void* kproj, uint16_t* tail_k,
                         uint16_t* tail_v, hipStream_t s);
hipError_t launch_scan_block(const UnitGeom& g, int n_tail, float sigma, bool query_nvfp4,
                             const _Float16* q, const uint8_t* codes, const uint8_t* scales,
                             const float* gscale, const float* center, const int32_t* seq_lens,
                             float* scores, hipStream_t s);
// hist0 (optional): the token selection's workspace, whose per-unit
// histograms (hist_stride words apart) the scan fills as tok_hist would.
hipError_t launch_scan_token(const UnitGeom& g, float sigma, int rank, bool fp8,
                             const _Float16* q, const void* kproj, const float* proj,
                             const int32_t* seq_lens, float* scores, uint32_t* hist0,
                             int64_t hist_stride, int budget, hipStream_t s);
size_t token_select_workspace(const UnitGeom& g, int budget, float top_p);
int64_t token_unit_words(const UnitGeom& g);  // words per unit of that workspace
hipError_t launch_select_block(const UnitGeom& g, int budget, int n_tail, const float* scores,
                               const int32_t* seq_lens, int32_t* idx, int32_t* count,
                               hipStream_t s);
// hist_ready: the histograms were filled by launch_scan_token (tok_hist is skipped).
// top_p > 0: the selection is then cut to the adaptive budget (tok_topp);
// budget <= kTopPMaxBudget.
// Token select in one launch (tokselect.hip): its LDS bitmaps hold up to
// kTokSelectMaxTokens tokens, and its threshold sample is sized for budgets up
// to kTokSelectOneMaxBudget; longer rows and larger budgets take the chunked
// launches (select.hip). lse (the adaptive budget, else null): where it leaves
// the softmax partials tok_topp reads.
constexpr int kTokSelectMaxTokens = 131072;
constexpr int kTokSelectOneMaxBudget = 2048;
bool token_select_one_group(const UnitGeom& g, int budget, float top_p);
size_t token_select_one_workspace(const UnitGeom& g);  // its region, after the chunked one's
hipError_t launch_select_token_one(const UnitGeom& g, int budget, const float* scores,
                                   const int32_t* seq_lens, void* ws, int32_t* idx,
                                   int32_t* count, uint32_t* lse, int64_t lse_stride,
                                   hipStream_t s);
hipError_t launch_select_token(const UnitGeom& g, int budget, const float* scores,
                               const int32_t* seq_lens, void* ws, int32_t* idx, int32_t* count,
                               hipStream_t s, bool hist_ready = false, float top_p = 0.0f);
// Largest token budget the adaptive (top-p) budget sorts in one work-group's LDS.
constexpr int kTopPMaxBudget = 4096;
// The attention launch merges the splits in its last group up to this many
// (more, up to 32, measured slower than the separate merge launch).
constexpr int kFusedMergeMaxSplits = 8;

// Largest budget for which the attention launch selects the blocks itself.
constexpr int kFusedSelectMax = 1024;

// sel_scores (block mode, budget <= kFusedSelectMax, optional): the launch
// also selects each unit's blocks from these scores, as select_topk would,
// and writes the selection to sel_idx / sel_count; idx and count are unused.
hipError_t launch_attention(const UnitGeom& g, int granularity, int budget, int n_tail,
                            float sigma, const _Float16* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* idx, const int32_t* count,
                            const uint16_t* tail_k, const uint16_t* tail_v, int splits,
                            float* part_o, float* part_lse, uint32_t* counters, float* out,
                            float* out_lse, const float* sel_scores, int32_t* sel_idx,
                            int32_t* sel_count, hipStream_t s);
hipError_t launch_combine(int rows, int splits, const float* part_o, const float* part_lse,
                          float* out, float* out_lse, hipStream_t s);

// Coarse semantic blocks (BSA_GRANULARITY_CLUSTER): at most this many per unit.
constexpr int kMaxClusters = 4096;
hipError_t launch_cluster_index(const UnitGeom& g, int C, const void* k, const int32_t* assign,
                                const int32_t* seq_lens, float* centroids, int32_t* offsets,
                                int32_t* members, hipStream_t s);
// score: score the centroids (into scores_out when set); else read scores_in.
// select: write the chosen blocks' tokens to idx [units][budget] and count.
hipError_t launch_cluster_step(const UnitGeom& g, int C, int budget, float sigma, bool score,
                               bool select, const _Float16* q, const float* centroids,
                               const int32_t* offsets, const int32_t* members,
                               const float* scores_in, float* scores_out, int32_t* idx,
                               int32_t* count, hipStream_t s);


}  // namespace bsa
