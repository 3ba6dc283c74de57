// Block-mode dense scan of one wave.
//
// Jet-QSparse abstract: every step scores all cached keys from the NVFP4 copy
// and selects 128-token blocks. Per (unit, block) the score is the
// largest estimated logit over the KV head's query heads and the block's valid
// tokens, sigma * (s_t * q . dequant(k) + q . c).
//
// gfx950 mapping. One wave scores one 128-token block as 8 steps of 16 tokens.
// In a step, lane l (n = l % 16, j = l / 16) holds token 16 i + n, channels
// 32 j .. 32 j + 31: one contiguous 16-byte load per lane, the packed layout
// puts the wave's 1 KiB in exactly that order. Each of the lane's 4 dwords is
// 8 E2M1 codes -> 4 x v_cvt_scalef32_pk_f16_fp4 (the hardware convert honours
// only the exponent of its scale, so it runs with scale 1 and the E4M3 group
// scale is applied by a packed f16 multiply: e2m1 * e4m3 has at most 6
// significant bits and lies in [2^-10, 2688], exact in f16). The dequantized
// dword is the B operand of one v_mfma_f32_16x16x32_f16 whose A operand holds
// the group's query heads (rows >= G are zero), so the matrix core forms the
// exact products and sums them in FP32. The output lane l holds heads
// 4 (l/16) + r of token n; the block maximum is a running VALU max followed by
// one 64-lane reduction.
#pragma once

#include "common.hpp"

namespace bsa {
namespace {

constexpr int kScanWaves = 4;

__device__ __forceinline__ half8 dequant8(uint32_t codes, half2v scale) {
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * scale;
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * scale;
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * scale;
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * scale;
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// The E4M3 scales of groups 2 j and 2 j + 1 of one token (bytes 2 hi, 2 hi + 1
// of word) as f16, by the hardware FP8 convert at scale 1 (every E4M3 value is
// exact in f16).
template <bool HI>
__device__ __forceinline__ half2v scale_halves(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, HI);
}

struct ScanBlockArgs {
  const _Float16* q;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  const float* center;
  const int32_t* seq_lens;
  float* scores;
  int Hkv, Hq, G, NBmax, Tmax, n_tail, bpw;
  int query_nvfp4;  // score with the NVFP4-quantized query (BSA_QUERY_NVFP4)
  float sigma;
};

// One block's code words, as one wave holds them (lane l: the 16 bytes of each
// 1 KiB code slice at offset 16 l); its scale words (lane l: 16 bytes of the
// scale record) are held apart.
struct ScanRec {
  uint4v cw[8];
};

__device__ __forceinline__ const uint4v* code_words(const ScanBlockArgs& a, int unit, int blk) {
  return reinterpret_cast<const uint4v*>(a.codes + (int64_t(unit) * a.NBmax + blk) * kCodeRecord);
}
__device__ __forceinline__ const uint4v* scale_words(const ScanBlockArgs& a, int unit, int blk) {
  return reinterpret_cast<const uint4v*>(a.scales + (int64_t(unit) * a.NBmax + blk) * kScaleRecord);
}

// The query side of one unit's scan, in the MFMA operand order.
struct ScanQuery {
  half8 qa[4];      // A operand: head row n = lane % 16 (zero beyond the group)
  float qc[4];      // q . c of the heads this output lane holds
  bool head_ok[4];
  float sc[4];      // s_t (times the head's query scale s_q for an NVFP4 query)
};

// The query side of one unit's scan, staged once per work-group (every thread
// calls it; it ends with a barrier): 16 threads per head, 8 channels each.
//
// Q4, the NVFP4 query (Jet-QSparse abstract: FP4 operands on both sides of the
// scan's query-key products): each head is quantized as the packer quantizes a
// key (no centering): per-head scale s_q = amax / 2688, per 16 channels the
// E4M3 scale of amax_g / (6 s_q), elements E2M1(q / (e4m3 * s_q)); every step
// one correctly rounded float32 operation. e2m1 * e4m3 (exact in f16) and s_q
// go to LDS; s_q multiplies the dot products instead.
//
// For either query the head's q . c (the centering term of the estimated
// logit, times s_q) goes to LDS too, so no wave holds the center vector.
template <bool Q4>
__device__ __forceinline__ void stage_query(const ScanBlockArgs& a, int b, int h,
                                            ScanQueryLds& ql) {
  const int t = threadIdx.x, head = t >> 4, chunk = t & 15;
  const bool ok = head < a.G;
  half8 v = half8{};
  if (ok) v = *reinterpret_cast<const half8*>(a.q + (int64_t(b) * a.Hq + h * a.G + head) * kHeadDim +
                                               8 * chunk);
  float s_q = 1.0f;
  if constexpr (Q4) {
#pragma clang fp contract(off)
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, __builtin_fabsf(float(v[e])));
    const float ag = fmaxf(am, __shfl_xor(am, 1, kWave));  // the 16-channel group
    float amax = ag;                                        // the head: 16 threads
#pragma unroll
    for (int off = 2; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    s_q = amax / 2688.0f;
    const uint32_t sb = e4m3_from_float(ag / (6.0f * s_q));  // 0 for a head of zeros
    const float e4 = e4m3_to_float(sb);
    const float S = e4 * s_q;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t code = S > 0.0f ? e2m1_from_float(float(v[e]) / S) : 0u;
      v[e] = _Float16(e2m1_to_float(code) * e4);
    }
    if (ok) {
      ql.q[t] = v;
      if (chunk == 0) ql.s_q[head] = s_q;
    }
  }
  float part = 0.0f;
  if (a.center && ok) {
    const float4v* cp = reinterpret_cast<const float4v*>(a.center + h * kHeadDim + 8 * chunk);
    const float4v c0 = cp[0], c1 = cp[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) part += float(v[e]) * c0[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) part += float(v[4 + e]) * c1[e];
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) part += __shfl_xor(part, off, kWave);
  if (ok && chunk == 0) ql.qc[head] = part * s_q;
  __syncthreads();
}

// The A operands (query head row n = lane % 16, channels 32 j + 8 c .. + 8) and
// per-output-lane factors, from the staged query side.
template <bool Q4>
__device__ __forceinline__ void scan_query(ScanQuery& sq, const ScanBlockArgs& a, int b, int h,
                                           int lane, const ScanQueryLds& ql) {
  const int n = lane & 15, j = lane >> 4;
  const int G = a.G;
  const bool row_ok = n < G;
  const _Float16* qrow = a.q + (int64_t(b) * a.Hq + h * G + (row_ok ? n : 0)) * kHeadDim + 32 * j;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    half8 v = Q4 ? ql.q[16 * (row_ok ? n : 0) + 4 * j + c]
                 : *reinterpret_cast<const half8*>(qrow + 8 * c);
    sq.qa[c] = row_ok ? v : half8{};
  }
  // output lane holds heads 4 j + r
  const float s_t = a.gscale[h];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * j + r;
    const bool ok = hh < G;
    sq.head_ok[r] = ok;
    sq.qc[r] = ok ? ql.qc[hh] : 0.0f;
    sq.sc[r] = s_t * (Q4 ? (ok ? ql.s_q[hh] : 0.0f) : 1.0f);
  }
}

// The score of one landed block with `valid` tokens (wave-uniform result):
// codes in r, scales in sw.
__device__ __forceinline__ float scan_score(const ScanRec& r, const uint4v& sw, const ScanQuery& sq,
                                            int valid, float sigma, int lane) {
  const int n = lane & 15;
  float m[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // scale bytes of (token 16 i + n, groups 2 j and 2 j + 1)
    const half2v sc = (i & 1) ? scale_halves<true>(sw[i >> 1]) : scale_halves<false>(sw[i >> 1]);
    const half2v s0 = {sc[0], sc[0]}, s1 = {sc[1], sc[1]};
    const half8 h0 = dequant8(r.cw[i][0], s0), h1 = dequant8(r.cw[i][1], s0);
    const half8 h2 = dequant8(r.cw[i][2], s1), h3 = dequant8(r.cw[i][3], s1);
    float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[0], h0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[1], h1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[2], h2, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[3], h3, acc, 0, 0, 0);
    const bool tok_ok = 16 * i + n < valid;
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = fmaxf(m[q], tok_ok ? acc[q] : -__builtin_inff());
  }
  float best = -__builtin_inff();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (sq.head_ok[q]) best = fmaxf(best, sq.sc[q] * m[q] + sq.qc[q]);
  return sigma * wave_max_uniform(best);
}

// The scan of one wave: blocks [blk_begin, blk_begin + bpw) of `unit`, where
// item counts the unit's runs of kScanWaves * bpw blocks, one block's loads in
// flight at a time (five waves per SIMD hide the latency; prefetching the next
// block needs registers that cost that occupancy and measured no faster). The
// scores are stored at the end, one per lane.
//
// Every wave of the work-group calls it for the same unit (the group stages the
// query side together in ql).
template <bool Q4>
__device__ __forceinline__ void scan_wave_blocks(const ScanBlockArgs& a, int lane, int wave,
                                                 int unit, int item, ScanQueryLds& ql) {
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  const int L = clamp_len(a.seq_lens[b], a.Tmax);
  const int npages = ceil_div(L, kBlock);
  const int packed = npages - a.n_tail > 0 ? npages - a.n_tail : 0;
  // a wave past the last block has nothing to load or score, but still takes
  // part in the query stage
  const int blk_begin = (item * kScanWaves + wave) * a.bpw;
  const int blk_end = min(blk_begin + a.bpw, a.NBmax);
  // blocks past the packed pages (tail pages, beyond the sequence) score -inf
  const int sc_end = min(blk_end, max(packed, blk_begin));
  auto valid_of = [&](int blk) { return min(kBlock, L - blk * kBlock); };

  stage_query<Q4>(a, b, h, ql);
  ScanQuery sq;
  scan_query<Q4>(sq, a, b, h, lane, ql);

  float mine = -__builtin_inff();  // lane k: the score of block blk_begin + k
  auto keep = [&](int blk, float s) {
    if (lane == blk - blk_begin) mine = s;
  };
  for (int blk = blk_begin; blk < sc_end; ++blk) {
    ScanRec r;
    const uint4v sw = __builtin_nontemporal_load(scale_words(a, unit, blk) + lane);
    const uint4v* cb = code_words(a, unit, blk);
#pragma unroll
    for (int i = 0; i < 8; ++i) r.cw[i] = __builtin_nontemporal_load(cb + i * 64 + lane);
    keep(blk, scan_score(r, sw, sq, valid_of(blk), a.sigma, lane));
  }
  if (lane < blk_end - blk_begin) {
    float* p = a.scores + int64_t(unit) * a.NBmax + blk_begin + lane;
    *p = blk_begin + lane < sc_end ? mine : -__builtin_inff();
  }
}

// Arguments and grid (runs of kScanWaves * bpw blocks, units) of one block scan.
ScanBlockArgs make_scan_args(const UnitGeom& g, int n_tail, float sigma, const _Float16* q,
                             const uint8_t* codes, const uint8_t* scales, const float* gscale,
                             const float* center, const int32_t* seq_lens, float* scores,
                             dim3& grid, int max_bpw, bool query_nvfp4) {
  const int units = g.B * g.Hkv;
  // enough work-groups to fill 256 CUs several times over
  int bpw = max_bpw;
  while (bpw > 1 && int64_t(units) * ceil_div(g.NBmax, kScanWaves * bpw) < 2048) bpw >>= 1;
  grid = dim3(ceil_div(g.NBmax, kScanWaves * bpw), units);
  ScanBlockArgs a;
  a.q = q;
  a.codes = codes;
  a.scales = scales;
  a.gscale = gscale;
  a.center = center;
  a.seq_lens = seq_lens;
  a.scores = scores;
  a.Hkv = g.Hkv;
  a.Hq = g.Hq;
  a.G = g.G;
  a.NBmax = g.NBmax;
  a.Tmax = g.Tmax;
  a.n_tail = n_tail;
  a.bpw = bpw;
  a.query_nvfp4 = query_nvfp4 ? 1 : 0;
  a.sigma = sigma;
  return a;
}

}  // namespace
}  // namespace bsa
