// Block-mode dense scan of one wave, shared by the scan kernel and the
// decode-step kernel.
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

__device__ __forceinline__ half2v scale_pair(uint32_t byte) {
  const _Float16 s = _Float16(e4m3_to_float(byte));
  half2v r;
  r[0] = s;
  r[1] = s;
  return r;
}

template <bool COHERENT>
__device__ __forceinline__ void put_score(float* p, float v) {
  if (COHERENT) store_coherent(p, v);
  else *p = v;
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

// One block's code and scale words, as one wave holds them (lane l: the 16
// bytes of each 1 KiB code slice at offset 16 l, and of the scale record).
struct ScanRec {
  uint4v cw[8];
  uint4v sw;
};

__device__ __forceinline__ void scan_load(ScanRec& r, const ScanBlockArgs& a, int unit, int blk,
                                          int lane) {
  const uint8_t* crec = a.codes + (int64_t(unit) * a.NBmax + blk) * kCodeRecord;
  const uint8_t* srec = a.scales + (int64_t(unit) * a.NBmax + blk) * kScaleRecord;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r.cw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint4v*>(crec + i * 1024) + lane);
  r.sw = __builtin_nontemporal_load(reinterpret_cast<const uint4v*>(srec) + lane);
}

// The query side of one unit's scan, in the MFMA operand order.
struct ScanQuery {
  half8 qa[4];      // A operand: head row n = lane % 16 (zero beyond the group)
  float qc[4];      // q . c of the heads this output lane holds
  bool head_ok[4];
  float sc[4];      // s_t (times the head's query scale s_q for an NVFP4 query)
};

// NVFP4 query (Jet-QSparse abstract: FP4 operands on both sides of the scan's
// query-key products). Each head is quantized as the packer quantizes a key
// (no centering): per-head scale s_q = amax / 2688, per 16 channels the E4M3
// scale of amax_g / (6 s_q), elements E2M1(q / (e4m3 * s_q)); every step one
// correctly rounded float32 operation. The work-group does it once per item,
// 16 threads per head with 8 channels each, and leaves e2m1 * e4m3 (exact in
// f16) and s_q in LDS (ScanQueryLds); s_q multiplies the dot products instead.
// Every thread of the work-group calls it (it ends with a barrier).
__device__ __forceinline__ void stage_nvfp4_query(const ScanBlockArgs& a, int b, int h,
                                                  ScanQueryLds& ql) {
#pragma clang fp contract(off)
  const int t = threadIdx.x, head = t >> 4, chunk = t & 15;
  const bool ok = head < a.G;
  half8 v = half8{};
  if (ok) v = *reinterpret_cast<const half8*>(a.q + (int64_t(b) * a.Hq + h * a.G + head) * kHeadDim +
                                               8 * chunk);
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, __builtin_fabsf(float(v[e])));
  const float ag = fmaxf(am, __shfl_xor(am, 1, kWave));  // the 16-channel group
  float amax = ag;                                        // the head: 16 threads
#pragma unroll
  for (int off = 2; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const float s_q = amax / 2688.0f;
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
  __syncthreads();
}

// ql: the staged NVFP4 query (query_nvfp4), else null.
__device__ __forceinline__ void scan_query(ScanQuery& sq, const ScanBlockArgs& a, int b, int h,
                                           int lane, const ScanQueryLds* ql) {
  const int n = lane & 15, j = lane >> 4;
  const int G = a.G;
  // A operand: query head row n, channels 32 j + 8 c .. + 8
  float qc_part = 0.0f;
  const bool row_ok = n < G;
  const _Float16* qrow = a.q + (int64_t(b) * a.Hq + h * G + (row_ok ? n : 0)) * kHeadDim + 32 * j;
  half8 v[4];
  float s_q = 1.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[c] = ql ? ql->q[16 * (row_ok ? n : 0) + 4 * j + c] : *reinterpret_cast<const half8*>(qrow + 8 * c);
    if (!row_ok) v[c] = half8{};
  }
  if (ql) s_q = row_ok ? ql->s_q[n] : 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    sq.qa[c] = v[c];
    if (a.center) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qc_part += float(v[c][e]) * a.center[h * kHeadDim + 32 * j + 8 * c + e];
    }
  }
  // q . c of head row n: sum over the 4 channel quarters (lanes n, n+16, n+32, n+48)
  qc_part += __shfl_xor(qc_part, 16, kWave);
  qc_part += __shfl_xor(qc_part, 32, kWave);
  qc_part *= s_q;
  // output lane holds heads 4 j + r: fetch their q . c and s_q from lanes 4 j + r
  const float s_t = a.gscale[h];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sq.qc[r] = __shfl(qc_part, 4 * j + r, kWave);
    sq.sc[r] = s_t * __shfl(s_q, 4 * j + r, kWave);
    sq.head_ok[r] = 4 * j + r < G;
  }
}

// The score of one landed block with `valid` tokens (wave-uniform result).
__device__ __forceinline__ float scan_score(const ScanRec& r, const ScanQuery& sq, int valid,
                                            float sigma, int lane) {
  const int n = lane & 15;
  float m[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // scale bytes of (token 16 i + n, groups 2 j and 2 j + 1)
    const uint32_t word = r.sw[i >> 1] >> (16 * (i & 1));
    const half2v s0 = scale_pair(word & 0xFFu);
    const half2v s1 = scale_pair((word >> 8) & 0xFFu);
    float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[0], dequant8(r.cw[i][0], s0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[1], dequant8(r.cw[i][1], s0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[2], dequant8(r.cw[i][2], s1), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sq.qa[3], dequant8(r.cw[i][3], s1), acc, 0, 0, 0);
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
// item counts the unit's runs of kScanWaves * bpw blocks. COHERENT: the scores
// are stored as device-scope atomics (read by other work-groups of the same
// launch). PIPE: two blocks in flight (the next block's loads are issued
// before the current block is scored), for launches whose register budget
// allows it; the scores are the same either way.
//
// Every wave of the work-group calls it for the same unit (with query_nvfp4 the
// group stages the query together); ql: LDS for that query. Without PIPE the
// query format is the template argument Q4 (the FP16 form keeps its registers).
template <bool COHERENT, bool PIPE = false, bool Q4 = false>
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
  float* out = a.scores + int64_t(unit) * a.NBmax;
  // blocks past the packed pages (tail pages, beyond the sequence) score -inf
  const int sc_end = min(blk_end, max(packed, blk_begin));
  if (lane == 0)
    for (int blk = sc_end; blk < blk_end; ++blk) put_score<COHERENT>(out + blk, -__builtin_inff());
  auto valid_of = [&](int blk) { return min(kBlock, L - blk * kBlock); };

  const ScanQueryLds* qp = a.query_nvfp4 ? &ql : nullptr;
  // The first block's loads (the first two with PIPE) go out before the query
  // is formed, so the query's own latency overlaps them.
  if constexpr (PIPE) {
    ScanRec r0, r1;
    if (blk_begin < sc_end) scan_load(r0, a, unit, blk_begin, lane);
    if (blk_begin + 1 < sc_end) scan_load(r1, a, unit, blk_begin + 1, lane);
    if (qp) stage_nvfp4_query(a, b, h, ql);
    ScanQuery sq;
    scan_query(sq, a, b, h, lane, qp);
    for (int blk = blk_begin; blk < sc_end; blk += 2) {
      const float s0 = scan_score(r0, sq, valid_of(blk), a.sigma, lane);
      if (lane == 0) put_score<COHERENT>(out + blk, s0);
      if (blk + 2 < sc_end) scan_load(r0, a, unit, blk + 2, lane);
      if (blk + 1 >= sc_end) break;
      const float s1 = scan_score(r1, sq, valid_of(blk + 1), a.sigma, lane);
      if (lane == 0) put_score<COHERENT>(out + blk + 1, s1);
      if (blk + 3 < sc_end) scan_load(r1, a, unit, blk + 3, lane);
    }
  } else if constexpr (Q4) {
    ScanRec r;
    if (blk_begin < sc_end) scan_load(r, a, unit, blk_begin, lane);
    stage_nvfp4_query(a, b, h, ql);
    ScanQuery sq;
    scan_query(sq, a, b, h, lane, &ql);
    for (int blk = blk_begin; blk < sc_end; ++blk) {
      if (blk > blk_begin) scan_load(r, a, unit, blk, lane);
      const float s = scan_score(r, sq, valid_of(blk), a.sigma, lane);
      if (lane == 0) put_score<COHERENT>(out + blk, s);
    }
  } else {
    ScanQuery sq;
    scan_query(sq, a, b, h, lane, nullptr);
    for (int blk = blk_begin; blk < sc_end; ++blk) {
      ScanRec r;
      scan_load(r, a, unit, blk, lane);
      const float s = scan_score(r, sq, valid_of(blk), a.sigma, lane);
      if (lane == 0) put_score<COHERENT>(out + blk, s);
    }
  }
}

// Arguments and grid (runs of kScanWaves * bpw blocks, units) of one block scan.
ScanBlockArgs make_scan_args(const UnitGeom& g, int n_tail, float sigma, const _Float16* q,
                             const uint8_t* codes, const uint8_t* scales, const float* gscale,
                             const float* center, const int32_t* seq_lens, float* scores,
                             dim3& grid, int max_bpw = 4, bool query_nvfp4 = false) {
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
