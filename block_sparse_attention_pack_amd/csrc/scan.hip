// Dense scan of one decode step over the whole key history.
//
// Block mode (Jet-QSparse abstract: every step scores all cached keys from the
// NVFP4 copy and selects 128-token blocks): per (unit, block) the score is the
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
//
// Token mode (JSSA Figure 1): qbar = mean of the group's query heads,
// p = P^T qbar in FP32 once per work-group, then each token's score is
// sigma * p . kproj_t, streamed 64 B per token with 16-byte loads.
#include "common.hpp"
#include "select_core.hpp"

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

struct ScanBlockArgs {
  const _Float16* q;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  const float* center;
  const int32_t* seq_lens;
  float* scores;
  int Hkv, Hq, G, NBmax, Tmax, n_tail, bpw;
  float sigma;
};

// The scan of one wave: blocks [blk_begin, blk_begin + bpw) of unit blockIdx.y.
__device__ __forceinline__ void scan_wave_blocks(const ScanBlockArgs& a, int lane, int wave) {
  const int unit = blockIdx.y;
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  const int L = clamp_len(a.seq_lens[b], a.Tmax);
  const int npages = ceil_div(L, kBlock);
  const int packed = npages - a.n_tail > 0 ? npages - a.n_tail : 0;
  const int blk_begin = (blockIdx.x * kScanWaves + wave) * a.bpw;
  if (blk_begin >= a.NBmax) return;
  const int blk_end = min(blk_begin + a.bpw, a.NBmax);
  const int G = a.G;
  float* out = a.scores + int64_t(unit) * a.NBmax;

  const int n = lane & 15, j = lane >> 4;
  // A operand: query head row n (zero beyond the group), channels 32 j + 8 c .. + 8
  half8 qa[4];
  float qc_part = 0.0f;
  const bool row_ok = n < G;
  const _Float16* qrow = a.q + (int64_t(b) * a.Hq + h * G + (row_ok ? n : 0)) * kHeadDim + 32 * j;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    half8 v = *reinterpret_cast<const half8*>(qrow + 8 * c);
    if (!row_ok) v = half8{};
    qa[c] = v;
    if (a.center) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qc_part += float(v[e]) * a.center[h * kHeadDim + 32 * j + 8 * c + e];
    }
  }
  // q . c of head row n: sum over the 4 channel quarters (lanes n, n+16, n+32, n+48)
  qc_part += __shfl_xor(qc_part, 16, kWave);
  qc_part += __shfl_xor(qc_part, 32, kWave);
  // output lane holds heads 4 j + r: fetch their q . c from lanes 4 j + r
  float qc[4];
  bool head_ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    qc[r] = __shfl(qc_part, 4 * j + r, kWave);
    head_ok[r] = 4 * j + r < G;
  }
  const float s_t = a.gscale[h];

  for (int blk = blk_begin; blk < blk_end; ++blk) {
    if (blk >= packed) {
      if (lane == 0) out[blk] = -__builtin_inff();
      continue;
    }
    const uint8_t* crec = a.codes + (int64_t(unit) * a.NBmax + blk) * kCodeRecord;
    const uint8_t* srec = a.scales + (int64_t(unit) * a.NBmax + blk) * kScaleRecord;
    uint4v cw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      cw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint4v*>(crec + i * 1024) + lane);
    const uint4v sw = __builtin_nontemporal_load(reinterpret_cast<const uint4v*>(srec) + lane);
    const int valid = min(kBlock, L - blk * kBlock);

    float m[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // scale bytes of (token 16 i + n, groups 2 j and 2 j + 1)
      const uint32_t word = sw[i >> 1] >> (16 * (i & 1));
      const half2v s0 = scale_pair(word & 0xFFu);
      const half2v s1 = scale_pair((word >> 8) & 0xFFu);
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[0], dequant8(cw[i][0], s0), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[1], dequant8(cw[i][1], s0), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[2], dequant8(cw[i][2], s1), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[3], dequant8(cw[i][3], s1), acc, 0, 0, 0);
      const bool tok_ok = 16 * i + n < valid;
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = fmaxf(m[r], tok_ok ? acc[r] : -__builtin_inff());
    }
    float best = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (head_ok[r]) best = fmaxf(best, s_t * m[r] + qc[r]);
    best = wave_max_uniform(best);
    if (lane == 0) out[blk] = a.sigma * best;
  }
}

// grid (ceil(NBmax / (kScanWaves * bpw)), B * Hkv), 256 threads.
__global__ __launch_bounds__(256) void scan_block_kernel(ScanBlockArgs a) {
  scan_wave_blocks(a, threadIdx.x & 63, threadIdx.x >> 6);
}

// Token mode. grid (ceil(Tmax / kTokPerWg), B * Hkv), 256 threads; each wave
// scores kTokPerWg / 4 consecutive tokens, one token per lane and step: a lane
// reads its token's whole projected row (R bf16 = R / 8 16-byte loads; together
// the wave's loads cover 64 consecutive rows, whole cache lines) and forms the
// dot product with p in its own registers, so the 64 scores of a step leave in
// one coalesced store.
constexpr int kTokPerWg = 16384;

template <int R>
__global__ __launch_bounds__(256) void scan_token_kernel(
    const _Float16* __restrict__ q, const uint16_t* __restrict__ kproj,
    const float* __restrict__ proj, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int Hkv, int Hq, int G, int Tmax, float sigma) {
  static_assert(R % 8 == 0 && R <= 128, "rank");
  constexpr int kVec = R / 8;               // 16-byte loads per token row
  constexpr bool kPinReg = R <= 32;         // p in registers (else read from LDS)
  constexpr int kUnroll = 1;                // tokens per lane in flight
  __shared__ float qbar[kHeadDim];
  __shared__ float part[256];
  __shared__ float p_lds[R];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.y;
  const int b = unit / Hkv, h = unit % Hkv;
  const int L = clamp_len(seq_lens[b], Tmax);

  // qbar = (sum of the group's queries) / G, then p = sigma * P^T qbar, in
  // float32; every thread issues all its loads of a stage before using them.
  if (threadIdx.x < kHeadDim) {
    const _Float16* qd = q + (int64_t(b) * Hq + h * G) * kHeadDim + threadIdx.x;
    float qs = 0.0f;
    for (int g = 0; g < G; ++g) qs += float(qd[int64_t(g) * kHeadDim]);
    qbar[threadIdx.x] = qs * (1.0f / float(G));
  }
  __syncthreads();
  {
    constexpr int kChunks = 256 / R;  // threads per output channel
    constexpr int kDPer = kHeadDim / kChunks;
    const int jj = threadIdx.x % R, ch = threadIdx.x / R;
    constexpr int kBatch = kDPer < 16 ? kDPer : 16;
    const float* pc = proj + (int64_t(h) * kHeadDim + ch * kDPer) * R + jj;
    float acc = 0.0f;
    for (int i0 = 0; i0 < kDPer; i0 += kBatch) {
      float pv[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) pv[i] = pc[int64_t(i0 + i) * R];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) acc += pv[i] * qbar[ch * kDPer + i0 + i];
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < R) {
      float sum = 0.0f;
      for (int c = 0; c < kChunks; ++c) sum += part[c * R + threadIdx.x];
      p_lds[threadIdx.x] = sum * sigma;
    }
    __syncthreads();
  }
  float p[kPinReg ? R : 1];
  if constexpr (kPinReg) {
#pragma unroll
    for (int j = 0; j < R; ++j) p[j] = p_lds[j];
  }

  const int t_wave = blockIdx.x * kTokPerWg + wave * (kTokPerWg / 4);
  const uint16_t* base = kproj + int64_t(unit) * Tmax * R;
  float* out = scores + int64_t(unit) * Tmax;
  const int t_end = min(t_wave + kTokPerWg / 4, Tmax);
  for (int t0 = t_wave; t0 < t_end; t0 += kUnroll * kWave) {
    uint4v w[kUnroll][kVec];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * kWave + lane;
      const uint4v* row = reinterpret_cast<const uint4v*>(base + int64_t(t < t_end ? t : t_wave) * R);
#pragma unroll
      for (int c = 0; c < kVec; ++c) w[u][c] = row[c];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * kWave + lane;
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < kVec; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 8 * c + 2 * e;
          const float p0 = kPinReg ? p[kPinReg ? j : 0] : p_lds[j];
          const float p1 = kPinReg ? p[kPinReg ? j + 1 : 0] : p_lds[j + 1];
          s = __builtin_fmaf(p0, bf16_bits_to_float(w[u][c][e] & 0xFFFFu), s);
          s = __builtin_fmaf(p1, bf16_bits_to_float(w[u][c][e] >> 16), s);
        }
      }
      if (t < t_end) out[t] = t < L ? s : -__builtin_inff();
    }
  }
}

}  // namespace

namespace {
ScanBlockArgs make_scan_args(const UnitGeom& g, int n_tail, float sigma, const _Float16* q,
                             const uint8_t* codes, const uint8_t* scales, const float* gscale,
                             const float* center, const int32_t* seq_lens, float* scores,
                             dim3& grid) {
  const int units = g.B * g.Hkv;
  // enough work-groups to fill 256 CUs several times over
  int bpw = 4;
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
  a.sigma = sigma;
  return a;
}
}  // namespace

hipError_t launch_scan_block(const UnitGeom& g, int n_tail, float sigma, const _Float16* q,
                             const uint8_t* codes, const uint8_t* scales, const float* gscale,
                             const float* center, const int32_t* seq_lens, float* scores,
                             hipStream_t s) {
  dim3 grid;
  const ScanBlockArgs a =
      make_scan_args(g, n_tail, sigma, q, codes, scales, gscale, center, seq_lens, scores, grid);
  hipLaunchKernelGGL(scan_block_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan_token(const UnitGeom& g, float sigma, int rank, const _Float16* q,
                             const uint16_t* kproj, const float* proj, const int32_t* seq_lens,
                             float* scores, hipStream_t s) {
  dim3 grid(ceil_div(g.Tmax, kTokPerWg), g.B * g.Hkv);
#define BSA_SCAN_TOKEN(RK)                                                                     \
  case RK:                                                                                     \
    hipLaunchKernelGGL(scan_token_kernel<RK>, grid, dim3(256), 0, s, q, kproj, proj, seq_lens, \
                       scores, g.Hkv, g.Hq, g.G, g.Tmax, sigma);                               \
    break;
  switch (rank) {
    BSA_SCAN_TOKEN(8)
    BSA_SCAN_TOKEN(16)
    BSA_SCAN_TOKEN(32)
    BSA_SCAN_TOKEN(64)
    BSA_SCAN_TOKEN(128)
    default:
      return hipErrorInvalidValue;
  }
#undef BSA_SCAN_TOKEN
  return hipGetLastError();
}

}  // namespace bsa
