// Dense scan kernels of one decode step (block and token mode).
//
// Token mode (JSSA Figure 1): qbar = mean of the group's query heads,
// p = P^T qbar in FP32 once per work-group, then each token's score is
// sigma * p . kproj_t, streamed 64 B per token with 16-byte loads.
#include "scan_core.hpp"
#include "select_core.hpp"

namespace bsa {
namespace {

// grid (ceil(NBmax / (kScanWaves * bpw)), B * Hkv), 256 threads.
__global__ __launch_bounds__(256) void scan_block_kernel(ScanBlockArgs a) {
  scan_wave_blocks<false>(a, threadIdx.x & 63, threadIdx.x >> 6, blockIdx.y, blockIdx.x);
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
