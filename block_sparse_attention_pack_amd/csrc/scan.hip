// Dense scan kernels of one decode step (block and token mode).
//
// Token mode (JSSA Figure 1): qbar = mean of the group's query heads,
// p = P^T qbar in FP32 once per work-group, then each token's score is
// sigma * p . kproj_t, streamed in contiguous 1 KiB loads: 2R bytes per token
// from a BF16 cache, R from an FP8 one (JSSA Figure 10), whose E4M3 bytes the
// gfx950 convert widens exactly (scale 1).
#include "scan_core.hpp"
#include "select_core.hpp"

namespace bsa {
namespace {

// Blocks per wave of the block scan (fewer when the grid would not fill the GPU).
constexpr int kScanBlocksPerWave = 4;

// grid (ceil(NBmax / (kScanWaves * bpw)), B * Hkv), 256 threads. Q4: the
// NVFP4 query (a.query_nvfp4).
template <bool Q4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void scan_block_kernel(ScanBlockArgs a) {
  __shared__ ScanQueryLds ql;
  scan_wave_blocks<Q4>(a, threadIdx.x & 63, threadIdx.x >> 6, blockIdx.y, blockIdx.x, ql);
}

// Token mode. grid (ceil(Tmax / kTokPerWg), B * Hkv), 256 threads; each wave
// scores kTokPerWg / 4 consecutive tokens, 64 per step. A token's projected row
// (2R bytes in BF16, R in FP8) is a run of 16-byte pieces, and a step's 64 rows
// are contiguous 1 KiB slices: lane l loads piece l % P of token l / P of each
// slice (P pieces per row), so every load instruction reads one contiguous
// KiB. A lane forms the dot product of its piece with the matching entries of
// p (8 in BF16, 16 in FP8), the P lanes of a token add theirs, and one
// exchange per slice moves token t's score to lane t. The scores collect in LDS and leave after the
// work-group's last read, in contiguous 16-byte-per-lane non-temporal stores:
// stores spread among the reads cost the HBM far more than their own bytes (23
// us of 120 at 128K context, batch 8, 8 KV heads). The next step's rows are
// loaded before the current ones are scored, and the first step's before p is
// formed. Each wave starts its run of steps at its own offset and wraps around,
// so the waves' concurrent reads are not all a power-of-two distance apart;
// with the non-temporal score stores this made the scan 4% (BF16) and 9% (FP8)
// faster at 128K context, batch 8, 8 KV heads.
constexpr int kTokPerWg = 16384;
constexpr int kTokThreads = 256;  // threads of a token-scan work-group
constexpr int kTokWaves = kTokThreads / kWave;
constexpr int kTokStagger = 13;  // steps between the starting points of consecutive waves

//
// With hist0 set, the work-group also counts its candidates' first select
// digits (the top 12 key bits of scores of tokens < L) as the token
// selection's tok_hist does: 16-bit counters, two per LDS word, filled while
// the scores are stored, then added to the unit's histogram at hist0 + unit *
// hist_stride. Units where the selection takes nothing or everything (picks 0
// or L) are not counted, as there.
template <int R, bool FP8>
__global__ __launch_bounds__(kTokThreads) void scan_token_kernel(
    const _Float16* __restrict__ q, const void* __restrict__ kproj,
    const float* __restrict__ proj, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int Hkv, int Hq, int G, int Tmax, float sigma,
    uint32_t* __restrict__ hist0, int64_t hist_stride, int budget) {
  constexpr int kRowBytes = FP8 ? R : 2 * R;
  constexpr int kPer = FP8 ? 16 : 8;      // entries of a row per 16-byte piece
  static_assert(kRowBytes % 16 == 0 && kRowBytes <= 256, "rank");
  constexpr int kLpt = kRowBytes / 16;    // lanes per token (one 16-byte piece each)
  constexpr int kTps = kWave / kLpt;  // tokens per 1 KiB slice
  constexpr int kSlices = kLpt;       // slices per 64-token step
  constexpr int kPerWave = kTokPerWg / kTokWaves;
  __shared__ float qbar[kHeadDim];
  __shared__ float part[kTokThreads];
  __shared__ float p_lds[R];
  __shared__ __attribute__((aligned(16))) float keep[kTokWaves][kPerWave];  // the scores, until the end
  __shared__ uint32_t h16[kTokHistBins / 2];  // bin d at half d & 1 of word d / 2
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.y;
  const int b = unit / Hkv, h = unit % Hkv;
  const int L = clamp_len(seq_lens[b], Tmax);
  const int picks = min(budget, L);
  const bool do_hist = hist0 != nullptr && picks > 0 && picks < L;  // uniform
  if (do_hist)
    for (int w = threadIdx.x; w < kTokHistBins / 2; w += kTokThreads) h16[w] = 0u;  // before the barriers below
  const int t_wave = blockIdx.x * kTokPerWg + wave * kPerWave;
  const int t_end = min(t_wave + kPerWave, Tmax);
  const uint8_t* base = static_cast<const uint8_t*>(kproj) + int64_t(unit) * Tmax * kRowBytes;
  float* out = scores + int64_t(unit) * Tmax;
  const int piece = lane % kLpt, tok_in_slice = lane / kLpt;

  // the 16-byte pieces this lane holds of the step at t0 (rows past t_end,
  // only possible in a partial last step, read row t0 instead and are dropped);
  // each load instruction takes whole 128-byte lines, read once: streaming
  // (non-temporal) loads, which measured about 10% faster than plain ones
  auto load_step = [&](uint4v (&w)[kSlices], int t0) {
#pragma unroll
    for (int c = 0; c < kSlices; ++c) {
      const int t = t0 + c * kTps + tok_in_slice;
      w[c] = __builtin_nontemporal_load(
          reinterpret_cast<const uint4v*>(base + int64_t(t < t_end ? t : t0) * kRowBytes) + piece);
    }
  };
  // the first step's rows are in flight while p is formed
  uint4v wa[kSlices], wb[kSlices];
  const int nsteps = t_end > t_wave ? (t_end - t_wave + kWave - 1) / kWave : 0;
  const int k0 =
      nsteps > 0
          ? int(((int64_t(blockIdx.y) * gridDim.x + blockIdx.x) * kTokWaves + wave) * kTokStagger %
                nsteps)
          : 0;
  auto step_t = [&](int i) {  // first token of the wave's i-th step
    int k = k0 + i;
    if (k >= nsteps) k -= nsteps;
    return t_wave + k * kWave;
  };
  if (nsteps > 0) load_step(wa, step_t(0));

  // qbar = (sum of the group's queries) / G, then p = sigma * P^T qbar, in
  // float32. The thread's entries of P are loaded with the queries, before
  // the first barrier.
  constexpr int kChunks = kTokThreads / R;  // threads per output channel
  constexpr int kDPer = kHeadDim / kChunks;
  const int jj = threadIdx.x % R, ch = threadIdx.x / R;
  float pv[kDPer];
  {
    const float* pc = proj + (int64_t(h) * kHeadDim + ch * kDPer) * R + jj;
#pragma unroll
    for (int i = 0; i < kDPer; ++i) pv[i] = pc[int64_t(i) * R];
  }
  if (threadIdx.x < kHeadDim) {
    const _Float16* qd = q + (int64_t(b) * Hq + h * G) * kHeadDim + threadIdx.x;
    float qs = 0.0f;
    for (int g = 0; g < G; ++g) qs += float(qd[int64_t(g) * kHeadDim]);
    qbar[threadIdx.x] = qs * (1.0f / float(G));
  }
  __syncthreads();
  {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kDPer; ++i) acc += pv[i] * qbar[ch * kDPer + i];
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < R) {
      float sum = 0.0f;
      for (int c = 0; c < kChunks; ++c) sum += part[c * R + threadIdx.x];
      p_lds[threadIdx.x] = sum * sigma;
    }
    __syncthreads();
  }
  float pq[kPer];  // the entries of p that meet this lane's piece
#pragma unroll
  for (int e = 0; e < kPer; ++e) pq[e] = p_lds[kPer * piece + e];

  // the 64 scores of the step at t0 from its landed pieces, stored by lane t
  auto score_step = [&](const uint4v (&w)[kSlices], int t0) {
    float mine = 0.0f;
#pragma unroll
    for (int c = 0; c < kSlices; ++c) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (FP8) {
          // bytes 0, 1 and 2, 3 of the dword are entries 4 e .. 4 e + 3
          const float2v lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[c][e], 1.0f, false);
          const float2v hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[c][e], 1.0f, true);
          s = __builtin_fmaf(pq[4 * e], lo[0], s);
          s = __builtin_fmaf(pq[4 * e + 1], lo[1], s);
          s = __builtin_fmaf(pq[4 * e + 2], hi[0], s);
          s = __builtin_fmaf(pq[4 * e + 3], hi[1], s);
        } else {
          s = __builtin_fmaf(pq[2 * e], bf16_bits_to_float(w[c][e] & 0xFFFFu), s);
          s = __builtin_fmaf(pq[2 * e + 1], bf16_bits_to_float(w[c][e] >> 16), s);
        }
      }
#pragma unroll
      for (int off = 1; off < kLpt; off <<= 1) s += __shfl_xor(s, off, kWave);
      // token c * kTps + k is complete in lane k * kLpt
      const float v = __shfl(s, (lane % kTps) * kLpt, kWave);
      if (lane / kTps == c) mine = v;
    }
    const int t = t0 + lane;
    if (t < t_end) keep[wave][t - t_wave] = t < L ? mine : -__builtin_inff();
  };
  // the next step's rows are in flight while a step is scored (a deeper
  // pipeline measured slower)
  for (int i = 0; i < nsteps; i += 2) {
    if (i + 1 < nsteps) load_step(wb, step_t(i + 1));
    score_step(wa, step_t(i));
    if (i + 1 >= nsteps) break;
    if (i + 2 < nsteps) load_step(wa, step_t(i + 2));
    score_step(wb, step_t(i + 1));
  }
  // the wave's scores, 1 KiB per store instruction (its own LDS rows: no barrier)
  wave_lds_sync();
  const int n = t_end > t_wave ? t_end - t_wave : 0;
  auto count_key = [&](float sc, int t) {
    if (t < L) {
      const uint32_t d = score_key(sc) >> kTokHistShift;
      atomicAdd(&h16[d >> 1], (d & 1u) ? 0x10000u : 1u);  // a count stays below 2^16
    }
  };
  for (int i = 4 * lane; i < n; i += 4 * kWave) {
    if (i + 4 <= n) {
      const float4v x = *reinterpret_cast<const float4v*>(&keep[wave][i]);
      __builtin_nontemporal_store(x, reinterpret_cast<float4v*>(out + t_wave + i));
      if (do_hist) {
#pragma unroll
        for (int k = 0; k < 4; ++k) count_key(x[k], t_wave + i + k);
      }
    } else {
      for (int k = i; k < n; ++k) {
        out[t_wave + k] = keep[wave][k];
        if (do_hist) count_key(keep[wave][k], t_wave + k);
      }
    }
  }
  if (do_hist) {
    __syncthreads();
    uint32_t* hist = hist0 + int64_t(unit) * hist_stride;
    for (int w = threadIdx.x; w < kTokHistBins / 2; w += kTokThreads) {
      const uint32_t x = h16[w];
      if (x & 0xFFFFu)
        __hip_atomic_fetch_add(&hist[2 * w], x & 0xFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (x >> 16)
        __hip_atomic_fetch_add(&hist[2 * w + 1], x >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_scan_block(const UnitGeom& g, int n_tail, float sigma, bool query_nvfp4,
                             const _Float16* q, const uint8_t* codes, const uint8_t* scales,
                             const float* gscale, const float* center, const int32_t* seq_lens,
                             float* scores, hipStream_t s) {
  dim3 grid;
  const ScanBlockArgs a = make_scan_args(g, n_tail, sigma, q, codes, scales, gscale, center,
                                         seq_lens, scores, grid, kScanBlocksPerWave, query_nvfp4);
  if (query_nvfp4) hipLaunchKernelGGL(scan_block_kernel<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(scan_block_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan_token(const UnitGeom& g, float sigma, int rank, bool fp8,
                             const _Float16* q, const void* kproj, const float* proj,
                             const int32_t* seq_lens, float* scores, uint32_t* hist0,
                             int64_t hist_stride, int budget, hipStream_t s) {
  dim3 grid(ceil_div(g.Tmax, kTokPerWg), g.B * g.Hkv);
#define BSA_SCAN_TOKEN(RK, F8)                                                                  \
  hipLaunchKernelGGL((scan_token_kernel<RK, F8>), grid, dim3(kTokThreads), 0, s, q, kproj, proj, \
                     seq_lens, scores, g.Hkv, g.Hq, g.G, g.Tmax, sigma, hist0, hist_stride, budget)
  if (fp8) {
    switch (rank) {
      case 16: BSA_SCAN_TOKEN(16, true); break;
      case 32: BSA_SCAN_TOKEN(32, true); break;
      case 64: BSA_SCAN_TOKEN(64, true); break;
      case 128: BSA_SCAN_TOKEN(128, true); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (rank) {
      case 8: BSA_SCAN_TOKEN(8, false); break;
      case 16: BSA_SCAN_TOKEN(16, false); break;
      case 32: BSA_SCAN_TOKEN(32, false); break;
      case 64: BSA_SCAN_TOKEN(64, false); break;
      case 128: BSA_SCAN_TOKEN(128, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef BSA_SCAN_TOKEN
  return hipGetLastError();
}

}  // namespace bsa
