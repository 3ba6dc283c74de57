// Coarse semantic blocks scored by their centroids (Coarse Semantic Blocks
// abstract: keys clustered into large blocks of noncontiguous tokens, each
// query picks blocks by scoring their centroids and attends the original keys
// and values of the picked blocks).
//
// Index (built once, off the decode step): from a token -> block assignment,
// the blocks' token lists (members ascending, so the step is deterministic)
// and centroids (the mean of the members' keys, summed in member order in
// FP32). The step: the scoring spreads every unit's centroids over 64-block
// work-groups (a wave takes 16 whole centroid rows at once, one coalesced
// 512-byte read per row, the G query heads' dot products reduced by DPP), so
// the whole GPU streams them; then one 1024-thread work-group per unit ranks
// the blocks by a bitonic sort of (key, block id) in LDS, takes the longest
// prefix of the ranking that fits the token budget, and writes the chosen
// blocks' tokens (block after block) as the index list the token-mode
// attention reads.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kClThreads = 1024;

// ---- index build -----------------------------------------------------------

// offsets[u][c] = the number of tokens t < L of unit u assigned to blocks
// before c; offsets[u][C] the total. One 1024-thread work-group per unit.
__global__ __launch_bounds__(kClThreads) void cluster_count_kernel(
    const int32_t* __restrict__ assign, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int C, int32_t* __restrict__ offsets) {
  __shared__ uint32_t cnt[kMaxClusters];
  __shared__ int wsum[kClThreads / kWave];
  const int unit = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = clamp_len(seq_lens[unit / Hkv], Tmax);
  for (int c = tid; c < C; c += kClThreads) cnt[c] = 0u;
  __syncthreads();
  const int32_t* a = assign + int64_t(unit) * Tmax;
  for (int t = tid; t < L; t += kClThreads) {
    const int c = a[t];
    if (c >= 0 && c < C) atomicAdd(&cnt[c], 1u);
  }
  __syncthreads();
  // exclusive scan of cnt[0 .. C) in order: thread t owns a run of P entries
  const int P = ceil_div(C, kClThreads);
  const int c0 = min(C, tid * P), c1 = min(C, c0 + P);
  int run = 0;
  for (int c = c0; c < c1; ++c) run += int(cnt[c]);
  int incl = run;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = incl - run;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int32_t* off = offsets + int64_t(unit) * (C + 1);
  for (int c = c0; c < c1; ++c) {
    off[c] = before;
    before += int(cnt[c]);
  }
  if (tid == kClThreads - 1) off[C] = before;  // the last thread's run ends the total
}

// members: block c's tokens, ascending, at offsets[c] .. offsets[c + 1].
// grid (B * Hkv, ceil(C / 64)), 256 threads: a work-group lists the tokens of
// 64 blocks, reading the unit's assignment 256 tokens at a time; a token's
// place is its block's cursor, plus its block's tokens in earlier waves of
// the round and in lower lanes of its own wave (found one block at a time by
// ballots: a wave of 64 tokens meets few of the work-group's blocks).
constexpr int kClGroup = 64;

__global__ __launch_bounds__(256) void cluster_members_kernel(
    const int32_t* __restrict__ assign, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int C, const int32_t* __restrict__ offsets, int32_t* __restrict__ members) {
  __shared__ int cur[kClGroup];
  __shared__ int cnt[4][kClGroup];
  const int unit = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g0 = blockIdx.y * kClGroup;
  const int L = clamp_len(seq_lens[unit / Hkv], Tmax);
  const int32_t* a = assign + int64_t(unit) * Tmax;
  const int32_t* off = offsets + int64_t(unit) * (C + 1);
  int32_t* mem = members + int64_t(unit) * Tmax;
  if (tid < kClGroup) cur[tid] = g0 + tid < C ? off[g0 + tid] : 0;
  for (int t0 = 0; t0 < L; t0 += 256) {
    const int t = t0 + tid;
    const int c = t < L ? a[t] : -1;
    const bool mine = c >= g0 && c < min(g0 + kClGroup, C);
    if (tid < 4 * kClGroup) cnt[tid / kClGroup][tid % kClGroup] = 0;
    __syncthreads();  // cur from the last round, cnt cleared
    // this wave's tokens per block, and each token's rank among them
    int rank = 0;
    uint64_t todo = __ballot(mine);
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int cl = __shfl(c, leader, kWave);
      const uint64_t same = __ballot(mine && c == cl);
      if (mine && c == cl) rank = __popcll(same & ((1ull << lane) - 1ull));
      if (lane == leader) cnt[wave][cl - g0] = __popcll(same);
      todo &= ~same;
    }
    __syncthreads();
    if (mine) {
      int pos = cur[c - g0] + rank;
      for (int w = 0; w < wave; ++w) pos += cnt[w][c - g0];
      mem[pos] = t;
    }
    __syncthreads();  // every place taken before the cursors move
    if (tid < kClGroup) cur[tid] += cnt[0][tid] + cnt[1][tid] + cnt[2][tid] + cnt[3][tid];
    __syncthreads();  // the counts read before the next round clears them
  }
}

// centroids[u][c] = mean of the members' keys (FP32 sum in member order).
// grid (B * Hkv, ceil(C / 4)), 256 threads: one wave per block, lane l
// holding channels 2 l and 2 l + 1.
template <int DT>
__global__ __launch_bounds__(256) void cluster_centroid_kernel(
    const uint16_t* __restrict__ k, int Hkv, int Tmax, int64_t sb, int64_t sh, int64_t st,
    int C, const int32_t* __restrict__ offsets, const int32_t* __restrict__ members,
    float* __restrict__ centroids) {
  const int unit = blockIdx.x, lane = threadIdx.x & 63;
  const int c = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (c >= C) return;
  const int b = unit / Hkv, h = unit % Hkv;
  const int32_t* off = offsets + int64_t(unit) * (C + 1);
  const int32_t* mem = members + int64_t(unit) * Tmax;
  const uint16_t* ku = k + b * sb + h * sh;
  const int m0 = off[c], m1 = off[c + 1];
  float s0 = 0.0f, s1 = 0.0f;
  for (int m = m0; m < m1; ++m) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(ku + int64_t(mem[m]) * st + 2 * lane);
    if (DT == BSA_DTYPE_F16) {
      s0 += half_bits_to_float(uint16_t(x & 0xFFFFu));
      s1 += half_bits_to_float(uint16_t(x >> 16));
    } else {
      s0 += bf16_bits_to_float(x & 0xFFFFu);
      s1 += bf16_bits_to_float(x >> 16);
    }
  }
  const int n = m1 - m0;
  float2v r = {0.0f, 0.0f};
  if (n > 0) {
    r[0] = s0 / float(n);
    r[1] = s1 / float(n);
  }
  *reinterpret_cast<float2v*>(centroids + (int64_t(unit) * C + c) * kHeadDim + 2 * lane) = r;
}

// ---- the step: score, rank, select ------------------------------------------

struct ClusterLds {
  uint64_t key[kMaxClusters];  // (score key, ~block id): descending = the ranking
  int pref[kMaxClusters + 1];  // sizes of the ranking's blocks, summed
  int wsum[kClThreads / kWave];
  int chosen;                  // blocks taken
};

// The centroids' scores: grid (B * Hkv, ceil(C / 64)), 256 threads; wave w
// scores blocks 64 blockIdx.y + 16 w .. + 15, lane l holding channels 2 l and
// 2 l + 1 of the rows and of each query head.
constexpr int kClRowsPerWave = 16;

template <int G>
__global__ __launch_bounds__(256) void cluster_score_kernel(
    const _Float16* __restrict__ q, const float* __restrict__ centroids,
    const int32_t* __restrict__ offsets, float* __restrict__ scores, int Hkv, int Hq, int C,
    float sigma) {
  const int unit = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = unit / Hkv, h = unit % Hkv;
  const int c0 = blockIdx.y * (4 * kClRowsPerWave) + wave * kClRowsPerWave;
  if (c0 >= C) return;  // wave-uniform
  const int32_t* off = offsets + int64_t(unit) * (C + 1);
  const float* cu = centroids + int64_t(unit) * C * kHeadDim;
  // every load is issued before the first use: the rows, the query heads and
  // the rows' offsets (lane j < 17 holds offsets[c0 + j])
  float2v x[kClRowsPerWave];
#pragma unroll
  for (int j = 0; j < kClRowsPerWave; ++j)
    x[j] = *reinterpret_cast<const float2v*>(cu + int64_t(min(c0 + j, C - 1)) * kHeadDim +
                                              2 * lane);
  const int ob = off[min(c0 + min(lane, kClRowsPerWave), C)];
  float qa[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const _Float16* qr = q + (int64_t(b) * Hq + h * G + g) * kHeadDim + 2 * lane;
    qa[g][0] = float(qr[0]);
    qa[g][1] = float(qr[1]);
  }
  float mine = -__builtin_inff();  // lane j < 16: the score of block c0 + j
#pragma unroll
  for (int j = 0; j < kClRowsPerWave; ++j) {
    float best = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < G; ++g)
      best = fmaxf(best, wave_sum_uniform(qa[g][0] * x[j][0] + qa[g][1] * x[j][1]));
    mine = lane == j ? best : mine;
  }
  const int c = c0 + lane;
  const int next = __shfl_down(ob, 1, kWave);  // offsets[c + 1]
  if (lane < kClRowsPerWave && c < C)
    scores[int64_t(unit) * C + c] = next > ob ? sigma * mine : -__builtin_inff();
}

// The choice from the scores: one 1024-thread work-group per unit.
__global__ __launch_bounds__(kClThreads) void cluster_select_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ members,
    const float* __restrict__ scores_in, int Tmax, int C, int budget, int32_t* __restrict__ idx,
    int32_t* __restrict__ count) {
  __shared__ ClusterLds s;
  const int unit = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* off = offsets + int64_t(unit) * (C + 1);
  int N = 1;  // sort size: a power of two >= C
  while (N < C) N <<= 1;
  for (int c = tid; c < C; c += kClThreads) {
    const float sc = off[c + 1] > off[c] ? scores_in[int64_t(unit) * C + c] : -__builtin_inff();
    s.key[c] = (uint64_t(score_key(sc)) << 32) | uint32_t(~uint32_t(c));
  }
  for (int c = C + tid; c < N; c += kClThreads) s.key[c] = 0ull;  // padding ranks last
  __syncthreads();
  // bitonic sort, descending. Up to 1024 keys each thread holds one, and the
  // compare-exchanges between lanes of one wave go through shuffles (no
  // barrier): only the steps whose partner lies in another wave use LDS.
  if (N <= kClThreads) {
    uint64_t v = tid < N ? s.key[tid] : 0ull;
    for (int kk = 2; kk <= N; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        uint64_t o;
        if (j >= kWave) {  // partner in another wave (uniform branch)
          if (tid < N) s.key[tid] = v;
          __syncthreads();
          o = tid < N ? s.key[tid ^ j] : 0ull;
          __syncthreads();  // read before the next publication overwrites it
        } else {
          const uint32_t lo = __shfl_xor(uint32_t(v), j, kWave);
          const uint32_t hi = __shfl_xor(uint32_t(v >> 32), j, kWave);
          o = (uint64_t(hi) << 32) | lo;
        }
        // in a descending run the lower position keeps the larger key
        const bool desc = (tid & kk) == 0, lower = (tid & j) == 0;
        v = (desc == lower) ? (v > o ? v : o) : (v < o ? v : o);
      }
    }
    if (tid < N) s.key[tid] = v;
    __syncthreads();
  } else {
    for (int kk = 2; kk <= N; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < N; i += kClThreads) {
          const int p = i ^ j;
          if (p > i) {
            const uint64_t a = s.key[i], e = s.key[p];
            const bool desc = (i & kk) == 0;
            if (desc ? a < e : a > e) {
              s.key[i] = e;
              s.key[p] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  // the ranking's sizes, summed (an empty block adds nothing), and the cut:
  // the first rank r whose sum exceeds the budget
  const int P = ceil_div(C, kClThreads);
  const int r0 = min(C, tid * P), r1 = min(C, r0 + P);
  auto size_at = [&](int r) {
    const int c = int(~uint32_t(s.key[r] & 0xFFFFFFFFull));
    return (c >= 0 && c < C) ? off[c + 1] - off[c] : 0;
  };
  int run = 0;
  for (int r = r0; r < r1; ++r) run += size_at(r);
  int incl = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) s.wsum[wave] = incl;
  if (tid == 0) s.chosen = C;
  __syncthreads();
  int before = incl - run;
  for (int w = 0; w < wave; ++w) before += s.wsum[w];
  for (int r = r0; r < r1; ++r) {
    s.pref[r] = before;
    before += size_at(r);
    if (before > budget) atomicMin(&s.chosen, r);  // rank r does not fit
  }
  if (tid == kClThreads - 1) s.pref[C] = before;
  __syncthreads();
  const int m = s.chosen;  // ranks 0 .. m-1 are taken (whole blocks)
  const int total = s.pref[m];
  int32_t* out = idx + int64_t(unit) * budget;
  const int32_t* mem = members + int64_t(unit) * Tmax;
  for (int p = tid; p < budget; p += kClThreads) {
    int tok = -1;
    if (p < total) {
      // the rank holding position p: the last r < m with pref[r] <= p
      int lo = 0, hi = m - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.pref[mid] <= p) lo = mid;
        else hi = mid - 1;
      }
      const int c = int(~uint32_t(s.key[lo] & 0xFFFFFFFFull));
      tok = mem[off[c] + (p - s.pref[lo])];
    }
    out[p] = tok;
  }
  if (tid == 0) count[unit] = total;
}

}  // namespace

hipError_t launch_cluster_index(const UnitGeom& g, int C, const void* k, const int32_t* assign,
                                const int32_t* seq_lens, float* centroids, int32_t* offsets,
                                int32_t* members, hipStream_t s) {
  const int units = g.B * g.Hkv;
  hipLaunchKernelGGL(cluster_count_kernel, dim3(units), dim3(kClThreads), 0, s, assign, seq_lens,
                     g.Hkv, g.Tmax, C, offsets);
  hipLaunchKernelGGL(cluster_members_kernel, dim3(units, ceil_div(C, kClGroup)), dim3(256), 0, s,
                     assign, seq_lens, g.Hkv, g.Tmax, C, offsets, members);
  const dim3 cg(units, ceil_div(C, 4));
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  if (g.dtype == BSA_DTYPE_F16)
    hipLaunchKernelGGL(cluster_centroid_kernel<BSA_DTYPE_F16>, cg, dim3(256), 0, s, kp, g.Hkv,
                       g.Tmax, g.sb, g.sh, g.st, C, offsets, members, centroids);
  else
    hipLaunchKernelGGL(cluster_centroid_kernel<BSA_DTYPE_BF16>, cg, dim3(256), 0, s, kp, g.Hkv,
                       g.Tmax, g.sb, g.sh, g.st, C, offsets, members, centroids);
  return hipGetLastError();
}

hipError_t launch_cluster_step(const UnitGeom& g, int C, int budget, float sigma, bool score,
                               bool select, const _Float16* q, const float* centroids,
                               const int32_t* offsets, const int32_t* members,
                               const float* scores_in, float* scores_out, int32_t* idx,
                               int32_t* count, hipStream_t s) {
  const int units = g.B * g.Hkv;
  if (score) {
    const dim3 grid(units, ceil_div(C, 4 * kClRowsPerWave));
#define BSA_CL(GG)                                                                              \
  hipLaunchKernelGGL((cluster_score_kernel<GG>), grid, dim3(256), 0, s, q, centroids, offsets, \
                     scores_out, g.Hkv, g.Hq, C, sigma)
    switch (g.G) {
      case 1: BSA_CL(1); break;
      case 2: BSA_CL(2); break;
      case 4: BSA_CL(4); break;
      case 8: BSA_CL(8); break;
      case 16: BSA_CL(16); break;
      default: return hipErrorInvalidValue;
    }
#undef BSA_CL
  }
  if (select)
    hipLaunchKernelGGL(cluster_select_kernel, dim3(units), dim3(kClThreads), 0, s, offsets,
                       members, score ? scores_out : scores_in, g.Tmax, C, budget, idx, count);
  return hipGetLastError();
}

}  // namespace bsa
