// Top-k selection of one unit by one 256-thread work-group (block mode).
//
// Scores become order-preserving 32-bit keys. A radix select over 8-bit digits
// (LDS histograms, at most four passes, stopping once the bucket that holds the
// boundary is taken whole) finds the exact key kappa of the picks-th largest
// candidate. Each thread owns a contiguous range of candidate indices, so
// block-wide scans of the taken-by-key and tied counts place every chosen index: the
// output is ascending, and of the candidates tied at kappa the lowest indices
// are taken. The forced tail pages follow the scanned blocks.
#pragma once

#include "common.hpp"

namespace bsa {

constexpr int kSelectThreads = 256;
constexpr int kSelectRegKeys = 8;  // rows up to 2048 candidates stay in registers

struct SelectLds {
  uint32_t hist[256];
  int wave_tot[kSelectThreads / kWave];
  int beta, above;
};

// Inclusive scan of one int per thread over the 256-thread work-group.
__device__ __forceinline__ int select_block_scan(int v, SelectLds& s, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(v, off, kWave);
    if (lane >= off) v += n;
  }
  if (lane == kWave - 1) s.wave_tot[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelectThreads / kWave; ++w) {
    const int x = s.wave_tot[w];
    before += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return v + before;
}

// Chooses `picks` of candidates 0 .. C-1 of `row` (largest scores, lower index
// first among equal ones), appends the forced entries f0 .. f1-1, writes them
// ascending to out[0 .. budget) padded with -1, and the number chosen to *count.
// Every thread of the work-group must call it (it synchronises the group).
// COHERENT: read the scores as device-scope loads (they were stored by other
// work-groups of the same launch).
template <bool COHERENT = false>
__device__ __forceinline__ void select_unit_rows(const float* row, int C, int picks, int f0,
                                                 int f1, int budget, int32_t* out,
                                                 int32_t* count, SelectLds& s) {
  auto score_at = [&](int i) -> float { return COHERENT ? load_coherent(row + i) : row[i]; };
  const int tid = threadIdx.x;
  picks = max(0, min(picks, C));
  const int per = ceil_div(C, kSelectThreads);
  const int i0 = min(C, tid * per), i1 = min(C, i0 + per);
  // Up to kSelectRegKeys candidates per thread are read once and kept in
  // registers; longer rows are re-read from memory on every pass.
  const bool in_regs = per <= kSelectRegKeys;
  uint32_t rk[kSelectRegKeys];
  if (in_regs) {
    if constexpr (COHERENT) {
      // device-scope loads are not reordered by the compiler: issue them all
      // before the first is used (indices past the thread's range are clamped
      // into the row and their values dropped)
      float f[kSelectRegKeys];
      const int last = max(C - 1, 0);
#pragma unroll
      for (int j = 0; j < kSelectRegKeys; ++j) f[j] = score_at(min(i0 + j, last));
#pragma unroll
      for (int j = 0; j < kSelectRegKeys; ++j) rk[j] = i0 + j < i1 ? score_key(f[j]) : 0u;
    } else {
#pragma unroll
      for (int j = 0; j < kSelectRegKeys; ++j)
        rk[j] = i0 + j < i1 ? score_key(score_at(i0 + j)) : 0u;
    }
  }
  auto for_each_key = [&](auto&& f) {
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kSelectRegKeys; ++j)
        if (i0 + j < i1) f(i0 + j, rk[j]);
    } else {
      for (int i = i0; i < i1; ++i) f(i, score_key(score_at(i)));
    }
  };

  // keys taken: key > kgt, plus the first r_eq (by index) with key == keq;
  // or every key >= kge when a whole bucket is taken
  uint32_t kgt = 0xFFFFFFFFu, keq = 0u, kge = 0u;
  int r_eq = 0;
  bool take_ge = false;
  const bool take_all = picks == C;
  if (!take_all && picks > 0) {
    uint32_t prefix = 0;
    int bits = 0, r = picks;
    while (true) {
      const int shift = 24 - bits;
      s.hist[tid] = 0;
      __syncthreads();
      for_each_key([&](int, uint32_t key) {
        if (bits == 0 || (key >> (shift + 8)) == prefix)
          atomicAdd(&s.hist[(key >> shift) & 0xFFu], 1u);
      });
      __syncthreads();
      // thread t looks at bin d = 255 - t; the inclusive scan counts bins >= d
      const int d = 255 - tid;
      const int hd = int(s.hist[d]);
      if (tid == 0) {  // defined results even if no bin qualifies (ordered by the scan's barriers)
        s.beta = 0;
        s.above = 0;
      }
      int total;
      const int ge = select_block_scan(hd, s, total);
      const int above = ge - hd;  // keys in bins above d
      if (above < r && r <= ge) {
        s.beta = d;
        s.above = above;
      }
      __syncthreads();
      const int beta = s.beta, above_beta = s.above;
      const int in_bucket = int(s.hist[beta]);
      __syncthreads();
      r -= above_beta;
      prefix = (prefix << 8) | uint32_t(beta);
      bits += 8;
      if (r == in_bucket) {  // the whole bucket is taken
        take_ge = true;
        kge = prefix << (32 - bits);
        break;
      }
      if (bits == 32) {
        kgt = keq = prefix;
        r_eq = r;
        break;
      }
    }
  }
  auto taken_by_key = [&](uint32_t key) {
    return take_all || (take_ge ? key >= kge : (picks > 0 && key > kgt));
  };
  auto tied = [&](uint32_t key) { return !take_all && !take_ge && picks > 0 && key == keq; };

  // counts of this thread's range: taken by key, and tied at kappa
  int ngt = 0, neq = 0;
  for_each_key([&](int, uint32_t key) {
    ngt += taken_by_key(key);
    neq += tied(key);
  });
  int tot_gt, tot_eq;
  const int gt_before = select_block_scan(ngt, s, tot_gt) - ngt;
  const int eq_before = select_block_scan(neq, s, tot_eq) - neq;
  const int nsel = max(0, min(tot_gt + min(tot_eq, r_eq), budget));
  int pos = gt_before + min(eq_before, r_eq);
  int eq_seen = eq_before;
  for_each_key([&](int i, uint32_t key) {
    bool take = taken_by_key(key);
    if (tied(key)) {
      take = eq_seen < r_eq;
      ++eq_seen;
    }
    if (take) {
      if (pos >= 0 && pos < budget) out[pos] = i;  // always true; guards the write
      ++pos;
    }
  });
  const int nf = max(0, f1 - f0);
  for (int k = tid; k < budget - nsel; k += kSelectThreads) out[nsel + k] = k < nf ? f0 + k : -1;
  if (tid == 0) *count = nsel + min(nf, budget - nsel);
}

// Candidates and forced pages of one unit in block mode.
__device__ __forceinline__ void block_candidates(int L, int n_tail, int row_len, int budget,
                                                 int& C, int& picks, int& f0, int& f1) {
  const int npg = ceil_div(L, kBlock);
  C = min(max(0, npg - n_tail), row_len);
  picks = budget - n_tail;
  f0 = max(0, npg - n_tail);
  f1 = npg;
}

}  // namespace bsa
