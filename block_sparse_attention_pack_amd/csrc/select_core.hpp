// Top-k selection of one unit by one 256-thread work-group (block mode).
//
// Scores become order-preserving 32-bit keys. A radix select finds the exact
// key kappa of the picks-th largest candidate: its first digit starts at the
// highest bit in which the candidates' keys differ (the bits above are common
// to all of them), digits are up to 8 bits wide, and the passes stop once the
// bucket that holds the boundary is taken whole. A pass costs two barriers: the
// histograms alternate between two LDS buffers (the next one is cleared while
// the current one fills), and one wave scans the 256 bins and names the
// boundary bucket. Each thread owns a contiguous range of candidate indices, so
// one block-wide scan of the taken-by-key and tied counts places every chosen
// index: the output is ascending, and of the candidates tied at kappa the lowest
// indices are taken. The forced tail pages follow the scanned blocks. Wave-wide
// scans and the key range use DPP moves, not LDS permutes: on a chain of six
// dependent lane exchanges the permutes' LDS latency set the pace.
#pragma once

#include "common.hpp"

namespace bsa {

constexpr int kSelectThreads = 256;
constexpr int kSelectRegKeys = 8;  // rows up to 2048 candidates stay in registers

struct SelectLds {
  uint32_t hist[256];
  uint32_t hist2[256];  // the block select's second histogram (passes alternate)
  int wave_tot[kSelectThreads / kWave];
  int wave_tot2[kSelectThreads / kWave];
  uint32_t wave_lo[kSelectThreads / kWave], wave_hi[kSelectThreads / kWave];
  int beta, above, inb;
};

// Inclusive scans of two ints per thread over the work-group, with one pair of
// barriers; tv, tw: the totals.
__device__ __forceinline__ void select_block_scan2(int& v, int& w, SelectLds& s, int& tv,
                                                   int& tw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_dpp(v);
  w = wave_scan_dpp(w);
  if (lane == kWave - 1) {
    s.wave_tot[wave] = v;
    s.wave_tot2[wave] = w;
  }
  __syncthreads();
  int bv = 0, bw = 0;
  tv = 0;
  tw = 0;
#pragma unroll
  for (int k = 0; k < kSelectThreads / kWave; ++k) {
    const int xv = s.wave_tot[k], xw = s.wave_tot2[k];
    bv += k < wave ? xv : 0;
    bw += k < wave ? xw : 0;
    tv += xv;
    tw += xw;
  }
  __syncthreads();
  v += bv;
  w += bw;
}

// Inclusive scan of one int per thread over the 256-thread work-group.
__device__ __forceinline__ int select_block_scan(int v, SelectLds& s, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_dpp(v);
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
  const int lane = tid & 63, wave = tid >> 6;
  if (!take_all && picks > 0) {
    // the candidates' key range
    uint32_t klo = 0xFFFFFFFFu, khi = 0u;
    for_each_key([&](int, uint32_t key) {
      klo = key < klo ? key : klo;
      khi = key > khi ? key : khi;
    });
    wave_minmax_dpp(klo, khi);
    if (lane == 0) {
      s.wave_lo[wave] = klo;
      s.wave_hi[wave] = khi;
    }
    s.hist[tid] = 0;  // the first pass's histogram
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSelectThreads / kWave; ++k) {
      klo = s.wave_lo[k] < klo ? s.wave_lo[k] : klo;
      khi = s.wave_hi[k] > khi ? s.wave_hi[k] : khi;
    }
    // bits [hi, 32) are common to every candidate; prefix holds them
    const uint32_t diff = klo ^ khi;
    int hi = diff ? 32 - __builtin_clz(diff) : 0;
    uint32_t prefix = hi < 32 ? khi >> hi : 0u;
    int r = picks;
    for (int pass = 0;; ++pass) {
      if (hi == 0) {  // every bit resolved: kappa = prefix, r of its ties are taken
        kgt = keq = prefix;
        r_eq = r;
        break;
      }
      const int width = hi < 8 ? hi : 8;
      const int shift = hi - width;
      uint32_t* cur = (pass & 1) ? s.hist2 : s.hist;
      uint32_t* nxt = (pass & 1) ? s.hist : s.hist2;
      nxt[tid] = 0;  // its last reader finished before the previous pass's last barrier
      for_each_key([&](int, uint32_t key) {
        if (hi == 32 || (key >> hi) == prefix)
          atomicAdd(&cur[(key >> shift) & ((1u << width) - 1u)], 1u);
      });
      __syncthreads();
      if (wave == 0) {
        // lane l takes bins 255 - 4 l .. 252 - 4 l (descending); ge counts the
        // keys in bins >= d, above those in bins > d
        if (lane == 0) {  // defined even if no bin qualified (the next writes win)
          s.beta = 0;
          s.above = 0;
          s.inb = 0;
        }
        int c[4];
        int run = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          run += int(cur[255 - 4 * lane - i]);
          c[i] = run;
        }
        const int incl = wave_scan_dpp(run);
        const int P = incl - run;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int above = P + (i ? c[i - 1] : 0), ge = P + c[i];
          if (above < r && r <= ge) {
            s.beta = 255 - 4 * lane - i;
            s.above = above;
            s.inb = ge - above;
          }
        }
      }
      __syncthreads();
      const int beta = s.beta, above_beta = s.above, in_bucket = s.inb;
      r -= above_beta;
      prefix = (prefix << width) | uint32_t(beta);
      hi = shift;
      if (r == in_bucket) {  // the whole bucket is taken
        take_ge = true;
        kge = prefix << hi;
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
  int sgt = ngt, seq = neq, tot_gt, tot_eq;
  select_block_scan2(sgt, seq, s, tot_gt, tot_eq);
  const int gt_before = sgt - ngt, eq_before = seq - neq;
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
