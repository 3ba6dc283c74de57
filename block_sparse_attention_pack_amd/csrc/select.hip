// Top-k selection per unit (Jet-QSparse abstract: top blocks per KV head;
// JSSA Figure 1 and Table 15: top-B tokens per KV head, shared by the group).
//
// Block mode: one 256-thread work-group per unit runs select_unit_rows
// (select_core.hpp).
//
// Token mode: one 1024-thread work-group per unit. Scores become
// order-preserving 32-bit keys. A radix select finds the exact key kappa of the
// picks-th largest candidate in at most three histogram passes (12 + 12 + 8
// bits, LDS histograms), stopping early once the bucket holding the boundary is
// taken whole. An index-ordered compaction then writes, in ascending order,
// every candidate with key > kappa plus the lowest-index candidates with key ==
// kappa up to the budget.
#include "common.hpp"
#include "select_core.hpp"

namespace bsa {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxDigitBits = 12;
constexpr int kLdsKeys = 8192;  // candidates staged in LDS (32 KiB) when they fit

struct ScanScratch {
  int wave_tot[kSelWaves];
  int wave_tot2[kSelWaves];
};

// Inclusive scan over the work-group of one int per thread; `total` gets the sum.
__device__ __forceinline__ int block_scan(int v, int* lds, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(v, off, kWave);
    if (lane >= off) v += n;
  }
  if (lane == kWave - 1) lds[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int x = lds[w];
    before += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return v + before;
}

__device__ __forceinline__ int wave_exclusive_scan(int v, int& total) {
  const int lane = threadIdx.x & 63;
  int inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += n;
  }
  total = __shfl(inc, kWave - 1, kWave);
  return inc - v;
}

// grid (B * Hkv), 1024 threads.
// block mode: row length NBmax, candidates n < ceil(L/128) - n_tail, forced pages after.
// token mode: row length Tmax, candidates t < L, no forced pages.
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int row_len, int block_mode, int budget, int n_tail, int32_t* __restrict__ idx,
    int32_t* __restrict__ count) {
  __shared__ uint32_t hist[1 << kMaxDigitBits];
  __shared__ uint32_t keys_lds[kLdsKeys];
  __shared__ ScanScratch scr;
  __shared__ int sh_beta, sh_above;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x;
  const int b = unit / Hkv;
  const int L = clamp_len(seq_lens[b], Tmax);
  int C, picks, f0, f1;
  if (block_mode) {
    const int npg = ceil_div(L, kBlock);
    C = max(0, npg - n_tail);
    C = min(C, row_len);
    picks = budget - n_tail;
    f0 = max(0, npg - n_tail);
    f1 = npg;
  } else {
    C = min(L, row_len);
    picks = budget;
    f0 = f1 = 0;
  }
  picks = max(0, min(picks, C));
  const float* row = scores + int64_t(unit) * row_len;
  // block-mode rows (and short token rows) are read from global memory once
  const bool in_lds = C <= kLdsKeys;
  if (in_lds) {
    for (int i = tid; i < C; i += kSelThreads) keys_lds[i] = score_key(row[i]);
    __syncthreads();
  }
  auto key_at = [&](int i) -> uint32_t { return in_lds ? keys_lds[i] : score_key(row[i]); };

  // --- radix select of the picks-th largest key ---------------------------
  // After the loop every candidate with key > kgt is taken, and of those with
  // key == keq the r_eq lowest indices are taken (r_eq = 0 when none are).
  uint32_t kgt = 0xFFFFFFFFu, keq = 0u;
  int r_eq = 0;
  bool take_all = picks == C, take_ge = false;
  uint32_t kge = 0u;
  if (!take_all && picks > 0) {
    uint32_t prefix = 0;
    int bits = 0, r = picks;
    while (true) {
      const int width = min(kMaxDigitBits, 32 - bits);
      const int nb = 1 << width;
      const int shift = 32 - bits - width;
      for (int d = tid; d < nb; d += kSelThreads) hist[d] = 0;
      __syncthreads();
      for (int i = tid; i < C; i += kSelThreads) {
        const uint32_t key = key_at(i);
        if (bits == 0 || (key >> (32 - bits)) == prefix)
          atomicAdd(&hist[(key >> shift) & uint32_t(nb - 1)], 1u);
      }
      __syncthreads();
      // bins per thread: nb / 1024 (4, or 1 for the last 8-bit digit)
      const int per = nb >= kSelThreads ? nb / kSelThreads : 1;
      const int lo = tid * per;
      int mine = 0;
      for (int d = lo; d < lo + per && d < nb; ++d) mine += int(hist[d]);
      int total;
      const int inc = block_scan(mine, scr.wave_tot, total);
      int above = total - inc;  // keys in bins above this thread's bins
      for (int d = lo + per - 1; d >= lo; --d) {
        if (d >= nb) continue;
        const int hd = int(hist[d]);
        if (above < r && r <= above + hd) {
          sh_beta = d;
          sh_above = above;
        }
        above += hd;
      }
      __syncthreads();
      const int beta = sh_beta;
      const int above_beta = sh_above;
      const int in_bucket = int(hist[beta]);
      __syncthreads();
      r -= above_beta;
      prefix = (prefix << width) | uint32_t(beta);
      bits += width;
      if (r == in_bucket) {  // the whole bucket is taken: key >= its lowest key
        take_ge = true;
        kge = prefix << (32 - bits);
        break;
      }
      if (bits == 32) {
        kgt = prefix;
        keq = prefix;
        r_eq = r;
        break;
      }
    }
  }

  // --- index-ordered compaction -------------------------------------------
  // Wave w owns candidates [w * seg, (w + 1) * seg); chunks of 256 (4 per lane).
  const int seg = ceil_div(ceil_div(C, kSelWaves), 256) * 256;
  const int s0 = wave * seg, s1 = min(C, s0 + seg);
  auto classify = [&](int i, uint32_t key, bool& gt, bool& eq) {
    if (take_all) {
      gt = true;
      eq = false;
    } else if (take_ge) {
      gt = key >= kge;
      eq = false;
    } else if (picks == 0) {
      gt = eq = false;
    } else {
      gt = key > kgt;
      eq = key == keq;
    }
  };
  // pass 1: per-wave counts of taken-by-key and of ties
  int n_gt = 0, n_eq = 0;
  for (int c0 = s0; c0 < s1; c0 += 256) {
    int cg = 0, ce = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = c0 + 4 * lane + k;
      if (i < s1) {
        bool gt, eq;
        classify(i, key_at(i), gt, eq);
        cg += gt;
        ce += eq;
      }
    }
    int t;
    wave_exclusive_scan(cg, t);
    n_gt += t;
    wave_exclusive_scan(ce, t);
    n_eq += t;
  }
  if (lane == 0) {
    scr.wave_tot[wave] = n_gt;
    scr.wave_tot2[wave] = n_eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += scr.wave_tot[w];
    eq_before += scr.wave_tot2[w];
  }
  // pass 2: write positions
  int32_t* out = idx + int64_t(unit) * budget;
  int pos = gt_before + min(eq_before, r_eq);
  int eq_seen = eq_before;
  for (int c0 = s0; c0 < s1; c0 += 256) {
    bool gt[4], eq[4];
    int ce = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = c0 + 4 * lane + k;
      gt[k] = eq[k] = false;
      if (i < s1) classify(i, key_at(i), gt[k], eq[k]);
      ce += eq[k];
    }
    int ce_tot;
    int eq_rank = eq_seen + wave_exclusive_scan(ce, ce_tot);
    int take = 0;
    bool sel[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sel[k] = gt[k] || (eq[k] && eq_rank < r_eq);
      eq_rank += eq[k];
      take += sel[k];
    }
    int take_tot;
    int p = pos + wave_exclusive_scan(take, take_tot);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (sel[k]) {
        if (p < budget) out[p] = c0 + 4 * lane + k;  // always true; guards the write
        ++p;
      }
    pos += take_tot;
    eq_seen += ce_tot;
  }
  __syncthreads();
  // the last wave's end position is the number chosen by score
  if (wave == kSelWaves - 1 && lane == 0) sh_above = pos;
  __syncthreads();
  const int nsel = min(sh_above, budget);
  const int nf = max(0, f1 - f0);
  for (int k = tid; k < budget - nsel; k += kSelThreads)
    out[nsel + k] = k < nf ? f0 + k : -1;
  if (tid == 0) count[unit] = nsel + min(nf, budget - nsel);
}

// Block mode: one 256-thread work-group per unit.
__global__ __launch_bounds__(kSelectThreads) void select_block_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int NBmax, int budget, int n_tail, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ SelectLds lds;
  const int unit = blockIdx.x;
  const int L = clamp_len(seq_lens[unit / Hkv], Tmax);
  int C, picks, f0, f1;
  block_candidates(L, n_tail, NBmax, budget, C, picks, f0, f1);
  select_unit_rows(scores + int64_t(unit) * NBmax, C, picks, f0, f1, budget,
                   idx + int64_t(unit) * budget, count + unit, lds);
}

}  // namespace

hipError_t launch_select_block(const UnitGeom& g, int budget, int n_tail, const float* scores,
                               const int32_t* seq_lens, int32_t* idx, int32_t* count,
                               hipStream_t s) {
  hipLaunchKernelGGL(select_block_kernel, dim3(g.B * g.Hkv), dim3(kSelectThreads), 0, s, scores,
                     seq_lens, g.Hkv, g.Tmax, g.NBmax, budget, n_tail, idx, count);
  return hipGetLastError();
}

size_t token_select_workspace(const UnitGeom&) { return 0; }

hipError_t launch_select_token(const UnitGeom& g, int budget, const float* scores,
                               const int32_t* seq_lens, void*, int32_t* idx, int32_t* count,
                               hipStream_t s) {
  hipLaunchKernelGGL(select_topk_kernel, dim3(g.B * g.Hkv), dim3(kSelThreads), 0, s, scores,
                     seq_lens, g.Hkv, g.Tmax, g.Tmax, 0, budget, 0, idx, count);
  return hipGetLastError();
}

}  // namespace bsa
