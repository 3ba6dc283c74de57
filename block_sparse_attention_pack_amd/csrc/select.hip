// Top-k selection per unit (Jet-QSparse abstract: top blocks per KV head;
// JSSA Figure 1 and Table 15: top-B tokens per KV head, shared by the group).
//
// Block mode: one 256-thread work-group per unit runs select_unit_rows
// (select_core.hpp); a unit has at most max_tokens/128 candidates.
//
// Token mode: a unit has up to max_tokens candidates (131072 at 128K context),
// too many for one work-group to read fast, so the selection is spread over
// kTokChunk-key chunks, one work-group each, in three launches:
//   hist    every group adds the histogram of its keys' top 12 bits (of the
//           order-preserving key) to its unit's, with device-scope atomics
//           (the histogram is zero on entry: the finish of the previous call
//           leaves it so); skipped when the token scan has already counted
//           them (bsa_score_select, bsa_decode_step);
//   filter  every group finds from that histogram the top digit beta that
//           holds the picks-th largest key and writes two bitmaps of its keys:
//           those with a larger top digit (taken), and those with top digit
//           beta (the bucket: usually about 1% of the keys);
//   finish  one group per unit lists the bucket's keys in token order, finds
//           the exact boundary key among them (radix select over the remaining
//           20 bits), compacts the taken tokens in index order (those above
//           the boundary key, and of its ties the lowest indices), and returns
//           the unit's histogram to zero.
#include "common.hpp"
#include "select_core.hpp"

namespace bsa {
namespace {

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

// ---------------------------------------------------------------------------
// Token mode
// ---------------------------------------------------------------------------
constexpr int kTokChunk = 16384;  // keys per work-group in hist and filter
constexpr int kTokBatch = 32;     // loads in flight per thread (hist)
constexpr int kTokBins = kTokHistBins;    // first digit: top 12 bits
constexpr int kTokShift = kTokHistShift;
constexpr int kTokSlot = 64;      // words of the state slot
constexpr int kTokWin = 4096;     // bitmap words per finish window
constexpr int kTokWpt = kTokWin / kSelectThreads;  // 16 words per thread and window
constexpr int kTokWinPad = kTokWin + kTokWin / 16;
constexpr int kTokStage = 8192;   // buckets up to this size are listed in LDS

// LDS index of window word k: one pad word per 16 keeps a thread's 16
// consecutive words in distinct banks from its neighbours'
__device__ __forceinline__ int tok_pad(int k) { return k + (k >> 4); }

// What the unit's state says is taken.
enum TokMode : uint32_t {
  kTokNone = 0,    // nothing (picks == 0)
  kTokAll = 1,     // every candidate
  kTokGe = 2,      // every key whose top digit is >= beta (the bucket is taken whole)
  kTokBucket = 3,  // top digit > beta, and r of the n keys whose top digit is beta
};

struct TokState {
  uint32_t mode, beta, r, n;
};

// Per-unit workspace: histogram, state and two bitmaps (taken by top digit;
// in the bucket), each on its own 256-byte boundary.
struct TokGeom {
  int W;               // 32-bit bitmap words per unit (a multiple of 2)
  int64_t w_bitmap;    // words reserved per bitmap
  int64_t unit_words;  // workspace words per unit
};

__host__ __device__ inline TokGeom tok_geom(int Tmax) {
  TokGeom t;
  t.W = ceil_div(Tmax, 64) * 2;
  t.w_bitmap = (int64_t(t.W) + 63) / 64 * 64;
  t.unit_words = kTokBins + kTokSlot + 2 * t.w_bitmap;
  return t;
}

struct TokUnit {
  uint32_t* hist;
  TokState* st;
  uint32_t* gt;  // bit t: token t taken by its top digit
  uint32_t* bk;  // bit t: token t in the bucket
};

__device__ __forceinline__ TokUnit tok_unit(void* ws, const TokGeom& t, int unit) {
  uint32_t* base = static_cast<uint32_t*>(ws) + int64_t(unit) * t.unit_words;
  TokUnit u;
  u.hist = base;
  u.st = reinterpret_cast<TokState*>(base + kTokBins);
  u.gt = base + kTokBins + kTokSlot;
  u.bk = u.gt + t.w_bitmap;
  return u;
}

__device__ __forceinline__ void tok_counts(const int32_t* seq_lens, int unit, int Hkv, int Tmax,
                                           int budget, int& C, int& picks) {
  C = clamp_len(seq_lens[unit / Hkv], Tmax);
  picks = max(0, min(budget, C));
}

// Histogram of the top 12 key bits of the unit's candidates.
// grid (ceil(Tmax / kTokChunk), B * Hkv), 256 threads.
__global__ __launch_bounds__(kSelectThreads) void tok_hist_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int budget, TokGeom tg, void* ws) {
  __shared__ uint32_t hist[kTokBins];
  const int unit = blockIdx.y, tid = threadIdx.x;
  int C, picks;
  tok_counts(seq_lens, unit, Hkv, Tmax, budget, C, picks);
  const int base = blockIdx.x * kTokChunk;
  if (picks == 0 || picks == C || base >= C) return;  // nothing to rank here
  for (int d = tid; d < kTokBins; d += kSelectThreads) hist[d] = 0u;
  __syncthreads();
  const float* row = scores + int64_t(unit) * Tmax;
  const int end = min(C, base + kTokChunk);
  for (int b0 = base; b0 < end; b0 += kTokBatch * kSelectThreads) {
    float v[kTokBatch];
#pragma unroll
    for (int j = 0; j < kTokBatch; ++j) {
      const int i = b0 + j * kSelectThreads + tid;
      v[j] = i < end ? row[i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kTokBatch; ++j) {
      const int i = b0 + j * kSelectThreads + tid;
      if (i < end) atomicAdd(&hist[score_key(v[j]) >> kTokShift], 1u);
    }
  }
  __syncthreads();
  const TokUnit u = tok_unit(ws, tg, unit);
  for (int d = tid; d < kTokBins; d += kSelectThreads) {
    const uint32_t h = hist[d];
    if (h) __hip_atomic_fetch_add(&u.hist[d], h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The top digit beta of the picks-th largest key, from the unit's histogram;
// `above` counts keys with a larger top digit, `in` those with digit beta.
__device__ __forceinline__ void tok_boundary(const uint32_t* ghist, int picks, SelectLds& lds,
                                             int& beta, int& above, int& in) {
  constexpr int kPer = kTokBins / kSelectThreads;  // 16 bins per thread, highest first
  const int tid = threadIdx.x;
  uint32_t h[kPer];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    h[j] = ghist[kTokBins - 1 - (tid * kPer + j)];
    mine += int(h[j]);
  }
  if (tid == 0) {  // defined results even if no bin qualifies (ordered by the scan's barriers)
    lds.beta = 0;
    lds.above = 0;
    lds.hist[0] = 0u;
  }
  int total;
  int ab = select_block_scan(mine, lds, total) - mine;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (ab < picks && picks <= ab + int(h[j])) {
      lds.beta = kTokBins - 1 - (tid * kPer + j);
      lds.above = ab;
      lds.hist[0] = h[j];
    }
    ab += int(h[j]);
  }
  __syncthreads();
  beta = lds.beta;
  above = lds.above;
  in = int(lds.hist[0]);
  __syncthreads();
}

// Bitmaps of the keys taken by their top digit and of the bucket (keys whose
// top digit is the boundary digit). grid (ceil(Tmax / kTokChunk), B * Hkv),
// 256 threads; wave w owns the 4096 keys from blockIdx.x * kTokChunk + 4096 w,
// as 64 rows of 64; lane j keeps row j's two words of each bitmap, so each
// bitmap is written with one 8-byte store per lane.
__global__ __launch_bounds__(kSelectThreads) void tok_filter_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int budget, TokGeom tg, void* ws) {
  constexpr int kRows = kTokChunk / kSelectThreads;
  static_assert(kRows == kWave, "one 64-key row per lane");
  __shared__ SelectLds lds;
  const int unit = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const TokUnit u = tok_unit(ws, tg, unit);
  int C, picks;
  tok_counts(seq_lens, unit, Hkv, Tmax, budget, C, picks);
  uint32_t mode = picks == 0 ? kTokNone : (picks == C ? kTokAll : kTokBucket);
  const float* row = scores + int64_t(unit) * Tmax;
  const int wbase = blockIdx.x * kTokChunk + wave * kRows * 64;
  // the keys are loaded before the boundary is known, so their latency
  // overlaps the histogram reads
  float v[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    const int i = wbase + j * 64 + lane;
    v[j] = (mode == kTokBucket && i < C) ? row[i] : 0.0f;
  }
  int beta = 0, above = 0, in = 0;
  if (mode == kTokBucket) {
    tok_boundary(u.hist, picks, lds, beta, above, in);
    if (picks - above == in) mode = kTokGe;
  }
  if (blockIdx.x == 0 && tid == 0) {
    TokState s;
    s.mode = mode;
    s.beta = uint32_t(beta);
    s.r = uint32_t(picks - above);
    s.n = uint32_t(in);
    *u.st = s;
  }
  uint32_t g0 = 0, g1 = 0, k0 = 0, k1 = 0;
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    const int i = wbase + j * 64 + lane;
    const uint32_t digit = score_key(v[j]) >> kTokShift;
    bool gt = false, inb = false;
    if (i < C) {
      if (mode == kTokAll) gt = true;
      else if (mode == kTokGe) gt = digit >= uint32_t(beta);
      else if (mode == kTokBucket) {
        gt = digit > uint32_t(beta);
        inb = digit == uint32_t(beta);
      }
    }
    const uint64_t bg = __ballot(gt), bb = __ballot(inb);
    if (lane == j) {
      g0 = uint32_t(bg);
      g1 = uint32_t(bg >> 32);
      k0 = uint32_t(bb);
      k1 = uint32_t(bb >> 32);
    }
  }
  const int word = wbase / 32 + 2 * lane;  // even; W is even
  if (word < tg.W) {
    *reinterpret_cast<uint2*>(u.gt + word) = make_uint2(g0, g1);
    *reinterpret_cast<uint2*>(u.bk + word) = make_uint2(k0, k1);
  }
}

// Resolve the bucket and compact the taken tokens in index order.
// grid (B * Hkv), 256 threads. The bitmaps are read in windows of kTokWin
// words (thread t owns window words 16 t .. 16 t + 15).
__global__ __launch_bounds__(kSelectThreads) void tok_finish_kernel(
    const float* __restrict__ scores, int Tmax, const int32_t* __restrict__ seq_lens, int Hkv,
    int budget, TokGeom tg, void* ws, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ uint32_t wgt[kTokWinPad];
  __shared__ uint32_t wbk[kTokWinPad];
  __shared__ uint32_t hist[kTokBins];
  __shared__ uint32_t skey[kTokStage];
  __shared__ int32_t stok[kTokStage];
  __shared__ SelectLds lds;
  const int unit = blockIdx.x, tid = threadIdx.x;
  const TokUnit u = tok_unit(ws, tg, unit);
  const TokState st = *u.st;
  int C, picks;
  tok_counts(seq_lens, unit, Hkv, Tmax, budget, C, picks);
  const float* row = scores + int64_t(unit) * Tmax;
  const int Wc = ceil_div(C, 32);
  const bool bucket = st.mode == kTokBucket;
  const int n = bucket ? int(st.n) : 0;
  const bool staged = n <= kTokStage;
  const bool one_window = Wc <= kTokWin;

  // window words [w0, w0 + kTokWin) of a bitmap into LDS; words >= Wc read as 0
  auto load_window = [&](const uint32_t* src, uint32_t* dst, int w0) {
#pragma unroll
    for (int m = 0; m < kTokWin / 4 / kSelectThreads; ++m) {
      const int k = (m * kSelectThreads + tid) * 4;
      const int w = w0 + k;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      // w < Wc <= W: the 4 words are inside the bitmap (its size is a multiple of 64)
      if (w < Wc) x = *reinterpret_cast<const uint4*>(src + w);
      dst[tok_pad(k)] = x.x;
      dst[tok_pad(k + 1)] = w + 1 < Wc ? x.y : 0u;
      dst[tok_pad(k + 2)] = w + 2 < Wc ? x.z : 0u;
      dst[tok_pad(k + 3)] = w + 3 < Wc ? x.w : 0u;
    }
  };
  // this thread's bucket bits of the window in wbk, and their number
  auto my_bucket_words = [&](uint32_t (&m)[kTokWpt]) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < kTokWpt; ++j) {
      m[j] = wbk[tok_pad(tid * kTokWpt + j)];
      c += __popc(m[j]);
    }
    return c;
  };

  // ---- list the bucket in token order (when it fits in LDS) ----------------
  int listed = 0;
  if (bucket && staged) {
    for (int w0 = 0; w0 < Wc; w0 += kTokWin) {
      load_window(u.bk, wbk, w0);
      __syncthreads();
      uint32_t m[kTokWpt];
      const int c = my_bucket_words(m);
      int tot;
      int off = listed + select_block_scan(c, lds, tot) - c;
#pragma unroll
      for (int j = 0; j < kTokWpt; ++j) {
        uint32_t b = m[j];
        while (b) {
          const int bit = __builtin_ctz(b);
          b &= b - 1;
          if (off < kTokStage) stok[off] = (w0 + tid * kTokWpt + j) * 32 + bit;
          ++off;
        }
      }
      listed += tot;
      if (!one_window) __syncthreads();  // the window buffer is reused
    }
    listed = min(listed, kTokStage);
    __syncthreads();
#pragma unroll 4
    for (int k = tid; k < listed; k += kSelectThreads) {
      const int t = stok[k];
      skey[k] = t < C ? score_key(row[t]) : 0u;  // t < C always
    }
    __syncthreads();
  }
  // calls f(key, token) for every bucket key; every thread must call it
  auto for_each = [&](auto&& f) {
    if (staged) {
      for (int k = tid; k < listed; k += kSelectThreads) f(skey[k], stok[k]);
    } else {
      for (int w0 = 0; w0 < Wc; w0 += kTokWin) {
        __syncthreads();
        load_window(u.bk, wbk, w0);
        __syncthreads();
        uint32_t m[kTokWpt];
        my_bucket_words(m);
        for (int j = 0; j < kTokWpt; ++j) {
          uint32_t b = m[j];
          while (b) {
            const int bit = __builtin_ctz(b);
            b &= b - 1;
            const int t = (w0 + tid * kTokWpt + j) * 32 + bit;
            if (t < C) f(score_key(row[t]), t);
          }
        }
      }
      __syncthreads();
    }
  };

  // ---- radix select of the r-th largest bucket key over its low 20 bits ----
  // (a 12-bit digit, then an 8-bit one)
  bool ge = false;
  uint32_t kb = 0;
  int r_eq = 0;
  if (bucket) {
    int r = int(st.r);
    uint32_t prefix = st.beta;
    int bits = 12;
    for (int level = 0; level < 2; ++level) {
      const int w = level == 0 ? 12 : 8;
      const int nb = 1 << w;
      const int shift = 32 - bits - w;
      for (int d = tid; d < nb; d += kSelectThreads) hist[d] = 0u;
      __syncthreads();
      for_each([&](uint32_t key, int) {
        if ((key >> (32 - bits)) == prefix) atomicAdd(&hist[(key >> shift) & uint32_t(nb - 1)], 1u);
      });
      __syncthreads();
      const int per = nb / kSelectThreads;  // 16 or 1 bins per thread, highest first
      int mine = 0;
      for (int j = 0; j < per; ++j) mine += int(hist[nb - 1 - (tid * per + j)]);
      if (tid == 0) {  // defined results even if no bin qualifies
        lds.beta = 0;
        lds.above = 0;
      }
      int total;
      int ab = select_block_scan(mine, lds, total) - mine;
      for (int j = 0; j < per; ++j) {
        const int d = nb - 1 - (tid * per + j);
        const int hd = int(hist[d]);
        if (ab < r && r <= ab + hd) {
          lds.beta = d;
          lds.above = ab;
        }
        ab += hd;
      }
      __syncthreads();
      const int beta = lds.beta;
      const int in_bucket = int(hist[beta]);
      r -= lds.above;
      prefix = (prefix << w) | uint32_t(beta);
      bits += w;
      __syncthreads();
      if (r == in_bucket) {  // the sub-bucket is taken whole
        ge = true;
        kb = bits == 32 ? prefix : prefix << (32 - bits);
        break;
      }
    }
    if (!ge) {
      kb = prefix;  // the exact boundary key; r of its ties are taken
      r_eq = max(0, min(r, n));
    }
  }

  // ---- compaction, window by window ---------------------------------------
  // A token is taken by key if its top digit is above the boundary digit, or
  // it is in the bucket with a key above kb (>= kb when ge); of the tokens tied
  // at kb the first r_eq in index order are taken. Its output position is the
  // number of tokens taken by key before it plus min(ties before it, r_eq).
  // With the bucket listed in LDS (in token order), each window's bucket
  // entries are one contiguous range of the list; its threads classify them
  // in parallel into the window's taken bitmap (wgt) and a tie bitmap (wbk,
  // free once the list is built). Otherwise each thread walks its own words'
  // bucket bits and reads their scores.
  int32_t* out = idx + int64_t(unit) * budget;
  int gt_run = 0, eq_run = 0;
  auto lower_bound = [&](int tok) {  // first list entry with token >= tok
    int lo = 0, hi = listed;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (stok[mid] < tok) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  for (int w0 = 0; w0 < Wc; w0 += kTokWin) {
    __syncthreads();
    load_window(u.gt, wgt, w0);
    if (bucket) {
      if (staged) {
        for (int k = tid; k < kTokWinPad; k += kSelectThreads) wbk[k] = 0u;
      } else {
        load_window(u.bk, wbk, w0);
      }
    }
    __syncthreads();
    if (bucket && staged) {
      const int lo = lower_bound(w0 * 32), hi = lower_bound((w0 + kTokWin) * 32);
      for (int k = lo + tid; k < hi; k += kSelectThreads) {
        const uint32_t key = skey[k];
        const int t = stok[k];
        const int wl = (t >> 5) - w0;  // in [0, kTokWin): t lies in this window
        const uint32_t bit = 1u << (t & 31);
        if (ge ? key >= kb : key > kb) atomicOr(&wgt[tok_pad(wl)], bit);
        else if (!ge && key == kb) atomicOr(&wbk[tok_pad(wl)], bit);
      }
      __syncthreads();
    }
    uint32_t tk[kTokWpt], te[kTokWpt];
    int ngt = 0, neq = 0;
    if (bucket && !staged) {
      uint32_t m[kTokWpt];
      my_bucket_words(m);
#pragma unroll
      for (int j = 0; j < kTokWpt; ++j) {
        uint32_t taken = wgt[tok_pad(tid * kTokWpt + j)], tie = 0u, b = m[j];
        while (b) {
          const int bit = __builtin_ctz(b);
          b &= b - 1;
          const int t = (w0 + tid * kTokWpt + j) * 32 + bit;
          const uint32_t key = t < C ? score_key(row[t]) : 0u;
          if (ge ? key >= kb : key > kb) taken |= 1u << bit;
          else if (!ge && key == kb) tie |= 1u << bit;
        }
        tk[j] = taken;
        te[j] = tie;
        ngt += __popc(taken);
        neq += __popc(tie);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kTokWpt; ++j) {
        tk[j] = wgt[tok_pad(tid * kTokWpt + j)];
        te[j] = bucket ? wbk[tok_pad(tid * kTokWpt + j)] : 0u;
        ngt += __popc(tk[j]);
        neq += __popc(te[j]);
      }
    }
    int win_gt, win_eq;
    const int gt_before = gt_run + select_block_scan(ngt, lds, win_gt) - ngt;
    int eq_seen = eq_run + select_block_scan(neq, lds, win_eq) - neq;
    int pos = gt_before + min(eq_seen, r_eq);
#pragma unroll
    for (int j = 0; j < kTokWpt; ++j) {
      uint32_t mm = tk[j] | te[j];
      while (mm) {
        const int bit = __builtin_ctz(mm);
        mm &= mm - 1;
        bool take = (tk[j] >> bit) & 1u;
        if (!take) {  // tied at kb
          take = eq_seen < r_eq;
          ++eq_seen;
        }
        if (take) {
          if (pos >= 0 && pos < budget) out[pos] = (w0 + tid * kTokWpt + j) * 32 + bit;
          ++pos;
        }
      }
    }
    gt_run += win_gt;
    eq_run += win_eq;
  }
  const int nsel = max(0, min(gt_run + min(eq_run, r_eq), budget));
  for (int k = nsel + tid; k < budget; k += kSelectThreads) out[k] = -1;
  if (tid == 0) count[unit] = nsel;
  // the unit's histogram back to zero for the next call (saves a launch)
  for (int d = tid; d < kTokBins; d += kSelectThreads) u.hist[d] = 0u;
}

}  // namespace

hipError_t launch_select_block(const UnitGeom& g, int budget, int n_tail, const float* scores,
                               const int32_t* seq_lens, int32_t* idx, int32_t* count,
                               hipStream_t s) {
  hipLaunchKernelGGL(select_block_kernel, dim3(g.B * g.Hkv), dim3(kSelectThreads), 0, s, scores,
                     seq_lens, g.Hkv, g.Tmax, g.NBmax, budget, n_tail, idx, count);
  return hipGetLastError();
}

size_t token_select_workspace(const UnitGeom& g) {
  return size_t(tok_geom(g.Tmax).unit_words) * 4 * size_t(g.B) * size_t(g.Hkv);
}

int64_t token_unit_words(const UnitGeom& g) { return tok_geom(g.Tmax).unit_words; }

hipError_t launch_select_token(const UnitGeom& g, int budget, const float* scores,
                               const int32_t* seq_lens, void* ws, int32_t* idx, int32_t* count,
                               hipStream_t s, bool hist_ready) {
  const TokGeom tg = tok_geom(g.Tmax);
  const int units = g.B * g.Hkv;
  const dim3 grid(ceil_div(g.Tmax, kTokChunk), units), block(kSelectThreads);
  if (!hist_ready)
    hipLaunchKernelGGL(tok_hist_kernel, grid, block, 0, s, scores, seq_lens, g.Hkv, g.Tmax, budget,
                       tg, ws);
  hipLaunchKernelGGL(tok_filter_kernel, grid, block, 0, s, scores, seq_lens, g.Hkv, g.Tmax, budget,
                     tg, ws);
  hipLaunchKernelGGL(tok_finish_kernel, dim3(units), block, 0, s, scores, g.Tmax, seq_lens, g.Hkv,
                     budget, tg, ws, idx, count);
  return hipGetLastError();
}

}  // namespace bsa
