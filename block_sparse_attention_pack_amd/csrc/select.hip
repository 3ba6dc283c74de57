// Top-k selection per unit (Jet-QSparse abstract: top blocks per KV head;
// JSSA Figure 1 and Table 15: top-B tokens per KV head, shared by the group).
//
// Block mode: one 256-thread work-group per unit runs select_unit_rows
// (select_core.hpp); a unit has at most max_tokens/128 candidates.
//
// Token mode: a unit has up to max_tokens candidates (131072 at 128K context),
// too many for one work-group to read fast. Budgets up to 2048 at up to 131072
// tokens take the one-launch select of tokselect.hip (then topp below, with
// the adaptive budget). Otherwise the selection is spread over kTokChunk-key
// chunks, one work-group each, in three launches (four with the adaptive
// budget):
//   hist    every group adds the histogram of its keys' top 12 bits (of the
//           order-preserving key) to its unit's, with device-scope atomics
//           (the histogram is zero on entry: the finish of the previous call
//           leaves it so); skipped when the token scan has already counted
//           them (bsa_score_select, bsa_decode_step);
//   filter  every group finds from that histogram the top digit beta that
//           holds the picks-th largest key and writes two bitmaps of its keys:
//           those with a larger top digit (taken), and those with top digit
//           beta (the bucket: usually about 1% of the keys);
//   finish  one group per chunk lists the bucket's keys, finds the exact
//           boundary key among them (radix select over the remaining 20 bits)
//           and writes its chunk's taken tokens in index order (those above
//           the boundary key, and of its ties the lowest indices) at offsets
//           counted from the bitmaps below the chunk; the groups share
//           returning the unit's histogram to zero;
//   topp    (only with top_p > 0, the adaptive budget) one group per unit
//           keeps the shortest top-ranked prefix of that selection whose
//           softmax shares reach top_p, from per-chunk partials the filter
//           then also stores.
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
constexpr int kTokChunkWords = kTokChunk / 32;
constexpr int kTokWin = 4096;     // bitmap words per finish window: 16 per thread
constexpr int kTokList = 4096;    // buckets up to this size are listed in LDS by the finish

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

// Per-unit workspace: histogram, state slot and two bitmaps, each on its own
// 256-byte boundary. The slot holds TokState and, from word kTokLseWord, three
// words per chunk that the filter leaves for the adaptive budget (the chunk's
// score maximum, its sum of exp(s - maximum), its count of +inf scores).
constexpr int kTokLseWord = 8;

struct TokGeom {
  int W;               // 32-bit bitmap words per unit (a multiple of 2)
  int chunks;          // kTokChunk-key chunks per unit
  int slot;            // words of the state slot
  int64_t w_bitmap;    // words reserved per bitmap
  int64_t unit_words;  // workspace words per unit
};

__host__ __device__ inline TokGeom tok_geom(int Tmax) {
  TokGeom t;
  t.W = ceil_div(Tmax, 64) * 2;
  t.chunks = ceil_div(Tmax, kTokChunk);
  t.slot = (kTokLseWord + 3 * t.chunks + 63) / 64 * 64;
  t.w_bitmap = (int64_t(t.W) + 63) / 64 * 64;
  t.unit_words = kTokBins + t.slot + 2 * t.w_bitmap;
  return t;
}

struct TokUnit {
  uint32_t* hist;
  TokState* st;
  uint32_t* lse;  // [chunks][3]: maximum (float bits), sum (float bits), +inf count
  uint32_t* gt;   // bit t: token t taken by its top digit
  uint32_t* bk;   // bit t: token t in the bucket
};

__device__ __forceinline__ TokUnit tok_unit(void* ws, const TokGeom& t, int unit) {
  uint32_t* base = static_cast<uint32_t*>(ws) + int64_t(unit) * t.unit_words;
  TokUnit u;
  u.hist = base;
  u.st = reinterpret_cast<TokState*>(base + kTokBins);
  u.lse = base + kTokBins + kTokLseWord;
  u.gt = base + kTokBins + t.slot;
  u.bk = u.gt + t.w_bitmap;
  return u;
}

__device__ __forceinline__ void tok_counts(const int32_t* seq_lens, int unit, int Hkv, int Tmax,
                                           int budget, int& C, int& picks) {
  C = clamp_len(seq_lens[unit / Hkv], Tmax);
  picks = max(0, min(budget, C));
}

// Histogram of the top 12 key bits of the unit's candidates.
// grid (B * Hkv, ceil(Tmax / kTokChunk)), 256 threads.
__global__ __launch_bounds__(kSelectThreads) void tok_hist_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int budget, TokGeom tg, void* ws) {
  __shared__ uint32_t hist[kTokBins];
  const int unit = blockIdx.x, tid = threadIdx.x;
  int C, picks;
  tok_counts(seq_lens, unit, Hkv, Tmax, budget, C, picks);
  const int base = blockIdx.y * kTokChunk;
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

// Merges a (maximum, sum of exp(x - maximum)) pair into another.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mx = fmaxf(m, m2);
  if (mx == -__builtin_inff()) {
    m = mx;
    s = 0.0f;
    return;
  }
  s = s * expf(m - mx) + s2 * expf(m2 - mx);
  m = mx;
}

// Bitmaps of the keys taken by their top digit and of the bucket (keys whose
// top digit is the boundary digit). grid (B * Hkv, ceil(Tmax / kTokChunk)),
// 256 threads; wave w owns the 4096 keys from blockIdx.y * kTokChunk + 4096 w,
// as 64 rows of 64; lane j keeps row j's two words of each bitmap, so each
// bitmap is written with one 8-byte store per lane.
// LSE: also store the chunk's softmax partial (for the adaptive budget).
template <bool LSE>
__global__ __launch_bounds__(kSelectThreads) void tok_filter_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int budget, TokGeom tg, void* ws) {
  constexpr int kRows = kTokChunk / kSelectThreads;
  static_assert(kRows == kWave, "one 64-key row per lane");
  __shared__ SelectLds lds;
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const TokUnit u = tok_unit(ws, tg, unit);
  int C, picks;
  tok_counts(seq_lens, unit, Hkv, Tmax, budget, C, picks);
  uint32_t mode = picks == 0 ? kTokNone : (picks == C ? kTokAll : kTokBucket);
  const float* row = scores + int64_t(unit) * Tmax;
  const int wbase = blockIdx.y * kTokChunk + wave * kRows * 64;
  // the keys are loaded before the boundary is known, so their latency
  // overlaps the histogram reads
  float v[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    const int i = wbase + j * 64 + lane;
    v[j] = ((mode == kTokBucket || LSE) && i < C) ? row[i] : 0.0f;
  }
  int beta = 0, above = 0, in = 0;
  if (mode == kTokBucket) {
    tok_boundary(u.hist, picks, lds, beta, above, in);
    if (picks - above == in) mode = kTokGe;
  }
  if (blockIdx.y == 0 && tid == 0) {
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
  if constexpr (LSE) {  // the chunk's softmax partial for the adaptive budget
    // branch-free: the lane's maximum over its finite scores, then its sum
    float m = -__builtin_inff(), sm = 0.0f;
    int ninf = 0;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const float x = v[j];
      const bool in = wbase + j * 64 + lane < C;
      ninf += (in && x == __builtin_inff()) ? 1 : 0;
      m = (in && x < __builtin_inff()) ? fmaxf(m, x) : m;  // fmaxf drops NaN
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const float x = v[j];
      const bool fin = wbase + j * 64 + lane < C && x > -__builtin_inff() && x < __builtin_inff();
      const float e = expf(x - m);
      sm += fin ? e : 0.0f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(m, off, kWave), s2 = __shfl_xor(sm, off, kWave);
      lse_merge(m, sm, m2, s2);
      ninf += __shfl_xor(ninf, off, kWave);
    }
    if (lane == 0) {
      lds.wave_lo[wave] = __builtin_bit_cast(uint32_t, m);
      lds.wave_hi[wave] = __builtin_bit_cast(uint32_t, sm);
      lds.wave_tot[wave] = ninf;
    }
    __syncthreads();
    if (tid == 0) {
      float M = __builtin_bit_cast(float, lds.wave_lo[0]);
      float S = __builtin_bit_cast(float, lds.wave_hi[0]);
      int NI = lds.wave_tot[0];
      for (int w = 1; w < kSelectThreads / kWave; ++w) {
        lse_merge(M, S, __builtin_bit_cast(float, lds.wave_lo[w]),
                  __builtin_bit_cast(float, lds.wave_hi[w]));
        NI += lds.wave_tot[w];
      }
      uint32_t* p = u.lse + 3 * blockIdx.y;
      p[0] = __builtin_bit_cast(uint32_t, M);
      p[1] = __builtin_bit_cast(uint32_t, S);
      p[2] = uint32_t(NI);
    }
  }
}

// Sums of N ints over the work-group (red: N ints per wave of LDS, used once).
template <int N>
__device__ __forceinline__ void tok_block_sum(int (&v)[N], int (*red)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < N; ++k) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off, kWave);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) red[wave][k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < kSelectThreads / kWave; ++w) t += red[w][k];
    v[k] = t;
  }
}

// A window of kTokWin bitmap words from word w0: thread t holds the 16 words
// tok_word(w0, j) (four aligned groups of 4, the groups of a wave adjacent in
// memory); words >= Wc read as 0. Every load is issued (at an address clamped
// to the last 4-word group holding a word < Wc, which lies inside the bitmap)
// and masked afterwards, so the loads of a window are all in flight together.
__device__ __forceinline__ int tok_word(int w0, int j) {
  return w0 + (j >> 2) * (kTokWin / 4) + 4 * int(threadIdx.x) + (j & 3);
}
__device__ __forceinline__ void tok_window(const uint32_t* src, int w0, int Wc,
                                           uint32_t (&m)[16]) {
  const int last = (Wc - 1) & ~3;  // Wc >= 1 here
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int w = tok_word(w0, 4 * q);
    const uint4 x = *reinterpret_cast<const uint4*>(src + min(w, last));
    m[4 * q] = w < Wc ? x.x : 0u;
    m[4 * q + 1] = w + 1 < Wc ? x.y : 0u;
    m[4 * q + 2] = w + 2 < Wc ? x.z : 0u;
    m[4 * q + 3] = w + 3 < Wc ? x.w : 0u;
  }
}

// The bin of a histogram of nb bins (nb / 256 per thread, highest first) that
// holds the r-th largest entry: d, and the count above it. Defined (0, 0) when
// no bin does. Synchronises the group.
__device__ __forceinline__ void tok_bin_of_rank(const uint32_t* hist, int nb, int r,
                                                SelectLds& lds, int& d_out, int& above_out) {
  const int tid = threadIdx.x;
  const int per = nb / kSelectThreads;
  int mine = 0;
  for (int j = 0; j < per; ++j) mine += int(hist[nb - 1 - (tid * per + j)]);
  if (tid == 0) {  // ordered before the writes below by the scan's barriers
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
  d_out = lds.beta;
  above_out = lds.above;
}

// Resolve the bucket and compact the taken tokens in index order.
// grid (B * Hkv, chunks), 256 threads: work-group c writes the output entries
// of chunk c's tokens (thread t owns the chunk's bitmap words 2t, 2t + 1).
// Every group of a unit first lists the bucket (keys and token indices) in LDS
// when it holds at most kTokList keys, and finds the boundary key kb by a
// radix select over the bucket's keys (their low 20 bits: a 12-bit digit, then
// an 8-bit one); a larger bucket is walked in the bitmap, with its scores read
// from memory, each time it is needed. A token is taken by key if its top
// digit is above the boundary digit (the taken bitmap), or it is in the bucket
// with a key above kb (>= kb when the 12-bit sub-bucket is taken whole); of the
// tokens tied at kb the first r_eq in index order are taken. Its output
// position is the number of tokens taken by key before it plus min(ties before
// it, r_eq); the counts before the chunk come from the taken bitmap's words
// below it and the bucket's keys below it. Group 0 also pads the output and
// writes the count; the groups share returning the histogram to zero.
__global__ __launch_bounds__(kSelectThreads) void tok_finish_kernel(
    const float* __restrict__ scores, int Tmax, const int32_t* __restrict__ seq_lens, int Hkv,
    int budget, TokGeom tg, void* ws, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ uint32_t skey[kTokList];
  __shared__ int32_t stok[kTokList];
  __shared__ uint32_t hist[kTokBins];   // the 12-bit digit below beta
  __shared__ uint32_t hist2[256];       // the last 8 bits
  __shared__ uint32_t wtk[kTokChunkWords], wte[kTokChunkWords];
  __shared__ int red[kSelectThreads / kWave][6];
  __shared__ SelectLds lds;
  const int unit = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
  const TokUnit u = tok_unit(ws, tg, unit);
  int C, picks;
  tok_counts(seq_lens, unit, Hkv, Tmax, budget, C, picks);
  const int cs = chunk * kTokChunk;  // the chunk's first token
  // the histogram is not read here (the filter has read it): clear it now
  for (int d = chunk * kSelectThreads + tid; d < kTokBins; d += int(gridDim.y) * kSelectThreads)
    u.hist[d] = 0u;
  if (chunk > 0 && cs >= C) return;  // no tokens here; group 0 always continues
  const float* row = scores + int64_t(unit) * Tmax;
  const int Wc = ceil_div(C, 32);
  const int w0 = chunk * kTokChunkWords + 2 * tid;  // this thread's two chunk words
  uint32_t tk[2], cb[2];  // their taken and bucket bits
  {
    const int wl = Wc > 0 ? min(w0, (Wc - 1) & ~1) : 0;  // even; a valid pair of words
    const uint2 x = *reinterpret_cast<const uint2*>(u.gt + wl);
    const uint2 y = *reinterpret_cast<const uint2*>(u.bk + wl);
    tk[0] = w0 < Wc ? x.x : 0u;
    tk[1] = w0 + 1 < Wc ? x.y : 0u;
    cb[0] = w0 < Wc ? y.x : 0u;
    cb[1] = w0 + 1 < Wc ? y.y : 0u;
  }
  const TokState st = *u.st;
  for (int d = tid; d < kTokBins; d += kSelectThreads) hist[d] = 0u;
  hist2[tid] = 0u;
  wtk[2 * tid] = wtk[2 * tid + 1] = 0u;
  wte[2 * tid] = wte[2 * tid + 1] = 0u;
  const bool bucket = st.mode == kTokBucket;
  const int n = bucket ? int(st.n) : 0;
  const bool listed = bucket && n <= kTokList;
  const uint32_t beta = st.beta;
  __syncthreads();

  // ---- taken-by-digit counts (before the chunk, all); the bucket listed ----
  // sums: 0, 1: taken by top digit (before the chunk, in all); 2, 3: bucket
  // keys taken by key (likewise); 4, 5: ties at kb (likewise)
  int sums[6] = {0, 0, 0, 0, 0, 0};
  int nlist = 0;  // bucket entries listed so far (in token order)
  for (int v0 = 0; v0 < Wc; v0 += kTokWin) {
    uint32_t g[16], m[16];
    tok_window(u.gt, v0, Wc, g);
    tok_window(u.bk, v0, Wc, m);
    int mine = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int x = __popc(g[j]);
      sums[1] += x;
      sums[0] += tok_word(v0, j) < chunk * kTokChunkWords ? x : 0;
      mine += __popc(m[j]);
    }
    if (listed) {  // uniform: every thread takes part in the scan
      int tot;
      int k = nlist + select_block_scan(mine, lds, tot) - mine;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        uint32_t b = m[j];
        while (b) {
          const int bit = __builtin_ctz(b);
          b &= b - 1;
          if (k < kTokList) stok[k] = tok_word(v0, j) * 32 + bit;
          ++k;
        }
      }
      nlist += tot;
    }
  }
  // calls f(key, token) for every bucket key (no barriers)
  int nl = 0;
  auto for_each = [&](auto&& f) {
    if (listed) {
      for (int k = tid; k < nl; k += kSelectThreads) f(skey[k], stok[k]);
    } else {
      for (int v0 = 0; v0 < Wc; v0 += kTokWin) {
        uint32_t m[16];
        tok_window(u.bk, v0, Wc, m);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          uint32_t b = m[j];
          while (b) {
            const int bit = __builtin_ctz(b);
            b &= b - 1;
            const int t = tok_word(v0, j) * 32 + bit;
            if (t < C) f(score_key(row[t]), t);
          }
        }
      }
    }
  };
  auto count1 = [&](uint32_t key) { atomicAdd(&hist[(key >> 8) & uint32_t(kTokBins - 1)], 1u); };

  // ---- the bucket's keys (listed: gathered), counted by their next 12 bits ----
  if (listed) {
    __syncthreads();
    nl = min(nlist, kTokList);
#pragma unroll 4
    for (int k = tid; k < nl; k += kSelectThreads) {
      const int t = stok[k];
      const uint32_t key = uint32_t(t) < uint32_t(C) ? score_key(row[t]) : 0u;  // always inside
      skey[k] = key;
      count1(key);
    }
  } else if (bucket) {
    for_each([&](uint32_t key, int) { count1(key); });
  }

  // ---- radix select of the r-th largest bucket key over its low 20 bits ----
  bool ge = false;
  uint32_t kb = 0;
  int r_eq = 0;
  if (bucket) {
    __syncthreads();
    int r = int(st.r), d1, ab1;
    tok_bin_of_rank(hist, kTokBins, r, lds, d1, ab1);
    r -= ab1;
    const uint32_t p1 = (beta << 12) | uint32_t(d1);  // the key's top 24 bits
    if (r == int(hist[d1])) {  // the sub-bucket is taken whole
      ge = true;
      kb = p1 << 8;
    } else {
      for_each([&](uint32_t key, int) {
        if ((key >> 8) == p1) atomicAdd(&hist2[key & 255u], 1u);
      });
      __syncthreads();
      int d2, ab2;
      tok_bin_of_rank(hist2, 256, r, lds, d2, ab2);
      kb = (p1 << 8) | uint32_t(d2);  // the exact boundary key; r of its ties are taken
      r_eq = max(0, min(r - ab2, n));
    }
  }
  auto by_key = [&](uint32_t key) { return ge ? key >= kb : key > kb; };
  auto tied = [&](uint32_t key) { return !ge && key == kb; };

  // ---- bucket counts before the chunk, and the chunk's bucket bits ----------
  if (bucket) {
    for_each([&](uint32_t key, int t) {
      const bool bk = by_key(key), te = tied(key);
      sums[2] += bk && t < cs ? 1 : 0;
      sums[3] += bk ? 1 : 0;
      sums[4] += te && t < cs ? 1 : 0;
      sums[5] += te ? 1 : 0;
      if (listed && t >= cs && t < cs + kTokChunk && (bk || te)) {
        const int wl = (t - cs) >> 5;
        atomicOr(bk ? &wtk[wl] : &wte[wl], 1u << (t & 31));
      }
    });
  }
  tok_block_sum(sums, red);  // also orders the bit marks above before the reads below
  int32_t* out = idx + int64_t(unit) * budget;
  if (chunk == 0) {
    const int nsel = max(0, min(sums[1] + sums[3] + min(sums[5], r_eq), budget));
    for (int k = nsel + tid; k < budget; k += kSelectThreads) out[k] = -1;
    if (tid == 0) count[unit] = nsel;
  }
  uint32_t te[2] = {0u, 0u};
  if (listed) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      tk[j] |= wtk[2 * tid + j];
      te[j] = wte[2 * tid + j];
    }
  } else if (bucket) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t b = cb[j];
      while (b) {
        const int bit = __builtin_ctz(b);
        b &= b - 1;
        const int t = (w0 + j) * 32 + bit;
        if (t >= C) continue;
        const uint32_t key = score_key(row[t]);
        if (by_key(key)) tk[j] |= 1u << bit;
        else if (tied(key)) te[j] |= 1u << bit;
      }
    }
  }

  // ---- positions and writes --------------------------------------------------
  const int own_gt = __popc(tk[0]) + __popc(tk[1]), own_eq = __popc(te[0]) + __popc(te[1]);
  int ngt = own_gt, neq = own_eq, tot_gt, tot_eq;
  select_block_scan2(ngt, neq, lds, tot_gt, tot_eq);  // inclusive
  int eq_seen = sums[4] + neq - own_eq;
  int pos = sums[0] + sums[2] + ngt - own_gt + min(eq_seen, r_eq);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
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
        if (pos >= 0 && pos < budget) out[pos] = (w0 + j) * 32 + bit;
        ++pos;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Adaptive budget (top-p retrieval, RaBitQCache abstract): of the unit's
// selection (its `budget` best tokens, ascending), keep the fewest top-ranked
// ones whose softmax shares over all candidates t < L reach top_p. A share is
// exp(s_t - max) / sum_u exp(s_u - max); NaN and -inf weigh nothing; if any
// score is +inf, the +inf candidates share the whole mass. With no weight at
// all the selection stays whole.
// grid (B * Hkv), kTopPThreads threads. The group merges the unit's total
// weight from the filter's per-chunk partials (maximum, rescaled sum, +inf
// count). Each selected token's weight is taken in fixed point (2^40 units,
// so every sum below is an exact integer, whatever its order), and the cut is
// found without sorting: a radix search over the 32-bit score keys, 8 bits a
// level, keeps the bin whose running weight (from the top) first reaches
// top_p times the total; at the boundary key, whose ties weigh the same,
// as many ties as needed are kept in index order.
// ---------------------------------------------------------------------------
constexpr int kTopPThreads = 1024;
constexpr int kTopPPer = kTopPMaxBudget / kTopPThreads;  // entries per thread (contiguous)
constexpr double kTopPFix = 1099511627776.0;               // 2^40

__global__ __launch_bounds__(kTopPThreads) void tok_topp_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int budget, float top_p, TokGeom tg, void* ws, int32_t* __restrict__ idx,
    int32_t* __restrict__ count) {
  __shared__ unsigned long long ew[kTopPMaxBudget];  // fixed-point weight by position
  __shared__ uint32_t ekey[kTopPMaxBudget];          // score key by position
  __shared__ int32_t tok[kTopPMaxBudget];            // token by position
  __shared__ unsigned long long hsum[256];
  __shared__ unsigned long long wtot[kTopPThreads / kWave];
  __shared__ float red_m[kTopPThreads / kWave], red_s[kTopPThreads / kWave];
  __shared__ int red_i[kTopPThreads / kWave];
  __shared__ unsigned long long sel_above, tie_w;
  __shared__ int sel_d, n_above, n_tie;
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kTopPThreads / kWave;
  const int C = clamp_len(seq_lens[unit / Hkv], Tmax);
  const float* row = scores + int64_t(unit) * Tmax;
  int32_t* out = idx + int64_t(unit) * budget;
  const int n = min(max(count[unit], 0), min(budget, kTopPMaxBudget));
  if (n == 0 || C <= 0) return;  // the group exits as one (n > 0 implies C > 0)

  // ---- the unit's total weight: the filter's per-chunk partials, merged ----
  const TokUnit u = tok_unit(ws, tg, unit);
  float m = -__builtin_inff(), s = 0.0f;
  int ninf = 0;
  for (int c = tid; c < tg.chunks; c += kTopPThreads) {
    const uint32_t* p = u.lse + 3 * c;
    lse_merge(m, s, __builtin_bit_cast(float, p[0]), __builtin_bit_cast(float, p[1]));
    ninf += int(p[2]);
  }
  // the wave's merge, complete in lane 63 (an empty partner is (-inf, 0))
  wave_dpp_steps([&](auto step) {
    const float m2 = __int_as_float(dpp_move(__float_as_int(-__builtin_inff()), __float_as_int(m), step));
    const float s2 = __int_as_float(dpp_move(0, __float_as_int(s), step));
    lse_merge(m, s, m2, s2);
    ninf += dpp_move(0, ninf, step);
  });
  if (lane == kWave - 1) {
    red_m[wave] = m;
    red_s[wave] = s;
    red_i[wave] = ninf;
  }
  // ---- the selection into LDS (its scores kept in registers) ----------------
  float x[kTopPPer];
#pragma unroll
  for (int j = 0; j < kTopPPer; ++j) {
    const int k = tid * kTopPPer + j;
    x[j] = __builtin_nanf("");
    if (k < n) {
      const int t = out[k];
      if (uint32_t(t) < uint32_t(C)) x[j] = row[t];
      tok[k] = t;
      ekey[k] = score_key(x[j]);
    }
  }
  if (tid < 256) hsum[tid] = 0ull;
  if (tid == 0) {
    n_above = 0;
    n_tie = 0;
    tie_w = 0ull;
    sel_d = -1;
  }
  __syncthreads();
  m = red_m[0];
  s = red_s[0];
  ninf = red_i[0];
  for (int w = 1; w < kWaves; ++w) {
    lse_merge(m, s, red_m[w], red_s[w]);
    ninf += red_i[w];
  }
  __syncthreads();  // red_i is reused below
  const bool inf_mode = ninf > 0;
  const float z = inf_mode ? float(ninf) : s;
  int mcut = n;
  uint32_t kappa = 0;  // the boundary key
  int j_tie = 0;       // ties at kappa kept
  if (z > 0.0f && z < __builtin_inff()) {  // uniform
    const unsigned long long thr =
        static_cast<unsigned long long>(ceil(double(top_p) * double(z) * kTopPFix));
#pragma unroll
    for (int j = 0; j < kTopPPer; ++j) {
      const int k = tid * kTopPPer + j;
      if (k < n) {
        const float w = inf_mode ? (x[j] == __builtin_inff() ? 1.0f : 0.0f)
                                 : ((x[j] == x[j] && x[j] > -__builtin_inff()) ? expf(x[j] - m)
                                                                               : 0.0f);
        ew[k] = static_cast<unsigned long long>(double(w) * kTopPFix);
      }
    }
    // ---- radix search for the boundary key, 8 bits a level ------------------
    uint32_t prefix = 0;
    unsigned long long above = 0ull;
    bool found = true;
    for (int level = 0; level < 4 && found; ++level) {
      const int shift = 24 - 8 * level;
      if (level > 0) {
        if (tid < 256) hsum[tid] = 0ull;
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < kTopPPer; ++j) {
        const int k = tid * kTopPPer + j;
        if (k < n) {
          const uint32_t key = ekey[k];
          if (level == 0 || (key >> (shift + 8)) == prefix)
            atomicAdd(&hsum[(key >> shift) & 255u], ew[k]);
        }
      }
      __syncthreads();
      // bins from the highest: the one where the running weight reaches thr
      unsigned long long v = 0ull, incl = 0ull;
      if (tid < 256) {
        v = hsum[255 - tid];
        incl = v;
        // inclusive 64-bit scan: both halves move by DPP, the sum carries
        wave_dpp_steps([&](auto step) {
          const uint32_t lo = uint32_t(dpp_move(0, int(uint32_t(incl)), step));
          const uint32_t hi = uint32_t(dpp_move(0, int(uint32_t(incl >> 32)), step));
          incl += (uint64_t(hi) << 32) | lo;
        });
        if (lane == kWave - 1) wtot[wave] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        unsigned long long before = incl - v;
        for (int w2 = 0; w2 < wave; ++w2) before += wtot[w2];
        if (above + before < thr && thr <= above + before + v) {
          sel_d = 255 - tid;
          sel_above = above + before;
        }
      }
      __syncthreads();
      found = sel_d >= 0;  // uniform; none at level 0: the selection's weight stays below thr
      if (found) {
        prefix = (prefix << 8) | uint32_t(sel_d);
        above = sel_above;
      }
      __syncthreads();  // every thread has read sel_d before it is reset
      if (tid == 0) sel_d = -1;
    }
    if (found) {
      kappa = prefix;
      // entries above kappa, and the ties at kappa (equal weights)
#pragma unroll
      for (int j = 0; j < kTopPPer; ++j) {
        const int k = tid * kTopPPer + j;
        if (k < n) {
          if (ekey[k] > kappa) atomicAdd(&n_above, 1);
          else if (ekey[k] == kappa) {
            atomicAdd(&n_tie, 1);
            tie_w = ew[k];  // every tie writes the same value
          }
        }
      }
      __syncthreads();
      const unsigned long long need = thr - above, wk = tie_w;  // need > 0
      int jt = wk > 0 ? int(min((need + wk - 1) / wk, (unsigned long long)n_tie)) : n_tie;
      j_tie = max(jt, 1);
      mcut = min(n_above + j_tie, n);
    }
  }

  // ---- keep the top mcut, compacted in token order ---------------------------
  // kept: keys above kappa, and the first j_tie ties at kappa by position
  // (everything when no cut was made)
  const bool cutting = mcut < n || j_tie > 0;
  int tie_mine = 0;
#pragma unroll
  for (int j = 0; j < kTopPPer; ++j) {
    const int k = tid * kTopPPer + j;
    tie_mine += (cutting && k < n && ekey[k] == kappa) ? 1 : 0;
  }
  const int tincl = wave_scan_dpp(tie_mine);
  if (lane == kWave - 1) red_i[wave] = tincl;
  __syncthreads();
  int tie_rank = tincl - tie_mine;
  for (int w2 = 0; w2 < wave; ++w2) tie_rank += red_i[w2];
  bool keep[kTopPPer];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kTopPPer; ++j) {
    const int k = tid * kTopPPer + j;
    bool kp = k < n;
    if (cutting && kp) {
      const uint32_t key = ekey[k];
      if (key == kappa) kp = tie_rank++ < j_tie;
      else kp = key > kappa;
    }
    keep[j] = kp;
    mine += kp ? 1 : 0;
  }
  const int incl = wave_scan_dpp(mine);
  __syncthreads();  // red_i is reused
  if (lane == kWave - 1) red_i[wave] = incl;
  __syncthreads();
  int pos = incl - mine;
  for (int w2 = 0; w2 < wave; ++w2) pos += red_i[w2];
#pragma unroll
  for (int j = 0; j < kTopPPer; ++j) {
    const int k = tid * kTopPPer + j;
    if (keep[j]) out[pos++] = tok[k];
  }
  int total = 0;
  for (int w2 = 0; w2 < kWaves; ++w2) total += red_i[w2];
  for (int k = total + tid; k < n; k += kTopPThreads) out[k] = -1;
  if (tid == 0) count[unit] = total;
}

}  // namespace

hipError_t launch_select_block(const UnitGeom& g, int budget, int n_tail, const float* scores,
                               const int32_t* seq_lens, int32_t* idx, int32_t* count,
                               hipStream_t s) {
  hipLaunchKernelGGL(select_block_kernel, dim3(g.B * g.Hkv), dim3(kSelectThreads), 0, s, scores,
                     seq_lens, g.Hkv, g.Tmax, g.NBmax, budget, n_tail, idx, count);
  return hipGetLastError();
}

// The chunked select's region (tok_geom words per unit), then, where the
// one-group select applies, its region.
size_t token_select_workspace(const UnitGeom& g, int budget, float top_p) {
  return size_t(tok_geom(g.Tmax).unit_words) * 4 * size_t(g.B) * size_t(g.Hkv) +
         (token_select_one_group(g, budget, top_p) ? token_select_one_workspace(g) : 0);
}

int64_t token_unit_words(const UnitGeom& g) { return tok_geom(g.Tmax).unit_words; }

hipError_t launch_select_token(const UnitGeom& g, int budget, const float* scores,
                               const int32_t* seq_lens, void* ws, int32_t* idx, int32_t* count,
                               hipStream_t s, bool hist_ready, float top_p) {
  const TokGeom tg = tok_geom(g.Tmax);
  const int units = g.B * g.Hkv;
  if (!hist_ready && token_select_one_group(g, budget, top_p)) {
    // with the adaptive budget its softmax partials go where the filter leaves
    // them (the chunked region's slots), and tok_topp follows
    uint32_t* w32 = static_cast<uint32_t*>(ws);
    const hipError_t e = launch_select_token_one(
        g, budget, scores, seq_lens, w32 + tg.unit_words * int64_t(units), idx, count,
        top_p > 0.0f ? w32 + kTokBins + kTokLseWord : nullptr, tg.unit_words, s);
    if (e == hipSuccess && top_p > 0.0f)
      hipLaunchKernelGGL(tok_topp_kernel, dim3(units), dim3(kTopPThreads), 0, s, scores, seq_lens,
                         g.Hkv, g.Tmax, budget, top_p, tg, ws, idx, count);
    return e == hipSuccess ? hipGetLastError() : e;
  }
  // the chunks of a unit share their unit's reads (histogram, bitmaps,
  // bucket scores): consecutive work-group ids are spread over the XCDs, so a
  // unit's groups are kept units apart to land on one XCD and its L2
  const dim3 grid(units, ceil_div(g.Tmax, kTokChunk)), block(kSelectThreads);
  if (!hist_ready)
    hipLaunchKernelGGL(tok_hist_kernel, grid, block, 0, s, scores, seq_lens, g.Hkv, g.Tmax, budget,
                       tg, ws);
  if (top_p > 0.0f)
    hipLaunchKernelGGL(tok_filter_kernel<true>, grid, block, 0, s, scores, seq_lens, g.Hkv, g.Tmax,
                       budget, tg, ws);
  else
    hipLaunchKernelGGL(tok_filter_kernel<false>, grid, block, 0, s, scores, seq_lens, g.Hkv,
                       g.Tmax, budget, tg, ws);
  hipLaunchKernelGGL(tok_finish_kernel, grid, block, 0, s, scores, g.Tmax, seq_lens, g.Hkv,
                     budget, tg, ws, idx, count);
  if (top_p > 0.0f)
    hipLaunchKernelGGL(tok_topp_kernel, dim3(units), dim3(kTopPThreads), 0, s, scores, seq_lens,
                       g.Hkv, g.Tmax, budget, top_p, tg, ws, idx, count);
  return hipGetLastError();
}

}  // namespace bsa
