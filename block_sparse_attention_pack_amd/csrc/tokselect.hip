// Top-B token selection per unit in one launch (JSSA Figure 1 and Table 15:
// the top-B tokens per KV head, shared by the group's query heads).
//
// Grid (unit, chunk of kTsChunk tokens), 1024 threads. Every work-group of a
// unit:
//   1. Threshold. With more than kTsCap candidates, a fixed sample of
//      kTsSample scores at evenly spaced tokens of the unit is ranked (radix
//      select in registers; every group of the unit computes the same T), and
//      T is the sample's key of rank r_s = ceil(5 picks S / (2 C)) + 8: about
//      2.5 picks + 8 C / S tokens have a key >= T. At 128K tokens and 2048
//      picks, r_s = 48 of S = 1024: T lies above the picks-th largest key only
//      if 48 sampled keys fall in the row's top 1.6% (16 expected), and the
//      list overflows only if fewer than 48 fall in its top 12.5% (128
//      expected). With at most kTsCap candidates, T = 0 and every candidate
//      is listed.
//   2. Listing. The chunk's keys >= T go to the chunk's list in the workspace
//      (key, token) with its count, staged in LDS and written with dense
//      stores.
// The unit's last group to arrive (an arrival counter, as the attention's
// merge uses) then:
//   3. finds the exact key kappa of the picks-th largest listed key by a radix
//      select over the list held in registers (the block select's procedure
//      over a 1024-thread group), and how many of its ties are taken;
//   4. sets a bit in an LDS "taken" bitmap of the unit's tokens for each
//      listed key above kappa, one in a "tied" bitmap for each key equal to
//      it, and writes the taken tokens and the lowest-index ties ascending in
//      one pass over the bitmap words (two block scans).
// With the adaptive budget, every group also leaves its two 16384-token
// halves' softmax partials for tok_topp, which then cuts the selection.
// If the lists hold fewer than picks or more than kTsCap candidates, or a chunk
// more than kTsChunkCap (a sample far from the unit's distribution, or many
// equal keys), steps 3 and 4 run over the unit's scores in memory instead: the
// same result, with one read of the scores per radix pass. The last group
// returns the counter to zero, so the workspace is ready for the next call.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kTsThreads = 1024;
constexpr int kTsWaves = kTsThreads / kWave;
constexpr int kTsCap = 16384;    // listed candidates
constexpr int kTsSample = 1024;  // sampled keys (one per thread)
constexpr int kTsPer = kTsCap / kTsThreads;
constexpr int kTsBatch = 8;      // 16-byte loads in flight per thread (fallback passes)
constexpr int kTsChunk = 32768;  // tokens listed per work-group

// A group's listed keys and tokens are staged in the bitmaps' words (used only
// by the unit's last group, after every group has stored its list), so the
// global list is written with dense stores.
constexpr int kTsStage = kTokSelectMaxTokens / 32;

struct TsLds {
  uint32_t taken[kTsStage + kWave];  // staging: the keys (and a dropped slot per lane)
  uint32_t tied[kTsStage + kWave];   // staging: their tokens
  uint32_t hist[2][256];
  uint32_t wlo[kTsWaves], whi[kTsWaves];
  int wtot[kTsWaves], wtot2[kTsWaves];
  int32_t out[kTokSelectOneMaxBudget];     // the selection, in order
  float pm[2][kTsWaves], ps[2][kTsWaves];  // the softmax partials' per-wave parts
  int pi[2][kTsWaves];
  int ncand, beta, above, inb, req, is_last;
};

constexpr float kTsLog2e = 1.4426950408889634f;

// (m, s) <- the log-sum-exp merge of (m, s) and (m2, s2): s a sum of exp(x - m)
// (the exponentials by the hardware exp2: the shares they feed decide a count
// within a tolerance of 1e-4, far above its few-ulp error)
__device__ __forceinline__ void ts_lse_merge(float& m, float& s, float m2, float s2) {
  const float mx = fmaxf(m, m2);
  if (mx == -__builtin_inff()) {
    m = mx;
    s = 0.0f;
    return;
  }
  s = s * __builtin_amdgcn_exp2f((m - mx) * kTsLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mx) * kTsLog2e);
  m = mx;
}

// Inclusive scans of two ints per thread over the work-group; tv, tw: totals.
__device__ __forceinline__ void ts_scan2(int& v, int& w, TsLds& s, int& tv, int& tw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int nv = __shfl_up(v, off, kWave), nw = __shfl_up(w, off, kWave);
    if (lane >= off) {
      v += nv;
      w += nw;
    }
  }
  if (lane == kWave - 1) {
    s.wtot[wave] = v;
    s.wtot2[wave] = w;
  }
  __syncthreads();
  int bv = 0, bw = 0;
  tv = 0;
  tw = 0;
#pragma unroll
  for (int k = 0; k < kTsWaves; ++k) {
    const int xv = s.wtot[k], xw = s.wtot2[k];
    bv += k < wave ? xv : 0;
    bw += k < wave ? xw : 0;
    tv += xv;
    tw += xw;
  }
  __syncthreads();
  v += bv;
  w += bw;
}

// What a radix select decided: keys > kgt are taken, and r_eq of the keys
// equal to keq (the lowest indices); or, with ge, every key >= kge.
struct TsCut {
  uint32_t kgt, keq, kge;
  int r_eq;
  bool ge;
};

// The key of the picks-th largest of the keys for_each_key visits (each
// thread visits its own share; picks >= 1 and at most their number), by radix
// digits of up to 8 bits from the highest bit in which the keys differ. Every
// thread of the work-group must call it.
template <class ForEach>
__device__ __forceinline__ TsCut ts_radix(int picks, ForEach&& for_each_key, TsLds& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t klo = 0xFFFFFFFFu, khi = 0u;
  for_each_key([&](uint32_t key) {
    klo = key < klo ? key : klo;
    khi = key > khi ? key : khi;
  });
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t ol = uint32_t(__shfl_xor(int(klo), off, kWave));
    const uint32_t oh = uint32_t(__shfl_xor(int(khi), off, kWave));
    klo = ol < klo ? ol : klo;
    khi = oh > khi ? oh : khi;
  }
  if (lane == 0) {
    s.wlo[wave] = klo;
    s.whi[wave] = khi;
  }
  if (tid < 256) s.hist[0][tid] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kTsWaves; ++k) {
    klo = s.wlo[k] < klo ? s.wlo[k] : klo;
    khi = s.whi[k] > khi ? s.whi[k] : khi;
  }
  const uint32_t diff = klo ^ khi;
  int hi = diff ? 32 - __builtin_clz(diff) : 0;  // bits [hi, 32) are common
  uint32_t prefix = hi < 32 ? khi >> hi : 0u;
  int r = picks;
  TsCut cut;
  cut.ge = false;
  cut.kge = 0u;
  for (int pass = 0;; ++pass) {
    if (hi == 0) {  // every bit resolved: kappa = prefix, r of its ties are taken
      cut.kgt = cut.keq = prefix;
      cut.r_eq = r;
      return cut;
    }
    const int width = hi < 8 ? hi : 8;
    const int shift = hi - width;
    uint32_t* cur = s.hist[pass & 1];
    uint32_t* nxt = s.hist[(pass & 1) ^ 1];
    if (tid < 256) nxt[tid] = 0;  // its last reader finished before the last barrier
    for_each_key([&](uint32_t key) {
      if (hi == 32 || (key >> hi) == prefix)
        atomicAdd(&cur[(key >> shift) & ((1u << width) - 1u)], 1u);
    });
    __syncthreads();
    if (wave == 0) {
      // lane l takes bins 255 - 4 l .. 252 - 4 l (descending)
      if (lane == 0) {
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
      int incl = run;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int n = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += n;
      }
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
      cut.ge = true;
      cut.kge = prefix << hi;
      cut.kgt = cut.keq = 0u;
      cut.r_eq = 0;
      return cut;
    }
  }
}

__device__ __forceinline__ void ts_mark(const TsCut& cut, uint32_t key, int t, TsLds& s) {
  const bool take = cut.ge ? key >= cut.kge : key > cut.kgt;
  const bool tie = !cut.ge && key == cut.keq;
  if (take) atomicOr(&s.taken[t >> 5], 1u << (t & 31));
  else if (tie) atomicOr(&s.tied[t >> 5], 1u << (t & 31));
}

// The unit's words in the one-launch region of the token workspace: the
// arrival counter, the chunks' candidate counts (each on its own 128-byte
// line), then per chunk a list of up to kTsChunkCap candidates (keys, then
// tokens).
constexpr int kTsChunkCap = 8192;
constexpr int kTsCounterWord = 0, kTsCountWord = 32, kTsListWord = 64;
constexpr int kTsMaxChunks = kTokSelectMaxTokens / kTsChunk;
static_assert(kTsMaxChunks <= 32, "the count words fit their line");

__host__ __device__ constexpr int64_t ts_unit_words(int chunks) {
  return kTsListWord + int64_t(chunks) * 2 * kTsChunkCap;
}

// grid (B * Hkv, ceil(Tmax / kTsChunk)), kTsThreads threads. lse (the adaptive
// budget, else null): where each 16384-token half-chunk's softmax partial goes
// (maximum over its finite scores, sum of exp(s - maximum), count of +inf), at
// lse + unit * lse_stride + 3 * half-chunk, as the chunked select's filter
// leaves them for tok_topp.
__global__ __launch_bounds__(kTsThreads) void tok_select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int Tmax,
    int budget, uint32_t* __restrict__ ws, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, uint32_t* __restrict__ lse, int64_t lse_stride) {
  __shared__ TsLds s;
  const int unit = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int C = clamp_len(seq_lens[unit / Hkv], Tmax);
  const int picks = max(0, min(budget, C));
  const float* row = scores + int64_t(unit) * Tmax;
  int32_t* out = idx + int64_t(unit) * budget;
  uint32_t* uw = ws + int64_t(unit) * ts_unit_words(gridDim.y);
  if (picks == 0 || picks == C) {  // nothing, or every candidate in order
    if (chunk == 0) {
      for (int k = tid; k < budget; k += kTsThreads) out[k] = k < picks ? k : -1;
      if (tid == 0) count[unit] = picks;
    }
    return;
  }

  // the sample's loads (always issued: inside the row whatever C), then the
  // chunk's: the sample is ranked while the chunk's scores are in flight
  constexpr int kPer = kTsSample / kTsThreads;
  float sv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j)  // an atomic load: issued here, not sunk into its branch
    sv[j] = __hip_atomic_load(row + (int64_t(tid + kTsThreads * j) * C) / kTsSample,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kQ = kTsChunk / 4 / kTsThreads;  // 16-byte pieces per thread
  const int nq = ceil_div(C, 4);                 // pieces of the row (Tmax % 4 == 0)
  const int qb = chunk * (kTsChunk / 4);
  float4v v[kQ];
#pragma unroll
  for (int b = 0; b < kQ; ++b) {
    const int q = min(qb + tid + kTsThreads * b, nq - 1);  // clamped: dropped below
    v[b] = *reinterpret_cast<const float4v*>(row + 4 * int64_t(q));
  }

  // ---- 1. threshold ----
  uint32_t T = 0u;
  if (C > kTsCap) {
    uint32_t sk[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) sk[j] = score_key(sv[j]);
    const int64_t want = (int64_t(picks) * kTsSample * 5 + 2 * C - 1) / (2 * C) + 8;
    if (want < kTsSample) {
      const TsCut c = ts_radix(int(want), [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) f(sk[j]);
      }, s);
      T = c.ge ? c.kge : c.keq;  // the sample's rank-want key (its ties included)
    }
  }

  if (lse) {  // the half-chunks' softmax partials (uniform branch)
    static_assert(kQ % 2 == 0, "two halves");
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float m = -__builtin_inff(), sm = 0.0f;
      int ninf = 0;
#pragma unroll
      for (int b = hh * kQ / 2; b < (hh + 1) * kQ / 2; ++b) {
        const int q = qb + tid + kTsThreads * b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[b][e];
          const bool in = q < nq && 4 * q + e < C;
          ninf += (in && x == __builtin_inff()) ? 1 : 0;
          m = (in && x < __builtin_inff()) ? fmaxf(m, x) : m;  // fmaxf drops NaN
        }
      }
#pragma unroll
      for (int b = hh * kQ / 2; b < (hh + 1) * kQ / 2; ++b) {
        const int q = qb + tid + kTsThreads * b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[b][e];
          const bool fin = q < nq && 4 * q + e < C && x > -__builtin_inff() && x < __builtin_inff();
          const float ex = __builtin_amdgcn_exp2f((x - m) * kTsLog2e);
          sm += fin ? ex : 0.0f;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off, kWave), s2 = __shfl_xor(sm, off, kWave);
        ts_lse_merge(m, sm, m2, s2);
        ninf += __shfl_xor(ninf, off, kWave);
      }
      if (lane == 0) {
        s.pm[hh][wave] = m;
        s.ps[hh][wave] = sm;
        s.pi[hh][wave] = ninf;
      }
    }
    __syncthreads();
    if (tid < 2) {
      const int half = 2 * chunk + tid;  // the 16384-token chunk
      if (half * (kTsChunk / 2) < Tmax) {
        float M = s.pm[tid][0], S = s.ps[tid][0];
        int NI = s.pi[tid][0];
        for (int w = 1; w < kTsWaves; ++w) {
          ts_lse_merge(M, S, s.pm[tid][w], s.ps[tid][w]);
          NI += s.pi[tid][w];
        }
        uint32_t* p = lse + int64_t(unit) * lse_stride + 3 * half;
        p[0] = __builtin_bit_cast(uint32_t, M);
        p[1] = __builtin_bit_cast(uint32_t, S);
        p[2] = uint32_t(NI);
      }
    }
  }

  // ---- 2. listing: this chunk's keys >= T ----
  int mine = 0;
#pragma unroll
  for (int b = 0; b < kQ; ++b) {
    const int q = qb + tid + kTsThreads * b;
#pragma unroll
    for (int e = 0; e < 4; ++e) mine += (q < nq && 4 * q + e < C && score_key(v[b][e]) >= T);
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += n;
  }
  if (lane == kWave - 1) s.wtot[wave] = incl;
  __syncthreads();
  int tot = 0, lpos = incl - mine;  // the group's total; this lane's first slot in the group
#pragma unroll
  for (int k = 0; k < kTsWaves; ++k) {
    tot += s.wtot[k];
    lpos += k < wave ? s.wtot[k] : 0;
  }
  uint32_t* lk = uw + kTsListWord + int64_t(chunk) * 2 * kTsChunkCap;  // keys, then tokens
  if (tid == 0) store_coherent(reinterpret_cast<int32_t*>(uw + kTsCountWord + chunk), tot);
  if (tot <= kTsStage) {  // the same in every thread
    // staged in LDS without branches (a lane's non-candidates go to a slot of
    // its own past the staging range), then stored densely
#pragma unroll
    for (int b = 0; b < kQ; ++b) {
      const int q = qb + tid + kTsThreads * b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = score_key(v[b][e]);
        const bool c = q < nq && 4 * q + e < C && key >= T;
        const int at = c ? lpos : kTsStage + lane;
        s.taken[at] = key;
        s.tied[at] = uint32_t(4 * q + e);
        lpos += c;
      }
    }
    __syncthreads();
    for (int i = tid; i < tot; i += kTsThreads) {
      store_coherent(reinterpret_cast<int32_t*>(lk + i), int32_t(s.taken[i]));
      store_coherent(reinterpret_cast<int32_t*>(lk + kTsChunkCap + i), int32_t(s.tied[i]));
    }
  } else {
#pragma unroll
    for (int b = 0; b < kQ; ++b) {
      const int q = qb + tid + kTsThreads * b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = score_key(v[b][e]);
        if (q < nq && 4 * q + e < C && key >= T) {
          if (lpos < kTsChunkCap) {
            store_coherent(reinterpret_cast<int32_t*>(lk + lpos), int32_t(key));
            store_coherent(reinterpret_cast<int32_t*>(lk + kTsChunkCap + lpos), 4 * q + e);
          }
          ++lpos;
        }
      }
    }
  }
  if (!last_group_of_unit(uw + kTsCounterWord, 0, gridDim.y, &s.is_last)) return;

  // ---- the unit's last group: 3. exact boundary, and the bitmaps ----
  // the chunks' counts; candidate i is in chunk k where pre[k] <= i < pre[k + 1]
  const int chunks = gridDim.y;
  int pre[kTsMaxChunks + 1];
  bool over = false;
  pre[0] = 0;
#pragma unroll
  for (int k = 0; k < kTsMaxChunks; ++k) {
    const int ck = k < chunks ? load_coherent(reinterpret_cast<const int32_t*>(uw + kTsCountWord + k))
                              : 0;
    over = over || ck > kTsChunkCap;
    pre[k + 1] = pre[k] + ck;
  }
  const int nc = pre[kTsMaxChunks];
  const int nwords = ceil_div(C, 32);
  for (int w = tid; w < nwords; w += kTsThreads) {
    s.taken[w] = 0u;
    s.tied[w] = 0u;
  }
  if (!over && nc >= picks && nc <= kTsCap) {
    uint32_t ck[kTsPer];
    int ct[kTsPer];
#pragma unroll
    for (int j = 0; j < kTsPer; ++j) {
      const int i = tid + kTsThreads * j;
      int k = 0;
#pragma unroll
      for (int m = 1; m < kTsMaxChunks; ++m) k += i >= pre[m];
      const int off = i < nc ? i - pre[k] : 0;  // past the list: a slot of chunk 0, dropped
      const uint32_t* l = uw + kTsListWord + int64_t(i < nc ? k : 0) * 2 * kTsChunkCap;
      ck[j] = uint32_t(load_coherent(reinterpret_cast<const int32_t*>(l + off)));
      ct[j] = load_coherent(reinterpret_cast<const int32_t*>(l + kTsChunkCap + off));
    }
#pragma unroll
    for (int j = 0; j < kTsPer; ++j)
      if (tid + kTsThreads * j >= nc) ct[j] = -1;
    __syncthreads();  // the bitmaps are clear
    const TsCut cut = ts_radix(picks, [&](auto&& f) {
#pragma unroll
      for (int j = 0; j < kTsPer; ++j)
        if (ct[j] >= 0) f(ck[j]);
    }, s);
#pragma unroll
    for (int j = 0; j < kTsPer; ++j)
      if (ct[j] >= 0) ts_mark(cut, ck[j], ct[j], s);
    s.req = cut.r_eq;  // the same in every thread; read after the barrier below
  } else {
    __syncthreads();  // the bitmaps are clear
    // the unit's scores in memory, 16-byte pieces, kTsBatch loads at a time
    auto each_global = [&](auto&& f) {
      for (int q0 = 0; q0 < nq; q0 += kTsThreads * kTsBatch) {
        float4v x[kTsBatch];
#pragma unroll
        for (int b = 0; b < kTsBatch; ++b)
          x[b] = *reinterpret_cast<const float4v*>(
              row + 4 * int64_t(min(q0 + tid + kTsThreads * b, nq - 1)));
#pragma unroll
        for (int b = 0; b < kTsBatch; ++b) {
          const int q = q0 + tid + kTsThreads * b;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (q < nq && 4 * q + e < C) f(score_key(x[b][e]), 4 * q + e);
        }
      }
    };
    const TsCut cut = ts_radix(picks, [&](auto&& f) {
      each_global([&](uint32_t key, int) { f(key); });
    }, s);
    each_global([&](uint32_t key, int t) { ts_mark(cut, key, t, s); });
    s.req = cut.r_eq;
  }
  __syncthreads();
  const int r_eq = s.req;

  // ---- 4. output in token order ----
  // Thread t owns bitmap words [t wpt, (t + 1) wpt) for the counts: its chosen
  // bits (taken, plus the ties whose rank among all ties is below r_eq) replace
  // its taken words and its words' first output positions its tied words. The
  // tokens are then written word by word with the words dealt out at a stride
  // of the group size, so a run of chosen tokens (a block of them) is spread
  // over several threads, into LDS, and leave in dense stores.
  constexpr int kMaxWpt = kTokSelectMaxTokens / 32 / kTsThreads;
  const int wpt = ceil_div(nwords, kTsThreads);
  const int w0 = min(nwords, tid * wpt), w1 = min(nwords, w0 + wpt);
  int ngt = 0, neq = 0;
  for (int w = w0; w < w1; ++w) {
    ngt += __builtin_popcount(s.taken[w]);
    neq += __builtin_popcount(s.tied[w]);
  }
  int sgt = ngt, seq = neq, tot_gt, tot_eq;
  ts_scan2(sgt, seq, s, tot_gt, tot_eq);
  const int nsel = min(tot_gt + min(tot_eq, r_eq), budget);
  int eq_seen = seq - neq, nmine = 0;
  uint32_t selw[kMaxWpt];
#pragma unroll
  for (int i = 0; i < kMaxWpt; ++i) {
    const int w = w0 + i;
    selw[i] = 0u;
    if (w < w1) {
      const uint32_t te = s.tied[w];
      // of this word's ties, the lowest-index (r_eq - eq_seen) are taken
      uint32_t keep = 0u, x = te;
      for (int k = r_eq - eq_seen; k > 0 && x; --k) {
        keep |= x & (0u - x);
        x &= x - 1u;
      }
      eq_seen += __builtin_popcount(te);
      selw[i] = s.taken[w] | keep;
      nmine += __builtin_popcount(selw[i]);
    }
  }
  int before = nmine, dummy = 0, tot_sel, tot_dummy;
  ts_scan2(before, dummy, s, tot_sel, tot_dummy);
  before -= nmine;
#pragma unroll
  for (int i = 0; i < kMaxWpt; ++i) {
    const int w = w0 + i;
    if (w < w1) {  // only this thread reads or writes its own words here
      s.taken[w] = selw[i];
      s.tied[w] = uint32_t(before);
      before += __builtin_popcount(selw[i]);
    }
  }
  __syncthreads();
  for (int w = tid; w < nwords; w += kTsThreads) {
    uint32_t m = s.taken[w];
    int p = int(s.tied[w]);
    while (m) {
      const int b = __builtin_ctz(m);
      m &= m - 1u;
      if (p < budget) s.out[p] = 32 * w + b;
      ++p;
    }
  }
  __syncthreads();
  for (int k = tid; k < budget; k += kTsThreads) out[k] = k < nsel ? s.out[k] : -1;
  if (tid == 0) count[unit] = nsel;
}

}  // namespace

bool token_select_one_group(const UnitGeom& g, int budget, float top_p) {
  (void)top_p;  // the adaptive budget's partials come with the listing
  return g.Tmax <= kTokSelectMaxTokens && g.Tmax % 4 == 0 && budget <= kTokSelectOneMaxBudget;
}

size_t token_select_one_workspace(const UnitGeom& g) {
  return size_t(ts_unit_words(ceil_div(g.Tmax, kTsChunk))) * 4 * size_t(g.B) * size_t(g.Hkv);
}

hipError_t launch_select_token_one(const UnitGeom& g, int budget, const float* scores,
                                   const int32_t* seq_lens, void* ws, int32_t* idx,
                                   int32_t* count, uint32_t* lse, int64_t lse_stride,
                                   hipStream_t s) {
  // a unit's chunks are units apart in the dispatch order, so with a unit count
  // that is a multiple of 8 they land on one XCD and share its L2
  const dim3 grid(g.B * g.Hkv, ceil_div(g.Tmax, kTsChunk));
  hipLaunchKernelGGL(tok_select_kernel, grid, dim3(kTsThreads), 0, s, scores, seq_lens, g.Hkv,
                     g.Tmax, budget, static_cast<uint32_t*>(ws), idx, count, lse, lse_stride);
  return hipGetLastError();
}

}  // namespace bsa
