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
//      (the score's bits, token) in token order, with its count, staged in
//      LDS and written with dense stores.
// The unit's last group to arrive (an arrival counter, as the attention's
// merge uses) then:
//   3. finds the exact key kappa of the picks-th largest listed key by a radix
//      select over the list held in registers (the block select's procedure
//      over a 1024-thread group), and how many of its ties are taken;
//   4. writes the listed tokens above kappa and the lowest-index ties in list
//      order, which is token order: each chosen slot's output position comes
//      from ballots over runs of 64 slots and one scan of the runs' counts.
// With the adaptive budget, every group also leaves its two 16384-token
// halves' softmax partials for tok_topp, which then cuts the selection.
// If the lists hold fewer than picks or more than kTsCap candidates, or a chunk
// more than kTsChunkCap (a sample far from the unit's distribution, or many
// equal keys), steps 3 and 4 run over the unit's scores in memory instead, with
// one read of the scores per radix pass, marks in LDS bitmaps of the unit's
// tokens and the output from scans of the bitmap words: the same result. The last group
// returns the counter to zero, so the workspace is ready for the next call.
#include <type_traits>

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

// A group's listed scores and tokens are staged in the bitmaps' words (used only
// by the unit's last group, after every group has stored its list), so the
// global list is written with dense stores.
constexpr int kTsStage = kTokSelectMaxTokens / 32;

struct TsLds {
  uint32_t taken[kTsStage + kWave];  // staging: the scores' bits (and a dropped slot per lane)
  uint32_t tied[kTsStage + kWave];   // staging: their tokens
  uint32_t hist[2][256];
  uint32_t wlo[kTsWaves], whi[kTsWaves];
  int wtot[4][kTsWaves];
  uint32_t slots[kTsPer * kTsWaves];  // per 64 list slots: chosen counts, then their bases
  int32_t out[kTokSelectOneMaxBudget];     // the selection, in order
  float pm[2][kTsWaves], ps[2][kTsWaves];  // the softmax partials' per-wave parts
  int pi[2][kTsWaves];
  int ncand, beta, above, inb, is_last;
};

constexpr float kTsLog2e = 1.4426950408889634f;

// For a key T > 0: the float f with key(x) >= T exactly when x >= f (x not
// NaN; NaN has key 0 and fails every compare). Keys up to that of -inf admit
// every number; above them a negative key is the complement of the float's
// bits and a positive one the float's bits with the sign bit set, and a key
// past +inf's gives a NaN, which admits nothing. The -0 and +0 share a key
// and compare equal, so either bound serves for them.
__device__ __forceinline__ float ts_key_floor(uint32_t T) {
  if (T <= 0x007FFFFFu) return -__builtin_inff();
  return __uint_as_float((T & 0x80000000u) ? (T & 0x7FFFFFFFu) : ~T);
}

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

// Inclusive scans of N ints per thread over the work-group (thread order);
// t: the totals.
template <int N>
__device__ __forceinline__ void ts_scan(int (&v)[N], int (&t)[N], TsLds& s) {
  static_assert(N <= 4, "scan width");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
#pragma unroll
  for (int n = 0; n < N; ++n) v[n] = wave_scan_dpp(v[n]);
  if (lane == kWave - 1)
#pragma unroll
    for (int n = 0; n < N; ++n) s.wtot[n][wave] = v[n];
  __syncthreads();
  // lane k < kTsWaves takes wave k's total: a scan over those lanes
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int x = wave_scan_dpp(lane < kTsWaves ? s.wtot[n][lane] : 0);
    t[n] = __builtin_amdgcn_readlane(x, kTsWaves - 1);
    v[n] += wave > 0 ? __builtin_amdgcn_readlane(x, wave > 0 ? wave - 1 : 0) : 0;
  }
  __syncthreads();
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
  wave_minmax_dpp(klo, khi);
  if (lane == 0) {
    s.wlo[wave] = klo;
    s.whi[wave] = khi;
  }
  if (tid < 256) s.hist[0][tid] = 0;
  __syncthreads();
  klo = lane < kTsWaves ? s.wlo[lane] : 0xFFFFFFFFu;  // lane k: wave k's
  khi = lane < kTsWaves ? s.whi[lane] : 0u;
  wave_minmax_dpp(klo, khi);
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
    // a thread adds a run of its keys that share a bin with one atomic: where
    // the keys crowd into few bins (candidates just above the threshold
    // below a few far larger ones), same-address lanes of one LDS atomic are
    // served one at a time
    uint32_t run_bin = 0u, run_n = 0u;
    for_each_key([&](uint32_t key) {
      if (hi == 32 || (key >> hi) == prefix) {
        const uint32_t bin = (key >> shift) & ((1u << width) - 1u);
        if (run_n && bin != run_bin) {
          atomicAdd(&cur[run_bin], run_n);
          run_n = 0u;
        }
        run_bin = bin;
        ++run_n;
      }
    });
    if (run_n) atomicAdd(&cur[run_bin], run_n);
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
      const int P = wave_scan_dpp(run) - run;
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
// line), then per chunk a list of up to kTsChunkCap candidates (score bits,
// then tokens).
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

  const bool whole_chunk = (chunk + 1) * kTsChunk <= C;  // no token of the chunk at or past C

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
    auto partials = [&](auto whole) {  // whole: every token of the chunk is below C
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
            const bool in = decltype(whole)::value || (q < nq && 4 * q + e < C);
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
            const bool in = decltype(whole)::value || (q < nq && 4 * q + e < C);
            const bool fin = in && x > -__builtin_inff() && x < __builtin_inff();
            const float ex = __builtin_amdgcn_exp2f((x - m) * kTsLog2e);
            sm += fin ? ex : 0.0f;
          }
        }
        // the wave's merge in lane 63 (an empty partner is (-inf, 0))
        wave_dpp_steps([&](auto step) {
          const float m2 = __int_as_float(dpp_move(__float_as_int(-__builtin_inff()), __float_as_int(m), step));
          const float s2 = __int_as_float(dpp_move(0, __float_as_int(sm), step));
          ts_lse_merge(m, sm, m2, s2);
          ninf += dpp_move(0, ninf, step);
        });
        if (lane == kWave - 1) {
          s.pm[hh][wave] = m;
          s.ps[hh][wave] = sm;
          s.pi[hh][wave] = ninf;
        }
      }
    };
    if (whole_chunk) partials(std::true_type{});
    else partials(std::false_type{});
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

  // ---- 2. listing: this chunk's keys >= T, in token order ----
  // Piece b of thread t holds tokens 4 (qb + t + kTsThreads b) .. + 3, so the
  // list runs piece by piece, thread by thread. A thread's count per piece (at
  // most 4) is scanned over the group two pieces to an int: a piece's total
  // stays below 2^16.
  static_assert(kQ * 4 == 32, "a candidate mask of 32 bits");
  uint32_t cm = 0u;  // bit 4 b + e: value e of piece b is a candidate
  // key(x) >= T as one float compare: x >= Tf for T > 0 (false for NaN)
  const float Tf = ts_key_floor(T);
  auto mark_candidates = [&](auto whole) {  // whole: every token of the chunk is below C
#pragma unroll
    for (int b = 0; b < kQ; ++b) {
      const int q = qb + tid + kTsThreads * b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = decltype(whole)::value || (q < nq && 4 * q + e < C);
        cm |= uint32_t(in && (T == 0u || v[b][e] >= Tf)) << (4 * b + e);
      }
    }
  };
  if (whole_chunk) mark_candidates(std::true_type{});
  else mark_candidates(std::false_type{});
  int pc[kQ / 2], incl[kQ / 2], tpc[kQ / 2];
#pragma unroll
  for (int hh = 0; hh < kQ / 2; ++hh)
    pc[hh] = __builtin_popcount((cm >> (8 * hh)) & 0xFu) +
             (__builtin_popcount((cm >> (8 * hh + 4)) & 0xFu) << 16);
#pragma unroll
  for (int hh = 0; hh < kQ / 2; ++hh) incl[hh] = pc[hh];
  ts_scan(incl, tpc, s);
  int tot = 0;
#pragma unroll
  for (int hh = 0; hh < kQ / 2; ++hh) {
    incl[hh] -= pc[hh];  // exclusive: the thread's slots in pieces 2 hh, 2 hh + 1
    tpc[hh] = __builtin_amdgcn_readfirstlane(tpc[hh]);
    tot += (tpc[hh] & 0xFFFF) + (tpc[hh] >> 16);
  }
  // this thread's first slot in piece b's run of the list
  auto first_slot = [&](int b) {
    int a = 0;
#pragma unroll
    for (int k = 0; k < b; ++k) a += (tpc[k >> 1] >> (16 * (k & 1))) & 0xFFFF;
    return a + ((incl[b >> 1] >> (16 * (b & 1))) & 0xFFFF);
  };
  uint32_t* lk = uw + kTsListWord + int64_t(chunk) * 2 * kTsChunkCap;  // scores, then tokens
  if (tid == 0) store_coherent(reinterpret_cast<int32_t*>(uw + kTsCountWord + chunk), tot);
  if (tot <= kTsStage) {  // the same in every thread
    // staged in LDS without branches (a lane's non-candidates go to a slot of
    // its own past the staging range), then stored densely
#pragma unroll
    for (int b = 0; b < kQ; ++b) {
      const int q = qb + tid + kTsThreads * b;
      int at = first_slot(b);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool c = (cm >> (4 * b + e)) & 1u;
        const int a = c ? at : kTsStage + lane;
        s.taken[a] = __float_as_uint(v[b][e]);
        s.tied[a] = uint32_t(4 * q + e);
        at += c;
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
      int at = first_slot(b);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((cm >> (4 * b + e)) & 1u) {
          if (at < kTsChunkCap) {
            store_coherent(reinterpret_cast<int32_t*>(lk + at), __float_as_int(v[b][e]));
            store_coherent(reinterpret_cast<int32_t*>(lk + kTsChunkCap + at), 4 * q + e);
          }
          ++at;
        }
      }
    }
  }
  if (!last_group_of_unit(uw + kTsCounterWord, 0, gridDim.y, &s.is_last)) return;

  // ---- the unit's last group: 3. exact boundary ----
  // the chunks' counts; candidate i is in chunk k where pre[k] <= i < pre[k + 1]
  const int chunks = gridDim.y;
  int pre[kTsMaxChunks + 1];
  bool over = false;
  pre[0] = 0;
  int cnt[kTsMaxChunks];  // every word of the counts' line is loaded at once
#pragma unroll
  for (int k = 0; k < kTsMaxChunks; ++k)
    cnt[k] = load_coherent(reinterpret_cast<const int32_t*>(uw + kTsCountWord + k));
#pragma unroll
  for (int k = 0; k < kTsMaxChunks; ++k) {
    const int ck = k < chunks ? cnt[k] : 0;
    over = over || ck > kTsChunkCap;
    pre[k + 1] = pre[k] + ck;
  }
  const int nc = pre[kTsMaxChunks];
  if (!over && nc >= picks && nc <= kTsCap) {
    // slot i = tid + kTsThreads j; from j = jn on no thread holds a candidate,
    // and every loop over j stops there (the group is bound by issue: its
    // per-slot instructions run once per wave)
    const int jn = ceil_div(nc, kTsThreads);
    uint32_t ck[kTsPer];
    int ct[kTsPer];
#pragma unroll
    for (int j = 0; j < kTsPer; ++j) {
      ck[j] = 0u;
      ct[j] = -1;
    }
#pragma unroll
    for (int j = 0; j < kTsPer; ++j) {
      if (j >= jn) continue;
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
    for (int j = 0; j < kTsPer; ++j) {  // after every load is issued
      if (j >= jn) continue;
      ck[j] = score_key(__uint_as_float(ck[j]));  // the lists hold the scores' bits
      if (j == jn - 1 && tid + kTsThreads * j >= nc) ct[j] = -1;  // past the list
    }
    const TsCut cut = ts_radix(picks, [&](auto&& f) {
#pragma unroll
      for (int j = 0; j < kTsPer; ++j) {
        if (j >= jn) continue;
        if (ct[j] >= 0) f(ck[j]);
      }
    }, s);

    // ---- 4. output: the chosen slots in slot order, which is token order ----
    // Chosen: the keys above the cut, and the ties whose rank among the ties
    // is below r_eq. Slot i = kTsThreads j + 64 wave + lane, so one ballot
    // counts a run of 64 slots; wave 0 scans the runs' counts (taken and
    // tied, two 16-bit fields) into their bases, and a chosen slot's output
    // position is the taken slots before it plus min(ties before it, r_eq).
    uint32_t fgt = 0u, feq = 0u;  // bit j: slot j is above the cut, is a tie
#pragma unroll
    for (int j = 0; j < kTsPer; ++j) {
      if (j >= jn) continue;
      const bool gt = ct[j] >= 0 && (cut.ge ? ck[j] >= cut.kge : ck[j] > cut.kgt);
      const bool eq = ct[j] >= 0 && !cut.ge && ck[j] == cut.keq;
      fgt |= uint32_t(gt) << j;
      feq |= uint32_t(eq) << j;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      if (lane == 0) s.slots[j * kTsWaves + wave] = uint32_t(__popcll(mg)) | uint32_t(__popcll(me)) << 16;
    }
    __syncthreads();
    if (wave == 0) {
      static_assert(kTsPer * kTsWaves == 4 * kWave, "four runs per lane");
      uint32_t c[4], x = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = 4 * lane + i < kTsWaves * jn ? s.slots[4 * lane + i] : 0u;
        x += c[i];  // each field stays below 2^16: at most kTsCap slots
      }
      const uint32_t inc = uint32_t(wave_scan_dpp(int(x)));
      uint32_t base = inc - x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s.slots[4 * lane + i] = base;
        base += c[i];
      }
      if (lane == kWave - 1) s.ncand = int(inc);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTsPer; ++j) {
      if (j >= jn) continue;
      const bool gt = (fgt >> j) & 1u, eq = (feq >> j) & 1u;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      const uint32_t base = s.slots[j * kTsWaves + wave];
      const int pg = int(base & 0xFFFFu) +
                     int(__builtin_amdgcn_mbcnt_hi(uint32_t(mg >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(uint32_t(mg), 0u)));
      const int pe = int(base >> 16) +
                     int(__builtin_amdgcn_mbcnt_hi(uint32_t(me >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(uint32_t(me), 0u)));
      const int p = gt ? pg + min(pe, cut.r_eq) : (eq && pe < cut.r_eq ? pg + pe : budget);
      if (p < budget) s.out[p] = ct[j];
    }
    const uint32_t tsel = uint32_t(s.ncand);
    const int nsel = min(int(tsel & 0xFFFFu) + min(int(tsel >> 16), cut.r_eq), budget);
    __syncthreads();
    for (int k = tid; k < budget; k += kTsThreads) out[k] = k < nsel ? s.out[k] : -1;
    if (tid == 0) count[unit] = nsel;
    return;
  }

  // ---- the fallback: marks in bitmaps of the unit's tokens ----
  const int nwords = ceil_div(C, 32);
  for (int w = tid; w < nwords; w += kTsThreads) {
    s.taken[w] = 0u;
    s.tied[w] = 0u;
  }
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
  __syncthreads();
  const int r_eq = cut.r_eq;

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
  int sc[2] = {ngt, neq}, st[2];
  ts_scan(sc, st, s);
  const int nsel = min(st[0] + min(st[1], r_eq), budget);
  int eq_seen = sc[1] - neq, nmine = 0;
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
  int sb[1] = {nmine}, stot[1];
  ts_scan(sb, stot, s);
  int before = sb[0] - nmine;
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
