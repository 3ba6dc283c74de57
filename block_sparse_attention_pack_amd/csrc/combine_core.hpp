// Log-sum-exp merge of split partials for one output channel:
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
// Shared by the combine kernel and the attention kernel's fused merge so both
// give the same bits: the maximum, the weights and their sum in split order,
// the weighted sum in four partial sums (split s into sum s % 4 while whole
// groups of four last, the rest into sum 0), fused multiply-adds throughout.
#pragma once

#include "common.hpp"

namespace bsa {

// One batch of up to B splits, s0 .. s0 + n - 1, whose log-sum-exps and
// partials are already in registers (lv, ov).
struct CombineState {
  float mx = -__builtin_inff();
  float sum = 0.0f;
  float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
};

template <int B>
__device__ __forceinline__ void combine_max(CombineState& st, const float (&lv)[B], int n) {
#pragma unroll
  for (int k = 0; k < B; ++k)
    if (k < n) st.mx = fmaxf(st.mx, lv[k]);
}

// s0 must be a multiple of 4; s4 = splits rounded down to a multiple of 4.
template <int B>
__device__ __forceinline__ void combine_accumulate(CombineState& st, const float (&lv)[B],
                                                   const float (&ov)[B], int s0, int n, int s4) {
  static_assert(B % 4 == 0, "batches keep the partial-sum pattern");
#pragma unroll
  for (int k = 0; k < B; ++k) {
    if (k < n) {
      const float w = __expf(lv[k] - st.mx);
      st.sum += w;
      if (s0 + k < s4) st.a4[k & 3] = __builtin_fmaf(w, ov[k], st.a4[k & 3]);
      else st.a4[0] = __builtin_fmaf(w, ov[k], st.a4[0]);
    }
  }
}

__device__ __forceinline__ void combine_finish(const CombineState& st, float& out, float& lse) {
  if (!(st.mx > -__builtin_inff())) {
    out = 0.0f;
    lse = -__builtin_inff();
    return;
  }
  out = ((st.a4[0] + st.a4[1]) + (st.a4[2] + st.a4[3])) / st.sum;
  lse = st.mx + __logf(st.sum);
}

// pl: the row's `splits` log-sum-exps; po: the row's partials [splits][128].
// Reads them in batches of kBatch (all loads of a batch in flight at once).
// COHERENT: device-scope loads (values written by other work-groups of the
// same launch).
template <bool COHERENT = false>
__device__ __forceinline__ void combine_channel(const float* pl, const float* po, int splits,
                                                int d, float& out, float& lse) {
  constexpr int kBatch = 8;
  auto ld = [](const float* p) -> float { return COHERENT ? load_coherent(p) : *p; };
  const int s4 = splits & ~3;
  CombineState st;
  // pass 1: the maximum
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    float lv[kBatch];
    const int n = min(kBatch, splits - s0);
#pragma unroll
    for (int k = 0; k < kBatch; ++k) lv[k] = k < n ? ld(pl + s0 + k) : -__builtin_inff();
    combine_max(st, lv, n);
  }
  if (!(st.mx > -__builtin_inff())) {
    combine_finish(st, out, lse);
    return;
  }
  // pass 2: weights and weighted partials
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    float lv[kBatch], ov[kBatch];
    const int n = min(kBatch, splits - s0);
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      lv[k] = k < n ? ld(pl + s0 + k) : 0.0f;
      ov[k] = k < n ? ld(po + int64_t(s0 + k) * kHeadDim + d) : 0.0f;
    }
    combine_accumulate(st, lv, ov, s0, n, s4);
  }
  combine_finish(st, out, lse);
}

// The same merge for at most MAXS splits, every value loaded once, all loads
// issued before the first is used.
template <int MAXS, bool COHERENT>
__device__ __forceinline__ void combine_channel_few(const float* pl, const float* po, int splits,
                                                    int d, float& out, float& lse) {
  auto ld = [](const float* p) -> float { return COHERENT ? load_coherent(p) : *p; };
  float lv[MAXS], ov[MAXS];
#pragma unroll
  for (int k = 0; k < MAXS; ++k) {
    lv[k] = k < splits ? ld(pl + k) : -__builtin_inff();
    ov[k] = k < splits ? ld(po + int64_t(k) * kHeadDim + d) : 0.0f;
  }
  CombineState st;
  combine_max(st, lv, splits);
  if (st.mx > -__builtin_inff()) combine_accumulate(st, lv, ov, 0, splits, splits & ~3);
  combine_finish(st, out, lse);
}

}  // namespace bsa
