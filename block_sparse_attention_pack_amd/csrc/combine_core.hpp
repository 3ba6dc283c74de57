// Log-sum-exp merge of split partials for one output channel:
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
// Shared by the combine kernel and the attention kernel's fused merge so both
// give the same bits (fixed summation order: weights in split order, the
// weighted sum in four interleaved partial sums).
#pragma once

#include "common.hpp"

namespace bsa {

// pl: the row's num_splits log-sum-exps; po: the row's partials [num_splits][128].
// COHERENT: read them with device-scope loads (written by other work-groups of
// the same launch).
template <bool COHERENT = false>
__device__ __forceinline__ void combine_channel(const float* pl, const float* po, int splits,
                                                int d, float& out, float& lse) {
  auto ld = [](const float* p) -> float { return COHERENT ? load_coherent(p) : *p; };
  float mx = -__builtin_inff();
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, ld(pl + s));
  if (!(mx > -__builtin_inff())) {
    out = 0.0f;
    lse = -__builtin_inff();
    return;
  }
  float sum = 0.0f;
  float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent partial sums keep loads in flight
  int s = 0;
  for (; s + 4 <= splits; s += 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float w = __expf(ld(pl + s + k) - mx);
      sum += w;
      a4[k] += w * ld(po + int64_t(s + k) * kHeadDim + d);
    }
  }
  for (; s < splits; ++s) {
    const float w = __expf(ld(pl + s) - mx);
    sum += w;
    a4[0] += w * ld(po + int64_t(s) * kHeadDim + d);
  }
  out = ((a4[0] + a4[1]) + (a4[2] + a4[3])) / sum;
  lse = mx + __logf(sum);
}

}  // namespace bsa
