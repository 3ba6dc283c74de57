// Log-sum-exp merge of split partials:
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
// One 128-thread work-group per row (sequence, query head), one channel per
// thread (combine_core.hpp). Up to 32 splits every value is loaded in one
// round trip (the one-pass form; the same bits as the batched one).
#include "combine_core.hpp"

namespace bsa {
namespace {

__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      float* __restrict__ out,
                                                      float* __restrict__ out_lse, int splits) {
  const int row = blockIdx.x, d = threadIdx.x;
  float o, lse;
  const float* pl = part_lse + int64_t(row) * splits;
  const float* po = part_o + int64_t(row) * splits * kHeadDim;
  if (splits <= 8) combine_channel_few<8, false>(pl, po, splits, d, o, lse);
  else if (splits <= 16) combine_channel_few<16, false>(pl, po, splits, d, o, lse);
  else if (splits <= 32) combine_channel_few<32, false>(pl, po, splits, d, o, lse);
  else combine_channel(pl, po, splits, d, o, lse);
  out[int64_t(row) * kHeadDim + d] = o;
  if (out_lse && d == 0) out_lse[row] = lse;
}

}  // namespace

hipError_t launch_combine(int rows, int splits, const float* part_o, const float* part_lse,
                          float* out, float* out_lse, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(rows), dim3(128), 0, s, part_o, part_lse, out, out_lse,
                     splits);
  return hipGetLastError();
}

}  // namespace bsa
