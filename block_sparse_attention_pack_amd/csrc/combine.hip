// Log-sum-exp merge of split partials:
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
// One 128-thread work-group per row (sequence, query head), one channel per
// thread; the split weights are computed once in LDS.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kMaxSplitsLds = 1024;

__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      float* __restrict__ out,
                                                      float* __restrict__ out_lse, int splits) {
  __shared__ float w[kMaxSplitsLds];
  __shared__ float sh_max, sh_sum;
  const int row = blockIdx.x, d = threadIdx.x;
  const float* pl = part_lse + int64_t(row) * splits;
  if (d < kWave) {
    float mx = -__builtin_inff();
    for (int s = d; s < splits; s += kWave) mx = fmaxf(mx, pl[s]);
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int s = d; s < splits; s += kWave) {
      const float e = mx > -__builtin_inff() ? __expf(pl[s] - mx) : 0.0f;
      w[s] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (d == 0) {
      sh_max = mx;
      sh_sum = sum;
    }
  }
  __syncthreads();
  const float mx = sh_max, sum = sh_sum;
  const bool empty = !(sum > 0.0f);
  float acc = 0.0f;
  if (!empty) {
    const float* po = part_o + int64_t(row) * splits * kHeadDim + d;
    float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent partial sums keep loads in flight
    int s = 0;
    for (; s + 4 <= splits; s += 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) a4[k] += w[s + k] * po[int64_t(s + k) * kHeadDim];
    }
    for (; s < splits; ++s) a4[0] += w[s] * po[int64_t(s) * kHeadDim];
    acc = ((a4[0] + a4[1]) + (a4[2] + a4[3])) / sum;
  }
  out[int64_t(row) * kHeadDim + d] = acc;
  if (out_lse && d == 0) out_lse[row] = empty ? -__builtin_inff() : mx + __logf(sum);
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
