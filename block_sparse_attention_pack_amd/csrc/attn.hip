// Sparse decode attention kernel (split partials, optional in-kernel selection
// and merge) and its host launcher. The device code is in attn_core.hpp.
#include "attn_core.hpp"

namespace bsa {
namespace {

// grid (splits, B * Hkv), 256 threads.
template <int G, bool MAIN_BF16>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a, int block_mode_i) {
  __shared__ AttnLds<G> lds;
  attn_item<G, MAIN_BF16, false>(a, block_mode_i != 0, blockIdx.x, blockIdx.y, lds, StepSync{});
}

template <int G>
void launch_g(dim3 grid, hipStream_t s, const AttnArgs& a, int block_mode, bool bf16) {
  if (bf16) hipLaunchKernelGGL((attn_kernel<G, true>), grid, dim3(256), 0, s, a, block_mode);
  else hipLaunchKernelGGL((attn_kernel<G, false>), grid, dim3(256), 0, s, a, block_mode);
}

}  // namespace

hipError_t launch_attention(const UnitGeom& g, int granularity, int budget, int n_tail,
                            float sigma, const _Float16* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* idx, const int32_t* count,
                            const uint16_t* tail_k, const uint16_t* tail_v, int splits,
                            float* part_o, float* part_lse, uint32_t* counters, float* out,
                            float* out_lse, const float* sel_scores, int32_t* sel_idx,
                            int32_t* sel_count, hipStream_t s) {
  if (sel_scores && (granularity != BSA_GRANULARITY_BLOCK || budget > kFusedSelectMax))
    return hipErrorInvalidValue;
  AttnArgs a;
  a.sel_scores = sel_scores;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.q = q;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.seq_lens = seq_lens;
  a.idx = idx;
  a.count = count;
  a.tail_k = tail_k;
  a.tail_v = tail_v;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.counters = counters;
  a.out = out;
  a.out_lse = out_lse;
  a.sb = g.sb;
  a.sh = g.sh;
  a.st = g.st;
  a.Hkv = g.Hkv;
  a.Hq = g.Hq;
  a.Tmax = g.Tmax;
  a.budget = budget;
  a.n_tail = n_tail;
  a.splits = splits;
  a.scale_log2 = sigma * kLog2e;
  const int block_mode = granularity == BSA_GRANULARITY_BLOCK;
  const bool bf16 = g.dtype == BSA_DTYPE_BF16;
  dim3 grid(splits, g.B * g.Hkv);
  switch (g.G) {
    case 1: launch_g<1>(grid, s, a, block_mode, bf16); break;
    case 2: launch_g<2>(grid, s, a, block_mode, bf16); break;
    case 4: launch_g<4>(grid, s, a, block_mode, bf16); break;
    case 8: launch_g<8>(grid, s, a, block_mode, bf16); break;
    case 16: launch_g<16>(grid, s, a, block_mode, bf16); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsa
