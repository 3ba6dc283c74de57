// Sparse decode attention kernel (split partials, optional in-kernel merge)
// and its host launcher. The device code is in attn_core.hpp.
#include "attn_core.hpp"

namespace bsa {
namespace {

// grid (splits, B * Hkv), 256 threads, at least two work-groups per CU. VM:
// where the values are read (kValCache, kValStore, kValStoreTail); RING: groups
// in flight per wave.
template <int G, bool MAIN_BF16, bool BLOCK, int VM, int RING>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(
    AttnArgs a) {
  __shared__ AttnLds<G> lds;
  attn_item<G, MAIN_BF16, BLOCK, VM, RING>(a, blockIdx.x, blockIdx.y, lds);
}

template <int G, bool BLOCK, int VM>
void launch_gbv(dim3 grid, hipStream_t s, const AttnArgs& a, bool bf16) {
  if (bf16) hipLaunchKernelGGL((attn_kernel<G, true, BLOCK, VM, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((attn_kernel<G, false, BLOCK, VM, 1>), grid, dim3(256), 0, s, a);
}

template <int G>
void launch_g(dim3 grid, hipStream_t s, const AttnArgs& a, int block_mode, bool bf16, bool vq,
              bool small_grid) {
  if (block_mode) {
    if (!vq && !bf16 && small_grid)
      hipLaunchKernelGGL((attn_kernel<G, false, true, kValCache, kRingSmallGrid>), grid,
                         dim3(256), 0, s, a);
    else if (!vq) launch_gbv<G, true, kValCache>(grid, s, a, bf16);
    else if (a.n_tail > 0) launch_gbv<G, true, kValStoreTail>(grid, s, a, bf16);
    else launch_gbv<G, true, kValStore>(grid, s, a, bf16);
  } else {
    if (!vq) launch_gbv<G, false, kValCache>(grid, s, a, bf16);
    else launch_gbv<G, false, kValStore>(grid, s, a, bf16);
  }
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
  a.vs = g.vq ? value_store(g, v) : ValueStore{nullptr, nullptr, nullptr};
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
  // fewer work-groups than two per CU of the 256
  const bool small = int64_t(splits) * g.B * g.Hkv < 512;
  switch (g.G) {
    case 1: launch_g<1>(grid, s, a, block_mode, bf16, g.vq, small); break;
    case 2: launch_g<2>(grid, s, a, block_mode, bf16, g.vq, small); break;
    case 4: launch_g<4>(grid, s, a, block_mode, bf16, g.vq, small); break;
    case 8: launch_g<8>(grid, s, a, block_mode, bf16, g.vq, small); break;
    case 16: launch_g<16>(grid, s, a, block_mode, bf16, g.vq, small); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsa
