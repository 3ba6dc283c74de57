// One block-mode decode step in a single launch: the dense scan, the per-unit
// top-k, the sparse attention and the log-sum-exp merge (Jet-QSparse abstract:
// every step scans the whole NVFP4 key history, then attends to the chosen
// 128-token blocks).
//
// Work items. A unit's scan is cut into scan items of kScanWaves * bpw blocks
// (bpw up to 8, two blocks in flight per wave); its attention into `splits`
// attention items (the attention kernel's work-groups). The units are dealt to
// K = min(8, U) classes (unit u to class u % K) and work-group b of the launch
// serves class b % K: it draws a ticket from its class's counter and runs the
// class item the ticket names, so a class's items start in ticket order
// whatever order the hardware dispatches in. Within a class all scan items
// come first, then the attention items, unit by unit.
//
// Hand-off. A scan item stores its scores as device-scope atomics, waits for
// them, and counts itself in its unit's scan-done counter. The item that
// completes the count selects the unit's blocks (select_topk's selection,
// made once per unit instead of once per attention work-group), stores idx
// and count the same way, and raises the counter one further. An attention
// item polls the counter for that value, then reads the selection. Every scan
// item of a unit holds a smaller ticket of the same class than any attention
// item of the unit, and a ticket is only drawn by a running work-group, so
// each awaited item is already running and finishes without waiting itself:
// no wait can block for good. (One ticket counter per class, each on its own
// 128-byte line, as are the scan-done counters: device-scope atomics on one
// address are served one at a time.)
//
// Why one launch: the scan is HBM-bound streaming; the selection, query
// staging and merge are latency chains. Run as two launches, every attention
// work-group starts together and the HBM idles while all of them select. Here
// the selections run while other items stream, attention items start as scan
// items retire, and no launch boundary drains the GPU in between. The cost:
// scan items run at the attention's register budget (three waves per SIMD,
// made up for by the second block in flight), and each waits for its score
// stores before it counts in.
//
// Counters (32-bit words; all return to zero by the end of the launch):
//   [0, U)                  arrival counters of the merge (the attention kernel's)
//   [U + 32 u]              scan-done counter of unit u (reset by its merging group)
//   [U + 32 U + 32 c]       ticket counter of class c < 8 (reset by the class's
//                           last work-group to draw)
//   [U + 32 U + 256]        fault flag: set only if a wait ran past its bound;
//                           never reset
#include "attn_core.hpp"
#include "scan_core.hpp"

namespace bsa {
namespace {

constexpr int kStepClasses = 8;
constexpr int kLineWords = 32;  // 128 bytes

struct StepArgs {
  ScanBlockArgs scan;
  AttnArgs attn;
  StepSync sync;
  uint32_t* tickets;     // class c's counter at tickets[kLineWords * c]
  int units, classes, scan_items, splits;
  uint32_t per_class;    // work-groups per class (the largest class's items)
};

struct Item {
  bool scan;
  int unit, index;  // scan item index within the unit, or the split
};

// Item t of a class of n units: their scan items (unit-major), then their
// attention items (unit-major). The unit is the class-local index.
__device__ __forceinline__ Item decode_ticket(int t, int n, int NS, int S) {
  Item it;
  it.scan = t < n * NS;
  if (it.scan) {
    it.unit = t / NS;
    it.index = t % NS;
  } else {
    t -= n * NS;
    it.unit = t / S;
    it.index = t % S;
  }
  return it;
}

// The unit's block selection (select_topk's), from its scores (device-scope
// loads), stored to idx / count as device-scope atomics. Every thread of the
// work-group calls it.
template <int G>
__device__ __forceinline__ void select_unit(const AttnArgs& a, int unit, AttnLds<G>& lds) {
  const int b = unit / a.Hkv;
  const int L = clamp_len(a.seq_lens[b], a.Tmax);
  const int nb = a.Tmax / kBlock;
  int C, picks, f0, f1;
  block_candidates(L, a.n_tail, nb, a.budget, C, picks, f0, f1);
  select_unit_rows<true>(a.sel_scores + int64_t(unit) * nb, C, picks, f0, f1, a.budget, lds.sel,
                         &lds.sel_cnt, lds.sel_s);
  __syncthreads();
  int32_t* idx = a.sel_idx + int64_t(unit) * a.budget;
  for (int i = threadIdx.x; i < a.budget; i += 256) store_coherent(idx + i, lds.sel[i]);
  if (threadIdx.x == 0) store_coherent(a.sel_count + unit, lds.sel_cnt);
}

template <int G, bool MAIN_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 3 : 1))) void step_kernel(
    StepArgs s) {
  __shared__ AttnLds<G> lds;
  __shared__ uint32_t ticket;
  const int cls = blockIdx.x % s.classes;
  const int n = (s.units - cls + s.classes - 1) / s.classes;  // units of this class
  const uint32_t items = uint32_t(n) * uint32_t(s.scan_items + s.splits);
  if (threadIdx.x == 0) {
    uint32_t* ctr = s.tickets + kLineWords * cls;
    const uint32_t t = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every other work-group of the class has drawn: ready the counter for the next step
    if (t == s.per_class - 1) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t >= s.per_class)  // the counter was not zero at the launch
      __hip_atomic_store(s.sync.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = t;
  }
  __syncthreads();
  if (ticket >= items) return;  // the class has fewer items than the largest one
  Item it = decode_ticket(int(ticket), n, s.scan_items, s.splits);
  it.unit = cls + s.classes * it.unit;
  if (it.scan) {
    scan_wave_blocks<true, true>(s.scan, threadIdx.x & 63, threadIdx.x >> 6, it.unit, it.index,
                                 lds.scan_q);
    wait_all_memory();  // the scores have reached the coherence point
    __syncthreads();
    uint32_t* ctr = s.sync.scan_done + kLineWords * it.unit;
    if (threadIdx.x == 0) {
      const uint32_t before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds.is_last = before == uint32_t(s.scan_items - 1);
    }
    __syncthreads();
    if (lds.is_last) {  // every score of the unit is stored: select for its attention
      select_unit(s.attn, it.unit, lds);
      wait_all_memory();
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(ctr, uint32_t(s.scan_items) + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    attn_item<G, MAIN_BF16, true>(s.attn, true, it.index, it.unit, lds, s.sync);
  }
}

template <int G>
void launch_step_g(uint32_t grid, hipStream_t st, const StepArgs& s, bool bf16) {
  if (bf16) hipLaunchKernelGGL((step_kernel<G, true>), dim3(grid), dim3(256), 0, st, s);
  else hipLaunchKernelGGL((step_kernel<G, false>), dim3(grid), dim3(256), 0, st, s);
}

}  // namespace

int step_counter_words(int units) {
  return units + kLineWords * units + kLineWords * kStepClasses + 1;
}

hipError_t launch_step(const UnitGeom& g, int budget, int n_tail, float sigma, bool query_nvfp4,
                       const _Float16* q,
                       const uint8_t* codes, const uint8_t* scales, const float* gscale,
                       const float* center, const void* k, const void* v,
                       const int32_t* seq_lens, const uint16_t* tail_k, const uint16_t* tail_v,
                       int splits, float* scores, int32_t* idx, int32_t* count, float* part_o,
                       float* part_lse, uint32_t* counters, float* out, float* out_lse,
                       hipStream_t st) {
  if (budget > kFusedSelectMax || splits < 1) return hipErrorInvalidValue;
  const int U = g.B * g.Hkv;
  StepArgs s;
  dim3 scan_grid;
  // up to 8 blocks per wave: each scan item ends with a wait for its stores
  s.scan = make_scan_args(g, n_tail, sigma, q, codes, scales, gscale, center, seq_lens, scores,
                          scan_grid, 8, query_nvfp4);
  AttnArgs& a = s.attn;
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
  a.sel_scores = scores;
  a.sel_idx = idx;
  a.sel_count = count;
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
  s.sync.scan_done = counters + U;
  s.sync.scan_stride = kLineWords;
  s.sync.fault = counters + U + kLineWords * U + kLineWords * kStepClasses;
  s.sync.scan_items = int(scan_grid.x);
  s.tickets = counters + U + kLineWords * U;
  s.units = U;
  s.classes = U < kStepClasses ? U : kStepClasses;
  s.scan_items = int(scan_grid.x);
  s.splits = splits;
  const int64_t per_class = int64_t(ceil_div(U, s.classes)) * (s.scan_items + splits);
  if (per_class * s.classes >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  s.per_class = uint32_t(per_class);
  const uint32_t grid = s.per_class * uint32_t(s.classes);
  const bool bf16 = g.dtype == BSA_DTYPE_BF16;
  switch (g.G) {
    case 1: launch_step_g<1>(grid, st, s, bf16); break;
    case 2: launch_step_g<2>(grid, st, s, bf16); break;
    case 4: launch_step_g<4>(grid, st, s, bf16); break;
    case 8: launch_step_g<8>(grid, st, s, bf16); break;
    case 16: launch_step_g<16>(grid, st, s, bf16); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsa
