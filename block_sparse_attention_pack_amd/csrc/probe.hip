// HBM read-rate probe: how fast can one launch read a given set of tiles?
//
// It measures the ceiling the decode-step kernels are held against: the block
// scan reads long contiguous runs of 9 KiB records, the block attention reads
// 32 KiB key and value tiles at the selected block offsets of a large cache.
// The probe reads the same byte patterns and does nothing else with them than
// fold them into one word (stored only when it equals a value no input here
// produces, so the loads stay live and nothing is written in practice).
//
// Two ways to land the data: ordinary 16-byte vector loads into registers,
// UNROLL loads in flight per thread; or gfx950's global-to-LDS loads, each
// wave streaming through its own ring of NSLOT 1 KiB LDS slots (64 lanes x 16
// bytes per load), one slot read back per load retired.
#include "common.hpp"
#include "../../include/bsa_probe.h"

namespace bsa {
namespace {

constexpr uint32_t kProbeMagic = 0x9E3779B9u;

// grid (ceil(n_tiles / tiles_per_wg)), 256 threads. Tile t starts at byte
// tile_off[t] (16-byte aligned) or, with tile_off null, at t * tile_bytes.
template <int UNROLL>
__global__ __launch_bounds__(256) void probe_vgpr_kernel(const uint8_t* __restrict__ buf,
                                                         const int64_t* __restrict__ tile_off,
                                                         int64_t tile_bytes, int tiles_per_wg,
                                                         int64_t n_tiles, uint32_t* sink) {
  const int64_t n16 = tile_bytes / 16;
  uint32_t acc = 0;
  const int64_t t0 = int64_t(blockIdx.x) * tiles_per_wg;
  const int64_t t1 = min(t0 + tiles_per_wg, n_tiles);
  for (int64_t t = t0; t < t1; ++t) {
    const uint4v* p = reinterpret_cast<const uint4v*>(buf + (tile_off ? tile_off[t] : t * tile_bytes));
    for (int64_t i = threadIdx.x; i < n16; i += 256 * UNROLL) {
      uint4v x[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int64_t j = i + 256 * u;
        x[u] = __builtin_nontemporal_load(p + (j < n16 ? j : i));
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
    }
  }
  if (acc == kProbeMagic) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Short tiles at scattered offsets (the token-mode attention's selected 256-byte
// key and value rows): the work-group's tile offsets are staged in LDS first
// (as the attention stages its row indices), then P = tile_bytes / 16 threads
// read one tile, one 16-byte piece each (P divides 256), so the work-group
// covers 256 / P tiles per step, UNROLL steps in flight per thread.
constexpr int kProbeRowsMax = 1024;  // tiles per work-group in this mode
template <int UNROLL>
__global__ __launch_bounds__(256) void probe_rows_kernel(const uint8_t* __restrict__ buf,
                                                         const int64_t* __restrict__ tile_off,
                                                         int64_t tile_bytes, int tiles_per_wg,
                                                         int64_t n_tiles, uint32_t* sink) {
  __shared__ int64_t offs[kProbeRowsMax];
  const int P = int(tile_bytes / 16);
  const int per_step = 256 / P;
  const int piece = threadIdx.x % P;
  const int64_t t0 = int64_t(blockIdx.x) * tiles_per_wg;
  const int n = int(min(int64_t(tiles_per_wg), n_tiles - t0));
  for (int i = threadIdx.x; i < n; i += 256) offs[i] = tile_off ? tile_off[t0 + i] : (t0 + i) * tile_bytes;
  __syncthreads();
  uint32_t acc = 0;
  for (int t = threadIdx.x / P; t < n; t += per_step * UNROLL) {
    uint4v x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int tt = t + per_step * u < n ? t + per_step * u : t;
      x[u] = __builtin_nontemporal_load(reinterpret_cast<const uint4v*>(buf + offs[tt]) + piece);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  if (acc == kProbeMagic) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// The same reads through LDS: wave w of the work-group takes the 1 KiB pieces
// w, w + 4, ... of each tile (tile_bytes a multiple of 1 KiB) and keeps NSLOT
// of them in flight in its ring.
template <int NSLOT>  // a power of two
__device__ __forceinline__ void probe_lds_body(const uint8_t* __restrict__ buf,
                                               const int64_t* __restrict__ tile_off,
                                               int64_t tile_bytes, int tiles_per_wg,
                                               int64_t n_tiles, uint32_t* sink,
                                               uint32_t (&ring)[4][NSLOT][256]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t pieces = tile_bytes / 1024;
  const int64_t t0 = int64_t(blockIdx.x) * tiles_per_wg;
  const int64_t t1 = min(t0 + tiles_per_wg, n_tiles);
  const int64_t per_tile = pieces > wave ? (pieces - wave + 3) / 4 : 0;
  const int64_t total = per_tile * (t1 > t0 ? t1 - t0 : 0);  // this wave's pieces
  // the next piece to issue: tile it, piece ip of it (no divisions in the loop)
  int64_t it = t0, ip = 0;
  auto issue = [&](int64_t k) {
    const int64_t pc = wave + 4 * ip;
    const uint8_t* src = buf + (tile_off ? tile_off[it] : it * tile_bytes) + pc * 1024 + 16 * lane;
    __builtin_amdgcn_global_load_lds(src, &ring[wave][k % NSLOT][0], 16, 0, 0);
    if (++ip == per_tile) {
      ip = 0;
      ++it;
    }
  };
  uint32_t acc = 0;
  const int pre = total < NSLOT ? int(total) : NSLOT;
  for (int k = 0; k < pre; ++k) issue(k);
  for (int64_t k = 0; k < total; ++k) {
    // the oldest load has landed once at most NSLOT - 1 newer ones are pending
    const int64_t left = total - 1 - k;
    const int newer = left < NSLOT - 1 ? int(left) : NSLOT - 1;
    switch (newer) {
#define BSA_PROBE_WAIT(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
      BSA_PROBE_WAIT(0) BSA_PROBE_WAIT(1) BSA_PROBE_WAIT(2) BSA_PROBE_WAIT(3)
      BSA_PROBE_WAIT(4) BSA_PROBE_WAIT(5) BSA_PROBE_WAIT(6) BSA_PROBE_WAIT(7)
      BSA_PROBE_WAIT(8) BSA_PROBE_WAIT(9) BSA_PROBE_WAIT(10) BSA_PROBE_WAIT(11)
      BSA_PROBE_WAIT(12) BSA_PROBE_WAIT(13) BSA_PROBE_WAIT(14) BSA_PROBE_WAIT(15)
      BSA_PROBE_WAIT(16) BSA_PROBE_WAIT(17) BSA_PROBE_WAIT(18) BSA_PROBE_WAIT(19)
      BSA_PROBE_WAIT(20) BSA_PROBE_WAIT(21) BSA_PROBE_WAIT(22) BSA_PROBE_WAIT(23)
      BSA_PROBE_WAIT(24) BSA_PROBE_WAIT(25) BSA_PROBE_WAIT(26) BSA_PROBE_WAIT(27)
      BSA_PROBE_WAIT(28) BSA_PROBE_WAIT(29) BSA_PROBE_WAIT(30) BSA_PROBE_WAIT(31)
#undef BSA_PROBE_WAIT
      default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
    const uint32_t* slot = &ring[wave][k % NSLOT][0];
    acc ^= slot[lane * 4] ^ slot[lane * 4 + 3];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read before it is refilled
    if (k + NSLOT < total) issue(k + NSLOT);
  }
  if (acc == kProbeMagic) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int NSLOT>
__global__ __launch_bounds__(256) void probe_lds_kernel(const uint8_t* __restrict__ buf,
                                                        const int64_t* __restrict__ tile_off,
                                                        int64_t tile_bytes, int tiles_per_wg,
                                                        int64_t n_tiles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint32_t ring[4][NSLOT][256];
  probe_lds_body<NSLOT>(buf, tile_off, tile_bytes, tiles_per_wg, n_tiles, sink, ring);
}

int probe_read(const void* buf, int64_t buf_bytes, const int64_t* tile_off, int64_t n_tiles,
               int64_t tile_bytes, int32_t tiles_per_group, int32_t mode, int32_t depth,
               uint32_t* sink, void* stream) {
  if (!buf || !sink || n_tiles <= 0 || tile_bytes <= 0 || tile_bytes % 16 || tiles_per_group <= 0)
    return BSA_ERR_INVALID_ARG;
  if (!tile_off && n_tiles > buf_bytes / tile_bytes) return BSA_ERR_INVALID_ARG;
  if (mode == 1 && tile_bytes % 1024) return BSA_ERR_INVALID_ARG;
  if (mode == 2 && (tile_bytes > 4096 || 4096 % tile_bytes || tiles_per_group > kProbeRowsMax))
    return BSA_ERR_INVALID_ARG;
  const int64_t groups = (n_tiles + tiles_per_group - 1) / tiles_per_group;
  if (groups > 0x7FFFFFFF) return BSA_ERR_INVALID_ARG;
  const dim3 grid{static_cast<uint32_t>(groups)}, block{256};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
#define BSA_PROBE(KERNEL, N) \
  hipLaunchKernelGGL((KERNEL<N>), grid, block, 0, s, b, tile_off, tile_bytes, tiles_per_group, n_tiles, sink)
  if (mode == 0) {
    switch (depth) {
      case 1: BSA_PROBE(probe_vgpr_kernel, 1); break;
      case 2: BSA_PROBE(probe_vgpr_kernel, 2); break;
      case 4: BSA_PROBE(probe_vgpr_kernel, 4); break;
      case 8: BSA_PROBE(probe_vgpr_kernel, 8); break;
      default: return BSA_ERR_UNSUPPORTED;
    }
  } else if (mode == 1) {
    switch (depth) {
      case 4: BSA_PROBE(probe_lds_kernel, 4); break;
      case 8: BSA_PROBE(probe_lds_kernel, 8); break;
      case 16: BSA_PROBE(probe_lds_kernel, 16); break;
      case 32: BSA_PROBE(probe_lds_kernel, 32); break;
      default: return BSA_ERR_UNSUPPORTED;
    }
  } else if (mode == 2) {
    switch (depth) {
      case 1: BSA_PROBE(probe_rows_kernel, 1); break;
      case 2: BSA_PROBE(probe_rows_kernel, 2); break;
      case 4: BSA_PROBE(probe_rows_kernel, 4); break;
      case 8: BSA_PROBE(probe_rows_kernel, 8); break;
      default: return BSA_ERR_UNSUPPORTED;
    }
  } else {
    return BSA_ERR_UNSUPPORTED;
  }
#undef BSA_PROBE
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace
}  // namespace bsa

extern "C" int bsa_probe_read(const void* buf, int64_t buf_bytes, const int64_t* tile_off,
                              int64_t n_tiles, int64_t tile_bytes, int32_t tiles_per_group,
                              int32_t mode, int32_t depth, uint32_t* sink, void* stream) {
  return bsa::probe_read(buf, buf_bytes, tile_off, n_tiles, tile_bytes, tiles_per_group, mode,
                         depth, sink, stream);
}
