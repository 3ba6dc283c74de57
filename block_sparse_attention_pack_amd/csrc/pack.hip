// Packers of the key copies (off the timed decode path).
//
// Block mode: NVFP4 -- E2M1 elements, one E4M3 scale per 16 channels, one FP32
// scale per KV head, keys centered first (Jet-QSparse abstract: NVFP4 cache,
// calibrated key centering, packed straight from the 16-bit activations).
// Token mode: projected keys kproj = P^T k, stored as BF16 or as E4M3FN bytes
// (JSSA Figure 1 and Figure 10).
// The 4-bit value store: value rows in NVFP4 like uncentred keys, one FP32
// scale per KV head (the NVFP4 cache of the Jet-QSparse abstract with its
// values compressed too).
//
// Every rounding step is a single IEEE float32 operation (no contraction into
// fused multiply-adds), so the bytes are reproducible bit for bit.
#pragma clang fp contract(off)

#include "common.hpp"

namespace bsa {
namespace {

template <int DT>
__device__ __forceinline__ void load16(const uint16_t* p, float* out) {
  const uint4v a = *reinterpret_cast<const uint4v*>(p);
  const uint4v b = *reinterpret_cast<const uint4v*>(p + 8);
  const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (DT == BSA_DTYPE_F16) {
      out[2 * i] = half_bits_to_float(uint16_t(w[i] & 0xFFFFu));
      out[2 * i + 1] = half_bits_to_float(uint16_t(w[i] >> 16));
    } else {
      out[2 * i] = bf16_bits_to_float(w[i] & 0xFFFFu);
      out[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
    }
  }
}

// One 16-channel group in NVFP4 under the FP32 scale s: the E4M3 scale byte is
// returned, the 16 E2M1 codes are packed into lo (channels 0..7) and hi (8..15),
// channel u in bits 4 (u % 8) .. +3. y holds the group's (centred) values.
__device__ __forceinline__ uint32_t nvfp4_group(const float (&y)[16], float s, uint32_t& lo,
                                                uint32_t& hi) {
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u) amax = fmaxf(amax, __builtin_fabsf(y[u]));
  const uint32_t sbyte = e4m3_from_float(amax / (6.0f * s));
  const float S = e4m3_to_float(sbyte) * s;
  lo = hi = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const uint32_t c = S > 0.0f ? e2m1_from_float(y[u] / S) : 0u;
    if (u < 8) lo |= c << (4 * u);
    else hi |= c << (4 * (u - 8));
  }
  return sbyte;
}

// One work-group packs one (unit, block): 1024 (token, 16-channel group) items,
// four per thread. Consecutive threads take consecutive groups of one token.
template <int DT>
__global__ __launch_bounds__(256) void pack_nvfp4_kernel(
    const uint16_t* __restrict__ k, const float* __restrict__ center,
    const float* __restrict__ gscale, int Hkv, int NBmax, int64_t sb, int64_t sh, int64_t st,
    int blk0, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int blk = blk0 + blockIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / Hkv, h = unit % Hkv;
  const float s_t = gscale[h];
  uint8_t* crec = codes + (int64_t(unit) * NBmax + blk) * kCodeRecord;
  uint8_t* srec = scales + (int64_t(unit) * NBmax + blk) * kScaleRecord;
  const uint16_t* kb = k + b * sb + h * sh + int64_t(blk) * kBlock * st;
#pragma unroll 1
  for (int r = 0; r < 4; ++r) {
    const int item = threadIdx.x + 256 * r;
    const int tau = item >> 3, g = item & 7;
    float y[16];
    load16<DT>(kb + tau * st + 16 * g, y);
#pragma unroll
    for (int u = 0; u < 16; ++u) y[u] = y[u] - (center ? center[h * kHeadDim + 16 * g + u] : 0.0f);
    uint32_t lo, hi;
    const uint32_t sbyte = nvfp4_group(y, s_t, lo, hi);
    const int i = tau >> 4, n = tau & 15, j = g >> 1, s = g & 1;
    uint32_t* dst = reinterpret_cast<uint32_t*>(crec + ((i * 4 + j) * 16 + n) * 16 + 8 * s);
    dst[0] = lo;
    dst[1] = hi;
    srec[((j * 16 + n) * 8 + i) * 2 + s] = uint8_t(sbyte);
  }
}

// The value store: one work-group packs the 128 rows of one (unit, block),
// four (row, 16-channel group) items per thread; work-group (0, 0) also copies
// the per-KV-head scales into the store.
template <int DT>
__global__ __launch_bounds__(256) void pack_values_kernel(
    const uint16_t* __restrict__ v, const float* __restrict__ vscale, int Hkv, int Tmax,
    int64_t sb, int64_t sh, int64_t st, int blk0, int blk1, ValueStore vs) {
  const int unit = blockIdx.y;
  if (blockIdx.x == 0 && unit == 0)
    for (int h = threadIdx.x; h < Hkv; h += 256) vs.s_v[h] = vscale[h];
  const int blk = blk0 + blockIdx.x;
  if (blk >= blk1) return;
  const int b = unit / Hkv, h = unit % Hkv;
  const float s_v = vscale[h];
  const uint16_t* vb = v + b * sb + h * sh + int64_t(blk) * kBlock * st;
  const int64_t row0 = int64_t(unit) * Tmax + int64_t(blk) * kBlock;
#pragma unroll 1
  for (int r = 0; r < 4; ++r) {
    const int item = threadIdx.x + 256 * r;
    const int tau = item >> 3, g = item & 7;
    float y[16];
    load16<DT>(vb + tau * st + 16 * g, y);
    uint32_t lo, hi;
    const uint32_t sbyte = nvfp4_group(y, s_v, lo, hi);
    uint32_t* dst = reinterpret_cast<uint32_t*>(vs.codes + (row0 + tau) * kValueCodeRow + 8 * g);
    dst[0] = lo;
    dst[1] = hi;
    vs.scales[(row0 + tau) * kValueScaleRow + g] = uint8_t(sbyte);
  }
}

// Projected keys: one thread per (token, output channel); the float32 sum runs
// over d in ascending order with separately rounded products and additions.
template <int DT, bool FP8>
__global__ __launch_bounds__(256) void pack_proj_kernel(
    const uint16_t* __restrict__ k, const float* __restrict__ proj, int Hkv, int Tmax,
    int64_t sb, int64_t sh, int64_t st, int rank, int tok0, int ntok,
    void* __restrict__ kproj) {
  const int unit = blockIdx.y;
  const int b = unit / Hkv, h = unit % Hkv;
  const int64_t item = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (item >= int64_t(ntok) * rank) return;
  const int t = tok0 + int(item / rank), j = int(item % rank);
  const uint16_t* kr = k + b * sb + h * sh + int64_t(t) * st;
  const float* P = proj + int64_t(h) * kHeadDim * rank + j;
  float acc = 0.0f;
  for (int d = 0; d < kHeadDim; d += 16) {
    float kv[16];
    load16<DT>(kr + d, kv);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float prod = P[(d + u) * rank] * kv[u];
      acc = acc + prod;
    }
  }
  const int64_t at = (int64_t(unit) * Tmax + t) * rank + j;
  const uint32_t u = __float_as_uint(acc);
  if constexpr (FP8) {
    // nearest E4M3FN code of |acc|, sign bit copied (inputs are finite)
    const uint32_t code = e4m3_from_float(__builtin_fabsf(acc)) | ((u >> 24) & 0x80u);
    static_cast<uint8_t*>(kproj)[at] = uint8_t(code);
  } else {
    // float32 -> bfloat16, round to nearest even (inputs are finite)
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    static_cast<uint16_t*>(kproj)[at] = uint16_t(rounded);
  }
}

// Decode-time append, one work-group per unit: the new token's cache rows, its
// 4-bit records (block mode; a token's records depend on its own row only) or
// projected key (token mode), and the BF16 tail store (slot s holds page
// n_pages - n_tail + s: a token that starts a page shifts the slots down by
// one, and the last slot then takes the new page).
struct AppendArgs {
  const uint16_t* k_new;  // [B][Hkv][128], cache dtype
  const uint16_t* v_new;
  const int32_t* seq_lens;
  uint16_t* k;
  uint16_t* v;
  int64_t sb, sh, st;
  const float* center;
  const float* gscale;
  uint8_t* codes;   // block mode (else null)
  uint8_t* scales;
  const float* proj;  // token mode (else null)
  void* kproj;
  bool fp8;
  uint16_t* tail_k;  // n_tail > 0 (else null)
  uint16_t* tail_v;
  ValueStore vs;     // codes non-null: v is the 4-bit value store
  int Hkv, Tmax, NBmax, rank, n_tail;
};

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {  // finite x
  const uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int DT>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  const int L = a.seq_lens[b];
  if (L < 0 || L >= a.Tmax) return;  // a full (or invalid) sequence is left unchanged
  const uint16_t* kn = a.k_new + int64_t(unit) * kHeadDim;
  const uint16_t* vn = a.v_new + int64_t(unit) * kHeadDim;
  // the cache rows
  if (tid < kHeadDim) {
    a.k[b * a.sb + h * a.sh + int64_t(L) * a.st + tid] = kn[tid];
    if (!a.vs.codes) a.v[b * a.sb + h * a.sh + int64_t(L) * a.st + tid] = vn[tid];
  }
  // the value store: the token's row, as pack_values_kernel packs it
  if (a.vs.codes && tid >= 64 && tid < 72) {
    const int g = tid - 64;
    float y[16];
    load16<DT>(vn + 16 * g, y);
    uint32_t lo, hi;
    const uint32_t sbyte = nvfp4_group(y, a.vs.s_v[h], lo, hi);
    const int64_t row = int64_t(unit) * a.Tmax + L;
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.vs.codes + row * kValueCodeRow + 8 * g);
    dst[0] = lo;
    dst[1] = hi;
    a.vs.scales[row * kValueScaleRow + g] = uint8_t(sbyte);
  }
  // block mode: the token's records, as pack_nvfp4_kernel writes them
  if (a.codes && tid < 8) {
    const int g = tid, blk = L / kBlock, tau = L % kBlock;
    const float s_t = a.gscale[h];
    float y[16];
    load16<DT>(kn + 16 * g, y);
#pragma unroll
    for (int u = 0; u < 16; ++u)
      y[u] = y[u] - (a.center ? a.center[h * kHeadDim + 16 * g + u] : 0.0f);
    uint32_t lo, hi;
    const uint32_t sbyte = nvfp4_group(y, s_t, lo, hi);
    uint8_t* crec = a.codes + (int64_t(unit) * a.NBmax + blk) * kCodeRecord;
    uint8_t* srec = a.scales + (int64_t(unit) * a.NBmax + blk) * kScaleRecord;
    const int i = tau >> 4, n = tau & 15, j = g >> 1, s = g & 1;
    uint32_t* dst = reinterpret_cast<uint32_t*>(crec + ((i * 4 + j) * 16 + n) * 16 + 8 * s);
    dst[0] = lo;
    dst[1] = hi;
    srec[((j * 16 + n) * 8 + i) * 2 + s] = uint8_t(sbyte);
  }
  // token mode: the projected key, as pack_proj_kernel forms it
  if (a.kproj && tid < a.rank) {
    const int j = tid;
    const float* P = a.proj + int64_t(h) * kHeadDim * a.rank + j;
    float acc = 0.0f;
    for (int d = 0; d < kHeadDim; d += 16) {
      float kv[16];
      load16<DT>(kn + d, kv);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float prod = P[(d + u) * a.rank] * kv[u];
        acc = acc + prod;
      }
    }
    const int64_t at = (int64_t(unit) * a.Tmax + L) * a.rank + j;
    if (a.fp8) {
      const uint32_t code = e4m3_from_float(__builtin_fabsf(acc)) | ((__float_as_uint(acc) >> 24) & 0x80u);
      static_cast<uint8_t*>(a.kproj)[at] = uint8_t(code);
    } else {
      static_cast<uint16_t*>(a.kproj)[at] = bf16_rne_bits(acc);
    }
  }
  // the BF16 tail store
  if (a.n_tail > 0) {
    constexpr int kSlotVec = kBlock * kHeadDim / 8;  // 16-byte vectors per slot
    uint4v* tk = reinterpret_cast<uint4v*>(a.tail_k + int64_t(unit) * a.n_tail * kBlock * kHeadDim);
    uint4v* tv = reinterpret_cast<uint4v*>(a.tail_v + int64_t(unit) * a.n_tail * kBlock * kHeadDim);
    if (L % kBlock == 0) {  // a new page: slots down by one, the last one cleared
      for (int sl = 0; sl + 1 < a.n_tail; ++sl) {
        for (int e = tid; e < kSlotVec; e += 256) {
          const uint4v xk = tk[(sl + 1) * kSlotVec + e], xv = tv[(sl + 1) * kSlotVec + e];
          tk[sl * kSlotVec + e] = xk;
          tv[sl * kSlotVec + e] = xv;
        }
        __syncthreads();  // slot sl + 1 is read before it is overwritten
      }
      const uint4v z = {0u, 0u, 0u, 0u};
      for (int e = tid; e < kSlotVec; e += 256) {
        tk[(a.n_tail - 1) * kSlotVec + e] = z;
        tv[(a.n_tail - 1) * kSlotVec + e] = z;
      }
      __syncthreads();  // cleared before the new row lands
    }
    if (tid < kHeadDim) {
      const int64_t at = (int64_t(unit) * a.n_tail + a.n_tail - 1) * kBlock * kHeadDim +
                         int64_t(L % kBlock) * kHeadDim + tid;
      if (DT == BSA_DTYPE_F16) {
        a.tail_k[at] = bf16_rne_bits(half_bits_to_float(kn[tid]));
        a.tail_v[at] = bf16_rne_bits(half_bits_to_float(vn[tid]));
      } else {
        a.tail_k[at] = kn[tid];
        a.tail_v[at] = vn[tid];
      }
    }
  }
}

}  // namespace

hipError_t launch_append(const UnitGeom& g, int n_tail, int rank, bool fp8, const void* k_new,
                         const void* v_new, const int32_t* seq_lens, void* k, void* v,
                         const float* center, const float* gscale, uint8_t* codes,
                         uint8_t* scales, const float* proj, void* kproj, uint16_t* tail_k,
                         uint16_t* tail_v, hipStream_t s) {
  AppendArgs a;
  a.vs = g.vq ? value_store(g, v) : ValueStore{nullptr, nullptr, nullptr};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.seq_lens = seq_lens;
  a.k = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.sb = g.sb;
  a.sh = g.sh;
  a.st = g.st;
  a.center = center;
  a.gscale = gscale;
  a.codes = codes;
  a.scales = scales;
  a.proj = proj;
  a.kproj = kproj;
  a.fp8 = fp8;
  a.tail_k = tail_k;
  a.tail_v = tail_v;
  a.Hkv = g.Hkv;
  a.Tmax = g.Tmax;
  a.NBmax = g.NBmax;
  a.rank = rank;
  a.n_tail = n_tail;
  if (g.dtype == BSA_DTYPE_F16)
    hipLaunchKernelGGL(append_kernel<BSA_DTYPE_F16>, dim3(g.B * g.Hkv), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<BSA_DTYPE_BF16>, dim3(g.B * g.Hkv), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack_block(const UnitGeom& g, const void* k, const float* center,
                             const float* gscale, int blk0, int blk1, uint8_t* codes,
                             uint8_t* scales, hipStream_t s) {
  if (blk1 <= blk0) return hipSuccess;
  dim3 grid(blk1 - blk0, g.B * g.Hkv);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  if (g.dtype == BSA_DTYPE_F16)
    hipLaunchKernelGGL(pack_nvfp4_kernel<BSA_DTYPE_F16>, grid, dim3(256), 0, s, kp, center,
                       gscale, g.Hkv, g.NBmax, g.sb, g.sh, g.st, blk0, codes, scales);
  else
    hipLaunchKernelGGL(pack_nvfp4_kernel<BSA_DTYPE_BF16>, grid, dim3(256), 0, s, kp, center,
                       gscale, g.Hkv, g.NBmax, g.sb, g.sh, g.st, blk0, codes, scales);
  return hipGetLastError();
}

hipError_t launch_pack_values(const UnitGeom& g, const void* v, const float* vscale, int blk0,
                              int blk1, void* store, hipStream_t s) {
  // an empty range still sets the store's scales
  dim3 grid(blk1 > blk0 ? blk1 - blk0 : 1, blk1 > blk0 ? g.B * g.Hkv : 1);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  const ValueStore vs = value_store(g, store);
  if (g.dtype == BSA_DTYPE_F16)
    hipLaunchKernelGGL(pack_values_kernel<BSA_DTYPE_F16>, grid, dim3(256), 0, s, vp, vscale,
                       g.Hkv, g.Tmax, g.sb, g.sh, g.st, blk0, blk1, vs);
  else
    hipLaunchKernelGGL(pack_values_kernel<BSA_DTYPE_BF16>, grid, dim3(256), 0, s, vp, vscale,
                       g.Hkv, g.Tmax, g.sb, g.sh, g.st, blk0, blk1, vs);
  return hipGetLastError();
}

hipError_t launch_pack_proj(const UnitGeom& g, const void* k, const float* proj, int rank,
                            bool fp8, int blk0, int blk1, void* kproj, hipStream_t s) {
  if (blk1 <= blk0) return hipSuccess;
  const int tok0 = blk0 * kBlock, ntok = (blk1 - blk0) * kBlock;
  const int64_t items = int64_t(ntok) * rank;
  dim3 grid(unsigned((items + 255) / 256), g.B * g.Hkv);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
#define BSA_PACK_PROJ(DT, F8)                                                                \
  hipLaunchKernelGGL((pack_proj_kernel<DT, F8>), grid, dim3(256), 0, s, kp, proj, g.Hkv, g.Tmax, \
                     g.sb, g.sh, g.st, rank, tok0, ntok, kproj)
  if (g.dtype == BSA_DTYPE_F16) {
    if (fp8) BSA_PACK_PROJ(BSA_DTYPE_F16, true);
    else BSA_PACK_PROJ(BSA_DTYPE_F16, false);
  } else {
    if (fp8) BSA_PACK_PROJ(BSA_DTYPE_BF16, true);
    else BSA_PACK_PROJ(BSA_DTYPE_BF16, false);
  }
#undef BSA_PACK_PROJ
  return hipGetLastError();
}

}  // namespace bsa
