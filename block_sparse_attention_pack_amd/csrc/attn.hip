// Sparse decode attention over the selected rows, as split partials.
//
// Jet-QSparse abstract: the chosen 128-token blocks are aggregated in FP16 with
// FP32 accumulation from contiguous tiles; up to two newest pages live in BF16.
// JSSA Figure 1: the KV head's query heads share one index set and read the
// original keys and values at those rows in place (no gather buffer).
//
// Work-group = (split s, unit); its 4 waves take the split's tiles round-robin
// and keep their own online-softmax state, merged through LDS at the end. A
// tile is one selected block (block mode) or 32 consecutive selected tokens
// (token mode), processed as groups of 16 rows:
//   QK^T: v_mfma_f32_16x16x32_f16, A = the group's query heads (rows >= G are
//         zero), B = 16 key rows, lane l holding row l % 16, channels
//         32 (l/16) .. +31 -- one 64-byte run of the row per lane. BF16 rows
//         (tail pages or a BF16 cache) use two bf16 MFMAs with q split exactly
//         into q_hi + q_lo (an fp16 value is the sum of two bf16 values).
//   softmax: FP32 in the log2 domain, one max/rescale per tile.
//   PV: VALU FMAs in FP32; lane owns DPL consecutive channels of one row subset,
//       so a wave load covers whole 256-byte value rows; probabilities come
//       from a per-wave LDS table.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kAttnWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int G>
struct PvShape {
  static constexpr int DPL = G <= 4 ? 8 : (G == 8 ? 4 : 2);  // channels per lane
  static constexpr int LPR = kHeadDim / DPL;                  // lanes per row
  static constexpr int NQ = kWave / LPR;                      // rows per wave load
};

__device__ __forceinline__ void split_bf16(const half8& q, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = float(q[e]);
    const __bf16 h = __bf16(f);
    hi[e] = h;
    lo[e] = __bf16(f - float(h));  // exact: f has 11 significant bits, h the top 8
  }
}

template <int DPL, bool BF16>
__device__ __forceinline__ void load_v(const uint16_t* p, float* v) {
  if constexpr (DPL == 8) {
    const uint4v w = *reinterpret_cast<const uint4v*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (BF16) {
        v[2 * e] = bf16_bits_to_float(w[e] & 0xFFFFu);
        v[2 * e + 1] = bf16_bits_to_float(w[e] >> 16);
      } else {
        v[2 * e] = half_bits_to_float(uint16_t(w[e] & 0xFFFFu));
        v[2 * e + 1] = half_bits_to_float(uint16_t(w[e] >> 16));
      }
    }
  } else if constexpr (DPL == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    const uint32_t ww[2] = {w.x, w.y};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      v[2 * e] = BF16 ? bf16_bits_to_float(ww[e] & 0xFFFFu) : half_bits_to_float(uint16_t(ww[e]));
      v[2 * e + 1] = BF16 ? bf16_bits_to_float(ww[e] >> 16) : half_bits_to_float(uint16_t(ww[e] >> 16));
    }
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = BF16 ? bf16_bits_to_float(w & 0xFFFFu) : half_bits_to_float(uint16_t(w));
    v[1] = BF16 ? bf16_bits_to_float(w >> 16) : half_bits_to_float(uint16_t(w >> 16));
  }
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct AttnArgs {
  const _Float16* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  const int32_t* idx;
  const int32_t* count;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
  float* part_o;
  float* part_lse;
  int64_t sb, sh, st;
  int Hkv, Hq, Tmax, budget, n_tail, splits;
  float scale_log2;  // sigma * log2(e)
};

template <int G, bool MAIN_BF16, int NG>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a, int block_mode) {
  using PV = PvShape<G>;
  constexpr int DPL = PV::DPL, LPR = PV::LPR, NQ = PV::NQ;
  constexpr int TROWS = 16 * NG;
  // the per-wave probability tables and, after the tile loop, the waves'
  // accumulators share one LDS buffer
  constexpr int kPFloats = TROWS * G, kAccFloats = G * kHeadDim;
  constexpr int kShare = kPFloats > kAccFloats ? kPFloats : kAccFloats;
  __shared__ float pa_lds[kAttnWaves * kShare];
  __shared__ float alpha_lds[kAttnWaves][16];
  __shared__ int row_lds[kAttnWaves][TROWS];
  __shared__ float m_lds[kAttnWaves][16], l_lds[kAttnWaves][16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, unit = blockIdx.y;
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  const int L = clamp_len(a.seq_lens[b], a.Tmax);
  const int npg = ceil_div(L, kBlock);
  const int tail0 = npg - a.n_tail;  // first page held in the tail store
  const int per = ceil_div(a.budget, a.splits);
  const int cnt = min(max(a.count[unit], 0), a.budget);
  const int e0 = split * per;
  const int e1 = min(min(e0 + per, a.budget), cnt);
  const int32_t* uidx = a.idx + int64_t(unit) * a.budget;

  // query operands: lane l holds head row l % 16, channels 32 (l/16) + 8 c .. + 8
  const int n16 = lane & 15, j4 = lane >> 4;
  half8 qa[4];
  {
    const bool ok = n16 < G;
    const _Float16* qrow =
        a.q + (int64_t(b) * a.Hq + h * G + (ok ? n16 : 0)) * kHeadDim + 32 * j4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      half8 v = *reinterpret_cast<const half8*>(qrow + 8 * c);
      qa[c] = ok ? v : half8{};
    }
  }

  float m[4], lsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -__builtin_inff();
    lsum[r] = 0.0f;
  }
  float acc[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.0f;

  const int dc = lane % LPR, qsub = lane / LPR;
  float* pw = pa_lds + wave * kShare;
  int* rw = row_lds[wave];

  // tiles of this split: block mode one entry per tile, token mode TROWS entries
  const int ent_per_tile = block_mode ? 1 : TROWS;
  const int ntiles = e1 > e0 ? ceil_div(e1 - e0, ent_per_tile) : 0;
  for (int tile = wave; tile < ntiles; tile += kAttnWaves) {
    // ---- row addressing ---------------------------------------------------
    bool tile_bf16 = MAIN_BF16;
    const uint16_t* kb = a.k + b * a.sb + h * a.sh;
    const uint16_t* vb = a.v + b * a.sb + h * a.sh;
    int64_t rstride = a.st;
    int nvalid_rows;
    if (block_mode) {
      const int blk = uidx[e0 + tile];
      if (blk < 0 || blk >= npg) continue;
      nvalid_rows = min(kBlock, L - blk * kBlock);
      if (a.n_tail > 0 && blk >= tail0) {
        const int64_t off = ((int64_t(unit) * a.n_tail + (blk - tail0)) * kBlock) * kHeadDim;
        kb = a.tail_k + off;
        vb = a.tail_v + off;
        rstride = kHeadDim;
        tile_bf16 = true;
      } else {
        kb += int64_t(blk) * kBlock * a.st;
        vb += int64_t(blk) * kBlock * a.st;
      }
      // rows are tau * rstride for tau < nvalid_rows
#pragma unroll
      for (int t = lane; t < TROWS; t += kWave) rw[t] = t < nvalid_rows ? t : -1;
    } else {
      const int t0 = e0 + tile * TROWS;
      for (int t = lane; t < TROWS; t += kWave) {
        const int e = t0 + t;
        const int tok = e < e1 ? uidx[e] : -1;
        rw[t] = (tok >= 0 && tok < L) ? tok : -1;
      }
      nvalid_rows = TROWS;
    }
    wave_lds_fence();

    // ---- scores: s[g][r] = log2-scaled logit of head 4 j4 + r, row 16 g + n16
    float s[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int row = rw[16 * g + n16];
      const bool ok = row >= 0;
      const uint16_t* kp = kb + int64_t(ok ? row : 0) * rstride + 32 * j4;
      uint4v w[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = reinterpret_cast<const uint4v*>(kp)[c];
      float4v d = {0.0f, 0.0f, 0.0f, 0.0f};
      if (!tile_bf16) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          half8 kv;
          __builtin_memcpy(&kv, &w[c], 16);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[c], kv, d, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8 kv, qh, ql;
          __builtin_memcpy(&kv, &w[c], 16);
          split_bf16(qa[c], qh, ql);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kv, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kv, d, 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[g][r] = ok ? d[r] * a.scale_log2 : -__builtin_inff();
    }

    // ---- online softmax update (per head row r of this lane) ----------------
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float tm = s[0][r];
#pragma unroll
      for (int g = 1; g < NG; ++g) tm = fmaxf(tm, s[g][r]);
      tm = row16_max(tm);
      const float mn = fmaxf(m[r], tm);
      const bool live = mn > -__builtin_inff();
      alpha[r] = live ? __builtin_amdgcn_exp2f(m[r] - mn) : 1.0f;
      float ps = 0.0f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float p = live ? __builtin_amdgcn_exp2f(s[g][r] - mn) : 0.0f;
        s[g][r] = p;
        ps += p;
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, kWave);
      lsum[r] = lsum[r] * alpha[r] + ps;
      m[r] = mn;
    }
    // probabilities and rescale factors to LDS (heads < G only)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 4 * j4 + r;
      if (hh < G) {
#pragma unroll
        for (int g = 0; g < NG; ++g) pw[(16 * g + n16) * G + hh] = s[g][r];
        if (n16 == 0) alpha_lds[wave][hh] = alpha[r];
      }
    }
    wave_lds_fence();

    // ---- PV: acc[hh][e] = acc * alpha + sum_rows p * v ----------------------
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float al = alpha_lds[wave][hh];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] *= al;
    }
#pragma unroll 2
    for (int rr = qsub; rr < TROWS; rr += NQ) {
      const int row = rw[rr];
      if (row < 0) continue;
      float vv[DPL];
      const uint16_t* vp = vb + int64_t(row) * rstride + dc * DPL;
      if (tile_bf16) load_v<DPL, true>(vp, vv);
      else load_v<DPL, false>(vp, vv);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = pw[rr * G + hh];
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[hh][e] = __builtin_fmaf(p, vv[e], acc[hh][e]);
      }
    }
    wave_lds_fence();
  }

  // ---- merge the waves' states -------------------------------------------
  __syncthreads();  // every wave is done with its probability table
  // rows of one channel chunk are spread over NQ lanes: sum them
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      float x = acc[hh][e];
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
      acc[hh][e] = x;
    }
  if (qsub == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) pa_lds[wave * kShare + hh * kHeadDim + dc * DPL + e] = acc[hh][e];
  }
  if (n16 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 4 * j4 + r;
      if (hh < G) {
        m_lds[wave][hh] = m[r];
        l_lds[wave][hh] = lsum[r];
      }
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < G * kHeadDim; o += 256) {
    const int hh = o / kHeadDim, d = o % kHeadDim;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_lds[w][hh]);
    float num = 0.0f, den = 0.0f;
    if (M > -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(m_lds[w][hh] - M);
        num += f * pa_lds[w * kShare + o];
        den += f * l_lds[w][hh];
      }
    }
    const int64_t rowq = int64_t(b) * a.Hq + h * G + hh;
    const bool empty = !(den > 0.0f);
    a.part_o[(rowq * a.splits + split) * kHeadDim + d] = empty ? 0.0f : num / den;
    if (d == 0)
      a.part_lse[rowq * a.splits + split] =
          empty ? -__builtin_inff() : (M + __builtin_amdgcn_logf(den)) * kLn2;
  }
}

template <int G, bool BF16, int NG>
void launch_one(dim3 grid, hipStream_t s, const AttnArgs& a, int block_mode) {
  hipLaunchKernelGGL((attn_kernel<G, BF16, NG>), grid, dim3(256), 0, s, a, block_mode);
}

template <int G>
void launch_g(dim3 grid, hipStream_t s, const AttnArgs& a, int block_mode, bool bf16) {
  if (block_mode) {
    if (bf16) launch_one<G, true, 8>(grid, s, a, 1);
    else launch_one<G, false, 8>(grid, s, a, 1);
  } else {
    if (bf16) launch_one<G, true, 2>(grid, s, a, 0);
    else launch_one<G, false, 2>(grid, s, a, 0);
  }
}

}  // namespace

hipError_t launch_attention(const UnitGeom& g, int granularity, int budget, int n_tail,
                            float sigma, const _Float16* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* idx, const int32_t* count,
                            const uint16_t* tail_k, const uint16_t* tail_v, int splits,
                            float* part_o, float* part_lse, hipStream_t s) {
  AttnArgs a;
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
