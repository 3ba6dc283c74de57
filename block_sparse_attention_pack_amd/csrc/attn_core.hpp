// Sparse decode attention over the selected rows, as split partials.
//
// Jet-QSparse abstract: the chosen 128-token blocks are aggregated in FP16 with
// FP32 accumulation from contiguous tiles; up to two newest pages live in BF16.
// JSSA Figure 1: the KV head's query heads share one index set and read the
// original keys and values at those rows in place (no gather buffer).
//
// Work-group = (split s, unit). Split s takes entries [s * per, min((s + 1) *
// per, count)) of the unit's selection, per = ceil(count / S). Its rows are cut
// into groups of 16 (an eighth of a selected block, or 16 consecutive selected
// tokens), dealt round-robin to the 4 waves. Each wave streams its groups
// through one software pipeline with no phases: the next group's keys and
// values are in flight while a group is used, so the HBM sees a steady stream
// from the first group to the last.
//
// Both products run on the matrix cores, in transposed form, so that the
// scores land in each lane exactly where the second product takes them: no
// LDS round trip and no lane exchange between the two. Lane l = (j, n),
// j = l / 16, n = l % 16, stands for head n throughout. Per group:
//   1. S^T = K Q^T on v_mfma_f32_16x16x32_f16. A = the group's 16 key rows,
//      lane l holding row l % 16 and, for MFMA step c, channels 8 (l/16 + 4 c)
//      .. +7, so each wave load reads 64 contiguous bytes of every row; B = the
//      query heads (heads >= G zero). Lane (j, n) receives the scores of head
//      n at rows 4 j .. 4 j + 3. BF16 rows (tail pages or a BF16 cache) take
//      two bf16 MFMAs with q split exactly into q_hi + q_lo (an fp16 value is
//      the sum of two bf16 values).
//   2. An online softmax in the log2 domain: head n's maximum and sum over the
//      16 rows are the lane's four values combined with those of the three
//      other lanes of head n by two lane-swap steps (v_permlane16_swap,
//      v_permlane32_swap), so those four lanes hold the same running maximum
//      and sum, bit for bit.
//   3. O^T += V^T P^T on v_mfma_f32_16x16x16. B = P^T is what step 2 left in
//      the lane (rows 4 j .. 4 j + 3 of head n). A = V^T, with channel slot m
//      of MFMA step c standing for channel 8 m + c: lane (j, n) loads the 16
//      contiguous bytes of channels 8 n .. 8 n + 7 of its rows 4 j .. 4 j + 3
//      (a wave load covers four whole 256-byte rows), and one byte permute per
//      operand dword puts the rows in the MFMA's K order. The probabilities
//      enter as two 16-bit parts p = p_hi + p_lo, each rounded to nearest, so
//      the products carry 22 (fp16) or 17 (bf16) significant bits of p, and
//      accumulate in FP32. Lane (j, n) accumulates head n, channels 32 j ..
//      32 j + 31. The accumulators are rescaled only when some head's maximum
//      grew.
//      From the 4-bit value store a lane loads the four code bytes of its
//      channels in each of its rows, and the one E4M3 scale byte they share.
//      The hardware FP4 convert (run at scale 1: it honours only the exponent
//      of its scale) and one packed f16 multiply by the E4M3 scale give
//      e2m1 * e4m3 exactly in f16 (at most 6 significant bits, in [2^-10,
//      2688]). Those rows accumulate apart from any BF16 tail rows, and the
//      KV head's FP32 scale s_v multiplies their sum at the end: the result
//      is the sum over e2m1 * fl32(e4m3 * s_v), the values the packer rounded
//      to, up to one rounding of each product's scale.
// With block scores given (block mode), every work-group of a unit first makes
// the unit's selection itself (select_unit_rows, the selection select_topk
// makes) into LDS, and the split-0 group also writes idx / count: the
// selection then costs its compute in each group instead of a launch of its
// own between the scan and the attention.
// The row indices (block ids or tokens) a wave needs are staged in LDS a
// window of groups at a time, so no load of the pipeline waits on an index
// load (a vector-memory wait would also wait for every key and value in
// flight). The waves' states are merged through LDS into one (O, lse) partial
// per head; with arrival counters the unit's last work-group also merges the
// splits.
#pragma once

#include "combine_core.hpp"
#include "common.hpp"
#include "select_core.hpp"

namespace bsa {
namespace {

constexpr int kAttnWaves = 4;
// RING (a template argument): 16-row groups of keys and values a wave has in
// flight. One when the grid fills the CUs: with 2048 waves streaming that is
// 16 MiB in flight, enough for the HBM; two groups per wave (32 MiB) queue so
// deep that the work-groups served first finish far ahead of the rest, and
// measured slower (16 x 4 heads at 128K, 64 blocks: 55.9 us with one group,
// 56.8 with two; with 16 splits 65.1 and 61.4). Two when a 16-bit block-mode
// grid leaves CUs with fewer than two work-groups (8 units, 32 splits: 18.8
// against 18.0 us).
constexpr int kRingSmallGrid = 2;

// Where a kernel reads the values: the 16-bit cache (BF16 tail pages too), the
// 4-bit store with no tail pages, or the 4-bit store with BF16 tail pages. In
// the last form every group issues the loads of both forms, the unused ones at
// one fixed line of the unit's store, so that no load sits behind a branch: a
// branch around loads makes the compiler copy the loaded registers at the loop
// end, which waits for every load in flight.
constexpr int kValCache = 0, kValStore = 1, kValStoreTail = 2;
constexpr int kWindow = 32;  // groups whose row indices a wave stages at a time
constexpr int kAccStride = kHeadDim + 4;  // floats per head in the merge table
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void split_bf16(const half8& q, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = float(q[e]);
    const __bf16 h = __bf16(f);
    hi[e] = h;
    lo[e] = __bf16(f - float(h));  // exact: f has 11 significant bits, h the top 8
  }
}

// v combined over lanes n, n + 16, n + 32, n + 48 (n = lane % 16), the same
// bits in all four: permlane16_swap leaves rows (0, 0, 2, 2) in one register
// and (1, 1, 3, 3) in the other, permlane32_swap the low and the high half.
// (The two results are copied out as scalars first: a bit cast applied to an
// element of the returned vector reads element 0.)
template <bool MAX>
__device__ __forceinline__ float heads_reduce(float v) {
  auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  uint32_t x0 = s[0], x1 = s[1];
  float a = __builtin_bit_cast(float, x0), b = __builtin_bit_cast(float, x1);
  v = MAX ? fmaxf(a, b) : a + b;
  s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                       __builtin_bit_cast(uint32_t, v), false, false);
  x0 = s[0];
  x1 = s[1];
  a = __builtin_bit_cast(float, x0);
  b = __builtin_bit_cast(float, x1);
  return MAX ? fmaxf(a, b) : a + b;
}

struct AttnArgs {
  const _Float16* q;
  const uint16_t* k;
  const uint16_t* v;
  ValueStore vs;  // the 4-bit value store (VM != kValCache), else unused
  const int32_t* seq_lens;
  const int32_t* idx;
  const int32_t* count;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
  float* part_o;
  float* part_lse;
  uint32_t* counters;  // non-null: the unit's last group also merges the partials
  float* out;
  float* out_lse;
  const float* sel_scores;  // non-null: select the blocks in the prologue (block mode)
  int32_t* sel_idx;         // where split 0 writes the selection, and its count
  int32_t* sel_count;
  int64_t sb, sh, st;
  int Hkv, Hq, Tmax, budget, n_tail, splits;
  float scale_log2;  // sigma * log2(e)
};

// Per-unit context shared by every row group of the work-group.
struct UnitCtx {
  const uint16_t* kunit;  // K and V of this (sequence, KV head)
  const uint16_t* vunit;
  const uint8_t* vcunit;  // its rows of the value store (VM != kValCache)
  const uint8_t* vsunit;
  float s_v;              // the value store's FP32 scale of this KV head
  const int32_t* uidx;
  const int* nulltoks;  // 16 entries of -1 in LDS (a null group's tokens)
  int e0, e1, L, npg, tail0, unit;
};

// One group of 16 rows: an eighth of a selected block, or 16 consecutive
// selected tokens. Row rho of the group is at kb/vb + row_offset(rho).
struct GroupRef {
  const uint16_t* kb;
  const uint16_t* vb;
  const uint8_t* vc;  // v4: row rho's value codes at vc + 64 row_index(rho),
  const uint8_t* vsb; // its scales at vsb + 8 row_index(rho)
  int64_t rs;       // elements between rows (block mode)
  int nvalid;       // block mode: rows 0 .. nvalid-1 are valid
  const int* toks;  // token mode: the group's 16 staged token indices (-1 = masked)
  bool bf16;
  bool v4;          // the values come from the 4-bit store (else vb, 16-bit)
};

// stage: the wave's staged window; tl: the group's index in it.
//   block mode: stage[tl] = block id of the group
//   token mode: stage[16 tl + rho] = token of row rho, or -1
// live == false gives a null group: every row masked (token mode: its tokens
// are the 16 -1 entries at nulltoks), addresses inside the unit (the same few
// lines every time, so its loads are served from cache).
template <bool MAIN_BF16, bool BLOCK, int VM>
__device__ __forceinline__ GroupRef describe(const AttnArgs& a, const UnitCtx& u, int q,
                                             const int* stage, int tl, bool live) {
  GroupRef r;
  r.toks = u.nulltoks;
  r.kb = u.kunit;
  r.vb = u.vunit;
  r.vc = u.vcunit;
  r.vsb = u.vsunit;
  r.rs = a.st;
  r.nvalid = 0;
  r.bf16 = MAIN_BF16;
  r.v4 = VM != kValCache;
  if (!live) return r;
  if constexpr (BLOCK) {
    // one block per group: its id (and so the branch below) is wave-uniform
    const int blk = __builtin_amdgcn_readfirstlane(stage[tl]);
    const int part = q & 7;
    const bool ok = blk >= 0 && blk < u.npg;
    const int b0 = ok ? blk : 0;
    r.nvalid = ok ? max(0, min(16, u.L - b0 * kBlock - 16 * part)) : 0;
    if (VM != kValStore && a.n_tail > 0 && ok && blk >= u.tail0) {
      const int64_t off =
          ((int64_t(u.unit) * a.n_tail + (blk - u.tail0)) * kBlock + 16 * part) * kHeadDim;
      r.kb = a.tail_k + off;
      r.vb = a.tail_v + off;
      r.rs = kHeadDim;
      r.bf16 = true;
      r.v4 = false;
    } else {
      const int64_t row0 = int64_t(b0) * kBlock + 16 * part;
      r.kb = u.kunit + row0 * a.st;
      r.vb = u.vunit + row0 * a.st;
      r.vc = u.vcunit + row0 * kValueCodeRow;
      r.vsb = u.vsunit + row0 * kValueScaleRow;
    }
  } else {
    r.nvalid = 16;
    r.toks = stage + 16 * tl;
  }
  return r;
}

// Whether row rho of the group holds a valid row.
template <bool BLOCK>
__device__ __forceinline__ bool row_valid(const GroupRef& r, int rho) {
  if constexpr (BLOCK) return rho < r.nvalid;
  else return r.toks[rho] >= 0;
}

// Row of group row rho counted from kb / vb / vc / vsb; masked rows read row 0
// of the group (block mode: a row of a selected block, or of the unit for a
// null group; token mode: row 0 of the unit), which is always inside the cache.
template <bool BLOCK>
__device__ __forceinline__ int row_index(const GroupRef& r, int rho) {
  if constexpr (BLOCK) {
    return rho < r.nvalid ? rho : 0;
  } else {
    const int tok = r.toks[rho];
    return tok >= 0 ? tok : 0;
  }
}

// Element offset of group row rho from kb / vb.
template <bool BLOCK>
__device__ __forceinline__ int64_t row_offset(const GroupRef& r, int rho) {
  return int64_t(row_index<BLOCK>(r, rho)) * r.rs;
}

// Key registers of one group: lane l holds row l % 16, channels 8 (l/16 + 4 c) .. +7
// for MFMA step c, so load c of the wave reads 64 contiguous bytes of each row.
struct KeySlot {
  uint4v w[4];
};

template <bool MAIN_BF16, bool BLOCK, int VM>
__device__ __forceinline__ void issue_keys(KeySlot& ks, const AttnArgs& a, const UnitCtx& u,
                                           int q, const int* stage, int tl, int lane, bool live) {
  const GroupRef r = describe<MAIN_BF16, BLOCK, VM>(a, u, q, stage, tl, live);
  const int64_t off = row_offset<BLOCK>(r, lane & 15);
  // plain loads: each 128-byte line is read by two of the wave's loads, and a
  // streaming (non-temporal) hint can evict it in between
  const uint4v* kp = reinterpret_cast<const uint4v*>(r.kb + off + 8 * (lane >> 4));
#pragma unroll
  for (int c = 0; c < 4; ++c) ks.w[c] = kp[4 * c];
}

// Value registers of one group: lane (j, n) holds channels 8 n .. 8 n + 7 of
// rows 4 j + i, i < 4: as 16-bit values in w[i][0..3] (dword e = channels
// 8 n + 2 e, 8 n + 2 e + 1), or from the 4-bit store as their codes in c4[i]
// and their shared scale byte in sc[i].
template <int VM>
struct ValSlot {
  static constexpr int R16 = VM == kValStore ? 1 : 4;
  static constexpr int R4 = VM == kValCache ? 1 : 4;
  uint32_t w[R16][4];
  uint32_t c4[R4];
  uint32_t sc[R4];
};

template <bool MAIN_BF16, bool BLOCK, int VM>
__device__ __forceinline__ void issue_values(ValSlot<VM>& vs, const AttnArgs& a,
                                             const UnitCtx& u, int q, const int* stage, int tl,
                                             int lane, bool live) {
  const GroupRef r = describe<MAIN_BF16, BLOCK, VM>(a, u, q, stage, tl, live);
  const int n = lane & 15, j = lane >> 4;
  if constexpr (VM != kValCache) {
    // a tail group (kValStoreTail) reads row 0 of the unit's store instead
    const uint8_t* cb = r.v4 ? r.vc : u.vcunit;
    const uint8_t* sb = r.v4 ? r.vsb : u.vsunit;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = r.v4 ? row_index<BLOCK>(r, 4 * j + i) : 0;
      vs.c4[i] = __builtin_nontemporal_load(
          reinterpret_cast<const uint32_t*>(cb + row * kValueCodeRow + 4 * n));
      vs.sc[i] = __builtin_nontemporal_load(sb + row * kValueScaleRow + (n >> 1));
    }
  }
  if constexpr (VM == kValStoreTail) {
    // the BF16 tail rows; a 4-bit group reads the first 256 bytes of the
    // unit's store codes instead (always cached, never used)
    const uint16_t* vb = r.v4 ? reinterpret_cast<const uint16_t*>(u.vcunit) : r.vb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t off = r.v4 ? 0 : row_offset<BLOCK>(r, 4 * j + i);
      const uint4v x = *reinterpret_cast<const uint4v*>(vb + off + 8 * n);
#pragma unroll
      for (int e = 0; e < 4; ++e) vs.w[i][e] = x[e];
    }
  }
  if constexpr (VM == kValCache) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t off = row_offset<BLOCK>(r, 4 * j + i);
      const uint4v x =
          __builtin_nontemporal_load(reinterpret_cast<const uint4v*>(r.vb + off + 8 * n));
#pragma unroll
      for (int e = 0; e < 4; ++e) vs.w[i][e] = x[e];
    }
  }
}

// LDS of one attention work-group.
template <int G>
struct AttnLds {
  int stage[kAttnWaves][16 * kWindow];     // each wave's staged row indices
  bf16x8 qsplit[8 * kWave];                // q = q_hi + q_lo in the MFMA operand order
  float acc[kAttnWaves][G * kAccStride];   // the waves' accumulators for the merge
  float m[kAttnWaves][G], l[kAttnWaves][G];
  int nulltoks[16];  // token mode: a null group's tokens (all -1)
  int is_last;
  int32_t sel[kFusedSelectMax];  // the unit's selection made in the prologue
  SelectLds sel_s;
  int32_t sel_cnt;
};

// The online-softmax state of one wave: lane (j, n) holds the running maximum
// (log2 domain) and sum of head n, the same in the four lanes of the head.
struct SoftState {
  float m, l;
};

// The A operands of the PV product from 16-bit rows: rw[i][e] holds channels
// 8 n + 2 e (low half) and 8 n + 2 e + 1 (high half) of row 4 j + i; MFMA step
// c = 2 e + h takes channel 8 n + c of rows 4 j .. 4 j + 3, as two dwords.
__device__ __forceinline__ void value_operands(const uint32_t (&rw)[4][4], uint2v (&av)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    av[2 * e][0] = __builtin_amdgcn_perm(rw[1][e], rw[0][e], 0x05040100u);
    av[2 * e][1] = __builtin_amdgcn_perm(rw[3][e], rw[2][e], 0x05040100u);
    av[2 * e + 1][0] = __builtin_amdgcn_perm(rw[1][e], rw[0][e], 0x07060302u);
    av[2 * e + 1][1] = __builtin_amdgcn_perm(rw[3][e], rw[2][e], 0x07060302u);
  }
}

// E2M1 codes x (channel 2 b + t in bits 8 b + 4 t .. +3) times the f16 scale
// pair s2, as f16 pairs (channels 2 b, 2 b + 1) in out[b]; the byte to
// convert is an immediate of the instruction.
__device__ __forceinline__ void fp4_row_to_f16(uint32_t x, half2v s2, uint32_t (&out)[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s2);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s2);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s2);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s2);
}

// acc[c] += A_c P^T over the group's 16 rows, P = hi + lo (16-bit parts).
template <bool BF>
__device__ __forceinline__ void pv_mfma(const uint2v (&av)[8], const float (&p)[4],
                                        float4v (&acc)[8]) {
  if constexpr (BF) {
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h = __bf16(p[i]);
      hi[i] = h;
      lo[i] = __bf16(p[i] - float(h));
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x4 a = __builtin_bit_cast(bf16x4, av[c]);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, hi, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, lo, acc[c], 0, 0, 0);
    }
  } else {
    half4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 h = _Float16(p[i]);
      hi[i] = h;
      lo[i] = _Float16(p[i] - float(h));
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const half4 a = __builtin_bit_cast(half4, av[c]);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, hi, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, lo, acc[c], 0, 0, 0);
    }
  }
}

// One landed group: S^T, the online softmax update, O^T += V^T P^T. The state
// and accumulators are updated in place: acc takes the 16-bit rows, or (VM !=
// kValCache) the 4-bit rows before their factor s_v; acct (kValStoreTail
// only) the BF16 tail rows. keys_done() runs once the key registers are read
// (it issues the next group's keys into them, so those loads are in flight
// during this group's softmax and PV).
template <int G, bool BLOCK, int VM, class KeysDone>
__device__ __forceinline__ void attend_group(const KeySlot& ks, const ValSlot<VM>& vs,
                                             const GroupRef& r, const half8 (&qa)[4],
                                             const bf16x8* qsplit, float scale_log2,
                                             SoftState& st, float4v (&acc)[8],
                                             float4v (&acct)[8], int lane, KeysDone&& keys_done) {
  // ---- S^T = K Q^T (lane (j, n): rows 4 j + i of head n) ----
  float4v d = {0.0f, 0.0f, 0.0f, 0.0f};
  if (!r.bf16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      half8 kv;
      __builtin_memcpy(&kv, &ks.w[c], 16);
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qa[c], d, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 kv;
      __builtin_memcpy(&kv, &ks.w[c], 16);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qsplit[(2 * c) * kWave + lane], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qsplit[(2 * c + 1) * kWave + lane], d, 0, 0,
                                                  0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  keys_done();
  __builtin_amdgcn_sched_barrier(0);
  // ---- online softmax ----
  const int n = lane & 15, j = lane >> 4;
  bool rv[4];
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rv[i] = row_valid<BLOCK>(r, 4 * j + i);
    s[i] = rv[i] ? d[i] * scale_log2 : -__builtin_inff();
  }
  const float mx = heads_reduce<true>(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  const float mo = st.m;
  const float mn = fmaxf(mo, mx);
  const bool live = mn > -__builtin_inff();
  const float alpha = live ? __builtin_amdgcn_exp2f(mo - mn) : 1.0f;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = live ? __builtin_amdgcn_exp2f(s[i] - mn) : 0.0f;
  st.m = mn;
  st.l = st.l * alpha + heads_reduce<false>((p[0] + p[1]) + (p[2] + p[3]));
  if (__ballot(n < G && mn > mo) != 0) {  // wave-uniform
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= alpha;
    if constexpr (VM == kValStoreTail) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acct[c] *= alpha;
    }
  }
  // ---- O^T += V^T P^T ----
  // a masked row has p = 0; its value bits are not data, so they are dropped
  // (zero bits, or a zero scale for a 4-bit row: E2M1 has no NaN code)
  uint32_t rw[4][4];
  uint2v av[8];
  if constexpr (VM != kValCache) {
    if (VM == kValStore || r.v4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the scale byte twice, so the convert gives the f16 pair (S, S)
        const uint32_t sb = rv[i] ? vs.sc[i] : 0u;
        fp4_row_to_f16(vs.c4[i], __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb * 0x101u, 1.0f, false),
                       rw[i]);
      }
      value_operands(rw, av);
      pv_mfma<false>(av, p, acc);
      return;
    }
  }
  if constexpr (VM != kValStore) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) rw[i][e] = rv[i] ? vs.w[i][e] : 0u;
    value_operands(rw, av);
    float4v (&dst)[8] = VM == kValStoreTail ? acct : acc;
    if (r.bf16) pv_mfma<true>(av, p, dst);
    else pv_mfma<false>(av, p, dst);
  }
}

// The attention of (split, unit): its rows' partial (O, lse) per head, and the
// merge when a.counters is set.
template <int G, bool MAIN_BF16, bool BLOCK, int VM, int RING>
__device__ __forceinline__ void attn_item(const AttnArgs& a, int split, int unit,
                                          AttnLds<G>& lds) {
  constexpr bool VQ = VM != kValCache;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  UnitCtx u;
  u.unit = unit;
  u.L = clamp_len(a.seq_lens[b], a.Tmax);
  u.npg = ceil_div(u.L, kBlock);
  u.tail0 = u.npg - a.n_tail;  // first page held in the tail store
  u.kunit = a.k + b * a.sb + h * a.sh;
  u.vunit = a.v + b * a.sb + h * a.sh;
  u.vcunit = VQ ? a.vs.codes + int64_t(unit) * a.Tmax * kValueCodeRow : nullptr;
  u.vsunit = VQ ? a.vs.scales + int64_t(unit) * a.Tmax * kValueScaleRow : nullptr;
  u.s_v = VQ ? a.vs.s_v[h] : 1.0f;
  u.nulltoks = lds.nulltoks;

  // query operands: lane l holds head l % 16, channels 8 (l/16 + 4 c) .. + 8
  // for MFMA step c (the key layout above); every wave loads its own, before
  // the selection so that their latency overlaps it
  const int n16 = lane & 15, j4 = lane >> 4;
  half8 qa[4];
  {
    const bool ok = n16 < G;
    const _Float16* qrow = a.q + (int64_t(b) * a.Hq + h * G + (ok ? n16 : 0)) * kHeadDim + 8 * j4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qa[c] = *reinterpret_cast<const half8*>(qrow + 32 * c);
      if (!ok) qa[c] = half8{};
    }
  }
  int cnt;
  if (BLOCK && a.sel_scores) {
    // the unit's selection, made by every group of the unit alike
    const int nb = a.Tmax / kBlock;
    int C, picks, f0, f1;
    block_candidates(u.L, a.n_tail, nb, a.budget, C, picks, f0, f1);
    select_unit_rows(a.sel_scores + int64_t(unit) * nb, C, picks, f0, f1, a.budget, lds.sel,
                     &lds.sel_cnt, lds.sel_s);
    __syncthreads();
    cnt = lds.sel_cnt;
    u.uidx = lds.sel;
    if (split == 0) {
      for (int i = threadIdx.x; i < a.budget; i += 256)
        a.sel_idx[int64_t(unit) * a.budget + i] = lds.sel[i];
      if (threadIdx.x == 0) a.sel_count[unit] = cnt;
    }
  } else {
    cnt = a.count[unit];
    u.uidx = a.idx + int64_t(unit) * a.budget;
  }
  cnt = min(max(cnt, 0), a.budget);
  const int per = ceil_div(cnt, a.splits);
  u.e0 = min(split * per, cnt);
  u.e1 = min(u.e0 + per, cnt);
  // BF16 rows need q = q_hi + q_lo, staged once by wave 0
  const bool any_bf16 = MAIN_BF16 || (BLOCK && a.n_tail > 0);
  if (any_bf16 || !BLOCK) {
    if (wave == 0) {
      if (any_bf16) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          split_bf16(qa[c], lds.qsplit[(2 * c) * kWave + lane],
                     lds.qsplit[(2 * c + 1) * kWave + lane]);
      }
      if (!BLOCK && lane < 16) lds.nulltoks[lane] = -1;
    }
    __syncthreads();
  }

  // 16-row groups of this split, dealt round-robin to the waves: wave w takes
  // groups w, w + 4, ...; t counts the wave's own groups
  const int nent = u.e1 - u.e0;
  const int ngroups = BLOCK ? 8 * nent : ceil_div(nent, 16);
  const int nmine = ngroups > wave ? ceil_div(ngroups - wave, kAttnWaves) : 0;
  int* stage = lds.stage[wave];

  SoftState st;
  st.m = -__builtin_inff();
  st.l = 0.0f;
  float4v acc[8], acct[8];  // acct: BF16 tail rows beside 4-bit rows (kValStoreTail)
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    acc[c] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    acct[c] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  }

#pragma unroll 1
  for (int w0 = 0; w0 < nmine; w0 += kWindow) {
    const int wend = min(w0 + kWindow, nmine);
    // stage the window's row indices (this wave's LDS rows only)
    wave_lds_sync();  // the previous window's last reads are done
    if constexpr (BLOCK) {
      for (int t = w0 + lane; t < wend; t += kWave)
        stage[t - w0] = u.uidx[u.e0 + ((wave + kAttnWaves * t) >> 3)];
    } else {
      for (int i = lane; i < 16 * (wend - w0); i += kWave) {
        const int t = w0 + (i >> 4);
        const int e = u.e0 + 16 * (wave + kAttnWaves * t) + (i & 15);
        const int tok = e < u.e1 ? u.uidx[e] : -1;
        stage[i] = (tok >= 0 && tok < u.L) ? tok : -1;
      }
    }
    wave_lds_sync();
    auto qof = [&](int t) { return wave + kAttnWaves * t; };
    KeySlot kr[RING];
    ValSlot<VM> vr[RING];
    // every slot is always issued (groups past the window are null groups), so
    // the ring registers are defined on every path
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      const int t = w0 + k;
      issue_keys<MAIN_BF16, BLOCK, VM>(kr[k], a, u, qof(t), stage, t - w0, lane, t < wend);
      issue_values<MAIN_BF16, BLOCK, VM>(vr[k], a, u, qof(t), stage, t - w0, lane, t < wend);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
    for (int t0 = w0; t0 < wend; t0 += RING) {
#pragma unroll
      for (int k = 0; k < RING; ++k) {
        const int t = t0 + k;
        const int tn = t + RING;  // the group this slot takes next
        // past the window (RING > 1) the slot holds a null group: every row
        // masked, which leaves the state as it is (no branch around the loads)
        const GroupRef r = describe<MAIN_BF16, BLOCK, VM>(a, u, qof(t), stage, t - w0, t < wend);
        // with one group per wave its next keys go out as soon as its keys are
        // read (during the softmax and PV); with two the next group is
        // already in flight then (measured: 0.5-1 us faster with one group
        // per wave at 16 x 4 heads, 128K; 0.3 us slower with two, 8 units)
        auto next_keys = [&] {
          issue_keys<MAIN_BF16, BLOCK, VM>(kr[k], a, u, qof(tn), stage, tn - w0, lane, tn < wend);
        };
        attend_group<G, BLOCK, VM>(kr[k], vr[k], r, qa, lds.qsplit, a.scale_log2, st, acc, acct,
                                   lane, [&] {
                                     if constexpr (RING == 1) next_keys();
                                   });
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (RING > 1) next_keys();
        issue_values<MAIN_BF16, BLOCK, VM>(vr[k], a, u, qof(tn), stage, tn - w0, lane,
                                           tn < wend);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- merge the waves' states -------------------------------------------
  // lane (j, n) holds head n, channels 32 j + 8 i + c in acc[c][i]
  if constexpr (VQ) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      acc[c] *= u.s_v;
      if constexpr (VM == kValStoreTail) acc[c] += acct[c];
    }
  }
  if (n16 < G) {
    float* dst = &lds.acc[wave][n16 * kAccStride + 32 * j4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<float4v*>(dst + 8 * i) = float4v{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *reinterpret_cast<float4v*>(dst + 8 * i + 4) =
          float4v{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
    if (j4 == 0) {
      lds.m[wave][n16] = st.m;
      lds.l[wave][n16] = st.l;
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < G * kHeadDim; o += 256) {
    const int hh = o / kHeadDim, d = o % kHeadDim;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, lds.m[w][hh]);
    float num = 0.0f, den = 0.0f;
    if (M > -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(lds.m[w][hh] - M);
        num += f * lds.acc[w][hh * kAccStride + d];
        den += f * lds.l[w][hh];
      }
    }
    const int64_t rowq = int64_t(b) * a.Hq + h * G + hh;
    const bool empty = !(den > 0.0f);
    const float po = empty ? 0.0f : num / den;
    const float pl = empty ? -__builtin_inff() : (M + __builtin_amdgcn_logf(den)) * kLn2;
    float* po_p = a.part_o + (rowq * a.splits + split) * kHeadDim + d;
    float* pl_p = a.part_lse + rowq * a.splits + split;
    if (a.counters) {  // read back by the unit's last group
      store_coherent(po_p, po);
      if (d == 0) store_coherent(pl_p, pl);
    } else {
      *po_p = po;
      if (d == 0) *pl_p = pl;
    }
  }
  if (!a.counters) return;

  // ---- fused merge: the unit's last group to finish combines the partials --
  if (!last_group_of_unit(a.counters, unit, a.splits, &lds.is_last)) return;
  for (int o = threadIdx.x; o < G * kHeadDim; o += 256) {
    const int hh = o / kHeadDim, d = o % kHeadDim;
    const int64_t rowq = int64_t(b) * a.Hq + h * G + hh;
    float val, lse;
    const float* pl = a.part_lse + rowq * a.splits;
    const float* po = a.part_o + rowq * a.splits * kHeadDim;
    static_assert(kFusedMergeMaxSplits == 8, "the one-pass form below");
    if (a.splits <= 8)
      combine_channel_few<8, true>(pl, po, a.splits, d, val, lse);
    else
      combine_channel<true>(pl, po, a.splits, d, val, lse);
    a.out[rowq * kHeadDim + d] = val;
    if (d == 0 && a.out_lse) a.out_lse[rowq] = lse;
  }
}

}  // namespace
}  // namespace bsa
