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
// from the first group to the last. Per group:
//   1. QK^T on v_mfma_f32_16x16x32_f16 (A = the group's query heads, rows >= G
//      zero; B = 16 key rows, lane l holding row l % 16 and, for MFMA step c,
//      channels 8 (l/16 + 4 c) .. +7, so each wave load reads 64 contiguous
//      bytes of every row). BF16 rows (tail pages or a BF16 cache) take two
//      bf16 MFMAs with q split exactly into q_hi + q_lo (an fp16 value is the
//      sum of two bf16 values).
//   2. An online softmax in the log2 domain, still in the MFMA output layout
//      (a 16-lane row holds four heads of the 16 rows): row maxima and sums by
//      DPP, the running maximum and sum per head kept by every lane of the row.
//      The probabilities and the heads' rescale factors go through a small
//      double-buffered LDS table to the value layout.
//   3. PV as FP32 VALU FMAs, a lane owning DPL consecutive channels of a subset
//      of the rows, so one wave load covers whole 256-byte value rows. The
//      accumulators are rescaled only when some head's maximum grew.
//      From the 4-bit value store a lane loads the DPL / 2 code bytes of its
//      channels and the one E4M3 scale byte they share; the codes become
//      floats by the hardware FP4 convert, and the row's scale times the KV
//      head's FP32 scale multiplies either the probabilities or the values,
//      whichever are fewer per lane (e2m1 * S is the value the packer rounded
//      to, S = fl32(e4m3 * s_v)).
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
// 16-row groups of keys, and of values, in flight per wave beyond the one being
// used. One: with 2048 waves streaming that is 16 MiB in flight, enough for
// the HBM; deeper rings (32 and 48 MiB) queue so deep that the work-groups
// served first finish far ahead of the rest, and measured slower (C3: 52.3 us
// with one group ahead, 54.2 with two, 56.8 with three).
constexpr int kRing = 1;
// The same with values from the 4-bit store (a group is 5 KiB instead of 8).
constexpr int kRingV4 = 1;

// Where a kernel reads the values: the 16-bit cache (BF16 tail pages too), the
// 4-bit store with no tail pages, or the 4-bit store with BF16 tail pages. In
// the last form every group issues the loads of both forms, the unused ones at
// one fixed line of the unit's store, so that no load sits behind a branch: a
// branch around loads makes the compiler copy the loaded registers at the loop
// end, which waits for every load in flight.
constexpr int kValCache = 0, kValStore = 1, kValStoreTail = 2;
constexpr int kWindow = 32;  // groups whose row indices a wave stages at a time
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int G>
struct PvShape {
  static constexpr int DPL = G <= 4 ? 8 : (G == 8 ? 4 : 2);  // channels per lane
  static constexpr int LPR = kHeadDim / DPL;                  // lanes per row
  static constexpr int NQ = kWave / LPR;                      // rows per wave load
  static constexpr int RPL = 16 / NQ;                         // value rows per lane per group
  static constexpr int VDW = DPL / 2;                         // dwords of a row per lane
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

// Value registers of one group: lane l holds channels (l % LPR) * DPL .. of rows
// l / LPR + NQ k: 16-bit values in w[k][..], or from the 4-bit store the
// channels' codes in c4[k] and their scale byte in sc[k].
template <int G, int VM>
struct ValSlot {
  static constexpr int R16 = VM == kValStore ? 1 : PvShape<G>::RPL;
  static constexpr int R4 = VM == kValCache ? 1 : PvShape<G>::RPL;
  uint32_t w[R16][PvShape<G>::VDW];
  uint32_t c4[R4];
  uint32_t sc[R4];
};

template <int G, bool MAIN_BF16, bool BLOCK, int VM>
__device__ __forceinline__ void issue_values(ValSlot<G, VM>& vs, const AttnArgs& a,
                                             const UnitCtx& u, int q, const int* stage, int tl,
                                             int lane, bool live) {
  using PV = PvShape<G>;
  const GroupRef r = describe<MAIN_BF16, BLOCK, VM>(a, u, q, stage, tl, live);
  const int dc = lane % PV::LPR, qsub = lane / PV::LPR;
  if constexpr (VM != kValCache) {
    // a tail group (kValStoreTail) reads row 0 of the unit's store instead
    const uint8_t* cb = r.v4 ? r.vc : u.vcunit;
    const uint8_t* sb = r.v4 ? r.vsb : u.vsunit;
#pragma unroll
    for (int k = 0; k < PV::RPL; ++k) {
      const int64_t row = r.v4 ? row_index<BLOCK>(r, qsub + PV::NQ * k) : 0;
      const uint8_t* cp = cb + row * kValueCodeRow + dc * (PV::DPL / 2);
      if constexpr (PV::DPL == 8)
        vs.c4[k] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(cp));
      else if constexpr (PV::DPL == 4)
        vs.c4[k] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(cp));
      else
        vs.c4[k] = __builtin_nontemporal_load(cp);
      vs.sc[k] = __builtin_nontemporal_load(sb + row * kValueScaleRow + (dc * PV::DPL) / 16);
    }
  }
  if constexpr (VM == kValStoreTail) {
    // the BF16 tail rows; a 4-bit group reads the first 256 bytes of the
    // unit's store codes instead (always cached, never used)
    const uint16_t* vb = r.v4 ? reinterpret_cast<const uint16_t*>(u.vcunit) : r.vb;
#pragma unroll
    for (int k = 0; k < PV::RPL; ++k) {
      const int64_t off = r.v4 ? 0 : row_offset<BLOCK>(r, qsub + PV::NQ * k);
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(vb + off + dc * PV::DPL);
#pragma unroll
      for (int e = 0; e < PV::VDW; ++e) vs.w[k][e] = vp[e];
    }
  }
  if constexpr (VM == kValCache) {
#pragma unroll
    for (int k = 0; k < PV::RPL; ++k) {
      const int64_t off = row_offset<BLOCK>(r, qsub + PV::NQ * k);
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(r.vb + off + dc * PV::DPL);
      if constexpr (PV::VDW == 4) {
        const uint4v x = __builtin_nontemporal_load(reinterpret_cast<const uint4v*>(vp));
#pragma unroll
        for (int e = 0; e < 4; ++e) vs.w[k][e] = x[e];
      } else {
#pragma unroll
        for (int e = 0; e < PV::VDW; ++e) vs.w[k][e] = __builtin_nontemporal_load(vp + e);
      }
    }
  }
}

// LDS of one attention work-group.
template <int G>
struct AttnLds {
  int stage[kAttnWaves][16 * kWindow];  // each wave's staged row indices
  float ptab[kAttnWaves][2][16][G];     // a group's probabilities [row][head] (double-buffered)
  float atab[kAttnWaves][2][G];         // a group's rescale factor per head
  bf16x8 qsplit[8 * kWave];             // q = q_hi + q_lo in the MFMA operand order
  float acc[kAttnWaves][G * kHeadDim];  // the waves' accumulators for the merge
  float m[kAttnWaves][G], l[kAttnWaves][G];
  int nulltoks[16];  // token mode: a null group's tokens (all -1)
  int is_last;
  int32_t sel[kFusedSelectMax];  // the unit's selection made in the prologue
  SelectLds sel_s;
  int32_t sel_cnt;
};

// The online-softmax state of one wave: lane (j, n) holds the running maximum
// (log2 domain) and sum of heads 4 j + r, r < 4; every lane of a 16-lane row
// holds the same maximum, and the row's lane 0 holds the sum that is kept.
struct SoftState {
  float m[4], l[4];
};

// The E2M1 codes of channels 0 .. N-1 (channel e in bits 4 e .. 4 e + 3) as
// floats, two per hardware convert (the byte to convert is an immediate).
template <int N>
__device__ __forceinline__ void fp4_to_floats(uint32_t x, float (&vv)[N]) {
  static_assert(N == 2 || N == 4 || N == 8, "channels per lane");
  float2v c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 0);
  vv[0] = c[0];
  vv[1] = c[1];
  if constexpr (N >= 4) {
    c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 1);
    vv[2] = c[0];
    vv[3] = c[1];
  }
  if constexpr (N == 8) {
    c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 2);
    vv[4] = c[0];
    vv[5] = c[1];
    c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 3);
    vv[6] = c[0];
    vv[7] = c[1];
  }
}

// One landed group: QK^T, the online softmax update, PV. Returns nothing; the
// state and accumulators are updated in place. ptab / atab: this wave's
// tables for the group's buffer.
template <int G, bool BLOCK, int VM>
__device__ __forceinline__ void attend_group(const KeySlot& ks, const ValSlot<G, VM>& vs,
                                             const GroupRef& r,
                                             const half8 (&qa)[4], const bf16x8* qsplit,
                                             float scale_log2, float s_v, SoftState& st,
                                             float (&acc)[G][PvShape<G>::DPL],
                                             float (&ptab)[16][G], float (&atab)[G], int lane) {
  using PV = PvShape<G>;
  constexpr int DPL = PV::DPL;
  // ---- QK^T ----
  float4v d = {0.0f, 0.0f, 0.0f, 0.0f};
  if (!r.bf16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      half8 kv;
      __builtin_memcpy(&kv, &ks.w[c], 16);
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[c], kv, d, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 kv;
      __builtin_memcpy(&kv, &ks.w[c], 16);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qsplit[(2 * c) * kWave + lane], kv, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qsplit[(2 * c + 1) * kWave + lane], kv, d, 0, 0, 0);
    }
  }
  // ---- online softmax (MFMA output layout: lane (j, n) = heads 4 j + r of row n) ----
  const int n16 = lane & 15, j4 = lane >> 4;
  const bool rok = row_valid<BLOCK>(r, n16);
  bool grew = false;
  float p[4], alpha[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const float s = rok ? d[q4] * scale_log2 : -__builtin_inff();
    const float mx = row16_max(s);
    const float mo = st.m[q4];
    const float mn = fmaxf(mo, mx);
    const bool live = mn > -__builtin_inff();
    alpha[q4] = live ? __builtin_amdgcn_exp2f(mo - mn) : 1.0f;
    p[q4] = live ? __builtin_amdgcn_exp2f(s - mn) : 0.0f;
    grew = grew || (4 * j4 + q4 < G && mn > mo);
    st.m[q4] = mn;
    st.l[q4] = st.l[q4] * alpha[q4] + row16_sum(p[q4]);
  }
  const bool rescale = __ballot(grew) != 0;  // wave-uniform
  if (4 * j4 < G) {
    if constexpr (G >= 4) {
      float4v pv = {p[0], p[1], p[2], p[3]};
      *reinterpret_cast<float4v*>(&ptab[n16][4 * j4]) = pv;
      if (n16 == 0) {
        float4v av = {alpha[0], alpha[1], alpha[2], alpha[3]};
        *reinterpret_cast<float4v*>(&atab[4 * j4]) = av;
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < G; ++q4) {
        ptab[n16][q4] = p[q4];
        if (n16 == 0) atab[q4] = alpha[q4];
      }
    }
  }
  wave_lds_sync();
  // ---- PV (value layout: lane (qsub, dc) = channels dc * DPL .. of rows qsub + NQ k) ----
  const int qsub = lane / PV::LPR;
  if (rescale) {
    float al[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) al[hh] = atab[hh];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] *= al[hh];
  }
  const bool full = BLOCK ? r.nvalid >= 16 : __ballot(rok) == ~0ull;  // all 16 rows valid
#pragma unroll
  for (int k = 0; k < PV::RPL; ++k) {
    const int row = qsub + PV::NQ * k;
    float pr[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) pr[hh] = ptab[row][hh];
    // a masked row has p = 0; its value bits are not data, so they are dropped
    const bool vok = full || row_valid<BLOCK>(r, row);
    float vv[DPL];
    if (VM != kValCache && r.v4) {
      // E2M1 code of channel e in bits 4 e .. 4 e + 3; a dropped row's scale is
      // zero (its byte could be a NaN code)
      fp4_to_floats<DPL>(vs.c4[k], vv);
      const float f =
          __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vok ? vs.sc[k] : 0u, 1.0f, false)[0] * s_v;
      if constexpr (G <= DPL) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) pr[hh] *= f;
      } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) vv[e] *= f;
      }
    } else if constexpr (VM != kValStore) {
#pragma unroll
      for (int e = 0; e < PV::VDW; ++e) {
        const uint32_t x = vok ? vs.w[k][e] : 0u;
        if (r.bf16) {
          vv[2 * e] = bf16_bits_to_float(x & 0xFFFFu);
          vv[2 * e + 1] = bf16_bits_to_float(x >> 16);
        } else {
          vv[2 * e] = half_bits_to_float(uint16_t(x & 0xFFFFu));
          vv[2 * e + 1] = half_bits_to_float(uint16_t(x >> 16));
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] = __builtin_fmaf(pr[hh], vv[e], acc[hh][e]);
    // with 8 or 16 heads a row's G probabilities are read where they are used
    // (hoisting every row's reads needs more registers than there are)
    if constexpr (G >= 8) __builtin_amdgcn_sched_barrier(0);
  }
}

// The attention of (split, unit): its rows' partial (O, lse) per head, and the
// merge when a.counters is set.
template <int G, bool MAIN_BF16, bool BLOCK, int VM>
__device__ __forceinline__ void attn_item(const AttnArgs& a, int split, int unit,
                                          AttnLds<G>& lds) {
  using PV = PvShape<G>;
  constexpr int DPL = PV::DPL, LPR = PV::LPR;
  constexpr int RING = VM != kValCache ? kRingV4 : kRing;
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

  // query operands: lane l holds head row l % 16, channels 8 (l/16 + 4 c) .. + 8
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
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    st.m[q4] = -__builtin_inff();
    st.l[q4] = 0.0f;
  }
  float acc[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.0f;

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
    ValSlot<G, VM> vr[RING];
    // every slot is always issued (groups past the window are null groups), so
    // the ring registers are defined on every path
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      const int t = w0 + k;
      issue_keys<MAIN_BF16, BLOCK, VM>(kr[k], a, u, qof(t), stage, t - w0, lane, t < wend);
      issue_values<G, MAIN_BF16, BLOCK, VM>(vr[k], a, u, qof(t), stage, t - w0, lane,
                                            t < wend);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
    for (int t0 = w0; t0 < wend; t0 += RING) {
#pragma unroll
      for (int k = 0; k < RING; ++k) {
        const int t = t0 + k;
        const int tn = t + RING;  // the group this slot takes next
        if (t < wend) {
          const GroupRef r = describe<MAIN_BF16, BLOCK, VM>(a, u, qof(t), stage, t - w0, true);
          attend_group<G, BLOCK, VM>(kr[k], vr[k], r, qa, lds.qsplit, a.scale_log2, u.s_v, st,
                                     acc, lds.ptab[wave][t & 1], lds.atab[wave][t & 1], lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_keys<MAIN_BF16, BLOCK, VM>(kr[k], a, u, qof(tn), stage, tn - w0, lane, tn < wend);
        issue_values<G, MAIN_BF16, BLOCK, VM>(vr[k], a, u, qof(tn), stage, tn - w0, lane,
                                              tn < wend);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- merge the waves' states -------------------------------------------
  const int dc = lane % LPR, qsub = lane / LPR;
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
      for (int e = 0; e < DPL; ++e) lds.acc[wave][hh * kHeadDim + dc * DPL + e] = acc[hh][e];
  }
  if (n16 == 0) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int hh = 4 * j4 + q4;
      if (hh < G) {
        lds.m[wave][hh] = st.m[q4];
        lds.l[wave][hh] = st.l[q4];
      }
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
        num += f * lds.acc[w][o];
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
