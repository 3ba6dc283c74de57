// Sparse decode attention over the selected rows, as split partials.
//
// Jet-QSparse abstract: the chosen 128-token blocks are aggregated in FP16 with
// FP32 accumulation from contiguous tiles; up to two newest pages live in BF16.
// JSSA Figure 1: the KV head's query heads share one index set and read the
// original keys and values at those rows in place (no gather buffer).
//
// Work-group = (split s, unit). The split's rows are cut into groups of 16
// (an eighth of a selected block, or 16 consecutive selected tokens), dealt
// round-robin to the 4 waves. A wave takes its groups in chunks of up to
// 1024 / G rows, each in three phases that keep a ring of kDepth groups of
// loads in flight:
//   1. keys stream in; QK^T on v_mfma_f32_16x16x32_f16 (A = the group's query
//      heads, rows >= G zero; B = 16 key rows, lane l holding row l % 16 and,
//      for MFMA step c, channels 8 (l/16 + 4 c) .. +7, so each wave load reads
//      64 contiguous bytes of every row); log2-scaled logits to an LDS table. BF16
//      rows (tail pages or a BF16 cache) take two bf16 MFMAs with q split
//      exactly into q_hi + q_lo (an fp16 value is the sum of two bf16 values).
//   2. an exact softmax update over the chunk per head (wave reductions), the
//      FP32 accumulators rescaled once per chunk.
//   3. values stream in; PV as FP32 VALU FMAs, a lane owning DPL consecutive
//      channels of a subset of the rows so one wave load covers whole
//      256-byte value rows.
// The waves' states are merged through LDS into one (O, lse) partial per head.
//
// With block scores given, every work-group of a unit first selects the unit's
// blocks itself (select_unit_rows, the same selection select_topk makes) into
// LDS, and the split-0 group also writes idx / count: the selection's latency
// then overlaps nothing but saves its own launch.
#pragma once

#include "combine_core.hpp"
#include "common.hpp"
#include "select_core.hpp"

namespace bsa {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kDepth = 2;  // 16-row groups in flight per wave in each streaming phase
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int G>
struct PvShape {
  static constexpr int DPL = G <= 4 ? 8 : (G == 8 ? 4 : 2);  // channels per lane
  static constexpr int LPR = kHeadDim / DPL;                  // lanes per row
  static constexpr int NQ = kWave / LPR;                      // rows per wave load
  static constexpr int RPL = 16 / NQ;                         // value rows per lane per group
  static constexpr int VDW = DPL / 2;                         // dwords of a row per lane
  static constexpr int CHUNK = 1024 / G;                      // rows per wave per chunk
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

// Decode-step launch only: every scan item of a unit counts itself in the
// unit's scan-done counter once its scores are stored; the last of them makes
// the unit's selection, stores idx and count, and raises the counter to
// scan_items + 1. The unit's attention waits for that value, then reads the
// selection; it sets *fault if the wait runs past its bound (which only a
// broken ordering could cause).
struct StepSync {
  uint32_t* scan_done;  // unit u's counter at scan_done[scan_stride * u]
  uint32_t* fault;
  int scan_items, scan_stride;
};

// Per-unit context shared by every row group of the work-group.
struct UnitCtx {
  const uint16_t* kunit;  // K and V of this (sequence, KV head)
  const uint16_t* vunit;
  const int32_t* uidx;
  int e0, e1, L, npg, tail0, unit;
};

// One group of 16 rows: an eighth of a selected block, or 16
// consecutive selected tokens. Row rho of the group is at kb/vb + off(rho).
struct GroupRef {
  const uint16_t* kb;
  const uint16_t* vb;
  int64_t rs;       // elements between rows (block mode)
  int nvalid;       // block mode: rows 0 .. nvalid-1 are valid
  const int* toks;  // token mode: the group's 16 staged token indices (-1 = masked)
  bool bf16;
};

// The selected block ids (block mode) or token indices (token mode) a wave
// needs for one chunk are staged in LDS before the chunk's streaming loops, so
// nothing inside them waits on a vector-memory index load (such a wait would
// also wait for every key and value load in flight).
//   block mode: stage[t] = block id of the wave's group t (relative to the chunk)
//   token mode: stage[16 t + rho] = token of row rho of group t, or -1
// live == false gives a null group: every row masked, addresses inside the unit.
template <bool MAIN_BF16>
__device__ __forceinline__ GroupRef describe(const AttnArgs& a, const UnitCtx& u, int q,
                                             const int* stage, int tl, bool block_mode,
                                             bool live) {
  GroupRef r;
  r.toks = stage;
  if (!live) {
    r.kb = u.kunit;
    r.vb = u.vunit;
    r.rs = a.st;
    r.nvalid = 0;
    r.bf16 = MAIN_BF16;
    return r;
  }
  if (block_mode) {
    const int blk = stage[tl];
    const int part = q & 7;
    const bool ok = blk >= 0 && blk < u.npg;
    const int b0 = ok ? blk : 0;
    r.nvalid = ok ? min(16, u.L - b0 * kBlock - 16 * part) : 0;
    if (a.n_tail > 0 && ok && blk >= u.tail0) {
      const int64_t off =
          ((int64_t(u.unit) * a.n_tail + (blk - u.tail0)) * kBlock + 16 * part) * kHeadDim;
      r.kb = a.tail_k + off;
      r.vb = a.tail_v + off;
      r.rs = kHeadDim;
      r.bf16 = true;
    } else {
      const int64_t off = (int64_t(b0) * kBlock + 16 * part) * a.st;
      r.kb = u.kunit + off;
      r.vb = u.vunit + off;
      r.rs = a.st;
      r.bf16 = MAIN_BF16;
    }
  } else {
    r.kb = u.kunit;
    r.vb = u.vunit;
    r.rs = a.st;
    r.nvalid = 16;
    r.toks = stage + 16 * tl;
    r.bf16 = MAIN_BF16;
  }
  return r;
}

// Element offset of group row rho from kb / vb, or -1 when masked.
__device__ __forceinline__ int64_t row_offset(const GroupRef& r, int rho, bool block_mode) {
  if (block_mode) return rho < r.nvalid ? int64_t(rho) * r.rs : -1;
  if (r.nvalid == 0) return -1;  // null group
  const int tok = r.toks[rho];
  return tok >= 0 ? int64_t(tok) * r.rs : -1;
}

// Key registers of one group: lane l holds row l % 16, channels 8 (l/16 + 4 c) .. +7
// for MFMA step c, so load c of the wave reads 64 contiguous bytes of each row.
struct KeySlot {
  uint4v w[4];
  bool ok, bf16;
};

template <bool MAIN_BF16>
__device__ __forceinline__ void issue_keys(KeySlot& ks, const AttnArgs& a, const UnitCtx& u,
                                           int q, const int* stage, int tl, int lane,
                                           bool block_mode, bool live) {
  const GroupRef r = describe<MAIN_BF16>(a, u, q, stage, tl, block_mode, live);
  const int64_t off = row_offset(r, lane & 15, block_mode);
  ks.ok = off >= 0;
  ks.bf16 = r.bf16;
  // plain loads: each 128-byte line is read by two of the wave's loads, and a
  // streaming (non-temporal) hint can evict it in between
  const uint4v* kp = reinterpret_cast<const uint4v*>(r.kb + (off >= 0 ? off : 0) + 8 * (lane >> 4));
#pragma unroll
  for (int c = 0; c < 4; ++c) ks.w[c] = kp[4 * c];
}

// Value registers of one group: lane l holds channels (l % LPR) * DPL .. of rows
// l / LPR + NQ k.
template <int G>
struct ValSlot {
  uint32_t w[PvShape<G>::RPL][PvShape<G>::VDW];
  bool bf16;
};

template <int G, bool MAIN_BF16>
__device__ __forceinline__ void issue_values(ValSlot<G>& vs, const AttnArgs& a, const UnitCtx& u,
                                             int q, const int* stage, int tl, int lane,
                                             bool block_mode, bool live) {
  using PV = PvShape<G>;
  const GroupRef r = describe<MAIN_BF16>(a, u, q, stage, tl, block_mode, live);
  vs.bf16 = r.bf16;
  const int dc = lane % PV::LPR, qsub = lane / PV::LPR;
#pragma unroll
  for (int k = 0; k < PV::RPL; ++k) {
    const int64_t off = row_offset(r, qsub + PV::NQ * k, block_mode);
    const uint32_t* vp =
        reinterpret_cast<const uint32_t*>(r.vb + (off >= 0 ? off : 0) + dc * PV::DPL);
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

// QK^T of one landed key group; the log2-scaled logits of rows 16 g .. +15 go
// to sc[head * CHUNK + 16 g + row] (masked rows -inf). qa: this lane's four
// FP16 query operands (registers); qsplit: the BF16 halves, in LDS.
template <int G>
__device__ __forceinline__ void group_scores(const KeySlot& ks, const half8* qa,
                                             const bf16x8* qsplit, float scale_log2, float* sc,
                                             int g, int lane) {
  constexpr int CHUNK = PvShape<G>::CHUNK;
  float4v d = {0.0f, 0.0f, 0.0f, 0.0f};
  if (!ks.bf16) {
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
  const int n16 = lane & 15, j4 = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * j4 + r;
    if (hh < G) sc[hh * CHUNK + 16 * g + n16] = ks.ok ? d[r] * scale_log2 : -__builtin_inff();
  }
}

// acc += p * v over one landed value group (p from sc, masked rows have p = 0).
template <int G>
__device__ __forceinline__ void group_pv(float (&acc)[G][PvShape<G>::DPL], const ValSlot<G>& vs,
                                         const float* sc, int g, int lane) {
  using PV = PvShape<G>;
  constexpr int DPL = PV::DPL, CHUNK = PV::CHUNK;
  const int qsub = lane / PV::LPR;
#pragma unroll
  for (int k = 0; k < PV::RPL; ++k) {
    const int rl = 16 * g + qsub + PV::NQ * k;
    float vv[DPL];
#pragma unroll
    for (int e = 0; e < PV::VDW; ++e) {
      const uint32_t x = vs.w[k][e];
      if (vs.bf16) {
        vv[2 * e] = bf16_bits_to_float(x & 0xFFFFu);
        vv[2 * e + 1] = bf16_bits_to_float(x >> 16);
      } else {
        vv[2 * e] = half_bits_to_float(uint16_t(x & 0xFFFFu));
        vv[2 * e + 1] = half_bits_to_float(uint16_t(x >> 16));
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float p = sc[hh * CHUNK + rl];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] = __builtin_fmaf(p, vv[e], acc[hh][e]);
    }
  }
}

// LDS of one attention work-group.
template <int G>
struct AttnLds {
  static constexpr int CHUNK = PvShape<G>::CHUNK;
  // per-wave score / probability tables [head][row]; after the row loop the
  // same LDS holds the waves' accumulators for the merge
  static constexpr int kScFloats = G * CHUNK, kAccFloats = G * kHeadDim;
  static constexpr int kShare = kScFloats > kAccFloats ? kScFloats : kAccFloats;
  union {
    float sc[kAttnWaves * kShare];
    ScanQueryLds scan_q;  // a decode-step scan item's query (no attention state then)
  };
  float m[kAttnWaves][16], l[kAttnWaves][16];
  half8 qa[4 * kWave];       // q in the MFMA operand order
  bf16x8 qsplit[8 * kWave];  // q = q_hi + q_lo in the MFMA operand order
  int stage[kAttnWaves][CHUNK];
  int is_last;
  int32_t sel[kFusedSelectMax];
  SelectLds sel_s;
  int32_t sel_cnt;
};

// Bound on the polls of the decode-step wait (about a second; a correct
// ordering needs a few microseconds).
constexpr uint32_t kStepWaitPolls = 1u << 20;

// The attention of (split, unit): its rows' partial (O, lse) per head, and the
// merge when a.counters is set. STEP: inside the decode-step launch (wait for
// the unit's scan items, read its scores as device-scope loads); sync is only
// read then.
template <int G, bool MAIN_BF16, bool STEP>
__device__ __forceinline__ void attn_item(const AttnArgs& a, bool block_mode, int split, int unit,
                                          AttnLds<G>& lds, const StepSync& sync) {
  using PV = PvShape<G>;
  constexpr int DPL = PV::DPL, LPR = PV::LPR, CHUNK = PV::CHUNK;
  constexpr int kShare = AttnLds<G>::kShare;
  float* sc_lds = lds.sc;
  auto& m_lds = lds.m;
  auto& l_lds = lds.l;
  half8* qa_lds = lds.qa;
  bf16x8* qsplit_lds = lds.qsplit;
  auto& stage_lds = lds.stage;
  int32_t* sel_lds = lds.sel;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = unit / a.Hkv, h = unit % a.Hkv;
  UnitCtx u;
  u.unit = unit;
  u.L = clamp_len(a.seq_lens[b], a.Tmax);
  u.npg = ceil_div(u.L, kBlock);
  u.tail0 = u.npg - a.n_tail;  // first page held in the tail store
  // query operands: lane l holds head row l % 16, channels 8 (l/16 + 4 c) .. + 8
  // for MFMA step c (the key layout above). For G <= 4 wave 0 issues the loads
  // first, so their latency overlaps the selection and the index loads below
  // (for larger groups the registers are needed there).
  constexpr bool kEarlyQ = G <= 4;
  const int n16 = lane & 15, j4 = lane >> 4;
  half8 qv[4];
  auto load_q = [&]() {
    const bool ok = n16 < G;
    const _Float16* qrow = a.q + (int64_t(b) * a.Hq + h * G + (ok ? n16 : 0)) * kHeadDim + 8 * j4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qv[c] = *reinterpret_cast<const half8*>(qrow + 32 * c);
      if (!ok) qv[c] = half8{};
    }
  };
  if (kEarlyQ && wave == 0) load_q();
  int cnt;
  if constexpr (STEP) {
    // the unit's selection is in idx / count once its last scan item has
    // raised the counter past the scan items
    if (threadIdx.x == 0) {
      uint32_t polls = 0;
      while (__hip_atomic_load(sync.scan_done + sync.scan_stride * unit, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) <
             uint32_t(sync.scan_items) + 1u) {
        if (++polls > kStepWaitPolls) {
          __hip_atomic_store(sync.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
    }
    __syncthreads();
    // device-scope loads into LDS, all issued before the first is stored
    // (indices past the budget are clamped and dropped)
    const int32_t* src = a.idx + int64_t(unit) * a.budget;
    constexpr int kPer = kFusedSelectMax / 256;
    int32_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = load_coherent(src + min(int(threadIdx.x) + 256 * k, a.budget - 1));
    const int32_t c = load_coherent(a.count + unit);
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (int(threadIdx.x) + 256 * k < a.budget) sel_lds[threadIdx.x + 256 * k] = v[k];
    __syncthreads();
    cnt = c;
    u.uidx = sel_lds;
  } else if (a.sel_scores) {
    // the unit's selection, made by every group of the unit alike
    const int nb = a.Tmax / kBlock;
    int C, picks, f0, f1;
    block_candidates(u.L, a.n_tail, nb, a.budget, C, picks, f0, f1);
    select_unit_rows(a.sel_scores + int64_t(unit) * nb, C, picks, f0, f1, a.budget, sel_lds,
                     &lds.sel_cnt, lds.sel_s);
    __syncthreads();
    cnt = lds.sel_cnt;
    u.uidx = sel_lds;
    if (split == 0) {
      for (int i = threadIdx.x; i < a.budget; i += 256)
        a.sel_idx[int64_t(unit) * a.budget + i] = sel_lds[i];
      if (threadIdx.x == 0) a.sel_count[unit] = cnt;
    }
  } else {
    cnt = a.count[unit];
    u.uidx = a.idx + int64_t(unit) * a.budget;
  }
  cnt = min(max(cnt, 0), a.budget);
  const int per = ceil_div(a.budget, a.splits);
  u.e0 = split * per;
  u.e1 = min(min(u.e0 + per, a.budget), cnt);
  u.kunit = a.k + b * a.sb + h * a.sh;
  u.vunit = a.v + b * a.sb + h * a.sh;

  // 16-row groups of this split, dealt round-robin to the waves: wave w takes
  // groups w, w + 4, ...; t counts the wave's own groups
  const int nent = u.e1 > u.e0 ? u.e1 - u.e0 : 0;
  const int ngroups = block_mode ? 8 * nent : ceil_div(nent, 16);
  const int nmine = ngroups > wave ? ceil_div(ngroups - wave, kAttnWaves) : 0;
  constexpr int kChunkGroups = CHUNK / 16;
  // stage the block ids / tokens of the wave's groups t0 .. tend-1
  auto stage_chunk = [&](int t0, int tend) {
    int* stage = stage_lds[wave];
    if (block_mode) {
      for (int t = t0 + lane; t < tend; t += kWave)
        stage[t - t0] = u.uidx[u.e0 + ((wave + kAttnWaves * t) >> 3)];
    } else {
      for (int i = lane; i < 16 * (tend - t0); i += kWave) {
        const int t = t0 + (i >> 4);
        const int e = u.e0 + 16 * (wave + kAttnWaves * t) + (i & 15);
        const int tok = e < u.e1 ? u.uidx[e] : -1;
        stage[i] = (tok >= 0 && tok < u.L) ? tok : -1;
      }
    }
  };
  // the first chunk's index loads overlap the query loads below
  if (nmine > 0) stage_chunk(0, min(kChunkGroups, nmine));

  // query operands: staged once in LDS by wave 0
  if (wave == 0) {
    if (!kEarlyQ) load_q();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qa_lds[c * kWave + lane] = qv[c];
      split_bf16(qv[c], qsplit_lds[(2 * c) * kWave + lane], qsplit_lds[(2 * c + 1) * kWave + lane]);
    }
  }
  __syncthreads();

  float m[G], lsum[G];  // wave-uniform running max (log2 domain) and sum per head
  float acc[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -__builtin_inff();
    lsum[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.0f;
  }
  float* sc = sc_lds + wave * kShare;

#pragma unroll 1
  for (int t0 = 0; t0 < nmine; t0 += kChunkGroups) {
    const int tend = min(t0 + kChunkGroups, nmine);
    int* stage = stage_lds[wave];
    if (t0 > 0) stage_chunk(t0, tend);  // the first chunk was staged before the loop
    wave_lds_sync();
    // ---- phase 1: keys stream through a ring of kDepth slots; QK^T -> sc ----
    // Every slot is always issued (groups past the chunk are null groups), so
    // the ring registers are defined on every path.
    {
      KeySlot ring[kDepth];
#pragma unroll
      for (int k = 0; k < kDepth; ++k)
        issue_keys<MAIN_BF16>(ring[k], a, u, wave + kAttnWaves * (t0 + k), stage, k, lane,
                              block_mode, t0 + k < tend);
      // the FP16 query operands stay in registers for the key phase only
      half8 qreg[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) qreg[c] = qa_lds[c * kWave + lane];
#pragma unroll 1
      for (int t = t0; t < tend; t += kDepth) {
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
          if (t + k < tend) group_scores<G>(ring[k], qreg, qsplit_lds, a.scale_log2, sc, t + k - t0, lane);
          issue_keys<MAIN_BF16>(ring[k], a, u, wave + kAttnWaves * (t + k + kDepth), stage,
                                t + k + kDepth - t0, lane, block_mode, t + k + kDepth < tend);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wave_lds_sync();
    __builtin_amdgcn_sched_barrier(0);
    // the value ring's first groups go out now, so their latency overlaps the
    // softmax (every slot is issued; groups past the chunk are null groups)
    ValSlot<G> vring[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k)
      issue_values<G, MAIN_BF16>(vring[k], a, u, wave + kAttnWaves * (t0 + k), stage, k, lane,
                                 block_mode, t0 + k < tend);
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase 2: exact softmax update over the chunk, per head -------------
    const int rows = 16 * (tend - t0);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float* sh = sc + hh * CHUNK;
      float mx = -__builtin_inff();
      for (int r = lane; r < rows; r += kWave) mx = fmaxf(mx, sh[r]);
      mx = wave_max_uniform(mx);
      const float mn = fmaxf(m[hh], mx);
      const bool live = mn > -__builtin_inff();
      const float alpha = live ? __builtin_amdgcn_exp2f(m[hh] - mn) : 1.0f;
      float ps = 0.0f;
      for (int r = lane; r < rows; r += kWave) {
        const float p = live ? __builtin_amdgcn_exp2f(sh[r] - mn) : 0.0f;
        sh[r] = p;
        ps += p;
      }
      // wave-uniform: keep the running state in scalar registers
      lsum[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                               __builtin_bit_cast(int, lsum[hh] * alpha + wave_sum_uniform(ps))));
      m[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mn)));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] *= alpha;
    }
    wave_lds_sync();
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase 3: values stream through the ring; PV -----------------------
    {
      ValSlot<G>(&ring)[kDepth] = vring;
#pragma unroll 1
      for (int t = t0; t < tend; t += kDepth) {
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
          if (t + k < tend) group_pv<G>(acc, ring[k], sc, t + k - t0, lane);
          issue_values<G, MAIN_BF16>(ring[k], a, u, wave + kAttnWaves * (t + k + kDepth), stage,
                                     t + k + kDepth - t0, lane, block_mode,
                                     t + k + kDepth < tend);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wave_lds_sync();
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- merge the waves' states -------------------------------------------
  __syncthreads();  // every wave is done with its score table
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
      for (int e = 0; e < DPL; ++e)
        sc_lds[wave * kShare + hh * kHeadDim + dc * DPL + e] = acc[hh][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m_lds[wave][hh] = m[hh];
      l_lds[wave][hh] = lsum[hh];
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
        num += f * sc_lds[w * kShare + o];
        den += f * l_lds[w][hh];
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
  // every group of the unit is past its wait: ready the counter for the next step
  if (STEP && threadIdx.x == 0)
    __hip_atomic_store(sync.scan_done + sync.scan_stride * unit, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  for (int o = threadIdx.x; o < G * kHeadDim; o += 256) {
    const int hh = o / kHeadDim, d = o % kHeadDim;
    const int64_t rowq = int64_t(b) * a.Hq + h * G + hh;
    float val, lse;
    const float* pl = a.part_lse + rowq * a.splits;
    const float* po = a.part_o + rowq * a.splits * kHeadDim;
    // up to 8 splits as launched by the attention entry points; the decode
    // step always merges here, in one pass up to 32 splits
    static_assert(kFusedMergeMaxSplits == 8, "the one-pass forms below");
    if (a.splits <= 8)
      combine_channel_few<8, true>(pl, po, a.splits, d, val, lse);
    else if (STEP && a.splits <= 16)
      combine_channel_few<16, true>(pl, po, a.splits, d, val, lse);
    else if (STEP && a.splits <= 32)
      combine_channel_few<32, true>(pl, po, a.splits, d, val, lse);
    else
      combine_channel<true>(pl, po, a.splits, d, val, lse);
    a.out[rowq * kHeadDim + d] = val;
    if (d == 0 && a.out_lse) a.out_lse[rowq] = lse;
  }
}

}  // namespace
}  // namespace bsa
