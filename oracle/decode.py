"""Decode-step sparse attention, step by step (oracle; test infrastructure only).

Sources (the only specification there is):

* "Jet-QSparse: Accelerating Agentic LLM Inference with 4-Bit Sparse
  Attention", abstract (Key points, Full text): the key history is stored as
  NVFP4 and scanned densely at every decode step to pick 128-token blocks;
  only those blocks' values enter the output, multiplied in FP16 and summed in
  FP32; keys are centered by a calibrated vector, and up to two of each
  sequence's newest pages stay in BF16; the budget is a block count per KV
  head (64 in the speed claim, 128 for the accuracy claim).
* "Joint Subspace Sparse Attention for Efficient Long-Context Decoding" (JSSA),
  Abstract and Figure 1: per KV head, the average of its query heads is
  compared with keys projected to a common rank-r basis; the B best positions
  become one index list that all of that head's queries use, and attention then
  reads the unprojected keys and values at those positions in place. Figure 3
  fixes the density (2048 of 128K); Figure 10 evaluates BF16 and FP8
  projected-key caches; Table 15 shows per-KV-head selection beats a
  head-shared vote.
* "Coarse Semantic Blocks for Efficient Training-Free Sparse Attention",
  Abstract: keys are clustered into large blocks of tokens from noncontiguous
  positions; a query picks blocks by scoring their centroids and attends the
  original keys and values inside the picked blocks, under a token budget.

Everything is per unit = one (sequence b, KV head h). Query head hq belongs to
KV head hq // G. Arithmetic is float64 except the steps whose result is a
stored float32/bfloat16 quantity (the packers), which follow float32 exactly.
Readings of points the pages leave open are stated where they are used.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from . import nvfp4

BLOCK = 128  # tokens per selectable block (Jet-QSparse abstract)
HEAD_DIM = 128
GROUP = 16  # NVFP4: one E4M3 scale per 16 consecutive channels
NGROUPS = HEAD_DIM // GROUP
E2M1_MAX = 6.0

F32 = np.float32


# --------------------------------------------------------------------------
# byte layout of the 4-bit key copy
#
# The pages fix only the number format. The library stores, per
# (sequence, KV head, block), an 8192-byte code record and a 1024-byte scale
# record. With token tau = 16*i + n (i < 8, n < 16), channel d = 32*j + e
# (j < 4, e < 32) and scale group g = 2*j + s (s < 2):
#   code of (tau, d)  -> byte ((i*4 + j)*16 + n)*16 + e//2, low nibble if e even
#   scale of (tau, g) -> byte ((j*16 + n)*8 + i)*2 + s
# --------------------------------------------------------------------------

def codes_to_cache_layout(codes: np.ndarray) -> np.ndarray:
    """[..., 128 tokens, 128 channels] one code per entry -> [..., 8192] bytes."""
    lead = codes.shape[:-2]
    c = codes.astype(np.uint8).reshape(*lead, 8, 16, 4, 32)  # i, n, j, e
    c = np.swapaxes(c, -3, -2)  # i, j, n, e
    packed = c[..., 0::2] | (c[..., 1::2] << 4)
    return np.ascontiguousarray(packed).reshape(*lead, 8192)


def cache_layout_to_codes(raw: np.ndarray) -> np.ndarray:
    lead = raw.shape[:-1]
    c = raw.reshape(*lead, 8, 4, 16, 16)  # i, j, n, byte
    out = np.empty((*lead, 8, 4, 16, 32), dtype=np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    out = np.swapaxes(out, -3, -2)  # i, n, j, e
    return np.ascontiguousarray(out).reshape(*lead, BLOCK, HEAD_DIM)


def scales_to_cache_layout(sb: np.ndarray) -> np.ndarray:
    """[..., 128 tokens, 8 groups] -> [..., 1024] bytes."""
    lead = sb.shape[:-2]
    s = sb.astype(np.uint8).reshape(*lead, 8, 16, 4, 2)  # i, n, j, s
    nd = s.ndim
    s = np.transpose(s, tuple(range(nd - 4)) + (nd - 2, nd - 3, nd - 4, nd - 1))  # j, n, i, s
    return np.ascontiguousarray(s).reshape(*lead, 1024)


def cache_layout_to_scales(raw: np.ndarray) -> np.ndarray:
    lead = raw.shape[:-1]
    s = raw.reshape(*lead, 4, 16, 8, 2)  # j, n, i, s
    nd = s.ndim
    s = np.transpose(s, tuple(range(nd - 4)) + (nd - 2, nd - 3, nd - 4, nd - 1))  # i, n, j, s
    return np.ascontiguousarray(s).reshape(*lead, BLOCK, NGROUPS)


# --------------------------------------------------------------------------
# helpers for the cache dtypes
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 values (bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bits, to nearest with ties to even.

    bfloat16 is the upper half of a binary32. Adding 0x7FFF plus the kept
    half's last bit to the 32-bit pattern carries into the upper half exactly
    when the dropped half is above 0x8000, or equal to it with an odd last
    bit; a carry out of the mantissa moves to the next binade or to infinity,
    as rounding does. NaN is kept a NaN, with the quiet bit set."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=F32))
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    quiet = (u >> 16) | 0x0040
    return np.where(nan, quiet, rounded).astype(np.uint16)


def n_pages(seq_len: int) -> int:
    return -(-int(seq_len) // BLOCK)


def packed_blocks(seq_len: int, n_tail: int) -> int:
    """Blocks held in the 4-bit copy: every page except the newest ``n_tail``."""
    return max(0, n_pages(seq_len) - n_tail)


# --------------------------------------------------------------------------
# A0: pack keys to the NVFP4 copy (Jet-QSparse abstract: the persistent cache is
# NVFP4, keys are centered by a calibrated vector first, and the packer reads the
# 16-bit activations directly)
#
# Reading: y = fl32(fl32(k) - c); per 16-channel group the E4M3 scale encodes
# amax(|y|) / (6 * s_t) so the group's largest element lands on the largest
# E2M1 magnitude; the effective scale is S = fl32(E4M3(sb) * s_t); each element
# is E2M1(fl32(y / S)); a group whose scale decodes to 0 stores code 0.
# --------------------------------------------------------------------------

def pack_nvfp4(k: np.ndarray, center: np.ndarray, global_scale: float
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize keys [..., 128] of one KV head.

    Returns (codes [..., 128] uint8, one 4-bit code per channel;
             scale bytes [..., 8] uint8, one E4M3 per 16-channel group).
    """
    y = (np.asarray(k).astype(F32) - np.asarray(center, dtype=F32)).astype(F32)
    yg = y.reshape(*y.shape[:-1], NGROUPS, GROUP)
    amax = np.abs(yg).max(axis=-1)
    st = F32(global_scale)
    six_st = F32(F32(E2M1_MAX) * st)
    ratio = (amax / six_st).astype(F32)
    sb = nvfp4.e4m3_encode_nonneg(ratio)
    S = (nvfp4.e4m3_decode(sb).astype(F32) * st).astype(F32)
    Sx = np.broadcast_to(S[..., None], yg.shape)
    x = np.divide(yg, Sx, out=np.zeros_like(yg), where=Sx > 0).astype(F32)
    codes = nvfp4.e2m1_encode(x)
    codes[np.broadcast_to((S == 0)[..., None], codes.shape)] = 0
    return codes.reshape(y.shape), sb


def pack_unit_blocks(k_unit: np.ndarray, center: np.ndarray, global_scale: float,
                     block_begin: int, block_end: int) -> Tuple[np.ndarray, np.ndarray]:
    """Pack blocks [block_begin, block_end) of one unit's keys [T, 128].

    Returns code records [n, 8192] and scale records [n, 1024].
    """
    kb = k_unit[block_begin * BLOCK:block_end * BLOCK].reshape(-1, BLOCK, HEAD_DIM)
    codes, sb = pack_nvfp4(kb, center, global_scale)
    return codes_to_cache_layout(codes), scales_to_cache_layout(sb)


def dequant_blocks(code_rec: np.ndarray, scale_rec: np.ndarray) -> np.ndarray:
    """Records [n, 8192] + [n, 1024] -> e2m1 * e4m3 values [n, 128, 128] (float64).

    The per-KV-head FP32 scale and the centering vector are not applied.
    """
    codes = cache_layout_to_codes(code_rec)
    sb = cache_layout_to_scales(scale_rec)
    return nvfp4.e2m1_decode(codes) * np.repeat(nvfp4.e4m3_decode(sb), GROUP, axis=-1)


# --------------------------------------------------------------------------
# A0v (option): NVFP4 value store (Jet-QSparse abstract: the persistent cache is
# NVFP4 -- its KV pools hold 2.58-2.76x BF16's tokens, more than a 4-bit copy of
# the keys alone can give -- while the chosen values are aggregated in FP16 with
# FP32 accumulation)
#
# Reading: a value row is quantized as a key row is (A0), without centering,
# with one FP32 scale s_v per KV head (s_v = fl32(amax |v|) / 2688 over the
# head's packed rows, as for keys). Row t of a unit stores 64 code bytes
# (channel 2i in the low nibble of byte i) and 8 scale bytes (byte g: the E4M3
# scale of channels 16g .. 16g + 15). The aggregation uses the value
# s_v * e2m1 * e4m3, of which e2m1 * e4m3 is exact in FP16 (at most 6
# significant bits, within [2^-10, 2688]).
# --------------------------------------------------------------------------

def value_scale(v_rows: np.ndarray) -> np.float32:
    """s_v of one KV head's packed value rows (any leading shape, last axis 128)."""
    amax = F32(np.abs(np.asarray(v_rows, dtype=F32)).max()) if np.size(v_rows) else F32(0)
    return F32(amax / F32(6.0 * 448.0)) if amax > 0 else F32(1.0)


def pack_values(v_rows: np.ndarray, s_v: float) -> Tuple[np.ndarray, np.ndarray]:
    """Value rows [T, 128] -> (code bytes [T, 64], scale bytes [T, 8]) uint8."""
    codes, sb = pack_nvfp4(v_rows, np.zeros(HEAD_DIM, dtype=F32), s_v)
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8), sb.astype(np.uint8)


def dequant_values(code_bytes: np.ndarray, scale_bytes: np.ndarray, s_v: float) -> np.ndarray:
    """(code bytes [T, 64], scale bytes [T, 8], s_v) -> value rows [T, 128] float64."""
    cb = np.asarray(code_bytes, dtype=np.uint8)
    codes = np.empty(cb.shape[:-1] + (HEAD_DIM,), dtype=np.uint8)
    codes[..., 0::2] = cb & 0xF
    codes[..., 1::2] = cb >> 4
    scale = np.repeat(nvfp4.e4m3_decode(np.asarray(scale_bytes, dtype=np.uint8)), GROUP, axis=-1)
    return float(np.float64(s_v)) * (nvfp4.e2m1_decode(codes) * scale)


# --------------------------------------------------------------------------
# A1: dense block scan (Jet-QSparse abstract: every decode step scores all cached
# keys from the 4-bit copy, and the scores pick blocks of 128 tokens)
#
# Readings: the estimated logit of query head h and token t is
#   sigma * (s_t * q_h . dequant(k_t) + q_h . c)
# (the centering vector is added back so the estimate targets q . k); a block's
# score is the largest estimated logit over the KV head's query heads and the
# block's valid tokens (t < L). Blocks outside the packed region score -inf.
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# A1q: NVFP4 query for the scan (Jet-QSparse abstract: the scan's query-key
# products run natively in FP4, on 4-bit operands on both sides)
#
# Reading: the pages give no query format or scale rule. Each query head's 128
# channels are quantized as the keys are (A0), without centering, with a
# per-head FP32 scale s_q = fl32(amax / 2688) -- amax / (6 * 448), so the group
# that holds the head's largest magnitude gets the largest E4M3 scale. A head of
# zeros quantizes to zeros. The scan then scores the dequantized query
# qtilde = e2m1 * e4m3 * s_q in place of q in both of its terms; attention keeps
# the FP16 query (the output is formed in FP16 on the pages).
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def quantize_query(q_group: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """q_group [G, 128] (fp16 values) -> (codes [G, 128], scale bytes [G, 8],
    per-head scales s_q [G] float32)."""
    q = np.asarray(q_group).astype(F32)
    G = q.shape[0]
    codes = np.zeros((G, HEAD_DIM), dtype=np.uint8)
    sb = np.zeros((G, NGROUPS), dtype=np.uint8)
    s_q = np.zeros(G, dtype=F32)
    for h in range(G):
        amax = F32(np.abs(q[h]).max())
        s_q[h] = F32(amax / F32(E2M1_MAX * E4M3_MAX))
        if s_q[h] > 0:  # else: every code and scale stays 0
            codes[h], sb[h] = pack_nvfp4(q[h], np.zeros(HEAD_DIM, dtype=F32), float(s_q[h]))
    return codes, sb, s_q


def dequant_query(codes: np.ndarray, sb: np.ndarray, s_q: np.ndarray) -> np.ndarray:
    """qtilde [G, 128] float64: e2m1 * e4m3 * s_q, exact."""
    e = nvfp4.e2m1_decode(codes) * np.repeat(nvfp4.e4m3_decode(sb), GROUP, axis=-1)
    return e * np.asarray(s_q, dtype=np.float64)[:, None]


def scan_query(q_group: np.ndarray, query_fmt: str = "f16") -> np.ndarray:
    """The query the block scan scores with: q itself, or qtilde for "nvfp4"."""
    if query_fmt == "f16":
        return np.asarray(q_group, dtype=np.float64)
    if query_fmt != "nvfp4":
        raise ValueError(query_fmt)
    return dequant_query(*quantize_query(q_group))


def scan_block_unit(q_group: np.ndarray, code_rec: np.ndarray, scale_rec: np.ndarray,
                    global_scale: float, center: np.ndarray, seq_len: int, n_tail: int,
                    sigma: float, max_blocks: Optional[int] = None) -> np.ndarray:
    """Block scores [max_blocks] (float64) of one unit; q_group is [G, 128]."""
    nb_total = code_rec.shape[0] if max_blocks is None else max_blocks
    scores = np.full(nb_total, -np.inf)
    nb = packed_blocks(seq_len, n_tail)
    if nb == 0:
        return scores
    qg = np.asarray(q_group, dtype=np.float64)
    kd = dequant_blocks(code_rec[:nb], scale_rec[:nb])  # [nb, 128, 128]
    dots = kd.reshape(-1, HEAD_DIM) @ qg.T  # [nb*128, G]
    qc = qg @ np.asarray(center, dtype=np.float64)  # [G]
    logits = sigma * (float(global_scale) * dots + qc[None, :])
    t = np.arange(nb * BLOCK)
    logits[t >= seq_len] = -np.inf
    scores[:nb] = logits.reshape(nb, BLOCK * qg.shape[0]).max(axis=1)
    return scores


# --------------------------------------------------------------------------
# A2 / A8: top-k selection per KV head
#
# Readings: the budget counts the forced BF16 pages (Jet-QSparse abstract: at
# most two BF16 pages), which are the two newest pages and are always chosen;
# the remaining budget - n_tail picks go to the highest-scoring candidates,
# equal scores going to the lower index; output ascending, padded with -1.
# Token mode (JSSA Figure 1): top-B token positions per KV head, no forced pages.
# --------------------------------------------------------------------------

def select_unit(scores: np.ndarray, n_candidates: int, budget: int,
                forced: Sequence[int] = (), picks: Optional[int] = None
                ) -> Tuple[np.ndarray, int]:
    """Pick from candidates 0..n_candidates-1; returns (idx [budget] int32, count).

    ``picks`` (default budget - len(forced)) candidates are chosen by score,
    then the forced entries are added.
    """
    if picks is None:
        picks = budget - len(forced)
    cand = np.arange(n_candidates)
    s = np.asarray(scores[:n_candidates], dtype=np.float64)
    order = np.lexsort((cand, -s))  # primary: score descending; then index ascending
    chosen = cand[order[:max(0, picks)]]
    sel = np.sort(np.concatenate([chosen, np.asarray(list(forced), dtype=np.int64)]))
    out = np.full(budget, -1, dtype=np.int32)
    out[:len(sel)] = sel
    return out, int(len(sel))


def select_blocks_unit(scores: np.ndarray, seq_len: int, n_tail: int, budget: int
                       ) -> Tuple[np.ndarray, int]:
    """Forced tail pages plus the top (budget - n_tail) scanned blocks."""
    npg = n_pages(seq_len)
    forced = list(range(max(0, npg - n_tail), npg))
    return select_unit(scores, packed_blocks(seq_len, n_tail), budget, forced,
                       picks=budget - n_tail)


def select_tokens_unit(scores: np.ndarray, seq_len: int, budget: int) -> Tuple[np.ndarray, int]:
    return select_unit(scores, min(int(seq_len), scores.shape[0]), budget)


# --------------------------------------------------------------------------
# A8p: an adaptive token budget. The RaBitQCache abstract (second page) takes
# top-p retrieval in place of a fixed top-k: the number of tokens follows how
# concentrated the estimated attention is. Reading on this path: the token
# scores are the estimated logits (score_t = sigma p . kproj_t, A1t); a
# candidate's share is its softmax weight over all candidates t < L; the
# selection is the shortest prefix of the ranking (score descending, lower
# index first) whose shares reach top_p, cut at the budget. Non-finite scores:
# NaN and -inf weigh nothing; if any score is +inf, the +inf candidates share
# the whole mass equally (the softmax's limit). With top_p = 0, or when no
# candidate has weight, the fixed budget applies.
# --------------------------------------------------------------------------

def token_weights(s: np.ndarray) -> np.ndarray:
    """Unnormalized softmax weights exp(s_t - max s) under the reading above (float64)."""
    s = np.asarray(s, dtype=np.float64)
    ok = ~np.isnan(s)
    if not ok.any():
        return np.zeros_like(s)
    m = s[ok].max()
    if m == np.inf:
        return (s == np.inf).astype(np.float64)
    if m == -np.inf:
        return np.zeros_like(s)
    w = np.exp(np.where(ok, s, -np.inf) - m)
    return w


def select_tokens_top_p(scores: np.ndarray, seq_len: int, budget: int, top_p: float
                        ) -> Tuple[np.ndarray, int]:
    """The fewest top-ranked candidates whose softmax shares reach top_p, at most budget.

    Returns (idx [budget] int32 ascending, padded with -1; count).
    """
    n = min(int(seq_len), scores.shape[0])
    s = np.asarray(scores[:n], dtype=np.float64)
    cand = np.arange(n)
    order = np.lexsort((cand, -s))  # score descending (NaN last), then index ascending
    picks = max(0, min(int(budget), n))
    m = picks
    w = token_weights(s)
    z = float(w.sum())
    if top_p > 0 and z > 0 and math.isfinite(z) and picks > 0:
        cum = np.cumsum(w[order[:picks]])
        hit = np.nonzero(cum >= top_p * z)[0]
        if len(hit):
            m = int(hit[0]) + 1
    sel = np.sort(cand[order[:m]])
    out = np.full(int(budget), -1, dtype=np.int32)
    out[:m] = sel
    return out, m


# --------------------------------------------------------------------------
# A3 / A9: sparse attention over the selected rows, split into partials
# (Jet-QSparse abstract: sparse value aggregation with FP32 accumulation over
# the selected blocks; JSSA Figure 1: the query heads share the index set and
# read the original keys and values)
# --------------------------------------------------------------------------

def gather_rows_block(k_unit, v_unit, blocks: Sequence[int], seq_len: int, n_tail: int,
                      tail_k_unit=None, tail_v_unit=None, v_store=None
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """float64 K and V rows [n, 128] of the selected blocks, in block order.

    Tail pages (the n_tail newest) come from the BF16 tail store, slot
    page - (n_pages - n_tail); tokens at or beyond seq_len are left out. With
    v_store = (code bytes [T, 64], scale bytes [T, 8], s_v) the values of the
    other pages are the NVFP4 store's (A0v).
    """
    if v_store is not None:
        v_unit = dequant_values(*v_store)
    npg = n_pages(seq_len)
    ks, vs = [], []
    for blk in blocks:
        lo, hi = blk * BLOCK, min((blk + 1) * BLOCK, seq_len)
        if hi <= lo:
            continue
        if n_tail and blk >= npg - n_tail:
            slot = blk - (npg - n_tail)
            ks.append(bf16_bits_to_f64(tail_k_unit[slot, :hi - lo]))
            vs.append(bf16_bits_to_f64(tail_v_unit[slot, :hi - lo]))
        else:
            ks.append(np.asarray(k_unit[lo:hi], dtype=np.float64))
            vs.append(np.asarray(v_unit[lo:hi], dtype=np.float64))
    if not ks:
        return np.zeros((0, HEAD_DIM)), np.zeros((0, HEAD_DIM))
    return np.concatenate(ks), np.concatenate(vs)


# --------------------------------------------------------------------------
# Decode-time state of the cache after L tokens (the Jet-QSparse abstract: the
# newest pages stay in BF16, older ones are packed into NVFP4 from the
# full-precision keys). Reading for appends: the BF16 tail store holds BF16
# roundings of the full-precision cache rows; slot s holds page
# n_pages(L) - n_tail + s, rows at or beyond L (and slots of pages below 0)
# are zero. The 4-bit records of a token depend on that token's row only (its
# scales cover 16 channels of one token), so the copy of every token < L is
# its bulk pack.
# --------------------------------------------------------------------------

def tail_store_from_cache(rows: np.ndarray, seq_len: int, n_tail: int) -> np.ndarray:
    """BF16 bits [n_tail, 128, 128] of the tail pages of one unit's cache rows
    [T, 128] (fp16 or bf16 values) at length seq_len."""
    out = np.zeros((n_tail, BLOCK, HEAD_DIM), dtype=np.uint16)
    npg = n_pages(seq_len)
    for s in range(n_tail):
        page = npg - n_tail + s
        if page < 0:
            continue
        lo, hi = page * BLOCK, min((page + 1) * BLOCK, seq_len)
        if hi > lo:
            out[s, :hi - lo] = f32_to_bf16_bits(np.asarray(rows[lo:hi], dtype=F32))
    return out


def gather_rows_token(k_unit, v_unit, tokens: Sequence[int], v_store=None
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """float64 K and V rows of the selected tokens (values from the NVFP4 store
    (A0v) when v_store = (code bytes, scale bytes, s_v) is given)."""
    t = np.asarray(tokens, dtype=np.int64)
    if v_store is not None:
        cb, sb, s_v = v_store
        return (np.asarray(k_unit[t], dtype=np.float64).reshape(-1, HEAD_DIM),
                dequant_values(cb[t], sb[t], s_v).reshape(-1, HEAD_DIM))
    return (np.asarray(k_unit[t], dtype=np.float64).reshape(-1, HEAD_DIM),
            np.asarray(v_unit[t], dtype=np.float64).reshape(-1, HEAD_DIM))


def attend(q_group: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, sigma: float
           ) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(sigma q K^T) V for each query head: (O [G, 128], lse [G]).

    An empty row set gives O = 0 and lse = -inf.
    """
    qg = np.asarray(q_group, dtype=np.float64)
    G = qg.shape[0]
    if k_rows.shape[0] == 0:
        return np.zeros((G, HEAD_DIM)), np.full(G, -np.inf)
    logits = sigma * (qg @ k_rows.T)  # [G, n]
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    z = w.sum(axis=1, keepdims=True)
    out = (w @ v_rows) / z
    lse = (m + np.log(z))[:, 0]
    return out, lse


def split_ranges(n: int, num_splits: int):
    """Split s covers entries [s*per, min((s+1)*per, n)) of the n selected
    entries, per = ceil(n / S): the splits share the entries actually selected,
    so an adaptive budget that keeps fewer rows still spreads them evenly."""
    per = -(-n // num_splits)
    return [(min(s * per, n), min((s + 1) * per, n)) for s in range(num_splits)]


def attend_splits(q_group, idx: np.ndarray, num_splits: int, rows_fn, sigma: float):
    """Per-split partials (O_s [S, G, 128], lse_s [S, G]) over the index list.

    idx holds the selection's entries followed by -1 padding; its count is the
    number of entries before the padding. ``rows_fn(list_of_indices)`` returns
    the (K, V) rows of those entries.
    """
    idx = np.asarray(idx)
    n = int(np.count_nonzero(idx >= 0))
    assert np.all(idx[:n] >= 0) and np.all(idx[n:] < 0), "padding must follow the entries"
    parts_o, parts_l = [], []
    for lo, hi in split_ranges(n, num_splits):
        sel = [int(x) for x in idx[lo:hi]]
        kr, vr = rows_fn(sel)
        o, l = attend(q_group, kr, vr, sigma)
        parts_o.append(o)
        parts_l.append(l)
    return np.stack(parts_o), np.stack(parts_l)


# --------------------------------------------------------------------------
# A4: log-sum-exp combine of split partials
#   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) * O_s
# --------------------------------------------------------------------------

def combine(part_o: np.ndarray, part_lse: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """part_o [S, ..., D], part_lse [S, ...] -> (O [..., D], lse [...])."""
    po = np.asarray(part_o, dtype=np.float64)
    pl = np.asarray(part_lse, dtype=np.float64)
    m = pl.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(pl - m_safe[None])
    z = w.sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, z)))
    out = (w[..., None] * po).sum(axis=0) / np.where(empty, 1.0, z)[..., None]
    out[empty] = 0.0
    return out, lse


# --------------------------------------------------------------------------
# A6: projected-key cache for token mode (JSSA Figure 1: keys projected onto a
# rank-r basis common to the heads; Figure 10: the cache held in BF16 or FP8)
#
# Reading: acc[t, j] is the float32 sum over d ascending of fl32(P[d, j] *
# k[t, d]), each addition rounded to float32, no fused multiply-add; the cache
# holds BF16(acc) (round to nearest even), or for the FP8 cache E4M3FN(acc)
# element by element (nearest, ties to even, saturating at 448, no further
# scale: the figure names only the storage precision).
# --------------------------------------------------------------------------

PROJ_FORMATS = ("bf16", "fp8")


def project_keys_f32(k_rows: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """Keys [n, 128] (fp16 values) and P [128, r] (float32) -> float32 acc [n, r]."""
    kf = np.asarray(k_rows).astype(F32)
    P = np.asarray(proj, dtype=F32)
    acc = np.zeros((kf.shape[0], P.shape[1]), dtype=F32)
    for d in range(HEAD_DIM):
        prod = (kf[:, d:d + 1] * P[d][None, :]).astype(F32)
        acc = (acc + prod).astype(F32)
    return acc


def project_keys(k_rows: np.ndarray, proj: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """The cache entries: BF16 bits (uint16) or E4M3 codes (uint8), [n, r]."""
    acc = project_keys_f32(k_rows, proj)
    if fmt == "fp8":
        return nvfp4.e4m3_encode(acc)
    if fmt != "bf16":
        raise ValueError(fmt)
    return f32_to_bf16_bits(acc)


def proj_values(kproj: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """Real values of cache entries."""
    if fmt == "fp8":
        return nvfp4.e4m3_decode(kproj)
    if fmt != "bf16":
        raise ValueError(fmt)
    return bf16_bits_to_f64(kproj)


# --------------------------------------------------------------------------
# A7: token scan (JSSA Figure 1: the mean of the KV head's query heads scores
# the projected keys)
#   qbar = mean_h q_h,  p = P^T qbar,  score_t = sigma * p . kproj_t   (t < L)
# --------------------------------------------------------------------------

def scan_token_unit(q_group: np.ndarray, kproj: np.ndarray, proj: np.ndarray,
                    seq_len: int, sigma: float, fmt: str = "bf16") -> np.ndarray:
    qbar = np.asarray(q_group, dtype=np.float64).mean(axis=0)
    p = np.asarray(proj, dtype=np.float64).T @ qbar  # [r]
    kt = proj_values(kproj, fmt)  # [T, r]
    scores = sigma * (kt @ p)
    scores[np.arange(kt.shape[0]) >= seq_len] = -np.inf
    return scores


def softmax_scale(head_dim: int = HEAD_DIM) -> float:
    return 1.0 / math.sqrt(head_dim)


# --------------------------------------------------------------------------
# A10: coarse semantic blocks scored by their centroids (Coarse Semantic
# Blocks abstract)
#
# Readings: the abstract leaves the clustering method open, so the index takes
# a token -> block assignment as given (a block id per token, -1 for none);
# block c holds the tokens t < L assigned to it, in ascending order, and its
# centroid is the mean of their keys (a block with no token has none and is
# never chosen). A KV head's query heads pick one block set together (the
# token and block modes' sharing): a block's score is the largest over the
# head's queries of sigma q . centroid. Blocks are ranked by score (descending,
# the lower block id first among equal scores, NaN last); the chosen blocks are
# the longest prefix of that ranking whose sizes add up to at most the token
# budget (whole blocks only). The attention reads the chosen blocks' tokens,
# block after block in ranking order, members ascending.
# --------------------------------------------------------------------------

def cluster_index(k_unit: np.ndarray, assign: np.ndarray, n_clusters: int, seq_len: int
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(centroids [C, 128] float64, offsets [C + 1], members [offsets[C]]) of
    one unit: block c's tokens are members[offsets[c]:offsets[c + 1]]."""
    L = int(seq_len)
    a = np.asarray(assign[:L], dtype=np.int64)
    members, offsets = [], [0]
    cent = np.zeros((n_clusters, HEAD_DIM))
    for c in range(n_clusters):
        toks = np.nonzero(a == c)[0]
        members.append(toks)
        offsets.append(offsets[-1] + len(toks))
        if len(toks):
            cent[c] = np.asarray(k_unit[toks], dtype=np.float64).mean(axis=0)
    return cent, np.asarray(offsets, dtype=np.int64), (
        np.concatenate(members) if members else np.zeros(0, dtype=np.int64))


def cluster_scores(q_group: np.ndarray, centroids: np.ndarray, sizes: np.ndarray,
                   sigma: float) -> np.ndarray:
    """score_c = max over the group's query heads of sigma q . centroid_c;
    -inf for a block with no token."""
    q = np.asarray(q_group, dtype=np.float64)
    s = sigma * (np.asarray(centroids, dtype=np.float64) @ q.T).max(axis=1)
    return np.where(np.asarray(sizes) > 0, s, -np.inf)


def select_clusters(scores: np.ndarray, sizes: np.ndarray, budget: int
                    ) -> Tuple[np.ndarray, int]:
    """Chosen block ids in ranking order: the longest prefix of the ranking of
    the non-empty blocks whose sizes sum to at most budget; and that sum."""
    s = np.asarray(scores, dtype=np.float64)
    ids = np.arange(len(s))
    key = np.where(np.isnan(s), -np.inf, s)
    nan_last = np.isnan(s).astype(np.int64)
    order = np.lexsort((ids, -key, nan_last))  # NaN last, then score desc, then id
    chosen, total = [], 0
    for c in order:
        if sizes[c] == 0:
            continue
        if total + int(sizes[c]) > budget:
            break
        chosen.append(int(c))
        total += int(sizes[c])
    return np.asarray(chosen, dtype=np.int64), total


def cluster_tokens(chosen: np.ndarray, offsets: np.ndarray, members: np.ndarray,
                   budget: int) -> Tuple[np.ndarray, int]:
    """The tokens the attention reads (the chosen blocks' members, block after
    block), padded with -1 to budget; and their count."""
    toks = [members[offsets[c]:offsets[c + 1]] for c in chosen]
    t = np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)
    out = np.full(budget, -1, dtype=np.int32)
    out[:len(t)] = t
    return out, int(len(t))

