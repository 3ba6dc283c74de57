"""Parity of the 4-bit value store with the oracle (through the C ABI).

The store is packed on the GPU (bsa_pack_values) and must equal the oracle's
packing bit for bit; the attention then reads the store's values (E2M1 codes
times the row's E4M3 scale times the KV head's FP32 scale) and must match the
oracle's attention over the dequantized values within 2e-3. Cases: block and
token mode, BF16 tail pages (read from the BF16 store, never from the 4-bit
one), query-group sizes 1..16, a BF16 cache, every block selected (dense
attention), and rows the attention must not read filled with NaN scale codes.
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_attention_pack_amd import workloads as W
from block_sparse_attention_pack_amd.step import upload

import parity_util as PU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_attention_pack_amd import binding

    binding.load()  # fails loudly when the library is missing


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.cpu().numpy()


def run_step(w, splits=None, kv_dtype="f16"):
    d = upload(w, splits=splits, kv_dtype=kv_dtype)
    assert d.value_store
    d.pack()
    d.run()
    torch.cuda.synchronize()
    return d


def v4(spec, name):
    return dataclasses.replace(spec, name=name, value_fmt="nvfp4")


CASES = {
    "block": W.reduced("jetqsparse_v4", 8192, batch=2),
    "ragged_tail2": v4(W.reduced("ragged", 16384, batch=3, budget=24), "ragged_v4"),
    "token": v4(W.reduced("token", 16384, batch=2), "token_v4"),
    "llama8b": v4(W.reduced("llama8b", 8192), "llama8b_v4"),
    "dense": W.reduced("jetqsparse_v4", 4096, batch=1, budget=32),
}


@pytest.mark.parametrize("name", list(CASES))
def test_value_store_workloads_match_oracle(name):
    spec = CASES[name]
    _say(f"[v4] {spec.name}")
    w = W.generate(spec)
    d = run_step(w)
    PU.check_units(w, d)
    PU.check_forms_match(d)


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_value_store_query_group_sizes(G):
    spec = dataclasses.replace(W.SPECS["tiny"], name=f"v4group{G}", seed=40 + G, batch=2,
                               kv_heads=2, q_heads=2 * G, max_tokens=2048, budget=5,
                               n_tail=1, value_fmt="nvfp4", lengths=(2048, 1500))
    w = W.generate(spec)
    d = run_step(w)
    PU.check_units(w, d)
    PU.check_forms_match(d)
    tspec = dataclasses.replace(W.SPECS["token"], name=f"v4tgroup{G}", seed=50 + G, batch=1,
                                kv_heads=2, q_heads=2 * G, max_tokens=4096, budget=96,
                                value_fmt="nvfp4")
    w = W.generate(tspec)
    d = run_step(w)
    PU.check_units(w, d)


def test_value_store_from_a_bf16_cache():
    spec = W.reduced("jetqsparse_v4", 4096, batch=2, budget=10)
    w = W.generate(spec)
    d = run_step(w, kv_dtype="bf16")
    # the oracle packs the bf16-rounded keys and values the GPU holds
    w16 = dataclasses.replace(w, k=host(d.k.float()), v=host(d.v_src.float()))
    PU.check_units(w16, d)


@pytest.mark.parametrize("n_tail", [0, 1])
def test_rows_past_the_length_and_tail_rows_are_not_read(n_tail):
    """Store rows the attention must skip (past each sequence's end, and the
    pages the BF16 tail store holds) are overwritten with 0xFF bytes, whose
    scale byte is an E4M3 NaN code: the outputs still match the oracle's, which
    never reads them."""
    spec = dataclasses.replace(W.SPECS["ragged"], name=f"v4mask{n_tail}", seed=70 + n_tail,
                               batch=5, kv_heads=2, q_heads=8, max_tokens=1024, budget=4,
                               n_tail=n_tail, needle_count=1, value_fmt="nvfp4",
                               lengths=(0, 1, 127, 129, 700))
    w = W.generate(spec)
    d = upload(w, splits=2)
    d.pack()
    codes, scales, _ = PU.store_views(d)
    for b in range(spec.batch):
        L = int(w.seq_lens[b])
        first = max(0, min(L, (w.n_pages(b) - n_tail) * 128)) if n_tail else L
        codes[b, :, first:] = 0xFF
        scales[b, :, first:] = 0xFF
    d.run()
    torch.cuda.synchronize()
    G = spec.group
    for b in range(spec.batch):
        for h in range(spec.kv_heads):
            rows = slice(h * G, (h + 1) * G)
            assert np.all(np.isfinite(host(d.out[b, rows])))
            PU.check_attention(w, b, h, host(d.idx[b, h]), d.splits, host(d.part_o[b, rows]),
                               host(d.part_lse[b, rows]), host(d.out[b, rows]),
                               host(d.out_lse[b, rows]), PU.oracle_value_store(w, b, h))
