"""bsa_decode_step_noalloc: the step with its intermediates in the library's
per-GPU scratch gives bsa_decode_step's output bits, call after call, with a
smaller step following a larger one on the same scratch."""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_attention_pack_amd import binding as B
from block_sparse_attention_pack_amd import workloads as W
from block_sparse_attention_pack_amd.step import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()


def _noalloc(d):
    out = torch.full_like(d.out, 7.0)
    lse = torch.full_like(d.out_lse, 7.0)
    B.decode_step_noalloc(d.layout, d.cfg, d.q, d.codes, d.scales, d.global_scale,
                          d.key_center, d.kproj, d.proj, d.k, d.v, d.seq_lens, d.tail_k, d.tail_v,
                          d.splits, out, lse)
    return out, lse


def _check(spec, splits=None):
    print(f"[noalloc] {spec.name} splits {splits}", flush=True)
    sys.stdout.flush()
    w = W.generate(spec)
    d = upload(w, splits=splits)
    d.pack()
    d.decode_step()
    torch.cuda.synchronize()
    ref = (d.out.cpu().numpy().copy(), d.out_lse.cpu().numpy().copy())
    out, lse = _noalloc(d)
    torch.cuda.synchronize()
    assert np.array_equal(ref[0], out.cpu().numpy()), spec.name
    assert np.array_equal(ref[1], lse.cpu().numpy(), equal_nan=True), spec.name


@pytest.mark.parametrize("mode", ["block", "token"])
def test_noalloc_matches_decode_step_twice_then_smaller(mode):
    if mode == "block":
        big = dataclasses.replace(W.reduced("ragged", 16384, batch=3, budget=24), name="na_big")
        small = dataclasses.replace(W.reduced("jetqsparse", 4096, batch=1, budget=8),
                                    name="na_small")
    else:
        big = dataclasses.replace(W.reduced("token", 16384, batch=2), name="na_tbig")
        small = dataclasses.replace(W.reduced("token", 4096, batch=1, budget=64),
                                    name="na_tsmall")
    _check(big)
    _check(big, splits=12)  # more splits than the in-kernel merge takes: the merge launch
    _check(small)


def test_noalloc_top_p_nvfp4_query_and_value_store():
    _check(W.reduced("token_topp", 16384, batch=2))
    _check(W.reduced("jetqsparse_q4", 8192, batch=2))
    _check(W.reduced("jetqsparse_v4", 8192, batch=2))
    _check(dataclasses.replace(W.reduced("ragged", 16384, batch=3, budget=24), name="na_v4_tail",
                               value_fmt="nvfp4"))
