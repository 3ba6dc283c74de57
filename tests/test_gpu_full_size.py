"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each workload is drawn at its full size (up to 128K tokens, batch 16), packed,
and run through the same calls bench.py times by default, with its default split
count (step.default_form). Every stage of sampled units (the first, the last
and others spread between them) is then checked against the oracle:
pack bytes bit-exact, scores within the FP32 accumulation bound, the selection
bit-exact on the GPU's own scores, outputs within 2e-3.
"""

import sys

import pytest

torch = pytest.importorskip("torch")

from block_sparse_attention_pack_amd import workloads as W
from block_sparse_attention_pack_amd.step import default_form, step_calls, upload

import parity_util as PU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_attention_pack_amd import binding

    binding.load()


def _sampled_units(spec, n=6):
    """n units spread over the batch and the KV heads, the first and last included."""
    U = spec.batch * spec.kv_heads
    picks = sorted(set([0, U - 1] + [(U * i) // (n - 1) + i % spec.kv_heads for i in range(1, n - 1)]))
    return [(u // spec.kv_heads, u % spec.kv_heads) for u in picks if u < U]


@pytest.mark.parametrize("name", W.ORDER)
def test_full_size_sampled_units(name):
    spec = W.SPECS[name]
    print(f"[full] {name}: generating", flush=True)
    w = W.generate(spec, threads=16)
    form = default_form(spec.granularity)
    d = upload(w)  # the default split count, as bench.py uses
    d.pack()
    for call in step_calls(d, form):
        call()
    torch.cuda.synchronize()
    assert int(d.counters.abs().sum()) == 0
    units = _sampled_units(spec)
    print(f"[full] {name}: {form}, splits {d.splits}, checking units {units}", flush=True)
    sys.stdout.flush()
    PU.check_units(w, d, units)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["jetqsparse", "token"])
def test_full_size_every_unit_selection_and_output(name):
    """Every unit of the bench's block and token workloads at full size, in the
    bench's launch configuration: the selection is exactly the oracle's on the
    GPU's own scores, and the partials, output and lse agree with the oracle's
    attention over that selection (the scan's scores are checked against the
    oracle's on the sampled units above, whose packing the oracle repeats)."""
    import numpy as np

    from oracle import decode as O

    spec = W.SPECS[name]
    print(f"[full-all] {name}: generating", flush=True)
    w = W.generate(spec, threads=16)
    d = upload(w)
    d.pack()
    for call in step_calls(d, default_form(spec.granularity)):
        call()
    torch.cuda.synchronize()
    assert int(d.counters.abs().sum()) == 0
    scores, idx, count = (t.cpu().numpy() for t in (d.scores, d.idx, d.count))
    part_o, part_lse, out, out_lse = (t.cpu().numpy() for t in (d.part_o, d.part_lse, d.out,
                                                                 d.out_lse))
    G = spec.group
    for b in range(spec.batch):
        L = int(w.seq_lens[b])
        for h in range(spec.kv_heads):
            sg = scores[b, h].astype(np.float64)
            if spec.granularity == "block":
                ref_idx, ref_cnt = O.select_blocks_unit(sg, L, spec.n_tail, spec.budget)
            else:
                ref_idx, ref_cnt = O.select_tokens_unit(sg, L, spec.budget)
            assert int(count[b, h]) == ref_cnt, (b, h)
            assert np.array_equal(idx[b, h], ref_idx), f"selection differs at {(b, h)}"
            rows = slice(h * G, (h + 1) * G)
            PU.check_attention(w, b, h, idx[b, h], d.splits, part_o[b, rows], part_lse[b, rows],
                               out[b, rows], out_lse[b, rows])
        print(f"[full-all] {name}: sequence {b} ok", flush=True)
    del d
    torch.cuda.empty_cache()
