"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each workload is drawn at its full size (up to 128K tokens, batch 16), packed,
and run through the same calls bench.py times by default, with its default split
count: one decode_step launch where that pays off (block mode, at least 16384
scanned blocks, sequence lengths that differ), else score_scan and
select_attend_combine. Every stage of a few sampled units
(the first, the last and one in between) is then checked against the oracle:
pack bytes bit-exact, scores within the FP32 accumulation bound, the selection
bit-exact on the GPU's own scores, outputs within 2e-3.
"""

import sys

import pytest

torch = pytest.importorskip("torch")

from block_sparse_attention_pack_amd import workloads as W
from block_sparse_attention_pack_amd.step import one_launch_pays, upload

import parity_util as PU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_attention_pack_amd import binding

    binding.load()


def _sampled_units(spec):
    units = [(0, 0), (spec.batch - 1, spec.kv_heads - 1),
             (spec.batch // 2, spec.kv_heads // 2)]
    return sorted(set(units))


@pytest.mark.parametrize("name", W.ORDER)
def test_full_size_sampled_units(name):
    spec = W.SPECS[name]
    print(f"[full] {name}: generating", flush=True)
    w = W.generate(spec, threads=16)
    one = one_launch_pays(spec.units, spec.max_blocks, spec.granularity,
                          len(set(int(x) for x in w.seq_lens)) > 1)
    d = upload(w, one_launch=one)  # the default split count, as bench.py uses
    d.pack()
    if one:
        d.decode_step()
    else:
        d.scan()
        d.select_attend_combine()
    torch.cuda.synchronize()
    assert int(d.counters.abs().sum()) == 0
    units = _sampled_units(spec)
    print(f"[full] {name}: {'decode_step' if one else 'two calls'}, splits {d.splits}, "
          f"checking units {units}", flush=True)
    sys.stdout.flush()
    PU.check_units(w, d, units)
    del d
    torch.cuda.empty_cache()
