"""Host checks of the synthetic workload shapes (no GPU, no arithmetic of
the method): the parameter counts the configurations are quoted with, and
the ZeRO-1 block sharding used for the per-GPU shard shape."""
import numpy as np
import pytest

import workloads


def _n(shapes):
    return sum(int(np.prod(s)) for _, s in shapes)


def _blocks(shapes):
    return sum(-(-int(np.prod(s)) // 2048) for _, s in shapes)


def test_parameter_counts():
    assert _n(workloads.vit_base_shapes()) == 86_567_656
    assert len(workloads.vit_base_shapes()) == 152
    assert _n(workloads.llama_7b_shapes()) == 6_738_415_616
    assert _blocks(workloads.llama_7b_shapes()) == 3_290_242
    assert _n(workloads.gpt_1p3b_shapes(with_tail_set=False)) == 1_315_819_520


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 8])
def test_zero1_shards_partition_the_blocks(n_ranks):
    full = workloads.llama_7b_shapes()
    sizes = {name: int(np.prod(s)) for name, s in full}
    seen = {name: [] for name in sizes}
    counts = []
    for r in range(n_ranks):
        shard = workloads.zero1_shard_shapes(full, r, n_ranks)
        counts.append(_blocks(shard))
        for name, (ln,) in shard:
            base, rng = name.rsplit("[", 1)
            lo, hi = (int(x) for x in rng.rstrip("]").split(":"))
            assert hi - lo == ln and lo % 2048 == 0      # cuts on block boundaries
            assert hi == sizes[base] or hi % 2048 == 0
            seen[base].append((lo, hi))
    # every element of every tensor lands in exactly one shard, in order
    for name, spans in seen.items():
        spans.sort()
        assert spans[0][0] == 0 and spans[-1][1] == sizes[name]
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
    assert sum(counts) == _blocks(full) and max(counts) - min(counts) <= 1


def test_llama_shard8_shape():
    shard = workloads.llama_7b_shard8_shapes()
    assert _n(shard) == 842_301_440 and _blocks(shard) == 411_280
