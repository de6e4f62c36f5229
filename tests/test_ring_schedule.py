"""The ring's step schedule (bench.py's caller-side rule, CPU only): the key
shards a query shard computes against are exactly those holding a key some
row of the shard can see (same document, not after the row), by brute force
over every (row, key) pair on small random document layouts."""

import numpy as np
import pytest

import bench


def _visible_shards(lengths, S, P, i):
    doc = np.repeat(np.arange(len(lengths)), lengths)   # document of each token
    L = S // P
    rows = np.arange(i * L, (i + 1) * L)
    out = set()
    for j in range(P):
        keys = np.arange(j * L, (j + 1) * L)
        seen = (keys[None, :] <= rows[:, None]) & (doc[keys][None, :] == doc[rows][:, None])
        if seen.any():
            out.add(j)
    return out


@pytest.mark.parametrize("seed", range(40))
def test_ring_schedule_is_the_set_of_visible_key_shards(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.choice([2, 4, 8]))
    S = P * int(rng.integers(1, 12))
    n_docs = int(rng.integers(1, min(S, 9) + 1))
    cuts = np.sort(rng.choice(np.arange(1, S), size=n_docs - 1, replace=False)) if n_docs > 1 else np.array([], int)
    cu = np.concatenate([[0], cuts, [S]]).astype(np.int32)
    lengths = np.diff(cu)
    for i in range(P):
        sched = bench.ring_schedule(cu, S, P, i)
        assert sched[0] == i                                   # own shard first
        assert len(set(sched)) == len(sched)
        want = _visible_shards(lengths, S, P, i)
        assert set(sched) == want, (cu.tolist(), P, i, sched, sorted(want))
        order = [(i - s) % P for s in range(P)]
        assert sched == [j for j in order if j in want]        # ring order kept
