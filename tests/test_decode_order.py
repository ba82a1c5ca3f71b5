"""kv_decode_order (host): a permutation of the batch, lengths non-increasing, equal
lengths in batch order; checked against Python's stable sort on random lengths."""

import numpy as np
import pytest

import paged_kv_cache_68_amd as pk


@pytest.mark.parametrize("seed", range(10))
def test_longest_first_stable(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 600))
    lens = rng.integers(-2, 50 if seed % 2 else 5000, size=n).astype(np.int32)
    order = pk.decode_order(lens)
    assert order.dtype == np.int32 and order.shape == (n,)
    assert sorted(order.tolist()) == list(range(n))
    want = sorted(range(n), key=lambda i: -int(lens[i]))       # Python's sort is stable
    assert order.tolist() == want


def test_edges():
    assert pk.decode_order(np.array([], dtype=np.int32)).shape == (0,)
    assert pk.decode_order([7]).tolist() == [0]
    assert pk.decode_order([1, 3, 3, 2]).tolist() == [1, 2, 3, 0]
    with pytest.raises(ValueError):
        pk.decode_order(np.zeros((2, 2), dtype=np.int32))
