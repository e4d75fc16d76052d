"""per_update_static, the update that allocates nothing (its bucketed
scratch lives in the library's static device array), against per_update on
the same inputs, through the C ABI: both trees and the running max bit for
bit, two calls in a row with the second smaller, for thin batches (four
partitions per update block), dense batches (one partition per block) and
crowded partitions (entries past a bucket go to the overflow list)."""
import numpy as np
import pytest
import torch

from parity_util import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu


def _pair(n, max_batch, seed):
    from sum_tree_sampling_amd import PerBuffer
    rng = np.random.default_rng(seed)
    p0 = (rng.random(n) ** 0.6).astype(np.float32)
    a = PerBuffer(n, 0, max_batch=max_batch)
    b = PerBuffer(n, 0, max_batch=max_batch)
    a.add(n, prio=dev(p0))
    b.add(n, prio=dev(p0))
    return a, b, rng


def _same(a, b, what):
    torch.cuda.synchronize()
    assert_bits_equal(host(b.sum_tree()), host(a.sum_tree()), what + " sum tree")
    assert_bits_equal(host(b.min_tree()), host(a.min_tree()), what + " min tree")
    assert_bits_equal(host(b.scalar("max_priority")), host(a.scalar("max_priority")),
                      what + " running max")


@pytest.mark.parametrize("L,batches,crowd", [
    (22, (4096, 2500), False),    # 1024 partitions: thin bucketed batches
    (20, (16384, 9000), False),   # 256 partitions, > 16 entries each: one partition per block
    (22, (6000, 2600), True),     # most entries in three partitions: overflow list
    (24, (65536, 30000), False),  # the largest capacity and batch the array holds
    (21, (300, 200), False),      # small batches: no scratch at all
])
def test_update_static_matches_update(L, batches, crowd):
    n = 1 << L
    say("update_static", L, batches, crowd)
    a, b, rng = _pair(n, max(batches), L + len(batches))
    for call, B in enumerate(batches):
        idx = rng.integers(0, n, B).astype(np.int64)
        if crowd:
            k = B * 3 // 4
            idx[:k] = rng.integers(0, 3, k) * 4096 + rng.integers(0, 4096, k)
        idx[: B // 10] = idx[B // 10: 2 * (B // 10)]   # repeats: the last one wins
        idx[-1] = -1                                   # skipped
        td = (rng.standard_normal(B) * 2).astype(np.float32)
        td[rng.integers(0, B, 3)] = np.nan
        a.update(dev(idx), dev(td))
        b.update_static(dev(idx), dev(td))
        _same(a, b, "L=%d call %d (B=%d)" % (L, call, B))
    a.close()
    b.close()


def test_update_static_limits():
    """Bucketed batches beyond the array's limits are refused before any work."""
    from sum_tree_sampling_amd import PerBuffer, PerError
    n = 1 << 25  # 8192 partitions: more than the array holds
    g = PerBuffer(n, 0, max_batch=4096)
    before = host(g.sum_tree()).copy()
    idx = torch.zeros(4096, dtype=torch.int64, device="cuda")
    td = torch.ones(4096, dtype=torch.float32, device="cuda")
    with pytest.raises(PerError) as e:
        g.update_static(idx, td)
    assert e.value.code == -1
    torch.cuda.synchronize()
    assert_bits_equal(host(g.sum_tree()), before, "refused call left the tree")
    g.close()
