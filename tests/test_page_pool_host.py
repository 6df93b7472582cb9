"""The library's native page pool (host code, no GPU) against the oracle's
model, step by step on seeded random scripts: block tables, lengths, copy
pairs, reference counts, free counts and error behaviour must be identical
(the allocation order is fixed, lowest free id first, so every entry is
comparable)."""
import numpy as np
import pytest
import torch

from flashattention_paged_kv_amd import ops
from oracle import pages
import test_oracle_pages as scripts

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(ops.LIB_PATH), reason="library not built")

NUM_PAGES, P, SEQS, MAXP = 24, 16, 6, 8


def _same(pool, model):
    assert np.array_equal(pool.block_table().numpy(), model.block_table())
    assert pool.lens().tolist() == model.lens
    assert pool.free_pages() == len(model.free_pages())
    assert [pool.refcount(p) for p in range(NUM_PAGES)] == model.refcount


@pytest.mark.parametrize("seed", range(8))
def test_native_pool_matches_model(seed):
    pool = ops.PagePool(NUM_PAGES, P, SEQS, MAXP)
    model = pages.PagePoolModel(NUM_PAGES, P, SEQS, MAXP)
    for op in scripts.random_script(100 + seed, n_ops=150):
        if op[0] == "extend":
            s = op[1]
            new = min(model.lens[s] + op[2], MAXP * P)
            try:
                want = model.extend(s, new)
            except MemoryError:
                with pytest.raises(ops.PagedAttnError) as e:
                    pool.extend(s, new)
                assert e.value.status == 5
            else:
                assert pool.extend(s, new) == want
        elif op[0] == "fork":
            parent, child, frac = op[1], op[2], op[3]
            if parent == child or model.lens[child] != 0 or model.lens[parent] == 0:
                with pytest.raises(ops.PagedAttnError) as e:
                    pool.fork(parent, child, max(1, int(frac * max(model.lens[parent], 1))) if parent != child else 1)
                assert e.value.status == 1
                continue
            n = max(1, int(frac * model.lens[parent]))
            model.fork(parent, child, n)
            pool.fork(parent, child, n)
        else:
            model.release(op[1])
            pool.release(op[1])
        _same(pool, model)


def test_native_pool_rejects_bad_arguments():
    pool = ops.PagePool(4, 16, 2, 2)
    for call, status in [(lambda: pool.extend(2, 1), 1), (lambda: pool.extend(0, 33), 1),
                         (lambda: pool.fork(0, 1, 1), 1), (lambda: pool.release(-1), 1)]:
        with pytest.raises(ops.PagedAttnError) as e:
            call()
        assert e.value.status == status
    pool.extend(0, 20)
    with pytest.raises(ops.PagedAttnError) as e:
        pool.extend(0, 10)            # sequences do not shrink
    assert e.value.status == 1
    pool.fork(0, 1, 20)
    with pytest.raises(ops.PagedAttnError) as e:
        pool.extend(1, 40)            # three pages for one sequence: beyond max_pages_per_seq
    assert e.value.status == 1


def test_native_pool_out_of_pages_changes_nothing():
    pool = ops.PagePool(3, 16, 2, 4)
    pool.extend(0, 33)                # all three pages
    pool.fork(0, 1, 20)
    before = (pool.block_table().clone(), pool.lens().clone(), [pool.refcount(p) for p in range(3)])
    with pytest.raises(ops.PagedAttnError) as e:
        pool.extend(1, 21)            # must copy the shared page 1: no free page
    assert e.value.status == 5
    assert torch.equal(pool.block_table(), before[0]) and torch.equal(pool.lens(), before[1])
    assert [pool.refcount(p) for p in range(3)] == before[2]
