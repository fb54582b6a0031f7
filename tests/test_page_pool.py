"""Host logic of the KV page allocator used by end-to-end generation (CPU)."""
import numpy as np
import pytest
import torch

import synth


class _FakeKV:
    def __init__(self, batch, max_pages, n_pages, ps=16):
        self.batch, self.max_pages, self.n_pages, self.page_size = batch, max_pages, n_pages, ps
        self.page_table = torch.zeros((batch, max_pages), dtype=torch.int32)


def test_pages_are_distinct_ordered_and_returned():
    from lossless_decoding_uno_amd.generate import PagePool
    kv = _FakeKV(batch=3, max_pages=8, n_pages=12)
    pool = PagePool(kv)
    pool.ensure(0, 40)          # 3 pages
    pool.ensure(1, 16)          # 1 page
    pool.ensure(0, 48)          # still 3 pages
    pool.ensure(2, 17)          # 2 pages
    pool.sync()
    owned = pool.owned
    assert [len(o) for o in owned] == [3, 1, 2]
    flat = [p for o in owned for p in o]
    assert len(set(flat)) == len(flat) and all(0 <= p < 12 for p in flat)
    for b in range(3):
        assert kv.page_table[b, : len(owned[b])].tolist() == owned[b]
    pool.release(0)
    assert pool.pages_in_use() == 3 and len(pool.free) == 9
    pool.ensure(1, 16 * 4)      # reuses the released pages
    assert len(set(pool.owned[1])) == 4
    with pytest.raises(RuntimeError):
        pool.ensure(2, 16 * 9)  # more than the table holds
    pool.ensure(1, 16 * 8)
    with pytest.raises(RuntimeError):   # pool exhausted: 8 + 2 + 3 > 12
        pool.ensure(0, 16 * 3)


def test_tpf_bounds_definition():
    """TPF = committed tokens per step / 2 passes lies in [1, (K+1)/2] when the
    first draft is always kept (paperglide reader, "The Uno Framework")."""
    K = 16
    for a in range(1, K + 1):
        tpf = (a + 1) / 2.0
        assert 1.0 <= tpf <= (K + 1) / 2.0
