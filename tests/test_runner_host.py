"""Host logic of the runner that needs no GPU: the page allocator behind continuous batching."""
import pytest

from tree_attention_verification_06_amd._abi import EagleError
from tree_attention_verification_06_amd.runner import PagePool


def test_page_pool_reserve_grow_release_reuse():
    pool = PagePool(n_pages=6, page_size=64, max_blocks=3, device="cpu")
    assert pool.reserve("a", 100) == [0, 1]          # ceil(100 / 64) pages
    assert pool.reserve("a", 120) == [0, 1]          # already enough
    assert pool.reserve("b", 64) == [2]
    assert pool.reserve("a", 129) == [0, 1, 3]       # grows page by page
    t = pool.table(["a", "b", "c"])
    assert t.tolist() == [[0, 1, 3], [2, -1, -1], [-1, -1, -1]]
    pool.release("a")
    # released pages are handed out first, in their order
    assert pool.reserve("c", 130) == [0, 1, 3]
    assert sorted(pool.free) == [4, 5]


def test_page_pool_limits():
    pool = PagePool(n_pages=3, page_size=64, max_blocks=2, device="cpu")
    with pytest.raises(EagleError):
        pool.reserve("a", 129)                        # more than max_blocks pages
    pool.reserve("a", 128)
    pool.reserve("b", 64)
    with pytest.raises(EagleError):
        pool.reserve("c", 1)                          # pool exhausted
    pool.release("b")
    assert pool.reserve("c", 1) == [2]
    pool.release("nobody")                            # releasing an unknown sequence is a no-op
