"""The oracle's plain pool model against the lease rules it states."""
import random

import oracle as O


def test_lease_all_or_nothing_and_conservation():
    order = list(range(40))
    random.Random(0).shuffle(order)
    p = O.PoolModel(order, 16, 8)
    assert p.lease("a", 100)                # 7 pages
    assert p.pages["a"] == order[:7]
    assert not p.lease("b", 16 * 34)        # 34 > 33 free: refused, unchanged
    assert len(p.free) == 33 and "b" not in p.pages
    assert p.lease("b", 16 * 33)
    assert len(p.free) == 0
    p.release("a")
    assert list(p.free) == order[:7]        # appended to the back in page order
    owned = [x for s in p.pages.values() for x in s] + list(p.free)
    assert sorted(owned) == list(range(40))


def test_page_table_and_slots():
    p = O.PoolModel(range(10), 16, 2)
    assert p.lease(5, 20) and p.lease(9, 1)
    assert not p.lease(3, 1)                # no slot left
    assert p.page_table([5, 9], 3) == [[0, 1, -1], [2, -1, -1]]
    assert p.slot == {5: 0, 9: 1}
    p.release(5)
    assert p.lease(3, 1) and p.slot[3] == 0
