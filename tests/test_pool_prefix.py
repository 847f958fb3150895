"""Prefix sharing in the page pool (host only), C ABI against the oracle's model.

Reading of the kern page, "The runtime": a finished request's pages freeze
in place as a checkpoint; a later request with the same prefix shares the
whole pages and gets a copy of only the page the prefix ends inside (at
most one writer per page); a token radix tree finds the longest checkpoint;
under pressure checkpoints are dropped, least recently used first.

- a worked example at 4 tokens per page, every expected value derived by
  hand from that reading (shared pages, matched length, page copies, slot
  and free-list order, eviction order, refusal when only held pages are
  left), checked against both the library and the oracle's model;
- seeded random mixes of prefix leases, extensions, finishes and releases
  over prompts that share prefixes: the library and the model agree on
  every result and page table, and the model's state keeps the invariants
  (every page free or held, never both; a page written by at most one
  sequence; shared pages hold the tokens the sharer's prompt has there);
- the error paths leave the pool unchanged.
"""
import random

import pytest

import decode_megakernel_persistent_amd as mk
import oracle as O

PT = 4


class Both:
    """The library's pool and the oracle's model driven in lockstep."""

    def __init__(self, n_pages, n_slots, order=None):
        order = list(range(n_pages)) if order is None else order
        self.lib = mk.mk_pool_create(n_pages, PT, n_slots, order)
        self.ref = O.PoolModel(order, PT, n_slots)
        self.live = {}

    def lease_prefix(self, seq, prompt, worst):
        want = self.ref.lease(seq, worst, prompt)
        try:
            got = mk.mk_pool_lease_prefix(self.lib, seq, prompt, worst)
        except mk.MkError as e:
            assert e.status == mk.MK_ENOMEM, e
            got = None
        assert got == want, f"lease {seq}: library {got}, model {want}"
        if got is not None:
            self.live[seq] = list(prompt)
        self.same()
        return got

    def lease(self, seq, worst):
        want = self.ref.lease(seq, worst)
        try:
            got = mk.mk_pool_lease(self.lib, seq, worst)
        except mk.MkError as e:
            assert e.status == mk.MK_ENOMEM, e
            got = None
        assert (got is None) == (want is None) and (got is None or got == want[0])
        if got is not None:
            self.live[seq] = []
        self.same()
        return want

    def extend(self, seq, tokens):
        want = self.ref.extend(seq, tokens)
        try:
            mk.mk_pool_extend(self.lib, seq, tokens)
            got = True
        except mk.MkError as e:
            assert e.status == mk.MK_ENOMEM
            got = False
        assert got == want
        self.same()
        return got

    def finish(self, seq, tokens):
        assert self.ref.finish(seq, tokens) == "ok"
        mk.mk_pool_finish(self.lib, seq, tokens)
        del self.live[seq]
        self.same()

    def release(self, seq):
        self.ref.release(seq)
        mk.mk_pool_release(self.lib, seq)
        del self.live[seq]
        self.same()

    def pages(self, seq):
        return self.ref.pages[seq]

    def same(self):
        assert mk.mk_pool_free_pages(self.lib) == len(self.ref.free)
        assert mk.mk_pool_cached_pages(self.lib) == self.ref.cached()
        seqs = sorted(self.ref.pages)
        if seqs:
            width = max(len(v) for v in self.ref.pages.values()) or 1
            assert mk.mk_pool_page_table(self.lib, seqs, width) == self.ref.page_table(seqs, width)


def test_worked_example():
    b = Both(16, 8)
    # A: nothing cached yet; pages 0, 1, 2 for 12 tokens
    assert b.lease_prefix(1, list(range(1, 11)), 12) == (0, 0, -1, -1)
    assert b.pages(1) == [0, 1, 2]
    # A ends after 10 tokens: [1..4]@0, [5..8]@1 and the tail [9, 10]@2 freeze
    b.finish(1, list(range(1, 11)))
    assert b.ref.cached() == 3 and list(b.ref.free) == list(range(3, 16))
    # B: at most 6 of its 7 tokens reused; page 0 shared, the match ends
    # inside page 1 (2 of its tokens), which is copied into fresh page 3
    assert b.lease_prefix(2, [1, 2, 3, 4, 5, 6, 99], 8) == (0, 6, 1, 3)
    assert b.pages(2) == [0, 3]
    # C: 10 of 11 reused; pages 0 and 1 shared, the tail page 2 copied to 4
    assert b.lease_prefix(3, list(range(1, 12)), 12) == (1, 10, 2, 4)
    assert b.pages(3) == [0, 1, 4]
    # B ends: page 0 is met on the tree, its own page 3 freezes as [5, 6, 99]
    b.finish(2, [1, 2, 3, 4, 5, 6, 99])
    assert b.ref.cached() == 4 and len(b.ref.free) == 11
    # D: [5, 6, 99] beats [5, 6, 7, 8] after page 0: 7 tokens, copy of page 3
    assert b.lease_prefix(4, [1, 2, 3, 4, 5, 6, 99, 7], 9) == (0, 7, 3, 5)
    assert b.pages(4) == [0, 5, 6]
    # C is dropped unfinished: only its private page 4 returns, to the back
    b.release(3)
    assert list(b.ref.free) == list(range(7, 16)) + [4]
    # E takes the 10 free pages; F then forces an eviction: the least
    # recently used leaf no one holds is the tail [9, 10] (page 2)
    assert b.lease(5, 40) is not None and b.pages(5) == list(range(7, 16)) + [4]
    assert b.lease(6, 4) is not None and b.pages(6) == [2]
    assert b.ref.cached() == 3
    # G needs two: [5..8]@1 (now a leaf) and then [5, 6, 99]@3
    assert b.lease(7, 8) is not None and b.pages(7) == [1, 3]
    assert b.ref.cached() == 1
    # H: the only checkpoint left (page 0) is held by D: refused, no change
    assert b.lease(8, 4) is None
    assert b.ref.cached() == 1 and len(b.ref.free) == 0
    # D ends after 8 tokens: page 5 freezes as [5, 6, 99, 7]; page 6 is freed
    b.finish(4, [1, 2, 3, 4, 5, 6, 99, 7])
    assert b.ref.cached() == 2 and list(b.ref.free) == [6]
    # I reuses 8 of 9 tokens as two whole pages and copies nothing
    assert b.lease_prefix(9, [1, 2, 3, 4, 5, 6, 99, 7, 8], 12) == (0, 8, -1, -1)
    assert b.pages(9) == [0, 5, 6]
    mk.mk_pool_free(b.lib)


def test_errors_leave_the_pool_unchanged():
    b = Both(8, 4)
    b.lease_prefix(1, [1, 2, 3, 4, 5], 8)
    b.finish(1, [1, 2, 3, 4, 5])
    b.lease_prefix(2, [1, 2, 3, 4, 5, 6], 8)          # shares page 0
    before = (mk.mk_pool_free_pages(b.lib), mk.mk_pool_cached_pages(b.lib),
              mk.mk_pool_page_table(b.lib, [2], 2))
    with pytest.raises(mk.MkError) as e:               # page 0 holds [1, 2, 3, 4], not [9, ...]
        mk.mk_pool_finish(b.lib, 2, [9, 9, 9, 9, 5, 6])
    assert e.value.status == mk.MK_EINVAL
    with pytest.raises(mk.MkError) as e:               # two pages hold at most 8 tokens
        mk.mk_pool_finish(b.lib, 2, list(range(9)))
    assert e.value.status == mk.MK_EBOUNDS
    with pytest.raises(mk.MkError) as e:               # worst case below the prompt
        mk.mk_pool_lease_prefix(b.lib, 3, [1, 2, 3], 2)
    assert e.value.status == mk.MK_EINVAL
    with pytest.raises(mk.MkError) as e:
        mk.mk_pool_lease_prefix(b.lib, 2, [1], 4)      # already leased
    assert e.value.status == mk.MK_ESTATE
    after = (mk.mk_pool_free_pages(b.lib), mk.mk_pool_cached_pages(b.lib),
             mk.mk_pool_page_table(b.lib, [2], 2))
    assert before == after
    assert b.ref.finish(2, [9, 9, 9, 9, 5, 6]) == "disagree"
    assert b.ref.finish(2, list(range(9))) == "bounds"
    mk.mk_pool_free(b.lib)


def check_invariants(model):
    held = {p for p, h in model.holders.items() if h}
    assert held.isdisjoint(model.free) and held | set(model.free) == set(model.holders)
    frozen = {n["page"] for n in model.nodes.values()}
    writers = {}
    for s, pages in model.pages.items():
        for p in pages:
            if p not in frozen:
                writers.setdefault(p, []).append(s)
    assert all(len(w) == 1 for w in writers.values()), "a page with two writers"


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_mixes_agree_with_the_model(seed):
    rng = random.Random(seed)
    n_pages = rng.choice([24, 40, 64])
    order = list(range(n_pages))
    rng.shuffle(order)
    b = Both(n_pages, 6, order)
    stems = [[rng.randrange(1, 6) for _ in range(rng.randrange(3, 20))] for _ in range(4)]
    made = {}
    reused = 0
    for step in range(400):
        op = rng.random()
        free_ids = [s for s in range(12) if s not in b.live]
        if op < 0.45 and free_ids:
            s = rng.choice(free_ids)
            stem = rng.choice(stems)
            prompt = stem[:rng.randrange(1, len(stem) + 1)] + [rng.randrange(1, 6) for _ in range(rng.randrange(0, 6))]
            worst = len(prompt) + rng.randrange(0, 10)
            got = b.lease_prefix(s, prompt, worst)
            if got is not None:
                reused += got[1]
                made[s] = (prompt, worst)
                # the shared pages hold the prompt's own tokens there
                m = got[1]
                for j in range(m // PT):
                    node = next(n for n in b.ref.nodes.values() if n["page"] == b.pages(s)[j])
                    assert node["run"] == prompt[j * PT:(j + 1) * PT]
        elif op < 0.6 and b.live:
            s = rng.choice(sorted(b.live))
            prompt, worst = made[s]
            worst += rng.randrange(1, 12)
            if b.extend(s, worst):
                made[s] = (prompt, worst)
        elif op < 0.85 and b.live:
            s = rng.choice(sorted(b.live))
            prompt, worst = made[s]
            tokens = prompt + [rng.randrange(1, 6) for _ in range(worst - len(prompt))]
            b.finish(s, tokens[:rng.randrange(len(prompt), worst + 1)])
        elif b.live:
            b.release(rng.choice(sorted(b.live)))
        check_invariants(b.ref)
    assert reused > 0 and b.ref.cached() > 0
    mk.mk_pool_free(b.lib)
