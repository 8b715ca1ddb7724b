"""Pins of the oracle's block-bookkeeping twin.

* A property run of 10,000 random events (admit with optional prefix share, grow by one
  token, finish) with the books checked after EVERY event against refcounts recomputed from
  the live block tables, over enough pressure for more than 100 pool exhaustions and more than
  100 shared admits ("P3: native paged-KV continuous-batching sampler", section "Evidence",
  item 4, allocator never leaks).
* The LIFO rule, all-or-nothing growth, typed exhaustion, the double-free guard and the
  read-only rule for shared blocks (same page, "Design > paged.py"; "Optional paged KV cache
  (vLLM-style) — v1 design", section "Design").
* Planted mistakes from the P3 page's mutant list (free leaks, free double-appends, incref
  removed, double-free guard removed, prefix sharing of a partial block) that the run must
  catch.
"""
from collections import Counter

import numpy as np
import pytest

from oracle import allocator as A
from oracle.allocator import BlockAllocator, DoubleFree, InvalidBlock, PoolExhausted, SharedWrite


def property_run(n_events=10_000, num_blocks=48, bs=4, seed=0, share_partial=False,
                 strict=True):
    """Random admit / grow / finish events; returns counters. Raises AssertionError on a
    broken book. Every written token goes through slots(), which refuses shared blocks."""
    rng = np.random.default_rng(seed)
    a = BlockAllocator(num_blocks)
    live = {}            # seq id -> [tokens, table]
    next_id = 0
    stats = Counter()
    for _ in range(n_events):
        r = rng.random()
        if r < 0.45 or not live:
            L = int(rng.integers(1, 7 * bs))
            share = None
            if live and rng.random() < 0.5:
                leader = list(live)[int(rng.integers(len(live)))]
                lt, ltab = live[leader]
                k = min(lt, L) // bs if not share_partial else -(-min(lt, L) // bs)
                if k > 0:
                    share = ltab[:k]
            nsh = len(share) if share else 0
            need = -(-L // bs) - nsh
            try:
                own = a.allocate(max(need, 0))
            except PoolExhausted:
                stats["exhausted"] += 1
                own = None
            if own is not None:
                if share:
                    a.incref(share)
                    stats["shared_admits"] += 1
                table = (share or []) + own
                a.slots(table, nsh * bs, L - nsh * bs, bs) if L > nsh * bs else None
                live[next_id] = [L, table]
                next_id += 1
        elif r < 0.8:
            sid = list(live)[int(rng.integers(len(live)))]
            t, tab = live[sid]
            grew = True
            if t % bs == 0:
                try:
                    tab.extend(a.allocate(1))
                except PoolExhausted:
                    stats["exhausted"] += 1
                    grew = False
            if grew:
                a.slots(tab, t, 1, bs)
                live[sid][0] = t + 1
        else:
            sid = list(live)[int(rng.integers(len(live)))]
            a.free(live.pop(sid)[1])
        # books after EVERY event
        if strict:
            assert a.check_consistent()
            recount = Counter(i for _, tab in live.values() for i in tab)
            for i in range(num_blocks):
                assert a.refcount[i] == recount.get(i, 0)
    for sid in list(live):
        a.free(live.pop(sid)[1])
    assert a.num_free() == num_blocks and a.check_consistent()
    return stats


def test_property_run_10k_events_books_hold_after_every_event():
    stats = property_run()
    assert stats["exhausted"] > 100 and stats["shared_admits"] > 100


def test_fresh_pool_hands_out_ascending_ids_and_is_lifo():
    a = BlockAllocator(6)
    assert a.allocate(3) == [0, 1, 2]
    a.free([1])
    assert a.allocate(1) == [1]
    a.free([2, 0])           # applied in array order: 2 pushed, then 0 on top
    assert a.allocate(2) == [0, 2]
    assert a.check_consistent()


def test_exhaustion_is_typed_and_all_or_nothing():
    a = BlockAllocator(4)
    a.allocate(3)
    before = (list(a.free_stack), list(a.refcount))
    with pytest.raises(PoolExhausted):
        a.allocate(2)
    assert (a.free_stack, a.refcount) == before


def test_double_free_and_incref_of_free_block_are_refused_without_change():
    a = BlockAllocator(4)
    ids = a.allocate(2)
    a.free([ids[0]])
    before = (list(a.free_stack), list(a.refcount))
    with pytest.raises(DoubleFree):
        a.free([ids[1], ids[0]])
    with pytest.raises(DoubleFree):
        a.free([ids[1], ids[1]])
    with pytest.raises(InvalidBlock):
        a.incref([ids[1], ids[0]])
    with pytest.raises(InvalidBlock):
        a.free([7])
    assert (a.free_stack, a.refcount) == before


def test_shared_block_is_read_only_for_everyone_owner_included():
    a = BlockAllocator(8)
    owner = a.allocate(2)
    assert a.slots(owner, 0, 8, 4) == [owner[0] * 4 + i for i in range(4)] + \
        [owner[1] * 4 + i for i in range(4)]
    a.incref(owner[:1])
    with pytest.raises(SharedWrite):
        a.slots(owner, 3, 1, 4)
    assert a.slots(owner, 4, 2, 4) == [owner[1] * 4, owner[1] * 4 + 1]
    a.free(owner[:1])
    assert a.slots(owner, 3, 1, 4) == [owner[0] * 4 + 3]


def test_refcount_sharing_frees_only_at_zero():
    a = BlockAllocator(3)
    x = a.allocate(1)[0]
    a.incref([x, x])
    a.free([x])
    a.free([x])
    assert a.num_free() == 2 and a.refcount[x] == 1
    a.free([x])
    assert a.num_free() == 3 and a.check_consistent()


# ---- planted mistakes --------------------------------------------------------------------

def _caught(monkeypatch_fn=None, **kw):
    try:
        property_run(n_events=3000, **kw)
    except (AssertionError, A.AllocatorError):
        return True
    return False


def test_unmutated_control_passes():
    assert not _caught()


def test_mutant_free_leaks(monkeypatch):
    def free(self, ids):
        for i in ids:
            self.refcount[i] -= 1
    monkeypatch.setattr(BlockAllocator, "free", free)
    assert _caught()


def test_mutant_free_double_appends(monkeypatch):
    def free(self, ids):
        for i in ids:
            self.refcount[i] -= 1
            if self.refcount[i] == 0:
                self.free_stack.append(i)
                self.free_stack.append(i)
    monkeypatch.setattr(BlockAllocator, "free", free)
    assert _caught()


def test_mutant_incref_removed(monkeypatch):
    monkeypatch.setattr(BlockAllocator, "incref", lambda self, ids: None)
    assert _caught()


def test_mutant_double_free_guard_removed(monkeypatch):
    def free(self, ids):
        for i in ids:
            self.refcount[i] -= 1
            if self.refcount[i] <= 0:
                self.free_stack.append(i)
    monkeypatch.setattr(BlockAllocator, "free", free)
    a = BlockAllocator(2)
    x = a.allocate(1)
    a.free(x)
    a.free(x)                     # silently accepted by the mutant
    assert not a.check_consistent()


def test_mutant_prefix_sharing_of_a_partial_block():
    assert _caught(share_partial=True)
