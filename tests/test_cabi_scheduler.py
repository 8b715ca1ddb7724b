"""The C++ host step builder (pkv_sched_* through the C ABI) against the scheduler oracle.

On identical seeded event traces (requests, steps, completions with random finishes, trims,
forks, and events that must be refused) both sides must build the same steps bit for bit: the
same scheduled sequences, row counts, context lengths, cu_seqlens, whole block tables, slots,
copy-on-write pairs and preemptions; the same sampled sequences; the same refusals; and after
every event the same per-sequence state, held blocks, counters, allocator free stack and
refcounts. Host only: no GPU is involved.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from oracle.scheduler import SchedConfig, Scheduler, SchedulerError


def _pair(nb, bs, chunk, budget, max_seqs, max_blocks, share):
    o = Scheduler(nb, SchedConfig(bs, chunk, budget, max_seqs, max_blocks, share))
    c = pkv.Scheduler(nb, bs, chunk, budget, max_seqs, max_blocks, share)
    return o, c


def _both(fo, fc):
    """Run one event on both sides; both succeed or both refuse."""
    eo = ec = None
    ro = rc = None
    try:
        ro = fo()
    except SchedulerError as e:
        eo = e
    try:
        rc = fc()
    except pkv.PkvError as e:
        ec = e
    assert (eo is None) == (ec is None), (eo, ec)
    return ro, rc, eo is not None


def _same_books(o, c):
    pre, shared, waiting, running = c.stats_tuple()
    assert (pre, shared, waiting, running) == (o.preemptions, o.shared_tokens, len(o.waiting),
                                               len(o.running))
    for sid, q in o.seqs.items():
        st, nt, nc, nb = c.seq_info(sid)
        assert (st, nt, nc, nb) == (q.state, q.n_tokens, q.num_computed, len(q.blocks)), sid
        assert c.seq_blocks(sid) == q.blocks
    stack, rc = c.allocator.snapshot()
    assert stack == o.alloc.free_stack and rc == o.alloc.refcount
    assert c.check()


def _same_plan(po, pc):
    assert pc.seq_ids == po.seq_ids
    assert pc.n_new == po.n_new
    assert pc.ctx_lens == po.ctx_lens
    assert pc.cu_seqlens == po.cu_seqlens
    assert pc.block_tables == po.block_tables
    assert pc.slots == po.slots
    assert pc.copies == po.copies
    assert pc.preempted == po.preempted


def _twin_run(seed, events=300):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 4, 5, 16]))
    max_blocks = int(rng.integers(2, 12))
    o, c = _pair(int(rng.integers(4, 48)), bs, int(rng.integers(1, 12)), int(rng.integers(1, 24)),
                 int(rng.integers(1, 8)), max_blocks, bool(rng.random() < 0.7))
    nxt = 0
    seen = {"steps": 0, "preempt": 0, "copies": 0, "refused": 0, "shared": 0}
    for _ in range(events):
        ev = rng.random()
        if ev < 0.3:
            plen = int(rng.integers(1, max_blocks * bs + 1))
            grp = int(rng.integers(0, 3)) if rng.random() < 0.6 else -1
            sid = nxt if rng.random() < 0.95 else max(nxt - 1, 0)   # sometimes a used id
            _, _, refused = _both(lambda: o.add(sid, plen, grp), lambda: c.add(sid, plen, grp))
            nxt += 0 if refused else 1
            seen["refused"] += refused
        elif ev < 0.36:
            pool = list(o.seqs) or [0]
            sid = int(rng.choice(pool))
            q = o.seqs.get(sid)
            n = int(rng.integers(0, (q.n_tokens if q else 3) + 2))
            _, _, refused = _both(lambda: o.trim(sid, n), lambda: c.trim(sid, n))
            seen["refused"] += refused
        elif ev < 0.42:
            pool = list(o.seqs) or [0]
            src = int(rng.choice(pool))
            _, _, refused = _both(lambda: o.fork(src, nxt), lambda: c.fork(src, nxt))
            nxt += 0 if refused else 1
            seen["refused"] += refused
        _same_books(o, c)
        po, pc, refused = _both(o.step, c.step)
        assert not refused
        _same_plan(po, pc)
        seen["steps"] += 1
        seen["preempt"] += len(po.preempted)
        seen["copies"] += len(po.copies)
        # events are refused while the step awaits completion
        _, _, refused = _both(o.step, c.step)
        assert refused
        fin = [i for i in po.seq_ids if rng.random() < 0.15]
        so, sc, refused = _both(lambda: o.complete(fin), lambda: c.complete(fin))
        assert not refused and so == sc
        _same_books(o, c)
    seen["shared"] = o.shared_tokens
    return seen


@pytest.mark.parametrize("seed", range(16))
def test_cpp_scheduler_equals_oracle_on_random_traces(seed):
    _twin_run(seed)


def test_twin_traces_exercise_every_path():
    tot = {"preempt": 0, "copies": 0, "refused": 0, "shared": 0}
    for seed in range(16):
        st = _twin_run(seed, events=200)
        for k in tot:
            tot[k] += st[k]
    assert all(v > 5 for v in tot.values()), tot


def test_scheduler_plan_feeds_the_slot_rule():
    # every slot of a plan is writable (refcount 1) and is the flat (block, offset) index of
    # its sequence's position through the plan's table
    o, c = _pair(24, 4, 6, 10, 4, 8, True)
    for sid, (plen, grp) in enumerate([(9, 0), (9, 0), (5, -1), (13, 1)]):
        c.add(sid, plen, grp)
    for _ in range(12):
        p = c.step()
        k = 0
        for sid, n, ctx, tab in zip(p.seq_ids, p.n_new, p.ctx_lens, p.block_tables):
            for pos in range(ctx - n, ctx):
                blk = tab[pos // 4]
                assert p.slots[k] == blk * 4 + pos % 4
                assert c.allocator.refcount(blk) == 1
                k += 1
        assert k == p.cu_seqlens[-1]
        c.complete()
        assert c.check()


def test_scheduler_validation():
    with pytest.raises(pkv.InvalidArgument):
        pkv.Scheduler(8, 0, 4, 4, 2, 4)
    c = pkv.Scheduler(8, 4, 4, 4, 2, 4)
    with pytest.raises(pkv.InvalidArgument):
        c.add(0, 17)                       # past max_blocks_per_seq * block_size
    c.add(0, 3)
    with pytest.raises(pkv.InvalidArgument):
        c.add(0, 3)                        # id exists
    with pytest.raises(pkv.InvalidArgument):
        c.complete()                       # no step pending
    c.step()
    for fn in (lambda: c.trim(0, 1), lambda: c.fork(0, 5), lambda: c.step()):
        with pytest.raises(pkv.InvalidArgument):
            fn()                           # a step awaits completion
    assert c.complete() == [0]
