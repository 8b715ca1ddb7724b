"""Pins of the scheduler oracle (oracle/scheduler.py) to the rules the pages state.

Each scenario below is derived by hand from the rules (decodes first, n_new = min(remaining,
chunk, budget), FIFO admission when the whole token list fits, preemption of the youngest
unscheduled running sequence by recompute, adoption of leading FULL blocks with the last prompt
token always recomputed, trim, copy-on-write on a divergent write). A randomized event run
checks the books after every step, and a CPU engine loop checks that whatever the schedule,
every computed token's attention equals a dense computation over its own keys: a wrong slot,
table, context length or block copy anywhere would change some token.
"""
import numpy as np
import pytest

from oracle.scheduler import FINISHED, RUNNING, SchedConfig, Scheduler, SchedulerError
from oracle.paged import attend_rows


def _sched(nb, bs=4, chunk=5, budget=8, max_seqs=4, max_blocks=8, share=False):
    return Scheduler(nb, SchedConfig(bs, chunk, budget, max_seqs, max_blocks, share))


def test_decodes_first_then_chunks_within_budget():
    s = _sched(16, chunk=5, budget=6)
    s.add(0, 2)
    s.add(1, 9)
    p = s.step()                       # both admitted; no decode yet; chunks oldest first
    assert (p.seq_ids, p.n_new) == ([0, 1], [2, 4])
    s.complete()
    p = s.step()                       # 0 now decodes (remaining 1) and goes first
    assert (p.seq_ids, p.n_new, p.ctx_lens) == ([0, 1], [1, 5], [3, 9])
    assert p.cu_seqlens == [0, 1, 6]
    s.complete()
    p = s.step()
    assert (p.seq_ids, p.n_new, p.ctx_lens) == ([0, 1], [1, 1], [4, 10])


def test_fifo_admission_needs_the_whole_token_list():
    s = _sched(4, bs=4, chunk=16, budget=16, max_seqs=8)
    s.add(0, 9)                        # 3 blocks
    s.add(1, 5)                        # 2 blocks: does not fit next to 0 -> waits
    s.add(2, 1)                        # would fit, but FIFO keeps it behind 1
    p = s.step()
    assert p.seq_ids == [0] and s.waiting == [1, 2]
    s.complete(finished=[0])
    p = s.step()
    assert p.seq_ids == [1, 2] and p.n_new == [5, 1] or p.seq_ids == [2, 1]
    assert s.seqs[1].state == RUNNING and s.seqs[2].state == RUNNING


def test_preemption_takes_the_youngest_and_recomputes_it():
    s = _sched(5, bs=4, chunk=8, budget=16, max_seqs=4)
    s.add(0, 8)                        # 2 blocks
    s.add(1, 8)                        # 2 blocks
    p = s.step()
    assert p.seq_ids == [0, 1]
    s.complete()                       # both sampled: 9 tokens each, need a third block
    p = s.step()
    # 0 decodes first: 1 free block -> takes it; 1 then needs one more -> no free block, the
    # youngest unscheduled sequence holding blocks is 1 itself -> preempted, waits this step
    assert p.seq_ids == [0] and p.preempted == [1]
    assert s.seqs[1].num_computed == 0 and s.seqs[1].blocks == [] and s.seqs[1].n_tokens == 9
    assert s.preemptions == 1
    s.complete(finished=[0])
    p = s.step()                       # 1 recomputes its 9 tokens as a chunk
    assert p.seq_ids == [1] and p.n_new == [8] and p.ctx_lens == [8]


def test_preemption_victim_is_youngest_other_sequence():
    s = _sched(4, bs=4, chunk=8, budget=16, max_seqs=4)
    for i in range(3):
        s.add(i, 4)                    # one block each; 1 block stays free
    p = s.step()
    assert p.seq_ids == [0, 1, 2]
    s.complete()                       # each has 5 tokens now: position 4 needs a 2nd block
    p = s.step()
    # 0 takes the free block; 1 finds none: the youngest unscheduled holder is 2 (not 1)
    assert p.seq_ids == [0, 1] and p.preempted == [2]
    assert s.seqs[2].blocks == [] and s.seqs[2].num_computed == 0 and s.seqs[2].n_tokens == 5
    s.complete(finished=[0, 1])
    p = s.step()                       # 2 recomputes from position 0
    assert p.seq_ids == [2] and p.n_new == [5] and p.ctx_lens == [5]


def test_prefix_adoption_defers_adopts_full_blocks_and_recomputes_last_token():
    bs = 4
    s = _sched(32, bs=bs, chunk=4, budget=4, max_seqs=8, share=True)
    s.add(0, 10, group=7)              # leader: 10 prompt tokens -> 2 full blocks to share
    s.add(1, 10, group=7)
    p = s.step()                       # leader computes 4; follower must wait (FIFO stops)
    assert p.seq_ids == [0] and s.waiting == [1]
    s.complete()
    p = s.step()
    assert s.waiting == [1]            # leader has 4 < 8 computed: still deferred
    s.complete()
    p = s.step()                       # leader has 8 computed -> follower adopts 2 blocks
    assert s.seqs[1].state == RUNNING
    lead = s.seqs[0].blocks
    assert s.seqs[1].blocks[:2] == lead[:2]
    assert s.alloc.refcount[lead[0]] == 2 and s.alloc.refcount[lead[1]] == 2
    assert s.shared_tokens == 8
    # admitted and scheduled in the same step: its chunk starts at position 8 (positions 8, 9 =
    # the last prompt tokens are recomputed) in a fresh block of its own
    i = p.seq_ids.index(1)
    assert p.ctx_lens[i] - p.n_new[i] == 8 and p.n_new[i] == 2
    fresh = s.seqs[1].blocks[2]
    assert fresh not in lead and s.alloc.refcount[fresh] == 1
    r0 = sum(p.n_new[:i])
    assert [sl // bs for sl in p.slots[r0:r0 + 2]] == [fresh, fresh]
    s.complete()
    s.check()


def test_prefix_adoption_never_shares_the_block_holding_the_last_prompt_token():
    bs = 4
    s = _sched(32, bs=bs, chunk=16, budget=16, max_seqs=8, share=True)
    s.add(0, 8, group=1)               # 8 tokens = exactly 2 blocks; last token in block 1
    s.add(1, 8, group=1)
    s.step()
    s.complete()
    s.step()                           # follower admitted: adopts (8 - 1) // 4 = 1 block only
    assert s.seqs[1].blocks[:1] == s.seqs[0].blocks[:1]
    assert s.seqs[1].num_computed == 4


def test_trim_frees_tail_blocks_and_regrowth_reallocates():
    s = _sched(16, bs=4, chunk=16, budget=16)
    s.add(0, 13)
    s.step()
    s.complete()                       # 13 computed, 14 tokens, 4 blocks
    assert len(s.seqs[0].blocks) == 4
    free_before = s.alloc.num_free()
    s.trim(0, 6)                       # 5 computed (token 5 is fed again): keep 2 blocks
    assert s.seqs[0].n_tokens == 6 and s.seqs[0].num_computed == 5
    assert len(s.seqs[0].blocks) == 2 and s.alloc.num_free() == free_before + 2
    s.check()
    s.trim(0, 5)                       # 4 computed: a block boundary, the tail block goes
    assert len(s.seqs[0].blocks) == 1 and s.seqs[0].num_computed == 4
    p = s.step()                       # position 4 again, in a newly allocated block
    assert p.seq_ids == [0] and p.n_new == [1] and p.ctx_lens == [5]
    assert len(p.block_tables[0]) == 2
    s.complete()                       # samples: 6 tokens
    p = s.step()
    assert p.ctx_lens == [6]
    s.complete()
    s.check()
    with pytest.raises(SchedulerError):
        s.trim(0, 999)


def test_fork_shares_blocks_and_copies_on_divergent_write():
    s = _sched(16, bs=4, chunk=16, budget=16)
    s.add(0, 6)
    s.step()
    s.complete()                       # 6 computed, 7 tokens, 2 blocks (second half full)
    s.fork(0, 1)
    b0 = list(s.seqs[0].blocks)
    assert s.seqs[1].blocks == b0 and all(s.alloc.refcount[b] == 2 for b in b0)
    p = s.step()                       # both decode position 6, in the shared block b0[1]
    assert p.seq_ids == [0, 1]
    # 0 writes first: copies b0[1] to a fresh block; then 1 is the only holder of b0[1]
    assert len(p.copies) == 1 and p.copies[0][0] == b0[1]
    assert s.seqs[0].blocks[1] == p.copies[0][1] and s.seqs[1].blocks[1] == b0[1]
    assert s.alloc.refcount[b0[1]] == 1 and s.alloc.refcount[b0[0]] == 2
    for sl, sid in zip(p.slots, p.seq_ids):
        assert s.alloc.refcount[sl // 4] == 1
    s.complete()
    s.check()


def _random_run(seed, steps=400, share=True):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 4, 5]))
    cfg = SchedConfig(bs, int(rng.integers(1, 12)), int(rng.integers(1, 24)),
                      int(rng.integers(1, 8)), int(rng.integers(2, 12)), share)
    s = Scheduler(int(rng.integers(4, 40)), cfg)
    nxt = 0
    stats = {"preempt": 0, "shared": 0, "copies": 0, "steps": 0}
    for _ in range(steps):
        ev = rng.random()
        if ev < 0.3:
            plen = int(rng.integers(1, cfg.max_blocks_per_seq * bs + 1))
            grp = int(rng.integers(0, 3)) if rng.random() < 0.5 else -1
            s.add(nxt, plen, grp)
            nxt += 1
        elif ev < 0.35 and s.running:
            rid = int(rng.choice(s.running))
            if s.seqs[rid].n_tokens > 1:
                s.trim(rid, int(rng.integers(1, s.seqs[rid].n_tokens + 1)))
        elif ev < 0.4 and s.running and len(s.running) < cfg.max_num_seqs:
            s.fork(int(rng.choice(s.running)), nxt)
            nxt += 1
        p = s.step()
        stats["steps"] += 1
        # plan invariants
        assert sum(p.n_new) <= cfg.token_budget
        assert len(set(p.seq_ids)) == len(p.seq_ids)
        kinds = [n == 1 and s.seqs[i].n_tokens - (c - n) == 1
                 for i, n, c in zip(p.seq_ids, p.n_new, p.ctx_lens)]
        assert kinds == sorted(kinds, reverse=True)         # decodes before chunks
        assert not set(p.preempted) & set(p.seq_ids)
        for i, n, c, t in zip(p.seq_ids, p.n_new, p.ctx_lens, p.block_tables):
            assert 1 <= n <= cfg.chunk_size and c == s.seqs[i].num_computed + n
            assert len(t) == -(-c // bs)
        for sl in p.slots:
            assert s.alloc.refcount[sl // bs] == 1            # never into a shared block
        stats["preempt"] += len(p.preempted)
        stats["copies"] += len(p.copies)
        fin = [i for i in p.seq_ids if rng.random() < 0.15]
        s.complete(fin)
        s.check()
    stats["shared"] = s.shared_tokens
    return stats


@pytest.mark.parametrize("seed", range(12))
def test_random_event_runs_keep_the_books(seed):
    _random_run(seed)


def test_random_runs_exercise_every_path():
    tot = {"preempt": 0, "shared": 0, "copies": 0}
    for seed in range(12):
        st = _random_run(seed)
        for k in tot:
            tot[k] += st[k]
    assert tot["preempt"] > 20 and tot["shared"] > 20 and tot["copies"] > 5


# ---- engine loop on the CPU: any schedule computes the same attention per token ----------

def _token_q(sid, pos, hq, d):
    return np.random.default_rng([sid, pos, 2]).standard_normal((hq, d))


class _Tokens:
    """Identity of every token: prompts of one group are the same tokens; a fork shares its
    parent's tokens (as they are at the fork); a trim discards the tokens past the cut, and
    tokens generated after it are new tokens."""

    def __init__(self):
        self.known = {}                                   # sid -> token ids by position
        self.epoch = {}

    def add(self, sid, plen, grp):
        self.known[sid] = [(0, grp, plen, p) for p in range(plen)] if grp >= 0 else []
        self.epoch[sid] = 0

    def key(self, sid, pos):
        k = self.known[sid]
        while len(k) <= pos:
            k.append((1, sid, self.epoch[sid], len(k)))
        return k[pos]

    def fork(self, src, new, n):
        self.known[new] = [self.key(src, p) for p in range(n)]
        self.epoch[new] = 0

    def trim(self, sid, n):
        self.known[sid] = [self.key(sid, p) for p in range(n)]
        self.epoch[sid] += 1


def _token_kv(key, hkv, d):
    r = np.random.default_rng([*key, 1])
    return r.standard_normal((hkv, d)), r.standard_normal((hkv, d))


def _dense(tok, sid, pos, hq=4, hkv=2, d=8):
    kv = [_token_kv(tok.key(sid, j), hkv, d) for j in range(pos + 1)]
    kc = np.stack([x[0] for x in kv], axis=1)
    vc = np.stack([x[1] for x in kv], axis=1)
    return attend_rows(_token_q(sid, pos, hq, d)[None], kc, vc, np.array([pos]), 0.3)[0]


def _engine_run(cfg, num_blocks, requests, steps, seed, hq=4, hkv=2, d=8):
    """Drive the scheduler with oracle pools and random forks, trims and finishes; every row
    computed is compared with the dense attention over its sequence's current tokens."""
    rng = np.random.default_rng(seed)
    s = Scheduler(num_blocks, cfg)
    bs = cfg.block_size
    K = np.full((num_blocks, bs, hkv, d), np.nan)
    V = np.full((num_blocks, bs, hkv, d), np.nan)
    tok = _Tokens()
    for sid, plen, grp in requests:
        s.add(sid, plen, grp)
        tok.add(sid, plen, grp)
    nxt, rows = 1000, 0
    st = {"preempt": 0, "copies": 0}
    for _ in range(steps):
        ev = rng.random()
        if ev < 0.08 and s.running and len(s.running) < cfg.max_num_seqs:
            src = int(rng.choice(s.running))
            s.fork(src, nxt)
            tok.fork(src, nxt, s.seqs[src].n_tokens)
            nxt += 1
        elif ev < 0.14 and s.running:
            sid = int(rng.choice(s.running))
            if s.seqs[sid].n_tokens > 2:
                n = int(rng.integers(2, s.seqs[sid].n_tokens + 1))
                s.trim(sid, n)
                tok.trim(sid, n)
        p = s.step()
        st["preempt"] += len(p.preempted)
        st["copies"] += len(p.copies)
        for src, dst in p.copies:
            K[dst] = K[src]
            V[dst] = V[src]
        r = 0
        for sid, n, c, table in zip(p.seq_ids, p.n_new, p.ctx_lens, p.block_tables):
            for pos in range(c - n, c):
                kk, vv = _token_kv(tok.key(sid, pos), hkv, d)
                slot = p.slots[r]
                K[slot // bs, slot % bs] = kk
                V[slot // bs, slot % bs] = vv
                r += 1
            kc = np.concatenate([K[b] for b in table], axis=0)[:c].transpose(1, 0, 2)
            vc = np.concatenate([V[b] for b in table], axis=0)[:c].transpose(1, 0, 2)
            qs = np.stack([_token_q(sid, pos, hq, d) for pos in range(c - n, c)])
            o = attend_rows(qs, kc, vc, np.arange(c - n, c), 0.3)
            for i, pos in enumerate(range(c - n, c)):
                assert np.abs(o[i] - _dense(tok, sid, pos)).max() < 1e-12, (sid, pos)
                rows += 1
        fin = [i for i in p.seq_ids if rng.random() < 0.05]
        s.complete(fin)
        s.check()
    st["shared"] = s.shared_tokens
    st["rows"] = rows
    return st


@pytest.mark.parametrize("variant", [
    dict(bs=4, chunk=3, budget=8, nb=40, share=False),
    dict(bs=4, chunk=16, budget=16, nb=14, share=True),     # tight pool: preemptions
    dict(bs=1, chunk=2, budget=5, nb=40, share=True),
    dict(bs=5, chunk=64, budget=64, nb=11, share=True),
])
def test_engine_loop_attention_is_schedule_independent(variant):
    cfg = SchedConfig(variant["bs"], variant["chunk"], variant["budget"], 6,
                      48 // variant["bs"], variant["share"])
    reqs = [(0, 11, 3), (1, 11, 3), (2, 7, -1), (3, 11, 3), (4, 2, -1), (5, 9, -1)]
    tot = {"preempt": 0, "copies": 0, "shared": 0, "rows": 0}
    for seed in range(3):
        st = _engine_run(cfg, variant["nb"], reqs, 50, seed)
        for k in tot:
            tot[k] += st[k]
    assert tot["rows"] > 100
    if variant["share"]:
        assert tot["shared"] > 0


def test_engine_loop_covers_preemption_sharing_and_copies():
    tot = {"preempt": 0, "copies": 0, "shared": 0, "rows": 0}
    cfg = SchedConfig(4, 16, 16, 6, 12, True)
    reqs = [(0, 11, 3), (1, 11, 3), (2, 7, -1), (3, 11, 3), (4, 2, -1), (5, 9, -1)]
    for seed in range(6):
        st = _engine_run(cfg, 14, reqs, 50, 100 + seed)
        for k in tot:
            tot[k] += st[k]
    assert tot["preempt"] > 0 and tot["copies"] > 0 and tot["shared"] > 0


# ---- planted mistakes: each must make at least one pin above fail -------------------------

def _mut_oldest_victim(self, scheduled):
    best = None
    for rid in self.running:
        r = self.seqs[rid]
        if rid in scheduled or not r.blocks:
            continue
        if best is None or r.order < best.order:
            best = r
    return best


def _mut_preempt_keeps_blocks(self, s):
    s.blocks = []                       # forgets to hand the blocks back


def _mut_share_partial(self):
    bs = self.cfg.block_size
    while self.waiting and len(self.running) < self.cfg.max_num_seqs:
        s = self.seqs[self.waiting[0]]
        adopted = []
        if self.cfg.prefix_sharing and s.group >= 0:
            leader = self._leader(s)
            target = -(-s.prompt_len // bs)        # also the block of the last prompt token
            if leader is not None:
                if leader.num_computed < min(target * bs, s.prompt_len):
                    return
                adopted = leader.blocks[:target]
        if -(-s.n_tokens // bs) - len(adopted) > self.alloc.num_free():
            return
        self.waiting.pop(0)
        self._admit(s, adopted)
        s.num_computed = min(s.num_computed, s.prompt_len - 1)


_ORIG_RESERVE = Scheduler._reserve


def _mut_cow_without_copy(self, s, n_new, scheduled, copies, preempted):
    ok = _ORIG_RESERVE(self, s, n_new, scheduled, copies, preempted)
    copies.clear()                      # the fresh block is used, its rows are never copied
    return ok


MUTANTS = {
    "preempts the oldest": ("_preempt_victim", _mut_oldest_victim),
    "preemption forgets to free": ("_free_blocks", _mut_preempt_keeps_blocks),
    "shares the last prompt block": ("_admission", _mut_share_partial),
    "copy-on-write without the copy": ("_reserve", _mut_cow_without_copy),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_scheduler_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(Scheduler, attr, fn)
    pins = [test_preemption_victim_is_youngest_other_sequence,
            test_prefix_adoption_never_shares_the_block_holding_the_last_prompt_token,
            test_fork_shares_blocks_and_copies_on_divergent_write,
            lambda: _random_run(3), lambda: _random_run(5),
            lambda: test_engine_loop_covers_preemption_sharing_and_copies()]
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, SchedulerError):
            failed += 1
    assert failed > 0, f"mutant '{name}' survived every pin"
