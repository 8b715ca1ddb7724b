"""Oracle: the host step builder (scheduler) around the paged path — test infrastructure only.

Follows "P3: native paged-KV continuous-batching sampler", section "Design > engine.py":
  * Every sequence is a token count plus num_computed; a step gives each scheduled sequence
    n_new = min(remaining, chunk_size, budget) new rows. Prefill, chunked prefill, decode and
    recompute after preemption are one path. Decodes are scheduled first; prefill chunks and
    decode rows share one flat ragged step.
  * Admission is FIFO and happens only if the whole current token list fits in the free blocks.
    When a scheduled sequence cannot get its blocks, the youngest running sequence not yet
    scheduled in this step is preempted by recompute: its blocks are freed and num_computed
    drops to 0 (its tokens are kept).
  * Prefix sharing (opt-in): a waiting sequence adopts the leading FULL blocks of a running
    sequence of its group, waits while that leader is still computing them, and always
    recomputes its own last prompt token.
and "Optional paged KV cache (vLLM-style) — v1 design", sections "Design" and "Follow-ups":
  * trim(n) rewinds a sequence to n tokens and frees the blocks nothing occupies any more.
  * Block-level copy-on-write: a fork shares every block (refcounts); the first write into a
    shared block copies it to a fresh block for the writer (fork on divergent write).

Readings where the pages leave a step open (each listed in the design notes):
  S1 Running sequences are kept in admission order (a fork is admitted when it is made); a
     preempted sequence stays running with num_computed 0 and no blocks.
  S2 Each step: admit waiting sequences (FIFO, stop at the first that does not fit or must
     wait, at most max_num_seqs running; "fits" = its whole token list fits in the free blocks
     not already promised to sequences admitted earlier in the same step; nothing is reserved
     for the residents' growth); then decodes (remaining == 1) oldest first, one row each,
     while budget lasts; then the others oldest first with n_new = min(remaining, chunk_size,
     budget).
  S3 "Youngest" = latest admitted. The victim is the youngest running sequence that holds at
     least one block and is not scheduled in this step; it may be the sequence asking. If no
     such sequence exists, the asking sequence waits for a later step; so does a sequence
     preempted while the step is being built.
  S4 Adoption: the leader is the oldest running sequence of the same group and prompt length;
     the follower takes its first (prompt_len - 1) // block_size blocks (full blocks that do
     not hold the last prompt token) once the leader has computed them, and starts with
     num_computed = adopted * block_size.
  S5 Blocks for a scheduled chunk: one fresh block to copy a shared block the chunk writes
     into (copy-on-write of the block holding position num_computed), then the missing tail
     blocks; all in one all-or-nothing allocation, popped in that order.
  S6 After the forward pass (complete): num_computed += n_new; a sequence whose num_computed
     reaches its token count samples: finished ones free their blocks, the others grow by
     one token (a sequence at max_blocks_per_seq * block_size tokens finishes).
  S7 trim(n): token count n, num_computed = min(num_computed, n - 1) (the last kept token is
     fed again, as after adoption, so that the sequence samples its next token), and the
     blocks past ceil(num_computed / block_size) are freed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

from .allocator import BlockAllocator, PoolExhausted, slot_of

WAITING, RUNNING, FINISHED = 0, 1, 2


class SchedulerError(Exception):
    pass


@dataclass
class SchedConfig:
    block_size: int
    chunk_size: int
    token_budget: int
    max_num_seqs: int
    max_blocks_per_seq: int
    prefix_sharing: bool = False


@dataclass
class Seq:
    sid: int
    prompt_len: int
    group: int
    n_tokens: int
    num_computed: int = 0
    blocks: List[int] = field(default_factory=list)
    state: int = WAITING
    order: int = -1          # admission counter; larger = younger


@dataclass
class StepPlan:
    seq_ids: List[int]
    n_new: List[int]
    ctx_lens: List[int]
    cu_seqlens: List[int]
    block_tables: List[List[int]]     # per scheduled sequence, its whole table after the step
    slots: List[int]                  # one per new row, in step order
    copies: List[Tuple[int, int]]     # (src block, dst block) to copy before the append
    preempted: List[int]              # sequences preempted while building this step


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class Scheduler:
    def __init__(self, num_blocks: int, cfg: SchedConfig):
        if min(cfg.block_size, cfg.chunk_size, cfg.token_budget, cfg.max_num_seqs,
               cfg.max_blocks_per_seq) < 1:
            raise SchedulerError("scheduler sizes must be >= 1")
        self.cfg = cfg
        self.alloc = BlockAllocator(num_blocks)
        self.seqs: Dict[int, Seq] = {}
        self.waiting: List[int] = []          # FIFO of sequence ids
        self.running: List[int] = []          # admission order (oldest first)
        self.counter = 0
        self.preemptions = 0
        self.shared_tokens = 0
        self.last_plan: Optional[StepPlan] = None

    # ---- requests ----------------------------------------------------------------------
    def add(self, sid: int, prompt_len: int, group: int = -1) -> None:
        if sid in self.seqs:
            raise SchedulerError(f"sequence {sid} exists")
        if not 1 <= prompt_len <= self.cfg.max_blocks_per_seq * self.cfg.block_size:
            raise SchedulerError("prompt length outside [1, max_blocks_per_seq * block_size]")
        self.seqs[sid] = Seq(sid, prompt_len, group, prompt_len)
        self.waiting.append(sid)

    def _admit(self, s: Seq, adopted: List[int]) -> None:
        if adopted:
            self.alloc.incref(adopted)
            self.shared_tokens += len(adopted) * self.cfg.block_size
        s.blocks = list(adopted)
        s.num_computed = len(adopted) * self.cfg.block_size
        s.state = RUNNING
        s.order = self.counter
        self.counter += 1
        self.running.append(s.sid)

    def _leader(self, s: Seq) -> Optional[Seq]:
        for rid in self.running:
            r = self.seqs[rid]
            if r.group == s.group and r.prompt_len == s.prompt_len:
                return r
        return None

    def _admission(self) -> None:
        bs = self.cfg.block_size
        room = self.alloc.num_free()        # free blocks not yet promised in this admission
        while self.waiting and len(self.running) < self.cfg.max_num_seqs:
            s = self.seqs[self.waiting[0]]
            adopted: List[int] = []
            if self.cfg.prefix_sharing and s.group >= 0:
                leader = self._leader(s)
                target = (s.prompt_len - 1) // bs
                if leader is not None and target > 0:
                    if leader.num_computed < target * bs:
                        return                      # defer: the leader is still computing them
                    adopted = leader.blocks[:target]
            need = _ceil_div(s.n_tokens, bs) - len(adopted)
            if need > room:
                return
            room -= need
            self.waiting.pop(0)
            self._admit(s, adopted)

    def _free_blocks(self, s: Seq) -> None:
        if s.blocks:
            self.alloc.free(s.blocks)
        s.blocks = []

    def _preempt_victim(self, scheduled: set) -> Optional[Seq]:
        best = None
        for rid in self.running:
            r = self.seqs[rid]
            if rid in scheduled or not r.blocks:
                continue
            if best is None or r.order > best.order:
                best = r
        return best

    def _blocks_for(self, s: Seq, n_new: int) -> Tuple[int, bool]:
        """(blocks to allocate, whether the first one is a copy-on-write target)."""
        bs = self.cfg.block_size
        j = s.num_computed // bs
        cow = j < len(s.blocks) and self.alloc.refcount[s.blocks[j]] > 1
        grow = max(0, _ceil_div(s.num_computed + n_new, bs) - len(s.blocks))
        return grow + (1 if cow else 0), cow

    def _reserve(self, s: Seq, n_new: int, scheduled: set, copies: list,
                 preempted: list) -> bool:
        """Get the blocks for s's chunk, preempting as needed; False if s does not run now."""
        while True:
            need, cow = self._blocks_for(s, n_new)
            try:
                ids = self.alloc.allocate(need)
            except PoolExhausted:
                victim = self._preempt_victim(scheduled)
                if victim is None:
                    return False
                self._free_blocks(victim)
                victim.num_computed = 0
                self.preemptions += 1
                preempted.append(victim.sid)
                if victim is s:
                    return False
                continue
            if cow:
                j = s.num_computed // self.cfg.block_size
                src = s.blocks[j]
                copies.append((src, ids[0]))
                self.alloc.free([src])
                s.blocks[j] = ids[0]
                ids = ids[1:]
            s.blocks.extend(ids)
            return True

    # ---- one step ----------------------------------------------------------------------
    def step(self) -> StepPlan:
        if self.last_plan is not None:
            raise SchedulerError("step while the previous step awaits completion")
        cfg = self.cfg
        self._admission()
        budget = cfg.token_budget
        order: List[Tuple[int, int]] = []
        scheduled: set = set()
        copies: List[Tuple[int, int]] = []
        preempted: List[int] = []
        # decodes first, oldest first; then chunks, oldest first. A sequence preempted while
        # this step is built waits for a later step.
        for decode_pass in (True, False):
            for rid in list(self.running):
                s = self.seqs[rid]
                if budget == 0:
                    break
                rem = s.n_tokens - s.num_computed
                if rem <= 0 or rid in scheduled or rid in preempted or (rem == 1) != decode_pass:
                    continue
                n_new = min(rem, cfg.chunk_size, budget)
                if self._reserve(s, n_new, scheduled, copies, preempted):
                    scheduled.add(rid)
                    order.append((rid, n_new))
                    budget -= n_new
        plan = StepPlan([], [], [], [0], [], [], copies, preempted)
        for rid, n_new in order:
            s = self.seqs[rid]
            plan.seq_ids.append(rid)
            plan.n_new.append(n_new)
            plan.ctx_lens.append(s.num_computed + n_new)
            plan.cu_seqlens.append(plan.cu_seqlens[-1] + n_new)
            plan.block_tables.append(list(s.blocks))
            plan.slots.extend(slot_of(s.blocks[p // cfg.block_size], p, cfg.block_size)
                              for p in range(s.num_computed, s.num_computed + n_new))
        self.last_plan = plan
        return plan

    def complete(self, finished: Sequence[int] = ()) -> List[int]:
        """Apply the last plan after its forward pass; returns the sequences that sampled."""
        plan = self.last_plan
        if plan is None:
            raise SchedulerError("complete without a step")
        self.last_plan = None
        fin = set(int(x) for x in finished)
        cap = self.cfg.max_blocks_per_seq * self.cfg.block_size
        sampled = []
        for rid, n_new in zip(plan.seq_ids, plan.n_new):
            s = self.seqs[rid]
            s.num_computed += n_new
            if s.num_computed == s.n_tokens:
                sampled.append(rid)
                if rid in fin or s.n_tokens >= cap:
                    self._free_blocks(s)
                    s.state = FINISHED
                    self.running.remove(rid)
                else:
                    s.n_tokens += 1
        return sampled

    # ---- trim / fork -------------------------------------------------------------------
    def trim(self, sid: int, n_tokens: int) -> None:
        if self.last_plan is not None:
            raise SchedulerError("trim while a step awaits completion")
        s = self.seqs.get(sid)
        if s is None or s.state != RUNNING or not 1 <= n_tokens <= s.n_tokens:
            raise SchedulerError("trim of a non-running sequence or past its tokens")
        s.n_tokens = n_tokens
        s.num_computed = min(s.num_computed, n_tokens - 1)
        keep = _ceil_div(s.num_computed, self.cfg.block_size)
        if len(s.blocks) > keep:
            self.alloc.free(s.blocks[keep:])
            s.blocks = s.blocks[:keep]

    def fork(self, src: int, new_sid: int) -> None:
        if self.last_plan is not None:
            raise SchedulerError("fork while a step awaits completion")
        s = self.seqs.get(src)
        if s is None or s.state != RUNNING:
            raise SchedulerError("fork of a non-running sequence")
        if new_sid in self.seqs:
            raise SchedulerError(f"sequence {new_sid} exists")
        if len(self.running) >= self.cfg.max_num_seqs:
            raise SchedulerError("fork beyond max_num_seqs")
        f = Seq(new_sid, s.prompt_len, s.group, s.n_tokens, s.num_computed, list(s.blocks))
        if f.blocks:
            self.alloc.incref(f.blocks)
        f.state = RUNNING
        f.order = self.counter
        self.counter += 1
        self.seqs[new_sid] = f
        self.running.append(new_sid)

    # ---- checks ------------------------------------------------------------------------
    def check(self) -> None:
        """Books: refcounts equal the references held by live tables; allocator consistent;
        every running sequence holds exactly the blocks its computed tokens need or fewer."""
        if not self.alloc.check_consistent():
            raise SchedulerError("allocator inconsistent")
        ref = [0] * self.alloc.num_blocks
        for s in self.seqs.values():
            if s.state != RUNNING:
                if s.blocks:
                    raise SchedulerError(f"sequence {s.sid} holds blocks while not running")
                continue
            for b in s.blocks:
                ref[b] += 1
            if len(s.blocks) < _ceil_div(s.num_computed, self.cfg.block_size):
                raise SchedulerError(f"sequence {s.sid} computed past its blocks")
        if ref != self.alloc.refcount:
            raise SchedulerError("refcounts differ from the live tables")
