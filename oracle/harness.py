"""Oracle: replay a synthetic step into oracle-owned pools — test infrastructure only.

A step is built the way the paged engine builds it ("P3: native paged-KV continuous-batching
sampler", sections "Design > paged.py" and "Design > engine.py"): a fully allocated pool is
freed in the workload's seeded order (so the LIFO list holds a permutation and block tables are
non-contiguous), sequences are admitted in order (a group member adopts its leader's full
prompt blocks), each sequence's prior context is written through the slot mapping, and the
step's new rows are written through the slot mapping before attention runs.

Nothing here comes from the GPU path: pools, tables and slots are the oracle's own.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Optional

import numpy as np

from .allocator import BlockAllocator
from .paged import paged_attention, write_kv


@dataclass
class OracleStep:
    workload: object
    allocator: BlockAllocator
    block_tables: np.ndarray       # int32 [B, max_blocks], -1 past each sequence's blocks
    k_pool: np.ndarray             # [NB, BS, Hkv, D] raw storage (uint16 bf16 bits / float32)
    v_pool: np.ndarray
    new_slots: np.ndarray          # int32 [T]: slot of each query row's new token
    k_new: np.ndarray              # [T, Hkv, D] the step's new K rows
    v_new: np.ndarray
    written_new: bool = False

    def write_new(self) -> None:
        """The step's append: scatter the new rows through their slots."""
        w = self.workload
        write_kv(self.k_pool, self.v_pool, self.k_new, self.v_new, self.new_slots, w.spec.BS)
        self.written_new = True

    def attention(self, rows: Optional[Iterable[int]] = None) -> np.ndarray:
        w = self.workload
        return paged_attention(w.q, self.k_pool, self.v_pool, self.block_tables, w.ctx_lens,
                               w.cu_seqlens_q, w.scale,
                               rows=None if rows is None else list(rows))


def _poison(shape, dtype):
    if dtype == np.uint16:
        return np.full(shape, 0x7FC0, dtype=np.uint16)     # bfloat16 quiet NaN
    return np.full(shape, np.nan, dtype=np.float32)


def build_oracle_step(w, seqs: Optional[Iterable[int]] = None, poison: bool = True,
                      write_new: bool = True) -> OracleStep:
    """Allocator replay, prior-context writes and (optionally) the step's append.

    ``seqs`` restricts the K/V writes to those sequences (the allocator replay always covers
    all of them, so block ids match the full step); other sequences' blocks stay poisoned.
    """
    s = w.spec
    B, NB, BS = w.B, w.num_blocks, s.BS
    alloc = BlockAllocator(NB)
    everything = alloc.allocate(NB)
    assert everything == list(range(NB))
    alloc.free([int(i) for i in w.free_order])

    tables = np.full((B, w.max_blocks), -1, dtype=np.int32)
    dt = w.np_dtype
    shape = (NB, BS, s.Hkv, s.D)
    k_pool = _poison(shape, dt) if poison else np.zeros(shape, dtype=dt)
    v_pool = _poison(shape, dt) if poison else np.zeros(shape, dtype=dt)
    chosen = set(range(B)) if seqs is None else set(int(b) for b in seqs)

    k_new = np.zeros((w.T, s.Hkv, s.D), dtype=dt)
    v_new = np.zeros((w.T, s.Hkv, s.D), dtype=dt)
    new_slots = np.full(w.T, -1, dtype=np.int32)
    kv_cache = {}

    for adm in w.admissions:
        b = adm.seq
        if adm.share_from >= 0:
            shared = [int(x) for x in tables[adm.share_from, :adm.n_shared_blocks]]
            alloc.incref(shared)
            own = alloc.allocate(adm.n_blocks - adm.n_shared_blocks)
            row = shared + own
        else:
            row = alloc.allocate(adm.n_blocks)
        tables[b, :len(row)] = row
        prior = w.prior_len(b)
        start = adm.n_shared_blocks * BS
        if b in chosen or any(a.share_from == b for a in w.admissions):
            kk, vv = w.kv(b)
            kv_cache[b] = (kk, vv)
            if prior > start:
                sl = alloc.slots(row, start, prior - start, BS)
                write_kv(k_pool, v_pool, kk[start:prior], vv[start:prior], sl, BS)

    for b in range(B):
        ql = int(w.q_lens[b])
        if ql == 0:
            continue
        prior = w.prior_len(b)
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        new_slots[lo:hi] = alloc.slots(tables[b], prior, ql, BS)
        if b in kv_cache:
            kk, vv = kv_cache[b]
            k_new[lo:hi] = kk[prior:prior + ql]
            v_new[lo:hi] = vv[prior:prior + ql]

    st = OracleStep(workload=w, allocator=alloc, block_tables=tables, k_pool=k_pool,
                    v_pool=v_pool, new_slots=new_slots, k_new=k_new, v_new=v_new)
    if write_new:
        if seqs is not None:
            # only chosen sequences' rows are meaningful; others write into their own blocks
            keep = np.full(w.T, -1, dtype=np.int32)
            for b in chosen:
                lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
                keep[lo:hi] = new_slots[lo:hi]
            write_kv(k_pool, v_pool, k_new, v_new, keep, BS)
            st.written_new = True
        else:
            st.write_new()
    return st
