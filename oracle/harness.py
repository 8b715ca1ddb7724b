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
from .fp8 import dequantize, quantize_rows
from .paged import attend_rows, bf16_bits_to_f64, gather, paged_attention, write_kv


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
        _write(w, self.k_pool, self.v_pool, self.k_new, self.v_new, self.new_slots)
        self.written_new = True

    def attention(self, rows: Optional[Iterable[int]] = None) -> np.ndarray:
        w = self.workload
        if not getattr(w, "kv_fp8", False):
            return paged_attention(w.q, self.k_pool, self.v_pool, self.block_tables, w.ctx_lens,
                                   w.cu_seqlens_q, w.scale,
                                   rows=None if rows is None else list(rows))
        # FP8 pools: each sequence's codes are gathered, then dequantised (code * scale) to
        # float64 and attended exactly like any other pool
        s = w.spec
        want = None if rows is None else set(int(r) for r in rows)
        out = np.full(w.q.shape, np.nan, dtype=np.float64)
        for b in range(w.B):
            lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
            ts = [t for t in range(lo, hi) if want is None or t in want]
            if not ts:
                continue
            ctx = int(w.ctx_lens[b])
            kc = dequantize(gather(self.k_pool, self.block_tables[b], ctx, s.BS), s.k_scale)
            vc = dequantize(gather(self.v_pool, self.block_tables[b], ctx, s.BS), s.v_scale)
            positions = [ctx - (hi - lo) + (t - lo) for t in ts]
            out[ts] = attend_rows(w.q[ts], kc, vc, positions, w.scale)
        return out


def _as_f32(rows: np.ndarray) -> np.ndarray:
    """bfloat16 bits or float32 rows -> float32 values (exact)."""
    if rows.dtype == np.uint16:
        return bf16_bits_to_f64(rows).astype(np.float32)
    return np.asarray(rows, dtype=np.float32)


def _write(w, k_pool, v_pool, k_rows, v_rows, slots) -> None:
    """The append of rows through slots; FP8 pools store the rows' E4M3 codes."""
    if getattr(w, "kv_fp8", False):
        k_rows = quantize_rows(_as_f32(k_rows), w.spec.k_scale)
        v_rows = quantize_rows(_as_f32(v_rows), w.spec.v_scale)
    write_kv(k_pool, v_pool, k_rows, v_rows, slots, w.spec.BS)


def _poison(shape, dtype):
    if dtype == np.uint8:
        return np.full(shape, 0x7F, dtype=np.uint8)        # E4M3 NaN
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
    pdt = np.uint8 if getattr(w, "kv_fp8", False) else dt
    shape = (NB, BS, s.Hkv, s.D)
    k_pool = _poison(shape, pdt) if poison else np.zeros(shape, dtype=pdt)
    v_pool = _poison(shape, pdt) if poison else np.zeros(shape, dtype=pdt)
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
                _write(w, k_pool, v_pool, kk[start:prior], vv[start:prior], sl)

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
            _write(w, k_pool, v_pool, k_new, v_new, keep)
            st.written_new = True
        else:
            st.write_new()
    return st
