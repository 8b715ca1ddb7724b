"""Oracle: KV write through a slot mapping, gather, and per-row softmax attention (float64).

Test infrastructure only (see the package docstring).

Definitions followed
  * Pool layout: per layer, K and V tensors [num_blocks, block_size, Hkv, D]; a new token is
    written in place at its (block, offset) slot, with no copy of the existing cache
    ("P3: native paged-KV continuous-batching sampler", section "Design > paged.py",
    PagedKVCache).
  * Slot encoding: slot = block * block_size + offset, the flat index of (block, offset) in
    [num_blocks, block_size]; a negative slot marks a padding row that writes nothing.
  * gather: a sequence's blocks in block-table order, concatenated and cut to its length, as a
    contiguous [Hkv, L, D] array (same page, PagedKVCache.gather; "Optional paged KV cache
    (vLLM-style) — v1 design", section "Design": take the table's blocks, transpose, reshape,
    slice to the offset).
  * Attention: each query row attends over exactly its own keys (P3 page, section
    "Design > paged.py", TorchPagedAttention 'row' mode). The rows of a segment are the last
    q_len positions of its context (chunked prefill advances the computed count; section
    "Design > engine.py", Scheduler), and key j is visible to the row at position pos iff
    j <= pos (a prefill row sees the prior context and the earlier rows of its own chunk; the
    same rule as delta = query_pos - key_pos >= 0 with no window in
    "mixle.utils.parallel.context_parallel_spine module", cp_window_attention_forward).
  * GQA: query head h reads kv head h // (Hq / Hkv), the blocked map (P3 page, section
    "Tensor parallelism (inference, opt-in) > Design", GQA bullet).
  * ctx_lens counts the keys in the cache after this step's append, new tokens included.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


class OracleError(ValueError):
    """Malformed input to the oracle (duplicate slot, slot out of range, bad shapes)."""


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64; exact (bfloat16 is the top half of float32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _to_f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def write_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             slots: Sequence[int], block_size: int) -> None:
    """Scatter row t of k_new / v_new ([T_w, Hkv, D]) to slot slots[t] of the pools, in place.

    Pools hold raw storage elements (uint16 bfloat16 bits or float32), so this is a byte copy.
    Rows are applied in ascending t; a negative slot skips its row; a slot >= num_blocks *
    block_size, or the same non-negative slot twice in one call, is an error and nothing is
    written.
    """
    nb, bs = k_pool.shape[0], k_pool.shape[1]
    if bs != block_size or v_pool.shape != k_pool.shape:
        raise OracleError("pool shape mismatch")
    slots = [int(s) for s in slots]
    if len(slots) != k_new.shape[0] or k_new.shape != v_new.shape:
        raise OracleError("k_new / v_new / slots length mismatch")
    if k_new.shape[1:] != k_pool.shape[2:]:
        raise OracleError("row shape does not match the pool's [Hkv, D]")
    seen = set()
    for s in slots:
        if s < 0:
            continue
        if s >= nb * bs:
            raise OracleError(f"slot {s} outside the pool ({nb} blocks of {bs})")
        if s in seen:
            raise OracleError(f"slot {s} appears twice in one write")
        seen.add(s)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(s, bs)
        k_pool[blk, off] = k_new[t]
        v_pool[blk, off] = v_new[t]


def gather(pool: np.ndarray, block_table_row: Sequence[int], length: int,
           block_size: int) -> np.ndarray:
    """Contiguous [Hkv, length, D] copy of a sequence's first ``length`` cached tokens."""
    if length == 0:
        return np.empty((pool.shape[2], 0, pool.shape[3]), dtype=pool.dtype)
    n_blocks = (length + block_size - 1) // block_size
    ids = [int(x) for x in block_table_row[:n_blocks]]
    if len(ids) < n_blocks:
        raise OracleError("block table shorter than the context")
    for i in ids:
        if not 0 <= i < pool.shape[0]:
            raise OracleError(f"block id {i} outside the pool")
    blocks = pool[ids]                                   # [n_blocks, BS, Hkv, D]
    flat = blocks.reshape(n_blocks * block_size, pool.shape[2], pool.shape[3])[:length]
    return np.ascontiguousarray(flat.transpose(1, 0, 2))  # [Hkv, length, D]


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """GQA blocked map: query head h reads kv head h // (Hq / Hkv)."""
    return h // (hq // hkv)


def n_visible(pos: int) -> int:
    """Keys visible to the row at absolute position pos: 0..pos (causal, no window)."""
    return pos + 1


def attend_rows(q_rows: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                positions: Sequence[int], scale: float) -> np.ndarray:
    """Softmax attention of each query row over exactly its visible keys, in float64.

    q_rows [n, Hq, D]; k_seq, v_seq [Hkv, L, D] contiguous (any storage type); positions[i] is
    the absolute position of row i, which sees keys 0..positions[i]. Returns [n, Hq, D] float64.
    """
    q = _to_f64(q_rows)
    k = _to_f64(k_seq)
    v = _to_f64(v_seq)
    n, hq, d = q.shape
    hkv = k.shape[0]
    if hq % hkv != 0:
        raise OracleError("Hq must be a multiple of Hkv")
    out = np.empty((n, hq, d), dtype=np.float64)
    for i in range(n):
        pos = int(positions[i])
        if not 0 <= pos < k.shape[1]:
            raise OracleError("row position outside the cached context")
        nv = n_visible(pos)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            keys = k[g, :nv]                      # [nv, D]
            vals = v[g, :nv]
            s = scale * (keys @ q[i, h])          # [nv]
            m = s.max()
            w = np.exp(s - m)
            out[i, h] = (w @ vals) / w.sum()
    return out


def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                    block_tables: np.ndarray, ctx_lens: Sequence[int],
                    cu_seqlens_q: Sequence[int], scale: float,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention for a flat ragged step over a paged cache.

    q [T, Hq, D]; pools [NB, BS, Hkv, D]; block_tables [B, max_blocks]; sequence b owns rows
    cu_seqlens_q[b]..cu_seqlens_q[b+1]-1, which are the last q_len positions of its ctx_lens[b]
    cached keys. Returns float64 [T, Hq, D]; when ``rows`` is given only those rows are computed
    and the others are NaN.
    """
    cu = [int(x) for x in cu_seqlens_q]
    ctx = [int(x) for x in ctx_lens]
    B = len(ctx)
    if len(cu) != B + 1 or cu[0] != 0 or cu[-1] != q.shape[0]:
        raise OracleError("cu_seqlens_q must run from 0 to T over B + 1 entries")
    bs = k_pool.shape[1]
    want = None if rows is None else set(int(r) for r in rows)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    for b in range(B):
        q_len = cu[b + 1] - cu[b]
        if q_len < 0 or q_len > ctx[b]:
            raise OracleError("need 0 <= q_len <= ctx_len")
        if q_len == 0:
            continue
        ts = [t for t in range(cu[b], cu[b + 1]) if want is None or t in want]
        if not ts:
            continue
        kc = gather(k_pool, block_tables[b], ctx[b], bs)
        vc = gather(v_pool, block_tables[b], ctx[b], bs)
        positions = [ctx[b] - q_len + (t - cu[b]) for t in ts]
        out[ts] = attend_rows(q[ts], kc, vc, positions, scale)
    return out
