"""Algorithmic byte and FLOP counts of the paged-KV path (what the method must move).

* KV bytes per token: layers x 2 (K and V) x kv heads x head_dim x element bytes, divided by
  the tensor-parallel degree when kv heads are sharded ("P3: native paged-KV
  continuous-batching sampler", sections "Memory accounting" and "Tensor parallelism >
  Evidence": 147,456 B for 36 x 8 x 128 bf16, 131,072 B for a 32-layer model, 36,864 B per
  rank at tp = 4).
* Decode reads every cached key and value of a row's sequence once: ctx x per-layer KV bytes
  per token. The same page's decode latency model ("Compute" table, KV ms column) is
  batch x ctx x bytes-per-token / HBM bandwidth.
* The append reads and writes each new row once: 2 x 2 x Hkv x D x e per row.
* Prefill: 4 x D x Hq FLOP per visible (query row, key) pair (QK^T and PV, multiply + add);
  the masked upper triangle is not counted.
Padded or split-partial traffic is overhead, never credited.
"""
from __future__ import annotations

from typing import Sequence


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int,
                       tp_degree: int = 1) -> int:
    if kv_heads % tp_degree != 0:
        raise ValueError("tp_degree must divide the kv heads")
    return layers * 2 * (kv_heads // tp_degree) * head_dim * elem_bytes


def decode_kv_bytes(ctx_lens: Sequence[int], kv_heads: int, head_dim: int,
                    elem_bytes: int) -> int:
    """Bytes of K and V one layer's decode step reads: every cached token once per row."""
    per_token = kv_bytes_per_token(1, kv_heads, head_dim, elem_bytes)
    return int(sum(int(c) for c in ctx_lens)) * per_token


def kv_read_time_ms(batch: int, ctx: int, bytes_per_token: int, hbm_bytes_per_s: float) -> float:
    """Decode KV-read time model: batch x ctx x bytes per token / bandwidth, in ms."""
    return batch * ctx * bytes_per_token / hbm_bytes_per_s * 1e3


def append_bytes(n_rows: int, kv_heads: int, head_dim: int, elem_bytes: int,
                 pool_elem_bytes: int = 0) -> int:
    """Bytes the KV append moves: read K and V of every new row (elem_bytes per element) and
    write them into the pools (pool_elem_bytes per element; 0 means the same type, 1 for E4M3
    codes)."""
    out_b = pool_elem_bytes or elem_bytes
    return 2 * n_rows * kv_heads * head_dim * (elem_bytes + out_b)


def visible_pairs(ctx: int, q_len: int) -> int:
    """(query row, key) pairs a segment of q_len rows ending at ctx attends over."""
    prior = ctx - q_len
    return q_len * prior + q_len * (q_len + 1) // 2


def attention_flops(ctx_lens: Sequence[int], q_lens: Sequence[int], num_q_heads: int,
                    head_dim: int) -> int:
    pairs = sum(visible_pairs(int(c), int(q)) for c, q in zip(ctx_lens, q_lens))
    return 4 * head_dim * num_q_heads * pairs


def unique_kv_bytes(block_ids_per_seq, ctx_lens, block_size: int, kv_heads: int, head_dim: int,
                    elem_bytes: int) -> int:
    """Bytes of distinct cached tokens a step reads (shared blocks counted once)."""
    seen = set()
    total_tokens = 0
    for ids, c in zip(block_ids_per_seq, ctx_lens):
        n = (int(c) + block_size - 1) // block_size
        for j in range(n):
            b = int(ids[j])
            if b in seen:
                continue
            seen.add(b)
            total_tokens += min(block_size, int(c) - j * block_size)
    return total_tokens * kv_bytes_per_token(1, kv_heads, head_dim, elem_bytes)
