"""CPU oracle for the paged-KV append and paged attention — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct reference that the HIP library is checked
against. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the library itself never does, and this package imports nothing
from the library. It shares no code with the GPU path: the two meet only in the seeded input
generators of ``workloads``, which hold none of the method's arithmetic.

Floating point is evaluated in float64 (bfloat16 and float32 inputs widen exactly).

Modules
  paged      write (slot scatter), gather to contiguous [Hkv, L, D], and softmax attention one
             query row at a time over exactly that row's keys.
  allocator  block bookkeeping twin: LIFO free list, refcounts, all-or-nothing allocation,
             read-only shared blocks, the slot rule.
  harness    replays a workload's admissions and prior-context writes into oracle pools.
  scheduler  the host step builder: decodes first, chunked prefill within a token budget, FIFO
             admission, preemption of the youngest by recompute, prefix adoption of full
             blocks with the last prompt token recomputed, trim, copy-on-write forks.
  fp8        the OCP E4M3 codec (nearest, ties to even, saturating at 448) and the FP8 KV
             write with per-tensor scales (one float32 multiply by the float32 reciprocal).

Every function is pinned by ``tests/test_oracle_*.py`` to something other than itself:
torch's float64 scaled_dot_product_attention on contiguous K/V, closed forms (one key, zero
query, constant values, a dominant key), storage equivalence, re-chunking invariance,
invariant-checked random allocator event runs, and planted mistakes that those pins must catch.
"""
from .paged import (bf16_bits_to_f64, write_kv, gather, attend_rows, paged_attention,
                    OracleError)
from .allocator import (BlockAllocator, AllocatorError, PoolExhausted, DoubleFree, SharedWrite,
                        InvalidBlock)
from .harness import OracleStep, build_oracle_step
from .scheduler import SchedConfig, Scheduler, SchedulerError, StepPlan
from . import fp8

__all__ = [
    "bf16_bits_to_f64", "write_kv", "gather", "attend_rows", "paged_attention", "OracleError",
    "BlockAllocator", "AllocatorError", "PoolExhausted", "DoubleFree", "SharedWrite",
    "InvalidBlock", "OracleStep", "build_oracle_step", "SchedConfig", "Scheduler",
    "SchedulerError", "StepPlan", "fp8",
]
