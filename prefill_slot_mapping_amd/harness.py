"""Build one synthetic step on the GPU through the library (allocator, slot mapping, append).

A step is replayed the way the paged engine builds it ("P3: native paged-KV
continuous-batching sampler", sections "Design > paged.py" and "Design > engine.py"): a fully
allocated pool is freed in the workload's seeded order so that the LIFO list holds a
permutation (non-contiguous block tables), sequences are admitted in order (a group member
adopts its leader's full prompt blocks with an incref), each sequence's prior context is
written with pkv_write_kv through pkv_slot_mapping slots, and the step's new rows are written
the same way before attention. Pools start filled with NaN (the E4M3 NaN code for FP8 pools)
so that a stray read shows. FP8 pools are written with pkv_write_kv_fp8 and read with
pkv_attention_fp8, with the workload's per-tensor scales.

Every method step here is a library call; torch only allocates device memory.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import _lib as L


def to_device(arr: np.ndarray, device):
    """uint16 bfloat16 bits or float32 numpy array -> torch tensor of the storage type."""
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def torch_dtype(w):
    import torch
    return torch.bfloat16 if w.spec.dtype == "bf16" else torch.float32


@dataclass
class GpuStep:
    workload: object
    allocator: L.BlockAllocator
    block_tables: np.ndarray      # host int32 [B, MB], -1 past each sequence's blocks
    block_tables_dev: object      # device int32 [B, MB]
    k_cache: object               # device [NB, BS, Hkv, D]
    v_cache: object
    q: object                     # device [T, Hq, D]
    new_slots: np.ndarray         # host int32 [T]
    new_slots_dev: object
    k_new: object                 # device [T, Hkv, D]
    v_new: object
    out: object = None
    workspace: object = None

    def write_new(self, stream=None):
        _write(self.workload, self.k_new, self.v_new, self.new_slots_dev, self.k_cache,
               self.v_cache, stream)

    def attention(self, kv_split: Optional[int] = None, stream=None,
                  phase_consistent: bool = False):
        import torch
        w = self.workload
        split = w.spec.kv_split if kv_split is None else kv_split
        if self.out is None:
            self.out = torch.empty((w.T, w.spec.Hq, w.spec.D), dtype=torch.float32,
                                   device=self.q.device)
        if w.kv_fp8:
            need = L.attention_fp8_workspace_size(w.ctx_lens, w.cu_seqlens_q, w.spec.Hq,
                                                  w.spec.Hkv, w.spec.D, split, phase_consistent)
            if self.workspace is None or self.workspace.numel() < need:
                self.workspace = torch.empty(max(need, 1), dtype=torch.uint8,
                                             device=self.q.device)
            return L.attention_fp8(self.q, self.k_cache, self.v_cache, self.block_tables_dev,
                                   w.ctx_lens, w.cu_seqlens_q, w.scale, w.spec.k_scale,
                                   w.spec.v_scale, out=self.out, workspace=self.workspace,
                                   kv_split=split, stream=stream,
                                   phase_consistent=phase_consistent)
        need = L.attention_workspace_size(w.ctx_lens, w.cu_seqlens_q, w.spec.Hq, w.spec.Hkv,
                                          w.spec.D, split,
                                          L.PKV_BF16 if w.spec.dtype == "bf16" else L.PKV_F32,
                                          phase_consistent)
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=self.q.device)
        return L.attention(self.q, self.k_cache, self.v_cache, self.block_tables_dev,
                           w.ctx_lens, w.cu_seqlens_q, w.scale, out=self.out,
                           workspace=self.workspace, kv_split=split, stream=stream,
                           phase_consistent=phase_consistent)


    def fused_step(self, kv_split: Optional[int] = None, stream=None,
                   phase_consistent: bool = False):
        """The step's KV append and attention in one pkv_write_kv_attention call
        (pkv_write_kv_attention_fp8 for E4M3 pools)."""
        import torch
        w = self.workload
        split = w.spec.kv_split if kv_split is None else kv_split
        if w.kv_fp8:
            if self.out is None:
                self.out = torch.empty((w.T, w.spec.Hq, w.spec.D), dtype=torch.float32,
                                       device=self.q.device)
            need = L.write_kv_attention_fp8_workspace_size(w.ctx_lens, w.cu_seqlens_q, w.spec.Hq,
                                                           w.spec.Hkv, w.spec.D, w.T, split,
                                                           phase_consistent)
            if self.workspace is None or self.workspace.numel() < need:
                self.workspace = torch.empty(max(need, 1), dtype=torch.uint8,
                                             device=self.q.device)
            return L.write_kv_attention_fp8(self.q, self.k_new, self.v_new, self.new_slots,
                                            self.k_cache, self.v_cache, self.block_tables_dev,
                                            w.ctx_lens, w.cu_seqlens_q, w.scale, w.spec.k_scale,
                                            w.spec.v_scale, out=self.out,
                                            workspace=self.workspace, kv_split=split,
                                            stream=stream, phase_consistent=phase_consistent)
        if self.out is None:
            self.out = torch.empty((w.T, w.spec.Hq, w.spec.D), dtype=torch.float32,
                                   device=self.q.device)
        need = L.write_kv_attention_workspace_size(
            w.ctx_lens, w.cu_seqlens_q, w.spec.Hq, w.spec.Hkv, w.spec.D, w.T, split,
            L.PKV_BF16 if w.spec.dtype == "bf16" else L.PKV_F32, phase_consistent)
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=self.q.device)
        return L.write_kv_attention(self.q, self.k_new, self.v_new, self.new_slots, self.k_cache,
                                    self.v_cache, self.block_tables_dev, w.ctx_lens,
                                    w.cu_seqlens_q, w.scale, out=self.out,
                                    workspace=self.workspace, kv_split=split, stream=stream,
                                    phase_consistent=phase_consistent)


def _write(w, k_rows, v_rows, slots, k_cache, v_cache, stream=None):
    if w.kv_fp8:
        L.write_kv_fp8(k_rows, v_rows, slots, k_cache, v_cache, w.spec.k_scale, w.spec.v_scale,
                       stream=stream)
    else:
        L.write_kv(k_rows, v_rows, slots, k_cache, v_cache, stream=stream)


def build_gpu_step(w, device="cuda", write_new: bool = True, workers: int = 8) -> GpuStep:
    import torch
    s = w.spec
    B, NB, BS = w.B, w.num_blocks, s.BS
    alloc = L.BlockAllocator(NB)
    ids = alloc.allocate(NB)
    assert ids == list(range(NB))
    alloc.free(w.free_order.tolist())

    dt = torch_dtype(w)
    if w.kv_fp8:
        k_cache = torch.full((NB, BS, s.Hkv, s.D), 0x7F, dtype=torch.uint8, device=device)
        v_cache = torch.full((NB, BS, s.Hkv, s.D), 0x7F, dtype=torch.uint8, device=device)
    else:
        k_cache = torch.full((NB, BS, s.Hkv, s.D), float("nan"), dtype=dt, device=device)
        v_cache = torch.full((NB, BS, s.Hkv, s.D), float("nan"), dtype=dt, device=device)
    tables = np.full((B, w.max_blocks), -1, dtype=np.int32)

    # admissions in order; each sequence writes its prior context right after its admission,
    # so a group leader's prompt is written before any member adopts (increfs) its blocks
    adm_of = {adm.seq: adm for adm in w.admissions}
    k_new = torch.empty((w.T, s.Hkv, s.D), dtype=dt, device=device)
    v_new = torch.empty((w.T, s.Hkv, s.D), dtype=dt, device=device)
    new_slots = np.full(w.T, -1, dtype=np.int32)
    for b, kk, vv in w.iter_kv(workers=workers):
        adm = adm_of[b]
        if adm.share_from >= 0:
            shared = tables[adm.share_from, :adm.n_shared_blocks].tolist()
            alloc.incref(shared)
            row = shared + alloc.allocate(adm.n_blocks - adm.n_shared_blocks)
        else:
            row = alloc.allocate(adm.n_blocks)
        tables[b, :len(row)] = row
        prior = w.prior_len(b)
        start = adm.n_shared_blocks * BS
        kd = to_device(kk, device)
        vd = to_device(vv, device)
        if prior > start:
            sl = alloc.slots(tables[b], start, prior - start, BS)
            _write(w, kd[start:prior].contiguous(), vd[start:prior].contiguous(), sl, k_cache,
                   v_cache)
        del kd, vd
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        if hi > lo:
            ql = hi - lo
            k_new[lo:hi] = to_device(kk[prior:prior + ql], device)
            v_new[lo:hi] = to_device(vv[prior:prior + ql], device)
    # the step's slots, once every sequence is admitted (shared blocks are read-only by now)
    for b in range(B):
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        if hi > lo:
            new_slots[lo:hi] = alloc.slots(tables[b], w.prior_len(b), hi - lo, BS)
    st = GpuStep(workload=w, allocator=alloc, block_tables=tables,
                 block_tables_dev=torch.from_numpy(tables).to(device), k_cache=k_cache,
                 v_cache=v_cache, q=to_device(w.q, device), new_slots=new_slots,
                 new_slots_dev=torch.from_numpy(new_slots).to(device), k_new=k_new, v_new=v_new)
    if write_new:
        st.write_new()
    torch.cuda.synchronize(device)
    return st
