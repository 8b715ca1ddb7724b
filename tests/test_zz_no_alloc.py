"""pkv_attention_noalloc (the library's own device scratch instead of a caller workspace)
against pkv_attention_ex on the same inputs, through the C ABI.

Two calls in a row, the second on a smaller step (the scratch keeps the first call's larger
lists and partials: the second must not read them), then the phase-consistent mode, then a
step too large for the scratch, which must be refused before anything is enqueued. The
entry point shares the kernels and the planner of pkv_attention_ex, so every output is
compared bitwise; the first step is also checked against the oracle. After the first call on
the device no staging allocation may happen.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from workloads import SMALL_CONFIGS, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _sub(gst, w, seqs):
    rows = np.concatenate([np.arange(w.cu_seqlens_q[b], w.cu_seqlens_q[b + 1])
                           for b in seqs]).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum([w.q_lens[b] for b in seqs])]).astype(np.int32)
    q = gst.q.index_select(0, torch.from_numpy(rows).to(DEV)).contiguous()
    bt = gst.block_tables_dev[torch.as_tensor(list(seqs), device=DEV)].contiguous()
    ctx = np.asarray([w.ctx_lens[b] for b in seqs], np.int32)
    return q, bt, ctx, cu


def _pair(gst, w, q, bt, ctx, cu, **kw):
    """(pkv_attention_ex result, pkv_attention_noalloc result) on the same inputs."""
    ref = pkv.attention(q, gst.k_cache, gst.v_cache, bt, ctx, cu, w.scale,
                        kv_split=w.spec.kv_split, **kw)
    out = torch.full_like(ref, float("nan"))
    pkv.attention_noalloc(q, gst.k_cache, gst.v_cache, bt, ctx, cu, w.scale, out,
                          kv_split=w.spec.kv_split, **kw)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def test_noalloc_equals_the_workspace_entry_point():
    from oracle import build_oracle_step
    from prefill_slot_mapping_amd.harness import build_gpu_step
    w = make_workload(SMALL_CONFIGS["mixed-ragged-step"])
    print(f"[noalloc] {w.spec.name} B={w.B} T={w.T}", flush=True)
    gst = build_gpu_step(w, device=DEV)
    all_seqs = list(range(w.B))

    # call 1: the whole step
    ref, got = _pair(gst, w, *_sub(gst, w, all_seqs))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    oracle = build_oracle_step(w).attention()
    assert float(np.abs(got.astype(np.float64) - oracle).max()) <= 2e-3
    slot_bytes, allocs = pkv.staging_info()
    assert slot_bytes >= 1 << 20

    # call 2: a smaller step (two of the sequences, reversed), right after
    small = [b for b in all_seqs if w.q_lens[b] > 0][-2:][::-1]
    ref2, got2 = _pair(gst, w, *_sub(gst, w, small))
    assert got2.shape[0] < got.shape[0]
    assert np.array_equal(got2.view(np.uint32), ref2.view(np.uint32))

    # the phase-consistent mode through the same scratch
    ref3, got3 = _pair(gst, w, *_sub(gst, w, all_seqs), phase_consistent=True)
    assert np.array_equal(got3.view(np.uint32), ref3.view(np.uint32))
    assert pkv.staging_info()[1] == allocs          # nothing allocated after set-up


def test_noalloc_refuses_a_step_larger_than_its_scratch():
    hq, hkv, d, bs, B = 32, 8, 128, 16, 64
    ctx = np.full(B, 300_000, np.int32)             # 586 splits per row: ~624 MB of partials
    cu = np.arange(B + 1, dtype=np.int32)
    need = pkv.attention_workspace_size(ctx, cu, hq, hkv, d, 512, pkv.PKV_BF16)
    assert need > pkv._lib.NOALLOC_SCRATCH_BYTES
    mb = -(-300_000 // bs)
    bt = torch.zeros((B, mb), dtype=torch.int32, device=DEV)
    q = torch.zeros((B, hq, d), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((4, bs, hkv, d), dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, hq, d), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(pkv.Unsupported, match="static scratch"):
        pkv.attention_noalloc(q, kc, kc, bt, ctx, cu, 0.1, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())                  # nothing ran
