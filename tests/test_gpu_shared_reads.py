"""Shared reads (pkv_write_kv_attention_shared) on the GPU, through the C ABI.

Decode splits that lie wholly in the same physical blocks for several rows (a shared prompt's
read-only blocks: "P3: native paged-KV continuous-batching sampler", section "Design >
engine.py", Prefix sharing) are read once per group of rows. Every row's arithmetic is that of
its per-row decode item, so the output must be bitwise the output of pkv_write_kv_attention on
the same step, and of each sequence alone; it must also stay within the bf16 tolerance of the
oracle. A row whose device table names other blocks than the host copy the planner used must
come out NaN, never another row's result.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from workloads import CONFIGS, SMALL_CONFIGS, Spec, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu_step(w):
    from prefill_slot_mapping_amd.harness import build_gpu_step
    return build_gpu_step(w, device=DEV)


def _shared(gst, w, bt_host=None):
    out = pkv.write_kv_attention_shared(
        gst.q, gst.k_new, gst.v_new, gst.new_slots, gst.k_cache, gst.v_cache,
        gst.block_tables_dev, gst.block_tables if bt_host is None else bt_host, w.ctx_lens,
        w.cu_seqlens_q, w.scale, kv_split=w.spec.kv_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _plain(gst, w):
    out = pkv.write_kv_attention(gst.q, gst.k_new, gst.v_new, gst.new_slots, gst.k_cache,
                                 gst.v_cache, gst.block_tables_dev, w.ctx_lens, w.cu_seqlens_q,
                                 w.scale, kv_split=w.spec.kv_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _alone(gst, w, b):
    lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
    out = pkv.attention(gst.q[lo:hi].contiguous(), gst.k_cache, gst.v_cache,
                        gst.block_tables_dev[b:b + 1].contiguous(), [int(w.ctx_lens[b])],
                        [0, hi - lo], w.scale, kv_split=w.spec.kv_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHARED_SPECS = [
    # (Hq, Hkv, D, BS, groups, per_group, prefix, tail_lo, tail_hi, kv_split)
    (16, 4, 128, 16, 3, 5, 1536, 1, 900, 512),
    (8, 4, 128, 16, 2, 4, 1024, 0, 600, 512),      # group 2; a tail of 0 (prompt only)
    (4, 4, 64, 32, 2, 6, 2048, 1, 400, 256),       # group 1, head_dim 64
    (16, 4, 128, 16, 2, 3, 512, 1, 64, 512),        # one whole shared split each
    (16, 4, 128, 8, 1, 7, 704, 1, 2000, 64),       # many short splits
    (32, 4, 128, 16, 2, 5, 1536, 1, 900, 512),     # group 8: two rows per group item
    (64, 8, 64, 32, 2, 3, 1024, 1, 700, 256),      # group 8, head_dim 64
]


@pytest.mark.parametrize("dims", SHARED_SPECS,
                         ids=[f"G{d[0] // d[1]}-D{d[2]}-BS{d[3]}-split{d[9]}" for d in SHARED_SPECS])
def test_shared_reads_equal_per_row_reads_bitwise(dims):
    from oracle import build_oracle_step
    hq, hkv, d, bs, groups, per, prefix, tlo, thi, split = dims
    spec = Spec(f"shared-{hq}-{hkv}-{d}-{bs}-{split}", "bf16", Hq=hq, Hkv=hkv, D=d, BS=bs,
                shared=(groups, per, prefix, max(tlo, 1), thi), kv_split=split)
    w = make_workload(spec)
    print(f"[shared] {spec.name} B={w.B}", flush=True)
    gst = _gpu_step(w)
    got = _shared(gst, w)
    assert np.isfinite(got).all()
    assert np.array_equal(got.view(np.uint32), _plain(gst, w).view(np.uint32))
    for b in range(0, w.B, 2):
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        assert np.array_equal(_alone(gst, w, b).view(np.uint32), got[lo:hi].view(np.uint32)), b
    ref = build_oracle_step(w).attention()
    assert float(np.abs(got.astype(np.float64) - ref).max()) <= 2e-3


def test_block_size_not_dividing_the_split():
    """Block 5, split 64: a split's first and last blocks are partly outside it; rows share a
    split only if every block it touches is the same."""
    spec = Spec("shared-bs5", "bf16", Hq=8, Hkv=2, D=128, BS=5, shared=(2, 4, 320, 1, 300),
                kv_split=64)
    w = make_workload(spec)
    gst = _gpu_step(w)
    got = _shared(gst, w)
    assert np.array_equal(got.view(np.uint32), _plain(gst, w).view(np.uint32))


def test_full_size_prefix_shared_step_bitwise_with_shared_reads():
    """The full prefix-shared step (16 groups x 8 samples on a 2048-token prompt): the shared
    call equals the per-row call, every sequence alone, and every group on its own."""
    w = make_workload(CONFIGS["prefix-shared-decode"])
    print(f"[shared] {w.spec.name} B={w.B}", flush=True)
    gst = _gpu_step(w)
    got = _shared(gst, w)
    assert np.array_equal(got.view(np.uint32), _plain(gst, w).view(np.uint32))
    for b in range(w.B):
        assert np.array_equal(_alone(gst, w, b).view(np.uint32), got[b:b + 1].view(np.uint32)), b
    for g in sorted(set(w.group_of.tolist())):
        members = np.flatnonzero(w.group_of == g)
        rows = [int(w.cu_seqlens_q[b]) for b in members]
        cu = np.arange(len(members) + 1, dtype=np.int32)
        sub_k = gst.k_new.index_select(0, torch.as_tensor(rows, device=DEV)).contiguous()
        sub_v = gst.v_new.index_select(0, torch.as_tensor(rows, device=DEV)).contiguous()
        out = pkv.write_kv_attention_shared(
            gst.q[rows].contiguous(), sub_k, sub_v, gst.new_slots[rows].copy(), gst.k_cache,
            gst.v_cache, gst.block_tables_dev[members].contiguous(), gst.block_tables[members],
            w.ctx_lens[members], cu, w.scale)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), got[rows].view(np.uint32)), g


def test_host_tables_that_differ_from_the_device_give_nan_rows():
    spec = Spec("shared-mismatch", "bf16", Hq=16, Hkv=4, D=128, BS=16, shared=(2, 3, 1024, 1, 200))
    w = make_workload(spec)
    gst = _gpu_step(w)
    good = _plain(gst, w)
    # the host copy claims the first sample of group 1 shares group 0's prompt blocks; the
    # device tables say otherwise
    a = int(np.flatnonzero(w.group_of == 0)[0])
    b = int(np.flatnonzero(w.group_of == 1)[0])
    bt = gst.block_tables.copy()
    n = int(w.prefix_tokens[a]) // spec.BS
    bt[b, :n] = bt[a, :n]
    got = _shared(gst, w, bt_host=bt)
    others = [r for r in range(w.B) if r != b]
    assert np.array_equal(got[others].view(np.uint32), good[others].view(np.uint32))
    assert np.isnan(got[b]).all()


FP8_SHARED_SPECS = [
    # (Hq, Hkv, D, BS, groups, per_group, prefix, tail_lo, tail_hi, kv_split)
    (16, 4, 128, 16, 3, 5, 1536, 1, 900, 512),     # group 4: four rows per group item
    (32, 4, 128, 16, 2, 5, 1536, 1, 900, 512),     # group 8: two rows per group item
    (4, 4, 64, 32, 2, 6, 2048, 1, 400, 256),       # group 1, head_dim 64
    (8, 4, 128, 8, 1, 7, 704, 1, 2000, 64),        # group 2, many short splits
]


@pytest.mark.parametrize("dims", FP8_SHARED_SPECS,
                         ids=[f"G{d[0] // d[1]}-D{d[2]}-BS{d[3]}-split{d[9]}"
                              for d in FP8_SHARED_SPECS])
def test_fp8_shared_reads_equal_per_row_reads_bitwise(dims):
    """E4M3 pools ("Finish RL Training Faster: Bitwise-Consistent ...", section 4.2: one read
    path for FP8 storage): the shared call equals pkv_write_kv_attention_fp8 and each row
    alone bitwise, and the dequantising oracle within the bar."""
    from oracle import build_oracle_step
    hq, hkv, d, bs, groups, per, prefix, tlo, thi, split = dims
    spec = Spec(f"shared-fp8-{hq}-{hkv}-{d}-{bs}-{split}", "bf16", Hq=hq, Hkv=hkv, D=d, BS=bs,
                shared=(groups, per, prefix, max(tlo, 1), thi), kv_split=split, kv_dtype="fp8",
                k_scale=1 / 32, v_scale=1 / 48)
    w = make_workload(spec)
    print(f"[shared-fp8] {spec.name} B={w.B}", flush=True)
    gst = _gpu_step(w)
    got = pkv.write_kv_attention_shared_fp8(
        gst.q, gst.k_new, gst.v_new, gst.new_slots, gst.k_cache, gst.v_cache,
        gst.block_tables_dev, gst.block_tables, w.ctx_lens, w.cu_seqlens_q, w.scale,
        spec.k_scale, spec.v_scale, kv_split=split)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.isfinite(got).all()
    plain = pkv.write_kv_attention_fp8(
        gst.q, gst.k_new, gst.v_new, gst.new_slots, gst.k_cache, gst.v_cache,
        gst.block_tables_dev, w.ctx_lens, w.cu_seqlens_q, w.scale, spec.k_scale, spec.v_scale,
        kv_split=split)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), plain.cpu().numpy().view(np.uint32))
    for b in range(0, w.B, 2):
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        alone = pkv.attention_fp8(gst.q[lo:hi].contiguous(), gst.k_cache, gst.v_cache,
                                  gst.block_tables_dev[b:b + 1].contiguous(),
                                  [int(w.ctx_lens[b])], [0, hi - lo], w.scale, spec.k_scale,
                                  spec.v_scale, kv_split=split)
        torch.cuda.synchronize()
        assert np.array_equal(alone.cpu().numpy().view(np.uint32), got[lo:hi].view(np.uint32)), b
    ref = build_oracle_step(w).attention()
    assert float(np.abs(got.astype(np.float64) - ref).max()) <= 2e-3
