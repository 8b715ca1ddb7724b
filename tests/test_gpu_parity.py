"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: the KV write and the block bookkeeping bit-exact; attention within max abs error 2e-3
for bfloat16 inputs and 1e-5 for float32 inputs (float64 oracle); a sequence's rows bitwise
identical alone and inside any batch, under any physical block placement, and run to run.
Sizes here are ones the oracle finishes in seconds while still spanning several 64-key tiles
and 512-key splits with ragged tails; full-size steps are checked on sampled rows.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from oracle import build_oracle_step
from workloads import CONFIGS, SMALL_CONFIGS, explicit_spec, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
DEV = "cuda:0"


def _harness():
    from prefill_slot_mapping_amd.harness import build_gpu_step
    return build_gpu_step


def _as_bits(t):
    a = t.detach().cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.view(torch.int32).numpy().view(np.uint32)


def _np_bits(a):
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def _run(gst, **kw):
    out = gst.attention(**kw)
    torch.cuda.synchronize()
    return out.detach().cpu().numpy().astype(np.float64)


def check_step(w, rows=None, seqs=None):
    print(f"[parity] {w.spec.name} B={w.B} T={w.T} NB={w.num_blocks}", flush=True)
    gst = _harness()(w, device=DEV)
    ost = build_oracle_step(w, seqs=seqs, poison=seqs is None)
    assert np.array_equal(gst.block_tables, ost.block_tables)
    assert np.array_equal(gst.new_slots, ost.new_slots)
    got = _run(gst)
    ref = ost.attention(rows)
    sel = np.arange(w.T) if rows is None else np.asarray(sorted(rows))
    assert np.isfinite(got[sel]).all()
    err = float(np.abs(got[sel] - ref[sel]).max()) if sel.size else 0.0
    print(f"[parity] {w.spec.name} max abs err {err:.3e}", flush=True)
    assert err <= TOL[w.spec.dtype]
    return gst, ost, got


@pytest.mark.parametrize("name", list(SMALL_CONFIGS))
def test_small_configs_match_oracle_and_pools_are_bit_exact(name):
    w = make_workload(SMALL_CONFIGS[name])
    gst, ost, _ = check_step(w)
    assert np.array_equal(_as_bits(gst.k_cache), _np_bits(ost.k_pool))
    assert np.array_equal(_as_bits(gst.v_cache), _np_bits(ost.v_pool))
    # bookkeeping: C++ allocator books equal the oracle twin's
    stack, rc = gst.allocator.snapshot()
    assert stack == ost.allocator.free_stack and rc == ost.allocator.refcount


EDGE = [
    # (dtype, Hq, Hkv, D, BS, sequences (ctx, q_len)[, spec keywords])
    ("bf16", 8, 2, 128, 16, [(1, 1), (2, 2), (16, 1), (17, 17), (513, 1), (1024, 1), (1025, 1),
                             (600, 0), (700, 130), (64, 64), (65, 1), (1100, 70)]),
    ("bf16", 4, 4, 128, 1, [(1, 1), (5, 5), (300, 1), (70, 3)]),
    ("bf16", 16, 8, 64, 32, [(3, 1), (100, 100), (1300, 1), (97, 33)]),
    ("bf16", 16, 2, 128, 5, [(7, 1), (129, 1), (642, 1), (88, 20)]),
    ("bf16", 8, 4, 64, 64, [(128, 1), (129, 2), (1, 1), (513, 1)]),
    ("f32", 8, 1, 128, 16, [(1, 1), (600, 1), (45, 45), (130, 9)]),
    ("f32", 4, 2, 64, 16, [(17, 1), (33, 1), (64, 1), (100, 1), (40, 12)]),
    ("f32", 2, 2, 64, 3, [(10, 10), (1030, 1), (77, 1)]),
    # every decode kernel instance: bf16 groups of 4 and 8 at head_dim 64 and 128 (16- and
    # 32-key tiles), and the smallest and largest KV splits
    ("bf16", 16, 4, 64, 16, [(1, 1), (300, 1), (1029, 1), (50, 20), (2100, 1)]),
    ("bf16", 32, 4, 64, 16, [(2, 1), (513, 1), (1500, 1), (40, 9)]),
    ("bf16", 32, 8, 128, 16, [(1, 1), (64, 1), (65, 1), (3000, 1), (90, 31)], {"kv_split": 64}),
    ("bf16", 64, 8, 128, 32, [(17, 1), (4097, 1), (2049, 1)], {"kv_split": 2048}),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}-G{c[1] // c[2]}-D{c[3]}-BS{c[4]}"
                                            + (f"-split{c[6]['kv_split']}" if len(c) > 6 else "")
                                            for c in EDGE])
def test_edge_cases_match_oracle(case):
    dt, hq, hkv, d, bs, seqs = case[:6]
    kw = case[6] if len(case) > 6 else {}
    w = make_workload(explicit_spec(f"edge-{dt}-{hq}-{hkv}-{d}-{bs}", dt, hq, hkv, d, bs, seqs,
                                    **kw))
    check_step(w)


def _alone(gst, b, w):
    """Sequence b run alone: its own table row, its own q rows, the same pools."""
    lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
    out = pkv.attention(gst.q[lo:hi].contiguous(), gst.k_cache, gst.v_cache,
                        gst.block_tables_dev[b:b + 1].contiguous(), [int(w.ctx_lens[b])],
                        [0, hi - lo], w.scale, kv_split=w.spec.kv_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["mixed-ragged-step", "prefix-shared-decode",
                                  "long-context-decode"])
def test_alone_equals_batched_bitwise(name):
    w = make_workload(SMALL_CONFIGS[name])
    gst = _harness()(w, device=DEV)
    batched = gst.attention().cpu().numpy()
    for b in range(w.B):
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        if hi == lo:
            continue
        assert np.array_equal(_alone(gst, b, w), batched[lo:hi]), f"sequence {b}"


def test_group_and_full_batch_bitwise_for_prefix_sharing():
    w = make_workload(SMALL_CONFIGS["prefix-shared-decode"])
    gst = _harness()(w, device=DEV)
    full = gst.attention().cpu().numpy()
    for g in sorted(set(w.group_of.tolist())):
        members = np.flatnonzero(w.group_of == g)
        rows = [int(w.cu_seqlens_q[b]) for b in members]
        out = pkv.attention(gst.q[rows].contiguous(), gst.k_cache, gst.v_cache,
                            gst.block_tables_dev[members].contiguous(), w.ctx_lens[members],
                            np.arange(len(members) + 1, dtype=np.int32), w.scale)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), full[rows])


@pytest.mark.parametrize("dims", [(32, 8, 128, 16), (16, 2, 128, 32), (8, 8, 64, 16),
                                  (16, 2, 64, 5)])
def test_prefill_rechunking_is_bitwise_invisible(dims):
    """A segment's rows give the same bits as one chunk, as several chunks (each over the cache
    as it stands after it), and as chunks batched together with strangers."""
    hq, hkv, d, bs = dims
    w = make_workload(explicit_spec(f"rechunk-{hq}-{hkv}-{d}-{bs}", "bf16", hq, hkv, d, bs,
                                    [(700, 300), (90, 2), (300, 1)]))
    gst = _harness()(w, device=DEV)
    full = gst.attention().cpu().numpy().copy()
    rows = full[0:300]
    bt = gst.block_tables_dev[0:1].contiguous()
    got = []
    for lo, hi in [(0, 37), (37, 101), (101, 102), (102, 103), (103, 300)]:
        if hi - lo == 1:
            continue                        # a 1-row segment is a decode row: another kind
        out = pkv.attention(gst.q[lo:hi].contiguous(), gst.k_cache, gst.v_cache, bt,
                            [400 + hi], [0, hi - lo], w.scale)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), rows[lo:hi]), (lo, hi)
    # two chunks of the same sequence as two segments of one step, next to a stranger
    q2 = torch.cat([gst.q[0:37], gst.q[300:302], gst.q[37:300]]).contiguous()
    bt2 = torch.cat([bt, gst.block_tables_dev[1:2], bt]).contiguous()
    out = pkv.attention(q2, gst.k_cache, gst.v_cache, bt2, [437, 90, 700], [0, 37, 39, 302],
                        w.scale)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(o[0:37], rows[0:37])
    assert np.array_equal(o[39:302], rows[37:300])
    assert np.array_equal(o[37:39], full[300:302])


def test_physical_block_permutation_is_bitwise_invisible():
    w = make_workload(SMALL_CONFIGS["mixed-ragged-step"])
    gst = _harness()(w, device=DEV)
    ref = gst.attention().cpu().numpy().copy()
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(7))
    inv = torch.argsort(perm).to(DEV)
    kc = gst.k_cache.index_select(0, inv).contiguous()   # block i now lives at perm[i]
    vc = gst.v_cache.index_select(0, inv).contiguous()
    t = gst.block_tables
    t2 = np.where(t >= 0, perm.numpy()[np.maximum(t, 0)], -1).astype(np.int32)
    out = pkv.attention(gst.q, kc, vc, torch.from_numpy(t2).to(DEV), w.ctx_lens, w.cu_seqlens_q,
                        w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


def test_run_to_run_determinism():
    w = make_workload(SMALL_CONFIGS["long-context-decode"])
    gst = _harness()(w, device=DEV)
    a = gst.attention().cpu().numpy().copy()
    for _ in range(3):
        assert np.array_equal(gst.attention().cpu().numpy(), a)


def test_out_of_range_block_id_gives_nan_not_a_fault():
    w = make_workload(explicit_spec("badblock", "bf16", 8, 2, 128, 16, [(40, 1), (40, 1)]))
    gst = _harness()(w, device=DEV)
    good = gst.attention().cpu().numpy().copy()
    t = gst.block_tables.copy()
    t[0, 1] = w.num_blocks + 1000            # a block the row needs
    out = pkv.attention(gst.q, gst.k_cache, gst.v_cache, torch.from_numpy(t).to(DEV),
                        w.ctx_lens, w.cu_seqlens_q, w.scale)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isnan(o[0]).all()
    assert np.array_equal(o[1], good[1])


def test_write_kv_skips_negative_and_out_of_range_slots():
    nb, bs, hkv, d = 4, 16, 2, 64
    kc = torch.zeros((nb, bs, hkv, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kn = torch.randn((3, hkv, d), device=DEV).to(torch.bfloat16)
    vn = torch.randn((3, hkv, d), device=DEV).to(torch.bfloat16)
    slots = torch.tensor([5, -1, nb * bs + 3], dtype=torch.int32, device=DEV)
    pkv.write_kv(kn, vn, slots, kc, vc)
    torch.cuda.synchronize()
    flat = kc.view(nb * bs, hkv, d)
    assert torch.equal(flat[5], kn[0])
    assert int((flat.float().abs().sum(dim=(1, 2)) > 0).sum()) == 1


FULL_SAMPLES = {
    "tiny-f32-decode": None,
    "batched-bf16-decode": "decode",
    "mixed-ragged-step": "mixed",
    "long-context-decode": "decode",
    "prefix-shared-decode": "decode",
}


@pytest.mark.parametrize("name", list(CONFIGS))
def test_full_size_configs_on_sampled_rows(name):
    w = make_workload(CONFIGS[name])
    rng = np.random.default_rng(11)
    if FULL_SAMPLES[name] is None:
        seqs, rows = None, None
    else:
        dec = [b for b in range(w.B) if w.q_lens[b] == 1]
        pre = [b for b in range(w.B) if w.q_lens[b] > 1]
        seqs = sorted(set(rng.choice(dec, size=min(4, len(dec)), replace=False).tolist()))
        seqs.append(int(np.argmax(w.ctx_lens)))          # the longest sequence too
        if pre:
            seqs += rng.choice(pre, size=2, replace=False).tolist()
        seqs = sorted(set(seqs))
        rows = []
        for b in seqs:
            lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
            cand = sorted(set([lo, hi - 1, (lo + hi) // 2] +
                              rng.integers(lo, hi, size=min(3, hi - lo)).tolist()))
            rows += cand
    check_step(w, rows=rows, seqs=seqs)


def _rows_of(w, seqs):
    return np.concatenate([np.arange(w.cu_seqlens_q[b], w.cu_seqlens_q[b + 1])
                           for b in seqs]).astype(np.int64)


def _sub_batch(gst, w, seqs, **kw):
    """The sequences `seqs` as a step of their own on the same pools (their q rows, table rows
    and lengths); returns their output rows."""
    rows = _rows_of(w, seqs)
    cu = np.concatenate([[0], np.cumsum([w.q_lens[b] for b in seqs])]).astype(np.int32)
    q = gst.q.index_select(0, torch.from_numpy(rows).to(DEV)).contiguous()
    bt = gst.block_tables_dev[torch.as_tensor(list(seqs), device=DEV)].contiguous()
    ctx = np.asarray([w.ctx_lens[b] for b in seqs], np.int32)
    out = pkv.attention(q, gst.k_cache, gst.v_cache, bt, ctx, cu, w.scale,
                        kv_split=w.spec.kv_split, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_full_size_prefix_shared_step_is_bitwise_invariant():
    """All 128 sequences of the full prefix-shared step (16 groups x 8 samples on a shared
    2048-token prompt): each alone, each group as a step, and the full batch give the same bits
    for every sequence."""
    w = make_workload(CONFIGS["prefix-shared-decode"])
    print(f"[invariance] {w.spec.name} B={w.B}", flush=True)
    gst = _harness()(w, device=DEV)
    full = gst.attention().cpu().numpy().copy()
    assert np.isfinite(full).all()
    for b in range(w.B):
        got = _sub_batch(gst, w, [b])
        assert np.array_equal(got.view(np.uint32), full[_rows_of(w, [b])].view(np.uint32)), b
    for g in sorted(set(w.group_of.tolist())):
        members = np.flatnonzero(w.group_of == g).tolist()
        got = _sub_batch(gst, w, members)
        assert np.array_equal(got.view(np.uint32), full[_rows_of(w, members)].view(np.uint32)), g
    # two groups together, in reverse order, as a third batch composition
    pair = np.flatnonzero(w.group_of == 3).tolist()[::-1] + np.flatnonzero(w.group_of == 0).tolist()
    got = _sub_batch(gst, w, pair)
    assert np.array_equal(got.view(np.uint32), full[_rows_of(w, pair)].view(np.uint32))


@pytest.mark.parametrize("name", ["mixed-ragged-step", "long-context-decode"])
def test_full_size_sequences_alone_equal_the_batch_bitwise(name):
    w = make_workload(CONFIGS[name])
    print(f"[invariance] {w.spec.name} B={w.B} T={w.T}", flush=True)
    gst = _harness()(w, device=DEV)
    full = gst.attention().cpu().numpy().copy()
    rng = np.random.default_rng(21)
    live = [b for b in range(w.B) if w.q_lens[b] > 0]
    seqs = sorted(set(rng.choice(live, size=min(12, len(live)), replace=False).tolist())
                  | {b for b in live if w.q_lens[b] > 1} | {int(np.argmax(w.ctx_lens))})
    for b in seqs:
        got = _sub_batch(gst, w, [b])
        assert np.array_equal(got.view(np.uint32), full[_rows_of(w, [b])].view(np.uint32)), b
