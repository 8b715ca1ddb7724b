"""Host side of the C ABI, on the CPU: symbols, block bookkeeping, slot mapping, validation.

The C++ allocator must equal the oracle's twin bit-exactly on identical event traces: same
returned ids, same error kinds, same free-stack order and refcounts after every event.
Device entry points are exercised only for their host-side validation (nothing reaches the GPU:
every call below is refused before any launch).
"""
import ctypes

import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from prefill_slot_mapping_amd import _lib as L
import oracle

pytestmark = []

# a fake device address, 256-byte aligned: validation never dereferences it
F = 0x1000


def test_library_exports_every_header_function():
    lib = pkv.lib()
    names = pkv.header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    assert pkv.version().startswith("pkv")


ERRMAP = {
    oracle.PoolExhausted: pkv.PoolExhausted,
    oracle.DoubleFree: pkv.DoubleFree,
    oracle.SharedWrite: pkv.SharedWrite,
    oracle.InvalidBlock: pkv.InvalidArgument,
}


def _both(fn_c, fn_o):
    """Run one event on both; return (c_result, o_result) or the matching error classes."""
    rc = ro = None
    ec = eo = None
    try:
        rc = fn_c()
    except pkv.PkvError as e:
        ec = type(e)
    try:
        ro = fn_o()
    except oracle.AllocatorError as e:
        eo = ERRMAP[type(e)]
    return rc, ro, ec, eo


def _books_equal(c, o):
    stack, rc = c.snapshot()
    assert stack == o.free_stack
    assert rc == o.refcount
    assert c.num_free() == o.num_free()
    assert c.check_consistent() == o.check_consistent()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cpp_allocator_equals_oracle_twin_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    nb = 37
    c = pkv.BlockAllocator(nb)
    o = oracle.BlockAllocator(nb)
    live = []      # references we hold (ids, possibly repeated)
    counts = {"exhausted": 0, "double_free": 0, "shared_write": 0, "invalid": 0}
    for step in range(4000):
        r = rng.random()
        if r < 0.35:
            n = int(rng.integers(0, 9))
            rc_, ro_, ec, eo = _both(lambda: c.allocate(n), lambda: o.allocate(n))
            assert ec == eo and rc_ == ro_
            if ec is None:
                live.extend(rc_)
            else:
                counts["exhausted"] += 1
        elif r < 0.5:
            if live and rng.random() < 0.8:
                ids = [live[int(i)] for i in rng.integers(0, len(live), size=int(rng.integers(1, 4)))]
            else:
                ids = [int(i) for i in rng.integers(-2, nb + 2, size=2)]
            _, _, ec, eo = _both(lambda: c.incref(ids), lambda: o.incref(ids))
            assert ec == eo
            if ec is None:
                live.extend(ids)
            else:
                counts["invalid"] += 1
        elif r < 0.8:
            if live and rng.random() < 0.85:
                k = int(rng.integers(1, min(4, len(live)) + 1))
                pick = sorted(rng.choice(len(live), size=k, replace=False).tolist(), reverse=True)
                ids = [live[i] for i in pick]
                if rng.random() < 0.15:
                    ids = ids + ids[:1]               # may be a double free
            else:
                ids = [int(rng.integers(0, nb))]
            _, _, ec, eo = _both(lambda: c.free(ids), lambda: o.free(ids))
            assert ec == eo
            if ec is None:
                for i in ids:
                    live.remove(i)
            elif ec is pkv.DoubleFree:
                counts["double_free"] += 1
        else:
            bs = int(rng.integers(1, 6))
            row = [live[int(i)] for i in rng.integers(0, len(live), size=3)] if live else [0, 1, 2]
            start = int(rng.integers(0, 3 * bs))
            n = int(rng.integers(0, 3 * bs - start + 2))
            rc_, ro_, ec, eo = _both(lambda: c.slots(row, start, n, bs).tolist(),
                                     lambda: o.slots(row, start, n, bs))
            assert ec == eo and (ec is not None or rc_ == ro_)
            if ec is pkv.SharedWrite:
                counts["shared_write"] += 1
        _books_equal(c, o)
    assert min(counts.values()) > 10, counts


def test_fresh_pool_order_and_lifo():
    c = pkv.BlockAllocator(5)
    assert c.allocate(3) == [0, 1, 2]
    c.free([2, 0])
    assert c.allocate(2) == [0, 2]
    assert c.snapshot() == ([4, 3], [1, 1, 1, 0, 0])


def test_exhaustion_is_all_or_nothing():
    c = pkv.BlockAllocator(3)
    c.allocate(2)
    before = c.snapshot()
    with pytest.raises(pkv.PoolExhausted):
        c.allocate(2)
    assert c.snapshot() == before


def test_slot_mapping_refuses_shared_blocks_and_writes_nothing():
    c = pkv.BlockAllocator(6)
    row = c.allocate(3)
    out = c.slots(row, 2, 6, 4)
    assert out.tolist() == [row[0] * 4 + 2, row[0] * 4 + 3] + [row[1] * 4 + i for i in range(4)]
    c.incref([row[1]])
    with pytest.raises(pkv.SharedWrite):
        c.slots(row, 3, 2, 4)
    with pytest.raises(pkv.InvalidArgument):
        c.slots(row, 10, 3, 4)            # past the table
    assert c.slots(row, 8, 4, 4).tolist() == [row[2] * 4 + i for i in range(4)]


def test_validate_slots():
    pkv.validate_slots([0, 5, -1, 7, -1], 8)
    with pytest.raises(pkv.InvalidArgument):
        pkv.validate_slots([0, 5, 5], 8)
    with pytest.raises(pkv.InvalidArgument):
        pkv.validate_slots([0, 8], 8)


def _attn(**kw):
    """Raw pkv_attention call with fake device pointers: only validation may run."""
    lib = pkv.lib()
    a = dict(q=F, k=F, v=F, bt=F, mb=8, ctx=[5, 9], cu=[0, 1, 3], T=3, hq=8, hkv=2, d=128,
             bs=16, nb=4, scale=0.1, split=512, dt=L.PKV_BF16, out=F, ws=F, wsb=1 << 30)
    a.update(kw)
    ctx = np.asarray(a["ctx"], np.int32)
    cu = np.asarray(a["cu"], np.int32)
    return lib.pkv_attention(a["q"], a["k"], a["v"], a["bt"], a["mb"], L._ptr(ctx), L._ptr(cu),
                             ctx.size, a["T"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"],
                             a["scale"], a["split"], a["dt"], a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=6, hkv=4), L.PKV_ERR_INVALID),                 # Hq % Hkv != 0
    (dict(d=96), L.PKV_ERR_UNSUPPORTED),                    # head_dim
    (dict(hq=24, hkv=2), L.PKV_ERR_UNSUPPORTED),            # group 12
    (dict(split=100), L.PKV_ERR_INVALID),                   # split not a multiple of 64
    (dict(split=2112), L.PKV_ERR_INVALID),                  # split above 2048
    (dict(ctx=[5, 1], cu=[0, 1, 3]), L.PKV_ERR_INVALID),    # q_len > ctx
    (dict(cu=[0, 2, 1], T=1), L.PKV_ERR_INVALID),           # cu decreasing
    (dict(cu=[1, 2, 3]), L.PKV_ERR_INVALID),                # cu[0] != 0
    (dict(T=4), L.PKV_ERR_INVALID),                         # cu[B] != T
    (dict(ctx=[5, 200]), L.PKV_ERR_INVALID),                # ctx > max_blocks * block_size
    (dict(wsb=16), L.PKV_ERR_INVALID),                      # workspace too small
    (dict(q=0), L.PKV_ERR_INVALID),                         # NULL q
    (dict(dt=7), L.PKV_ERR_INVALID),                        # dtype
    (dict(scale=float("nan")), L.PKV_ERR_INVALID),
])
def test_attention_validation_refuses_before_any_launch(kw, status):
    assert _attn(**kw) == status
    assert pkv.lib().pkv_last_error() != b""


def test_attention_empty_step_is_a_no_op():
    assert _attn(ctx=[], cu=[0], T=0) == L.PKV_OK
    assert _attn(ctx=[4, 4], cu=[0, 0, 0], T=0) == L.PKV_OK


def test_workspace_size_counts_splits():
    # decode rows: ctx 512 -> 1 split (direct, no partials); ctx 513 -> 2 splits (+ partials)
    a = pkv.attention_workspace_size([512], [0, 1], 8, 2, 128, 512)
    b = pkv.attention_workspace_size([513], [0, 1], 8, 2, 128, 512)
    assert b > a > 0
    # partials: 2 splits x 8 heads x (128 + 2) floats, at least
    assert b - a >= 2 * 8 * 130 * 4
    with pytest.raises(pkv.Unsupported):
        pkv.attention_workspace_size([5], [0, 1], 8, 2, 96, 512)


def test_write_kv_validation():
    lib = pkv.lib()
    assert lib.pkv_write_kv(F, F, F, 4, F, F, 4, 16, 2, 128, 9, None) == L.PKV_ERR_INVALID
    assert lib.pkv_write_kv(F, F, F, -1, F, F, 4, 16, 2, 128, 1, None) == L.PKV_ERR_INVALID
    assert lib.pkv_write_kv(0, F, F, 4, F, F, 4, 16, 2, 128, 1, None) == L.PKV_ERR_INVALID
    assert lib.pkv_write_kv(F, F, F, 0, F, F, 4, 16, 2, 128, 1, None) == L.PKV_OK
    assert lib.pkv_write_kv(F, F, F, 4, F, F, 4, 16, 1, 4, 1, None) == L.PKV_ERR_UNSUPPORTED


def _attn_ex(flags, **kw):
    """Raw pkv_attention_ex call with fake device pointers: only validation may run."""
    lib = pkv.lib()
    a = dict(q=F, k=F, v=F, bt=F, mb=8, ctx=[5, 9], cu=[0, 1, 3], T=3, hq=8, hkv=2, d=128,
             bs=16, nb=4, scale=0.1, split=512, dt=L.PKV_BF16, out=F, ws=F, wsb=16)
    a.update(kw)
    ctx = np.asarray(a["ctx"], np.int32)
    cu = np.asarray(a["cu"], np.int32)
    return lib.pkv_attention_ex(a["q"], a["k"], a["v"], a["bt"], a["mb"], L._ptr(ctx),
                                L._ptr(cu), ctx.size, a["T"], a["hq"], a["hkv"], a["d"], a["bs"],
                                a["nb"], a["scale"], a["split"], a["dt"], flags, a["out"],
                                a["ws"], a["wsb"], None)


def test_phase_consistent_flag_validation():
    # unknown bits and float32 (no MFMA tile path) are refused before any launch
    assert _attn_ex(2) == L.PKV_ERR_INVALID
    assert _attn_ex(L.PKV_ATTN_PHASE_CONSISTENT, dt=L.PKV_F32) == L.PKV_ERR_UNSUPPORTED
    assert _attn_ex(L.PKV_ATTN_PHASE_CONSISTENT, d=96) == L.PKV_ERR_UNSUPPORTED
    # a valid call with a 16-byte workspace fails on the workspace size, i.e. after the flags
    assert _attn_ex(L.PKV_ATTN_PHASE_CONSISTENT) == L.PKV_ERR_INVALID
    assert b"workspace" in pkv.lib().pkv_last_error()
    with pytest.raises(pkv.Unsupported):
        pkv.attention_workspace_size([5], [0, 1], 8, 2, 128, 512, L.PKV_F32,
                                     phase_consistent=True)


def test_phase_consistent_workspace_holds_tile_split_partials():
    # a 4096-key decode row is cut into kv_split splits in both modes: 8 partial slots of
    # 8 heads x (128 + 2) floats at kv_split 512, 2 at 2048, none when one split covers it
    part = 8 * (128 + 2) * 4
    for split, n in [(512, 8), (2048, 2)]:
        normal = pkv.attention_workspace_size([4096], [0, 1], 8, 2, 128, split)
        cons = pkv.attention_workspace_size([4096], [0, 1], 8, 2, 128, split, phase_consistent=True)
        assert n * part <= normal < n * part + 4096
        assert n * part <= cons < n * part + 4096
    assert 0 < pkv.attention_workspace_size([2048], [0, 1], 8, 2, 128, 2048,
                                            phase_consistent=True) < 1024
    # a prefill segment: partial slots for every row times the segment's splits
    cons = pkv.attention_workspace_size([1100], [0, 100], 8, 2, 128, 512, phase_consistent=True)
    assert 100 * 3 * part <= cons < 100 * 3 * part + 8192


def test_kv_split_beyond_2048_only_in_the_consistent_mode():
    with pytest.raises(pkv.InvalidArgument):
        pkv.attention_workspace_size([5000], [0, 1], 8, 2, 128, 4096)
    assert pkv.attention_workspace_size([5000], [0, 1], 8, 2, 128, 4096,
                                        phase_consistent=True) > 2 * 8 * 130 * 4
    # one split longer than every context: no partials
    assert pkv.attention_workspace_size([5000], [0, 1], 8, 2, 128, 1 << 20,
                                        phase_consistent=True) < 1024
    with pytest.raises(pkv.InvalidArgument):
        pkv.attention_workspace_size([5000], [0, 1], 8, 2, 128, 4100, phase_consistent=True)


def test_consistent_workspace_sums_the_segments():
    # partials of a multi-segment step: per segment, q_len rows x ceil(ctx / kv_split) slots
    # when ctx > kv_split, none otherwise; decode rows count as 1-row segments
    hq, hkv, d, split = 8, 2, 128, 256
    ctx = [1000, 300, 256, 5000, 40]
    ql = [100, 1, 1, 1, 40]
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    slots = sum(q * -(-c // split) for c, q in zip(ctx, ql) if c > split)
    got = pkv.attention_workspace_size(ctx, cu, hq, hkv, d, split, phase_consistent=True)
    part = slots * hq * (d + 2) * 4
    assert part <= got < part + 64 * 1024


def _fused(**kw):
    """Raw pkv_write_kv_attention call with fake device pointers: only validation may run."""
    lib = pkv.lib()
    a = dict(q=F, kn=F, vn=F, slots=[3, -1, 60], n=3, k=F, v=F, bt=F, mb=8, ctx=[5, 9],
             cu=[0, 1, 3], T=3, hq=8, hkv=2, d=128, bs=16, nb=4, scale=0.1, split=512,
             dt=L.PKV_BF16, flags=0, out=F, ws=F, wsb=1 << 30)
    a.update(kw)
    ctx = np.asarray(a["ctx"], np.int32)
    cu = np.asarray(a["cu"], np.int32)
    sl = np.asarray(a["slots"] if a["slots"] is not None else [0], np.int32)
    sp = L._ptr(sl) if a["slots"] is not None else None
    return lib.pkv_write_kv_attention(a["q"], a["kn"], a["vn"], sp, a["n"], a["k"], a["v"],
                                      a["bt"], a["mb"], L._ptr(ctx), L._ptr(cu), ctx.size,
                                      a["T"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"],
                                      a["scale"], a["split"], a["dt"], a["flags"], a["out"],
                                      a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(slots=[3, -1, 64]), L.PKV_ERR_INVALID),           # slot == num_blocks * block_size
    (dict(slots=[3, -1, 3]), L.PKV_ERR_INVALID),            # one slot twice
    (dict(slots=[60, 2, 60]), L.PKV_ERR_INVALID),
    (dict(n=-1), L.PKV_ERR_INVALID),                        # negative row count
    (dict(slots=None), L.PKV_ERR_INVALID),                  # NULL host slots
    (dict(kn=0), L.PKV_ERR_INVALID),                        # NULL k_new
    (dict(dt=5), L.PKV_ERR_INVALID),                        # dtype
    (dict(hkv=1, hq=4, d=4, dt=L.PKV_BF16), L.PKV_ERR_UNSUPPORTED),  # 8-byte rows
    (dict(hq=6, hkv=4), L.PKV_ERR_INVALID),                 # attention part still validated
    (dict(T=4), L.PKV_ERR_INVALID),
    (dict(wsb=16), L.PKV_ERR_INVALID),                      # workspace too small
    (dict(flags=2), L.PKV_ERR_INVALID),
])
def test_fused_step_validation_refuses_before_any_copy(kw, status):
    assert _fused(**kw) == status
    assert pkv.lib().pkv_last_error() != b""


def test_fused_step_workspace_holds_the_slots():
    a = pkv.attention_workspace_size([513, 40], [0, 1, 2], 8, 2, 128, 512)
    b = pkv.write_kv_attention_workspace_size([513, 40], [0, 1, 2], 8, 2, 128, 1000, 512)
    assert b >= a + 4 * 1000
    assert pkv.write_kv_attention_workspace_size([513, 40], [0, 1, 2], 8, 2, 128, 0, 512) == a
    # a pure append (no sequences) still needs room for its slots
    assert pkv.write_kv_attention_workspace_size([], [0], 8, 2, 128, 10, 512) >= 40
    with pytest.raises(pkv.InvalidArgument):
        pkv.write_kv_attention_workspace_size([5], [0, 1], 8, 2, 128, -1, 512)


def test_profile_kind_mask_validation():
    assert pkv.lib().pkv_profile_set_kinds(0x20) == L.PKV_ERR_INVALID
    assert pkv.lib().pkv_profile_set_kinds(0x1F) == L.PKV_OK
    pkv.profile_set_kinds(["decode"])
    pkv.profile_set_kinds(["write_kv", "prefill", "decode", "merge"])


def test_copy_blocks_validation():
    lib = pkv.lib()
    pairs = np.asarray([1, 2, 3, 4], np.int32)
    call = lambda pr, n=2, nb=8, dt=L.PKV_BF16, wsb=256: lib.pkv_copy_blocks(
        F, F, L._ptr(np.asarray(pr, np.int32)), n, nb, 16, 2, 128, dt, F, wsb, None)
    assert call([1, 2, 3, 8]) == L.PKV_ERR_INVALID          # id outside the pool
    assert call([1, 2, 3, 2]) == L.PKV_ERR_INVALID          # destination twice
    assert call([1, 2, 2, 4]) == L.PKV_ERR_INVALID          # destination is also a source
    assert call([1, 2, 3, 4], wsb=8) == L.PKV_ERR_INVALID   # workspace too small
    assert call([1, 2, 3, 4], dt=3) == L.PKV_ERR_INVALID
    assert call([1, 2], n=0) == L.PKV_OK                    # nothing to copy
    assert lib.pkv_copy_blocks(F, F, L._ptr(pairs), 1, 8, 1, 1, 4, L.PKV_BF16, F, 256,
                               None) == L.PKV_ERR_UNSUPPORTED   # 8-byte blocks
    # E4M3 pools: one-byte elements (a 4-code block is too small; a 16-code block passes the
    # type and size checks and stops at the 8-byte workspace)
    assert lib.pkv_copy_blocks(F, F, L._ptr(pairs), 1, 8, 1, 1, 4, L.PKV_E4M3, F, 256,
                               None) == L.PKV_ERR_UNSUPPORTED
    assert lib.pkv_copy_blocks(F, F, L._ptr(pairs), 1, 8, 1, 1, 16, L.PKV_E4M3, F, 4,
                               None) == L.PKV_ERR_INVALID
    assert b"workspace" in lib.pkv_last_error()
    # the other entry points do not take PKV_E4M3
    assert lib.pkv_write_kv(F, F, F, 4, F, F, 4, 16, 2, 128, L.PKV_E4M3, None) == L.PKV_ERR_INVALID


def test_write_kv_fp8_validation():
    lib = pkv.lib()
    call = lambda n=4, hkv=2, d=128, ks=0.5, vs=0.5, k=F: lib.pkv_write_kv_fp8(
        k, F, F, n, F, F, 4, 16, hkv, d, ks, vs, None)
    assert call(n=0) == L.PKV_OK                               # nothing to write
    assert call(n=-1) == L.PKV_ERR_INVALID
    assert call(k=0) == L.PKV_ERR_INVALID                      # NULL k_new
    assert call(ks=0.0) == L.PKV_ERR_INVALID
    assert call(vs=-1.0) == L.PKV_ERR_INVALID
    assert call(ks=float("inf")) == L.PKV_ERR_INVALID
    assert call(vs=float("nan")) == L.PKV_ERR_INVALID
    assert call(hkv=1, d=8) == L.PKV_ERR_UNSUPPORTED           # 8-byte pool rows
    assert pkv.lib().pkv_last_error() != b""


def _attn_fp8(**kw):
    """Raw pkv_attention_fp8 call with fake device pointers: only validation may run."""
    lib = pkv.lib()
    a = dict(q=F, k=F, v=F, bt=F, mb=8, ctx=[5, 9], cu=[0, 1, 3], T=3, hq=8, hkv=2, d=128,
             bs=16, nb=4, scale=0.1, ks=0.5, vs=0.5, split=512, flags=0, out=F, ws=F, wsb=16)
    a.update(kw)
    ctx = np.asarray(a["ctx"], np.int32)
    cu = np.asarray(a["cu"], np.int32)
    return lib.pkv_attention_fp8(a["q"], a["k"], a["v"], a["bt"], a["mb"], L._ptr(ctx),
                                 L._ptr(cu), ctx.size, a["T"], a["hq"], a["hkv"], a["d"],
                                 a["bs"], a["nb"], a["scale"], a["ks"], a["vs"], a["split"],
                                 a["flags"], a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=32, hkv=2), L.PKV_ERR_UNSUPPORTED),            # group 16 has no instance
    (dict(d=96), L.PKV_ERR_UNSUPPORTED),
    (dict(ks=0.0), L.PKV_ERR_INVALID),
    (dict(vs=float("nan")), L.PKV_ERR_INVALID),
    (dict(ks=float("inf")), L.PKV_ERR_INVALID),
    (dict(split=100), L.PKV_ERR_INVALID),
    (dict(ctx=[5, 1]), L.PKV_ERR_INVALID),                  # q_len > ctx
    (dict(flags=2), L.PKV_ERR_INVALID),                     # unknown flag bits
])
def test_attention_fp8_validation_refuses_before_any_launch(kw, status):
    assert _attn_fp8(**kw) == status
    assert pkv.lib().pkv_last_error() != b""


def test_attention_fp8_reaches_the_workspace_check_and_routes_rows_as_bf16():
    assert _attn_fp8() == L.PKV_ERR_INVALID                 # 16-byte workspace
    assert b"workspace" in pkv.lib().pkv_last_error()
    assert _attn_fp8(flags=L.PKV_ATTN_PHASE_CONSISTENT) == L.PKV_ERR_INVALID
    assert b"workspace" in pkv.lib().pkv_last_error()
    assert _attn_fp8(ctx=[], cu=[0], T=0) == L.PKV_OK
    # the same work lists as bfloat16 pools: a prefill chunk on tiles, decode rows split
    for ctx, cu in (([2000], [0, 300]), ([2000, 700], [0, 1, 2])):
        for pc in (False, True):
            f8 = pkv.attention_fp8_workspace_size(ctx, cu, 8, 2, 128, 512, pc)
            bf = pkv.attention_workspace_size(ctx, cu, 8, 2, 128, 512, phase_consistent=pc)
            assert f8 == bf
    with pytest.raises(pkv.Unsupported):
        pkv.attention_fp8_workspace_size([5], [0, 1], 32, 2, 128, 512)


def test_misaligned_device_pointers_are_refused():
    assert _attn(q=F + 2) == L.PKV_ERR_INVALID
    assert b"aligned" in pkv.lib().pkv_last_error()
    assert _attn(ws=F + 8) == L.PKV_ERR_INVALID
    assert _attn(out=F + 2) == L.PKV_ERR_INVALID
    lib = pkv.lib()
    assert lib.pkv_write_kv(F + 4, F, F, 4, F, F, 4, 16, 2, 128, 1, None) == L.PKV_ERR_INVALID
    assert b"aligned" in pkv.lib().pkv_last_error()
    assert lib.pkv_write_kv_fp8(F, F, F, 4, F + 8, F, 4, 16, 2, 128, 0.5, 0.5,
                                None) == L.PKV_ERR_INVALID
    assert b"aligned" in pkv.lib().pkv_last_error()


def test_fused_fp8_step_validation():
    lib = pkv.lib()
    ctx = np.asarray([5, 9], np.int32)
    cu = np.asarray([0, 1, 3], np.int32)

    def call(slots=(3, -1, 60), ks=0.5, hq=8, wsb=1 << 30, flags=0):
        sl = np.asarray(slots, np.int32)
        return lib.pkv_write_kv_attention_fp8(F, F, F, L._ptr(sl), sl.size, F, F, F, 8,
                                              L._ptr(ctx), L._ptr(cu), 2, 3, hq, 2, 128, 16, 4,
                                              0.1, ks, 0.5, 512, flags, F, F, wsb, None)
    assert call(slots=(3, -1, 64)) == L.PKV_ERR_INVALID       # slot outside the pool
    assert b"outside" in pkv.lib().pkv_last_error()
    assert call(slots=(7, 7, -1)) == L.PKV_ERR_INVALID        # one slot twice
    assert b"twice" in pkv.lib().pkv_last_error()
    assert call(ks=-1.0) == L.PKV_ERR_INVALID
    assert call(hq=32) == L.PKV_ERR_UNSUPPORTED
    assert call(wsb=16) == L.PKV_ERR_INVALID
    assert b"workspace" in pkv.lib().pkv_last_error()
    assert call(flags=4) == L.PKV_ERR_INVALID
    a = pkv.attention_fp8_workspace_size([5, 9], [0, 1, 3], 8, 2, 128, 512)
    b = pkv.write_kv_attention_fp8_workspace_size([5, 9], [0, 1, 3], 8, 2, 128, 1000, 512)
    assert b >= a + 4 * 1000


def test_fused_step_refuses_duplicate_slots_on_both_check_paths():
    """Duplicates are found whether the slots' range is dense (bitmap) or sparse (sorted copy);
    negative slots may repeat (padding)."""
    big = 1 << 20
    assert _fused(slots=[5, 1, 5], nb=big // 16) == L.PKV_ERR_INVALID
    assert b"appears twice" in pkv.lib().pkv_last_error()
    assert _fused(slots=[0, big - 1, 0], nb=big // 16) == L.PKV_ERR_INVALID
    assert b"appears twice" in pkv.lib().pkv_last_error()
    # distinct slots and repeated padding pass the slot check (then stop at the workspace)
    assert _fused(slots=[0, -1, -1], n=3, wsb=16) == L.PKV_ERR_INVALID
    assert b"workspace" in pkv.lib().pkv_last_error()
