"""A large mixed step runs its decode pass on the library's second stream, beside the prefill
pass (it forks when the prefill grid has more than 512 workgroups and the decode grid at least
1024; its prefill pass is then two launches, one round of the longest items at one workgroup
per compute unit first, with bf16 and with E4M3 pools). Its rows must be bitwise those the same rows get from
steps that do not fork (the prefill segments alone, one launch; the decode rows alone), and
work enqueued on the caller's stream after the call must see the finished output (the join
back to that stream).
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from workloads import ALL_CONFIGS, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
M_ROWS = 128   # prefill tile rows (query rows x heads of one kv head)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def _grids(w):
    """Workgroups of the prefill and decode launches of step w."""
    s = w.spec
    rows = M_ROWS // (s.Hq // s.Hkv)
    n_pre = n_dec = 0
    for b in range(w.B):
        ql = int(w.cu_seqlens_q[b + 1] - w.cu_seqlens_q[b])
        if ql > 1:
            n_pre += -(-ql // rows)
        elif ql == 1:
            n_dec += -(-int(w.ctx_lens[b]) // s.kv_split)
    return n_pre * s.Hkv, n_dec * s.Hkv


def _sub_step(gst, w, seqs):
    """The sequences `seqs` as a step of their own: their q rows, table rows and lengths."""
    cu = w.cu_seqlens_q
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in seqs])
    lens = [int(cu[b + 1] - cu[b]) for b in seqs]
    sub_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    idx = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    q = gst.q.index_select(0, idx).contiguous()
    bt = gst.block_tables_dev[torch.as_tensor(seqs, device=DEV)].contiguous()
    ctx = np.asarray([w.ctx_lens[b] for b in seqs], dtype=np.int32)
    s = w.spec
    if w.kv_fp8:
        out = pkv.attention_fp8(q, gst.k_cache, gst.v_cache, bt, ctx, sub_cu, w.scale,
                                s.k_scale, s.v_scale, kv_split=s.kv_split)
    else:
        out = pkv.attention(q, gst.k_cache, gst.v_cache, bt, ctx, sub_cu, w.scale,
                            kv_split=s.kv_split)
    return rows, out


@pytest.mark.parametrize("name", ["mixed-ragged-step", "mixed-fp8-step"])
def test_forked_step_equals_unforked_parts_bitwise(name):
    from prefill_slot_mapping_amd.harness import build_gpu_step
    w = make_workload(ALL_CONFIGS[name])
    pre_wgs, dec_wgs = _grids(w)
    print(f"[overlap] {name} B={w.B} T={w.T} prefill wgs {pre_wgs} decode wgs {dec_wgs}",
          flush=True)
    assert pre_wgs > 512 and dec_wgs >= 1024      # the step forks
    gst = build_gpu_step(w, device=DEV)
    full = _bits(gst.attention())
    ql = np.diff(w.cu_seqlens_q)
    pre = [b for b in range(w.B) if ql[b] > 1]
    dec = [b for b in range(w.B) if ql[b] == 1]
    for part in (pre, dec):
        rows, out = _sub_step(gst, w, part)
        torch.cuda.synchronize()
        assert np.array_equal(full[rows], _bits(out))


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "write_kv_attention"])
def test_caller_stream_waits_for_the_decode_pass(fused):
    from prefill_slot_mapping_amd.harness import build_gpu_step
    w = make_workload(ALL_CONFIGS["mixed-ragged-step"])
    gst = build_gpu_step(w, device=DEV, write_new=not fused)
    ref = gst.fused_step() if fused else gst.attention()
    torch.cuda.synchronize()
    ref = _bits(ref)
    side = torch.cuda.Stream(device=DEV)
    for rep in range(3):
        with torch.cuda.stream(side):
            gst.out.fill_(float("nan"))
            out = gst.fused_step(stream=side) if fused else gst.attention(stream=side)
            snap = out.clone()     # enqueued right behind the call on the caller's stream
        side.synchronize()
        print(f"[overlap] fused={fused} repeat {rep}", flush=True)
        assert np.array_equal(_bits(snap), ref)


def test_forked_steps_from_two_threads():
    """Two host threads run forked mixed steps on streams of their own: the library's lock
    around the fork and the join and its staging ring keep every result whole."""
    import threading
    from prefill_slot_mapping_amd.harness import build_gpu_step
    w = make_workload(ALL_CONFIGS["mixed-ragged-step"])
    steps = [build_gpu_step(w, device=DEV) for _ in range(2)]
    refs = []
    for gst in steps:
        refs.append(_bits(gst.attention()))
        torch.cuda.synchronize()
    errors = []

    def run(i):
        try:
            gst = steps[i]
            s = torch.cuda.Stream(device=DEV)
            for rep in range(4):
                with torch.cuda.stream(s):
                    gst.out.fill_(float("nan"))
                    snap = gst.attention(stream=s).clone()
                s.synchronize()
                if not np.array_equal(_bits(snap), refs[i]):
                    errors.append(f"thread {i} repeat {rep}")
        except Exception as e:   # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    print(f"[overlap] two threads: {errors or 'ok'}", flush=True)
    assert not any(t.is_alive() for t in threads) and not errors, errors
