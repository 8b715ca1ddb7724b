"""GPU: the fused step (pkv_write_kv_attention: KV append through host slots + attention in one
call; one launch copies the staged work lists and appends the rows, reading the slots from the
pinned staging buffer in place) equals pkv_write_kv followed by pkv_attention bit for bit, on
the pools and on the output; repeated calls cycle the library's pinned staging ring (and its
fences) without changing a bit, on one stream and alternating between two, and with different
steps alternating while the GPU lags far behind the host.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from oracle import build_oracle_step
from workloads import SMALL_CONFIGS, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 2e-3, "f32": 1e-5}


def _bits(t):
    a = t.detach().cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy()
    return a.view(torch.int32).numpy()


def _pair(w):
    from prefill_slot_mapping_amd.harness import build_gpu_step
    a = build_gpu_step(w, device=DEV, write_new=False)
    b = build_gpu_step(w, device=DEV, write_new=False)
    return a, b


@pytest.mark.parametrize("name", ["mixed-ragged-step", "batched-bf16-decode", "tiny-f32-decode",
                                  "prefix-shared-decode", "long-context-decode"])
def test_fused_step_equals_separate_calls_bitwise(name):
    w = make_workload(SMALL_CONFIGS[name])
    print(f"[fused] {name} B={w.B} T={w.T}", flush=True)
    a, b = _pair(w)
    a.write_new()
    ref = a.attention().clone()
    got = b.fused_step().clone()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a.k_cache), _bits(b.k_cache))
    assert np.array_equal(_bits(a.v_cache), _bits(b.v_cache))
    assert np.array_equal(_bits(ref), _bits(got))
    # and the fused result is the oracle's
    o = build_oracle_step(w).attention()
    err = float(np.abs(got.cpu().numpy().astype(np.float64) - o).max())
    assert err <= TOL[w.spec.dtype], err


def test_repeated_fused_steps_cycle_the_staging_ring():
    w = make_workload(SMALL_CONFIGS["mixed-ragged-step"])
    a, _ = _pair(w)
    first = _bits(a.fused_step().clone())
    s2 = torch.cuda.Stream(device=DEV)
    outs = []
    for i in range(40):
        stream = s2 if (i // 3) % 2 else None    # runs of three calls per stream
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                o = a.fused_step(stream=stream).clone()
            torch.cuda.current_stream().wait_stream(stream)
        else:
            o = a.fused_step().clone()
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(_bits(o), first)


def test_ring_wraps_while_the_gpu_lags_with_different_steps_alternating():
    """A long matmul holds the GPU while the host enqueues 40 fused steps of two different
    workloads in turn: the 16-slot staging ring wraps before the first step has run, so the
    host must wait for the fences before rewriting a slot the device still reads."""
    from prefill_slot_mapping_amd.harness import build_gpu_step
    steps = [build_gpu_step(make_workload(SMALL_CONFIGS[n]), device=DEV)
             for n in ("mixed-ragged-step", "batched-bf16-decode")]
    refs = [_bits(st.fused_step().clone()) for st in steps]
    big = torch.randn((8192, 8192), device=DEV)
    prod = torch.empty_like(big)
    torch.cuda.synchronize()
    for _ in range(4):
        torch.mm(big, big, out=prod)          # tens of milliseconds of GPU work
    outs = [(i % 2, steps[i % 2].fused_step().clone()) for i in range(40)]
    torch.cuda.synchronize()
    for k, o in outs:
        assert np.array_equal(_bits(o), refs[k])


def test_fused_step_without_rows_or_sequences():
    w = make_workload(SMALL_CONFIGS["batched-bf16-decode"])
    a, b = _pair(w)
    a.write_new()
    b.write_new()
    ref = a.attention().clone()
    # no append rows: the plain attention call
    empty = torch.empty((0, w.spec.Hkv, w.spec.D), dtype=a.k_new.dtype, device=DEV)
    got = pkv.write_kv_attention(b.q, empty, empty, np.zeros(0, np.int32), b.k_cache, b.v_cache,
                                 b.block_tables_dev, w.ctx_lens, w.cu_seqlens_q, w.scale,
                                 kv_split=w.spec.kv_split)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ref), _bits(got))
    # no sequences: the plain append (into a third step whose new rows are not written yet)
    c, _ = _pair(w)
    q0 = torch.empty((0, w.spec.Hq, w.spec.D), dtype=c.q.dtype, device=DEV)
    bt0 = torch.empty((0, 1), dtype=torch.int32, device=DEV)
    pkv.write_kv_attention(q0, c.k_new, c.v_new, c.new_slots, c.k_cache, c.v_cache, bt0, [], [0],
                           w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a.k_cache), _bits(c.k_cache))
    assert np.array_equal(_bits(a.v_cache), _bits(c.v_cache))
