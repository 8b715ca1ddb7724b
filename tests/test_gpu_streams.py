"""The Python binding's temporaries follow the stream the library enqueues on.

With ``stream=s`` the wrappers make their device copy of host slots, the workspace and the
output inside ``torch.cuda.stream(s)``: the copy runs before the kernel that reads it, and the
caching allocator reuses that memory only for work ordered after ours on ``s``. Here ``s`` is
held busy by a bounded sleep kernel while the caller's current stream allocates and overwrites
memory right after each call; the results must still be those of the plain calls.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from workloads import SMALL_CONFIGS, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SLEEP_CYCLES = 20_000_000   # ~10 ms of a spinning kernel: long enough to reorder, bounded


def _churn():
    """Allocate and overwrite memory on the current stream, as a caller would next."""
    for _ in range(8):
        junk = torch.empty(1 << 20, dtype=torch.int32, device=DEV)
        junk.fill_(-7)
        del junk


def test_write_kv_with_host_slots_on_a_busy_side_stream():
    nb, bs, hkv, d = 64, 16, 2, 64
    g = torch.Generator(device="cpu").manual_seed(3)
    kn = torch.randn((40, hkv, d), generator=g).to(torch.bfloat16).to(DEV)
    vn = torch.randn((40, hkv, d), generator=g).to(torch.bfloat16).to(DEV)
    slots = np.random.default_rng(5).permutation(nb * bs)[:40].astype(np.int32)
    ref_k = torch.zeros((nb, bs, hkv, d), dtype=torch.bfloat16, device=DEV)
    ref_v = torch.zeros_like(ref_k)
    pkv.write_kv(kn, vn, slots, ref_k, ref_v)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=DEV)
    kc = torch.zeros_like(ref_k)
    vc = torch.zeros_like(ref_v)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SLEEP_CYCLES)
    pkv.write_kv(kn, vn, slots, kc, vc, stream=s)
    _churn()
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), ref_k.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), ref_v.view(torch.int16))


@pytest.mark.parametrize("fused", [False, True])
def test_attention_temporaries_on_a_busy_side_stream(fused):
    from prefill_slot_mapping_amd.harness import build_gpu_step
    w = make_workload(SMALL_CONFIGS["mixed-ragged-step"])
    gst = build_gpu_step(w, device=DEV)
    ref = gst.attention().detach().clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(s):
        torch.cuda._sleep(SLEEP_CYCLES)
    if fused:
        # the step's append again (same rows into the same slots: the pools do not change)
        out = pkv.write_kv_attention(gst.q, gst.k_new, gst.v_new, gst.new_slots, gst.k_cache,
                                     gst.v_cache, gst.block_tables_dev, w.ctx_lens,
                                     w.cu_seqlens_q, w.scale, stream=s)
    else:
        out = pkv.attention(gst.q, gst.k_cache, gst.v_cache, gst.block_tables_dev, w.ctx_lens,
                            w.cu_seqlens_q, w.scale, stream=s)
    _churn()
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
