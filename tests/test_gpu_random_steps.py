"""Seeded random ragged steps on the GPU against the oracle, through the C ABI.

Each case draws its shape: group size, kv heads, head_dim, block size, KV split, pool element
type (bf16, float32, or E4M3 codes), and a batch that mixes decode rows with chunked-prefill
segments of ragged lengths over ragged prior contexts. The bars are those of the other parity
tests: attention within max abs error 2e-3 (bf16 inputs) or 1e-5 (float32) of the float64
oracle, in the default mode and (bf16 and E4M3 pools) the phase-consistent mode, and every
sequence run alone bitwise equal to its rows in the batch. The draws cover what fixed cases
rarely combine: segments whose rows start inside a 64-key tile, waves of a prefill item that
hold only padding rows, splits that end inside a tile, blocks of 1 and 3 keys. A second, smaller
set draws contexts of up to 6000 keys, chunks of up to 300 rows and splits of up to 2048 keys, so
that rows span many splits; a third set does the same in the phase-consistent mode alone at
splits of 4096 and 8192 keys (beyond the default mode's limit of 2048).
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from oracle import build_oracle_step
from workloads import explicit_spec, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
DEV = "cuda:0"
N_CASES = 144
N_LONG = 24    # contexts to 6000 keys and chunks to 300 rows: many splits per row
N_PC = 12      # the same, phase-consistent mode only, at splits beyond the default mode's 2048
SEED_BASE = {"short": 20260000, "long": 20270000, "pc": 20280000}


def _draw(i, set_="short"):
    long = set_ != "short"
    rng = np.random.default_rng(SEED_BASE[set_] + i)
    group = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2])) if group < 8 else 1
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([1, 3, 8, 16, 32, 64]))
    kind = ("fp8", "bf16" if set_ == "pc" else "f32", "bf16", "bf16")[i % 4]
    kv_split = int(rng.choice([4096, 8192] if set_ == "pc" else
                              [64, 512, 1024, 2048] if long else [64, 128, 512, 1024]))
    seqs = []
    for _ in range(int(rng.integers(1, 6))):
        q = 1 if rng.random() < 0.4 else int(rng.integers(2, 300 if long else 140))
        prior = int(rng.integers(0, 6000 if long else 600))
        seqs.append((prior + q, q))
    kw = {"kv_split": kv_split}
    if kind == "fp8":
        kw.update(kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 64)
    dtype = "f32" if kind == "f32" else "bf16"
    name = f"random-{set_}-{i}-{kind}-G{group}-Hkv{hkv}-D{d}-BS{bs}-S{kv_split}"
    return explicit_spec(name, dtype, group * hkv, hkv, d, bs, seqs, **kw), kind


def _alone(gst, w, b, phase_consistent):
    lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
    q = gst.q[lo:hi].contiguous()
    bt = gst.block_tables_dev[b:b + 1].contiguous()
    ctx, cu = [int(w.ctx_lens[b])], [0, hi - lo]
    if w.kv_fp8:
        out = pkv.attention_fp8(q, gst.k_cache, gst.v_cache, bt, ctx, cu, w.scale,
                                w.spec.k_scale, w.spec.v_scale, kv_split=w.spec.kv_split,
                                phase_consistent=phase_consistent)
    else:
        out = pkv.attention(q, gst.k_cache, gst.v_cache, bt, ctx, cu, w.scale,
                            kv_split=w.spec.kv_split, phase_consistent=phase_consistent)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("i", [(i, "short") for i in range(N_CASES)] +
                         [(i, "long") for i in range(N_LONG)] + [(i, "pc") for i in range(N_PC)],
                         ids=lambda x: f"{x[1]}-{x[0]}")
def test_random_step_matches_oracle_and_is_batch_invariant(i):
    from prefill_slot_mapping_amd.harness import build_gpu_step
    spec, kind = _draw(*i)
    w = make_workload(spec)
    print(f"[random] {spec.name} seqs={list(zip(w.ctx_lens.tolist(), w.q_lens.tolist()))}",
          flush=True)
    gst = build_gpu_step(w, device=DEV)
    ref = build_oracle_step(w).attention()
    modes = [True] if i[1] == "pc" else [False] if kind == "f32" else [False, True]
    for pc in modes:
        out = gst.attention(phase_consistent=pc).cpu().numpy().copy()
        torch.cuda.synchronize()
        got = out.astype(np.float64)
        assert np.isfinite(got).all()
        err = float(np.abs(got - ref).max())
        print(f"[random] {spec.name} phase_consistent={pc} max abs err {err:.3e}", flush=True)
        assert err <= TOL[spec.dtype]
        for b in range(w.B):
            lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
            assert np.array_equal(_alone(gst, w, b, pc), out[lo:hi]), f"sequence {b}, pc={pc}"
