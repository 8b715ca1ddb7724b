"""The seeded synthetic steps have the shapes and structure their recipes state."""
import numpy as np

from workloads import CONFIGS, DIAGNOSTIC_CONFIGS, SMALL_CONFIGS, make_workload, stable_seed


def test_seeds_are_stable_and_distinct():
    assert stable_seed("pkv-config-a") == stable_seed("pkv-config-a")
    assert stable_seed("pkv-config-a") != stable_seed("pkv-config-b")
    w1 = make_workload(SMALL_CONFIGS["batched-bf16-decode"])
    w2 = make_workload(SMALL_CONFIGS["batched-bf16-decode"])
    assert np.array_equal(w1.ctx_lens, w2.ctx_lens) and np.array_equal(w1.q, w2.q)
    assert np.array_equal(w1.kv(3)[0], w2.kv(3)[0])


def test_tiny_f32_decode_shape():
    w = make_workload(CONFIGS["tiny-f32-decode"])
    assert list(w.ctx_lens) == [17, 33, 64, 100] and w.num_blocks == 64
    assert w.T == 4 and w.spec.dtype == "f32" and w.q.dtype == np.float32
    assert sorted(w.free_order) == list(range(64))
    assert w.scale == 1.0 / 8.0


def test_batched_decode_lengths_are_clipped_lognormal():
    w = make_workload(CONFIGS["batched-bf16-decode"])
    assert w.B == 64 and w.T == 64
    assert w.ctx_lens.min() >= 16 and w.ctx_lens.max() <= 16384
    needed = int(((w.ctx_lens + 15) // 16).sum())
    assert w.num_blocks == int(np.ceil(1.2 * needed))
    assert 1000 < np.median(w.ctx_lens) < 4000


def test_mixed_step_is_one_flat_ragged_batch():
    w = make_workload(CONFIGS["mixed-ragged-step"])
    assert w.T == 8 * 512 + 120 and w.B == 128
    assert sorted(set(w.q_lens.tolist())) == [1, 512]
    pre = w.q_lens == 512
    assert (w.ctx_lens[pre] - 512).min() >= 0 and (w.ctx_lens[pre] - 512).max() <= 8192
    # prefill segments are interleaved with decodes
    first = np.flatnonzero(pre)
    assert first.max() - first.min() > 8


def test_long_context_decode():
    w = make_workload(CONFIGS["long-context-decode"])
    assert list(w.ctx_lens) == [40960] * 8 and w.spec.BS == 32 and w.spec.G == 8


def test_prefix_shared_groups():
    w = make_workload(CONFIGS["prefix-shared-decode"])
    assert w.B == 128
    sharers = [a for a in w.admissions if a.share_from >= 0]
    assert len(sharers) == 16 * 7 and all(a.n_shared_blocks == 128 for a in sharers)
    assert ((w.ctx_lens - 2048) >= 1).all() and ((w.ctx_lens - 2048) <= 4096).all()


def test_outliers_scale_about_one_percent_of_k_rows():
    w = make_workload(SMALL_CONFIGS["long-context-decode"])
    k, v = w.kv(0)
    from oracle import bf16_bits_to_f64
    rows = np.abs(bf16_bits_to_f64(k)).max(axis=-1)     # [ctx, Hkv]
    frac = (rows > 6.0).mean()
    assert 0.002 < frac < 0.03


def test_prefill_rows_workload_is_the_mixed_steps_segments():
    w = make_workload(CONFIGS["mixed-ragged-step"])
    pre = w.q_lens > 1
    d = make_workload(DIAGNOSTIC_CONFIGS["mixed-step-prefill-rows"])
    assert (d.q_lens > 1).all()
    assert sorted(zip(d.ctx_lens.tolist(), d.q_lens.tolist())) == \
        sorted(zip(w.ctx_lens[pre].tolist(), w.q_lens[pre].tolist()))
