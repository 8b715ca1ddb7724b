"""Pins of the oracle's write / gather / attention against things other than itself.

* torch's float64 scaled_dot_product_attention on contiguous K/V with an explicit boolean
  mask (a library routine independent of the oracle's per-row loop);
* closed forms: one key, zero query, constant values, a row at position 0, a dominant key;
* flat-index semantics of a slot (numpy's own reshape of the pool);
* storage equivalence: a paged layout gives bitwise the same result as a contiguous cache and
  as any permutation of the physical blocks ("Optional paged KV cache (vLLM-style) — v1
  design", section "Motivation": tolerance 0 for a storage-layout change);
* re-chunking and batch-composition invariance ("P3: native paged-KV continuous-batching
  sampler", section "Evidence", batch invariance);
* planted mistakes (the kernel-relevant mutants of the P3 page's "Evidence" list) that these
  pins must catch.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import paged as P
from oracle import allocator as A
from oracle import build_oracle_step, attend_rows, gather, write_kv, paged_attention
from workloads import explicit_spec, make_workload, SMALL_CONFIGS, round_f32_to_bf16_bits

pytestmark = []


def to64(x):
    return P.bf16_bits_to_f64(x) if x.dtype == np.uint16 else np.asarray(x, np.float64)


def sdpa_rows(q_rows, k_seq, v_seq, positions, scale):
    """torch float64 SDPA, contiguous K/V, explicit [n, L] causal mask, GQA by repeat."""
    q = torch.from_numpy(to64(q_rows))            # [n, Hq, D]
    k = torch.from_numpy(to64(k_seq))             # [Hkv, L, D]
    v = torch.from_numpy(to64(v_seq))
    hq, hkv = q.shape[1], k.shape[0]
    k = k.repeat_interleave(hq // hkv, dim=0)     # [Hq, L, D]
    v = v.repeat_interleave(hq // hkv, dim=0)
    L = k.shape[1]
    mask = torch.arange(L)[None, :] <= torch.tensor(list(positions))[:, None]
    out = F.scaled_dot_product_attention(q.permute(1, 0, 2), k, v, attn_mask=mask,
                                         scale=scale)
    return out.permute(1, 0, 2).numpy()


def step_vs_sdpa(w, st):
    """Max |oracle - SDPA| over every row of the step (SDPA on the generator's own K/V)."""
    out = st.attention()
    worst = 0.0
    for b in range(w.B):
        ql = int(w.q_lens[b])
        if ql == 0:
            continue
        kk, vv = w.kv(b)                                  # [ctx, Hkv, D] from the generator
        ks = np.ascontiguousarray(kk.transpose(1, 0, 2))
        vs = np.ascontiguousarray(vv.transpose(1, 0, 2))
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        pos = [w.prior_len(b) + i for i in range(ql)]
        ref = sdpa_rows(w.q[lo:hi], ks, vs, pos, w.scale)
        worst = max(worst, float(np.abs(out[lo:hi] - ref).max()))
    return worst


def tiny_spec(dtype, G, D, BS, seqs, name="tiny"):
    return explicit_spec(f"{name}-{dtype}-{G}-{D}-{BS}", dtype, Hq=2 * G, Hkv=2, D=D, BS=BS,
                         seqs=seqs)


TINY_CASES = [
    ("f32", 1, 8, 4, [(1, 1), (5, 5), (9, 3), (13, 1)]),
    ("bf16", 2, 16, 2, [(3, 2), (17, 1), (20, 7)]),
    ("f32", 4, 8, 1, [(6, 6), (11, 4), (2, 1)]),
    ("bf16", 4, 16, 16, [(40, 13), (33, 1), (16, 16), (7, 0)]),
]


@pytest.mark.parametrize("dtype,G,D,BS,seqs", TINY_CASES)
def test_oracle_matches_torch_sdpa_float64(dtype, G, D, BS, seqs):
    w = make_workload(tiny_spec(dtype, G, D, BS, seqs))
    st = build_oracle_step(w)
    assert step_vs_sdpa(w, st) <= 1e-12


@pytest.mark.parametrize("name", ["batched-bf16-decode", "mixed-ragged-step",
                                  "prefix-shared-decode", "tiny-f32-decode"])
def test_oracle_matches_sdpa_on_small_configs(name):
    w = make_workload(SMALL_CONFIGS[name])
    st = build_oracle_step(w)
    assert step_vs_sdpa(w, st) <= 1e-12


def test_gather_round_trip_is_byte_exact():
    """Write through the slot mapping, gather back: the generator's rows, byte for byte."""
    w = make_workload(SMALL_CONFIGS["prefix-shared-decode"])
    st = build_oracle_step(w)
    for b in range(w.B):
        kk, vv = w.kv(b)
        g = gather(st.k_pool, st.block_tables[b], int(w.ctx_lens[b]), w.spec.BS)
        assert g.dtype == kk.dtype
        assert np.array_equal(g.transpose(1, 0, 2).view(np.uint16), kk.view(np.uint16))
        g = gather(st.v_pool, st.block_tables[b], int(w.ctx_lens[b]), w.spec.BS)
        assert np.array_equal(g.transpose(1, 0, 2).view(np.uint16), vv.view(np.uint16))


def test_slot_is_flat_index_of_block_and_offset():
    rng = np.random.default_rng(3)
    nb, bs, hkv, d = 7, 4, 2, 3
    kp = np.zeros((nb, bs, hkv, d), np.float32)
    vp = np.zeros_like(kp)
    slots = rng.permutation(nb * bs)[:11]
    slots[2] = -1
    kn = rng.standard_normal((11, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((11, hkv, d)).astype(np.float32)
    write_kv(kp, vp, kn, vn, slots, bs)
    flat = kp.reshape(nb * bs, hkv, d)
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(flat[s], kn[t])
    assert np.count_nonzero(flat.reshape(nb * bs, -1).any(axis=1)) == 10


def test_write_rejects_duplicates_and_out_of_range_without_writing():
    kp = np.zeros((2, 4, 1, 2), np.float32)
    vp = np.zeros_like(kp)
    kn = np.ones((3, 1, 2), np.float32)
    with pytest.raises(oracle.OracleError):
        write_kv(kp, vp, kn, kn, [1, 5, 1], 4)
    with pytest.raises(oracle.OracleError):
        write_kv(kp, vp, kn, kn, [0, 8, 2], 4)
    assert not kp.any() and not vp.any()


# ---- closed forms ----------------------------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_key_returns_its_value_exactly():
    q = _rand((1, 4, 8), 0)
    k = _rand((2, 1, 8), 1)
    v = _rand((2, 1, 8), 2)
    out = attend_rows(q, k, v, [0], 0.3)
    for h in range(4):
        assert np.array_equal(out[0, h], v[h // 2, 0])


def test_zero_query_gives_mean_of_visible_values():
    v = _rand((1, 9, 5), 4)
    k = _rand((1, 9, 5), 5)
    out = attend_rows(np.zeros((3, 2, 5)), k, v, [2, 5, 8], 1.0)
    for i, pos in enumerate([2, 5, 8]):
        np.testing.assert_allclose(out[i, 0], v[0, :pos + 1].mean(axis=0), rtol=0, atol=1e-15)
    out0 = attend_rows(_rand((1, 2, 5), 6), k, v, [8], 0.0)   # scale 0: same thing
    np.testing.assert_allclose(out0[0, 1], v[0].mean(axis=0), rtol=0, atol=1e-15)


def test_constant_values_give_that_constant():
    k = _rand((2, 30, 8), 7)
    v = np.full((2, 30, 8), -1.75)
    out = attend_rows(_rand((4, 4, 8), 8), k, v, [0, 3, 17, 29], 0.5)
    np.testing.assert_allclose(out, -1.75, rtol=0, atol=1e-15)


def test_row_at_position_zero_sees_only_the_first_key():
    k = _rand((1, 12, 4), 9)
    v = _rand((1, 12, 4), 10)
    out = attend_rows(_rand((1, 3, 4), 11), k, v, [0], 1.0)
    for h in range(3):
        assert np.array_equal(out[0, h], v[0, 0])


def test_dominant_key_takes_the_whole_weight():
    d = 8
    k = _rand((1, 20, d), 12) * 0.01
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    k[0, 13, 0] = 80.0                    # score gap ~ 80 → other weights < 20 e^-79
    v = _rand((1, 20, d), 13)
    out = attend_rows(q, k, v, [19], 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, 13], rtol=0, atol=1e-30 + 20 * np.exp(-79.0) * 5)


# ---- invariances ------------------------------------------------------------------------

def _contiguous_copy(st):
    """Same sequences in a fresh pool whose tables are identity ranges."""
    w = st.workload
    bs = w.spec.BS
    nblk = [(int(c) + bs - 1) // bs for c in w.ctx_lens]
    nb = sum(nblk)
    kp = np.zeros((nb,) + st.k_pool.shape[1:], st.k_pool.dtype)
    vp = np.zeros_like(kp)
    tables = np.full_like(st.block_tables, -1)
    base = 0
    for b, n in enumerate(nblk):
        ids = st.block_tables[b, :n]
        kp[base:base + n] = st.k_pool[ids]
        vp[base:base + n] = st.v_pool[ids]
        tables[b, :n] = np.arange(base, base + n)
        base += n
    return kp, vp, tables


def test_storage_equivalence_paged_equals_contiguous_bitwise():
    w = make_workload(SMALL_CONFIGS["mixed-ragged-step"])
    st = build_oracle_step(w)
    out = st.attention()
    kp, vp, tables = _contiguous_copy(st)
    out2 = paged_attention(w.q, kp, vp, tables, w.ctx_lens, w.cu_seqlens_q, w.scale)
    assert np.array_equal(out, out2)


def test_permuting_physical_blocks_is_bitwise_invisible():
    w = make_workload(SMALL_CONFIGS["batched-bf16-decode"])
    st = build_oracle_step(w)
    out = st.attention()
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    inv = np.argsort(perm)
    kp = st.k_pool[inv]          # block i moves to slot perm[i]
    vp = st.v_pool[inv]
    tables = np.where(st.block_tables >= 0, perm[np.maximum(st.block_tables, 0)], -1)
    out2 = paged_attention(w.q, kp, vp, tables, w.ctx_lens, w.cu_seqlens_q, w.scale)
    assert np.array_equal(out, out2)


def test_rechunking_and_batch_composition_are_bitwise_invisible():
    spec = explicit_spec("rechunk", "bf16", Hq=8, Hkv=2, D=16, BS=4, seqs=[(50, 21)])
    w = make_workload(spec)
    st = build_oracle_step(w)
    whole = st.attention()                      # one 21-row segment on a 29-token prior
    kc, vc = st.k_pool, st.v_pool
    tab = st.block_tables
    # the same 21 rows as chunks 5 + 9 + 7, each over the cache as it stands after the chunk
    parts = []
    done = 29
    for c in (5, 9, 7):
        done += c
        parts.append(paged_attention(w.q[done - 29 - c:done - 29], kc, vc, tab, [done],
                                     [0, c], w.scale))
    assert np.array_equal(np.concatenate(parts), whole)
    # the same rows inside a batch of strangers
    other = make_workload(explicit_spec("strangers", "bf16", Hq=8, Hkv=2, D=16, BS=4,
                                        seqs=[(33, 1), (12, 12), (70, 9), (5, 0), (9, 1)]))
    ost = build_oracle_step(other)
    nb = ost.k_pool.shape[0]
    kp = np.concatenate([ost.k_pool, kc])
    vp = np.concatenate([ost.v_pool, vc])
    mb = max(tab.shape[1], ost.block_tables.shape[1])
    tables = np.full((other.B + 1, mb), -1, np.int32)
    tables[:other.B, :ost.block_tables.shape[1]] = ost.block_tables
    tables[other.B, :tab.shape[1]] = np.where(tab[0] >= 0, tab[0] + nb, -1)
    q = np.concatenate([other.q, w.q])
    ctx = list(other.ctx_lens) + [50]
    cu = list(other.cu_seqlens_q) + [other.T + 21]
    batched = paged_attention(q, kp, vp, tables, ctx, cu, w.scale)
    assert np.array_equal(batched[other.T:], whole)


# ---- planted mistakes (oracle mutants) must be caught ------------------------------------

def _pins_hold():
    try:
        for dtype, G, D, BS, seqs in TINY_CASES:
            w = make_workload(tiny_spec(dtype, G, D, BS, seqs))
            st = build_oracle_step(w)
            if not step_vs_sdpa(w, st) <= 1e-12:
                return False
            for b in range(w.B):
                kk, _ = w.kv(b)
                g = gather(st.k_pool, st.block_tables[b], int(w.ctx_lens[b]), BS)
                if not np.array_equal(g.transpose(1, 0, 2).view(np.uint8), kk.view(np.uint8)):
                    return False
        return True
    except (oracle.OracleError, oracle.AllocatorError, IndexError, ValueError):
        return False


def test_unmutated_control_passes():
    assert _pins_hold()


def test_mutant_gather_drops_last_key(monkeypatch):
    real = P.gather
    monkeypatch.setattr(P, "gather", lambda pool, row, n, bs: real(pool, row, n, bs)[:, :-1]
                        if n > 1 else real(pool, row, n, bs))
    assert not _pins_hold()


def test_mutant_slot_ignores_block_offset(monkeypatch):
    monkeypatch.setattr(A, "slot_of", lambda block, pos, bs: block * bs)
    assert not _pins_hold()


def test_mutant_k_heads_flipped(monkeypatch):
    monkeypatch.setattr(P, "kv_head_of", lambda h, hq, hkv: (hkv - 1) - h // (hq // hkv))
    assert not _pins_hold()


@pytest.mark.parametrize("delta", [-1, +1])
def test_mutant_causal_mask_off_by_one(monkeypatch, delta):
    monkeypatch.setattr(P, "n_visible", lambda pos: max(pos + 1 + delta, 1))
    assert not _pins_hold()


def test_bf16_rounding_of_draws_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3e38],
                 dtype=np.float32)
    bits = round_f32_to_bf16_bits(x)
    back = P.bf16_bits_to_f64(bits)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 → 1; 1 + 3*2^-8 → 1 + 2^-6
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6
    assert back[3] == 1.0 and back[4] == -2.5
    assert abs(back[5] - 3e38) / 3e38 < 2 ** -8
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, bits)
