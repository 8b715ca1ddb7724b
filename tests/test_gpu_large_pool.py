"""Maximum sizes: K/V pools larger than 4 GiB each, with the step's sequences on the highest
block ids, so that every byte offset the append, the decode pass and the tile path form exceeds
32 bits. The oracle attends over each sequence's rows directly (float64, keys 0..pos), so it
never holds the pools on the host.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from oracle.fp8 import dequantize, quantize_rows
from oracle.paged import attend_rows, bf16_bits_to_f64
from workloads import round_f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HQ, HKV, D, BS = 32, 8, 128, 16
SEQS = [(600, 1), (700, 130), (100, 1), (1030, 1)]   # (ctx, q_len): decode, prefill, decode, 3 splits
TOL = 2e-3


def _bits_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _case(fp8: bool):
    elem = 1 if fp8 else 2
    block_bytes = BS * HKV * D * elem
    nb = (4 << 30) // block_bytes + 4096               # > 4 GiB per pool
    rng = np.random.default_rng(2024 + fp8)
    B = len(SEQS)
    nblk = [(c + BS - 1) // BS for c, _ in SEQS]
    top = np.arange(nb - sum(nblk), nb, dtype=np.int32)
    rng.shuffle(top)
    tables = np.full((B, max(nblk)), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = top[o:o + n]
        o += n
    ks = [round_f32_to_bf16_bits(rng.standard_normal((c, HKV, D), dtype=np.float32)) for c, _ in SEQS]
    vs = [round_f32_to_bf16_bits(rng.standard_normal((c, HKV, D), dtype=np.float32)) for c, _ in SEQS]
    T = sum(q for _, q in SEQS)
    q = round_f32_to_bf16_bits(rng.standard_normal((T, HQ, D), dtype=np.float32))
    ctx = np.asarray([c for c, _ in SEQS], dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum([q_ for _, q_ in SEQS])]).astype(np.int32)
    return nb, tables, ks, vs, q, ctx, cu


def _slots(tables, b, n):
    pos = np.arange(n)
    return (tables[b, pos // BS].astype(np.int64) * BS + pos % BS).astype(np.int32)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
def test_pools_over_4gib_match_oracle(fp8):
    nb, tables, ks, vs, q, ctx, cu = _case(fp8)
    scale = 1.0 / np.sqrt(D)
    k_scale, v_scale = 1 / 48, 1 / 40
    print(f"[large-pool] fp8={fp8} NB={nb} pool bytes={nb * BS * HKV * D * (1 if fp8 else 2)}",
          flush=True)
    shape = (nb, BS, HKV, D)
    if fp8:
        kc = torch.full(shape, 0x7F, dtype=torch.uint8, device=DEV)
        vc = torch.full(shape, 0x7F, dtype=torch.uint8, device=DEV)
    else:
        kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    try:
        for b, (c, _) in enumerate(SEQS):
            sl = _slots(tables, b, c)
            kd, vd = _bits_to_dev(ks[b]), _bits_to_dev(vs[b])
            if fp8:
                pkv.write_kv_fp8(kd, vd, sl, kc, vc, k_scale, v_scale)
            else:
                pkv.write_kv(kd, vd, sl, kc, vc)
        bt = torch.from_numpy(tables).to(DEV)
        qd = _bits_to_dev(q)
        for pc in (False, True):
            if fp8:
                out = pkv.attention_fp8(qd, kc, vc, bt, ctx, cu, scale, k_scale, v_scale,
                                        phase_consistent=pc)
            else:
                out = pkv.attention(qd, kc, vc, bt, ctx, cu, scale, phase_consistent=pc)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            err = 0.0
            for b, (c, ql) in enumerate(SEQS):
                lo = int(cu[b])
                if fp8:
                    kf = dequantize(quantize_rows(bf16_bits_to_f64(ks[b]).astype(np.float32),
                                                  k_scale), k_scale)
                    vf = dequantize(quantize_rows(bf16_bits_to_f64(vs[b]).astype(np.float32),
                                                  v_scale), v_scale)
                    # the codes stored in the pool are the oracle's (write bit-exact)
                    sl = _slots(tables, b, c)
                    got_codes = kc.view(-1, HKV, D)[torch.from_numpy(sl.astype(np.int64)).to(DEV)]
                    want_codes = quantize_rows(bf16_bits_to_f64(ks[b]).astype(np.float32), k_scale)
                    assert np.array_equal(got_codes.cpu().numpy(), want_codes)
                else:
                    kf, vf = bf16_bits_to_f64(ks[b]), bf16_bits_to_f64(vs[b])
                ref = attend_rows(q[lo:lo + ql], np.ascontiguousarray(kf.transpose(1, 0, 2)),
                                  np.ascontiguousarray(vf.transpose(1, 0, 2)),
                                  list(range(c - ql, c)), scale)
                err = max(err, float(np.abs(got[lo:lo + ql] - ref).max()))
            print(f"[large-pool] fp8={fp8} phase_consistent={pc} max abs err {err:.3e}", flush=True)
            assert np.isfinite(got).all() and err <= TOL
    finally:
        del kc, vc
        torch.cuda.empty_cache()
