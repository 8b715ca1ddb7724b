"""Pins of the FP8 (OCP E4M3) codec and the FP8 KV write of the oracle (oracle/fp8.py).

The codec is checked against the format's definition (printed points of the OCP 8-bit
floating point specification's E4M3 encoding), against a library routine (torch's
float8_e4m3fn cast, which rounds to nearest even inside the finite range), and by brute
force (round trips of every code, every midpoint between neighbours, monotonicity). Planted
mistakes (ties rounded up, no saturation, a wrong exponent bias, truncation) each fail.
"""
import numpy as np
import pytest

from oracle import fp8

torch = pytest.importorskip("torch")


def test_format_points():
    d = fp8.e4m3_decode
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x3C) == 1.5 and d(0x30) == 0.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0                 # largest finite
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9          # min normal, min subnormal
    assert d(0x07) == 7 * 2.0 ** -9                                # max subnormal
    assert d(0x00) == 0.0 and np.signbit(d(0x80))                  # signed zeros
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))                 # the only NaNs
    assert np.isfinite(fp8.e4m3_decode(np.arange(256))[[c for c in range(256) if c & 0x7F != 0x7F]]).all()


def test_every_finite_code_round_trips_and_the_grid_is_monotone():
    codes = np.arange(256, dtype=np.uint8)
    v = fp8.e4m3_decode(codes)
    fin = ~np.isnan(v)
    assert (fp8.e4m3_encode(v[fin].astype(np.float32)) == codes[fin]).all()
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()


def test_midpoints_round_to_the_even_code_and_neighbours_to_the_nearer():
    mags = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)       # exact in float32
    assert (mids.astype(np.float64) == (mags[:-1] + mags[1:]) / 2).all()
    got = fp8.e4m3_encode(mids)
    lo = np.arange(0x7E, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert (got == want).all()
    assert (fp8.e4m3_encode(np.nextafter(mids, np.float32(np.inf))) == lo + 1).all()
    assert (fp8.e4m3_encode(np.nextafter(mids, np.float32(-np.inf))) == lo).all()
    assert (fp8.e4m3_encode(-mids) == (want | 0x80)).all()


def test_saturation_and_signed_zero():
    e = fp8.e4m3_encode
    assert e(np.float32(448.5))[()] == 0x7E and e(np.float32(1e30))[()] == 0x7E
    assert e(np.float32(464.0))[()] == 0x7E and e(np.float32(-5e5))[()] == 0xFE
    assert e(np.float32(-0.0))[()] == 0x80 and e(np.float32(-1e-30))[()] == 0x80
    assert e(np.float32(2.0 ** -10))[()] == 0x00         # half the min subnormal: tie to even 0
    assert e(np.float32(3 * 2.0 ** -10))[()] == 0x02     # 1.5 min subnormals: tie to even 2
    with pytest.raises(ValueError):
        e(np.float32(np.nan))


def test_agrees_with_torch_inside_the_finite_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (1e-3, 0.05, 1, 30, 120)])
    mags = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    x = np.concatenate([x, (mags[:-1] + mags[1:]) / 2, -(mags[:-1] + mags[1:]) / 2]).astype(np.float32)
    x = x[np.abs(x) < 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (fp8.e4m3_encode(x) == t).all()


def test_quantize_is_one_float32_multiply_by_the_float32_reciprocal():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(4096).astype(np.float32)
    for scale in (1 / 64, 0.0123, 3.0):
        inv = np.float32(1) / np.float32(scale)
        assert fp8.inv_scale_f32(scale) == inv
        assert (fp8.quantize_rows(x, scale) == fp8.e4m3_encode(x * inv)).all()
        # dequantised values are within half a grid step (relative 2^-4) of the input
        dq = fp8.dequantize(fp8.quantize_rows(x, scale), scale)
        big = np.abs(x) > 2 ** -6 * scale * 8
        assert (np.abs(dq[big] - x[big]) <= np.abs(x[big]) * 2.0 ** -4 + 1e-12).all()


def _encode_mutant(x, mode):
    mags = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(np.asarray(x, np.float64))
    if mode != "no_saturation":
        a = np.minimum(a, 448.0)
    lo = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    if mode == "ties_up":
        pick = (mags[hi] - a) <= (a - mags[lo])
    elif mode == "truncate":
        pick = np.zeros_like(a, dtype=bool)
    else:
        pick = ((mags[hi] - a) < (a - mags[lo])) | (((mags[hi] - a) == (a - mags[lo])) & (hi % 2 == 0))
    code = np.where(pick, hi, lo).astype(np.uint8)
    if mode == "no_saturation":
        code = np.where(a > 464, 0x7F, code).astype(np.uint8)
    return code


@pytest.mark.parametrize("mode", ["ties_up", "truncate", "no_saturation"])
def test_planted_codec_mistakes_are_caught(mode):
    mags = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    probe = np.concatenate([(mags[:-1] + mags[1:]) / 2, mags * 1.01, [500.0, 1e6]]).astype(np.float32)
    assert (_encode_mutant(probe, "ok") == fp8.e4m3_encode(probe)).all()
    assert not (_encode_mutant(probe, mode) == fp8.e4m3_encode(probe)).all()


def test_planted_bias_mistake_is_caught():
    c = np.arange(0x7F, dtype=np.uint8)
    e = (c.astype(np.int64) >> 3) & 0xF
    m = c & 7
    wrong = np.where(e == 0, m * 2.0 ** -10, (1 + m / 8) * np.exp2(e - 8.0))   # bias 8
    assert not np.array_equal(wrong, fp8.e4m3_decode(c))
    assert fp8.e4m3_decode(0x38) == 1.0 and wrong[0x38] != 1.0


# ---- the FP8 oracle step -------------------------------------------------------------------

from oracle import build_oracle_step                       # noqa: E402
from oracle.paged import bf16_bits_to_f64, gather          # noqa: E402
from workloads import FP8_SMALL_CONFIGS, make_workload     # noqa: E402


@pytest.mark.parametrize("name", list(FP8_SMALL_CONFIGS))
def test_fp8_pools_hold_the_codes_of_every_written_row(name):
    w = make_workload(FP8_SMALL_CONFIGS[name])
    st = build_oracle_step(w)
    s = w.spec
    for b in range(w.B):
        kk, vv = w.kv(b)
        ctx = int(w.ctx_lens[b])
        kc = gather(st.k_pool, st.block_tables[b], ctx, s.BS)      # [Hkv, ctx, D] codes
        vc = gather(st.v_pool, st.block_tables[b], ctx, s.BS)
        k32 = bf16_bits_to_f64(kk[:ctx]).astype(np.float32)
        v32 = bf16_bits_to_f64(vv[:ctx]).astype(np.float32)
        assert (kc.transpose(1, 0, 2) == fp8.quantize_rows(k32, s.k_scale)).all()
        assert (vc.transpose(1, 0, 2) == fp8.quantize_rows(v32, s.v_scale)).all()


@pytest.mark.parametrize("name", list(FP8_SMALL_CONFIGS))
def test_fp8_attention_equals_sdpa_over_the_dequantised_cache(name):
    w = make_workload(FP8_SMALL_CONFIGS[name])
    st = build_oracle_step(w)
    got = st.attention()
    s = w.spec
    q = bf16_bits_to_f64(w.q)
    for b in range(w.B):
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        if hi == lo:
            continue
        ctx = int(w.ctx_lens[b])
        kd = fp8.dequantize(gather(st.k_pool, st.block_tables[b], ctx, s.BS), s.k_scale)
        vd = fp8.dequantize(gather(st.v_pool, st.block_tables[b], ctx, s.BS), s.v_scale)
        kq = torch.from_numpy(kd).repeat_interleave(s.G, dim=0)       # [Hq, ctx, D]
        vq = torch.from_numpy(vd).repeat_interleave(s.G, dim=0)
        qq = torch.from_numpy(q[lo:hi]).transpose(0, 1)               # [Hq, n, D]
        pos = torch.arange(ctx - (hi - lo), ctx)[:, None]
        mask = torch.arange(ctx)[None, :] <= pos
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq, attn_mask=mask,
                                                                scale=w.scale)
        assert np.abs(got[lo:hi] - ref.transpose(0, 1).numpy()).max() < 1e-12


def test_fp8_attention_is_close_to_the_unquantised_attention():
    w = make_workload(FP8_SMALL_CONFIGS["batched-fp8-decode"])
    st = build_oracle_step(w)
    import dataclasses
    wb = make_workload(dataclasses.replace(w.spec, kv_dtype=""))
    ref = build_oracle_step(wb).attention()
    # same seeded values (same spec name); E4M3 keeps 3 mantissa bits: errors of a few 1e-2
    err = np.abs(st.attention() - ref).max()
    assert 1e-4 < err < 0.15, err
