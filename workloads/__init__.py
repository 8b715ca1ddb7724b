"""Seeded synthetic inputs for the paged-KV append and paged attention.

Both sides of every comparison (the HIP library and the CPU oracle) take their inputs from
here, so this module holds none of the method's arithmetic: no slot computation, no block
bookkeeping, no attention. It only draws random numbers, rounds the draws to the storage type,
and describes the structure of a step (which sequences exist, how long they are, which ones
share a prompt, in which order blocks are handed out).

Workload shapes follow the length mixes the pages describe: heavy-tailed rollout lengths
("P3: native paged-KV continuous-batching sampler", section "Why": most samples end at a few
thousand tokens, some run to 16k/40k), chunked prefill sharing a flat ragged step with decodes
(same page, "Design > engine.py", Scheduler), and G samples that share one prompt through
full read-only blocks (same page, "Prefix sharing").

Seeds are sha256-derived, so a label always gives the same stream, whatever the interpreter's
hash salt (same page, "Review": bench seeds).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "stable_seed", "round_f32_to_bf16_bits", "Spec", "Admission", "Workload",
    "make_workload", "CONFIGS", "SMALL_CONFIGS", "DIAGNOSTIC_CONFIGS", "explicit_spec",
]


def stable_seed(label: str) -> int:
    """64-bit seed from the first 8 bytes (little-endian) of sha256(label)."""
    return int.from_bytes(hashlib.sha256(label.encode("utf-8")).digest()[:8], "little")


def round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite draws; a NaN is kept as a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    r = bits >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += bits
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


# --------------------------------------------------------------------------------------------
# Step description
# --------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Spec:
    """Recipe of one synthetic step.

    Sequence kinds, all optional and concatenated in the order decode, prefill, shared (then
    shuffled when ``interleave``):
      decode_ctx:  ("fixed", [ctx...]) or ("lognormal", median, sigma, lo, hi, count);
                   each such sequence has one query row (its last position).
      prefill:     (count, q_len, prior_lo, prior_hi): chunked-prefill segments whose prior
                   context is uniform on {prior_lo..prior_hi} and whose q_len new rows follow it.
      shared:      (groups, per_group, prefix_tokens, tail_lo, tail_hi): each group shares a
                   prompt of prefix_tokens (a whole number of blocks), every sample adds a
                   private tail uniform on {tail_lo..tail_hi}; one query row each.
      explicit:    [(ctx, q_len), ...] exact sequences (edge cases).
    pool: ("fixed", NB) or ("factor", f): NB = ceil(f * blocks needed).
    k_outlier: (prob, factor): each K row (sequence, position, kv head) is scaled by factor with
               probability prob.
    """
    name: str
    dtype: str
    Hq: int
    Hkv: int
    D: int
    BS: int
    decode_ctx: Optional[tuple] = None
    prefill: Optional[tuple] = None
    shared: Optional[tuple] = None
    explicit: Optional[tuple] = None
    pool: tuple = ("factor", 1.2)
    k_outlier: Optional[tuple] = None
    interleave: bool = False
    kv_split: int = 512
    # "fp8": the pools hold OCP E4M3 codes with per-tensor scales (q and the K/V rows that
    # are written stay in `dtype`); "" keeps the pools in `dtype`
    kv_dtype: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


@dataclass
class Admission:
    """One admission event in sequence order.

    A sequence with ``share_from >= 0`` adopts the first ``n_shared_blocks`` blocks of sequence
    ``share_from`` (already admitted and written) and then takes ``n_blocks - n_shared_blocks``
    fresh blocks; otherwise it takes ``n_blocks`` fresh blocks.
    """
    seq: int
    share_from: int
    n_shared_blocks: int
    n_blocks: int


@dataclass
class Workload:
    spec: Spec
    seed: int
    ctx_lens: np.ndarray          # int32 [B]
    q_lens: np.ndarray            # int32 [B]
    cu_seqlens_q: np.ndarray      # int32 [B + 1]
    num_blocks: int               # NB
    free_order: np.ndarray        # int32 [NB]: order in which a fully allocated pool is freed
    admissions: List[Admission]
    group_of: np.ndarray          # int32 [B]: shared-prompt group or -1
    prefix_tokens: np.ndarray     # int32 [B]: tokens of the shared prompt (0 if none)
    q: np.ndarray                 # [T, Hq, D]  uint16 bf16 bits or float32
    scale: float
    _kv_seed: int = 0
    _prefix_cache: dict = field(default_factory=dict)

    # ---- shapes ------------------------------------------------------------------------
    @property
    def B(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def n_blocks_per_seq(self) -> np.ndarray:
        bs = self.spec.BS
        return (self.ctx_lens + bs - 1) // bs

    @property
    def max_blocks(self) -> int:
        return max(1, int(self.n_blocks_per_seq.max(initial=0)))

    @property
    def np_dtype(self):
        return np.uint16 if self.spec.dtype == "bf16" else np.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.spec.dtype == "bf16" else 4

    @property
    def kv_fp8(self) -> bool:
        return self.spec.kv_dtype == "fp8"

    @property
    def kv_elem_bytes(self) -> int:
        """Bytes per stored K/V element (the pools' element type)."""
        return 1 if self.kv_fp8 else self.elem_bytes

    # ---- K/V values ---------------------------------------------------------------------
    def _draw(self, rng: np.random.Generator, n: int) -> Tuple[np.ndarray, np.ndarray]:
        s = self.spec
        k = rng.standard_normal((n, s.Hkv, s.D), dtype=np.float32)
        v = rng.standard_normal((n, s.Hkv, s.D), dtype=np.float32)
        if s.k_outlier is not None and n:
            prob, factor = s.k_outlier
            mask = rng.random((n, s.Hkv)) < prob
            k[mask] *= np.float32(factor)
        if s.dtype == "bf16":
            return round_f32_to_bf16_bits(k), round_f32_to_bf16_bits(v)
        return k, v

    def _stream(self, kind: str, idx: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([self._kv_seed, 0 if kind == "seq" else 1, idx])))

    def kv(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V of sequence b at positions [0, ctx_b): arrays [ctx_b, Hkv, D]."""
        ctx = int(self.ctx_lens[b])
        npre = int(self.prefix_tokens[b])
        tail_k, tail_v = self._draw(self._stream("seq", b), ctx - npre)
        if npre == 0:
            return tail_k, tail_v
        g = int(self.group_of[b])
        if g not in self._prefix_cache:
            self._prefix_cache[g] = self._draw(self._stream("group", g), npre)
        pk, pv = self._prefix_cache[g]
        return np.concatenate([pk, tail_k]), np.concatenate([pv, tail_v])

    def iter_kv(self, seqs=None, workers: int = 8):
        """Yield (b, k, v) for the given sequences (default all) in order, drawn in threads."""
        from concurrent.futures import ThreadPoolExecutor
        seqs = list(range(self.B)) if seqs is None else [int(b) for b in seqs]
        for g in sorted(set(int(self.group_of[b]) for b in seqs if self.prefix_tokens[b] > 0)):
            if g not in self._prefix_cache:
                b0 = next(b for b in seqs if self.group_of[b] == g)
                self.kv(b0)
        if workers <= 1 or len(seqs) <= 1:
            for b in seqs:
                yield (b,) + self.kv(b)
            return
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for b, (k, v) in zip(seqs, ex.map(self.kv, seqs)):
                yield b, k, v

    def prior_len(self, b: int) -> int:
        return int(self.ctx_lens[b] - self.q_lens[b])

    def q_rows(self, b: int) -> np.ndarray:
        return self.q[self.cu_seqlens_q[b]:self.cu_seqlens_q[b + 1]]


def _lognormal_lengths(rng, median, sigma, lo, hi, count) -> np.ndarray:
    z = rng.standard_normal(count)
    return np.clip(np.rint(np.exp(np.log(median) + sigma * z)), lo, hi).astype(np.int64)


def make_workload(spec: Spec, seed: Optional[int] = None) -> Workload:
    """Draw one step from ``spec``. ``seed`` defaults to stable_seed('pkv-config-' + name)."""
    if seed is None:
        seed = stable_seed("pkv-config-" + spec.name)
    ss = np.random.SeedSequence(seed)
    s_len, s_perm, s_q, s_kv, s_order = ss.spawn(5)
    rng_len = np.random.Generator(np.random.PCG64(s_len))

    ctx: List[int] = []
    qlen: List[int] = []
    group: List[int] = []
    prefix: List[int] = []
    if spec.decode_ctx is not None:
        if spec.decode_ctx[0] == "fixed":
            vals = list(spec.decode_ctx[1])
        else:
            _, median, sigma, lo, hi, count = spec.decode_ctx
            vals = list(_lognormal_lengths(rng_len, median, sigma, lo, hi, count))
        for c in vals:
            ctx.append(int(c)); qlen.append(1); group.append(-1); prefix.append(0)
    if spec.prefill is not None:
        count, ql, plo, phi = spec.prefill
        priors = rng_len.integers(plo, phi + 1, size=count)
        for p in priors:
            ctx.append(int(p) + ql); qlen.append(ql); group.append(-1); prefix.append(0)
    if spec.shared is not None:
        groups, per_group, npre, tlo, thi = spec.shared
        assert npre % spec.BS == 0, "a shared prompt is a whole number of blocks"
        for g in range(groups):
            tails = rng_len.integers(tlo, thi + 1, size=per_group)
            for t in tails:
                ctx.append(npre + int(t)); qlen.append(1); group.append(g); prefix.append(npre)
    if spec.explicit is not None:
        for c, ql in spec.explicit:
            ctx.append(int(c)); qlen.append(int(ql)); group.append(-1); prefix.append(0)

    B = len(ctx)
    order = np.arange(B)
    if spec.interleave and B > 1:
        order = np.random.Generator(np.random.PCG64(s_order)).permutation(B)
    ctx_a = np.asarray(ctx, dtype=np.int32)[order]
    q_a = np.asarray(qlen, dtype=np.int32)[order]
    grp_a = np.asarray(group, dtype=np.int32)[order]
    pre_a = np.asarray(prefix, dtype=np.int32)[order]
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_a)

    # admissions in sequence order; the first member of a group owns the prompt blocks
    bs = spec.BS
    nblk = (ctx_a.astype(np.int64) + bs - 1) // bs
    leaders = {}
    admissions = []
    needed = 0
    for b in range(B):
        g = int(grp_a[b])
        if g >= 0 and g in leaders:
            nsh = int(pre_a[b]) // bs
            admissions.append(Admission(b, leaders[g], nsh, int(nblk[b])))
            needed += int(nblk[b]) - nsh
        else:
            if g >= 0:
                leaders[g] = b
            admissions.append(Admission(b, -1, 0, int(nblk[b])))
            needed += int(nblk[b])

    if spec.pool[0] == "fixed":
        NB = int(spec.pool[1])
    else:
        NB = int(np.ceil(spec.pool[1] * needed))
    NB = max(NB, needed, 1)
    free_order = np.random.Generator(np.random.PCG64(s_perm)).permutation(NB).astype(np.int32)

    T = int(cu[-1])
    rng_q = np.random.Generator(np.random.PCG64(s_q))
    qf = rng_q.standard_normal((T, spec.Hq, spec.D), dtype=np.float32)
    q = round_f32_to_bf16_bits(qf) if spec.dtype == "bf16" else qf

    w = Workload(spec=spec, seed=seed, ctx_lens=ctx_a, q_lens=q_a, cu_seqlens_q=cu,
                 num_blocks=NB, free_order=free_order, admissions=admissions,
                 group_of=grp_a, prefix_tokens=pre_a, q=q, scale=1.0 / float(np.sqrt(spec.D)))
    w._kv_seed = int(s_kv.generate_state(1, np.uint64)[0])
    return w


def explicit_spec(name: str, dtype: str, Hq: int, Hkv: int, D: int, BS: int,
                  seqs: Sequence[Tuple[int, int]], pool=("factor", 1.5), **kw) -> Spec:
    """A step made of exactly the given (ctx, q_len) sequences."""
    return Spec(name=name, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, BS=BS, explicit=tuple(seqs),
                pool=pool, **kw)


# --------------------------------------------------------------------------------------------
# The five measured workloads and their small twins
# --------------------------------------------------------------------------------------------

CONFIGS = {
    # 1 layer, 4 sequences with ctx {17, 33, 64, 100}, one query row each, 64-block pool.
    "tiny-f32-decode": Spec("tiny-f32-decode", "f32", Hq=4, Hkv=2, D=64, BS=16,
                            decode_ctx=("fixed", [17, 33, 64, 100]), pool=("fixed", 64)),
    # 64 decode rows, lognormal lengths (median 2048, sigma 1) clipped to [16, 16384].
    "batched-bf16-decode": Spec("batched-bf16-decode", "bf16", Hq=32, Hkv=8, D=128, BS=16,
                                decode_ctx=("lognormal", 2048, 1.0, 16, 16384, 64)),
    # 8 chunked-prefill segments of 512 rows on priors U{0..8192} + 120 decode rows
    # (lognormal, median 3000), in one flat ragged batch.
    "mixed-ragged-step": Spec("mixed-ragged-step", "bf16", Hq=32, Hkv=8, D=128, BS=16,
                              decode_ctx=("lognormal", 3000, 1.0, 16, 16384, 120),
                              prefill=(8, 512, 0, 8192), interleave=True),
    # 8 sequences of 40960 tokens, block 32, G = 8; 1 % of K rows scaled by 8.
    "long-context-decode": Spec("long-context-decode", "bf16", Hq=64, Hkv=8, D=128, BS=32,
                                decode_ctx=("fixed", [40960] * 8), k_outlier=(0.01, 8.0)),
    # 16 groups x 8 samples sharing a 2048-token prompt (128 blocks of 16) + tails U{1..4096}.
    "prefix-shared-decode": Spec("prefix-shared-decode", "bf16", Hq=16, Hkv=4, D=128, BS=16,
                                 shared=(16, 8, 2048, 1, 4096)),
}

# Reduced sizes the oracle finishes in seconds; each still spans several 64-token tiles and
# several 512-token splits with ragged tails.
SMALL_CONFIGS = {
    "tiny-f32-decode": CONFIGS["tiny-f32-decode"],
    "batched-bf16-decode": Spec("batched-bf16-decode-small", "bf16", Hq=32, Hkv=8, D=128,
                                BS=16, decode_ctx=("lognormal", 300, 1.0, 1, 1500, 6)),
    "mixed-ragged-step": Spec("mixed-ragged-step-small", "bf16", Hq=32, Hkv=8, D=128, BS=16,
                              decode_ctx=("lognormal", 300, 1.0, 1, 1200, 5),
                              prefill=(3, 130, 0, 700), interleave=True),
    "long-context-decode": Spec("long-context-decode-small", "bf16", Hq=64, Hkv=8, D=128,
                                BS=32, decode_ctx=("fixed", [1100, 1537]),
                                k_outlier=(0.01, 8.0)),
    "prefix-shared-decode": Spec("prefix-shared-decode-small", "bf16", Hq=16, Hkv=4, D=128,
                                 BS=16, shared=(2, 3, 64, 1, 600)),
}


# The batched decode and mixed steps with FP8 (OCP E4M3) pools and per-tensor scales 1/64
# (N(0, 1) values of a few units stay far inside the E4M3 range): q and the written K/V rows are
# bfloat16, the pools hold their codes.
FP8_CONFIGS = {
    "batched-fp8-decode": Spec("batched-fp8-decode", "bf16", Hq=32, Hkv=8, D=128, BS=16,
                               decode_ctx=("lognormal", 2048, 1.0, 16, 16384, 64),
                               kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 64),
    "mixed-fp8-step": Spec("mixed-fp8-step", "bf16", Hq=32, Hkv=8, D=128, BS=16,
                           decode_ctx=("lognormal", 3000, 1.0, 16, 16384, 120),
                           prefill=(8, 512, 0, 8192), interleave=True,
                           kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 64),
    # the long-context step (G 8, 8 x 40960 keys, 1 % of K rows x 8) over E4M3 pools; the K
    # scale 1/8 keeps the outlier rows (|k| up to about 40) inside the +-448 code range
    "long-context-fp8-decode": Spec("long-context-fp8-decode", "bf16", Hq=64, Hkv=8, D=128,
                                    BS=32, decode_ctx=("fixed", [40960] * 8),
                                    k_outlier=(0.01, 8.0), kv_dtype="fp8", k_scale=1 / 8,
                                    v_scale=1 / 64),
}

FP8_SMALL_CONFIGS = {
    "batched-fp8-decode": Spec("batched-fp8-decode-small", "bf16", Hq=32, Hkv=8, D=128, BS=16,
                               decode_ctx=("lognormal", 300, 1.0, 1, 1500, 6),
                               kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 64),
    "mixed-fp8-step": Spec("mixed-fp8-step-small", "bf16", Hq=32, Hkv=8, D=128, BS=16,
                           decode_ctx=("lognormal", 300, 1.0, 1, 1200, 5),
                           prefill=(3, 130, 0, 700), interleave=True,
                           kv_dtype="fp8", k_scale=1 / 64, v_scale=1 / 32),
    "prefix-shared-fp8-decode": Spec("prefix-shared-fp8-decode-small", "bf16", Hq=16, Hkv=4,
                                     D=64, BS=16, shared=(2, 3, 64, 1, 600),
                                     kv_dtype="fp8", k_scale=0.02, v_scale=0.015),
    "long-context-fp8-decode": Spec("long-context-fp8-decode-small", "bf16", Hq=64, Hkv=8,
                                    D=128, BS=32, decode_ctx=("fixed", [1100, 1537]),
                                    k_outlier=(0.01, 8.0), kv_dtype="fp8", k_scale=1 / 8,
                                    v_scale=1 / 64),
}

# Measurement only: the mixed step's eight chunked-prefill segments (the (ctx, q_len) pairs its
# draw gives) with no decode rows, so that the prefill tile kernel runs alone, in one launch.
DIAGNOSTIC_CONFIGS = {
    "mixed-step-prefill-rows": Spec("mixed-step-prefill-rows", "bf16", Hq=32, Hkv=8, D=128,
                                    BS=16, explicit=((2620, 512), (795, 512), (5169, 512),
                                                     (3436, 512), (2650, 512), (8095, 512),
                                                     (5333, 512), (6535, 512))),
}

ALL_CONFIGS = {**CONFIGS, **FP8_CONFIGS, **DIAGNOSTIC_CONFIGS}
