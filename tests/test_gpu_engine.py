"""GPU: the host step builder driving the device path end to end, through the C ABI.

Each step: the C++ scheduler (pkv_sched_*) builds a plan; its copy-on-write pairs are applied
with pkv_copy_blocks; pkv_write_kv_attention appends the step's new rows through the plan's
slots and attends over the plan's tables, cu_seqlens_q and ctx_lens. Whatever the schedule
(chunked prefill, decodes, preemption by recompute, prefix adoption, forks, trims), every row
computed must equal float64 dense attention over its own sequence's current tokens, within the
element type's tolerance. Token K/V and queries are seeded functions of the token's identity.
"""
import numpy as np
import pytest

import prefill_slot_mapping_amd as pkv
from oracle.fp8 import dequantize, quantize_rows
from oracle.paged import attend_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 2e-3, "f32": 1e-5, "e4m3": 2e-3}
HQ, HKV, D, SCALE = 8, 2, 64, 0.125
K_SCALE, V_SCALE = 1 / 40, 1 / 48      # E4M3 pools: the rows are bf16, the pools their codes


def _bf16_round(a):
    """float32 -> nearest-even bfloat16, returned as float32 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32)


class Tokens:
    """Identity of every token: a group's prompts are the same tokens; a fork shares its
    parent's tokens; after a trim, new tokens past the cut are new identities."""

    def __init__(self):
        self.known, self.epoch = {}, {}

    def add(self, sid, plen, grp):
        self.known[sid] = [(0, grp, plen, p) for p in range(plen)] if grp >= 0 else []
        self.epoch[sid] = 0

    def key(self, sid, pos):
        k = self.known[sid]
        while len(k) <= pos:
            k.append((1, sid, self.epoch[sid], len(k)))
        return k[pos]

    def fork(self, src, new, n):
        self.known[new] = [self.key(src, p) for p in range(n)]
        self.epoch[new] = 0

    def trim(self, sid, n):
        self.known[sid] = [self.key(sid, p) for p in range(n)]
        self.epoch[sid] += 1


def _kv(key, dt):
    r = np.random.default_rng([*key, 1])
    k, v = r.standard_normal((HKV, D)).astype(np.float32), r.standard_normal((HKV, D)).astype(np.float32)
    return (_bf16_round(k), _bf16_round(v)) if dt != "f32" else (k, v)


def _kv_stored(key, dt):
    """The values a pool holds for a token: E4M3 pools hold codes of the bf16 rows."""
    k, v = _kv(key, dt)
    if dt == "e4m3":
        return dequantize(quantize_rows(k, K_SCALE), K_SCALE), dequantize(quantize_rows(v, V_SCALE), V_SCALE)
    return k, v


def _q(sid, pos, dt):
    q = np.random.default_rng([sid, pos, 2]).standard_normal((HQ, D)).astype(np.float32)
    return _bf16_round(q) if dt != "f32" else q


def _dense(tok, sid, pos, dt):
    kv = [_kv_stored(tok.key(sid, j), dt) for j in range(pos + 1)]
    kc = np.stack([x[0] for x in kv], axis=1)
    vc = np.stack([x[1] for x in kv], axis=1)
    return attend_rows(_q(sid, pos, dt)[None], kc, vc, np.array([pos]), SCALE)[0]


def _engine(dt, bs, chunk, budget, nb, share, steps, seed):
    rng = np.random.default_rng(seed)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    mb = 64 // bs
    sched = pkv.Scheduler(nb, bs, chunk, budget, 6, mb, share)
    if dt == "e4m3":
        kc = torch.full((nb, bs, HKV, D), 0x7F, dtype=torch.uint8, device=DEV)
        vc = torch.full((nb, bs, HKV, D), 0x7F, dtype=torch.uint8, device=DEV)
    else:
        kc = torch.full((nb, bs, HKV, D), float("nan"), dtype=tdt, device=DEV)
        vc = torch.full((nb, bs, HKV, D), float("nan"), dtype=tdt, device=DEV)
    tok = Tokens()
    reqs = [(0, 11, 3), (1, 11, 3), (2, 7, -1), (3, 37, 3), (4, 2, -1), (5, 9, -1), (6, 37, 3)]
    for sid, plen, grp in reqs:
        sched.add(sid, plen, grp)
        tok.add(sid, plen, grp)
    nxt = 1000
    st = {"rows": 0, "prefill_rows": 0, "preempt": 0, "copies": 0, "err": 0.0}
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    for _ in range(steps):
        ev = rng.random()
        pre, _, _, running = sched.stats_tuple()
        live = [s for s in list(tok.known) if sched.seq_info(s)[0] == 1]
        if ev < 0.08 and live and running < 6:
            src = int(rng.choice(live))
            n_tok = sched.seq_info(src)[1]
            sched.fork(src, nxt)
            tok.fork(src, nxt, n_tok)
            nxt += 1
        elif ev < 0.14 and live:
            sid = int(rng.choice(live))
            n_tok = sched.seq_info(sid)[1]
            if n_tok > 2:
                n = int(rng.integers(2, n_tok + 1))
                sched.trim(sid, n)
                tok.trim(sid, n)
        p = sched.step()
        st["preempt"] += len(p.preempted)
        st["copies"] += len(p.copies)
        if p.copies:
            pkv.copy_blocks(p.copies, kc, vc)
        if p.seq_ids:
            T = p.cu_seqlens[-1]
            q = np.zeros((T, HQ, D), np.float32)
            kn = np.zeros((T, HKV, D), np.float32)
            vn = np.zeros((T, HKV, D), np.float32)
            rows = []
            for sid, n, c in zip(p.seq_ids, p.n_new, p.ctx_lens):
                for pos in range(c - n, c):
                    t = len(rows)
                    q[t] = _q(sid, pos, dt)
                    kn[t], vn[t] = _kv(tok.key(sid, pos), dt)
                    rows.append((sid, pos, n > 1))
            bt = np.full((len(p.seq_ids), mb), -1, np.int32)
            for b, tab in enumerate(p.block_tables):
                bt[b, :len(tab)] = tab
            args = (torch.from_numpy(q).to(DEV, tdt), torch.from_numpy(kn).to(DEV, tdt),
                    torch.from_numpy(vn).to(DEV, tdt), np.asarray(p.slots, np.int32), kc, vc,
                    torch.from_numpy(bt).to(DEV), p.ctx_lens, p.cu_seqlens, SCALE)
            if dt == "e4m3":
                out = pkv.write_kv_attention_fp8(*args, K_SCALE, V_SCALE, workspace=ws)
            else:
                out = pkv.write_kv_attention(*args, workspace=ws)
            got = out.cpu().numpy().astype(np.float64)
            for t, (sid, pos, pre_row) in enumerate(rows):
                err = float(np.abs(got[t] - _dense(tok, sid, pos, dt)).max())
                assert err <= TOL[dt], (dt, sid, pos, err)
                st["err"] = max(st["err"], err)
                st["rows"] += 1
                st["prefill_rows"] += pre_row
        fin = [i for i in p.seq_ids if rng.random() < 0.05]
        sched.complete(fin)
        assert sched.check()
    return st


@pytest.mark.parametrize("dt", ["bf16", "f32", "e4m3"])
@pytest.mark.parametrize("cfg", [dict(bs=4, chunk=16, budget=24, nb=30, share=True),
                                 dict(bs=16, chunk=40, budget=64, nb=9, share=True),
                                 dict(bs=1, chunk=5, budget=12, nb=120, share=False)],
                         ids=["bs4-tight", "bs16-tight", "bs1"])
def test_engine_rows_equal_dense_attention_whatever_the_schedule(dt, cfg):
    tot = {"rows": 0, "prefill_rows": 0, "preempt": 0, "copies": 0}
    for seed in range(2):
        st = _engine(dt, steps=40, seed=seed, **cfg)
        print(f"[engine] {dt} {cfg} seed {seed}: {st}", flush=True)
        for k in tot:
            tot[k] += st[k]
    assert tot["rows"] > 100 and tot["prefill_rows"] > 20
