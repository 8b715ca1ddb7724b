#!/usr/bin/env python3
"""Benchmark of the paged-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--extra A,B]

One step = one pass of the whole path over one synthetic batch: the step's slot mapping on the
host (pkv_slot_mapping_step), then one pkv_write_kv_attention_shared call (E4M3 pools:
pkv_write_kv_attention_fp8) with the step's host block tables: host work planning (a decode
split whose blocks several rows share is read once per group of rows), one host-to-device copy
of the slots and work lists, the KV append, the prefill tiles, the decode split pass and the
split merge. Inputs
are resident in HBM before timing starts; the timed region is bracketed by device
synchronisation. The headline workload is the batched bf16 decode step (64 sequences,
lognormal lengths with median 2048, Hq 32, Hkv 8, D 128, block 16), reported as algorithmic
GB/s (KV bytes read + append bytes moved, per step time). The mixed ragged step
(8 x 512-row prefill chunks + 120 decodes) is reported alongside in tokens/s, and the same
batched decode step over E4M3 pools with per-tensor scales (pkv_write_kv_attention_fp8; its
bytes counted at one byte per cached element).

The long-context decode step (8 x 40960 keys, G 8, block 32; also over E4M3 pools) and the
prefix-shared group decode step (16 groups x 8 samples sharing a 2048-token prompt) are timed
the same way; decode-only
steps carry a `roofline` object for their decode kernel (the prefix-shared step also on unique
bytes). Each workload also gets the flushed-cache protocol (median, p10 and p90 of HIP-event
step times over `--protocol-reps` reps, each after a 2 GiB scratch write that evicts L2 and the
MALL) and bitwise invariance verdicts (sampled sequences alone, and for shared prompts each
group, against the batched step). The cpu_baseline leg times the oracle on the headline
workload and compares the oracle's rows with sampled GPU rows of every timed workload
(`parity_vs_oracle`).

Order per workload: build the step (host work, the GPU idle); 64 untimed steps (the first steps
after the set-up run up to twice as long, steady from about the 50th); the untimed pass that
brackets every kernel; the W warm-up steps and the K timed steps; the cold-cache pass, the
protocol and the invariance checks.

Prints ONE JSON line (rank 0, N = 1). `--gpus N` with N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
EVENT_STRIDE = 5                 # timed steps per step whose dominant kernel is bracketed
SETTLE_STEPS = 64                # untimed steps after a workload's set-up, before any figure
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="batched-bf16-decode")
    ap.add_argument("--extra", default="mixed-ragged-step,long-context-decode,"
                                       "prefix-shared-decode,batched-fp8-decode,mixed-fp8-step,"
                                       "long-context-fp8-decode",
                    help="comma-separated workloads timed the same way, reported under 'extra'")
    ap.add_argument("--protocol-reps", type=int, default=50,
                    help="reps of the flushed-cache protocol per workload (median, p10, p90 of "
                         "HIP-event step times, a 2 GiB scratch write before each rep); 0: off")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--consistent", default="batched-bf16-decode,mixed-ragged-step",
                    help="comma-separated workloads also timed in the phase-consistent mode, "
                         "reported under 'extra' as '<name>/phase-consistent'")
    ap.add_argument("--consistent-split", type=int, default=4096,
                    help="kv_split of the phase-consistent runs (the tile path's KV split; "
                         "4096 is the fastest of 2048 / 4096 / 8192 on both default "
                         "consistent workloads)")
    ap.add_argument("--kernel-events", choices=("timed", "separate"), default="timed",
                    help="take the per-kernel HIP-event times inside the timed steps (default) "
                         "or in a second pass of the same steps")
    ap.add_argument("--stream-reference", action="store_true",
                    help="only time torch's 2 GiB device copy and float32 sum (HBM rate "
                         "references) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device copies (scale reference for PMC byte "
                         "counters) and exit")
    return ap.parse_args()


def copy_calibration(reps=5, nbytes=1 << 30):
    """Plain device-to-device copies of known size: FETCH_SIZE / WRITE_SIZE per copy dispatch
    over nbytes gives the factor that turns those counters into HBM bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_per_copy": nbytes, "reps": reps,
                                           "kib_per_copy": nbytes / 1024}}))


def stream_reference(reps=20, nbytes=2 << 30):
    """Bandwidth that torch's own device streams reach on this GPU, as a reference for the
    kernels' HBM rates: a copy of nbytes (read + write) and a float32 sum over nbytes (read),
    each averaged over reps launches between two HIP events."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e-3

    t_copy = timed(lambda: y.copy_(x))
    t_sum = timed(lambda: x.sum())
    print(json.dumps({"stream_reference": {
        "bytes": nbytes, "reps": reps,
        "copy_us": t_copy * 1e6, "copy_tbs_read_plus_write": 2 * nbytes / t_copy / 1e12,
        "sum_us": t_sum * 1e6, "sum_tbs_read": nbytes / t_sum / 1e12}}))


def _step_inputs(w, gst):
    """Host arrays the step's slot mapping needs (prior lengths and new-row counts)."""
    import numpy as np
    starts = (w.ctx_lens - w.q_lens).astype(np.int32)
    return starts, w.q_lens.astype(np.int32)


def _kv_bytes(w):
    from prefill_slot_mapping_amd import accounting as acc
    return acc.decode_kv_bytes(w.ctx_lens, w.spec.Hkv, w.spec.D, w.kv_elem_bytes)


def _sample_rows(w, seed=11):
    """Sequences and query rows whose outputs are compared with the oracle: four decode
    sequences, the longest sequence and two prefill segments, a few rows of each."""
    import numpy as np
    rng = np.random.default_rng(seed)
    dec = [b for b in range(w.B) if w.q_lens[b] == 1]
    pre = [b for b in range(w.B) if w.q_lens[b] > 1]
    seqs = set(rng.choice(dec, size=min(4, len(dec)), replace=False).tolist()) if dec else set()
    seqs.add(int(np.argmax(w.ctx_lens)))
    if pre:
        seqs |= set(rng.choice(pre, size=min(2, len(pre)), replace=False).tolist())
    rows = []
    for b in sorted(seqs):
        lo, hi = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        rows += sorted(set([lo, hi - 1, (lo + hi) // 2] +
                           rng.integers(lo, hi, size=min(3, hi - lo)).tolist()))
    return sorted(int(b) for b in seqs), rows


def _invariance(w, gst, out, split, phase_consistent):
    """Bitwise verdicts of the step's rows against the same rows computed in other batches:
    each sequence of a sample alone (all sequences of a prefix-sharing step, each also with
    its group), through the attention entry point on the same pools."""
    import numpy as np
    import torch
    import prefill_slot_mapping_amd as pkv
    s = w.spec
    full = out.detach().cpu().numpy()

    def run(seqs):
        seqs = list(seqs)
        rows = np.concatenate([np.arange(w.cu_seqlens_q[b], w.cu_seqlens_q[b + 1])
                               for b in seqs]).astype(np.int64)
        cu = np.concatenate([[0], np.cumsum([w.q_lens[b] for b in seqs])]).astype(np.int32)
        q = gst.q.index_select(0, torch.from_numpy(rows).to(gst.q.device)).contiguous()
        bt = gst.block_tables_dev[torch.as_tensor(seqs, device=gst.q.device)].contiguous()
        ctx = np.asarray([w.ctx_lens[b] for b in seqs], np.int32)
        if w.kv_fp8:
            o = pkv.attention_fp8(q, gst.k_cache, gst.v_cache, bt, ctx, cu, w.scale, s.k_scale,
                                  s.v_scale, kv_split=split, phase_consistent=phase_consistent)
        else:
            o = pkv.attention(q, gst.k_cache, gst.v_cache, bt, ctx, cu, w.scale, kv_split=split,
                              phase_consistent=phase_consistent)
        return rows, o.cpu().numpy()

    live = [b for b in range(w.B) if w.q_lens[b] > 0]
    if (w.group_of >= 0).any():
        alone = live
    else:
        rng = np.random.default_rng(5)
        alone = sorted(set(rng.choice(live, size=min(8, len(live)), replace=False).tolist())
                       | {int(np.argmax(w.ctx_lens))} | {b for b in live if w.q_lens[b] > 1})
    bad_alone = 0
    for b in alone:
        rows, o = run([b])
        bad_alone += int(not np.array_equal(o.view(np.uint32), full[rows].view(np.uint32)))
    verdict = {"alone_vs_batch": {"sequences": len(alone), "bitwise_equal": len(alone) - bad_alone}}
    groups = sorted(set(int(g) for g in w.group_of if g >= 0))
    if groups:
        bad = 0
        for g in groups:
            rows, o = run(np.flatnonzero(w.group_of == g).tolist())
            bad += int(not np.array_equal(o.view(np.uint32), full[rows].view(np.uint32)))
        verdict["group_vs_batch"] = {"groups": len(groups), "bitwise_equal": len(groups) - bad}
    verdict["all_bitwise"] = all(v.get("bitwise_equal") == v.get("sequences", v.get("groups"))
                                 for v in verdict.values() if isinstance(v, dict))
    return verdict


def _clean_scratch(n_floats, device):
    """A scratch buffer for cache eviction, written once and then read once, so that none of
    its lines is still dirty in L2 or the MALL when the reads that evict start."""
    import torch
    buf = torch.ones(n_floats, dtype=torch.float32, device=device)
    buf.sum()
    torch.cuda.synchronize(device)
    return buf


def _evict(buf):
    """Read the whole scratch buffer (a reduction): evicts L2 and the 256 MB MALL. A write
    would leave its lines dirty there, and their write-back would then compete with the step
    that follows for HBM bandwidth."""
    buf.sum()


def _protocol(step, reps, device, value_of):
    """Flushed-cache timing: before each rep a 2 GiB scratch write evicts L2 and the 256 MB
    MALL (and keeps the GPU busy while the host enqueues the step); HIP events on the stream
    bracket the step. Returns the median and p10 / p90 of the reps."""
    import numpy as np
    import torch
    flush = torch.empty(1 << 29, dtype=torch.float32, device=device)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for i in range(reps):
        flush.fill_(float(i))
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize(device)
    ms = np.array([a.elapsed_time(z) for a, z in evs])
    del flush
    p10, med, p90 = (float(x) for x in np.percentile(ms, [10, 50, 90]))
    return {"reps": reps, "flush_bytes": 1 << 31, "median_ms": med, "p10_ms": p10,
            "p90_ms": p90, "median_value": value_of(med), "p10_value": value_of(p90),
            "p90_value": value_of(p10)}


def time_workload(name, steps, warmup, device="cuda:0", phase_consistent=False,
                  kernel_events="timed", cold_steps=20, kv_split=None, protocol_reps=0):
    """Build the step, then time `steps` whole steps; returns a result dict. With
    phase_consistent the attention runs with PKV_ATTN_PHASE_CONSISTENT (decode rows on the
    prefill tile path, bitwise equal to the same tokens inside prefill chunks)."""
    import numpy as np
    import torch
    import prefill_slot_mapping_amd as pkv
    from prefill_slot_mapping_amd import accounting as acc
    from prefill_slot_mapping_amd.harness import build_gpu_step
    from workloads import ALL_CONFIGS, make_workload

    w = make_workload(ALL_CONFIGS[name])
    split = w.spec.kv_split if kv_split is None else kv_split
    t_build = time.time()
    gst = build_gpu_step(w, device=device)
    t_build = time.time() - t_build
    s = w.spec
    starts, n_new = _step_inputs(w, gst)
    slots_np = np.zeros(max(w.T, 1), dtype=np.int32)
    ctx_np = np.ascontiguousarray(w.ctx_lens, dtype=np.int32)
    cu_np = np.ascontiguousarray(w.cu_seqlens_q, dtype=np.int32)
    bt_np = np.ascontiguousarray(gst.block_tables, dtype=np.int32)
    if w.kv_fp8:
        ws_bytes = pkv.write_kv_attention_fp8_workspace_size(ctx_np, cu_np, s.Hq, s.Hkv, s.D,
                                                             w.T, split, phase_consistent)
    else:
        ws_bytes = pkv.write_kv_attention_shared_workspace_size(
            ctx_np, cu_np, s.Hq, s.Hkv, s.D, w.T, bt_np, s.BS, split,
            pkv.PKV_BF16 if s.dtype == "bf16" else pkv.PKV_F32, phase_consistent)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
    out = torch.empty((w.T, s.Hq, s.D), dtype=torch.float32, device=device)

    def step():
        # host slot mapping of the step's new rows, then one library call: the slots and the
        # attention work lists go to the device in one copy, then append, attention, merge
        sl = pkv.slot_mapping_step(gst.allocator, bt_np, s.BS, starts, n_new, out=slots_np)
        if w.kv_fp8:
            pkv.write_kv_attention_fp8(gst.q, gst.k_new, gst.v_new, sl, gst.k_cache, gst.v_cache,
                                       gst.block_tables_dev, ctx_np, cu_np, w.scale, s.k_scale,
                                       s.v_scale, out=out, workspace=workspace,
                                       kv_split=split, phase_consistent=phase_consistent)
            return
        # the host copy of the tables lets the planner read a split shared by several rows
        # (a common prompt's blocks) once per group of rows; same bits as per-row reads
        pkv.write_kv_attention_shared(gst.q, gst.k_new, gst.v_new, sl, gst.k_cache,
                                      gst.v_cache, gst.block_tables_dev, bt_np, ctx_np, cu_np,
                                      w.scale, out=out, workspace=workspace, kv_split=split,
                                      phase_consistent=phase_consistent)

    # After the set-up (seconds of host work, the GPU idle) the first steps run up to twice as
    # long and the next few dozen 10-20 % longer (measured on the long-context and mixed steps:
    # steady from about the 50th step). SETTLE_STEPS untimed steps come first, then the
    # untimed pass that brackets every kernel, then the W warm-up and the K timed steps, so
    # that every figure is taken in the steady state whatever the warm-up count.
    dominant = "decode" if (w.q_lens == 1).any() and not phase_consistent else "prefill"
    # a decode pass may be two launches (per-row items, group items): both are bracketed
    dominant_kinds = [dominant, "decode_group"] if dominant == "decode" else [dominant]
    # long-lived objects (torch, the workload) go to the permanent generation, as serving
    # loops do after start-up, so a collection inside the loop does not walk all of them; done
    # here, not between the warm-up and the timed steps, where its tens of milliseconds of host
    # work would leave the GPU idle again
    gc.collect()
    gc.freeze()
    for _ in range(SETTLE_STEPS):
        step()
    kinds = ("write_kv", "prefill", "decode", "merge", "decode_group")
    pkv.profile_set_kinds(list(kinds))
    pkv.profile_enable(True)
    for _ in range(steps):
        step()
    kern = {k: pkv.profile_read(k) for k in kinds}
    dspan = pkv.profile_read_span(["decode", "decode_group"])
    pkv.profile_enable(False)
    torch.cuda.synchronize(device)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(device)
    gc_pauses = []

    def on_gc(phase, info, _t=[0.0]):
        if phase == "start":
            _t[0] = time.perf_counter()
        else:
            gc_pauses.append(time.perf_counter() - _t[0])

    # The dominant kernel's device time is taken inside the timed steps: the library brackets
    # its launch with HIP events on the launch stream in every EVENT_STRIDE-th step (an event
    # record costs the stream a few microseconds, so bracketing every launch of every kernel
    # would stretch the step it times). Every kernel's time came from the untimed pass above,
    # with all launches bracketed.
    gc.callbacks.append(on_gc)
    if kernel_events == "timed":
        pkv.profile_set_kinds([])
        pkv.profile_enable(True)
    torch.cuda.synchronize(device)
    stage0 = pkv.staging_info()
    host_ends = []
    t0 = time.perf_counter()
    for i in range(steps):
        if kernel_events == "timed":
            pkv.profile_set_kinds(dominant_kinds if i % EVENT_STRIDE == 0 else [])
        step()
        host_ends.append(time.perf_counter())
    torch.cuda.synchronize(device)
    dt = time.perf_counter() - t0
    stage1 = pkv.staging_info()
    gc.callbacks.remove(on_gc)
    gc.unfreeze()
    host_ms = np.diff(np.array([t0] + host_ends)) * 1e3
    timed = {}
    if kernel_events == "timed":
        # the decode pass of a bracketed step: its per-row launch and any group launch beside
        # it, from the first start to the last end
        tms, tn = pkv.profile_read_span(dominant_kinds)
        gn = pkv.profile_read("decode_group")[1] if dominant == "decode" else 0
        timed = {"kernel": dominant, "launches_bracketed": tn,
                 "avg_ms": tms / tn if tn else None, "group_launches": gn}
    assert np.array_equal(slots_np[:w.T], gst.new_slots)
    ms_step = dt / steps * 1e3

    # Cold caches: before each of these steps a 1 GiB scratch read evicts L2 and the 256 MB
    # MALL, so the dominant kernel reads its K/V from HBM; its events give the cold time
    # (untimed passes, not part of ms_per_step). A read leaves no dirty lines behind; after a
    # scratch write (also measured, the protocol's flush), up to 256 MB of dirty MALL lines are
    # written back while the step reads, which the step's own traffic does not include.
    cold = {}
    if cold_steps > 0:
        def cold_pass(evict_read):
            scratch = (_clean_scratch(1 << 28, device) if evict_read else
                       torch.empty(1 << 28, dtype=torch.float32, device=device))
            pkv.profile_set_kinds(dominant_kinds)
            pkv.profile_enable(True)
            for i in range(cold_steps):
                if evict_read:
                    _evict(scratch)
                else:
                    scratch.fill_(float(i))
                step()
            cms, cn = pkv.profile_read_span(dominant_kinds)
            pkv.profile_enable(False)
            torch.cuda.synchronize(device)
            del scratch
            return cms / cn if cn else None, cn
        ms_r, n_r = cold_pass(True)
        ms_w, _ = cold_pass(False)
        cold = {"kernel": dominant, "launches": n_r, "avg_ms": ms_r, "flush_bytes": 1 << 30,
                "evict": "scratch read", "avg_ms_after_scratch_write": ms_w}

    kv = _kv_bytes(w)
    app0 = acc.append_bytes(w.T, s.Hkv, s.D, w.elem_bytes, w.kv_elem_bytes)
    decode_only0 = bool((w.q_lens <= 1).all())

    def value_of(ms):
        # decode-only steps: GB/s of KV read + append; steps with prefill rows: tokens/s
        return (kv + app0) / (ms * 1e-3) / 1e9 if decode_only0 else w.T / (ms * 1e-3)

    proto = _protocol(step, protocol_reps, device, value_of) if protocol_reps > 0 else None
    inv = _invariance(w, gst, out, split, phase_consistent)
    seqs_s, rows_s = _sample_rows(w)
    sample = {"seqs": seqs_s, "rows": rows_s,
              "gpu": out[rows_s].detach().cpu().numpy().astype("float64")}
    app = acc.append_bytes(w.T, s.Hkv, s.D, w.elem_bytes, w.kv_elem_bytes)
    decode_rows = w.q_lens == 1
    decode_only = bool((w.q_lens <= 1).all())
    uq = acc.unique_kv_bytes(gst.block_tables, w.ctx_lens, s.BS, s.Hkv, s.D, w.kv_elem_bytes)
    dec_kv = acc.decode_kv_bytes(w.ctx_lens[decode_rows], s.Hkv, s.D, w.kv_elem_bytes)
    flops = acc.attention_flops(w.ctx_lens[~decode_rows], w.q_lens[~decode_rows], s.Hq, s.D)
    res = {
        "workload": name, "phase_consistent": phase_consistent, "kv_split": split,
        "B": w.B, "T": w.T,
        "kv_dtype": s.kv_dtype or s.dtype,
        "ms_per_step": ms_step,
        "step_gbs": (kv + app) / (ms_step * 1e-3) / 1e9, "tokens_per_s": w.T / (ms_step * 1e-3),
        "kv_bytes": kv, "append_bytes": app, "decode_kv_bytes": dec_kv, "prefill_flops": flops,
        # distinct cached bytes (a block shared by several sequences counted once) and, for
        # decode-only steps, the rate they give over the decode kernel's time
        "unique_kv_bytes": uq,
        "decode_unique_gbs": (uq / (dspan[0] / dspan[1] * 1e-3) / 1e9
                              if decode_only and dspan[1] else None),
        "build_s": t_build,
        "host_enqueue_ms": {"median": float(np.median(host_ms)), "max": float(host_ms.max())},
        "gc_pauses_in_timed_region": {"count": len(gc_pauses),
                                      "max_ms": max(gc_pauses, default=0.0) * 1e3},
        "kernels_ms": {k: (v[0] / v[1] if v[1] else None) for k, v in kern.items()},
        # the decode pass per step: from the first start to the last end of its per-row
        # launch and its group launch (when there is one, on the second stream beside it)
        "decode_pass_ms": dspan[0] / dspan[1] if dspan[1] else None,
        "timed_region_kernel": timed,
        "cold_cache_kernel": cold,
        "kernel_launches": {k: v[1] for k, v in kern.items()},
        "staging_allocations_in_timed_region": stage1[1] - stage0[1],
        "staging_slot_bytes": stage1[0],
        "protocol": proto,
        "protocol_unit": "GB/s" if decode_only0 else "tokens/s",
        "invariance": inv,
    }
    t_roof = max((kv + app) / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    res["roofline_frac_step"] = t_roof / (ms_step * 1e-3)
    res["_gst"] = gst
    res["_w"] = w
    res["_out"] = out
    res["_sample"] = sample
    return res


def oracle_parity(samples):
    """Part of the cpu_baseline leg: for each timed workload, the oracle's rows for the
    sampled sequences against the GPU rows copied out of that workload's last timed step.
    Returns {workload: {rows, max_abs_err, tolerance, within}}."""
    import numpy as np
    from oracle import build_oracle_step
    out = {}
    for key, (w, smp) in samples.items():
        st = build_oracle_step(w, seqs=smp["seqs"], poison=False)
        ref = st.attention(rows=smp["rows"])[smp["rows"]]
        err = float(np.abs(smp["gpu"] - ref).max()) if len(smp["rows"]) else 0.0
        tol = 2e-3 if w.spec.dtype == "bf16" else 1e-5
        out[key] = {"rows": len(smp["rows"]), "sequences": len(smp["seqs"]),
                    "max_abs_err": err, "tolerance": tol,
                    "within": bool(np.isfinite(smp["gpu"]).all() and err <= tol)}
    return out


def cpu_baseline(w, budget_s, gpu_out=None):
    """The oracle as it stands, on a bounded sample of the same workload's rows; with gpu_out
    (the last timed step's output) the sampled rows are also compared with the GPU's."""
    import numpy as np
    from oracle import build_oracle_step
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    order = list(range(w.B))
    # calibrate on the first sequence, then take as many as fit the budget
    per_token = None
    chosen = []
    est = 0.0
    for b in order:
        if w.q_lens[b] == 0:
            continue
        if per_token is not None and est + per_token * int(w.ctx_lens[b]) * int(w.q_lens[b]) > budget_s:
            continue
        chosen.append(b)
        if per_token is None:
            st = build_oracle_step(w, seqs=[b], poison=False)
            t = time.perf_counter()
            st.attention(rows=range(int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])))
            el = time.perf_counter() - t
            per_token = el / (int(w.ctx_lens[b]) * int(w.q_lens[b]))
            est += el
        else:
            est += per_token * int(w.ctx_lens[b]) * int(w.q_lens[b])
    st = build_oracle_step(w, seqs=chosen, poison=False)
    rows = [r for b in chosen for r in range(int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1]))]
    # repeat the sample until about `budget_s` of CPU work has been timed
    reps = 0
    t = time.perf_counter()
    while True:
        ref = st.attention(rows=rows)
        reps += 1
        spent = time.perf_counter() - t
        if spent >= 0.66 * budget_s or spent / reps * (reps + 1) > budget_s:
            break
    from prefill_slot_mapping_amd import accounting as acc
    kv_done = reps * acc.decode_kv_bytes(w.ctx_lens[chosen], w.spec.Hkv, w.spec.D, w.elem_bytes)
    sample = f"{len(chosen)} of {w.B} sequences ({len(rows)} query rows, " \
             f"{int(w.ctx_lens[chosen].sum())} cached tokens) x {reps} passes, float64 " \
             f"per-row oracle"
    parity = None
    if gpu_out is not None:
        got = gpu_out[rows].detach().cpu().numpy().astype(np.float64)
        parity = {"rows": len(rows), "max_abs_err": float(np.abs(got - ref[rows]).max()),
                  "tolerance": 2e-3 if w.spec.dtype == "bf16" else 1e-5}
    return {"value": kv_done / spent / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle", "sample": sample, "seconds": spent,
            "affinity_cores": len(os.sched_getaffinity(0)), "parity_vs_gpu": parity}


def _traffic_for(workload):
    """HBM bytes per launch of the workload's decode kernel (FETCH_SIZE + WRITE_SIZE, each
    scaled by what the counter reads for a plain copy of known size) from the committed
    rocprofv3 PMC summary, or None when that kernel's source has changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        ent = rec[workload]
        src_path = ent.get("kernel_source") or rec["kernel_source"]
        sha = ent.get("kernel_sha256") or rec["kernel_sha256"]
        src = open(os.path.join(ROOT, src_path), "rb").read()
        if sha != hashlib.sha256(src).hexdigest():
            return None
        return ent["hbm_bytes"]
    except (OSError, KeyError, ValueError):
        return None


def _decode_roofline(res, name, kernel):
    """Roofline object of a result's decode kernel: algorithmic KV bytes / its average launch
    in the timed steps; the cold-cache launch (L2 and MALL flushed first) is given beside it."""
    tr = res["timed_region_kernel"]
    ms = tr.get("avg_ms") if tr.get("kernel") == "decode" else res["decode_pass_ms"]
    achieved = res["decode_kv_bytes"] / (ms * 1e-3) / 1e9 if ms else None
    cold = res.get("cold_cache_kernel") or {}
    cms = cold.get("avg_ms") if cold.get("kernel") == "decode" else None
    wms = cold.get("avg_ms_after_scratch_write") if cold.get("kernel") == "decode" else None
    kvb = res["decode_kv_bytes"]
    r = {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS if achieved else None,
         "traffic": _traffic_for(name), "bytes_per_launch": kvb,
         "avg_launch_ms": ms,
         "cold_cache": {"evict": "1 GiB scratch read", "avg_launch_ms": cms,
                        "achieved": kvb / (cms * 1e-3) / 1e9 if cms else None,
                        "frac": kvb / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS if cms else None,
                        "after_scratch_write": {
                            "avg_launch_ms": wms,
                            "frac": kvb / (wms * 1e-3) / 1e9 / HBM_PEAK_GBS if wms else None}}}
    uq = res["unique_kv_bytes"]
    if uq != res["decode_kv_bytes"] and ms:
        # blocks shared by several sequences: `achieved` counts every sequence's reads
        # (logical bytes); this counts each distinct cached byte once
        r["logical_bytes_per_launch"] = res["decode_kv_bytes"]
        r["unique"] = {"bytes_per_launch": uq, "achieved": uq / (ms * 1e-3) / 1e9,
                       "frac": uq / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "cold_cache_frac": uq / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS if cms else None}
    return r


def _decode_kernel_name(w):
    """The decode kernel a decode-only workload runs on (its group and pool type)."""
    return "decode_mfma_kernel" if (w.kv_fp8 or w.spec.dtype == "bf16") else "decode_f32_kernel"


def _clocks():
    """Current GPU clocks as rocm-smi reports them (a child process), or None. The script is
    handed to this interpreter directly: its `#!/usr/bin/env` line would make the child replace
    itself once more, which profilers that set up the GPU in every process do not allow."""
    import shutil
    import subprocess
    smi = shutil.which("rocm-smi")
    if smi is None:
        return None
    try:
        r = subprocess.run([sys.executable, os.path.realpath(smi), "--showclocks", "--json"],
                           capture_output=True, text=True, timeout=30)
        if r.returncode != 0:
            return None
        d = json.loads(r.stdout[r.stdout.index("{"):])
        card = next(iter(d.values()))
        return {k: v for k, v in card.items() if "clock" in k.lower() or "level" in k.lower()}
    except (OSError, ValueError, StopIteration, subprocess.SubprocessError):
        return None


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1 "
                                   "(sharding across GPUs is not run)"}))
        sys.exit(2)
    import torch
    import prefill_slot_mapping_amd as pkv
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.stream_reference:
        stream_reference()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    pkv.lib()   # fail loudly if the HIP library is not built

    samples = {}
    print(f"[bench] {args.workload}", file=sys.stderr, flush=True)
    main_res = time_workload(args.workload, args.steps, args.warmup,
                             kernel_events=args.kernel_events, protocol_reps=args.protocol_reps)
    w = main_res["_w"]
    samples[args.workload] = (w, main_res.pop("_sample"))
    extra = {}
    for name in [n for n in args.extra.split(",") if n and n != args.workload]:
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        r = time_workload(name, args.steps, args.warmup, kernel_events=args.kernel_events,
                          protocol_reps=args.protocol_reps)
        if r["decode_kv_bytes"] and not (r["_w"].q_lens > 1).any():
            r["roofline"] = _decode_roofline(r, name, _decode_kernel_name(r["_w"]))
        samples[name] = (r["_w"], r.pop("_sample"))
        r.pop("_gst"); r.pop("_w"); r.pop("_out")
        extra[name] = r
        torch.cuda.empty_cache()

    for name in [n for n in args.consistent.split(",") if n]:
        print(f"[bench] {name}/phase-consistent", file=sys.stderr, flush=True)
        r = time_workload(name, args.steps, args.warmup, phase_consistent=True,
                          kernel_events=args.kernel_events, kv_split=args.consistent_split,
                          protocol_reps=args.protocol_reps)
        samples[name + "/phase-consistent"] = (r["_w"], r.pop("_sample"))
        r.pop("_gst"); r.pop("_w"); r.pop("_out")
        extra[name + "/phase-consistent"] = r
        torch.cuda.empty_cache()

    roofline = _decode_roofline(main_res, args.workload, _decode_kernel_name(w))
    clocks = _clocks()
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        # the cpu_baseline leg: the oracle timed on the host cores, and its rows compared
        # with every timed workload's sampled GPU rows
        print("[bench] cpu_baseline leg", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds, main_res["_out"])
        parity = oracle_parity(samples)
    main_res.pop("_gst")
    main_res.pop("_w")
    main_res.pop("_out")
    s = w.spec
    line = {
        "metric": "paged decode KV GB/s (% HBM peak); mixed ragged step tokens/s",
        "value": main_res["step_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": ("e4m3 KV, bf16 q" if w.kv_fp8 else s.dtype), "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "Hq": s.Hq, "Hkv": s.Hkv, "D": s.D,
                   "block_size": s.BS, "kv_split": s.kv_split, "kv_dtype": s.kv_dtype or s.dtype,
                   "cached_tokens": int(w.ctx_lens.sum()), "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "invariance": {k: v["invariance"]["all_bitwise"]
                       for k, v in [(args.workload, main_res)] + list(extra.items())},
        "gpu_clocks_after_timing": clocks,
        "detail": main_res,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
