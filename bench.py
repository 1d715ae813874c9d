#!/usr/bin/env python3
"""Benchmark: one rank's lap of ring attention on one MI355X.

A step is one whole lap: the empty state, P block steps (each block after the
rank's own arrives through an emulated ring transfer on a side stream), and the
finalize pass, on seeded synthetic bf16 inputs already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rank R] [--lap-only]

Prints ONE JSON line.  ``value`` is useful attention TFLOP/s: 4 * head_dim flops
per allowed (query, key) pair per query head, over the timed laps.  The
``roofline`` object prices the step kernel alone (its flops per launch over its
average launch time, from HIP events recorded around each launch on the compute
stream) against the MI355X dense bf16 MFMA peak; ``cpu_baseline`` times the
fp64 oracle on this host's cores over a bounded sample of the same workload.

On a bf16 workload the line's ``detail`` also holds, unless ``--lap-only`` (or only some of
them are named by flag): the HBM-bound passes (finalize, short KV blocks, the merge of shard
states), the backward lap, and the split-KV decode step, the last two each with the oracle
timed beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU (MI355X)
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "noncausal_n131072_p8_h32"
MASK_CODE = {"none": 0, "causal_contiguous": 1, "causal_striped": 2, "causal_zigzag": 3}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_bf16_traffic.txt")
STEP_SOURCE = os.path.join(ROOT, "exact_long_context_amd", "csrc", "ra_step_bf16.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    return hashlib.sha256(open(STEP_SOURCE, "rb").read()).hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per step-kernel launch from the committed rocprofv3 counter summary,
    or None if it is missing, for another workload, or older than the kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for ln in open(TRAFFIC_FILE):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha() or kv.get("workload") != workload:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, rank: int, q, k, v, seconds: float):
    """Time the fp64 oracle on this host over whole row chunks of one head (all keys)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    causal = w.mask != "none"
    q_pos = oracle.tokens_of_rank(w.N, w.P, w.layout, rank)
    k_pos = np.arange(w.N)
    g = 0
    q64 = q[0, 0:1].double().numpy()[None]
    k64 = k[0, g:g + 1].double().numpy()[None]
    v64 = v[0, g:g + 1].double().numpy()[None]
    chunk = 256 if w.N <= 262144 else 32    # keeps the fp64 score chunk near 256 MiB
    done_rows = 0
    flops = 0
    t0 = time.perf_counter()
    while done_rows < w.n_local and time.perf_counter() - t0 < seconds:
        rows = np.arange(done_rows, min(done_rows + chunk, w.n_local))
        oracle.dense_attention(q64, k64, v64, q_pos, k_pos, causal, rows=rows, row_chunk=chunk)
        pairs = oracle.live_pair_count(q_pos[rows], k_pos, causal)
        flops += 4 * w.head_dim * pairs
        done_rows += rows.size
    el = time.perf_counter() - t0
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "blas": host_blas(),
        "kind": "oracle",
        "sample": (f"fp64 dense attention (oracle.dense_attention) of head 0, local rows 0..{done_rows - 1} "
                   f"of rank {rank} against all {w.N} keys, {el:.1f} s; same useful-flop accounting"),
        "seconds": round(el, 3),
    }


def host_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def host_blas() -> str:
    """The BLAS library NumPy's fp64 products run on, as threadpoolctl names it."""
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                for i in threadpool_info() if i.get("user_api") == "blas"]
        return ", ".join(libs) if libs else "unknown"
    except Exception:
        return "unknown"


def cpu_backward_baseline(w, rank: int, j: int, q, kb, vb, d_out, seconds: float):
    """Time the fp64 oracle's backward step (oracle.backward_block) on this host: query head 0,
    whole chunks of local rows against all keys of block j, until `seconds` of timed work.
    Its inputs lse and D for those rows come from the oracle's own forward against that block
    (untimed).  Useful flops as on the GPU: 10*d per allowed pair."""
    import numpy as np
    import oracle
    causal = w.mask != "none"
    q_pos = oracle.tokens_of_rank(w.N, w.P, w.layout, rank)
    k_pos = oracle.tokens_of_rank(w.N, w.P, w.layout, j)
    k64 = kb[j][0:1, 0:1].double().cpu().numpy()
    v64 = vb[j][0:1, 0:1].double().cpu().numpy()
    chunk, done, flops, timed = 512, 0, 0, 0.0
    while done < w.n_local and timed < seconds:
        rows = np.arange(done, min(done + chunk, w.n_local))
        q64 = q[0:1, 0:1, done:done + rows.size].double().cpu().numpy()
        do64 = d_out[0:1, 0:1, done:done + rows.size].double().cpu().numpy()
        o, lse = oracle.dense_attention(q64, k64, v64, q_pos[rows], k_pos, causal)
        D = oracle.backward_row_terms(do64, o)
        t0 = time.perf_counter()
        oracle.backward_block(q64, k64, v64, do64, lse, D, q_pos[rows], k_pos, causal)
        timed += time.perf_counter() - t0
        flops += 10 * w.head_dim * oracle.live_pair_count(q_pos[rows], k_pos, causal)
        done += rows.size
    return {"value": round(flops / timed / 1e12, 5) if timed > 0 else 0.0, "unit": "TFLOP/s",
            "cores": host_threads(), "blas": host_blas(), "kind": "oracle",
            "sample": (f"fp64 oracle.backward_block of query head 0, local rows 0..{done - 1} of rank {rank} "
                       f"against the {k_pos.size} keys of block {j}, {timed:.1f} s timed; 10*d flops per allowed pair"),
            "seconds": round(timed, 3)}


def cpu_decode_baseline(seconds: float):
    """Time the fp64 oracle's block update (oracle.online_block_update) for one decode token of
    64 query heads over 8 KV heads (d = 128) against a 16K-key block on this host, repeated
    until `seconds`; reported in the decode unit, bf16 K+V bytes of the block per second."""
    import numpy as np
    import oracle
    import synth
    B, Hq, Hkv, d, nk = 1, 64, 8, 128, 16384
    sc = 1 / math.sqrt(128)
    q = synth.round_to_dtype(synth.draw(5, synth.Q_ID, 0, B, Hq, 1, d, sc), "bf16").double().numpy()
    k = synth.round_to_dtype(synth.draw(5, synth.K_ID, -1, B, Hkv, nk, d, sc), "bf16").double().numpy()
    v = synth.round_to_dtype(synth.draw(5, synth.V_ID, -1, B, Hkv, nk, d, sc), "bf16").double().numpy()
    st = oracle.online_state_init(B, Hq, 1, d)
    q_pos, k_pos = np.array([nk - 1]), np.arange(nk)
    calls, t0 = 0, time.perf_counter()
    while calls == 0 or time.perf_counter() - t0 < seconds:
        oracle.online_block_update(st, q, k, v, q_pos, k_pos, False)
        calls += 1
    el = time.perf_counter() - t0
    kv_bytes = 2 * B * Hkv * nk * d * 2
    return {"value": round(kv_bytes * calls / el / 1e9, 3), "unit": "GB/s",
            "cores": host_threads(), "blas": host_blas(), "kind": "oracle",
            "sample": (f"fp64 oracle.online_block_update, 1 token x 64 query heads over 8 KV heads against "
                       f"{nk} keys, {calls} calls in {el:.1f} s; K+V bytes as bf16"),
            "seconds": round(el, 3)}


def cpu_hbm_baselines(d: int, seconds: float):
    """The oracle's finalize, merge of 8 shard states and short-block update on this host:
    one head of 16384 query rows, fp64, each repeated for about `seconds`; reported in the
    same algorithmic bytes per second as the GPU passes (fp32 state, bf16 K/V)."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(3)
    n = 16384

    def state():
        return {"m": rng.standard_normal((1, 1, n)), "l": rng.random((1, 1, n)) + 1.0,
                "o": rng.standard_normal((1, 1, n, d))}

    def rate(fn, nbytes):
        calls, t0 = 0, time.perf_counter()
        while calls == 0 or time.perf_counter() - t0 < seconds:
            fn()
            calls += 1
        el = time.perf_counter() - t0
        return {"value": round(nbytes * calls / el / 1e9, 3), "unit": "GB/s", "calls": calls,
                "seconds": round(el, 3)}

    res = {}
    st = state()
    res["finalize"] = rate(lambda: oracle.online_finalize(st), n * (4 * d + 8) + n * (4 * d + 4))
    parts = [state() for _ in range(8)]
    res["merge_8_parts"] = rate(lambda: oracle.merge_states(parts), 8 * n * (4 * d + 8) + n * (4 * d + 4))
    q = rng.standard_normal((1, 1, n, d))
    for nk in (256, 1024):
        kk, vv = rng.standard_normal((1, 1, nk, d)), rng.standard_normal((1, 1, nk, d))
        nbytes = 2 * n * (4 * d + 8) + n * d * 2 + 2 * nk * d * 2
        res[f"step_nk{nk}"] = rate(lambda: oracle.online_block_update(st, q, kk, vv, np.arange(n),
                                                                      np.arange(nk), False), nbytes)
    return {"kind": "oracle", "cores": host_threads(), "blas": host_blas(),
            "sample": "fp64 oracle online_finalize, merge_states of 8 parts and online_block_update "
                      "(Nk 256, 1024) on one head of 16384 rows", "passes": res}


def hbm_passes(ra, q, k, v, ws, w, desc, reps: int = 20, cpu_seconds: float = 0.0):
    """The HBM-bound passes beside the lap: finalize over the lap's state, and block steps
    with short KV blocks (the state read and write then outweigh the MFMA work).  Each is
    timed with events on the current stream over `reps` launches; bytes are algorithmic."""
    import torch
    rows = w.batch * w.q_heads * w.n_local
    d = w.head_dim
    elem = q.element_size()
    res = {}

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = torch.empty((w.batch, w.q_heads, w.n_local, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((w.batch, w.q_heads, w.n_local), dtype=torch.float32, device=q.device)
    # a state finalizes once: one resumed handle on the lap's state per launch, made beforehand
    fin = [ra.RingState(q, k, w.P, workspace=ws, resume=True) for _ in range(reps + 1)]
    it = iter(fin)
    ms = timed(lambda: next(it).finalize(out, lse))
    for f in fin:
        f.close()
    st = ra.RingState(q, k, w.P, workspace=ws, resume=True)
    nbytes = rows * (4 * d + 8) + rows * (4 * d + 4)
    res["finalize"] = {"ms": round(ms, 4), "bytes": nbytes, "GB_s": round(nbytes / ms / 1e6, 1),
                       "frac_of_8TB_s": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)}
    for nk in (256, 512, 1024):
        kk, vv = k[:, :, :nk], v[:, :, :nk]
        ms = timed(lambda: st.step(kk, vv, 0))
        nbytes = 2 * rows * (4 * d + 8) + rows * d * elem + 2 * w.batch * w.kv_heads * nk * d * elem
        flops = 4 * d * w.n_local * nk * w.q_heads * w.batch
        res[f"step_nk{nk}"] = {"ms": round(ms, 4), "bytes": nbytes, "GB_s": round(nbytes / ms / 1e6, 1),
                               "frac_of_8TB_s": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3),
                               "TFLOP_s": round(flops / ms / 1e9, 1)}
    st.close()
    # the reduction of shard states (split-KV decode): 8 parts of this state's size, here
    # copies of the lap's state, into O and lse
    parts = [ws] + [ws.clone() for _ in range(7)]
    ms = timed(lambda: ra.merge_states(desc, parts, out=out, lse=lse))
    nbytes = len(parts) * rows * (4 * d + 8) + rows * (4 * d + 4)
    res["merge_8_parts"] = {"ms": round(ms, 4), "bytes": nbytes, "GB_s": round(nbytes / ms / 1e6, 1),
                            "frac_of_8TB_s": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)}
    del parts
    if cpu_seconds > 0:
        log("[bench] timing the oracle's HBM-bound passes on host cores")
        res["cpu_oracle"] = cpu_hbm_baselines(d, cpu_seconds)
    return res


def decode_passes(ra, reps: int = 20, cpu_seconds: float = 0.0):
    """The split-KV block step (ra_decode_step) for few query rows of the long-context GQA
    head shape (64 query heads over 8 KV heads, d = 128, bf16): one block of n_k keys per call
    into a resumed state, for blocks from one ring block (16K keys) to the whole 1M-token
    context.  Timed with events on the current stream over `reps` calls, beside the tiled
    ra_block_step on the same block.  Bytes are algorithmic: K and V once, Q, the state read
    and written, and the chunk states written and read back."""
    import torch
    import synth
    B, Hq, Hkv, d = 1, 64, 8, 128
    res = {}

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for n_q in (1, 8, 16):
        q = synth.draw_device(5, synth.Q_ID, 0, B, Hq, n_q, d, 1 / math.sqrt(128), "bf16", "cuda")
        for nk in (16384, 131072, 1048576):
            k = synth.draw_device(5, synth.K_ID, -1, B, Hkv, nk, d, 1 / math.sqrt(128), "bf16", "cuda")
            v = synth.draw_device(5, synth.V_ID, -1, B, Hkv, nk, d, 1 / math.sqrt(128), "bf16", "cuda")
            st = ra.RingState(q, k)
            ws = torch.empty(ra.decode_workspace_bytes(st.desc, nk), dtype=torch.uint8, device="cuda")
            st.decode_step(k, v, 0, workspace=ws)      # the state now holds a valid lap state
            ms = timed(lambda: st.decode_step(k, v, 0, workspace=ws))
            ms_tiled = timed(lambda: st.step(k, v, 0))
            st.close()
            rows = B * Hq * n_q
            kv_bytes = 2 * B * Hkv * nk * d * 2
            parts = ws.numel() // (rows * (d + 2) * 4) if rows else 0
            nbytes = kv_bytes + rows * d * 2 + 2 * rows * (d + 2) * 4 + 2 * parts * rows * (d + 2) * 4
            res[f"decode_q{n_q}_nk{nk}"] = {
                "ms": round(ms, 4), "bytes": nbytes, "GB_s": round(nbytes / ms / 1e6, 1),
                "frac_of_8TB_s": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3),
                "tiled_step_ms": round(ms_tiled, 4), "speedup_vs_tiled": round(ms_tiled / ms, 2)}
            del k, v, ws
    res.update(decode_lap_graph(ra, reps))
    if cpu_seconds > 0:
        log("[bench] timing the oracle decode update on host cores")
        res["cpu_oracle"] = cpu_decode_baseline(cpu_seconds)
    return res


def decode_lap_graph(ra, reps: int = 20, P: int = 8, nk: int = 16384):
    """A whole decode lap (P blocks of nk keys through ra_decode_step, then ra_finalize; the
    newest tokens at the end of the context, causal) issued eagerly from Python, against the
    same lap captured once in a HIP graph on the state's stream and replayed.  Short blocks
    leave the GPU waiting on the host's launches; the graph removes that wait."""
    import torch
    import synth
    B, Hq, Hkv, d = 1, 64, 8, 128
    N = P * nk
    res = {}
    s = torch.cuda.Stream()
    for n_q in (1, 8):
        q = synth.draw_device(6, synth.Q_ID, 0, B, Hq, n_q, d, 1 / math.sqrt(128), "bf16", "cuda")
        k = synth.draw_device(6, synth.K_ID, -1, B, Hkv, N, d, 1 / math.sqrt(128), "bf16", "cuda")
        v = synth.draw_device(6, synth.V_ID, -1, B, Hkv, N, d, 1 / math.sqrt(128), "bf16", "cuda")
        kb = [k[:, :, j * nk:(j + 1) * nk] for j in range(P)]
        vb = [v[:, :, j * nk:(j + 1) * nk] for j in range(P)]
        desc = ra.desc_for(q, kb[0], P, stream=s)
        ws = torch.empty(ra.decode_workspace_bytes(desc, nk), dtype=torch.uint8, device="cuda")
        state_ws = torch.empty(ra.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device="cuda")
        q_off = N - n_q

        def lap():
            st = ra.RingState(q, kb[0], ring_size=P, stream=s, workspace=state_ws)
            for j in range(P - 1, -1, -1):        # the diagonal block first, as rank P-1 visits them
                st.decode_step(kb[j], vb[j], 1, q_off, j * nk, workspace=ws)
            st.finalize(out=out, lse=lse)
            st.close()

        def timed(fn):
            with torch.cuda.stream(s):
                fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                for _ in range(reps):
                    fn()
                e1.record(s)
            s.synchronize()
            return e0.elapsed_time(e1) / reps

        ms_eager = timed(lap)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            lap()
        ms_graph = timed(g.replay)
        kv_bytes = 2 * B * Hkv * N * d * 2
        res[f"decode_lap_q{n_q}_p{P}x{nk}"] = {
            "eager_ms": round(ms_eager, 4), "graph_ms": round(ms_graph, 4),
            "graph_kv_GB_s": round(kv_bytes / ms_graph / 1e6, 1), "blocks": P, "keys_per_block": nk}
        del g
    return res


def backward_lap(ra, q, kb, vb, out, lse, w, rank, mask, order, step_flops, laps, cpu_seconds=0.0):
    """Time the backward lap: ra_bwd_init, one ra_bwd_block_step per block in ring order
    (each block's dK, dV accumulating in its own buffer), ra_bwd_finalize.  Useful flops:
    10*d per allowed pair (the five products of the standard backward: the recomputed scores,
    dP, dV, dK, dQ); the kernels recompute the scores and dP once more for the dQ side."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(1)
    d_out = torch.randn(q.shape, generator=g).to(q.dtype).to(q.device)
    dks = [torch.zeros(kb[j].shape, dtype=torch.float32, device=q.device) for j in range(w.P)]
    dvs = [torch.zeros(vb[j].shape, dtype=torch.float32, device=q.device) for j in range(w.P)]
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = torch.empty(ra.bwd_workspace_bytes(ra.desc_for(q, kb[0], w.P)), dtype=torch.uint8, device=q.device)

    def one():
        bw = ra.RingBackward(q, d_out, out, lse, kb[0], ring_size=w.P, workspace=ws)
        for j in order:
            qo, ko = ra.block_offsets(mask, rank, j, w.n_local, w.n_local)
            bw.step(kb[j], vb[j], dks[j], dvs[j], mask, qo, ko)
        bw.finalize(dq)
        bw.close()

    one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(laps):
        one()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / laps
    flops = sum(step_flops) // 4 * 10      # 10*d per pair (step_flops holds 4*d per pair)
    res = {"ms_per_lap": round(ms, 4), "useful_flops_per_lap": flops,
           "TFLOP_s": round(flops / ms / 1e9, 1), "pct_of_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS * 100, 2),
           "flop_convention": "10*d per allowed pair per query head"}
    if cpu_seconds > 0:
        log("[bench] timing the oracle backward on host cores")
        res["cpu_oracle"] = cpu_backward_baseline(w, rank, order[0], q, kb, vb, d_out, cpu_seconds)
    return res


def lap_timing(ring, qd, rank: int, mask: int, w, step_flops, warmup: int, laps: int, ws, out, lse):
    """Emulated laps with HIP events around each step's launch: (ms per lap by the host clock,
    step-kernel ms per live launch, useful TFLOP/s of the laps, of the step kernels)."""
    import torch
    for _ in range(warmup):
        ring.lap(qd, rank, mask, workspace=ws, out=out, lse=lse)
    events = []
    for _ in range(laps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * w.P)]
        for e in evs:
            e.record()
        events.append(evs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(laps):
        ring.lap(qd, rank, mask, workspace=ws, out=out, lse=lse, step_events=events[i])
    torch.cuda.synchronize()
    lap_s = (time.perf_counter() - t0) / laps
    live = [s for s in range(w.P) if step_flops[s] > 0]
    kern = [events[i][2 * s].elapsed_time(events[i][2 * s + 1]) for i in range(laps) for s in live]
    kern_ms = sum(kern) / max(len(kern), 1)
    lap_flops = sum(step_flops)
    return {
        "lap_ms": round(1000.0 * lap_s, 4),
        "useful_tflops_lap": round(lap_flops / lap_s / 1e12, 2),
        "step_kernel_ms_mean": round(kern_ms, 4),
        "step_kernel_tflops": round(sum(step_flops[s] for s in live) / len(live) / (kern_ms / 1e3) / 1e12, 2)
        if live and kern_ms > 0 else None,
        "live_steps": len(live),
        "useful_flops_per_lap": lap_flops,
    }


def plan_flops(ra, desc, w, rank: int, mask: int):
    from exact_long_context_amd.workload import useful_flops
    order = [((rank - s) % w.P + w.P) % w.P for s in range(w.P)]
    flops = []
    for j in order:
        qo, ko = ra.block_offsets(mask, rank, j, w.n_local, w.n_local)
        flops.append(useful_flops(ra.plan_block(desc, w.n_local, mask, qo, ko)["live_pairs"], w.head_dim))
    return order, flops


# every other measured (workload, rank): the causal-contiguous ramp, the striped and
# long-context GQA laps, and the zigzag layout, each timed in the bench's own launch
# configuration (emulated lap with transfers)
OTHER_CONFIGS = [
    ("causal_contig_n131072_p8_h32", 0),
    ("causal_contig_n131072_p8_h32", 7),
    ("zigzag_n131072_p8_h32", 0),
    ("zigzag_n131072_p8_h32", 7),
    ("striped_n262144_p16_h32", 5),
    ("gqa_striped_n1m_p64_h64kv8", 5),
]


def other_configs(ra, warmup: int = 1, laps: int = 3):
    import torch
    import synth
    from exact_long_context_amd.workload import shard_blocks
    dev = torch.device("cuda", 0)
    res = {}
    cache = {}
    for name, rank in OTHER_CONFIGS:
        w = synth.WORKLOADS[name]
        mask = MASK_CODE[w.mask]
        log(f"[bench] {name} rank {rank}")
        key = (w.N, w.P, w.q_heads, w.kv_heads, w.value_scale)
        if key not in cache:   # K and V are drawn in global order: shared by the layouts
            cache.clear()
            torch.cuda.empty_cache()
            _, k, v = synth.workload_tensors(w, rank, heads_q=[])
            cache[key] = (k.to(dev), v.to(dev))
        kd, vd = cache[key]
        q, _, _ = synth.workload_tensors(w, rank, heads_kv=[])
        qd = q.to(dev)
        kb, vb = shard_blocks(kd, vd, w.P, w.layout)
        ring = ra.EmulatedRing(kb, vb)
        desc = ra.desc_for(qd, kb[0], w.P)
        ws = torch.empty(ra.workspace_bytes(desc), dtype=torch.uint8, device=dev)
        out = torch.empty((w.batch, w.q_heads, w.n_local, w.head_dim), dtype=torch.float32, device=dev)
        lse = torch.empty((w.batch, w.q_heads, w.n_local), dtype=torch.float32, device=dev)
        _, flops = plan_flops(ra, desc, w, rank, mask)
        r = lap_timing(ring, qd, rank, mask, w, flops, warmup, laps, ws, out, lse)
        r.update({"rank": rank, "mask": w.mask, "value_scale": round(w.value_scale, 6),
                  "pct_of_peak_lap": round(100.0 * r["useful_tflops_lap"] / PEAK_BF16_TFLOPS, 2)})
        res[f"{name}/r{rank}"] = r
        del ring, kb, vb, qd, ws, out, lse
    cache.clear()
    torch.cuda.empty_cache()
    return res


def copy_cost(ra, qd, kb, vb, ws, w, rank: int, mask: int, order, step_flops, laps: int, lap_kernel_ms):
    """What the emulated ring's copies cost the step kernel: the same steps, in the same
    process, with no transfer beside them (each block read in place from the pool)."""
    import torch
    n = w.n_local
    live = [s for s in range(w.P) if step_flops[s] > 0]
    ms = []
    for _ in range(laps + 1):
        st = ra.RingState(qd, kb[0], ring_size=w.P, workspace=ws)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * w.P)]
        for s, j in enumerate(order):
            evs[2 * s].record()
            st.step(kb[j], vb[j], mask, *ra.block_offsets(mask, rank, j, n, n))
            evs[2 * s + 1].record()
        torch.cuda.synchronize()
        ms.append([evs[2 * s].elapsed_time(evs[2 * s + 1]) for s in live])
        st.close()
    alone = [x for lap in ms[1:] for x in lap]
    alone_ms = sum(alone) / len(alone)
    return {"step_kernel_ms_with_copies": round(lap_kernel_ms, 4),
            "step_kernel_ms_without_copies": round(alone_ms, 4),
            "slowdown_from_copies": round(lap_kernel_ms / alone_ms, 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed laps")
    ap.add_argument("--warmup", type=int, default=3, help="untimed laps")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rank", type=int, default=None, help="measured rank (default: the workload's first)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle timing budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lap-only", action="store_true",
                    help="time the forward lap only: none of the passes below")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward lap (ra_bwd_*) after the forward laps")
    ap.add_argument("--decode", action="store_true",
                    help="time the split-KV step for few query rows (decode) against 16K..1M keys")
    ap.add_argument("--hbm-passes", action="store_true",
                    help="time the HBM-bound passes (finalize, short KV blocks, state merge)")
    ap.add_argument("--copy-cost", action="store_true",
                    help="time the same step kernels without the ring's concurrent copies")
    ap.add_argument("--configs", action="store_true",
                    help="time the other measured workloads and ranks (causal-contiguous, zigzag, "
                         "striped, long-context GQA)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs one rank's lap on one GPU; --gpus {args.gpus} is not supported "
              "(the ring is emulated on a single device and nothing here spans GPUs)", file=sys.stderr)
        return 2

    import torch
    import synth
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks, useful_flops

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 2
    w = synth.WORKLOADS[args.workload]
    rank = w.ranks[0] if args.rank is None else args.rank
    mask = MASK_CODE[w.mask]
    dev = torch.device("cuda", 0)

    log(f"[bench] generating {w.name} rank {rank}")
    t0 = time.perf_counter()
    q, k, v = synth.workload_tensors(w, rank)
    if w.global_q:   # the tiny workload draws Q globally: keep this rank's rows
        n = w.n_local
        q = q[:, :, rank * n:(rank + 1) * n] if w.layout == "contiguous" else q[:, :, rank::w.P]
        q = q.contiguous()
    qd = q.to(dev)
    kd, vd = k.to(dev), v.to(dev)
    kb, vb = shard_blocks(kd, vd, w.P, w.layout)
    del kd, vd
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")

    ring = ra.EmulatedRing(kb, vb)
    desc = ra.desc_for(qd, kb[0], w.P)
    ws = torch.empty(ra.workspace_bytes(desc), dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, w.q_heads, w.n_local, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.q_heads, w.n_local), dtype=torch.float32, device=dev)

    # per-step work from the host planner (the same decisions the kernels take)
    order = [((rank - s) % w.P + w.P) % w.P for s in range(w.P)]
    step_flops = []
    for j in order:
        qo, ko = ra.block_offsets(mask, rank, j, w.n_local, w.n_local)
        step_flops.append(useful_flops(ra.plan_block(desc, w.n_local, mask, qo, ko)["live_pairs"], w.head_dim))
    lap_flops = sum(step_flops)

    def mk_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * w.P)]
        for e in evs:
            e.record()
        return evs

    for i in range(args.warmup):
        ring.lap(qd, rank, mask, workspace=ws, out=out, lse=lse)
    events = [mk_events() for _ in range(args.steps)]
    torch.cuda.synchronize()

    t_start = time.perf_counter()
    stats = None
    for i in range(args.steps):
        _, _, stats = ring.lap(qd, rank, mask, workspace=ws, out=out, lse=lse, step_events=events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_lap = 1000.0 * elapsed / args.steps
    value = lap_flops * args.steps / elapsed / 1e12
    assert stats["live_pairs"] * 4 * w.head_dim == lap_flops

    # step-kernel launch times from the events (steps that launched a kernel only)
    per_step_ms = [[evs[2 * s].elapsed_time(evs[2 * s + 1]) for s in range(w.P)] for evs in events]
    # end of step s-1 to start of step s: launch gap plus any wait for the block's transfer
    gaps_ms = [[evs[2 * s - 1].elapsed_time(evs[2 * s]) for s in range(1, w.P)] for evs in events]
    # each timed lap from its first step's start to its last step's end (init and finalize,
    # ~0.1 ms, fall outside)
    lap_span_ms = sorted(evs[0].elapsed_time(evs[2 * w.P - 1]) for evs in events)
    live_steps = [s for s in range(w.P) if step_flops[s] > 0]
    kern_ms = sum(per_step_ms[i][s] for i in range(args.steps) for s in live_steps)
    kern_launches = len(live_steps) * args.steps
    achieved = sum(step_flops) * args.steps / (kern_ms / 1000.0) / 1e12 if kern_ms > 0 else 0.0
    avg_kernel_ms = kern_ms / max(kern_launches, 1)

    traffic = read_traffic(w.name)
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "kernel": "step_bf16_kernel<128>",
        "flops_per_launch": step_flops[live_steps[0]] if live_steps else 0,
        "avg_launch_ms": round(avg_kernel_ms, 4),
    }

    # the passes beside the lap: those named by flag, else all of them on a bf16 workload
    # (none with --lap-only)
    named = args.backward or args.decode or args.hbm_passes or args.configs or args.copy_cost
    every = not args.lap_only and not named and w.dtype == "bf16"
    hbm = bwd = dec = cfgs = cost = None
    if every or args.copy_cost:
        log("[bench] step kernels without concurrent transfers")
        cost = copy_cost(ra, qd, kb, vb, ws, w, rank, mask, order, step_flops, args.steps, avg_kernel_ms)
    side_cpu = 0.0 if args.no_cpu_baseline else 5.0
    if args.hbm_passes or every:
        log("[bench] HBM-bound passes: finalize, short KV blocks, state merge")
        hbm = hbm_passes(ra, qd, kb[0], vb[0], ws, w, desc, cpu_seconds=side_cpu / 4)
    if args.backward or every:
        log("[bench] backward lap")
        bwd = backward_lap(ra, qd, kb, vb, out, lse, w, rank, mask, order, step_flops, args.steps, side_cpu)
    if args.decode or every:
        log("[bench] split-KV decode steps")
        dec = decode_passes(ra, cpu_seconds=side_cpu)
    if args.configs or every:
        del ring, kb, vb
        torch.cuda.empty_cache()
        cfgs = other_configs(ra)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on host cores")
        cpu = cpu_baseline(w, rank, q, k, v, args.cpu_seconds)

    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": "useful attention TFLOP/s per GPU (one rank's lap) and % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_lap, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. Gaussian Q/K/V, see synth/)",
        "config": {
            "workload": w.name, "N": w.N, "P": w.P, "rank": rank, "batch": w.batch,
            "q_heads": w.q_heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
            "q_len": w.n_local, "kv_block": w.n_local, "mask": w.mask, "layout": w.layout,
            "value_scale": w.value_scale,
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {
            "useful_flops_per_lap": lap_flops,
            "live_pairs_per_lap": stats["live_pairs"],
            "blocks_run": stats["blocks_run"], "blocks_skipped": stats["blocks_skipped"],
            "tiles": {"full": stats["tiles_full"], "partial": stats["tiles_partial"],
                      "empty": stats["tiles_empty"], "tile_q": stats["tile_q"], "tile_k": stats["tile_k"]},
            "lap_steps_ms_median": round(lap_span_ms[len(lap_span_ms) // 2], 4),
            "lap_steps_ms_min": round(lap_span_ms[0], 4),
            "step_kernel_ms_median": [round(sorted(col)[len(col) // 2], 4) for col in zip(*per_step_ms)],
            "gap_before_step_ms_median": [round(sorted(col)[len(col) // 2], 4) for col in zip(*gaps_ms)],
            "peak_mem_gib": round(torch.cuda.max_memory_allocated() / 2**30, 2),
            "gpu": props.name, "cus": props.multi_processor_count,
            "torch": torch.__version__, "hip": torch.version.hip,
            "kernel_source_sha": kernel_source_sha(),
            "hbm_passes": hbm,
            "backward": bwd,
            "decode": dec,
            "copy_cost": cost,
            "configs": cfgs,
        },
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
