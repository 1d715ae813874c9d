"""Shared helpers for the GPU parity tests (inputs, laps through the C ABI, tolerances)."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth

LAYOUT_OF_MASK = {0: "contiguous", 1: "contiguous", 2: "striped", 3: "zigzag"}

# bf16 inputs with fp32 accumulation, against the fp64 oracle on the same bf16 values
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_NORMWISE = 1e-2     # stricter check of our own: ||err||_F / ||ref||_F
# fp32 path: normwise relative error ||err||_inf / ||ref||_inf
F32_REL = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X: run them with -m gpu on a machine that has one"
    import exact_long_context_amd  # noqa: F401  (fails loudly if librocring.so is missing)


def lap_with_steps(q, k_blocks, v_blocks, rank, mask_kind, P, order=None, softmax_scale=0.0,
                   debug_counters=None):
    """One lap through ra_state_init / ra_block_step / ra_finalize in ring order."""
    import exact_long_context_amd as ra
    n = q.shape[2]
    nk = k_blocks[0].shape[2]
    st = ra.RingState(q, k_blocks[0], ring_size=P, softmax_scale=softmax_scale)
    if debug_counters is not None:
        st.set_debug_counters(debug_counters)
    order = oracle.ring_visit_order(P, rank) if order is None else order
    for j in order:
        qo, ko = ra.block_offsets(mask_kind, rank, j, n, nk)
        st.step(k_blocks[j], v_blocks[j], mask_kind, qo, ko)
    o, lse = st.finalize()
    stats = st.stats()
    st.close()
    return o, lse, stats


def oracle_rows(q64, k64, v64, q_pos, causal, heads, rows, group, row_chunk=16):
    """fp64 reference rows: q64 [Hq, n, d] (numpy), k64/v64 [Hkv, N, d] in global order."""
    N = k64.shape[1]
    out = {}
    for h in heads:
        g = h // group
        o, lse = oracle.dense_attention(q64[None, h:h + 1], k64[None, g:g + 1], v64[None, g:g + 1],
                                        q_pos, np.arange(N), causal, rows=rows, row_chunk=row_chunk)
        out[h] = (o[0, 0, rows], lse[0, 0, rows])
    return out


def bf16_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got.astype(np.float64) - ref)
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "normwise": float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)),
    }


# per-row bound of our own for outputs: ||err_row|| <= BF16_ROWWISE * ||ref_row|| + 1e-6, so
# that a few wrong rows cannot hide inside whole-tensor norms (rows are the last axis)
BF16_ROWWISE = 2e-2


def assert_bf16_close(got, ref, what="", rowwise=BF16_ROWWISE):
    e = bf16_errors(got, ref)
    msg = f"    {what} max_abs={e['max_abs']:.3e} mean_abs={e['mean_abs']:.3e} normwise={e['normwise']:.3e}"
    if rowwise is not None and np.asarray(ref).size:
        g = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
        r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
        row = np.linalg.norm(g - r, axis=1) / (np.linalg.norm(r, axis=1) + 1e-6 / rowwise)
        e["worst_row"] = float(row.max())
        msg += f" worst_row={e['worst_row']:.3e}"
        assert e["worst_row"] <= rowwise, (what, e, int(row.argmax()))
    say(msg)
    assert e["max_abs"] <= BF16_MAX_ABS, (what, e)
    assert e["mean_abs"] <= BF16_MEAN_ABS, (what, e)
    assert e["normwise"] <= BF16_NORMWISE, (what, e)
    return e


def assert_f32_close(got, ref, what="", tol=F32_REL):
    got = got.astype(np.float64)
    rel = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))
    elem = float(np.max(np.abs(got - ref) / (np.abs(ref) + 1e-6)))
    say(f"    {what} normwise_rel={rel:.3e} elementwise={elem:.3e}")
    assert rel <= tol, (what, rel, tol)
    return rel


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def seeded_rows(n: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    edge = list(range(min(16, n))) + list(range(max(0, n - 16), n))
    extra = rng.choice(n, size=min(count, n), replace=False).tolist()
    return np.array(sorted(set(edge + extra)), dtype=np.int64)


def plant_score_levels(q, k, levels, q_amp: float = 8.0) -> None:
    """Plant score structure through channel 0, in place on CPU tensors q [B, Hq, n, d] and
    k [B, Hkv, N, d]: every query row gets q[..., 0] = q_amp and key t gets
    k[..., t, 0] = levels[t] * sqrt(d) / q_amp (rounded to k's dtype), so that with the softmax
    scale 1/sqrt(d) the planted part of any row's score against key t is levels[t] in natural
    units; the other channels keep their (small) random values.  The oracle reads the same
    rounded tensors, so the planted values need not be exact."""
    d = q.shape[-1]
    q[..., 0] = q_amp
    lv = torch.from_numpy(np.asarray(levels, dtype=np.float64) * (math.sqrt(d) / q_amp))
    k[..., :, 0] = lv.to(k.dtype)


def ladder_levels(u: int, nk: int, rng) -> np.ndarray:
    """Planted score levels (natural units) for the block visited at step u of a lap, built so
    that the state's reference must move by far more than 32 (base 2) on rows that already
    hold keys:
      u = 0: every key near -40 (a row's first visible keys score very low);
      u = 1: keys near 0, about 58 base-2 units above: the first tile of the launch rescales;
      u even >= 2: keys 0..127 at the previous plateau, then every 8th key 35 units higher:
               the rescale happens inside the launch, after visible tiles;
      u odd >= 3: keys within a few units of the current plateau, taken without a rescale,
               so the outputs mix several keys of the top plateau."""
    t = np.arange(nk)
    if u == 0:
        return -40.0 + rng.uniform(-1.0, 0.0, nk)
    if u == 1:
        return rng.uniform(-1.0, 0.0, nk)
    top = 30.0 + 35.0 * ((u - 2) // 2)          # plateau after this step
    prev = 0.0 if u < 4 else top - 35.0 if u % 2 == 0 else top
    lv = (prev if u % 2 == 0 else top - 3.0) + rng.uniform(-1.0, 0.0, nk)
    if u % 2 == 0:
        sel = (t >= 128) & (t % 8 == 3)
        lv[sel] = top + rng.uniform(-1.0, 0.0, int(sel.sum()))
    else:
        sel = t % 4 == 1
        lv[sel] = top + rng.uniform(-1.0, 2.0, int(sel.sum()))
    return lv


def oracle_head_rows_threaded(q64, k64, v64, q_pos, causal, rows, threads=None, budget=1 << 22):
    """oracle.dense_attention on some rows of one head, run over a thread pool.

    q64 [1, n, d], k64 / v64 [1, N, d] (numpy fp64; keys in global token order, so key t sits
    at position t).  Rows go in chunks whose score matrix holds about ``budget`` elements;
    for causal rows a chunk is given only the key prefix its last row may see (no key past it
    is allowed to any row of the chunk, so the result is the same).  BLAS runs one thread per
    pool thread.  Returns (O [len(rows), d], lse [len(rows)])."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    rows = np.asarray(rows, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    N = k64.shape[1]
    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    def keys_seen(r):   # keys a chunk ending at local row r is given
        return min(N, int(q_pos[r]) + 1) if causal else N

    chunks = []
    i = 0
    while i < rows.size:   # rows ascend, so a chunk's last row sees the most keys
        c = 1
        while i + c < rows.size and (c + 1) * keys_seen(rows[i + c]) <= budget:
            c += 1
        chunks.append(rows[i:i + c])
        i += c

    def one(rc):
        kc = keys_seen(rc[-1])
        o, lse = oracle.dense_attention(q64[None, :, rc], k64[None, :, :kc], v64[None, :, :kc],
                                        q_pos[rc], np.arange(kc), causal, row_chunk=rc.size)
        return o[0, 0], lse[0, 0]

    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, chunks))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
