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


def assert_f32_close(got, ref, what=""):
    got = got.astype(np.float64)
    rel = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))
    elem = float(np.max(np.abs(got - ref) / (np.abs(ref) + 1e-6)))
    say(f"    {what} normwise_rel={rel:.3e} elementwise={elem:.3e}")
    assert rel <= F32_REL, (what, rel)
    return rel


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def seeded_rows(n: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    edge = list(range(min(16, n))) + list(range(max(0, n - 16), n))
    extra = rng.choice(n, size=min(count, n), replace=False).tolist()
    return np.array(sorted(set(edge + extra)), dtype=np.int64)
