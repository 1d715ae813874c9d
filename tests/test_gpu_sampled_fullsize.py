"""GPU parity at the full workload sizes, in the launch configuration bench.py times
(one emulated lap through ra_ring_lap_emulated), checked against the fp64 oracle
computed row by row over every key of the sequence: sampled rows of every measured
workload and rank, every row of the first and the last query head of the 16K x 8-block
and the 1M-token GQA workloads, and 512 seeded (head, row) pairs of each."""

import dataclasses
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_bf16_close, oracle_head_rows_threaded, oracle_rows, require_gpu, say,
                      seeded_rows)

pytestmark = pytest.mark.gpu

MASK_CODE = {"none": 0, "causal_contiguous": 1, "causal_striped": 2, "causal_zigzag": 3}

_LAPS = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    _LAPS.clear()


def _run(name, rank, vs):
    """One emulated lap of a workload; the CPU copies of its inputs and outputs are kept for
    the other tests of the same (workload, rank, inputs), one at a time."""
    key = (name, rank, vs)
    if key in _LAPS:
        return _LAPS[key]
    _LAPS.clear()
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks
    w = synth.WORKLOADS[name]
    if vs is not None:
        w = dataclasses.replace(w, value_scale=vs)
    say(f"  generating {w.name} rank {rank} (value_scale={w.value_scale:.5f})")
    q, k, v = synth.workload_tensors(w, rank)
    kd, vd = k.cuda(), v.cuda()
    kb, vb = shard_blocks(kd, vd, w.P, w.layout)
    del kd, vd
    mask = MASK_CODE[w.mask]
    ring = ra.EmulatedRing(kb, vb)
    say(f"  lap {w.name} rank {rank}")
    o, lse, stats = ring.lap(q.cuda(), rank, mask)
    torch.cuda.synchronize()
    del ring, kb, vb
    out = (w, q, k, v, o.cpu(), lse.cpu(), stats)
    torch.cuda.empty_cache()
    _LAPS[key] = out
    return out


def _head_inputs(w, q, k, v, h):
    g = h // (w.q_heads // w.kv_heads)
    return q[0, h:h + 1].double().numpy(), k[0, g:g + 1].double().numpy(), v[0, g:g + 1].double().numpy()


def _sampled_rows(name, rank, vs):
    w, q, k, v, o_cpu, lse_cpu, stats = _run(name, rank, vs)
    causal = w.mask != "none"
    q_pos = oracle.tokens_of_rank(w.N, w.P, w.layout, rank)
    n = w.n_local
    # pair counts of the whole lap, from the oracle's enumeration
    want_pairs = 0
    for j in range(w.P):
        want_pairs += oracle.live_pair_count(q_pos, oracle.tokens_of_rank(w.N, w.P, w.layout, j), causal)
    assert stats["live_pairs"] == want_pairs * w.q_heads * w.batch
    rng = np.random.default_rng(rank + 100)
    heads = sorted({0, w.q_heads - 1, int(rng.integers(w.q_heads)), int(rng.integers(w.q_heads))})
    assert torch.isfinite(o_cpu).all()
    gots, refs = [], []
    for h in heads:
        rows = seeded_rows(n, 16, 1000 * rank + h)
        q64, k64, v64 = _head_inputs(w, q, k, v, h)
        ref = oracle_rows(q64, k64, v64, q_pos, causal, [0], rows, 1)[0]
        got = o_cpu[0, h, rows].double().numpy()
        gots.append(got)
        refs.append(ref[0])
        fin = np.isfinite(ref[1])
        assert np.array_equal(np.isfinite(lse_cpu[0, h, rows].numpy()), fin)
        assert np.max(np.abs(lse_cpu[0, h, rows].double().numpy()[fin] - ref[1][fin])) <= 2e-2
        say(f"    head {h}: {rows.size} rows")
    assert_bf16_close(np.concatenate(gots), np.concatenate(refs), f"{name} r{rank}")


def _every_row_of_a_head(name, rank, head):
    """Every row of one query head against every key of the sequence."""
    w, q, k, v, o_cpu, lse_cpu, _ = _run(name, rank, None)
    causal = w.mask != "none"
    q_pos = oracle.tokens_of_rank(w.N, w.P, w.layout, rank)
    rows = np.arange(w.n_local)
    q64, k64, v64 = _head_inputs(w, q, k, v, head)
    say(f"  oracle: all {rows.size} rows of head {head} against {w.N} keys")
    t0 = time.perf_counter()
    ref, ref_lse = oracle_head_rows_threaded(q64, k64, v64, q_pos, causal, rows)
    say(f"    oracle took {time.perf_counter() - t0:.1f} s")
    got = o_cpu[0, head].double().numpy()
    assert_bf16_close(got, ref, f"{name} r{rank} head {head}")
    fin = np.isfinite(ref_lse)
    got_lse = lse_cpu[0, head].double().numpy()
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.max(np.abs(got_lse[fin] - ref_lse[fin])) <= 2e-2


def _seeded_pairs(name, rank):
    """512 (head, row) pairs drawn with a fixed seed over the whole rank's output."""
    w, q, k, v, o_cpu, lse_cpu, _ = _run(name, rank, None)
    causal = w.mask != "none"
    q_pos = oracle.tokens_of_rank(w.N, w.P, w.layout, rank)
    rng = np.random.default_rng(4242 + rank)
    flat = rng.choice(w.q_heads * w.n_local, size=512, replace=False)
    heads, rows = np.divmod(flat, w.n_local)
    gots, refs = [], []
    for h in np.unique(heads):
        r = np.sort(rows[heads == h])
        q64, k64, v64 = _head_inputs(w, q, k, v, int(h))
        ref, ref_lse = oracle_head_rows_threaded(q64, k64, v64, q_pos, causal, r)
        gots.append(o_cpu[0, int(h), r].double().numpy())
        refs.append(ref)
        got_lse = lse_cpu[0, int(h), r].double().numpy()
        assert np.max(np.abs(got_lse - ref_lse)) <= 2e-2
    say(f"  {name} r{rank}: 512 pairs over {np.unique(heads).size} heads")
    assert_bf16_close(np.concatenate(gots), np.concatenate(refs), f"{name} r{rank} 512 pairs")


# (check, workload, rank, argument), grouped by workload so each lap runs once.  "rows":
# sampled rows of four heads (argument: a value scale other than the workload's, or None);
# "head": every row of that query head (the first and the last: for the GQA workload they
# read KV heads 0 and 7, the first and the last group); "pairs": 512 seeded (head, row) pairs.
CHECKS = [
    ("rows", "noncausal_n131072_p8_h32", 0, None),
    ("head", "noncausal_n131072_p8_h32", 0, 0),
    ("head", "noncausal_n131072_p8_h32", 0, 31),
    ("pairs", "noncausal_n131072_p8_h32", 0, None),
    ("rows", "noncausal_n131072_p8_h32", 0, 1.0),      # the other reading: plain N(0,1) inputs
    ("rows", "causal_contig_n131072_p8_h32", 0, None),
    ("rows", "causal_contig_n131072_p8_h32", 7, None),
    ("rows", "zigzag_n131072_p8_h32", 0, None),
    ("rows", "zigzag_n131072_p8_h32", 7, None),
    ("rows", "striped_n262144_p16_h32", 5, None),
    ("rows", "gqa_striped_n1m_p64_h64kv8", 5, None),
    ("head", "gqa_striped_n1m_p64_h64kv8", 5, 0),
    ("head", "gqa_striped_n1m_p64_h64kv8", 5, 63),
    ("pairs", "gqa_striped_n1m_p64_h64kv8", 5, None),
]


def _check_id(c):
    kind, name, rank, arg = c
    tail = {"rows": "-plain" if arg else "", "head": f"-h{arg}", "pairs": "-512pairs"}[kind]
    return f"{kind}-{name}-r{rank}{tail}"


@pytest.mark.parametrize("check", CHECKS, ids=[_check_id(c) for c in CHECKS])
def test_full_size(check):
    kind, name, rank, arg = check
    if kind == "rows":
        _sampled_rows(name, rank, arg)
    elif kind == "head":
        _every_row_of_a_head(name, rank, arg)
    else:
        _seeded_pairs(name, rank)
