"""GPU parity at the full workload sizes, in the launch configuration bench.py times
(one emulated lap through ra_ring_lap_emulated), checked on sampled rows that the
fp64 oracle computes one by one over every key of the sequence."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bf16_close, oracle_rows, require_gpu, say, seeded_rows

pytestmark = pytest.mark.gpu

MASK_CODE = {"none": 0, "causal_contiguous": 1, "causal_striped": 2, "causal_zigzag": 3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _run(w, rank):
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks
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
    return q, k, v, o, lse, stats


FULL = [
    ("noncausal_n131072_p8_h32", 0, None),
    ("noncausal_n131072_p8_h32", 0, 1.0),      # the other reading: plain N(0,1) inputs
    ("causal_contig_n131072_p8_h32", 0, None),
    ("causal_contig_n131072_p8_h32", 7, None),
    ("zigzag_n131072_p8_h32", 0, None),
    ("zigzag_n131072_p8_h32", 7, None),
    ("striped_n262144_p16_h32", 5, None),
    ("gqa_striped_n1m_p64_h64kv8", 5, None),
]


@pytest.mark.parametrize("name,rank,vs", FULL, ids=[f"{n}-r{r}" + ("-plain" if v else "") for n, r, v in FULL])
def test_full_size_sampled_rows(name, rank, vs):
    w = synth.WORKLOADS[name]
    if vs is not None:
        w = dataclasses.replace(w, value_scale=vs)
    q, k, v, o, lse, stats = _run(w, rank)
    causal = w.mask != "none"
    q_pos = oracle.tokens_of_rank(w.N, w.P, w.layout, rank)
    n = w.n_local
    G = w.q_heads // w.kv_heads
    # pair counts of the whole lap, from the oracle's enumeration
    want_pairs = 0
    for j in range(w.P):
        want_pairs += oracle.live_pair_count(q_pos, oracle.tokens_of_rank(w.N, w.P, w.layout, j), causal)
    assert stats["live_pairs"] == want_pairs * w.q_heads * w.batch
    rng = np.random.default_rng(rank + 100)
    heads = sorted({0, w.q_heads - 1, int(rng.integers(w.q_heads)), int(rng.integers(w.q_heads))})
    o_cpu = o.cpu()
    lse_cpu = lse.cpu()
    assert torch.isfinite(o_cpu).all()
    gots, refs = [], []
    for h in heads:
        rows = seeded_rows(n, 16, 1000 * rank + h)
        g = h // G
        q64 = q[0, h:h + 1].double().numpy()
        k64 = k[0, g:g + 1].double().numpy()
        v64 = v[0, g:g + 1].double().numpy()
        ref = oracle_rows(q64, k64, v64, q_pos, causal, [0], rows, 1)[0]
        got = o_cpu[0, h, rows].double().numpy()
        gots.append(got)
        refs.append(ref[0])
        fin = np.isfinite(ref[1])
        assert np.array_equal(np.isfinite(lse_cpu[0, h, rows].numpy()), fin)
        assert np.max(np.abs(lse_cpu[0, h, rows].double().numpy()[fin] - ref[1][fin])) <= 2e-2
        say(f"    head {h}: {rows.size} rows")
    assert_bf16_close(np.concatenate(gots), np.concatenate(refs), f"{name} r{rank}")
