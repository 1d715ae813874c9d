"""GPU parity of ra_merge_states, the global online-softmax reduction of shard states
(split-KV decode), against the fp64 oracle, plus its exact identities."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_bf16_close, assert_f32_close, lap_with_steps, require_gpu, say, to64)

pytestmark = pytest.mark.gpu

NONE, CONTIG, STRIPED = 0, 1, 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _shard_states(q, k, v, cuts):
    """One state per key range [cuts[s], cuts[s+1]) of k/v (views: the strides are shared)."""
    import exact_long_context_amd as ra
    states = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        st = ra.RingState(q, k)
        st.step(k[:, :, a:b], v[:, :, a:b], NONE)
        assert st.stats()["blocks_run"] == 1
        states.append(st)
    return states


@pytest.mark.parametrize("dtype,Hq,Hkv,d,n", [("bf16", 8, 2, 128, 1), ("bf16", 8, 2, 128, 5),
                                             ("bf16", 4, 4, 64, 130), ("f32", 4, 2, 128, 3),
                                             ("f32", 2, 2, 64, 70)])
def test_split_kv_decode_matches_oracle(dtype, Hq, Hkv, d, n):
    import exact_long_context_amd as ra
    cuts = [0, 300, 301, 1078, 1142, 2048, 2500]          # six shards, ragged sizes
    N = cuts[-1]
    q, k, v = synth.random_case(40 + n, 1, Hq, Hkv, n, N, d, dtype)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say(f"  split-KV {dtype} Hq={Hq} Hkv={Hkv} d={d} n={n} shards={len(cuts) - 1}")
    states = _shard_states(qd, kd, vd, cuts)
    o = torch.empty((1, Hq, n, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, Hq, n), dtype=torch.float32, device="cuda")
    ra.merge_states(states[0].desc, [s.workspace for s in states], out=o, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), np.arange(n), np.arange(N), False)
    if dtype == "bf16":
        assert_bf16_close(to64(o), ref, "merged O")
        tol = 2e-2
    else:
        assert_f32_close(to64(o), ref, "merged O")
        tol = 1e-5
    assert np.max(np.abs(to64(lse) - ref_lse)) <= tol * max(1.0, float(np.max(np.abs(ref_lse))))
    for s in states:
        s.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mask", [CONTIG, STRIPED])
def test_merged_lap_halves_match_oracle_with_empty_rows(dtype, mask):
    """Two states over two halves of a causal lap's blocks, merged.  With the striped layout
    the second half holds only blocks after the rank, where query row 0 sees no key: its
    reference maximum is -inf there and must contribute nothing."""
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks
    N, P, rank, Hq, Hkv = 2048, 4, 1, 4, 2
    layout = "striped" if mask == STRIPED else "contiguous"
    q_pos = oracle.tokens_of_rank(N, P, layout, rank)
    n = q_pos.size
    q, k, v = synth.random_case(60 + mask, 1, Hq, Hkv, n, N, 128, dtype)
    kb, vb = shard_blocks(k.cuda(), v.cuda(), P, layout)
    qd = q.cuda()
    halves = ([0, 1], [2, 3]) if mask == STRIPED else ([1], [0])
    states = []
    for blocks in halves:
        st = ra.RingState(qd, kb[0], ring_size=P)
        for j in blocks:
            qo, ko = ra.block_offsets(mask, rank, j, n, n)
            st.step(kb[j], vb[j], mask, qo, ko)
        assert st.stats()["blocks_run"] == len(blocks)
        states.append(st)
    if mask == STRIPED:   # row 0 (position rank) sees no key of blocks 2, 3
        _, m_b, _ = states[1].state_views()
        torch.cuda.synchronize()
        assert torch.isneginf(m_b[0, :, 0]).all()
    o = torch.empty((1, Hq, n, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, Hq, n), dtype=torch.float32, device="cuda")
    ra.merge_states(states[0].desc, [s.workspace for s in states], out=o, lse=lse)
    o_lap, lse_lap, _ = lap_with_steps(qd, kb, vb, rank, mask, P)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), True)
    if dtype == "bf16":
        assert_bf16_close(to64(o), ref, "merged halves")
        assert_bf16_close(to64(o), to64(o_lap), "merged halves vs one lap")
    else:
        assert_f32_close(to64(o), ref, "merged halves")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), fin)
    for s in states:
        s.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_identities_are_bitwise(dtype):
    """merge -> state -> finalize equals merge -> O directly; merging in place over the first
    part equals merging into a fresh workspace; a single part equals finalizing that part."""
    import exact_long_context_amd as ra
    Hq, Hkv, d, n = 4, 2, 128, 200
    cuts = [0, 500, 900, 1500]
    q, k, v = synth.random_case(77, 1, Hq, Hkv, n, cuts[-1], d, dtype)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    states = _shard_states(qd, kd, vd, cuts)
    desc = states[0].desc
    parts = [s.workspace for s in states]
    o_direct = torch.empty((1, Hq, n, d), dtype=torch.float32, device="cuda")
    lse_direct = torch.empty((1, Hq, n), dtype=torch.float32, device="cuda")
    ra.merge_states(desc, parts, out=o_direct, lse=lse_direct)
    merged = torch.empty_like(parts[0])
    ra.merge_states(desc, parts, merged=merged)
    o_via, lse_via = ra.RingState(qd, kd, workspace=merged, resume=True).finalize()
    in_place = [p.clone() for p in parts]
    ra.merge_states(desc, in_place, merged=in_place[0])
    o_inpl, _ = ra.RingState(qd, kd, workspace=in_place[0], resume=True).finalize()
    o_one = torch.empty_like(o_direct)
    ra.merge_states(desc, parts[1:2], out=o_one)
    o_fin1, _ = ra.RingState(qd, kd, workspace=parts[1].clone(), resume=True).finalize()
    torch.cuda.synchronize()
    assert torch.equal(o_direct, o_via) and torch.equal(lse_direct, lse_via)
    assert torch.equal(o_direct, o_inpl)
    assert torch.equal(o_one, o_fin1)
    for s in states:
        s.close()
