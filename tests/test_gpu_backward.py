"""GPU parity of the backward ring step (ra_bwd_*) against the fp64 oracle.

The oracle runs its own forward for O and lse; the library's backward consumes the
library's forward outputs.  Each rank's dQ and its contribution to every block's dK, dV are
compared block by block."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bf16_close, assert_f32_close, lap_with_steps, require_gpu, say, to64

pytestmark = pytest.mark.gpu

NONE, CONTIG, STRIPED, ZIGZAG = 0, 1, 2, 3
LAYOUT = {NONE: "contiguous", CONTIG: "contiguous", STRIPED: "striped", ZIGZAG: "zigzag"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _close(got, ref, dtype, what):
    if dtype == "bf16":
        return assert_bf16_close(got, ref, what, rowwise=None)
    return assert_f32_close(got, ref, what)


CASES = [
    # dtype, B, Hq, Hkv, d, N, P, rank, mask
    ("f32", 1, 2, 1, 64, 512, 4, 2, CONTIG),
    ("f32", 1, 2, 2, 128, 600, 3, 1, STRIPED),
    ("f32", 2, 2, 1, 64, 480, 4, 3, ZIGZAG),
    ("f32", 1, 3, 3, 128, 400, 4, 1, NONE),
    ("bf16", 1, 4, 2, 128, 1024, 4, 2, CONTIG),
    ("bf16", 1, 4, 1, 128, 1200, 4, 3, STRIPED),
    ("bf16", 1, 2, 2, 64, 1000, 5, 4, ZIGZAG),
    ("bf16", 2, 2, 1, 128, 900, 3, 0, NONE),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}-H{c[2]}x{c[3]}-d{c[4]}-N{c[5]}-P{c[6]}-r{c[7]}-m{c[8]}"
                                             for c in CASES])
def test_backward_lap_matches_oracle(case):
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks
    dtype, B, Hq, Hkv, d, N, P, rank, mask = case
    layout = LAYOUT[mask]
    causal = mask != NONE
    seed = zlib.crc32(repr(case).encode()) % 1000
    q_pos = oracle.tokens_of_rank(N, P, layout, rank)
    n = q_pos.size
    q, k, v = synth.random_case(seed, B, Hq, Hkv, n, N, d, dtype)
    g = np.random.default_rng(seed + 1)
    d_out = torch.from_numpy(g.standard_normal((B, Hq, n, d)).astype(np.float32)).to(q.dtype)
    kb, vb = shard_blocks(k.cuda(), v.cuda(), P, layout)
    qd, dod = q.cuda(), d_out.cuda()
    say(f"  backward case {case}")
    o, lse, _ = lap_with_steps(qd, kb, vb, rank, mask, P)
    bw = ra.RingBackward(qd, dod, o, lse, kb[0], ring_size=P)
    dks = [torch.zeros(kb[j].shape, dtype=torch.float32, device="cuda") for j in range(P)]
    dvs = [torch.zeros(vb[j].shape, dtype=torch.float32, device="cuda") for j in range(P)]
    for j in oracle.ring_visit_order(P, rank):
        qo, ko = ra.block_offsets(mask, rank, j, n, n)
        bw.step(kb[j], vb[j], dks[j], dvs[j], mask, qo, ko)
    dq = bw.finalize()
    stats = bw.stats()
    bw.close()
    torch.cuda.synchronize()
    # the oracle: its own forward, then the same lap of backward steps
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(d_out)
    o_ref, lse_ref = oracle.dense_attention(q64, k64, v64, q_pos, np.arange(N), causal)
    D = oracle.backward_row_terms(do64, o_ref)
    dq_ref = np.zeros_like(q64)
    for j in oracle.ring_visit_order(P, rank):
        kp = oracle.tokens_of_rank(N, P, layout, j)
        gq, gk, gv = oracle.backward_block(q64, k64[:, :, kp], v64[:, :, kp], do64, lse_ref, D, q_pos, kp, causal)
        dq_ref += gq
        _close(to64(dks[j]), gk, dtype, f"dK block {j}")
        _close(to64(dvs[j]), gv, dtype, f"dV block {j}")
    _close(to64(dq), dq_ref, dtype, "dQ")
    assert stats["live_pairs"] == B * Hq * sum(
        oracle.live_pair_count(q_pos, oracle.tokens_of_rank(N, P, layout, j), causal) for j in range(P))


def test_backward_rows_without_keys_and_accumulation():
    """A rank-0 causal shard against a block wholly in the future adds nothing; dK, dV
    accumulate onto what the block already carries."""
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks
    N, P, Hq, d = 512, 4, 2, 128
    q, k, v = synth.random_case(5, 1, Hq, Hq, N // P, N, d, "f32")
    kb, vb = shard_blocks(k.cuda(), v.cuda(), P, "contiguous")
    qd = q.cuda()
    dod = torch.randn(qd.shape, device="cuda")
    o, lse, _ = lap_with_steps(qd, kb, vb, 0, CONTIG, P)
    bw = ra.RingBackward(qd, dod, o, lse, kb[0], ring_size=P)
    carried = torch.randn(kb[2].shape, device="cuda")
    dk = carried.clone()
    dv = carried.clone()
    qo, ko = ra.block_offsets(CONTIG, 0, 2, N // P, N // P)
    bw.step(kb[2], vb[2], dk, dv, CONTIG, qo, ko)
    assert bw.stats()["blocks_skipped"] == 1
    dq = bw.finalize()
    torch.cuda.synchronize()
    assert torch.equal(dk, carried) and torch.equal(dv, carried)
    assert not dq.any()
    bw.close()


def test_backward_full_size_sampled_rows_and_keys():
    """The 16K x 16K causal diagonal block at full size (rank 0 of the 131072-token,
    8-rank contiguous ring, 32 heads): sampled dQ rows and sampled keys of dK, dV against the
    oracle, whose forward for head 0 (lse, O) it computes itself."""
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks
    from gpu_util import seeded_rows
    w = synth.WORKLOADS["causal_contig_n131072_p8_h32"]
    rank = 0
    say(f"  generating {w.name} rank {rank}")
    q, k, v = synth.workload_tensors(w, rank)
    n = w.n_local
    d_out = synth.random_case(9, 1, w.q_heads, 1, n, 1, w.head_dim, "bf16")[0]
    kb, vb = shard_blocks(k.cuda(), v.cuda(), w.P, w.layout)
    qd, dod = q.cuda(), d_out.cuda()
    ring = ra.EmulatedRing(kb, vb)
    o, lse, _ = ring.lap(qd, rank, CONTIG)
    bw = ra.RingBackward(qd, dod, o, lse, kb[0], ring_size=w.P)
    dk0 = torch.zeros(kb[0].shape, dtype=torch.float32, device="cuda")
    dv0 = torch.zeros_like(dk0)
    scratch_k = torch.zeros_like(dk0)
    scratch_v = torch.zeros_like(dk0)
    for j in oracle.ring_visit_order(w.P, rank):
        qo, ko = ra.block_offsets(CONTIG, rank, j, n, n)
        bw.step(kb[j], vb[j], dk0 if j == 0 else scratch_k, dv0 if j == 0 else scratch_v, CONTIG, qo, ko)
    dq = bw.finalize()
    assert bw.stats()["blocks_skipped"] == w.P - 1
    bw.close()
    torch.cuda.synchronize()
    assert not scratch_k.any() and not scratch_v.any()   # every other block is in the future
    # oracle, head 0: rank 0's rows against block 0 (the only keys they may see)
    q_pos = np.arange(n)
    q64 = to64(q[:, :1])
    k64 = to64(k[:, :1, :n])
    v64 = to64(v[:, :1, :n])
    do64 = to64(d_out[:, :1])
    say("  oracle forward, head 0")
    o_ref, lse_ref = oracle.dense_attention(q64, k64, v64, q_pos, q_pos, True)
    D = oracle.backward_row_terms(do64, o_ref)
    rows = seeded_rows(n, 48, 3)
    gq, _, _ = oracle.backward_block(q64[:, :, rows], k64, v64, do64[:, :, rows], lse_ref[:, :, rows],
                                     D[:, :, rows], q_pos[rows], q_pos, True)
    assert_bf16_close(to64(dq[:, :1, rows]), gq, "dQ sampled rows", rowwise=None)
    keys = seeded_rows(n, 48, 4)
    _, gk, gv = oracle.backward_block(q64, k64[:, :, keys], v64[:, :, keys], do64, lse_ref, D, q_pos,
                                      q_pos[keys], True)
    assert_bf16_close(to64(dk0[:, :1, keys]), gk, "dK sampled keys", rowwise=None)
    assert_bf16_close(to64(dv0[:, :1, keys]), gv, "dV sampled keys", rowwise=None)


def test_backward_full_size_noncausal_lap_sampled():
    """The backward lap that bench.py times: the non-causal 131072-token, 8-rank ring, rank 0,
    32 heads, all 8 blocks through ra_bwd_block_step in ring order.  Sampled dQ rows of head 0
    against every key of the sequence, and sampled keys of one travelling block's dK and dV
    (this rank's contribution: every one of its rows), against the oracle, whose forward for
    head 0 (O, lse over all keys) it computes itself."""
    import exact_long_context_amd as ra
    from exact_long_context_amd.workload import shard_blocks
    from gpu_util import seeded_rows
    w = synth.WORKLOADS["noncausal_n131072_p8_h32"]
    rank, j_check = 0, 3
    say(f"  generating {w.name} rank {rank}")
    q, k, v = synth.workload_tensors(w, rank)
    n = w.n_local
    d_out = synth.random_case(10, 1, w.q_heads, 1, n, 1, w.head_dim, "bf16")[0]
    kb, vb = shard_blocks(k.cuda(), v.cuda(), w.P, w.layout)
    qd, dod = q.cuda(), d_out.cuda()
    o, lse, _ = ra.EmulatedRing(kb, vb).lap(qd, rank, NONE)
    bw = ra.RingBackward(qd, dod, o, lse, kb[0], ring_size=w.P)
    dks = {j: torch.zeros(kb[j].shape, dtype=torch.float32, device="cuda") for j in range(w.P)}
    dvs = {j: torch.zeros(kb[j].shape, dtype=torch.float32, device="cuda") for j in range(w.P)}
    for j in oracle.ring_visit_order(w.P, rank):
        bw.step(kb[j], vb[j], dks[j], dvs[j], NONE, 0, 0)
    dq = bw.finalize()
    bw.close()
    torch.cuda.synchronize()
    # oracle, head 0: the rank's rows against the whole sequence
    q64, k64, v64, do64 = to64(q[:, :1]), to64(k[:, :1]), to64(v[:, :1]), to64(d_out[:, :1])
    q_pos, k_pos = np.arange(n), np.arange(w.N)
    say("  oracle forward, head 0, all keys")
    o_ref, lse_ref = oracle.dense_attention(q64, k64, v64, q_pos, k_pos, False, row_chunk=512)
    D = oracle.backward_row_terms(do64, o_ref)
    rows = seeded_rows(n, 48, 5)
    gq, _, _ = oracle.backward_block(q64[:, :, rows], k64, v64, do64[:, :, rows], lse_ref[:, :, rows],
                                     D[:, :, rows], q_pos[rows], k_pos, False)
    assert_bf16_close(to64(dq[:, :1, rows]), gq, "dQ sampled rows, all keys", rowwise=None)
    keys = seeded_rows(n, 48, 6)                       # local keys of block j_check
    gk_keys = j_check * n + keys                       # their global positions
    _, gk, gv = oracle.backward_block(q64, k64[:, :, gk_keys], v64[:, :, gk_keys], do64, lse_ref, D,
                                      q_pos, gk_keys, False)
    assert_bf16_close(to64(dks[j_check][:, :1, keys]), gk, f"dK block {j_check} sampled keys", rowwise=None)
    assert_bf16_close(to64(dvs[j_check][:, :1, keys]), gv, f"dV block {j_check} sampled keys", rowwise=None)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_is_bitwise_repeatable(dtype):
    """Twenty identical backward steps over 4096 rows x 8 heads (many workgroups on every CU):
    dQ, dK and dV must be bit-identical every time, so no workgroup reads a buffer another one
    is still writing."""
    import exact_long_context_amd as ra
    g = torch.Generator(device="cpu").manual_seed(79)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H, n = 8, 4096
    q = (torch.randn(1, H, n, 128, generator=g) * 0.3).to(tdt).cuda()
    k = (torch.randn(1, H, n, 128, generator=g) * 0.3).to(tdt).cuda()
    v = torch.randn(1, H, n, 128, generator=g).to(tdt).cuda()
    dod = torch.randn(1, H, n, 128, generator=g).to(tdt).cuda()
    o, lse, _ = lap_with_steps(q, [k], [v], 0, CONTIG, 1)
    say(f"  backward repeatability {dtype}: {H} heads x {n} rows, causal diagonal block")
    runs = []
    for _ in range(20):
        bw = ra.RingBackward(q, dod, o, lse, k, ring_size=1)
        dk = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
        dv = torch.zeros(v.shape, dtype=torch.float32, device="cuda")
        bw.step(k, v, dk, dv, CONTIG, 0, 0)
        dq = bw.finalize()
        torch.cuda.synchronize()
        bw.close()
        runs.append((dq.clone(), dk, dv))
    for other in runs[1:]:
        for a, b in zip(runs[0], other):
            assert torch.equal(a, b)
