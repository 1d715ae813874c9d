"""Laps captured in a HIP graph (torch.cuda.CUDAGraph on the state's stream) and replayed.
Every entry point that a lap calls only launches kernels on the state's stream under capture:
no allocation, no memset, no synchronisation (ra_block_step grows its key-norm buffer only
outside capture, and steps a block it does not fit without bounds).  A lap therefore captures
whole: the split-KV decode lap, the tiled forward lap, the backward lap and a split-KV merge.  Each graph is
replayed several times, with eager work of the program between replays, and every replay
must reproduce the eager run bit for bit; the eager run itself is checked against the fp64
oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bf16_close, require_gpu, say, to64

pytestmark = pytest.mark.gpu

NONE, CONTIG = 0, 1
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _blocks(x, P):
    nk = x.shape[2] // P
    return [x[:, :, j * nk:(j + 1) * nk] for j in range(P)]


def _forward_lap(ra, q, kb, vb, mask, q_off, nk, stream, out, lse, ws, decode, state_ws):
    """One rank's lap through a fresh state on `stream`: every block in ring order, then
    finalize into the caller's buffers.  Allocates nothing on the device."""
    P = len(kb)
    rank = q_off // nk
    st = ra.RingState(q, kb[0], ring_size=P, stream=stream, workspace=state_ws)
    for j in oracle.ring_visit_order(P, rank):
        if decode:
            st.decode_step(kb[j], vb[j], mask, q_off, j * nk, workspace=ws)
        else:
            st.step(kb[j], vb[j], mask, q_off, j * nk)
    st.finalize(out=out, lse=lse)
    return st


def _eager_noise(q):
    """Unrelated work of the program between replays, on the default stream."""
    x = torch.randn(1 << 20, device=q.device)
    torch.cuda.synchronize()
    return float((x * x).sum())


@pytest.mark.parametrize("decode,n,mask,nk", [(True, 1, CONTIG, 2500), (True, 8, NONE, 2500),
                                              (False, 300, CONTIG, 2500), (False, 300, NONE, 4096)],
                         ids=["decode_q1_causal", "decode_q8_noncausal", "tiled_q300_causal",
                              "tiled_q300_noncausal_bounds_eager_only"])
def test_forward_lap_graph_replays_match_eager(decode, n, mask, nk):
    """With blocks of 4096 keys the eager lap's steps use key-norm bounds, while the captured
    lap's fresh state cannot allocate them under capture and runs the full guard: a bound only
    ever skips a maximum that would have moved no reference, so the two agree bit for bit."""
    import exact_long_context_amd as ra
    B, Hq, Hkv, d, P = 1, 16, 2, 128, 4
    N = P * nk
    say(f"  graph lap: decode={decode} n={n} mask={mask}, {P} blocks of {nk} keys")
    q, k, v = synth.random_case(930 + n, B, Hq, Hkv, n, N, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kb, vb = _blocks(kd, P), _blocks(vd, P)
    q_off = N - n if mask == CONTIG else 0          # the newest tokens of the context
    s = torch.cuda.Stream()
    desc = ra.desc_for(qd, kb[0], P, stream=s)
    ws = torch.empty(max(ra.decode_workspace_bytes(desc, nk), 256), dtype=torch.uint8, device="cuda")
    state_ws = torch.empty(ra.workspace_bytes(desc), dtype=torch.uint8, device="cuda")

    out_e = torch.empty((B, Hq, n, d), dtype=torch.float32, device="cuda")
    lse_e = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        st = _forward_lap(ra, qd, kb, vb, mask, q_off, nk, s, out_e, lse_e, ws, decode, state_ws)
    s.synchronize()
    st.close()
    q_pos, k_pos = q_off + np.arange(n), np.arange(N)
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, k_pos, mask != NONE)
    assert_bf16_close(to64(out_e), ref, "eager lap O")
    assert np.max(np.abs(to64(lse_e) - ref_lse)) <= 2e-2

    out_g = torch.full_like(out_e, float("nan"))
    lse_g = torch.full_like(lse_e, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st_g = _forward_lap(ra, qd, kb, vb, mask, q_off, nk, s, out_g, lse_g, ws, decode, state_ws)
    for r in range(REPLAYS):
        with torch.cuda.stream(s):
            out_g.fill_(float("nan"))
            lse_g.fill_(float("nan"))
            ws.fill_(0xAB)                             # chunk states left by other work
            state_ws.fill_(0xCD)                       # a stale running state
            g.replay()
        s.synchronize()
        assert torch.equal(out_g, out_e), f"replay {r}: O differs from the eager lap"
        assert torch.equal(lse_g, lse_e), f"replay {r}: lse differs from the eager lap"
        _eager_noise(qd)
    st_g.close()


def test_backward_lap_graph_replays_match_eager():
    """ra_bwd_init, one ra_bwd_block_step per block, ra_bwd_finalize, captured whole."""
    import exact_long_context_amd as ra
    B, Hq, Hkv, n, d, P = 1, 8, 2, 384, 128, 4
    N = P * n
    rank = 2
    say(f"  graph backward lap: {Hq} heads, {P} blocks of {n}, rank {rank}, causal")
    q_all, k, v = synth.random_case(951, B, Hq, Hkv, N, N, d, "bf16")
    q = q_all[:, :, rank * n:(rank + 1) * n].contiguous()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kb, vb = _blocks(kd, P), _blocks(vd, P)
    q_off = rank * n
    s = torch.cuda.Stream()
    out = torch.empty((B, Hq, n, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        st = _forward_lap(ra, qd, kb, vb, CONTIG, q_off, n, s, out, lse, None, False, None)
    s.synchronize()
    st.close()
    g_cpu = torch.Generator(device="cpu").manual_seed(952)
    d_out = torch.randn((B, Hq, n, d), generator=g_cpu).to(torch.bfloat16).cuda()
    desc = ra.desc_for(qd, kb[0], P, stream=s)
    ws = torch.empty(ra.bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")

    def lap(dks, dvs, dq):
        bw = ra.RingBackward(qd, d_out, out, lse, kb[0], ring_size=P, workspace=ws, stream=s)
        for j in oracle.ring_visit_order(P, rank):
            bw.step(kb[j], vb[j], dks[j], dvs[j], CONTIG, q_off, j * n)
        bw.finalize(dq)
        return bw

    def buffers():
        return ([torch.zeros(kb[j].shape, dtype=torch.float32, device="cuda") for j in range(P)],
                [torch.zeros(vb[j].shape, dtype=torch.float32, device="cuda") for j in range(P)],
                torch.empty((B, Hq, n, d), dtype=torch.float32, device="cuda"))

    dks_e, dvs_e, dq_e = buffers()
    with torch.cuda.stream(s):
        lap(dks_e, dvs_e, dq_e).close()
    s.synchronize()
    # the eager gradients against the oracle's own forward and backward steps
    q64, k64, v64, do64 = to64(q), to64(k), to64(v), to64(d_out)
    q_pos = q_off + np.arange(n)
    o_ref, lse_ref = oracle.dense_attention(q64, k64, v64, q_pos, np.arange(N), True)
    D = oracle.backward_row_terms(do64, o_ref)
    dq_ref = np.zeros_like(q64)
    for j in range(P):
        kp = np.arange(j * n, (j + 1) * n)
        gq, gk, gv = oracle.backward_block(q64, k64[:, :, kp], v64[:, :, kp], do64, lse_ref, D, q_pos, kp, True)
        dq_ref += gq
        assert_bf16_close(to64(dks_e[j]), gk, f"eager dK block {j}", rowwise=None)
        assert_bf16_close(to64(dvs_e[j]), gv, f"eager dV block {j}", rowwise=None)
    assert_bf16_close(to64(dq_e), dq_ref, "eager dQ", rowwise=None)

    dks_g, dvs_g, dq_g = buffers()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bw_g = lap(dks_g, dvs_g, dq_g)
    for r in range(REPLAYS):
        with torch.cuda.stream(s):
            for x in dks_g + dvs_g:                    # the step accumulates into dK_j, dV_j
                x.zero_()
            dq_g.fill_(float("nan"))
            g.replay()
        s.synchronize()
        assert torch.equal(dq_g, dq_e), f"replay {r}: dQ differs"
        for j in range(P):
            assert torch.equal(dks_g[j], dks_e[j]), f"replay {r}: dK of block {j} differs"
            assert torch.equal(dvs_g[j], dvs_e[j]), f"replay {r}: dV of block {j} differs"
        _eager_noise(qd)
    bw_g.close()


def test_split_kv_merge_graph_replays_match_eager():
    """Shard states over ragged key ranges, then ra_merge_states into a merged state and O, lse:
    the steps and the merge captured whole on one stream."""
    import exact_long_context_amd as ra
    Hq, Hkv, n, d = 8, 2, 3, 128
    cuts = [0, 700, 701, 1900, 2600]
    N = cuts[-1]
    say(f"  graph merge: {len(cuts) - 1} shard states over {N} keys")
    q, k, v = synth.random_case(961, 1, Hq, Hkv, n, N, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    s = torch.cuda.Stream()
    desc = ra.desc_for(qd, kd, 1, stream=s)
    nbytes = ra.workspace_bytes(desc)
    part_ws = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in cuts[:-1]]
    merged = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def run(out, lse):
        sts = []
        for w, a, b in zip(part_ws, cuts[:-1], cuts[1:]):
            st = ra.RingState(qd, kd, stream=s, workspace=w)
            st.step(kd[:, :, a:b], vd[:, :, a:b], NONE)
            sts.append(st)
        ra.merge_states(desc, part_ws, merged=merged, out=out, lse=lse)
        return sts

    out_e = torch.empty((1, Hq, n, d), dtype=torch.float32, device="cuda")
    lse_e = torch.empty((1, Hq, n), dtype=torch.float32, device="cuda")
    merged.fill_(0xEE)                                 # the layout's padding is never written
    with torch.cuda.stream(s):
        for st in run(out_e, lse_e):
            st.close()
    s.synchronize()
    merged_e = merged.clone()
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), np.arange(n), np.arange(N), False)
    assert_bf16_close(to64(out_e), ref, "eager merged O")
    assert np.max(np.abs(to64(lse_e) - ref_lse)) <= 2e-2

    out_g = torch.full_like(out_e, float("nan"))
    lse_g = torch.full_like(lse_e, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sts = run(out_g, lse_g)
    for r in range(REPLAYS):
        with torch.cuda.stream(s):
            out_g.fill_(float("nan"))
            merged.fill_(0xEE)
            for w in part_ws:
                w.fill_(0x5A)
            g.replay()
        s.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), f"replay {r}: O or lse differs"
        assert torch.equal(merged, merged_e), f"replay {r}: merged state differs"
        _eager_noise(qd)
    for st in sts:
        st.close()
