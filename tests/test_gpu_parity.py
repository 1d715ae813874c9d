"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Sizes here let the oracle compute every output element, span several tiles
and end on ragged tails.  Full-size workloads are in test_gpu_sampled_fullsize.py.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (F32_REL, assert_bf16_close, assert_f32_close, lap_with_steps, require_gpu, say,
                      to64)

pytestmark = pytest.mark.gpu

NONE, CONTIG, STRIPED, ZIGZAG = 0, 1, 2, 3
LAYOUT = {NONE: "contiguous", CONTIG: "contiguous", STRIPED: "striped", ZIGZAG: "zigzag"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import exact_long_context_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


def _blocks(k, v, P, layout, dev="cuda"):
    from exact_long_context_amd.workload import shard_blocks
    return shard_blocks(k.to(dev), v.to(dev), P, layout)


# ---------------------------------------------------------------------------
# tiny exactness workload: N=256, P=4, one head, d=64, fp32
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mask", [NONE, CONTIG, ZIGZAG])
@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_tiny_fp32_workload(mask, rank):
    w = synth.WORKLOADS["tiny_fp32_n256_p4"]
    q_all, k, v = synth.workload_tensors(w, rank)
    n = w.n_local
    q_pos = oracle.tokens_of_rank(w.N, w.P, LAYOUT[mask], rank)
    q = q_all[:, :, q_pos].contiguous()
    kb, vb = _blocks(k, v, w.P, LAYOUT[mask])
    say(f"  tiny fp32 rank={rank} mask={mask}")
    o, lse, stats = lap_with_steps(q.cuda(), kb, vb, rank, mask, w.P)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(w.N), mask != NONE)
    assert_f32_close(to64(o), ref, f"O rank {rank}")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), fin)
    assert np.max(np.abs(to64(lse)[fin] - ref_lse[fin])) <= 1e-5 * max(1.0, np.max(np.abs(ref_lse)))
    pairs = oracle.live_pair_count(q_pos, np.arange(w.N), mask != NONE)
    assert stats["live_pairs"] == pairs
    if mask == CONTIG:
        assert stats["blocks_skipped"] == w.P - 1 - rank
    if mask == ZIGZAG:   # chunk 2P-1-r is later than every rank's first chunk: no block is empty
        assert stats["blocks_skipped"] == 0


# ---------------------------------------------------------------------------
# random small shapes: both dtypes, GQA, every mask, ragged tails
# ---------------------------------------------------------------------------

CASES = [
    # dtype, B, Hq, Hkv, d, N, P, rank, mask
    ("bf16", 1, 2, 2, 128, 1024, 4, 2, NONE),
    ("bf16", 2, 4, 2, 128, 1200, 4, 3, CONTIG),      # 300-token blocks: ragged tiles
    ("bf16", 1, 8, 1, 128, 1024, 8, 5, STRIPED),     # GQA 8:1
    ("bf16", 1, 4, 4, 64, 800, 4, 1, STRIPED),       # d = 64, 200-token blocks
    ("bf16", 2, 6, 3, 64, 1000, 2, 1, CONTIG),       # 500-token blocks
    ("bf16", 1, 2, 1, 128, 4 * 1037, 4, 3, CONTIG),  # odd block length
    ("f32", 1, 2, 1, 128, 768, 4, 2, STRIPED),
    ("f32", 2, 4, 2, 64, 600, 3, 1, CONTIG),         # 200-token blocks
    ("f32", 1, 3, 3, 128, 500, 5, 4, NONE),          # 100-token blocks
    ("bf16", 1, 4, 2, 128, 2048, 4, 1, ZIGZAG),      # 256-token chunks
    ("bf16", 2, 2, 1, 128, 1800, 3, 2, ZIGZAG),      # 300-token chunks: ragged tiles
    ("bf16", 1, 4, 4, 64, 1600, 4, 0, ZIGZAG),       # d = 64, 200-token chunks
    ("f32", 1, 2, 1, 128, 1200, 3, 1, ZIGZAG),       # 200-token chunks
    ("f32", 2, 2, 2, 64, 960, 4, 3, ZIGZAG),         # 120-token chunks
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}-H{c[2]}x{c[3]}-d{c[4]}-N{c[5]}-P{c[6]}-r{c[7]}-m{c[8]}"
                                             for c in CASES])
def test_random_small_lap(case):
    dtype, B, Hq, Hkv, d, N, P, rank, mask = case
    layout = LAYOUT[mask]
    seed = zlib.crc32(repr(case).encode()) % 1000
    q_pos = oracle.tokens_of_rank(N, P, layout, rank)
    n = q_pos.size
    q, k, v = synth.random_case(seed, B, Hq, Hkv, n, N, d, dtype)
    kb, vb = _blocks(k, v, P, layout)
    say(f"  case {case}")
    o, lse, stats = lap_with_steps(q.cuda(), kb, vb, rank, mask, P)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), mask != NONE)
    got = to64(o)
    assert np.isfinite(got).all()
    if dtype == "bf16":
        assert_bf16_close(got, ref, "O")
    else:
        assert_f32_close(got, ref, "O")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), fin)
    assert np.max(np.abs(to64(lse)[fin] - ref_lse[fin])) <= (2e-2 if dtype == "bf16" else 1e-5) * \
        max(1.0, float(np.max(np.abs(ref_lse[fin]))))
    assert stats["live_pairs"] == B * Hq * oracle.live_pair_count(q_pos, np.arange(N), mask != NONE)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mask,rank", [(STRIPED, 1), (STRIPED, 6), (CONTIG, 5), (NONE, 2), (ZIGZAG, 1),
                                       (ZIGZAG, 6)])
def test_lap_in_shuffled_block_order(dtype, mask, rank):
    """Blocks in a seeded random order: the first blocks may leave rows with no visible key
    (striped blocks after the rank's own), which the state must carry through unchanged."""
    N, P, Hq, Hkv = 2048, 8, 4, 2
    layout = LAYOUT[mask]
    q_pos = oracle.tokens_of_rank(N, P, layout, rank)
    q, k, v = synth.random_case(23 + rank, 1, Hq, Hkv, q_pos.size, N, 128, dtype)
    kb, vb = _blocks(k, v, P, layout)
    order = [int(j) for j in np.random.default_rng(rank).permutation(P)]
    if mask == STRIPED:   # start with a block that sees strictly fewer keys than the rows
        order.remove(P - 1)
        order.insert(0, P - 1)
    if mask == ZIGZAG and rank < P - 1:
        # start with a block whose two chunks are both later than the rank's first chunk:
        # that chunk's rows get no allowed pair in the first step of a fresh state
        order.remove(P - 1)
        order.insert(0, P - 1)
    say(f"  order {order}")
    o, lse, _ = lap_with_steps(q.cuda(), kb, vb, rank, mask, P, order=order)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), mask != NONE)
    got = to64(o)
    assert np.isfinite(got).all()
    if dtype == "bf16":
        assert_bf16_close(got, ref, "O")
    else:
        assert_f32_close(got, ref, "O")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mask", [CONTIG, STRIPED, ZIGZAG])
def test_mask_and_skip_decisions_bit_exact(dtype, mask):
    """The kernel's own counts of unmasked tiles, masked tiles and scored pairs equal the
    oracle's enumeration with the kernel's tile sizes, block by block."""
    import exact_long_context_amd as ra
    N, P, rank, Hq = 2048, 4, 2, 2
    layout = LAYOUT[mask]
    q_pos = oracle.tokens_of_rank(N, P, layout, rank)
    n = q_pos.size
    q, k, v = synth.random_case(7, 1, Hq, 1, n, N, 128, dtype)
    kb, vb = _blocks(k, v, P, layout)
    qd = q.cuda()
    for j in range(P):
        kp = oracle.tokens_of_rank(N, P, layout, j)
        counters = torch.zeros(5, dtype=torch.int64, device="cuda")
        st = ra.RingState(qd, kb[0], ring_size=P)
        st.set_debug_counters(counters)
        qo, ko = ra.block_offsets(mask, rank, j, n, n)
        st.step(kb[j], vb[j], mask, qo, ko)
        plan = st.stats()
        st.finalize()
        torch.cuda.synchronize()
        c = counters.cpu().tolist()[:3]
        if mask == ZIGZAG:   # the kernel tiles each (query chunk, key chunk) pair on its own
            cl = n // 2
            cls = np.concatenate([oracle.tile_classes(q_pos[a * cl:(a + 1) * cl], kp[b * cl:(b + 1) * cl],
                                                      plan["tile_q"], plan["tile_k"], True)
                                  for a in range(2) for b in range(2)], axis=None)
        else:
            cls = oracle.tile_classes(q_pos, kp, plan["tile_q"], plan["tile_k"], True)
        want = [Hq * int((cls == oracle.FULL).sum()), Hq * int((cls == oracle.PARTIAL).sum()),
                Hq * oracle.live_pair_count(q_pos, kp, True)]
        say(f"    block {j}: kernel {c} oracle {want}")
        if want[2] == 0:
            assert c == [0, 0, 0] and plan["blocks_skipped"] == 1
        else:
            assert c == want
        st.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout,mask", [("contiguous", CONTIG), ("striped", STRIPED), ("zigzag", ZIGZAG)])
def test_single_visible_key_row_is_exact(dtype, layout, mask):
    """Global position 0 (rank 0, local row 0) may see only key 0: O = V[key 0] exactly."""
    N, P, d = 1024, 4, 128
    q_pos = oracle.tokens_of_rank(N, P, layout, 0)
    q, k, v = synth.random_case(11, 1, 2, 1, q_pos.size, N, d, dtype)
    kb, vb = _blocks(k, v, P, layout)
    o, lse, _ = lap_with_steps(q.cuda(), kb, vb, 0, mask, P)
    torch.cuda.synchronize()
    got = o[0, :, 0].cpu()
    want = v[0, 0, 0].to(torch.float32).expand_as(got)
    assert torch.equal(got, want)


def test_order_invariance_and_state_resume_bitwise():
    import exact_long_context_amd as ra
    N, P, rank = 2048, 4, 1
    q_pos = oracle.tokens_of_rank(N, P, "striped", rank)
    q, k, v = synth.random_case(13, 1, 4, 2, q_pos.size, N, 128, "bf16")
    kb, vb = _blocks(k, v, P, "striped")
    qd = q.cuda()
    base, _, _ = lap_with_steps(qd, kb, vb, rank, STRIPED, P)
    rev, _, _ = lap_with_steps(qd, kb, vb, rank, STRIPED, P, order=list(reversed(oracle.ring_visit_order(P, rank))))
    ref, _ = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), True)
    assert_bf16_close(to64(rev), ref, "reversed order")
    # checkpoint after two blocks, resume from a copy of the workspace, finish: bit-identical
    order = oracle.ring_visit_order(P, rank)
    n = q_pos.size
    st = ra.RingState(qd, kb[0], ring_size=P)
    for j in order[:2]:
        st.step(kb[j], vb[j], STRIPED, *ra.block_offsets(STRIPED, rank, j, n, n))
    saved = st.workspace.clone()
    st.close()
    st2 = ra.RingState(qd, kb[0], ring_size=P, workspace=saved, resume=True)
    for j in order[2:]:
        st2.step(kb[j], vb[j], STRIPED, *ra.block_offsets(STRIPED, rank, j, n, n))
    o2, _ = st2.finalize()
    torch.cuda.synchronize()
    assert torch.equal(o2, base)
    # the exported state satisfies its invariant: m is the running max (base 2) per row
    st3 = ra.RingState(qd, kb[0], ring_size=P)
    for j in order:
        st3.step(kb[j], vb[j], STRIPED, *ra.block_offsets(STRIPED, rank, j, n, n))
    torch.cuda.synchronize()
    o_acc, m, l_ = (t.cpu().double().numpy() for t in st3.state_views())
    s = np.einsum("hid,htd->hit", to64(q)[0], np.repeat(to64(k)[0], 2, axis=0)) / math.sqrt(128)
    ok = oracle.allowed_mask(q_pos, np.arange(N), True)
    xmax = np.where(ok, s, -np.inf).max(axis=-1) * math.log2(math.e)
    assert np.all(m[0] >= xmax - 32.0) and np.all(m[0] <= xmax + 1e-3)
    st3.close()


@pytest.mark.parametrize("N", [4096, 32768], ids=["blocks512", "blocks4096"])
def test_emulated_ring_lap_matches_steps_and_poison(N):
    """The emulated lap equals the same blocks stepped one by one and then finalized, bit for
    bit, with and without poisoned receive buffers.  The non-causal lap's last step finalizes in
    its own write-back; the other layouts' last steps leave rows without a visible key (or skip
    the block), so their laps run the separate finalize pass."""
    import exact_long_context_amd as ra
    P = 8
    # contiguous ranks 0 and 2 skip seven and five blocks: their receive buffers are freed on
    # arrival, while the poison fill and the copies still run
    cases = ((NONE, 3), (CONTIG, 6), (STRIPED, 5), (CONTIG, 0), (CONTIG, 2))
    if N > 4096:
        cases += ((ZIGZAG, 1),)
    for mask, rank in cases:
        layout = LAYOUT[mask]
        q_pos = oracle.tokens_of_rank(N, P, layout, rank)
        q, k, v = synth.random_case(17 + mask, 1, 4, 4 if N == 4096 else 2, q_pos.size, N, 128, "bf16")
        kb, vb = _blocks(k, v, P, layout)
        qd = q.cuda()
        o_steps, lse_steps, st_steps = lap_with_steps(qd, kb, vb, rank, mask, P)
        ring = ra.EmulatedRing(kb, vb)
        o_ring, lse_ring, st_ring = ring.lap(qd, rank, mask)
        o_pois, lse_pois, _ = ring.lap(qd, rank, mask, poison=True)
        torch.cuda.synchronize()
        say(f"  emulated lap mask={mask} rank={rank} stats={st_ring}")
        assert torch.equal(o_ring, o_steps) and torch.equal(o_pois, o_steps)
        assert torch.equal(lse_ring, lse_steps) and torch.equal(lse_pois, lse_steps)
        assert st_ring == st_steps


def test_degenerate_inputs():
    import exact_long_context_amd as ra
    # empty query slice
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((1, 2, 64, 128), device="cuda").to(torch.bfloat16)
    st = ra.RingState(q, k, ring_size=2)
    st.step(k, k, NONE)
    o, lse = st.finalize()
    assert o.numel() == 0
    st.close()
    # every block strictly in the future (a partial lap of rank 0): O = 0, lse = -inf
    q = torch.randn((1, 2, 100, 128), device="cuda").to(torch.bfloat16)
    st = ra.RingState(q, k, ring_size=4)
    for j in (1, 2, 3):
        st.step(k, k, CONTIG, 0, j * 100)
    o, lse = st.finalize()
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0 and torch.isneginf(lse).all()
    assert st.stats()["blocks_run"] == 0
    st.close()
    # zero-length blocks are no-ops
    st = ra.RingState(q, k, ring_size=4)
    st.step(k[:, :, :0], k[:, :, :0], NONE)
    st.step(k, k, NONE)
    o, _ = st.finalize()
    st2 = ra.RingState(q, k, ring_size=4)
    st2.step(k, k, NONE)
    o2, _ = st2.finalize()
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    st.close()
    st2.close()
    # a single-row, single-key lap
    q1 = torch.randn((1, 1, 1, 64), device="cuda")
    k1 = torch.randn((1, 1, 1, 64), device="cuda")
    v1 = torch.randn((1, 1, 1, 64), device="cuda")
    st = ra.RingState(q1, k1, ring_size=1)
    st.step(k1, v1, CONTIG, 0, 0)
    o, lse = st.finalize()
    torch.cuda.synchronize()
    assert torch.equal(o[0, 0, 0], v1[0, 0, 0])
    st.close()


def test_strided_views_without_copies():
    """Q and KV given as [B, n, H, d] views (token-major) through the stride arguments."""
    N, P, rank, Hq, Hkv, d = 1024, 4, 2, 4, 2, 128
    q_pos = oracle.tokens_of_rank(N, P, "contiguous", rank)
    q, k, v = synth.random_case(19, 1, Hq, Hkv, q_pos.size, N, d, "bf16")
    n = q_pos.size
    q_tm = q.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)   # strides (n*H*d, d, H*d)
    kb = [k[:, :, j * n:(j + 1) * n].permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3) for j in range(P)]
    vb = [v[:, :, j * n:(j + 1) * n].permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3) for j in range(P)]
    o, _, _ = lap_with_steps(q_tm, kb, vb, rank, CONTIG, P)
    torch.cuda.synchronize()
    ref, _ = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), True)
    assert_bf16_close(to64(o), ref, "token-major views")


@pytest.mark.parametrize("dtype,nk", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 320),
                                      ("f32", 320)])
def test_steps_are_bitwise_repeatable_across_many_workgroups(dtype, nk):
    """The same fresh step and resumed step, twenty times over: the state (m, l, O~) must be
    bit-identical every time.  16384 rows x 16 heads fill the chip with co-resident
    workgroups, so a race between workgroups or between the waves of one (a tile buffer reused
    too early, a read not yet landed) shows up as rows that change from run to run.  Blocks of
    64 to 256 keys cover the bf16 kernel's first step, whose look-ahead copy refills the K
    buffer the prologue's scores read: past the block's end those copies return zeros almost
    at once, so a wave that started them before the others had read the buffer would corrupt
    their first tile."""
    import exact_long_context_amd as ra
    H, n = 16, 16384
    g = torch.Generator(device="cpu").manual_seed(77)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = (torch.randn(1, H, n, 128, generator=g) * 0.3).to(tdt).cuda()
    k = (torch.randn(1, H, 2 * nk, 128, generator=g) * 0.3).to(tdt).cuda()
    v = torch.randn(1, H, 2 * nk, 128, generator=g).to(tdt).cuda()
    say(f"  repeatability {dtype}: {H} heads x {n} rows, two blocks of {nk} keys")
    states = []
    for _ in range(20):
        st = ra.RingState(q, k[:, :, :nk], ring_size=1)
        st.step(k[:, :, :nk], v[:, :, :nk], NONE)
        st.step(k[:, :, nk:], v[:, :, nk:], CONTIG, 10 * nk, 0)
        torch.cuda.synchronize()
        states.append(st.workspace.clone())
        st.close()
    for other in states[1:]:
        diff = (states[0] != other).nonzero()
        assert diff.numel() == 0, f"{diff.numel()} workspace bytes differ between identical runs"


# ---------------------------------------------------------------------------
# the rescale of rows that already hold keys (exp(old max - new max) on a new maximum)
# ---------------------------------------------------------------------------

def _planted_lap_inputs(dtype, mask, rank, N, P, Hq, Hkv, order, seed):
    """Small random inputs with planted score ladders: the block visited at step u carries
    ladder_levels(u) through channel 0, so rows' maxima climb by 35-40 natural units between
    blocks and inside blocks."""
    from gpu_util import ladder_levels, plant_score_levels
    layout = LAYOUT[mask]
    q_pos = oracle.tokens_of_rank(N, P, layout, rank)
    q, k, v = synth.random_case(seed, 1, Hq, Hkv, q_pos.size, N, 128, dtype, value_scale=0.3)
    v = synth.random_case(seed + 1, 1, Hq, Hkv, q_pos.size, N, 128, dtype)[2]
    rng = np.random.default_rng(seed)
    levels = np.zeros(N)
    for u, j in enumerate(order):
        kp = oracle.tokens_of_rank(N, P, layout, j)
        levels[kp] = ladder_levels(u, kp.size, rng)
    plant_score_levels(q, k, levels)
    return q_pos, q, k, v


def _assert_live_rescales_ran(q, kb, vb, rank, mask, P, order, dtype, bounded=None):
    """Run the lap twice, with and without the kernels' debug counters: the counting variant
    must report (row, tile) events in which a row holding keys moved its reference, and give
    bit for bit the product kernel's result.  The product run also checks, from the state
    after every step, that some rows holding keys raised m by more than 32 (base 2) in one
    step, which only the rescale path does."""
    import exact_long_context_amd as ra
    counters = torch.zeros(5, dtype=torch.int64, device="cuda")
    o_dbg, lse_dbg, _ = lap_with_steps(q, kb, vb, rank, mask, P, order=order, debug_counters=counters)
    n = q.shape[2]
    st = ra.RingState(q, kb[0], ring_size=P)
    jumps = 0
    m_prev = l_prev = None
    for j in order:
        st.step(kb[j], vb[j], mask, *ra.block_offsets(mask, rank, j, n, n))
        _, m, l_ = (t.clone() for t in st.state_views())
        if m_prev is not None:
            live = (l_prev > 0) & torch.isfinite(m_prev)
            jumps += int(((m - m_prev > 32.0) & live).sum().item())
        m_prev, l_prev = m, l_
    o, lse = st.finalize()
    st.close()
    torch.cuda.synchronize()
    c = counters.cpu().tolist()
    say(f"    live-row reference moves counted: {c[3]}; rows jumping > 32 between steps: {jumps}")
    assert c[3] > 0, "no row that held keys moved its reference: the rescale path did not run"
    assert jumps > 0
    if bounded is not None:
        say(f"    (wave, tile) events decided by the key-norm bound: {c[4]}")
        assert (c[4] > 0) == bounded
    assert torch.equal(o, o_dbg) and torch.equal(lse, lse_dbg)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shuffled", [False, True], ids=["ring", "shuffled"])
@pytest.mark.parametrize("mask,rank", [(NONE, 2), (CONTIG, 7), (STRIPED, 5), (ZIGZAG, 1)])
def test_live_rows_rescale_on_planted_score_ladders(dtype, shuffled, mask, rank):
    """Extreme scores ("Ring Attention：把超长序列沿设备环流动", section 正确性测试应覆盖哪些边界,
    online-softmax stability at extreme scores): each row's first block scores near -40, and
    later blocks raise the row maximum by 35-40 natural units, at a block's first tile and in
    the middle of a launch.  Rows that already hold keys must rescale l and O~ by
    2^(m_old - m_new) ("Ring attention" MCQ page, body)."""
    N, P, Hq, Hkv = 4096, 8, 4, 2
    layout = LAYOUT[mask]
    order = oracle.ring_visit_order(P, rank)
    if shuffled:
        order = [int(j) for j in np.random.default_rng(100 + rank).permutation(P)]
    q_pos, q, k, v = _planted_lap_inputs(dtype, mask, rank, N, P, Hq, Hkv, order, 31 + rank + 7 * mask)
    kb, vb = _blocks(k, v, P, layout)
    say(f"  planted ladders {dtype} mask={mask} rank={rank} order={order}")
    o, lse = _assert_live_rescales_ran(q.cuda(), kb, vb, rank, mask, P, order, dtype)
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), mask != NONE)
    got = to64(o)
    assert np.isfinite(got).all()
    if dtype == "bf16":
        assert_bf16_close(got, ref, "O")
    else:
        # An fp32 score s carries a rounding error of about |s| * 2^-24 per operation, and its
        # weight e^s inherits it as a relative error: the bound that holds for unit-scale
        # logits (|s| up to about 5, as in the tiny exactness workload) grows linearly with
        # the largest logit here (about 100).  A plain all-fp32 evaluation of the definition
        # on these inputs is off by 5.7e-5 normwise.
        kk = np.repeat(to64(k)[0], Hq // Hkv, 0)
        s_max = float(np.max(np.abs(to64(q)[0] @ kk.transpose(0, 2, 1)))) / math.sqrt(128)
        rel = assert_f32_close(got, ref, "O", tol=F32_REL * max(1.0, s_max / 5.0))
        say(f"    largest |logit| {s_max:.1f}: fp32 bound {F32_REL * max(1.0, s_max / 5.0):.2e}, measured {rel:.2e}")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), fin)
    tol = (2e-2 if dtype == "bf16" else 1e-5) * max(1.0, float(np.max(np.abs(ref_lse[fin]))))
    assert np.max(np.abs(to64(lse)[fin] - ref_lse[fin])) <= tol


@pytest.mark.parametrize("mask,rank", [(NONE, 3), (STRIPED, 6), (ZIGZAG, 2)])
def test_key_norm_bound_with_planted_ladders(mask, rank):
    """Blocks of 4096 keys, long enough for the key-norm bound on the reference (|x| <= |q| |k|,
    checked once per tile in place of the scores' maximum).  On the planted ladders it holds
    on the plateau blocks and fails where a block climbs, so both paths run in one lap: the
    bound must decide some tiles, rows holding keys must still rescale, and the result must
    match the oracle and the counting variant bit for bit."""
    N, P, Hq, Hkv = 32768, 8, 4, 2
    layout = LAYOUT[mask]
    order = oracle.ring_visit_order(P, rank)
    q_pos, q, k, v = _planted_lap_inputs("bf16", mask, rank, N, P, Hq, Hkv, order, 71 + rank + 7 * mask)
    kb, vb = _blocks(k, v, P, layout)
    say(f"  key-norm bound, planted ladders: mask={mask} rank={rank}, {P} blocks of {N // P} keys")
    o, lse = _assert_live_rescales_ran(q.cuda(), kb, vb, rank, mask, P, order, "bf16", bounded=True)
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), mask != NONE)
    assert_bf16_close(to64(o), ref, "O")
    fin = np.isfinite(ref_lse)
    assert np.max(np.abs(to64(lse)[fin] - ref_lse[fin])) <= 2e-2 * max(1.0, float(np.max(np.abs(ref_lse[fin]))))


@pytest.mark.parametrize("case", ["loose", "ragged_zigzag", "d64"])
def test_key_norm_bound_edges(case):
    """Where the bound cannot help.  loose: queries and keys of scale 4 make |q| |k| far larger
    than any score, so the bound never decides a tile and every tile takes the scores' maximum.
    ragged_zigzag: chunks of 4100 keys, so the second key chunk of each block does not start
    on a 32-key tile; its launches go without bounds while the first chunk's use them.  d64:
    head dimension 64 (the other instantiation of the norm pass and of the step kernel).  All
    must match the oracle."""
    import exact_long_context_amd as ra
    d = 128
    if case == "loose":
        N, P, rank, mask, Hq, Hkv, vs = 32768, 8, 5, STRIPED, 4, 2, 4.0
    elif case == "d64":
        N, P, rank, mask, Hq, Hkv, vs, d = 32768, 8, 3, STRIPED, 4, 2, None, 64
    else:
        N, P, rank, mask, Hq, Hkv, vs = 16400, 2, 1, ZIGZAG, 4, 2, None
    layout = LAYOUT[mask]
    q_pos = oracle.tokens_of_rank(N, P, layout, rank)
    kw = {} if vs is None else {"value_scale": vs}
    q, k, _ = synth.random_case(83 + P, 1, Hq, Hkv, q_pos.size, N, d, "bf16", **kw)
    v = synth.random_case(84 + P, 1, Hq, Hkv, q_pos.size, N, d, "bf16")[2]   # unit-scale outputs
    kb, vb = _blocks(k, v, P, layout)
    counters = torch.zeros(5, dtype=torch.int64, device="cuda")
    say(f"  key-norm bound, {case}: {P} blocks of {kb[0].shape[2]} keys")
    o, lse, _ = lap_with_steps(q.cuda(), kb, vb, rank, mask, P, debug_counters=counters)
    torch.cuda.synchronize()
    c = counters.cpu().tolist()
    say(f"    (wave, tile) events decided by the bound: {c[4]}")
    if case == "loose":
        assert c[4] == 0
    else:
        assert c[4] > 0
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), True)
    assert_bf16_close(to64(o), ref, "O")
    fin = np.isfinite(ref_lse)
    assert np.max(np.abs(to64(lse)[fin] - ref_lse[fin])) <= 2e-2 * max(1.0, float(np.max(np.abs(ref_lse[fin]))))


def test_live_rows_rescale_after_resume():
    """Checkpoint after two blocks of a planted ladder, resume from a copy of the workspace
    and finish: the resumed launches load states that hold keys and must move their
    reference; the result is bit-identical to the uninterrupted lap and matches the oracle."""
    import exact_long_context_amd as ra
    N, P, rank, mask = 4096, 8, 5, STRIPED
    order = oracle.ring_visit_order(P, rank)
    q_pos, q, k, v = _planted_lap_inputs("bf16", mask, rank, N, P, 4, 2, order, 57)
    kb, vb = _blocks(k, v, P, "striped")
    qd = q.cuda()
    n = q_pos.size
    base, _, _ = lap_with_steps(qd, kb, vb, rank, mask, P, order=order)
    st = ra.RingState(qd, kb[0], ring_size=P)
    for j in order[:2]:
        st.step(kb[j], vb[j], mask, *ra.block_offsets(mask, rank, j, n, n))
    saved = st.workspace.clone()
    st.close()
    counters = torch.zeros(5, dtype=torch.int64, device="cuda")
    st2 = ra.RingState(qd, kb[0], ring_size=P, workspace=saved, resume=True)
    st2.set_debug_counters(counters)
    for j in order[2:]:
        st2.step(kb[j], vb[j], mask, *ra.block_offsets(mask, rank, j, n, n))
    o2, _ = st2.finalize()
    st2.close()
    torch.cuda.synchronize()
    say(f"  resumed lap: live-row reference moves {counters[3].item()}")
    assert counters[3].item() > 0
    assert torch.equal(o2, base)
    ref, _ = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, np.arange(N), True)
    assert_bf16_close(to64(o2), ref, "resumed O")
