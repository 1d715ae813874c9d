"""Pins for the fp64 oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped
rescale term, a sign flip in exp(old - new), an off-by-one in k <= q, a
transposed operand, a wrong striped map, a missing softmax scale) fails at
least one of them:

* torch's scaled_dot_product_attention in float64 on the CPU (one block, the
  library special case) -- catches scale, transposes, the causal diagonal;
* the whole lap reassembled over all ranks equals causal attention on the
  unsharded sequence -- pins positions and both layouts with no position code;
* a pure-Python scalar evaluation with math.exp on tiny inputs;
* closed forms (uniform scores give prefix means; live-pair counts n(n+1)/2);
* exact special cases (single allowed key returns V exactly; masked pairs get
  exactly zero weight);
* the ring table printed on the pages.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import EMPTY, FULL, PARTIAL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _golden_rows(name):
    return [[int(x) for x in ln.split()] for ln in open(os.path.join(GOLDEN, name))
            if ln.strip() and not ln.startswith("#")]


def _blocks_for(k, v, N, P, layout):
    """Per-rank KV blocks with their global positions (from token ownership)."""
    out = []
    for j in range(P):
        pos = oracle.tokens_of_rank(N, P, layout, j)
        out.append((k[:, :, pos], v[:, :, pos], pos))
    return out


# ---------------------------------------------------------------------------
# The ring itself
# ---------------------------------------------------------------------------

def test_ring_table_matches_page():
    rows = [tuple(int(x) for x in ln.split()) for ln in open(os.path.join(GOLDEN, "ring_table_4dev.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 8
    for rnd, dev, blk in rows:
        assert oracle.ring_visit_order(4, dev)[rnd] == blk


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16, 64])
def test_lap_visits_every_block_once(P):
    for r in range(P):
        order = oracle.ring_visit_order(P, r)
        assert order[0] == r
        assert sorted(order) == list(range(P))


def test_lap_block_counts_match_page():
    rows = [tuple(int(x) for x in ln.split()) for ln in open(os.path.join(GOLDEN, "lap_block_counts.txt"))
            if ln.strip() and not ln.startswith("#")]
    for P, local, remote in rows:
        for r in range(P):
            order = oracle.ring_visit_order(P, r)
            assert sum(1 for j in order if j == r) == local
            assert sum(1 for j in order if j != r) == remote


def test_token_layouts():
    # contiguous: device p local index i -> global p * N_local + i ([P3] 位置编码必须使用全局位置)
    N, P = 64, 4
    for p in range(P):
        pos = oracle.tokens_of_rank(N, P, "contiguous", p)
        assert list(pos) == [p * (N // P) + i for i in range(N // P)]
    # striped: token t lives on rank t mod P
    for p in range(P):
        pos = oracle.tokens_of_rank(N, P, "striped", p)
        assert all(int(t) % P == p for t in pos)
        assert len(pos) == N // P
    # zigzag: 2P chunks, rank p holds chunks p and 2P-1-p ([P1] "Striping the sequence to
    # flatten the triangle"), written out in tests/golden/zigzag_chunks_p4.txt
    table = _golden_rows("zigzag_chunks_p4.txt")
    Nz, Pz = 16, 4
    for p, *toks in table:
        assert list(oracle.tokens_of_rank(Nz, Pz, "zigzag", p)) == toks
    # every token has exactly one owner
    for layout in ("contiguous", "striped", "zigzag"):
        allpos = np.concatenate([oracle.tokens_of_rank(N, P, layout, p) for p in range(P)])
        assert sorted(allpos.tolist()) == list(range(N))


def test_token_layouts_when_P_does_not_divide_N():
    # [P3] 正确性测试应覆盖哪些边界: N not a multiple of P, tail-rank padding.  Every shard has
    # ceil(N/P) slots; contiguous device p local index i -> global p * ceil(N/P) + i for the
    # slots that hold a real token; striped keeps token t on rank t mod P.
    assert oracle.shard_capacity(23, 4) == 6 and oracle.shard_capacity(24, 4) == 6
    assert oracle.shard_capacity(25, 4) == 7 and oracle.shard_capacity(1, 8) == 1
    expect_contig = {0: [0, 1, 2, 3, 4, 5], 1: [6, 7, 8, 9, 10, 11], 2: [12, 13, 14, 15, 16, 17],
                     3: [18, 19, 20, 21, 22]}
    expect_striped = {0: [0, 4, 8, 12, 16, 20], 1: [1, 5, 9, 13, 17, 21], 2: [2, 6, 10, 14, 18, 22],
                      3: [3, 7, 11, 15, 19]}
    for p in range(4):
        assert oracle.tokens_of_rank(23, 4, "contiguous", p).tolist() == expect_contig[p]
        assert oracle.tokens_of_rank(23, 4, "striped", p).tolist() == expect_striped[p]
    # N = 9 over 4 ranks: 3 slots each, the last rank holds no real token
    assert [oracle.tokens_of_rank(9, 4, "contiguous", p).tolist() for p in range(4)] == \
        [[0, 1, 2], [3, 4, 5], [6, 7, 8], []]
    with pytest.raises(ValueError):
        oracle.token_owner(23, 4, "zigzag")


# ---------------------------------------------------------------------------
# Dense attention against independent references
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,d", [(1, 1, 64), (4, 2, 32), (8, 1, 16)])
def test_dense_matches_torch_sdpa_fp64(causal, Hq, Hkv, d):
    rng = _rng(1)
    B, N = 2, 96
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    pos = np.arange(N)
    o, lse = oracle.dense_attention(q, k, v, pos, pos, causal)
    G = Hq // Hkv
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=causal).numpy()
    assert _rel(o, ref) <= 1e-12
    # lse: log of the softmax denominator, checked with a direct logsumexp
    s = torch.from_numpy(q) @ kt.transpose(-1, -2) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12


def test_dense_matches_scalar_python_loops():
    rng = _rng(2)
    n, N, d = 5, 7, 3
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    q_pos = np.array([2, 3, 5, 6, 9])
    k_pos = np.array([0, 1, 2, 4, 6, 7, 8])
    for causal in (False, True):
        o, _ = oracle.dense_attention(q, k, v, q_pos, k_pos, causal)
        for i in range(n):
            keys = [t for t in range(N) if (not causal) or k_pos[t] <= q_pos[i]]
            sc = {t: sum(q[0, 0, i, c] * k[0, 0, t, c] for c in range(d)) / math.sqrt(d) for t in keys}
            mx = max(sc.values())
            w = {t: math.exp(sc[t] - mx) for t in keys}
            den = sum(w.values())
            for c in range(d):
                ref = sum(w[t] * v[0, 0, t, c] for t in keys) / den
                assert abs(o[0, 0, i, c] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_dense_rows_and_heads_subset():
    rng = _rng(3)
    q = rng.standard_normal((1, 4, 40, 8))
    k = rng.standard_normal((1, 2, 60, 8))
    v = rng.standard_normal((1, 2, 60, 8))
    qp = np.arange(20, 60)
    kp = np.arange(60)
    full, full_lse = oracle.dense_attention(q, k, v, qp, kp, True)
    rows = np.array([0, 7, 39])
    part, part_lse = oracle.dense_attention(q, k, v, qp, kp, True, heads=[1, 3], rows=rows)
    for h in (1, 3):
        assert np.array_equal(part[0, h, rows], full[0, h, rows])
        assert np.array_equal(part_lse[0, h, rows], full_lse[0, h, rows])
    assert np.isnan(part[0, 0]).all()


# ---------------------------------------------------------------------------
# The ring recipe (blockwise merge) against dense and against the unsharded sequence
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_equals_dense(layout, P, causal):
    rng = _rng(10 + P)
    N, d, Hq, Hkv = 128, 16, 4, 2
    k = rng.standard_normal((1, Hkv, N, d))
    v = rng.standard_normal((1, Hkv, N, d))
    blocks = _blocks_for(k, v, N, P, layout)
    for r in range(P):
        qp = oracle.tokens_of_rank(N, P, layout, r)
        q = rng.standard_normal((1, Hq, qp.size, d))
        o_ring, lse_ring = oracle.blockwise_attention(q, blocks, qp, causal,
                                                      order=oracle.ring_visit_order(P, r))
        o_ref, lse_ref = oracle.dense_attention(q, k, v, qp, np.arange(N), causal)
        assert _rel(o_ring, o_ref) <= 1e-12
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse_ring))
        assert np.max(np.abs(lse_ring[fin] - lse_ref[fin])) <= 1e-12


@pytest.mark.parametrize("layout,N", [("contiguous", 64), ("striped", 64), ("zigzag", 64),
                                      ("contiguous", 61), ("striped", 61), ("contiguous", 9)])
@pytest.mark.parametrize("P", [2, 4])
def test_whole_ring_equals_unsharded_causal_sdpa(layout, N, P):
    """Reassemble every rank's lap; it must equal causal attention on the full sequence.

    The reference here is torch's is_causal lower-triangular mask over global
    token order: no position or layout code of the oracle is involved.  N = 61 and 9 are
    not multiples of P: padded shards whose tail rank holds fewer real tokens (for N = 9,
    P = 4 the last rank holds none).
    """
    rng = _rng(20 + P + N)
    d, H = 8, 2
    q = rng.standard_normal((1, H, N, d))
    k = rng.standard_normal((1, H, N, d))
    v = rng.standard_normal((1, H, N, d))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                         torch.from_numpy(v), is_causal=True).numpy()
    blocks = _blocks_for(k, v, N, P, layout)
    got = np.full_like(q, np.nan)
    for r in range(P):
        qp = oracle.tokens_of_rank(N, P, layout, r)
        o, _ = oracle.blockwise_attention(q[:, :, qp], blocks, qp, True,
                                          order=oracle.ring_visit_order(P, r))
        got[:, :, qp] = o
    assert _rel(got, ref) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_visit_order_invariance(causal):
    rng = _rng(30)
    N, P, d = 128, 8, 16
    k = rng.standard_normal((1, 2, N, d))
    v = rng.standard_normal((1, 2, N, d))
    blocks = _blocks_for(k, v, N, P, "contiguous")
    r = 5
    qp = oracle.tokens_of_rank(N, P, "contiguous", r)
    q = rng.standard_normal((1, 2, qp.size, d))
    base, _ = oracle.blockwise_attention(q, blocks, qp, causal, order=oracle.ring_visit_order(P, r))
    orders = [list(reversed(oracle.ring_visit_order(P, r)))]
    orders += [list(_rng(100 + i).permutation(P)) for i in range(5)]
    for order in orders:
        o, _ = oracle.blockwise_attention(q, blocks, qp, causal, order=order)
        assert _rel(o, base) <= 1e-12


def test_blockwise_stable_at_extreme_scores():
    # logits in the hundreds: without max subtraction exp would overflow
    rng = _rng(31)
    N, P, d = 96, 4, 8
    q = 60.0 * rng.standard_normal((1, 1, N // P, d))
    k = 60.0 * rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    blocks = _blocks_for(k, v, N, P, "contiguous")
    qp = oracle.tokens_of_rank(N, P, "contiguous", 3)
    for causal in (False, True):
        o, lse = oracle.blockwise_attention(q, blocks, qp, causal, order=oracle.ring_visit_order(P, 3))
        ref, lse_ref = oracle.dense_attention(q, k, v, qp, np.arange(N), causal)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        assert _rel(o, ref) <= 1e-12
        assert np.max(np.abs(lse - lse_ref)) <= 1e-9 * np.max(np.abs(lse_ref))


def test_state_resume_is_identical():
    rng = _rng(32)
    N, P, d = 64, 4, 8
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    blocks = _blocks_for(k, v, N, P, "striped")
    qp = oracle.tokens_of_rank(N, P, "striped", 1)
    q = rng.standard_normal((1, 1, qp.size, d))
    order = oracle.ring_visit_order(P, 1)
    st = oracle.online_state_init(1, 1, qp.size, d)
    for j in order:
        st = oracle.online_block_update(st, q, blocks[j][0], blocks[j][1], qp, blocks[j][2], True)
    st2 = oracle.online_state_init(1, 1, qp.size, d)
    for j in order[:2]:
        st2 = oracle.online_block_update(st2, q, blocks[j][0], blocks[j][1], qp, blocks[j][2], True)
    saved = {key: val.copy() for key, val in st2.items()}
    for j in order[2:]:
        saved = oracle.online_block_update(saved, q, blocks[j][0], blocks[j][1], qp, blocks[j][2], True)
    a = oracle.online_finalize(st)
    b = oracle.online_finalize(saved)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Masks: zero weight for masked pairs, brute force, single-key rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_masked_pairs_get_exactly_zero_weight(layout):
    # V = identity turns the output into the probability matrix itself
    N, P, r = 32, 4, 2
    rng = _rng(40)
    qp = oracle.tokens_of_rank(N, P, layout, r)
    q = rng.standard_normal((1, 1, qp.size, 6))
    k = rng.standard_normal((1, 1, N, 6))
    v = np.eye(N)[None, None]
    w, _ = oracle.dense_attention(q, k, v, qp, np.arange(N), True)
    w = w[0, 0]
    allowed = np.array([[t <= qp[i] for t in range(N)] for i in range(qp.size)])
    assert (w[~allowed] == 0.0).all()
    assert (w[allowed] > 0.0).all()
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # the ring recipe gives the same exact zeros
    blocks = _blocks_for(k, v, N, P, layout)
    wr, _ = oracle.blockwise_attention(q, blocks, qp, True, order=oracle.ring_visit_order(P, r))
    assert (wr[0, 0][~allowed] == 0.0).all()


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_perturbing_masked_keys_leaves_output_bit_identical(layout):
    N, P, r, d = 64, 4, 1, 8
    rng = _rng(41)
    qp = oracle.tokens_of_rank(N, P, layout, r)
    q = rng.standard_normal((1, 1, qp.size, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    blocks = _blocks_for(k, v, N, P, layout)
    order = oracle.ring_visit_order(P, r)
    base, _ = oracle.blockwise_attention(q, blocks, qp, True, order=order)
    future = np.arange(N) > qp.max()           # masked for every local row
    k2, v2 = k.copy(), v.copy()
    k2[:, :, future] += rng.standard_normal(k2[:, :, future].shape)
    v2[:, :, future] += rng.standard_normal(v2[:, :, future].shape)
    got, _ = oracle.blockwise_attention(q, _blocks_for(k2, v2, N, P, layout), qp, True, order=order)
    assert np.array_equal(got, base)
    # per row: perturb only what that row may not see
    i = qp.size // 2
    row_future = np.arange(N) > qp[i]
    k3, v3 = k.copy(), v.copy()
    k3[:, :, row_future] *= -3.0
    v3[:, :, row_future] += 7.0
    d0, _ = oracle.dense_attention(q, k, v, qp, np.arange(N), True, rows=np.array([i]))
    d1, _ = oracle.dense_attention(q, k3, v3, qp, np.arange(N), True, rows=np.array([i]))
    assert np.array_equal(d0[0, 0, i], d1[0, 0, i])


def test_mask_matches_brute_force_positions():
    for layout in ("contiguous", "striped"):
        for P in (1, 2, 4, 16):
            N = 64 if P < 16 else 256
            for r in range(P):
                qp = oracle.tokens_of_rank(N, P, layout, r)
                for j in range(P):
                    kp = oracle.tokens_of_rank(N, P, layout, j)
                    m = oracle.allowed_mask(qp, kp, True)
                    for i in range(0, qp.size, 3):
                        for t in range(0, kp.size, 5):
                            assert m[i, t] == (int(kp[t]) <= int(qp[i]))


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_single_allowed_key_row_returns_that_value_exactly(layout):
    # global position 0 lives on rank 0 at local row 0; only key 0 is allowed
    N, P, d = 256, 4, 64
    rng = _rng(42)
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    qp = oracle.tokens_of_rank(N, P, layout, 0)
    q = rng.standard_normal((1, 1, qp.size, d))
    o, lse = oracle.dense_attention(q, k, v, qp, np.arange(N), True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    blocks = _blocks_for(k, v, N, P, layout)
    o2, _ = oracle.blockwise_attention(q, blocks, qp, True, order=oracle.ring_visit_order(P, 0))
    assert np.array_equal(o2[0, 0, 0], v[0, 0, 0])
    s0 = float(q[0, 0, 0] @ k[0, 0, 0]) / math.sqrt(d)
    assert abs(lse[0, 0, 0] - s0) <= 1e-12 * max(1.0, abs(s0))


def test_uniform_scores_give_prefix_means():
    # Q = 0 makes every allowed score equal: O[i] is the mean of V over the allowed keys
    N, P, d = 128, 4, 8
    rng = _rng(43)
    v = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    for layout in ("contiguous", "striped"):
        for r in range(P):
            qp = oracle.tokens_of_rank(N, P, layout, r)
            q = np.zeros((1, 1, qp.size, d))
            o, _ = oracle.blockwise_attention(q, _blocks_for(k, v, N, P, layout), qp, True,
                                              order=oracle.ring_visit_order(P, r))
            csum = np.cumsum(v[0, 0], axis=0)
            ref = csum[qp] / (qp[:, None] + 1.0)
            assert _rel(o[0, 0], ref) <= 1e-12
            o_nc, _ = oracle.blockwise_attention(q, _blocks_for(k, v, N, P, layout), qp, False)
            assert _rel(o_nc[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), o_nc[0, 0].shape)) <= 1e-12


def test_row_without_any_allowed_key_is_zero():
    # a partial lap (only future blocks) leaves rows empty: O = 0, lse = -inf
    N, P, d = 64, 4, 8
    rng = _rng(44)
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    qp = oracle.tokens_of_rank(N, P, "contiguous", 0)
    q = rng.standard_normal((1, 1, qp.size, d))
    blocks = _blocks_for(k, v, N, P, "contiguous")
    o, lse = oracle.blockwise_attention(q, blocks, qp, True, order=[1, 2, 3])
    assert (o == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------------------
# Live-pair counts and tile classes
# ---------------------------------------------------------------------------

def test_live_pairs_match_brute_force():
    for layout in ("contiguous", "striped"):
        for P in (1, 2, 4, 16):
            N = 64
            for r in range(P):
                qp = oracle.tokens_of_rank(N, P, layout, r)
                for j in range(P):
                    kp = oracle.tokens_of_rank(N, P, layout, j)
                    for causal in (False, True):
                        assert oracle.live_pair_count(qp, kp, causal) == \
                            oracle.brute_force_pair_count(qp, kp, causal)


@pytest.mark.parametrize("name,N,P,r,layout,per_head", [
    ("causal contiguous rank 0", 131072, 8, 0, "contiguous", 134_225_920),
    ("causal contiguous rank 7", 131072, 8, 7, "contiguous", 2_013_274_112),
    ("causal striped P=16 rank 5", 262144, 16, 5, "striped", 2_147_450_880),
    ("causal striped P=64 rank 5", 1048576, 64, 5, "striped", 8_589_508_608),
])
def test_live_pair_closed_forms_at_full_size(name, N, P, r, layout, per_head):
    """Closed forms: a diagonal block holds n(n+1)/2 pairs; a striped block from
    source s holds n(n+1)/2 when s <= r and n(n-1)/2 when s > r; a past
    contiguous block holds n^2 and a future one 0."""
    n = N // P
    qp = oracle.tokens_of_rank(N, P, layout, r)
    total = 0
    for j in range(P):
        kp = oracle.tokens_of_rank(N, P, layout, j)
        c = oracle.live_pair_count(qp, kp, True)
        if layout == "contiguous":
            expect = n * n if j < r else (n * (n + 1) // 2 if j == r else 0)
        else:
            expect = n * (n + 1) // 2 if j <= r else n * (n - 1) // 2
        assert c == expect
        total += c
    assert total == per_head


def _shard_state(q, k, v, q_pos, k_pos, keys, causal):
    st = oracle.online_state_init(q.shape[0], q.shape[1], q.shape[2], v.shape[-1])
    if keys.size:
        st = oracle.online_block_update(st, q, k[:, :, keys], v[:, :, keys], q_pos, k_pos[keys], causal)
    return st


@pytest.mark.parametrize("causal", [False, True])
def test_merged_shard_states_equal_sdpa_over_all_keys(causal):
    """Split-KV: disjoint random key shards, one state each, merged, equal exact attention
    over every key (torch SDPA in float64; no oracle position or layout code involved)."""
    rng = _rng(50)
    N, d, Hq, Hkv, n = 96, 16, 4, 2, 7
    q = rng.standard_normal((1, Hq, n, d))
    k = rng.standard_normal((1, Hkv, N, d))
    v = rng.standard_normal((1, Hkv, N, d))
    q_pos = np.sort(rng.choice(N, size=n, replace=False)) if causal else np.arange(n)
    k_pos = np.arange(N)
    shard = rng.integers(0, 5, size=N)                       # 5 shards, random sizes
    parts = [_shard_state(q, k, v, q_pos, k_pos, np.nonzero(shard == s)[0], causal) for s in range(5)]
    o, lse = oracle.online_finalize(oracle.merge_states(parts))
    kk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
    vv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
    mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None]) if causal else None
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), kk, vv, attn_mask=mask).numpy()
    assert _rel(o, ref) <= 1e-12
    # lse against a direct log-sum-exp over the allowed scores
    s = np.einsum("bhnd,bhkd->bhnk", q, kk.numpy()) / math.sqrt(d)
    if causal:
        s = np.where(mask.numpy(), s, -np.inf)
    ref_lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_merge_order_empty_and_single_parts():
    rng = _rng(51)
    N, d, H, n = 64, 8, 2, 5
    q = rng.standard_normal((1, H, n, d))
    k = rng.standard_normal((1, H, N, d))
    v = rng.standard_normal((1, H, N, d))
    q_pos, k_pos = np.arange(n), np.arange(N)
    parts = [_shard_state(q, k, v, q_pos, k_pos, np.arange(s, N, 3), False) for s in range(3)]
    a = oracle.merge_states(parts)
    b = oracle.merge_states(parts[::-1])
    assert _rel(a["o"] / a["l"][..., None], b["o"] / b["l"][..., None]) <= 1e-14
    # a single part and an added empty part leave the state exactly as it was
    one = oracle.merge_states([parts[0]])
    assert all(np.array_equal(one[x], parts[0][x]) for x in ("m", "l", "o"))
    empty = oracle.online_state_init(1, H, n, d)
    with_empty = oracle.merge_states([parts[1], empty])
    assert all(np.array_equal(with_empty[x], parts[1][x]) for x in ("m", "l", "o"))
    # rows no part has seen: O = 0 and lse = -inf after the merge
    o, lse = oracle.online_finalize(oracle.merge_states([empty, empty]))
    assert not o.any() and np.isneginf(lse).all()


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_ring_backward_sums_to_autograd(layout, Hq, Hkv):
    """Every rank's dQ (summed over its lap's blocks) and every block's dK, dV (summed over
    the ranks it visits) equal torch autograd of causal attention on the whole sequence, in
    float64; the forward lse and O come from torch too, so no oracle forward is involved."""
    rng = _rng(70 + Hq)
    N, P, d = 48, 4, 8
    G = Hq // Hkv
    q = torch.from_numpy(rng.standard_normal((1, Hq, N, d))).requires_grad_()
    k = torch.from_numpy(rng.standard_normal((1, Hkv, N, d))).requires_grad_()
    v = torch.from_numpy(rng.standard_normal((1, Hkv, N, d))).requires_grad_()
    d_out = torch.from_numpy(rng.standard_normal((1, Hq, N, d)))
    kk, vv = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    mask = torch.tril(torch.ones(N, N, dtype=torch.bool))
    s = (q @ kk.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(~mask, -math.inf)
    out = torch.softmax(s, -1) @ vv
    lse = torch.logsumexp(s, -1).detach().numpy()
    out.backward(d_out)
    q_np, k_np, v_np, do_np = q.detach().numpy(), k.detach().numpy(), v.detach().numpy(), d_out.numpy()
    o_np = out.detach().numpy()
    dq = np.zeros_like(q_np)
    dk = np.zeros_like(k_np)
    dv = np.zeros_like(v_np)
    for r in range(P):
        qp = oracle.tokens_of_rank(N, P, layout, r)
        D = oracle.backward_row_terms(do_np[:, :, qp], o_np[:, :, qp])
        for j in oracle.ring_visit_order(P, r):
            kp = oracle.tokens_of_rank(N, P, layout, j)
            gq, gk, gv = oracle.backward_block(q_np[:, :, qp], k_np[:, :, kp], v_np[:, :, kp],
                                               do_np[:, :, qp], lse[:, :, qp], D, qp, kp, True)
            dq[:, :, qp] += gq
            dk[:, :, kp] += gk
            dv[:, :, kp] += gv
    assert _rel(dq, q.grad.numpy()) <= 1e-12
    assert _rel(dk, k.grad.numpy()) <= 1e-12
    assert _rel(dv, v.grad.numpy()) <= 1e-12


def test_backward_terms_against_scalar_loops():
    """D and one block's gradients written out as scalar Python loops over the pairs."""
    rng = _rng(71)
    n, nk, d = 3, 4, 2
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, nk, d))
    v = rng.standard_normal((1, 1, nk, d))
    do = rng.standard_normal((1, 1, n, d))
    o = rng.standard_normal((1, 1, n, d))
    q_pos, k_pos = np.array([1, 2, 3]), np.array([0, 1, 2, 3])
    sc = 0.7
    lse = rng.standard_normal((1, 1, n)) + 2.0
    D = oracle.backward_row_terms(do, o)
    for i in range(n):
        assert abs(D[0, 0, i] - sum(do[0, 0, i, c] * o[0, 0, i, c] for c in range(d))) <= 1e-14
    gq, gk, gv = oracle.backward_block(q, k, v, do, lse, D, q_pos, k_pos, True, scale=sc)
    eq, ek, ev = np.zeros((n, d)), np.zeros((nk, d)), np.zeros((nk, d))
    for i in range(n):
        for t in range(nk):
            if k_pos[t] > q_pos[i]:
                continue
            s_it = sc * sum(q[0, 0, i, c] * k[0, 0, t, c] for c in range(d))
            p_it = math.exp(s_it - lse[0, 0, i])
            dp_it = sum(do[0, 0, i, c] * v[0, 0, t, c] for c in range(d))
            ds_it = p_it * (dp_it - D[0, 0, i])
            for c in range(d):
                ev[t, c] += p_it * do[0, 0, i, c]
                eq[i, c] += sc * ds_it * k[0, 0, t, c]
                ek[t, c] += sc * ds_it * q[0, 0, i, c]
    assert np.max(np.abs(gq[0, 0] - eq)) <= 1e-13
    assert np.max(np.abs(gk[0, 0] - ek)) <= 1e-13
    assert np.max(np.abs(gv[0, 0] - ev)) <= 1e-13


def test_zigzag_balances_the_causal_work():
    """[P1] "Striping the sequence to flatten the triangle": every rank gets one early and
    one late chunk, so the causal work is shared evenly.  Closed form: queries in chunk i
    (c tokens) see i*c^2 + c(c+1)/2 keys in all, so rank r, holding chunks r and 2P-1-r,
    sees (2P-1)c^2 + c^2 + c = 2P c^2 + c, the same for every rank; per block, a chunk pair
    (query chunk a, key chunk b) holds c^2 pairs when b < a, c(c+1)/2 when b == a, else 0."""
    N, P = 131072, 8
    c = N // (2 * P)
    for r in range(P):
        qp = oracle.tokens_of_rank(N, P, "zigzag", r)
        total = 0
        for j in range(P):
            kp = oracle.tokens_of_rank(N, P, "zigzag", j)
            got = oracle.live_pair_count(qp, kp, True)
            expect = 0
            for a in (r, 2 * P - 1 - r):
                for b in (j, 2 * P - 1 - j):
                    expect += c * c if b < a else (c * (c + 1) // 2 if b == a else 0)
            assert got == expect
            total += got
        assert total == 2 * P * c * c + c == 1_073_750_016
    # the contiguous ramp it replaces: rank 0 and rank 7 differ fifteen-fold
    n = N // P
    ramp = [oracle.live_pair_count(oracle.tokens_of_rank(N, P, "contiguous", r), np.arange(N), True)
            for r in (0, P - 1)]
    assert ramp == [n * (n + 1) // 2, (P - 1) * n * n + n * (n + 1) // 2]


def test_zigzag_pair_counts_match_brute_force():
    for P in (1, 2, 3, 4):
        N = 2 * P * 6
        for r in range(P):
            qp = oracle.tokens_of_rank(N, P, "zigzag", r)
            for j in range(P):
                kp = oracle.tokens_of_rank(N, P, "zigzag", j)
                assert oracle.live_pair_count(qp, kp, True) == oracle.brute_force_pair_count(qp, kp, True)


def _brute_tile_classes(qp, kp, tq, tk):
    nqt = -(-len(qp) // tq)
    nkt = -(-len(kp) // tk)
    out = np.empty((nqt, nkt), dtype=np.uint8)
    for a in range(nqt):
        for c in range(nkt):
            rows = [int(x) for x in qp[a * tq:(a + 1) * tq]]
            keys = [int(x) for x in kp[c * tk:(c + 1) * tk]]
            ok = [kk <= qq for qq in rows for kk in keys]
            out[a, c] = EMPTY if not any(ok) else (FULL if all(ok) else PARTIAL)
    return out


def test_tile_classes_match_brute_force():
    for layout in ("contiguous", "striped"):
        for P in (1, 2, 4, 16):
            N = 128 if P < 16 else 512
            for r in (0, P // 2, P - 1):
                qp = oracle.tokens_of_rank(N, P, layout, r)
                for j in range(P):
                    kp = oracle.tokens_of_rank(N, P, layout, j)
                    for tq, tk in ((8, 4), (16, 16), (32, 8), (5, 3)):
                        got = oracle.tile_classes(qp, kp, tq, tk, True)
                        assert np.array_equal(got, _brute_tile_classes(qp, kp, tq, tk))
                    assert (oracle.tile_classes(qp, kp, 8, 8, False) == FULL).all()


def test_diagonal_block_tile_counts_closed_form():
    # T x T tiles on an n x n diagonal block: nT(nT-1)/2 EMPTY, as many FULL, nT PARTIAL
    n, T = 16384, 128
    qp = np.arange(n)
    cls = oracle.tile_classes(qp, qp, T, T, True)
    nT = n // T
    assert int((cls == EMPTY).sum()) == nT * (nT - 1) // 2 == 8128
    assert int((cls == FULL).sum()) == nT * (nT - 1) // 2
    assert int((cls == PARTIAL).sum()) == nT == 128
