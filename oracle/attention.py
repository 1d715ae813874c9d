"""fp64 reference computations for one rank's lap of ring attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Everything here is written from the definitions on the pages, in float64 with
NumPy, with no blocking, fusion or reordering beyond what those definitions
state:

* ``dense_attention`` is exact attention, softmax(scale * Q K^T) V, over every
  key the mask allows -- the result the ring reaches exactly ([P1] "Why partial
  results are allowed to merge"; [P3] section 局部 Softmax 为什么不能直接相加).
* ``online_state_init`` / ``online_block_update`` / ``online_finalize`` /
  ``blockwise_attention`` are the ring's own recipe: a per-row running maximum
  m, running exponential sum l and unnormalised output O~, rescaled by
  exp(old max - new max) when a block arrives, the block's contribution added,
  and O = O~ / l at the end ([P1] "Why partial results are allowed to merge";
  [P2] body, the rescale by exp(old_max - new_max); [P3] 局部 Softmax
  为什么不能直接相加, whose update equations were lost in extraction -- the
  standard form is used, see the readings in the design notes).
* ``ring_visit_order`` is the lap: rank r sends to r+1 and receives from r-1,
  so at step s it holds the block that started on rank (r - s) mod P ([P1] "One
  lap around the ring"; the four-device table in [P3] 环是怎样工作的).
* ``token_owner`` / ``tokens_of_rank`` give each rank its tokens: contiguous
  slices ([P1] "Sharding the sequence, pinning the queries"; [P3] 位置编码必须使用
  全局位置, device p local index i -> global position p * N_local + i) or the
  round-robin striped layout, token t to rank t mod P (named as "striped" on
  [P2] body and [P3] Causal section; the map itself is this project's reading),
  or the paired "zigzag" layout: 2P chunks of N/(2P) tokens, rank r holding
  chunks r and 2P-1-r ([P1] "Striping the sequence to flatten the triangle").
  When P does not divide N, contiguous shards are padded to ceil(N/P) slots and
  the tail rank holds fewer real tokens ([P3] 正确性测试应覆盖哪些边界, tail-rank
  padding with a valid-length mask): ``shard_capacity``.
* The causal rule is on global positions: query q sees key k iff k <= q ([P3]
  Causal Attention 让环不再完全对称, and 位置编码必须使用全局位置).
* ``merge_states`` is the global online-softmax reduction of shard states for
  decode ([P3] 训练与推理的适用方式不同: the query is sent to the KV shards, each
  computes a local attention state, and the states are reduced), the same
  rescale-and-add as a block update.
* ``backward_row_terms`` / ``backward_block`` are one ring step of the backward
  pass ([P3] Backward 需要让梯度也沿环传播: dQ stays with the query owner, dK and dV
  accumulate on the travelling block, probabilities are recomputed from the saved
  per-row logsumexp); the gradient formulas are the standard ones, not printed on
  the pages.
* ``tile_classes`` enumerates pairs per (query tile, key tile) and names a tile
  EMPTY (no allowed pair), FULL (every pair allowed) or PARTIAL ([P3] Causal
  section's three-way block rule: strictly future -> skip, crossing the
  diagonal -> masked, otherwise unmasked; [P1] "Striping the sequence to
  flatten the triangle": wholly masked blocks are skipped).

Tensor layout: Q is [B, Hq, n, d]; K and V are [B, Hkv, n_k, d]; query head h
reads KV head h // (Hq // Hkv) (contiguous GQA groups; [P1] "When the ring
stops paying for itself" names grouped-query attention, the head map is this
project's reading).
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

EMPTY, FULL, PARTIAL = 0, 1, 2


# ----------------------------------------------------------------------------
# The lap and the token layouts
# ----------------------------------------------------------------------------

def ring_visit_order(P: int, r: int) -> list[int]:
    """Blocks rank r holds at steps 0..P-1 of one lap.

    Step 0 is the rank's own block; each step it passes what it holds to r+1
    and receives from r-1 ([P1] "One lap around the ring").  Simulated here
    literally by passing blocks around a ring of P ranks, not by a formula.
    """
    if not 0 <= r < P:
        raise ValueError("rank out of range")
    holding = list(range(P))           # holding[x] = block on rank x at step 0
    seen = []
    for _ in range(P):
        seen.append(holding[r])
        # every rank sends to its successor: rank x now holds what x-1 had
        holding = [holding[(x - 1) % P] for x in range(P)]
    return seen


def shard_capacity(N: int, P: int) -> int:
    """Token slots per rank when N is split over P ranks: ceil(N / P).  When P does not
    divide N, the shards are padded to this common size and the tail rank holds fewer real
    tokens ([P3] 正确性测试应覆盖哪些边界: divisible and non-divisible N, tail-rank padding
    with a valid-length mask)."""
    return -(-N // P)


def token_owner(N: int, P: int, layout: str) -> np.ndarray:
    """Rank that owns each global token 0..N-1 under a layout.

    Contiguous: rank r owns [r * c, min(N, (r + 1) * c)) with c = shard_capacity(N, P), so
    for N not a multiple of P the last ranks own fewer tokens (possibly none).  Striped:
    token t goes to rank t mod P for any N.  Zigzag needs N to be a multiple of 2P."""
    t = np.arange(N, dtype=np.int64)
    if layout == "contiguous":
        return t // shard_capacity(N, P)
    if layout == "striped":
        return t % P
    if layout == "zigzag":
        if N % (2 * P):
            raise ValueError("zigzag needs N to be a multiple of 2P")
        chunk = t // (N // (2 * P))
        return np.where(chunk < P, chunk, 2 * P - 1 - chunk)
    raise ValueError(f"unknown layout {layout!r}")


def tokens_of_rank(N: int, P: int, layout: str, r: int) -> np.ndarray:
    """Global positions of rank r's tokens, in local order (ascending)."""
    return np.nonzero(token_owner(N, P, layout) == r)[0].astype(np.int64)


def allowed_mask(q_pos: np.ndarray, k_pos: np.ndarray, causal: bool) -> np.ndarray:
    """[n_q, n_k] boolean: may query at q_pos[i] see key at k_pos[t]?"""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if not causal:
        return np.ones((q_pos.size, k_pos.size), dtype=bool)
    return k_pos[None, :] <= q_pos[:, None]


# ----------------------------------------------------------------------------
# Exact attention (the plain definition)
# ----------------------------------------------------------------------------

def _group(Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("q_heads must be a multiple of kv_heads")
    return Hq // Hkv


def dense_attention(q, k, v, q_pos, k_pos, causal: bool, scale: float | None = None,
                    row_chunk: int = 256, heads: Iterable[int] | None = None,
                    rows: np.ndarray | None = None):
    """Exact softmax(scale * Q K^T) V over the allowed keys, in float64.

    q: [B, Hq, n, d]; k, v: [B, Hkv, N, d] (all keys the rows may see);
    q_pos: [n] global positions of the query rows; k_pos: [N] of the keys.
    Rows with no allowed key get O = 0 and lse = -inf.

    ``heads`` restricts the computation to some query heads and ``rows`` to
    some local query rows (other outputs are left NaN), so that single rows of
    very long sequences can be checked one by one.

    Returns (O [B, Hq, n, d] float64, lse [B, Hq, n] float64) where lse is the
    natural log of the softmax denominator, sum_t exp(scale * <q, k_t>).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    G = _group(Hq, Hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    out = np.full((B, Hq, n, v.shape[-1]), np.nan)
    lse = np.full((B, Hq, n), np.nan)
    row_ids = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    head_ids = range(Hq) if heads is None else heads
    for b in range(B):
        for h in head_ids:
            kh = k[b, h // G]
            vh = v[b, h // G]
            for c0 in range(0, row_ids.size, row_chunk):
                ri = row_ids[c0:c0 + row_chunk]
                s = scale * (q[b, h, ri] @ kh.T)                  # [rows, N]
                ok = allowed_mask(q_pos[ri], k_pos, causal)
                s = np.where(ok, s, -np.inf)
                mx = s.max(axis=1, keepdims=True, initial=-np.inf)
                has = np.isfinite(mx[:, 0])
                mx_safe = np.where(np.isfinite(mx), mx, 0.0)
                p = np.where(ok, np.exp(s - mx_safe), 0.0)
                den = p.sum(axis=1, keepdims=True)
                o = np.where(has[:, None], (p @ vh) / np.where(den > 0, den, 1.0), 0.0)
                out[b, h, ri] = o
                lse[b, h, ri] = np.where(has, mx[:, 0] + np.log(np.where(den[:, 0] > 0, den[:, 0], 1.0)),
                                         -np.inf)
    return out, lse


# ----------------------------------------------------------------------------
# The ring's recipe: online-softmax state, block update, finalize
# ----------------------------------------------------------------------------

def online_state_init(B: int, Hq: int, n: int, d: int) -> dict:
    """Empty per-row state for the local queries: m = -inf, l = 0, O~ = 0.

    [P3] 环是怎样工作的: the lap starts from an empty online-softmax state built
    for the local queries.  m is kept in natural-log units of the scaled
    logits scale * <q, k>.
    """
    return {
        "m": np.full((B, Hq, n), -np.inf),
        "l": np.zeros((B, Hq, n)),
        "o": np.zeros((B, Hq, n, d)),
    }


def online_block_update(state: dict, q, k_j, v_j, q_pos, k_pos_j, causal: bool,
                        scale: float | None = None) -> dict:
    """Merge one arriving KV block into the running state (float64).

    In the pages' order: score the block, take its per-row max, form the new
    running max, rescale both accumulators by exp(old max - new max), add the
    block's contribution ([P1] "Why partial results are allowed to merge";
    [P2] body).  Rows that see no key of this block keep their state.
    Returns a new state dict; the input is not modified.
    """
    q = np.asarray(q, dtype=np.float64)
    k_j = np.asarray(k_j, dtype=np.float64)
    v_j = np.asarray(v_j, dtype=np.float64)
    B, Hq, n, d = q.shape
    G = _group(Hq, k_j.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ok = allowed_mask(q_pos, k_pos_j, causal)                       # [n, Nk]
    m_old, l_old, o_old = state["m"], state["l"], state["o"]
    m_new = np.empty_like(m_old)
    l_new = np.empty_like(l_old)
    o_new = np.empty_like(o_old)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k_j[b, h // G].T)                 # block scores S^(j)
            s = np.where(ok, s, -np.inf)
            block_max = s.max(axis=1, initial=-np.inf)               # local max (-inf: no key)
            mn = np.maximum(m_old[b, h], block_max)                  # new running max
            # rows with no key seen so far: keep everything at the empty state
            live = np.isfinite(mn)
            mn_safe = np.where(live, mn, 0.0)
            alpha = np.where(live, np.exp(m_old[b, h] - mn_safe), 1.0)   # exp(old max - new max)
            p = np.where(ok, np.exp(s - mn_safe[:, None]), 0.0)
            l_new[b, h] = alpha * l_old[b, h] + p.sum(axis=1)
            o_new[b, h] = alpha[:, None] * o_old[b, h] + p @ v_j[b, h // G]
            m_new[b, h] = mn
    return {"m": m_new, "l": l_new, "o": o_new}


def online_finalize(state: dict):
    """O = O~ / l and lse = m + ln l; rows that saw no key give O = 0, lse = -inf."""
    m, l, o = state["m"], state["l"], state["o"]
    seen = l > 0
    out = np.where(seen[..., None], o / np.where(seen, l, 1.0)[..., None], 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return out, lse


def merge_states(parts: Sequence[dict]) -> dict:
    """Global online-softmax reduction of states over disjoint key sets (float64).

    For decode the query goes to the KV shards, each shard computes a local
    attention state, and one reduction combines them ([P3] 训练与推理的适用方式不同).
    The combination is the same rescale-and-add as a block update ([P1] "Why
    partial results are allowed to merge"): with m = max_s m_s,
    l = sum_s exp(m_s - m) l_s and O~ = sum_s exp(m_s - m) O~_s.  Rows that no
    part has seen stay at the empty state.
    """
    m = parts[0]["m"]
    for st in parts[1:]:
        m = np.maximum(m, st["m"])
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    l = np.zeros_like(parts[0]["l"])
    o = np.zeros_like(parts[0]["o"])
    for st in parts:
        w = np.where(np.isfinite(st["m"]), np.exp(st["m"] - m_safe), 0.0)
        l = l + w * st["l"]
        o = o + w[..., None] * st["o"]
    return {"m": m, "l": l, "o": o}


def blockwise_attention(q, blocks: Sequence[tuple], q_pos, causal: bool,
                        order: Sequence[int] | None = None, scale: float | None = None):
    """One lap: fold every (K_j, V_j, k_pos_j) block into the state, then finalize.

    ``order`` is the visit order (defaults to the blocks' order); the result
    does not depend on it in exact arithmetic ([P3] 正确性测试应覆盖哪些边界 lists
    ring-order float differences as something to test).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, n, d = q.shape
    st = online_state_init(B, Hq, n, np.asarray(blocks[0][1]).shape[-1])
    for j in (range(len(blocks)) if order is None else order):
        k_j, v_j, kp = blocks[j]
        st = online_block_update(st, q, k_j, v_j, q_pos, kp, causal, scale)
    return online_finalize(st)


# ----------------------------------------------------------------------------
# Backward: gradients of one rank's lap, block by block
# ----------------------------------------------------------------------------

def backward_row_terms(d_out, out):
    """D_i = sum_c dO[i, c] * O[i, c]: the per-row term of the softmax gradient."""
    return np.einsum("bhnd,bhnd->bhn", np.asarray(d_out, np.float64), np.asarray(out, np.float64))


def backward_block(q, k_j, v_j, d_out, lse, D, q_pos, k_pos_j, causal: bool,
                   scale: float | None = None):
    """One ring step of the backward pass (float64): this query shard's contribution to
    dQ and to the travelling block's dK_j, dV_j.

    [P3] Backward 需要让梯度也沿环传播: the query owner accumulates dQ over every KV
    block; dK, dV of a travelling block accumulate over the query owners it passes; the
    probabilities are recomputed per block from the saved per-row logsumexp instead of
    storing the attention matrix.  The gradient of softmax attention (not printed on the
    pages; the standard form) with P = exp(scale * q.k - lse) on allowed pairs:
        dV_j = P^T dO,   dP = dO V_j^T,   dS = P * (dP - D),
        dQ   = scale * dS K_j,   dK_j = scale * dS^T Q.
    Query head h reads (and writes gradients to) KV head h // (Hq / Hkv).
    """
    q = np.asarray(q, dtype=np.float64)
    k_j = np.asarray(k_j, dtype=np.float64)
    v_j = np.asarray(v_j, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    B, Hq, n, d = q.shape
    Hkv = k_j.shape[1]
    G = _group(Hq, Hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ok = allowed_mask(q_pos, k_pos_j, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_j)
    dv = np.zeros((B, Hkv, k_j.shape[2], v_j.shape[-1]))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = scale * (q[b, h] @ k_j[b, g].T)
            fin = np.isfinite(lse[b, h])[:, None]
            p = np.where(ok & fin, np.exp(s - np.where(fin, lse[b, h][:, None], 0.0)), 0.0)
            dv[b, g] += p.T @ d_out[b, h]
            dp = d_out[b, h] @ v_j[b, g].T
            ds = p * (dp - D[b, h][:, None])
            dq[b, h] += scale * (ds @ k_j[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Pair enumeration: live pairs and per-tile classes
# ----------------------------------------------------------------------------

def brute_force_pair_count(q_pos, k_pos, causal: bool) -> int:
    """Count allowed (q, k) pairs with a double loop (tiny inputs only)."""
    n = 0
    for qp in (int(x) for x in q_pos):
        for kp in (int(x) for x in k_pos):
            if (not causal) or kp <= qp:
                n += 1
    return n


def live_pair_count(q_pos, k_pos, causal: bool) -> int:
    """Count allowed pairs at any size: per query, the keys at or before it.

    Uses a sort and a binary search per row, so full-size blocks (16384 x
    16384) are counted without forming the pair matrix.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if not causal:
        return int(q_pos.size) * int(k_pos.size)
    ks = np.sort(k_pos)
    return int(np.searchsorted(ks, q_pos, side="right").sum())


def tile_classes(q_pos, k_pos, tile_q: int, tile_k: int, causal: bool) -> np.ndarray:
    """EMPTY / FULL / PARTIAL per (query tile, key tile), by counting pairs.

    Tiles cover consecutive local rows [a*tile_q, (a+1)*tile_q) and keys
    [c*tile_k, (c+1)*tile_k); the last tile of each may be short.  A tile is
    EMPTY when it holds no allowed pair, FULL when every pair is allowed and
    PARTIAL otherwise.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    nqt = -(-q_pos.size // tile_q)
    nkt = -(-k_pos.size // tile_k)
    out = np.empty((nqt, nkt), dtype=np.uint8)
    for c in range(nkt):
        kt = np.sort(k_pos[c * tile_k:(c + 1) * tile_k])
        for a in range(nqt):
            qt = q_pos[a * tile_q:(a + 1) * tile_q]
            total = qt.size * kt.size
            if causal:
                live = int(np.searchsorted(kt, qt, side="right").sum())
            else:
                live = total
            out[a, c] = EMPTY if live == 0 else (FULL if live == total else PARTIAL)
    return out
