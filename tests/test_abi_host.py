"""Host-only checks of librocring.so: it loads, exports every declared symbol,
its planner takes exactly the oracle's mask/skip decisions, and misuse returns
the documented error codes.  No device work is enqueued by any call here."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import exact_long_context_amd as ra
from exact_long_context_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_lap_entry_points():
    names = declared_functions()
    for must in ("ra_state_init", "ra_block_step", "ra_finalize", "ra_ring_lap_emulated"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(_abi.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each
    assert set(declared_functions()) == set(_abi.SIGNATURES)


def test_version_and_status_strings():
    lib = ra.lib()
    assert lib.ra_version() == 1
    assert lib.ra_status_string(0) == b"ok"
    assert lib.ra_status_string(12345) == b"unknown status"


def _desc(q_len=256, q_heads=4, kv_heads=2, d=128, dtype=ra.RA_DTYPE_BF16, P=4, B=1):
    qs = (q_heads * q_len * d, q_len * d, d)
    ks = (kv_heads * 512 * d, 512 * d, d)
    return ra.make_desc(B, q_heads, kv_heads, q_len, d, dtype, qs, ks, ring_size=P)


# ---------------------------------------------------------------------------
# planner vs the oracle's enumeration (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [ra.RA_DTYPE_BF16, ra.RA_DTYPE_F32])
@pytest.mark.parametrize("layout,mask", [("contiguous", ra.RA_MASK_CAUSAL_CONTIGUOUS),
                                         ("striped", ra.RA_MASK_CAUSAL_STRIPED),
                                         ("contiguous", ra.RA_MASK_NONE)])
def test_tile_classes_match_oracle(dtype, layout, mask):
    for P, N in ((1, 640), (2, 640), (4, 1024), (16, 4096)):
        n = N // P
        for r in sorted({0, P // 2, P - 1}):
            qp = oracle.tokens_of_rank(N, P, layout, r)
            d = _desc(q_len=n, dtype=dtype, P=P)
            for j in range(P):
                kp = oracle.tokens_of_rank(N, P, layout, j)
                q_off, k_off = ra.block_offsets(mask, r, j, n, n)
                got = ra.tile_classes(d, n, mask, q_off, k_off)
                st = ra.plan_block(d, n, mask, q_off, k_off)
                want = oracle.tile_classes(qp, kp, st["tile_q"], st["tile_k"], mask != ra.RA_MASK_NONE)
                assert np.array_equal(got, want), (P, r, j)
                heads = d.batch * d.q_heads
                assert st["live_pairs"] == heads * oracle.live_pair_count(qp, kp, mask != ra.RA_MASK_NONE)
                assert st["tiles_full"] == heads * int((want == oracle.FULL).sum())
                assert st["tiles_partial"] == heads * int((want == oracle.PARTIAL).sum())
                assert st["tiles_empty"] == heads * int((want == oracle.EMPTY).sum())
                assert st["blocks_run"] + st["blocks_skipped"] == 1
                assert st["blocks_skipped"] == int(st["live_pairs"] == 0)


def _zigzag_tile_classes(N, P, r, j, tq, tk):
    """The oracle's classes per (query chunk, key chunk), assembled on the chunk tiling."""
    qp = oracle.tokens_of_rank(N, P, "zigzag", r)
    kp = oracle.tokens_of_rank(N, P, "zigzag", j)
    c = qp.size // 2
    rows = []
    for qa in range(2):
        rows.append(np.concatenate([oracle.tile_classes(qp[qa * c:(qa + 1) * c], kp[ka * c:(ka + 1) * c],
                                                        tq, tk, True) for ka in range(2)], axis=1))
    return np.concatenate(rows, axis=0), qp, kp


@pytest.mark.parametrize("dtype", [ra.RA_DTYPE_BF16, ra.RA_DTYPE_F32])
def test_zigzag_tile_classes_and_counts_match_oracle(dtype):
    for P, N in ((1, 512), (2, 1200), (3, 1536), (4, 4096), (8, 4 * 8 * 300)):
        n = N // P
        d = _desc(q_len=n, dtype=dtype, P=P)
        for r in sorted({0, P // 2, P - 1}):
            for j in range(P):
                st = ra.plan_block(d, n, ra.RA_MASK_CAUSAL_ZIGZAG, r, j)
                got = ra.tile_classes(d, n, ra.RA_MASK_CAUSAL_ZIGZAG, r, j)
                want, qp, kp = _zigzag_tile_classes(N, P, r, j, st["tile_q"], st["tile_k"])
                assert np.array_equal(got, want), (P, r, j)
                heads = d.batch * d.q_heads
                assert st["live_pairs"] == heads * oracle.live_pair_count(qp, kp, True)
                assert st["tiles_full"] == heads * int((want == oracle.FULL).sum())
                assert st["tiles_partial"] == heads * int((want == oracle.PARTIAL).sum())
                assert st["tiles_empty"] == heads * int((want == oracle.EMPTY).sum())
                assert st["blocks_skipped"] == int(st["live_pairs"] == 0)


def test_zigzag_full_size_ranks_do_equal_work():
    # the 131072-token, 8-rank ring: every rank's lap holds 2P c^2 + c pairs per head
    N, P, Hq = 131072, 8, 32
    n, c = N // P, N // (2 * P)
    d = _desc(q_len=n, q_heads=Hq, kv_heads=Hq, P=P)
    for r in range(P):
        total = sum(ra.plan_block(d, n, ra.RA_MASK_CAUSAL_ZIGZAG, r, j)["live_pairs"] for j in range(P))
        assert total == Hq * (2 * P * c * c + c)


def test_zigzag_argument_validation():
    lib = ra.lib()
    s = ra.ra_stats()
    d = _desc(q_len=64, P=4)
    Z = ra.RA_MASK_CAUSAL_ZIGZAG
    assert lib.ra_plan_block(C.byref(d), 64, Z, 0, 3, C.byref(s)) == ra.RA_OK
    assert lib.ra_plan_block(C.byref(d), 64, Z, 4, 0, C.byref(s)) == ra.RA_E_INVALID    # rank >= P
    assert lib.ra_plan_block(C.byref(d), 64, Z, 0, -1, C.byref(s)) == ra.RA_E_INVALID
    assert lib.ra_plan_block(C.byref(d), 32, Z, 0, 0, C.byref(s)) == ra.RA_E_INVALID    # kv_len != q_len
    d_odd = _desc(q_len=63, P=4)
    assert lib.ra_plan_block(C.byref(d_odd), 63, Z, 0, 0, C.byref(s)) == ra.RA_E_INVALID
    assert lib.ra_plan_block(C.byref(d), 64, 4, 0, 0, C.byref(s)) == ra.RA_E_INVALID     # unknown mask


@pytest.mark.parametrize("q_len,kv_len,q_off,k_off", [
    (200, 150, 0, 0), (200, 150, 149, 0), (200, 150, 0, 57), (1, 1, 0, 0), (1, 1, 0, 1),
    (129, 65, 3, 1), (64, 64, -10, 0), (300, 10, 1000, 0), (0, 64, 0, 0), (64, 0, 0, 0)])
def test_ragged_tiles_match_oracle(q_len, kv_len, q_off, k_off):
    for dtype in (ra.RA_DTYPE_BF16, ra.RA_DTYPE_F32):
        d = _desc(q_len=q_len, dtype=dtype)
        qp = q_off + np.arange(q_len)
        kp = k_off + np.arange(kv_len)
        st = ra.plan_block(d, kv_len, ra.RA_MASK_CAUSAL_CONTIGUOUS, q_off, k_off)
        got = ra.tile_classes(d, kv_len, ra.RA_MASK_CAUSAL_CONTIGUOUS, q_off, k_off)
        if q_len and kv_len:
            want = oracle.tile_classes(qp, kp, st["tile_q"], st["tile_k"], True)
            assert np.array_equal(got, want)
        assert st["live_pairs"] == d.q_heads * oracle.live_pair_count(qp, kp, True)


def test_striped_large_ring_offsets():
    # P = 64 striped: diag is 0 for blocks at or before the rank, -1 after it
    N, P, r = 64 * 256, 64, 5
    n = N // P
    d = _desc(q_len=n, P=P)
    qp = oracle.tokens_of_rank(N, P, "striped", r)
    for j in (0, 4, 5, 6, 63):
        kp = oracle.tokens_of_rank(N, P, "striped", j)
        st = ra.plan_block(d, n, ra.RA_MASK_CAUSAL_STRIPED, r, j)
        assert st["live_pairs"] == d.q_heads * oracle.live_pair_count(qp, kp, True)
        got = ra.tile_classes(d, n, ra.RA_MASK_CAUSAL_STRIPED, r, j)
        assert np.array_equal(got, oracle.tile_classes(qp, kp, st["tile_q"], st["tile_k"], True))


@pytest.mark.parametrize("name,N,P,r,mask,Hq,per_head", [
    ("causal contiguous rank 0", 131072, 8, 0, ra.RA_MASK_CAUSAL_CONTIGUOUS, 32, 134_225_920),
    ("causal contiguous rank 7", 131072, 8, 7, ra.RA_MASK_CAUSAL_CONTIGUOUS, 32, 2_013_274_112),
    ("causal striped P=16 rank 5", 262144, 16, 5, ra.RA_MASK_CAUSAL_STRIPED, 32, 2_147_450_880),
    ("causal striped P=64 rank 5", 1048576, 64, 5, ra.RA_MASK_CAUSAL_STRIPED, 64, 8_589_508_608),
    ("non-causal P=8", 131072, 8, 0, ra.RA_MASK_NONE, 32, 16384 * 131072),
])
def test_full_size_lap_pair_counts(name, N, P, r, mask, Hq, per_head):
    n = N // P
    d = _desc(q_len=n, q_heads=Hq, kv_heads=8 if Hq == 64 else Hq, P=P)
    total = 0
    run = skipped = 0
    for s in range(P):
        j = oracle.ring_visit_order(P, r)[s]
        q_off, k_off = ra.block_offsets(mask, r, j, n, n)
        st = ra.plan_block(d, n, mask, q_off, k_off)
        total += st["live_pairs"]
        run += st["blocks_run"]
        skipped += st["blocks_skipped"]
    assert total == per_head * Hq
    if mask == ra.RA_MASK_CAUSAL_CONTIGUOUS:
        assert (run, skipped) == ((1, 7) if r == 0 else (8, 0))


def test_full_size_diagonal_tiles_match_oracle():
    # the 16384 x 16384 diagonal block, bf16 tiles, contiguous and striped (both sides of r)
    n = 16384
    d = _desc(q_len=n, P=16)
    cases = [(ra.RA_MASK_CAUSAL_CONTIGUOUS, 7 * n, 7 * n, np.arange(n) + 7 * n, np.arange(n) + 7 * n),
             (ra.RA_MASK_CAUSAL_STRIPED, 5, 5, np.arange(n) * 16 + 5, np.arange(n) * 16 + 5),
             (ra.RA_MASK_CAUSAL_STRIPED, 5, 9, np.arange(n) * 16 + 5, np.arange(n) * 16 + 9)]
    for mask, q_off, k_off, qp, kp in cases:
        got = ra.tile_classes(d, n, mask, q_off, k_off)
        st = ra.plan_block(d, n, mask, q_off, k_off)
        assert np.array_equal(got, oracle.tile_classes(qp, kp, st["tile_q"], st["tile_k"], True))


# ---------------------------------------------------------------------------
# error codes (host-side validation; nothing reaches the device)
# ---------------------------------------------------------------------------

def _init(desc, q=0x10000, ws=0x20000):
    h = C.c_void_p()
    rc = ra.lib().ra_state_init(C.byref(desc) if desc is not None else None, q, ws, C.byref(h))
    return rc, h


def test_invalid_descriptors():
    lib = ra.lib()
    assert lib.ra_workspace_bytes(None) == 0
    assert _init(None)[0] == ra.RA_E_INVALID
    assert _init(_desc(q_heads=6, kv_heads=4))[0] == ra.RA_E_INVALID
    assert _init(_desc(d=96))[0] == ra.RA_E_UNSUPPORTED
    bad = _desc()
    bad.dtype = 7
    assert _init(bad)[0] == ra.RA_E_UNSUPPORTED
    bad = _desc()
    bad.softmax_scale = -1.0
    assert _init(bad)[0] == ra.RA_E_INVALID
    bad = _desc()
    bad.softmax_scale = float("nan")
    assert _init(bad)[0] == ra.RA_E_INVALID
    bad = _desc()
    bad.q_strides[2] = 100           # not a multiple of 8 bf16 elements
    assert _init(bad)[0] == ra.RA_E_INVALID
    bad = _desc()
    bad.ring_size = 0
    assert _init(bad)[0] == ra.RA_E_INVALID
    bad = _desc()
    bad.batch = 0
    assert _init(bad)[0] == ra.RA_E_INVALID
    assert _init(_desc(), q=0)[0] == ra.RA_E_INVALID
    assert _init(_desc(), ws=0)[0] == ra.RA_E_INVALID
    assert _init(_desc(), q=0x10008)[0] == ra.RA_E_INVALID       # misaligned Q
    assert _init(_desc(), ws=0x20010)[0] == ra.RA_E_INVALID      # workspace not 256-aligned
    assert b"multiple" in lib.ra_status_string(ra.RA_E_INVALID) or True
    # more query tiles than one launch can hold (2^30 rows x 16 heads: 2^28 tiles of 64 rows)
    big = _desc(q_len=1 << 30, q_heads=16, kv_heads=16)
    assert _init(big)[0] == ra.RA_E_UNSUPPORTED
    assert lib.ra_workspace_bytes(C.byref(big)) == 0
    ok = _desc(q_len=1 << 20, q_heads=64, kv_heads=8)      # 2^20 tiles x 256 threads: fits
    assert lib.ra_workspace_bytes(C.byref(ok)) > 0


def test_workspace_layout():
    d = _desc(q_len=100, q_heads=3, kv_heads=1, d=64, B=2)
    o, m, l_ = ra.workspace_layout(d)
    rows = 2 * 3 * 100
    assert o == 0 and m >= rows * 64 * 4 and l_ >= m + rows * 4
    assert m % 256 == 0 and l_ % 256 == 0
    assert ra.workspace_bytes(d) >= l_ + rows * 4
    assert ra.workspace_bytes(_desc(q_len=0)) == 0


def test_state_machine_without_device_work():
    lib = ra.lib()
    assert lib.ra_block_step(None, 0, 0, 0, 0, 0, 0) == ra.RA_E_INVALID
    d = _desc(q_len=0)                      # q_len 0: finalize has nothing to launch
    rc, h = _init(d, q=0, ws=0)
    assert rc == ra.RA_OK
    assert lib.ra_block_step(h, 0x30000, 0x40000, 64, ra.RA_MASK_NONE, 0, 0) == ra.RA_OK
    assert lib.ra_block_step(h, 0x30000, 0x40000, 64, 9, 0, 0) == ra.RA_E_INVALID
    assert lib.ra_block_step(h, 0x30000, 0x40000, -1, 0, 0, 0) == ra.RA_E_INVALID
    assert lib.ra_finalize(h, None, None) == ra.RA_OK
    assert lib.ra_finalize(h, None, None) == ra.RA_E_STATE
    assert lib.ra_block_step(h, 0x30000, 0x40000, 64, ra.RA_MASK_NONE, 0, 0) == ra.RA_E_STATE
    assert lib.ra_state_destroy(h) == ra.RA_OK


def test_fully_masked_blocks_launch_nothing():
    # rank 0 of a contiguous causal ring: every block but its own is strictly in the future
    lib = ra.lib()
    d = _desc(q_len=256)
    rc, h = _init(d)
    assert rc == ra.RA_OK
    for j in (1, 2, 3):
        assert lib.ra_block_step(h, 0x30000, 0x40000, 256, ra.RA_MASK_CAUSAL_CONTIGUOUS,
                                 0, j * 256) == ra.RA_OK
    assert lib.ra_block_step(h, 0, 0, 0, ra.RA_MASK_NONE, 0, 0) == ra.RA_OK   # empty block
    s = ra.ra_stats()
    assert lib.ra_get_stats(h, C.byref(s)) == ra.RA_OK
    assert s.blocks_skipped == 4 and s.blocks_run == 0 and s.live_pairs == 0
    assert lib.ra_block_step(h, 0, 0x40000, 256, ra.RA_MASK_NONE, 0, 0) == ra.RA_E_INVALID  # NULL K
    assert lib.ra_block_step(h, 0x30004, 0x40000, 256, ra.RA_MASK_NONE, 0, 0) == ra.RA_E_INVALID
    lib.ra_state_destroy(h)


def test_merge_argument_validation():
    # every check happens on the host before anything is enqueued
    lib = ra.lib()
    d = _desc(q_len=64)
    ok = 0x100000
    parts = (C.c_void_p * 2)(ok, ok + 0x100000)
    E = ra.RA_E_INVALID
    assert lib.ra_merge_states(C.byref(d), 0, parts, ok, None, None) == E             # no parts
    big = (C.c_void_p * 65)(*([ok] * 65))
    assert lib.ra_merge_states(C.byref(d), 65, big, ok, None, None) == E              # too many
    assert lib.ra_merge_states(C.byref(d), 2, None, ok, None, None) == E              # NULL array
    assert lib.ra_merge_states(C.byref(d), 2, parts, None, None, None) == E           # no output
    assert lib.ra_merge_states(C.byref(d), 2, parts, ok, None, ok) == E               # lse without O
    bad = (C.c_void_p * 2)(ok, ok + 64)
    assert lib.ra_merge_states(C.byref(d), 2, bad, ok, None, None) == E               # misaligned part
    nul = (C.c_void_p * 2)(ok, None)
    assert lib.ra_merge_states(C.byref(d), 2, nul, ok, None, None) == E               # NULL part
    assert lib.ra_merge_states(C.byref(d), 2, parts, ok + 16, None, None) == E        # misaligned merged
    assert lib.ra_merge_states(C.byref(d), 2, parts, None, ok + 4, None) == E         # misaligned O
    assert ra.RA_MERGE_MAX_PARTS == 64


def test_lap_argument_validation():
    lib = ra.lib()
    d = _desc(q_len=64, P=4)
    lap = ra.ra_lap()
    lap.rank = 4                           # out of range
    assert lib.ra_ring_lap_emulated(C.byref(d), 0x10000, 0x20000, C.byref(lap), 0x50000, None,
                                    None) == ra.RA_E_INVALID
    assert lib.ra_ring_lap_emulated(None, 0, 0, None, 0, None, None) == ra.RA_E_INVALID
    # per-block valid key counts must lie in [0, kv_len]; checked before any work is enqueued
    kp = (C.c_void_p * 4)(0x100000, 0x200000, 0x300000, 0x400000)
    lap = ra.ra_lap()
    lap.k_blocks = C.cast(kp, C.POINTER(C.c_void_p))
    lap.v_blocks = C.cast(kp, C.POINTER(C.c_void_p))
    for i in range(2):
        lap.recv_k[i] = 0x500000 + i * 0x100000
        lap.recv_v[i] = 0x700000 + i * 0x100000
    lap.block_bytes = 64 * 128 * 2
    lap.rank = 1
    lap.kv_len = 64
    for bad in ([64, 64, 65, 3], [64, -1, 64, 64]):
        valid = (C.c_int32 * 4)(*bad)
        lap.kv_valid = C.cast(valid, C.POINTER(C.c_int32))
        assert lib.ra_ring_lap_emulated(C.byref(d), 0x10000, 0x20000, C.byref(lap), 0x50000, None,
                                        None) == ra.RA_E_INVALID


def test_one_hip_runtime_per_process():
    """The library binds to the HIP runtime torch ships; a second copy of libamdhip64 in
    the process would receive torch's stream handles and crash."""
    import torch  # noqa: F401
    assert len(_abi._hip_runtimes_mapped()) == 1


def test_decode_workspace_bytes():
    # chunk states of rows * (d + 2) floats, each section 256-byte aligned.  One row group per
    # KV head: min(ceil(T / (B * Hkv)), ceil(kv_len / 256)) parts, T = 2048 waves for at most
    # 8 packed rows, else 1024.  Two row groups: below 131072 keys
    # min(ceil(1024 / (B * Hkv * 2)), ceil(kv_len / 256)); from there the larger of that and
    # 2 * min(ceil(512 / (B * Hkv)), ceil(kv_len / (2 * 512))).  More: R = 4 row groups per
    # workgroup, min(ceil(512 / (B * Hkv * ceil(groups / 4))), ceil(kv_len / 512)) parts.
    lib = ra.lib()
    d = _desc(q_len=1, q_heads=64, kv_heads=8)            # 8 packed rows per KV head: one group
    rows = 64

    def expect(parts):
        a = lambda x: (x + 255) // 256 * 256               # noqa: E731
        return a(parts * rows * 128 * 4) + 2 * a(parts * rows * 4)

    assert lib.ra_decode_workspace_bytes(C.byref(d), 1 << 20) == expect(256)
    assert lib.ra_decode_workspace_bytes(C.byref(d), 300) == expect(2)
    assert lib.ra_decode_workspace_bytes(C.byref(d), 1) == expect(1)
    assert lib.ra_decode_workspace_bytes(C.byref(d), 0) == 0
    assert lib.ra_decode_workspace_bytes(C.byref(d), -1) == 0
    a = lambda x: (x + 255) // 256 * 256                   # noqa: E731

    def states(parts, rows):
        return a(parts * rows * 128 * 4) + 2 * a(parts * rows * 4)

    d2 = _desc(q_len=5, q_heads=16, kv_heads=2)           # 40 packed rows: two groups per KV head
    assert lib.ra_decode_workspace_bytes(C.byref(d2), 1 << 20) == states(512, 80)
    assert lib.ra_decode_workspace_bytes(C.byref(d2), 600) == states(3, 80)
    assert lib.ra_decode_workspace_bytes(C.byref(d2), 300) == states(2, 80)
    d4 = _desc(q_len=4, q_heads=64, kv_heads=4)           # 64 packed rows, 4 KV heads
    assert lib.ra_decode_workspace_bytes(C.byref(d4), 1 << 17) == states(max(128, 2 * 128), 64 * 4)
    assert lib.ra_decode_workspace_bytes(C.byref(d4), 1 << 20) == states(max(128, 2 * 128), 64 * 4)
    assert lib.ra_decode_workspace_bytes(C.byref(d4), 5000) == states(20, 64 * 4)
    d3 = _desc(q_len=24, q_heads=64, kv_heads=8)          # 192 packed rows: six groups, two workgroups
    assert lib.ra_decode_workspace_bytes(C.byref(d3), 1 << 20) == states(-(-512 // (8 * 2)), 64 * 24)
    assert lib.ra_decode_workspace_bytes(C.byref(d3), 1000) == states(2, 64 * 24)
    d5 = _desc(q_len=2, q_heads=64, kv_heads=8)           # 16 packed rows: one group, 1024 waves
    assert lib.ra_decode_workspace_bytes(C.byref(d5), 1 << 20) == states(128, 128)
    assert lib.ra_decode_workspace_bytes(C.byref(d5), 3000) == states(12, 128)
    bad = _desc(q_len=1, d=96)
    assert lib.ra_decode_workspace_bytes(C.byref(bad), 1000) == 0


def test_decode_argument_validation():
    # every check below is taken on the host before anything is enqueued
    lib = ra.lib()
    d = _desc(q_len=4, q_heads=8, kv_heads=2)
    h = C.c_void_p()
    assert lib.ra_state_init(C.byref(d), 0x10000, 0x20000, C.byref(h)) == ra.RA_OK
    ws, K, V = 0x100000, 0x300000, 0x500000
    need = lib.ra_decode_workspace_bytes(C.byref(d), 512)
    E = ra.RA_E_INVALID
    assert lib.ra_decode_step(None, K, V, 512, 0, 0, 0, ws, need) == E                      # no state
    assert lib.ra_decode_step(h, K, V, 512, ra.RA_MASK_CAUSAL_ZIGZAG, 0, 0, ws, need) == ra.RA_E_UNSUPPORTED
    assert lib.ra_decode_step(h, None, V, 512, 0, 0, 0, ws, need) == E                      # NULL K
    assert lib.ra_decode_step(h, K + 4, V, 512, 0, 0, 0, ws, need) == E                     # misaligned
    assert lib.ra_decode_step(h, K, V, 512, 0, 0, 0, None, need) == E                       # no workspace
    assert lib.ra_decode_step(h, K, V, 512, 0, 0, 0, ws + 16, need) == E                    # misaligned
    assert lib.ra_decode_step(h, K, V, 512, 0, 0, 0, ws, need - 1) == E                     # too short
    assert lib.ra_decode_step(h, K, V, -1, 0, 0, 0, ws, need) == E                          # bad length
    assert lib.ra_decode_step(h, K, V, 512, 9, 0, 0, ws, need) == E                         # bad mask
    # blocks without an allowed pair launch nothing and need no workspace
    assert lib.ra_decode_step(h, K, V, 512, ra.RA_MASK_CAUSAL_CONTIGUOUS, 0, 4, None, 0) == ra.RA_OK
    assert lib.ra_decode_step(h, None, None, 0, 0, 0, 0, None, 0) == ra.RA_OK
    s = ra.ra_stats()
    assert lib.ra_get_stats(h, C.byref(s)) == ra.RA_OK
    assert s.blocks_skipped == 2 and s.blocks_run == 0 and s.live_pairs == 0
    lib.ra_state_destroy(h)
    d32 = _desc(q_len=4, q_heads=8, kv_heads=2, dtype=ra.RA_DTYPE_F32)
    assert lib.ra_state_init(C.byref(d32), 0x10000, 0x20000, C.byref(h)) == ra.RA_OK
    # fp32 is the tiled step's: its checks, then (not run here) its launch
    assert lib.ra_decode_step(h, None, V, 512, 0, 0, 0, None, 0) == E
    assert lib.ra_decode_step(h, K, V, 512, ra.RA_MASK_CAUSAL_ZIGZAG, 0, 0, ws, need) == ra.RA_E_UNSUPPORTED
    lib.ra_state_destroy(h)
