"""A CPU model of the bf16 step kernel's use of LDS, in three parts.

Layouts: the kernel's direct copies (buffer_load ... lds: lane i of one instruction writes
16 bytes at [16 i, 16 i + 16) after the instruction's LDS base, from the global offset it
computes) and its operand reads (16-byte score reads, 8-byte transposing value reads) are
replayed byte by byte on random tiles, the fragments handed to the MFMA are assembled in the
32x32x16 operand layouts, and both products are checked against K Q^T and V^T P^T computed
directly, with P in the key order the score accumulators hold.

Schedule: which buffer every wave's copies write and reads read, tile by tile, when each copy
may still be in flight (the barrier after tile t waits until all but the newest LPW copy
instructions of the wave have landed), and whether any copy can overlap a read of, or another
copy into, the same bytes.  The kernel's schedule (three buffers per tensor, copies two tiles
ahead, vmcnt(LPW) at each barrier) has no such overlap; two buffers, or a looser wait, do.

Epilogue: the accumulators leave through the tile buffers, each wave in its own, written in
the accumulator layout and read back row-major; the model replays it element by element."""

import itertools

import numpy as np
import pytest

BK = 32          # keys per tile
WAVES = 4


def lpw(D):
    """Copy instructions per wave per tile: K copies D/16/4, V copies 2*(D/32)/4."""
    return D // 64 + D // 64


# ---- layouts -------------------------------------------------------------------------------

def lds_after_copies(D, K, V):
    """K and V tiles (BK x D, as uint16) as the kernel's copies leave them in LDS (byte
    arrays), with rows past the block's end (rows of K beyond its length) returning zeros."""
    row_bytes = 2 * D
    kg = np.zeros(BK * row_bytes, np.uint8)
    vg = np.zeros(BK * row_bytes, np.uint8)
    kg[:K.size * 2] = K.view(np.uint8).reshape(-1)
    vg[:V.size * 2] = V.view(np.uint8).reshape(-1)
    klds = np.full(BK * row_bytes, 0xAB, np.uint8)
    vlds = np.full(BK * row_bytes, 0xAB, np.uint8)
    KS, VB = D // 16, D // 32
    for ks in range(KS):                      # one K copy per 16-dim slice
        for lane in range(64):
            goff = (lane & 31) * row_bytes + (lane >> 5) * 16 + ks * 32
            dst = ks * 1024 + 16 * lane
            klds[dst:dst + 16] = kg[goff:goff + 16]
    for vb, h in itertools.product(range(VB), range(2)):   # two V copies per 32-dim block
        for lane in range(64):
            goff = (lane >> 2) * row_bytes + (lane & 3) * 16 + vb * 64 + h * 16 * row_bytes
            dst = vb * 2048 + h * 1024 + 16 * lane
            vlds[dst:dst + 16] = vg[goff:goff + 16]
    return klds, vlds


def u16(buf, off, n):
    return buf[off:off + 2 * n].view(np.uint16)


def score_operand(klds, ks):
    """Operand A of the score product for k-step ks: 8 bf16 per lane, read at
    ks*1024 + hi*512 + r32*16."""
    return np.stack([u16(klds, ks * 1024 + (l >> 5) * 512 + (l & 31) * 16, 8) for l in range(64)])


def read_tr16_b64(lds, addrs):
    """ds_read_b64_tr_b16 over a wave: within each 16-lane group, lane 4a + c gets element c
    of the 4-element pieces addressed by lanes a, a + 4, a + 8, a + 12 (in that order)."""
    pieces = [u16(lds, a, 4) for a in addrs]
    out = np.zeros((64, 4), np.uint16)
    for lane in range(64):
        g, a, c = lane >> 4, (lane & 15) >> 2, lane & 3
        for t in range(4):
            out[lane, t] = pieces[16 * g + a + 4 * t][c]
    return out


def value_operand(vlds, vb, kk):
    """Operand A of the value product for value block vb and key half kk: two transposing
    reads at vb*2048 + kk*16*64 + vb0 and 8 key rows further."""
    vb0 = [(4 * (l >> 5) + ((l >> 2) & 3)) * 64 + (16 * ((l >> 4) & 1) + 4 * (l & 3)) * 2 for l in range(64)]
    base = [vb * 2048 + kk * 16 * 64 + x for x in vb0]
    lo = read_tr16_b64(vlds, base)
    hi = read_tr16_b64(vlds, [x + 8 * 64 for x in base])
    return np.concatenate([lo, hi], axis=1)


def bf16_to_f64(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def mfma_32x32x16(a, b):
    """v_mfma_f32_32x32x16_bf16 operand and result layouts: lane l holds A[l & 31][8(l >> 5)
    + i] and B[8(l >> 5) + i][l & 31]; result register j of lane l is C[8(j >> 2) +
    4(l >> 5) + (j & 3)][l & 31]."""
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for l in range(64):
        A[l & 31, 8 * (l >> 5):8 * (l >> 5) + 8] = a[l]
        B[8 * (l >> 5):8 * (l >> 5) + 8, l & 31] = b[l]
    C = A @ B
    out = np.zeros((64, 16))
    for l, j in itertools.product(range(64), range(16)):
        out[l, j] = C[8 * (j >> 2) + 4 * (l >> 5) + (j & 3), l & 31]
    return out


def random_bf16(rng, shape):
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_keys", [BK, 19])
def test_operands_reproduce_both_products(D, n_keys):
    rng = np.random.default_rng(D + n_keys)
    K = random_bf16(rng, (n_keys, D))
    V = random_bf16(rng, (n_keys, D))
    Q = random_bf16(rng, (32, D))
    klds, vlds = lds_after_copies(D, K, V)
    Kf = np.zeros((BK, D))
    Vf = np.zeros((BK, D))
    Kf[:n_keys] = bf16_to_f64(K)
    Vf[:n_keys] = bf16_to_f64(V)
    Qf = bf16_to_f64(Q)

    # scores, transposed: lane l's B fragment of k-step ks is q row l & 31, dims 16ks + 8(l >> 5) ..
    acc = np.zeros((64, 16))
    for ks in range(D // 16):
        qb = np.stack([Qf[l & 31, 16 * ks + 8 * (l >> 5):16 * ks + 8 * (l >> 5) + 8] for l in range(64)])
        acc += mfma_32x32x16(bf16_to_f64(score_operand(klds, ks)), qb)
    S_T = Kf @ Qf.T                                   # [key, row]
    for l, j in itertools.product(range(64), range(16)):
        key = 8 * (j >> 2) + 4 * (l >> 5) + (j & 3)
        assert acc[l, j] == pytest.approx(S_T[key, l & 31], rel=1e-12, abs=1e-12)

    # value product: lane l's probabilities for half kk are its score registers 8kk .. 8kk+7,
    # used directly as the B fragment, so B's k index i stands for key
    # 16kk + 4(l >> 5) + 8(i >> 2) + (i & 3)
    P = rng.random((32, BK))                          # [row, key]
    out = np.zeros((64, D // 32, 16))
    for kk in range(2):
        pb = np.stack([[P[l & 31, 16 * kk + 4 * (l >> 5) + 8 * (i >> 2) + (i & 3)] for i in range(8)]
                       for l in range(64)])
        for vb in range(D // 32):
            out[:, vb] += mfma_32x32x16(bf16_to_f64(value_operand(vlds, vb, kk)), pb)
    O_T = Vf.T @ P.T                                  # [value dim, row]
    for l, vb, j in itertools.product(range(64), range(D // 32), range(16)):
        dim = 32 * vb + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3)
        assert out[l, vb, j] == pytest.approx(O_T[dim, l & 31], rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("D", [64, 128])
def test_each_tile_byte_is_written_by_one_copy_of_one_wave(D):
    """Wave w issues K copies ks = w*KPW .. and V copies c = w*VPW .., each one 1 KB region
    of its buffer, so the four waves' regions tile each buffer exactly."""
    KPW, VPW = D // 64, D // 64
    for per_wave, n in ((KPW, D // 16), (VPW, 2 * (D // 32))):
        regions = [set(range(1024 * c, 1024 * c + 1024)) for w in range(WAVES) for c in range(w * per_wave, (w + 1) * per_wave)]
        assert len(regions) == n
        assert set().union(*regions) == set(range(BK * 2 * D))
        assert sum(map(len, regions)) == BK * 2 * D


# ---- schedule ------------------------------------------------------------------------------

def events(kt_live, n_buf, ahead, lpw_, wait_n):
    """Every wave runs the same program, so one wave's view suffices for the intervals; the
    hazard is between any wave's copy and any wave's (or its own) reads, which the barrier
    alone orders.  Returns (copies, reads): copies as (buffer, tile, first phase, last phase
    it may still be in flight), reads as (buffer, tile, phase).  Phase t is the stretch
    between the barrier before tile t's compute and the one after it; the prologue is phase -1."""
    issued = []                       # (instruction index, phase, tile)
    n = 0
    for t in range(ahead):            # prologue copies
        issued += [(n + i, -1, t) for i in range(lpw_)]
        n += lpw_
    done_by = {}
    barriers = []                     # instructions issued by each barrier, phase -1 .. kt_live-1
    barriers.append(n)
    for kt in range(kt_live):
        issued += [(n + i, kt, kt + ahead) for i in range(lpw_)]
        n += lpw_
        barriers.append(n)
    for idx, ph, tile in issued:
        # landed by the first barrier, at or after its own phase, that leaves at most wait_n
        # newer instructions pending; the final vmcnt(0) catches the rest
        last = kt_live
        for b_ph, count in zip(range(-1, kt_live), barriers):
            if b_ph >= ph and count - idx - 1 >= wait_n:
                last = b_ph
                break
        done_by[(idx, tile)] = last
    copies = sorted({(tile % n_buf, tile, ph, done_by[(idx, tile)]) for idx, ph, tile in issued})
    reads = [(kt % n_buf, kt, kt) for kt in range(kt_live)]
    return copies, reads


def hazards(kt_live, n_buf=3, ahead=2, wait_n=None, lpw_=4):
    wait_n = lpw_ if wait_n is None else wait_n
    copies, reads = events(kt_live, n_buf, ahead, lpw_, wait_n)
    found = []
    for buf, tile, first, last in copies:
        for rbuf, rtile, ph in reads:
            if rbuf == buf and first <= ph <= last:
                found.append(("read", tile, rtile, ph))
        for buf2, tile2, first2, last2 in copies:
            if buf2 == buf and tile2 != tile and first <= last2 and first2 <= last:
                found.append(("copy", tile, tile2))
    return found


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kt_live", [1, 2, 3, 4, 7, 64])
def test_kernel_schedule_has_no_overlap(D, kt_live):
    assert hazards(kt_live, lpw_=lpw(D)) == []


@pytest.mark.parametrize("kt_live", [1, 2, 3, 7])
def test_every_read_tile_has_landed(kt_live):
    """The copies of tile t land at or before the barrier that opens phase t."""
    copies, reads = events(kt_live, 3, 2, 4, 4)
    for buf, tile, first, last in copies:
        if tile < kt_live:
            assert last <= tile - 1


def test_two_buffers_race():
    # tile t + 2 would refill the buffer tile t is read from, in the same phase
    assert ("read", 2, 0, 0) in hazards(4, n_buf=2)


def test_a_looser_wait_races():
    # with vmcnt(2 LPW) the copies of tile t + 1 may still land while it is read
    assert any(h[0] == "read" and h[1] == h[2] for h in hazards(4, wait_n=8))


# ---- the epilogue: O~ out through the tile buffers -------------------------------------------
# After the loop every wave waits for all its copies and the workgroup meets at a barrier; then
# wave w stages its accumulators through tile buffer w (K buffers 0-2, V buffer 0), one 32-wide
# value block of a 32-row sub-tile at a time, in 4 KB regions: written in the accumulator layout
# (lane (r, hi) holds row r, columns 8a + 4hi .. +3 of the block for a = 0..3), read back
# row-major (lane l: row 8j + l // 8, 16-byte chunk l % 8, j = 0..3) and stored.  Row R of a
# region sits at R * 128 with chunk C at slot C ^ ((R >> 1) & 7).

def stage_base(D, s, vb):
    """Offset of the region of (sub-tile s, value block vb) in the wave's tile buffer: two
    regions used in turn where the buffer holds 8 KB (d = 128), one at d = 64 (4 KB)."""
    return ((s * (D // 32) + vb) & 1) * 4096 if BK * 2 * D == 8192 else 0


def acc_write(lane, a):
    r, hi = lane & 31, lane >> 5
    return r * 128 + (((2 * a + hi) ^ ((r >> 1) & 7)) * 16), r, 8 * a + 4 * hi


def row_read(lane, j):
    R, C = 8 * j + (lane >> 3), lane & 7
    return R * 128 + ((C ^ ((R >> 1) & 7)) * 16), R, 4 * C


@pytest.mark.parametrize("D", [64, 128])
def test_epilogue_staging_round_trip(D):
    """Every accumulator element reaches its row and column, and no region leaves the wave's
    tile buffer (the neighbouring buffers are other waves' staging areas)."""
    TB = BK * 2 * D
    lds = np.full(TB // 4, np.nan)
    out = np.full((64, D), np.nan)
    tag = lambda row, col: row * 1000.0 + col
    for s in range(2):
        for vb in range(D // 32):
            base = stage_base(D, s, vb)
            assert 0 <= base and base + 4096 <= TB
            for a in range(4):
                for lane in range(64):
                    off, r, c0 = acc_write(lane, a)
                    for e in range(4):
                        lds[(base + off) // 4 + e] = tag(32 * s + r, vb * 32 + c0 + e)
            for j in range(4):
                for lane in range(64):
                    off, R, c0 = row_read(lane, j)
                    for e in range(4):
                        out[32 * s + R, vb * 32 + c0 + e] = lds[(base + off) // 4 + e]
    expect = np.array([[tag(r, c) for c in range(D)] for r in range(64)])
    assert np.array_equal(out, expect)


def test_epilogue_staging_is_free_of_bank_conflicts():
    """A 16-byte LDS access of 16 lanes covers 256 bytes, all 64 banks, when the lanes' 16-byte
    slots (address / 16 mod 16) are distinct; both access patterns meet that."""
    for a in range(4):
        for g in range(4):
            assert len({(acc_write(l, a)[0] // 16) % 16 for l in range(16 * g, 16 * g + 16)}) == 16
    for j in range(4):
        for g in range(4):
            assert len({(row_read(l, j)[0] // 16) % 16 for l in range(16 * g, 16 * g + 16)}) == 16


@pytest.mark.parametrize("kt_live", [1, 2, 3, 7, 64])
def test_every_copy_lands_before_the_epilogue(kt_live):
    """The staging phase comes after the barrier that follows the loop's final vmcnt(0): no copy,
    including the two past the last live tile, can still write a tile buffer there."""
    copies, _ = events(kt_live, 3, 2, 4, 4)
    assert max(last for _, _, _, last in copies) <= kt_live
