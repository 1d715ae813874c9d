"""A CPU model of the bf16 step kernel's LDS traffic: which bytes each wave reads and which
bytes each wave's direct copies (buffer_load ... lds) write, phase by phase, where a phase is
the stretch between two workgroup barriers.

Ordering rules the model relies on: a wave's direct copies land in LDS before its
s_waitcnt vmcnt(0) returns, every wave waits so before the barrier that ends the phase, and
the barrier orders everything before it against everything after it.  Inside one phase
nothing orders one wave's accesses against another's, so a byte one wave's copy writes must
not be read or written by any other wave in the same phase.

The address formulas are the kernel's (64-key tiles of d bf16 per buffer, four waves; a
copy of one 1 KB span per instruction, lane i writing bytes [16 i, 16 i + 16) after the
instruction's base; the score operand reads 16 bytes per lane, the value operand two 8-byte
transposing reads per lane).  The model checks the schedule of the shipped kernel and shows
that the schedule without the barrier after the prologue's scores races: the first step's
copy of K tile 2 refills the K buffer every wave reads for tile 0's scores."""

import itertools

import pytest

BK = 64        # keys per tile
WAVES = 4


def k_phys(D, t, c):
    return c ^ (t & 15) if D == 128 else c ^ ((t >> 1) & 7)


def v_phys(D, t, c):
    return c ^ (4 * (t & 3)) if D == 128 else c ^ (4 * ((t >> 1) & 1))


def copy_bytes(D, wave):
    """Bytes of one tile buffer that `wave`'s direct copies write."""
    RB, CPR = 2 * D, D // 8
    RPL = 64 // CPR
    LPW = BK * RB // 1024 // WAVES
    out = set()
    for u in range(LPW):
        row0 = (wave * LPW + u) * RPL
        base = row0 * RB
        for lane in range(64):
            out.update(range(base + 16 * lane, base + 16 * lane + 16))
    return out


def score_read_bytes(D):
    """Bytes of a K buffer one wave's score operand reads (every wave reads the same)."""
    RB, KS = 2 * D, D // 16
    out = set()
    for lane, ks, kh in itertools.product(range(64), range(KS), range(2)):
        r32, hi = lane & 31, lane >> 5
        off = r32 * RB + (k_phys(D, r32, 2 * ks + hi) << 4) + kh * 32 * RB
        out.update(range(off, off + 16))
    return out


def value_read_bytes(D):
    """Bytes of a V buffer one wave's transposing value-operand reads touch."""
    RB, VB = 2 * D, D // 32
    out = set()
    for lane in range(64):
        g, a, e = lane >> 4, lane & 3, (lane >> 2) & 3
        key = 4 * (g >> 1) + e
        for vb, kk, half in itertools.product(range(VB), range(4), range(2)):
            dv = 32 * vb + 16 * (g & 1) + 4 * a
            off = key * RB + (v_phys(D, key, dv >> 3) << 4) + ((dv & 7) << 1) + kk * 16 * RB + half * 8 * RB
            out.update(range(off, off + 8))
    return out


def schedule(kt_live, barrier_after_prologue):
    """Phases of one workgroup: lists of (wave, op, buffer), op 'w' (copy) or 'r' (read).
    Buffers: ('k', 0 or 1) and ('v', 0 or 1)."""
    phases = []
    ph = []
    for w in range(WAVES):   # prologue copies: K0 -> k0, V0 -> v0, K1 -> k1; vmcnt(0); barrier
        ph += [(w, "w", ("k", 0)), (w, "w", ("v", 0)), (w, "w", ("k", 1))]
    phases.append(ph)
    ph = [(w, "r", ("k", 0)) for w in range(WAVES)]   # scores of tile 0
    if barrier_after_prologue:
        phases.append(ph)
        ph = []
    for kt in range(kt_live):
        B = kt & 1
        for w in range(WAVES):
            ph += [(w, "w", ("k", B)),          # copy of K tile kt + 2
                   (w, "w", ("v", 1 - B)),      # copy of V tile kt + 1
                   (w, "r", ("v", B)),          # value product of tile kt
                   (w, "r", ("k", 1 - B))]      # scores of tile kt + 1
        phases.append(ph)                       # vmcnt(0); barrier
        ph = []
    return phases


def hazards(D, phases):
    reads = {"k": score_read_bytes(D), "v": value_read_bytes(D)}
    found = []
    for i, ph in enumerate(phases):
        for (w1, op1, b1), (w2, op2, b2) in itertools.permutations(ph, 2):
            if w1 == w2 or b1 != b2 or op1 != "w":
                continue
            mine = copy_bytes(D, w1)
            theirs = copy_bytes(D, w2) if op2 == "w" else reads[b2[0]]
            if mine & theirs:
                found.append((i, w1, w2, op2, b1))
    return found


@pytest.mark.parametrize("D", [64, 128])
def test_copies_tile_the_buffer_and_reads_stay_inside(D):
    size = BK * 2 * D
    parts = [copy_bytes(D, w) for w in range(WAVES)]
    assert set().union(*parts) == set(range(size))
    assert sum(len(p) for p in parts) == size          # each byte written by exactly one wave
    assert score_read_bytes(D) == set(range(size))     # every wave's scores read the whole K tile
    assert value_read_bytes(D) == set(range(size))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kt_live", [1, 2, 3, 6])
def test_shipped_schedule_has_no_cross_wave_hazard(D, kt_live):
    assert hazards(D, schedule(kt_live, barrier_after_prologue=True)) == []


@pytest.mark.parametrize("D", [64, 128])
def test_schedule_without_the_prologue_barrier_races(D):
    found = hazards(D, schedule(2, barrier_after_prologue=False))
    # every wave's copy of K tile 2 overlaps every other wave's reads of tile 0's keys
    assert {(w1, w2) for (i, w1, w2, op, b) in found if op == "r" and b == ("k", 0)} == \
        {(a, b) for a in range(WAVES) for b in range(WAVES) if a != b}


def test_epilogue_staging_through_private_buffers_is_hazard_free():
    """The LDS-staged epilogue tried earlier: after the last barrier each wave writes its 32
    rows of O~ (16 KB of fp32) into one tile buffer of its own (k0, k1, v0, v1 for waves 0-3)
    and reads them back.  The buffers are disjoint, so nothing in that phase crosses waves;
    its wrong results came from the prologue hazard above, which it shared."""
    own = {0: ("k", 0), 1: ("k", 1), 2: ("v", 0), 3: ("v", 1)}
    assert len(set(own.values())) == WAVES
    ph = [(w, op, own[w]) for w in range(WAVES) for op in ("w", "r")]
    assert all(b1 != b2 for (w1, _, b1), (w2, _, b2) in itertools.permutations(ph, 2) if w1 != w2)
