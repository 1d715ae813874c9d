"""GPU parity of ra_decode_step, the split-KV block step for a few query rows, against the
fp64 oracle: single blocks under every single-range mask, ragged and tiny key counts, rows
that see no key, blocks that are skipped, laps that mix it with ra_block_step, and a
full-size decode against one million keys checked on sampled heads."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bf16_close, require_gpu, say, to64

pytestmark = pytest.mark.gpu

NONE, CONTIG, STRIPED = 0, 1, 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _positions(mask, P, q_off, k_off, n, nk):
    s = P if mask == STRIPED else 1
    return q_off + s * np.arange(n), k_off + s * np.arange(nk)


def _check(o, lse, q, k, v, q_pos, k_pos, causal, what):
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_pos, k_pos, causal)
    got = to64(o)
    empty = ~np.isfinite(ref_lse)
    assert np.array_equal(~np.isfinite(to64(lse)), empty), "rows with no key differ"
    assert np.all(got[empty[..., None].repeat(got.shape[-1], -1)] == 0.0)
    assert_bf16_close(got, ref, what)
    ok = ~empty
    assert np.max(np.abs(to64(lse)[ok] - ref_lse[ok]), initial=0.0) <= 2e-2


# (B, Hq, Hkv, n_q, d, kv_len, mask, P, q_off, k_off)
CASES = [
    (1, 8, 1, 1, 128, 5000, NONE, 1, 0, 0),          # one token, GQA 8:1, ragged keys
    (2, 16, 2, 4, 64, 3000, CONTIG, 1, 2996, 0),      # 4 new tokens at the end of the block
    (1, 12, 3, 5, 128, 4099, STRIPED, 4, 16003, 1),   # striped positions, diagonal in the tail
    (1, 8, 1, 7, 128, 2500, CONTIG, 1, 2493, 0),      # 56 packed rows: two row groups
    (1, 4, 4, 3, 64, 700, CONTIG, 1, 300, 200),       # causal cut in the block's middle
    (1, 2, 1, 2, 128, 1, NONE, 1, 0, 0),              # a single key
    (1, 2, 2, 3, 128, 17, NONE, 1, 0, 0),             # fewer keys than one tile
    (1, 4, 2, 6, 64, 600, CONTIG, 1, 100, 103),       # rows 0..2 see no key
    (1, 64, 8, 1, 128, 20000, NONE, 1, 0, 0),         # the long-context GQA head shape
    (1, 32, 32, 1, 128, 9000, CONTIG, 1, 9000, 0),    # MHA decode, whole block visible
    (1, 16, 2, 16, 128, 3001, CONTIG, 1, 2985, 0),    # 128 packed rows: four waves share tiles
    (1, 8, 2, 20, 64, 2000, NONE, 1, 0, 0),           # 80 packed rows: three waves and an idle one
    (1, 8, 1, 20, 128, 1500, STRIPED, 4, 6003, 3),    # 160 packed rows: two four-wave workgroups
    (2, 8, 2, 10, 64, 40000, CONTIG, 1, 39990, 0),    # two row groups at d = 64, many chunks
    (1, 8, 1, 6, 128, 140000, CONTIG, 1, 139995, 0),  # two row groups on a long block: the ring
    (1, 8, 1, 6, 64, 140000, CONTIG, 1, 100000, 0),   # long block, but only 100006 keys visible
    (1, 8, 1, 6, 64, 133000, NONE, 1, 0, 0),          # two row groups, ring at d = 64
    (2, 8, 1, 12, 128, 5000, STRIPED, 4, 19997, 2),   # batch 2, three row groups on the ring
    (1, 64, 8, 16, 128, 16461, CONTIG, 1, 16445, 0),  # ring chunks at their 512-key floor, 77-key tail
    (1, 64, 8, 8, 128, 33000, NONE, 1, 0, 0),         # two row groups, 1024 waves, ragged chunks
    (1, 64, 8, 2, 128, 20000, NONE, 1, 0, 0),         # 16 packed rows: one group, 1024-wave target
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}h{c[1]}x{c[2]}n{c[3]}d{c[4]}k{c[5]}m{c[6]}")
def test_decode_step_matches_oracle(case):
    import exact_long_context_amd as ra
    B, Hq, Hkv, n, d, nk, mask, P, q_off, k_off = case
    say(f"  decode case {case}")
    q, k, v = synth.random_case(700 + nk % 97, B, Hq, Hkv, n, nk, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    st = ra.RingState(qd, kd, ring_size=P)
    ws = torch.empty(max(ra.decode_workspace_bytes(st.desc, nk), 256), dtype=torch.uint8, device="cuda")
    st.decode_step(kd, vd, mask, q_off, k_off, workspace=ws)
    stats = st.stats()
    o, lse = st.finalize()
    torch.cuda.synchronize()
    st.close()
    q_pos, k_pos = _positions(mask, P, q_off, k_off, n, nk)
    _check(o, lse, q, k, v, q_pos, k_pos, mask != NONE, "decode O")
    plan = ra.plan_block(st.desc, nk, mask, q_off, k_off)
    assert stats["live_pairs"] == plan["live_pairs"]
    assert stats["blocks_run"] == 1


def test_decode_lap_mixed_with_block_steps():
    """A lap of six blocks through one state, alternating ra_decode_step and ra_block_step,
    in ring order (the first block is the diagonal one); the result is the oracle's dense
    attention over all keys, so every chunk state and the running state were combined right."""
    import exact_long_context_amd as ra
    Hq, Hkv, n, d, nk, P = 16, 4, 3, 128, 1111, 6
    N = P * nk
    q, k, v = synth.random_case(811, 1, Hq, Hkv, n, N, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    q_off = 4 * nk + 500                      # rank 4's rows near the middle of its block
    q_pos = q_off + np.arange(n)
    st = ra.RingState(qd, kd[:, :, :nk], ring_size=P)
    ws = torch.empty(ra.decode_workspace_bytes(st.desc, nk), dtype=torch.uint8, device="cuda")
    say("  decode lap: 6 blocks, alternating split-KV and tiled steps")
    for u, j in enumerate(oracle.ring_visit_order(P, 4)):
        kj, vj = kd[:, :, j * nk:(j + 1) * nk], vd[:, :, j * nk:(j + 1) * nk]
        if u % 2 == 0:
            st.decode_step(kj, vj, CONTIG, q_off, j * nk, workspace=ws)
        else:
            st.step(kj, vj, CONTIG, q_off, j * nk)
    stats = st.stats()
    o, lse = st.finalize()
    torch.cuda.synchronize()
    st.close()
    assert stats["blocks_run"] == 5 and stats["blocks_skipped"] == 1
    _check(o, lse, q, k, v, q_pos, np.arange(N), True, "decode lap O")


def test_decode_skips_and_empty_blocks():
    """A block wholly in the future and an empty block launch nothing; the state stays fresh
    and a later block still starts it from the empty state."""
    import exact_long_context_amd as ra
    Hq, Hkv, n, d, nk = 8, 2, 2, 64, 500
    q, k, v = synth.random_case(820, 1, Hq, Hkv, n, nk, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    st = ra.RingState(qd, kd)
    ws = torch.zeros(ra.decode_workspace_bytes(st.desc, nk), dtype=torch.uint8, device="cuda")
    st.decode_step(kd, vd, CONTIG, 0, 10, workspace=ws)      # every key after every row
    st.decode_step(kd[:, :, :0], vd[:, :, :0], NONE, 0, 0, workspace=ws)
    s = st.stats()
    assert s["blocks_run"] == 0 and s["blocks_skipped"] == 2
    # garbage in the state's workspace must not leak into a fresh start
    st.workspace.fill_(0x7f)
    st.decode_step(kd, vd, NONE, 0, 0, workspace=ws)
    o, lse = st.finalize()
    torch.cuda.synchronize()
    st.close()
    _check(o, lse, q, k, v, np.arange(n), np.arange(nk), False, "after skips O")


def test_decode_rejects_short_workspace():
    import exact_long_context_amd as ra
    q, k, v = synth.random_case(830, 1, 4, 2, 1, 4096, 128, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    st = ra.RingState(qd, kd)
    need = ra.decode_workspace_bytes(st.desc, 4096)
    short = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ra.RaError):
        st.decode_step(kd, vd, NONE, workspace=short)
    st.close()


def test_decode_fp32_takes_the_exact_path():
    """fp32 inputs go through the tiled fp32 step: the result meets the fp32 bar."""
    import exact_long_context_amd as ra
    from gpu_util import assert_f32_close
    q, k, v = synth.random_case(831, 1, 8, 2, 3, 2000, 64, "f32")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    st = ra.RingState(qd, kd)
    st.decode_step(kd, vd, CONTIG, 1997, 0)
    o, lse = st.finalize()
    torch.cuda.synchronize()
    st.close()
    ref, _ = oracle.dense_attention(to64(q), to64(k), to64(v), 1997 + np.arange(3), np.arange(2000), True)
    assert_f32_close(to64(o), ref, "fp32 decode O")


def test_decode_fullsize_million_keys_sampled_heads():
    """One token of 64 query heads over 8 KV heads against 1,048,576 keys (the long-context
    GQA head shape with the whole context local), inputs N(0,1) / sqrt(128); the oracle
    checks four sampled query heads of two KV groups one by one."""
    import exact_long_context_amd as ra
    B, Hq, Hkv, n, d, nk = 1, 64, 8, 1, 128, 1 << 20
    say(f"  decode full size: Hq={Hq} Hkv={Hkv} keys={nk}")
    vs = 1 / np.sqrt(128)
    qd = synth.draw_device(901, synth.Q_ID, 0, B, Hq, n, d, vs, "bf16", "cuda")
    kd = synth.draw_device(901, synth.K_ID, -1, B, Hkv, nk, d, vs, "bf16", "cuda")
    vd = synth.draw_device(901, synth.V_ID, -1, B, Hkv, nk, d, vs, "bf16", "cuda")
    st = ra.RingState(qd, kd)
    st.decode_step(kd, vd, NONE)
    o, lse = st.finalize()
    torch.cuda.synchronize()
    st.close()
    kv64 = {}
    for h in [0, 7, 40, 47]:
        g = h // (Hq // Hkv)
        if g not in kv64:
            kv64.clear()
            kv64[g] = (to64(kd[:, g:g + 1]), to64(vd[:, g:g + 1]))
        ref, ref_lse = oracle.dense_attention(to64(qd[:, h:h + 1]), *kv64[g], np.arange(n), np.arange(nk), False)
        assert_bf16_close(to64(o[:, h:h + 1]), ref, f"head {h} O")
        assert abs(float(lse[0, h, 0]) - float(ref_lse[0, 0, 0])) <= 2e-2


def test_decode_fullsize_ring_sixteen_tokens():
    """Sixteen tokens of 64 query heads over 8 KV heads (128 packed rows per KV head: four row
    groups in one workgroup sharing an LDS ring) against 1,048,576 keys; the oracle checks
    every row of four sampled query heads of two KV groups."""
    import exact_long_context_amd as ra
    B, Hq, Hkv, n, d, nk = 1, 64, 8, 16, 128, 1 << 20
    say(f"  decode ring full size: Hq={Hq} Hkv={Hkv} tokens={n} keys={nk}")
    vs = 1 / np.sqrt(128)
    qd = synth.draw_device(902, synth.Q_ID, 0, B, Hq, n, d, vs, "bf16", "cuda")
    kd = synth.draw_device(902, synth.K_ID, -1, B, Hkv, nk, d, vs, "bf16", "cuda")
    vd = synth.draw_device(902, synth.V_ID, -1, B, Hkv, nk, d, vs, "bf16", "cuda")
    st = ra.RingState(qd, kd)
    st.decode_step(kd, vd, NONE)
    o, lse = st.finalize()
    torch.cuda.synchronize()
    st.close()
    kv64 = {}
    for h in [3, 4, 56, 63]:
        g = h // (Hq // Hkv)
        if g not in kv64:
            kv64.clear()
            kv64[g] = (to64(kd[:, g:g + 1]), to64(vd[:, g:g + 1]))
        ref, ref_lse = oracle.dense_attention(to64(qd[:, h:h + 1]), *kv64[g], np.arange(n), np.arange(nk), False)
        assert_bf16_close(to64(o[:, h:h + 1]), ref, f"head {h} O")
        assert np.max(np.abs(to64(lse[:, h:h + 1]) - ref_lse)) <= 2e-2


def test_decode_is_bitwise_repeatable():
    """Twenty identical split-KV steps (four-wave workgroups sharing tiles, many chunks) give
    bit-identical states."""
    import exact_long_context_amd as ra
    g = torch.Generator(device="cpu").manual_seed(78)
    q = (torch.randn(2, 64, 8, 128, generator=g) * 0.3).to(torch.bfloat16).cuda()
    k = (torch.randn(2, 8, 70000, 128, generator=g) * 0.3).to(torch.bfloat16).cuda()
    v = torch.randn(2, 8, 70000, 128, generator=g).to(torch.bfloat16).cuda()
    say("  decode repeatability: 2 x 64 heads x 8 tokens, 70000 keys")
    states = []
    for _ in range(20):
        st = ra.RingState(q, k)
        st.decode_step(k, v, NONE)
        st.decode_step(k[:, :, :1000], v[:, :, :1000], NONE)
        torch.cuda.synchronize()
        states.append(st.workspace.clone())
        st.close()
    for other in states[1:]:
        assert torch.equal(states[0], other)
    # the same with two row groups on a long block (four-wave workgroups on an LDS ring, two
    # tile subsets per row group)
    q = synth.draw_device(79, synth.Q_ID, 0, 1, 64, 8, 128, 0.3, "bf16", "cuda")
    k = synth.draw_device(79, synth.K_ID, -1, 1, 8, 200000, 128, 0.3, "bf16", "cuda")
    v = synth.draw_device(79, synth.V_ID, -1, 1, 8, 200000, 128, 1.0, "bf16", "cuda")
    say("  decode repeatability: 64 heads x 8 tokens, 200000 keys")
    states = []
    for _ in range(20):
        st = ra.RingState(q, k)
        st.decode_step(k, v, NONE)
        torch.cuda.synchronize()
        states.append(st.workspace.clone())
        st.close()
    for other in states[1:]:
        assert torch.equal(states[0], other)


def test_decode_token_major_views():
    """Q, K and V as token-major [B, n, H, d] storage seen through [B, H, n, d] views (the
    strides go through the ABI; nothing is copied)."""
    import exact_long_context_amd as ra
    B, Hq, Hkv, n, d, nk = 2, 16, 4, 3, 128, 2500
    q, k, v = synth.random_case(840, B, Hq, Hkv, n, nk, d, "bf16")
    qt = q.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    kt = k.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    vt = v.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    assert kt.stride()[2] == Hkv * d and not kt.is_contiguous()
    st = ra.RingState(qt, kt)
    st.decode_step(kt, vt, CONTIG, nk - n, 0)
    o, lse = st.finalize()
    torch.cuda.synchronize()
    st.close()
    _check(o, lse, q, k, v, nk - n + np.arange(n), np.arange(nk), True, "token-major decode O")


def _sawtooth_levels(nk, rng):
    """Planted score levels (natural units) for a decode block: plateaus 0, 40, 80, 120 of 128
    keys each, repeating.  Inside the 120 plateau only every 16th key reaches it (the rest stay
    near 80), so the outputs mix a few dozen keys.  A chunk that starts low meets plateaus 40
    or more units higher in later tiles: rows holding keys must move their reference."""
    t = np.arange(nk)
    seg = (t // 128) % 4
    lv = 40.0 * seg - 3.0 * rng.uniform(0.0, 1.0, nk)
    top = (seg == 3) & (t % 16 != 5)
    lv[top] = 80.0 - 3.0 * rng.uniform(0.0, 1.0, int(top.sum()))
    return lv


# (B, Hq, Hkv, n_q, d, kv_len): one row group (decode_kernel, one wave), two row groups on a
# short block (decode_kernel, two waves), four row groups (ring kernel 4 x 1), two row groups
# on a long block (ring kernel 2 x 2)
PLANTED = [
    (1, 8, 1, 1, 128, 4096),
    (1, 8, 1, 7, 128, 2500),
    (1, 16, 2, 16, 128, 3001),
    (1, 8, 1, 6, 64, 140000),
]


@pytest.mark.parametrize("case", PLANTED, ids=lambda c: f"h{c[1]}x{c[2]}n{c[3]}d{c[4]}k{c[5]}")
def test_decode_live_rows_rescale_on_planted_sawtooth(case):
    """Extreme scores in the split-KV step ("Ring Attention：把超长序列沿设备环流动", section
    正确性测试应覆盖哪些边界): scores climb by 40 natural units from tile to tile inside a chunk,
    so every chunk wave must rescale rows that already hold keys ("Ring attention" MCQ page,
    body).  The debug counter proves the path ran; the result matches the oracle."""
    import exact_long_context_amd as ra
    from gpu_util import plant_score_levels
    B, Hq, Hkv, n, d, nk = case
    q, k, _ = synth.random_case(900 + nk % 89, B, Hq, Hkv, n, nk, d, "bf16", value_scale=0.3)
    v = synth.random_case(901 + nk % 89, B, Hq, Hkv, n, nk, d, "bf16")[2]
    plant_score_levels(q, k, _sawtooth_levels(nk, np.random.default_rng(nk)))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say(f"  planted decode {case}")
    outs = []
    for counted in (True, False):
        st = ra.RingState(qd, kd)
        counters = torch.zeros(5, dtype=torch.int64, device="cuda")
        if counted:
            st.set_debug_counters(counters)
        st.decode_step(kd, vd, NONE)
        outs.append(st.finalize())
        st.close()
        torch.cuda.synchronize()
        if counted:
            moves = counters[3].item()
            say(f"    live-row reference moves: {moves}")
            assert moves > 0, "no row that held keys moved its reference"
    assert torch.equal(outs[0][0], outs[1][0])
    _check(outs[1][0], outs[1][1], q, k, v, np.arange(n), np.arange(nk), False, "planted decode O")
