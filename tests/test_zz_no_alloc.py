"""ra_decode_step_noalloc, the split-KV step for callers that cannot allocate, through the C
ABI: its result equals ra_decode_step's with a caller workspace, bit for bit, on two calls in
a row (the second smaller, so the library's scratch still holds the first call's chunk
states), and both match the fp64 oracle.  Requests larger than the scratch are refused."""

import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bf16_close, require_gpu, say, to64

pytestmark = pytest.mark.gpu

NONE, CONTIG = 0, 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


# (B, Hq, Hkv, n_q, d, kv_len, mask, q_offset): about 32 MiB of chunk states, then a small one
CALLS = [
    (1, 64, 8, 16, 128, 131072, NONE, 0),
    (1, 16, 2, 3, 128, 5000, CONTIG, 4997),
]


def _lap_pair(case, seed):
    import exact_long_context_amd as ra
    from exact_long_context_amd._abi import check, lib
    B, Hq, Hkv, n, d, nk, mask, q_off = case
    q, k, v = synth.random_case(seed, B, Hq, Hkv, n, nk, d, "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    st = ra.RingState(qd, kd)
    need = ra.decode_workspace_bytes(st.desc, nk)
    say(f"  case {case}: {need / 2**20:.2f} MiB of chunk states")
    assert 0 < need <= ra.RA_DECODE_NOALLOC_MAX_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st.decode_step(kd, vd, mask, q_off, 0, workspace=ws)
    o_ws, lse_ws = st.finalize()
    st.close()
    st2 = ra.RingState(qd, kd)
    check(lib().ra_decode_step_noalloc(C.c_void_p(st2._handle().value), kd.data_ptr(), vd.data_ptr(),
                                       nk, mask, q_off, 0))
    o_na, lse_na = st2.finalize()
    stats = st2.stats()
    st2.close()
    torch.cuda.synchronize()
    assert stats["blocks_run"] == 1
    assert torch.equal(o_na, o_ws) and torch.equal(lse_na, lse_ws)
    ref, ref_lse = oracle.dense_attention(to64(q), to64(k), to64(v), q_off + np.arange(n), np.arange(nk),
                                          mask != NONE)
    assert_bf16_close(to64(o_na), ref, "no-alloc O")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse_na)), fin)
    assert np.max(np.abs(to64(lse_na)[fin] - ref_lse[fin])) <= 2e-2


def test_noalloc_decode_matches_the_workspace_entry_point_twice():
    for i, case in enumerate(CALLS):
        _lap_pair(case, 60 + i)


def test_noalloc_decode_refuses_more_than_its_scratch():
    import exact_long_context_amd as ra
    from exact_long_context_amd._abi import RA_E_UNSUPPORTED, lib
    # 4096 tokens of 64 query heads (one chunk per KV head): 262144 rows of chunk state are
    # 130 MiB, more than the scratch; the call is refused before any work is enqueued (and the
    # tensors are real, so the refused call would be in bounds anyway)
    n, nk = 4096, 512
    q = torch.zeros((1, 64, n, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, nk, 128), dtype=torch.bfloat16, device="cuda")
    st = ra.RingState(q, k)
    assert ra.decode_workspace_bytes(st.desc, nk) > ra.RA_DECODE_NOALLOC_MAX_BYTES
    rc = lib().ra_decode_step_noalloc(C.c_void_p(st._handle().value), k.data_ptr(), k.data_ptr(), nk,
                                      NONE, 0, 0)
    assert rc == RA_E_UNSUPPORTED
    assert st.stats()["blocks_run"] == 0
    st.close()
