"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds only random-number draws and the workload shapes; none of
the attention arithmetic, no positions and no masks.  Both the oracle (CPU,
float64) and the HIP path (bf16 / fp32 on the device) are fed from here, so
they see identical values.

Recipe (one independent stream per (tensor, slab)):

* Every [n, d] slab -- one (batch, head) of one tensor -- is drawn with NumPy's
  Philox generator seeded by ``SeedSequence([seed, tensor_id, part, b, h])``
  as ``standard_normal((n, d), float32)``; tensor_id is Q=0, K=1, V=2, and
  ``part`` is -1 for a tensor drawn in global token order and the rank for a
  query slice drawn directly in local order.
* The slab is multiplied in float32 by ``value_scale`` (1/sqrt(128) for the
  16K x 8-block workloads, 1.0 otherwise), then rounded to the workload dtype
  (bf16 round-to-nearest-even, via torch) or kept as fp32.
* K and V are always drawn in global token order, [B, Hkv, N, d]; each side
  cuts its own blocks from them.  The tiny exactness workload also draws Q
  globally; the large ones draw only the measured rank's slice, [B, Hq, n, d],
  since a global Q at 1M tokens would not fit host memory comfortably.

Because each slab has its own stream, any single head can be regenerated on
its own (the sampled-row parity checks at full size rely on this).

Device draws (``draw_device``): for inputs too large to draw on the host in a
test's time (decode against a million keys), each slab is drawn on the GPU with
torch's device generator seeded from the same SeedSequence words, as
``randn((n, d), float32) * value_scale`` rounded to the dtype.  These are other
numbers than the host draws of the same slab; the oracle side is then fed a
host copy of the very tensors the device side reads.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

Q_ID, K_ID, V_ID = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    N: int                     # global sequence length
    P: int                     # ring size
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: str                 # "bf16" or "f32"
    mask: str                  # "none", "causal_contiguous", "causal_striped", "causal_zigzag"
    ranks: tuple               # ranks measured / checked
    value_scale: float = 1.0   # inputs multiplied by this before rounding
    seed: int = 0
    global_q: bool = False     # draw Q for the whole sequence (tiny cases)
    masks: tuple = field(default=())  # extra masks run on the same tensors

    @property
    def n_local(self) -> int:
        return self.N // self.P

    @property
    def layout(self) -> str:
        return {"causal_striped": "striped", "causal_zigzag": "zigzag"}.get(self.mask, "contiguous")


WORKLOADS = {
    # Tiny exactness case: N=256, P=4, one head, d=64, fp32, rank 2, both masks.
    "tiny_fp32_n256_p4": Workload("tiny_fp32_n256_p4", 256, 4, 1, 1, 1, 64, "f32", "none", (2,),
                                  global_q=True, masks=("none", "causal_contiguous")),
    # Non-causal lap: N=131072, P=8, 32 heads, d=128, bf16, inputs scaled by 1/sqrt(128).
    "noncausal_n131072_p8_h32": Workload("noncausal_n131072_p8_h32", 131072, 8, 1, 32, 32, 128,
                                         "bf16", "none", (0,), value_scale=1 / math.sqrt(128)),
    # Causal contiguous imbalance: the same tensors, ranks 0 and 7.
    "causal_contig_n131072_p8_h32": Workload("causal_contig_n131072_p8_h32", 131072, 8, 1, 32, 32,
                                             128, "bf16", "causal_contiguous", (0, 7),
                                             value_scale=1 / math.sqrt(128)),
    # Causal zigzag: the non-causal tensors' shapes, rank r holding chunks r and 15 - r of 16;
    # the first and the last rank (equal work, unlike the contiguous ramp).
    "zigzag_n131072_p8_h32": Workload("zigzag_n131072_p8_h32", 131072, 8, 1, 32, 32, 128, "bf16",
                                      "causal_zigzag", (0, 7), value_scale=1 / math.sqrt(128)),
    # Causal striped: N=262144, P=16, token t on rank t mod 16, rank 5.
    "striped_n262144_p16_h32": Workload("striped_n262144_p16_h32", 262144, 16, 1, 32, 32, 128,
                                        "bf16", "causal_striped", (5,)),
    # Long-context GQA: N=1048576, P=64, 64 query heads over 8 KV heads, striped, rank 5.
    "gqa_striped_n1m_p64_h64kv8": Workload("gqa_striped_n1m_p64_h64kv8", 1048576, 64, 1, 64, 8, 128,
                                           "bf16", "causal_striped", (5,)),
}


def _slab(seed: int, tensor_id: int, part: int, b: int, h: int, n: int, d: int,
          value_scale: float) -> np.ndarray:
    ss = np.random.SeedSequence([seed, tensor_id, part + 1, b, h])
    g = np.random.Generator(np.random.Philox(ss))
    x = g.standard_normal((n, d), dtype=np.float32)
    if value_scale != 1.0:
        x *= np.float32(value_scale)
    return x


def draw(seed: int, tensor_id: int, part: int, B: int, H: int, n: int, d: int,
         value_scale: float = 1.0, heads=None, threads: int = 8) -> np.ndarray:
    """float32 [B, len(heads), n, d] before dtype rounding (heads default: all)."""
    heads = list(range(H)) if heads is None else list(heads)
    out = np.empty((B, len(heads), n, d), dtype=np.float32)

    def one(bi_hi):
        bi, hi = bi_hi
        out[bi, hi] = _slab(seed, tensor_id, part, bi, heads[hi], n, d, value_scale)

    jobs = [(bi, hi) for bi in range(B) for hi in range(len(heads))]
    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return out


def draw_device(seed: int, tensor_id: int, part: int, B: int, H: int, n: int, d: int,
                value_scale: float, dtype: str, device):
    """[B, H, n, d] drawn on ``device`` in the workload dtype (see the module docstring)."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    out = torch.empty((B, H, n, d), dtype=tdt, device=device)
    for b in range(B):
        for h in range(H):
            word = np.random.SeedSequence([seed, tensor_id, part + 1, b, h]).generate_state(1, np.uint64)[0]
            g = torch.Generator(device=device)
            g.manual_seed(int(word) & ((1 << 63) - 1))
            x = torch.randn((n, d), generator=g, device=device, dtype=torch.float32)
            if value_scale != 1.0:
                x.mul_(value_scale)
            out[b, h].copy_(x)
    return out


def round_to_dtype(x: np.ndarray, dtype: str):
    """Round float32 to the workload dtype; returns a CPU torch tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def workload_tensors(w: Workload, rank: int, heads_q=None, heads_kv=None, threads: int = 8):
    """(Q, K, V) CPU torch tensors in the workload dtype.

    K, V: [B, Hkv_sel, N, d] in global token order.
    Q: [B, Hq_sel, n_local, d] -- the rank's slice in local order; for
    ``global_q`` workloads the whole [B, Hq_sel, N, d] is returned instead and
    the caller slices it.
    """
    d = w.head_dim
    if w.global_q:
        q = draw(w.seed, Q_ID, -1, w.batch, w.q_heads, w.N, d, w.value_scale, heads_q, threads)
    else:
        q = draw(w.seed, Q_ID, rank, w.batch, w.q_heads, w.n_local, d, w.value_scale, heads_q,
                 threads)
    k = draw(w.seed, K_ID, -1, w.batch, w.kv_heads, w.N, d, w.value_scale, heads_kv, threads)
    v = draw(w.seed, V_ID, -1, w.batch, w.kv_heads, w.N, d, w.value_scale, heads_kv, threads)
    return round_to_dtype(q, w.dtype), round_to_dtype(k, w.dtype), round_to_dtype(v, w.dtype)


def random_case(seed: int, B: int, Hq: int, Hkv: int, n_q: int, N: int, d: int, dtype: str,
                value_scale: float = 1.0):
    """Small random Q [B,Hq,n_q,d], K/V [B,Hkv,N,d] for parity sweeps."""
    q = draw(seed, Q_ID, 0, B, Hq, n_q, d, value_scale, threads=1)
    k = draw(seed, K_ID, -1, B, Hkv, N, d, value_scale, threads=1)
    v = draw(seed, V_ID, -1, B, Hkv, N, d, value_scale, threads=1)
    return round_to_dtype(q, dtype), round_to_dtype(k, dtype), round_to_dtype(v, dtype)
