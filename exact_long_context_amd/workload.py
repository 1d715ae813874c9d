"""Device-side data placement for the emulated ring (torch plumbing only).

Cuts global K/V [B, Hkv, N, d] into the P per-rank blocks a ring would hold:
contiguous slices (rank j owns tokens j*N/P .. (j+1)*N/P - 1), the striped
round-robin layout (rank j owns tokens t with t mod P == j) or the zigzag layout
(rank j owns chunks j and 2P-1-j of 2P, in that order), each block made
contiguous [B, Hkv, N/P, d] so it can be moved with one copy.  The positions of
those tokens are not materialised: the library derives them from the block
index (include/ra.h).
"""

from __future__ import annotations


def shard_blocks(k_global, v_global, P: int, layout: str):
    N = k_global.shape[2]
    if N % P:
        raise ValueError("N must be a multiple of P")
    n = N // P
    ks, vs = [], []
    for j in range(P):
        if layout == "contiguous":
            ks.append(k_global[:, :, j * n:(j + 1) * n].contiguous())
            vs.append(v_global[:, :, j * n:(j + 1) * n].contiguous())
        elif layout == "striped":
            ks.append(k_global[:, :, j::P].contiguous())
            vs.append(v_global[:, :, j::P].contiguous())
        elif layout == "zigzag":
            import torch
            c = n // 2
            if n % 2:
                raise ValueError("zigzag needs N to be a multiple of 2P")
            lo, hi = j * c, (2 * P - 1 - j) * c
            ks.append(torch.cat([k_global[:, :, lo:lo + c], k_global[:, :, hi:hi + c]], dim=2).contiguous())
            vs.append(torch.cat([v_global[:, :, lo:lo + c], v_global[:, :, hi:hi + c]], dim=2).contiguous())
        else:
            raise ValueError(layout)
    return ks, vs


def shard_blocks_padded(k_global, v_global, P: int, layout: str, fill: float = float("nan")):
    """Blocks of ceil(N/P) slots for any N (contiguous or striped): block j holds its real
    tokens first and ``fill`` in the slots past them.  Returns (k_blocks, v_blocks, valid)
    with valid[j] the count of real tokens of block j."""
    import torch
    B, H, N, d = k_global.shape
    c = -(-N // P)
    ks, vs, valid = [], [], []
    for j in range(P):
        if layout == "contiguous":
            idx = torch.arange(j * c, min(N, (j + 1) * c), device=k_global.device)
        elif layout == "striped":
            idx = torch.arange(j, N, P, device=k_global.device)
        else:
            raise ValueError(f"padded shards for {layout!r} are not defined")
        kb = torch.full((B, H, c, d), fill, dtype=k_global.dtype, device=k_global.device)
        vb = torch.full((B, H, c, d), fill, dtype=v_global.dtype, device=v_global.device)
        kb[:, :, :idx.numel()] = k_global[:, :, idx]
        vb[:, :, :idx.numel()] = v_global[:, :, idx]
        ks.append(kb)
        vs.append(vb)
        valid.append(int(idx.numel()))
    return ks, vs, valid


def useful_flops(live_pairs: int, head_dim: int) -> int:
    """4*d flops per allowed (query, key) pair per query head: 2d for the score, 2d for PV."""
    return 4 * head_dim * live_pairs
