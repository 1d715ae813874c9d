"""exact_long_context_amd -- one rank's lap of ring attention on MI355X (gfx950).

A thin Python layer over librocring.so (include/ra.h).  The C entry points are
available under their C names through ``lib()``; the helpers below only
marshal torch tensors (device memory and streams) into those calls.  Every step
of the computation runs in the library's HIP kernels; if the library is not
built, importing this package raises ImportError.
"""

from __future__ import annotations

import ctypes as C

import numpy as np

from ._abi import (  # noqa: F401
    RA_DECODE_NOALLOC_MAX_BYTES,
    RA_DTYPE_BF16,
    RA_DTYPE_F32,
    RA_E_HIP,
    RA_E_INVALID,
    RA_E_STATE,
    RA_E_UNSUPPORTED,
    RA_MASK_CAUSAL_CONTIGUOUS,
    RA_MASK_CAUSAL_STRIPED,
    RA_MASK_CAUSAL_ZIGZAG,
    RA_MASK_NONE,
    RA_MERGE_MAX_PARTS,
    RA_OK,
    RA_TILE_EMPTY,
    RA_TILE_FULL,
    RA_TILE_PARTIAL,
    SIGNATURES,
    RaError,
    check,
    lib,
    ra_desc,
    ra_lap,
    ra_stats,
)

lib()  # fail loudly at import when the library is missing

MASKS = {
    "none": RA_MASK_NONE,
    "causal_contiguous": RA_MASK_CAUSAL_CONTIGUOUS,
    "causal_striped": RA_MASK_CAUSAL_STRIPED,
    "causal_zigzag": RA_MASK_CAUSAL_ZIGZAG,
}


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return RA_DTYPE_BF16
    if t.dtype == torch.float32:
        return RA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def make_desc(batch: int, q_heads: int, kv_heads: int, q_len: int, head_dim: int, dtype: int,
              q_strides, kv_strides, ring_size: int = 1, softmax_scale: float = 0.0,
              stream: int = 0) -> ra_desc:
    d = ra_desc()
    d.batch, d.q_heads, d.kv_heads, d.q_len, d.head_dim = batch, q_heads, kv_heads, q_len, head_dim
    d.dtype = dtype
    d.softmax_scale = softmax_scale
    d.ring_size = ring_size
    for i in range(3):
        d.q_strides[i] = int(q_strides[i])
        d.kv_strides[i] = int(kv_strides[i])
    d.stream = stream
    return d


def desc_for(q, k, ring_size: int = 1, softmax_scale: float = 0.0, stream=None) -> ra_desc:
    """Descriptor for Q_r [B, Hq, n, d] and KV blocks shaped/strided like k [B, Hkv, nk, d]."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("Q and K must be 4-D [B, H, n, d]")
    if q.stride(-1) != 1 or k.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous")
    if q.dtype != k.dtype:
        raise TypeError("Q and K dtypes differ")
    B, Hq, n, d = q.shape
    return make_desc(B, Hq, k.shape[1], n, d, _dtype_code(q), q.stride()[:3], k.stride()[:3],
                     ring_size, softmax_scale, _stream_handle(stream) if q.is_cuda else 0)


def workspace_bytes(desc: ra_desc) -> int:
    return int(lib().ra_workspace_bytes(C.byref(desc)))


def decode_workspace_bytes(desc: ra_desc, kv_len: int) -> int:
    return int(lib().ra_decode_workspace_bytes(C.byref(desc), kv_len))


def bwd_workspace_bytes(desc: ra_desc) -> int:
    return lib().ra_bwd_workspace_bytes(C.byref(desc))


def workspace_layout(desc: ra_desc) -> tuple[int, int, int]:
    o, m, l_ = C.c_size_t(), C.c_size_t(), C.c_size_t()
    check(lib().ra_workspace_layout(C.byref(desc), C.byref(o), C.byref(m), C.byref(l_)))
    return o.value, m.value, l_.value


def plan_block(desc: ra_desc, kv_len: int, mask_kind: int, q_offset: int = 0,
               k_offset: int = 0) -> dict:
    s = ra_stats()
    check(lib().ra_plan_block(C.byref(desc), kv_len, mask_kind, q_offset, k_offset, C.byref(s)))
    return s.as_dict()


def tile_classes(desc: ra_desc, kv_len: int, mask_kind: int, q_offset: int = 0,
                 k_offset: int = 0) -> np.ndarray:
    s = plan_block(desc, kv_len, mask_kind, q_offset, k_offset)
    if mask_kind == RA_MASK_CAUSAL_ZIGZAG:   # tiles follow the two chunks on each axis
        c = desc.q_len // 2
        nqt = 2 * -(-c // s["tile_q"])
        nkt = 2 * -(-c // s["tile_k"])
    else:
        nqt = -(-desc.q_len // s["tile_q"])
        nkt = -(-kv_len // s["tile_k"])
    out = np.zeros((nqt, nkt), dtype=np.uint8)
    check(lib().ra_tile_classes(C.byref(desc), kv_len, mask_kind, q_offset, k_offset,
                                out.ctypes.data_as(C.c_void_p), out.nbytes))
    return out


class RingState:
    """The online-softmax state of one rank's lap (ra_state_init / ra_block_step / ra_finalize).

    ``q`` is the resident query slice (a CUDA tensor [B, Hq, n, d], bf16 or fp32);
    ``kv_like`` any tensor with the shape and strides the KV blocks will have.  The
    workspace (state buffer) is allocated by torch unless given.
    """

    def __init__(self, q, kv_like, ring_size: int = 1, softmax_scale: float = 0.0,
                 workspace=None, stream=None, resume: bool = False):
        import torch
        self.q = q
        self.desc = desc_for(q, kv_like, ring_size, softmax_scale, stream)
        nbytes = workspace_bytes(self.desc)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        elif workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        self.workspace = workspace
        h = C.c_void_p()
        fn = lib().ra_state_resume if resume else lib().ra_state_init
        check(fn(C.byref(self.desc), q.data_ptr(), workspace.data_ptr(), C.byref(h)))
        self._h = h

    def _handle(self):
        if self._h is None:
            raise RuntimeError("state destroyed")
        return self._h

    def step(self, k, v, mask_kind: int, q_offset: int = 0, k_offset: int = 0) -> None:
        if k.stride() != v.stride() or tuple(k.stride()[:3]) != tuple(self.desc.kv_strides):
            raise ValueError("K and V must have the strides the state was created for")
        check(lib().ra_block_step(self._handle(), k.data_ptr(), v.data_ptr(), k.shape[2], mask_kind,
                                  q_offset, k_offset))

    def decode_step(self, k, v, mask_kind: int, q_offset: int = 0, k_offset: int = 0,
                    workspace=None) -> None:
        """ra_decode_step: the split-KV form of step() for a few query rows.  ``workspace`` is a
        torch uint8 device tensor of at least decode_workspace_bytes(desc, k.shape[2]) bytes,
        allocated here if not given."""
        import torch
        if k.stride() != v.stride() or tuple(k.stride()[:3]) != tuple(self.desc.kv_strides):
            raise ValueError("K and V must have the strides the state was created for")
        if workspace is None:
            nbytes = decode_workspace_bytes(self.desc, k.shape[2])
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.q.device)
        check(lib().ra_decode_step(self._handle(), k.data_ptr(), v.data_ptr(), k.shape[2], mask_kind,
                                   q_offset, k_offset, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size()))

    def decode_step_noalloc(self, k, v, mask_kind: int, q_offset: int = 0, k_offset: int = 0) -> None:
        """ra_decode_step_noalloc: decode_step() with the chunk states in the library's own
        per-device scratch (nothing is allocated, here or in the library)."""
        if k.stride() != v.stride() or tuple(k.stride()[:3]) != tuple(self.desc.kv_strides):
            raise ValueError("K and V must have the strides the state was created for")
        check(lib().ra_decode_step_noalloc(self._handle(), k.data_ptr(), v.data_ptr(), k.shape[2],
                                           mask_kind, q_offset, k_offset))

    def finalize(self, out=None, lse=None, want_lse: bool = True):
        import torch
        B, Hq, n, d = self.q.shape
        if out is None:
            out = torch.empty((B, Hq, n, d), dtype=torch.float32, device=self.q.device)
        if lse is None and want_lse:
            lse = torch.empty((B, Hq, n), dtype=torch.float32, device=self.q.device)
        check(lib().ra_finalize(self._handle(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None))
        return out, lse

    def stats(self) -> dict:
        s = ra_stats()
        check(lib().ra_get_stats(self._handle(), C.byref(s)))
        return s.as_dict()

    def set_debug_counters(self, counters) -> None:
        check(lib().ra_state_set_debug_counters(self._handle(),
                                                counters.data_ptr() if counters is not None else None))

    def state_views(self):
        """(O~, m, l) as torch views of the workspace (fp32)."""
        import torch
        B, Hq, n, d = self.q.shape
        o_off, m_off, l_off = workspace_layout(self.desc)
        ws = self.workspace
        rows = B * Hq * n
        o = ws[o_off:o_off + rows * d * 4].view(torch.float32).view(B, Hq, n, d)
        m = ws[m_off:m_off + rows * 4].view(torch.float32).view(B, Hq, n)
        l_ = ws[l_off:l_off + rows * 4].view(torch.float32).view(B, Hq, n)
        return o, m, l_

    def close(self) -> None:
        if self._h is not None:
            lib().ra_state_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def merge_states(desc: ra_desc, parts, merged=None, out=None, lse=None) -> None:
    """ra_merge_states: reduce the states held in the workspaces ``parts`` (torch uint8 device
    tensors laid out for ``desc``) into the workspace ``merged`` and/or O and lse (fp32 device
    tensors [B, Hq, n, d] and [B, Hq, n]), on desc.stream."""
    arr = (C.c_void_p * len(parts))(*[w.data_ptr() for w in parts])
    check(lib().ra_merge_states(C.byref(desc), len(parts), arr,
                                merged.data_ptr() if merged is not None else None,
                                out.data_ptr() if out is not None else None,
                                lse.data_ptr() if lse is not None else None))


class RingBackward:
    """The backward of one rank's lap (ra_bwd_init / ra_bwd_block_step / ra_bwd_finalize).

    ``q`` and ``d_out`` are Q_r and dO_r (same dtype and strides), ``out`` and ``lse`` the
    forward's O_r and lse_r (fp32, as ``RingState.finalize`` returns them); ``kv_like`` any
    tensor with the KV blocks' shape and strides.
    """

    def __init__(self, q, d_out, out, lse, kv_like, ring_size: int = 1, softmax_scale: float = 0.0,
                 workspace=None, stream=None):
        import torch
        if d_out.dtype != q.dtype or d_out.stride() != q.stride() or d_out.shape != q.shape:
            raise ValueError("dO_r must have Q_r's shape, dtype and strides")
        self.q, self.d_out, self.out, self.lse = q, d_out, out.contiguous(), lse.contiguous()
        self.desc = desc_for(q, kv_like, ring_size, softmax_scale, stream)
        nbytes = lib().ra_bwd_workspace_bytes(C.byref(self.desc))
        if workspace is None:
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        self.workspace = workspace
        h = C.c_void_p()
        check(lib().ra_bwd_init(C.byref(self.desc), q.data_ptr(), d_out.data_ptr(), self.out.data_ptr(),
                                self.lse.data_ptr(), workspace.data_ptr(), C.byref(h)))
        self._h = h

    def step(self, k, v, dk, dv, mask_kind: int, q_offset: int = 0, k_offset: int = 0) -> None:
        if k.stride() != v.stride() or tuple(k.stride()[:3]) != tuple(self.desc.kv_strides):
            raise ValueError("K and V must have the strides the state was created for")
        if not (dk.is_contiguous() and dv.is_contiguous()) or dk.shape != k.shape or dv.shape != v.shape:
            raise ValueError("dK and dV must be contiguous fp32 tensors of the block's shape")
        check(lib().ra_bwd_block_step(self._h, k.data_ptr(), v.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                      k.shape[2], mask_kind, q_offset, k_offset))

    def finalize(self, dq=None):
        import torch
        if dq is None:
            dq = torch.empty(self.q.shape, dtype=torch.float32, device=self.q.device)
        check(lib().ra_bwd_finalize(self._h, dq.data_ptr()))
        return dq

    def stats(self) -> dict:
        s = ra_stats()
        check(lib().ra_bwd_get_stats(self._h, C.byref(s)))
        return s.as_dict()

    def close(self) -> None:
        if self._h is not None:
            lib().ra_bwd_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def block_offsets(mask_kind: int, rank: int, block: int, q_len: int, kv_len: int) -> tuple[int, int]:
    """(q_offset, k_offset) of a block under a mask's layout (include/ra.h conventions)."""
    if mask_kind == RA_MASK_CAUSAL_CONTIGUOUS:
        return rank * q_len, block * kv_len
    if mask_kind in (RA_MASK_CAUSAL_STRIPED, RA_MASK_CAUSAL_ZIGZAG):
        return rank, block
    return 0, 0


class EmulatedRing:
    """Buffers and streams for ra_ring_lap_emulated: two receive buffers and a side stream."""

    def __init__(self, k_blocks, v_blocks, side_stream=None, valid=None):
        """``valid``: optional per-block counts of real keys (the rest of each block is padding;
        see ra_lap.kv_valid)."""
        import torch
        if len(k_blocks) != len(v_blocks) or not k_blocks:
            raise ValueError("need one K and one V tensor per block")
        ref = k_blocks[0]
        for t in list(k_blocks) + list(v_blocks):
            if t.shape != ref.shape or t.stride() != ref.stride() or not t.is_contiguous():
                raise ValueError("all blocks must be contiguous with the same shape")
        self.k_blocks = list(k_blocks)
        self.v_blocks = list(v_blocks)
        self.recv_k = [torch.empty_like(ref) for _ in range(2)]
        self.recv_v = [torch.empty_like(ref) for _ in range(2)]
        self.side = side_stream if side_stream is not None else torch.cuda.Stream(device=ref.device)
        P = len(k_blocks)
        self._kp = (C.c_void_p * P)(*[t.data_ptr() for t in self.k_blocks])
        self._vp = (C.c_void_p * P)(*[t.data_ptr() for t in self.v_blocks])
        self.block_bytes = ref.numel() * ref.element_size()
        self._valid = None
        if valid is not None:
            if len(valid) != P:
                raise ValueError("need one valid count per block")
            self._valid = (C.c_int32 * P)(*[int(x) for x in valid])

    def lap(self, q, rank: int, mask_kind: int, softmax_scale: float = 0.0, workspace=None,
            out=None, lse=None, poison: bool = False, stream=None, step_events=None):
        """One emulated lap (ra_ring_lap_emulated).  ``step_events``: optional list of 2P
        recorded torch.cuda.Event objects, re-recorded around each step's kernel."""
        import torch
        P = len(self.k_blocks)
        desc = desc_for(q, self.k_blocks[0], P, softmax_scale, stream)
        B, Hq, n, d = q.shape
        nbytes = workspace_bytes(desc)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty((B, Hq, n, d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
        lap = ra_lap()
        lap.k_blocks = C.cast(self._kp, C.POINTER(C.c_void_p))
        lap.v_blocks = C.cast(self._vp, C.POINTER(C.c_void_p))
        for i in range(2):
            lap.recv_k[i] = self.recv_k[i].data_ptr()
            lap.recv_v[i] = self.recv_v[i].data_ptr()
        lap.block_bytes = self.block_bytes
        lap.rank = rank
        lap.kv_len = self.k_blocks[0].shape[2]
        lap.mask_kind = mask_kind
        lap.poison = 1 if poison else 0
        lap.side_stream = int(self.side.cuda_stream)
        if step_events is not None:
            if len(step_events) != 2 * P:
                raise ValueError("need 2P events")
            evs = (C.c_void_p * (2 * P))(*[int(e.cuda_event) for e in step_events])
            lap.step_events = C.cast(evs, C.POINTER(C.c_void_p))
        if self._valid is not None:
            lap.kv_valid = C.cast(self._valid, C.POINTER(C.c_int32))
        st = ra_stats()
        check(lib().ra_ring_lap_emulated(C.byref(desc), q.data_ptr(), workspace.data_ptr(),
                                         C.byref(lap), out.data_ptr(), lse.data_ptr(), C.byref(st)))
        return out, lse, st.as_dict()
