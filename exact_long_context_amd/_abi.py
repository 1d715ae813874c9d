"""ctypes declarations of include/ra.h (argument marshalling only).

Every function of the C ABI is exposed under its C name with its C signature;
device pointers are passed as Python ints.  Loading fails loudly when the
library has not been built: there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librocring.so")

RA_OK = 0
RA_E_INVALID = -1
RA_E_UNSUPPORTED = -2
RA_E_STATE = -3
RA_E_HIP = -4

RA_MASK_NONE = 0
RA_MASK_CAUSAL_CONTIGUOUS = 1
RA_MASK_CAUSAL_STRIPED = 2
RA_MASK_CAUSAL_ZIGZAG = 3
RA_MERGE_MAX_PARTS = 64
RA_DECODE_NOALLOC_MAX_BYTES = 64 << 20

RA_DTYPE_BF16 = 0
RA_DTYPE_F32 = 1

RA_TILE_EMPTY = 0
RA_TILE_FULL = 1
RA_TILE_PARTIAL = 2


class ra_desc(C.Structure):
    _fields_ = [
        ("batch", C.c_int32),
        ("q_heads", C.c_int32),
        ("kv_heads", C.c_int32),
        ("q_len", C.c_int32),
        ("head_dim", C.c_int32),
        ("dtype", C.c_int32),
        ("softmax_scale", C.c_float),
        ("ring_size", C.c_int32),
        ("q_strides", C.c_int64 * 3),
        ("kv_strides", C.c_int64 * 3),
        ("stream", C.c_void_p),
    ]


class ra_stats(C.Structure):
    _fields_ = [
        ("live_pairs", C.c_int64),
        ("tiles_full", C.c_int64),
        ("tiles_partial", C.c_int64),
        ("tiles_empty", C.c_int64),
        ("blocks_run", C.c_int64),
        ("blocks_skipped", C.c_int64),
        ("tile_q", C.c_int32),
        ("tile_k", C.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class ra_lap(C.Structure):
    _fields_ = [
        ("k_blocks", C.POINTER(C.c_void_p)),
        ("v_blocks", C.POINTER(C.c_void_p)),
        ("recv_k", C.c_void_p * 2),
        ("recv_v", C.c_void_p * 2),
        ("block_bytes", C.c_size_t),
        ("rank", C.c_int32),
        ("kv_len", C.c_int32),
        ("mask_kind", C.c_int32),
        ("poison", C.c_int32),
        ("side_stream", C.c_void_p),
        ("step_events", C.POINTER(C.c_void_p)),
        ("kv_valid", C.POINTER(C.c_int32)),
    ]


# name -> (restype, argtypes); the order and types follow include/ra.h
SIGNATURES = {
    "ra_workspace_bytes": (C.c_size_t, [C.POINTER(ra_desc)]),
    "ra_workspace_layout": (C.c_int, [C.POINTER(ra_desc), C.POINTER(C.c_size_t),
                                      C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "ra_state_init": (C.c_int, [C.POINTER(ra_desc), C.c_void_p, C.c_void_p, C.POINTER(C.c_void_p)]),
    "ra_state_resume": (C.c_int, [C.POINTER(ra_desc), C.c_void_p, C.c_void_p, C.POINTER(C.c_void_p)]),
    "ra_block_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                C.c_int64, C.c_int64]),
    "ra_finalize": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "ra_decode_workspace_bytes": (C.c_size_t, [C.POINTER(ra_desc), C.c_int32]),
    "ra_decode_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                 C.c_int64, C.c_int64, C.c_void_p, C.c_size_t]),
    "ra_decode_step_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                         C.c_int64, C.c_int64]),
    "ra_bwd_workspace_bytes": (C.c_size_t, [C.POINTER(ra_desc)]),
    "ra_bwd_init": (C.c_int, [C.POINTER(ra_desc), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.POINTER(C.c_void_p)]),
    "ra_bwd_block_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_int32, C.c_int32, C.c_int64, C.c_int64]),
    "ra_bwd_finalize": (C.c_int, [C.c_void_p, C.c_void_p]),
    "ra_bwd_get_stats": (C.c_int, [C.c_void_p, C.POINTER(ra_stats)]),
    "ra_bwd_destroy": (C.c_int, [C.c_void_p]),
    "ra_merge_states": (C.c_int, [C.POINTER(ra_desc), C.c_int32, C.POINTER(C.c_void_p), C.c_void_p,
                                  C.c_void_p, C.c_void_p]),
    "ra_state_destroy": (C.c_int, [C.c_void_p]),
    "ra_get_stats": (C.c_int, [C.c_void_p, C.POINTER(ra_stats)]),
    "ra_state_set_debug_counters": (C.c_int, [C.c_void_p, C.c_void_p]),
    "ra_plan_block": (C.c_int, [C.POINTER(ra_desc), C.c_int32, C.c_int32, C.c_int64, C.c_int64,
                                C.POINTER(ra_stats)]),
    "ra_tile_classes": (C.c_int, [C.POINTER(ra_desc), C.c_int32, C.c_int32, C.c_int64, C.c_int64,
                                  C.c_void_p, C.c_size_t]),
    "ra_ring_lap_emulated": (C.c_int, [C.POINTER(ra_desc), C.c_void_p, C.c_void_p, C.POINTER(ra_lap),
                                       C.c_void_p, C.c_void_p, C.POINTER(ra_stats)]),
    "ra_status_string": (C.c_char_p, [C.c_int]),
    "ra_version": (C.c_int, []),
}


class RaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def _hip_runtimes_mapped() -> set:
    """Distinct HIP runtime files mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {os.path.realpath(ln.split()[-1]) for ln in f if "libamdhip64" in ln}
    except OSError:
        return set()


def load(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python exact_long_context_amd/build.py` "
            "(there is no fallback implementation)")
    # One HIP runtime per process: torch ships its own libamdhip64 (soname
    # libamdhip64.so.7).  Loading torch first lets the library's NEEDED entry bind to
    # that copy; loading the library first would map /opt/rocm's copy as well, and
    # torch's streams would then be handed to a different runtime.
    import torch  # noqa: F401
    lib = C.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped in this process: {sorted(runtimes)}; "
                          "import torch before anything that loads /opt/rocm's libamdhip64")
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def check(code: int) -> int:
    if code != RA_OK:
        raise RaError(code, lib().ra_status_string(code).decode())
    return code
