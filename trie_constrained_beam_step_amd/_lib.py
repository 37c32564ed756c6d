"""ctypes declarations of the C ABI in include/gr.h (argument marshalling only).

The library runs inside the HIP runtime that PyTorch already loaded: torch is
imported before libgr.so so that libgr's dependency on libamdhip64.so.7
resolves to that same runtime (one runtime, one set of streams).  There is
no fallback: if libgr.so is missing or fails to load, importing raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GR_LIBRARY names another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("GR_LIBRARY") or os.path.join(HERE, "libgr.so")

GR_OK, GR_ERR_INVALID_ARG, GR_ERR_BAD_TRIE, GR_ERR_STATE = 0, 1, 2, 3
GR_ERR_OUT_OF_MEMORY, GR_ERR_HIP, GR_ERR_UNSUPPORTED = 4, 5, 6
GR_F32, GR_BF16 = 0, 1
GR_STATIC_SCRATCH_BYTES = 16 << 20  # the static workspace of gr_beam_step_static, per GPU


class BeamConfig(C.Structure):
    _fields_ = [("batch", C.c_int32), ("beam_width", C.c_int32), ("vocab", C.c_int32),
                ("max_steps", C.c_int32), ("eos_token", C.c_int32), ("logits_dtype", C.c_int32),
                ("logits_row_stride", C.c_int64)]


class BeamView(C.Structure):
    _fields_ = [("step", C.c_int32), ("batch", C.c_int32), ("beam_width", C.c_int32),
                ("vocab", C.c_int32), ("max_steps", C.c_int32),
                ("scores", C.c_void_p), ("nodes", C.c_void_p), ("finished", C.c_void_p),
                ("sequences", C.c_void_p), ("parents", C.c_void_p), ("tokens", C.c_void_p),
                ("lse", C.c_void_p)]


class StepIO(C.Structure):
    _fields_ = [("config", BeamConfig), ("trie", C.c_void_p), ("step", C.c_int32),
                ("live_bound", C.c_int32), ("temperature", C.c_float), ("seed", C.c_uint64),
                ("logits", C.c_void_p), ("scores", C.c_void_p), ("nodes", C.c_void_p),
                ("finished", C.c_void_p), ("sequences", C.c_void_p), ("scores_out", C.c_void_p),
                ("nodes_out", C.c_void_p), ("finished_out", C.c_void_p), ("sequences_out", C.c_void_p),
                ("parents_out", C.c_void_p), ("tokens_out", C.c_void_p), ("lse_out", C.c_void_p)]


class StepStats(C.Structure):
    _fields_ = [("rows_read", C.c_int64), ("candidates", C.c_int64), ("survivors", C.c_int64),
                ("slow_path_requests", C.c_int64), ("rescanned_rows", C.c_int64),
                ("fused_requests", C.c_int64)]


_VP = C.c_void_p
_I32, _I64, _SZ = C.c_int32, C.c_int64, C.c_size_t
_PP = C.POINTER(C.c_void_p)

# name -> (restype, argtypes); every function of include/gr.h
SIGNATURES = {
    "gr_trie_validate": (C.c_int, [_I32, _I32, _VP, _PP, _PP, _PP]),
    "gr_trie_build": (C.c_int, [_I32, _I32, _VP, _PP, _PP, _PP, _VP, C.POINTER(_VP)]),
    "gr_trie_info": (C.c_int, [_VP, C.POINTER(_I32), C.POINTER(_I32), _VP, _VP]),
    "gr_trie_free": (None, [_VP]),
    "gr_trie_densify": (C.c_int, [_VP, _I32, _I64, _VP, C.POINTER(_I64)]),
    "gr_beam_init": (C.c_int, [C.POINTER(BeamConfig), _VP, _VP, C.POINTER(_VP)]),
    "gr_beam_reset": (C.c_int, [_VP, _VP]),
    "gr_beam_step": (C.c_int, [_VP, _VP, _VP]),
    "gr_beam_rewind": (C.c_int, [_VP]),
    "gr_beam_search": (C.c_int, [_VP, C.POINTER(_VP), C.c_int32, _VP]),
    "gr_beam_step_static": (C.c_int, [C.POINTER(StepIO), _VP]),
    "gr_beam_backward": (C.c_int, [_VP, _VP, _VP, _VP, _VP, _VP]),
    "gr_beam_backward_scatter": (C.c_int, [_VP, C.c_int32, _VP, _VP, _VP, _VP, C.c_int64, _VP]),
    "gr_beam_view_get": (C.c_int, [_VP, C.POINTER(BeamView)]),
    "gr_beam_set_state": (C.c_int, [_VP, _I32, _VP, _VP, _VP, _VP, _VP]),
    "gr_beam_free": (None, [_VP]),
    "gr_beam_set_sampling": (C.c_int, [_VP, C.c_float, C.c_uint64]),
    "gr_beam_set_penalties": (C.c_int, [_VP, C.c_float, _I32, _VP, _I32, _VP]),
    "gr_beam_set_normalization": (C.c_int, [_VP, _I32, _I32, _I32]),
    "gr_beam_set_fused": (C.c_int, [_VP, _I32]),
    "gr_beam_timing_enable": (C.c_int, [_VP, _I32]),
    "gr_beam_timing_get": (C.c_int, [_VP, C.POINTER(C.c_double), C.POINTER(C.c_double),
                                     C.POINTER(_I64)]),
    "gr_beam_timing_reset": (C.c_int, [_VP]),
    "gr_beam_last_stats": (C.c_int, [_VP, C.POINTER(StepStats)]),
    "gr_probe_read": (C.c_int, [_VP, _SZ, _VP, _VP]),
    "gr_probe_copy": (C.c_int, [_VP, _VP, _SZ, _VP]),
    "gr_probe_draw_error": (C.c_int, [C.c_uint32, C.c_uint64, _VP, _VP]),
    "gr_draw_error_bound": (C.c_double, []),
    "gr_memcpy": (C.c_int, [_VP, _VP, _SZ, _VP]),
    "gr_status_string": (C.c_char_p, [C.c_int]),
    "gr_last_error": (C.c_char_p, []),
    "gr_version": (C.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libgr.so (after torch, see the module docstring)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m trie_constrained_beam_step_amd.build` "
            "(there is no CPU fallback)")
    import torch  # noqa: F401  -- loads the HIP runtime libgr must share
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process (should be one)."""
    out = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    out.add(line.split()[-1])
    except OSError:
        pass
    return sorted(out)
