"""ctypes binding of libgptoss_attn.so.

Argument marshalling only: every step of the computation runs in the HIP
library.  torch supplies device memory and the current HIP stream.  There is
no fallback: if the library is missing or a call fails, an exception is
raised.
"""

import ctypes
import os

from .build import LIB_PATH

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "HIP"}

EXPORTS = [
    "gptoss_attn_abi_version", "gptoss_attn_last_error", "gptoss_attn_fwd",
    "gptoss_attn_bwd_workspace_size", "gptoss_attn_bwd",
    "gptoss_attn_decode_workspace_size", "gptoss_attn_decode", "gptoss_attn_decode_noalloc",
    "gptoss_attn_decode_paged",
    "gptoss_attn_fwd_varlen", "gptoss_attn_bwd_varlen_workspace_size", "gptoss_attn_bwd_varlen",
    "gptoss_attn_rope_table", "gptoss_attn_rope_rows", "gptoss_attn_fwd_rope", "gptoss_attn_decode_rope",
    "gptoss_attn_bwd_rope_workspace_size", "gptoss_attn_bwd_rope",
]

_lib = None

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_double = ctypes.c_double


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load(path=None):
    """Load (once) and return the ctypes library handle.  GPTOSS_ATTN_LIBRARY,
    when set, names another build of the same ABI to load instead (the CPU
    tests use it for a sanitizer build of the host layer)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or os.environ.get("GPTOSS_ATTN_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run "
                           "`python -m attention_attn_fwd_amd.build` first")
    lib = ctypes.CDLL(path)
    lib.gptoss_attn_abi_version.restype = c_int
    lib.gptoss_attn_abi_version.argtypes = []
    lib.gptoss_attn_last_error.restype = ctypes.c_char_p
    lib.gptoss_attn_last_error.argtypes = []
    lib.gptoss_attn_fwd.restype = c_int
    lib.gptoss_attn_fwd.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                    c_int, c_int, c_float, c_void_p, c_void_p, c_void_p]
    lib.gptoss_attn_bwd_workspace_size.restype = c_size_t
    lib.gptoss_attn_bwd_workspace_size.argtypes = [c_int] * 6
    lib.gptoss_attn_bwd.restype = c_int
    lib.gptoss_attn_bwd.argtypes = [c_void_p] * 7 + [c_int] * 6 + [c_float] + [c_void_p] * 5 + \
        [c_size_t, c_void_p]
    lib.gptoss_attn_decode_workspace_size.restype = c_size_t
    lib.gptoss_attn_decode_workspace_size.argtypes = [c_int] * 6
    lib.gptoss_attn_decode.restype = c_int
    lib.gptoss_attn_decode.argtypes = [c_void_p] * 5 + [c_int] * 6 + [c_float] + [c_void_p] * 3 + \
        [c_size_t, c_void_p]
    lib.gptoss_attn_decode_noalloc.restype = c_int
    lib.gptoss_attn_decode_noalloc.argtypes = [c_void_p] * 5 + [c_int] * 6 + [c_float] + [c_void_p] * 3
    lib.gptoss_attn_decode_paged.restype = c_int
    lib.gptoss_attn_decode_paged.argtypes = [c_void_p] * 6 + [c_int] * 9 + [c_float] + [c_void_p] * 3 + \
        [c_size_t, c_void_p]
    lib.gptoss_attn_fwd_varlen.restype = c_int
    lib.gptoss_attn_fwd_varlen.argtypes = [c_void_p] * 5 + [c_int] * 7 + [c_float] + [c_void_p] * 3
    lib.gptoss_attn_bwd_varlen_workspace_size.restype = c_size_t
    lib.gptoss_attn_bwd_varlen_workspace_size.argtypes = [c_int] * 4
    lib.gptoss_attn_bwd_varlen.restype = c_int
    lib.gptoss_attn_bwd_varlen.argtypes = [c_void_p] * 8 + [c_int] * 7 + [c_float] + [c_void_p] * 5 + \
        [c_size_t, c_void_p]
    lib.gptoss_attn_rope_table.restype = c_int
    lib.gptoss_attn_rope_table.argtypes = [c_void_p, c_int, c_int] + [c_double] * 5 + [c_void_p]
    lib.gptoss_attn_rope_rows.restype = c_int
    lib.gptoss_attn_rope_rows.argtypes = [c_void_p] * 3 + [c_int] * 3 + [c_void_p, c_int, c_int, c_void_p]
    lib.gptoss_attn_fwd_rope.restype = c_int
    lib.gptoss_attn_fwd_rope.argtypes = [c_void_p] * 5 + [c_int] * 7 + [c_float] + [c_void_p] * 4
    lib.gptoss_attn_decode_rope.restype = c_int
    lib.gptoss_attn_decode_rope.argtypes = [c_void_p] * 6 + [c_int] * 7 + [c_float] + [c_void_p] * 3 + \
        [c_size_t, c_void_p]
    lib.gptoss_attn_bwd_rope_workspace_size.restype = c_size_t
    lib.gptoss_attn_bwd_rope_workspace_size.argtypes = [c_int] * 5
    lib.gptoss_attn_bwd_rope.restype = c_int
    lib.gptoss_attn_bwd_rope.argtypes = [c_void_p] * 5 + [c_int] + [c_void_p] * 3 + [c_int] * 6 + [c_float] + \
        [c_void_p] * 5 + [c_size_t, c_void_p]
    if path in (LIB_PATH, os.environ.get("GPTOSS_ATTN_LIBRARY")):
        _lib = lib
    return lib


def check(status, lib=None):
    if status != OK:
        lib = lib or load()
        raise AttnError(status, lib.gptoss_attn_last_error().decode())
