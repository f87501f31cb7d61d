"""ctypes binding of ``libw4a16.so`` (the C ABI in include/w4a16.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every computation happens in the library's kernels.  If the library
is missing, every call raises -- there is no fallback path.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16.so")

_c = ctypes
_i32, _i64, _p = _c.c_int32, _c.c_int64, _c.c_void_p

# name -> (restype, argtypes); mirrors include/w4a16.h
SIGNATURES = {
    "w4a16_status_string": (_c.c_char_p, [_c.c_int]),
    "w4a16_version": (_c.c_int, []),
    "w4a16_set_timing_events": (_c.c_int, [_p, _p]),
    "w4a16_repacked_bytes": (_i64, [_i64, _i64, _i32, _i32]),
    "w4a16_make_perm": (_c.c_int, [_p, _i64, _i32, _p, _p, _p]),
    "w4a16_quantize_rtn": (_c.c_int, [_p, _p, _p, _i64, _i64, _i32, _p, _p, _p, _p]),
    "w4a16_repack": (_c.c_int, [_p, _p, _p, _p, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p]),
    "w4a16_workspace_bytes": (_i64, [_i64, _i64, _i64, _i32]),
    "w4a16_gemm": (_c.c_int, [_p, _p, _p, _p, _p, _i32, _p, _i64, _i64, _i64, _i32, _p, _i64, _p]),
    "w4a16_gemm_xscale": (_c.c_int, [_p, _p, _p, _p, _p, _p, _i32, _p, _i64, _i64, _i64, _i32, _p,
                                     _i64, _p]),
    "w4a16_dequant": (_c.c_int, [_p, _p, _p, _i64, _i64, _i32, _i32, _p, _p]),
    "w4a16_repacked_bytes_bits": (_i64, [_i64, _i64, _i32, _i32, _i32]),
    "w4a16_quantize_rtn_bits": (_c.c_int, [_p, _p, _p, _i64, _i64, _i32, _i32, _p, _p, _p, _p]),
    "w4a16_repack_bits": (_c.c_int, [_p, _p, _p, _p, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _p,
                                     _p]),
    "w4a16_gemm_bits": (_c.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _p, _i64, _i64, _i64, _i32,
                                   _p, _i64, _p]),
    "w4a16_dequant_bits": (_c.c_int, [_p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p, _p]),
    "nf4_codebook": (_c.c_int, [_p]),
    "nf4_quantize": (_c.c_int, [_p, _i64, _i64, _i32, _p, _p, _p, _p]),
    "nf4_workspace_bytes": (_i64, [_i64, _i64, _i64, _i32]),
    "nf4_gemm": (_c.c_int, [_p, _p, _p, _p, _i32, _p, _i64, _i64, _i64, _i32, _p, _i64, _p]),
    "nf4_dequant": (_c.c_int, [_p, _p, _p, _i64, _i64, _i32, _i32, _p, _p]),
    "w4a16_gemm_plan": (_c.c_int, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _p,
                                   _i64, _p]),
    "nf4_gemm_plan": (_c.c_int, [_i64, _i64, _i64, _i32, _i32, _i32, _p, _i64, _p]),
    "nf4_gemm_repacked_plan": (_c.c_int, [_i64, _i64, _i64, _i32, _i32, _i32, _p, _i64, _p]),
    "nf4_repacked_bytes": (_i64, [_i64, _i64, _i32]),
    "nf4_repack": (_c.c_int, [_p, _i64, _i64, _i32, _p, _p]),
    "nf4_gemm_repacked": (_c.c_int, [_p, _p, _p, _p, _i32, _p, _i64, _i64, _i64, _i32, _p, _i64,
                                     _p]),
    "w4a16_stream_read": (_c.c_int, [_p, _i64, _i32, _p, _p]),
    "w4a16_gemm_noalloc": (_c.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _p, _i64, _i64, _i64,
                                      _i32, _p]),
}

_lib = None


def load():
    """Load the library (once); raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libw4a16.so not built (expected at %s); run __graft_entry__.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def lib():
    return load()


class W4A16Error(RuntimeError):
    pass


def check(status, what):
    if status != 0:
        msg = load().w4a16_status_string(status).decode()
        raise W4A16Error("%s failed: status %d (%s)" % (what, status, msg))
