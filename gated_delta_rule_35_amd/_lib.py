"""ctypes view of libagnes_gdn.so (the C ABI declared in include/agnes_gdn.h)."""
import atexit
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libagnes_gdn.so")

c_int, c_int64, c_float, c_size_t, c_void_p = (ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                              ctypes.c_size_t, ctypes.c_void_p)

# name -> (restype, argtypes), in the order of include/agnes_gdn.h
SIGNATURES = {
    "agnes_gdn_conv": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int, c_void_p, c_void_p,
                               c_void_p, c_int, c_int64, c_int, c_int, c_void_p, c_int, c_int,
                               c_float, c_void_p]),
    "agnes_gdn_prefill_workspace_size": (c_size_t, [c_int, c_int64, c_int, c_int, c_int, c_int]),
    "agnes_gdn_prefill_chunked": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int64, c_int64,
                                          c_void_p, c_void_p, c_void_p, c_int, c_int64, c_int, c_int,
                                          c_int, c_float, c_void_p, c_void_p, c_void_p, c_int,
                                          c_void_p, c_size_t, c_void_p]),
    "agnes_gdn_prefill_fused": (c_int, [c_void_p, c_int64, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_int, c_int64, c_int, c_int, c_int, c_float,
                                        c_float, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_size_t,
                                        c_void_p]),
    "agnes_gdn_decode_step": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int64, c_int64,
                                      c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_float,
                                      c_void_p, c_void_p, c_int, c_void_p]),
    "agnes_gdn_gated_rmsnorm": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_float,
                                        c_int64, c_int, c_void_p, c_int, c_void_p]),
    "agnes_gdn_decode_fused": (c_int, [c_void_p, c_int64, c_int, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_int, c_int, c_int, c_int, c_int, c_float, c_float, c_float,
                                       c_void_p, c_void_p, c_int, c_void_p]),
    "agnes_gdn_layer_prefill_workspace_size": (c_size_t, [c_int, c_int64, c_int, c_int, c_int]),
    "agnes_gdn_layer_prefill": (c_int, [c_void_p, c_int64, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_int, c_int64, c_int, c_int, c_int, c_float,
                                        c_float, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_float,
                                        c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "agnes_gdn_layer_prefill_noalloc": (c_int, [c_void_p, c_int64, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                                c_void_p, c_void_p, c_int, c_int64, c_int, c_int, c_int, c_float,
                                                c_float, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_float,
                                                c_void_p, c_void_p, c_int, c_void_p]),
    "agnes_attn_prefill_workspace_size": (c_size_t, [c_int, c_int64]),
    "agnes_attn_prefill": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                   c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_int64, c_int,
                                   c_int, c_int, c_int, c_float, c_float, c_float, c_void_p, c_int64,
                                   c_void_p, c_int64, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "agnes_attn_decode_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int64]),
    "agnes_attn_decode": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                  c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_void_p,
                                  c_int, c_int, c_int, c_int, c_int, c_float, c_float, c_float, c_void_p, c_int,
                                  c_void_p, c_size_t, c_void_p]),
    "agnes_gdn_workspace_status": (c_int, [c_void_p, c_void_p, c_void_p]),
    "agnes_gdn_set_wait_limit": (c_int, [ctypes.c_uint32]),
    "agnes_gdn_set_prefill_stages": (c_int, [c_void_p, c_int]),
    "agnes_gdn_ceiling_rmw_stream": (c_int, [c_void_p, c_size_t, c_void_p]),
    "agnes_gdn_ceiling_mfma": (c_int, [c_void_p, c_int, c_int, c_void_p]),
    "agnes_gdn_release": (c_int, []),
    "agnes_gdn_status_string": (ctypes.c_char_p, [c_int]),
    "agnes_gdn_last_hip_error": (c_int, []),
    "agnes_gdn_version": (ctypes.c_char_p, []),
}

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
WS_WAIT_LDS, WS_WAIT_EXCHANGE, WS_WAIT_ROLE, WS_RANGE = 1, 2, 4, 8
F32, BF16 = 0, 1

_lib = None


def load():
    """Load the built library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_35_amd.build` "
                "(the layer has no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        # release the library's side streams and events while the HIP runtime (and any profiler
        # attached to it) is still whole: interpreter exit handlers run before the C runtime's
        atexit.register(_release_at_exit)
    return _lib


def _release_at_exit():
    try:
        _lib.agnes_gdn_release()
    except Exception:  # pragma: no cover - nothing to do at exit
        pass
