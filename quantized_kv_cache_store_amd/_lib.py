"""ctypes loader for libkvq.so and the C declarations of include/kvq.h."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

c_i32 = ctypes.c_int32
c_u32 = ctypes.c_uint32
c_size = ctypes.c_size_t
c_vp = ctypes.c_void_p
c_f = ctypes.c_float

HAD_INT4, Q4_0, Q6_0, ASYM_INT4_G32, Q8_0 = 0, 1, 2, 3, 4
LAYOUT_IDS = {"had_int4": HAD_INT4, "q4_0": Q4_0, "q6_0": Q6_0, "asym_int4_g32": ASYM_INT4_G32, "q8_0": Q8_0}
PREFILL_NO_CAUSAL_SKIP = 1

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP launch failure"}


class KvqCacheDesc(ctypes.Structure):
    _fields_ = [
        ("layout", c_i32), ("head_dim", c_i32), ("num_kv_heads", c_i32), ("page_size", c_i32),
        ("num_pages", c_i32), ("n_recent", c_i32), ("max_batch", c_i32), ("reserved", c_i32),
        ("k_payload", c_vp), ("v_payload", c_vp), ("k_scale", c_vp), ("v_scale", c_vp),
        ("k_recent", c_vp), ("v_recent", c_vp),
    ]


P = ctypes.POINTER(KvqCacheDesc)

# name -> (restype, argtypes); mirrors include/kvq.h
SIGNATURES = {
    "kvq_payload_bytes": (c_size, [c_i32, c_i32]),
    "kvq_scale_bytes": (c_size, [c_i32, c_i32]),
    "kvq_store": (c_i32, [P, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "kvq_debug_stream_read": (c_i32, [c_i32, c_vp, c_vp, c_vp]),
    "kvq_store_chunk": (c_i32, [P, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp]),
    "kvq_prefill_full_then_store": (c_i32, [P, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_f, c_i32, c_vp,
                                            c_vp, c_i32, c_i32, c_vp, c_size, c_vp]),
    "kvq_decode_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "kvq_attend_decode": (c_i32, [P, c_vp, c_vp, c_i32, c_i32, c_f, c_vp, c_i32, c_vp, c_i32, c_i32,
                                  c_vp, c_size, c_vp]),
    "kvq_attend_decode_float_q": (c_i32, [P, c_vp, c_vp, c_i32, c_i32, c_f, c_vp, c_i32, c_vp, c_i32, c_i32,
                                          c_vp, c_size, c_vp]),
    "kvq_decode_split": (c_i32, [P, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "kvq_decode_split_lengths": (c_i32, [P, c_i32, c_i32, c_vp, c_i32, c_i32, c_vp, c_vp]),
    "kvq_attend_decode_noalloc": (c_i32, [P, c_vp, c_vp, c_i32, c_i32, c_f, c_vp, c_i32, c_vp, c_i32, c_i32,
                                          c_vp]),
    "kvq_attend_decode_partial": (c_i32, [P, c_vp, c_i32, c_i32, c_f, c_vp, c_i32, c_vp, c_i32, c_i32,
                                          c_vp, c_size, c_vp]),
    "kvq_attend_decode_reduce": (c_i32, [P, c_vp, c_i32, c_i32, c_vp, c_i32, c_i32, c_vp, c_size, c_vp]),
    "kvq_prefill_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "kvq_attend_prefill_causal": (c_i32, [P, c_vp, c_vp, c_i32, c_i32, c_i32, c_f, c_i32, c_vp, c_vp, c_i32,
                                          c_vp, c_i32, c_u32, c_vp, c_size, c_vp]),
    "kvq_debug_quantize_q": (c_i32, [c_i32, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "kvq_debug_qk_i32": (c_i32, [P, c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_vp, c_vp, c_size, c_vp]),
    "kvq_status_string": (ctypes.c_char_p, [c_i32]),
    "kvq_last_error": (ctypes.c_char_p, []),
}

_lib = None


class KvqError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


def load():
    """Load libkvq.so (built in-tree); raises if it is missing -- there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn_name, status):
    if status != 0:
        msg = load().kvq_last_error().decode(errors="replace")
        raise KvqError(fn_name, status, msg)
