"""ctypes loader of the HIP decode library (libld.so, built for gfx950).

There is no fallback: if the library is missing this raises, so nothing can
silently run a CPU path in its place.
"""
import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libld.so")

LD_OK = 0
LD_E_INVAL = -1
LD_E_RANGE = -2
LD_E_ARENA = -3
LD_E_HIP = -4
LD_E_NONFINITE = -5
LD_E_SCRATCH = -6
LD_STATIC_SCRATCH_BYTES = 32 << 20

LD_K_QKV, LD_K_ATTN, LD_K_WO, LD_K_W13, LD_K_W2, LD_K_CLS = range(6)

# every entry point declared in include/ld.h
EXPORTS = [
    "ld_arena_bytes", "ld_model_init", "ld_prefill", "ld_decode_step", "ld_decode_step_noalloc",
    "ld_generate", "ld_kv_reset",
    "ld_set_pos", "ld_get_pos", "ld_read_weights", "ld_weights_checksum", "ld_status", "ld_profile",
    "ld_profile_read", "ld_synth_prompt", "ld_model_free", "ld_strerror",
]


class LdConfig(C.Structure):
    _fields_ = [("dim", C.c_int32), ("n_layers", C.c_int32), ("n_heads", C.c_int32),
                ("hidden_dim", C.c_int32), ("vocab_size", C.c_int32), ("max_seq", C.c_int32),
                ("max_batch", C.c_int32), ("tied_classifier", C.c_int32),
                ("n_kv_heads", C.c_int32), ("weight_bf16", C.c_int32), ("max_pos", C.c_int32),
                ("rope_theta", C.c_double),
                ("norm_eps", C.c_double)]


class LdError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (what, strerror(code), code))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("HIP decode library not built: %s is missing (run __graft_entry__.build())"
                              % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, u64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_size_t
        L.ld_arena_bytes.argtypes = [C.POINTER(LdConfig), C.POINTER(sz)]
        L.ld_model_init.argtypes = [C.POINTER(LdConfig), u64, vp, sz, vp, C.POINTER(vp)]
        L.ld_prefill.argtypes = [vp, i32, i32, C.POINTER(i32), vp, vp, i32]
        L.ld_decode_step.argtypes = [vp, i32, vp, i32, vp, vp]
        L.ld_decode_step_noalloc.argtypes = [vp, i32, vp, i32, vp, vp]
        L.ld_generate.argtypes = [vp, i32, i32, vp, i32, vp, vp]
        L.ld_kv_reset.argtypes = [vp]
        L.ld_set_pos.argtypes = [vp, i32]
        L.ld_get_pos.argtypes = [vp, C.POINTER(i32)]
        L.ld_read_weights.argtypes = [vp, i64, u64, u64, C.POINTER(C.c_float)]
        L.ld_weights_checksum.argtypes = [vp, C.POINTER(u64)]
        L.ld_status.argtypes = [vp]
        L.ld_profile.argtypes = [vp, i32, i32]
        L.ld_profile_read.argtypes = [vp, i32, C.POINTER(C.c_double), C.POINTER(i64)]
        L.ld_synth_prompt.argtypes = [u64, u64, i32, i32, i32, C.POINTER(i32)]
        L.ld_model_free.argtypes = [vp]
        L.ld_model_free.restype = None
        L.ld_strerror.argtypes = [C.c_int]
        L.ld_strerror.restype = C.c_char_p
        for name in EXPORTS:
            if name not in ("ld_model_free", "ld_strerror"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def strerror(code):
    try:
        return lib().ld_strerror(code).decode()
    except ImportError:
        return "error %d" % code


def check(code, what):
    if code != LD_OK:
        raise LdError(code, what)
    return code
