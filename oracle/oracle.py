"""ctypes binding of the CPU oracle -- TEST INFRASTRUCTURE, not part of the product.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
module.  It loads oracle/liboracle.so (plain single-threaded C, fp32 storage,
fp64 accumulation) and never touches the HIP library.
"""
import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32P = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


class OrConfig(C.Structure):
    _fields_ = [("dim", C.c_int32), ("n_layers", C.c_int32), ("n_heads", C.c_int32),
                ("hidden_dim", C.c_int32), ("vocab_size", C.c_int32), ("max_seq", C.c_int32),
                ("tied", C.c_int32), ("n_kv_heads", C.c_int32), ("weight_bf16", C.c_int32),
                ("max_pos", C.c_int32), ("rope_theta", C.c_double), ("norm_eps", C.c_double)]


def lib(path=None):
    """Load liboracle.so (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _bind(C.CDLL(path))
    if _lib is None:
        override = os.environ.get("LD_ORACLE_LIB")   # a planted-mistake build, for the pin tests
        if override:
            _lib = _bind(C.CDLL(override))
            return _lib
        if not os.path.exists(_LIB_PATH):
            from . import _build
            _build.build()
        _lib = _bind(C.CDLL(_LIB_PATH))
    return _lib


def _bind(L):
    L.or_rmsnorm.argtypes = [F32P, F32P, F32P, C.c_int, C.c_double]
    L.or_matvec.argtypes = [F32P, F32P, F32P, C.c_int, C.c_int]
    L.or_rope_table.argtypes = [F32P, F32P, C.c_int, C.c_int, C.c_double]
    L.or_rope.argtypes = [F32P, C.c_int, C.c_int, F32P, F32P]
    L.or_softmax.argtypes = [F64P, C.c_int]
    L.or_attention.argtypes = [F32P, F32P, F32P, F32P, C.c_int, C.c_int, C.c_int, C.c_int]
    L.or_swiglu.argtypes = [F32P, F32P, F32P, C.c_int]
    L.or_residual_add.argtypes = [F32P, F32P, C.c_int]
    L.or_argmax.argtypes = [F32P, C.c_int]
    L.or_argmax.restype = C.c_int
    L.or_bf16_round.argtypes = [C.c_float]
    L.or_bf16_round.restype = C.c_float
    L.or_model_create.argtypes = [C.POINTER(OrConfig), C.c_uint64, C.c_int]
    L.or_model_create.restype = C.c_void_p
    L.or_model_free.argtypes = [C.c_void_p]
    L.or_model_tensor.argtypes = [C.c_void_p, C.c_int64, C.POINTER(C.c_size_t)]
    L.or_model_tensor.restype = C.POINTER(C.c_float)
    L.or_state_create.argtypes = [C.c_void_p]
    L.or_state_create.restype = C.c_void_p
    L.or_state_free.argtypes = [C.c_void_p]
    L.or_forward.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, F32P]
    L.or_forward.restype = C.c_int
    L.or_forward_recompute.argtypes = [C.c_void_p, I32P, C.c_int, F32P]
    L.or_forward_recompute.restype = C.c_int
    L.synth_normal.argtypes = [F32P, C.c_uint64, C.c_uint64, C.c_uint64, C.c_size_t, C.c_double]
    L.synth_normal_mt.argtypes = [F32P, C.c_uint64, C.c_uint64, C.c_uint64, C.c_size_t,
                                  C.c_double, C.c_int]
    L.synth_prompt.argtypes = [I32P, C.c_uint64, C.c_uint64, C.c_size_t, C.c_int32, C.c_int32]
    L.synth_u64.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64]
    L.synth_u64.restype = C.c_uint64
    return L


# ------------------------------------------------------------------ ops ----
def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def rmsnorm(x, gain, eps, L=None):
    L = L or lib()
    x = _f32(x)
    out = np.empty_like(x)
    L.or_rmsnorm(out, x, _f32(gain), x.size, eps)
    return out


def matvec(w, x, L=None):
    L = L or lib()
    w = _f32(w)
    out = np.empty(w.shape[0], np.float32)
    L.or_matvec(out, w, _f32(x), w.shape[0], w.shape[1])
    return out


def rope_table(max_seq, head_dim, theta, L=None):
    L = L or lib()
    c = np.empty((max_seq, head_dim // 2), np.float32)
    s = np.empty_like(c)
    L.or_rope_table(c, s, max_seq, head_dim, theta)
    return c, s


def rope(v, head_dim, cos_row, sin_row, L=None):
    L = L or lib()
    v = _f32(v).copy()
    L.or_rope(v, v.size, head_dim, _f32(cos_row), _f32(sin_row))
    return v


def softmax(s, L=None):
    L = L or lib()
    s = np.ascontiguousarray(s, dtype=np.float64).copy()
    L.or_softmax(s, s.size)
    return s


def attention(q, k_rows, v_rows, n_heads, n_kv_heads=None, L=None):
    """k_rows, v_rows: [n_pos][n_kv_heads * head_dim] (n_kv_heads defaults to n_heads)"""
    L = L or lib()
    q = _f32(q)
    k_rows = _f32(k_rows)
    out = np.empty_like(q)
    L.or_attention(out, q, k_rows, _f32(v_rows), k_rows.shape[0], q.size, n_heads,
                   n_heads if n_kv_heads is None else n_kv_heads)
    return out


def swiglu(h1, h3, L=None):
    L = L or lib()
    h1 = _f32(h1)
    out = np.empty_like(h1)
    L.or_swiglu(out, h1, _f32(h3), h1.size)
    return out


def residual_add(x, t, L=None):
    L = L or lib()
    x = _f32(x).copy()
    L.or_residual_add(x, _f32(t), x.size)
    return x


def argmax(v, L=None):
    L = L or lib()
    v = _f32(v)
    return int(L.or_argmax(v, v.size))


def bf16_round(x, L=None):
    """Each element rounded to the nearest bfloat16 (ties to even), as float32."""
    L = L or lib()
    x = _f32(x)
    out = np.empty_like(x)
    flat, src = out.reshape(-1), x.reshape(-1)
    for i in range(src.size):
        flat[i] = L.or_bf16_round(float(src[i]))
    return out


def synth_normal(seed, stream, start, n, std=0.02, nthreads=1, L=None):
    L = L or lib()
    out = np.empty(n, np.float32)
    if nthreads > 1:
        L.synth_normal_mt(out, seed, stream, start, n, std, nthreads)
    else:
        L.synth_normal(out, seed, stream, start, n, std)
    return out


def synth_prompt(seed, seq, n, lo=3, hi=32000, L=None):
    L = L or lib()
    out = np.empty(n, np.int32)
    L.synth_prompt(out, seed, seq, n, lo, hi)
    return out


# ---------------------------------------------------------------- model ----
class OracleModel:
    """One model instance: weights drawn from `seed` (std 0.02, gains 1.0).

    cfg is any object with attributes dim, n_layers, n_heads, hidden_dim,
    vocab_size, max_seq, tied, rope_theta, norm_eps (and optionally n_kv_heads,
    weight_bf16, max_pos).
    """

    def __init__(self, cfg, seed, nthreads=8, L=None):
        self.L = L or lib()
        self.cfg = cfg
        c = OrConfig(cfg.dim, cfg.n_layers, cfg.n_heads, cfg.hidden_dim, cfg.vocab_size,
                     cfg.max_seq, int(cfg.tied), int(getattr(cfg, "n_kv_heads", 0) or 0),
                     int(bool(getattr(cfg, "weight_bf16", False))),
                     int(getattr(cfg, "max_pos", 0) or 0),
                     float(cfg.rope_theta), float(cfg.norm_eps))
        self._h = self.L.or_model_create(C.byref(c), seed, nthreads)
        if not self._h:
            raise ValueError("oracle rejected config %r" % (cfg,))

    def close(self):
        if self._h:
            self.L.or_model_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def tensor(self, tid):
        """Writable numpy view of a weight tensor (synth stream id) or a gain (negative id)."""
        n = C.c_size_t(0)
        p = self.L.or_model_tensor(self._h, tid, C.byref(n))
        if not p:
            raise KeyError(tid)
        return np.ctypeslib.as_array(p, shape=(n.value,))

    def new_state(self):
        return OracleState(self)

    def forward(self, state, token, pos, logits=None):
        if logits is None:
            logits = np.empty(self.cfg.vocab_size, np.float32)
        r = self.L.or_forward(self._h, state._h, int(token), int(pos), logits)
        return r, logits

    def recompute(self, tokens):
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        logits = np.empty(self.cfg.vocab_size, np.float32)
        r = self.L.or_forward_recompute(self._h, tokens, tokens.size, logits)
        return r, logits


class OracleState:
    def __init__(self, model):
        self.m = model
        self._h = model.L.or_state_create(model._h)
        if not self._h:
            raise MemoryError("oracle state")

    def __del__(self):
        try:
            if self._h:
                self.m.L.or_state_free(self._h)
                self._h = None
        except Exception:
            pass


def run_sequence(model, prompt, n_positions, feed=None, keep_logits=None, sub_idx=None):
    """Greedy run of one sequence through positions 0..n_positions-1.

    Position p < len(prompt) consumes prompt[p]; later positions consume the
    previous position's greedy token, or feed[p] when `feed` (teacher tokens,
    indexed by position) is given.  Returns (tokens_in[n_positions],
    greedy_out[n_positions], top1_val, top2_val, kept) where `kept` maps each
    position in `keep_logits` to its full logits vector.  With `sub_idx` (logit
    indices), kept["sub"] is also an [n_positions, len(sub_idx)] array of those
    logits at every position.
    """
    st = model.new_state()
    V = model.cfg.vocab_size
    tin = np.zeros(n_positions, np.int32)
    tout = np.zeros(n_positions, np.int32)
    top1 = np.zeros(n_positions, np.float32)
    top2 = np.zeros(n_positions, np.float32)
    kept = {}
    keep = set(keep_logits or ())
    logits = np.empty(V, np.float32)
    sub = None
    if sub_idx is not None:
        sub_idx = np.asarray(sub_idx, np.int64)
        sub = np.zeros((n_positions, sub_idx.size), np.float32)
        kept["sub"] = sub
    nxt = None
    for p in range(n_positions):
        if p < len(prompt):
            t = int(prompt[p])
        elif feed is not None:
            t = int(feed[p])
        else:
            t = nxt
        tin[p] = t
        r, _ = model.forward(st, t, p, logits)
        if r < 0:
            raise FloatingPointError("oracle produced a non-finite logit at position %d" % p)
        tout[p] = r
        top1[p] = logits[r]
        masked = logits.copy()
        masked[r] = -np.inf
        top2[p] = masked.max()
        if p in keep:
            kept[p] = logits.copy()
        if sub is not None:
            sub[p] = logits[sub_idx]
        nxt = r
    return tin, tout, top1, top2, kept
