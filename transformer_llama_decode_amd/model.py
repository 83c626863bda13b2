"""Python face of the decode library: argument marshalling over the C ABI.

PyTorch only provides device memory (one arena tensor plus caller-owned output
tensors) and the stream; every step of the forward pass runs in the library's
HIP kernels.
"""
import ctypes as C

import numpy as np

from ._lib import LdConfig, check, lib, LD_OK
from .configs import ModelConfig


def _cfg_struct(cfg: ModelConfig):
    return LdConfig(cfg.dim, cfg.n_layers, cfg.n_heads, cfg.hidden_dim, cfg.vocab_size, cfg.max_seq,
                    cfg.max_batch, int(cfg.tied), int(cfg.n_kv_heads or 0), int(bool(cfg.weight_bf16)),
                    int(cfg.max_pos or 0), float(cfg.rope_theta), float(cfg.norm_eps))


def arena_bytes(cfg: ModelConfig) -> int:
    n = C.c_size_t()
    check(lib().ld_arena_bytes(C.byref(_cfg_struct(cfg)), C.byref(n)), "ld_arena_bytes")
    return n.value


def synth_prompt(seed, seq, n, lo=3, hi=32000):
    out = np.empty(n, np.int32)
    check(lib().ld_synth_prompt(seed, seq, n, lo, hi, out.ctypes.data_as(C.POINTER(C.c_int32))),
          "ld_synth_prompt")
    return out


def _i32p(a):
    return a.ctypes.data_as(C.POINTER(C.c_int32))


class LlamaDecoder:
    """One model on one GPU: weights drawn from `seed`, KV cache for cfg.max_batch sequences."""

    def __init__(self, cfg: ModelConfig, seed: int, device=0, stream=None):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.L = lib()
        self._c = _cfg_struct(cfg)
        self.device = torch.device("cuda", device)
        nbytes = arena_bytes(cfg)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        h = C.c_void_p()
        with torch.cuda.device(self.device):
            check(self.L.ld_model_init(C.byref(self._c), seed, self.arena.data_ptr(), nbytes,
                                       self.stream.cuda_stream, C.byref(h)), "ld_model_init")
        self._h = h
        self.next = torch.zeros(cfg.max_batch, dtype=torch.int32, device=self.device)

    # ---------------------------------------------------------------- calls
    def prefill(self, tokens, logits=None, next_out=None, all_pos=False):
        """tokens: int32 array [batch, n] (host).  Returns the next-token tensor."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        if t.ndim == 1:
            t = t[None, :]
        B, n = t.shape
        nxt = next_out if next_out is not None else self.next[:B]
        check(self.L.ld_prefill(self._h, B, n, _i32p(t),
                                logits.data_ptr() if logits is not None else None,
                                nxt.data_ptr(), int(all_pos)), "ld_prefill")
        return nxt

    def decode_step(self, tokens, logits=None, next_out=None):
        """tokens: int32 host array [batch] or int32 device tensor [batch]."""
        torch = self.torch
        if isinstance(tokens, torch.Tensor) and tokens.is_cuda:
            assert tokens.dtype == torch.int32 and tokens.is_contiguous()
            B, ptr, on_dev = tokens.numel(), tokens.data_ptr(), 1
            keep = None
        else:
            keep = np.ascontiguousarray(np.atleast_1d(tokens), dtype=np.int32)
            B, ptr, on_dev = keep.size, keep.ctypes.data, 0
        nxt = next_out if next_out is not None else self.next[:B]
        check(self.L.ld_decode_step(self._h, B, ptr, on_dev,
                                    logits.data_ptr() if logits is not None else None,
                                    nxt.data_ptr()), "ld_decode_step")
        return nxt

    def decode_step_noalloc(self, tokens, logits=None, next_out=None):
        """decode_step with the step's scratch in the library's static device array
        (ld_decode_step_noalloc).  Returns the status code (LD_OK, or LD_E_SCRATCH
        when the step needs more than the array holds) and the next-token tensor."""
        torch = self.torch
        if isinstance(tokens, torch.Tensor) and tokens.is_cuda:
            assert tokens.dtype == torch.int32 and tokens.is_contiguous()
            B, ptr, on_dev = tokens.numel(), tokens.data_ptr(), 1
            keep = None
        else:
            keep = np.ascontiguousarray(np.atleast_1d(tokens), dtype=np.int32)
            B, ptr, on_dev = keep.size, keep.ctypes.data, 0
        nxt = next_out if next_out is not None else self.next[:B]
        rc = self.L.ld_decode_step_noalloc(self._h, B, ptr, on_dev,
                                           logits.data_ptr() if logits is not None else None,
                                           nxt.data_ptr())
        return rc, nxt

    def generate(self, tokens, n_steps, logits=None, out=None):
        """Greedy on-device generation of n_steps positions (one HIP graph replay each).

        tokens: the first input ids, int32 host array [batch] or device tensor [batch].
        Returns the int32 device tensor [n_steps, batch] of generated tokens (`out` if given).
        """
        torch = self.torch
        if isinstance(tokens, torch.Tensor) and tokens.is_cuda:
            assert tokens.dtype == torch.int32 and tokens.is_contiguous()
            B, ptr, on_dev = tokens.numel(), tokens.data_ptr(), 1
            keep = None
        else:
            keep = np.ascontiguousarray(np.atleast_1d(tokens), dtype=np.int32)
            B, ptr, on_dev = keep.size, keep.ctypes.data, 0
        if out is None:
            out = torch.empty((max(n_steps, 0), B), dtype=torch.int32, device=self.device)
        assert out.dtype == torch.int32 and out.is_contiguous() and out.numel() >= n_steps * B
        check(self.L.ld_generate(self._h, B, n_steps, ptr, on_dev,
                                 logits.data_ptr() if logits is not None else None,
                                 out.data_ptr()), "ld_generate")
        return out

    def generate_rc(self, tokens, n_steps):
        """Like generate (host tokens, no outputs) but returns the status code."""
        keep = np.ascontiguousarray(np.atleast_1d(tokens), dtype=np.int32)
        return self.L.ld_generate(self._h, keep.size, n_steps, keep.ctypes.data, 0, None, None)

    def decode_step_rc(self, tokens, logits=None, next_out=None):
        """Like decode_step but returns the status code instead of raising."""
        keep = np.ascontiguousarray(np.atleast_1d(tokens), dtype=np.int32)
        nxt = next_out if next_out is not None else self.next[:keep.size]
        return self.L.ld_decode_step(self._h, keep.size, keep.ctypes.data, 0,
                                     logits.data_ptr() if logits is not None else None,
                                     nxt.data_ptr())

    def prefill_rc(self, tokens, logits=None, all_pos=False):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        if t.ndim == 1:
            t = t[None, :]
        B, n = t.shape
        return self.L.ld_prefill(self._h, B, n, _i32p(t),
                                 logits.data_ptr() if logits is not None else None,
                                 self.next.data_ptr(), int(all_pos))

    def kv_reset(self):
        check(self.L.ld_kv_reset(self._h), "ld_kv_reset")

    def set_pos(self, p):
        check(self.L.ld_set_pos(self._h, p), "ld_set_pos")

    def set_pos_rc(self, p):
        return self.L.ld_set_pos(self._h, p)

    @property
    def pos(self):
        p = C.c_int32()
        check(self.L.ld_get_pos(self._h, C.byref(p)), "ld_get_pos")
        return p.value

    def read_weights(self, stream_id, start, n):
        out = np.empty(n, np.float32)
        check(self.L.ld_read_weights(self._h, stream_id, start, n,
                                     out.ctypes.data_as(C.POINTER(C.c_float))), "ld_read_weights")
        return out

    def weights_checksum(self):
        v = C.c_uint64(0)
        check(self.L.ld_weights_checksum(self._h, C.byref(v)), "ld_weights_checksum")
        return v.value

    def status(self):
        return self.L.ld_status(self._h)

    def profile(self, kernel_class, enable=True):
        check(self.L.ld_profile(self._h, kernel_class, int(enable)), "ld_profile")

    def profile_read(self, kernel_class):
        avg = C.c_double()
        cnt = C.c_int64()
        check(self.L.ld_profile_read(self._h, kernel_class, C.byref(avg), C.byref(cnt)),
              "ld_profile_read")
        return avg.value, cnt.value

    def close(self):
        if getattr(self, "_h", None):
            self.L.ld_model_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
