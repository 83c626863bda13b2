"""The C-ABI library loads and exports every entry point of include/ld.h (CPU only).

No compute calls: only the host-side entry points that touch no GPU
(arena sizing / config validation, the synthetic prompt generator).
"""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from transformer_llama_decode_amd import _lib
from transformer_llama_decode_amd.configs import WORKLOADS, TINY, ModelConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ld.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from transformer_llama_decode_amd import _build
        _build.build()
    return _lib.lib()


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ld_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = declared()
    assert names == sorted(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (ld_[a-z_]+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(L, n)


def test_library_is_built_for_gfx950_only():
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          "--input=" + _lib.LIB_PATH], capture_output=True, text=True)
    if out.returncode != 0:
        # shared objects carry the device code in a .hip_fatbin section instead
        sec = subprocess.run(["readelf", "-S", _lib.LIB_PATH], capture_output=True, text=True).stdout
        assert ".hip_fatbin" in sec
        blob = open(_lib.LIB_PATH, "rb").read()
        assert b"gfx950" in blob
        assert b"gfx942" not in blob and b"gfx90a" not in blob


def _cfg(m, **kw):
    from transformer_llama_decode_amd.model import _cfg_struct
    from dataclasses import replace
    return _cfg_struct(replace(m, **kw))


@pytest.mark.parametrize("bad", [dict(dim=100), dict(n_heads=5), dict(hidden_dim=100), dict(vocab_size=0),
                                 dict(max_seq=0), dict(max_batch=0), dict(rope_theta=0.0),
                                 dict(dim=64, n_heads=1, hidden_dim=64, vocab_size=10, max_seq=4) | {"n_layers": 0},
                                 dict(dim=512, n_heads=1), dict(n_kv_heads=3), dict(n_kv_heads=-1),
                                 dict(weight_bf16=2), dict(max_pos=50), dict(max_pos=-1),
                                 dict(hidden_dim=39936 + 32), dict(hidden_dim=65536)])
def test_arena_bytes_rejects_unsupported_configs(L, bad):
    n = C.c_size_t(0)
    raw = {k: bad.pop(k) for k in list(bad) if k in ("weight_bf16", "max_pos")}   # set on the C struct as is
    c = _cfg(TINY, **bad)
    for k, v in raw.items():
        setattr(c, k, v)
    assert L.ld_arena_bytes(C.byref(c), C.byref(n)) == _lib.LD_E_INVAL


def test_longest_gemv_input_is_accepted(L):
    # the batch-1 W2 projection stages its whole input (hidden_dim floats) in LDS:
    # 39936 floats fit beside its static arrays in gfx950's 160 KiB
    n = C.c_size_t(0)
    c = _cfg(TINY, hidden_dim=39936)
    assert L.ld_arena_bytes(C.byref(c), C.byref(n)) == _lib.LD_OK and n.value > 0


def test_arena_sizes_of_the_workloads(L):
    for name, w in WORKLOADS.items():
        n = C.c_size_t(0)
        assert L.ld_arena_bytes(C.byref(_cfg(w.model)), C.byref(n)) == 0
        weights = w.model.n_params() * w.model.weight_elem_bytes
        assert weights <= n.value < weights * 1.3 + 3 * 2 ** 30, name
    n = C.c_size_t(0)
    L.ld_arena_bytes(C.byref(_cfg(WORKLOADS["C5"].model)), C.byref(n))
    assert n.value < 40 * 2 ** 30          # 7B shape fits one 288 GB MI355X many times over


def test_null_arguments_are_rejected(L):
    assert L.ld_arena_bytes(None, None) == _lib.LD_E_INVAL
    assert L.ld_kv_reset(None) == _lib.LD_E_INVAL
    assert L.ld_decode_step(None, 1, None, 0, None, None) == _lib.LD_E_INVAL
    assert L.ld_prefill(None, 1, 1, None, None, None, 0) == _lib.LD_E_INVAL
    h = C.c_void_p()
    assert L.ld_model_init(C.byref(_cfg(TINY)), 0, None, 0, None, C.byref(h)) == _lib.LD_E_INVAL
    assert L.ld_strerror(_lib.LD_E_RANGE).decode().startswith("position")


def test_prompt_generator_is_the_shared_one(L):
    from oracle import oracle as O
    from transformer_llama_decode_amd.model import synth_prompt
    for seed, seq in [(1, 0), (2, 255), (4, 0)]:
        assert np.array_equal(synth_prompt(seed, seq, 512), O.synth_prompt(seed, seq, 512))


def test_grouped_query_arena_saves_the_key_value_rows_and_cache(L):
    from dataclasses import replace
    mha = ModelConfig(dim=256, n_layers=2, n_heads=8, hidden_dim=320, vocab_size=301, max_seq=128,
                      max_batch=3)
    sizes = {}
    for kvh in (0, 2, 1):
        n = C.c_size_t(0)
        assert L.ld_arena_bytes(C.byref(_cfg(replace(mha, n_kv_heads=kvh))), C.byref(n)) == 0
        sizes[kvh] = n.value
    hd, d, Lr, B, S = 32, 256, 2, 3, 128
    for kvh in (2, 1):
        saved = 4 * Lr * (2 * (d - kvh * hd) * d + 2 * B * S * (d - kvh * hd))
        assert abs((sizes[0] - sizes[kvh]) - saved) <= 8 * 256, kvh


def test_bfloat16_arena_halves_the_matrices(L):
    from dataclasses import replace
    for tied in (True, False):
        m = ModelConfig(dim=256, n_layers=3, n_heads=8, hidden_dim=320, vocab_size=301, max_seq=64,
                        max_batch=2, tied=tied)
        n32, n16 = C.c_size_t(0), C.c_size_t(0)
        assert L.ld_arena_bytes(C.byref(_cfg(m)), C.byref(n32)) == 0
        assert L.ld_arena_bytes(C.byref(_cfg(replace(m, weight_bf16=True))), C.byref(n16)) == 0
        matrices = m.n_params() - (2 * m.n_layers + 1) * m.dim      # all but the norm gains
        assert abs((n32.value - n16.value) - 2 * matrices) <= 16 * 256, tied


def test_window_arena_adds_the_ring_slack_and_rotary_rows(L):
    """past max_seq: 64 more KV slots per sequence and rotary rows for every position"""
    from dataclasses import replace
    m = ModelConfig(dim=128, n_layers=2, n_heads=4, hidden_dim=160, vocab_size=301, max_seq=100,
                    max_batch=3, n_kv_heads=2)
    n0, n1 = C.c_size_t(0), C.c_size_t(0)
    assert L.ld_arena_bytes(C.byref(_cfg(m)), C.byref(n0)) == 0
    assert L.ld_arena_bytes(C.byref(_cfg(replace(m, max_pos=1000))), C.byref(n1)) == 0
    kv_slack = 2 * 4 * m.n_layers * m.max_batch * m.kv_dim * 64        # K and V, 64 slots
    rope = 2 * 4 * (1000 - 100) * (m.head_dim // 2)                  # cos and sin rows
    ring = 3 * 4 * (1000 - 100)                                      # generated-token ring
    assert abs((n1.value - n0.value) - (kv_slack + rope + ring)) <= 16 * 256
    n2 = C.c_size_t(0)
    assert L.ld_arena_bytes(C.byref(_cfg(replace(m, max_pos=100))), C.byref(n2)) == 0
    assert n2.value == n0.value                                      # max_pos = max_seq: no window


def test_model_init_rejects_a_small_or_misaligned_arena_before_touching_it(L):
    """checked on the host before any device call: the pointers are never dereferenced"""
    n = C.c_size_t(0)
    c = _cfg(TINY)
    assert L.ld_arena_bytes(C.byref(c), C.byref(n)) == 0
    h = C.c_void_p()
    fake = C.c_void_p(1 << 40)                       # 256-byte aligned, never dereferenced
    assert L.ld_model_init(C.byref(c), 0, fake, n.value - 256, None, C.byref(h)) == _lib.LD_E_ARENA
    assert L.ld_model_init(C.byref(c), 0, C.c_void_p((1 << 40) + 64), n.value, None, C.byref(h)) == _lib.LD_E_ARENA
    assert not h.value


def test_calls_on_a_null_handle_are_rejected(L):
    i32 = C.c_int32()
    u64 = C.c_uint64()
    assert L.ld_get_pos(None, C.byref(i32)) == _lib.LD_E_INVAL
    assert L.ld_set_pos(None, 0) == _lib.LD_E_INVAL
    assert L.ld_weights_checksum(None, C.byref(u64)) == _lib.LD_E_INVAL
    assert L.ld_generate(None, 1, 1, None, 0, None, None) == _lib.LD_E_INVAL
    assert L.ld_status(None) == _lib.LD_E_INVAL
    assert L.ld_read_weights(None, 0, 0, 1, None) == _lib.LD_E_INVAL
