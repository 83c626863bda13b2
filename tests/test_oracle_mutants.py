"""Planted mistakes: each plausible error in the oracle must fail at least one pin.

Each case copies oracle/oracle.c to a temporary directory, applies one textual
change (a dropped term, a wrong sign, index or operand), builds it on the CPU and
runs tests/test_oracle_pins.py against that build in a child process.  The case
passes when the pin suite FAILS on the mutant.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "rmsnorm_eps_outside_root": ("1.0 / sqrt((double)ss / (double)n + eps)",
                                 "1.0 / (sqrt((double)ss / (double)n) + eps)"),
    "rmsnorm_sum_not_mean": ("(double)ss / (double)n + eps", "(double)ss + eps"),
    "rmsnorm_gain_dropped": ("* inv * (double)gain[i]", "* inv"),
    "matvec_transposed": ("acc += (or_acc)row[k] * (or_acc)x[k];",
                          "acc += (or_acc)w[(size_t)k * rows + r % cols] * (or_acc)x[k % rows];"),
    "matvec_float_accumulator": ("    or_acc acc = 0;\n    for (int k = 0; k < cols; ++k)",
                                 "    float acc = 0.0f;\n    for (int k = 0; k < cols; ++k)"),
    "rope_sign": ("(float)(a * c - b * s)", "(float)(a * c + b * s)"),
    "rope_second_sign": ("(float)(a * s + b * c)", "(float)(-a * s + b * c)"),
    "rope_half_split_pairs": ("double a = vh[2 * i], b = vh[2 * i + 1];",
                              "double a = vh[i], b = vh[i + half];"),
    "rope_frequency_exponent": ("-(2.0 * (double)i) / (double)head_dim", "-(double)i / (double)head_dim"),
    "rope_not_applied_to_k": ("    or_rope(s->k, kvd, hd,", "    if (0) or_rope(s->k, kvd, hd,"),
    "attention_scale_1_over_hd": ("(double)dot / sqrt((double)hd)", "(double)dot / (double)hd"),
    "attention_excludes_current_position": ("vl + (size_t)lo * kvd, pos - lo + 1, d,",
                                            "vl + (size_t)lo * kvd, pos - lo > 0 ? pos - lo : 1, d,"),
    "window_one_too_wide": ("int lo = pos - c->max_seq + 1 > 0 ? pos - c->max_seq + 1 : 0;",
                            "int lo = pos - c->max_seq > 0 ? pos - c->max_seq : 0;"),
    "window_ignored": ("int lo = pos - c->max_seq + 1 > 0 ? pos - c->max_seq + 1 : 0;", "int lo = 0;"),
    "recompute_window_one_too_narrow": ("int lo = i - c->max_seq + 1 > 0 ? i - c->max_seq + 1 : 0;",
                                        "int lo = i - c->max_seq + 2 > 0 ? i - c->max_seq + 2 : 0;"),
    "bf16_truncates": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;"),
    "bf16_ties_away_from_zero": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    "bf16_not_applied_to_weights": ("if (c->weight_bf16)\n    for", "if (0)\n    for"),
    "attention_v_head_offset": ("v_rows[(size_t)j * kvd + kv_off + i]", "v_rows[(size_t)j * kvd + i]"),
    "gqa_kv_head_modulo": ("const size_t kv_off = (size_t)(h / group) * hd;",
                           "const size_t kv_off = (size_t)(h % n_kv_heads) * hd;"),
    "gqa_key_row_stride_dim": ("const float* kj = k_rows + (size_t)j * kvd + kv_off;",
                               "const float* kj = k_rows + (size_t)j * dim + kv_off;"),
    "softmax_not_normalised": ("for (int j = 0; j < n; ++j) s[j] /= sum;", ""),
    "swiglu_gate_on_w3": ("double z = h1[i];\n    g[i] = (float)((z / (1.0 + exp(-z))) * (double)h3[i]);",
                          "double z = h3[i];\n    g[i] = (float)((z / (1.0 + exp(-z))) * (double)h1[i]);"),
    "silu_sign": ("(z / (1.0 + exp(-z)))", "(z / (1.0 + exp(z)))"),
    "residual_dropped": ("x[i] = x[i] + t[i];", "x[i] = t[i];"),
    "cache_written_one_back": ("memcpy(kl + (size_t)pos * kvd, s->k",
                               "memcpy(kl + (size_t)(pos > 0 ? pos - 1 : 0) * kvd, s->k"),
    "value_cache_gets_keys": ("memcpy(vl + (size_t)pos * kvd, s->v", "memcpy(vl + (size_t)pos * kvd, s->k"),
    "query_uses_wk": ("or_matvec(s->q, m->wq[l], s->xn, d, d);", "or_matvec(s->q, m->wk[l], s->xn, d, d);"),
    "argmax_highest_index_on_ties": ("if (v[i] > v[best]) best = i;", "if (v[i] >= v[best]) best = i;"),
    "classifier_ignores_untied": ("or_matvec(logits, m->wcls, xn,", "or_matvec(logits, m->emb, xn,"),
    "final_norm_dropped": ("or_matvec(logits, m->wcls, xn, m->c.vocab_size",
                           "or_matvec(logits, m->wcls, x, m->c.vocab_size"),
    "ffn_norm_skipped": ("  or_matvec(h1, m->w1[l], xn, f, d);\n  or_matvec(h3, m->w3[l], xn, f, d);",
                         "  or_matvec(h1, m->w1[l], x, f, d);\n  or_matvec(h3, m->w3[l], x, f, d);"),
}


def _check(name):
    find, repl = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, "mutation anchor for %s not unique/absent" % name
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "oracle.c")
        with open(path, "w") as f:
            f.write(src.replace(find, repl))
        so = os.path.join(td, "liboracle_mutant.so")
        _build.build_oracle(path, so)
        env = dict(os.environ, LD_ORACLE_LIB=so, PYTHONDONTWRITEBYTECODE="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        return r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin():
    if not os.path.exists(_build.SYNTH_OBJ):
        _build.build_synth()
    names = sorted(MUTANTS)
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip(names, ex.map(_check, names)))
    survivors = [n for n, (rc, _) in results.items() if rc == 0]
    assert not survivors, "planted mistakes not caught by any pin: %s" % survivors


def test_unmutated_oracle_passes_pins():
    # the harness itself: the real source, rebuilt the same way, passes
    with tempfile.TemporaryDirectory() as td:
        so = os.path.join(td, "liboracle_copy.so")
        _build.build_oracle(SRC, so)
        env = dict(os.environ, LD_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout[-3000:]
