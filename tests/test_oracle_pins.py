"""Pins of the CPU oracle against what the mathematics fixes, CPU only.

Every check compares the oracle with something other than itself: exact
rational arithmetic, closed forms of special cases, invariants of the
operations, hand-worked values, or a brute-force path with no KV cache.
tests/test_oracle_mutants.py plants plausible mistakes in a copy of the oracle
and shows that at least one of these pins fails for each.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from transformer_llama_decode_amd.configs import ModelConfig

F32_EPS = float(np.finfo(np.float32).eps)


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ dot ----
def _exact_dot_f32(w_row, x):
    s = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(w_row, x)), Fraction(0))
    return s


def test_matvec_is_correctly_rounded_dot():
    r = _rng(1)
    rows, cols = 7, 300                       # non-square: a transposed W fails
    w = r.standard_normal((rows, cols)).astype(np.float32)
    x = r.standard_normal(cols).astype(np.float32)
    w[3, :] = np.float32(1e4) * w[3, :]      # one row with heavy cancellation
    x[:150] *= np.float32(-1.0)
    got = O.matvec(w, x)
    for i in range(rows):
        ex = _exact_dot_f32(w[i], x)
        near = np.float32(float(ex))          # correctly rounded (via double, ties aside)
        # the exact value must round to the oracle's value: |got - exact| <= half ulp
        ulp = np.spacing(np.abs(near))
        assert abs(Fraction(float(got[i])) - ex) <= Fraction(float(ulp)) / 2 * (1 + 1e-9), i


def test_matvec_identity_and_selection():
    x = np.arange(1, 10, dtype=np.float32)
    assert np.array_equal(O.matvec(np.eye(9, dtype=np.float32), x), x)
    sel = np.zeros((2, 9), np.float32)
    sel[0, 8] = 1
    sel[1, 0] = 2
    assert O.matvec(sel, x).tolist() == [9.0, 2.0]


# -------------------------------------------------------------- RMSNorm ----
def test_rmsnorm_unit_rms_before_gain():
    r = _rng(2)
    for n in (7, 288, 4096):
        x = (r.standard_normal(n) * 3).astype(np.float32)
        y = O.rmsnorm(x, np.ones(n, np.float32), 1e-5).astype(np.float64)
        ms = np.mean(x.astype(np.float64) ** 2)
        want = math.sqrt(ms / (ms + 1e-5))
        assert abs(math.sqrt(np.mean(y ** 2)) - want) < 4 * F32_EPS


def test_rmsnorm_closed_form_constant_vector_eps_inside_root():
    # x = c everywhere: y = c / sqrt(c^2 + eps).  With c = 1e-3 and eps = 1e-5
    # this is 0.30151..., far from 0.990 (eps outside the root) or from the
    # value with a sum instead of a mean.
    n = 16
    x = np.full(n, 1e-3, np.float32)
    y = O.rmsnorm(x, np.ones(n, np.float32), 1e-5)
    c = float(np.float32(1e-3))
    assert np.allclose(y, c / math.sqrt(c * c + 1e-5), rtol=2 * F32_EPS, atol=0)


def test_rmsnorm_gain_and_scale_invariance():
    r = _rng(3)
    n = 512
    x = r.standard_normal(n).astype(np.float32)
    g = r.uniform(0.5, 2.0, n).astype(np.float32)
    y1 = O.rmsnorm(x, np.ones(n, np.float32), 1e-5)
    yg = O.rmsnorm(x, g, 1e-5)
    assert np.allclose(yg, y1 * g, rtol=3 * F32_EPS, atol=0)
    y8 = O.rmsnorm(x * np.float32(8.0), np.ones(n, np.float32), 1e-5)
    assert np.allclose(y8, y1, rtol=1e-5, atol=0)     # eps breaks it only at 1e-5/ms


# -------------------------------------------------------------- softmax ----
def test_softmax_sums_to_one_shift_invariant_and_single():
    r = _rng(4)
    s = r.standard_normal(1000) * 10
    p = O.softmax(s)
    assert abs(p.sum() - 1.0) < 1000 * 2.3e-16
    assert np.all(p > 0)
    assert np.allclose(O.softmax(s + 123.0), p, rtol=1e-12, atol=0)
    assert O.softmax(np.array([-7.5]))[0] == 1.0


def test_softmax_hand_worked():
    # softmax(0, ln 3) = (1/4, 3/4)
    p = O.softmax(np.array([0.0, math.log(3.0)]))
    assert abs(p[0] - 0.25) < 1e-15 and abs(p[1] - 0.75) < 1e-15


# ----------------------------------------------------------------- RoPE ----
def test_rope_position_zero_is_identity():
    c, s = O.rope_table(4, 48, 10000.0)
    v = _rng(5).standard_normal(288).astype(np.float32)
    assert np.array_equal(O.rope(v, 48, c[0], s[0]), v)


def test_rope_preserves_pair_norms():
    hd = 64
    c, s = O.rope_table(1024, hd, 10000.0)
    v = _rng(6).standard_normal(512).astype(np.float32)
    for p in (1, 17, 1023):
        w = O.rope(v, hd, c[p], s[p]).astype(np.float64)
        a = v.astype(np.float64).reshape(-1, 2)
        b = w.reshape(-1, 2)
        na, nb = np.hypot(a[:, 0], a[:, 1]), np.hypot(b[:, 0], b[:, 1])
        assert np.all(np.abs(nb - na) <= 4 * F32_EPS * na)


def test_rope_pairs_are_adjacent_and_rotate_counterclockwise():
    hd = 8
    c, s = O.rope_table(8, hd, 10000.0)
    v = np.zeros(16, np.float32)
    v[0] = 1.0                                 # head 0, pair 0 (freq 1): angle = p
    v[8 + 2] = 1.0                             # head 1, pair 1
    w = O.rope(v, hd, c[1], s[1])
    nz = set(np.nonzero(w)[0].tolist())
    assert nz == {0, 1, 10, 11}                # only partners 2i+1 are touched
    assert w[0] == np.float32(math.cos(1.0)) and w[1] == np.float32(math.sin(1.0))
    assert w[11] > 0                           # (1,0) turns toward +second component


def test_rope_frequencies_and_linear_angles():
    hd, theta = 128, 10000.0
    c, s = O.rope_table(64, hd, theta)
    # recover theta_i from the angle at p = 1 (all angles < pi there)
    ang = np.arctan2(s[1].astype(np.float64), c[1].astype(np.float64))
    want = theta ** (-(2.0 * np.arange(hd // 2)) / hd)
    assert np.allclose(ang, want, rtol=1e-6, atol=1e-7)
    # angles grow linearly in p: Chebyshev recurrence cos((p+1)t)+cos((p-1)t) = 2cos(t)cos(pt)
    cc = c.astype(np.float64)
    for p in (5, 31, 62):
        lhs = cc[p + 1] + cc[p - 1]
        rhs = 2 * cc[1] * cc[p]
        assert np.allclose(lhs, rhs, atol=8 * F32_EPS)


def test_rope_relative_position_property():
    hd = 32
    c, s = O.rope_table(300, hd, 10000.0)
    r = _rng(7)
    q = r.standard_normal(hd).astype(np.float32)
    k = r.standard_normal(hd).astype(np.float32)

    def ip(m, n):
        return float(np.dot(O.rope(q, hd, c[m], s[m]).astype(np.float64),
                            O.rope(k, hd, c[n], s[n]).astype(np.float64)))
    for m, n, sh in [(10, 3, 100), (5, 5, 250), (0, 40, 7)]:
        assert abs(ip(m, n) - ip(m + sh, n + sh)) < 1e-5 * (1 + abs(ip(m, n)))


# ------------------------------------------------------------ attention ----
def test_attention_single_position_returns_v0_exactly():
    r = _rng(8)
    d, H = 96, 2
    q = r.standard_normal(d).astype(np.float32)
    k = r.standard_normal((1, d)).astype(np.float32)
    v = r.standard_normal((1, d)).astype(np.float32)
    assert np.array_equal(O.attention(q, k, v, H), v[0])


def test_attention_equal_keys_give_mean_and_dominant_key_selects():
    r = _rng(9)
    d, H, n = 64, 4, 9
    q = r.standard_normal(d).astype(np.float32)
    k = np.tile(r.standard_normal(d).astype(np.float32), (n, 1))
    v = r.standard_normal((n, d)).astype(np.float32)
    assert np.allclose(O.attention(q, k, v, H), v.astype(np.float64).mean(0), rtol=0, atol=1e-6)
    q2 = np.ones(d, np.float32)
    k2 = np.zeros((n, d), np.float32)
    k2[6] = 100.0                             # score 100*16/4 = 400 above the rest
    assert np.array_equal(O.attention(q2, k2, v, H), v[6])


def test_attention_hand_worked_scale():
    # one head, hd = 4 (scale 1/2): q = (2,0,0,0), k0 = 0, k1 = (ln 3,0,0,0)
    # scores (0, ln 3) -> weights (1/4, 3/4) -> o = v0/4 + 3 v1/4
    q = np.array([2, 0, 0, 0], np.float32)
    k = np.zeros((2, 4), np.float32)
    k[1, 0] = math.log(3.0)
    v = np.array([[4, 8, -4, 0], [8, 0, 4, 12]], np.float32)
    l3 = float(np.float32(math.log(3.0)))
    w1 = 3 ** (l3 / math.log(3.0)) / (1 + 3 ** (l3 / math.log(3.0)))
    want = (1 - w1) * v[0].astype(np.float64) + w1 * v[1].astype(np.float64)
    assert np.allclose(O.attention(q, k, v, 1), want, rtol=2 * F32_EPS, atol=1e-6)


def test_attention_heads_are_independent():
    r = _rng(10)
    d, H, n = 48, 3, 5
    q = r.standard_normal(d).astype(np.float32)
    k = r.standard_normal((n, d)).astype(np.float32)
    v = r.standard_normal((n, d)).astype(np.float32)
    o = O.attention(q, k, v, H)
    k2, v2 = k.copy(), v.copy()
    k2[:, 16:32] = r.standard_normal((n, 16))
    v2[:, 16:32] = r.standard_normal((n, 16))
    o2 = O.attention(q, k2, v2, H)
    assert np.array_equal(o[:16], o2[:16]) and np.array_equal(o[32:], o2[32:])
    assert not np.array_equal(o[16:32], o2[16:32])


# --------------------------------------------------------------- SwiGLU ----
def test_swiglu_special_values():
    h1 = np.array([0.0, 1.0, 30.0, -30.0, -1.0], np.float32)
    h3 = np.array([5.0, 1.0, 2.0, 2.0, 1.0], np.float32)
    g = O.swiglu(h1, h3)
    assert g[0] == 0.0
    assert g[1] == np.float32(1.0 / (1.0 + math.exp(-1.0)))      # silu(1) = 1/(1+1/e)
    assert abs(g[2] - 60.0) < 1e-6                                # silu(z) -> z
    assert abs(g[3]) < 30 * 2 * math.exp(-30) * 1.01              # silu(z) -> 0
    assert g[4] == np.float32(-1.0 / (1.0 + math.e))              # silu(-1) = -1/(1+e)


def test_argmax_lowest_index_on_ties_and_nonfinite():
    assert O.argmax(np.array([1, 3, 3, 2], np.float32)) == 1
    assert O.argmax(np.array([-5, -5], np.float32)) == 0
    assert O.argmax(np.array([0, np.nan, 1], np.float32)) == -1
    assert O.argmax(np.array([0, np.inf], np.float32)) == -1


def test_residual_add_fp32():
    x = np.array([1.0, 1e8], np.float32)
    t = np.array([2.0 ** -24, 1.0], np.float32)
    y = O.residual_add(x, t)
    assert y[0] == np.float32(1.0) + np.float32(2.0 ** -24) and y[1] == np.float32(1e8)


# ---------------------------------------------------------- whole model ----
TINY = ModelConfig(dim=32, n_layers=2, n_heads=4, hidden_dim=48, vocab_size=61, max_seq=12)
TINY_U = ModelConfig(dim=24, n_layers=3, n_heads=2, hidden_dim=40, vocab_size=37, max_seq=10,
                     tied=False)


def _zero_mix(m, cfg, kinds):
    for l in range(cfg.n_layers):
        for kd in kinds:
            m.tensor(1 + 7 * l + kd)[:] = 0


def test_closed_form_when_blocks_are_zero_tied():
    # With Wo = W2 = 0 every block adds nothing, so x stays E[t] and
    # logits_j = E_j . E_t / sqrt(mean(E_t^2) + eps).
    cfg = TINY
    m = O.OracleModel(cfg, 11)
    _zero_mix(m, cfg, (3, 5))
    E = m.tensor(0).reshape(cfg.vocab_size, cfg.dim).astype(np.float64)
    st = m.new_state()
    for pos, t in enumerate([5, 0, 60, 17]):
        r, logits = m.forward(st, t, pos)
        xn = E[t] / math.sqrt(np.mean(E[t] ** 2) + cfg.norm_eps)
        want = E @ xn
        assert np.allclose(logits, want, rtol=1e-6, atol=1e-7)
        assert r == int(np.argmax(want))


def test_closed_form_when_blocks_are_zero_untied():
    cfg = TINY_U
    m = O.OracleModel(cfg, 12)
    _zero_mix(m, cfg, (3, 5))
    E = m.tensor(0).reshape(cfg.vocab_size, cfg.dim).astype(np.float64)
    W = m.tensor(1 + 7 * cfg.n_layers).reshape(cfg.vocab_size, cfg.dim).astype(np.float64)
    st = m.new_state()
    r, logits = m.forward(st, 9, 0)
    xn = E[9] / math.sqrt(np.mean(E[9] ** 2) + cfg.norm_eps)
    assert np.allclose(logits, W @ xn, rtol=1e-6, atol=1e-7)


def test_single_layer_at_position_zero_reduces_to_value_path():
    # At p = 0 attention returns V[0] = Wv n(x), so with the FFN silenced
    # (W2 = 0) the block is x + Wo Wv n(x): Wq and Wk must not matter.
    cfg = ModelConfig(dim=16, n_layers=1, n_heads=2, hidden_dim=24, vocab_size=23, max_seq=4)
    m = O.OracleModel(cfg, 13)
    m.tensor(1 + 5)[:] = 0                               # W2
    E = m.tensor(0).reshape(23, 16).astype(np.float64)
    Wv = m.tensor(1 + 2).reshape(16, 16).astype(np.float64)
    Wo = m.tensor(1 + 3).reshape(16, 16).astype(np.float64)
    x = E[4]
    x1 = x + Wo @ (Wv @ (x / math.sqrt(np.mean(x ** 2) + 1e-5)))
    want = E @ (x1 / math.sqrt(np.mean(x1 ** 2) + 1e-5))
    _, logits = m.forward(m.new_state(), 4, 0)
    assert np.allclose(logits, want, rtol=1e-5, atol=1e-6)
    m.tensor(1 + 0)[:] = 7.0                              # Wq, Wk are irrelevant at p = 0
    m.tensor(1 + 1)[:] = -3.0
    _, logits2 = m.forward(m.new_state(), 4, 0)
    assert np.array_equal(logits, logits2)


def test_ffn_hand_worked():
    # d = 2, f = 2, one layer, attention silenced (Wo = 0).  x = E[0] = (a, a):
    # n(x) = (1, 1) up to eps;  W1 = diag(1, 2), W3 = diag(3, 1), W2 = [[1, 0], [0, 1]]
    # -> g = (silu(1) * 3, silu(2) * 1) -> x' = x + g.
    cfg = ModelConfig(dim=2, n_layers=1, n_heads=1, hidden_dim=2, vocab_size=3, max_seq=2)
    m = O.OracleModel(cfg, 14)
    E = m.tensor(0)
    E[:] = [2.0, 2.0, 0.0, 1.0, 1.0, 0.0]
    m.tensor(4)[:] = 0                                    # Wo
    m.tensor(5)[:] = [1, 0, 2, 0]                         # W1 rows: (1,0), (2,0)... see below
    m.tensor(7)[:] = [3, 0, 0, 1]                         # W3
    m.tensor(6)[:] = [1, 0, 0, 1]                         # W2
    # W1 = [[1,0],[2,0]] so W1 n(x) = (n1, 2 n1) with n1 = 2/sqrt(4+eps)
    n1 = 2.0 / math.sqrt(4.0 + 1e-5)
    silu = lambda z: z / (1 + math.exp(-z))
    n1f = float(np.float32(n1))
    g = [silu(n1f) * 3 * n1f, silu(2 * n1f) * n1f]
    x1 = np.array([2.0 + g[0], 2.0 + g[1]])
    logits_want = E.reshape(3, 2).astype(np.float64) @ (x1 / math.sqrt(np.mean(x1 ** 2) + 1e-5))
    _, logits = m.forward(m.new_state(), 0, 0)
    assert np.allclose(logits, logits_want, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("cfg,seed", [(TINY, 21), (TINY_U, 22)])
def test_incremental_cache_equals_full_recomputation(cfg, seed):
    m = O.OracleModel(cfg, seed)
    toks = O.synth_prompt(seed, 0, cfg.max_seq, 0, cfg.vocab_size)
    st = m.new_state()
    for p in range(cfg.max_seq):
        r, logits = m.forward(st, int(toks[p]), p)
        r2, logits2 = m.recompute(toks[: p + 1])
        assert r == r2
        assert np.array_equal(logits, logits2), p


def test_forward_rejects_bad_input():
    m = O.OracleModel(TINY, 1)
    st = m.new_state()
    assert m.forward(st, TINY.vocab_size, 0)[0] == -2
    assert m.forward(st, -1, 0)[0] == -2
    assert m.forward(st, 0, TINY.max_seq)[0] == -2


def test_weights_come_from_the_generator():
    m = O.OracleModel(TINY_U, 5)
    L = TINY_U.n_layers
    for sid in (0, 1, 7, 1 + 7 * (L - 1) + 6, 1 + 7 * L):
        w = m.tensor(sid)
        assert np.array_equal(w, O.synth_normal(5, sid, 0, w.size))
    assert np.all(m.tensor(-1) == 1.0) and np.all(m.tensor(-1 - 2 * L) == 1.0)


# ------------------------------------------------ grouped-query attention ----
# n_kv_heads key/value heads, each shared by n_heads / n_kv_heads consecutive
# query heads (Ainslie et al. 2023, sec. 2.2); one key/value head is multi-query
# attention (the pages' "multi-query support" TODO).
GQA = ModelConfig(dim=64, n_layers=2, n_heads=4, hidden_dim=96, vocab_size=301, max_seq=24,
                  tied=False, n_kv_heads=2)
MQA = ModelConfig(dim=64, n_layers=2, n_heads=4, hidden_dim=96, vocab_size=301, max_seq=24,
                  tied=True, n_kv_heads=1)


def test_gqa_attention_equals_mha_with_repeated_kv_heads():
    r = _rng(31)
    H, hd, n = 6, 8, 5
    for Hkv in (1, 2, 3, 6):
        g = H // Hkv
        q = r.standard_normal(H * hd).astype(np.float32)
        k = r.standard_normal((n, Hkv * hd)).astype(np.float32)
        v = r.standard_normal((n, Hkv * hd)).astype(np.float32)
        # MHA head h gets key/value head h // g (np.repeat keeps each head's hd columns together)
        k_rep = np.repeat(k.reshape(n, Hkv, hd), g, axis=1).reshape(n, H * hd)
        v_rep = np.repeat(v.reshape(n, Hkv, hd), g, axis=1).reshape(n, H * hd)
        assert np.array_equal(O.attention(q, k, v, H, Hkv), O.attention(q, k_rep, v_rep, H)), Hkv


@pytest.mark.parametrize("cfg", [GQA, MQA])
def test_gqa_model_equals_mha_model_with_repeated_kv_rows(cfg):
    """A GQA model and an MHA model whose Wk / Wv repeat each key/value head's
    rows for its query-head group give bit-identical logits."""
    seed = 33
    gm = O.OracleModel(cfg, seed)
    mha = ModelConfig(**{**cfg.__dict__, "n_kv_heads": 0})
    mm = O.OracleModel(mha, seed)
    H, Hkv, hd, d = cfg.n_heads, cfg.kv_heads, cfg.head_dim, cfg.dim
    g = H // Hkv
    for l in range(cfg.n_layers):
        for kind in (1, 2):                       # Wk, Wv of layer l
            sid = 1 + 7 * l + kind
            src = gm.tensor(sid).reshape(Hkv, hd, d)
            mm.tensor(sid)[:] = np.repeat(src, g, axis=0).reshape(-1)
    toks = O.synth_prompt(seed, 0, cfg.max_seq, 0, cfg.vocab_size)
    s1, s2 = gm.new_state(), mm.new_state()
    for p in range(cfg.max_seq):
        r1, l1 = gm.forward(s1, int(toks[p]), p)
        r2, l2 = mm.forward(s2, int(toks[p]), p)
        assert r1 == r2 and np.array_equal(l1, l2), p


@pytest.mark.parametrize("cfg,seed", [(GQA, 34), (MQA, 35)])
def test_gqa_incremental_cache_equals_full_recomputation(cfg, seed):
    m = O.OracleModel(cfg, seed)
    toks = O.synth_prompt(seed, 0, cfg.max_seq, 0, cfg.vocab_size)
    st = m.new_state()
    for p in range(cfg.max_seq):
        r, logits = m.forward(st, int(toks[p]), p)
        r2, logits2 = m.recompute(toks[: p + 1])
        assert r == r2
        assert np.array_equal(logits, logits2), p


def test_gqa_weight_shapes_and_bad_head_counts():
    m = O.OracleModel(GQA, 36)
    kvd = GQA.kv_dim
    assert m.tensor(2).size == kvd * GQA.dim and m.tensor(3).size == kvd * GQA.dim   # Wk, Wv
    assert m.tensor(1).size == GQA.dim * GQA.dim                                   # Wq
    assert np.array_equal(m.tensor(2), O.synth_normal(36, 2, 0, kvd * GQA.dim))
    with pytest.raises(ValueError):
        O.OracleModel(ModelConfig(dim=64, n_layers=1, n_heads=4, hidden_dim=32, vocab_size=10,
                                  max_seq=4, n_kv_heads=3), 1)


# ------------------------------------------------------ bfloat16 weights ----
# bfloat16 is the upper half of an IEEE binary32: sign, 8 exponent bits, 7
# fraction bits (Kalamkar et al. 2019, sec. 2); the weights are the fp32 draws
# rounded to nearest, ties to even.  torch's CPU conversion (round to nearest
# even) is the independent reference.
def _torch_bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def test_bf16_round_matches_torch_on_every_kind_of_value():
    r = _rng(41)
    parts = [r.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)]   # any bit pattern
    hi = r.integers(0, 2**16, 4000, dtype=np.uint64).astype(np.uint32) << 16
    parts.append(hi | 0x8000)                      # exactly halfway, both parities of the kept bit
    parts.append(hi | 0x7FFF)
    parts.append(hi | 0x8001)
    parts.append(np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001,
                           0x007FFFFF, 0x3F808000, 0x3F818000], np.uint32))
    u = np.concatenate(parts)
    x = u.view(np.float32)
    got, want = O.bf16_round(x), _torch_bf16(x)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(_bits(got)[~nan], _bits(want)[~nan])


def test_bf16_round_hand_worked():
    one = 1.0
    cases = [
        (one, one),
        (one + 2**-8, one),                        # halfway, kept bit 0: stays
        (one + 3 * 2**-8, one + 2**-6),            # halfway, kept bit 1: rounds up to even
        (one + 2**-8 + 2**-20, one + 2**-7),       # just past halfway
        (-(one + 2**-8), -one),
        (3.4028234663852886e38, math.inf),         # largest float: past the largest bfloat16
        (2.0**-149, 0.0),                          # smallest subnormal: below half a bf16 quantum
    ]
    for x, want in cases:
        assert float(O.bf16_round(np.array([x], np.float32))[0]) == want, x
    # 0.02 to the nearest multiple of its bfloat16 quantum 2^-13 (7 fraction bits, 2^-6 <= 0.02 < 2^-5)
    x = float(np.float32(0.02))
    q = 2.0**-13
    assert float(O.bf16_round(np.array([x], np.float32))[0]) == round(x / q) * q


BF = ModelConfig(dim=32, n_layers=2, n_heads=4, hidden_dim=48, vocab_size=61, max_seq=12,
                 tied=False, weight_bf16=True)


def test_bf16_model_weights_are_the_rounded_draws():
    seed = 42
    m = O.OracleModel(BF, seed)
    L = BF.n_layers
    changed = 0
    for sid in [0] + list(range(1, 1 + 7 * L)) + [1 + 7 * L]:
        w = m.tensor(sid)
        draw = O.synth_normal(seed, sid, 0, w.size)
        assert np.array_equal(_bits(w), _bits(_torch_bf16(draw))), sid
        assert np.all(_bits(w) & 0xFFFF == 0), sid
        assert np.all(np.abs(w - draw) <= np.abs(draw) * 2.0**-8), sid   # half a unit in the 8th bit
        changed += int(np.count_nonzero(w != draw))
    assert changed > 0
    for g in range(2 * L + 1):
        assert np.all(m.tensor(-1 - g) == 1.0)     # norm gains stay fp32 ones


def test_bf16_model_is_the_fp32_model_with_rounded_weights():
    """only storage changes: an fp32 model given the rounded weights computes the same logits"""
    seed = 43
    bm = O.OracleModel(BF, seed)
    fm = O.OracleModel(ModelConfig(**{**BF.__dict__, "weight_bf16": False}), seed)
    L = BF.n_layers
    for sid in [0] + list(range(1, 1 + 7 * L)) + [1 + 7 * L]:
        fm.tensor(sid)[:] = _torch_bf16(fm.tensor(sid))
    toks = O.synth_prompt(seed, 0, BF.max_seq, 0, BF.vocab_size)
    s1, s2 = bm.new_state(), fm.new_state()
    for p in range(BF.max_seq):
        r1, l1 = bm.forward(s1, int(toks[p]), p)
        r2, l2 = fm.forward(s2, int(toks[p]), p)
        assert r1 == r2 and np.array_equal(l1, l2), p


# --------------------------------------------- decoding past max_seq ----
# The KV cache holds max_seq positions; past that, position p attends to the
# window p-max_seq+1 .. p (sliding-window attention: Longformer, Beltagy et al.
# 2020, sec. 3.1; Mistral 7B, Jiang et al. 2023, sec. 2), rotary angles of the
# absolute position.
def _win(n_layers, W, P, seed_cfg=0):
    return ModelConfig(dim=32, n_layers=n_layers, n_heads=4, hidden_dim=48, vocab_size=61,
                       max_seq=W, max_pos=P, tied=True)


def _run(m, toks, upto):
    st = m.new_state()
    out = []
    for p in range(upto):
        r, lg = m.forward(st, int(toks[p]), p)
        assert r >= 0
        out.append(lg.copy())
    return np.stack(out)


def test_window_is_inactive_before_max_seq():
    seed, W, P = 44, 8, 30
    a = O.OracleModel(_win(2, W, P), seed)
    b = O.OracleModel(_win(2, P, 0), seed)          # no window: the cache holds every position
    toks = O.synth_prompt(seed, 0, P, 0, 61)
    la, lb = _run(a, toks, P), _run(b, toks, P)
    assert np.array_equal(la[:W], lb[:W])
    assert all(not np.array_equal(la[p], lb[p]) for p in range(W, P))


@pytest.mark.parametrize("n_layers,W", [(1, 6), (2, 5), (3, 4)])
def test_window_receptive_field_is_exact(n_layers, W):
    """logits at p depend on the tokens at p - L(W-1) .. p and on no earlier one
    (each layer reaches W-1 positions further back)"""
    seed, P = 45, 26
    m = O.OracleModel(_win(n_layers, W, P), seed)
    toks = O.synth_prompt(seed, 0, P, 0, 61)
    base = _run(m, toks, P)
    p = P - 1
    edge = p - n_layers * (W - 1)
    assert edge >= 1
    for q, same in ((edge - 1, True), (edge, False)):
        t2 = toks.copy()
        t2[q] = (t2[q] + 1) % 61
        lg = _run(m, t2, P)
        assert np.array_equal(lg[p], base[p]) == same, q
        assert np.array_equal(lg[:q], base[:q])       # causality


def test_window_depends_on_relative_positions_only():
    """one layer: the logits at p >= W equal those at W-1 of the same W tokens
    started at position 0 (rotary scores depend on p - j; fp32 rounding of the
    rotations at other absolute angles is the only difference)"""
    seed, W, P = 46, 7, 24
    m = O.OracleModel(_win(1, W, P), seed)
    toks = O.synth_prompt(seed, 0, P, 0, 61)
    lg = _run(m, toks, P)
    for p in range(W, P):
        ref = _run(m, toks[p - W + 1: p + 1], W)[-1]
        assert np.allclose(lg[p], ref, rtol=1e-5, atol=1e-6), p


def test_window_incremental_cache_equals_full_recomputation():
    seed, W, P = 47, 5, 17
    m = O.OracleModel(_win(2, W, P), seed)
    toks = O.synth_prompt(seed, 0, P, 0, 61)
    st = m.new_state()
    for p in range(P):
        r, lg = m.forward(st, int(toks[p]), p)
        r2, lg2 = m.recompute(toks[: p + 1])
        assert r == r2 and np.array_equal(lg, lg2), p


def test_window_bounds():
    m = O.OracleModel(_win(1, 4, 9), 1)
    st = m.new_state()
    assert m.forward(st, 0, 9)[0] == -2               # past max_pos
    with pytest.raises(ValueError):
        O.OracleModel(_win(1, 8, 5), 1)                # max_pos below max_seq
