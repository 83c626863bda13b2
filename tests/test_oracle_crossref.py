"""A second, independent forward pass in float64 NumPy against the oracle.

The pages check their C engine against a separate PyTorch implementation
("the same result"); this is that check for the oracle.  The NumPy version is
written from the mathematics in a different shape: the whole sequence at once
with matrix products, the rotary embedding as multiplication of adjacent pairs
read as complex numbers by e^(i p theta_j), attention as one masked softmax over
a [positions x positions] score matrix (keys repeated per query-head group for
grouped-query attention, a band mask for the window past max_seq), and every
intermediate kept in float64 (the oracle stores fp32 between steps, so the two
agree to float32 rounding, not bit for bit).  It shares no code with the
oracle; weights are read from the oracle's tensors.
"""
import numpy as np
import pytest

from oracle import oracle as O
from transformer_llama_decode_amd.configs import ModelConfig


def _weights(om, cfg):
    L = cfg.n_layers
    w = {"E": om.tensor(0).astype(np.float64).reshape(cfg.vocab_size, cfg.dim)}
    for l in range(L):
        for kind, name in enumerate(["wq", "wk", "wv", "wo", "w1", "w2", "w3"]):
            t = om.tensor(1 + 7 * l + kind).astype(np.float64)
            rows = {"wk": cfg.kv_dim, "wv": cfg.kv_dim, "w1": cfg.hidden_dim, "w3": cfg.hidden_dim}.get(name, cfg.dim)
            w[(name, l)] = t.reshape(rows, -1)
        w[("g_att", l)] = om.tensor(-1 - l).astype(np.float64)
        w[("g_ffn", l)] = om.tensor(-1 - L - l).astype(np.float64)
    w["g_out"] = om.tensor(-1 - 2 * L).astype(np.float64)
    w["cls"] = w["E"] if cfg.tied else om.tensor(1 + 7 * L).astype(np.float64).reshape(cfg.vocab_size, cfg.dim)
    return w


def _rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def _rotate(x, n_heads, hd, theta):
    """x [T, n_heads*hd]: pairs (2j, 2j+1) of each head as complex numbers times e^(i t theta^(-2j/hd))"""
    T = x.shape[0]
    z = x.reshape(T, n_heads, hd // 2, 2)
    zc = z[..., 0] + 1j * z[..., 1]
    freqs = theta ** (-np.arange(0, hd, 2) / hd)
    rot = np.exp(1j * np.outer(np.arange(T), freqs))[:, None, :]
    zc = zc * rot
    return np.stack([zc.real, zc.imag], axis=-1).reshape(T, n_heads * hd)


def numpy_forward(om, cfg, tokens):
    """logits [T, V] of every position of `tokens` (positions 0..T-1)"""
    w = _weights(om, cfg)
    T, d, H, Hk, hd = len(tokens), cfg.dim, cfg.n_heads, cfg.kv_heads, cfg.head_dim
    x = w["E"][np.asarray(tokens)]
    pos = np.arange(T)
    # query t sees key j iff t - max_seq < j <= t
    mask = (pos[None, :] <= pos[:, None]) & (pos[None, :] > pos[:, None] - cfg.max_seq)
    for l in range(cfg.n_layers):
        xn = _rms(x, w[("g_att", l)], cfg.norm_eps)
        q = _rotate(xn @ w[("wq", l)].T, H, hd, cfg.rope_theta).reshape(T, H, hd)
        k = _rotate(xn @ w[("wk", l)].T, Hk, hd, cfg.rope_theta).reshape(T, Hk, hd)
        v = (xn @ w[("wv", l)].T).reshape(T, Hk, hd)
        k = np.repeat(k, H // Hk, axis=1)          # query head h uses key/value head h // (H / Hk)
        v = np.repeat(v, H // Hk, axis=1)
        s = np.einsum("thd,jhd->htj", q, k) / np.sqrt(hd)
        s = np.where(mask[None], s, -np.inf)
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        p = p / p.sum(axis=-1, keepdims=True)
        o = np.einsum("htj,jhd->thd", p, v).reshape(T, d)
        x = x + o @ w[("wo", l)].T
        xn = _rms(x, w[("g_ffn", l)], cfg.norm_eps)
        h1, h3 = xn @ w[("w1", l)].T, xn @ w[("w3", l)].T
        x = x + (h1 / (1 + np.exp(-h1)) * h3) @ w[("w2", l)].T
    return _rms(x, w["g_out"], cfg.norm_eps) @ w["cls"].T


CASES = [
    (ModelConfig(dim=32, n_layers=2, n_heads=4, hidden_dim=48, vocab_size=61, max_seq=12), 71, 12),
    (ModelConfig(dim=48, n_layers=3, n_heads=2, hidden_dim=64, vocab_size=53, max_seq=10, tied=False), 72, 10),
    (ModelConfig(dim=64, n_layers=2, n_heads=4, hidden_dim=96, vocab_size=97, max_seq=16, n_kv_heads=2), 73, 16),
    (ModelConfig(dim=64, n_layers=2, n_heads=4, hidden_dim=96, vocab_size=97, max_seq=16, n_kv_heads=1,
                 weight_bf16=True), 74, 16),
    # past max_seq: a window of 6 positions over 20
    (ModelConfig(dim=32, n_layers=2, n_heads=4, hidden_dim=48, vocab_size=61, max_seq=6, max_pos=20), 75, 20),
]


@pytest.mark.parametrize("cfg,seed,T", CASES)
def test_oracle_agrees_with_independent_numpy_forward(cfg, seed, T):
    om = O.OracleModel(cfg, seed)
    toks = O.synth_prompt(seed, 0, T, 0, cfg.vocab_size)
    ref = numpy_forward(om, cfg, toks)
    st = om.new_state()
    for p in range(T):
        r, lg = om.forward(st, int(toks[p]), p)
        assert r >= 0
        # float32 rounding of the oracle's stored intermediates: <= 1e-7 of the logits' scale
        err = np.abs(lg - ref[p]).max() / np.abs(ref[p]).max()
        assert err < 1e-6, (p, float(err))
        # and the greedy token wherever the top two are apart by more than the rounding
        srt = np.sort(ref[p])
        if srt[-1] - srt[-2] > 1e-4:
            assert r == int(np.argmax(ref[p])), p


def test_numpy_forward_is_sensitive_to_the_pieces_it_checks():
    """a window one wider, or (almost) no rotation, moves the logits by far more
    than the 1e-6 agreement above"""
    cfg, seed, T = CASES[4]
    om = O.OracleModel(cfg, seed)
    toks = O.synth_prompt(seed, 0, T, 0, cfg.vocab_size)
    ref = numpy_forward(om, cfg, toks)
    scale = np.abs(ref[-1]).max()
    wide = numpy_forward(om, ModelConfig(**{**cfg.__dict__, "max_seq": 7}), toks)
    assert np.abs(wide[-1] - ref[-1]).max() > 1e-2 * scale
    flat = numpy_forward(om, ModelConfig(**{**cfg.__dict__, "rope_theta": 1e9}), toks)
    assert np.abs(flat[-1] - ref[-1]).max() > 1e-4 * scale
