"""Decoding past max_seq on the GPU: the sliding window over a ring KV cache.

A model with max_pos > max_seq keeps running past max_seq; position p then
attends to positions p - max_seq + 1 .. p (the oracle's definition, pinned in
tests/test_oracle_pins.py).  Every logit is compared with the oracle through
and well past the point where the ring of KV slots wraps: batch-1 decode (GEMV
path), batched lockstep decode (GEMM path), prompts that cross max_seq and the
ring in one call (chunked so no chunk overwrites a slot it still reads) or in
pieces, matrix-core and vector prompt attention, bfloat16 weights, on-device
generation, and the rewind rule.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from transformer_llama_decode_amd.configs import ModelConfig
from tests.parity import assert_logits, assert_token

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# ring = round_up(max_seq, 64) + 64 slots per sequence
WIN_HD32 = ModelConfig(dim=128, n_layers=2, n_heads=4, hidden_dim=160, vocab_size=1001, max_seq=100,
                       max_pos=330, max_batch=3)                                   # ring 192
WIN_GQA64 = ModelConfig(dim=256, n_layers=2, n_heads=4, hidden_dim=192, vocab_size=1001, max_seq=70,
                        max_pos=300, max_batch=2, n_kv_heads=2)                    # ring 192
WIN_HD16 = ModelConfig(dim=64, n_layers=2, n_heads=4, hidden_dim=96, vocab_size=1003, max_seq=64,
                       max_pos=260, max_batch=3)                                   # ring 128
WIN_HD48_BF16 = ModelConfig(dim=192, n_layers=2, n_heads=4, hidden_dim=160, vocab_size=1001,
                            max_seq=90, max_pos=300, max_batch=2, weight_bf16=True)  # ring 192
WINDOWED = [(WIN_HD32, 51), (WIN_GQA64, 52), (WIN_HD16, 53), (WIN_HD48_BF16, 54)]


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_llama_decode_amd import model  # noqa: F401  (fails loudly if libld.so is missing)
    return torch.device("cuda", 0)


def _models(cfg, seed):
    from transformer_llama_decode_amd.model import LlamaDecoder
    return LlamaDecoder(cfg, seed), O.OracleModel(cfg, seed)


def _oracle_stream(om, prompt, n_pos):
    """oracle greedy run: tokens fed per position and logits per position"""
    st = om.new_state()
    feed, logits = [], []
    nxt = None
    for p in range(n_pos):
        t = int(prompt[p]) if p < len(prompt) else nxt
        r, lg = om.forward(st, t, p)
        assert r >= 0
        feed.append(t)
        logits.append(lg.copy())
        nxt = r
    return np.array(feed, np.int32), np.stack(logits)


@pytest.mark.parametrize("cfg,seed", WINDOWED)
def test_window_batch1_decode_every_logit(dev, cfg, seed):
    _say("window b1 decode", cfg)
    gm, om = _models(cfg, seed)
    feed, ref = _oracle_stream(om, [1], cfg.max_pos)
    logits = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    for p in range(cfg.max_pos):
        nxt = gm.decode_step(feed[p:p + 1], logits=logits)
        assert_logits(logits.cpu().numpy(), ref[p], "pos %d" % p)
        assert_token(int(nxt.cpu()[0]), ref[p], "pos %d" % p)
    assert gm.pos == cfg.max_pos
    assert gm.decode_step_rc([1]) == -2          # past max_pos
    assert gm.status() == 0
    gm.close()


@pytest.mark.parametrize("cfg,seed", [WINDOWED[0], WINDOWED[2]])
def test_window_batched_lockstep_every_logit(dev, cfg, seed):
    _say("window batched", cfg)
    B = cfg.max_batch
    gm, om = _models(cfg, seed)
    P, n = 5, cfg.max_pos
    prompts = np.stack([O.synth_prompt(seed, b, P, 0, cfg.vocab_size) for b in range(B)])
    refs = [_oracle_stream(om, prompts[b], n) for b in range(B)]
    lg = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    gm.prefill(prompts, logits=lg)
    for p in range(P, n):
        toks = np.array([refs[b][0][p] for b in range(B)], np.int32)
        nxt = gm.decode_step(toks, logits=lg).cpu().numpy()
        g = lg.cpu().numpy()
        for b in range(B):
            assert_logits(g[b], refs[b][1][p], "seq %d pos %d" % (b, p))
            assert_token(nxt[b], refs[b][1][p], "seq %d pos %d" % (b, p))
    gm.close()


@pytest.mark.parametrize("cfg,seed", WINDOWED)
def test_window_long_prompt_every_logit(dev, cfg, seed):
    """one prompt call past max_seq and past the ring (chunked by the library),
    every position's logits, then decoding on top of it"""
    _say("window long prompt", cfg)
    gm, om = _models(cfg, seed)
    B, P = 2, cfg.max_pos - 20
    prompts = np.stack([O.synth_prompt(seed, 40 + b, P, 0, cfg.vocab_size) for b in range(B)])
    allp = torch.empty((B, P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompts, logits=allp, all_pos=True).cpu().numpy()
    allp = allp.cpu().numpy()
    streams = [_oracle_stream(om, prompts[b], cfg.max_pos) for b in range(B)]
    for b in range(B):
        for p in range(P):
            assert_logits(allp[b, p], streams[b][1][p], "seq %d pos %d" % (b, p))
        assert_token(nxt[b], streams[b][1][P - 1], "seq %d next" % b)
    lg = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    for p in range(P, cfg.max_pos):
        gm.decode_step(np.array([streams[b][0][p] for b in range(B)], np.int32), logits=lg)
        g = lg.cpu().numpy()
        for b in range(B):
            assert_logits(g[b], streams[b][1][p], "seq %d decode pos %d" % (b, p))
    gm.close()


@pytest.mark.parametrize("cfg,seed", [WINDOWED[0], WINDOWED[1]])
def test_window_prompt_in_pieces_every_logit(dev, cfg, seed):
    """pieces that start before and after the ring wraps"""
    _say("window prompt pieces", cfg)
    gm, om = _models(cfg, seed)
    cuts = [0, 90, 170, 240, cfg.max_pos]
    prompt = O.synth_prompt(seed, 60, cfg.max_pos, 0, cfg.vocab_size)
    _, ref = _oracle_stream(om, prompt, cfg.max_pos)
    for a, b in zip(cuts[:-1], cuts[1:]):
        allp = torch.empty((1, b - a, cfg.vocab_size), dtype=torch.float32, device=dev)
        gm.prefill(prompt[None, a:b], logits=allp, all_pos=True)
        allp = allp.cpu().numpy()
        for i in range(b - a):
            assert_logits(allp[0, i], ref[a + i], "pos %d" % (a + i))
    assert gm.pos == cfg.max_pos
    gm.close()


@pytest.mark.parametrize("cfg,seed,B", [(WIN_HD32, 55, 1), (WIN_HD32, 56, 3), (WIN_GQA64, 57, 2)])
def test_window_generate_matches_oracle(dev, cfg, seed, B):
    """on-device generation (HIP graph, position in device memory) across the wrap"""
    _say("window generate", cfg, B)
    gm, om = _models(cfg, seed)
    P = 40
    prompts = np.stack([O.synth_prompt(seed, b, P, 0, cfg.vocab_size) for b in range(B)])
    first = gm.prefill(prompts).clone()
    n = cfg.max_pos - P
    logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    toks = gm.generate(first, n, logits=logits).cpu().numpy()
    assert gm.pos == cfg.max_pos and gm.status() == 0
    first = first.cpu().numpy()
    last = logits.cpu().numpy()
    for b in range(B):
        feed = np.concatenate([prompts[b], [first[b]], toks[:-1, b]])
        st = om.new_state()
        ref = []
        for p, t in enumerate(feed):
            r, lg = om.forward(st, int(t), p)
            assert r >= 0
            ref.append(lg.copy())
        assert_token(first[b], ref[P - 1], "seq %d prefill next" % b)
        for i in range(n):
            assert_token(toks[i, b], ref[P + i], "seq %d pos %d" % (b, P + i))
        assert_logits(last[b], ref[-1], "seq %d last step" % b)
    gm.close()


def test_window_rewind_rule_and_rerun(dev):
    """a rewind is allowed while the ring still holds the new position's window,
    and the rerun from there reproduces the logits bit for bit"""
    cfg, seed = WIN_HD32, 58                      # window 100, ring 192
    gm, _ = _models(cfg, seed)
    prompt = O.synth_prompt(seed, 0, 300, 0, cfg.vocab_size)
    gm.prefill(prompt[None, :250])
    assert gm.set_pos_rc(100) == -2               # 100 - 100 < 250 - 192: overwritten
    assert gm.pos == 250
    assert gm.set_pos_rc(157) == -2
    lg1 = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    lg2 = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    outs = []
    for p in range(250, 300):
        gm.decode_step(prompt[p:p + 1], logits=lg1)
        outs.append(lg1.cpu().numpy().copy())
    assert gm.set_pos_rc(258) == 0                # 258 - 100 >= 300 - 192
    for p in range(258, 300):
        gm.decode_step(prompt[p:p + 1], logits=lg2)
        assert np.array_equal(lg2.cpu().numpy(), outs[p - 250]), p
    gm.close()
