"""On-device greedy generation (ld_generate: HIP graphs of 8 steps, then of one step, replayed).

The generated tokens are checked against the oracle teacher-forced with those
same tokens: at every position the GPU's token must be the oracle's arg-max
wherever the oracle's top-1 minus top-2 exceeds the margin, and the last
step's logits must match the oracle's element by element.  Both the GEMV path
(batch 1) and the GEMM path (batch > 1), prompts that cross 64-position tiles,
and runs to the end of the KV cache.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from transformer_llama_decode_amd.configs import (TINY, TINY_UNTIED, SMALL, TINY_GQA, SMALL_MQA,
                                                   TINY_BF16, SMALL_BF16, ModelConfig)
from tests.parity import assert_logits, assert_token

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_llama_decode_amd import model  # noqa: F401  (fails loudly if libld.so is missing)
    return torch.device("cuda", 0)


def _gpu(cfg, seed):
    from transformer_llama_decode_amd.model import LlamaDecoder
    return LlamaDecoder(cfg, seed)


def _oracle_forced(om, feed):
    """oracle logits at positions 0..len(feed)-1 with the given input tokens"""
    st = om.new_state()
    out = []
    for p, t in enumerate(feed):
        r, lg = om.forward(st, int(t), p)
        assert r >= 0
        out.append(lg.copy())
    return np.stack(out)


CASES = [
    (TINY, 7, 1),
    (TINY, 7, 5),
    (TINY_UNTIED, 8, 1),
    (SMALL, 9, 1),
    (SMALL, 9, 3),
    (ModelConfig(dim=96, n_layers=2, n_heads=6, hidden_dim=160, vocab_size=777, max_seq=70,
                 max_batch=3), 10, 2),
    (TINY_GQA, 17, 1),
    (TINY_GQA, 17, 5),
    (SMALL_MQA, 18, 3),
    (TINY_BF16, 25, 1),
    (SMALL_BF16, 26, 4),
]


@pytest.mark.parametrize("cfg,seed,B", CASES)
def test_generate_matches_oracle(dev, cfg, seed, B):
    _say("generate", cfg, "batch", B)
    gm = _gpu(cfg, seed)
    om = O.OracleModel(cfg, seed)
    P = min(cfg.max_seq // 2, 67)
    prompts = np.stack([O.synth_prompt(seed, b, P, 0, cfg.vocab_size) for b in range(B)])
    first = gm.prefill(prompts).clone()
    n = cfg.max_seq - P                              # to the end of the cache
    logits = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    toks = gm.generate(first, n, logits=logits).cpu().numpy()
    assert toks.shape == (n, B)
    assert gm.pos == cfg.max_seq
    assert gm.status() == 0
    last = logits.cpu().numpy()
    first = first.cpu().numpy()
    for b in range(B):
        feed = np.concatenate([prompts[b], [first[b]], toks[:-1, b]])
        ref = _oracle_forced(om, feed)
        assert_token(first[b], ref[P - 1], "seq %d prefill next" % b)
        for i in range(n):
            assert_token(toks[i, b], ref[P + i], "seq %d pos %d" % (b, P + i))
        assert_logits(last[b], ref[-1], "seq %d last step" % b)
    gm.close()


@pytest.mark.parametrize("B", [1, 4])
def test_generate_in_pieces_equals_one_call(dev, B):
    """the device position and token feedback carry across calls: n1 + n2 steps == one call"""
    cfg, seed = TINY, 11
    a, b = _gpu(cfg, seed), _gpu(cfg, seed)
    prompt = np.stack([O.synth_prompt(seed, s, 20, 0, cfg.vocab_size) for s in range(B)])
    fa, fb = a.prefill(prompt).clone(), b.prefill(prompt).clone()
    la = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    lb = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    whole = a.generate(fa, 30, logits=la)
    p1 = b.generate(fb, 13, logits=lb)
    p2 = b.generate(p1[-1].clone(), 17, logits=lb)
    assert torch.equal(whole, torch.cat([p1, p2]))
    assert torch.equal(la, lb)
    assert a.pos == b.pos == 50
    a.close()
    b.close()


def test_generate_rewind_is_bit_identical(dev):
    cfg, seed = SMALL, 12
    gm = _gpu(cfg, seed)
    prompt = O.synth_prompt(seed, 0, 70, 0, cfg.vocab_size)
    first = gm.prefill(prompt).clone()
    l1 = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    l2 = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    t1 = gm.generate(first, 40, logits=l1).clone()
    gm.set_pos(70)
    t2 = gm.generate(first, 40, logits=l2)        # a new logits buffer: the step is recaptured
    assert torch.equal(t1, t2)
    assert torch.equal(l1, l2)
    gm.close()


def test_generate_agrees_with_decode_step_loop(dev):
    """same tokens as the eager per-step path fed with its own device tokens"""
    cfg, seed = SMALL, 13
    a, b = _gpu(cfg, seed), _gpu(cfg, seed)
    prompt = O.synth_prompt(seed, 0, 30, 0, cfg.vocab_size)
    fa, fb = a.prefill(prompt).clone(), b.prefill(prompt).clone()
    n = 60
    gen = a.generate(fa, n).cpu().numpy()[:, 0]
    lg = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    cur = fb
    for i in range(n):
        cur = b.decode_step(cur, logits=lg).clone()
        # near-ties may legitimately resolve differently (different attention split)
        v = np.sort(lg.cpu().numpy())
        if v[-1] - v[-2] <= 1e-3:
            break
        assert int(cur.cpu()[0]) == gen[i], "step %d" % i
    a.close()
    b.close()


def test_generate_errors_leave_state(dev):
    cfg, seed = TINY, 14
    gm = _gpu(cfg, seed)
    gm.prefill(O.synth_prompt(seed, 0, 10, 0, cfg.vocab_size))
    assert gm.generate_rc([1], cfg.max_seq) == -2            # past max_seq
    assert gm.pos == 10
    assert gm.generate_rc([cfg.vocab_size], 3) == -1         # bad host token
    assert gm.generate_rc([1] * (cfg.max_batch + 1), 3) == -1
    assert gm.generate_rc([1], -1) == -1
    assert gm.pos == 10
    assert gm.generate_rc([1], 0) == 0                       # nothing to do
    assert gm.pos == 10
    assert gm.generate_rc([1], cfg.max_seq - 10) == 0        # exactly to the end
    assert gm.pos == cfg.max_seq
    assert gm.status() == 0
    gm.close()


def test_generate_out_of_range_device_token_is_flagged(dev):
    cfg, seed = TINY, 15
    gm = _gpu(cfg, seed)
    bad = torch.tensor([cfg.vocab_size + 5], dtype=torch.int32, device=dev)
    gm.generate(bad, 2)
    assert gm.status() == -5
    assert gm.status() == 0
    gm.close()
