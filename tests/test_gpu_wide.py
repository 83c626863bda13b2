"""Every kernel at the 7B shape's real sizes, element by element against the oracle.

Two layers of the 7B shape (4096 wide, 32 heads of 128, 11008 hidden, 32000
vocabulary, untied classifier) run the same launches the 7B decode and prefill
time: the Q/K/V GEMV [12288 x 4096], W1/W3 [22016 x 4096], W2 [4096 x 11008],
the classifier [32000 x 4096], the split-K MFMA GEMMs with fp64 carries and the
matrix-core prompt attention at head dim 128.  Every logit of a 40-token prompt
and of 4 decode steps after it is compared with the oracle, for fp32 weights
with multi-head attention and for bfloat16 weights with 8 key/value heads, and
one layer run past max_seq over a wrapped ring.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

from oracle import oracle as O
from transformer_llama_decode_amd.configs import ModelConfig
from tests.parity import assert_logits, assert_token

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WIDE = ModelConfig(dim=4096, n_layers=2, n_heads=32, hidden_dim=11008, vocab_size=32000, max_seq=128,
                   tied=False)
WIDE_BF16_GQA = replace(WIDE, weight_bf16=True, n_kv_heads=8)


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_llama_decode_amd import model  # noqa: F401  (fails loudly if libld.so is missing)
    return torch.device("cuda", 0)


@pytest.mark.parametrize("cfg,seed", [(WIDE, 81), (WIDE_BF16_GQA, 82)])
def test_seven_b_shapes_every_logit(dev, cfg, seed):
    from transformer_llama_decode_amd.model import LlamaDecoder
    _say("7B-shape layers", cfg)
    P, D = 40, 4
    gm = LlamaDecoder(cfg, seed)
    prompt = O.synth_prompt(seed, 0, P, 3, cfg.vocab_size)
    allp = torch.empty((1, P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompt[None, :], logits=allp, all_pos=True)
    allp = allp.cpu().numpy()[0]
    first = int(nxt.cpu()[0])
    gpu_dec = []
    lg = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    feed = [first]
    for i in range(D):
        t = int(gm.decode_step(np.array([feed[-1]], np.int32), logits=lg).cpu()[0])
        gpu_dec.append(lg.cpu().numpy().copy())
        feed.append(t)
    gm.close()
    _say("oracle", cfg)
    om = O.OracleModel(cfg, seed, nthreads=16)
    st = om.new_state()
    for p in range(P):
        r, ref = om.forward(st, int(prompt[p]), p)
        assert r >= 0
        assert_logits(allp[p], ref, "prefill pos %d" % p)
    assert_token(first, ref, "prefill next")
    for i in range(D):
        r, ref = om.forward(st, feed[i], P + i)
        assert r >= 0
        assert_logits(gpu_dec[i], ref, "decode pos %d" % (P + i))
        assert_token(feed[i + 1], ref, "decode pos %d" % (P + i))
    om.close()


WIDE_WINDOW = replace(WIDE, n_layers=1, max_seq=64, max_pos=160)   # ring of 128 slots


def test_seven_b_shapes_past_max_seq_every_logit(dev):
    """the window at head dim 128: a 100-token prompt crosses max_seq (matrix-core prompt
    attention with window masks), 50 decode steps run past the 128-slot ring's wrap"""
    from transformer_llama_decode_amd.model import LlamaDecoder
    cfg, seed = WIDE_WINDOW, 83
    _say("7B-shape layer past max_seq", cfg)
    P, D = 100, 50
    gm = LlamaDecoder(cfg, seed)
    prompt = O.synth_prompt(seed, 0, P, 3, cfg.vocab_size)
    allp = torch.empty((1, P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompt[None, :], logits=allp, all_pos=True)
    allp = allp.cpu().numpy()[0]
    feed = [int(nxt.cpu()[0])]
    gpu_dec = []
    lg = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    for i in range(D):
        t = int(gm.decode_step(np.array([feed[-1]], np.int32), logits=lg).cpu()[0])
        gpu_dec.append(lg.cpu().numpy().copy())
        feed.append(t)
    assert gm.pos == P + D
    gm.close()
    om = O.OracleModel(cfg, seed, nthreads=16)
    st = om.new_state()
    for p in range(P):
        r, ref = om.forward(st, int(prompt[p]), p)
        assert r >= 0
        assert_logits(allp[p], ref, "prefill pos %d" % p)
    for i in range(D):
        r, ref = om.forward(st, feed[i], P + i)
        assert r >= 0
        assert_logits(gpu_dec[i], ref, "decode pos %d" % (P + i))
        assert_token(feed[i + 1], ref, "decode pos %d" % (P + i))
    om.close()
