"""Every kernel at the 7B shape's real sizes, element by element against the oracle.

Two layers of the 7B shape (4096 wide, 32 heads of 128, 11008 hidden, 32000
vocabulary, untied classifier) run the same launches the 7B decode and prefill
time: the Q/K/V GEMV [12288 x 4096], W1/W3 [22016 x 4096], W2 [4096 x 11008],
the classifier [32000 x 4096], the split-K MFMA GEMMs with fp64 carries and the
fp64 prompt attention that wide models keep (head dim 128).  Every logit of a 40-token prompt
and of 4 decode steps after it is compared with the oracle, for fp32 weights
with multi-head attention and for bfloat16 weights with 8 key/value heads, and
one layer run past max_seq over a wrapped ring.  A 2048-wide layer run as a
batch of sequences takes the small-problem GEMM with 32-wide tiles, K split
over workgroups and fp64 carries; the same layer under a 520-token prompt takes
the LDS-tiled GEMM with fp64 carries.
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
    """the window at head dim 128: a 100-token prompt crosses max_seq (prompt attention
    with window masks), 50 decode steps run past the 128-slot ring's wrap"""
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


# 2048 wide: fp64 carries in the matrix-core sums; at 4 x 8 rows (and 4 in decode)
# the Q/K/V GEMM takes 192 tiles of 32 x 32 in one K slice each (with 4 key/value
# heads: 96 tiles, K split over 6 workgroups), Wo and W2 64 such tiles with K split
# over 8 workgroups
MID_BATCH = ModelConfig(dim=2048, n_layers=1, n_heads=16, hidden_dim=5632, vocab_size=4096, max_seq=32,
                        max_batch=4, tied=False)


@pytest.mark.parametrize("cfg,seed", [(MID_BATCH, 84), (replace(MID_BATCH, weight_bf16=True, n_kv_heads=4), 85)])
def test_batched_split_k_with_carries_every_logit(dev, cfg, seed):
    from transformer_llama_decode_amd.model import LlamaDecoder
    _say("2048-wide batch", cfg)
    B, P, D = cfg.max_batch, 8, 3
    gm = LlamaDecoder(cfg, seed)
    prompts = np.stack([O.synth_prompt(seed, b, P, 3, cfg.vocab_size) for b in range(B)])
    allp = torch.empty((B, P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompts, logits=allp, all_pos=True)
    allp = allp.cpu().numpy()
    feed = [nxt.cpu().numpy().astype(np.int32)]
    dec = []
    lg = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    for i in range(D):
        t = gm.decode_step(feed[-1], logits=lg).cpu().numpy().astype(np.int32)
        dec.append(lg.cpu().numpy().copy())
        feed.append(t)
    gm.close()
    om = O.OracleModel(cfg, seed, nthreads=16)
    for b in range(B):
        st = om.new_state()
        for p in range(P):
            r, ref = om.forward(st, int(prompts[b, p]), p)
            assert r >= 0
            assert_logits(allp[b, p], ref, "seq %d prefill pos %d" % (b, p))
        assert_token(int(feed[0][b]), ref, "seq %d prefill next" % b)
        for i in range(D):
            r, ref = om.forward(st, int(feed[i][b]), P + i)
            assert r >= 0
            assert_logits(dec[i][b], ref, "seq %d decode pos %d" % (b, P + i))
            assert_token(int(feed[i + 1][b]), ref, "seq %d decode pos %d" % (b, P + i))
    om.close()


# 2048 wide, a 520-token prompt: more than 256 rows, so every projection takes the
# LDS-tiled MFMA GEMM with fp64 carries (128-row tiles and a ragged 8-row tail), and
# prompt attention the fp64 vector path that wide models keep
MID_PROMPT = ModelConfig(dim=2048, n_layers=1, n_heads=16, hidden_dim=5632, vocab_size=4096, max_seq=576,
                         tied=False)


@pytest.mark.parametrize("cfg,seed", [(MID_PROMPT, 86), (replace(MID_PROMPT, weight_bf16=True, n_kv_heads=4), 87)])
def test_wide_long_prompt_tiled_gemm_every_logit(dev, cfg, seed):
    from transformer_llama_decode_amd.model import LlamaDecoder
    _say("2048-wide 520-token prompt", cfg)
    P = 520
    gm = LlamaDecoder(cfg, seed)
    prompt = O.synth_prompt(seed, 0, P, 3, cfg.vocab_size)
    allp = torch.empty((1, P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompt[None, :], logits=allp, all_pos=True)
    allp = allp.cpu().numpy()[0]
    first = int(nxt.cpu()[0])
    gm.close()
    om = O.OracleModel(cfg, seed, nthreads=16)
    st = om.new_state()
    for p in range(P):
        r, ref = om.forward(st, int(prompt[p]), p)
        assert r >= 0
        assert_logits(allp[p], ref, "prefill pos %d" % p)
    assert_token(first, ref, "prefill next")
    om.close()
