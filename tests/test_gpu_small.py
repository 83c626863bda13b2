"""GPU parity at sizes the oracle finishes in seconds, element by element.

Every logit of every step is compared with the oracle (teacher forcing on the
oracle's own greedy tokens), over shapes that span several tiles and ragged
tails: widths that are not multiples of the 128-wide GEMM tiles, vocabularies
of odd size, head dims 16..64, prompts that cross 64-position KV tiles.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from transformer_llama_decode_amd.configs import (TINY, TINY_UNTIED, SMALL, TINY_GQA, SMALL_MQA,
                                                   GQA_HD64, TINY_BF16, SMALL_BF16, ModelConfig)
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


CASES = [
    (TINY, 7),
    (TINY_UNTIED, 8),
    (SMALL, 9),
    (ModelConfig(dim=96, n_layers=2, n_heads=6, hidden_dim=160, vocab_size=777, max_seq=70,
                 max_batch=3), 10),
    # grouped-query / multi-query attention (key/value heads shared by query-head groups)
    (TINY_GQA, 17),
    (SMALL_MQA, 18),
    (GQA_HD64, 19),
    # bfloat16 weights
    (TINY_BF16, 23),
    (SMALL_BF16, 24),
    # a long FFN: the batch-1 W2 projection stages 20480 inputs (80 KiB) in LDS,
    # past the default 64 KiB dynamic limit
    (ModelConfig(dim=64, n_layers=2, n_heads=4, hidden_dim=20480, vocab_size=301, max_seq=24,
                 max_batch=3), 25),
]


@pytest.mark.parametrize("cfg,seed", CASES)
def test_weights_on_device_are_the_generator_values(dev, cfg, seed):
    """bit-identical to the oracle's weights: the generator's draws, for bfloat16
    weights rounded to nearest even (the library rounds by scaling on the host,
    the oracle on the bit pattern)"""
    _say("weights", cfg)
    gm, om = _models(cfg, seed)
    L = cfg.n_layers
    ids = [0] + list(range(1, 1 + 7 * L)) + ([] if cfg.tied else [1 + 7 * L])
    for sid in ids:
        if sid == 0 or sid == 1 + 7 * L:
            n = cfg.vocab_size * cfg.dim
        else:
            kind = (sid - 1) % 7
            n = cfg.dim * (cfg.hidden_dim if kind in (4, 5, 6) else
                           cfg.kv_dim if kind in (1, 2) else cfg.dim)
        got = gm.read_weights(sid, 0, n)
        want = om.tensor(sid)
        assert want.size == n
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), sid
        if not cfg.weight_bf16:
            assert np.array_equal(want, O.synth_normal(seed, sid, 0, n)), sid
    # the library's whole-model checksum: sum of the elements' 32-bit patterns mod 2^64
    want_sum = 0
    for sid in ids:
        want_sum = (want_sum + int(om.tensor(sid).view(np.uint32).astype(np.uint64).sum(dtype=np.uint64))) % 2**64
    assert gm.weights_checksum() == want_sum
    gm.close()


@pytest.mark.parametrize("cfg,seed", CASES)
def test_batch1_decode_every_logit(dev, cfg, seed):
    _say("b1 decode", cfg)
    gm, om = _models(cfg, seed)
    feed, ref = _oracle_stream(om, [1], cfg.max_seq)
    logits = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    for p in range(cfg.max_seq):
        nxt = gm.decode_step(feed[p:p + 1], logits=logits)
        g = logits.cpu().numpy()
        assert_logits(g, ref[p], "pos %d" % p)
        assert_token(int(nxt.cpu()[0]), ref[p], "pos %d" % p)
    assert gm.pos == cfg.max_seq
    assert gm.status() == 0
    gm.close()


@pytest.mark.parametrize("cfg,seed", CASES)
def test_prefill_then_decode_every_logit(dev, cfg, seed):
    _say("prefill", cfg)
    gm, om = _models(cfg, seed)
    P = min(cfg.max_seq - 3, 67)   # crosses a 64-position tile
    prompt = O.synth_prompt(seed, 0, P, 0, cfg.vocab_size)
    feed, ref = _oracle_stream(om, prompt, cfg.max_seq)
    allp = torch.empty((P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompt[None, :], logits=allp, all_pos=True)
    allp = allp.cpu().numpy()
    for p in range(P):
        assert_logits(allp[p], ref[p], "prefill pos %d" % p)
    assert_token(int(nxt.cpu()[0]), ref[P - 1], "prefill next")
    logits = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    for p in range(P, cfg.max_seq):
        gm.decode_step(feed[p:p + 1], logits=logits)
        assert_logits(logits.cpu().numpy(), ref[p], "decode pos %d" % p)
    gm.close()


@pytest.mark.parametrize("cfg,seed", CASES)
def test_prefill_last_logits_equal_sequential_decode(dev, cfg, seed):
    gm, _ = _models(cfg, seed)
    P = min(cfg.max_seq, 40)
    prompt = O.synth_prompt(seed, 1, P, 0, cfg.vocab_size)
    lg_pre = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    gm.prefill(prompt[None, :], logits=lg_pre)
    lg_pre = lg_pre.cpu().numpy()
    gm.kv_reset()
    lg = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    for p in range(P):
        gm.decode_step(prompt[p:p + 1], logits=lg)
    # GEMM (MFMA) and GEMV paths accumulate differently: equal within the tolerance
    assert_logits(lg_pre, lg.cpu().numpy(), "prefill vs decode")
    gm.close()


@pytest.mark.parametrize("cfg,seed", CASES)
def test_batched_lockstep_matches_each_sequence_alone(dev, cfg, seed):
    _say("batched", cfg)
    B = cfg.max_batch
    if B < 2:
        pytest.skip("single-sequence config")
    gm, om = _models(cfg, seed)
    P = 5
    prompts = np.stack([O.synth_prompt(seed, b, P, 0, cfg.vocab_size) for b in range(B)])
    refs = [_oracle_stream(om, prompts[b], cfg.max_seq) for b in range(B)]
    lg = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompts, logits=lg)
    g = lg.cpu().numpy()
    for b in range(B):
        assert_logits(g[b], refs[b][1][P - 1], "seq %d prefill" % b)
        assert_token(int(nxt.cpu()[b]), refs[b][1][P - 1], "seq %d prefill" % b)
    for p in range(P, cfg.max_seq):
        toks = np.array([refs[b][0][p] for b in range(B)], np.int32)
        nxt = gm.decode_step(toks, logits=lg)
        g = lg.cpu().numpy()
        nn = nxt.cpu().numpy()
        for b in range(B):
            assert_logits(g[b], refs[b][1][p], "seq %d pos %d" % (b, p))
            assert_token(nn[b], refs[b][1][p], "seq %d pos %d" % (b, p))
    gm.close()


@pytest.mark.parametrize("cfg,seed", [(TINY, 11), (SMALL, 12), (SMALL_MQA, 13), (SMALL_BF16, 14)])
def test_many_row_prefill_every_logit(dev, cfg, seed):
    # more than 256 rows per forward pass: the LDS-tiled MFMA GEMM path
    # (smaller row counts take the split-K path exercised above)
    _say("many-row prefill", cfg)
    B = cfg.max_batch
    P = min(cfg.max_seq, 300 // B + 1)
    assert B * P > 256
    gm, om = _models(cfg, seed)
    prompts = np.stack([O.synth_prompt(seed, 10 + b, P, 0, cfg.vocab_size) for b in range(B)])
    allp = torch.empty((B, P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompts, logits=allp, all_pos=True)
    allp = allp.cpu().numpy()
    nn = nxt.cpu().numpy()
    for b in range(B):
        _, ref = _oracle_stream(om, prompts[b], P)
        for p in range(P):
            assert_logits(allp[b, p], ref[p], "seq %d pos %d" % (b, p))
        assert_token(nn[b], ref[P - 1], "seq %d next" % b)
    gm.close()


def test_device_token_feedback_equals_host_tokens(dev):
    cfg, seed = TINY, 3
    gm, _ = _models(cfg, seed)
    lg = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)
    out_host, toks = [], [1]
    for p in range(20):
        nxt = gm.decode_step(np.array(toks[-1:], np.int32), logits=lg)
        out_host.append(lg.cpu().numpy().copy())
        toks.append(int(nxt.cpu()[0]))
    gm.kv_reset()
    nxt = torch.tensor([1], dtype=torch.int32, device=dev)
    buf = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(2)]
    for p in range(20):
        out = buf[p % 2]
        gm.decode_step(nxt, logits=lg, next_out=out)
        nxt = out
        assert np.array_equal(lg.cpu().numpy(), out_host[p]), p
        assert int(out.cpu()[0]) == toks[p + 1]
    gm.close()


def test_reset_rerun_and_run_to_run_bit_identical(dev):
    cfg, seed = SMALL, 4
    gm, _ = _models(cfg, seed)
    prompt = O.synth_prompt(seed, 0, 17, 0, cfg.vocab_size)
    lg = torch.empty(cfg.vocab_size, dtype=torch.float32, device=dev)

    def run():
        gm.kv_reset()
        gm.prefill(prompt[None, :])
        outs = []
        t = np.array([5], np.int32)
        for _ in range(30):
            nxt = gm.decode_step(t, logits=lg)
            outs.append(lg.cpu().numpy().copy())
            t = nxt.cpu().numpy()
        return outs
    a = run()
    b = run()
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    gm.close()


def test_error_paths_leave_state_unchanged(dev):
    from transformer_llama_decode_amd._lib import LD_E_INVAL, LD_E_RANGE
    cfg, seed = TINY, 5
    gm, _ = _models(cfg, seed)
    assert gm.decode_step_rc([cfg.vocab_size]) == LD_E_INVAL
    assert gm.decode_step_rc([-1]) == LD_E_INVAL
    assert gm.decode_step_rc(np.zeros(cfg.max_batch + 1, np.int32)) == LD_E_INVAL
    assert gm.pos == 0
    assert gm.prefill_rc(np.zeros((1, cfg.max_seq + 1), np.int32)) == LD_E_RANGE
    assert gm.pos == 0
    gm.prefill(np.zeros((1, cfg.max_seq - 1), np.int32))
    assert gm.prefill_rc(np.zeros((1, 2), np.int32)) == LD_E_RANGE
    assert gm.pos == cfg.max_seq - 1
    gm.decode_step([3])
    assert gm.decode_step_rc([3]) == LD_E_RANGE
    assert gm.pos == cfg.max_seq
    from transformer_llama_decode_amd._lib import LdError
    with pytest.raises(LdError):
        gm.set_pos(cfg.max_seq + 1)
    gm.set_pos(10)
    assert gm.pos == 10
    assert gm.status() == 0
    gm.close()


@pytest.mark.parametrize("batch", [1, 3])
def test_poisoned_weight_is_reported(dev, batch):
    """a NaN planted in one embedding row reaches exactly one logit through the
    tied classifier; the classifier's non-finite check must report it"""
    from transformer_llama_decode_amd._lib import LD_E_NONFINITE
    cfg, seed = TINY, 6
    gm, _ = _models(cfg, seed)
    V, d = cfg.vocab_size, cfg.dim
    j, t = 17, 5                                   # poisoned row j, fed token t != j
    E = gm.arena[:V * d * 4].view(torch.float32)  # the embedding sits at arena offset 0
    E[j * d + 3] = float("nan")
    logits = torch.empty((batch, V), dtype=torch.float32, device=dev)
    gm.decode_step(np.full(batch, t, np.int32), logits=logits)
    assert gm.status() == LD_E_NONFINITE
    assert gm.status() == 0                        # cleared after reporting
    g = logits.cpu().numpy()
    assert np.isnan(g[:, j]).all()
    assert np.isfinite(np.delete(g, j, axis=1)).all()
    # the prompt path (per-row classifier of each sequence's last position)
    gm.kv_reset()
    prompts = np.full((batch, 6), t, np.int32)
    gm.prefill(prompts, logits=logits)
    assert gm.status() == LD_E_NONFINITE
    # a finite table again: no report
    E[j * d + 3] = 0.0
    gm.kv_reset()
    gm.decode_step(np.full(batch, t, np.int32), logits=logits)
    assert gm.status() == 0
    gm.close()


def test_out_of_range_device_token_is_reported(dev):
    from transformer_llama_decode_amd._lib import LD_E_NONFINITE
    cfg, seed = TINY, 6
    gm, _ = _models(cfg, seed)
    bad = torch.tensor([cfg.vocab_size + 5], dtype=torch.int32, device=dev)
    gm.decode_step(bad)
    assert gm.status() == LD_E_NONFINITE
    assert gm.status() == 0          # cleared after reporting
    gm.close()



LONG = [
    # head dim 32 and 64 (grouped-query): the matrix-core prompt attention
    (ModelConfig(dim=128, n_layers=2, n_heads=4, hidden_dim=160, vocab_size=1001, max_seq=330,
                 max_batch=2), 41),
    (ModelConfig(dim=256, n_layers=2, n_heads=4, hidden_dim=192, vocab_size=1001, max_seq=330,
                 max_batch=2, n_kv_heads=2), 42),
    # head dim 96 (three 32-dimension output tiles) and 128 (multi-query)
    (ModelConfig(dim=192, n_layers=2, n_heads=2, hidden_dim=160, vocab_size=1001, max_seq=330,
                 max_batch=2), 43),
    (ModelConfig(dim=256, n_layers=2, n_heads=2, hidden_dim=192, vocab_size=1001, max_seq=330,
                 max_batch=2, n_kv_heads=1), 44),
    # bfloat16 weights, grouped-query
    (ModelConfig(dim=256, n_layers=2, n_heads=4, hidden_dim=192, vocab_size=1001, max_seq=330,
                 max_batch=2, n_kv_heads=2, weight_bf16=True), 46),
    # head dim 48: not a multiple of 32, rows share K/V tiles on the vector units
    (ModelConfig(dim=192, n_layers=2, n_heads=4, hidden_dim=160, vocab_size=1001, max_seq=330,
                 max_batch=2), 45),
]


@pytest.mark.parametrize("cfg,seed", LONG)
def test_long_prompt_prefill_every_logit(dev, cfg, seed):
    """prompts of 301 rows (ragged against 32-row and 8-row groups, 64-key tiles)"""
    _say("long prompt", cfg)
    gm, om = _models(cfg, seed)
    B, P = 2, 301                           # ragged: 301 rows = 37 groups of 8 + 5
    prompts = np.stack([O.synth_prompt(seed, 20 + b, P, 0, cfg.vocab_size) for b in range(B)])
    allp = torch.empty((B, P, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompts, logits=allp, all_pos=True)
    allp = allp.cpu().numpy()
    nn = nxt.cpu().numpy()
    for b in range(B):
        _, ref = _oracle_stream(om, prompts[b], P)
        for p in range(P):
            assert_logits(allp[b, p], ref[p], "seq %d pos %d" % (b, p))
        assert_token(nn[b], ref[P - 1], "seq %d next" % b)
    # then decode on top of the prompt's cache
    lg = torch.empty((B, cfg.vocab_size), dtype=torch.float32, device=dev)
    feed, refs = [], []
    for b in range(B):
        f, r = _oracle_stream(om, prompts[b], P + 8)
        feed.append(f)
        refs.append(r)
    for p in range(P, P + 8):
        gm.decode_step(np.array([feed[b][p] for b in range(B)], np.int32), logits=lg)
        g = lg.cpu().numpy()
        for b in range(B):
            assert_logits(g[b], refs[b][p], "seq %d decode pos %d" % (b, p))
    gm.close()


@pytest.mark.parametrize("cfg,seed", [LONG[1], LONG[3], LONG[4]])
def test_prompt_in_two_pieces_every_logit(dev, cfg, seed):
    """a prompt fed as 100 + 201 tokens: the second piece attends to the first
    piece's cache entries at positions below its own rows"""
    _say("prompt in two pieces", cfg)
    gm, om = _models(cfg, seed)
    B, P1, P2 = 2, 100, 201
    prompts = np.stack([O.synth_prompt(seed, 30 + b, P1 + P2, 0, cfg.vocab_size) for b in range(B)])
    gm.prefill(prompts[:, :P1])
    allp = torch.empty((B, P2, cfg.vocab_size), dtype=torch.float32, device=dev)
    nxt = gm.prefill(prompts[:, P1:], logits=allp, all_pos=True)
    assert gm.pos == P1 + P2
    allp = allp.cpu().numpy()
    nn = nxt.cpu().numpy()
    for b in range(B):
        _, ref = _oracle_stream(om, prompts[b], P1 + P2)
        for i in range(P2):
            assert_logits(allp[b, i], ref[P1 + i], "seq %d pos %d" % (b, P1 + i))
        assert_token(nn[b], ref[P1 + P2 - 1], "seq %d next" % b)
    gm.close()
