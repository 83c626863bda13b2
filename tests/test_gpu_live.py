"""GPU parity of the two batch-1 TinyStories-shape workloads against the oracle
run live, every logit of every step.

The 15M shape (288/6L/6H, start token 1, positions 0..255) and the 44M shape
(512/8L/8H, a 64-token prompt, then decode to position 1023) are small enough
for the oracle to follow the GPU step by step in seconds: the oracle runs each
position first, the GPU is fed the same token (teacher forcing on the oracle's
greedy stream) in the configuration the benchmark times (prefill of the prompt,
then one decode step per position), and all 32000 logits are compared at the
last prompt position and at every decode step, together with the greedy token
wherever the oracle's top-1 margin exceeds 1e-3.  The worst |gpu - oracle| /
tolerance is printed.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from transformer_llama_decode_amd.configs import WORKLOADS
from tests.parity import REL, ABS, MARGIN

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _live(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_llama_decode_amd.model import LlamaDecoder
    w = WORKLOADS[name]
    cfg, V = w.model, w.model.vocab_size
    dev = torch.device("cuda", 0)
    gm = LlamaDecoder(cfg, w.model_seed)
    om = O.OracleModel(cfg, w.model_seed)
    st = om.new_state()
    prompt = (O.synth_prompt(w.prompt_seed, 0, w.prompt_len) if w.prompt_len > 0
              else np.array([w.start_token], np.int32))
    P = len(prompt)
    ref = np.empty(V, np.float32)
    logits = torch.empty((1, V), dtype=torch.float32, device=dev)
    fails, worst, nchk = [], 0.0, 0

    def compare(p, nxt):
        nonlocal worst, nchk
        g = logits[0].cpu().numpy().astype(np.float64)
        o = ref.astype(np.float64)
        r = np.abs(g - o) / np.maximum(REL * np.abs(o), ABS)
        worst = max(worst, float(r.max()))
        nchk += 1
        if (r > 1).any():
            i = int(np.argmax(r))
            fails.append("pos %d: %d of %d logits out of tolerance; worst at %d: gpu %.9g oracle %.9g"
                         % (p, int((r > 1).sum()), V, i, g[i], o[i]))
        top = int(np.argmax(ref))
        second = np.max(np.delete(ref, top))
        if ref[top] - second > MARGIN and int(nxt) != top:
            fails.append("pos %d: gpu token %d, oracle token %d" % (p, int(nxt), top))

    # the prompt: oracle position by position, the GPU in one prefill
    nxt_o = None
    for p in range(P):
        nxt_o, _ = om.forward(st, int(prompt[p]), p, ref)
        assert nxt_o >= 0
    if w.prompt_len > 0:
        nxt = gm.prefill(prompt[None, :], logits=logits)
        compare(P - 1, nxt.cpu().numpy()[0])
    else:
        nxt = gm.decode_step(prompt[:1], logits=logits)
        compare(0, nxt.cpu().numpy()[0])
    # decode: both fed the oracle's greedy token of the previous position
    for p in range(P, w.end_pos):
        t = nxt_o
        nxt_o, _ = om.forward(st, t, p, ref)
        assert nxt_o >= 0
        nxt = gm.decode_step(np.array([t], np.int32), logits=logits)
        compare(p, nxt.cpu().numpy()[0])
        if p % 256 == 0:
            _say("%s: pos %d" % (name, p))
    assert gm.status() == 0
    gm.close()
    om.close()
    _say("%s live parity: %d positions x %d logits, worst |gpu - oracle| / tol %.3f, %d failures"
         % (name, nchk, V, worst, len(fails)))
    assert nchk == w.end_pos - (P - 1 if w.prompt_len > 0 else 0)
    assert not fails, fails[:10]


@pytest.mark.timeout(300)
def test_live_C1_every_logit_every_step():
    _live("C1")


@pytest.mark.timeout(600)
def test_live_C2_every_logit_every_step():
    _live("C2")
