"""The allocation-free decode entry point (ld_decode_step_noalloc) against the
ordinary one (ld_decode_step), through the C ABI.

Two handles of the same model and seed are fed the same tokens, one through
each entry point, and every logit and greedy token must be identical bit for
bit (the same kernels run on the same values; only where the step's scratch
lives differs), on consecutive calls whose second one is smaller (fewer rows,
so the static array's contents from the larger call are still there), on the
batch-1 path (GEMV projections, split attention heads) and the batched one
(split-K GEMMs with their tickets in the static array).  A step that needs more
scratch than the array holds is refused with LD_E_SCRATCH and changes nothing.
"""
import sys

import numpy as np
import pytest

from transformer_llama_decode_amd.configs import TINY, ModelConfig
from oracle import oracle as O
from tests.parity import assert_logits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_llama_decode_amd import model  # noqa: F401
    return torch.device("cuda", 0)


def _pair(cfg, seed):
    from transformer_llama_decode_amd.model import LlamaDecoder
    return LlamaDecoder(cfg, seed), LlamaDecoder(cfg, seed)


# (model, seed, batches of consecutive calls: each later call no larger)
CASES = [
    (TINY, 31, [5, 5, 3, 1, 1]),
    (ModelConfig(dim=128, n_layers=2, n_heads=2, hidden_dim=352, vocab_size=4099, max_seq=200,
                 max_batch=4, n_kv_heads=1), 32, [4, 2, 1]),
]


@pytest.mark.parametrize("cfg,seed,batches", CASES)
def test_noalloc_step_equals_the_ordinary_step(dev, cfg, seed, batches):
    from transformer_llama_decode_amd._lib import LD_OK
    _say("noalloc vs ordinary", cfg, batches)
    a, b = _pair(cfg, seed)
    om = O.OracleModel(cfg, seed)
    V = cfg.vocab_size
    # a prompt long enough that batch-1 attention splits heads into chunks (tickets)
    P = 150 if cfg.max_seq >= 200 else 40
    B0 = batches[0]
    prompts = np.stack([O.synth_prompt(seed, 60 + s, P, 0, V) for s in range(B0)])
    a.prefill(prompts)
    b.prefill(prompts)
    toks = [int(t) for t in prompts[:, -1]]
    refs = [om.new_state() for _ in range(B0)]
    for s in range(B0):
        for p in range(P):
            om.forward(refs[s], int(prompts[s, p]), p)
    la = torch.empty((B0, V), dtype=torch.float32, device=dev)
    lb = torch.full((B0, V), float("nan"), dtype=torch.float32, device=dev)
    for i, B in enumerate(batches):
        p = P + i
        tok = np.array([(7 * i + 11 * s + 5) % V for s in range(B)], np.int32)
        na = a.decode_step(tok, logits=la[:B]).clone()
        rc, nb = b.decode_step_noalloc(tok, logits=lb[:B])
        assert rc == LD_OK
        assert torch.equal(la[:B].view(torch.int32), lb[:B].view(torch.int32)), "call %d (batch %d)" % (i, B)
        assert torch.equal(na, nb[:B]), "call %d (batch %d)" % (i, B)
        # and both against the oracle (sequence s of this call)
        g = lb[:B].cpu().numpy()
        for s in range(B):
            ref = np.empty(V, np.float32)
            om.forward(refs[s], int(tok[s]), p, ref)
            assert_logits(g[s], ref, "call %d seq %d" % (i, s))
    assert a.pos == b.pos == P + len(batches)
    assert a.status() == 0 and b.status() == 0
    a.close()
    b.close()


def test_noalloc_refuses_a_step_larger_than_its_array(dev):
    from transformer_llama_decode_amd._lib import LD_E_SCRATCH, LD_STATIC_SCRATCH_BYTES
    from transformer_llama_decode_amd.model import LlamaDecoder
    # 256 rows of a 2048-wide model: 4 x 2 MiB of activations + 8 MiB of gate rows +
    # 16 MiB of split-K partials, more than the 32 MiB array
    assert LD_STATIC_SCRATCH_BYTES == 32 << 20
    cfg = ModelConfig(dim=2048, n_layers=1, n_heads=16, hidden_dim=8192, vocab_size=301, max_seq=8,
                      max_batch=256)
    gm = LlamaDecoder(cfg, 3)
    rc, _ = gm.decode_step_noalloc(np.full(256, 7, np.int32))
    assert rc == LD_E_SCRATCH
    assert gm.pos == 0
    # a step that fits still runs, on the same handle
    rc, nxt = gm.decode_step_noalloc(np.full(4, 7, np.int32))
    assert rc == 0 and gm.pos == 1
    ref = LlamaDecoder(cfg, 3)
    lr = torch.empty((4, cfg.vocab_size), dtype=torch.float32, device=dev)
    ref.decode_step(np.full(4, 7, np.int32), logits=lr)
    lg = torch.empty((4, cfg.vocab_size), dtype=torch.float32, device=dev)
    gm.set_pos(0)
    rc, _ = gm.decode_step_noalloc(np.full(4, 7, np.int32), logits=lg)
    assert rc == 0
    assert torch.equal(lg.view(torch.int32), lr.view(torch.int32))
    assert gm.status() == 0
    gm.close()
    ref.close()
