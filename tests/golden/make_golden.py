"""Write the oracle's reference outputs for the full-size workloads.

Calls only oracle/ (and the shared input generator through it).  For each
workload and each stored sequence it runs the oracle greedily over every
position and records, per position: the token fed in, the greedy token out, the
top-1 and top-2 logit values.  For the sequences listed in `full_seqs` it also
records the full logit vector at the last prompt position, the two after it,
every 32nd position after it and the last two, and a fixed set of SUB_N logit indices
(drawn once from SUB_SEED, stored with the file) at every position.  Those greedy
sequences are the teacher-forcing inputs of the GPU parity tests.

    python tests/golden/make_golden.py C2 C3 ...     (default: all but C5)
    python tests/golden/make_golden.py C5            (~1.5 h, ~30 GB of RAM)
    python tests/golden/make_golden.py C5bf16        (the same with bfloat16 weights)
    python tests/golden/make_golden.py C5w           (past max_seq: ~2.5 h)

GOLDEN_PROCS sets the worker processes (default 6), GOLDEN_THREADS the threads
each uses to draw its weights (default 4; the draw is counter-based, so the
weights do not depend on it, and the forward pass is single-threaded).
"""
import hashlib
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402
from transformer_llama_decode_amd.configs import WORKLOADS  # noqa: E402

SOURCES = ["oracle/oracle.c", "oracle/oracle.h", "synth/synth.c", "synth/synth.h"]

# sequences whose greedy streams are stored, and those with full logits
PLAN = {
    "C1": dict(seqs=[0], full_seqs=[0]),
    "C2": dict(seqs=[0], full_seqs=[0]),
    "C3": dict(seqs=list(range(256)), full_seqs=[0, 255]),
    "C4b32": dict(seqs=list(range(32)), full_seqs=[0, 31]),
    "C5": dict(seqs=[0], full_seqs=[0]),
    "C5bf16": dict(seqs=[0], full_seqs=[0]),
    "C5w": dict(seqs=[0], full_seqs=[0]),
}


def source_hash():
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# logit indices stored at every position: SUB_N distinct indices from a fixed seed
SUB_N, SUB_SEED, FULL_EVERY = 256, 20240, 32


def sub_indices(V):
    return np.sort(np.random.default_rng(SUB_SEED).choice(V, SUB_N, replace=False)).astype(np.int32)


def keep_positions(w):
    """Positions whose full logits are stored: the last prompt position (the
    first one the GPU is compared at), every FULL_EVERY-th position after it,
    the two after the prompt and the last two."""
    P = max(w.prompt_len, 1)
    E = w.end_pos
    return sorted(set(range(P - 1, E, FULL_EVERY)) | {P, P + 1, E - 2, E - 1})


def prompt_of(w, seq):
    if w.prompt_len == 0:
        return np.array([w.start_token], np.int32)
    return O.synth_prompt(w.prompt_seed, seq, w.prompt_len)


def _run_one(args):
    name, seq, keep = args
    w = WORKLOADS[name]
    m = O.OracleModel(w.model, w.model_seed, nthreads=int(os.environ.get("GOLDEN_THREADS", "4")))
    t0 = time.time()
    sub = sub_indices(w.model.vocab_size) if keep else None
    tin, tout, t1, t2, kept = O.run_sequence(m, prompt_of(w, seq), w.end_pos, keep_logits=keep,
                                             sub_idx=sub)
    m.close()
    return seq, tin, tout, t1, t2, kept, time.time() - t0


def make(name, procs):
    w = WORKLOADS[name]
    plan = PLAN[name]
    keep = keep_positions(w)
    jobs = [(name, s, keep if s in plan["full_seqs"] else []) for s in plan["seqs"]]
    n = len(jobs)
    tin = np.zeros((n, w.end_pos), np.int32)
    tout = np.zeros((n, w.end_pos), np.int32)
    top1 = np.zeros((n, w.end_pos), np.float32)
    top2 = np.zeros((n, w.end_pos), np.float32)
    full = {}
    subs = {}
    t0 = time.time()
    with ProcessPoolExecutor(max_workers=min(procs, n)) as ex:
        for k, (seq, a, b, c, d, kept, dt) in enumerate(ex.map(_run_one, jobs)):
            i = plan["seqs"].index(seq)
            tin[i], tout[i], top1[i], top2[i] = a, b, c, d
            for p, v in kept.items():
                if p == "sub":
                    subs[seq] = v
                else:
                    full[(seq, p)] = v
            print("%s seq %d done (%.1fs, %d/%d)" % (name, seq, dt, k + 1, n), flush=True)
    fs = sorted(full)
    ss = sorted(subs)
    out = os.path.join(HERE, "%s.npz" % name)
    np.savez_compressed(
        out, workload=np.array(name), source_hash=np.array(source_hash()),
        seqs=np.array(plan["seqs"], np.int32), tokens_in=tin, greedy=tout, top1=top1, top2=top2,
        full_seq=np.array([s for s, _ in fs], np.int32), full_pos=np.array([p for _, p in fs], np.int32),
        full_logits=np.stack([full[k] for k in fs]) if fs else np.zeros((0, w.model.vocab_size), np.float32),
        sub_idx=sub_indices(w.model.vocab_size), sub_seq=np.array(ss, np.int32),
        sub_logits=np.stack([subs[k] for k in ss]) if ss else np.zeros((0, w.end_pos, SUB_N), np.float32))
    print("wrote %s in %.0fs" % (out, time.time() - t0), flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or ["C1", "C2", "C3", "C4b32"]
    procs = int(os.environ.get("GOLDEN_PROCS", "6"))
    for nm in names:
        make(nm, procs)
