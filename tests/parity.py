"""Shared helpers of the GPU parity tests (tolerances and comparisons).

The tolerance is the one the decode path is held to: a logit passes when
|gpu - oracle| <= max(1e-4 * |oracle|, 1e-5); greedy tokens must be identical
wherever the oracle's top-1 minus top-2 logit exceeds 1e-3.
"""
import numpy as np

REL, ABS, MARGIN = 1e-4, 1e-5, 1e-3


def logits_close(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return np.abs(g - o) <= np.maximum(REL * np.abs(o), ABS)


def assert_logits(g, o, ctx=""):
    ok = logits_close(g, o)
    if not ok.all():
        g = np.asarray(g, np.float64).ravel()
        o = np.asarray(o, np.float64).ravel()
        okr = ok.ravel()
        i = int(np.argmax(np.abs(g - o) / np.maximum(REL * np.abs(o), ABS)))
        raise AssertionError("%s: %d of %d logits out of tolerance; worst at %d: gpu %.9g oracle %.9g"
                             % (ctx, int((~okr).sum()), okr.size, i, g[i], o[i]))


def top2(o):
    o = np.asarray(o, np.float32)
    i = int(np.argmax(o))
    m = o.copy()
    m[i] = -np.inf
    return i, float(o[i]), float(m.max())


def assert_token(g_tok, o_logits, ctx=""):
    i, v1, v2 = top2(o_logits)
    if v1 - v2 > MARGIN:
        assert int(g_tok) == i, "%s: gpu token %d, oracle token %d (margin %.3g)" % (ctx, g_tok, i, v1 - v2)
