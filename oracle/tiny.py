"""Pure-Python loop versions of the attention definitions, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

These restate the masked-softmax definition element by element with ``math``
and Python lists (no numpy, no matrix products), so they serve as brute force
against the vectorised oracle on inputs of a few dozen tokens.
"""

import math


def masked_softmax_attention(q, k, v, allowed, scale):
    """q, k, v: lists of rows (lists of floats); allowed(t, s) -> bool.

    Returns (o, lse) as lists; a query with no allowed key gets o = 0 and
    lse = -inf.
    """
    n_q = len(q)
    n_k = len(k)
    d = len(v[0]) if n_k else 0
    o, lse = [], []
    for t in range(n_q):
        keys = [s for s in range(n_k) if allowed(t, s)]
        if not keys:
            o.append([0.0] * d)
            lse.append(-math.inf)
            continue
        sc = [scale * sum(q[t][c] * k[s][c] for c in range(len(q[t]))) for s in keys]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        tot = sum(w)
        o.append([sum(w[n] * v[s][c] for n, s in enumerate(keys)) / tot for c in range(d)])
        lse.append(m + math.log(tot))
    return o, lse


def block_rows_allowed(rows, block, causal):
    """allowed(t, s) for a list of per-query-block key-block sets."""
    def allowed(t, s):
        if causal and s > t:
            return False
        return (s // block) in rows[t // block]
    return allowed


def offsets_allowed(offsets):
    """allowed(t, s) for a set of distances: s = t - delta, delta in offsets."""
    offs = set(offsets)

    def allowed(t, s):
        return (t - s) in offs
    return allowed


def explicit_keys_attention(q, keys, values, scale):
    """Softmax attention of one query over an explicit list of key / value
    vectors, in pure Python loops (no numpy reductions).  Returns (o, lse);
    an empty list gives o = 0 and lse = -inf."""
    d = len(q)
    if not keys:
        return [0.0] * d, -math.inf
    sc = []
    for kv in keys:
        acc = 0.0
        for x in range(d):
            acc += q[x] * kv[x]
        sc.append(scale * acc)
    m = max(sc)
    ws = [math.exp(x - m) for x in sc]
    tot = sum(ws)
    o = [0.0] * d
    for wgt, vv in zip(ws, values):
        for x in range(d):
            o[x] += wgt * vv[x]
    return [x / tot for x in o], m + math.log(tot)
