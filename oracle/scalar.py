"""Pure-Python brute-force tree attention for tiny inputs (test infrastructure).

Independent of ``oracle.attention`` in the parts most likely to go wrong:
visibility comes from walking parent pointers (key node p is visible to
query node c iff p is c or an ancestor of c), not from DFS intervals; the
softmax is a direct sum of exp() without max-shifting; every dot product is
a Python loop. Only for contiguous tree attention without rotary embedding
("tree_attn.py" page, CPU tree-attention kernel), at sizes of a few dozen
tokens.
"""

from __future__ import annotations

import math


def ancestors_or_self(parent, c: int) -> set:
    out = set()
    while c >= 0:
        out.add(c)
        c = int(parent[c])
    return out


def tree_attn_bruteforce(q, k, v, q_indptr, parents, h_q: int, h_kv: int, sm_scale: float):
    """q [total, h_q, d], k/v [total, h_kv, d] nested lists or arrays of floats;
    parents: one parent array per sequence (parent[0] = -1), queries and keys
    are the sequence's tree nodes in order.
    Returns (out, lse) as nested Python lists; lse in base 2."""
    g = h_q // h_kv
    total = int(q_indptr[-1])
    d = len(q[0][0]) if total else 0
    out = [[[0.0] * d for _ in range(h_q)] for _ in range(total)]
    lse = [[float("-inf")] * h_q for _ in range(total)]
    for b in range(len(q_indptr) - 1):
        base = int(q_indptr[b])
        n = int(q_indptr[b + 1]) - base
        par = parents[b]
        for c in range(n):
            anc = ancestors_or_self(par, c)
            for h in range(h_q):
                kvh = h // g
                weights = []
                for p in sorted(anc):
                    dot = 0.0
                    for t in range(d):
                        dot += float(q[base + c][h][t]) * float(k[base + p][kvh][t])
                    weights.append((p, math.exp(sm_scale * dot)))
                z = sum(w for _, w in weights)
                for t in range(d):
                    acc = 0.0
                    for p, w in weights:
                        acc += w * float(v[base + p][kvh][t])
                    out[base + c][h][t] = acc / z
                lse[base + c][h] = math.log(z) / math.log(2.0)
    return out, lse
