"""Exact output distribution of per-path rejection on a small fixed tree.

Per-path rejection (ReDrafter page, "The Full Speculative Decoding Loop",
Step 5, under the library's readings of it): candidate node t is accepted with
probability a_t = min(1, p_par(x_t) / q_par(x_t)), independently of every other
node; a node survives when it and all its ancestors are accepted; the deepest
survivor is the stop node (lowest node index among equals); the next token is
drawn from norm(max(0, p_s - q_s)) when the stop node s has children (all of
them rejected, or one would be deeper), else from p_s.

Summing over every accept pattern of the candidate nodes gives
P(stop = s, next token = x) exactly.  The variants build the same table under
plausible mistakes, so a test can show that its sample tells them apart from
the exact table.
"""
import itertools

import numpy as np
from scipy.special import softmax

VARIANTS = ("exact", "ties_highest", "residual_from_p", "no_ancestors", "ratio_swapped",
            "residual_root_rows")


def per_path_table(parent, token, lp, lq, dft_row, variant="exact"):
    """(T, V) table of P(stop node, next token) for candidate nodes 1..N with the
    given parent node indices and tokens; lp: target logits row of every node,
    lq: draft logits rows, dft_row[t]: draft row of node t's children."""
    assert variant in VARIANTS
    par = [-1] + [int(x) for x in parent]
    tok = [-1] + [int(x) for x in token]
    T = len(par)
    assert all(0 <= par[t] < t for t in range(1, T)), "parents precede their children"
    p = softmax(np.asarray(lp, np.float64), axis=1)
    q = softmax(np.asarray(lq, np.float64), axis=1)
    V = p.shape[1]
    depth = [0] * T
    for t in range(1, T):
        depth[t] = depth[par[t]] + 1
    has_child = [any(par[c] == t for c in range(1, T)) for t in range(T)]
    a = np.zeros(T)
    for t in range(1, T):
        pp, qq, x = p[par[t]], q[dft_row[par[t]]], tok[t]
        a[t] = min(1.0, qq[x] / pp[x] if variant == "ratio_swapped" else pp[x] / qq[x])
    table = np.zeros((T, V))
    for pattern in itertools.product((False, True), repeat=T - 1):
        acc = (True,) + pattern
        w = 1.0
        for t in range(1, T):
            w *= a[t] if acc[t] else 1.0 - a[t]
        if w == 0.0:
            continue
        surv = list(acc)
        if variant != "no_ancestors":
            for t in range(1, T):
                surv[t] = acc[t] and surv[par[t]]
        deepest = max(depth[t] for t in range(T) if surv[t])
        at_depth = [t for t in range(T) if surv[t] and depth[t] == deepest]
        s = max(at_depth) if variant == "ties_highest" else min(at_depth)
        if has_child[s] and variant != "residual_from_p":
            r_node = 0 if variant == "residual_root_rows" else s
            res = np.maximum(0.0, p[r_node] - q[dft_row[r_node]])
            dist = res / res.sum()
        else:
            dist = p[s]
        table[s] += w * dist
    return table
