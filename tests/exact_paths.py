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


RECURSIVE_VARIANTS = ("exact", "draw_from_p", "reverse_order", "no_residual_update", "root_rows")


def recursive_table(parent, token, lp, lq, dft_row, variant="exact"):
    """(T, V) table of P(stop node, next token) under sequential rejection
    ([ResiSpec] section 4, with the library's readings): the children of the
    current node s are tested in node-index order against p', which starts as
    p_s; child x is accepted with probability min(1, p'(x) / q_s(x)) and the
    walk moves to it; each rejection sets p' <- norm(max(0, p' - q_s)); with no
    child left the next token is drawn from p' (from p_s at a leaf).  The
    process follows one path, so the table is a sum over the tree's nodes and
    the number of rejections before each acceptance.  Variants: the final draw
    from p_s, children tested in reverse order, p' never updated, every node's
    residual built from the root's rows."""
    assert variant in RECURSIVE_VARIANTS
    par = [-1] + [int(x) for x in parent]
    tok = [-1] + [int(x) for x in token]
    T = len(par)
    p = softmax(np.asarray(lp, np.float64), axis=1)
    q = softmax(np.asarray(lq, np.float64), axis=1)
    V = p.shape[1]
    children = [[c for c in range(1, T) if par[c] == s] for s in range(T)]
    table = np.zeros((T, V))

    def visit(s, prob):
        ch = children[s]
        if not ch:
            table[s] += prob * p[s]
            return
        rows = 0 if variant == "root_rows" else s
        pr, qq = p[rows].copy(), q[dft_row[rows]]
        if variant == "reverse_order":
            ch = ch[::-1]
        rem = prob
        for c in ch:
            x = tok[c]
            acc = min(1.0, pr[x] / qq[x]) if qq[x] > 0 else (1.0 if pr[x] > 0 else 0.0)
            if acc > 0:
                visit(c, rem * acc)
            rem *= 1.0 - acc
            if variant != "no_residual_update":
                r = np.maximum(0.0, pr - qq)
                pr = r / r.sum()
        table[s] += rem * (p[s] if variant == "draw_from_p" else pr)

    visit(0, 1.0)
    return table
