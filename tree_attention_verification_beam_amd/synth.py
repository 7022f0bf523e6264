"""Seeded synthetic inputs for the verification step (numpy only).

This module produces inputs and nothing else: it builds no tree, computes no
attention and takes no acceptance decision.  The HIP path and the CPU oracle
both consume exactly these arrays.  The only arithmetic here is the drafter's
side of the step, which lies outside the verification step itself: a static
tree's tokens are the top-ranked entries of synthetic head logits, and the
i.i.d. multi-candidate tokens are inverse-CDF draws from the draft
distribution.

Workloads (shapes of the pages' settings, values synthetic):
  0 tiny-f32-beams      B=1, ctx 64, H=Hkv=4, D=64, fp32; 4 beams x 4 over V=1000
  1 redrafter-7b-beams  B=1, ctx 2048, H=Hkv=32, D=128, bf16; 8 beams x 5, V=32000
  2 clover-static-b64   B=64, ctx 1024, H=Hkv=32, D=128, bf16; 16-node static tree
                        from 4 heads with top-(4,2,1,1) fan-out, V=128000, greedy
  3 gqa70b-beams-b16    B=16, ctx 8192, H=64, Hkv=8, D=128, bf16; 16 beams x 4,
                        V=128256, per-path rejection sampling
  4 multicand-32k       B=4, ctx 32768, H=32, Hkv=8, D=128, bf16; 8 i.i.d.
                        candidates per position over a chain of 6 positions,
                        V=152064, sequential (recursive) rejection
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAMS = ("tree", "q", "k", "v", "tgt", "dft", "u_node", "u_final", "cand")


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    ctx: int
    H: int
    Hkv: int
    D: int
    dtype: str            # "f32" | "bf16"
    tree: str             # "beams" | "static" | "caterpillar"
    V: int
    modes: tuple
    W: int = 0
    L: int = 0
    N: int = 0            # explicit trees: candidate count
    draft_sigma: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def T_cap(self) -> int:
        if self.tree == "beams":
            return 1 + self.W * self.L
        return 1 + self.N

    @property
    def cap(self) -> int:
        return self.ctx + self.T_cap

    @property
    def group(self) -> int:
        return self.H // self.Hkv


WORKLOADS = [
    Workload(0, "tiny-f32-beams", B=1, ctx=64, H=4, Hkv=4, D=64, dtype="f32", tree="beams",
             V=1000, modes=("greedy", "reject_path"), W=4, L=4, draft_sigma=1.0),
    Workload(1, "redrafter-7b-beams", B=1, ctx=2048, H=32, Hkv=32, D=128, dtype="bf16",
             tree="beams", V=32000, modes=("greedy", "reject_path"), W=8, L=5, draft_sigma=1.0),
    Workload(2, "clover-static-b64", B=64, ctx=1024, H=32, Hkv=32, D=128, dtype="bf16",
             tree="static", V=128000, modes=("greedy",), N=16),
    Workload(3, "gqa70b-beams-b16", B=16, ctx=8192, H=64, Hkv=8, D=128, dtype="bf16",
             tree="beams", V=128256, modes=("reject_path",), W=16, L=4, draft_sigma=1.0),
    Workload(4, "multicand-32k", B=4, ctx=32768, H=32, Hkv=8, D=128, dtype="bf16",
             tree="caterpillar", V=152064, modes=("reject_recursive",), N=48, draft_sigma=1.5,
             extra=dict(depth=6, per=8)),
]

# Static tree of the parallel-head workload, as rank tuples in BFS order, then
# lexicographic: head k contributes its top-r_k with fan-out (4, 2, 1, 1) along
# the two best depth-2 branches of the best depth-1 branch.
STATIC_TREE = (
    [(a,) for a in range(4)]
    + [(a, r) for a in range(4) for r in range(2)]
    + [(0, 0, 0), (0, 1, 0)]
    + [(0, 0, 0, 0), (0, 1, 0, 0)]
)


def static_tree_parents():
    """Parent tree index of every node of STATIC_TREE (node j+1 <- tuple j)."""
    index = {(): 0}
    for j, tup in enumerate(STATIC_TREE):
        index[tup] = j + 1
    return [index[tup[:-1]] for tup in STATIC_TREE]


def caterpillar_parents(depth: int, per: int):
    """Parent tree index of candidates of a chain with `per` siblings per position.

    Candidate j at depth d is node 1 + per*(d-1) + j; all siblings at depth d
    hang off the spine node (candidate 0) of depth d-1, the root at depth 1.
    """
    out = []
    for d in range(1, depth + 1):
        spine_parent = 0 if d == 1 else 1 + per * (d - 2)
        out += [spine_parent] * per
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def exact_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """U[0,1) drawn as k * 2^-24: exactly representable in fp32 and fp64."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * (2.0 ** -24)).astype(np.float32)


def _normal(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def _draw_beams(rng, B, W, L, V):
    beams = rng.integers(0, V, size=(B, W, L), dtype=np.int64)
    shared = rng.integers(0, L, size=(B, W), dtype=np.int64)
    for b in range(B):
        for i in range(1, W):
            k = int(shared[b, i])
            beams[b, i, :k] = beams[b, 0, :k]
    return beams.astype(np.int32)


def _inverse_cdf_draws(logits_row: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Drafter-side sampling of candidates from softmax(logits_row), fp64."""
    z = logits_row.astype(np.float64)
    w = np.exp(z - z.max())
    cdf = np.cumsum(w / w.sum())
    idx = np.searchsorted(cdf, u, side="right")
    return np.minimum(idx, len(cdf) - 1).astype(np.int32)


def make_inputs(wid: int, seed_offset: int = 0, *, with_kv: bool = True,
                ctx_override: int | None = None, B_override: int | None = None) -> dict:
    """All inputs of one step of workload `wid`, seeded by SeedSequence(1234 + wid + offset).

    Overrides shrink ctx or B for the oracle-sized parity cases while keeping
    every other shape, distribution and structure of the workload.
    """
    w = WORKLOADS[wid]
    B = B_override or w.B
    ctx = w.ctx if ctx_override is None else ctx_override
    T_cap = w.T_cap
    cap = ctx + T_cap
    ss = np.random.SeedSequence(1234 + wid + seed_offset)
    rngs = dict(zip(STREAMS, [np.random.default_rng(s) for s in ss.spawn(len(STREAMS))]))
    out = dict(wid=wid, name=w.name, B=B, ctx=ctx, T_cap=T_cap, cap=cap, H=w.H, Hkv=w.Hkv,
               D=w.D, V=w.V, dtype=w.dtype, tree=w.tree, modes=w.modes)

    out["root_token"] = rngs["tree"].integers(0, w.V, size=B, dtype=np.int64).astype(np.int32)
    tgt = _normal(rngs["tgt"], (B, T_cap, w.V), 3.0)
    out["tgt"] = tgt
    if w.tree == "beams":
        out["W"], out["L"] = w.W, w.L
        out["beams"] = _draw_beams(rngs["tree"], B, w.W, w.L, w.V)
        out["dft"] = tgt + _normal(rngs["dft"], (B, T_cap, w.V), w.draft_sigma)
        out["dft_row"] = np.tile(np.arange(T_cap, dtype=np.int32), (B, 1))
    elif w.tree == "static":
        parents = static_tree_parents()
        out["cand_parent"] = np.tile(np.array(parents, np.int32), (B, 1))
        # head k (1-based) reads the target row of the best branch at depth k-1
        spine = [0, 1, 5, 13]
        sigmas = [0.5 * k for k in range(1, 5)]
        heads = np.stack([tgt[:, spine[k]] + _normal(rngs["dft"], (B, w.V), sigmas[k])
                          for k in range(4)], axis=1)  # [B][4][V]
        order = np.argsort(-heads, axis=2, kind="stable")
        cand_token = np.zeros((B, len(STATIC_TREE)), np.int32)
        for j, tup in enumerate(STATIC_TREE):
            cand_token[:, j] = order[:, len(tup) - 1, tup[-1]]
        out["cand_token"] = cand_token
        out["dft"] = None
        out["dft_row"] = None
    elif w.tree == "caterpillar":
        depth, per = w.extra["depth"], w.extra["per"]
        parents = caterpillar_parents(depth, per)
        out["cand_parent"] = np.tile(np.array(parents, np.int32), (B, 1))
        spine_nodes = [0] + [1 + per * (d - 1) for d in range(1, depth)]
        dft = np.stack([tgt[:, s] + _normal(rngs["dft"], (B, w.V), w.draft_sigma)
                        for s in spine_nodes], axis=1)  # [B][depth][V]
        dft_row = np.full((B, T_cap), -1, np.int32)
        for r, s in enumerate(spine_nodes):
            dft_row[:, s] = r
        u_c = rngs["cand"].random(size=(B, depth, per))
        cand_token = np.zeros((B, depth * per), np.int32)
        for b in range(B):
            for d in range(depth):
                cand_token[b, d * per:(d + 1) * per] = _inverse_cdf_draws(dft[b, d], u_c[b, d])
        out["cand_token"] = cand_token
        out["dft"] = dft
        out["dft_row"] = dft_row
    else:
        raise ValueError(w.tree)

    out["u_node"] = exact_uniforms(rngs["u_node"], (B, T_cap))
    out["u_final"] = exact_uniforms(rngs["u_final"], (B,))
    out["ctx_len"] = np.full(B, ctx, np.int32)

    if with_kv:
        if w.dtype == "f32":
            conv = lambda a: a
        else:
            conv = f32_to_bf16_bits
        out["q"] = conv(_normal(rngs["q"], (B, T_cap, w.H, w.D)))
        out["k"] = conv(_normal(rngs["k"], (B, w.Hkv, cap, w.D)))
        out["v"] = conv(_normal(rngs["v"], (B, w.Hkv, cap, w.D)))
    return out


def make_custom_inputs(seed: int, *, B: int, H: int, Hkv: int, D: int, V: int, dtype: str,
                       ctx_lens, tree: str = "beams", W: int = 0, L: int = 0, parents=None,
                       draft_sigma: float = 1.0) -> dict:
    """Inputs of one step with free shapes, for edge cases of the parity tests.

    tree = "beams": W beams of L tokens with shared prefixes drawn as in the
    workloads.  tree = "explicit": every sequence uses the parent list
    `parents` (node j+1's parent) with uniform tokens.  Each node's children
    are drawn from that node's own draft row (dft_row = identity).  Context
    lengths may differ per sequence; the cache holds the longest context plus
    the tree.
    """
    ss = np.random.SeedSequence(seed)
    rngs = dict(zip(STREAMS, [np.random.default_rng(s) for s in ss.spawn(len(STREAMS))]))
    ctx_lens = np.asarray(ctx_lens, np.int32)
    assert ctx_lens.shape == (B,)
    if tree == "beams":
        T_cap = 1 + W * L
    else:
        T_cap = 1 + len(parents)
    cap = int(ctx_lens.max()) + T_cap
    out = dict(wid=-1, name="custom", B=B, ctx=int(ctx_lens.max()), T_cap=T_cap, cap=cap, H=H,
               Hkv=Hkv, D=D, V=V, dtype=dtype, tree=tree if tree == "beams" else "explicit",
               modes=("greedy", "reject_path", "reject_recursive"))
    out["root_token"] = rngs["tree"].integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    tgt = _normal(rngs["tgt"], (B, T_cap, V), 3.0)
    out["tgt"] = tgt
    if tree == "beams":
        out["W"], out["L"] = W, L
        out["beams"] = _draw_beams(rngs["tree"], B, W, L, V)
    else:
        out["cand_parent"] = np.tile(np.asarray(parents, np.int32), (B, 1))
        out["cand_token"] = rngs["tree"].integers(0, V, size=(B, len(parents)),
                                                  dtype=np.int64).astype(np.int32)
    out["dft"] = tgt + _normal(rngs["dft"], (B, T_cap, V), draft_sigma)
    out["dft_row"] = np.tile(np.arange(T_cap, dtype=np.int32), (B, 1))
    out["u_node"] = exact_uniforms(rngs["u_node"], (B, T_cap))
    out["u_final"] = exact_uniforms(rngs["u_final"], (B,))
    out["ctx_len"] = ctx_lens.copy()
    conv = (lambda a: a) if dtype == "f32" else f32_to_bf16_bits
    out["q"] = conv(_normal(rngs["q"], (B, T_cap, H, D)))
    out["k"] = conv(_normal(rngs["k"], (B, Hkv, cap, D)))
    out["v"] = conv(_normal(rngs["v"], (B, Hkv, cap, D)))
    return out


def make_two_level_trials(rng: np.random.Generator, B: int, lp0: np.ndarray, lq0: np.ndarray,
                          lp1: np.ndarray, lq1: np.ndarray, N1: int, N2: int) -> dict:
    """B independent two-position trials whose rows depend only on the token prefix.

    A root with N1 children drawn i.i.d. from softmax(lq0), each child with
    token x having N2 children drawn i.i.d. from softmax(lq1[x]); the target row
    of the root is lp0 and of a depth-1 node with token x is lp1[x] (as a model's
    rows depend on the prefix only), and the draft rows match.  Depth-2 nodes are
    leaves (target row lp0, unused by the first two emitted tokens).  Node
    numbering: depth-1 candidate i is node 1 + i, its j-th child node
    1 + N1 + i*N2 + j.
    """
    V = len(lp0)
    N = N1 + N1 * N2
    T_cap = 1 + N
    cand_parent = np.zeros((B, N), np.int32)
    cand_token = np.zeros((B, N), np.int32)
    tok1 = _inverse_cdf_draws(lq0, rng.random((B, N1)).ravel()).reshape(B, N1)
    cand_token[:, :N1] = tok1
    u2 = rng.random((B, N1, N2))
    for x in range(V):
        sel = tok1 == x
        if sel.any():
            draws = _inverse_cdf_draws(lq1[x], u2[sel].ravel()).reshape(-1, N2)
            idx_b, idx_i = np.nonzero(sel)
            for j in range(N2):
                cand_token[idx_b, N1 + idx_i * N2 + j] = draws[:, j]
    for i in range(N1):
        cand_parent[:, N1 + i * N2:N1 + (i + 1) * N2] = 1 + i
    tgt = np.empty((B, T_cap, V), np.float32)
    tgt[:] = lp0
    tgt[:, 1:1 + N1] = lp1[tok1]
    dft = np.empty((B, 1 + N1, V), np.float32)
    dft[:, 0] = lq0
    dft[:, 1:] = lq1[tok1]
    dft_row = np.full((B, T_cap), -1, np.int32)
    dft_row[:, :1 + N1] = np.arange(1 + N1, dtype=np.int32)
    return dict(B=B, T_cap=T_cap, V=V, tree="explicit", cand_parent=cand_parent,
                cand_token=cand_token, root_token=np.zeros(B, np.int32), tgt=tgt, dft=dft,
                dft_row=dft_row, u_node=exact_uniforms(rng, (B, T_cap)),
                u_final=exact_uniforms(rng, (B,)))


# one fixed small tree with siblings at several depths: parent node of candidate
# nodes 1..7 and their tokens (vocabulary of 6); nodes 0, 1, 2 and 4 have children
FIXED_TREE_PARENTS = (0, 0, 0, 1, 1, 2, 4)
FIXED_TREE_TOKENS = (0, 1, 2, 3, 4, 0, 5)
FIXED_TREE_TOKENS_DUP = (0, 0, 2, 3, 4, 0, 5)  # nodes 1 and 2: the same token under the root


def make_fixed_tree_trials(rng: np.random.Generator, B: int, cand_parent, cand_token,
                           lp: np.ndarray, lq: np.ndarray, dft_row) -> dict:
    """B independent trials of one fixed explicit tree; only the uniforms differ.

    `cand_parent` / `cand_token` name candidate nodes 1..N (parents are node
    indices, the root is node 0), `lp` holds the target logits row of every node
    (T = N + 1 rows), `lq` the draft logits rows and `dft_row[t]` the draft row
    of node t's children (-1 for a leaf).
    """
    cand_parent = np.asarray(cand_parent, np.int32)
    cand_token = np.asarray(cand_token, np.int32)
    lp = np.asarray(lp, np.float32)
    lq = np.asarray(lq, np.float32)
    N = len(cand_parent)
    T_cap = N + 1
    V = lp.shape[1]
    return dict(B=B, T_cap=T_cap, V=V, tree="explicit",
                cand_parent=np.ascontiguousarray(np.broadcast_to(cand_parent, (B, N))),
                cand_token=np.ascontiguousarray(np.broadcast_to(cand_token, (B, N))),
                root_token=np.zeros(B, np.int32),
                tgt=np.ascontiguousarray(np.broadcast_to(lp, (B, T_cap, V))),
                dft=np.ascontiguousarray(np.broadcast_to(lq, (B,) + lq.shape)),
                dft_row=np.ascontiguousarray(np.broadcast_to(np.asarray(dft_row, np.int32),
                                                             (B, T_cap))),
                u_node=exact_uniforms(rng, (B, T_cap)), u_final=exact_uniforms(rng, (B,)))


FIXED_TREE_DFT_ROW = (0, 1, 2, -1, 3, -1, -1, -1)


def fixed_tree_logits(seed: int, tokens=FIXED_TREE_TOKENS, raise_drafted: float = 0.5) -> tuple:
    """Logits rows of the fixed tree: target row of every node ~ N(0, 1.5^2),
    draft row of each node with children = its target row + N(0, 1), with each
    child's token raised by 0.5 in its parent's draft row (drafted tokens are
    the draft's likely ones; `raise_drafted` sets the amount).  Returns
    (lp (8, 6), lq (4, 6), dft_row)."""
    rng = np.random.default_rng(seed)
    T = len(FIXED_TREE_PARENTS) + 1
    lp = (1.5 * rng.standard_normal((T, 6))).astype(np.float32)
    lq = np.empty((4, 6), np.float32)
    for node, r in enumerate(FIXED_TREE_DFT_ROW):
        if r >= 0:
            lq[r] = lp[node] + rng.standard_normal(6).astype(np.float32)
    for par, tok in zip(FIXED_TREE_PARENTS, tokens):
        lq[FIXED_TREE_DFT_ROW[par], tok] += np.float32(raise_drafted)
    return lp, lq, np.asarray(FIXED_TREE_DFT_ROW, np.int32)
