"""Pins of the oracle's tree construction against what the pages fix.

- the worked dedup example of the ReDrafter page ("Dynamic Tree Attention");
- a second formulation: the broadcast-compare / cumulative-sum / argmax
  description of dedup_prefix on the same page, written here in numpy;
- the round trip: walking parents from each beam's last node gives the beam back;
- the node count equals the number of distinct prefixes (brute force over a set);
- parents precede children and the mask is the transitive closure of parent
  plus self (Clover page, tree mask M_ij).
"""
import json
from pathlib import Path

import numpy as np
import pytest

from tree_attention_verification_beam_amd import synth

GOLDEN = Path(__file__).resolve().parent / "golden"


def dedup_prefix_numpy(beam: np.ndarray) -> np.ndarray:
    """dedup_prefix as the ReDrafter page describes it, for one [W][L] beam.

    matches[i][j][k] = beam[i][k] == beam[j][k]; candidates i and j share the
    prefix of length k+1 when the running count of matches equals k+1; argmax
    over j picks the smallest such candidate.
    """
    W, L = beam.shape
    matches = beam[:, None, :] == beam[None, :, :]               # [W][W][L]
    counts = np.cumsum(matches, axis=2)                          # [W][W][L]
    seq_matches = counts == np.arange(1, L + 1)[None, None, :]   # [W][W][L]
    return np.argmax(seq_matches, axis=1)                        # [W][L]


def with_root(beams, root):
    return np.concatenate([np.asarray(root)[:, None, None].repeat(beams.shape[1], 1), beams], 2)


def anc_bits(anc_row):
    out = set()
    for w, word in enumerate(anc_row):
        word = int(word)
        for bit in range(64):
            if (word >> bit) & 1:
                out.add(64 * w + bit)
    return out


def test_worked_example(oracle):
    ex = json.loads((GOLDEN / "redrafter_dedup_example.json").read_text())
    words = sorted({w for row in ex["beam"] for w in row})
    ids = np.array([[words.index(w) for w in row] for row in ex["beam"]], np.int32)
    # stated shares: candidate i shares its prefix of length n with candidate 0
    pt = dedup_prefix_numpy(ids)
    for s in ex["stated_shared_prefix"]:
        i, j, n = s["candidate"], s["with"], s["length"]
        assert all(pt[i, k] == j for k in range(n))
        assert pt[i, n] == i
    # the tree: column 0 is the root
    root = ids[:, 0][:1]
    beams = ids[None, :, 1:]
    tr = oracle.build_tree_beams(beams, root, T_cap=1 + beams.shape[1] * beams.shape[2])
    # 8 distinct tokens in the packed beam: quiet morning sipping coffee and reading on her
    assert tr["n_nodes"][0] == 8
    bn = tr["beam_node"][0]
    for s in ex["stated_shared_prefix"]:
        i, j, n = s["candidate"], s["with"], s["length"]
        assert list(bn[i, :n - 1]) == list(bn[j, :n - 1])     # n-1 draft tokens + root
        assert bn[i, n - 1] != bn[j, n - 1]
    # tokens of the packed beam in first-appearance order
    packed = [words[t] for t in tr["token"][0, :8]]
    assert packed == ["quiet", "morning", "sipping", "coffee", "and", "reading", "on", "her"]


def _random_beams(seed, B, W, L, V):
    rng = np.random.default_rng(seed)
    beams = rng.integers(0, V, size=(B, W, L)).astype(np.int32)
    for b in range(B):
        for i in range(1, W):
            src = rng.integers(0, i)
            k = rng.integers(0, L + 1)
            beams[b, i, :k] = beams[b, src, :k]
    return beams, rng.integers(0, V, size=B).astype(np.int32)


@pytest.mark.parametrize("W,L,V", [(4, 4, 1000), (8, 5, 3), (16, 4, 2), (1, 7, 5), (9, 1, 4)])
def test_second_formulation_and_first_appearance(oracle, W, L, V):
    beams, root = _random_beams(7 + W * L + V, 24, W, L, V)
    tr = oracle.build_tree_beams(beams, root, T_cap=1 + W * L)
    for b in range(beams.shape[0]):
        pt = dedup_prefix_numpy(with_root(beams[b:b + 1], root[b:b + 1])[0])  # [W][L+1]
        new = pt[:, 1:] == np.arange(W)[:, None]                             # [W][L]
        # every new (i, k) in beam-major order gets the next id 1, 2, 3, ...
        order = np.flatnonzero(new.reshape(-1))
        assert tr["n_nodes"][b] == 1 + len(order)
        bn = tr["beam_node"][b]
        assert list(bn.reshape(-1)[order]) == list(range(1, 1 + len(order)))
        # an old (i, k) reuses the node of the smallest candidate sharing the prefix
        for i in range(W):
            for k in range(L):
                assert bn[i, k] == bn[pt[i, k + 1], k]


@pytest.mark.parametrize("W,L,V", [(4, 4, 1000), (8, 5, 2), (16, 4, 3)])
def test_round_trip_and_distinct_prefixes(oracle, W, L, V):
    beams, root = _random_beams(99 + W, 32, W, L, V)
    T_cap = 1 + W * L + 3
    tr = oracle.build_tree_beams(beams, root, T_cap=T_cap)
    for b in range(beams.shape[0]):
        T = tr["n_nodes"][b]
        prefixes = {tuple(beams[b, i, :k + 1]) for i in range(W) for k in range(L)}
        assert T == 1 + len(prefixes)
        par, tok, dep = tr["parent"][b], tr["token"][b], tr["depth"][b]
        assert tok[0] == root[b] and par[0] == -1 and dep[0] == 0
        for i in range(W):
            node = tr["beam_node"][b, i, L - 1]
            seq = []
            while node != 0:
                seq.append(tok[node])
                node = par[node]
            assert seq[::-1] == list(beams[b, i])
        for t in range(1, T):
            assert 0 <= par[t] < t
            assert dep[t] == dep[par[t]] + 1
            closure, cur = {t}, t
            while cur != 0:
                cur = par[cur]
                closure.add(cur)
            assert anc_bits(tr["anc"][b, t]) == closure
        for t in range(T, T_cap):
            assert par[t] == -1 and tok[t] == -1 and dep[t] == -1
            assert anc_bits(tr["anc"][b, t]) == set()


def test_wide_tree_two_mask_words(oracle):
    beams, root = _random_beams(5, 4, 16, 4, 100000)
    tr = oracle.build_tree_beams(beams, root, T_cap=65)
    assert tr["anc"].shape[2] == 2
    for b in range(4):
        T = tr["n_nodes"][b]
        for t in range(T):
            bits = anc_bits(tr["anc"][b, t])
            assert max(bits) == t and 0 in bits


def test_explicit_static_and_caterpillar(oracle):
    parents = np.array([synth.static_tree_parents()], np.int32)
    tokens = np.arange(16, dtype=np.int32)[None] + 10
    tr = oracle.build_tree_explicit(parents, tokens, np.array([3], np.int32), T_cap=17)
    assert tr["n_nodes"][0] == 17 and tr["bad"][0] == 0
    # rank tuples give the depth directly
    assert list(tr["depth"][0, 1:]) == [len(t) for t in synth.STATIC_TREE]
    # the node of tuple (0,1,0,0) sees exactly its own rank prefixes and the root
    idx = {tup: j + 1 for j, tup in enumerate(synth.STATIC_TREE)}
    want = {0, idx[(0,)], idx[(0, 1)], idx[(0, 1, 0)], idx[(0, 1, 0, 0)]}
    assert anc_bits(tr["anc"][0, idx[(0, 1, 0, 0)]]) == want

    cp = np.array([synth.caterpillar_parents(6, 8)], np.int32)
    tr = oracle.build_tree_explicit(cp, np.zeros((1, 48), np.int32), np.array([0], np.int32),
                                    T_cap=49)
    assert tr["n_nodes"][0] == 49
    assert list(tr["depth"][0, 1:]) == [d for d in range(1, 7) for _ in range(8)]


def test_explicit_rejects_non_topological(oracle):
    cp = np.array([[0, 0, 3], [0, 1, 1]], np.int32)     # row 0: candidate 2 names node 3
    tr = oracle.build_tree_explicit(cp, np.ones((2, 3), np.int32), np.zeros(2, np.int32), T_cap=4)
    assert list(tr["bad"]) == [1, 0]
    assert tr["n_nodes"][0] == 1 and tr["n_nodes"][1] == 4
