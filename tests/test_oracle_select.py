"""Pins of the oracle's dynamic tree selection (history-of-drafters page, the
EAGLE-2 paragraph: a branch scores the product of the drafter's confidences
along its path; the highest-scoring branches are kept, and a parent always
scores at least as high as its children).

- On random trees whose log-confidences are multiples of 1/8 (so every fp32
  path sum is exact), the kept set equals the top N by an independent exact
  score: integer path sums found by walking each node's ancestors, the lower
  index on ties.
- Every kept node's parent is kept, and the renumbered parent list points at it.
- A hand-worked five-candidate example with three-way ties.
- Special cases: keeping everything returns the input; all confidences 1
  keep the first N candidates; invalid input is refused.
"""
import numpy as np
import pytest


def _random_tree(rng, B, N):
    par = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(N):
            par[b, i] = rng.integers(0, i + 1)      # candidate i is node i + 1
    k = rng.integers(0, 24, size=(B, N))            # log-confidence -k/8
    tok = rng.integers(0, 1000, size=(B, N)).astype(np.int32)
    return par, tok, k


@pytest.mark.parametrize("N,N_keep", [(40, 10), (200, 63), (128, 127), (30, 1)])
def test_top_n_by_exact_path_score(oracle, N, N_keep):
    rng = np.random.default_rng(N + N_keep)
    B = 6
    par, tok, k = _random_tree(rng, B, N)
    res = oracle.select_tree(par, tok, (-k / 8.0).astype(np.float32), N_keep)
    for b in range(B):
        # exact score: minus the sum of k over the node and its ancestors
        exact = []
        for i in range(N):
            total, node = 0, i + 1
            while node > 0:
                total += int(k[b, node - 1])
                node = int(par[b, node - 1])
            exact.append((total, i))
        want = sorted(i for _, i in sorted(exact)[:N_keep])
        assert res["src"][b].tolist() == want
        assert np.array_equal(res["token"][b], tok[b, want])
        assert np.array_equal(res["score"][b], np.array([-exact[i][0] / 8.0 for i in want],
                                                        np.float32))
        # closure and renumbering: kept candidate k is node k + 1
        for kk, i in enumerate(want):
            p = int(par[b, i])
            q = int(res["parent"][b, kk])
            assert 0 <= q <= kk
            assert (p == 0 and q == 0) or (q > 0 and want[q - 1] == p - 1)


def test_hand_example_with_ties(oracle):
    """a (root child, 0.5), b (root child, 0.25), c (child of a, 0.5), d (child
    of a, 0.1), e (child of b, 1.0).  Path products: a 0.5, b 0.25, c 0.25,
    d 0.05, e 0.25.  Budget 3: a, then b and c win the three-way tie at 0.25
    by index.  Budget 4 adds e, whose parent b is new node 2."""
    par = np.array([[0, 0, 1, 1, 2]], np.int32)
    tok = np.array([[10, 11, 12, 13, 14]], np.int32)
    lp = np.log(np.array([[0.5, 0.25, 0.5, 0.1, 1.0]])).astype(np.float32)
    r3 = oracle.select_tree(par, tok, lp, 3)
    assert r3["src"].tolist() == [[0, 1, 2]]
    assert r3["parent"].tolist() == [[0, 0, 1]]
    assert r3["token"].tolist() == [[10, 11, 12]]
    r4 = oracle.select_tree(par, tok, lp, 4)
    assert r4["src"].tolist() == [[0, 1, 2, 4]]
    assert r4["parent"].tolist() == [[0, 0, 1, 2]]


def test_special_cases(oracle):
    rng = np.random.default_rng(3)
    par, tok, k = _random_tree(rng, 3, 50)
    lp = (-k / 8.0).astype(np.float32)
    everything = oracle.select_tree(par, tok, lp, 50)
    assert np.array_equal(everything["src"], np.tile(np.arange(50, dtype=np.int32), (3, 1)))
    assert np.array_equal(everything["parent"], par)
    ones = oracle.select_tree(par, tok, np.zeros_like(lp), 20)
    assert np.array_equal(ones["src"], np.tile(np.arange(20, dtype=np.int32), (3, 1)))
    bad = lp.copy()
    bad[1, 7] = 0.5                                   # a confidence above 1
    with pytest.raises(RuntimeError):
        oracle.select_tree(par, tok, bad, 20)
    bad_par = par.copy()
    bad_par[0, 3] = 9                                 # a parent after its child
    with pytest.raises(RuntimeError):
        oracle.select_tree(bad_par, tok, lp, 20)
