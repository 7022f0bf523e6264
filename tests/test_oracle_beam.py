"""Pins of the oracle's beam-search pruning step (ReDrafter page, "Beam Search
During Inference", steps 1 and 3: every (beam, token) extension scores
score[j] + logp[j][v]; the K best of the K x |V| extensions become the next beams).

- The selection property itself, checked element by element on random inputs:
  outputs in descending (score, then lower flattened index) order, each output
  score equal to its own extension's fp32 sum, no two outputs alike, and no
  unselected extension ahead of the last selected one.
- Pure-Python brute force (heapq.nlargest over every extension) on tiny cases.
- A hand example with ties across beams and the history gather; the first
  step (one row, no beam scores); -inf tokens, and a full ordering.
"""
import heapq

import numpy as np
import pytest


def _scores(logp, beam_score):
    B, K, V = logp.shape
    bs = np.zeros((B, K), np.float32) if beam_score is None else beam_score.astype(np.float32)
    return (bs[:, :, None] + logp.astype(np.float32)).astype(np.float32)  # fp32 sum


def _rank_key(s, idx):
    return (float(s), -int(idx))


@pytest.mark.parametrize("K_in,V,K_out", [(8, 1000, 8), (8, 1000, 16), (1, 5000, 16), (16, 257, 3)])
def test_selection_property(oracle, K_in, V, K_out):
    rng = np.random.default_rng(K_in * 1000 + V + K_out)
    B = 5
    logp = rng.standard_normal((B, K_in, V)).astype(np.float32)
    logp[:, :, ::7] = np.round(logp[:, :, ::7], 1)          # many exact ties
    bs = np.round(rng.standard_normal((B, K_in)), 1).astype(np.float32)
    res = oracle.beam_topk(logp, bs, K_out)
    s = _scores(logp, bs).reshape(B, -1)
    for b in range(B):
        idx = res["parent"][b].astype(np.int64) * V + res["token"][b]
        assert len(set(idx.tolist())) == K_out
        assert np.array_equal(res["score"][b], s[b, idx])
        keys = [_rank_key(s[b, i], i) for i in idx]
        assert keys == sorted(keys, reverse=True)
        worst = keys[-1]
        chosen = set(idx.tolist())
        for i in range(s.shape[1]):
            if i not in chosen:
                assert _rank_key(s[b, i], i) < worst


def test_brute_force_tiny(oracle):
    rng = np.random.default_rng(7)
    for trial in range(20):
        K_in, V = int(rng.integers(1, 5)), int(rng.integers(1, 9))
        K_out = int(rng.integers(1, K_in * V + 1))
        logp = rng.integers(-3, 1, size=(2, K_in, V)).astype(np.float32)   # integers: ties
        bs = rng.integers(-2, 1, size=(2, K_in)).astype(np.float32)
        res = oracle.beam_topk(logp, bs, K_out)
        for b in range(2):
            ext = [(float(bs[b, j] + logp[b, j, v]), -(j * V + v))
                   for j in range(K_in) for v in range(V)]
            best = heapq.nlargest(K_out, ext)
            assert [(-i // V, -i % V) for _, i in best] == list(
                zip(res["parent"][b].tolist(), res["token"][b].tolist())), trial
            assert [x for x, _ in best] == res["score"][b].tolist()


def test_hand_example_ties_and_history(oracle):
    """Two beams of three tokens.  Beam scores 0 and -1; rows [-1, -2, -1] and
    [0, 0, -5] give extension scores [-1, -2, -1, -1, -1, -6].  Four extensions
    tie at -1: flattened indices 0, 2, 3, 4.  The best three are 0, 2, 3: beam 0
    token 0, beam 0 token 2, beam 1 token 0; histories [7] and [9] grow to
    [7, 0], [7, 2] and [9, 0]."""
    logp = np.array([[[-1, -2, -1], [0, 0, -5]]], np.float32)
    bs = np.array([[0, -1]], np.float32)
    hist = np.array([[[7], [9]]], np.int32)
    res = oracle.beam_topk(logp, bs, 3, hist=hist)
    assert res["parent"].tolist() == [[0, 0, 1]]
    assert res["token"].tolist() == [[0, 2, 0]]
    assert res["score"].tolist() == [[-1.0, -1.0, -1.0]]
    assert res["hist"].tolist() == [[[7, 0], [7, 2], [9, 0]]]


def test_first_step_and_infinities(oracle):
    """One row, no beam scores: the K largest logits by value, lower index on
    ties.  Tokens at -inf come last; asking for every extension orders them all."""
    row = np.array([[[2.0, -np.inf, 5.0, 2.0, -1.0, -np.inf]]], np.float32)
    res = oracle.beam_topk(row, None, 6)
    assert res["parent"].tolist() == [[0] * 6]
    assert res["token"].tolist() == [[2, 0, 3, 4, 1, 5]]
    assert res["score"][0, :4].tolist() == [5.0, 2.0, 2.0, -1.0]
    assert np.all(np.isneginf(res["score"][0, 4:]))
