"""GPU parity of the beam-search pruning step (spec_beam_topk) against the oracle,
through the C ABI: parents, tokens, scores and histories bit for bit.

- beam widths 1, 8 and 16; vocabularies that are and are not multiples of 4
  (16-byte and scalar loads); K_out of 1, 8 and 16;
- many exact ties across beams and slices (lower flattened index first), -inf
  tokens, and asking for every extension of a small grid;
- a 70B-scale step (16 sequences x 16 beams x 128256 tokens), checked on
  every sequence;
- five chained steps from one row: the histories become the [B][W][L] beams of
  spec_build_tree, whose tree matches the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_beam_amd import binding as sv

from test_gpu_parity import log

pytestmark = pytest.mark.gpu


def gpu_topk(logp, beam_score, K_out, hist=None):
    B, K_in, V = logp.shape
    dev = torch.device("cuda:0")
    t_logp = torch.from_numpy(np.ascontiguousarray(logp, np.float32)).to(dev)
    t_bs = None if beam_score is None else torch.from_numpy(
        np.ascontiguousarray(beam_score, np.float32)).to(dev)
    par = torch.full((B, K_out), -7, dtype=torch.int32, device=dev)
    tok = torch.full((B, K_out), -7, dtype=torch.int32, device=dev)
    sc = torch.full((B, K_out), float("nan"), dtype=torch.float32, device=dev)
    nb = sv.spec_beam_topk_workspace_size(B, K_in, K_out, V)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    h_in = h_out = None
    length = 0
    if hist is not None:
        length = hist.shape[2]
        h_in = torch.from_numpy(np.ascontiguousarray(hist, np.int32)).to(dev)
        h_out = torch.full((B, K_out, length + 1), -7, dtype=torch.int32, device=dev)
    sv.spec_beam_topk(B, K_in, K_out, V, t_logp, t_bs, par, tok, sc, h_in, length, h_out, ws, nb)
    torch.cuda.synchronize()
    out = dict(parent=par.cpu().numpy(), token=tok.cpu().numpy(), score=sc.cpu().numpy())
    if h_out is not None:
        out["hist"] = h_out.cpu().numpy()
    return out


def log_softmax(rng, shape):
    """Synthetic drafter rows: log-softmax of N(0, 3^2) logits, in fp32."""
    x = 3.0 * rng.standard_normal(shape)
    x -= x.max(axis=-1, keepdims=True)
    return (x - np.log(np.exp(x).sum(axis=-1, keepdims=True))).astype(np.float32)


def assert_same(res, ref, what):
    for key in ("parent", "token", "score") + (("hist",) if "hist" in ref else ()):
        assert np.array_equal(res[key], ref[key]), (what, key, res[key][:2], ref[key][:2])


@pytest.mark.parametrize("B,K_in,V,K_out", [(2, 8, 32000, 8), (3, 1, 5001, 16), (4, 16, 1000, 16),
                                            (2, 8, 32000, 1), (5, 2, 7, 14),
                                            (64, 4, 128000, 4)])
def test_beam_topk_matches_oracle(gpu, B, K_in, V, K_out):
    rng = np.random.default_rng(B * 100 + K_in * 10 + K_out)
    log(f"case beam top-K B={B} K_in={K_in} V={V} K_out={K_out}")
    logp = (rng.standard_normal((B, K_in, V)) - 8.0).astype(np.float32)
    logp[:, :, 1::5] = np.round(logp[:, :, 1::5], 0)        # exact ties across beams
    logp[:, :, 3::11] = -np.inf
    bs = None if K_in == 1 else np.round(rng.standard_normal((B, K_in)), 0).astype(np.float32)
    hist = rng.integers(0, V, size=(B, K_in, 3)).astype(np.int32)
    ref = oracle.beam_topk(logp, bs, K_out, hist=hist)
    res = gpu_topk(logp, bs, K_out, hist=hist)
    assert_same(res, ref, f"B={B} K_in={K_in} V={V} K_out={K_out}")


def test_beam_topk_70b_scale(gpu):
    B, K_in, V, K_out = 16, 16, 128256, 16
    rng = np.random.default_rng(11)
    log(f"case beam top-K B={B} K_in={K_in} V={V} K_out={K_out}")
    logp = log_softmax(rng, (B, K_in, V))
    bs = np.sort(rng.standard_normal((B, K_in)).astype(np.float32) - 3.0, axis=1)[:, ::-1].copy()
    res = gpu_topk(logp, bs, K_out)
    ref = oracle.beam_topk(logp, bs, K_out)
    assert_same(res, ref, "70B scale")


def test_beam_search_feeds_the_tree_build(gpu):
    """Five steps of pruning (fresh synthetic rows each step, as a drafter would
    give): the final histories are the beams input of spec_build_tree."""
    B, W, L, V = 3, 8, 5, 32000
    rng = np.random.default_rng(5)
    log("case beam search chain -> build tree")
    logp = log_softmax(rng, (B, 1, V))
    ref = oracle.beam_topk(logp, None, W, hist=np.zeros((B, 1, 0), np.int32))
    res = gpu_topk(logp, None, W, hist=np.zeros((B, 1, 0), np.int32))
    assert_same(res, ref, "step 1")
    for step in range(2, L + 1):
        logp = log_softmax(rng, (B, W, V))
        ref = oracle.beam_topk(logp, ref["score"], W, hist=ref["hist"])
        res = gpu_topk(logp, res["score"], W, hist=res["hist"])
        assert_same(res, ref, f"step {step}")
    beams = res["hist"]
    assert beams.shape == (B, W, L)
    root = rng.integers(0, V, size=B).astype(np.int32)
    T_cap = 1 + W * L
    tr = oracle.build_tree_beams(beams, root, T_cap)
    dev = torch.device("cuda:0")
    i32 = dict(dtype=torch.int32, device=dev)
    n_nodes = torch.zeros(B, **i32)
    parent = torch.zeros((B, T_cap), **i32)
    token = torch.zeros((B, T_cap), **i32)
    depth = torch.zeros((B, T_cap), **i32)
    anc = torch.zeros((B, T_cap, (T_cap + 63) // 64), dtype=torch.int64, device=dev)
    beam_node = torch.zeros((B, W, L), **i32)
    status = torch.zeros(1, **i32)
    sv.spec_build_tree(sv.SPEC_TREE_BEAMS, B, W, L, T_cap, torch.from_numpy(beams).to(dev), None,
                       torch.from_numpy(root).to(dev), n_nodes, parent, token, depth, anc,
                       beam_node, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(n_nodes.cpu().numpy(), tr["n_nodes"])
    assert np.array_equal(parent.cpu().numpy(), tr["parent"])
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), tr["anc"])
    # beams share prefixes: the tree is smaller than W * L + 1
    assert (tr["n_nodes"] < T_cap).any()
