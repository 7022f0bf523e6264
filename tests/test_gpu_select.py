"""GPU parity of dynamic draft-tree selection (spec_select_tree) against the
oracle, through the C ABI: kept candidates, renumbered parents, tokens, source
indices and fp32 path scores bit for bit.

- random trees of 40 to 1024 candidates with budgets from 1 to 127, with many
  exact ties (log-confidences on a 1/8 grid) and with continuous confidences;
- a deep chain (the level-by-level scoring takes one round per depth);
- a sequence with a confidence above 1: its list is flagged, and the explicit
  tree build turns it into a root-only tree;
- the kept list feeds spec_build_tree (explicit), whose tree matches the
  oracle's build of the oracle's list.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_beam_amd import binding as sv

from test_gpu_parity import log

pytestmark = pytest.mark.gpu


def gpu_select(par, tok, lp, N_keep):
    B, N = par.shape
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = dict(parent=torch.full((B, N_keep), -7, dtype=torch.int32, device=dev),
               token=torch.full((B, N_keep), -7, dtype=torch.int32, device=dev),
               src=torch.full((B, N_keep), -7, dtype=torch.int32, device=dev),
               score=torch.full((B, N_keep), float("nan"), device=dev))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sv.spec_select_tree(B, N, N_keep, t(par.astype(np.int32)), t(tok.astype(np.int32)),
                        t(lp.astype(np.float32)), out["parent"], out["token"], out["src"],
                        out["score"], status)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["status"] = int(status.item())
    return res


def random_tree(rng, B, N, grid=True):
    par = np.array([[rng.integers(0, i + 1) for i in range(N)] for _ in range(B)], np.int32)
    tok = rng.integers(0, 128000, size=(B, N)).astype(np.int32)
    if grid:
        lp = (-rng.integers(0, 24, size=(B, N)) / 8.0).astype(np.float32)
    else:
        lp = np.log(rng.uniform(0.01, 1.0, size=(B, N))).astype(np.float32)
    return par, tok, lp


def assert_same(res, ref, what):
    for key in ("parent", "token", "src", "score"):
        assert np.array_equal(res[key], ref[key]), (what, key, res[key][:1], ref[key][:1])


@pytest.mark.parametrize("B,N,N_keep,grid", [(8, 40, 10, True), (4, 1024, 127, True),
                                            (16, 232, 16, False), (3, 300, 1, True),
                                            (2, 777, 63, False)])
def test_select_matches_oracle(gpu, B, N, N_keep, grid):
    rng = np.random.default_rng(N + N_keep)
    log(f"case select tree B={B} N={N} keep={N_keep} grid={grid}")
    par, tok, lp = random_tree(rng, B, N, grid)
    res = gpu_select(par, tok, lp, N_keep)
    assert res["status"] == 0
    assert_same(res, oracle.select_tree(par, tok, lp, N_keep), f"N={N} keep={N_keep}")


def test_select_deep_chain(gpu):
    N = 300
    par = np.arange(N, dtype=np.int32)[None, :]          # candidate i hangs below node i
    tok = np.arange(N, dtype=np.int32)[None, :]
    lp = np.full((1, N), -0.125, np.float32)
    log("case select tree, a 300-deep chain")
    res = gpu_select(par, tok, lp, 100)
    assert_same(res, oracle.select_tree(par, tok, lp, 100), "chain")
    assert res["src"][0].tolist() == list(range(100))


def test_select_flags_bad_input_and_feeds_the_build(gpu):
    rng = np.random.default_rng(9)
    B, N, K = 4, 232, 16
    par, tok, lp = random_tree(rng, B, N, grid=False)
    lp[2, 17] = 0.25                                    # a confidence above 1
    log("case select tree -> explicit build, one flagged sequence")
    res = gpu_select(par, tok, lp, K)
    assert res["status"] & 0x1
    assert np.all(res["parent"][2] == -1)
    good = [0, 1, 3]
    ref = oracle.select_tree(par[good], tok[good], lp[good], K)
    for key in ("parent", "token", "src", "score"):
        assert np.array_equal(res[key][good], ref[key]), key
    # the kept lists (flagged one included) through the explicit tree build
    dev = torch.device("cuda:0")
    T_cap = K + 1
    i32 = dict(dtype=torch.int32, device=dev)
    n_nodes, status = torch.zeros(B, **i32), torch.zeros(1, **i32)
    parent, token, depth = (torch.zeros((B, T_cap), **i32) for _ in range(3))
    anc = torch.zeros((B, T_cap, 1), dtype=torch.int64, device=dev)
    root = torch.arange(B, **i32)
    sv.spec_build_tree(sv.SPEC_TREE_EXPLICIT, B, 1, K, T_cap,
                       torch.from_numpy(res["token"]).to(dev),
                       torch.from_numpy(res["parent"]).to(dev), root, n_nodes, parent, token,
                       depth, anc, None, status)
    torch.cuda.synchronize()
    nn = n_nodes.cpu().numpy()
    assert nn[2] == 1 and int(status.item()) & 0x1
    tr = oracle.build_tree_explicit(ref["parent"], ref["token"], np.array(good, np.int32), T_cap)
    assert np.array_equal(nn[good], tr["n_nodes"])
    assert np.array_equal(parent.cpu().numpy()[good], tr["parent"])
    assert np.array_equal(anc.cpu().numpy().view(np.uint64)[good], tr["anc"])
