"""GPU parity of the rejection-mode walks (SPEC_REJECT_PATH_WALK and
SPEC_REJECT_RECURSIVE_WALK: rejection sampling that reads only the rows of
nodes whose path is accepted) against the oracle's walks, through the C ABI.

Bar as in test_gpu_parity.py: acceptance length, path, next token and the
decisions of tested nodes bit-exact (sequences with a near-tie on either side
excepted and counted), p / q of the tested nodes within 1e-5.

- every rejection workload at oracle-sized shapes and the 70B-class GQA and
  32k-context multi-candidate workloads at full size (all 16 and 4 sequences,
  full vocabularies);
- the largest tree (127 positions) and a star tree, a vocabulary that is not a
  multiple of 4 (scalar loads), a bad tree;
- one million trials of sequential rejection at V = 16 with N = 4 i.i.d.
  candidates from q: chi-square against p, with element-wise parity against the
  oracle on the first call.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from tree_attention_verification_beam_amd import pipeline, synth

from test_gpu_distribution import _chi2_pvalue, _first_emitted, _logits
from test_gpu_parity import assert_tree_equal, assert_verify_equal, log, oracle_tree

pytestmark = pytest.mark.gpu

WALK = {"reject_path_walk": "reject_path", "reject_recursive_walk": "reject_recursive"}


def oracle_walk(inp, tr, mode):
    return oracle.verify_reject_walk(WALK[mode], inp["tgt"], inp["dft"], inp["dft_row"],
                                     tr["n_nodes"], tr["parent"], tr["token"], tr["depth"],
                                     inp["u_node"], inp["u_final"])


def run_case(gpu, inp, mode, what):
    tr = oracle_tree(inp)
    step = pipeline.Step(inp, mode, with_kv=False)
    res = step.run()
    assert res["status"] == 0, gpu.decode_status(res["status"])
    assert_tree_equal(res, tr)
    ref = oracle_walk(inp, tr, mode)
    assert_verify_equal(res, ref, f"{what} {mode}")
    return res, ref


CASES = [(0, 0, {}), (0, 1, {}), (1, 0, {}), (1, 2, {}), (3, 0, dict(B_override=3)),
         (4, 0, dict(B_override=2)), (4, 1, dict(B_override=1))]


@pytest.mark.parametrize("mode", list(WALK))
@pytest.mark.parametrize("wid,seed,ov", CASES)
def test_reduced(gpu, mode, wid, seed, ov):
    inp = synth.make_inputs(wid, 600 + seed, with_kv=False, **ov)
    log(f"case {mode} wid={wid} seed={seed} B={inp['B']} V={inp['V']}")
    run_case(gpu, inp, mode, f"wid {wid}")


@pytest.mark.parametrize("wid,mode", [(3, "reject_path_walk"), (4, "reject_recursive_walk"),
                                      (3, "reject_recursive_walk")])
def test_full_size(gpu, wid, mode):
    inp = synth.make_inputs(wid, 700, with_kv=False)
    log(f"case full size {mode} wid={wid} B={inp['B']} V={inp['V']}")
    res, ref = run_case(gpu, inp, mode, f"full wid {wid}")
    log(f"  rows read per sequence: target {ref['rows_tgt'].mean():.1f}, "
        f"draft {ref['rows_dft'].mean():.1f}")


@pytest.mark.parametrize("mode", list(WALK))
def test_largest_tree_star_odd_vocab(gpu, mode):
    inp = synth.make_custom_inputs(9101, B=3, H=4, Hkv=4, D=64, V=3001, dtype="f32",
                                   ctx_lens=[4, 4, 4], tree="beams", W=9, L=14)
    log(f"case {mode} largest tree, V=3001")
    run_case(gpu, inp, mode, "T_cap 127 odd V")
    inp = synth.make_custom_inputs(9102, B=4, H=4, Hkv=4, D=64, V=2048, dtype="f32",
                                   ctx_lens=[4] * 4, tree="explicit", parents=[0] * 60)
    log(f"case {mode} star tree")
    run_case(gpu, inp, mode, "star")


@pytest.mark.parametrize("mode", list(WALK))
def test_bad_tree(gpu, mode):
    """A token outside the vocabulary: that sequence accepts nothing, takes the
    root's greedy token and raises SPEC_DEV_BAD_TOKEN; the other is exact."""
    inp = synth.make_inputs(1, 610, with_kv=False)
    inp2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    for k in ("tgt", "dft", "dft_row", "u_node", "u_final", "root_token", "ctx_len"):
        inp2[k] = np.concatenate([inp[k], inp[k]], axis=0)
    inp2["beams"] = np.concatenate([inp["beams"], inp["beams"]], axis=0)
    inp2["beams"][1, 0, 0] = inp["V"] + 5
    inp2["B"] = 2
    log(f"case {mode} bad token in sequence 1")
    step = pipeline.Step(inp2, mode, with_kv=False)
    res = step.run()
    assert res["status"] & 0x2
    assert res["acc_len"][1] == 0
    assert res["next_token"][1] == int(np.argmax(inp2["tgt"][1, 0]))
    tr = oracle_tree(inp)
    ref = oracle_walk(inp, tr, mode)
    one = {k: v[:1] for k, v in res.items() if isinstance(v, np.ndarray)}
    assert_verify_equal(one, ref, f"{mode} good sequence beside a bad one")


def test_sequential_walk_reproduces_target(gpu):
    """One million trials, V = 16, a root with 4 i.i.d. children from q."""
    N, TRIALS, CHUNK, V = 4, 1_000_000, 250_000, 16
    lp, lq = _logits(104, 1.5)
    q = softmax(lq.astype(np.float64))
    rng = np.random.default_rng(4)
    counts = np.zeros(V, np.int64)
    log(f"case sequential walk chi-square, N={N}, {TRIALS} trials")
    for start in range(0, TRIALS, CHUNK):
        B = min(CHUNK, TRIALS - start)
        T_cap = N + 1
        cand = rng.choice(V, size=(B, N), p=q).astype(np.int32)
        tgt = np.ascontiguousarray(np.broadcast_to(lp, (B, T_cap, V)))
        dft = np.ascontiguousarray(np.broadcast_to(lq, (B, 1, V)))
        dft_row = np.full((B, T_cap), -1, np.int32)
        dft_row[:, 0] = 0
        inp = dict(B=B, T_cap=T_cap, V=V, tree="explicit", cand_token=cand,
                   cand_parent=np.zeros((B, N), np.int32), root_token=np.zeros(B, np.int32),
                   tgt=tgt, dft=dft, dft_row=dft_row, u_node=synth.exact_uniforms(rng, (B, T_cap)),
                   u_final=synth.exact_uniforms(rng, (B,)))
        res = pipeline.Step(inp, "reject_recursive_walk", with_kv=False).run()
        assert res["status"] == 0, res["status"]
        x = _first_emitted(res["token"], res["acc_len"], res["acc_path"], res["next_token"])
        counts += np.bincount(x, minlength=V)
        if start == 0:
            tr = oracle.build_tree_explicit(inp["cand_parent"], cand, inp["root_token"], T_cap)
            ref = oracle_walk(inp, tr, "reject_recursive_walk")
            ok = (res["near_tie"] == 0) & (ref["near_tie"] == 0)
            assert int((~ok).sum()) <= B // 1000
            for k in ("acc_len", "acc_path", "next_token", "decision"):
                assert np.array_equal(res[k][ok], ref[k][ok]), k
    pv = _chi2_pvalue(counts, softmax(lp.astype(np.float64)))
    log(f"  chi-square p-value {pv:.4f}")
    assert pv >= 1e-3
