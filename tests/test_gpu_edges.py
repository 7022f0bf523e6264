"""GPU parity on the edge cases of the method, through the C ABI, against the oracle.

- the largest tree (127 positions: two mask words) with ragged context lengths,
  including a sequence with no context at all (its first key tile holds only
  tree keys), in all three verify modes and a planted greedy path;
- head dimension 64 on the bf16 path and a grouped fp32 case;
- a star tree (every candidate a child of the root) in all modes;
- a context that overflows the launch bound: that sequence gets zero rows and
  the device status bit, the others stay exact;
- B = 0 calls (host-only, in test_abi.py);
- one attention call launched forty times, each checked (intermittent errors),
  on the staged plan and on the direct-to-LDS GQA plan;
- the greedy walk on explicit trees whose siblings share tokens (several
  survivors per depth), on a vocabulary that is not a multiple of 4 (scalar
  loads) and on a tree that fails validation.
Bar as in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_beam_amd import pipeline, synth

from test_gpu_parity import (assert_tree_equal, assert_verify_equal, attn_bar, log, oracle_tree,
                             oracle_verify)

pytestmark = pytest.mark.gpu

MODES = ("greedy", "reject_path", "reject_recursive", "greedy_walk")


def run_all_modes(gpu, inp, what, planted=True):
    tr = oracle_tree(inp)
    for mode in MODES:
        step = pipeline.Step(inp, mode)
        res = step.run(compact=False)
        assert res["status"] == 0, gpu.decode_status(res["status"])
        assert_tree_equal(res, tr)
        assert_verify_equal(res, oracle_verify(inp, tr, mode), f"{what} {mode}")
        if mode == "greedy":
            ref = oracle.tree_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"],
                                        tr["n_nodes"], tr["anc"])
            attn_bar(res["attn"], ref, what)
            k0, v0 = inp["k"].copy(), inp["v"].copy()
            step.compact()
            torch.cuda.synchronize()
            new_ctx = oracle.kv_compact(k0, v0, inp["ctx_len"], res["acc_len"], res["acc_path"])
            view = torch.int16 if step.k.dtype == torch.bfloat16 else torch.int32
            assert np.array_equal(step.k.view(view).cpu().numpy().view(k0.dtype), k0)
            assert np.array_equal(step.v.view(view).cpu().numpy().view(v0.dtype), v0)
            assert np.array_equal(step.ctx_len[:inp["B"]].cpu().numpy(), new_ctx)
    if planted:
        # plant a full path so greedy accepts every node of one branch and the
        # bonus token comes from the leaf
        tgt = inp["tgt"].copy()
        for b in range(inp["B"]):
            t = int(tr["n_nodes"][b]) - 1          # the last node: walk its path
            path = []
            while t > 0:
                path.append(t)
                t = int(tr["parent"][b, t])
            for t in path:
                par = int(tr["parent"][b, t])
                tgt[b, par, tr["token"][b, t]] = tgt[b, par].max() + 20.0
        inp2 = dict(inp, tgt=tgt)
        for mode in ("greedy", "greedy_walk"):
            step = pipeline.Step(inp2, mode, with_kv=False)
            res = step.run()
            ref = oracle_verify(inp2, tr, mode)
            assert_verify_equal(res, ref, f"{what} {mode} planted")
            assert ref["acc_len"].min() >= 1


def test_largest_tree_ragged_context(gpu):
    inp = synth.make_custom_inputs(9001, B=3, H=8, Hkv=2, D=128, V=3000, dtype="bf16",
                                   ctx_lens=[0, 77, 300], tree="beams", W=18, L=7)
    assert inp["T_cap"] == 127
    log(f"case largest tree T_cap={inp['T_cap']} ctx={inp['ctx_len'].tolist()}")
    run_all_modes(gpu, inp, "T_cap=127")


def test_head_dim_64_bf16(gpu):
    inp = synth.make_custom_inputs(9002, B=2, H=4, Hkv=1, D=64, V=2000, dtype="bf16",
                                   ctx_lens=[200, 129], tree="beams", W=4, L=4)
    log("case D=64 bf16 G=4")
    run_all_modes(gpu, inp, "D=64")


def test_fp32_grouped(gpu):
    inp = synth.make_custom_inputs(9003, B=2, H=8, Hkv=2, D=32, V=1500, dtype="f32",
                                   ctx_lens=[50, 0], tree="beams", W=3, L=5)
    log("case fp32 G=4 D=32")
    run_all_modes(gpu, inp, "fp32 GQA")


def test_star_tree(gpu):
    inp = synth.make_custom_inputs(9004, B=2, H=4, Hkv=4, D=128, V=4000, dtype="bf16",
                                   ctx_lens=[130, 64], tree="explicit", parents=[0] * 40)
    log("case star tree, 40 children of the root")
    run_all_modes(gpu, inp, "star")


def test_context_overflow_flags_one_sequence(gpu):
    inp = synth.make_custom_inputs(9005, B=3, H=8, Hkv=8, D=128, V=1000, dtype="bf16",
                                   ctx_lens=[100, 120, 90], tree="beams", W=4, L=3)
    log("case context past the launch bound in sequence 1")
    tr = oracle_tree(inp)
    step = pipeline.Step(inp, "greedy")
    step.build_tree()
    step.ctx_len[1] = step.max_ctx + 1        # beyond the host bound of the launch
    step.attention()
    torch.cuda.synchronize()
    status = int(step.status.item())
    assert status & 0x8, gpu.decode_status(status)
    got = step.out.float().cpu().numpy()
    assert np.all(got[1] == 0)
    ref = oracle.tree_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tr["n_nodes"],
                                tr["anc"])
    for b in (0, 2):
        attn_bar(got[b], ref[b], f"overflow case, sequence {b}")


def test_large_batch_large_vocab(gpu):
    """Many sequences with a large vocabulary: each sequence gets few select
    workgroups, so their vocabulary slices exceed what the register cache of
    the row pair holds and the residual passes read the rows from memory."""
    inp = synth.make_custom_inputs(9006, B=64, H=1, Hkv=1, D=64, V=100000, dtype="bf16",
                                   ctx_lens=[16] * 64, tree="beams", W=2, L=2)
    log("case B=64, V=100000 (uncached residual passes)")
    tr = oracle_tree(inp)
    for mode in ("reject_path", "reject_recursive"):
        step = pipeline.Step(inp, mode, with_kv=False)
        res = step.run()
        assert res["status"] == 0, gpu.decode_status(res["status"])
        assert_verify_equal(res, oracle_verify(inp, tr, mode), f"B=64 V=1e5 {mode}")


def test_attention_repeated_launches_match(gpu):
    """Forty launches of one attention call whose plan has two query tiles per
    wave, two 4-wave row blocks of direct loads (196 rows) and two-tile context
    splits (the tree keys fall in the first tile of the last split).  Every launch must match
    the oracle: a wrongly unmasked tree key shows up as an intermittent error,
    so one launch is not enough."""
    inp = synth.make_inputs(4, 100, B_override=1, ctx_override=3000)
    log("case repeated attention launches, B=1 ctx=3000 G=4")
    tr = oracle_tree(inp)
    ref = oracle.tree_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tr["n_nodes"],
                                tr["anc"])
    step = pipeline.Step(inp, "greedy")
    step.build_tree()
    for rep in range(40):
        step.out.fill_(float("nan"))
        step.attention()
        torch.cuda.synchronize()
        assert int(step.status.item()) == 0
        attn_bar(step.out.float().cpu().numpy(), ref, f"launch {rep}")


def test_direct_load_attention_repeated_launches_match(gpu):
    """Forty launches of the 70B-class GQA plan that loads its K/V tiles
    straight into LDS and computes the next tile's scores beside this tile's
    softmax (two sequences, 1000-key contexts: five 128-row blocks per key
    range, six context splits, the tree keys in the last split).  Every
    launch must match the oracle, so that a race between the loads into LDS
    and the barrier that hands a stage over would show."""
    inp = synth.make_inputs(3, 100, B_override=2, ctx_override=1000)
    log("case repeated direct-load attention launches, B=2 ctx=1000 G=8")
    tr = oracle_tree(inp)
    ref = oracle.tree_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tr["n_nodes"],
                                tr["anc"])
    step = pipeline.Step(inp, "greedy")
    step.build_tree()
    for rep in range(40):
        step.out.fill_(float("nan"))
        step.attention()
        torch.cuda.synchronize()
        assert int(step.status.item()) == 0
        attn_bar(step.out.float().cpu().numpy(), ref, f"launch {rep}")


def test_greedy_walk_duplicate_siblings_and_odd_vocab(gpu):
    """Explicit trees whose siblings repeat a token: several nodes of one depth
    survive, and the walk scans all their rows in node order.  V = 3001 takes the
    scalar-load scan; V = 3000 the 16-byte one."""
    parents = [0, 0, 0, 1, 1, 2, 3, 3, 4, 6, 6, 7, 9, 9, 10, 0, 15, 15]
    for V in (3000, 3001):
        inp = synth.make_custom_inputs(9010 + V, B=6, H=4, Hkv=4, D=64, V=V, dtype="bf16",
                                       ctx_lens=[8] * 6, tree="explicit", parents=parents)
        rng = np.random.default_rng(V)
        inp["cand_token"] = rng.integers(0, 3, size=inp["cand_token"].shape).astype(np.int32)
        tr = oracle_tree(inp)
        tgt = inp["tgt"].copy()
        for b in range(inp["B"]):
            for t in range(int(tr["n_nodes"][b])):
                if rng.random() < 0.7:
                    tgt[b, t, rng.integers(0, 3)] = tgt[b, t].max() + 5.0
        inp2 = dict(inp, tgt=tgt)
        log(f"case greedy walk, duplicate siblings, V={V}")
        ref = oracle_verify(inp2, tr, "greedy_walk")
        assert (ref["rows_read"] >= 3).any()
        step = pipeline.Step(inp2, "greedy_walk", with_kv=False)
        res = step.run()
        assert res["status"] == 0, gpu.decode_status(res["status"])
        assert_verify_equal(res, ref, f"walk duplicates V={V}")
        full = oracle_verify(inp2, tr, "greedy")
        for key in ("acc_len", "acc_path", "next_token"):
            assert np.array_equal(res[key], full[key]), key


def test_greedy_walk_bad_tree(gpu):
    """A candidate naming a later parent: the tree build flags the sequence and
    the walk accepts nothing and takes the root's greedy token."""
    inp = synth.make_inputs(4, 301, B_override=2, ctx_override=100)
    inp["cand_parent"] = inp["cand_parent"].copy()
    inp["cand_parent"][1, 5] = 9
    log("case greedy walk on a flagged tree")
    step = pipeline.Step(inp, "greedy_walk")
    res = step.run()
    assert res["status"] & 0x1
    assert res["acc_len"][1] == 0 and res["acc_path"][1, 0] == 0
    assert np.all(res["acc_path"][1, 1:] == -1) and np.all(res["decision"][1] == -1)
    assert res["next_token"][1] == int(np.argmax(inp["tgt"][1, 0]))
    tr = oracle_tree(inp)
    ref = oracle.verify_greedy_walk(inp["tgt"][:1], tr["n_nodes"][:1], tr["parent"][:1],
                                    tr["token"][:1], tr["depth"][:1])
    for key in ("acc_len", "acc_path", "next_token", "decision"):
        assert np.array_equal(res[key][:1], ref[key]), key


def test_greedy_walk_reuses_its_workspace(gpu):
    """The walk's meeting counters return to zero after every call: two input
    sets alternate on one workspace (a stale counter would let a meeting read
    entries of the other set), each call checked against the oracle.  The row
    slices of a 32k vocabulary go to several workgroups per sequence."""
    sets = []
    for seed in (302, 303):
        inp = synth.make_inputs(1, seed)
        tr = oracle_tree(inp)
        inp2 = dict(inp, tgt=plant_greedy_all(inp, tr) if seed == 302 else inp["tgt"])
        sets.append((inp2, oracle_verify(inp2, tr, "greedy_walk")))
    assert sets[0][1]["acc_len"][0] >= 2
    log("case greedy walk, two input sets alternating on one workspace")
    steps = [pipeline.Step(inp, "greedy_walk", with_kv=False) for inp, _ in sets]
    steps[1].ver_ws, steps[1].ver_ws_bytes = steps[0].ver_ws, steps[0].ver_ws_bytes
    for rep in range(6):
        st, (_, ref) = steps[rep % 2], sets[rep % 2]
        res = st.run()
        assert res["status"] == 0, gpu.decode_status(res["status"])
        assert_verify_equal(res, ref, f"walk call {rep}")


def plant_greedy_all(inp, tr):
    """Make the first beam's whole path the greedy path of every sequence."""
    tgt = inp["tgt"].copy()
    for b in range(inp["B"]):
        for k in range(inp["L"]):
            par = 0 if k == 0 else tr["beam_node"][b, 0, k - 1]
            tgt[b, par, inp["beams"][b, 0, k]] = tgt[b, par].max() + 20.0
    return tgt


def test_meeting_kernels_launched_cooperatively(gpu, monkeypatch):
    """SPEC_COOPERATIVE_LAUNCH=1 launches the grids whose workgroups meet (the
    split select of the rejection modes, the greedy walk) cooperatively; the
    results are the same as the oracle's."""
    monkeypatch.setenv("SPEC_COOPERATIVE_LAUNCH", "1")
    inp = synth.make_inputs(4, 303, B_override=1, ctx_override=200)
    tr = oracle_tree(inp)
    log("case cooperative launches: sequential rejection, greedy walk")
    step = pipeline.Step(inp, "reject_recursive", with_kv=False)
    res = step.run()
    assert res["status"] == 0, gpu.decode_status(res["status"])
    assert_verify_equal(res, oracle_verify(inp, tr, "reject_recursive"), "cooperative recursive")
    inp1 = synth.make_inputs(1, 304)
    tr1 = oracle_tree(inp1)
    step = pipeline.Step(inp1, "greedy_walk", with_kv=False)
    res = step.run()
    assert res["status"] == 0, gpu.decode_status(res["status"])
    assert_verify_equal(res, oracle_verify(inp1, tr1, "greedy_walk"), "cooperative walk")
