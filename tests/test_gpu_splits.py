"""Tree attention across the context-split counts the plan can choose.

The context of a (sequence, KV head) is split over workgroups so that the grid
covers the CUs; a merge kernel then combines the (max, sum, O) partials.  The
shapes below make the plan choose 1, 2, 4, 21 and 32 splits (the last two with
two and with one key group), for 1024 (sequence, head) streams 4-wave groups,
24 splits of the 4-wave GQA plan that loads its tiles straight into LDS, one
8-wave row block of register-staged tiles (5 query tiles) and two 4-wave
direct-load row blocks (9 query tiles);
each is compared with the oracle within 1e-2 of the largest output, with
ragged contexts where B > 1.  The same GQA plan is also run without splits on
the 70B shape and on ranges shorter than one key tile.
"""
import numpy as np
import pytest

import oracle
from tree_attention_verification_beam_amd import pipeline, synth

from test_gpu_parity import attn_bar, log

pytestmark = pytest.mark.gpu

# (B, H, Hkv, context lengths): splits chosen by the plan for 4 beams of 4
CASES = {
    "1 split": (1, 2, 2, [150]),
    "2 splits": (4, 16, 16, [300, 41, 299, 0]),
    "4 splits": (2, 32, 32, [1000, 777]),
    "21 splits": (1, 1, 1, [4000]),
    "32 splits, GQA": (1, 4, 1, [8000]),
    # 1024 (sequence, head) streams of at most 32 rows: 4-wave groups
    "1024 streams": (32, 32, 32, [40 + 7 * i for i in range(32)]),
    # 272 rows per KV head: the 4-wave plan whose tiles go straight to LDS
    "24 splits, GQA direct loads": (1, 32, 2, [3000]),
    # 68 rows per KV head (5 query tiles): one 8-wave row block of
    # register-staged tiles, two query tiles per wave
    "one 8-wave row block": (2, 8, 2, [2000, 1500]),
    # 136 rows per KV head (9 query tiles): two 4-wave row blocks of direct
    # loads, the second with one live query tile
    "two direct-load row blocks": (2, 16, 2, [2000, 1500]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_attention_split_counts(gpu, case):
    B, H, Hkv, ctx = CASES[case]
    inp = synth.make_custom_inputs(9100 + len(case), B=B, H=H, Hkv=Hkv, D=128, V=500,
                                   dtype="bf16", ctx_lens=ctx, tree="beams", W=4, L=4)
    log(f"case {case}: B={B} H={H} Hkv={Hkv} ctx={ctx}")
    tr = oracle.build_tree_beams(inp["beams"], inp["root_token"], inp["T_cap"])
    res = pipeline.Step(inp, "greedy").run(compact=False)
    assert res["status"] == 0, gpu.decode_status(res["status"])
    ref = oracle.tree_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tr["n_nodes"],
                                tr["anc"])
    attn_bar(res["attn"], ref, case)
    for b in range(B):
        assert np.all(res["attn"][b, tr["n_nodes"][b]:] == 0)


def test_gqa_row_blocks_every_row(gpu):
    """The 70B-class GQA plan without context splits (16 sequences, 64 query
    heads on 8 KV heads, 16 beams of 4: up to 65 nodes, five 128-row blocks per
    (sequence, KV head) reading one key range), every row of every sequence
    against the oracle, with ragged contexts."""
    B, H, Hkv = 16, 64, 8
    ctx = [200 + 23 * i for i in range(B)]
    inp = synth.make_custom_inputs(9200, B=B, H=H, Hkv=Hkv, D=128, V=500, dtype="bf16",
                                   ctx_lens=ctx, tree="beams", W=16, L=4)
    log(f"case GQA row blocks: B={B} H={H} Hkv={Hkv} T_cap={inp['T_cap']} ctx={ctx[0]}..{ctx[-1]}")
    tr = oracle.build_tree_beams(inp["beams"], inp["root_token"], inp["T_cap"])
    res = pipeline.Step(inp, "greedy").run(compact=False)
    assert res["status"] == 0, gpu.decode_status(res["status"])
    ref = oracle.tree_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tr["n_nodes"],
                                tr["anc"])
    attn_bar(res["attn"], ref, "GQA row blocks")
    for b in range(B):
        assert np.all(res["attn"][b, tr["n_nodes"][b]:] == 0)


def test_gqa_direct_loads_short_ranges(gpu):
    """The direct-to-LDS GQA plan (16 query heads per KV head, 17 nodes: 272
    rows, three row blocks) on key ranges that end inside the first tile (no
    context, 5 context keys: the first tile is loaded over every cache slot
    and its rows past the range are zeroed in LDS) and inside the second tile
    (the loads' range check returns zeros), against the oracle; the cache
    slots past each sequence's keys hold NaN."""
    B, H, Hkv = 4, 32, 2
    ctx = [0, 5, 64, 130]
    inp = synth.make_custom_inputs(9300, B=B, H=H, Hkv=Hkv, D=128, V=500, dtype="bf16",
                                   ctx_lens=ctx, tree="beams", W=4, L=4)
    log(f"case GQA direct loads: B={B} H={H} Hkv={Hkv} T_cap={inp['T_cap']} ctx={ctx}")
    assert (H // Hkv) * inp["T_cap"] > 256
    tr = oracle.build_tree_beams(inp["beams"], inp["root_token"], inp["T_cap"])
    # cache slots past each sequence's keys hold NaN: none may reach an output
    assert inp["k"].dtype == np.uint16
    for b in range(B):
        end = ctx[b] + int(tr["n_nodes"][b])
        inp["k"][b, :, end:] = 0x7FC0
        inp["v"][b, :, end:] = 0x7FC0
    res = pipeline.Step(inp, "greedy").run(compact=False)
    assert res["status"] == 0, gpu.decode_status(res["status"])
    ref = oracle.tree_attention(inp["q"], inp["k"], inp["v"], inp["ctx_len"], tr["n_nodes"],
                                tr["anc"])
    attn_bar(res["attn"], ref, "GQA direct loads")
    for b in range(B):
        assert np.all(res["attn"][b, tr["n_nodes"][b]:] == 0)
