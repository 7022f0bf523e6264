"""Host-side arithmetic of the benchmark: algorithmic bytes and flops of the
calls, and the roofline bound they imply (no GPU needed).

Hand-worked values on small shapes; the 70B-class GQA shape sits above the
bf16 ridge (2.5 PFLOP/s over 8 TB/s = 312.5 flop/B) and the 7B-class shape
below it, as the arithmetic intensity of attention over a long context with
G query heads per KV head predicts (about G*T flops per K/V byte read).
"""
import numpy as np

import bench
from tree_attention_verification_beam_amd import synth


def _inp(B, ctx, H, Hkv, D, T_cap, V=100, dtype="bf16"):
    return dict(B=B, ctx_len=np.full(B, ctx, np.int32), H=H, Hkv=Hkv, D=D, T_cap=T_cap, V=V,
                dtype=dtype)


def test_attention_bytes_hand_worked():
    inp = _inp(B=2, ctx=10, H=4, Hkv=2, D=8, T_cap=5)
    n_nodes = np.array([3, 5], np.int32)
    # per sequence: K and V of ctx+T slots of 2 KV heads, q and out of T*H rows, masks
    want = 0
    for T in (3, 5):
        want += 2 * 2 * (10 + T) * 8 * 2 + 2 * T * 4 * 8 * 2 + T * 1 * 8
    assert bench.attention_bytes(inp, n_nodes) == want
    # fp32 doubles the element size; more than 64 tree slots need two mask words
    inp32 = _inp(B=1, ctx=0, H=1, Hkv=1, D=4, T_cap=65, dtype="f32")
    assert bench.attention_bytes(inp32, np.array([65])) == 2 * 65 * 4 * 4 + 2 * 65 * 4 * 4 + 65 * 2 * 8


def test_attention_flops_hand_worked():
    inp = _inp(B=2, ctx=10, H=4, Hkv=2, D=8, T_cap=5)
    # two MACs (Q K^T and P V) per (node, head, visible-or-not key, dim), 2 flops each
    assert bench.attention_flops(inp, np.array([3, 5])) == 4 * 4 * 8 * (3 * 13 + 5 * 15)


def test_ridge_separates_the_gqa_shape():
    ridge = bench.BF16_MFMA_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBPS * 1e9)
    assert abs(ridge - 312.5) < 1e-9
    for wid, above in ((1, False), (2, False), (3, True), (4, False)):
        w = synth.WORKLOADS[wid]
        T = w.T_cap * 2 // 3  # a typical tree size
        inp = _inp(B=w.B, ctx=w.ctx, H=w.H, Hkv=w.Hkv, D=w.D, T_cap=w.T_cap)
        nn = np.full(w.B, T, np.int32)
        ai = bench.attention_flops(inp, nn) / bench.attention_bytes(inp, nn)
        assert (ai > ridge) == above, (wid, ai)


def test_verify_bytes_modes():
    V = 10
    inp = dict(B=1, V=V)
    n_nodes = np.array([4])
    parent = np.array([[-1, 0, 0, 1]])         # node 1 has a child, the root has two
    dft_row = np.array([[0, 1, -1, -1]])
    # greedy: every target row of the tree
    assert bench.verify_bytes(inp, n_nodes, parent, dft_row, "greedy") == 4 * V * 4
    # rejection: plus the draft rows of the nodes with children (root and node 1)
    assert bench.verify_bytes(inp, n_nodes, parent, dft_row, "reject_path") == 6 * V * 4
    # walk: the root's row and one row per accepted tested node
    decision = np.array([[-1, 1, 0, 1]])
    assert bench.verify_bytes(inp, n_nodes, parent, dft_row, "greedy_walk", decision) == 3 * V * 4
