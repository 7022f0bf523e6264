"""GPU tests of the C-ABI contract beyond parity, through the C ABI:

- spec_last_device_status reads a caller's status word and the library's own
  word (used by calls passed no word), clearing only the library's;
- spec_kv_compact on paths of up to 127 nodes (a workgroup's LDS buffer
  full), against the oracle, with its arrival counters back at zero;
- the greedy walk and the one-pass verify on workspaces filled with arbitrary
  bytes before the first call (no initial contents are needed);
- the bandwidth probes read (and copy) exactly their buffers.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_attention_verification_beam_amd import binding as sv
from tree_attention_verification_beam_amd import pipeline, synth

from test_gpu_parity import assert_verify_equal, log, oracle_tree, oracle_verify

pytestmark = pytest.mark.gpu


def test_last_device_status_library_and_caller_words(gpu):
    """A bad explicit parent list raises SPEC_DEV_BAD_PARENT into the caller's
    word when one is passed and into the library's word when none is."""
    dev = torch.device("cuda:0")
    i32 = dict(dtype=torch.int32, device=dev)
    B, N, T_cap = 2, 4, 5
    cand_parent = torch.tensor([[0, 0, 1, 2], [0, 3, 1, 1]], **i32)  # b=1: parent 3 of node 2
    cand_token = torch.arange(B * N, **i32).reshape(B, N)
    root = torch.zeros(B, **i32)
    n_nodes = torch.zeros(B, **i32)
    par, tok, dep = (torch.zeros((B, T_cap), **i32) for _ in range(3))
    anc = torch.zeros((B, T_cap, 1), dtype=torch.int64, device=dev)
    log("case last device status: library word, then caller word")
    sv.spec_last_device_status(None)  # clear what earlier calls without a word left
    assert sv.spec_last_device_status(None) == 0
    sv.spec_build_tree(sv.SPEC_TREE_EXPLICIT, B, 1, N, T_cap, cand_token, cand_parent, root,
                       n_nodes, par, tok, dep, anc, None, None)
    assert sv.spec_last_device_status(None) == 0x1
    assert sv.spec_last_device_status(None) == 0          # read once, then cleared
    assert n_nodes.cpu().tolist() == [5, 1]
    word = torch.zeros(1, **i32)
    sv.spec_build_tree(sv.SPEC_TREE_EXPLICIT, B, 1, N, T_cap, cand_token, cand_parent, root,
                       n_nodes, par, tok, dep, anc, None, word)
    assert sv.spec_last_device_status(word) == 0x1
    assert sv.spec_last_device_status(word) == 0x1        # a caller's word is left as it is
    assert sv.spec_last_device_status(None) == 0          # the library's word was not used


@pytest.mark.parametrize("Hkv,D,dtype", [(32, 128, "bf16"), (8, 128, "f32"), (3, 64, "bf16")])
def test_compact_long_paths(gpu, Hkv, D, dtype):
    """Paths of up to 127 nodes over every (head, K|V) block: at 128 fp32
    values a 127-node path fills a workgroup's LDS buffer with one head, at 32
    heads of bf16 the workgroups take a few heads each; overlapping moves
    (path [0, 2, 3, ...]), an identity path, an empty path and a bad path (not
    increasing) in one call, with the arrival counters back at zero after it."""
    rng = np.random.default_rng(9100 + Hkv)
    T_cap, B, ctx0 = 128, 5, 300
    cap = ctx0 + T_cap + 7
    np_dt = np.float32 if dtype == "f32" else np.uint16
    k = rng.integers(0, 1 << 15, size=(B, Hkv, cap, D)).astype(np_dt) if dtype == "bf16" else \
        rng.standard_normal((B, Hkv, cap, D)).astype(np_dt)
    v = rng.integers(0, 1 << 15, size=(B, Hkv, cap, D)).astype(np_dt) if dtype == "bf16" else \
        rng.standard_normal((B, Hkv, cap, D)).astype(np_dt)
    ctx = np.array([ctx0, ctx0 - 17, 3, ctx0 + 1, 0], np.int32)
    acc_len = np.array([127, 60, 5, 0, 4], np.int32)
    path = np.full((B, T_cap), -1, np.int32)
    path[:, 0] = 0
    path[0, 1:128] = np.arange(1, 128)                              # identity, whole tree
    path[1, 1:61] = np.sort(rng.choice(np.arange(1, 128), 60, replace=False))
    path[2, 1:6] = [2, 3, 9, 10, 100]                               # overlapping moves
    path[4, 1:5] = [3, 2, 5, 6]                                     # not increasing: refused
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tk = torch.from_numpy(k.view(np.int16) if dtype == "bf16" else k).to(dev)
    tv = torch.from_numpy(v.view(np.int16) if dtype == "bf16" else v).to(dev)
    if dtype == "bf16":
        tk, tv = tk.view(tdt), tv.view(tdt)
    t_ctx = torch.from_numpy(ctx).to(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    nw = sv.spec_kv_compact_workspace_size(B)
    ws = torch.zeros(nw, dtype=torch.uint8, device=dev)
    log(f"case compact long paths Hkv={Hkv} D={D} {dtype}")
    sv.spec_kv_compact(sv.SPEC_BF16 if dtype == "bf16" else sv.SPEC_F32, B, Hkv, D, cap, T_cap,
                       tk, tv, t_ctx, torch.from_numpy(acc_len).to(dev),
                       torch.from_numpy(path).to(dev), ws, nw, status)
    torch.cuda.synchronize()
    assert int(ws.sum().item()) == 0  # the arrival counters are back at zero
    # the oracle commits the four valid sequences; the refused one is untouched
    k_ref, v_ref = k.copy(), v.copy()
    k4, v4 = np.ascontiguousarray(k_ref[:4]), np.ascontiguousarray(v_ref[:4])
    new_ctx = oracle.kv_compact(k4, v4, ctx[:4], acc_len[:4], path[:4])
    k_ref[:4], v_ref[:4] = k4, v4
    view = torch.int16 if dtype == "bf16" else torch.float32
    assert np.array_equal(tk.view(view).cpu().numpy().view(np_dt), k_ref)
    assert np.array_equal(tv.view(view).cpu().numpy().view(np_dt), v_ref)
    got_ctx = t_ctx.cpu().numpy()
    assert np.array_equal(got_ctx[:4], new_ctx)
    assert got_ctx.tolist() == [ctx0 + 128, ctx0 - 17 + 61, 9, ctx0 + 2, 0]
    assert int(status.item()) == 0x8  # the refused path of sequence 4


@pytest.mark.parametrize("mode", ["greedy_walk", "reject_recursive", "greedy", "reject_path_walk",
                                  "reject_recursive_walk"])
def test_verify_on_a_workspace_of_arbitrary_bytes(gpu, mode):
    """No initial workspace contents are needed: the workspace is filled with
    random bytes (and, for the walk, with words that carry plausible tags of
    other calls) before each of two calls on two input sets."""
    sets = []
    for seed in (312, 313):
        inp = synth.make_inputs(1, seed) if "recursive" not in mode else \
            synth.make_inputs(4, seed, B_override=2, ctx_override=100)
        tr = oracle_tree(inp)
        ref = oracle_verify(inp, tr, mode) if "walk" not in mode or mode == "greedy_walk" else \
            oracle.verify_reject_walk(mode.replace("_walk", ""), inp["tgt"], inp["dft"],
                                      inp["dft_row"], tr["n_nodes"], tr["parent"], tr["token"],
                                      tr["depth"], inp["u_node"], inp["u_final"])
        sets.append((inp, ref))
    steps = [pipeline.Step(inp, mode, with_kv=False) for inp, _ in sets]
    ws = steps[0].ver_ws
    steps[1].ver_ws, steps[1].ver_ws_bytes = ws, steps[0].ver_ws_bytes
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7)
    for rep in range(4):
        log(f"case {mode} on a workspace of arbitrary bytes, call {rep}")
        noise = torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=ws.device,
                              generator=gen)
        ws.copy_(noise)
        if rep == 3:
            ws.view(torch.int64)[:] = (rep << 40) | 5  # tag-like words, all equal
        st, (_, ref) = steps[rep % 2], sets[rep % 2]
        res = st.run()
        assert res["status"] == 0, sv.decode_status(res["status"])
        assert_verify_equal(res, ref, f"{mode} arbitrary workspace call {rep}")


@pytest.mark.parametrize("n_bytes,n_blocks", [(3 * (256 << 10) + 4096 + 48, 2), (256 << 10, 8), (16, 1)])
def test_read_probe_reads_every_byte_once(gpu, n_bytes, n_blocks):
    """The bandwidth probes read exactly their buffer: the streaming read's
    per-workgroup sums over a buffer of fp32 twos (whole 256 KiB chunks, a
    partial last chunk, fewer workgroups than chunks) add up to 2 * n_bytes / 4;
    the copy reproduces its source."""
    log(f"case read probe n_bytes={n_bytes} blocks={n_blocks}")
    src = torch.full((n_bytes // 4,), 2.0, dtype=torch.float32, device="cuda")
    out = torch.full((n_blocks,), -1.0, dtype=torch.float32, device="cuda")
    sv.spec_read_probe(src, n_bytes, out, n_blocks)
    torch.cuda.synchronize()
    assert float(out.double().sum()) == 2.0 * (n_bytes // 4)
    dst = torch.zeros_like(src)
    sv.spec_copy_probe(src, dst, n_bytes)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
