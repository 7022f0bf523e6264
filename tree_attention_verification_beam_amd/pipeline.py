"""One verification step on the GPU: the four C-ABI calls in order.

``Step`` places a step's inputs in device memory (torch allocations), owns the
output and workspace buffers, and enqueues spec_build_tree ->
spec_tree_attention -> spec_verify -> spec_kv_compact on one stream.  All
arithmetic happens in the HIP library; this module only allocates and copies.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as sv


def _dev(a, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


class Step:
    """Device-resident buffers of one step of a synthetic workload (see synth)."""

    def __init__(self, inp: dict, mode: str, device="cuda:0", with_kv: bool = True):
        self.inp = inp
        self.mode = sv.MODES[mode]
        self.device = torch.device(device)
        B, T_cap, V = inp["B"], inp["T_cap"], inp["V"]
        self.B, self.T_cap, self.V = B, T_cap, V
        self.n_words = (T_cap + 63) // 64
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        # tree inputs
        if inp["tree"] == "beams":
            self.kind, self.W, self.L = sv.SPEC_TREE_BEAMS, inp["W"], inp["L"]
            self.cand_token = _dev(inp["beams"], dev)
            self.cand_parent = None
            self.beam_node = torch.zeros((B, self.W, self.L), **i32)
        else:
            self.kind, self.W, self.L = sv.SPEC_TREE_EXPLICIT, 1, inp["cand_token"].shape[1]
            self.cand_token = _dev(inp["cand_token"], dev)
            self.cand_parent = _dev(inp["cand_parent"], dev)
            self.beam_node = None
        self.root_token = _dev(inp["root_token"], dev)
        # tree outputs
        self.n_nodes = torch.zeros(B, **i32)
        self.parent = torch.zeros((B, T_cap), **i32)
        self.token = torch.zeros((B, T_cap), **i32)
        self.depth = torch.zeros((B, T_cap), **i32)
        self.anc = torch.zeros((B, T_cap, self.n_words), dtype=torch.int64, device=dev)
        self.status = torch.zeros(1, **i32)
        # attention
        self.with_kv = with_kv
        if with_kv:
            self.dt = sv.SPEC_F32 if inp["dtype"] == "f32" else sv.SPEC_BF16
            tdt = torch.float32 if self.dt == sv.SPEC_F32 else torch.bfloat16
            self.q = _dev(inp["q"], dev, None if self.dt == sv.SPEC_F32 else torch.bfloat16)
            self.k = _dev(inp["k"], dev, None if self.dt == sv.SPEC_F32 else torch.bfloat16)
            self.v = _dev(inp["v"], dev, None if self.dt == sv.SPEC_F32 else torch.bfloat16)
            # context lengths padded to 16 bytes, so the library's copy kernel
            # can restore them from ctx0 (kernels read the first B entries)
            nb = (B + 3) // 4 * 4
            ctx_pad = np.zeros(nb, np.int32)
            ctx_pad[:B] = inp["ctx_len"]
            self.ctx0 = _dev(ctx_pad, dev)
            self.ctx_len = self.ctx0.clone()
            self.ctx_bytes = nb * 4
            self.H, self.Hkv, self.D = inp["H"], inp["Hkv"], inp["D"]
            self.cap = self.k.shape[2]
            self.max_ctx = int(inp["ctx_len"].max())
            self.out = torch.empty((B, T_cap, self.H, self.D), dtype=tdt, device=dev)
            nb = sv.spec_tree_attention_workspace_size(self.dt, B, T_cap, self.H, self.Hkv,
                                                       self.D, self.max_ctx)
            self.attn_ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
            self.attn_ws_bytes = nb
        # verify
        self.tgt = _dev(inp["tgt"], dev)
        if self.mode not in (sv.SPEC_GREEDY, sv.SPEC_GREEDY_WALK):
            self.dft = _dev(inp["dft"], dev)
            self.dft_row = _dev(inp["dft_row"], dev)
            self.R = int(self.dft.shape[1])
        else:
            self.dft = self.dft_row = None
            self.R = 0
        self.u_node = _dev(inp["u_node"], dev)
        self.u_final = _dev(inp["u_final"], dev)
        self.acc_len = torch.zeros(B, **i32)
        self.acc_path = torch.zeros((B, T_cap), **i32)
        self.next_token = torch.zeros(B, **i32)
        self.p_tok = torch.zeros((B, T_cap), dtype=torch.float32, device=dev)
        self.q_tok = torch.zeros((B, T_cap), dtype=torch.float32, device=dev)
        self.decision = torch.zeros((B, T_cap), dtype=torch.int8, device=dev)
        self.near_tie = torch.zeros(B, **i32)
        nb = sv.spec_verify_workspace_size(self.mode, B, T_cap, V, self.R)
        # no initial contents are needed; zero-filled for reproducible tests
        self.ver_ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
        self.ver_ws_bytes = nb
        # the commit's arrival counters: zero before the first call, and every
        # call leaves them at zero
        nc = sv.spec_kv_compact_workspace_size(B)
        self.cmp_ws = torch.zeros(max(nc, 256), dtype=torch.uint8, device=dev)
        self.cmp_ws_bytes = nc

    # ------------------------------------------------------------------ prepared calls
    def prepare(self, stream=None):
        """Marshal the four calls once (and a reset of ctx_len from its initial
        value through the library's copy kernel), for timing loops."""
        P = sv.prepare
        self.p_build = P("spec_build_tree", self.kind, self.B, self.W, self.L, self.T_cap,
                         self.cand_token, self.cand_parent, self.root_token, self.n_nodes,
                         self.parent, self.token, self.depth, self.anc, self.beam_node,
                         self.status, stream=stream)
        self.p_verify = P("spec_verify", self.mode, self.B, self.T_cap, self.V, self.R, self.tgt,
                          self.dft, self.dft_row, self.n_nodes, self.parent, self.token,
                          self.depth, self.u_node, self.u_final, self.acc_len, self.acc_path,
                          self.next_token, self.p_tok, self.q_tok, self.decision,
                          self.near_tie, self.ver_ws, self.ver_ws_bytes, self.status,
                          stream=stream)
        if self.with_kv:
            self.p_attention = P("spec_tree_attention", self.dt, self.B, self.T_cap, self.H,
                                 self.Hkv, self.D, self.cap, self.max_ctx, self.q, self.k, self.v,
                                 self.ctx_len, self.n_nodes, self.anc, 0.0, self.out,
                                 self.attn_ws, self.attn_ws_bytes, self.status, stream=stream)
            self.p_compact = P("spec_kv_compact", self.dt, self.B, self.Hkv, self.D, self.cap,
                               self.T_cap, self.k, self.v, self.ctx_len, self.acc_len,
                               self.acc_path, self.cmp_ws, self.cmp_ws_bytes, self.status,
                               stream=stream)
            self.p_reset = P("spec_copy_probe", self.ctx0, self.ctx_len, self.ctx_bytes,
                             stream=stream)

    def prepare_verify_mode(self, mode: str, stream=None):
        """spec_verify in another mode on this step's tree and rows, with a
        workspace of its own (outputs shared with the step's own verify call),
        for timing the modes side by side."""
        m = sv.MODES[mode]
        R = self.R if m not in (sv.SPEC_GREEDY, sv.SPEC_GREEDY_WALK) else 0
        nb = sv.spec_verify_workspace_size(m, self.B, self.T_cap, self.V, R)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=self.device)
        call = sv.prepare("spec_verify", m, self.B, self.T_cap, self.V, R, self.tgt,
                          self.dft if R else None, self.dft_row if R else None, self.n_nodes,
                          self.parent, self.token, self.depth, self.u_node, self.u_final,
                          self.acc_len, self.acc_path, self.next_token, self.p_tok, self.q_tok,
                          self.decision, self.near_tie, ws, nb, self.status, stream=stream)
        call.workspace = ws  # keep it alive with the call
        return call

    def prepare_fresh_contexts(self, n, stream=None):
        """n copies of the initial context lengths, each with its own prepared
        attention and commit calls.  A timing loop that uses copy k for the
        k-th step of this input set starts every step from the same context
        without a restore in the timed region (the commit advances the copy
        it was given)."""
        P = sv.prepare
        self.fresh_ctx = [self.ctx0.clone() for _ in range(n)]
        self.p_attention_fresh = [
            P("spec_tree_attention", self.dt, self.B, self.T_cap, self.H, self.Hkv, self.D,
              self.cap, self.max_ctx, self.q, self.k, self.v, c, self.n_nodes, self.anc, 0.0,
              self.out, self.attn_ws, self.attn_ws_bytes, self.status, stream=stream)
            for c in self.fresh_ctx]
        self.p_compact_fresh = [
            P("spec_kv_compact", self.dt, self.B, self.Hkv, self.D, self.cap, self.T_cap, self.k,
              self.v, c, self.acc_len, self.acc_path, self.cmp_ws, self.cmp_ws_bytes,
              self.status, stream=stream)
            for c in self.fresh_ctx]

    # ------------------------------------------------------------------ calls
    def build_tree(self, stream=None):
        sv.spec_build_tree(self.kind, self.B, self.W, self.L, self.T_cap, self.cand_token,
                           self.cand_parent, self.root_token, self.n_nodes, self.parent,
                           self.token, self.depth, self.anc, self.beam_node, self.status, stream)

    def attention(self, stream=None):
        sv.spec_tree_attention(self.dt, self.B, self.T_cap, self.H, self.Hkv, self.D, self.cap,
                               self.max_ctx, self.q, self.k, self.v, self.ctx_len, self.n_nodes,
                               self.anc, 0.0, self.out, self.attn_ws, self.attn_ws_bytes,
                               self.status, stream)

    def verify(self, stream=None):
        sv.spec_verify(self.mode, self.B, self.T_cap, self.V, self.R, self.tgt, self.dft,
                       self.dft_row, self.n_nodes, self.parent, self.token, self.depth,
                       self.u_node, self.u_final, self.acc_len, self.acc_path, self.next_token,
                       self.p_tok, self.q_tok, self.decision, self.near_tie, self.ver_ws,
                       self.ver_ws_bytes, self.status, stream)

    def compact(self, stream=None):
        sv.spec_kv_compact(self.dt, self.B, self.Hkv, self.D, self.cap, self.T_cap, self.k, self.v,
                           self.ctx_len, self.acc_len, self.acc_path, self.cmp_ws,
                           self.cmp_ws_bytes, self.status, stream)

    def launch(self, compact: bool = True, stream=None):
        """Enqueue one whole step (no host synchronisation)."""
        self.build_tree(stream)
        if self.with_kv:
            self.attention(stream)
        self.verify(stream)
        if compact and self.with_kv:
            self.compact(stream)

    def run(self, compact: bool = False) -> dict:
        """One step, then copy every output back to host numpy arrays."""
        self.launch(compact=compact)
        torch.cuda.synchronize(self.device)
        out = dict(
            n_nodes=self.n_nodes.cpu().numpy(), parent=self.parent.cpu().numpy(),
            token=self.token.cpu().numpy(), depth=self.depth.cpu().numpy(),
            anc=self.anc.cpu().numpy().view(np.uint64),
            acc_len=self.acc_len.cpu().numpy(), acc_path=self.acc_path.cpu().numpy(),
            next_token=self.next_token.cpu().numpy(), p_tok=self.p_tok.cpu().numpy(),
            q_tok=self.q_tok.cpu().numpy(), decision=self.decision.cpu().numpy(),
            near_tie=self.near_tie.cpu().numpy(), status=int(self.status.item()),
        )
        if self.beam_node is not None:
            out["beam_node"] = self.beam_node.cpu().numpy()
        if self.with_kv:
            out["attn"] = self.out.float().cpu().numpy()
            out["ctx_len"] = self.ctx_len[:self.B].cpu().numpy()
        return out
