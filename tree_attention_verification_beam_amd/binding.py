"""ctypes binding of libspecverify.so: the C-ABI entry points under the same names.

Argument marshalling only.  Buffers are torch tensors on the GPU (or raw device
addresses as ints); the stream defaults to torch's current stream.  A non-zero
return code raises SpecError.  The library must have been built in-tree
(``build.py``); load() fails loudly otherwise, and there is no fallback.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libspecverify.so"

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_TREE_BEAMS, SPEC_TREE_EXPLICIT = 0, 1
SPEC_GREEDY, SPEC_REJECT_PATH, SPEC_REJECT_RECURSIVE, SPEC_GREEDY_WALK = 0, 1, 2, 3
SPEC_REJECT_PATH_WALK, SPEC_REJECT_RECURSIVE_WALK = 4, 5
MODES = {"greedy": SPEC_GREEDY, "reject_path": SPEC_REJECT_PATH,
         "reject_recursive": SPEC_REJECT_RECURSIVE, "greedy_walk": SPEC_GREEDY_WALK,
         "reject_path_walk": SPEC_REJECT_PATH_WALK,
         "reject_recursive_walk": SPEC_REJECT_RECURSIVE_WALK}

DEV_BITS = {
    0x1: "BAD_PARENT", 0x2: "BAD_TOKEN", 0x4: "BAD_ROW", 0x8: "CTX_RANGE",
    0x10: "RESIDUAL_ZERO", 0x20: "SYNC_TIMEOUT", 0x40: "BAD_TREE",
}

_c_int, _c_size, _vp, _c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

# name -> (restype, argtypes), in the order of include/specverify.h
SIGNATURES = {
    "spec_version": (_c_int, []),
    "spec_status_string": (ctypes.c_char_p, [_c_int]),
    "spec_build_tree": (_c_int, [_c_int] * 5 + [_vp] * 10 + [_vp]),
    "spec_tree_attention_workspace_size": (_c_size, [_c_int] * 7),
    "spec_tree_attention": (_c_int, [_c_int] * 8 + [_vp] * 6 + [_c_float, _vp, _vp, _c_size, _vp,
                                                                 _vp]),
    "spec_verify_workspace_size": (_c_size, [_c_int] * 5),
    "spec_verify": (_c_int, [_c_int] * 5 + [_vp] * 17 + [_c_size, _vp, _vp]),
    "spec_verify_noalloc": (_c_int, [_c_int] * 5 + [_vp] * 16 + [_vp, _vp]),
    "spec_kv_compact_workspace_size": (_c_size, [_c_int]),
    "spec_kv_compact": (_c_int, [_c_int] * 6 + [_vp] * 6 + [_c_size, _vp, _vp]),
    "spec_beam_topk_workspace_size": (_c_size, [_c_int] * 4),
    "spec_beam_topk": (_c_int, [_c_int] * 4 + [_vp] * 6 + [_c_int, _vp, _vp, _c_size, _vp]),
    "spec_select_tree": (_c_int, [_c_int] * 3 + [_vp] * 9),
    "spec_last_device_status": (_c_int, [_vp, _vp]),
    "spec_copy_probe": (_c_int, [_vp, _vp, _c_size, _vp]),
    "spec_read_probe": (_c_int, [_vp, _c_size, _vp, _c_int, _vp]),
}

_lib = None


class SpecError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        name = _lib.spec_status_string(code).decode() if _lib is not None else str(code)
        super().__init__(f"{fn} returned {code} ({name})")


def load() -> ctypes.CDLL:
    """Load the in-tree library (no fallback of any kind)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int):
    if rc != 0:
        raise SpecError(fn, rc)


def spec_version() -> int:
    return load().spec_version()


def spec_build_tree(kind, B, W, L, T_cap, cand_token, cand_parent, root_token, n_nodes, parent,
                    token, depth, anc, beam_node=None, status=None, stream=None):
    rc = load().spec_build_tree(kind, B, W, L, T_cap, _ptr(cand_token), _ptr(cand_parent),
                                _ptr(root_token), _ptr(n_nodes), _ptr(parent), _ptr(token),
                                _ptr(depth), _ptr(anc), _ptr(beam_node), _ptr(status),
                                _stream(stream))
    _check("spec_build_tree", rc)


def spec_tree_attention_workspace_size(dt, B, T_cap, H, Hkv, D, max_ctx) -> int:
    return load().spec_tree_attention_workspace_size(dt, B, T_cap, H, Hkv, D, max_ctx)


def spec_tree_attention(dt, B, T_cap, H, Hkv, D, cache_cap, max_ctx, q, k_cache, v_cache,
                        ctx_len, n_nodes, anc, scale, out, ws=None, ws_bytes=0, status=None,
                        stream=None):
    rc = load().spec_tree_attention(dt, B, T_cap, H, Hkv, D, cache_cap, max_ctx, _ptr(q),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), _ptr(n_nodes),
                                    _ptr(anc), float(scale), _ptr(out), _ptr(ws), ws_bytes,
                                    _ptr(status), _stream(stream))
    _check("spec_tree_attention", rc)


def spec_verify_workspace_size(mode, B, T_cap, V, R) -> int:
    return load().spec_verify_workspace_size(mode, B, T_cap, V, R)


def spec_verify(mode, B, T_cap, V, R, tgt, dft, dft_row, n_nodes, parent, token, depth, u_node,
                u_final, acc_len, acc_path, next_token, p_tok, q_tok, decision, near_tie, ws,
                ws_bytes, status=None, stream=None):
    rc = load().spec_verify(mode, B, T_cap, V, R, _ptr(tgt), _ptr(dft), _ptr(dft_row),
                            _ptr(n_nodes), _ptr(parent), _ptr(token), _ptr(depth), _ptr(u_node),
                            _ptr(u_final), _ptr(acc_len), _ptr(acc_path), _ptr(next_token),
                            _ptr(p_tok), _ptr(q_tok), _ptr(decision), _ptr(near_tie), _ptr(ws),
                            ws_bytes, _ptr(status), _stream(stream))
    _check("spec_verify", rc)


def spec_verify_noalloc(mode, B, T_cap, V, R, tgt, dft, dft_row, n_nodes, parent, token, depth,
                        u_node, u_final, acc_len, acc_path, next_token, p_tok, q_tok, decision,
                        near_tie, status=None, stream=None):
    rc = load().spec_verify_noalloc(mode, B, T_cap, V, R, _ptr(tgt), _ptr(dft), _ptr(dft_row),
                                    _ptr(n_nodes), _ptr(parent), _ptr(token), _ptr(depth),
                                    _ptr(u_node), _ptr(u_final), _ptr(acc_len), _ptr(acc_path),
                                    _ptr(next_token), _ptr(p_tok), _ptr(q_tok), _ptr(decision),
                                    _ptr(near_tie), _ptr(status), _stream(stream))
    _check("spec_verify_noalloc", rc)


def spec_kv_compact_workspace_size(B) -> int:
    return load().spec_kv_compact_workspace_size(B)


def spec_kv_compact(dt, B, Hkv, D, cache_cap, T_cap, k_cache, v_cache, ctx_len, acc_len,
                    acc_path, ws, ws_bytes, status=None, stream=None):
    rc = load().spec_kv_compact(dt, B, Hkv, D, cache_cap, T_cap, _ptr(k_cache), _ptr(v_cache),
                                _ptr(ctx_len), _ptr(acc_len), _ptr(acc_path), _ptr(ws),
                                ws_bytes, _ptr(status), _stream(stream))
    _check("spec_kv_compact", rc)


def spec_beam_topk_workspace_size(B, K_in, K_out, V) -> int:
    return load().spec_beam_topk_workspace_size(B, K_in, K_out, V)


def spec_beam_topk(B, K_in, K_out, V, logp, beam_score, out_parent, out_token, out_score,
                   hist_in=None, hist_len=0, hist_out=None, ws=None, ws_bytes=0, stream=None):
    rc = load().spec_beam_topk(B, K_in, K_out, V, _ptr(logp), _ptr(beam_score), _ptr(out_parent),
                               _ptr(out_token), _ptr(out_score), _ptr(hist_in), hist_len,
                               _ptr(hist_out), _ptr(ws), ws_bytes, _stream(stream))
    _check("spec_beam_topk", rc)


def spec_select_tree(B, N, N_keep, cand_parent, cand_token, cand_logp, keep_parent, keep_token,
                     keep_src=None, keep_score=None, status=None, stream=None):
    rc = load().spec_select_tree(B, N, N_keep, _ptr(cand_parent), _ptr(cand_token),
                                 _ptr(cand_logp), _ptr(keep_parent), _ptr(keep_token),
                                 _ptr(keep_src), _ptr(keep_score), _ptr(status), _stream(stream))
    _check("spec_select_tree", rc)


def spec_copy_probe(src, dst, n_bytes, stream=None):
    rc = load().spec_copy_probe(_ptr(src), _ptr(dst), n_bytes, _stream(stream))
    _check("spec_copy_probe", rc)


def spec_read_probe(src, n_bytes, out, n_blocks, stream=None):
    rc = load().spec_read_probe(_ptr(src), n_bytes, _ptr(out), n_blocks, _stream(stream))
    _check("spec_read_probe", rc)


def spec_last_device_status(status=None, stream=None) -> int:
    """SPEC_DEV_* bits of a device status word (the library's own word when
    status is None) once the stream has finished; the library's word is
    cleared after it is read."""
    rc = load().spec_last_device_status(_ptr(status), _stream(stream))
    if rc < 0:
        raise SpecError("spec_last_device_status", rc)
    return rc


def decode_status(word: int) -> list[str]:
    return [name for bit, name in DEV_BITS.items() if word & bit]


class Prepared:
    """A C-ABI call with its arguments marshalled once (device addresses, sizes
    and the stream fixed at preparation time), for loops that issue the same
    call many times: calling it costs one ctypes call and a status check."""

    def __init__(self, name: str, *args):
        lib = load()
        fn = getattr(lib, name)
        self.name = name
        self.fn = fn
        conv = []
        for a, t in zip(args, SIGNATURES[name][1]):
            if t is _vp:
                conv.append(_vp(_ptr(a)))
            elif t is _c_float:
                conv.append(_c_float(a))
            elif t is _c_size:
                conv.append(_c_size(a))
            else:
                conv.append(_c_int(a))
        assert len(conv) == len(SIGNATURES[name][1]), name
        self.args = tuple(conv)

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            raise SpecError(self.name, rc)


def prepare(name: str, *args, stream=None) -> Prepared:
    """Prepared(name, *args) with the stream (torch's current one by default)
    appended as the last argument, as every launching entry point takes it."""
    return Prepared(name, *args, _stream(stream))
