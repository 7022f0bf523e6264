"""CPU oracle of the speculative verification step (test infrastructure).

Plain, slow, single-threaded fp64 C (``oracle.c``) behind a numpy-facing ctypes
wrapper.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and imports nothing from it.

The functions follow the pages' statement of the problem; the citations sit
beside each C function in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"

GREEDY, REJECT_PATH, REJECT_RECURSIVE = 0, 1, 2
MODES = {"greedy": GREEDY, "reject_path": REJECT_PATH, "reject_recursive": REJECT_RECURSIVE}


def build(force: bool = False) -> Path:
    """Compile oracle.c with gcc (IEEE fp64, no contraction, no fast-math)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-shared",
             "-fPIC", "-o", str(tmp), str(_SRC), "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(str(build()))
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"oracle {what} failed (rc={rc})")


def n_words(T_cap: int) -> int:
    return (T_cap + 63) // 64


def build_tree_beams(beams: np.ndarray, root_token: np.ndarray, T_cap: int):
    """beams [B][W][L] int -> dict(n_nodes, parent, token, depth, anc, beam_node)."""
    beams = _i32(beams)
    B, W, L = beams.shape
    out = dict(
        n_nodes=np.zeros(B, np.int32),
        parent=np.zeros((B, T_cap), np.int32),
        token=np.zeros((B, T_cap), np.int32),
        depth=np.zeros((B, T_cap), np.int32),
        anc=np.zeros((B, T_cap, n_words(T_cap)), np.uint64),
        beam_node=np.zeros((B, W, L), np.int32),
    )
    root = _i32(root_token)
    f = lib().orc_build_tree_beams
    f.restype = ctypes.c_int
    rc = f(B, W, L, T_cap, _p(beams), _p(root), _p(out["n_nodes"]), _p(out["parent"]),
           _p(out["token"]), _p(out["depth"]), _p(out["anc"]), _p(out["beam_node"]))
    _check(rc, "build_tree_beams")
    return out


def build_tree_explicit(cand_parent: np.ndarray, cand_token: np.ndarray, root_token: np.ndarray,
                        T_cap: int):
    """cand_parent/cand_token [B][N] -> dict(n_nodes, parent, token, depth, anc, bad)."""
    cand_parent = _i32(cand_parent)
    cand_token = _i32(cand_token)
    B, N = cand_parent.shape
    out = dict(
        n_nodes=np.zeros(B, np.int32),
        parent=np.zeros((B, T_cap), np.int32),
        token=np.zeros((B, T_cap), np.int32),
        depth=np.zeros((B, T_cap), np.int32),
        anc=np.zeros((B, T_cap, n_words(T_cap)), np.uint64),
        bad=np.zeros(B, np.int32),
    )
    root = _i32(root_token)
    f = lib().orc_build_tree_explicit
    f.restype = ctypes.c_int
    rc = f(B, N, T_cap, _p(cand_parent), _p(cand_token), _p(root), _p(out["n_nodes"]),
           _p(out["parent"]), _p(out["token"]), _p(out["depth"]), _p(out["anc"]), _p(out["bad"]))
    _check(rc, "build_tree_explicit")
    return out


def tree_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, ctx_len, n_nodes, anc,
                   scale: float = 0.0, rows: np.ndarray | None = None) -> np.ndarray:
    """q [B][T_cap][H][D], k/v [B][Hkv][cap][D] as float32 or bf16 bits (uint16).

    Returns fp64 [B][T_cap][H][D], or [n][D] for rows = int array [n][3] of (b,t,h).
    """
    if q.dtype == np.float32:
        dtype = 0
    elif q.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("q must be float32 or uint16 (bf16 bits)")
    assert k.dtype == q.dtype and v.dtype == q.dtype
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, T_cap, H, D = q.shape
    _, Hkv, cap, _ = k.shape
    ctx_len = _i32(ctx_len)
    n_nodes = _i32(n_nodes)
    anc = np.ascontiguousarray(anc, dtype=np.uint64)
    if rows is None:
        out = np.zeros((B, T_cap, H, D), np.float64)
        n_sel, sel = 0, None
    else:
        sel = _i32(rows).reshape(-1, 3)
        n_sel = sel.shape[0]
        out = np.zeros((n_sel, D), np.float64)
    f = lib().orc_tree_attention
    f.restype = ctypes.c_int
    rc = f(dtype, B, T_cap, H, Hkv, D, cap, _p(q), _p(k), _p(v), _p(ctx_len), _p(n_nodes),
           _p(anc), ctypes.c_double(scale), n_sel, _p(sel), _p(out))
    _check(rc, "tree_attention")
    return out


def verify(mode, tgt: np.ndarray, dft, dft_row, n_nodes, parent, token, depth, u_node, u_final):
    """Verification of packed trees; see orc_verify in oracle.c for the semantics."""
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    tgt = np.ascontiguousarray(tgt, dtype=np.float32)
    B, T_cap, V = tgt.shape
    if dft is not None:
        dft = np.ascontiguousarray(dft, dtype=np.float32)
        R = dft.shape[1]
        dft_row = _i32(dft_row)
    else:
        R = 0
    out = dict(
        acc_len=np.zeros(B, np.int32),
        acc_path=np.zeros((B, T_cap), np.int32),
        next_token=np.zeros(B, np.int32),
        p_tok=np.zeros((B, T_cap), np.float64),
        q_tok=np.zeros((B, T_cap), np.float64),
        decision=np.zeros((B, T_cap), np.int8),
        near_tie=np.zeros(B, np.int32),
        fallback=np.zeros(B, np.int32),
    )
    f = lib().orc_verify
    f.restype = ctypes.c_int
    rc = f(mode, B, T_cap, V, R, _p(tgt), _p(dft), _p(dft_row if dft is not None else None),
           _p(_i32(n_nodes)), _p(_i32(parent)), _p(_i32(token)), _p(_i32(depth)),
           _p(np.ascontiguousarray(u_node, dtype=np.float32)),
           _p(np.ascontiguousarray(u_final, dtype=np.float32)),
           _p(out["acc_len"]), _p(out["acc_path"]), _p(out["next_token"]), _p(out["p_tok"]),
           _p(out["q_tok"]), _p(out["decision"]), _p(out["near_tie"]), _p(out["fallback"]))
    _check(rc, "verify")
    return out


def verify_greedy_walk(tgt: np.ndarray, n_nodes, parent, token, depth):
    """Greedy verification by a depth-by-depth walk over the surviving nodes; see
    orc_verify_greedy_walk in oracle.c.  Only tested nodes carry decision/p_tok."""
    tgt = np.ascontiguousarray(tgt, dtype=np.float32)
    B, T_cap, V = tgt.shape
    out = dict(
        acc_len=np.zeros(B, np.int32),
        acc_path=np.zeros((B, T_cap), np.int32),
        next_token=np.zeros(B, np.int32),
        p_tok=np.zeros((B, T_cap), np.float64),
        q_tok=np.zeros((B, T_cap), np.float64),
        decision=np.zeros((B, T_cap), np.int8),
        near_tie=np.zeros(B, np.int32),
        rows_read=np.zeros(B, np.int32),
    )
    f = lib().orc_verify_greedy_walk
    f.restype = ctypes.c_int
    rc = f(B, T_cap, V, _p(tgt), _p(_i32(n_nodes)), _p(_i32(parent)), _p(_i32(token)),
           _p(_i32(depth)), _p(out["acc_len"]), _p(out["acc_path"]), _p(out["next_token"]),
           _p(out["p_tok"]), _p(out["decision"]), _p(out["rows_read"]))
    _check(rc, "verify_greedy_walk")
    return out


def verify_reject_walk(mode, tgt: np.ndarray, dft, dft_row, n_nodes, parent, token, depth, u_node,
                       u_final):
    """Rejection-mode verification walking the surviving nodes and reading only
    their rows; see orc_verify_reject_walk in oracle.c.  Only tested nodes carry
    decision / p_tok / q_tok; rows_tgt / rows_dft count the rows read."""
    mode = MODES[mode] if isinstance(mode, str) else int(mode)
    tgt = np.ascontiguousarray(tgt, dtype=np.float32)
    dft = np.ascontiguousarray(dft, dtype=np.float32)
    B, T_cap, V = tgt.shape
    out = dict(
        acc_len=np.zeros(B, np.int32),
        acc_path=np.zeros((B, T_cap), np.int32),
        next_token=np.zeros(B, np.int32),
        p_tok=np.zeros((B, T_cap), np.float64),
        q_tok=np.zeros((B, T_cap), np.float64),
        decision=np.zeros((B, T_cap), np.int8),
        near_tie=np.zeros(B, np.int32),
        fallback=np.zeros(B, np.int32),
        rows_tgt=np.zeros(B, np.int32),
        rows_dft=np.zeros(B, np.int32),
    )
    f = lib().orc_verify_reject_walk
    f.restype = ctypes.c_int
    rc = f(mode, B, T_cap, V, dft.shape[1], _p(tgt), _p(dft), _p(_i32(dft_row)),
           _p(_i32(n_nodes)), _p(_i32(parent)), _p(_i32(token)), _p(_i32(depth)),
           _p(np.ascontiguousarray(u_node, dtype=np.float32)),
           _p(np.ascontiguousarray(u_final, dtype=np.float32)),
           _p(out["acc_len"]), _p(out["acc_path"]), _p(out["next_token"]), _p(out["p_tok"]),
           _p(out["q_tok"]), _p(out["decision"]), _p(out["near_tie"]), _p(out["fallback"]),
           _p(out["rows_tgt"]), _p(out["rows_dft"]))
    _check(rc, "verify_reject_walk")
    return out


def beam_topk(logp: np.ndarray, beam_score, K_out: int, hist=None):
    """One beam-search pruning step; see orc_beam_topk in oracle.c.
    logp [B][K_in][V] fp32, beam_score [B][K_in] or None, hist [B][K_in][len] or None."""
    logp = np.ascontiguousarray(logp, dtype=np.float32)
    B, K_in, V = logp.shape
    out = dict(parent=np.zeros((B, K_out), np.int32), token=np.zeros((B, K_out), np.int32),
               score=np.zeros((B, K_out), np.float32))
    length = 0
    if hist is not None:
        hist = _i32(hist)
        length = hist.shape[2]
        out["hist"] = np.zeros((B, K_out, length + 1), np.int32)
    bs = None if beam_score is None else np.ascontiguousarray(beam_score, dtype=np.float32)
    f = lib().orc_beam_topk
    f.restype = ctypes.c_int
    rc = f(B, K_in, K_out, V, _p(logp), _p(bs), _p(out["parent"]), _p(out["token"]),
           _p(out["score"]), _p(hist), length, _p(out.get("hist")))
    _check(rc, "beam_topk")
    return out


def select_tree(cand_parent, cand_token, cand_logp, N_keep: int):
    """Dynamic tree selection under a node budget; see orc_select_tree in oracle.c."""
    cand_parent, cand_token = _i32(cand_parent), _i32(cand_token)
    cand_logp = np.ascontiguousarray(cand_logp, dtype=np.float32)
    B, N = cand_parent.shape
    out = dict(parent=np.zeros((B, N_keep), np.int32), token=np.zeros((B, N_keep), np.int32),
               src=np.zeros((B, N_keep), np.int32), score=np.zeros((B, N_keep), np.float32))
    f = lib().orc_select_tree
    f.restype = ctypes.c_int
    rc = f(B, N, N_keep, _p(cand_parent), _p(cand_token), _p(cand_logp), _p(out["parent"]),
           _p(out["token"]), _p(out["src"]), _p(out["score"]))
    _check(rc, "select_tree")
    return out


def residual_chain(p: np.ndarray, q: np.ndarray, K: int, literal: bool = False):
    """Residual distributions after 0..K rejections: (dist [K+1][V], mass [K+1], filled)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    V = p.shape[0]
    dist = np.zeros((K + 1, V), np.float64)
    mass = np.zeros(K + 1, np.float64)
    f = lib().orc_residual_chain
    f.restype = ctypes.c_int
    filled = f(V, _p(p), _p(q), K, int(bool(literal)), _p(dist), _p(mass))
    return dist, mass, filled


def kv_compact(k: np.ndarray, v: np.ndarray, ctx_len, acc_len, acc_path):
    """In-place commit of the accepted path on numpy caches [B][Hkv][cap][D]."""
    assert k.flags["C_CONTIGUOUS"] and v.flags["C_CONTIGUOUS"]
    B, Hkv, cap, D = k.shape
    acc_path = _i32(acc_path)
    T_cap = acc_path.shape[1]
    ctx_len_io = _i32(ctx_len).copy()
    f = lib().orc_kv_compact
    f.restype = ctypes.c_int
    rc = f(k.itemsize, B, Hkv, D, cap, T_cap, _p(k), _p(v), _p(ctx_len_io), _p(_i32(acc_len)),
           _p(acc_path))
    _check(rc, "kv_compact")
    return ctx_len_io


def resispec_proxy(p, q, x0: int, fill: int = 0, x0_mode: int = 0):
    """The literal GetProxy steps for a rejected candidate x0: (r, k, Z)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    V = p.shape[0]
    r = np.zeros(V, np.float64)
    k = np.zeros(V, np.float64)
    z = ctypes.c_double(0.0)
    f = lib().orc_resispec_proxy
    f.restype = ctypes.c_int
    rc = f(V, _p(p), _p(q), int(x0), int(fill), int(x0_mode), _p(r), _p(k), ctypes.byref(z))
    _check(rc, "resispec_proxy")
    return r, k, z.value


def multicand_marginal(p, q, n: int, shape: int = 0, fill: int = 0, x0_mode: int = 0):
    """Output distribution of n i.i.d. candidates from q verified sequentially
    (every path summed): shape 0 standard residuals, 1 the literal ResiSpec ones."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    out = np.zeros(p.shape[0], np.float64)
    f = lib().orc_multicand_marginal
    f.restype = ctypes.c_int
    rc = f(p.shape[0], int(n), _p(p), _p(q), int(shape), int(fill), int(x0_mode), _p(out))
    _check(rc, "multicand_marginal")
    return out
