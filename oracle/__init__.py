"""Python access to the CPU oracle (oracle.c).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this package. The GPU library's Python binding never
imports it, and the product path never falls back to it.

`build()` compiles oracle.c with gcc into liboracle.so next to this file; the
functions below marshal numpy arrays (float32 logits, int32 ids) into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

BAD_TOKEN = 1
NONFINITE = 2
MARGIN_ACCEPT = 1
MARGIN_SAMPLE = 2
MARGIN_REL = 1e-6


def build(verbose: bool = False) -> str:
    """Compile the oracle (plain C, fp64, OpenMP across sequences)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.orc_transform_row.argtypes = [P, I, D, I, P]
    lib.orc_transform_row.restype = I
    lib.orc_argmax_row.argtypes = [P, I]
    lib.orc_argmax_row.restype = I
    lib.orc_verify_chain.argtypes = [P, P, P, P, P, I, I, I, D, I, D, P, P, P, P, P, P, I]
    lib.orc_verify_chain.restype = None
    lib.orc_verify_greedy.argtypes = [P, P, P, I, I, I, P, P, P, P, I]
    lib.orc_verify_greedy.restype = None
    lib.orc_build_tree.argtypes = [P, I, I, I, I, P, P, P, P, P, P, I]
    lib.orc_build_tree.restype = None
    lib.orc_verify_tree.argtypes = [P, P, P, P, I, I, I, P, P, P, I]
    lib.orc_verify_tree.restype = None
    lib.orc_verify_tree_sampled.argtypes = [P, P, P, P, P, I, I, I, D, I, D, P, P, P, P, P, I]
    lib.orc_verify_tree_sampled.restype = None
    lib.orc_select_len.argtypes = [P, I, I, ctypes.c_float, P, P, P, P]
    lib.orc_select_len.restype = None
    lib.orc_verify_chain_capped.argtypes = [P, P, P, P, P, I, I, I, D, I, D, P, P, P, P, P, P, P, I]
    lib.orc_verify_chain_capped.restype = None
    lib.orc_select_len_table.argtypes = [P, I, I, P, P, P, P, P]
    lib.orc_select_len_table.restype = None
    lib.orc_compact_kv.argtypes = [P, ctypes.c_longlong, ctypes.c_longlong, P, P, P, I, I]
    lib.orc_compact_kv.restype = None
    lib.orc_rerank_tree.argtypes = [P, P, P, P, I, I, I, P, P, P, P, P, P, P]
    lib.orc_rerank_tree.restype = None
    lib.orc_expand_tree.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I]
    lib.orc_expand_tree.restype = None
    lib.orc_check_chain.argtypes = [P, P, P, P, P, I, I, I, D, I, D, P, P, P, P, I]
    lib.orc_check_chain.restype = None
    lib.orc_check_tree_sampled.argtypes = [P, P, P, P, P, I, I, I, D, I, D, P, P, P, P, I]
    lib.orc_check_tree_sampled.restype = None
    lib.orc_check_select_len.argtypes = [P, I, I, ctypes.c_float, D, P, P]
    lib.orc_check_select_len.restype = None
    _lib = lib
    return lib


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _t32(temperature) -> float:
    """The temperature crosses the GPU boundary as an fp32 value; use that value."""
    return float(np.float32(temperature))


def transform_row(logits, temperature: float, top_k: int = 0):
    """(valid, p[V]) for one row of logits."""
    x = _f32(logits)
    p = np.zeros(x.shape[0], dtype=np.float64)
    ok = _load().orc_transform_row(_ptr(x), x.shape[0], _t32(temperature), int(top_k), _ptr(p))
    return bool(ok), p


def argmax_row(logits) -> int:
    x = _f32(logits)
    return int(_load().orc_argmax_row(_ptr(x), x.shape[0]))


def verify_chain(target, draft, tokens, uniforms, cu, B, K_max, V, temperature, top_k=0,
                 margin_rel=MARGIN_REL, threads=None, want_probs=True):
    """Stochastic (T > 0) or greedy (T == 0) chain verification.

    Returns a dict of numpy arrays: A, next, probs ([R_d, 2] fp64), R, status, margin.
    """
    t = _f32(target).reshape(-1)
    d = _f32(draft).reshape(-1) if draft is not None else np.zeros(1, np.float32)
    y = _i32(tokens).reshape(-1)
    u = _f32(uniforms).reshape(-1)
    c = None if cu is None else _i32(cu)
    R_d = y.shape[0]
    A = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    probs = np.zeros((max(R_d, 1), 2), np.float64) if want_probs else None
    R = np.zeros(B, np.float64)
    st = np.zeros(B, np.int32)
    mg = np.zeros(B, np.int32)
    _load().orc_verify_chain(_ptr(t), _ptr(d), _ptr(y), _ptr(u), _ptr(c), int(B), int(K_max), int(V),
                             _t32(temperature), int(top_k), float(margin_rel),
                             _ptr(A), _ptr(nxt), _ptr(probs), _ptr(R), _ptr(st), _ptr(mg),
                             int(threads or default_threads()))
    return {"A": A, "next": nxt, "probs": None if probs is None else probs[:R_d], "R": R,
            "status": st, "margin": mg}


def verify_greedy(target, tokens, cu, B, K_max, V, threads=None):
    t = _f32(target).reshape(-1)
    y = _i32(tokens).reshape(-1)
    c = None if cu is None else _i32(cu)
    R_t = t.shape[0] // V
    A = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    g = np.zeros(R_t, np.int32)
    _load().orc_verify_greedy(_ptr(t), _ptr(y), _ptr(c), int(B), int(K_max), int(V),
                              _ptr(A), _ptr(nxt), _ptr(st), _ptr(g),
                              int(threads or default_threads()))
    return {"A": A, "next": nxt, "status": st, "argmax": g}


def build_tree(marginals, B, K, V, N, threads=None):
    m = _f32(marginals).reshape(-1)
    tok = np.zeros((B, N), np.int32)
    par = np.zeros((B, N), np.int32)
    dep = np.zeros((B, N), np.int32)
    sc = np.zeros((B, N), np.float32)
    anc = np.zeros((B, N), np.uint64)
    nn = np.zeros(B, np.int32)
    _load().orc_build_tree(_ptr(m), int(B), int(K), int(V), int(N), _ptr(tok), _ptr(par), _ptr(dep),
                           _ptr(sc), _ptr(anc), _ptr(nn), int(threads or default_threads()))
    return {"token": tok, "parent": par, "depth": dep, "score": sc, "anc_mask": anc, "n_nodes": nn}


def verify_tree(target, token, parent, n_nodes, B, N, V, threads=None):
    t = _f32(target).reshape(-1)
    tok = _i32(token).reshape(-1)
    par = _i32(parent).reshape(-1)
    nn = _i32(n_nodes)
    path = np.zeros((B, N), np.int32)
    A = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    _load().orc_verify_tree(_ptr(t), _ptr(tok), _ptr(par), _ptr(nn), int(B), int(N), int(V),
                            _ptr(path), _ptr(A), _ptr(nxt), int(threads or default_threads()))
    return {"path": path, "A": A, "next": nxt}


def verify_tree_sampled(target, token, parent, n_nodes, uniforms, B, N, V, temperature, top_k=0,
                        margin_rel=MARGIN_REL, threads=None):
    """Sampled tree walk: at each node the target's token is drawn from its own
    transformed row with that node's uniform (uniforms [B, N]).

    Returns path, A, next, status, margin.
    """
    t = _f32(target).reshape(-1)
    tok = _i32(token).reshape(-1)
    par = _i32(parent).reshape(-1)
    nn = _i32(n_nodes)
    u = _f32(uniforms).reshape(-1)
    path = np.zeros((B, N), np.int32)
    A = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    mg = np.zeros(B, np.int32)
    _load().orc_verify_tree_sampled(_ptr(t), _ptr(tok), _ptr(par), _ptr(nn), _ptr(u), int(B), int(N),
                                    int(V), ctypes.c_double(temperature), int(top_k),
                                    ctypes.c_double(margin_rel), _ptr(path), _ptr(A), _ptr(nxt),
                                    _ptr(st), _ptr(mg), int(threads or default_threads()))
    return {"path": path, "A": A, "next": nxt, "status": st, "margin": mg}


def select_len(conf, B, K, cost):
    c = _f32(conf).reshape(-1)
    k = np.zeros(B, np.int32)
    adv = np.zeros(B, np.float64)
    cu = np.zeros(B + 1, np.int32)
    mg = np.zeros(B, np.int32)
    _load().orc_select_len(_ptr(c), int(B), int(K), ctypes.c_float(cost), _ptr(k), _ptr(adv),
                           _ptr(cu), _ptr(mg))
    return {"k": k, "adv": adv, "cu": cu, "margin": mg}


def verify_chain_capped(target, draft, tokens, uniforms, cap, B, K, V, temperature, top_k=0,
                        margin_rel=MARGIN_REL, threads=None):
    """Cap-accept verification over a padded window (B sequences x K positions).

    Returns A (committed, <= cap), next, A_full (first rejection over the whole
    window), probs ([B*K, 2]), R, status, margin.
    """
    t = _f32(target).reshape(-1)
    d = _f32(draft).reshape(-1)
    y = _i32(tokens).reshape(-1)
    u = _f32(uniforms).reshape(-1)
    c = _i32(cap)
    A = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    Af = np.zeros(B, np.int32)
    probs = np.zeros((max(B * K, 1), 2), np.float64)
    R = np.zeros(B, np.float64)
    st = np.zeros(B, np.int32)
    mg = np.zeros(B, np.int32)
    _load().orc_verify_chain_capped(_ptr(t), _ptr(d), _ptr(y), _ptr(u), _ptr(c), int(B), int(K),
                                    int(V), _t32(temperature), int(top_k), float(margin_rel),
                                    _ptr(A), _ptr(nxt), _ptr(Af), _ptr(probs), _ptr(R), _ptr(st),
                                    _ptr(mg), int(threads or default_threads()))
    return {"A": A, "next": nxt, "A_full": Af, "probs": probs[:B * K], "R": R, "status": st,
            "margin": mg}


def select_len_table(conf, B, K, cost_table):
    """Verify length with a per-position cost table (cost_table[j-1] for position j)."""
    assert K <= 64
    c = _f32(conf).reshape(-1)
    tab = _f32(cost_table).reshape(-1)
    assert tab.shape[0] >= K
    k = np.zeros(B, np.int32)
    adv = np.zeros(B, np.float64)
    cu = np.zeros(B + 1, np.int32)
    mg = np.zeros(B, np.int32)
    _load().orc_select_len_table(_ptr(c), int(B), int(K), _ptr(tab), _ptr(k), _ptr(adv), _ptr(cu),
                                 _ptr(mg))
    return {"k": k, "adv": adv, "cu": cu, "margin": mg}


def compact_kv(kv, row_base, path, accepted_len, B, N):
    """Accepted-path KV compaction on a host copy; kv is a 2-D uint8 array
    [n_rows, row_bytes]. Returns the compacted copy."""
    out = np.ascontiguousarray(np.array(kv, dtype=np.uint8, copy=True))
    n_rows, row_bytes = out.shape
    rb = np.ascontiguousarray(np.asarray(row_base, dtype=np.int64))
    p = _i32(path).reshape(-1)
    a = _i32(accepted_len)
    _load().orc_compact_kv(_ptr(out), int(row_bytes), int(n_rows), _ptr(rb), _ptr(p), _ptr(a),
                           int(B), int(N))
    return out


def rerank_tree(cand_parent, cand_token, cand_prob, n_cand, B, M, N):
    """EAGLE-2-style tree from an expanded candidate tree (see oracle.c)."""
    par = _i32(cand_parent).reshape(-1)
    tok = _i32(cand_token).reshape(-1)
    prob = _f32(cand_prob).reshape(-1)
    nc = _i32(n_cand)
    out = {"token": np.zeros((B, N), np.int32), "parent": np.zeros((B, N), np.int32),
           "depth": np.zeros((B, N), np.int32), "score": np.zeros((B, N), np.float32),
           "anc_mask": np.zeros((B, N), np.uint64), "cand": np.zeros((B, N), np.int32),
           "n_nodes": np.zeros(B, np.int32)}
    _load().orc_rerank_tree(_ptr(par), _ptr(tok), _ptr(prob), _ptr(nc), int(B), int(M), int(N),
                            _ptr(out["token"]), _ptr(out["parent"]), _ptr(out["depth"]),
                            _ptr(out["score"]), _ptr(out["anc_mask"]), _ptr(out["cand"]),
                            _ptr(out["n_nodes"]))
    return out


CHECK_A = 1
CHECK_NEXT = 2


def check_chain(target, draft, tokens, uniforms, cu, B, K_max, V, temperature, A, nxt, top_k=0,
                tol=MARGIN_REL, threads=None):
    """Validity of another implementation's (A, next) per sequence, within the
    rounding slack tol (see orc_check_chain). Returns (valid bits [B], status
    bits the chain rule raises at that A [B])."""
    t = _f32(target).reshape(-1)
    d = _f32(draft).reshape(-1)
    y = _i32(tokens).reshape(-1)
    u = _f32(uniforms).reshape(-1)
    c = None if cu is None else _i32(cu)
    a = _i32(A)
    n = _i32(nxt)
    valid = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    _load().orc_check_chain(_ptr(t), _ptr(d), _ptr(y), _ptr(u), _ptr(c), int(B), int(K_max), int(V),
                            _t32(temperature), int(top_k), float(tol), _ptr(a), _ptr(n), _ptr(valid),
                            _ptr(st), int(threads or default_threads()))
    return valid, st


def check_tree_sampled(target, token, parent, n_nodes, uniforms, B, N, V, temperature, path, A, nxt,
                       top_k=0, tol=MARGIN_REL, threads=None):
    """1 per sequence whose sampled walk (path, A, next) is a valid walk within
    the rounding slack tol (see orc_check_tree_sampled)."""
    t = _f32(target).reshape(-1)
    tok = _i32(token).reshape(-1)
    par = _i32(parent).reshape(-1)
    nn = _i32(n_nodes)
    u = _f32(uniforms).reshape(-1)
    pa = _i32(path).reshape(-1)
    a = _i32(A)
    n = _i32(nxt)
    valid = np.zeros(B, np.int32)
    _load().orc_check_tree_sampled(_ptr(t), _ptr(tok), _ptr(par), _ptr(nn), _ptr(u), int(B), int(N),
                                   int(V), ctypes.c_double(temperature), int(top_k),
                                   ctypes.c_double(tol), _ptr(pa), _ptr(a), _ptr(n), _ptr(valid),
                                   int(threads or default_threads()))
    return valid


def check_select_len(conf, B, K, cost, k, tol=MARGIN_REL):
    """1 per sequence whose verify length k is the rule's choice within slack tol."""
    c = _f32(conf).reshape(-1)
    kk = _i32(k)
    valid = np.zeros(B, np.int32)
    _load().orc_check_select_len(_ptr(c), int(B), int(K), ctypes.c_float(cost), float(tol), _ptr(kk),
                                 _ptr(valid))
    return valid


def expand_tree(cand, expand_in, child_token, child_prob, B, M, W, C):
    """One EAGLE-2-style expansion step on host copies (see orc_expand_tree).

    cand: dict of parent, token, prob, conf ([B, M]) and n_cand ([B]); a new
    dict is returned with the grown arrays and "expand" ([B, W])."""
    out = {"parent": _i32(cand["parent"]).reshape(B, M).copy(),
           "token": _i32(cand["token"]).reshape(B, M).copy(),
           "prob": _f32(cand["prob"]).reshape(B, M).copy(),
           "conf": _f32(cand["conf"]).reshape(B, M).copy(),
           "n_cand": _i32(cand["n_cand"]).copy(),
           "expand": np.zeros((B, W), np.int32)}
    ei = _i32(expand_in).reshape(-1)
    ct = _i32(child_token).reshape(-1)
    cp = _f32(child_prob).reshape(-1)
    _load().orc_expand_tree(_ptr(out["parent"]), _ptr(out["token"]), _ptr(out["prob"]), _ptr(out["conf"]),
                            _ptr(out["n_cand"]), _ptr(ei), _ptr(out["expand"]), _ptr(ct), _ptr(cp),
                            int(B), int(M), int(W), int(C))
    return out


def empty_candidates(B, M):
    """Candidate arrays of B sequences before the first expansion step."""
    return {"parent": np.full((B, M), -1, np.int32), "token": np.full((B, M), -1, np.int32),
            "prob": np.zeros((B, M), np.float32), "conf": np.full((B, M), -1.0, np.float32),
            "n_cand": np.zeros(B, np.int32)}
