"""Python binding of libsd: batched speculative-decoding draft verification on
AMD Instinct MI355X (gfx950).

Argument marshalling only. Every step of the verification runs in the HIP
kernels of libsd.so behind the C ABI of include/sd.h; torch provides device
memory (inputs, outputs, workspace) and the current HIP stream. There is no
CPU fallback: if libsd.so is missing or no GPU is present, the calls raise.

Functions mirror the C entry points:
  verify_chain   sd_verify_chain   (stochastic chain, or greedy when T == 0)
  verify_greedy  sd_verify_greedy
  build_tree     sd_build_tree     (DDTree best-first tree from marginals)
  verify_tree    sd_verify_tree    (walk along the target's argmax)
  verify_tree_sampled  sd_verify_tree_sampled  (walk along the target's own draws)
  select_len     sd_select_len     (DSpark verify length, packed offsets)
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsd.so")

SD_OK, SD_EINVAL, SD_EUNSUPPORTED, SD_EWORKSPACE, SD_EHIP = 0, 1, 2, 3, 4
SD_F32, SD_BF16 = 0, 1
OP_CHAIN, OP_GREEDY, OP_BUILD_TREE, OP_VERIFY_TREE, OP_SELECT_LEN, OP_VERIFY_TREE_SAMPLED = 0, 1, 2, 3, 4, 5
SEQ_BAD_TOKEN, SEQ_NONFINITE = 1, 2

_lib = None


class SDError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _load().sd_status_str(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg}")
        self.status = status


def _load():
    """Load libsd.so (built in-tree by `_build.build()`); fails loudly if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libsd.so not found at {LIB_PATH}: build it with "
                           "rejection_sampling_verify_softmax_amd._build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.sd_abi_version.argtypes = []
    lib.sd_abi_version.restype = ctypes.c_int
    lib.sd_status_str.argtypes = [ctypes.c_int]
    lib.sd_status_str.restype = ctypes.c_char_p
    lib.sd_workspace_bytes.argtypes = [ctypes.c_int, I, I, I, I, I, ctypes.POINTER(Z)]
    lib.sd_workspace_bytes.restype = ctypes.c_int
    lib.sd_verify_chain.argtypes = [P, P, ctypes.c_int, P, P, P, I, I, I, F, I, P, P, P, P, P, P, Z, P]
    lib.sd_verify_chain.restype = ctypes.c_int
    lib.sd_verify_greedy.argtypes = [P, ctypes.c_int, P, P, I, I, I, P, P, P, P, Z, P]
    lib.sd_verify_greedy.restype = ctypes.c_int
    lib.sd_build_tree.argtypes = [P, I, I, I, I, P, P, P, P, P, P, P, Z, P]
    lib.sd_build_tree.restype = ctypes.c_int
    lib.sd_verify_tree.argtypes = [P, ctypes.c_int, P, P, P, I, I, I, P, P, P, P, Z, P]
    lib.sd_verify_tree.restype = ctypes.c_int
    lib.sd_verify_tree_sampled.argtypes = [P, ctypes.c_int, P, P, P, P, I, I, I, F, I, P, P, P, P, P, Z, P]
    lib.sd_verify_tree_sampled.restype = ctypes.c_int
    lib.sd_select_len.argtypes = [P, I, I, F, P, P, P, P]
    lib.sd_select_len.restype = ctypes.c_int
    lib.sd_verify_chain_capped.argtypes = [P, P, ctypes.c_int, P, P, P, I, I, I, F, I, P, P, P, P, P,
                                           P, P, Z, P]
    lib.sd_verify_chain_capped.restype = ctypes.c_int
    lib.sd_select_len_table.argtypes = [P, I, I, P, P, P, P, P]
    lib.sd_select_len_table.restype = ctypes.c_int
    lib.sd_compact_kv.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P, P, I, I, P]
    lib.sd_compact_kv.restype = ctypes.c_int
    lib.sd_rerank_tree.argtypes = [P, P, P, P, I, I, I, P, P, P, P, P, P, P, P]
    lib.sd_rerank_tree.restype = ctypes.c_int
    lib.sd_expand_tree.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, P]
    lib.sd_expand_tree.restype = ctypes.c_int
    lib.sd_verify_chain_noalloc.argtypes = [P, P, ctypes.c_int, P, P, P, I, I, I, F, I, P, P, P, P, P, P]
    lib.sd_verify_chain_noalloc.restype = ctypes.c_int
    lib.sd_stream_read.argtypes = [P, Z, P, I, P]
    lib.sd_stream_read.restype = ctypes.c_int
    lib.sd_stream_read_rows.argtypes = [P, Z, I, Z, P, P]
    lib.sd_stream_read_rows.restype = ctypes.c_int
    lib.sd_time_next_stream_pass.argtypes = [P, P]
    lib.sd_time_next_stream_pass.restype = ctypes.c_int
    _lib = lib
    return lib


def lib():
    return _load()


def _ptr(t: Optional[torch.Tensor]):
    # a device address as a plain int (the entry points' argtypes take ints)
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    """The HIP stream handle (an int) a call runs on: `stream`, else torch's
    current stream on the current device."""
    if stream is not None:
        return stream.cuda_stream
    return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SD_BF16
    if t.dtype == torch.float32:
        return SD_F32
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check(t: Optional[torch.Tensor], name: str, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _out(o: dict, key: str, shape, dtype, dev):
    """An output tensor: o[key] when the caller passed one (checked, so that no
    kernel writes past it), else a new one."""
    t = o.get(key)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _check(t, key, dtype, dev)
    n = 1
    for d in (shape if isinstance(shape, tuple) else (shape,)):
        n *= d
    if t.numel() < n:
        raise ValueError(f"out[{key!r}] holds {t.numel()} elements, {n} needed")
    return t


def _raise(status: int, where: str):
    if status != SD_OK:
        raise SDError(status, where)


def time_next_stream_pass(start: Optional["torch.cuda.Event"], stop: Optional["torch.cuda.Event"]):
    """sd_time_next_stream_pass: the next call's streaming kernel is bracketed by
    these events on its stream. torch creates an event's HIP handle on its first
    record(), so both must have been recorded once before."""
    s = None if start is None else ctypes.c_void_p(start.cuda_event)
    e = None if stop is None else ctypes.c_void_p(stop.cuda_event)
    if (start is not None and not s.value) or (stop is not None and not e.value):
        raise ValueError("record() each event once before passing it (its HIP event is created lazily)")
    _raise(_load().sd_time_next_stream_pass(s, e), "sd_time_next_stream_pass")


def stream_read(data: torch.Tensor, sink: torch.Tensor, n_blocks: int, stream=None):
    """sd_stream_read: a plain streaming read of `data` (the device's read ceiling)."""
    _check(data, "data")
    _check(sink, "sink", torch.int32, data.device)
    nbytes = data.numel() * data.element_size()
    if sink.numel() < n_blocks:
        raise ValueError("sink needs one word per workgroup")
    _raise(_load().sd_stream_read(_ptr(data), nbytes, _ptr(sink), int(n_blocks),
                                  _stream(stream)), "sd_stream_read")


def stream_read_rows(data: torch.Tensor, chunk_bytes: int, sink: torch.Tensor, stream=None):
    """sd_stream_read_rows: a plain read of the rows of `data` (2-D, row-major),
    one workgroup per (row, chunk of chunk_bytes): the row passes' grid."""
    _check(data, "data")
    _check(sink, "sink", torch.int32, data.device)
    if data.dim() != 2:
        raise ValueError("data must be 2-D (rows)")
    row_bytes = data.shape[1] * data.element_size()
    chunks = -(-row_bytes // int(chunk_bytes))
    if sink.numel() < data.shape[0] * chunks:
        raise ValueError("sink needs one word per (row, chunk)")
    _raise(_load().sd_stream_read_rows(_ptr(data), row_bytes, int(data.shape[0]), int(chunk_bytes),
                                       _ptr(sink), _stream(stream)), "sd_stream_read_rows")


def workspace_bytes(op: int, B: int, K_max: int = 0, V: int = 1, top_k: int = 0, N: int = 2) -> int:
    return _workspace_bytes(int(op), int(B), int(K_max), int(V), int(top_k), int(N))


@functools.lru_cache(maxsize=256)
def _workspace_bytes(op: int, B: int, K_max: int, V: int, top_k: int, N: int) -> int:
    # a pure function of its sizes: remembered, so repeated calls skip the query
    out = ctypes.c_size_t(0)
    _raise(_load().sd_workspace_bytes(op, B, K_max, V, top_k, N, ctypes.byref(out)), "sd_workspace_bytes")
    return int(out.value)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor], stream=None):
    n = max(int(nbytes), 256)
    if ws is not None:
        if ws.numel() * ws.element_size() < n:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {n} needed")
        return ws
    t = torch.empty(n, dtype=torch.uint8, device=device)
    if stream is not None:
        # allocated on the current stream, used on `stream`: the allocator
        # must not hand the block out again before `stream` is done with it
        t.record_stream(stream)
    return t


def _check_rows(t: Optional[torch.Tensor], name: str, rows: int, V: int):
    if t is not None and t.numel() < rows * V:
        raise ValueError(f"{name} holds {t.numel()} elements, the batch layout needs {rows * V}")


def _check_layout(target, draft, tokens, uniforms, cu, B, K_max, V, greedy, validate, stream=None):
    """Size checks of the batch layout (include/sd.h) so that no kernel reads
    past a tensor. For a packed layout the row counts depend on cu, which lives
    on the device: validate=True reads it on the host after the call's stream
    has finished its earlier work (a synchronisation); with validate=False
    (the default) the caller vouches for cu and nothing is read back."""
    if cu is not None:
        if cu.numel() != B + 1:
            raise ValueError(f"cu must hold B+1 = {B + 1} offsets")
        if not validate:
            return
        (torch.cuda.current_stream() if stream is None else stream).synchronize()
        c = cu.cpu()
        lens = c[1:] - c[:-1]
        if int(c[0]) != 0 or (B > 0 and (int(lens.min()) < 0 or int(lens.max()) > K_max)):
            raise ValueError("cu must start at 0 and have lengths in [0, K_max]")
        R_d = int(c[-1])
    else:
        R_d = B * K_max
    _check_rows(target, "target", R_d + B, V)
    _check_rows(tokens, "tokens", R_d, 1)
    if not greedy:
        _check_rows(draft, "draft", R_d, V)
        _check_rows(uniforms, "uniforms", R_d + B, 1)


def verify_chain(target: torch.Tensor, draft: Optional[torch.Tensor], tokens: torch.Tensor,
                 uniforms: Optional[torch.Tensor], temperature: float, top_k: int = 0,
                 cu: Optional[torch.Tensor] = None, B: Optional[int] = None,
                 K_max: Optional[int] = None, want_probs: bool = False,
                 want_resid: bool = False, workspace: Optional[torch.Tensor] = None,
                 out: Optional[dict] = None, stream=None, validate: bool = False) -> dict:
    """sd_verify_chain. Dense batch (cu None): target [B*(K+1), V], draft [B*K, V],
    tokens [B*K] (or [B, K]). Packed batch: pass cu [B+1] (device int32) and K_max
    (required: the call never reads cu back to the host unless validate=True).
    Returns dict with accepted_len, next_token, status (+ probs [R_d, 2], resid)."""
    dev = target.device
    _check(target, "target", device=dev)
    dt = _dtype_code(target)
    V = int(target.shape[-1])
    if cu is not None:
        _check(cu, "cu", torch.int32, dev)
        if B is None:
            B = cu.numel() - 1
        if K_max is None:
            raise ValueError("a packed batch (cu given) needs K_max, the largest draft length")
    else:
        if K_max is None:
            K_max = int(tokens.shape[-1]) if tokens.dim() == 2 else None
        if B is None:
            if K_max is None:
                raise ValueError("pass K_max (or 2-D tokens) for a dense batch")
            B = target.numel() // V // (K_max + 1)
    _check(tokens, "tokens", torch.int32, dev)
    greedy = float(temperature) == 0.0
    if not greedy:
        _check(draft, "draft", target.dtype, dev)
        _check(uniforms, "uniforms", torch.float32, dev)
    _check_layout(target, draft, tokens, uniforms, cu, B, K_max, V, greedy, validate, stream)
    o = out or {}
    A = _out(o, "accepted_len", B, torch.int32, dev)
    nxt = _out(o, "next_token", B, torch.int32, dev)
    st = _out(o, "status", B, torch.int32, dev)
    probs = None
    if want_probs and not greedy:
        probs = _out(o, "probs", (max(tokens.numel(), 1), 2), torch.float32, dev)
    resid = None
    if want_resid and not greedy:
        resid = _out(o, "resid", B, torch.float32, dev)
    nbytes = workspace_bytes(OP_CHAIN, B, K_max, V, top_k)
    ws = _workspace(nbytes, dev, workspace, stream)
    r = _load().sd_verify_chain(_ptr(target), _ptr(draft) if not greedy else None, dt, _ptr(tokens),
                                _ptr(uniforms) if not greedy else None, _ptr(cu), int(B), int(K_max),
                                int(V), float(temperature), int(top_k), _ptr(A),
                                _ptr(nxt), _ptr(probs), _ptr(resid), _ptr(st), _ptr(ws),
                                ws.numel(), _stream(stream))
    _raise(r, "sd_verify_chain")
    res = {"accepted_len": A, "next_token": nxt, "status": st}
    if probs is not None:
        res["probs"] = probs
    if resid is not None:
        res["resid"] = resid
    return res


def verify_chain_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor], tokens: torch.Tensor,
                         uniforms: Optional[torch.Tensor], temperature: float, top_k: int = 0,
                         cu: Optional[torch.Tensor] = None, B: Optional[int] = None,
                         K_max: Optional[int] = None, out: dict = None, want_probs: bool = False,
                         want_resid: bool = False, stream=None) -> dict:
    """sd_verify_chain_noalloc: verify_chain with the library's own static
    scratch instead of a workspace. With every output passed in `out`
    (accepted_len, next_token, status, and probs / resid when asked for) the
    call allocates nothing, so it may run under graph capture."""
    dev = target.device
    _check(target, "target", device=dev)
    dt = _dtype_code(target)
    V = int(target.shape[-1])
    if cu is not None:
        _check(cu, "cu", torch.int32, dev)
        B = cu.numel() - 1 if B is None else B
        if K_max is None:
            raise ValueError("a packed batch (cu given) needs K_max, the largest draft length")
    else:
        if K_max is None:
            if tokens.dim() != 2:
                raise ValueError("pass K_max (or 2-D tokens) for a dense batch")
            K_max = int(tokens.shape[-1])
        B = target.numel() // V // (K_max + 1) if B is None else B
    _check(tokens, "tokens", torch.int32, dev)
    greedy = float(temperature) == 0.0
    if not greedy:
        _check(draft, "draft", target.dtype, dev)
        _check(uniforms, "uniforms", torch.float32, dev)
    _check_layout(target, draft, tokens, uniforms, cu, B, K_max, V, greedy, False, stream)
    o = out or {}
    A = _out(o, "accepted_len", B, torch.int32, dev)
    nxt = _out(o, "next_token", B, torch.int32, dev)
    st = _out(o, "status", B, torch.int32, dev)
    probs = None
    if want_probs and not greedy:
        probs = _out(o, "probs", (max(tokens.numel(), 1), 2), torch.float32, dev)
    resid = None
    if want_resid and not greedy:
        resid = _out(o, "resid", B, torch.float32, dev)
    r = _load().sd_verify_chain_noalloc(_ptr(target), _ptr(draft) if not greedy else None, dt,
                                        _ptr(tokens), _ptr(uniforms) if not greedy else None, _ptr(cu),
                                        int(B), int(K_max), int(V), float(temperature),
                                        int(top_k), _ptr(A), _ptr(nxt), _ptr(probs), _ptr(resid), _ptr(st),
                                        _stream(stream))
    _raise(r, "sd_verify_chain_noalloc")
    res = {"accepted_len": A, "next_token": nxt, "status": st}
    if probs is not None:
        res["probs"] = probs
    if resid is not None:
        res["resid"] = resid
    return res


def verify_chain_capped(target: torch.Tensor, draft: Optional[torch.Tensor], tokens: torch.Tensor,
                        uniforms: Optional[torch.Tensor], k_cap: torch.Tensor, temperature: float,
                        top_k: int = 0, want_probs: bool = False, want_resid: bool = False,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """sd_verify_chain_capped (cap-accept). Padded window: target [B*(K+1), V],
    draft [B*K, V], tokens [B, K], uniforms [B*(K+1)], k_cap [B] int32 (device).
    Returns accepted_len (committed), next_token, accepted_full, status
    (+ probs [B*K, 2], resid)."""
    dev = target.device
    _check(target, "target", device=dev)
    dt = _dtype_code(target)
    V = int(target.shape[-1])
    if tokens.dim() != 2:
        raise ValueError("tokens must be [B, K]")
    B, K = (int(x) for x in tokens.shape)
    _check(tokens, "tokens", torch.int32, dev)
    _check(k_cap, "k_cap", torch.int32, dev)
    if k_cap.numel() != B:
        raise ValueError("k_cap must hold one entry per sequence")
    greedy = float(temperature) == 0.0
    if not greedy:
        _check(draft, "draft", target.dtype, dev)
        _check(uniforms, "uniforms", torch.float32, dev)
    _check_layout(target, draft, tokens, uniforms, None, B, K, V, greedy, False)
    A = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    Af = torch.empty(B, dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    probs = torch.empty(max(B * K, 1), 2, dtype=torch.float32, device=dev) if want_probs and not greedy else None
    resid = torch.empty(B, dtype=torch.float32, device=dev) if want_resid and not greedy else None
    ws = _workspace(workspace_bytes(OP_CHAIN, B, K, V, top_k), dev, workspace, stream)
    r = _load().sd_verify_chain_capped(_ptr(target), _ptr(draft) if not greedy else None, dt,
                                       _ptr(tokens), _ptr(uniforms) if not greedy else None,
                                       _ptr(k_cap), B, K, V, float(temperature),
                                       int(top_k), _ptr(A), _ptr(nxt), _ptr(Af), _ptr(probs),
                                       _ptr(resid), _ptr(st), _ptr(ws), ws.numel(),
                                       _stream(stream))
    _raise(r, "sd_verify_chain_capped")
    res = {"accepted_len": A, "next_token": nxt, "accepted_full": Af, "status": st}
    if probs is not None:
        res["probs"] = probs
    if resid is not None:
        res["resid"] = resid
    return res


def verify_greedy(target: torch.Tensor, tokens: torch.Tensor, cu: Optional[torch.Tensor] = None,
                  B: Optional[int] = None, K_max: Optional[int] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  validate: bool = False) -> dict:
    """sd_verify_greedy; same layout as verify_chain (K_max required with cu)."""
    dev = target.device
    _check(target, "target", device=dev)
    _check(tokens, "tokens", torch.int32, dev)
    dt = _dtype_code(target)
    V = int(target.shape[-1])
    if cu is not None:
        _check(cu, "cu", torch.int32, dev)
        B = cu.numel() - 1 if B is None else B
        if K_max is None:
            raise ValueError("a packed batch (cu given) needs K_max, the largest draft length")
    else:
        if K_max is None:
            if tokens.dim() != 2:
                raise ValueError("pass K_max (or 2-D tokens) for a dense batch")
            K_max = int(tokens.shape[-1])
        B = target.numel() // V // (K_max + 1) if B is None else B
    _check_layout(target, None, tokens, None, cu, B, K_max, V, True, validate, stream)
    A = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(workspace_bytes(OP_GREEDY, B, K_max, V), dev, workspace, stream)
    r = _load().sd_verify_greedy(_ptr(target), dt, _ptr(tokens), _ptr(cu), int(B), int(K_max), int(V),
                                 _ptr(A), _ptr(nxt), _ptr(st), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _raise(r, "sd_verify_greedy")
    return {"accepted_len": A, "next_token": nxt, "status": st}


def build_tree(marginals: torch.Tensor, N: int, workspace: Optional[torch.Tensor] = None,
               stream=None) -> dict:
    """sd_build_tree. marginals [B, K, V] float32 on the GPU."""
    dev = marginals.device
    _check(marginals, "marginals", torch.float32, dev)
    B, K, V = (int(s) for s in marginals.shape)
    out = {
        "token": torch.empty(B, N, dtype=torch.int32, device=dev),
        "parent": torch.empty(B, N, dtype=torch.int32, device=dev),
        "depth": torch.empty(B, N, dtype=torch.int32, device=dev),
        "score": torch.empty(B, N, dtype=torch.float32, device=dev),
        "anc_mask": torch.empty(B, N, dtype=torch.int64, device=dev),
        "n_nodes": torch.empty(B, dtype=torch.int32, device=dev),
    }
    ws = _workspace(workspace_bytes(OP_BUILD_TREE, B, K, V, 0, N), dev, workspace, stream)
    r = _load().sd_build_tree(_ptr(marginals), B, K, V, int(N), _ptr(out["token"]), _ptr(out["parent"]),
                              _ptr(out["depth"]), _ptr(out["score"]), _ptr(out["anc_mask"]),
                              _ptr(out["n_nodes"]), _ptr(ws), ws.numel(),
                              _stream(stream))
    _raise(r, "sd_build_tree")
    return out


def verify_tree(target: torch.Tensor, tree: dict, workspace: Optional[torch.Tensor] = None,
                stream=None, out: Optional[dict] = None) -> dict:
    """sd_verify_tree. target [B, N, V] (bf16 or fp32); tree from build_tree.
    The walk needs no workspace (the argument is accepted and ignored)."""
    dev = target.device
    _check(target, "target", device=dev)
    dt = _dtype_code(target)
    B, N, V = (int(s) for s in target.shape)
    for k in ("token", "parent", "n_nodes"):
        _check(tree[k], k, torch.int32, dev)
    if tree["token"].numel() < B * N or tree["parent"].numel() < B * N or tree["n_nodes"].numel() < B:
        raise ValueError("tree arrays do not cover [B, N]")
    o = out or {}
    path = _out(o, "path", (B, N), torch.int32, dev)
    A = _out(o, "accepted_len", B, torch.int32, dev)
    nxt = _out(o, "next_token", B, torch.int32, dev)
    r = _load().sd_verify_tree(_ptr(target), dt, _ptr(tree["token"]), _ptr(tree["parent"]),
                               _ptr(tree["n_nodes"]), B, N, V, _ptr(path), _ptr(A), _ptr(nxt),
                               None, 0, _stream(stream))
    _raise(r, "sd_verify_tree")
    return {"path": path, "accepted_len": A, "next_token": nxt}


def verify_tree_sampled(target: torch.Tensor, tree: dict, uniforms: Optional[torch.Tensor],
                        temperature: float, top_k: int = 0, out: Optional[dict] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """sd_verify_tree_sampled. target [B, N, V] (bf16 or fp32); tree from build_tree;
    uniforms [B, N] float32 (None when temperature == 0); top_k 0 = no truncation.
    The walk needs no workspace; the argument is accepted and ignored."""
    dev = target.device
    _check(target, "target", device=dev)
    dt = _dtype_code(target)
    B, N, V = (int(s) for s in target.shape)
    for k in ("token", "parent", "n_nodes"):
        _check(tree[k], k, torch.int32, dev)
    if tree["token"].numel() < B * N or tree["parent"].numel() < B * N or tree["n_nodes"].numel() < B:
        raise ValueError("tree arrays do not cover [B, N]")
    if uniforms is not None:
        _check(uniforms, "uniforms", torch.float32, dev)
        if uniforms.numel() < B * N:
            raise ValueError("uniforms needs one entry per (sequence, node)")
    o = out or {}
    path = _out(o, "path", (B, N), torch.int32, dev)
    A = _out(o, "accepted_len", B, torch.int32, dev)
    nxt = _out(o, "next_token", B, torch.int32, dev)
    st = _out(o, "status", B, torch.int32, dev)
    r = _load().sd_verify_tree_sampled(_ptr(target), dt, _ptr(tree["token"]), _ptr(tree["parent"]),
                                       _ptr(tree["n_nodes"]), _ptr(uniforms), B, N, V,
                                       float(temperature), int(top_k), _ptr(path),
                                       _ptr(A), _ptr(nxt), _ptr(st), None, 0,
                                       _stream(stream))
    _raise(r, "sd_verify_tree_sampled")
    return {"path": path, "accepted_len": A, "next_token": nxt, "status": st}


def select_len(conf: torch.Tensor, cost: float, out: Optional[dict] = None, stream=None) -> dict:
    """sd_select_len. conf [B, K_max] float32 on the GPU."""
    dev = conf.device
    _check(conf, "conf", torch.float32, dev)
    B, K = (int(s) for s in conf.shape)
    o = out or {}
    k = _out(o, "k", B, torch.int32, dev)
    adv = _out(o, "adv", B, torch.float32, dev)
    cu = _out(o, "cu", B + 1, torch.int32, dev)
    r = _load().sd_select_len(_ptr(conf), B, K, float(cost), _ptr(k), _ptr(adv),
                              _ptr(cu), _stream(stream))
    _raise(r, "sd_select_len")
    return {"k": k, "adv": adv, "cu": cu}


def select_len_table(conf: torch.Tensor, cost_table: torch.Tensor, out: Optional[dict] = None,
                     stream=None) -> dict:
    """sd_select_len_table. conf [B, K_max] float32, cost_table [K_max] float32, on the GPU."""
    dev = conf.device
    _check(conf, "conf", torch.float32, dev)
    _check(cost_table, "cost_table", torch.float32, dev)
    B, K = (int(s) for s in conf.shape)
    if cost_table.numel() < K:
        raise ValueError("cost_table needs one entry per position")
    o = out or {}
    k = _out(o, "k", B, torch.int32, dev)
    adv = _out(o, "adv", B, torch.float32, dev)
    cu = _out(o, "cu", B + 1, torch.int32, dev)
    r = _load().sd_select_len_table(_ptr(conf), B, K, _ptr(cost_table), _ptr(k), _ptr(adv), _ptr(cu),
                                    _stream(stream))
    _raise(r, "sd_select_len_table")
    return {"k": k, "adv": adv, "cu": cu}


def compact_kv(kv: torch.Tensor, row_base: torch.Tensor, path: torch.Tensor,
               accepted_len: torch.Tensor, stream=None) -> torch.Tensor:
    """sd_compact_kv, in place. kv: contiguous GPU tensor whose first dimension
    is the row (token) index; row_base [B] int64; path [B, N] int32 and
    accepted_len [B] int32 as returned by verify_tree. Returns kv."""
    dev = kv.device
    _check(kv, "kv", device=dev)
    _check(row_base, "row_base", torch.int64, dev)
    _check(path, "path", torch.int32, dev)
    _check(accepted_len, "accepted_len", torch.int32, dev)
    if path.dim() != 2:
        raise ValueError("path must be [B, N]")
    B, N = (int(x) for x in path.shape)
    if row_base.numel() != B or accepted_len.numel() != B:
        raise ValueError("row_base and accepted_len need one entry per sequence")
    n_rows = int(kv.shape[0])
    row_bytes = kv.numel() * kv.element_size() // max(n_rows, 1)
    r = _load().sd_compact_kv(_ptr(kv), row_bytes, n_rows, _ptr(row_base), _ptr(path),
                              _ptr(accepted_len), B, N, _stream(stream))
    _raise(r, "sd_compact_kv")
    return kv


def empty_candidates(B: int, M: int, device="cuda") -> dict:
    """Candidate arrays for sd_expand_tree before its first call: n_cand = 0
    (the first call writes the root); the other arrays need no values."""
    return {"parent": torch.empty(B, M, dtype=torch.int32, device=device),
            "token": torch.empty(B, M, dtype=torch.int32, device=device),
            "prob": torch.empty(B, M, dtype=torch.float32, device=device),
            "conf": torch.empty(B, M, dtype=torch.float32, device=device),
            "n_cand": torch.zeros(B, dtype=torch.int32, device=device)}


def expand_tree(cand: dict, expand_in: Optional[torch.Tensor], child_token: torch.Tensor,
                child_prob: torch.Tensor, expand_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sd_expand_tree: one EAGLE-2 expansion step, in place on the candidate
    arrays of `cand` (parent, token, prob, conf [B, M]; n_cand [B]).
    child_token / child_prob [B, W, C]: the draft's children of the node in
    each expand_in slot. Returns expand_out [B, W] (may be expand_in itself)."""
    dev = cand["parent"].device
    for k, dt in (("parent", torch.int32), ("token", torch.int32), ("prob", torch.float32),
                  ("conf", torch.float32), ("n_cand", torch.int32)):
        _check(cand[k], k, dt, dev)
    _check(child_token, "child_token", torch.int32, dev)
    _check(child_prob, "child_prob", torch.float32, dev)
    B, M = (int(x) for x in cand["parent"].shape)
    if child_token.dim() != 3 or child_token.shape != child_prob.shape or int(child_token.shape[0]) != B:
        raise ValueError("child_token and child_prob must both be [B, W, C]")
    W, C = int(child_token.shape[1]), int(child_token.shape[2])
    for k in ("token", "prob", "conf"):
        if tuple(cand[k].shape) != (B, M):
            raise ValueError(f"cand[{k!r}] must be [B, M] like cand['parent']")
    if cand["n_cand"].numel() != B:
        raise ValueError("n_cand needs one entry per sequence")
    if expand_in is not None:
        _check(expand_in, "expand_in", torch.int32, dev)
        if expand_in.numel() != B * W:
            raise ValueError("expand_in must be [B, W]")
    out = torch.empty(B, W, dtype=torch.int32, device=dev) if expand_out is None else expand_out
    _check(out, "expand_out", torch.int32, dev)
    if out.numel() != B * W:
        raise ValueError("expand_out must be [B, W]")
    r = _load().sd_expand_tree(_ptr(cand["parent"]), _ptr(cand["token"]), _ptr(cand["prob"]),
                               _ptr(cand["conf"]), _ptr(cand["n_cand"]), _ptr(expand_in), _ptr(out),
                               _ptr(child_token), _ptr(child_prob), B, M, W, C, _stream(stream))
    _raise(r, "sd_expand_tree")
    return out


_RERANK_OUT = (("token", torch.int32), ("parent", torch.int32), ("depth", torch.int32),
               ("score", torch.float32), ("anc_mask", torch.int64), ("cand", torch.int32))


def rerank_tree(cand_parent: torch.Tensor, cand_token: torch.Tensor, cand_prob: torch.Tensor,
                n_cand: torch.Tensor, N: int, stream=None, out: Optional[dict] = None) -> dict:
    """sd_rerank_tree. cand_* [B, M] (int32, int32, float32) and n_cand [B] int32 on the GPU.
    Returns the tree as build_tree does, plus "cand" (the candidate behind each node).
    `out` may hold the output tensors of an earlier call of the same sizes, to be
    overwritten instead of allocated."""
    dev = cand_parent.device
    _check(cand_parent, "cand_parent", torch.int32, dev)
    _check(cand_token, "cand_token", torch.int32, dev)
    _check(cand_prob, "cand_prob", torch.float32, dev)
    _check(n_cand, "n_cand", torch.int32, dev)
    B, M = (int(x) for x in cand_parent.shape)
    if cand_token.shape != cand_parent.shape or cand_prob.shape != cand_parent.shape or n_cand.numel() != B:
        raise ValueError("candidate arrays must be [B, M] and n_cand [B]")
    if out is None:
        out = {k: torch.empty(B, N, dtype=t, device=dev) for k, t in _RERANK_OUT}
        out["n_nodes"] = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        for k, t in _RERANK_OUT + (("n_nodes", torch.int32),):
            _check(out[k], k, t, dev)
            if out[k].numel() != (B if k == "n_nodes" else B * N):
                raise ValueError(f"out[{k!r}] must be [B, N] ([B] for n_nodes)")
    r = _load().sd_rerank_tree(_ptr(cand_parent), _ptr(cand_token), _ptr(cand_prob), _ptr(n_cand), B, M,
                               int(N), _ptr(out["token"]), _ptr(out["parent"]), _ptr(out["depth"]),
                               _ptr(out["score"]), _ptr(out["anc_mask"]), _ptr(out["cand"]),
                               _ptr(out["n_nodes"]), _stream(stream))
    _raise(r, "sd_rerank_tree")
    return out
