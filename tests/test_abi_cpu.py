"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/sd.h declares, and rejects invalid calls before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sd.h")


@pytest.fixture(scope="module")
def L():
    import rejection_sampling_verify_softmax_amd as sd
    if not os.path.exists(sd.LIB_PATH):
        from rejection_sampling_verify_softmax_amd import _build
        _build.build()
    return sd.lib()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_symbols()
    for n in ("sd_verify_chain", "sd_verify_greedy", "sd_build_tree", "sd_verify_tree", "sd_select_len",
              "sd_verify_chain_capped", "sd_select_len_table", "sd_compact_kv", "sd_rerank_tree",
              "sd_verify_tree_sampled",
              "sd_workspace_bytes", "sd_abi_version", "sd_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    import rejection_sampling_verify_softmax_amd as sd
    out = os.popen(f"nm -D --defined-only {sd.LIB_PATH}").read()
    exported = set(re.findall(r" T (sd_\w+)", out))
    missing = [n for n in declared_symbols() if n not in exported]
    assert not missing, missing
    for n in declared_symbols():
        assert hasattr(L, n)


def test_version_and_status_strings(L):
    assert L.sd_abi_version() == 1
    for s in range(5):
        assert L.sd_status_str(s).startswith(b"SD_")
    assert L.sd_status_str(99) == b"unknown sd status"


def _chain(L, **kw):
    a = dict(target=16, draft=16, dtype=1, tokens=16, uni=16, cu=None, B=2, K=3, V=100, T=1.0, top_k=0,
             A=16, nxt=16, probs=None, resid=None, st=None, ws=16, wsb=1 << 30, stream=None)
    a.update(kw)
    f = lambda v: None if v is None else ctypes.c_void_p(v)
    return L.sd_verify_chain(f(a["target"]), f(a["draft"]), a["dtype"], f(a["tokens"]), f(a["uni"]),
                             f(a["cu"]), a["B"], a["K"], a["V"], ctypes.c_float(a["T"]), a["top_k"],
                             f(a["A"]), f(a["nxt"]), f(a["probs"]), f(a["resid"]), f(a["st"]),
                             f(a["ws"]), ctypes.c_size_t(a["wsb"]), f(a["stream"]))


@pytest.mark.parametrize("bad", [
    dict(B=0), dict(B=-1), dict(V=0), dict(V=1 << 24), dict(K=65), dict(K=-1),
    dict(T=-1.0), dict(T=float("nan")), dict(T=float("inf")), dict(top_k=-1), dict(top_k=257),
    dict(dtype=7), dict(target=None), dict(A=None), dict(nxt=None), dict(ws=None),
    dict(tokens=None), dict(uni=None), dict(draft=None),
])
def test_chain_rejects_invalid_arguments(L, bad):
    assert _chain(L, **bad) == 1          # SD_EINVAL, nothing launched


def test_chain_greedy_needs_no_draft_or_uniforms_but_checks_workspace(L):
    # T == 0: draft and uniforms may be NULL; a 1-byte workspace is too small
    assert _chain(L, T=0.0, draft=None, uni=None, wsb=1) == 3      # SD_EWORKSPACE


def test_workspace_too_small(L):
    assert _chain(L, wsb=16) == 3


@pytest.mark.parametrize("which", ["target", "draft", "ws"])
def test_chain_rejects_misaligned_rows(L, which):
    # logit rows and the workspace are read in 16-byte vectors: a base pointer
    # off a 16-byte boundary (a view at an odd storage offset) is refused
    assert _chain(L, **{which: 16 + 2}) == 1
    assert _chain(L, **{which: 16 + 8}) == 1


def test_other_calls_reject_misaligned_rows(L):
    v = ctypes.c_void_p
    one, odd = v(16), v(18)
    assert L.sd_verify_greedy(odd, 1, one, None, 2, 3, 100, one, one, None, one, 1 << 30, None) == 1
    assert L.sd_build_tree(odd, 2, 4, 100, 8, one, one, one, one, one, one, one, 1 << 30, None) == 1
    assert L.sd_verify_tree(odd, 1, one, one, one, 2, 8, 100, one, one, one, one, 1 << 30, None) == 1
    assert L.sd_verify_tree_sampled(odd, 1, one, one, one, one, 2, 8, 100, ctypes.c_float(1.0), 0, one,
                                    one, one, None, None, 0, None) == 1
    assert L.sd_compact_kv(odd, 64, 10, one, one, one, 2, 8, None) == 1


def test_workspace_bytes(L):
    import rejection_sampling_verify_softmax_amd as sd
    n = sd.workspace_bytes(sd.OP_CHAIN, 512, 8, 128256, 0)
    assert n > 0 and n % 256 == 0
    assert sd.workspace_bytes(sd.OP_CHAIN, 256, 5, 151936, 50) >= 256 * 6 * 2 * 50 * 8
    assert sd.workspace_bytes(sd.OP_BUILD_TREE, 32, 16, 32000, 0, 64) >= 32 * 16 * 63 * 8
    assert sd.workspace_bytes(sd.OP_SELECT_LEN, 512, 8) == 0
    out = ctypes.c_size_t(0)
    assert L.sd_workspace_bytes(0, 0, 8, 100, 0, 0, ctypes.byref(out)) == 1
    assert L.sd_workspace_bytes(2, 4, 17, 100, 0, 64, ctypes.byref(out)) == 1   # tree K > 16
    assert L.sd_workspace_bytes(2, 4, 16, 100, 0, 65, ctypes.byref(out)) == 1   # N > 64
    assert L.sd_workspace_bytes(9, 4, 16, 100, 0, 64, ctypes.byref(out)) == 1   # unknown op
    assert L.sd_workspace_bytes(0, 4, 4, 100, 0, 0, None) == 1


def test_other_calls_reject_invalid_arguments(L):
    v = ctypes.c_void_p
    one = v(16)
    # greedy
    assert L.sd_verify_greedy(None, 1, one, None, 2, 3, 100, one, one, None, one, 1 << 30, None) == 1
    assert L.sd_verify_greedy(one, 1, one, None, 2, 3, 100, one, one, None, one, 8, None) == 3
    # tree build: N out of range, K out of range, null outputs
    assert L.sd_build_tree(one, 2, 4, 100, 1, one, one, one, one, one, one, one, 1 << 30, None) == 1
    assert L.sd_build_tree(one, 2, 17, 100, 8, one, one, one, one, one, one, one, 1 << 30, None) == 1
    assert L.sd_build_tree(one, 2, 4, 100, 8, None, one, one, one, one, one, one, 1 << 30, None) == 1
    assert L.sd_build_tree(one, 2, 4, 100, 8, one, one, one, one, one, one, one, 8, None) == 3
    # tree verify
    assert L.sd_verify_tree(one, 1, one, one, one, 2, 65, 100, one, one, one, one, 1 << 30, None) == 1
    assert L.sd_verify_tree(one, 5, one, one, one, 2, 8, 100, one, one, one, one, 1 << 30, None) == 1
    # select_len
    assert L.sd_select_len(one, 0, 8, ctypes.c_float(0.1), one, None, None, None) == 1
    assert L.sd_select_len(one, 4, 65, ctypes.c_float(0.1), one, None, None, None) == 1
    assert L.sd_select_len(one, 4, 8, ctypes.c_float(float("nan")), one, None, None, None) == 1
    assert L.sd_select_len(one, 4, 8, ctypes.c_float(0.1), None, None, None, None) == 1


def test_capped_and_cost_table_reject_invalid_arguments(L):
    one = ctypes.c_void_p(16)
    f = ctypes.c_float

    def capped(cap=one, B=2, K=3, A=one, wsb=1 << 30, T=1.0):
        return L.sd_verify_chain_capped(one, one, 1, one, one, cap, B, K, 100, f(T), 0, A, one, None,
                                        None, None, None, one, wsb, None)
    assert capped(cap=None) == 1
    assert capped(B=0) == 1
    assert capped(K=65) == 1
    assert capped(A=None) == 1
    assert capped(T=-1.0) == 1
    assert capped(wsb=16) == 3
    assert L.sd_select_len_table(one, 4, 8, None, one, None, None, None) == 1
    assert L.sd_select_len_table(None, 4, 8, one, one, None, None, None) == 1
    assert L.sd_select_len_table(one, 4, 65, one, one, None, None, None) == 1
    assert L.sd_select_len_table(one, 0, 8, one, one, None, None, None) == 1
    assert L.sd_select_len_table(one, 4, 8, one, None, None, None, None) == 1


def test_compact_kv_rejects_invalid_arguments(L):
    one = ctypes.c_void_p(16)
    assert L.sd_compact_kv(None, 64, 10, one, one, one, 2, 8, None) == 1
    assert L.sd_compact_kv(one, 24, 10, one, one, one, 2, 8, None) == 1      # not a multiple of 16
    assert L.sd_compact_kv(one, 0, 10, one, one, one, 2, 8, None) == 1
    assert L.sd_compact_kv(one, 64, 0, one, one, one, 2, 8, None) == 1
    assert L.sd_compact_kv(one, 64, 10, one, one, one, 0, 8, None) == 1
    assert L.sd_compact_kv(one, 64, 10, one, one, one, 2, 65, None) == 1
    assert L.sd_compact_kv(one, 64, 10, None, one, one, 2, 8, None) == 1


def test_rerank_tree_rejects_invalid_arguments(L):
    one = ctypes.c_void_p(16)

    def rr(B=2, M=100, N=64, first=one, out=one):
        return L.sd_rerank_tree(first, one, one, one, B, M, N, out, one, one, one, one, None, one, None)
    assert rr(B=0) == 1
    assert rr(M=0) == 1
    assert rr(M=1025) == 1
    assert rr(N=1) == 1
    assert rr(N=65) == 1
    assert rr(first=None) == 1
    assert rr(out=None) == 1


def test_tree_sampled_rejects_invalid_arguments(L):
    one = ctypes.c_void_p(16)
    f = ctypes.c_float

    def ts(dtype=1, uni=one, B=2, N=8, V=100, T=1.0, top_k=0, out=one, ws=None, wsb=0):
        return L.sd_verify_tree_sampled(one, dtype, one, one, one, uni, B, N, V, f(T), top_k, out, one,
                                        one, None, ws, wsb, None)
    assert ts(B=0) == 1
    assert ts(N=1) == 1
    assert ts(N=65) == 1
    assert ts(V=0) == 1
    assert ts(V=1 << 24) == 1
    assert ts(dtype=5) == 1
    assert ts(T=-0.5) == 1
    assert ts(T=float("inf")) == 1
    assert ts(top_k=-1) == 1
    assert ts(uni=None) == 1              # uniforms are required when T > 0
    assert ts(out=None) == 1
    assert ts(top_k=257) == 1             # above SD_MAX_TOPK
    assert ts(top_k=50, uni=None) == 1
    assert ts(top_k=50, uni=None, T=0.0, out=None) == 1
    import rejection_sampling_verify_softmax_amd as sd
    # both walks read their rows on demand: no workspace with or without top-k
    assert sd.workspace_bytes(sd.OP_VERIFY_TREE_SAMPLED, 32, 0, 32000, 0, 64) == 0
    assert sd.workspace_bytes(sd.OP_VERIFY_TREE_SAMPLED, 32, 0, 32000, 50, 64) == 0
    assert sd.workspace_bytes(sd.OP_VERIFY_TREE_SAMPLED, 32, 0, 40, 50, 64) == 0


def test_binding_fails_loudly_without_gpu():
    import torch
    import rejection_sampling_verify_softmax_amd as sd
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    x = torch.zeros(8, 16)
    with pytest.raises(ValueError):
        sd.verify_chain(x, x, torch.zeros(4, dtype=torch.int32), torch.zeros(8), 1.0, K_max=1)


def test_tree_binding_checks_inputs_without_gpu():
    import torch
    import rejection_sampling_verify_softmax_amd as sd
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    rows = torch.zeros(2, 4, 16)
    tree = {"token": torch.zeros(2, 4, dtype=torch.int32), "parent": torch.zeros(2, 4, dtype=torch.int32),
            "n_nodes": torch.zeros(2, dtype=torch.int32)}
    with pytest.raises(ValueError):                    # host tensors
        sd.verify_tree_sampled(rows, tree, torch.zeros(2, 4), 1.0)
    with pytest.raises(ValueError):
        sd.verify_tree(rows, tree)



def test_noalloc_rejects_before_any_hip_call(L):
    v, f = ctypes.c_void_p, ctypes.c_float
    one = v(16)

    def na(B=2, K=3, V=100, T=1.0, top_k=0, target=one, draft=one, A=one, uni=one, dtype=1):
        return L.sd_verify_chain_noalloc(target, draft, dtype, one, uni, None, B, K, V, f(T), top_k, A, one,
                                         None, None, None, None)
    assert na(B=0) == 1
    assert na(K=65) == 1
    assert na(T=-1.0) == 1
    assert na(top_k=300) == 1
    assert na(target=None) == 1
    assert na(A=None) == 1
    assert na(uni=None) == 1
    assert na(draft=v(24)) == 1                   # misaligned logit rows
    # a batch whose scratch need exceeds the library's static array
    # (V = 128256, K = 8: bf16 fits up to B = 4999, fp32 up to B = 2577)
    assert na(B=5000, K=8, V=128256) == 3        # SD_EWORKSPACE, nothing launched
    assert na(B=2578, K=8, V=128256, dtype=0) == 3
    ws = ctypes.c_size_t()
    assert L.sd_workspace_bytes(0, 2577, 8, 128256, 0, 0, ctypes.byref(ws)) == 0   # fp32 needs the most
    assert ws.value <= 16 << 20
    assert L.sd_workspace_bytes(0, 2578, 8, 128256, 0, 0, ctypes.byref(ws)) == 0
    assert ws.value > 16 << 20


def test_expand_tree_rejects_invalid_arguments(L):
    one = ctypes.c_void_p(16)

    def ex(B=2, M=100, W=10, C=10, first=one, kids=one, out=one):
        return L.sd_expand_tree(first, one, one, one, one, None, out, kids, one, B, M, W, C, None)
    assert ex(B=0) == 1
    assert ex(M=0) == 1
    assert ex(M=1025) == 1
    assert ex(W=0) == 1
    assert ex(W=65) == 1
    assert ex(C=0) == 1
    assert ex(first=None) == 1
    assert ex(kids=None) == 1
    assert ex(out=None) == 1


def test_stream_reads_reject_invalid_arguments(L):
    v, z = ctypes.c_void_p, ctypes.c_size_t
    one, odd = v(16), v(18)
    assert L.sd_stream_read(None, z(1024), one, 4, None) == 1
    assert L.sd_stream_read(odd, z(1024), one, 4, None) == 1
    assert L.sd_stream_read(one, z(1000), one, 4, None) == 1          # not a multiple of 16
    assert L.sd_stream_read(one, z(1024), None, 4, None) == 1
    assert L.sd_stream_read(one, z(1024), one, 0, None) == 1

    def rows(data=one, row_bytes=4096, n_rows=8, chunk=1024, sink=one):
        return L.sd_stream_read_rows(data, z(row_bytes), n_rows, z(chunk), sink, None)
    assert rows(data=None) == 1
    assert rows(data=odd) == 1
    assert rows(sink=None) == 1
    assert rows(row_bytes=0) == 1
    assert rows(row_bytes=4100) == 1
    assert rows(chunk=0) == 1
    assert rows(chunk=1000) == 1
    assert rows(n_rows=0) == 1
    assert rows(row_bytes=(1 << 32) + 16) == 1
    assert rows(row_bytes=1 << 20, n_rows=1 << 16, chunk=16) == 1    # more than 2^24 workgroups
