"""sd_verify_chain_noalloc (the entry point that allocates nothing: its
scratch is the library's static device array) against sd_verify_chain with a
caller workspace, on calls in a row of decreasing size; both run the same
kernels, so every output must be bit-identical, and the small case also
matches the oracle."""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_softmax_amd as sd
from rejection_sampling_verify_softmax_amd import workloads as wl

from parity import compare_chain, oracle_chain

pytestmark = pytest.mark.gpu


def _same(a, b):
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_noalloc_matches_the_workspace_entry_point():
    print("no-alloc chain: adaptive B=512 K_max=8 V=128256, then top-k B=64, then B=24 f32", flush=True)
    ad = wl.gen_adaptive_chain(device="cuda")
    sel = sd.select_len(ad.conf, ad.cost)
    torch.cuda.synchronize()
    packed = ad.packed(sel["k"])
    cases = [
        (packed, dict(cu=sel["cu"], B=ad.B, K_max=ad.K_max), 1.0, 0, False),
        (wl.gen_topk_chain(device="cuda", seed=5, B=64, K=5, V=60000, top_k=50), {}, None, None, True),
        (wl.gen_base_noise_chain(6, B=24, K=4, V=20003, base_sigma=2.0, noise_sigma=0.7, temperature=0.9,
                                 dtype="f32", device="cuda"), {}, None, None, True),
    ]
    for case, kw, T, top_k, probs in cases:
        T = case.temperature if T is None else T
        top_k = case.top_k if top_k is None else top_k
        kw = kw or dict(B=case.B, K_max=case.K_max)
        ref = sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, T, top_k=top_k,
                              want_probs=probs, want_resid=True, **kw)
        # outputs pre-allocated: the call itself allocates nothing
        out = {k: torch.full_like(v, -7) for k, v in ref.items()}
        got = sd.verify_chain_noalloc(case.target, case.draft, case.tokens, case.uniforms, T, top_k=top_k,
                                      out=out, want_probs=probs, want_resid=True, **kw)
        torch.cuda.synchronize()
        _same(ref, got)
        print(f"  B={kw['B']} K_max={kw['K_max']} V={case.V} top_k={top_k}: identical", flush=True)
    # the last (smallest) call against the oracle as well
    compare_chain(got, oracle_chain(case))


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    x = torch.zeros(16, 8, dtype=torch.bfloat16, device="cuda")
    tok = torch.zeros(8, dtype=torch.int32, device="cuda")
    u = torch.zeros(16, dtype=torch.float32, device="cuda")
    lib = sd.lib()
    import ctypes
    r = lib.sd_verify_chain_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), sd.SD_BF16,
                                    ctypes.c_void_p(tok.data_ptr()), ctypes.c_void_p(u.data_ptr()), None,
                                    5000, 8, 128256, ctypes.c_float(1.0), 0, ctypes.c_void_p(tok.data_ptr()),
                                    ctypes.c_void_p(tok.data_ptr()), None, None, None, None)
    assert r == sd.SD_EWORKSPACE
