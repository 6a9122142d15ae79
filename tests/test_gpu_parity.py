"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases (several 16-byte-vector tiles, several chunks, ragged tails) run
the oracle on every sequence; the five full-size workloads run the oracle on a
sample of sequences, in the launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_softmax_amd as sd
from rejection_sampling_verify_softmax_amd import workloads as wl

from parity import close_rel, compare_chain, oracle_chain, sample_seqs, subset_host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_chain(case, probs=True, **kw):
    # probs=False is the serving configuration: positions are then verified in
    # phases and rows after an early rejection are never read
    kw.setdefault("validate", True)
    return sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, case.temperature,
                           top_k=case.top_k, cu=case.cu, B=case.B, K_max=case.K_max,
                           want_probs=probs, want_resid=True, **kw)


# --------------------------------------------------------------------------
# stochastic chain, full vocabulary
# --------------------------------------------------------------------------

def test_chain_B1_K4_V1000_f32():
    _say("chain: B=1 K=4 V=1000 fp32")
    case = wl.gen_chain_small(device="cuda")
    out = run_chain(case)
    info = compare_chain(out, oracle_chain(case))
    _say(f"  {info}")


@pytest.mark.parametrize("dtype,V,T", [("bf16", 40000, 0.9), ("bf16", 16384 * 2 + 8, 1.0),
                                       ("f32", 20000, 1.3), ("f32", 1001, 1.0), ("bf16", 777, 0.6),
                                       ("bf16", 40001, 0.8), ("f32", 20003, 1.1)])
def test_chain_small_all_sequences(dtype, V, T):
    _say(f"chain small {dtype} V={V} T={T}")
    case = wl.gen_base_noise_chain(11 + V, B=24, K=5, V=V, base_sigma=2.0, noise_sigma=0.6,
                                   temperature=T, dtype=dtype, device="cuda")
    out = run_chain(case)
    info = compare_chain(out, oracle_chain(case))
    _say(f"  {info}")
    A = out["accepted_len"].cpu().numpy()
    assert (A < case.K_max).any()


# Windows of at least 2^24 logits are verified in phases when no per-position
# probabilities are asked for (smaller ones in one pass); these cases are sized
# to take the phased path, and are checked against the oracle and against the
# one-pass call.
@pytest.mark.parametrize("dtype,V,T,B", [("bf16", 40000, 0.9, 96), ("bf16", 16384 * 2 + 8, 1.0, 96),
                                         ("f32", 20000, 1.3, 160)])
def test_chain_phased_all_sequences(dtype, V, T, B):
    K = 5
    assert B * (K + 1) * V >= 1 << 24
    _say(f"chain phased {dtype} V={V} T={T} B={B}")
    case = wl.gen_base_noise_chain(13 + V, B=B, K=K, V=V, base_sigma=2.0, noise_sigma=0.6,
                                   temperature=T, dtype=dtype, device="cuda")
    one = run_chain(case)
    ph = run_chain(case, probs=False)
    for key in ("accepted_len", "next_token", "status", "resid"):
        assert torch.equal(one[key], ph[key]), key
    info = compare_chain(ph, oracle_chain(case, sample_seqs(B, 32, seed=V)))
    _say(f"  {info}")


# A batch of at least 256 sequences takes the last decision, the residual mass
# and the final draw in one workgroup per sequence (smaller batches with rows
# longer than one mass chunk use the chunked launches above); vocabularies
# that are not a whole number of 16-byte vectors take the element-wise loads.
@pytest.mark.parametrize("dtype,V,T,B,K", [("bf16", 40003, 0.8, 256, 2), ("bf16", 40000, 1.0, 300, 3),
                                           ("f32", 12001, 1.0, 300, 3)])
def test_chain_large_batch_all_sequences(dtype, V, T, B, K):
    _say(f"chain large batch {dtype} V={V} T={T} B={B} K={K}")
    case = wl.gen_base_noise_chain(17 + V, B=B, K=K, V=V, base_sigma=2.0, noise_sigma=0.6,
                                   temperature=T, dtype=dtype, device="cuda")
    one = run_chain(case)
    ph = run_chain(case, probs=False)
    for key in ("accepted_len", "next_token", "status", "resid"):
        assert torch.equal(one[key], ph[key]), key
    info = compare_chain(one, oracle_chain(case))
    _say(f"  {info}")
    A = one["accepted_len"].cpu().numpy()
    assert (A < K).any() and (A == K).any()


def test_chain_extra_token_in_every_chunk():
    # drafts equal to the targets: every position is accepted and every
    # sequence draws its extra token from p of its last row, whose chunk the
    # last launch finds from the row's chunk partials; V spans four 32K-token
    # chunks (the last one short) and the uniforms a grid, so the draws land
    # in every chunk, in the phased and the one-pass launches
    B, K, V = 256, 2, 3 * 32768 + 1000
    _say(f"chain extra token across chunks B={B} K={K} V={V} bf16")
    g = torch.Generator(device="cuda").manual_seed(41)
    target = (torch.randn(B * (K + 1), V, generator=g, device="cuda") * 2.0).to(torch.bfloat16)
    rows = torch.arange(B * (K + 1), device="cuda").view(B, K + 1)[:, :K].reshape(-1)
    draft = target[rows].contiguous()
    tokens = torch.randint(0, V, (B * K,), generator=g, device="cuda", dtype=torch.int32)
    uniforms = wl.grid_uniforms((B * (K + 1),), g, "cuda")
    case = wl.ChainCase(B=B, K_max=K, V=V, temperature=1.0, top_k=0, target=target, draft=draft,
                        tokens=tokens, uniforms=uniforms)
    one = run_chain(case)
    ph = run_chain(case, probs=False)
    for key in ("accepted_len", "next_token", "status", "resid"):
        assert torch.equal(one[key], ph[key]), key
    assert (one["accepted_len"].cpu().numpy() == K).all()
    info = compare_chain(one, oracle_chain(case))
    chunks = np.bincount(one["next_token"].cpu().numpy() // 32768, minlength=4)
    _say(f"  {info}, draws per chunk {chunks.tolist()}")
    assert (chunks > 0).all()


def test_chain_phased_ragged():
    lengths = [0, 3, 1, 5, 0, 2, 8, 4, 1, 0, 6, 7, 8, 8, 2, 2, 3, 8, 1, 5]
    V = 100000
    assert len(lengths) * 9 * V >= 1 << 24
    case = wl.ragged_chain(7, lengths, V, dtype="bf16", device="cuda")
    one = run_chain(case)
    ph = run_chain(case, probs=False)
    for key in ("accepted_len", "next_token", "status", "resid"):
        assert torch.equal(one[key], ph[key]), key
    compare_chain(ph, oracle_chain(case))


def test_chain_packed_ragged_lengths():
    lengths = [0, 3, 1, 5, 0, 2, 8, 4, 1, 0, 6, 7]
    _say(f"packed chain lengths {lengths}")
    case = wl.ragged_chain(5, lengths, 30000, dtype="bf16", device="cuda")
    out = run_chain(case)
    info = compare_chain(out, oracle_chain(case))
    _say(f"  {info}")
    # a packed call matches the dense call of the same rows sequence by sequence
    for b, k in enumerate(lengths):
        cu = case.cu.cpu().numpy()
        sub = wl.ChainCase(B=1, K_max=k, V=case.V, temperature=case.temperature, top_k=0,
                           target=case.target[cu[b] + b: cu[b + 1] + b + 1].contiguous(),
                           draft=case.draft[cu[b]: cu[b + 1]].contiguous(),
                           tokens=case.tokens[cu[b]: cu[b + 1]].contiguous(),
                           uniforms=case.uniforms[cu[b] + b: cu[b + 1] + b + 1].contiguous())
        o1 = run_chain(sub)
        assert int(o1["accepted_len"][0]) == int(out["accepted_len"][b])
        assert int(o1["next_token"][0]) == int(out["next_token"][b])


@pytest.mark.parametrize("probs", [True, False])
def test_chain_edge_cases(probs):
    # 64 sequences x 4 rows x 65536 = 2^24 logits: without probabilities the
    # window is verified in phases
    _say(f"chain edge cases probs={probs}")
    V, K, B = 65536, 3, 64
    g = torch.Generator(device="cuda").manual_seed(3)
    tgt = torch.randn(B * (K + 1), V, generator=g, device="cuda") * 2
    dft = torch.randn(B * K, V, generator=g, device="cuda") * 2
    tok = torch.randint(0, V, (B * K,), generator=g, device="cuda", dtype=torch.int32)
    uni = wl.grid_uniforms((B * (K + 1),), g, "cuda")
    # seq 0: draft equals target -> everything accepted
    dft[0:K] = tgt[0:K]
    # seq 1: bad token at position 1
    tok[K + 1] = V + 5
    # seq 2: NaN target row at position 0
    tgt[2 * (K + 1)] = float("nan")
    # seq 3: -inf except one entry in its target row 1, and a -inf-only draft chunk region
    tgt[3 * (K + 1) + 1] = float("-inf")
    tgt[3 * (K + 1) + 1, 17] = 0.0
    dft[3 * K + 2, :40000] = float("-inf")
    # seq 4: +inf in the extra-token row
    tgt[4 * (K + 1) + K, 5] = float("inf")
    # seq 5: extreme logits (one-pass reference far below the max)
    tgt[5 * (K + 1), 3000] = 400.0
    dft[5 * K, 100] = -300.0
    for dtype in (torch.float32, torch.bfloat16):
        case = wl.ChainCase(B=B, K_max=K, V=V, temperature=1.0, top_k=0, target=tgt.to(dtype),
                            draft=dft.to(dtype), tokens=tok, uniforms=uni)
        out = run_chain(case, probs)
        ref = oracle_chain(case)
        info = compare_chain(out, ref)
        _say(f"  {dtype}: {info} A={out['accepted_len'].tolist()} st={out['status'].tolist()}")
        assert int(out["accepted_len"][0]) == K
        assert int(out["status"][1]) & sd.SEQ_BAD_TOKEN or int(out["accepted_len"][1]) < 1
        assert int(out["status"][2]) & sd.SEQ_NONFINITE and int(out["next_token"][2]) == -1


def test_chain_tiny_vocab_and_k0():
    _say("V=1, K_max=0 and all-zero packed lengths")
    for V in (1, 2, 8):
        for K in (1, 2, 3):
            case = wl.gen_base_noise_chain(1, B=5, K=K, V=V, base_sigma=1.0, noise_sigma=0.5,
                                           temperature=1.0, dtype="f32", device="cuda")
            compare_chain(run_chain(case), oracle_chain(case))
    case = wl.gen_base_noise_chain(2, B=7, K=0, V=300, base_sigma=1.0, noise_sigma=0.5,
                                   temperature=1.0, dtype="bf16", device="cuda")
    compare_chain(run_chain(case), oracle_chain(case))
    case = wl.ragged_chain(3, [0, 0, 0], 500, dtype="bf16", device="cuda")
    compare_chain(run_chain(case), oracle_chain(case))
    case = wl.ragged_chain(4, [1, 2, 3, 2, 1, 0, 9], 700, dtype="bf16", device="cuda")
    compare_chain(run_chain(case), oracle_chain(case))


@pytest.mark.parametrize("mode", ["full", "topk", "greedy"])
def test_chain_window_of_64_positions(mode):
    # K_max = 64, the largest window: its final uniform and extra-token row sit
    # at position 64, past the 64 lanes of the deciding wave
    B, K, V = 3, 64, 600
    T = 0.0 if mode == "greedy" else 1.0
    case = wl.gen_base_noise_chain(41, B=B, K=K, V=V, base_sigma=2.0, noise_sigma=0.5,
                                   temperature=max(T, 1.0), dtype="f32", device="cuda")
    tgt = case.target.view(B, K + 1, V).clone()
    dft = case.draft.view(B, K, V)
    tgt[0, :K] = dft[0]                                   # sequence 0 accepts all 64 drafts
    if mode == "greedy":
        tok = case.tokens.view(B, K).clone()
        tok[0] = torch.argmax(tgt[0, :K], dim=-1).to(torch.int32)
        case.tokens = tok.reshape(-1).contiguous()
    case.target = tgt.reshape(B * (K + 1), V).contiguous()
    case.temperature = T
    case.top_k = 20 if mode == "topk" else 0
    if mode == "topk":
        # sequence 0's drafts must come from the kept set: re-draw them
        g = torch.Generator(device="cuda").manual_seed(3)
        case.tokens = wl.gumbel_draft_tokens(case.draft, 1.0, 20, g)
    out = run_chain(case, probs=mode != "greedy")
    ref = oracle_chain(case)
    compare_chain(out, ref, check_probs=mode != "greedy", check_resid=mode != "greedy")
    assert int(out["accepted_len"][0]) == K


# The largest vocabulary the ABI accepts (V < 2^24): the 16-byte vector path
# (V a multiple of 8) and the element-wise path (odd V), for the stochastic
# chain, greedy verification and the sampled tree walk.
@pytest.mark.parametrize("V", [(1 << 24) - 8, (1 << 24) - 1])
def test_maximum_vocabulary(V):
    B, K = 2, 2
    _say(f"maximum vocabulary V={V}")
    case = wl.gen_base_noise_chain(23, B=B, K=K, V=V, base_sigma=2.0, noise_sigma=0.6,
                                   temperature=1.0, dtype="bf16", device="cuda")
    info = compare_chain(run_chain(case), oracle_chain(case))
    _say(f"  chain {info}")
    # greedy: sequence 0 drafts the target argmax, sequence 1 the draft tokens
    tok = case.tokens.clone()
    rows0 = torch.arange(0, K, device="cuda")
    tok[:K] = wl.first_argmax(case.target.index_select(0, rows0)).to(torch.int32)
    g = sd.verify_greedy(case.target, tok, B=B, K_max=K)
    host = wl.to_host_f32(case.target)
    ref = oracle.verify_greedy(host, tok.cpu().numpy(), None, B, K, V)
    np.testing.assert_array_equal(g["accepted_len"].cpu().numpy(), ref["A"])
    np.testing.assert_array_equal(g["next_token"].cpu().numpy(), ref["next"])
    assert ref["A"][0] == K
    # sampled walk over a two-node tree whose child carries the root row's argmax
    rows = case.target[:2].reshape(1, 2, V).contiguous()
    tree = {"token": torch.tensor([[-1, int(wl.first_argmax(rows[0, :1])[0])]], dtype=torch.int32, device="cuda"),
            "parent": torch.tensor([[-1, 0]], dtype=torch.int32, device="cuda"),
            "n_nodes": torch.tensor([2], dtype=torch.int32, device="cuda")}
    for T in (0.0, 0.05, 1.0):
        u = torch.tensor([[0.25, 0.75]], device="cuda")
        _sampled_walk_check(tree, rows, T, None if T == 0.0 else u)
    del host


# Extreme temperatures: at T = 0.05 the exponent range per row is in the
# hundreds of binary orders (most weights underflow), at T = 8 the weights are
# nearly flat; both through the full-vocabulary chain (one pass and phases),
# the top-k chain and the sampled tree walk.
@pytest.mark.parametrize("T", [0.05, 8.0])
def test_extreme_temperatures(T):
    _say(f"extreme temperature T={T}")
    case = wl.gen_base_noise_chain(29, B=24, K=5, V=40000, base_sigma=2.0, noise_sigma=0.6,
                                   temperature=T, dtype="bf16", device="cuda")
    info = compare_chain(run_chain(case), oracle_chain(case))
    _say(f"  chain {info}")
    tk = wl.gen_topk_chain(device="cuda", seed=31, B=16, K=4, V=30000, top_k=50, temperature=T)
    info = compare_chain(run_chain(tk), oracle_chain(tk))
    _say(f"  top-k {info}")
    tr = wl.gen_tree(device="cuda", seed=33, B=16, K=16, V=32000, N=64)
    tree = sd.build_tree(tr.marginals, 64)
    target = tr.target_for_depths(tree["depth"], tree["n_nodes"])
    u = wl.grid_uniforms((16, 64), torch.Generator(device="cuda").manual_seed(34), "cuda")
    _sampled_walk_check(tree, target, T, u)


# The library only enqueues kernels on the caller's stream (no allocation, no
# synchronisation, no memset), so a step can be captured in a HIP graph. The
# graph is replayed several times, with eager work and synchronisations in
# between, and every replay must equal the eager result.
def test_graph_capture_replays_equal_eager():
    case = wl.gen_adaptive_chain(device="cuda", seed=41, B=64, K=6, V=30000)
    sel0 = sd.select_len(case.conf, case.cost)
    torch.cuda.synchronize()
    packed = case.packed(sel0["k"])
    B, K, V = case.B, case.K_max, case.V
    ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, B, K, V), dtype=torch.uint8, device="cuda")
    tr = wl.gen_tree(device="cuda", seed=42, B=8, K=16, V=20000, N=64)
    ws_b = torch.empty(sd.workspace_bytes(sd.OP_BUILD_TREE, 8, 16, 20000, 0, 64), dtype=torch.uint8,
                       device="cuda")
    tree0 = sd.build_tree(tr.marginals, 64, workspace=ws_b)
    target = tr.target_for_depths(tree0["depth"], tree0["n_nodes"])
    u = wl.grid_uniforms((8, 64), torch.Generator(device="cuda").manual_seed(43), "cuda")

    def step(o):
        s = sd.select_len(case.conf, case.cost, out=o.get("sel"))
        o["sel"] = s
        o["chain"] = sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0,
                                     cu=s["cu"], B=B, K_max=K, workspace=ws, out=o.get("chain"),
                                     validate=False)
        o["tree"] = sd.build_tree(tr.marginals, 64, workspace=ws_b)
        o["walk"] = sd.verify_tree_sampled(target, o["tree"], u, 0.8, out=o.get("walk"))
        return o

    eager = step({})
    torch.cuda.synchronize()
    ref = {k: {kk: vv.clone() for kk, vv in v.items()} for k, v in eager.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(eager)                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = step(eager)
    for rep in range(4):
        for v in cap.values():
            for t in v.values():
                t.fill_(-7)                           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            for kk in ref[k]:
                assert torch.equal(cap[k][kk], ref[k][kk]), (rep, k, kk)
    del g


def test_calls_on_a_side_stream_match_the_current_stream():
    # every call given `stream=` runs there, its internally allocated workspace
    # held for that stream; results equal those of the same calls on the
    # current stream, while the current stream keeps allocating and writing
    case = wl.gen_adaptive_chain(device="cuda", seed=51, B=64, K=6, V=30000)
    tr = wl.gen_tree(device="cuda", seed=52, B=8, K=16, V=20000, N=64)
    gr = wl.gen_greedy_chain(device="cuda", seed=53, B=8, K=3, V=20000)
    _say("side stream: select_len + packed chain, greedy, build_tree")
    packed = case.packed(sd.select_len(case.conf, case.cost)["k"])
    torch.cuda.synchronize()
    B, K = case.B, case.K_max

    def run(stream):
        sel = sd.select_len(case.conf, case.cost, stream=stream)
        ch = sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0, cu=sel["cu"],
                             B=B, K_max=K, stream=stream)
        g = sd.verify_greedy(gr.target, gr.tokens, K_max=gr.K_max, stream=stream)
        t = sd.build_tree(tr.marginals, 64, stream=stream)
        return {"sel": sel, "chain": ch, "greedy": g, "tree": t}

    ref = run(None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    side = run(s)
    junk = [torch.full((1 << 20,), 3, dtype=torch.uint8, device="cuda") for _ in range(16)]
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    del junk
    for k in ref:
        for kk in ref[k]:
            assert torch.equal(side[k][kk], ref[k][kk]), (k, kk)


def test_binding_rejects_unfit_output_tensors():
    # outputs passed in are checked before any launch: a tensor too small, of
    # the wrong type, on the host or not contiguous raises, and the outputs
    # that were given are left as they were
    case = wl.gen_chain_small(device="cuda")
    good = sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, 1.0, B=1, K_max=4)
    A = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    bad = [{"accepted_len": torch.empty(0, dtype=torch.int32, device="cuda")},
           {"accepted_len": torch.empty(1, dtype=torch.int64, device="cuda")},
           {"accepted_len": torch.empty(1, dtype=torch.int32)},
           {"next_token": torch.empty(2, 2, dtype=torch.int32, device="cuda").t()[0]},
           {"accepted_len": A, "probs": torch.empty(3, 2, dtype=torch.float32, device="cuda")}]
    for out in bad:
        with pytest.raises((ValueError, TypeError)):
            sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, 1.0, B=1, K_max=4, out=out,
                            want_probs=True)
    torch.cuda.synchronize()
    assert int(A[0]) == -7
    sel = sd.select_len(case.conf if hasattr(case, "conf") else torch.rand(1, 4, device="cuda"), 0.1)
    with pytest.raises(ValueError):
        sd.select_len(torch.rand(4, 8, device="cuda"), 0.1, out={"cu": torch.empty(4, dtype=torch.int32,
                                                                                       device="cuda")})
    tree_out = {"path": torch.empty(1, 2, dtype=torch.int32, device="cuda")}
    tc = wl.gen_tree(device="cuda", seed=3, B=2, K=2, V=64, N=4)
    tree = sd.build_tree(tc.marginals, 4)
    target = tc.target_for_depths(tree["depth"], tree["n_nodes"])
    with pytest.raises(ValueError):
        sd.verify_tree(target, tree, out=tree_out)
    assert good["accepted_len"].numel() == 1 and int(sel["cu"][0]) == 0


def test_chain_run_twice_bit_identical():
    case = wl.gen_base_noise_chain(9, B=16, K=6, V=50000, base_sigma=2.0, noise_sigma=0.7,
                                   temperature=1.0, dtype="bf16", device="cuda")
    a = run_chain(case)
    b = run_chain(case)
    for k in a:
        assert torch.equal(a[k], b[k]), k


# --------------------------------------------------------------------------
# greedy
# --------------------------------------------------------------------------

def _greedy_ref(case):
    h = subset_host(case, range(case.B))
    return oracle.verify_greedy(h["target"], h["tokens"], h["cu"], case.B, case.K_max, case.V)


def test_greedy_B64_K3_V128256_full():
    _say("greedy chain: B=64 K=3 V=128256 bf16 (all sequences)")
    case = wl.gen_greedy_chain(device="cuda")
    out = sd.verify_greedy(case.target, case.tokens, K_max=case.K_max, B=case.B)
    ref = _greedy_ref(case)
    np.testing.assert_array_equal(out["accepted_len"].cpu().numpy(), ref["A"])
    np.testing.assert_array_equal(out["next_token"].cpu().numpy(), ref["next"])
    np.testing.assert_array_equal(out["status"].cpu().numpy(), ref["status"])
    # the same through sd_verify_chain with T = 0
    o2 = sd.verify_chain(case.target, None, case.tokens, None, 0.0, K_max=case.K_max, B=case.B)
    assert torch.equal(o2["accepted_len"], out["accepted_len"])
    assert torch.equal(o2["next_token"], out["next_token"])
    _say(f"  mean A = {ref['A'].mean():.3f}")


def test_greedy_ties_and_nan():
    V, K, B = 3000, 2, 4
    t = torch.zeros(B * (K + 1), V, device="cuda")
    t[0, [5, 2900, 17]] = 3.0           # tie: lowest id 5
    t[1, :] = float("-inf")             # all -inf: argmax 0
    t[2, :] = float("nan")              # all NaN: no argmax
    t[3, 1000] = float("nan"); t[3, 999] = 1.0
    tok = torch.tensor([5, 0, 1, 0, 0, 0, 0, 0], dtype=torch.int32, device="cuda")
    for dtype in (torch.float32, torch.bfloat16):
        case = wl.GreedyCase(B=B, K_max=K, V=V, target=t.to(dtype), tokens=tok)
        out = sd.verify_greedy(case.target, case.tokens, K_max=K, B=B)
        ref = _greedy_ref(case)
        np.testing.assert_array_equal(out["accepted_len"].cpu().numpy(), ref["A"])
        np.testing.assert_array_equal(out["next_token"].cpu().numpy(), ref["next"])
        np.testing.assert_array_equal(out["status"].cpu().numpy(), ref["status"])


# --------------------------------------------------------------------------
# top-k chain
# --------------------------------------------------------------------------

@pytest.mark.parametrize("top_k,V", [(50, 3000), (1, 2000), (7, 151), (256, 40000), (50, 999)])
def test_topk_small_all_sequences(top_k, V):
    _say(f"top-k {top_k} V={V}")
    case = wl.gen_topk_chain(device="cuda", seed=77 + top_k, B=12, K=4, V=V, top_k=top_k)
    info = compare_chain(run_chain(case), oracle_chain(case))
    _say(f"  {info}")


@pytest.mark.parametrize("top_k", [50, 3])
def test_topk_phased_all_sequences(top_k):
    # 64 x 6 x 50000 >= 2^24 logits: without probabilities, verified in phases
    B, K, V = 64, 5, 50000
    assert B * (K + 1) * V >= 1 << 24
    case = wl.gen_topk_chain(device="cuda", seed=91 + top_k, B=B, K=K, V=V, top_k=top_k)
    one = run_chain(case)
    ph = run_chain(case, probs=False)
    for key in ("accepted_len", "next_token", "status", "resid"):
        assert torch.equal(one[key], ph[key]), key
    info = compare_chain(ph, oracle_chain(case))
    _say(f"  top-k {top_k} phased: {info}")


def test_topk_ties_at_kth_value():
    # many equal bf16 values straddle the k-th position
    V, K, B = 5000, 3, 8
    g = torch.Generator(device="cuda").manual_seed(4)
    base = torch.randint(-4, 5, (B * (K + 1), V), generator=g, device="cuda").float()
    dft = torch.randint(-4, 5, (B * K, V), generator=g, device="cuda").float()
    case = wl.ChainCase(B=B, K_max=K, V=V, temperature=0.8, top_k=50,
                        target=base.to(torch.bfloat16), draft=dft.to(torch.bfloat16),
                        tokens=wl.gumbel_draft_tokens(dft.to(torch.bfloat16), 0.8, 50, g),
                        uniforms=wl.grid_uniforms((B * (K + 1),), g, "cuda"))
    info = compare_chain(run_chain(case), oracle_chain(case))
    _say(f"  ties: {info}")


@pytest.mark.parametrize("layout", ["descending", "ascending", "front_heavy", "strided_top", "constant",
                                    "few_finite"])
def test_topk_structured_rows(layout):
    # Rows whose largest values sit where a threshold guessed from the start of
    # the row is too high (front-heavy, strided) or too low (ascending), or
    # where every value ties or almost every logit is -inf.
    _say(f"top-k structured rows: {layout}")
    V, K, B, top_k = 40000, 2, 4, 50
    R = B * (K + 1)
    g = torch.Generator(device="cuda").manual_seed(11)
    noise = torch.randn(R, V, generator=g, device="cuda")
    ramp = torch.linspace(6.0, -6.0, V, device="cuda")
    if layout == "descending":
        tgt = ramp.expand(R, V) + 0.01 * noise
    elif layout == "ascending":
        tgt = ramp.flip(0).expand(R, V) + 0.01 * noise
    elif layout == "front_heavy":
        tgt = noise.clone()
        tgt[:, :4000] += 8.0
    elif layout == "strided_top":
        # the row's 50 largest values one per 8-token vector at the row's
        # start: a threshold guessed from the start's maxima is too high
        tgt = noise.clone()
        tgt[:, 0:400:8] += 20.0
    elif layout == "constant":
        tgt = torch.full((R, V), 1.5, device="cuda")
    else:
        tgt = torch.full((R, V), float("-inf"), device="cuda")
        tgt[:, 100:130] = noise[:, 100:130]
    tgt = tgt.contiguous().to(torch.bfloat16)
    dft = tgt.view(B, K + 1, V)[:, :K].reshape(B * K, V).contiguous()
    case = wl.ChainCase(B=B, K_max=K, V=V, temperature=1.0, top_k=top_k, target=tgt, draft=dft,
                        tokens=wl.gumbel_draft_tokens(dft, 1.0, top_k, g),
                        uniforms=wl.grid_uniforms((R,), g, "cuda"))
    info = compare_chain(run_chain(case), oracle_chain(case))
    _say(f"  {info}")


def test_topk_chain_B256_K5_V151936_full():
    _say("top-k chain: B=256 K=5 V=151936 bf16 T=0.7 top-k 50 (every sequence)")
    case = wl.gen_topk_chain(device="cuda")
    out = run_chain(case)
    margins = 0
    for g0 in range(0, case.B, 128):
        info = compare_chain(out, oracle_chain(case, range(g0, min(case.B, g0 + 128))))
        margins += info["margin"]
    A = out["accepted_len"].float().mean().item()
    _say(f"  {case.B} sequences, {margins} margin cases checked for validity, mean A={A:.3f}")
    # the benchmark's call (no per-position probabilities): verified in phases
    o2 = run_chain(case, False)
    for key in ("accepted_len", "next_token", "status", "resid"):
        assert torch.equal(o2[key], out[key]), key


# --------------------------------------------------------------------------
# DDTree build and walk
# --------------------------------------------------------------------------

def _tree_compare(out, ref):
    for k in ("token", "parent", "depth", "n_nodes"):
        np.testing.assert_array_equal(out[k].cpu().numpy(), ref[k], err_msg=k)
    np.testing.assert_array_equal(out["anc_mask"].cpu().numpy().view(np.uint64), ref["anc_mask"])
    np.testing.assert_array_equal(out["score"].cpu().numpy(), ref["score"])   # same fp32 products


# (3, 3, ...) and (1, 1, ...): an odd number of rows, so the candidate kernel's
# last workgroup (two rows each) holds one row
@pytest.mark.parametrize("B,K,V,N", [(4, 3, 5, 20), (6, 16, 700, 64), (3, 2, 3, 64), (5, 16, 31, 64),
                                     (2, 1, 1000, 10), (3, 3, 500, 40), (1, 1, 50, 8)])
def test_tree_build_small(B, K, V, N):
    case = wl.gen_tree(device="cuda", seed=5 + V, B=B, K=K, V=V, N=N, sigma=1.5)
    out = sd.build_tree(case.marginals, N)
    ref = oracle.build_tree(wl.to_host_f32(case.marginals), B, K, V, N)
    _tree_compare(out, ref)


# Peaked marginals make deep trees, where a child often beats the next
# sibling: many build rounds of one or two pops each.
@pytest.mark.parametrize("sigma", [4.0, 8.0])
def test_tree_build_deep(sigma):
    B, K, V, N = 16, 16, 2000, 64
    case = wl.gen_tree(device="cuda", seed=17 + int(sigma), B=B, K=K, V=V, N=N, sigma=sigma)
    out = sd.build_tree(case.marginals, N)
    ref = oracle.build_tree(wl.to_host_f32(case.marginals), B, K, V, N)
    _tree_compare(out, ref)
    assert ref["depth"].max() >= 4


def test_tree_build_candidate_overflow():
    """Two heavy tokens per depth: the prefixes scoring at least the depth-1
    list's last entry double at every depth, past what the threshold path
    holds, so these trees come from the pop loop; a flat sequence beside them
    takes the threshold path in the same launch."""
    B, K, V, N = 3, 16, 200, 64
    m = torch.full((B, K, V), 0.1 / (V - 2), device="cuda")
    m[:, :, 3] = 0.45
    m[:, :, 150] = 0.45
    m[2] = torch.softmax(torch.randn(K, V, generator=torch.Generator(device="cuda").manual_seed(4),
                                     device="cuda") * 0.5, dim=-1)
    out = sd.build_tree(m, N)
    ref = oracle.build_tree(m.cpu().numpy(), B, K, V, N)
    _tree_compare(out, ref)
    assert ref["depth"][0].max() >= 5


def test_tree_build_ties():
    B, K, V, N = 3, 4, 40, 30
    m = torch.full((B, K, V), 1.0 / V, device="cuda")        # every score ties
    m[1, :, :8] = 0.05
    out = sd.build_tree(m, N)
    ref = oracle.build_tree(m.cpu().numpy(), B, K, V, N)
    _tree_compare(out, ref)
    # zero marginals, half of them -0 (the products tie with +0 ones): rows
    # with fewer positive entries than the budget
    z = torch.zeros(B, K, V, device="cuda")
    z[:, :, 5:9] = 0.25
    z[:, 1::2, 20:] = -0.0
    z[2, 0] = -0.0
    z[2, 0, 3] = 1.0
    out = sd.build_tree(z, N)
    ref = oracle.build_tree(z.cpu().numpy(), B, K, V, N)
    _tree_compare(out, ref)


# Rows of up to 32768 fp32 marginals take the register-resident top-k (one
# workgroup holds the row); longer rows take the streaming top-k.
@pytest.mark.parametrize("V", [32768, 32767, 32769, 40000])
def test_tree_build_row_length_paths(V):
    B, K, N = 3, 4, 64
    case = wl.gen_tree(device="cuda", seed=9 + V, B=B, K=K, V=V, N=N, sigma=2.5)
    out = sd.build_tree(case.marginals, N)
    ref = oracle.build_tree(wl.to_host_f32(case.marginals), B, K, V, N)
    _tree_compare(out, ref)


def test_tree_build_mass_ties():
    # thousands of equal marginals at the top of a row: more tokens than the
    # short top-k ranks at once reach its first bound, which is then raised
    B, K, V, N = 2, 3, 30000, 64
    g = torch.Generator(device="cuda").manual_seed(3)
    m = torch.rand(B, K, V, generator=g, device="cuda") * 1e-5
    m[0, :, ::7] = 1e-4
    m[1, 1, :] = 1.0 / V
    m[1, 2, 5000:9000] = 2e-4
    out = sd.build_tree(m, N)
    ref = oracle.build_tree(m.cpu().numpy(), B, K, V, N)
    _tree_compare(out, ref)


def test_tree_B32_K16_V32000_N64_full():
    _say("tree: B=32 K=16 V=32000 N=64")
    case = wl.gen_tree(device="cuda")
    tree = sd.build_tree(case.marginals, case.N)
    ref = oracle.build_tree(wl.to_host_f32(case.marginals), case.B, case.K, case.V, case.N)
    _tree_compare(tree, ref)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    walk = sd.verify_tree(target, tree)
    wref = oracle.verify_tree(wl.to_host_f32(target), ref["token"], ref["parent"], ref["n_nodes"],
                              case.B, case.N, case.V)
    np.testing.assert_array_equal(walk["accepted_len"].cpu().numpy(), wref["A"])
    np.testing.assert_array_equal(walk["next_token"].cpu().numpy(), wref["next"])
    np.testing.assert_array_equal(walk["path"].cpu().numpy(), wref["path"])
    _say(f"  mean depth-1 nodes {(ref['depth'] == 1).sum() / case.B:.1f}, mean walk {wref['A'].mean():.2f}")


@pytest.mark.parametrize("row_bytes", [16, 4096, 131072 + 48])
def test_compact_kv_matches_oracle(row_bytes):
    # paths from a real tree walk plus synthetic increasing paths with gaps,
    # chains where each destination is the previous move's source, full-depth
    # and empty paths, and a region past the buffer (left alone)
    g = torch.Generator(device="cuda").manual_seed(17)
    case = wl.gen_tree(device="cuda", seed=23, B=6, K=16, V=3000, N=64, sigma=1.5)
    tree = sd.build_tree(case.marginals, case.N)
    walk = sd.verify_tree(case.target_for_depths(tree["depth"], tree["n_nodes"]), tree)
    B, N = 12, 64
    path = torch.full((B, N), -1, dtype=torch.int32, device="cuda")
    alen = torch.zeros(B, dtype=torch.int32, device="cuda")
    path[:6] = walk["path"]
    alen[:6] = walk["accepted_len"]
    for b in range(6, B):
        A = [0, 5, 20, 63, 17, 9][b - 6]
        nodes = torch.sort(torch.randperm(N - 1, generator=g, device="cuda")[:A] + 1).values
        if b == 8:
            nodes = torch.arange(2, 2 + A, device="cuda")        # each target is the last source
        path[b, :A] = nodes.to(torch.int32)
        alen[b] = A
    n_rows = B * (N - 1) + 40
    base = torch.arange(B, dtype=torch.int64, device="cuda") * (N - 1)
    base[B - 1] = n_rows - (N - 1) + 1                        # one row past the end: untouched
    kv = torch.randint(0, 256, (n_rows, row_bytes), generator=g, device="cuda", dtype=torch.int32)
    kv = kv.to(torch.uint8)
    ref = oracle.compact_kv(kv.cpu().numpy(), base.cpu().numpy(), path.cpu().numpy(),
                            alen.cpu().numpy(), B, N)
    sd.compact_kv(kv, base, path, alen)
    np.testing.assert_array_equal(kv.cpu().numpy(), ref)


def _eagle2_candidates(rng, B, M, layers, topk, V=32000):
    """Expanded candidate trees as an EAGLE-2 drafter would leave them: per
    layer, the topk candidates of the newest layer by cumulative confidence each
    get topk children (conditional probabilities of a random softmax)."""
    par = np.full((B, M), -1, np.int32)
    tok = np.zeros((B, M), np.int32)
    prob = np.zeros((B, M), np.float32)
    n = np.zeros(B, np.int32)
    for b in range(B):
        conf = [1.0]
        par_l, tok_l, prob_l = [-1], [-1], [1.0]
        layer = [0]
        for _ in range(layers):
            grow = sorted(layer, key=lambda c: (-conf[c], c))[:topk]
            layer = []
            for c in grow:
                z = rng.normal(0, 2.0, 64)
                q = np.exp(z - z.max())
                q = (q / q.sum()).astype(np.float32)
                for r in np.argsort(-q, kind="stable")[:topk]:
                    if len(par_l) >= M:
                        break
                    par_l.append(c)
                    tok_l.append(int(rng.integers(0, V)))
                    prob_l.append(float(q[r]))
                    conf.append(float(np.float32(conf[c] * np.float32(q[r]))))
                    layer.append(len(par_l) - 1)
        k = len(par_l)
        par[b, :k], tok[b, :k], prob[b, :k], n[b] = par_l, tok_l, prob_l, k
    return par, tok, prob, n


@pytest.mark.parametrize("M,layers,topk,N", [(400, 6, 8, 64), (1024, 8, 10, 64), (60, 3, 4, 12)])
def test_rerank_tree_matches_oracle(M, layers, topk, N):
    rng = np.random.default_rng(M + N)
    B = 16
    par, tok, prob, n = _eagle2_candidates(rng, B, M, layers, topk)
    par[3, 7] = 9                         # a bad parent and a bad probability drop subtrees
    prob[4, 5] = 1.25
    ref = oracle.rerank_tree(par, tok, prob, n, B, M, N)
    t = lambda a: torch.as_tensor(a, device="cuda")
    out = sd.rerank_tree(t(par), t(tok), t(prob), t(n), N)
    for key in ("token", "parent", "depth", "score", "cand", "n_nodes"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(out["anc_mask"].cpu().numpy().view(np.uint64), ref["anc_mask"])


def test_rerank_tree_ties_and_short_lists():
    """Sequence 0: a full 5-ary tree of four levels with every probability
    0.2, so whole levels tie in confidence and more candidates reach the
    selection bound than it ranks at once (the sort path). Sequence 1: 20
    candidates, fewer than N - 1, some with probability 0 (every candidate
    competes). Sequences 2-3: random expansions (the threshold path)."""
    N, M, B = 64, 1024, 4
    rng = np.random.default_rng(12)
    par, tok, prob, n = _eagle2_candidates(rng, B, M, 6, 8)
    par[0:2], tok[0:2], prob[0:2], n[0:2] = 0, 0, 0.0, 0
    cand = [(-1, 1.0)]
    level = [0]
    for _ in range(4):
        nxt = []
        for c in level:
            for _ in range(5):
                cand.append((c, 0.2))
                nxt.append(len(cand) - 1)
        level = nxt
    n[0] = len(cand)
    for i, (p, q) in enumerate(cand):
        par[0, i], prob[0, i], tok[0, i] = p, q, 1000 + i
    n[1] = 20
    for i in range(1, 20):
        par[1, i], prob[1, i], tok[1, i] = (i - 1) // 3, (0.0 if i % 4 == 0 else 0.3), 50 + i
    par[0, 0] = par[1, 0] = -1
    ref = oracle.rerank_tree(par, tok, prob, n, B, M, N)
    t = lambda a: torch.as_tensor(a, device="cuda")
    out = sd.rerank_tree(t(par), t(tok), t(prob), t(n), N)
    for key in ("token", "parent", "depth", "score", "cand", "n_nodes"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(out["anc_mask"].cpu().numpy().view(np.uint64), ref["anc_mask"])
    assert ref["n_nodes"][0] == N and ref["n_nodes"][1] == 20


def _cand_equal(g, ref, B):
    np.testing.assert_array_equal(g["n_cand"].cpu().numpy(), ref["n_cand"])
    gh = {k: g[k].cpu().numpy() for k in ("parent", "token", "prob", "conf")}
    for b in range(B):
        n = int(ref["n_cand"][b])
        for k in ("parent", "token"):
            np.testing.assert_array_equal(gh[k][b, :n], ref[k][b, :n], err_msg=f"{k} seq {b}")
        for k in ("prob", "conf"):          # bit patterns: NaN, -0 and products exactly
            np.testing.assert_array_equal(gh[k][b, :n].view(np.int32), ref[k][b, :n].view(np.int32),
                                          err_msg=f"{k} seq {b}")


@pytest.mark.parametrize("B,M,W,C,layers,kind", [(32, 1024, 10, 10, 8, "eagle"), (300, 200, 7, 5, 6, "coarse"),
                                                 (5, 1024, 64, 16, 3, "coarse"), (9, 64, 3, 40, 4, "bad")])
def test_expand_tree_matches_oracle(B, M, W, C, layers, kind):
    _say(f"EAGLE-2 expansion B={B} M={M} W={W} C={C} layers={layers} {kind}")
    g = torch.Generator(device="cuda").manual_seed(B + M + W + C)
    if kind == "eagle":
        kids = wl.gen_eagle_children(device="cuda", seed=B, B=B, layers=layers, W=W, C=C)
    else:
        kids = []
        for _ in range(layers):
            ct = torch.randint(0, 1000, (B, W, C), generator=g, device="cuda", dtype=torch.int32)
            cp = torch.randint(0, 9, (B, W, C), generator=g, device="cuda").float() / 8   # ties
            if kind == "bad":      # probabilities outside [0, 1], NaN and -0 (stored, never expanded)
                r = torch.rand(B, W, C, generator=g, device="cuda")
                cp = torch.where(r < 0.1, torch.full_like(cp, float("nan")), cp)
                cp = torch.where((r >= 0.1) & (r < 0.2), cp + 1.5, cp)
                cp = torch.where((r >= 0.2) & (r < 0.3), torch.full_like(cp, -0.0), cp)
            kids.append((ct.contiguous(), cp.contiguous()))
    cand = sd.empty_candidates(B, M)
    ref = oracle.empty_candidates(B, M)
    exp = torch.full((B, W), -1, dtype=torch.int32, device="cuda")
    ref_exp = np.full((B, W), -1, np.int32)
    for layer, (ct, cp) in enumerate(kids):
        if kind == "bad" and layer == 2:   # slots naming nothing, past the candidates, or unusable
            exp[:, 0] = -1
            exp[:, 1] = M + 5
            conf = cand["conf"].cpu().numpy()
            unusable = [int(np.nonzero(conf[b, :int(ref["n_cand"][b])] < 0)[0][0])
                        if (conf[b, :int(ref["n_cand"][b])] < 0).any() else 0 for b in range(B)]
            exp[:, 2] = torch.tensor(unusable, dtype=torch.int32, device="cuda")
            ref_exp = exp.cpu().numpy()
        sd.expand_tree(cand, exp, ct, cp, expand_out=exp)
        ref = oracle.expand_tree(ref, ref_exp, ct.cpu().numpy(), cp.cpu().numpy(), B, M, W, C)
        ref_exp = ref["expand"]
        _cand_equal(cand, ref, B)
        np.testing.assert_array_equal(exp.cpu().numpy(), ref_exp, err_msg=f"expand, layer {layer}")
    N = 64
    out = sd.rerank_tree(cand["parent"], cand["token"], cand["prob"], cand["n_cand"], N)
    rr = oracle.rerank_tree(ref["parent"], ref["token"], ref["prob"], ref["n_cand"], B, M, N)
    for k in ("token", "parent", "depth", "score", "cand", "n_nodes"):
        np.testing.assert_array_equal(out[k].cpu().numpy(), rr[k], err_msg=k)
    np.testing.assert_array_equal(out["anc_mask"].cpu().numpy().view(np.uint64), rr["anc_mask"])
    _say(f"  candidates {int(ref['n_cand'].min())}..{int(ref['n_cand'].max())}, "
         f"tree nodes {int(rr['n_nodes'].min())}..{int(rr['n_nodes'].max())}")


def test_rerank_tree_then_walks():
    """The re-ranked tree has the built tree's layout, so both walks take it:
    target rows that favour each node's children, argmax and sampled walks
    against the oracle on the same tree."""
    rng = np.random.default_rng(7)
    B, M, N, V = 8, 400, 64, 3000
    par, tok, prob, n = _eagle2_candidates(rng, B, M, 6, 8, V=V)
    t = lambda a: torch.as_tensor(a, device="cuda")
    tree = sd.rerank_tree(t(par), t(tok), t(prob), t(n), N)
    g = torch.Generator(device="cuda").manual_seed(11)
    rows = torch.randn(B, N, V, generator=g, device="cuda")
    tk, pr, nn = tree["token"].cpu().numpy(), tree["parent"].cpu().numpy(), tree["n_nodes"].cpu().numpy()
    for b in range(B):
        for c in range(1, int(nn[b])):
            rows[b, int(pr[b, c]), int(tk[b, c])] += 4.0      # children's tokens likely under the target
    rows = rows.to(torch.bfloat16)
    w = sd.verify_tree(rows, tree)
    ref = oracle.verify_tree(wl.to_host_f32(rows), tk, pr, nn, B, N, V)
    np.testing.assert_array_equal(w["accepted_len"].cpu().numpy(), ref["A"])
    np.testing.assert_array_equal(w["path"].cpu().numpy(), ref["path"])
    np.testing.assert_array_equal(w["next_token"].cpu().numpy(), ref["next"])
    u = wl.grid_uniforms((B, N), torch.Generator(device="cuda").manual_seed(12), "cuda")
    _, sref = _sampled_walk_check(tree, rows, 1.0, u)
    assert ref["A"].max() >= 2 and sref["A"].max() >= 1


def test_tree_walk_planted():
    V, N, B = 12, 6, 2
    tok = torch.tensor([[-1, 4, 7, 2, 9, -1]] * B, dtype=torch.int32, device="cuda")
    par = torch.tensor([[-1, 0, 0, 1, 3, -1]] * B, dtype=torch.int32, device="cuda")
    nn = torch.tensor([5, 5], dtype=torch.int32, device="cuda")
    rows = torch.full((B, N, V), -5.0, device="cuda")
    for n, t in enumerate([4, 2, 0, 9, 11, 0]):
        rows[0, n, t] = 5.0
    for n, t in enumerate([3, 0, 0, 0, 0, 0]):
        rows[1, n, t] = 5.0
    out = sd.verify_tree(rows.to(torch.bfloat16), {"token": tok, "parent": par, "n_nodes": nn})
    assert out["accepted_len"].tolist() == [3, 0]
    assert out["next_token"].tolist() == [11, 3]
    assert out["path"][0].tolist()[:4] == [1, 3, 4, -1]


# --------------------------------------------------------------------------
# DDTree walk under a sampling target (rows read on demand, one per step)
# --------------------------------------------------------------------------

def _sampled_walk_check(tree, target, T, u, top_k=0):
    B, N, V = (int(x) for x in target.shape)
    out = sd.verify_tree_sampled(target, tree, u, T, top_k=top_k)
    ref = oracle.verify_tree_sampled(wl.to_host_f32(target), tree["token"].cpu().numpy(),
                                     tree["parent"].cpu().numpy(), tree["n_nodes"].cpu().numpy(),
                                     (u.cpu().numpy() if u is not None else np.zeros((B, N), np.float32)),
                                     B, N, V, T, top_k)
    ok = ref["margin"] == 0
    for kg, kr in (("accepted_len", "A"), ("next_token", "next"), ("status", "status")):
        got = out[kg].cpu().numpy()
        bad = np.nonzero(ok & (got != ref[kr]))[0]
        assert len(bad) == 0, f"{kg}: seqs {bad[:5]} gpu {got[bad[:5]]} oracle {ref[kr][bad[:5]]}"
    np.testing.assert_array_equal(out["path"].cpu().numpy()[ok], ref["path"][ok])
    if (~ok).any():
        # margin cases: the GPU's walk must be one that rounding allows (every
        # committed token inside its node's fp64 CDF interval widened by 1e-6)
        valid = oracle.check_tree_sampled(wl.to_host_f32(target), tree["token"].cpu().numpy(),
                                          tree["parent"].cpu().numpy(), tree["n_nodes"].cpu().numpy(),
                                          u.cpu().numpy(), B, N, V, T, out["path"].cpu().numpy(),
                                          out["accepted_len"].cpu().numpy(),
                                          out["next_token"].cpu().numpy(), top_k=top_k)
        bad = np.nonzero(~ok & (valid != 1))[0]
        assert len(bad) == 0, f"margin walks not allowed by rounding: seqs {bad[:5]}"
    return out, ref


@pytest.mark.parametrize("dtype,V,T", [("bf16", 32000, 1.0), ("bf16", 32000, 0.3), ("bf16", 70000, 0.8),
                                       ("bf16", 32001, 0.6), ("f32", 40000, 1.2), ("f32", 999, 0.5),
                                       ("bf16", 8, 1.0)])
def test_tree_walk_sampled_matches_oracle(dtype, V, T):
    B, K, N = 24, 16, 64
    _say(f"sampled walk {dtype} V={V} T={T}")
    case = wl.gen_tree(device="cuda", seed=31 + V, B=B, K=K, V=V, N=N)
    tree = sd.build_tree(case.marginals, N)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    if dtype == "f32":
        target = target.float()
    u = wl.grid_uniforms((B, N), torch.Generator(device="cuda").manual_seed(V), "cuda")
    out, ref = _sampled_walk_check(tree, target, T, u)
    _say(f"  mean walk {ref['A'].mean():.2f}, max {ref['A'].max()}, margin {int((ref['margin'] != 0).sum())}")


# Top-k truncation inside the sampled walk: every node row is reduced to its
# kept list first (ties at the k-th value keep the lower ids).
@pytest.mark.parametrize("dtype,V,T,top_k", [("bf16", 32000, 1.0, 50), ("bf16", 32001, 0.7, 256),
                                             ("f32", 20000, 1.3, 1), ("bf16", 60, 1.0, 50),
                                             ("f32", 999, 0.5, 7)])
def test_tree_walk_sampled_topk_matches_oracle(dtype, V, T, top_k):
    B, K, N = 24, 16, 64
    _say(f"sampled walk top-k {top_k} {dtype} V={V} T={T}")
    case = wl.gen_tree(device="cuda", seed=37 + V, B=B, K=K, V=V, N=N)
    tree = sd.build_tree(case.marginals, N)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    if dtype == "f32":
        target = target.float()
    u = wl.grid_uniforms((B, N), torch.Generator(device="cuda").manual_seed(V + top_k), "cuda")
    out, ref = _sampled_walk_check(tree, target, T, u, top_k=top_k)
    if top_k == 1:                 # one kept id: the argmax walk for every uniform
        g = sd.verify_tree(target, tree)
        assert torch.equal(out["path"], g["path"]) and torch.equal(out["next_token"], g["next_token"])
    _say(f"  mean walk {ref['A'].mean():.2f}, margin {int((ref['margin'] != 0).sum())}")


# The top-k walk holds a row of up to 4096 16-byte vectors in registers (bf16
# V <= 32768, fp32 V <= 16384) and streams longer rows; a tile whose bound
# admits too many candidates (heavy ties) is streamed too. Each case checks one
# side of those limits: the largest tiles and one vector past them, rows of
# negative log-probabilities, coarse ties, and flat rows (every id tied).
@pytest.mark.parametrize("dtype,V,top_k,kind", [("bf16", 32768, 50, "normal"), ("bf16", 32776, 50, "normal"),
                                                ("f32", 16384, 20, "normal"), ("f32", 16388, 20, "normal"),
                                                ("bf16", 32000, 50, "logprob"), ("bf16", 32000, 200, "coarse"),
                                                ("f32", 8000, 64, "flat"), ("bf16", 32000, 256, "flat")])
def test_tree_walk_sampled_topk_tile_limits(dtype, V, top_k, kind):
    B, K, N = 16, 16, 64
    _say(f"sampled walk top-k {top_k} {dtype} V={V} rows {kind}")
    case = wl.gen_tree(device="cuda", seed=91 + V + top_k, B=B, K=K, V=V, N=N)
    tree = sd.build_tree(case.marginals, N)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"]).float()
    if kind == "logprob":
        target = torch.log_softmax(target, dim=-1)
    elif kind == "coarse":
        target = torch.round(target * 2.0) / 2.0
    elif kind == "flat":
        target[0::2] = 0.0             # even sequences: every row one tied value
    target = target.to(torch.bfloat16) if dtype == "bf16" else target
    u = wl.grid_uniforms((B, N), torch.Generator(device="cuda").manual_seed(V + 3), "cuda")
    out, ref = _sampled_walk_check(tree, target, 1.0, u, top_k=top_k)
    _say(f"  mean walk {ref['A'].mean():.2f}, margin {int((ref['margin'] != 0).sum())}")


def test_tree_walk_sampled_topk_ties_and_nonfinite():
    V, N, B = 12, 6, 3
    tok = torch.tensor([[-1, 4, 7, 2, 9, -1]] * B, dtype=torch.int32, device="cuda")
    par = torch.tensor([[-1, 0, 0, 1, 3, -1]] * B, dtype=torch.int32, device="cuda")
    nn = torch.tensor([5] * B, dtype=torch.int32, device="cuda")
    rows = torch.zeros((B, N, V), device="cuda")
    rows[:, :, 4] = 1.0                 # row max at id 4 ...
    rows[:, :, 7] = 1.0                 # ... tied with id 7: top-1 keeps id 4
    rows[1, 1, :] = float("nan")        # sequence 1: no kept finite entry at node 1
    rows[2, 0, 3] = float("inf")        # sequence 2: an infinite maximum at the root
    tree = {"token": tok, "parent": par, "n_nodes": nn}
    u = torch.full((B, N), 0.9, device="cuda")
    out = sd.verify_tree_sampled(rows, tree, u, 1.0, top_k=1)
    ref = oracle.verify_tree_sampled(rows.cpu().numpy(), tok.cpu().numpy(), par.cpu().numpy(),
                                     nn.cpu().numpy(), u.cpu().numpy(), B, N, V, 1.0, 1)
    for kg, kr in (("accepted_len", "A"), ("next_token", "next"), ("status", "status")):
        np.testing.assert_array_equal(out[kg].cpu().numpy(), ref[kr], err_msg=kg)
    assert out["accepted_len"].tolist()[0] == 1 and out["status"].tolist() == [0, 2, 2]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tree_walk_sampled_topk_rows_mostly_neg_inf(dtype):
    # rows of -inf but for 30 finite logits, top-k 50: the kept set holds the 30
    # and 20 of the -inf entries (lowest ids); the register tile's bound sits
    # at -inf there
    V, N, B = 4096, 6, 4
    g = torch.Generator(device="cuda").manual_seed(21)
    tok = torch.tensor([[-1, 104, 117, 110, 121, -1]] * B, dtype=torch.int32, device="cuda")
    par = torch.tensor([[-1, 0, 0, 1, 3, -1]] * B, dtype=torch.int32, device="cuda")
    nn = torch.tensor([5] * B, dtype=torch.int32, device="cuda")
    rows = torch.full((B, N, V), float("-inf"), device="cuda")
    rows[:, :, 100:130] = torch.randn(B, N, 30, generator=g, device="cuda")
    rows[:, :, 104] += 2.0
    rows = rows.to(dtype)
    tree = {"token": tok, "parent": par, "n_nodes": nn}
    u = wl.grid_uniforms((B, N), g, "cuda")
    out, ref = _sampled_walk_check(tree, rows, 1.0, u, top_k=50)
    assert (out["status"] == 0).all()


def test_tree_walk_sampled_T0_is_the_argmax_walk():
    case = wl.gen_tree(device="cuda", seed=77, B=16, K=16, V=32000, N=64)
    tree = sd.build_tree(case.marginals, 64)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    for tgt in (target, target.float()):
        out, _ = _sampled_walk_check(tree, tgt, 0.0, None)
        ref = sd.verify_tree(tgt, tree)
        for k in ("path", "accepted_len", "next_token"):
            assert torch.equal(out[k], ref[k]), k


def test_tree_sampled_walk_B32_V32000_full():
    _say("sampled tree walk: B=32 K=16 V=32000 N=64 T=1")
    case = wl.gen_tree(device="cuda")
    tree = sd.build_tree(case.marginals, case.N)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    u = wl.grid_uniforms((case.B, case.N), torch.Generator(device="cuda").manual_seed(1004), "cuda")
    out, ref = _sampled_walk_check(tree, target, 1.0, u)
    _say(f"  mean walk {ref['A'].mean():.2f}")


def test_tree_walk_sampled_nonfinite_and_planted():
    V, N, B = 12, 6, 3
    tok = torch.tensor([[-1, 4, 7, 2, 9, -1]] * B, dtype=torch.int32, device="cuda")
    par = torch.tensor([[-1, 0, 0, 1, 3, -1]] * B, dtype=torch.int32, device="cuda")
    nn = torch.tensor([5] * B, dtype=torch.int32, device="cuda")
    rows = torch.full((B, N, V), float("-inf"), device="cuda")
    for b in range(B):
        for n, t in enumerate([4, 2, 0, 9, 11, 0]):
            rows[b, n, t] = 0.0                        # one-hot p: the draw is certain
    rows[1, 3, :] = float("nan")                       # sequence 1 meets a NaN row at node 3
    rows[2, 0, :] = float("inf")                       # sequence 2: no finite maximum at the root
    u = torch.full((B, N), 0.5, device="cuda")
    tree = {"token": tok, "parent": par, "n_nodes": nn}
    out = sd.verify_tree_sampled(rows, tree, u, 0.9)
    assert out["accepted_len"].tolist() == [3, 2, 0]
    assert out["next_token"].tolist() == [11, -1, -1]
    assert out["status"].tolist() == [0, 2, 2]
    assert out["path"][0].tolist()[:4] == [1, 3, 4, -1]


def test_gpu_sampled_walk_tokens_follow_target():
    """One call over 2^18 copies of a small tree: the committed tokens follow
    the target's rows (first token ~ p_root; second ~ p_child given the child)."""
    from scipy import stats
    P = np.array([[.1, .4, .2, .3], [.5, .1, .3, .1], [.25, .25, .25, .25],
                  [.2, .6, .1, .1], [.7, .1, .1, .1], [.1, .1, .1, .7]])
    tok0 = [-1, 1, 3, 0, 2, 1]
    par0 = [-1, 0, 0, 1, 1, 3]
    n, N, V = 1 << 18, 6, 4
    rows = torch.log(torch.tensor(P, dtype=torch.float32, device="cuda"))[None].expand(n, N, V).contiguous()
    tree = {"token": torch.tensor([tok0] * n, dtype=torch.int32, device="cuda"),
            "parent": torch.tensor([par0] * n, dtype=torch.int32, device="cuda"),
            "n_nodes": torch.full((n,), N, dtype=torch.int32, device="cuda")}
    u = wl.grid_uniforms((n, N), torch.Generator(device="cuda").manual_seed(99), "cuda")
    out = sd.verify_tree_sampled(rows, tree, u, 1.0)
    A = out["accepted_len"].cpu().numpy()
    path = out["path"].cpu().numpy()
    nxt = out["next_token"].cpu().numpy()
    tk = np.array(tok0)
    first = np.where(A >= 1, tk[np.maximum(path[:, 0], 0)], nxt)
    assert stats.chisquare(np.bincount(first, minlength=V), P[0] * n).pvalue >= 1e-3
    for c in (1, 2):
        sel = (A >= 1) & (path[:, 0] == c)
        second = np.where(A[sel] >= 2, tk[np.maximum(path[sel, 1], 0)], nxt[sel])
        assert stats.chisquare(np.bincount(second, minlength=V), P[c] * sel.sum()).pvalue >= 1e-3


# --------------------------------------------------------------------------
# DSpark length selection and the packed verify of the selected windows
# --------------------------------------------------------------------------

def test_select_len_parity():
    g = torch.Generator(device="cuda").manual_seed(8)
    # up to 8192 sequences one workgroup; beyond, one thread per sequence and a scan workgroup
    for B, K, cost in ((512, 8, 0.15), (3, 64, 0.01), (1000, 5, 0.5), (700, 0, 0.1), (8192, 8, 0.15),
                       (8193, 8, 0.15), (300001, 8, 0.15), (1 << 20, 3, 0.3), (20000, 0, 0.1)):
        conf = torch.sort(torch.rand(B, K, 6, generator=g, device="cuda"), dim=-1).values[..., 4].contiguous() \
            if K > 0 else torch.zeros(B, 0, device="cuda")
        out = sd.select_len(conf, cost)
        ref = oracle.select_len(conf.cpu().numpy(), B, K, cost)
        np.testing.assert_array_equal(out["k"].cpu().numpy(), ref["k"])
        np.testing.assert_array_equal(out["cu"].cpu().numpy(), ref["cu"])
        np.testing.assert_allclose(out["adv"].cpu().numpy(), ref["adv"], rtol=1e-5)


def test_select_len_table_parity():
    g = torch.Generator(device="cuda").manual_seed(9)
    for B, K in ((512, 8), (5, 64), (300, 3), (40, 0), (70000, 8)):
        conf = torch.sort(torch.rand(B, K, 6, generator=g, device="cuda"), dim=-1).values[..., 4].contiguous() \
            if K > 0 else torch.zeros(B, 0, device="cuda")
        table = (torch.rand(max(K, 1), generator=g, device="cuda") * 0.4).contiguous()
        out = sd.select_len_table(conf, table)
        ref = oracle.select_len_table(conf.cpu().numpy(), B, K, table.cpu().numpy())
        np.testing.assert_array_equal(out["k"].cpu().numpy(), ref["k"])
        np.testing.assert_array_equal(out["cu"].cpu().numpy(), ref["cu"])
        np.testing.assert_allclose(out["adv"].cpu().numpy(), ref["adv"], rtol=1e-5)
        # a constant table selects what the scalar call selects
        flat = torch.full((max(K, 1),), 0.15, device="cuda")
        a = sd.select_len_table(conf, flat)["k"].cpu().numpy()
        b = sd.select_len(conf, 0.15)["k"].cpu().numpy()
        np.testing.assert_array_equal(a, b)


def _padded_case(mode, seed):
    if mode == "topk":
        return wl.gen_topk_chain(device="cuda", seed=seed, B=48, K=6, V=30000, top_k=20)
    if mode == "greedy":
        g = wl.gen_greedy_chain(device="cuda", seed=seed, B=48, K=6, V=30000)
        return wl.ChainCase(B=g.B, K_max=g.K_max, V=g.V, temperature=0.0, top_k=0, target=g.target,
                            draft=None, tokens=g.tokens, uniforms=None)
    return wl.gen_base_noise_chain(seed, B=48, K=6, V=30000, base_sigma=2.0, noise_sigma=0.7,
                                   temperature=1.0, dtype="bf16", device="cuda")


@pytest.mark.parametrize("mode", ["full", "topk", "greedy"])
def test_capped_commits_what_compact_commits(mode):
    _say(f"cap-accept vs compact ({mode})")
    case = _padded_case(mode, 31)
    B, K, V = case.B, case.K_max, case.V
    g = torch.Generator(device="cuda").manual_seed(12)
    cap = torch.randint(0, K + 1, (B,), generator=g, device="cuda", dtype=torch.int32)
    cap[:3] = torch.tensor([-2, K + 5, K], dtype=torch.int32)      # clamped to [0, K]
    greedy = case.temperature == 0.0
    out = sd.verify_chain_capped(case.target, case.draft, case.tokens.view(B, K), case.uniforms, cap,
                                 case.temperature, top_k=case.top_k, want_probs=not greedy,
                                 want_resid=not greedy)
    # compact: the first kc positions only (rows gathered as an engine would)
    kc = cap.clamp(0, K).long()
    ar_d, ar_t = torch.arange(K, device="cuda"), torch.arange(K + 1, device="cuda")
    dmask = (ar_d[None, :] < kc[:, None]).reshape(-1)
    tmask = (ar_t[None, :] <= kc[:, None]).reshape(-1)
    cu = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    cu[1:] = torch.cumsum(kc, 0).to(torch.int32)
    packed = wl.ChainCase(B=B, K_max=K, V=V, temperature=case.temperature, top_k=case.top_k,
                          target=case.target[tmask].contiguous(),
                          draft=None if greedy else case.draft[dmask].contiguous(),
                          tokens=case.tokens[dmask].contiguous(),
                          uniforms=None if greedy else case.uniforms[tmask].contiguous(), cu=cu)
    comp = sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms,
                           case.temperature, top_k=case.top_k, cu=cu, B=B, K_max=K)
    for key in ("accepted_len", "next_token", "status"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), comp[key].cpu().numpy(), err_msg=key)
    full = sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, case.temperature,
                           top_k=case.top_k, B=B, K_max=K)
    np.testing.assert_array_equal(out["accepted_full"].cpu().numpy(), full["accepted_len"].cpu().numpy())
    # and the oracle's cap-accept verification
    t = wl.to_host_f32(case.target)
    if greedy:
        ref = oracle.verify_chain_capped(t, np.zeros((B * K, V), np.float32), case.tokens.cpu().numpy(),
                                         np.zeros(B * (K + 1), np.float32), cap.cpu().numpy(), B, K, V,
                                         0.0)
    else:
        ref = oracle.verify_chain_capped(t, wl.to_host_f32(case.draft), case.tokens.cpu().numpy(),
                                         case.uniforms.cpu().numpy(), cap.cpu().numpy(), B, K, V,
                                         case.temperature, case.top_k)
    ok = ref["margin"] == 0
    for key, rk in (("accepted_len", "A"), ("next_token", "next"), ("accepted_full", "A_full")):
        got = out[key].cpu().numpy()
        assert (got[ok] == ref[rk][ok]).all(), (key, np.nonzero(got[ok] != ref[rk][ok]))
    if not greedy and (~ok).any():
        # margin cases: the committed result must be one that rounding allows
        # on the compact window, and the full-window rejection on the whole one
        valid, st_exp = oracle.check_chain(wl.to_host_f32(packed.target), wl.to_host_f32(packed.draft),
                                           packed.tokens.cpu().numpy(), packed.uniforms.cpu().numpy(),
                                           cu.cpu().numpy(), B, K, V, case.temperature,
                                           out["accepted_len"].cpu().numpy(),
                                           out["next_token"].cpu().numpy(), top_k=case.top_k)
        assert (valid[~ok] == 3).all() and (st_exp[~ok] == out["status"].cpu().numpy()[~ok]).all()
        valid, _ = oracle.check_chain(t, wl.to_host_f32(case.draft), case.tokens.cpu().numpy(),
                                      case.uniforms.cpu().numpy(), None, B, K, V, case.temperature,
                                      out["accepted_full"].cpu().numpy(), full["next_token"].cpu().numpy(),
                                      top_k=case.top_k)
        assert ((valid[~ok] & oracle.CHECK_A) != 0).all()
    if not greedy:
        good, worst = close_rel(out["probs"].cpu().numpy(), ref["probs"])
        assert good, worst
    _say(f"  margin cases {int((~ok).sum())}, mean committed {out['accepted_len'].float().mean().item():.2f}")


def test_adaptive_chain_B512_K8_V128256_sampled():
    _say("adaptive chain: select_len + packed chain B=512 K_max=8 V=128256 bf16 (sampled)")
    case = wl.gen_adaptive_chain(device="cuda")
    sel = sd.select_len(case.conf, case.cost)
    ref_sel = oracle.select_len(case.conf.cpu().numpy(), case.B, case.K_max, case.cost)
    np.testing.assert_array_equal(sel["k"].cpu().numpy(), ref_sel["k"])
    np.testing.assert_array_equal(sel["cu"].cpu().numpy(), ref_sel["cu"])
    np.testing.assert_allclose(sel["adv"].cpu().numpy(), ref_sel["adv"], rtol=1e-5)
    packed = case.packed(sel["k"])
    # launch exactly as the benchmark does: device cu from select_len, no host read
    out = sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0,
                          cu=sel["cu"], B=case.B, K_max=case.K_max, want_probs=True,
                          want_resid=True, validate=False)
    # every sequence, in groups of 128 (host copies of about 0.7 GB each)
    margins = 0
    for g0 in range(0, case.B, 128):
        info = compare_chain(out, oracle_chain(packed, range(g0, min(case.B, g0 + 128))))
        margins += info["margin"]
    _say(f"  {case.B} sequences, {margins} margin cases checked for validity, "
         f"E[k*]={ref_sel['k'].mean():.3f} mean A={out['accepted_len'].float().mean().item():.3f}")
    # the benchmark's own call: no per-position probabilities, so positions are
    # verified in phases; the decisions are those of the one-phase call
    o2 = sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0,
                         cu=sel["cu"], B=case.B, K_max=case.K_max, want_resid=True, validate=False)
    for key in ("accepted_len", "next_token", "status"):
        assert torch.equal(o2[key], out[key]), key
    np.testing.assert_array_equal(o2["resid"].cpu().numpy(), out["resid"].cpu().numpy())


# --------------------------------------------------------------------------
# distribution: chi-square on a large batch of tiny-vocabulary sequences
# --------------------------------------------------------------------------

def test_gpu_chi_square_tokens_follow_target():
    from scipy import stats
    P = np.array([[.05, .15, .5, .3, 0, 0], [.6, .1, .1, .1, .05, .05], [0, 0, 0, .5, .5, 0],
                  [.3, .3, .1, .1, .1, .1]])
    Q = np.array([[1 / 6] * 6, [.5, .5, 0, 0, 0, 0], [0, 0, .2, .2, .3, .3]])
    K, V, n = 3, 6, 1 << 18
    with np.errstate(divide="ignore"):
        lp = torch.tensor(np.log(P), dtype=torch.float32, device="cuda")
        lq = torch.tensor(np.log(Q), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(99)
    tgt = lp.repeat(n, 1).contiguous()
    dft = lq.repeat(n, 1).contiguous()
    y = torch.stack([torch.multinomial(torch.tensor(Q[i], device="cuda", dtype=torch.float32), n,
                                       replacement=True, generator=g) for i in range(K)], 1)
    tok = y.to(torch.int32).reshape(-1).contiguous()
    uni = wl.grid_uniforms((n * (K + 1),), g, "cuda")
    out = sd.verify_chain(tgt, dft, tok, uni, 1.0, K_max=K, B=n)
    A = out["accepted_len"].cpu().numpy()
    nx = out["next_token"].cpu().numpy()
    yk = y.cpu().numpy()
    for j in range(K + 1):
        reach = A >= j
        if reach.sum() < 5000:
            continue
        t = np.where(A[reach] > j, yk[reach][:, j] if j < K else -1, nx[reach])
        obs = np.bincount(t, minlength=V)
        z = P[j] == 0
        assert obs[z].sum() == 0
        pv = stats.chisquare(obs[~z], P[j][~z] * reach.sum()).pvalue
        _say(f"  position {j}: n={reach.sum()} p-value {pv:.3g}")
        assert pv >= 1e-3
