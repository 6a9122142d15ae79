#!/usr/bin/env python3
"""Benchmark of the verify hot path on one MI355X.

Default workload (the one the headline metric is quoted on, V = 128256 bf16):
DSpark-style adaptive chain verification. One step is the whole path over one
batch: sd_select_len on the per-position confidences (B = 512, K_max = 8,
cost 0.15 per position), then a packed stochastic sd_verify_chain (T = 1) over
the selected windows only, with the packed offsets read by the kernels from
device memory (no host round trip). Inputs are seeded synthetic arrays already
resident in HBM when timing starts.

Printed: one JSON line with the throughput in verified draft positions per
second, the roofline of the dominant kernel (the streaming pass over the logit
rows, timed with HIP events on its own stream), the CPU oracle timed on a
bounded sample of the same workload, and the parity of the timed step against
that oracle run (verify lengths of every sequence, committed results of the
sampled sequences; bit-exact outside the oracle's margin cases).

Other workloads (--workload greedy|topk|tree|tree_sampled|tree_sampled_topk|chain1|kv|rerank)
measure the other kernels
for the design notes; their inputs are rotated across copies so that the
working set exceeds the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak), V=128256 bf16"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (string
    and character literals kept), so that a comment edit keeps the digest."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest() -> str:
    """Digest of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rejection_sampling_verify_softmax_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy-kernel calibration), if recorded for the
    current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = source_digest()
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = dict(kv.split("=", 1) for kv in line.split())
        if f.get("kernel") == kernel and f.get("workload") == workload and f.get("sources") == digest:
            return float(f["bytes_per_launch"])
    return None


# --------------------------------------------------------------------------
# workloads: each returns (step_fn, meta) where step_fn(i, timer_events) runs
# one step on the current stream.
# --------------------------------------------------------------------------

def setup_adaptive(torch, sd, wl):
    import numpy as np

    case = wl.gen_adaptive_chain(device="cuda")
    sel = sd.select_len(case.conf, case.cost)
    torch.cuda.synchronize()
    packed = case.packed(sel["k"])
    B, K, V = case.B, case.K_max, case.V
    positions = int(sel["cu"][-1].item())
    R_d, R_t = positions, positions + B
    out = {k: v for k, v in sd.verify_chain(packed.target, packed.draft, packed.tokens,
                                            packed.uniforms, 1.0, cu=sel["cu"], B=B, K_max=K,
                                            validate=True).items()}
    ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, B, K, V), dtype=torch.uint8, device="cuda")
    sel_out = {"k": sel["k"], "adv": sel["adv"], "cu": sel["cu"]}
    # Rows the verification streams: positions 0 and 1 (and the extra-token
    # row of a shorter draft) of every sequence in the first phase, the rest of
    # the window only for sequences whose first two drafts were both accepted.
    k_sel = sel["k"].cpu().numpy().astype(np.int64)
    A = out["accepted_len"].cpu().numpy().astype(np.int64)
    split = 2
    t1, d1 = np.minimum(k_sel + 1, split), np.minimum(k_sel, split)
    alive = (k_sel >= split) & (A >= split)
    t2 = np.where(alive, k_sel + 1 - split, 0)
    d2 = np.where(alive, k_sel - split, 0)
    rows1, rows2 = int(t1.sum() + d1.sum()), int(t2.sum() + d2.sum())
    stats_bytes = rows1 * V * 2 + int(d1.sum()) * 4           # first-phase rows once + draft tokens
    step_bytes = ((rows1 + rows2) * V * 2 + R_d * 4 + R_t * 4  # rows streamed, tokens, uniforms
                  + B * K * 4 + B * (4 + 4 + 4) + (B + 1) * 4  # conf in; k, adv, cu out
                  + B * 12)                                    # A, next, status out

    def step(ev=None):
        s = sd.select_len(case.conf, case.cost, out=sel_out)
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0,
                        cu=s["cu"], B=B, K_max=K, workspace=ws, out=out, validate=False)

    meta = {
        "workload": (f"DSpark-adaptive chain verify: select_len (Beta(5,2) confidences, cost 0.15) "
                     f"+ packed stochastic verify over the selected windows, B={B}, K_max={K}, "
                     f"V={V}, bf16 logits, T=1.0"),
        "global_batch": B, "K_max": K, "V": V, "logits": "bf16", "temperature": 1.0,
        "positions_per_step": positions, "target_rows": R_t, "draft_rows": R_d,
        "kernel": "k_chain_stats", "kernel_bytes": stats_bytes, "step_bytes": step_bytes,
        "mean_k": positions / B, "mean_A": float(A.mean()),
        "rows_streamed": rows1 + rows2, "rows_in_windows": R_t + R_d,
    }
    cpu = {"case": case, "packed": packed, "k": sel["k"].cpu().numpy(), "cu": sel["cu"].cpu().numpy(),
           "out": out}
    return step, meta, cpu


def setup_greedy(torch, sd, wl):
    case = wl.gen_greedy_chain(device="cuda")
    B, K, V = case.B, case.K_max, case.V
    copies = [case.target] + [case.target.clone() for _ in range(7)]    # 8 x 66 MB > LLC
    ws = torch.empty(sd.workspace_bytes(sd.OP_GREEDY, B, K, V), dtype=torch.uint8, device="cuda")
    st = {"i": 0}

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        t = copies[st["i"] % len(copies)]
        st["i"] += 1
        sd.verify_greedy(t, case.tokens, B=B, K_max=K, workspace=ws)

    rows = B * (K + 1)
    meta = {"workload": f"greedy chain verify B={B} K={K} V={V} bf16 (8 rotated input copies)",
            "global_batch": B, "K_max": K, "V": V, "positions_per_step": B * K,
            "kernel": "k_argmax", "kernel_bytes": rows * V * 2, "step_bytes": rows * V * 2 + B * K * 4}
    return step, meta, None


def setup_topk(torch, sd, wl):
    case = wl.gen_topk_chain(device="cuda")
    B, K, V = case.B, case.K_max, case.V
    ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, B, K, V, case.top_k), dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, case.temperature,
                        top_k=case.top_k, B=B, K_max=K, workspace=ws, validate=False)

    # rows streamed: slots 0-1 of every sequence, the rest only where both
    # first drafts were accepted (as in the adaptive workload)
    A = sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, case.temperature,
                        top_k=case.top_k, B=B, K_max=K, workspace=ws)["accepted_len"].cpu()
    split = 2
    rows1 = B * (split + split)
    alive = int((A >= split).sum())
    rows2 = alive * ((K + 1 - split) + (K - split))
    meta = {"workload": f"top-k chain verify B={B} K={K} V={V} bf16 T=0.7 top-k 50",
            "global_batch": B, "K_max": K, "V": V, "positions_per_step": B * K,
            "kernel": "k_topk_rows", "kernel_bytes": rows1 * V * 2,
            "step_bytes": (rows1 + rows2) * V * 2 + B * K * 4 + B * (K + 1) * 4,
            "mean_A": float(A.float().mean()), "rows_streamed": rows1 + rows2,
            "rows_in_windows": B * (K + 1) + B * K}
    return step, meta, None


def setup_tree(torch, sd, wl):
    case = wl.gen_tree(device="cuda")
    B, K, V, N = case.B, case.K, case.V, case.N
    tree = sd.build_tree(case.marginals, N)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    # 8 copies: 8 x 65.5 MB of marginals pass between two uses of one copy, more
    # than the 256 MB last-level cache, so neither the marginals nor the few
    # target rows a walk visits are still cached when their copy comes round
    margs = [case.marginals] + [case.marginals.clone() for _ in range(7)]
    targets = [target] + [target.clone() for _ in range(7)]
    st = {"i": 0}
    ws_b = torch.empty(sd.workspace_bytes(sd.OP_BUILD_TREE, B, K, V, 0, N), dtype=torch.uint8, device="cuda")
    walk_out = sd.verify_tree(target, tree)
    A = walk_out["accepted_len"].cpu()
    rows_read = int(A.sum()) + B              # the walk reads the rows on its path only

    def step(ev=None):
        i = st["i"] % len(margs)
        st["i"] += 1
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.build_tree(margs[i], N, workspace=ws_b)
        sd.verify_tree(targets[i], tree, out=walk_out)

    meta = {"workload": (f"DDTree build (B={B}, K={K}, V={V} fp32 marginals, N={N}) + argmax walk over "
                         f"bf16 target rows (read on demand)"),
            "global_batch": B, "K_max": K, "V": V, "positions_per_step": B * (N - 1),
            "kernel": "k_topk_short<f32>", "kernel_bytes": B * K * V * 4,
            "step_bytes": B * K * V * 4 + rows_read * V * 2, "mean_A": float(A.float().mean()),
            "rows_streamed": rows_read}
    return step, meta, None


def setup_tree_sampled(torch, sd, wl):
    # the tree workload's build, then the walk under a sampling target (T = 1):
    # at each node the target draws its own token; only the walk's rows are read
    case = wl.gen_tree(device="cuda")
    B, K, V, N = case.B, case.K, case.V, case.N
    tree = sd.build_tree(case.marginals, N)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    u = wl.grid_uniforms((B, N), torch.Generator(device="cuda").manual_seed(1004), "cuda")
    # 8 copies: 8 x 65.5 MB of marginals pass between two uses of one copy, more
    # than the 256 MB last-level cache, so neither the marginals nor the few
    # target rows a walk visits are still cached when their copy comes round
    margs = [case.marginals] + [case.marginals.clone() for _ in range(7)]
    targets = [target] + [target.clone() for _ in range(7)]
    st = {"i": 0}
    ws_b = torch.empty(sd.workspace_bytes(sd.OP_BUILD_TREE, B, K, V, 0, N), dtype=torch.uint8, device="cuda")
    walk_out = sd.verify_tree_sampled(target, tree, u, 1.0)
    A = walk_out["accepted_len"].cpu()
    rows_read = int(A.sum()) + B

    def step(ev=None):
        i = st["i"] % len(margs)
        st["i"] += 1
        sd.build_tree(margs[i], N, workspace=ws_b)
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.verify_tree_sampled(targets[i], tree, u, 1.0, out=walk_out)

    meta = {"workload": (f"DDTree build (B={B}, K={K}, V={V} fp32 marginals, N={N}) + walk under a "
                         f"sampling target (T=1, bf16 rows read on demand)"),
            "global_batch": B, "K_max": K, "V": V, "positions_per_step": B * (N - 1),
            "kernel": "k_tree_walk_rows", "kernel_bytes": rows_read * V * 2 + B * N * 12,
            "step_bytes": B * K * V * 4 + rows_read * V * 2, "mean_A": float(A.float().mean()),
            "rows_streamed": rows_read}
    return step, meta, None


def setup_tree_sampled_topk(torch, sd, wl):
    # the walk under a sampling target with top-k 50 (T = 1): at each visited
    # node the workgroup takes the exact top-50 of that row on the fly; only
    # the walk's rows are read. The tree itself is built once, outside the step
    case = wl.gen_tree(device="cuda")
    B, K, V, N = case.B, case.K, case.V, case.N
    tree = sd.build_tree(case.marginals, N)
    target = case.target_for_depths(tree["depth"], tree["n_nodes"])
    # 8 copies (8 x 131 MB): the rows a walk visits are not still cached when
    # their copy comes round
    targets = [target] + [target.clone() for _ in range(7)]
    u = wl.grid_uniforms((B, N), torch.Generator(device="cuda").manual_seed(1004), "cuda")
    walk_out = sd.verify_tree_sampled(target, tree, u, 1.0, top_k=50)
    A = walk_out["accepted_len"].cpu()
    rows_read = int(A.sum()) + B
    st = {"i": 0}

    def step(ev=None):
        i = st["i"] % len(targets)
        st["i"] += 1
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.verify_tree_sampled(targets[i], tree, u, 1.0, top_k=50, out=walk_out)

    meta = {"workload": (f"DDTree walk under a sampling target with top-k 50 (T=1): B={B}, N={N}, "
                         f"V={V} bf16 rows read on demand, the exact top-50 of each visited row"),
            "global_batch": B, "V": V, "positions_per_step": B * (N - 1),
            "kernel": "k_tree_walk_topk_rows", "kernel_bytes": rows_read * V * 2 + B * N * 12,
            "step_bytes": rows_read * V * 2, "mean_A": float(A.float().mean()),
            "rows_streamed": rows_read, "max_A": int(A.max())}
    return step, meta, None


def setup_kv(torch, sd, wl):
    # accepted-path KV compaction after a tree walk of the tree workload: one
    # 128 KB row per token (32 layers x 8 KV heads x 128 x (K, V) x bf16)
    case = wl.gen_tree(device="cuda")
    tree = sd.build_tree(case.marginals, case.N)
    walk = sd.verify_tree(case.target_for_depths(tree["depth"], tree["n_nodes"]), tree)
    B, N, row_bytes = case.B, case.N, 32 * 8 * 128 * 2 * 2
    n_rows = B * (N - 1)
    kv = torch.empty(n_rows, row_bytes, dtype=torch.uint8, device="cuda")
    base = torch.arange(B, dtype=torch.int64, device="cuda") * (N - 1)
    path, alen = walk["path"], walk["accepted_len"]
    p, a = path.cpu(), alen.cpu()
    moved = sum(1 for b in range(B) for i in range(int(a[b])) if int(p[b, i]) - 1 != i)

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.compact_kv(kv, base, path, alen)

    meta = {"workload": (f"accepted-path KV compaction after the tree walk: B={B}, N={N}, "
                         f"{row_bytes} B per token row"),
            "global_batch": B, "positions_per_step": int(a.sum()),
            "kernel": "k_compact_kv", "kernel_bytes": 2 * moved * row_bytes,
            "step_bytes": 2 * moved * row_bytes}
    return step, meta, None


def setup_rerank(torch, sd, wl):
    # EAGLE-2-style tree choice: 32 sequences, 1024 expanded candidates each
    # (8 layers, the 10 best of each layer expanded 10 ways), budget 64
    import numpy as np
    B, M, N = 32, 1024, 64
    rng = np.random.default_rng(1006)
    par = np.full((B, M), -1, np.int32)
    tok = np.zeros((B, M), np.int32)
    prob = np.zeros((B, M), np.float32)
    n = np.zeros(B, np.int32)
    for b in range(B):
        conf, pl, tl, ql, layer = [1.0], [-1], [-1], [1.0], [0]
        for _ in range(8):
            grow = sorted(layer, key=lambda c: (-conf[c], c))[:10]
            layer = []
            for c in grow:
                z = rng.normal(0, 2.0, 64)
                q = np.exp(z - z.max())
                q = (q / q.sum()).astype(np.float32)
                for r in np.argsort(-q, kind="stable")[:10]:
                    if len(pl) >= M:
                        break
                    pl.append(c)
                    tl.append(int(rng.integers(0, 128256)))
                    ql.append(float(q[r]))
                    conf.append(float(np.float32(conf[c] * q[r])))
                    layer.append(len(pl) - 1)
        k = len(pl)
        par[b, :k], tok[b, :k], prob[b, :k], n[b] = pl, tl, ql, k
    t = lambda a: torch.as_tensor(a, device="cuda")
    par_t, tok_t, prob_t, n_t = t(par), t(tok), t(prob), t(n)

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.rerank_tree(par_t, tok_t, prob_t, n_t, N)

    meta = {"workload": f"EAGLE-2-style tree choice: B={B}, {M} candidates, budget N={N}",
            "global_batch": B, "positions_per_step": B * (N - 1),
            "kernel": "k_rerank_tree", "kernel_bytes": B * M * 12 + B * N * 28,
            "step_bytes": B * M * 12 + B * N * 28}
    return step, meta, None


def setup_chain1(torch, sd, wl):
    case = wl.gen_chain_small(device="cuda")
    ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, 1, 4, 1000), dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, 1.0, B=1, K_max=4,
                        workspace=ws, validate=False)

    meta = {"workload": "chain verify B=1 K=4 V=1000 fp32 (latency-bound)", "global_batch": 1,
            "K_max": 4, "V": 1000, "positions_per_step": 4, "kernel": "k_chain_stats",
            "kernel_bytes": 9 * 1000 * 4 + 16, "step_bytes": 9 * 1000 * 4 + 16 + 20}
    return step, meta, None


WORKLOADS = {"adaptive": setup_adaptive, "greedy": setup_greedy, "topk": setup_topk,
             "tree": setup_tree, "tree_sampled": setup_tree_sampled,
             "tree_sampled_topk": setup_tree_sampled_topk, "chain1": setup_chain1,
             "kv": setup_kv, "rerank": setup_rerank}


def run_cpu_baseline(cpu, target_seconds: float):
    import numpy as np
    import torch

    import oracle
    from rejection_sampling_verify_softmax_amd import workloads as wl

    case, packed = cpu["case"], cpu["packed"]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    threads = min(threads, oracle.default_threads())
    conf = case.conf.cpu().numpy()
    t0 = time.perf_counter()
    sel = oracle.select_len(conf, case.B, case.K_max, case.cost)
    t_sel = time.perf_counter() - t0
    cu = sel["cu"].astype(np.int64)
    B, V = case.B, case.V
    group, n_groups = 16, min(8, (B + 15) // 16)
    # the sample: the first n_groups * group sequences, copied to host once
    # (fp32), then verified group after group, cycling, until the time is spent
    groups = []
    for g in range(n_groups):
        seqs = [s for s in range(g * group, (g + 1) * group) if s < B]
        t_rows = np.concatenate([np.arange(cu[s] + s, cu[s + 1] + s + 1) for s in seqs])
        d_rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
        ti = torch.as_tensor(t_rows, device="cuda")
        di = torch.as_tensor(d_rows, device="cuda")
        lens = [int(cu[s + 1] - cu[s]) for s in seqs]
        groups.append(dict(
            seqs=np.array(seqs),
            tgt=wl.to_host_f32(packed.target.index_select(0, ti)),
            dft=wl.to_host_f32(packed.draft.index_select(0, di)),
            tok=packed.tokens.index_select(0, di).cpu().numpy(),
            uni=packed.uniforms.index_select(0, ti).cpu().numpy(),
            cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
            n=len(seqs), k_max=max(lens), pos=int(sum(lens))))
    # Parity of the timed GPU step on the same inputs: its verify lengths for
    # every sequence, and its committed results for the sampled sequences (the
    # first visit of each group), bit-exact outside the oracle's margin cases.
    out = cpu["out"]
    A_g, nx_g = out["accepted_len"].cpu().numpy(), out["next_token"].cpu().numpy()
    st_g = out["status"].cpu().numpy()
    sel_margin = sel["margin"] != 0
    par = {"select_len_sequences": int(B),
           "select_len_mismatches": int(((cpu["k"] != sel["k"]) & ~sel_margin).sum()),
           "select_len_margin_cases": int(sel_margin.sum()),
           "verify_sequences": 0, "verify_mismatches": 0, "verify_margin_cases": 0}
    done_pos, done_seq, spent, calls = 0, 0, t_sel, 0
    while spent < target_seconds or calls < n_groups:
        g = groups[calls % n_groups]
        t0 = time.perf_counter()
        ref = oracle.verify_chain(g["tgt"], g["dft"], g["tok"], g["uni"], g["cu"], g["n"], g["k_max"], V,
                                  1.0, threads=threads, want_probs=False)
        spent += time.perf_counter() - t0
        if calls < n_groups:
            sq, mg = g["seqs"], ref["margin"] != 0
            bad = ~mg & ((A_g[sq] != ref["A"]) | (nx_g[sq] != ref["next"]) | (st_g[sq] != ref["status"]))
            par["verify_sequences"] += len(sq)
            par["verify_mismatches"] += int(bad.sum())
            par["verify_margin_cases"] += int(mg.sum())
        done_pos += g["pos"]
        done_seq += g["n"]
        calls += 1
    par["pass"] = par["select_len_mismatches"] == 0 and par["verify_mismatches"] == 0
    cpu["parity"] = par
    return {"value": done_pos / spent, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "sample": (f"CPU oracle (fp64 C, OpenMP over sequences): length selection for all {B} "
                       f"sequences, then packed chain verification of the first {n_groups * group} "
                       f"sequences in groups of {group}, cycled ({done_seq} sequences, "
                       f"{done_pos} draft positions), "
                       f"{spent:.1f} s of oracle time; transfer and conversion not timed")}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="adaptive", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--event-every", type=int, default=5,
                    help="time the dominant kernel with events on every n-th timed step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as HIP-graph replays (8 captured steps, cycled); the "
                         "dominant kernel is still timed live on eager steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "sequences are independent and the batch shards with no communication, so the "
              "single-GPU figure is the per-GPU throughput.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rejection_sampling_verify_softmax_amd as sd
    from rejection_sampling_verify_softmax_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sd.lib()
    log(f"setting up workload {args.workload}")
    step, meta, cpu = WORKLOADS[args.workload](torch, sd, wl)
    torch.cuda.synchronize()

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device-to-device copies")
        del a, b

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")

    # The dominant kernel is timed by a pair of events on every event_every-th
    # step of the timed region (each bound event leaves the stream idle for a
    # few microseconds around that launch, so not every step carries them).
    timed = list(range(0, args.steps, max(1, args.event_every)))
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in timed}
    for s_ev, e_ev in evs.values():  # torch creates the HIP event on its first record
        s_ev.record()
        e_ev.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = [s.elapsed_time(e) for s, e in evs.values()]
    kernel_ms_avg = sum(kernel_ms) / len(kernel_ms)
    if args.graph:
        # The library only enqueues kernels (no allocation, synchronisation or
        # memset), so a step captures as it is. Eight captured steps keep any
        # rotation over input copies that the workload does.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for _ in range(8):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        log(f"graph replays: {elapsed * 1e3 / args.steps:.4f} ms/step")
    ms_per_step = elapsed * 1e3 / args.steps
    positions = meta["positions_per_step"]
    value = positions * args.steps / elapsed
    achieved = meta["kernel_bytes"] / (kernel_ms_avg * 1e-3) / 1e9
    traffic = load_traffic(meta["kernel"], args.workload)
    log(f"{ms_per_step:.4f} ms/step, {meta['kernel']} {kernel_ms_avg * 1e3:.1f} us avg -> "
        f"{achieved:.0f} GB/s ({achieved / PEAK_HBM_GBPS:.1%} of 8 TB/s)")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {k: meta[k] for k in ("workload", "global_batch", "K_max", "V") if k in meta},
        "launch": "hip graph replays (8 captured steps)" if args.graph else "eager",
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "traffic_GBps": (traffic / (kernel_ms_avg * 1e-3) / 1e9) if traffic else None,
            "kernel": meta["kernel"],
            "kernel_us": kernel_ms_avg * 1e3,
            "launches_timed": len(kernel_ms),
            "algorithmic_bytes_per_launch": meta["kernel_bytes"],
        },
        "step": {
            "positions_per_step": positions,
            "algorithmic_bytes": meta["step_bytes"],
            "effective_GBps": meta["step_bytes"] / (ms_per_step * 1e-3) / 1e9,
        },
    }
    result["config"]["parallelism"] = "none (one GPU)"
    for k in ("logits", "temperature", "mean_k"):
        if k in meta:
            result["config"][k] = meta[k]
    for k in ("mean_A", "max_A", "rows_streamed", "rows_in_windows"):
        if k in meta:
            result["step"][k] = meta[k]
    if cpu is not None and not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = run_cpu_baseline(cpu, args.cpu_seconds)
        result["parity"] = cpu.get("parity")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
