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

Other workloads (--workload adaptive_table|greedy|topk|tree|tree_sampled|tree_sampled_topk|chain1|kv|rerank|
readceiling_66m|readceiling_523m|readceiling_523m_64k|readceiling_523m_rows|readceiling_1g)
measure the other kernels
for the design notes; their inputs are rotated across copies so that the
working set exceeds the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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

def adaptive_bytes(k_sel, A, B, K, V):
    """Algorithmic bytes of a packed adaptive step (bf16 rows): (first-phase
    streaming launch, whole step, rows of phase 1, rows of phase 2). Phase 1
    streams positions 0 and 1 (and the extra-token row of a shorter draft) of
    every sequence; phase 2 the rest of the window only for sequences whose
    first two drafts were both accepted."""
    import numpy as np
    k_sel = k_sel.cpu().numpy().astype(np.int64)
    A = A.cpu().numpy().astype(np.int64)
    R_d = int(k_sel.sum())
    R_t = R_d + B
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
    return stats_bytes, step_bytes, rows1, rows2


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
    stats_bytes, step_bytes, rows1, rows2 = adaptive_bytes(sel["k"], out["accepted_len"], B, K, V)

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
        "mean_k": positions / B, "mean_A": out["accepted_len"].float().mean().item(),
        "rows_streamed": rows1 + rows2, "rows_in_windows": R_t + R_d,
        # the step's two calls, timed alone after the timed region
        "parts": {
            "select_len": lambda: sd.select_len(case.conf, case.cost, out=sel_out),
            "verify": lambda: sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0,
                                              cu=sel_out["cu"], B=B, K_max=K, workspace=ws, out=out,
                                              validate=False),
        },
    }
    cpu = {"leg": cpu_leg_adaptive, "case": case, "packed": packed, "out": out, "sel": sel_out}
    return step, meta, cpu


def measure_cost_table(torch, sd, case, reps=30):
    """Per-position cost table of the verify step on this GPU (the DSpark
    scheduler's table, profiled on the deployment that uses it). For every
    fixed window k = 0..K_max the packed verification of all B sequences over
    their first k positions is timed (median of `reps` calls, HIP events on the
    stream it runs on); dt_j = t(j) - t(j-1) is the verify time that position
    j adds to the batch. In tokens of advance, at the full window's operating
    point (throughput E[adv(K)] * B / t(K) tokens per second, with the
    expected advance from sd_select_len), position j costs
    cost[j-1] = E[adv(K)] * dt_j / t(K) per sequence. Only the verify step's
    own time is in it, not the target forward's."""
    import statistics
    B, K = case.B, case.K_max
    times = []
    for k in range(K + 1):
        pk = case.packed(torch.full((B,), k, dtype=torch.int64))
        ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, B, k, case.V), dtype=torch.uint8, device="cuda")
        out = sd.verify_chain(pk.target, pk.draft, pk.tokens, pk.uniforms, 1.0, cu=pk.cu, B=B, K_max=k,
                              workspace=ws)
        for _ in range(3):
            sd.verify_chain(pk.target, pk.draft, pk.tokens, pk.uniforms, 1.0, cu=pk.cu, B=B, K_max=k,
                            workspace=ws, out=out)
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            sd.verify_chain(pk.target, pk.draft, pk.tokens, pk.uniforms, 1.0, cu=pk.cu, B=B, K_max=k,
                            workspace=ws, out=out)
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        times.append(statistics.median(ms))
        del pk, ws, out
    adv_full = float(sd.select_len(case.conf, -1.0)["adv"].mean())     # every s_j > -1: k = K_max
    dt = [times[j] - times[j - 1] for j in range(1, K + 1)]
    table = [adv_full * d / times[K] for d in dt]
    return {"t_ms": times, "dt_ms": dt, "adv_full_window": adv_full, "cost": table}


def setup_adaptive_table(torch, sd, wl):
    # the adaptive step with verify lengths chosen from the per-position cost
    # table measured on this GPU (instead of the constant 0.15)
    case = wl.gen_adaptive_chain(device="cuda")
    log("measuring the per-position cost table (fixed windows k = 0..8)")
    ct = measure_cost_table(torch, sd, case)
    table = torch.tensor(ct["cost"], dtype=torch.float32, device="cuda")
    log("cost table: " + " ".join(f"{c:.4f}" for c in ct["cost"]) +
        "  (t(k) ms: " + " ".join(f"{t:.4f}" for t in ct["t_ms"]) + ")")
    sel = sd.select_len_table(case.conf, table)
    torch.cuda.synchronize()
    packed = case.packed(sel["k"])
    B, K, V = case.B, case.K_max, case.V
    positions = int(sel["cu"][-1].item())
    ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, B, K, V), dtype=torch.uint8, device="cuda")
    out = sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0, cu=sel["cu"],
                          B=B, K_max=K, workspace=ws)
    sel_out = {"k": sel["k"], "adv": sel["adv"], "cu": sel["cu"]}

    def step(ev=None):
        s = sd.select_len_table(case.conf, table, out=sel_out)
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms, 1.0,
                        cu=s["cu"], B=B, K_max=K, workspace=ws, out=out)

    torch.cuda.synchronize()
    A = out["accepted_len"].float().mean().item()
    stats_bytes, step_bytes, rows1, rows2 = adaptive_bytes(sel["k"], out["accepted_len"], B, K, V)
    meta = {"workload": (f"DSpark-adaptive chain verify with a measured cost table: select_len_table "
                         f"(per-position costs measured on this GPU) + packed stochastic verify, "
                         f"B={B}, K_max={K}, V={V}, bf16 logits, T=1.0"),
            "global_batch": B, "K_max": K, "V": V, "logits": "bf16", "temperature": 1.0,
            "positions_per_step": positions, "kernel": "k_chain_stats",
            "kernel_bytes": stats_bytes, "step_bytes": step_bytes, "mean_k": positions / B, "mean_A": A,
            "mean_adv": float(sel["adv"].mean()), "cost_table": ct, "rows_streamed": rows1 + rows2,
            "rows_in_windows": 2 * positions + B,
            "parts": {
                "select_len": lambda: sd.select_len_table(case.conf, table, out=sel_out),
                "verify": lambda: sd.verify_chain(packed.target, packed.draft, packed.tokens, packed.uniforms,
                                                  1.0, cu=sel_out["cu"], B=B, K_max=K, workspace=ws, out=out),
            }}
    cpu = {"leg": cpu_leg_adaptive, "case": case, "packed": packed, "out": out, "sel": sel_out,
           "table": table.cpu().numpy()}
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
        st["out"] = sd.verify_greedy(t, case.tokens, B=B, K_max=K, workspace=ws)

    rows = B * (K + 1)
    A = sd.verify_greedy(case.target, case.tokens, B=B, K_max=K, workspace=ws)["accepted_len"].cpu()
    meta = {"workload": f"greedy chain verify B={B} K={K} V={V} bf16 (8 rotated input copies)",
            "global_batch": B, "K_max": K, "V": V, "positions_per_step": B * K,
            "kernel": "k_argmax", "kernel_bytes": rows * V * 2, "step_bytes": rows * V * 2 + B * K * 4,
            "mean_A": float(A.float().mean())}
    return step, meta, {"leg": cpu_leg_greedy, "case": case, "state": st}


def setup_topk(torch, sd, wl):
    case = wl.gen_topk_chain(device="cuda")
    B, K, V = case.B, case.K_max, case.V
    ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, B, K, V, case.top_k), dtype=torch.uint8, device="cuda")

    st = {}

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        st["out"] = sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, case.temperature,
                                    top_k=case.top_k, B=B, K_max=K, workspace=ws)

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
    return step, meta, {"leg": cpu_leg_chain, "case": case, "state": st}


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
        st["tree"] = sd.build_tree(margs[i], N, workspace=ws_b)
        sd.verify_tree(targets[i], st["tree"], out=walk_out)

    st["walk"] = walk_out
    meta = {"workload": (f"DDTree build (B={B}, K={K}, V={V} fp32 marginals, N={N}) + argmax walk over "
                         f"bf16 target rows (read on demand)"),
            "global_batch": B, "K_max": K, "V": V, "positions_per_step": B * (N - 1),
            "kernel": "k_topk_short<f32>", "kernel_bytes": B * K * V * 4,
            "step_bytes": B * K * V * 4 + rows_read * V * 2, "mean_A": float(A.float().mean()),
            "rows_streamed": rows_read}
    return step, meta, {"leg": cpu_leg_tree, "case": case, "target": target, "state": st}


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
        st["tree"] = sd.build_tree(margs[i], N, workspace=ws_b)
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.verify_tree_sampled(targets[i], st["tree"], u, 1.0, out=walk_out)

    st["walk"] = walk_out

    meta = {"workload": (f"DDTree build (B={B}, K={K}, V={V} fp32 marginals, N={N}) + walk under a "
                         f"sampling target (T=1, bf16 rows read on demand)"),
            "global_batch": B, "K_max": K, "V": V, "positions_per_step": B * (N - 1),
            "kernel": "k_tree_walk_rows", "kernel_bytes": rows_read * V * 2 + B * N * 12,
            "step_bytes": B * K * V * 4 + rows_read * V * 2, "mean_A": float(A.float().mean()),
            "rows_streamed": rows_read}
    return step, meta, {"leg": cpu_leg_tree, "case": case, "target": target, "state": st, "u": u,
                        "T": 1.0, "top_k": 0}


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

    st["tree"], st["walk"] = tree, walk_out

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
    return step, meta, {"leg": cpu_leg_tree, "case": case, "target": target, "state": st, "u": u,
                        "T": 1.0, "top_k": 50, "walk_only": True}


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

    g = torch.Generator(device="cuda").manual_seed(1007)
    kv.copy_(torch.randint(0, 256, kv.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))
    kv0 = kv.clone()

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.compact_kv(kv, base, path, alen)

    meta = {"workload": (f"accepted-path KV compaction after the tree walk: B={B}, N={N}, "
                         f"{row_bytes} B per token row"),
            "global_batch": B, "positions_per_step": int(a.sum()),
            "kernel": "k_compact_kv", "kernel_bytes": 2 * moved * row_bytes,
            "step_bytes": 2 * moved * row_bytes}
    return step, meta, {"leg": cpu_leg_kv, "kv": kv, "kv0": kv0, "base": base, "path": path, "alen": alen,
                        "B": B, "N": N}


def setup_rerank(torch, sd, wl):
    # EAGLE-2-style dynamic tree: 8 expansion steps (each expands the 10 best
    # new candidates by cumulative confidence, 10 children each, from the
    # stand-in drafter's proposals), then the re-ranking of the candidates into
    # a verification tree of budget 64, for 32 sequences
    B, M, N, layers, W, C = 32, 1024, 64, 8, 10, 10
    kids = wl.gen_eagle_children(device="cuda", B=B, layers=layers, W=W, C=C)
    cand = sd.empty_candidates(B, M)
    exp = torch.empty(B, W, dtype=torch.int32, device="cuda")
    st = {}

    def step(ev=None):
        cand["n_cand"].zero_()                  # a new tree: the first step writes the root
        for ct, cp in kids:
            sd.expand_tree(cand, exp, ct, cp, expand_out=exp)
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        st["out"] = sd.rerank_tree(cand["parent"], cand["token"], cand["prob"], cand["n_cand"], N,
                                   out=st.get("out"))

    step()
    torch.cuda.synchronize()
    n_cand = int(cand["n_cand"].max())
    meta = {"workload": (f"EAGLE-2-style dynamic tree: {layers} expansion steps (W={W} nodes x C={C} "
                         f"children each) + re-ranking into a budget-{N} tree, B={B}, {n_cand} candidates"),
            "global_batch": B, "positions_per_step": B * (N - 1),
            "kernel": "k_rerank_tree", "kernel_bytes": B * n_cand * 12 + B * N * 28,
            "step_bytes": B * n_cand * 12 + B * N * 28 + layers * B * W * C * 8}
    return step, meta, {"leg": cpu_leg_rerank, "kids": kids, "cand": cand, "B": B, "M": M, "N": N,
                        "W": W, "C": C, "state": st}


def setup_chain1(torch, sd, wl):
    case = wl.gen_chain_small(device="cuda")
    ws = torch.empty(sd.workspace_bytes(sd.OP_CHAIN, 1, 4, 1000), dtype=torch.uint8, device="cuda")

    st = {}

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        st["out"] = sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, 1.0, B=1,
                                    K_max=4, workspace=ws)

    A = sd.verify_chain(case.target, case.draft, case.tokens, case.uniforms, 1.0, B=1, K_max=4,
                        workspace=ws)["accepted_len"].cpu()
    meta = {"workload": "chain verify B=1 K=4 V=1000 fp32 (latency-bound)", "global_batch": 1,
            "K_max": 4, "V": 1000, "positions_per_step": 4, "kernel": "k_chain_stats",
            "kernel_bytes": 9 * 1000 * 4 + 16, "step_bytes": 9 * 1000 * 4 + 16 + 20,
            "mean_A": float(A.float().mean())}
    return step, meta, {"leg": cpu_leg_chain, "case": case, "state": st}


def setup_readceiling(torch, sd, wl, nbytes, copies, chunk=16384):
    # a plain streaming read of nbytes (16-byte non-temporal loads, the load of
    # the row passes), rotated over `copies` buffers so that a copy is not still
    # in the 256 MB last-level cache when its turn comes
    n_blocks = nbytes // chunk          # 16 KB per workgroup: the fastest chunk measured
    bufs = [torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(copies)]
    sink = torch.empty(n_blocks, dtype=torch.int32, device="cuda")
    st = {"i": 0}

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.stream_read(bufs[st["i"] % copies], sink, n_blocks)
        st["i"] += 1

    meta = {"workload": (f"plain streaming read of {nbytes / 1e6:.1f} MB ({copies} rotated copies), "
                         f"{n_blocks} workgroups x 256 threads ({chunk // 1024} KB each), 16-byte non-temporal loads"),
            "positions_per_step": 0, "kernel": "k_stream_read", "kernel_bytes": nbytes,
            "step_bytes": nbytes}
    return step, meta, None


def setup_readceiling_66m(torch, sd, wl):
    return setup_readceiling(torch, sd, wl, 64 * 4 * 128256 * 2, 8)     # the greedy workload's rows


def setup_readceiling_1g(torch, sd, wl):
    return setup_readceiling(torch, sd, wl, 1 << 30, 2)


def setup_readceiling_523m(torch, sd, wl):
    # the bytes of the adaptive step's first streaming launch
    return setup_readceiling(torch, sd, wl, 523032028 // 16 * 16, 2)


def setup_readceiling_523m_64k(torch, sd, wl):
    # the same bytes in the row passes' chunk size (64 KB per workgroup and row)
    return setup_readceiling(torch, sd, wl, 523032028 // 16 * 16, 2, chunk=65536)


def setup_readceiling_523m_rows(torch, sd, wl):
    # the adaptive step's first launch as a plain read: its 2039 bf16 rows of
    # V = 128256 (a 256,512-byte pitch), one workgroup per 64 KB chunk of a row
    rows, V, copies = 2039, 128256, 2
    bufs = [torch.empty(rows, V, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(copies)]
    n_chunks = -(-V * 2 // 65536)
    sink = torch.empty(rows * n_chunks, dtype=torch.int32, device="cuda")
    st = {"i": 0}

    def step(ev=None):
        if ev is not None:
            sd.time_next_stream_pass(*ev)
        sd.stream_read_rows(bufs[st["i"] % copies], 65536, sink)
        st["i"] += 1

    nbytes = rows * V * 2
    meta = {"workload": (f"plain streaming read of {rows} bf16 rows of V = {V} ({nbytes / 1e6:.1f} MB, "
                         f"{copies} rotated copies), one workgroup x 256 threads per 64 KB chunk of a row "
                         f"({rows * n_chunks} workgroups, the row passes' grid), 16-byte non-temporal loads"),
            "positions_per_step": 0, "kernel": "k_stream_read_rows", "kernel_bytes": nbytes,
            "step_bytes": nbytes}
    return step, meta, None


WORKLOADS = {"adaptive": setup_adaptive, "adaptive_table": setup_adaptive_table, "greedy": setup_greedy, "topk": setup_topk,
             "tree": setup_tree, "tree_sampled": setup_tree_sampled,
             "tree_sampled_topk": setup_tree_sampled_topk, "chain1": setup_chain1,
             "kv": setup_kv, "rerank": setup_rerank, "readceiling_66m": setup_readceiling_66m,
             "readceiling_1g": setup_readceiling_1g, "readceiling_523m": setup_readceiling_523m,
             "readceiling_523m_64k": setup_readceiling_523m_64k,
             "readceiling_523m_rows": setup_readceiling_523m_rows}


# --------------------------------------------------------------------------
# CPU oracle legs: each returns (sample, parity, about). sample(threads) runs
# the oracle once on a bounded piece of the workload and returns the
# positions it covered; parity() compares the timed step's GPU results with
# the oracle on the whole batch (bit-exact, the oracle's margin cases checked
# for validity instead); about says what the sample is. Only this leg of the
# benchmark touches the oracle.
# --------------------------------------------------------------------------

def _groups(n, size):
    return [list(range(g, min(n, g + size))) for g in range(0, n, size)]


def _chain_parity(oracle, h, A, nx, st, V, T, top_k, threads):
    """Oracle verification of host rows h (re-packed sequences) against the
    GPU's A, next and status for those sequences: (sequences, mismatches,
    margin cases)."""
    import numpy as np
    ref = oracle.verify_chain(h["target"], h["draft"], h["tokens"], h["uniforms"], h["cu"], h["B"],
                              h["K_max"], V, T, top_k, threads=threads, want_probs=False)
    mg = ref["margin"] != 0
    bad = ~mg & ((A != ref["A"]) | (nx != ref["next"]) | (st != ref["status"]))
    if mg.any() and T != 0.0:
        valid, st_exp = oracle.check_chain(h["target"], h["draft"], h["tokens"], h["uniforms"], h["cu"],
                                           h["B"], h["K_max"], V, T, A, nx, top_k=top_k, threads=threads)
        sample_only = (ref["margin"] & oracle.MARGIN_ACCEPT) == 0
        bad |= mg & ((valid != 3) | (st != st_exp) | (sample_only & (A != ref["A"])))
    return len(A), int(bad.sum()), int(mg.sum())


def _host_chain(case, seqs):
    """Host float32 rows of sequences seqs of a chain case, re-packed."""
    import numpy as np
    import torch
    from rejection_sampling_verify_softmax_amd import workloads as wl
    cu = (np.arange(case.B + 1, dtype=np.int64) * case.K_max if case.cu is None
          else case.cu.cpu().numpy().astype(np.int64))
    t_rows = np.concatenate([np.arange(cu[b] + b, cu[b + 1] + b + 1) for b in seqs])
    d_parts = [np.arange(cu[b], cu[b + 1]) for b in seqs]
    d_rows = np.concatenate(d_parts)
    lens = [int(cu[b + 1] - cu[b]) for b in seqs]
    ti = torch.as_tensor(t_rows, device=case.target.device)
    di = torch.as_tensor(d_rows, device=case.target.device)
    h = {"target": wl.to_host_f32(case.target.index_select(0, ti)),
         "tokens": case.tokens.index_select(0, di).cpu().numpy() if len(d_rows) else np.zeros(0, np.int32),
         "cu": np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), "B": len(seqs),
         "K_max": max(lens), "pos": int(sum(lens)), "seqs": np.array(seqs)}
    if case.draft is not None:
        h["draft"] = wl.to_host_f32(case.draft.index_select(0, di))
        h["uniforms"] = case.uniforms.index_select(0, ti).cpu().numpy()
    else:
        h["draft"], h["uniforms"] = None, np.zeros(len(t_rows), np.float32)
    return h


def cpu_leg_adaptive(cpu, threads):
    import numpy as np
    import oracle
    case, packed = cpu["case"], cpu["packed"]
    B, V = case.B, case.V
    conf = case.conf.cpu().numpy()
    groups = [_host_chain(packed, g) for g in _groups(B, 16)[:8]]     # the first 128 sequences
    state = {"i": 0, "sel": True}

    table = cpu.get("table")

    def select():
        if table is None:
            return oracle.select_len(conf, B, case.K_max, case.cost)
        return oracle.select_len_table(conf, B, case.K_max, table)

    def sample(nt):
        if state["sel"]:                    # length selection for the whole batch, once per pass
            select()
        g = groups[state["i"] % len(groups)]
        state["i"] += 1
        state["sel"] = state["i"] % len(groups) == 0
        oracle.verify_chain(g["target"], g["draft"], g["tokens"], g["uniforms"], g["cu"], g["B"],
                            g["K_max"], V, 1.0, threads=nt, want_probs=False)
        return g["pos"]

    def parity():
        k_g = cpu["sel"]["k"].cpu().numpy()
        sel = select()
        sel_mg = sel["margin"] != 0
        if table is None:
            ok_sel = oracle.check_select_len(conf, B, case.K_max, case.cost, k_g) == 1
        else:                               # no validity check for the table rule: margins must match
            ok_sel = k_g == sel["k"]
        out = cpu["out"]
        A, nx, st = (out[k].cpu().numpy() for k in ("accepted_len", "next_token", "status"))
        par = {"select_len_sequences": B,
               "select_len_mismatches": int(((k_g != sel["k"]) & ~sel_mg).sum() + (~ok_sel & sel_mg).sum()),
               "select_len_margin_cases": int(sel_mg.sum()),
               "verify_sequences": 0, "verify_mismatches": 0, "verify_margin_cases": 0}
        for g in _groups(B, 64):
            h = _host_chain(packed, g)
            n, bad, mg = _chain_parity(oracle, h, A[g], nx[g], st[g], V, 1.0, 0, threads)
            par["verify_sequences"] += n
            par["verify_mismatches"] += bad
            par["verify_margin_cases"] += mg
        par["pass"] = par["select_len_mismatches"] == 0 and par["verify_mismatches"] == 0
        return par

    about = (f"length selection for all {B} sequences, then packed chain verification of the first "
             f"{sum(g['B'] for g in groups)} sequences in groups of 16, cycled")
    return sample, parity, about


def cpu_leg_chain(cpu, threads):
    import oracle
    case = cpu["case"]
    V, T, top_k = case.V, case.temperature, case.top_k
    size = 1 if case.B == 1 else (4 if top_k else 16)
    groups = [_host_chain(case, g) for g in _groups(case.B, size)[:8]]
    state = {"i": 0}

    def sample(nt):
        g = groups[state["i"] % len(groups)]
        state["i"] += 1
        oracle.verify_chain(g["target"], g["draft"], g["tokens"], g["uniforms"], g["cu"], g["B"],
                            g["K_max"], V, T, top_k, threads=nt, want_probs=False)
        return g["pos"]

    def parity():
        out = cpu["state"]["out"]
        A, nx, st = (out[k].cpu().numpy() for k in ("accepted_len", "next_token", "status"))
        par = {"verify_sequences": 0, "verify_mismatches": 0, "verify_margin_cases": 0}
        for g in _groups(case.B, 32):
            n, bad, mg = _chain_parity(oracle, _host_chain(case, g), A[g], nx[g], st[g], V, T, top_k,
                                       threads)
            par["verify_sequences"] += n
            par["verify_mismatches"] += bad
            par["verify_margin_cases"] += mg
        par["pass"] = par["verify_mismatches"] == 0
        return par

    about = (f"chain verification{' with top-k ' + str(top_k) if top_k else ''} of the first "
             f"{sum(g['B'] for g in groups)} sequences in groups of {size}, cycled")
    return sample, parity, about


def cpu_leg_greedy(cpu, threads):
    import oracle
    from rejection_sampling_verify_softmax_amd import workloads as wl
    case = cpu["case"]
    B, K, V = case.B, case.K_max, case.V
    host_t = wl.to_host_f32(case.target).reshape(B, K + 1, V)
    host_y = case.tokens.cpu().numpy().reshape(B, K)
    groups = _groups(B, 8)
    state = {"i": 0}

    def sample(nt):
        g = groups[state["i"] % len(groups)]
        state["i"] += 1
        oracle.verify_greedy(host_t[g[0]:g[-1] + 1], host_y[g[0]:g[-1] + 1], None, len(g), K, V, threads=nt)
        return len(g) * K

    def parity():
        out = cpu["state"]["out"]
        ref = oracle.verify_greedy(host_t, host_y, None, B, K, V, threads=threads)
        bad = sum(int((out[kg].cpu().numpy() != ref[kr]).sum())
                  for kg, kr in (("accepted_len", "A"), ("next_token", "next"), ("status", "status")))
        return {"verify_sequences": B, "verify_mismatches": bad, "pass": bad == 0}

    return sample, parity, f"greedy verification of all {B} sequences in groups of 8, cycled"


def cpu_leg_tree(cpu, threads):
    import numpy as np
    import oracle
    from rejection_sampling_verify_softmax_amd import workloads as wl
    case, st = cpu["case"], cpu["state"]
    B, K, V, N = case.B, case.K, case.V, case.N
    marg = wl.to_host_f32(case.marginals)
    tgt = wl.to_host_f32(cpu["target"])
    T, top_k = cpu.get("T", 0.0), cpu.get("top_k", 0)
    walk_only = cpu.get("walk_only", False)
    u = cpu["u"].cpu().numpy() if "u" in cpu else None
    groups = _groups(B, 4)
    tree_h = {k: v.cpu().numpy() for k, v in st["tree"].items()}
    state = {"i": 0}

    def sample(nt):
        g = groups[state["i"] % len(groups)]
        state["i"] += 1
        s = slice(g[0], g[-1] + 1)
        tr = tree_h if walk_only else oracle.build_tree(marg[s], len(g), K, V, N, threads=nt)
        tok, par_, nn = (tr[k][s] if walk_only else tr[k] for k in ("token", "parent", "n_nodes"))
        if T == 0.0:
            oracle.verify_tree(tgt[s], tok, par_, nn, len(g), N, V, threads=nt)
        else:
            oracle.verify_tree_sampled(tgt[s], tok, par_, nn, u[s], len(g), N, V, T, top_k, threads=nt)
        return len(g) * (N - 1)

    def parity():
        tree = {k: v.cpu().numpy() for k, v in st["tree"].items()}
        walk = {k: v.cpu().numpy() for k, v in st["walk"].items()}
        bad = 0
        if not walk_only:
            ref_t = oracle.build_tree(marg, B, K, V, N, threads=threads)
            for k in ("token", "parent", "depth", "score", "n_nodes"):
                bad += int((tree[k] != ref_t[k]).reshape(B, -1).any(axis=1).sum())
            bad += int((tree["anc_mask"].view(np.uint64) != ref_t["anc_mask"]).any(axis=1).sum())
        margins = 0
        if T == 0.0:
            ref = oracle.verify_tree(tgt, tree["token"], tree["parent"], tree["n_nodes"], B, N, V,
                                     threads=threads)
            mg = np.zeros(B, bool)
        else:
            ref = oracle.verify_tree_sampled(tgt, tree["token"], tree["parent"], tree["n_nodes"], u, B, N,
                                             V, T, top_k, threads=threads)
            mg = ref["margin"] != 0
            margins = int(mg.sum())
        diff = ((walk["path"] != ref["path"]).any(axis=1) | (walk["accepted_len"] != ref["A"])
                | (walk["next_token"] != ref["next"]))
        bad += int((diff & ~mg).sum())
        if mg.any():
            valid = oracle.check_tree_sampled(tgt, tree["token"], tree["parent"], tree["n_nodes"], u, B, N, V,
                                              T, walk["path"], walk["accepted_len"], walk["next_token"],
                                              top_k=top_k, threads=threads)
            bad += int((mg & (valid != 1)).sum())
        return {"tree_sequences": B, "mismatches": bad, "walk_margin_cases": margins, "pass": bad == 0}

    what = ("the sampled walk" + (f" with top-k {top_k}" if top_k else "") if T else "the argmax walk")
    about = (("" if walk_only else "tree build and ") + what +
             f" for all {B} sequences in groups of 4, cycled")
    return sample, parity, about


def cpu_leg_kv(cpu, threads):
    import numpy as np
    import oracle
    kv0 = cpu["kv0"].cpu().numpy()
    base, path, alen = (cpu[k].cpu().numpy() for k in ("base", "path", "alen"))
    B, N = cpu["B"], cpu["N"]
    state = {}

    def sample(nt):
        state["ref"] = oracle.compact_kv(kv0, base, path, alen, B, N)
        return int(alen.sum())

    def parity():
        # the library moves rows in place: a step applied to the compacted rows
        # again is not the one-step result, so compare one fresh call
        import rejection_sampling_verify_softmax_amd as sd
        import torch
        kv = cpu["kv0"].clone()
        sd.compact_kv(kv, cpu["base"], cpu["path"], cpu["alen"])
        torch.cuda.synchronize()
        ref = oracle.compact_kv(kv0, base, path, alen, B, N)
        bad = int((kv.cpu().numpy() != ref).any(axis=1).sum())
        return {"rows": int(kv0.shape[0]), "row_mismatches": bad, "pass": bad == 0}

    return sample, parity, f"accepted-path KV compaction of all {B} sequences (host copy of the rows)", True


def cpu_leg_rerank(cpu, threads):
    import numpy as np
    import oracle
    B, M, N, W, C = cpu["B"], cpu["M"], cpu["N"], cpu["W"], cpu["C"]
    kids = [(t.cpu().numpy(), p.cpu().numpy()) for t, p in cpu["kids"]]

    def run():
        cand = oracle.empty_candidates(B, M)
        exp = np.full((B, W), -1, np.int32)
        for ct, cp in kids:
            cand = oracle.expand_tree(cand, exp, ct, cp, B, M, W, C)
            exp = cand["expand"]
        return cand, oracle.rerank_tree(cand["parent"], cand["token"], cand["prob"], cand["n_cand"], B, M, N)

    def sample(nt):
        run()
        return B * (N - 1)

    def parity():
        ref_c, ref = run()
        g = {k: v.cpu().numpy() for k, v in cpu["cand"].items()}
        bad = int((g["n_cand"] != ref_c["n_cand"]).sum())
        for b in range(B):
            n = int(ref_c["n_cand"][b])
            for k in ("parent", "token"):
                bad += int((g[k][b, :n] != ref_c[k][b, :n]).any())
            for k in ("prob", "conf"):
                bad += int((g[k][b, :n].view(np.int32) != ref_c[k][b, :n].view(np.int32)).any())
        out = {k: v.cpu().numpy() for k, v in cpu["state"]["out"].items()}
        for k in ("token", "parent", "depth", "score", "cand", "n_nodes"):
            bad += int((out[k] != ref[k]).reshape(B, -1).any(axis=1).sum())
        bad += int((out["anc_mask"].view(np.uint64) != ref["anc_mask"]).any(axis=1).sum())
        return {"tree_sequences": B, "mismatches": bad, "pass": bad == 0}

    return sample, parity, (f"{len(kids)} expansion steps and the re-ranking for all {B} sequences "
                            f"(single-threaded C)"), True


def run_cpu_baseline(cpu, target_seconds: float):
    """The oracle timed on the host's cores on a bounded sample of the
    workload (all cores, then one thread for a quarter of the time), and the
    parity of the timed step against it. Returns (cpu_baseline, parity)."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    threads = min(threads, oracle.default_threads())
    leg = cpu["leg"](cpu, threads)
    sample, parity, about = leg[:3]
    if len(leg) > 3 and leg[3]:         # a single-threaded oracle routine
        threads = 1

    def timed(nt, seconds):
        units, spent, calls = 0, 0.0, 0
        while spent < seconds or calls == 0:
            t0 = time.perf_counter()
            units += sample(nt)
            spent += time.perf_counter() - t0
            calls += 1
        return units, spent

    units, spent = timed(threads, target_seconds)
    units1, spent1 = (units, spent) if threads == 1 else timed(1, target_seconds / 4)
    base = {"value": units / spent, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "value_1thread": units1 / spent1,
            "sample": (f"CPU oracle (fp64 C, OpenMP over sequences): {about}; {units} positions in "
                       f"{spent:.1f} s on {threads} threads, {units1} positions in {spent1:.1f} s on one "
                       f"thread; host copies and conversions not timed")}
    return base, parity()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: at least 200, and enough for 40 steps with kernel "
                         "events at the default event spacing)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="adaptive", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--event-every", type=int, default=None,
                    help="time the dominant kernel with events on every n-th timed step (default: "
                         "spaced so that the events add about 1 %% to the timed region, at least 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-parts", action="store_true",
                    help="do not time the step's calls alone after the timed region")
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
    # The step's own time, without events, sets how far apart the evented steps
    # are: a launch bound to an event pair costs the step about 10-80 us (the
    # stream idles around it, and the host issues it more slowly), which would
    # dominate a launch-bound step of a few microseconds if every fifth step
    # carried one.
    n_cal = 1
    while True:
        t0 = time.perf_counter()
        for _ in range(n_cal):
            step()
        torch.cuda.synchronize()
        cal = time.perf_counter() - t0
        if cal >= 0.01 or n_cal >= 1 << 16:
            break
        n_cal *= 2
    t_step = cal / n_cal
    event_cost_s = 50e-6
    if args.event_every is None:
        args.event_every = max(5, math.ceil(event_cost_s / (0.01 * t_step)))
        if args.steps is not None:
            args.event_every = min(args.event_every, max(5, args.steps // 20))
    if args.steps is None:
        args.steps = min(max(200, 40 * args.event_every), max(200, int(2.0 / t_step)))
    log(f"warmup {args.warmup} done ({t_step * 1e6:.1f} us per step without events); timing "
        f"{args.steps} steps, events on every {args.event_every}")

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
            "event_every": args.event_every,
            "algorithmic_bytes_per_launch": meta["kernel_bytes"],
        },
        "step": {
            "positions_per_step": positions,
            "algorithmic_bytes": meta["step_bytes"],
            "effective_GBps": meta["step_bytes"] / (ms_per_step * 1e-3) / 1e9,
            "us_per_step_without_events": t_step * 1e6,
        },
    }
    result["config"]["parallelism"] = "none (one GPU)"
    for k in ("logits", "temperature", "mean_k"):
        if k in meta:
            result["config"][k] = meta[k]
    for k in ("mean_A", "max_A", "rows_streamed", "rows_in_windows", "mean_adv"):
        if k in meta:
            result["step"][k] = meta[k]
    if "cost_table" in meta:
        result["cost_table"] = meta["cost_table"]
    result["roofline"]["kernel_us_median"] = sorted(kernel_ms)[len(kernel_ms) // 2] * 1e3
    if "parts" in meta and not args.skip_parts:
        # each call of the step alone, 100 back to back between two events
        # after 5 warm-ups (outside the timed region; same inputs and outputs)
        for name, fn in meta["parts"].items():
            for _ in range(5):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(100):
                fn()
            b.record()
            b.synchronize()
            result["step"][f"{name}_us"] = a.elapsed_time(b) * 1e3 / 100
    if cpu is not None and not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample; parity of the timed step against it")
        result["cpu_baseline"], result["parity"] = run_cpu_baseline(cpu, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
