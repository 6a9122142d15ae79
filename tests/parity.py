"""Shared helpers of the GPU parity tests: run the oracle on (a sample of) a
case and compare it with the library's outputs.

Parity rule (the tolerance regime stated for this path):
* accepted length, next token and status bit-exact, except sequences the
  oracle flags as margin cases (an accept test with |u q - p| < 1e-6 p, or a
  sampled point within 1e-6 of a CDF step); those are counted and returned,
  and still checked: the GPU's result must be one that rounding allows
  (oracle.check_chain: every accepted position passes the ratio test and the
  rejected one fails it, each within 1e-6 relative, and the next token lies in
  the fp64 CDF interval of the chain rule's final draw at that A, widened by
  1e-6 of the total); where only the final draw is at a margin, the accepted
  length and the status must still match exactly;
* p_i(y_i), q_i(y_i) and the residual mass within 1e-5 relative; values below
  1e-30 must be below 1e-30 on both sides.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from rejection_sampling_verify_softmax_amd import workloads as wl

REL_TOL = 1e-5
TINY = 1e-30


def seq_layout(case):
    """(cu as numpy int64 [B+1]) for a dense or packed chain case."""
    if case.cu is None:
        return np.arange(case.B + 1, dtype=np.int64) * case.K_max
    return case.cu.cpu().numpy().astype(np.int64)


def subset_host(case, seqs):
    """Host float32 copies of the rows of the chosen sequences, re-packed."""
    cu = seq_layout(case)
    seqs = [int(b) for b in seqs]
    t_rows = np.concatenate([np.arange(cu[b] + b, cu[b + 1] + b + 1) for b in seqs])
    d_parts = [np.arange(cu[b], cu[b + 1]) for b in seqs]
    d_rows = np.concatenate(d_parts) if d_parts else np.zeros(0, np.int64)
    dev = case.target.device
    ti = torch.as_tensor(t_rows, device=dev)
    di = torch.as_tensor(d_rows, device=dev)
    lens = [cu[b + 1] - cu[b] for b in seqs]
    new_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = {
        "target": wl.to_host_f32(case.target.index_select(0, ti)),
        "tokens": case.tokens.index_select(0, di).cpu().numpy() if len(d_rows) else np.zeros(0, np.int32),
        "cu": new_cu,
        "B": len(seqs),
        "K_max": int(max(lens)) if lens else 0,
        "d_rows": d_rows,
    }
    if getattr(case, "draft", None) is not None:
        out["draft"] = (wl.to_host_f32(case.draft.index_select(0, di)) if len(d_rows)
                        else np.zeros((0, case.V), np.float32))
    if getattr(case, "uniforms", None) is not None:
        out["uniforms"] = case.uniforms.index_select(0, ti).cpu().numpy()
    return out


def oracle_chain(case, seqs=None):
    seqs = list(range(case.B)) if seqs is None else list(seqs)
    h = subset_host(case, seqs)
    ref = oracle.verify_chain(h["target"], h["draft"], h["tokens"], h["uniforms"], h["cu"], h["B"],
                              h["K_max"], case.V, case.temperature, case.top_k)
    ref["seqs"] = np.array(seqs)
    ref["d_rows"] = h["d_rows"]
    ref["host"] = h
    ref["V"], ref["temperature"], ref["top_k"] = case.V, case.temperature, case.top_k
    return ref


def repack_host(h, idx):
    """The host rows of the sequences idx (positions within h), re-packed."""
    cu = h["cu"].astype(np.int64)
    idx = [int(i) for i in idx]
    t_rows = np.concatenate([np.arange(cu[i] + i, cu[i + 1] + i + 1) for i in idx])
    d_parts = [np.arange(cu[i], cu[i + 1]) for i in idx]
    d_rows = np.concatenate(d_parts) if d_parts else np.zeros(0, np.int64)
    lens = [int(cu[i + 1] - cu[i]) for i in idx]
    return {"target": h["target"][t_rows], "draft": h["draft"][d_rows], "tokens": h["tokens"][d_rows],
            "uniforms": h["uniforms"][t_rows], "B": len(idx), "K_max": max(lens) if lens else 0,
            "cu": np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)}


def check_margin_cases(ref, A, nx, st, idx):
    """Asserts that the GPU's results on the oracle's margin cases idx
    (positions within ref's sample) are results that rounding allows."""
    if len(idx) == 0:
        return
    h = repack_host(ref["host"], idx)
    valid, st_exp = oracle.check_chain(h["target"], h["draft"], h["tokens"], h["uniforms"], h["cu"],
                                       h["B"], h["K_max"], ref["V"], ref["temperature"], A[idx], nx[idx],
                                       top_k=ref["top_k"])
    seqs = ref["seqs"][idx]
    bad = valid != 3
    assert not bad.any(), (f"margin cases not allowed by rounding, seqs {seqs[bad][:5]}: "
                           f"gpu A/next={A[idx][bad][:5]}/{nx[idx][bad][:5]} check bits {valid[bad][:5]} "
                           f"oracle A/next={ref['A'][idx][bad][:5]}/{ref['next'][idx][bad][:5]}")
    bad = st[idx] != st_exp
    assert not bad.any(), f"status on margin cases, seqs {seqs[bad][:5]}: {st[idx][bad][:5]} vs {st_exp[bad][:5]}"
    # a margin in the final draw alone leaves the accept decisions exact
    sample_only = (ref["margin"][idx] & oracle.MARGIN_ACCEPT) == 0
    bad = sample_only & (A[idx] != ref["A"][idx])
    assert not bad.any(), f"accepted length differs where only the draw is at a margin: seqs {seqs[bad][:5]}"


def close_rel(a, b, tol=REL_TOL):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    tiny = (np.abs(a) < TINY) & (np.abs(b) < TINY)
    rel = np.abs(a - b) / np.maximum(np.abs(b), TINY)
    bad = ~tiny & ~(rel <= tol)
    return not bad.any(), (rel[~tiny].max() if (~tiny).any() else 0.0)


def compare_chain(gpu: dict, ref: dict, check_probs=True, check_resid=True) -> dict:
    """Assert parity on the oracle's sample; returns counts for reporting."""
    seqs = ref["seqs"]
    A = gpu["accepted_len"].cpu().numpy()[seqs]
    nx = gpu["next_token"].cpu().numpy()[seqs]
    st = gpu["status"].cpu().numpy()[seqs]
    margin = ref["margin"] != 0
    ok = ~margin
    bad = np.nonzero(ok & ((A != ref["A"]) | (nx != ref["next"]) | (st != ref["status"])))[0]
    assert len(bad) == 0, (
        f"{len(bad)} non-margin mismatches, first seqs {seqs[bad[:5]]}: "
        f"gpu A/next/st={A[bad[:5]]}/{nx[bad[:5]]}/{st[bad[:5]]} "
        f"oracle={ref['A'][bad[:5]]}/{ref['next'][bad[:5]]}/{ref['status'][bad[:5]]}")
    info = {"seqs": len(seqs), "margin": int(margin.sum()),
            "margin_mismatch": int((margin & ((A != ref["A"]) | (nx != ref["next"]))).sum())}
    if "host" in ref and ref["temperature"] != 0.0:
        check_margin_cases(ref, A, nx, st, np.nonzero(margin)[0])
    if check_probs and "probs" in gpu and len(ref["d_rows"]):
        pg = gpu["probs"].cpu().numpy()[ref["d_rows"]]
        good, worst = close_rel(pg, ref["probs"])
        assert good, f"p(y)/q(y) beyond {REL_TOL} relative (worst {worst:.3e})"
        info["probs_rel"] = float(worst)
    if check_resid and "resid" in gpu:
        rg = gpu["resid"].cpu().numpy()[seqs]
        same = ok | (A == ref["A"])          # R depends on A only, not on the final draw
        good, worst = close_rel(rg[same], ref["R"][same])
        assert good, f"residual mass beyond {REL_TOL} relative (worst {worst:.3e})"
        info["resid_rel"] = float(worst)
    return info


def sample_seqs(B, n, seed=0):
    if B <= n:
        return list(range(B))
    rng = np.random.default_rng(seed)
    s = set(rng.choice(B, size=n, replace=False).tolist())
    s.update([0, B - 1])
    return sorted(s)
