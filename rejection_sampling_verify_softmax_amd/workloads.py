"""Seeded synthetic inputs for the five verification workloads.

This module draws random numbers and nothing else: it holds none of the
verification arithmetic (no transform of logits into probabilities, no accept
test, no residual, no tree scoring, no survival product). Both the GPU library's
tests/benchmark and the CPU oracle receive the arrays made here.

Two stand-ins for systems outside the verify step live here, because their
outputs are the verify step's inputs:

* a drafter that picks each draft token y_i from its own proposal distribution
  with the Gumbel-max trick (argmax of logit/T + Gumbel noise over its kept set),
  which never forms the probabilities themselves;
* a block drafter whose per-position marginals are the softmax of Gaussian
  logits (the DDTree workload feeds these marginals in as data);
* an EAGLE-2-style drafter that proposes, for each node it is asked to
  expand, C children with their conditional probabilities (the C largest of
  a softmax of Gaussian logits over a few dozen proposals) and uniform ids.

Every generator takes a torch device. Full-size workloads are drawn on the GPU
(the host's RNG is far too slow for a billion draws); small test cases are drawn
on the CPU. Within one run the same arrays feed both sides, so the device used
for drawing does not matter for parity.

Uniforms are drawn on the grid n / 2**24, n in [0, 2**24), so that an fp32 and
an fp64 consumer see exactly the same value in [0, 1).

Workload recipes (sigma is a standard deviation throughout):

* gen_chain_small -- chain, B=1, K=4, V=1000, fp32: draft base D ~ N(0, 2) with K+1 rows; draft
  rows are D[0..K-1]; target rows are D + N(0, 0.5); T = 1.
* gen_greedy_chain -- greedy chain, B=64, K=3, V=128256, bf16 target ~ N(0, 3) with K+1 rows;
  y_i is the target argmax (lowest id) with probability 0.7, otherwise a
  uniform id.
* gen_topk_chain -- chain, B=256, K=5, V=151936, bf16 target N(0, 3) plus, per row, 20 distinct
  uniformly chosen ids boosted by 12/r (r = 1..20) before rounding; draft rows
  are bf16(target + N(0, 1)); T = 0.7, top-k 50 on both.
* gen_tree -- tree, B=32, K=16, V=32000, N=64: Z ~ N(0, 2.5) per (sequence, depth);
  marginals are softmax(Z) in fp32; the target row of a node at depth d < K is
  bf16(Z[d] + N(0, 1)), and a node at depth K gets fresh N(0, 2.5).
* gen_eagle_children -- EAGLE-2 expansion, B=32 sequences, 8 layers, W=10 nodes expanded per
  layer, C=10 children each: probabilities are the 10 largest of softmax(N(0, 2)) over 64
  proposals (largest first), tokens uniform in [0, 128256).
* gen_adaptive_chain -- adaptive chain, B=512, K_max=8, V=128256: confidences c ~ Beta(5, 2) (the
  5th smallest of 6 uniforms); draft base D ~ N(0, 2) with K_max+1 rows;
  target = bf16(D + N(0, 0.7)); draft rows bf16(D); T = 1.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

# Independent RNG streams per kind of draw, so that changing one size does not
# shift the draws of another kind.
_STREAMS = {"base": 0, "noise": 1, "draft_sample": 2, "uniform": 3,
            "boost": 4, "conf": 5, "tree_target": 6, "accept_mix": 7}


def _gen(seed: int, stream: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 16 + _STREAMS[stream])
    return g


def grid_uniforms(shape, gen: torch.Generator, device) -> torch.Tensor:
    """fp32 uniforms on the 2**-24 grid in [0, 1) (exact in fp32 and fp64)."""
    n = torch.randint(0, 1 << 24, shape, generator=gen, device=device, dtype=torch.int64)
    return (n.to(torch.float64) / float(1 << 24)).to(torch.float32)


def kept_set(logits: torch.Tensor, top_k: int) -> torch.Tensor:
    """Ids kept by a drafter that truncates to its top_k logits, ties to the lower id.

    Returns an int64 [rows, top_k] tensor. A stable sort of -logit keeps equal
    values in ascending id order.
    """
    order = torch.sort(-logits.float(), dim=-1, stable=True).indices
    return order[:, :top_k]


def gumbel_draft_tokens(draft_logits: torch.Tensor, temperature: float, top_k: int,
                        gen: torch.Generator) -> torch.Tensor:
    """Drafter stand-in: y = argmax over the kept set of (logit/T + Gumbel).

    draft_logits: [rows, V] (any float dtype). Returns int32 [rows].
    The Gumbel-max trick draws from the drafter's proposal without ever
    forming that proposal's probabilities.
    """
    rows, V = draft_logits.shape
    out = torch.empty(rows, dtype=torch.int32, device=draft_logits.device)
    step = max(1, (1 << 26) // max(V, 1))
    for r0 in range(0, rows, step):
        x = draft_logits[r0:r0 + step].to(torch.float64)
        if 0 < top_k < V:
            ids = kept_set(x, top_k)
            xs = torch.gather(x, 1, ids)
        else:
            ids = None
            xs = x
        u = torch.rand(xs.shape, generator=gen, device=xs.device, dtype=torch.float64)
        u = u.clamp_(min=1e-300, max=1.0 - 2.0 ** -53)
        score = xs / float(temperature) - torch.log(-torch.log(u))
        pick = torch.argmax(score, dim=1, keepdim=True)
        tok = pick if ids is None else torch.gather(ids, 1, pick)
        out[r0:r0 + step] = tok.squeeze(1).to(torch.int32)
    return out


def first_argmax(logits: torch.Tensor) -> torch.Tensor:
    """Lowest id among the row maxima (torch.argmax returns the first maximum)."""
    return torch.argmax(logits.float(), dim=-1).to(torch.int32)


# --------------------------------------------------------------------------
# Case containers. Logit tensors live on the generating device in their wire
# dtype (float32 or bfloat16); `.to_host()` gives float32 numpy copies for the
# oracle (bf16 -> fp32 is exact).
# --------------------------------------------------------------------------

@dataclass
class ChainCase:
    B: int
    K_max: int
    V: int
    temperature: float
    top_k: int
    target: torch.Tensor        # [R_t, V]; sequence b owns rows cu[b]+b .. cu[b+1]+b
    draft: torch.Tensor         # [R_d, V]; sequence b owns rows cu[b] .. cu[b+1]-1
    tokens: torch.Tensor        # int32 [R_d]
    uniforms: torch.Tensor      # float32 [R_t]
    cu: Optional[torch.Tensor] = None   # int32 [B+1] or None (every k_b = K_max)
    name: str = ""

    @property
    def dtype(self) -> str:
        return "bf16" if self.target.dtype == torch.bfloat16 else "f32"

    def lengths(self):
        if self.cu is None:
            return [self.K_max] * self.B
        c = self.cu.cpu().tolist()
        return [c[i + 1] - c[i] for i in range(self.B)]

    def positions(self) -> int:
        return int(sum(self.lengths()))


@dataclass
class GreedyCase:
    B: int
    K_max: int
    V: int
    target: torch.Tensor        # [R_t, V]
    tokens: torch.Tensor        # int32 [R_d]
    cu: Optional[torch.Tensor] = None
    name: str = ""


@dataclass
class TreeCase:
    B: int
    K: int
    V: int
    N: int
    marginals: torch.Tensor     # float32 [B, K, V]
    Z: torch.Tensor             # float32 [B, K, V] pre-softmax draws behind the marginals
    seed: int = 0
    name: str = ""

    def target_for_depths(self, depth: torch.Tensor, n_nodes: torch.Tensor) -> torch.Tensor:
        """bf16 target logits [B, N, V] for a tree with the given node depths.

        In a serving engine these rows come out of the target model's forward
        over the tree; here a node at depth d < K sees bf16(Z[d] + N(0, 1)) and a
        node at depth K (or an unused slot) sees fresh N(0, 2.5).
        """
        dev = self.Z.device
        g = _gen(self.seed, "tree_target", dev)
        B, N, V, K = self.B, self.N, self.V, self.K
        depth = depth.to(dev).long()
        nn = n_nodes.to(dev).long()
        out = torch.empty(B, N, V, dtype=torch.bfloat16, device=dev)
        for b in range(B):
            noise = torch.randn(N, V, generator=g, device=dev)
            fresh = torch.randn(N, V, generator=g, device=dev) * 2.5
            d = depth[b].clamp(min=0)
            used = torch.arange(N, device=dev) < nn[b]
            src = self.Z[b][d.clamp(max=K - 1)] + noise
            take_src = used & (d < K)
            rows = torch.where(take_src[:, None], src, fresh)
            out[b] = rows.to(torch.bfloat16)
        return out


@dataclass
class AdaptiveCase:
    B: int
    K_max: int
    V: int
    temperature: float
    cost: float
    conf: torch.Tensor          # float32 [B, K_max]
    target_full: torch.Tensor   # bf16 [B, K_max+1, V]
    draft_full: torch.Tensor    # bf16 [B, K_max, V]
    tokens_full: torch.Tensor   # int32 [B, K_max]
    uniforms_full: torch.Tensor  # float32 [B, K_max+1]
    name: str = ""

    def packed(self, k_sel) -> ChainCase:
        """Packed ragged chain case over the first k_sel[b] positions of each sequence.

        k_sel may come from either side's length selection; this is plain
        indexing (the rows an engine's target forward would have produced for
        the selected window). Uniform cu[b]+b+i for i < k_b drives accept test i
        and uniform cu[b]+b+k_b the final sample, exactly as in the full window.
        """
        dev = self.target_full.device
        k = torch.as_tensor(k_sel, dtype=torch.int64).to(dev)
        B, Km = self.B, self.K_max
        ar_d = torch.arange(Km, device=dev)
        ar_t = torch.arange(Km + 1, device=dev)
        dmask = ar_d[None, :] < k[:, None]             # [B, Km]
        tmask = ar_t[None, :] <= k[:, None]            # [B, Km+1]
        cu = torch.zeros(B + 1, dtype=torch.int32, device=dev)
        cu[1:] = torch.cumsum(k, 0).to(torch.int32)
        draft = self.draft_full[dmask]
        tokens = self.tokens_full[dmask]
        target = self.target_full[tmask]
        uni = self.uniforms_full[tmask]
        return ChainCase(B=B, K_max=Km, V=self.V, temperature=self.temperature, top_k=0,
                         target=target.contiguous(), draft=draft.contiguous(),
                         tokens=tokens.contiguous(), uniforms=uni.contiguous(),
                         cu=cu, name=self.name + "-packed")


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

def gen_base_noise_chain(seed: int, B: int, K: int, V: int, *, base_sigma: float,
                         noise_sigma: float, temperature: float, dtype: str,
                         top_k: int = 0, device="cpu", name: str = "") -> ChainCase:
    """The small and the adaptive chains' recipe: D ~ N(0, base_sigma) with K+1 rows per sequence,
    draft rows D[0..K-1], target rows D + N(0, noise_sigma), y ~ drafter."""
    gb, gn = _gen(seed, "base", device), _gen(seed, "noise", device)
    gs, gu = _gen(seed, "draft_sample", device), _gen(seed, "uniform", device)
    D = torch.randn(B, K + 1, V, generator=gb, device=device) * base_sigma
    tgt = D + torch.randn(B, K + 1, V, generator=gn, device=device) * noise_sigma
    wire = torch.bfloat16 if dtype == "bf16" else torch.float32
    target = tgt.to(wire).reshape(B * (K + 1), V)
    draft = D[:, :K].to(wire).reshape(B * K, V).contiguous()
    del D, tgt
    tokens = gumbel_draft_tokens(draft, temperature, top_k, gs)
    uniforms = grid_uniforms((B * (K + 1),), gu, device)
    return ChainCase(B=B, K_max=K, V=V, temperature=temperature, top_k=top_k,
                     target=target, draft=draft, tokens=tokens, uniforms=uniforms,
                     name=name)


def gen_chain_small(device="cpu", seed: int = 1001, B: int = 1, K: int = 4, V: int = 1000) -> ChainCase:
    return gen_base_noise_chain(seed, B, K, V, base_sigma=2.0, noise_sigma=0.5,
                                temperature=1.0, dtype="f32", device=device,
                                name=f"chain-f32-B{B}-K{K}-V{V}")


def gen_greedy_chain(device="cpu", seed: int = 1002, B: int = 64, K: int = 3, V: int = 128256) -> GreedyCase:
    gb, gm, gs = _gen(seed, "base", device), _gen(seed, "accept_mix", device), _gen(seed, "draft_sample", device)
    tgt = (torch.randn(B, K + 1, V, generator=gb, device=device) * 3.0).to(torch.bfloat16)
    amax = first_argmax(tgt[:, :K].reshape(B * K, V))
    take = torch.rand(B * K, generator=gm, device=device) < 0.7
    rand_ids = torch.randint(0, V, (B * K,), generator=gs, device=device, dtype=torch.int32)
    tokens = torch.where(take, amax, rand_ids).to(torch.int32)
    return GreedyCase(B=B, K_max=K, V=V, target=tgt.reshape(B * (K + 1), V), tokens=tokens,
                      name=f"greedy-bf16-B{B}-K{K}-V{V}")


def gen_topk_chain(device="cpu", seed: int = 1003, B: int = 256, K: int = 5, V: int = 151936,
                top_k: int = 50, n_boost: int = 20, temperature: float = 0.7) -> ChainCase:
    gb, gn = _gen(seed, "base", device), _gen(seed, "noise", device)
    gx, gs, gu = _gen(seed, "boost", device), _gen(seed, "draft_sample", device), _gen(seed, "uniform", device)
    rows = B * (K + 1)
    tgt = torch.randn(rows, V, generator=gb, device=device) * 3.0
    nb = min(n_boost, V)
    # distinct boosted ids per row: the nb smallest of V iid uniform keys
    ids = torch.empty(rows, nb, dtype=torch.int64, device=device)
    step = max(1, (1 << 25) // V)
    for r0 in range(0, rows, step):
        keys = torch.rand(min(step, rows - r0), V, generator=gx, device=device)
        ids[r0:r0 + step] = torch.topk(keys, nb, dim=1, largest=False).indices
    boost = 12.0 / torch.arange(1, nb + 1, device=device, dtype=torch.float32)
    tgt.scatter_add_(1, ids, boost.expand(rows, nb).contiguous())
    target = tgt.to(torch.bfloat16)
    del tgt
    t3 = target.reshape(B, K + 1, V)
    draft = (t3[:, :K].float() + torch.randn(B, K, V, generator=gn, device=device)).to(torch.bfloat16)
    draft = draft.reshape(B * K, V).contiguous()
    tokens = gumbel_draft_tokens(draft, temperature, top_k, gs)
    uniforms = grid_uniforms((rows,), gu, device)
    return ChainCase(B=B, K_max=K, V=V, temperature=temperature, top_k=top_k,
                     target=target, draft=draft, tokens=tokens, uniforms=uniforms,
                     name=f"chain-topk{top_k}-bf16-B{B}-K{K}-V{V}")


def gen_tree(device="cpu", seed: int = 1004, B: int = 32, K: int = 16, V: int = 32000,
                N: int = 64, sigma: float = 2.5) -> TreeCase:
    gb = _gen(seed, "base", device)
    Z = torch.randn(B, K, V, generator=gb, device=device) * sigma
    marg = torch.softmax(Z, dim=-1).to(torch.float32).contiguous()
    return TreeCase(B=B, K=K, V=V, N=N, marginals=marg, Z=Z, seed=seed,
                    name=f"tree-B{B}-K{K}-V{V}-N{N}")


def gen_eagle_children(device="cpu", seed: int = 1006, B: int = 32, layers: int = 8, W: int = 10,
                       C: int = 10, V: int = 128256, width: int = 64, sigma: float = 2.0):
    """Stand-in drafter outputs for the EAGLE-2 expansion steps: per layer a pair
    (child_token [B, W, C] int32, child_prob [B, W, C] fp32), slot w holding the
    children of the node expanded in that slot."""
    gb, gt = _gen(seed, "base", device), _gen(seed, "draft_sample", device)
    z = torch.randn(layers, B, W, width, generator=gb, device=device) * sigma
    probs = torch.topk(torch.softmax(z, dim=-1), C, dim=-1).values.to(torch.float32)
    tokens = torch.randint(0, V, (layers, B, W, C), generator=gt, device=device, dtype=torch.int32)
    return [(tokens[i].contiguous(), probs[i].contiguous()) for i in range(layers)]


def gen_adaptive_chain(device="cpu", seed: int = 1005, B: int = 512, K: int = 8, V: int = 128256,
                cost: float = 0.15) -> AdaptiveCase:
    gc = _gen(seed, "conf", device)
    six = torch.rand(B, K, 6, generator=gc, device=device)
    conf = torch.sort(six, dim=-1).values[..., 4].contiguous()    # Beta(5, 2)
    base = gen_base_noise_chain(seed, B, K, V, base_sigma=2.0, noise_sigma=0.7,
                                temperature=1.0, dtype="bf16", device=device)
    return AdaptiveCase(B=B, K_max=K, V=V, temperature=1.0, cost=cost, conf=conf,
                        target_full=base.target.reshape(B, K + 1, V),
                        draft_full=base.draft.reshape(B, K, V),
                        tokens_full=base.tokens.reshape(B, K),
                        uniforms_full=base.uniforms.reshape(B, K + 1),
                        name=f"adaptive-bf16-B{B}-K{K}-V{V}")


def ragged_chain(seed: int, lengths, V: int, *, dtype: str = "bf16", temperature: float = 1.0,
                 top_k: int = 0, base_sigma: float = 2.0, noise_sigma: float = 0.7,
                 device="cpu") -> ChainCase:
    """A packed chain case with the given per-sequence draft lengths (any k_b >= 0)."""
    lengths = [int(k) for k in lengths]
    B, Km = len(lengths), max(lengths) if lengths else 0
    full = gen_base_noise_chain(seed, B, Km, V, base_sigma=base_sigma, noise_sigma=noise_sigma,
                                temperature=temperature, dtype=dtype, top_k=top_k, device=device)
    ad = AdaptiveCase(B=B, K_max=Km, V=V, temperature=temperature, cost=0.0,
                      conf=torch.zeros(B, Km), target_full=full.target.reshape(B, Km + 1, V),
                      draft_full=full.draft.reshape(B, Km, V),
                      tokens_full=full.tokens.reshape(B, Km),
                      uniforms_full=full.uniforms.reshape(B, Km + 1))
    c = ad.packed(lengths)
    c.top_k = top_k
    c.name = f"ragged-{dtype}-B{B}-V{V}"
    return c


def to_host_f32(t: torch.Tensor):
    """float32 numpy copy (bf16 -> fp32 is exact)."""
    return t.detach().float().cpu().contiguous().numpy()
