"""Seeded synthetic inputs for the EAGLE-3 draft-tree and tree-verification round.

This module only draws numbers and builds tree topologies; it contains none of the
method's arithmetic (no fusion, norm, RoPE, attention, softmax, selection or acceptance).
Both the HIP path and the CPU oracle are fed from here, so the same seed gives the same
inputs on either side.

Shapes follow the five workloads this library is exercised on (weights N(0, 1/fan_in),
embedding N(0, 1), norm gains 1, hidden states / KV / queries N(0, 1), tokens uniform).
bf16 tensors are the round-to-nearest-even of float32 draws.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

# ---------------------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    dtype: str          # "f32" or "bf16": activations, weights, KV and logits
    B: int              # requests
    d: int              # target / drafter hidden size
    Hq: int
    Hkv: int
    Dh: int
    F: int              # drafter FFN width (SiLU-gated)
    V: int              # vocabulary
    prefix: tuple       # ("fixed", P) or ("uniform", lo, hi)
    depth: int          # D: draft depth
    topk: int           # K: children per expanded node
    width: int          # W: nodes expanded per depth
    n_nodes: int        # N: draft nodes kept after the final prune
    noise: float        # sigma of target-logit noise around draft logits
    temperature: float  # acceptance temperature (0 = greedy)
    verify_tree: str    # "draft" (verify the drafted tree) or "random" (random topology)
    verify_max_nodes: int = 0
    verify_max_depth: int = 0
    branch: int = 0     # long-context branch length (chain)


TINY = Shape("tiny_fp32", "f32", 1, 256, 4, 4, 64, 1024, 1024, ("fixed", 128),
             3, 2, 4, 14, 0.5, 1.0, "draft")
LLAMA8B = Shape("llama8b_bf16", "bf16", 1, 4096, 32, 8, 128, 14336, 128256, ("fixed", 2048),
                6, 10, 10, 60, 1.0, 0.0, "draft")
BATCH16 = Shape("batch16_ragged_bf16", "bf16", 16, 4096, 32, 8, 128, 14336, 128256,
                ("uniform", 512, 4096), 6, 10, 10, 48, 1.0, 0.0, "random",
                verify_max_nodes=48, verify_max_depth=6)
LLAMA70B = Shape("llama70b_bf16", "bf16", 4, 8192, 64, 8, 128, 28672, 128256, ("fixed", 8192),
                 6, 10, 10, 60, 1.0, 0.7, "draft")
LONGCTX = Shape("longctx_branch_bf16", "bf16", 1, 4096, 32, 8, 128, 14336, 128256,
                ("fixed", 65536), 0, 0, 0, 0, 0.0, 0.0, "chain", branch=7)

SHAPES = {s.name: s for s in (TINY, LLAMA8B, BATCH16, LLAMA70B, LONGCTX)}


def scaled(shape: Shape, **kw) -> Shape:
    """A copy of `shape` with some fields replaced (used for reduced-size parity cases)."""
    return dataclasses.replace(shape, **kw)


def torch_dtype(shape: Shape) -> torch.dtype:
    return torch.float32 if shape.dtype == "f32" else torch.bfloat16


# ---------------------------------------------------------------------------------------
# Drawing helpers
# ---------------------------------------------------------------------------------------


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal(shape, std, seed, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """N(0, std^2) drawn in float32, then rounded (RNE) to `dtype`."""
    dev = torch.device(device)
    x = torch.randn(shape, generator=_gen(seed, dev), dtype=torch.float32, device=dev)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform_int(n, high, seed, device="cpu") -> torch.Tensor:
    dev = torch.device(device)
    return torch.randint(0, high, (n,), generator=_gen(seed, dev), dtype=torch.int32, device=dev)


# ---------------------------------------------------------------------------------------
# Drafter weights (layout: every projection is [out_features, in_features], row-major)
# ---------------------------------------------------------------------------------------


def drafter_weights(shape: Shape, seed: int = 1234, device="cpu") -> dict:
    dt = torch_dtype(shape)
    d, Hq, Hkv, Dh, F, V = shape.d, shape.Hq, shape.Hkv, shape.Dh, shape.F, shape.V
    nqkv = (Hq + 2 * Hkv) * Dh
    w = {
        "embed": normal((V, d), 1.0, seed + 1, dt, device),
        "w_fuse": normal((d, 3 * d), 1.0 / math.sqrt(3 * d), seed + 2, dt, device),
        "w_qkv": normal((nqkv, 2 * d), 1.0 / math.sqrt(2 * d), seed + 3, dt, device),
        "w_o": normal((d, Hq * Dh), 1.0 / math.sqrt(Hq * Dh), seed + 4, dt, device),
        "w_gate_up": normal((2 * F, d), 1.0 / math.sqrt(d), seed + 5, dt, device),
        "w_down": normal((d, F), 1.0 / math.sqrt(F), seed + 6, dt, device),
        "w_lm": normal((V, d), 1.0 / math.sqrt(d), seed + 7, dt, device),
    }
    for k in ("g_embed", "g_feat", "g_mlp", "g_final"):
        w[k] = torch.ones(d, dtype=dt, device=device)
    return w


# ---------------------------------------------------------------------------------------
# Per-request prefix lengths and draft-side inputs
# ---------------------------------------------------------------------------------------


def prefix_lengths(shape: Shape, seed: int) -> List[int]:
    if shape.prefix[0] == "fixed":
        return [int(shape.prefix[1])] * shape.B
    lo, hi = int(shape.prefix[1]), int(shape.prefix[2])
    g = _gen(seed + 11)
    return [int(v) for v in torch.randint(lo, hi + 1, (shape.B,), generator=g)]


def cu_from_lengths(lengths: List[int]) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def draft_inputs(shape: Shape, seed: int = 99, device="cpu", prefix: Optional[List[int]] = None) -> dict:
    dt = torch_dtype(shape)
    P = prefix if prefix is not None else prefix_lengths(shape, seed)
    total = sum(P)
    return {
        "h_low": normal((shape.B, shape.d), 1.0, seed + 1, dt, device),
        "h_mid": normal((shape.B, shape.d), 1.0, seed + 2, dt, device),
        "h_high": normal((shape.B, shape.d), 1.0, seed + 3, dt, device),
        "root_tok": uniform_int(shape.B, shape.V, seed + 4, device),
        "kpre": normal((total, shape.Hkv, shape.Dh), 1.0, seed + 5, dt, device),
        "vpre": normal((total, shape.Hkv, shape.Dh), 1.0, seed + 6, dt, device),
        "prefix": P,
        "cu_prefix": cu_from_lengths(P).to(device),
    }


# ---------------------------------------------------------------------------------------
# Tree topologies (parents are request-local, root = node 0 with parent -1,
# every parent index is smaller than its child's)
# ---------------------------------------------------------------------------------------


def random_tree(n_nodes: int, max_depth: int, seed: int) -> List[int]:
    """Parents of a random tree: node i's parent is uniform among earlier nodes whose
    depth is below `max_depth` (so no node is deeper than `max_depth`)."""
    g = _gen(seed)
    parents = [-1]
    depth = [0]
    for i in range(1, n_nodes):
        allowed = [j for j in range(i) if depth[j] < max_depth]
        j = allowed[int(torch.randint(0, len(allowed), (1,), generator=g))]
        parents.append(j)
        depth.append(depth[j] + 1)
    return parents


def chain_tree(n_nodes: int) -> List[int]:
    return [-1] + list(range(n_nodes - 1))


def star_tree(n_nodes: int) -> List[int]:
    return [-1] + [0] * (n_nodes - 1)


def full_tree(k: int, depth: int) -> List[int]:
    """Level-ordered full k-ary tree of the given depth (root included)."""
    parents = [-1]
    level = [0]
    for _ in range(depth):
        nxt = []
        for p in level:
            for _ in range(k):
                parents.append(p)
                nxt.append(len(parents) - 1)
        level = nxt
    return parents


def verify_inputs(shape: Shape, trees: List[List[int]], prefix: List[int], seed: int = 77,
                  device="cpu", with_logits: bool = True) -> dict:
    """Verify-layer tensors for the given trees: queries and tree K/V for every node,
    an independent prefix KV, and N(0, 1) target logits (callers may overwrite them)."""
    dt = torch_dtype(shape)
    n = [len(t) for t in trees]
    T = sum(n)
    out = {
        "parents": torch.tensor([p for t in trees for p in t], dtype=torch.int32, device=device),
        "cu_nodes": cu_from_lengths(n).to(device),
        "q": normal((T, shape.Hq, shape.Dh), 1.0, seed + 1, dt, device),
        "k_tree": normal((T, shape.Hkv, shape.Dh), 1.0, seed + 2, dt, device),
        "v_tree": normal((T, shape.Hkv, shape.Dh), 1.0, seed + 3, dt, device),
        "kpre": normal((sum(prefix), shape.Hkv, shape.Dh), 1.0, seed + 4, dt, device),
        "vpre": normal((sum(prefix), shape.Hkv, shape.Dh), 1.0, seed + 5, dt, device),
        "cu_prefix": cu_from_lengths(prefix).to(device),
        "prefix": list(prefix),
        "T": T,
    }
    if with_logits:
        out["logits"] = normal((T, shape.V), 1.0, seed + 6, dt, device)
    out["tokens"] = uniform_int(T, shape.V, seed + 7, device)
    return out


def sampled_tree_inputs(trees: List[List[int]], V: int, seed: int, dtype=torch.bfloat16,
                        device="cpu", n_hot: int = 16, hot_boost: float = 6.0,
                        target_noise: float = 0.5) -> dict:
    """Inputs of one acceptance round over sampled candidates.  Every node with children gets
    a draft logit row: N(0, 1) plus `hot_boost` on `n_hot` random tokens; its children carry
    distinct tokens of that hot set (uniform without replacement; beyond n_hot children the
    rest are distinct uniform tokens).  A node's target logits are its draft row plus
    N(0, target_noise^2); a node without children gets a fresh hot-boosted row and draft row
    -1.  Returns cu_nodes, tokens, parents, logits [T, V], draft_logits [R, V], draft_row [T]."""
    g = _gen(seed)
    parents = [p for t in trees for p in t]
    T = len(parents)
    tokens = torch.zeros(T, dtype=torch.int32)
    draft_row = torch.full((T,), -1, dtype=torch.int32)
    zq_rows, z = [], torch.empty((T, V), dtype=torch.float32)

    def hot_row():
        row = torch.randn(V, generator=g)
        hot = torch.randperm(V, generator=g)[:n_hot]
        row[hot] += hot_boost
        return row, hot

    n0 = 0
    for t in trees:
        kids = {}
        for j in range(1, len(t)):
            kids.setdefault(t[j], []).append(j)
        for i in range(len(t)):
            row, hot = hot_row()
            ch = kids.get(i, [])
            if ch:
                draft_row[n0 + i] = len(zq_rows)
                zq_rows.append(row)
                pick = hot[torch.randperm(len(hot), generator=g)].tolist()
                while len(pick) < len(ch):
                    x = int(torch.randint(0, V, (1,), generator=g))
                    if x not in pick:
                        pick.append(x)
                for c, x in zip(ch, pick):
                    tokens[n0 + c] = x
                z[n0 + i] = row + target_noise * torch.randn(V, generator=g)
            else:
                z[n0 + i] = row
        n0 += len(t)
    zq = torch.stack(zq_rows) if zq_rows else torch.zeros((1, V))
    return {"cu_nodes": cu_from_lengths([len(t) for t in trees]).to(device),
            "tokens": tokens.to(device), "parents": torch.tensor(parents, dtype=torch.int32, device=device),
            "logits": z.to(dtype).to(device), "draft_logits": zq.to(dtype).to(device),
            "draft_row": draft_row.to(device), "T": T}


def plant_path(logits: torch.Tensor, tokens: torch.Tensor, parents: List[int], node0: int,
               end_node: int, bump: float = 1.0) -> None:
    """Make the root->end_node path of one request the target's greedy choice: for every
    edge (parent -> child) on it, raise the parent's logit at the child's token to the
    row maximum plus `bump`.  `node0` is the request's first global node index."""
    j = end_node
    while parents[j] >= 0:
        p = parents[j]
        row = logits[node0 + p]
        tok = int(tokens[node0 + j])
        row[tok] = (row.float().max() + bump).to(row.dtype)
        j = p
