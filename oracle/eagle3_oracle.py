"""CPU oracle for one EAGLE-3 draft-tree round and one tree-verification round.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, obviously-correct restatement of
what the method computes.  It is imported only by tests/, by __graft_entry__.smoke() (to
check the GPU result) and by bench.py's cpu_baseline leg.  The product path (the HIP
library and its Python binding) never imports, calls or links it, and it shares no code
with that path: its inputs are plain numpy arrays.

Precision: floating-point arithmetic runs in float64 on the exact upcast of the (bf16 or
fp32) inputs.  Where a floating-point value decides an integer result (draft scores that
drive selection, the Gumbel perturbation that drives sampling), the decision is made in
float32, the precision of the kernels, with every operation rounded separately.

Sources (the pages this restates):
  [P1] "EAGLE-3: Training-time Test 的投机推理加速" (paper deep-dive page):
       sections 论文位置, 推理流程：多层特征融合 + 单层 draft decoder,
       训练细节 (component table), Draft tree 配置.
  [P2] EAGLE 系列演进 page (EAGLE-1 -> EAGLE-2 -> EAGLE-3, DFlash): section
       二、EAGLE-2动态草稿树 (K=3 expansion, flattening, positional encoding, 0/1 tree
       mask, one-pass verification, rollback).
  [P3] "SpecForge：把 EAGLE3 从训练样本交付到 SGLang": sections
       多层特征融合到底融合了什么 (g_t = W_f[h_low;h_mid;h_high], a_{t+1} = D(e(x_t), g_t)),
       第二步为什么没有“正确隐藏状态”可用 (later steps feed the drafter output a),
       从序列到动态草稿树 (ancestor-only tree attention), 先看 checkpoint 最终要参与什么计算
       (accept the continuous prefix, correct at the rejection).
  [P4] "EAGLE-3 投机解码与 USP 长序列训练优化": section USP 核心设计：三步走
       (Out_main/LSE_main, Out_branch/LSE_branch, streaming-softmax fusion).
  [P5] speculative-decoding thinking-budget page: section 一棵候选树怎样被验证
       (assign positions, ancestor-only mask, one forward, accept by target
       probabilities, commit only the path).

Readings where the pages are silent (each is listed with its reason in the design notes):
Llama-style drafter layer (RMSNorm eps 1e-5, no biases, half-split RoPE with
theta 500000, final RMSNorm before the LM head); embedding and feature concatenated into
a 2d-wide QKV input; tree expansion by per-depth top-W of cumulative log-probability; the
stochastic acceptance rule in its deterministic-candidate form (Gumbel-max draw of the
target token at every node, descend while the draw equals a child token); in its
sampled-candidate form, siblings drawn without replacement and tested in the order drawn,
each rejection taking its token out of q and replacing p by the normalised positive part
of p - q (the probabilities of that form in float64).
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")

# =======================================================================================
# Elementary pieces of the drafter layer
# =======================================================================================


def f64(x) -> np.ndarray:
    """Exact upcast of an array-like (numpy, or a torch tensor via .numpy()) to float64."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma (reading of the
    'single decoder layer' in [P1] 训练细节 as a Llama-style layer)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def project(x, w) -> np.ndarray:
    """One projection of the drafter, y = x W^T with W stored [out, in] (the fusion W_f of
    [P3] 多层特征融合到底融合了什么; the QKV, O and MLP projections of the single decoder
    layer and the LM head, [P1] 训练细节), in float64 on the exact upcast of the inputs."""
    return f64(x) @ f64(w).T


def fuse_features(h_low, h_mid, h_high, w_fuse) -> np.ndarray:
    """[P3] 多层特征融合到底融合了什么 / [P1] 推理流程: concatenate the low, middle and
    high target features (3k wide) and project back to k with one fully connected layer:
    g = W_f [h_low; h_mid; h_high].  w_fuse is stored [d, 3d] (out x in)."""
    x = np.concatenate([h_low, h_mid, h_high], axis=-1)
    return x @ w_fuse.T


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary position embedding on the last axis (Dh), half-split pairs (i, i + Dh/2),
    angle pos * theta^(-2i/Dh).  Positions carry the tree structure ([P2] 位置编码,
    [P5] 给节点分配 position): a node at tree depth t sits at prefix_len + t."""
    Dh = x.shape[-1]
    half = Dh // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / Dh)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def log_sum_exp(z: np.ndarray) -> float:
    """ln sum_t e^{z_t}, max-shifted."""
    m = np.max(z)
    return float(m + np.log(np.sum(np.exp(z - m))))


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
           visible: Optional[np.ndarray] = None) -> Tuple[np.ndarray, float]:
    """Softmax attention of one query over an explicit key list (two passes: scores and
    max, then weights).  Keys outside `visible` get weight exactly 0.  Returns (o, lse)
    with lse = ln sum_j e^{scale q.k_j} over the visible keys; an empty key set gives
    (0, -inf)."""
    if visible is None:
        visible = np.ones(keys.shape[0], dtype=bool)
    if keys.shape[0] == 0 or not np.any(visible):
        return np.zeros(values.shape[-1]), NEG_INF
    s = (keys @ q) * scale
    m = np.max(s[visible])
    w = np.zeros_like(s)
    w[visible] = np.exp(s[visible] - m)
    tot = np.sum(w)
    return (w @ values) / tot, float(m + np.log(tot))


def attend_rows(Q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                visible: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """`attend` for many queries that share one key list, each with its own visibility
    row (visible[r, j]).  Same definition, evaluated with matrix products."""
    R = Q.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((R, values.shape[-1])), np.full(R, NEG_INF)
    S = (Q @ keys.T) * scale
    S = np.where(visible, S, NEG_INF)
    m = np.max(S, axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    Wt = np.where(visible, np.exp(S - m_safe[:, None]), 0.0)
    tot = np.sum(Wt, axis=1)
    O = np.zeros((R, values.shape[-1]))
    O[has] = (Wt[has] @ values) / tot[has, None]
    lse = np.full(R, NEG_INF)
    lse[has] = m[has] + np.log(tot[has])
    return O, lse


def topk_desc(z: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k of one row ordered by (value descending, token id ascending)."""
    ids = np.arange(z.shape[0])
    order = np.lexsort((ids, -z))
    sel = order[:k]
    return sel.astype(np.int64), z[sel]


# =======================================================================================
# O2: one drafter node (a single decoder layer, [P1] 训练细节 / [P3] a = D(e(x), g))
# =======================================================================================


class Drafter:
    """Drafter weights upcast to float64.  Layout of every projection: [out, in]."""

    def __init__(self, w: Dict[str, object], Hq: int, Hkv: int, Dh: int,
                 eps: float = 1e-5, theta: float = 500000.0):
        self.embed = f64(w["embed"])
        self.w_fuse = f64(w["w_fuse"])
        self.w_qkv = f64(w["w_qkv"])
        self.w_o = f64(w["w_o"])
        self.w_gate_up = f64(w["w_gate_up"])
        self.w_down = f64(w["w_down"])
        self.w_lm = f64(w["w_lm"])
        self.g_embed = f64(w["g_embed"])
        self.g_feat = f64(w["g_feat"])
        self.g_mlp = f64(w["g_mlp"])
        self.g_final = f64(w["g_final"])
        self.Hq, self.Hkv, self.Dh = Hq, Hkv, Dh
        self.d = self.embed.shape[1]
        self.F = self.w_down.shape[1]
        self.eps, self.theta = eps, theta
        self.scale = float(np.float32(1.0 / math.sqrt(Dh)))

    def qkv(self, tokens: Sequence[int], feats: np.ndarray, pos: Sequence[int]):
        """Input u = [rms(E[x]) * g_e ; rms(f) * g_f] (2d wide), then q, k, v with RoPE."""
        e = self.embed[np.asarray(tokens, dtype=np.int64)]
        u = np.concatenate([rmsnorm(e, self.g_embed, self.eps),
                            rmsnorm(feats, self.g_feat, self.eps)], axis=-1)
        y = u @ self.w_qkv.T
        Hq, Hkv, Dh = self.Hq, self.Hkv, self.Dh
        q = y[:, :Hq * Dh].reshape(-1, Hq, Dh)
        k = y[:, Hq * Dh:(Hq + Hkv) * Dh].reshape(-1, Hkv, Dh)
        v = y[:, (Hq + Hkv) * Dh:].reshape(-1, Hkv, Dh)
        q = np.stack([rope(q[r], pos[r], self.theta) for r in range(q.shape[0])])
        k = np.stack([rope(k[r], pos[r], self.theta) for r in range(k.shape[0])])
        return q, k, v

    def after_attention(self, feats: np.ndarray, attn: np.ndarray):
        """O projection + residual on the feature stream, SiLU-gated MLP + residual, final
        norm, LM head, log-sum-exp.  Returns (a, z, lse)."""
        h1 = feats + attn @ self.w_o.T
        m = rmsnorm(h1, self.g_mlp, self.eps)
        gu = m @ self.w_gate_up.T
        t = silu(gu[:, :self.F]) * gu[:, self.F:]
        a = h1 + t @ self.w_down.T
        z = rmsnorm(a, self.g_final, self.eps) @ self.w_lm.T
        lse = np.array([log_sum_exp(z[r]) for r in range(z.shape[0])])
        return a, z, lse

    def forward_nodes(self, tokens, feats, pos, kpre: np.ndarray, vpre: np.ndarray,
                      anc_k: List[np.ndarray], anc_v: List[np.ndarray]):
        """Evaluate several nodes of one request.  Node r attends, per query head h (KV head
        h // (Hq/Hkv)), to the drafter prefix keys followed by its ancestors' keys
        (anc_k[r]: [n_anc, Hkv, Dh], root first) and its own key.
        Returns dict(k, v, a, z, lse) with k, v the nodes' own keys/values."""
        feats = np.asarray(feats, dtype=np.float64)
        q, k, v = self.qkv(tokens, feats, pos)
        G = self.Hq // self.Hkv
        attn = np.zeros((len(tokens), self.Hq * self.Dh))
        for r in range(len(tokens)):
            keys = np.concatenate([kpre, anc_k[r], k[r:r + 1]], axis=0)
            vals = np.concatenate([vpre, anc_v[r], v[r:r + 1]], axis=0)
            for h in range(self.Hq):
                c = h // G
                o, _ = attend(q[r, h], keys[:, c, :], vals[:, c, :], self.scale)
                attn[r, h * self.Dh:(h + 1) * self.Dh] = o
        a, z, lse = self.after_attention(feats, attn)
        return {"k": k, "v": v, "a": a, "z": z, "lse": lse, "q": q, "attn": attn}


# =======================================================================================
# O3: dynamic draft tree ([P1] Draft tree 配置, [P2] 二、EAGLE-2动态草稿树,
#     [P3] 从序列到动态草稿树)
# =======================================================================================
#
# Per request: the root (root token, fused feature g, depth 0, score 0) is evaluated first.
# Every evaluated node v creates its top-K children (value desc, id asc) with cumulative
# log-probability  s_child = s_v + (z_v[t] - lse_v)  computed in float32.  Candidates get
# a creation index that increases in generation order.  At depth t = 1 .. D-1 the top-W
# depth-t candidates by (s desc, creation asc) are evaluated (in that rank order, which is
# also the order their children are created in), each with feature a_parent and position
# prefix_len + t, attending to the drafter prefix plus its evaluated ancestors and itself.
# After D evaluation steps the top-N candidates of the whole pool by (s desc, creation
# asc) are kept and relabelled by (depth asc, creation asc); the root is node 0.
#
# Evaluation slots: slot 0 is the root; the j-th node evaluated at depth t >= 1 takes
# slot 1 + (t-1)*W + j.


def _f32(x) -> np.float32:
    return np.float32(x)


def child_score(s_parent: np.float32, val, lse) -> np.float32:
    """s_child = s_parent + (z[t] - lse), each operation rounded to float32."""
    return _f32(_f32(s_parent) + _f32(_f32(val) - _f32(lse)))


def rank_select(scores: List[np.float32], creation: List[int], k: int) -> List[int]:
    """Indices of the k best entries by (score desc, creation asc), best first."""
    order = sorted(range(len(scores)), key=lambda i: (-float(scores[i]), creation[i]))
    return order[:k]


def expand_tree(D: int, K: int, W: int, N: int, root_token: int,
                evaluate: Callable[[int, List[dict]], List[dict]]) -> dict:
    """Grow one request's draft tree.  `evaluate(depth, nodes)` receives the nodes to
    evaluate at that depth (dicts with slot, token, parent_slot, depth) and returns, per
    node, dict(topk_ids, topk_vals, lse).  Returns the final tree and the evaluation log."""
    slots = [{"slot": 0, "token": int(root_token), "parent_slot": -1, "depth": 0,
              "cand": -1, "score": _f32(0.0)}]
    cands: List[dict] = []
    res = evaluate(0, [slots[0]])
    frontier = [slots[0]]
    results = {0: res[0]}
    for t in range(1, D + 1):
        # children of the nodes evaluated at depth t-1, in frontier order then child rank
        new = []
        for v in frontier:
            r = results[v["slot"]]
            run = None
            for rank in range(K):
                # a child never scores above a sibling created before it (for a top-K list, whose
                # values fall with the rank, this changes nothing; for sampled children it keeps
                # every kept sibling set a prefix of the draw order)
                sc = child_score(v["score"], r["topk_vals"][rank], r["lse"])
                run = sc if run is None else min(run, sc)
                c = {"token": int(r["topk_ids"][rank]), "parent_slot": v["slot"],
                     "depth": t, "score": _f32(run),
                     "creation": len(cands), "slot": -1}
                cands.append(c)
                new.append(c)
        if t == D:
            break
        pick = rank_select([c["score"] for c in new], [c["creation"] for c in new], W)
        frontier = []
        for j, ci in enumerate(pick):
            c = new[ci]
            c["slot"] = 1 + (t - 1) * W + j
            node = {"slot": c["slot"], "token": c["token"], "parent_slot": c["parent_slot"],
                    "depth": t, "cand": c["creation"], "score": c["score"]}
            slots.append(node)
            frontier.append(node)
        res = evaluate(t, frontier)
        for node, r in zip(frontier, res):
            results[node["slot"]] = r
    # final prune and relabel
    keep = rank_select([c["score"] for c in cands], [c["creation"] for c in cands], N)
    keep = sorted(keep, key=lambda i: (cands[i]["depth"], cands[i]["creation"]))
    label_of_cand = {ci: 1 + n for n, ci in enumerate(keep)}
    cand_of_slot = {s["slot"]: s["cand"] for s in slots}
    tokens = [int(root_token)]
    parents = [-1]
    depth = [0]
    score = [_f32(0.0)]
    for ci in keep:
        c = cands[ci]
        ps = c["parent_slot"]
        tokens.append(c["token"])
        parents.append(0 if ps == 0 else label_of_cand[cand_of_slot[ps]])
        depth.append(c["depth"])
        score.append(c["score"])
    return {"tokens": tokens, "parents": parents, "depth": depth,
            "score": np.array(score, dtype=np.float32), "slots": slots, "cands": cands,
            "results": results}


def draft_round(drafter: Drafter, D: int, K: int, W: int, N: int,
                h_low, h_mid, h_high, root_tok, kpre, vpre, prefix: Sequence[int],
                feature_override: Optional[Callable[[int, int], Optional[np.ndarray]]] = None,
                schedule: Optional[List[List[dict]]] = None) -> List[dict]:
    """One draft-tree round for every request, the drafter evaluated in float64.

    feature_override(b, slot) may return the feature a_parent to feed instead of the
    oracle's own (teacher forcing against another implementation's per-node outputs).
    schedule[b] (optional) is another implementation's evaluation log: when given, the
    oracle evaluates exactly those slots (token, parent) rather than its own selection,
    and returns its per-slot outputs for comparison ("score mode")."""
    g = fuse_features(f64(h_low), f64(h_mid), f64(h_high), drafter.w_fuse)
    kpre, vpre = f64(kpre), f64(vpre)
    cu = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int64)
    out = []
    for b in range(len(prefix)):
        kp, vp = kpre[cu[b]:cu[b + 1]], vpre[cu[b]:cu[b + 1]]
        P = int(prefix[b])
        store: Dict[int, dict] = {}

        def evaluate(t: int, nodes: List[dict], b=b, kp=kp, vp=vp, P=P, store=store):
            toks, feats, pos, ak, av = [], [], [], [], []
            for nd in nodes:
                toks.append(nd["token"])
                f = None
                if feature_override is not None and nd["parent_slot"] >= 0:
                    f = feature_override(b, nd["parent_slot"])
                if f is None:
                    f = g[b] if nd["parent_slot"] < 0 else store[nd["parent_slot"]]["a"]
                feats.append(np.asarray(f, dtype=np.float64))
                pos.append(P + t)
                chain = []
                ps = nd["parent_slot"]
                while ps >= 0:
                    chain.append(ps)
                    ps = store[ps]["parent_slot"]
                chain.reverse()
                ak.append(np.stack([store[s]["k"] for s in chain]) if chain
                          else np.zeros((0, drafter.Hkv, drafter.Dh)))
                av.append(np.stack([store[s]["v"] for s in chain]) if chain
                          else np.zeros((0, drafter.Hkv, drafter.Dh)))
            r = drafter.forward_nodes(toks, np.stack(feats), pos, kp, vp, ak, av)
            res = []
            for j, nd in enumerate(nodes):
                ids, vals = topk_desc(r["z"][j], K)
                store[nd["slot"]] = {"k": r["k"][j], "v": r["v"][j], "a": r["a"][j],
                                     "parent_slot": nd["parent_slot"], "z": r["z"][j],
                                     "lse": r["lse"][j], "topk_ids": ids, "topk_vals": vals,
                                     "feat": feats[j]}
                res.append({"topk_ids": ids, "topk_vals": vals, "lse": r["lse"][j]})
            return res

        if schedule is None:
            tree = expand_tree(D, K, W, N, int(root_tok[b]), evaluate)
        else:
            by_depth: Dict[int, List[dict]] = {}
            for nd in schedule[b]:
                by_depth.setdefault(nd["depth"], []).append(nd)
            for t in sorted(by_depth):
                evaluate(t, sorted(by_depth[t], key=lambda n: n["slot"]))
            tree = {}
        tree["store"] = store
        tree["g"] = g[b]
        out.append(tree)
    return out


# =======================================================================================
# After acceptance: commit the accepted path's KV ([P5] 一棵候选树怎样被验证, step 5) and
# rebuild the drafter's prefix KV of the committed positions from the target's real
# features ([P3] 第二步为什么没有“正确隐藏状态”可用)
# =======================================================================================


def commit_kv(cu_nodes, path, accept_len, k_tree, v_tree, dst_row, k_cache, v_cache):
    """[P5] 一棵候选树怎样被验证, step 5: only the KV of the accepted path is committed and
    the other branches are released.  For request b the path's nodes path[b][0..accept_len[b]]
    (root first) are tree rows cu_nodes[b] + path[b][i]; their K and V rows are copied, in
    path order, to cache rows dst_row[b] + i.  Every other cache row is left as it was.
    Returns new (k_cache, v_cache) arrays."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    for b in range(len(cu_nodes) - 1):
        for i in range(int(accept_len[b]) + 1):
            src = int(cu_nodes[b]) + int(path[b][i])
            kc[int(dst_row[b]) + i] = k_tree[src]
            vc[int(dst_row[b]) + i] = v_tree[src]
    return kc, vc


def drafter_catchup(drafter: "Drafter", tokens, h_low, h_mid, h_high, pos):
    """Drafter catch-up over committed positions.  [P3] 第二步为什么没有“正确隐藏状态”可用:
    the first draft step reads the real fused target feature g with its token; later steps
    substitute the drafter's own output a only because the target has not run on the drafted
    tokens yet.  Once the target has verified positions, their real features exist, and the
    drafter's prefix KV for them is built as for a first step: per row,
    g = W_f [h_low; h_mid; h_high] ([P3] 多层特征融合到底融合了什么),
    u = [rms(E[x]) g_e ; rms(g) g_f], and the layer's key (RoPE at the row's position) and
    value.  Returns (g [n, d], k [n, Hkv, Dh], v [n, Hkv, Dh]) in float64."""
    g = fuse_features(f64(h_low), f64(h_mid), f64(h_high), drafter.w_fuse)
    _, k, v = drafter.qkv([int(t) for t in tokens], g, [int(p) for p in pos])
    return g, k, v


# =======================================================================================
# O4: tree mask, depth, positions ([P2] 树因果掩码, [P3] 每个节点只能关注它的祖先路径,
#     [P5] 给节点分配 position / 节点只能看到自己的祖先)
# =======================================================================================


def build_tree_mask(parents: Sequence[int], cu_nodes: Sequence[int], cu_prefix: Sequence[int],
                    words: int = 1):
    """For every node i of every request: mask bit j set iff j is i or an ancestor of i
    (request-local indices), depth = number of edges to the root, pos = P_b + depth.
    Found by walking parent pointers.  Returns (mask [T, words] uint64, depth, pos, ok);
    ok is False if a parent is not an earlier node of the same request (root: -1)."""
    T = len(parents)
    mask = np.zeros((T, words), dtype=np.uint64)
    depth = np.zeros(T, dtype=np.int32)
    pos = np.zeros(T, dtype=np.int32)
    ok = True
    for b in range(len(cu_nodes) - 1):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        P = int(cu_prefix[b + 1]) - int(cu_prefix[b])
        for i in range(n1 - n0):
            p = int(parents[n0 + i])
            if (i == 0 and p != -1) or (i > 0 and not (0 <= p < i)) or i >= 64 * words:
                ok = False
                continue
            j, dep = i, 0
            while j >= 0:
                mask[n0 + i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
                nxt = int(parents[n0 + j]) if j > 0 else -1
                if nxt >= 0:
                    dep += 1
                j = nxt
            depth[n0 + i] = dep
            pos[n0 + i] = P + dep
    return mask, depth, pos, ok


def mask_bit(mask: np.ndarray, i: int, j: int) -> bool:
    return bool((int(mask[i, j // 64]) >> (j % 64)) & 1)


# =======================================================================================
# O5: tree attention over prefix KV + tree KV ([P3] 从序列到动态草稿树, [P5] step 2-3)
# =======================================================================================


def tree_attention(q, k_tree, v_tree, cu_nodes, mask, kpre, vpre, cu_prefix, scale: float,
                   key_filter: Optional[Callable[[int, int], Tuple[np.ndarray, np.ndarray]]] = None):
    """For node i (request b) and query head h (KV head h // (Hq/Hkv)): softmax attention
    over the key list [prefix keys 0..P_b-1] ++ [tree nodes j with mask bit j set].
    Returns O [T, Hq, Dh] and natural-log LSE [T, Hq].

    key_filter(b, P_b) -> (prefix_keep [P_b] bool, tree_keep [n_b] bool) restricts the key
    list to a subset (a partial, as one split of the prefix or the tree alone would give)."""
    q, k_tree, v_tree = f64(q), f64(k_tree), f64(v_tree)
    kpre, vpre = f64(kpre), f64(vpre)
    T, Hq, Dh = q.shape
    Hkv = k_tree.shape[1]
    G = Hq // Hkv
    O = np.zeros((T, Hq, Dh))
    L = np.full((T, Hq), NEG_INF)
    for b in range(len(cu_nodes) - 1):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        p0, p1 = int(cu_prefix[b]), int(cu_prefix[b + 1])
        n, P = n1 - n0, p1 - p0
        if n == 0:
            continue
        vis_tree = np.array([[mask_bit(mask, n0 + i, j) for j in range(n)] for i in range(n)],
                            dtype=bool).reshape(n, n)
        pk = np.ones(P, dtype=bool)
        tk = np.ones(n, dtype=bool)
        if key_filter is not None:
            pk, tk = key_filter(b, P)
        vis = np.concatenate([np.broadcast_to(pk, (n, P)), vis_tree & tk[None, :]], axis=1)
        for c in range(Hkv):
            keys = np.concatenate([kpre[p0:p1, c], k_tree[n0:n1, c]], axis=0)
            vals = np.concatenate([vpre[p0:p1, c], v_tree[n0:n1, c]], axis=0)
            heads = list(range(c * G, (c + 1) * G))
            Q = q[n0:n1][:, heads, :].reshape(n * G, Dh)
            visr = np.repeat(vis, G, axis=0)
            o, l = attend_rows(Q, keys, vals, scale, visr)
            O[n0:n1, c * G:(c + 1) * G] = o.reshape(n, G, Dh)
            L[n0:n1, c * G:(c + 1) * G] = l.reshape(n, G)
    return O, L


# =======================================================================================
# The training form of the long-context shape ([P4] USP 核心设计：三步走): every position
# of the sequence is a query.  Step 1: causal attention over the main sequence (Out_main,
# LSE_main); Step 2: each position's own TTT branch keys, the at most seven keys that the
# unrolled draft steps produced at that position (Out_branch, LSE_branch); Step 3: the
# streaming-softmax fusion, which is lse_merge below.
# =======================================================================================


def causal_attention(q, k, v, scale: float, rows=None):
    """Step 1: position t, query head h (KV head h // (Hq/Hkv)) attends to the main keys
    0 .. t.  q [L, Hq, Dh], k, v [L, Hkv, Dh].  Returns (O [L, Hq, Dh], LSE [L, Hq]) in
    float64; with `rows` (positions), only those rows are computed (the others are left 0 /
    -inf)."""
    q, k, v = f64(q), f64(k), f64(v)
    L, Hq, Dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    O = np.zeros((L, Hq, Dh))
    LSE = np.full((L, Hq), NEG_INF)
    for t in (range(L) if rows is None else rows):
        for h in range(Hq):
            O[t, h], LSE[t, h] = attend(q[t, h], k[:t + 1, h // G], v[:t + 1, h // G], scale)
    return O, LSE


def branch_attention(q, kb, vb, scale: float):
    """Step 2: position t, query head h attends to its own branch keys kb[0 .. s-1, t]
    (the unrolled steps' keys at position t, KV head h // (Hq/Hkv)), computed as per-position
    dot products.  q [L, Hq, Dh], kb, vb [s, L, Hkv, Dh].  Returns (O [L, Hq, Dh],
    LSE [L, Hq])."""
    q, kb, vb = f64(q), f64(kb), f64(vb)
    L, Hq, Dh = q.shape
    Hkv = kb.shape[2]
    G = Hq // Hkv
    O = np.zeros((L, Hq, Dh))
    LSE = np.full((L, Hq), NEG_INF)
    for t in range(L):
        for h in range(Hq):
            O[t, h], LSE[t, h] = attend(q[t, h], kb[:, t, h // G], vb[:, t, h // G], scale)
    return O, LSE


# =======================================================================================
# O6: log-sum-exp merge of partials ([P4] USP 核心设计 Step 3: streaming-softmax fusion of
#     Out_branch/LSE_branch into Out_main/LSE_main with one consistent normalisation)
# =======================================================================================


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """o_parts [S, rows, Dh], lse_parts [S, rows] (natural log).  Per row:
    m = max_s LSE_s, w_s = e^{LSE_s - m}, O = sum_s w_s O_s / sum_s w_s,
    LSE = m + ln sum_s w_s.  A partial with LSE = -inf has weight 0; if every partial of a
    row is -inf the row gives O = 0 and LSE = -inf."""
    o_parts, lse_parts = f64(o_parts), f64(lse_parts)
    S, R, Dh = o_parts.shape
    O = np.zeros((R, Dh))
    L = np.full(R, NEG_INF)
    for r in range(R):
        m = np.max(lse_parts[:, r])
        if not np.isfinite(m):
            continue
        w = np.exp(lse_parts[:, r] - m)
        O[r] = (w[:, None] * o_parts[:, r, :]).sum(axis=0) / w.sum()
        L[r] = m + np.log(w.sum())
    return O, L


# =======================================================================================
# O7: acceptance ([P1] 论文位置: accept the longest correct prefix, standard speculative
#     sampling keeps the target distribution; [P2] rollback to the last accepted node;
#     [P3] 接受连续前缀，拒绝处进行校正; [P5] 按目标概率与采样规则确定被接受路径)
# =======================================================================================
#
# Deterministic-candidate form: the candidates are top-K (not sampled), so the proposal
# at a child is a point mass and min(1, p/q) accepts child x with probability p(x); the
# rejection residual is p with x removed.  Walking the siblings this way is the same as
# drawing one y ~ p at the node and descending into the child whose token is y (if any),
# otherwise emitting y as the correction.  The draw y_i = argmax_t(z_i[t]/T + Gumbel)
# (greedy: argmax_t z_i[t]) is made independently at every node from a counter-based
# generator, so the accepted path is the longest root path whose every token equals the
# draw at its parent; the bonus token is the draw at the path's end.

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
    easy as 1, 2, 3", SC'11): each round multiplies words 0 and 2 by M0 and M1 (32x32->64),
    and forms (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is bumped by the Weyl
    constants W0, W1 between rounds.  Works elementwise on numpy uint64 arrays holding
    32-bit values."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & MASK32
    M0, M1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & np.uint64(MASK32)
            k1 = (k1 + np.uint64(PHILOX_W1)) & np.uint64(MASK32)
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform23(x) -> np.ndarray:
    """u = ((x >> 9) + 0.5) * 2^-23: the top 23 bits of a 32-bit word mapped to the
    centre of one of 2^23 equal cells, strictly inside (0, 1).  (x >> 9) + 0.5 needs at
    most 24 significant bits, so every step is exact in float32; with 24 bits the top
    cell would round to exactly 1.0.)"""
    x = np.asarray(x, dtype=np.uint64)
    return ((x >> np.uint64(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


LN2_HI = np.float32(0.693145751953125)        # 0x3f317200: ln 2 rounded to 15 bits
LN2_LO = np.float32(1.42860676e-06)           # ln 2 - LN2_HI, rounded to float32
SQRT2_F32 = np.float32(1.41421354)            # 0x3fb504f3
C3, C5, C7, C9 = (np.float32(1.0 / 3.0), np.float32(1.0 / 5.0), np.float32(1.0 / 7.0),
                  np.float32(1.0 / 9.0))


def ln_spec(v) -> np.ndarray:
    """Natural log of positive normal float32 values by the textbook reduction
    v = 2^e * m with m in [sqrt(1/2), sqrt(2)), ln v = e ln2 + 2 atanh(s), s = (m-1)/(m+1),
    atanh(s) = s + s^3/3 + s^5/5 + s^7/7 + s^9/9 (Horner in s^2), ln 2 split in a
    short high part and a float32 low part.  Every operation is a separately rounded
    float32 add, multiply or correctly rounded divide, in the order written, so the
    result is reproducible bit for bit by any IEEE float32 implementation."""
    v = np.asarray(v, dtype=np.float32)
    bits = v.view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32) - 127
    m = ((bits & np.uint32(0x7FFFFF)) | np.uint32(0x3F800000)).view(np.float32)
    big = m >= SQRT2_F32
    m = np.where(big, m * np.float32(0.5), m).astype(np.float32)
    e = np.where(big, e + 1, e)
    ef = e.astype(np.float32)
    s = (m - np.float32(1.0)) / (m + np.float32(1.0))
    t = s * s
    p = C9
    p = p * t + C7
    p = p * t + C5
    p = p * t + C3
    r = s + (s * t) * p
    return (ef * LN2_HI + (ef * LN2_LO + np.float32(2.0) * r)).astype(np.float32)


def gumbel(seed: int, rnd: int, b: int, i: int, t: np.ndarray) -> np.ndarray:
    """Gumbel noise for token ids t at node i of request b: counter (t>>2, i, b, round),
    key (seed_lo, seed_hi); word t & 3 of the Philox output; G = -ln(-ln u)."""
    t = np.asarray(t, dtype=np.uint64)
    n = t.shape[0]
    c0 = t >> np.uint64(2)
    w = philox4x32_10(c0, np.full(n, i), np.full(n, b), np.full(n, rnd & MASK32),
                      np.full(n, seed & MASK32), np.full(n, (seed >> 32) & MASK32))
    sel = (t & np.uint64(3)).astype(np.int64)
    x = np.choose(sel, w)
    u = uniform23(x)
    inner = -ln_spec(u)
    return (-ln_spec(inner)).astype(np.float32)


def draws_over_rounds(z_row, temperature: float, seed: int, rounds: np.ndarray, b: int,
                      i: int) -> np.ndarray:
    """`node_draw` for many rounds at once (the same rule, vectorised over the round
    counter); used for the statistical checks.  Returns y [len(rounds)]."""
    z = np.asarray(z_row, dtype=np.float32)
    V = z.shape[0]
    R = rounds.shape[0]
    # one Philox block per (round, counter t >> 2): its four words serve tokens 4c .. 4c+3
    C = (V + 3) // 4
    c0 = np.tile(np.arange(C, dtype=np.uint64), R)
    rr = np.repeat(np.asarray(rounds, dtype=np.uint64), C)
    w = philox4x32_10(c0, np.full(c0.shape, i), np.full(c0.shape, b), rr & np.uint64(MASK32),
                      np.full(c0.shape, seed & MASK32), np.full(c0.shape, (seed >> 32) & MASK32))
    x = np.stack(w, axis=-1).reshape(R, 4 * C)[:, :V]
    g = (-ln_spec(-ln_spec(uniform23(x.reshape(-1))))).astype(np.float32).reshape(R, V)
    invT = np.float32(1.0) / np.float32(temperature)
    vals = (z[None, :] * invT + g).astype(np.float32)
    return np.argmax(vals, axis=1)


def node_draw(z_row, temperature: float, seed: int, rnd: int, b: int, i: int) -> int:
    """Target draw at one node: greedy argmax_t z[t] (temperature 0), else
    argmax_t (z[t] * invT + G_t) in float32 with invT = 1/T rounded to float32; ties go to
    the lowest token id."""
    z = np.asarray(z_row, dtype=np.float32)
    if temperature == 0.0:
        vals = z
    else:
        invT = np.float32(1.0) / np.float32(temperature)
        vals = (z * invT + gumbel(seed, rnd, b, i, np.arange(z.shape[0]))).astype(np.float32)
    return int(np.argmax(vals))     # numpy argmax returns the first maximum


def accept(cu_nodes, tokens, parents, logits, temperature: float, seed: int, rnd: int,
           max_depth: int):
    """Per request: y_i = draw at every node; the accepted end node is the deepest node
    whose root path has every token equal to the draw at its parent (ties: lowest node
    index); bonus = y at that node.  Returns (accept_len [B], path [B, max_depth+1],
    out_tokens [B, max_depth+1], bonus [B]) with -1 padding; the path is node indices
    root first, out_tokens the accepted draft tokens then the bonus."""
    B = len(cu_nodes) - 1
    acc = np.zeros(B, dtype=np.int32)
    path = np.full((B, max_depth + 1), -1, dtype=np.int32)
    outt = np.full((B, max_depth + 1), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    lg = np.asarray(logits.float().numpy() if hasattr(logits, "float") else logits,
                    dtype=np.float32)
    for b in range(B):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        n = n1 - n0
        y = [node_draw(lg[n0 + i], temperature, seed, rnd, b, i) for i in range(n)]
        best, best_len = 0, 0
        for i in range(n):
            j, L, good = i, 0, True
            while j > 0:
                p = int(parents[n0 + j])
                if int(tokens[n0 + j]) != y[p]:
                    good = False
                    break
                L += 1
                j = p
            if good and L > best_len:
                best, best_len = i, L
        chain = []
        j = best
        while j >= 0:
            chain.append(j)
            j = int(parents[n0 + j]) if j > 0 else -1
        chain.reverse()
        acc[b] = best_len
        bonus[b] = y[best]
        for s, j in enumerate(chain):
            path[b, s] = j
        for s, j in enumerate(chain[1:]):
            outt[b, s] = int(tokens[n0 + j])
        outt[b, best_len] = y[best]
    return acc, path, outt, bonus


# =======================================================================================
# O8: sampled candidates ([P2] 四 DFlash: every drafted token is kept with probability
#     min(1, p_target / p_draft), the dice are thrown left to right and the first rejection
#     ends the kept prefix; [P3] 先看 checkpoint 最终要参与什么计算: the continuous prefix is
#     kept, the rejection point is corrected, and the output then follows the target model
#     alone).  Tree form (a reading: the pages give the one-candidate rule): the children of
#     a node are draws without replacement from the drafter's distribution q at that node,
#     tested in the order drawn; after a rejection the target side becomes the normalised
#     positive part of (p - q) and the rejected token is taken out of q (q renormalised).
#     When every child is rejected, or the node has none, the next token is drawn from the
#     target side as it then stands.
# =======================================================================================

ACCEPT_UNIFORM_C0 = 0x40000000   # counter word 0 of the acceptance uniforms (t >> 2 never reaches it)


def softmax64(z_row, temperature: float) -> np.ndarray:
    """softmax(z / T) in float64: a_t = z_t * (1 / T) (z upcast exactly, 1 / T the float64
    reciprocal of the float32 temperature, rounded once), p_t = exp(a_t - A) with
    A = max a + ln sum exp(a - max a)."""
    a = np.asarray(z_row, dtype=np.float64) * (1.0 / float(np.float32(temperature)))
    m = a.max()
    A = m + math.log(float(np.exp(a - m).sum()))
    return np.exp(a - A)


def rrs_node(p: np.ndarray, q: np.ndarray, cand: Sequence[int], u: Sequence[float]):
    """The rejection chain at one node.  cand: the children's tokens in the order drawn,
    u: one uniform in (0, 1) per child.  Candidate x (not already rejected here, inside the
    vocabulary) is kept when u < p(x) / q(x) for the current p and q (q(x) = 0 keeps it
    whenever p(x) > 0); otherwise p <- max(p - q, 0) / sum, q(x) <- 0, q <- q / sum.
    Returns (index of the kept child or -1, the target side p after the chain, the list of
    thresholds p(x)/q(x) met by each tested child, None for a skipped child)."""
    p = np.array(p, dtype=np.float64)
    q = np.array(q, dtype=np.float64)
    V = p.shape[0]
    tried, thr = set(), []
    for k, x in enumerate(cand):
        x = int(x)
        if x < 0 or x >= V or x in tried:
            thr.append(None)
            continue
        tried.add(x)
        t = math.inf if q[x] == 0.0 else p[x] / q[x]
        thr.append(t)
        if float(u[k]) < t:
            return k, p, thr
        r = np.maximum(p - q, 0.0)
        s = r.sum()
        if s > 0.0:                 # a rejection leaves s > 0 unless p and q agree to rounding
            p = r / s
        q[x] = 0.0
        sq = q.sum()
        if sq <= 0.0:               # the drafter's mass is used up: nothing more to test
            break
        q = q / sq
    return -1, p, thr


def residual_draw(p: np.ndarray, g: np.ndarray) -> int:
    """Gumbel-max draw from p: argmax over p_t > 0 of ln p_t + g_t (float64; g the float32
    Gumbel noise upcast), lowest token id on ties."""
    with np.errstate(divide="ignore"):
        v = np.where(p > 0.0, np.log(p) + np.asarray(g, dtype=np.float64), -np.inf)
    return int(np.argmax(v))


def accept_uniform(seed: int, rnd: int, b: int, j: int) -> float:
    """The uniform met by child node j of request b: Philox4x32-10 with counter
    (ACCEPT_UNIFORM_C0, j, b, round), key (seed lo, seed hi), word 0, mapped as uniform23."""
    w = philox4x32_10(ACCEPT_UNIFORM_C0, j, b, rnd & MASK32, seed & MASK32, (seed >> 32) & MASK32)
    return float(uniform23(w[0]))


DRAFT_NOISE_C1 = 0x80000000      # counter word 1 of the drafter's noise: above every node index


def draft_gumbel(seed: int, rnd: int, b: int, slot: int, t: np.ndarray) -> np.ndarray:
    """The drafter's Gumbel noise at evaluation slot `slot` of request b: as `gumbel`, with
    counter word 1 = DRAFT_NOISE_C1 | slot (a stream apart from the verifier's)."""
    t = np.asarray(t, dtype=np.uint64)
    n = t.shape[0]
    w = philox4x32_10(t >> np.uint64(2), np.full(n, DRAFT_NOISE_C1 | slot), np.full(n, b),
                      np.full(n, rnd & MASK32), np.full(n, seed & MASK32),
                      np.full(n, (seed >> 32) & MASK32))
    x = np.choose((t & np.uint64(3)).astype(np.int64), w)
    u = uniform23(x)
    return (-ln_spec(-ln_spec(u))).astype(np.float32)


def sample_children(z_row, temperature: float, K: int, seed: int, rnd: int, b: int, slot: int):
    """K children drawn without replacement from softmax(z / T) by the Gumbel-top-K rule: the K
    best tokens by zs_t + G_t (zs = z * invT, invT = 1/T, each rounded to float32, then the sum
    rounded; ties to the lowest id), best first, which is the order they are drawn in.
    Returns (ids, zs at the ids) -- the scaled logits without noise, which the scores use."""
    z = np.asarray(z_row, dtype=np.float32)
    invT = np.float32(1.0) / np.float32(temperature)
    zs = (z * invT).astype(np.float32)
    v = (zs + draft_gumbel(seed, rnd, b, slot, np.arange(z.shape[0]))).astype(np.float32)
    ids = np.lexsort((np.arange(z.shape[0]), -v.astype(np.float64)))[:K]
    return ids.astype(np.int64), zs[ids]


def accept_sampled(cu_nodes, tokens, parents, logits, draft_logits, draft_row,
                   temperature: float, seed: int, rnd: int, max_depth: int,
                   max_children: int = 1 << 30):
    """Sampled-candidate acceptance.  Per request, from the root: at node i the target side
    is p = softmax(z_i / T) and the draft side q = softmax(draft_logits[draft_row[i]] / T);
    its first max_children children (nodes whose parent is i, in increasing node index) go
    through rrs_node with their uniforms; a kept child becomes the next node; otherwise the bonus token is
    residual_draw of the resulting target side with the Gumbel noise of node i (the noise
    of the deterministic form).  A node whose draft row is outside draft_logits draws from
    p directly.  Returns (accept_len, path, out_tokens, bonus) laid out as by `accept`."""
    B = len(cu_nodes) - 1
    acc = np.zeros(B, dtype=np.int32)
    path = np.full((B, max_depth + 1), -1, dtype=np.int32)
    outt = np.full((B, max_depth + 1), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    lg = np.asarray(logits.float().numpy() if hasattr(logits, "float") else logits, dtype=np.float32)
    dl = np.asarray(draft_logits.float().numpy() if hasattr(draft_logits, "float") else draft_logits,
                    dtype=np.float32)
    V, R = lg.shape[1], dl.shape[0]
    for b in range(B):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        if n1 <= n0:                         # empty request: nothing accepted, no bonus
            bonus[b] = -1
            continue
        kids: Dict[int, List[int]] = {}
        for j in range(1, n1 - n0):
            pj = int(parents[n0 + j])
            if 0 <= pj < j:                  # a parent outside [0, j) makes j nobody's child
                kids.setdefault(pj, []).append(j)
        i, chain = 0, [0]
        while True:
            p = softmax64(lg[n0 + i], temperature)
            ch = kids.get(i, [])[:max_children]
            r = int(draft_row[n0 + i])
            if ch and 0 <= r < R:
                q = softmax64(dl[r], temperature)
                k, p, _ = rrs_node(p, q, [int(tokens[n0 + j]) for j in ch],
                                   [accept_uniform(seed, rnd, b, j) for j in ch])
                if k >= 0:
                    i = ch[k]
                    chain.append(i)
                    continue
            y = residual_draw(p, gumbel(seed, rnd, b, i, np.arange(V)))
            break
        L = len(chain) - 1
        acc[b], bonus[b] = L, y
        path[b, :L + 1] = chain
        for s, j in enumerate(chain[1:]):
            outt[b, s] = int(tokens[n0 + j])
        outt[b, L] = y
    return acc, path, outt, bonus


# =======================================================================================
# Speculative-budget controller ([P5] 执行控制器): a host-side policy that adjusts the draft
# tree budget from observed acceptance and latency, never the target decoding itself
# =======================================================================================


class BudgetController:
    """[P5] 执行控制器.  The page lists what the controller watches (proposed, accepted and
    committed tokens, mean accepted length, drafter and verify latency) and a simplified
    policy: lower the tree budget when recent accepted length is low or drafting is
    expensive; raise it cautiously when acceptance is stable and verification has spare
    capacity; every adjustment bounded, with a cooldown and a fallback baseline so that
    short-term noise does not make it oscillate.  The quality rule (deadline-driven thinking
    allowance) changes answers and is a product decision, not part of this controller.

    Reading taken (the page gives no numbers): budgets are a ladder of tree configurations in
    increasing size; statistics are the last `window` rounds at the current level (cleared on
    every change); with c = tokens committed per round (accept_len + 1), D the level's depth:
      frac = mean(c) / (D + 1), cv = std(c) / mean(c) (population std),
      draft share = mean(draft_ms) / mean(draft_ms + verify_ms),
      goodput = mean(c) / mean(draft_ms + verify_ms).
    A decision is taken only when the window is full and `cooldown` rounds have passed since
    the last change, in this order:
      1. after a raise, the first full window is compared with the goodput measured before
         it; a drop of more than `revert_drop` (a fraction) steps back down (the fallback)
         and blocks raises for 4 * cooldown rounds;
      2. frac < low_frac or draft share > draft_share_max: one level down (not below 0);
      3. frac >= high_frac and cv <= max_cv and mean(verify_ms) < verify_ms_max, raises not
         blocked: one level up (not above the top).
    Every change resets the round counter and the window.  All statistics in float64, sums
    in round order."""

    def __init__(self, n_levels, depths, start, cooldown, window, low_frac, high_frac, max_cv,
                 draft_share_max, verify_ms_max, revert_drop):
        self.n, self.depths = int(n_levels), [int(x) for x in depths]
        self.level = int(start)
        self.cooldown, self.window = int(cooldown), int(window)
        self.low_frac, self.high_frac, self.max_cv = float(low_frac), float(high_frac), float(max_cv)
        self.draft_share_max, self.verify_ms_max = float(draft_share_max), float(verify_ms_max)
        self.revert_drop = float(revert_drop)
        self.hist = []
        self.since = 0
        self.block = 0            # rounds during which raises are blocked
        self.check = False        # the last change was a raise, goodput to be compared
        self.g_before = 0.0

    def _change(self, new_level):
        self.level = new_level
        self.since = 0
        self.hist = []

    def update(self, accept_len, draft_ms, verify_ms) -> int:
        self.hist.append((float(accept_len) + 1.0, float(draft_ms), float(verify_ms)))
        if len(self.hist) > self.window:
            self.hist.pop(0)
        self.since += 1
        if self.block > 0:
            self.block -= 1
        if len(self.hist) < self.window or self.since < self.cooldown:
            return self.level
        n = float(len(self.hist))
        mc = sum(h[0] for h in self.hist) / n
        var = sum((h[0] - mc) ** 2 for h in self.hist) / n
        cv = math.sqrt(var) / mc
        md = sum(h[1] for h in self.hist) / n
        mv = sum(h[2] for h in self.hist) / n
        mr = sum(h[1] + h[2] for h in self.hist) / n
        frac = mc / (self.depths[self.level] + 1)
        good = mc / mr
        if self.check:
            self.check = False
            if good < self.g_before * (1.0 - self.revert_drop) and self.level > 0:
                self.block = 4 * self.cooldown
                self._change(self.level - 1)
                return self.level
        if (frac < self.low_frac or md / mr > self.draft_share_max) and self.level > 0:
            self._change(self.level - 1)
        elif (frac >= self.high_frac and cv <= self.max_cv and mv < self.verify_ms_max
              and self.block == 0 and self.level < self.n - 1):
            self.g_before = good
            self.check = True
            self._change(self.level + 1)
        return self.level
