"""GPU parity of eagle3_draft_expand against the oracle, following the teacher-forced
protocol: (1) top-K ids equal the oracle's top-K of the GPU's own logits, bit for bit;
(2) replaying the oracle's selection on the GPU's per-slot (top-K, lse) reproduces the
GPU's tree bit for bit; (3) per-slot floats (g, a, logits, lse) match the oracle's
float64 drafter run on the GPU's tree with the GPU's parent features, within 1e-4 (fp32)
or 2e-2 (bf16) relative."""
import math

import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import capi, synth
from tests.gpu_util import TOL, need_gpu, np32, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_gpu(shape, prefix, wseed, iseed, logits=True):
    w = synth.drafter_weights(shape, seed=wseed, device=DEV)
    di = synth.draft_inputs(shape, seed=iseed, device=DEV, prefix=prefix)
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    tree = capi.Eagle3TreeCfg(depth=shape.depth, topk=shape.topk, width=shape.width,
                              n_nodes=shape.n_nodes)
    out = capi.eagle3_draft_expand(dr, tree, di["h_low"], di["h_mid"], di["h_high"], di["root_tok"],
                                   di["kpre"], di["vpre"], di["cu_prefix"], max(prefix), debug=True,
                                   debug_logits=logits)
    torch.cuda.synchronize()
    return w, di, out


def gpu_schedule(dbg, b, W):
    st = dbg["slot_token"][b].cpu().numpy()
    sp = dbg["slot_parent"][b].cpu().numpy()
    nodes = []
    for s in range(st.shape[0]):
        if sp[s] == -2:
            continue
        nodes.append({"slot": s, "token": int(st[s]), "parent_slot": int(sp[s]),
                      "depth": 0 if s == 0 else 1 + (s - 1) // W})
    return nodes


def check_topk_on_gpu_logits(shape, dbg, B):
    lg = dbg["slot_logits"].cpu().numpy()
    ids = dbg["slot_topk_id"].cpu().numpy()
    vals = dbg["slot_topk_val"].cpu().numpy()
    sp = dbg["slot_parent"].cpu().numpy()
    for b in range(B):
        for s in range(lg.shape[1]):
            if sp[b, s] == -2:
                continue
            ri, rv = O.topk_desc(lg[b, s], shape.topk)
            assert np.array_equal(ids[b, s], ri), (b, s)
            assert np.array_equal(vals[b, s], rv.astype(np.float32)), (b, s)


def check_selection_replay(shape, out, B):
    """Oracle selection driven by the GPU's per-slot (top-K, lse) must give the GPU tree."""
    dbg = out["debug"]
    ids = dbg["slot_topk_id"].cpu().numpy()
    vals = dbg["slot_topk_val"].cpu().numpy()
    lse = dbg["slot_lse"].cpu().numpy()
    st = dbg["slot_token"].cpu().numpy()
    sp = dbg["slot_parent"].cpu().numpy()
    root = st[:, 0]
    for b in range(B):
        def evaluate(t, nodes, b=b):
            res = []
            for nd in nodes:
                s = nd["slot"]
                assert st[b, s] == nd["token"] and sp[b, s] == nd["parent_slot"], (b, s)
                res.append({"topk_ids": ids[b, s], "topk_vals": vals[b, s], "lse": lse[b, s]})
            return res
        ref = O.expand_tree(shape.depth, shape.topk, shape.width, shape.n_nodes, int(root[b]), evaluate)
        n = int(out["n_nodes"][b])
        assert n == len(ref["tokens"])
        assert out["tokens"][b, :n].tolist() == ref["tokens"]
        assert out["parents"][b, :n].tolist() == ref["parents"]
        assert out["depth"][b, :n].tolist() == ref["depth"]
        assert np.array_equal(out["score"][b, :n].cpu().numpy(), ref["score"])
        assert all(x == -1 for x in out["tokens"][b, n:].tolist())
        # every slot the oracle did not use is marked unused on the GPU too
        used = {nd["slot"] for nd in ref["slots"]}
        for s in range(st.shape[1]):
            assert (s in used) == (sp[b, s] != -2), (b, s)


def check_teacher_forced(shape, w, di, out, B, prefix, slots_per_request=None):
    dbg = out["debug"]
    dt = synth.torch_dtype(shape)
    tol = TOL[dt]
    drafter = O.Drafter({k: v.cpu() for k, v in w.items()}, shape.Hq, shape.Hkv, shape.Dh)
    a_gpu = dbg["slot_a"].cpu().numpy()
    sched = [gpu_schedule(dbg, b, shape.width) for b in range(B)]
    if slots_per_request is not None:
        sched = [slots_per_request(b, s) for b, s in enumerate(sched)]
    res = O.draft_round(drafter, shape.depth, shape.topk, shape.width, shape.n_nodes,
                        di["h_low"].cpu(), di["h_mid"].cpu(), di["h_high"].cpu(),
                        di["root_tok"].cpu(), di["kpre"].cpu(), di["vpre"].cpu(), prefix,
                        feature_override=lambda b, ps: a_gpu[b, ps], schedule=sched)
    g_ref = np.stack([r["g"] for r in res])
    assert rel_err(np32(dbg["g"]), g_ref) <= tol
    lse_g = dbg["slot_lse"].cpu().numpy()
    lg = dbg["slot_logits"].cpu().numpy() if "slot_logits" in dbg else None
    for b in range(B):
        for s, rec in res[b]["store"].items():
            assert rel_err(a_gpu[b, s], rec["a"]) <= tol, ("a", b, s, rel_err(a_gpu[b, s], rec["a"]))
            assert abs(lse_g[b, s] - rec["lse"]) / max(1.0, abs(rec["lse"])) <= tol, ("lse", b, s)
            if lg is not None:
                assert rel_err(lg[b, s], rec["z"]) <= tol, ("z", b, s, rel_err(lg[b, s], rec["z"]))
    return res


def test_draft_tiny_fp32_full_protocol():
    need_gpu()
    shape = synth.TINY
    prefix = [128]
    w, di, out = run_gpu(shape, prefix, 1234, 99)
    check_topk_on_gpu_logits(shape, out["debug"], 1)
    check_selection_replay(shape, out, 1)
    check_teacher_forced(shape, w, di, out, 1, prefix)
    # full binary tree for (D, K, W, N) = (3, 2, 4, 14)
    assert out["n_nodes"].tolist() == [15]
    assert sorted(out["depth"][0].tolist()) == [0] + [1] * 2 + [2] * 4 + [3] * 8
    # untethered: the oracle's own float64 round gives the same tree
    drafter = O.Drafter({k: v.cpu() for k, v in w.items()}, shape.Hq, shape.Hkv, shape.Dh)
    ref = O.draft_round(drafter, 3, 2, 4, 14, di["h_low"].cpu(), di["h_mid"].cpu(),
                        di["h_high"].cpu(), di["root_tok"].cpu(), di["kpre"].cpu(),
                        di["vpre"].cpu(), prefix)[0]
    assert out["tokens"][0].tolist() == ref["tokens"]
    assert out["parents"][0].tolist() == ref["parents"]
    np.testing.assert_allclose(out["score"][0].cpu().numpy(), ref["score"], rtol=1e-4, atol=1e-4)


SMALL_BF16 = synth.scaled(synth.LLAMA8B, d=512, Hq=8, Hkv=2, Dh=128, F=1536, V=8192, B=3,
                          depth=4, topk=5, width=6, n_nodes=20)


@pytest.mark.parametrize("shape,prefix", [
    (SMALL_BF16, [300, 0, 1000]),
    (synth.scaled(SMALL_BF16, dtype="f32", B=2, Dh=64, Hq=8, Hkv=8), [77, 513]),
    (synth.scaled(SMALL_BF16, B=1, depth=1, topk=16, width=1, n_nodes=16), [64]),
    (synth.scaled(SMALL_BF16, B=2, depth=6, topk=10, width=10, n_nodes=60, V=4096), [2048, 5]),
    # EAGLE-3's depth 8 at the 60 / 50 / 48-node budgets: 71 evaluation slots (two mask words)
    (synth.scaled(SMALL_BF16, B=2, depth=8, topk=10, width=10, n_nodes=60, V=4096), [1500, 40]),
    (synth.scaled(SMALL_BF16, B=1, depth=8, topk=10, width=10, n_nodes=50, V=4096), [700]),
    (synth.scaled(SMALL_BF16, B=1, depth=8, topk=10, width=10, n_nodes=48, V=4096), [33]),
    # 177 slots (three mask words), a 200-node tree
    (synth.scaled(SMALL_BF16, B=1, depth=12, topk=5, width=16, n_nodes=200, V=4096), [256]),
    # the largest vocabulary the drafter takes: 64 chunks of 4096 logits, one per lane of the
    # selection's merge wave
    (synth.scaled(SMALL_BF16, B=1, depth=3, topk=4, width=3, n_nodes=10, V=64 * 4096), [100]),
], ids=["bf16_ragged", "fp32_mha", "bf16_depth1_k16", "bf16_llama_budget", "bf16_depth8_n60",
        "bf16_depth8_n50", "bf16_depth8_n48", "bf16_177_slots", "bf16_max_vocab"])
def test_draft_small_full_protocol(shape, prefix):
    need_gpu()
    B = shape.B
    w, di, out = run_gpu(shape, prefix, 7, 8)
    check_topk_on_gpu_logits(shape, out["debug"], B)
    check_selection_replay(shape, out, B)
    check_teacher_forced(shape, w, di, out, B, prefix)
    # invariants of the returned tree
    for b in range(B):
        n = int(out["n_nodes"][b])
        par = out["parents"][b, :n].tolist()
        dep = out["depth"][b, :n].tolist()
        sc = out["score"][b, :n].cpu().numpy()
        assert par[0] == -1 and dep == sorted(dep)
        for i in range(1, n):
            assert 0 <= par[i] < i and dep[i] == dep[par[i]] + 1 and sc[i] <= sc[par[i]]


def test_draft_llama8b_full_size_sampled():
    """The 8B-shaped bf16 workload at full size: top-K and selection checked on every slot;
    floats teacher-forced on the root-to-leaf chains of two sampled deepest slots."""
    need_gpu()
    shape = synth.LLAMA8B
    prefix = [2048]
    w, di, out = run_gpu(shape, prefix, 1234, 99)
    check_topk_on_gpu_logits(shape, out["debug"], 1)
    check_selection_replay(shape, out, 1)
    assert out["n_nodes"].tolist() == [61]

    def chains(b, nodes):
        by = {n["slot"]: n for n in nodes}
        deepest = [n["slot"] for n in nodes if n["depth"] == shape.depth - 1][:2]
        keep = set()
        for s in deepest:
            while s >= 0:
                keep.add(s)
                s = by[s]["parent_slot"]
        return [by[s] for s in sorted(keep)]
    check_teacher_forced(shape, w, di, out, 1, prefix, slots_per_request=chains)


def test_draft_llama70b_full_size_sampled():
    """The 70B-shaped drafter (d 8192, 64 q / 8 kv heads, FFN 28672, fusion 24576 -> 8192) for
    4 requests over 8192-token prefixes: top-K and selection checked on every slot of every
    request; floats teacher-forced on the root-to-leaf chain of one deepest slot each."""
    need_gpu()
    shape = synth.LLAMA70B
    prefix = synth.prefix_lengths(shape, seed=71)
    w, di, out = run_gpu(shape, prefix, 7070, 7071)
    check_topk_on_gpu_logits(shape, out["debug"], shape.B)
    check_selection_replay(shape, out, shape.B)
    assert out["n_nodes"].tolist() == [shape.n_nodes + 1] * shape.B

    def chain(b, nodes):
        by = {n["slot"]: n for n in nodes}
        s = [n["slot"] for n in nodes if n["depth"] == shape.depth - 1][0]
        keep = set()
        while s >= 0:
            keep.add(s)
            s = by[s]["parent_slot"]
        return [by[x] for x in sorted(keep)]
    check_teacher_forced(shape, w, di, out, shape.B, prefix, slots_per_request=chain)


def test_draft_batch16_full_size_sampled():
    """16 requests with the 8B-shaped drafter over ragged prefixes (uniform 512..4096):
    160 evaluated rows per step.  Top-K and selection on every slot of every request; floats
    teacher-forced on one root-to-leaf chain of requests 0, 7 and 15."""
    need_gpu()
    shape = synth.BATCH16
    prefix = synth.prefix_lengths(shape, seed=161)
    w, di, out = run_gpu(shape, prefix, 1616, 1617)
    check_topk_on_gpu_logits(shape, out["debug"], shape.B)
    check_selection_replay(shape, out, shape.B)

    def chain(b, nodes):
        if b not in (0, 7, 15):
            return []
        by = {n["slot"]: n for n in nodes}
        s = max(nodes, key=lambda n: (n["depth"], -n["slot"]))["slot"]
        keep = set()
        while s >= 0:
            keep.add(s)
            s = by[s]["parent_slot"]
        return [by[x] for x in sorted(keep)]
    check_teacher_forced(shape, w, di, out, shape.B, prefix, slots_per_request=chain)


def test_draft_topk_statistics_at_the_widest_vocabulary():
    """The LM-head statistics path at its widest vocabulary (V = 131064: 1024 blocks of 128
    columns, the last holding 120) with the largest top-K and width (16): every lane of the
    selection holds 16 blocks, the candidate gather takes the most blocks, and top-K ids stay
    exact against the GPU's own logits."""
    need_gpu()
    shape = synth.scaled(SMALL_BF16, V=131064, B=1, depth=3, topk=16, width=16, n_nodes=40)
    prefix = [300]
    w = synth.drafter_weights(shape, seed=51, device=DEV)
    di = synth.draft_inputs(shape, seed=52, device=DEV, prefix=prefix)
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    tree = capi.Eagle3TreeCfg(depth=shape.depth, topk=shape.topk, width=shape.width,
                              n_nodes=shape.n_nodes)
    out = capi.eagle3_draft_expand(dr, tree, di["h_low"], di["h_mid"], di["h_high"], di["root_tok"],
                                   di["kpre"], di["vpre"], di["cu_prefix"], max(prefix), debug=True,
                                   debug_logits=True)
    torch.cuda.synchronize()
    check_topk_on_gpu_logits(shape, out["debug"], shape.B)
    check_selection_replay(shape, out, shape.B)
    # the log-sum-exp formed from the blocks' (best, sum) pairs against float64 over the logits
    dbg = out["debug"]
    lg = dbg["slot_logits"].cpu().numpy().astype(np.float64)
    lse = dbg["slot_lse"].cpu().numpy()
    sp = dbg["slot_parent"].cpu().numpy()
    for s_ in range(lg.shape[1]):
        if sp[0, s_] == -2:
            continue
        z = lg[0, s_]
        ref = z.max() + np.log(np.exp(z - z.max()).sum())
        assert abs(lse[0, s_] - ref) <= 1e-5 * max(1.0, abs(ref)), (s_, lse[0, s_], ref)


@pytest.mark.parametrize("kind,V,B", [("plain", 4104, 4), ("periodic3", 8192, 4), ("paired", 4104, 4),
                                      ("plain", 65544, 4), ("plain", 4104, 16), ("periodic3", 8192, 16)])
def test_draft_topk_wide_lm_head_statistics(kind, V, B):
    """40 evaluated rows per step (4 requests x width 10): the LM head runs in the wide
    kernel and emits statistics per 128 columns, from which the selection takes each row's
    top-K and log-sum-exp.  Top-K ids stay exact with plain logits, with heavy ties (the
    exact path), and when the vocabulary ends 8 columns into a block (V = 4104: the last
    256-column workgroup has a half wholly past the end; V = 65544: 32 tiles per workgroup,
    one round of 129 workgroups, the last with three 128-column quarters past the end).
    With 16 requests (160 rows) the wide kernel holds ten row tiles (waves 0 and 1 three
    each, waves 2 and 3 two) at 16 tiles per workgroup."""
    need_gpu()
    shape = synth.scaled(SMALL_BF16, V=V, B=B, depth=3, topk=10, width=10, n_nodes=20)
    prefix = [100, 257, 33, 1] * (B // 4)
    w = synth.drafter_weights(shape, seed=41, device=DEV)
    _tied_lm_head(w, kind)
    di = synth.draft_inputs(shape, seed=42, device=DEV, prefix=prefix)
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    tree = capi.Eagle3TreeCfg(depth=shape.depth, topk=shape.topk, width=shape.width,
                              n_nodes=shape.n_nodes)
    out = capi.eagle3_draft_expand(dr, tree, di["h_low"], di["h_mid"], di["h_high"], di["root_tok"],
                                   di["kpre"], di["vpre"], di["cu_prefix"], max(prefix), debug=True,
                                   debug_logits=True)
    torch.cuda.synchronize()
    check_topk_on_gpu_logits(shape, out["debug"], shape.B)
    check_selection_replay(shape, out, shape.B)
    check_teacher_forced(shape, w, di, out, shape.B, prefix)


def test_draft_ignores_stale_workspace_contents():
    """Unused evaluation slots sit inside the drafter's tree-key range (masked out); the
    round must not depend on what the workspace held before (here: all NaN bytes)."""
    need_gpu()
    shape = SMALL_BF16
    prefix = [300, 0, 1000]
    w = synth.drafter_weights(shape, seed=7, device=DEV)
    di = synth.draft_inputs(shape, seed=8, device=DEV, prefix=prefix)
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    tree = capi.Eagle3TreeCfg(depth=shape.depth, topk=shape.topk, width=shape.width,
                              n_nodes=shape.n_nodes)
    nbytes = capi.eagle3_draft_expand_workspace_size(dr, tree, shape.B, max(prefix))
    outs = []
    for fill in (0xFF, 0x00):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        outs.append(capi.eagle3_draft_expand(dr, tree, di["h_low"], di["h_mid"], di["h_high"],
                                             di["root_tok"], di["kpre"], di["vpre"], di["cu_prefix"],
                                             max(prefix), workspace=ws))
    torch.cuda.synchronize()
    for k in ("tokens", "parents", "depth", "score", "n_nodes"):
        assert torch.equal(outs[0][k], outs[1][k]), k
    assert torch.isfinite(outs[0]["score"][:, :shape.n_nodes + 1]).all()


def _tied_lm_head(w, kind):
    """Rewrite the LM head so that its logits tie: "periodic3" gives every row only three
    distinct logit values (ids t = r mod 3 tie), "paired" makes rows 2j and 2j+1 equal (each
    value appears twice, at adjacent ids)."""
    lm = w["w_lm"]
    if kind == "periodic3":
        base = lm[:3].clone()
        lm.copy_(base.repeat((lm.shape[0] + 2) // 3, 1)[:lm.shape[0]])
    elif kind == "paired":
        lm[1::2].copy_(lm[0::2][:lm[1::2].shape[0]])


@pytest.mark.parametrize("kind,V", [("periodic3", 8192), ("paired", 8192), ("plain", 4104),
                                    ("paired", 4104)])
def test_draft_topk_with_tied_logits_and_short_tail_chunk(kind, V):
    """Top-K ids (value desc, id asc) stay exact when logits tie heavily (every wave falls
    back to exact argmax rounds), when ties sit at the selection threshold, and when the
    last 4096-logit chunk holds fewer than K logits (V = 4104, K = 10)."""
    need_gpu()
    shape = synth.scaled(SMALL_BF16, V=V, B=2, depth=3, topk=10, width=4, n_nodes=20)
    prefix = [100, 257]
    w = synth.drafter_weights(shape, seed=31, device=DEV)
    _tied_lm_head(w, kind)
    di = synth.draft_inputs(shape, seed=32, device=DEV, prefix=prefix)
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    tree = capi.Eagle3TreeCfg(depth=shape.depth, topk=shape.topk, width=shape.width,
                              n_nodes=shape.n_nodes)
    out = capi.eagle3_draft_expand(dr, tree, di["h_low"], di["h_mid"], di["h_high"], di["root_tok"],
                                   di["kpre"], di["vpre"], di["cu_prefix"], max(prefix), debug=True,
                                   debug_logits=True)
    torch.cuda.synchronize()
    check_topk_on_gpu_logits(shape, out["debug"], shape.B)
    check_selection_replay(shape, out, shape.B)
    check_teacher_forced(shape, w, di, out, shape.B, prefix)
