"""GPU parity of the verify side against the oracle: tree mask (bit-exact), tree attention
and LSE merge (fp32 1e-4 / bf16 2e-2 relative), acceptance (bit-exact), sampling
(chi-square) -- all through the C-ABI."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import capi, synth
from tests.gpu_util import TOL, lse_err, need_gpu, np32, rel_err, rel_err_rows, u64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cu_of(trees):
    cu = [0]
    for t in trees:
        cu.append(cu[-1] + len(t))
    return cu


# --------------------------------------------------------------------------- tree mask
GOLD = os.path.join(os.path.dirname(__file__), "golden", "tree_masks.json")


def test_mask_worked_examples():
    need_gpu()
    cases = json.load(open(GOLD))["cases"]
    trees = [c["parents"] for c in cases]
    cu = cu_of(trees)
    par = torch.tensor([p for t in trees for p in t], dtype=torch.int32, device=DEV)
    cup = torch.tensor([0, 7, 7, 107], dtype=torch.int32, device=DEV)
    out = capi.eagle3_build_tree_mask(torch.tensor(cu, dtype=torch.int32, device=DEV), par, cup,
                                      max_nodes=max(len(t) for t in trees))
    m = u64(out["mask"])[:, 0]
    dep = out["depth"].cpu().numpy()
    pos = out["pos"].cpu().numpy()
    P = [7, 0, 100]
    for b, c in enumerate(cases):
        for i, hx in enumerate(c["mask_hex"]):
            assert int(m[cu[b] + i]) == int(hx, 16)
            assert dep[cu[b] + i] == c["depth"][i]
            assert pos[cu[b] + i] == P[b] + c["depth"][i]


@pytest.mark.parametrize("W64,sizes", [(1, [1, 5, 64, 17, 33]), (2, [65, 128, 3]), (4, [256, 200])])
def test_mask_random_trees_bitexact(W64, sizes):
    need_gpu()
    trees = [synth.random_tree(n, 6 if W64 == 1 else 40, 1000 + n) for n in sizes]
    trees.append(synth.chain_tree(64 * W64))
    cu = cu_of(trees)
    pre = [0]
    for i in range(len(trees)):
        pre.append(pre[-1] + 13 * i)
    par = [p for t in trees for p in t]
    om, od, op, ok = O.build_tree_mask(par, cu, pre, words=W64)
    assert ok
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = capi.eagle3_build_tree_mask(torch.tensor(cu, dtype=torch.int32, device=DEV),
                                      torch.tensor(par, dtype=torch.int32, device=DEV),
                                      torch.tensor(pre, dtype=torch.int32, device=DEV),
                                      max_nodes=64 * W64, W64=W64, dev_status=status)
    assert np.array_equal(u64(out["mask"]), om)
    assert np.array_equal(out["depth"].cpu().numpy(), od)
    assert np.array_equal(out["pos"].cpu().numpy(), op)
    assert int(status.item()) == 0


def test_mask_flags_bad_parents():
    need_gpu()
    par = torch.tensor([-1, 0, 5, 1, -1, 0, 0], dtype=torch.int32, device=DEV)   # node 2 bad
    cu = torch.tensor([0, 4, 7], dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = capi.eagle3_build_tree_mask(cu, par, None, max_nodes=4, dev_status=status)
    assert int(status.item()) & 1
    m = u64(out["mask"])[:, 0]
    assert int(m[2]) == 0b101       # treated as a child of the root
    assert [int(x) for x in m[4:]] == [1, 3, 5]


# --------------------------------------------------------------------------- attention
def attn_case(shape, trees, prefix, seed):
    vi = synth.verify_inputs(shape, trees, prefix, seed=seed, device=DEV, with_logits=False)
    cu = vi["cu_nodes"]
    mk = capi.eagle3_build_tree_mask(cu, vi["parents"], vi["cu_prefix"], max_nodes=max(len(t) for t in trees))
    return vi, mk


def oracle_attention(vi, mask_np, scale):
    return O.tree_attention(vi["q"].cpu(), vi["k_tree"].cpu(), vi["v_tree"].cpu(),
                            vi["cu_nodes"].tolist(), mask_np, vi["kpre"].cpu(), vi["vpre"].cpu(),
                            vi["cu_prefix"].tolist(), scale)


ATTN_CASES = [
    # name, dtype, Hq, Hkv, Dh, tree sizes, prefix lengths, splits
    ("tiny_fp32", torch.float32, 4, 4, 64, [15], [128], 0),
    ("gqa_bf16_ragged", torch.bfloat16, 32, 8, 128, [61, 1, 17], [2048, 0, 333], 0),
    ("gqa_bf16_splits", torch.bfloat16, 8, 2, 128, [9, 30], [700, 129], 5),
    ("fp32_dh128_many_splits", torch.float32, 4, 2, 128, [7, 64], [65, 1000], 9),
    ("bf16_dh64_no_prefix", torch.bfloat16, 8, 8, 64, [40, 2], [0, 0], 0),
    ("gqa8_bf16", torch.bfloat16, 64, 8, 128, [61], [515], 0),
    # prefix lengths 0 and 8192 in one call: a lone root's output is its own value (large),
    # a long prefix's output is an average of 8192 values (small); per-row tolerance
    ("bf16_prefix_0_and_8192", torch.bfloat16, 32, 8, 128, [1, 61, 5], [0, 8192, 8192], 0),
    # automatic splits where each (request, KV head) has a single row block: 80 rows per KV
    # head in one 128-row block (the 70B-shaped drafter steps) and 40 rows in one 64-row
    # block (the 8B-shaped ones), ragged prefixes down to less than one key tile
    ("rows80_one_block_auto_splits", torch.bfloat16, 64, 8, 128, [10, 3, 10], [8192, 77, 1000], 0),
    ("rows40_one_block_auto_splits", torch.bfloat16, 32, 8, 128, [10, 10, 1], [2048, 333, 40], 0),
    # head size 64 with a prefix in both bf16 workgroup shapes (96 and 48 rows per KV head)
    ("dh64_rows96_prefix", torch.bfloat16, 16, 2, 64, [12, 5], [1000, 64], 0),
    ("dh64_rows48_prefix", torch.bfloat16, 8, 2, 64, [12, 3], [500, 129], 0),
]


@pytest.mark.parametrize("name,dt,Hq,Hkv,Dh,sizes,prefix,splits", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_tree_attention_matches_oracle(name, dt, Hq, Hkv, Dh, sizes, prefix, splits):
    need_gpu()
    shape = synth.scaled(synth.LLAMA8B, dtype="f32" if dt == torch.float32 else "bf16",
                         Hq=Hq, Hkv=Hkv, Dh=Dh)
    trees = [synth.random_tree(n, 6, 50 + n) for n in sizes]
    vi, mk = attn_case(shape, trees, prefix, seed=len(name))
    scale = float(np.float32(1.0 / math.sqrt(Dh)))
    out = capi.eagle3_tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], vi["cu_nodes"],
                                     max(sizes), mk["mask"], vi["kpre"], vi["vpre"], vi["cu_prefix"],
                                     max(prefix), scale, n_splits=splits, partials=True, merged=True)
    torch.cuda.synchronize()
    mask_np = u64(mk["mask"])
    Oref, Lref = oracle_attention(vi, mask_np, scale)
    assert rel_err(np32(out["o"]), Oref) <= TOL[dt]
    assert rel_err_rows(np32(out["o"]), Oref, Dh) <= TOL[dt]
    assert lse_err(np32(out["lse"]), Lref) <= TOL[dt]
    # each partial equals the oracle restricted to that split's keys
    S = out["splits"]
    cp = vi["cu_prefix"].tolist()
    for s in range(S + 1):
        def filt(b, P, s=s):
            keep = np.zeros(P, dtype=bool)
            if s < S:
                ch = (-(-P // S) + 127) // 128 * 128   # split size: ceil(P/S) up to a multiple of 128
                keep[min(P, s * ch):min(P, s * ch + ch)] = True
            return keep, np.full(sizes[b], s == S)
        o_s, l_s = O.tree_attention(vi["q"].cpu(), vi["k_tree"].cpu(), vi["v_tree"].cpu(),
                                    vi["cu_nodes"].tolist(), mask_np, vi["kpre"].cpu(), vi["vpre"].cpu(),
                                    cp, scale, key_filter=filt)
        assert rel_err(np32(out["o_part"][s]), o_s) <= max(TOL[dt], 1e-4) or np.all(o_s == 0)
        assert rel_err_rows(np32(out["o_part"][s]), o_s, Dh) <= max(TOL[dt], 1e-4)
        assert lse_err(np32(out["lse_part"][s]), l_s) <= TOL[dt]


def test_tree_attention_path_invariant_chain():
    """A chain tree must equal causal attention over [prefix; chain] (bf16 and fp32)."""
    need_gpu()
    for dt in (torch.float32, torch.bfloat16):
        shape = synth.scaled(synth.LLAMA8B, dtype="f32" if dt == torch.float32 else "bf16",
                             Hq=8, Hkv=2, Dh=128)
        trees = [synth.chain_tree(64)]
        vi, mk = attn_case(shape, trees, [100], seed=3)
        out = capi.eagle3_tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], vi["cu_nodes"], 64,
                                         mk["mask"], vi["kpre"], vi["vpre"], vi["cu_prefix"], 100,
                                         float(np.float32(1 / math.sqrt(128))))
        q = vi["q"].double().cpu()
        keys = torch.cat([vi["kpre"], vi["k_tree"]]).double().cpu()
        vals = torch.cat([vi["vpre"], vi["v_tree"]]).double().cpu()
        qs = torch.cat([torch.zeros(100, 8, 128, dtype=torch.float64), q]).permute(1, 0, 2)[None]
        kk = keys.permute(1, 0, 2)[None].repeat_interleave(4, 1)
        vv = vals.permute(1, 0, 2)[None].repeat_interleave(4, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qs, kk, vv, is_causal=True, scale=float(np.float32(1 / math.sqrt(128))))
        ref = ref[0].permute(1, 0, 2)[100:].numpy()
        assert rel_err(np32(out["o"]), ref) <= TOL[dt]


def test_lse_merge_matches_oracle():
    need_gpu()
    g = torch.Generator().manual_seed(0)
    S, rows, Dh = 6, 333, 128
    o = torch.randn(S, rows, Dh, generator=g)
    l = torch.randn(S, rows, generator=g) * 3
    l[2, :50] = -math.inf
    l[:, 60:64] = -math.inf       # rows with every partial empty
    for dt in (torch.float32, torch.bfloat16):
        out = capi.eagle3_lse_merge(o.to(DEV), l.to(DEV), out_dtype=dt)
        Oref, Lref = O.lse_merge(o.numpy(), l.numpy())
        assert rel_err(np32(out["o"]), Oref) <= (1e-5 if dt == torch.float32 else 1e-2)
        assert lse_err(np32(out["lse"]), Lref) <= 1e-6
        assert np.all(np32(out["o"])[60:64] == 0)


# --------------------------------------------------------------------------- accept
def accept_case(V, sizes, dt, seed, plant=True):
    rng = np.random.default_rng(seed)
    trees = [synth.random_tree(n, 6, seed * 7 + n) for n in sizes]
    cu = cu_of(trees)
    tokens = torch.tensor(rng.integers(0, V, cu[-1]), dtype=torch.int32)
    logits = torch.tensor(rng.standard_normal((cu[-1], V)), dtype=torch.float32).to(dt)
    if plant:
        for b, t in enumerate(trees):
            synth.plant_path(logits, tokens, t, cu[b], int(rng.integers(0, len(t))))
    return trees, cu, tokens, logits


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("temperature", [0.0, 1.0, 0.7])
def test_accept_bitexact(dt, temperature):
    need_gpu()
    V = 5003
    sizes = [1, 61, 13, 48, 7]
    trees, cu, tokens, logits = accept_case(V, sizes, dt, seed=int(temperature * 10) + 3)
    par = [p for t in trees for p in t]
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    par_t = torch.tensor(par, dtype=torch.int32, device=DEV)
    mk = capi.eagle3_build_tree_mask(cu_t, par_t, None, max_nodes=max(sizes))
    for rnd in (0, 1, 12345):
        out = capi.eagle3_accept(cu_t, tokens.to(DEV), par_t, mk["mask"], logits.to(DEV),
                                 temperature, seed=0xDEADBEEF12345678, round=rnd, max_depth=6)
        acc, path, outt, bonus = O.accept(cu, tokens.tolist(), par, logits, temperature,
                                          0xDEADBEEF12345678, rnd, 6)
        assert np.array_equal(out["accept_len"].cpu().numpy(), acc)
        assert np.array_equal(out["path"].cpu().numpy(), path)
        assert np.array_equal(out["out_tokens"].cpu().numpy(), outt)
        assert np.array_equal(out["bonus"].cpu().numpy(), bonus)
        if temperature == 0.0:
            break


def test_accept_full_vocab_and_no_match():
    need_gpu()
    V = 128256
    trees, cu, tokens, logits = accept_case(V, [61, 61], torch.bfloat16, seed=9, plant=False)
    par = [p for t in trees for p in t]
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    par_t = torch.tensor(par, dtype=torch.int32, device=DEV)
    mk = capi.eagle3_build_tree_mask(cu_t, par_t, None, max_nodes=61)
    for T_ in (0.0, 0.7):
        out = capi.eagle3_accept(cu_t, tokens.to(DEV), par_t, mk["mask"], logits.to(DEV), T_,
                                 seed=7, round=3, max_depth=6)
        acc, path, outt, bonus = O.accept(cu, tokens.tolist(), par, logits, T_, 7, 3, 6)
        assert np.array_equal(out["accept_len"].cpu().numpy(), acc)
        assert np.array_equal(out["bonus"].cpu().numpy(), bonus)
        assert np.array_equal(out["out_tokens"].cpu().numpy(), outt)


def test_accept_chi_square_on_gpu():
    """Losslessness on the GPU path: the first emitted token of the K=3 two-level tree with
    V=16, T=1 follows softmax(z_root) over 1e6 draws (chi-square p > 0.01); the second token,
    given the accepted depth-1 child c, follows softmax(z_c) (p > 0.01); and the GPU's draws
    equal the oracle's for sampled rounds."""
    need_gpu()
    from scipy import stats
    V = 16
    rng = np.random.default_rng(5)
    par = synth.full_tree(3, 2)
    n = len(par)
    z = (rng.standard_normal((n, V)) * 1.2).astype(np.float32)
    # the depth-1 children carry the root's three most likely tokens, so that about half of
    # the 1e6 rounds go through a child and the conditional test below sees many draws
    tok = [0] + [int(x) for x in np.argsort(-z[0])[:3]] + [int(x) for x in rng.integers(0, V, 9)]
    B = 100000
    cu = torch.arange(0, (B + 1) * n, n, dtype=torch.int32, device=DEV)
    par_t = torch.tensor(par * B, dtype=torch.int32, device=DEV)
    tok_t = torch.tensor(tok * B, dtype=torch.int32, device=DEV)
    lg = torch.tensor(np.tile(z, (B, 1)), dtype=torch.float32, device=DEV)
    mk = capi.eagle3_build_tree_mask(cu, par_t, None, max_nodes=n)
    firsts, seconds, vias = [], [], []
    for rnd in range(10):
        out = capi.eagle3_accept(cu, tok_t, par_t, mk["mask"], lg, 1.0, seed=424242, round=rnd,
                                 max_depth=2)
        firsts.append(out["out_tokens"][:, 0].cpu().numpy())
        went = out["accept_len"].cpu().numpy() >= 1
        seconds.append(out["out_tokens"][:, 1].cpu().numpy()[went])
        vias.append(out["path"][:, 1].cpu().numpy()[went])
        if rnd == 0:
            for b in (0, 1, 777, B - 1):
                acc, path, outt, bonus = O.accept([0, n], tok, par, z, 1.0, 424242, 0, 2)
                # request b uses counter word b: recompute its draw for the root directly
                y = O.node_draw(z[0], 1.0, 424242, 0, b, 0)
                assert out["out_tokens"][b, 0].item() == y
    y = np.concatenate(firsts)
    p = np.exp(z[0].astype(np.float64) - z[0].max())
    p /= p.sum()
    obs = np.bincount(y, minlength=V)
    assert stats.chisquare(obs, p * obs.sum()).pvalue > 0.01
    # the second token, given that the walk went through depth-1 child c (path[1] == c), is the
    # draw at c: it follows softmax(z_c) (one chi-square over the three children's tables)
    chi, dof = 0.0, 0
    sec = np.concatenate(seconds)
    via = np.concatenate(vias)
    for c in (1, 2, 3):
        yc = sec[via == c]
        pc = np.exp(z[c].astype(np.float64) - z[c].max())
        pc /= pc.sum()
        e = pc * len(yc)
        keep = e >= 5
        o = np.bincount(yc, minlength=V)[keep]
        e = e[keep] / e[keep].sum() * o.sum()
        chi += ((o - e) ** 2 / e).sum()
        dof += int(keep.sum()) - 1
    assert len(sec) > 300000 and stats.chi2.sf(chi, dof) > 0.01, (chi, dof)


def test_accept_duplicate_siblings_and_ties_on_gpu():
    """Greedy acceptance with sibling nodes carrying the same token (possible in random-topology
    trees): both are length-1 matches, the lower index wins; a deeper match under the
    higher-index sibling wins by length; greedy ties inside a row go to the lowest token id.
    Then random trees whose siblings repeat tokens, GPU against the oracle bit for bit."""
    need_gpu()
    par = [-1, 0, 0, 2]
    tok = [9, 4, 4, 6]
    z = np.zeros((4, 10), dtype=np.float32)
    z[0, 4] = 1
    z[1, 1] = 1
    z[2, 7] = 1
    z[3, 2] = 1
    cu = torch.tensor([0, 4], dtype=torch.int32, device=DEV)
    par_t = torch.tensor(par, dtype=torch.int32, device=DEV)
    tok_t = torch.tensor(tok, dtype=torch.int32, device=DEV)
    mk = capi.eagle3_build_tree_mask(cu, par_t, None, max_nodes=4)
    out = capi.eagle3_accept(cu, tok_t, par_t, mk["mask"], torch.tensor(z, device=DEV), 0.0, seed=0,
                             round=0, max_depth=2)
    assert out["accept_len"].item() == 1 and out["path"][0, 1].item() == 1 and out["bonus"].item() == 1
    z[2, 7] = 0
    z[2, 6] = 1
    out = capi.eagle3_accept(cu, tok_t, par_t, mk["mask"], torch.tensor(z, device=DEV), 0.0, seed=0,
                             round=0, max_depth=2)
    assert out["accept_len"].item() == 2 and out["path"][0].tolist() == [0, 2, 3] and out["bonus"].item() == 2
    zt = np.zeros((1, 6), dtype=np.float32)
    zt[0, [2, 4]] = 3.0
    one = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    root = torch.tensor([-1], dtype=torch.int32, device=DEV)
    mk1 = capi.eagle3_build_tree_mask(one, root, None, max_nodes=1)
    out = capi.eagle3_accept(one, torch.zeros(1, dtype=torch.int32, device=DEV), root, mk1["mask"],
                             torch.tensor(zt, device=DEV), 0.0, seed=0, round=0, max_depth=0)
    assert out["bonus"].item() == 2
    # random trees, tokens drawn from a 3-token alphabet so siblings repeat; each parent row
    # favours one of those tokens
    rng = np.random.default_rng(17)
    V, sizes = 64, [40, 61, 17, 2, 33]
    trees = [synth.random_tree(n, 6, 900 + n) for n in sizes]
    cuh = cu_of(trees)
    parh = [p for t in trees for p in t]
    tokh = rng.integers(0, 3, cuh[-1]).tolist()
    zr = rng.standard_normal((cuh[-1], V)).astype(np.float32)
    zr[np.arange(cuh[-1]), rng.integers(0, 3, cuh[-1])] += 4.0
    for dt in (torch.float32, torch.bfloat16):
        zd = torch.tensor(zr).to(dt)
        cu_t = torch.tensor(cuh, dtype=torch.int32, device=DEV)
        p_t = torch.tensor(parh, dtype=torch.int32, device=DEV)
        mk = capi.eagle3_build_tree_mask(cu_t, p_t, None, max_nodes=max(sizes))
        out = capi.eagle3_accept(cu_t, torch.tensor(tokh, dtype=torch.int32, device=DEV), p_t, mk["mask"],
                                 zd.to(DEV), 0.0, seed=0, round=0, max_depth=6)
        acc, path, outt, bonus = O.accept(cuh, tokh, parh, zd, 0.0, 0, 0, 6)
        assert np.array_equal(out["accept_len"].cpu().numpy(), acc)
        assert np.array_equal(out["path"].cpu().numpy(), path)
        assert np.array_equal(out["out_tokens"].cpu().numpy(), outt)
        assert np.array_equal(out["bonus"].cpu().numpy(), bonus)
        assert acc.max() >= 1
    # the random trees do hold siblings with equal tokens
    kids = {}
    for b, t in enumerate(trees):
        for j in range(1, len(t)):
            kids.setdefault((b, t[j]), []).append(tokh[cuh[b] + j])
    assert any(len(v) != len(set(v)) for v in kids.values())
