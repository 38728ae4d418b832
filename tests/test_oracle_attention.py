"""Pins for the oracle's tree attention (O5) and LSE merge (O6).

Independent references: torch's scaled_dot_product_attention (a library routine) on the
explicit root-to-node path sequence, closed forms for one or two keys, and the identity
"merge of partials == one softmax over the concatenated keys"."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import synth


def make(trees, prefix, Hq=4, Hkv=2, Dh=16, seed=0):
    shape = synth.scaled(synth.TINY, Hq=Hq, Hkv=Hkv, Dh=Dh, V=32)
    vi = synth.verify_inputs(shape, trees, prefix, seed=seed, with_logits=False)
    par = [p for t in trees for p in t]
    cu = vi["cu_nodes"].tolist()
    mask, depth, pos, ok = O.build_tree_mask(par, cu, vi["cu_prefix"].tolist())
    assert ok
    return vi, mask, cu


def sdpa_last(q, keys, vals):
    """Attention of one query (Hq, Dh) at the end of a key sequence (L, Hkv, Dh) via torch
    SDPA with grouped heads; returns (Hq, Dh)."""
    Hq, Dh = q.shape
    Hkv = keys.shape[1]
    qt = torch.tensor(q, dtype=torch.float64).reshape(1, Hq, 1, Dh)
    kt = torch.tensor(keys, dtype=torch.float64).permute(1, 0, 2).unsqueeze(0)
    vt = torch.tensor(vals, dtype=torch.float64).permute(1, 0, 2).unsqueeze(0)
    kt = kt.repeat_interleave(Hq // Hkv, dim=1)
    vt = vt.repeat_interleave(Hq // Hkv, dim=1)
    out = Fnn.scaled_dot_product_attention(qt, kt, vt, scale=1.0 / math.sqrt(Dh))
    return out.reshape(Hq, Dh).numpy()


@pytest.mark.parametrize("seed", range(4))
def test_tree_equals_path_attention_bruteforce(seed):
    trees = [synth.random_tree(n, 6, 100 + seed * 7 + i) for i, n in enumerate([1, 9, 23])]
    prefix = [0, 13, 40]
    vi, mask, cu = make(trees, prefix, seed=seed)
    scale = 1.0 / math.sqrt(16)
    Ot, Lt = O.tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], cu, mask, vi["kpre"],
                              vi["vpre"], vi["cu_prefix"].tolist(), scale)
    q = vi["q"].double().numpy()
    kt, vt = vi["k_tree"].double().numpy(), vi["v_tree"].double().numpy()
    kp, vp = vi["kpre"].double().numpy(), vi["vpre"].double().numpy()
    cp = vi["cu_prefix"].tolist()
    for b, t in enumerate(trees):
        for i in range(len(t)):
            path = []
            j = i
            while j >= 0:
                path.append(j)
                j = t[j]
            path.reverse()
            keys = np.concatenate([kp[cp[b]:cp[b + 1]], kt[cu[b] + np.array(path)]], axis=0)
            vals = np.concatenate([vp[cp[b]:cp[b + 1]], vt[cu[b] + np.array(path)]], axis=0)
            ref = sdpa_last(q[cu[b] + i], keys, vals)
            np.testing.assert_allclose(Ot[cu[b] + i], ref, rtol=1e-10, atol=1e-12)


def test_chain_tree_is_causal_attention():
    n, P = 12, 20
    vi, mask, cu = make([synth.chain_tree(n)], [P], Hq=4, Hkv=4, Dh=8, seed=3)
    Ot, _ = O.tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], cu, mask, vi["kpre"],
                             vi["vpre"], [0, P], 1.0 / math.sqrt(8))
    # causal SDPA over the whole sequence [prefix; chain]; prefix queries are unused
    L = P + n
    keys = torch.cat([vi["kpre"], vi["k_tree"]]).double().permute(1, 0, 2).unsqueeze(0)
    vals = torch.cat([vi["vpre"], vi["v_tree"]]).double().permute(1, 0, 2).unsqueeze(0)
    qs = torch.cat([torch.zeros(P, 4, 8, dtype=torch.float64), vi["q"].double()])
    qs = qs.permute(1, 0, 2).unsqueeze(0)
    ref = Fnn.scaled_dot_product_attention(qs, keys, vals, is_causal=True, scale=1 / math.sqrt(8))
    ref = ref[0].permute(1, 0, 2)[P:].numpy()
    np.testing.assert_allclose(Ot, ref, rtol=1e-10, atol=1e-12)


def test_star_and_closed_forms():
    # star tree, no prefix: the root sees itself only -> O = v_root, LSE = scale q.k
    vi, mask, cu = make([synth.star_tree(5)], [0], Hq=2, Hkv=2, Dh=8, seed=5)
    s = 1.0 / math.sqrt(8)
    Ot, Lt = O.tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], cu, mask, vi["kpre"],
                              vi["vpre"], [0, 0], s)
    q, k, v = (vi[x].double().numpy() for x in ("q", "k_tree", "v_tree"))
    for h in range(2):
        np.testing.assert_allclose(Ot[0, h], v[0, h], rtol=1e-12)
        assert abs(Lt[0, h] - s * q[0, h] @ k[0, h]) < 1e-12
        # leaf i sees {root, i}: two keys -> closed form two-way softmax
        for i in range(1, 5):
            a, c = s * q[i, h] @ k[0, h], s * q[i, h] @ k[i, h]
            w0, w1 = 1 / (1 + math.exp(c - a)), 1 / (1 + math.exp(a - c))
            np.testing.assert_allclose(Ot[i, h], w0 * v[0, h] + w1 * v[i, h], rtol=1e-10)
            assert abs(Lt[i, h] - (max(a, c) + math.log1p(math.exp(-abs(a - c))))) < 1e-12


def test_identical_keys_lse_ln2():
    q = np.array([0.3, -1.0, 2.0])
    k = np.array([[1.0, 0.5, -0.25]] * 2)
    v = np.array([[1.0, 2.0, 3.0], [5.0, 6.0, 7.0]])
    o, lse = O.attend(q, k, v, 0.5)
    assert abs(lse - (0.5 * q @ k[0] + math.log(2))) < 1e-14
    np.testing.assert_allclose(o, [3.0, 4.0, 5.0])


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_merge_equals_single_softmax(splits):
    trees = [synth.random_tree(17, 6, 9), synth.random_tree(5, 6, 10)]
    prefix = [50, 3]
    vi, mask, cu = make(trees, prefix, seed=11)
    s = 0.25
    args = (vi["q"], vi["k_tree"], vi["v_tree"], cu, mask, vi["kpre"], vi["vpre"],
            vi["cu_prefix"].tolist(), s)
    Ofull, Lfull = O.tree_attention(*args)
    parts_o, parts_l = [], []
    for sp in range(splits):
        def filt(b, P, sp=sp):
            ch = -(-P // splits)
            keep = np.zeros(P, dtype=bool)
            keep[sp * ch:min(P, (sp + 1) * ch)] = True
            return keep, np.zeros(len(trees[b]), dtype=bool)
        o, l = O.tree_attention(*args, key_filter=filt)
        parts_o.append(o)
        parts_l.append(l)
    o, l = O.tree_attention(*args, key_filter=lambda b, P: (np.zeros(P, bool), np.ones(len(trees[b]), bool)))
    parts_o.append(o)
    parts_l.append(l)
    T, Hq, Dh = Ofull.shape
    po = np.stack(parts_o).reshape(splits + 1, T * Hq, Dh)
    pl = np.stack(parts_l).reshape(splits + 1, T * Hq)
    Om, Lm = O.lse_merge(po, pl)
    np.testing.assert_allclose(Om.reshape(T, Hq, Dh), Ofull, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Lm.reshape(T, Hq), Lfull, rtol=1e-12)
    # order independence
    perm = np.random.default_rng(0).permutation(splits + 1)
    Op, Lp = O.lse_merge(po[perm], pl[perm])
    np.testing.assert_allclose(Op, Om, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lp, Lm, rtol=1e-13)


def test_merge_empty_partials():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, 4, 8))
    l = rng.standard_normal((3, 4))
    base_o, base_l = O.lse_merge(o, l)
    o2 = np.concatenate([o, rng.standard_normal((1, 4, 8))])
    l2 = np.concatenate([l, np.full((1, 4), -np.inf)])
    o3, l3 = O.lse_merge(o2, l2)
    np.testing.assert_allclose(o3, base_o, rtol=1e-14)
    np.testing.assert_allclose(l3, base_l, rtol=1e-14)
    oz, lz = O.lse_merge(o, np.full((3, 4), -np.inf))
    assert np.all(oz == 0) and np.all(np.isneginf(lz))
    # a single partial passes through unchanged
    o1, l1 = O.lse_merge(o[:1], l[:1])
    np.testing.assert_allclose(o1, o[0], rtol=1e-15)
    np.testing.assert_allclose(l1, l[0], rtol=1e-15)


def test_empty_prefix_split_is_neg_inf():
    vi, mask, cu = make([synth.random_tree(4, 6, 1)], [0])
    o, l = O.tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], cu, mask, vi["kpre"],
                            vi["vpre"], [0, 0], 0.25,
                            key_filter=lambda b, P: (np.ones(P, bool), np.zeros(4, bool)))
    assert np.all(np.isneginf(l)) and np.all(o == 0)
