"""Pins for the oracle's training form of the long-context shape ([P4] USP 核心设计：三步走):
causal main attention, per-position branch attention, and their streaming-softmax fusion."""
import numpy as np

from oracle import eagle3_oracle as O


def _inputs(L, s, Hq=4, Hkv=2, Dh=8, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, Hq, Dh))
    k = rng.standard_normal((L, Hkv, Dh))
    v = rng.standard_normal((L, Hkv, Dh))
    kb = rng.standard_normal((s, L, Hkv, Dh))
    vb = rng.standard_normal((s, L, Hkv, Dh))
    return q, k, v, kb, vb


def test_causal_equals_chain_tree_attention():
    """Causal attention over a sequence is tree attention over a chain with no prefix: the
    chain's ancestor mask is the lower triangle (an independent path through the oracle)."""
    L = 23
    q, k, v, _, _ = _inputs(L, 1)
    sc = 0.3
    o, lse = O.causal_attention(q, k, v, sc)
    par = [-1] + list(range(L - 1))
    mask, _, _, _ = O.build_tree_mask(par, [0, L], [0, 0], words=1)
    ot, lt = O.tree_attention(q, k, v, [0, L], mask, np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), [0, 0], sc)
    np.testing.assert_allclose(o, ot, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lt, rtol=1e-12, atol=1e-12)


def test_causal_first_position_and_uniform_keys():
    """Position 0 sees only its own key: O = v_0, LSE = scale q.k_0.  With all keys equal,
    position t averages its t+1 values and LSE = scale q.k + ln(t+1)."""
    L = 9
    q, k, v, _, _ = _inputs(L, 1, seed=2)
    o, lse = O.causal_attention(q, k, v, 0.5)
    np.testing.assert_allclose(o[0, 1], v[0, 0], rtol=1e-13)
    np.testing.assert_allclose(lse[0, 3], 0.5 * q[0, 3] @ k[0, 1], rtol=1e-13)
    k2 = np.broadcast_to(k[:1], k.shape).copy()
    o2, l2 = O.causal_attention(q, k2, v, 0.5)
    for t in range(L):
        np.testing.assert_allclose(o2[t, 2], v[:t + 1, 1].mean(axis=0), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l2[t, 2], 0.5 * q[t, 2] @ k[0, 1] + np.log(t + 1), rtol=1e-12)


def test_branch_single_step_and_rows_independent():
    """One branch step: weight 1 on that key (O = its value, LSE = its score).  Positions do
    not interact: permuting positions permutes the result."""
    L = 11
    q, _, _, kb, vb = _inputs(L, 1, seed=3)
    o, lse = O.branch_attention(q, kb, vb, 0.7)
    np.testing.assert_allclose(o[:, 1], vb[0, :, 0], rtol=1e-13)
    np.testing.assert_allclose(lse[:, 1], 0.7 * np.einsum("ld,ld->l", q[:, 1], kb[0, :, 0]), rtol=1e-12)
    q, _, _, kb, vb = _inputs(L, 5, seed=4)
    o, lse = O.branch_attention(q, kb, vb, 0.7)
    perm = np.random.default_rng(0).permutation(L)
    o2, l2 = O.branch_attention(q[perm], kb[:, perm], vb[:, perm], 0.7)
    np.testing.assert_allclose(o2, o[perm], rtol=1e-13)


def test_fusion_equals_softmax_over_main_and_branch_keys():
    """Step 3: merging (Out_main, LSE_main) with (Out_branch, LSE_branch) equals one softmax
    over the concatenated key list (main keys 0..t, then the position's branch keys)."""
    L, s, sc = 17, 7, 0.4
    q, k, v, kb, vb = _inputs(L, s, seed=5)
    om, lm = O.causal_attention(q, k, v, sc)
    ob, lb = O.branch_attention(q, kb, vb, sc)
    Hq, Dh = q.shape[1], q.shape[2]
    o, lse = O.lse_merge(np.stack([om.reshape(-1, Dh), ob.reshape(-1, Dh)]),
                         np.stack([lm.reshape(-1), lb.reshape(-1)]))
    for t in (0, 5, 16):
        for h in range(Hq):
            c = h // 2
            keys = np.concatenate([k[:t + 1, c], kb[:, t, c]])
            vals = np.concatenate([v[:t + 1, c], vb[:, t, c]])
            ref, rl = O.attend(q[t, h], keys, vals, sc)
            np.testing.assert_allclose(o.reshape(L, Hq, Dh)[t, h], ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse.reshape(L, Hq)[t, h], rl, rtol=1e-12)


def test_causal_rows_subset():
    L = 15
    q, k, v, _, _ = _inputs(L, 1, seed=6)
    o, lse = O.causal_attention(q, k, v, 0.2)
    o2, l2 = O.causal_attention(q, k, v, 0.2, rows=[3, 14])
    np.testing.assert_allclose(o2[[3, 14]], o[[3, 14]], rtol=0, atol=0)
    assert np.all(np.isneginf(l2[[0, 1, 2, 4]]))
