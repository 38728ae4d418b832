"""Pins for the oracle's sampled-candidate acceptance (keep a drafted token with probability
min(1, p/q), dice left to right, correct at the first rejection; siblings drawn without
replacement, the rejected token taken out of q and the target side replaced by the
normalised positive part of p - q).  The pins: the page's E/F/G chain walk, chains worked
out by hand, the exact output distribution of one node (every ordered candidate list
enumerated) equal to p, and a chi-square test of the whole walk with Philox uniforms and
Gumbel corrections on a two-level tree."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import eagle3_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def test_efg_chain_golden():
    g = json.load(open(os.path.join(HERE, "golden", "sampled_chain_efg.json")))
    kept = []
    for nd in g["nodes"]:
        k, p, thr = O.rrs_node(np.array(nd["p"]), np.array(nd["q"]), [nd["candidate"]], [nd["u"]])
        assert thr[0] == pytest.approx(nd["ratio"], rel=1e-12)
        if k < 0:
            np.testing.assert_allclose(p, g["residual_at_rejection"], rtol=0, atol=1e-15)
            assert O.residual_draw(p, np.zeros(4)) == g["correction_token"]
            break
        kept.append(nd["candidate"])
    assert kept == g["kept"]


def test_three_siblings_by_hand():
    """p = [.1 .2 .3 .4], q = [.4 .3 .2 .1], children drawn as tokens 0, 1, 2.
    Child 0: p/q = 1/4.  Rejected: p <- [0 0 .1 .3]/.4 = [0 0 1/4 3/4], q <- [0 .3 .2 .1]/.6.
    Child 1: p/q = 0.  Rejected: p <- max([0 0 1/4 3/4] - [0 1/2 1/3 1/6], 0) = [0 0 0 7/12]
    -> [0 0 0 1], q <- [0 0 .2 .1]/.3.  Child 2: p/q = 0.  Rejected: p stays [0 0 0 1]."""
    p = np.array([0.1, 0.2, 0.3, 0.4])
    q = np.array([0.4, 0.3, 0.2, 0.1])
    k, pr, thr = O.rrs_node(p, q, [0, 1, 2], [np.inf] * 3)
    assert k == -1
    assert thr[0] == pytest.approx(0.25, rel=1e-14) and thr[1] == 0.0 and thr[2] == 0.0
    np.testing.assert_allclose(pr, [0, 0, 0, 1], atol=1e-15)
    # the first uniform below 1/4 keeps child 0; above it, children 1 and 2 can never be kept
    assert O.rrs_node(p, q, [0, 1, 2], [0.2, 0.0, 0.0])[0] == 0
    assert O.rrs_node(p, q, [0, 1, 2], [0.3, 0.0, 0.0])[0] == -1


def test_two_siblings_second_always_kept():
    """p = [.5 .3 .2], q = [.2 .6 .2], drawn 1 then 0.  Child 1: p/q = 1/2.  Rejected:
    p <- [.3 0 0]/.3 = [1 0 0], q <- [.2 0 .2]/.4 = [1/2 0 1/2].  Child 0: p/q = 2: kept
    whatever its uniform."""
    k, _, thr = O.rrs_node(np.array([0.5, 0.3, 0.2]), np.array([0.2, 0.6, 0.2]), [1, 0], [0.9, 0.999])
    assert k == 1 and thr == [pytest.approx(0.5), pytest.approx(2.0)]


def test_skips_repeated_and_out_of_vocabulary_candidates():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    q = np.array([0.4, 0.3, 0.2, 0.1])
    k, pr, thr = O.rrs_node(p, q, [0, 0, 9, -1, 3], [np.inf, 0.0, 0.0, 0.0, np.inf])
    assert thr[1] is None and thr[2] is None and thr[3] is None
    assert k == -1 and thr[4] == pytest.approx(4.5)       # after child 0: p(3) = 3/4, q(3) = 1/6
    _, pr1, _ = O.rrs_node(p, q, [0, 3], [np.inf, np.inf])
    np.testing.assert_array_equal(pr, pr1)


def test_equal_distributions_keep_the_first_child():
    rng = np.random.default_rng(0)
    p = rng.dirichlet(np.ones(16))
    for u in (0.0, 0.5, 0.999999):
        assert O.rrs_node(p, p.copy(), [3, 5, 7], [u, u, u])[0] == 0


def _exact_output(p, q, K):
    """Probability of each output token when K children are drawn without replacement from q
    (every ordered list enumerated with its probability) and go through rrs_node; a child is
    kept with probability min(1, threshold)."""
    V = len(p)
    out = np.zeros(V)
    for seq in itertools.permutations(range(V), K):
        pr, left = 1.0, 1.0
        for x in seq:
            pr *= q[x] / left
            left -= q[x]
        _, pfin, thr = O.rrs_node(p, q, list(seq), [np.inf] * K)
        reach = 1.0
        for x, t in zip(seq, thr):
            a = min(1.0, t)
            out[x] += pr * reach * a
            reach *= 1.0 - a
        out += pr * reach * pfin
    return out


@pytest.mark.parametrize("V", [3, 4, 5])
def test_one_node_output_is_exactly_the_target(V):
    """Losslessness at one node, by enumeration: for every number of children K (1 .. V) the
    output distribution equals p (to rounding).  Dropping the renormalisation of q, keeping a
    rejected token in q, or correcting from max(q - p, 0) each break this."""
    rng = np.random.default_rng(V)
    for trial in range(4):
        p = rng.dirichlet(np.ones(V) * 0.7)
        q = rng.dirichlet(np.ones(V) * 0.7)
        if trial == 3:
            q[0] = 0.0            # a token the drafter never proposes
            q /= q.sum()
        for K in range(1, V + 1):
            if K > np.count_nonzero(q):
                continue
            np.testing.assert_allclose(_exact_output(p, q, K), p, rtol=0, atol=1e-12)


def test_residual_of_one_candidate_is_the_standard_correction():
    rng = np.random.default_rng(3)
    p, q = rng.dirichlet(np.ones(7)), rng.dirichlet(np.ones(7))
    x = int(np.argmax(q / p))                          # a token with p < q
    k, pr, thr = O.rrs_node(p, q, [x], [np.inf])
    r = np.maximum(p - q, 0)
    np.testing.assert_allclose(pr, r / r.sum(), rtol=1e-14)
    assert thr[0] == pytest.approx(p[x] / q[x], rel=1e-14)


def test_softmax64_closed_form():
    z = np.array([0.0, np.log(3.0), np.log(6.0)], dtype=np.float32)
    np.testing.assert_allclose(O.softmax64(z, 1.0), [0.1, 0.3, 0.6], rtol=1e-7)
    np.testing.assert_allclose(O.softmax64(2 * z, 2.0), O.softmax64(z, 1.0), rtol=1e-15)


def test_accept_uniform_is_uniform_and_distinct_from_the_gumbel_stream():
    us = np.array([O.accept_uniform(11, r, 0, 5) for r in range(4000)])
    assert 0 < us.min() and us.max() < 1
    assert abs(us.mean() - 0.5) < 0.02 and abs(us.var() - 1 / 12) < 0.01
    assert len({O.accept_uniform(11, 0, b, j) for b in range(4) for j in range(8)}) == 32


def _path_logits(path, V, rng_seed, shift=0.0):
    r = np.random.default_rng([rng_seed] + [t + 1 for t in path])
    return (r.normal(size=V) * 1.5 + shift).astype(np.float32)


def test_walk_is_lossless_chi_square():
    """Two-level trees: the root draws K1 children without replacement from its draft
    distribution, each child K2 of its own; target and draft logits depend on the token path.
    Over many rounds (fresh Philox uniforms and Gumbel noise per round) the first output token
    must follow p(. | root) and, when the first token was a kept child, the second must
    follow p(. | root, first)."""
    V, K1, K2, T = 6, 3, 2, 0.8
    n_rounds = 3000
    rng = np.random.default_rng(1)
    first = np.zeros(V)
    pair = np.zeros((V, V))
    for rnd in range(n_rounds):
        zr = _path_logits([], V, 7)
        qr = O.softmax64(_path_logits([], V, 8), T)
        c1 = rng.choice(V, size=K1, replace=False, p=qr)
        toks, par, tgt, drf = [0], [-1], [zr], [_path_logits([], V, 8)]
        for x in c1:
            toks.append(int(x)); par.append(0)
            tgt.append(_path_logits([int(x)], V, 7)); drf.append(_path_logits([int(x)], V, 8))
        for a in range(1, K1 + 1):
            qa = O.softmax64(drf[a], T)
            for y in rng.choice(V, size=K2, replace=False, p=qa):
                toks.append(int(y)); par.append(a)
                tgt.append(_path_logits([toks[a], int(y)], V, 7)); drf.append(np.zeros(V, np.float32))
        n = len(toks)
        drow = np.array([i if i <= K1 else -1 for i in range(n)], dtype=np.int32)
        acc, path, outt, bonus = O.accept_sampled([0, n], np.array(toks), np.array(par), np.stack(tgt),
                                                  np.stack(drf), drow, T, 99, rnd, 2)
        first[outt[0, 0]] += 1
        if acc[0] >= 1:
            pair[outt[0, 0], outt[0, 1]] += 1
    p1 = O.softmax64(_path_logits([], V, 7), T)
    chi1 = ((first - n_rounds * p1) ** 2 / (n_rounds * p1)).sum()
    assert chi1 < 20.5, chi1          # chi-square, 5 degrees of freedom, p ~ 1e-3
    chi2, dof = 0.0, 0
    for a in range(V):
        na = pair[a].sum()
        if na < 50:
            continue
        e = na * O.softmax64(_path_logits([a], V, 7), T)
        chi2 += ((pair[a] - e) ** 2 / e).sum()
        dof += V - 1
    assert dof >= 10
    from scipy.stats import chi2 as C
    assert C.sf(chi2, dof) > 1e-3, (chi2, dof)


# ---- the drafter's side: children drawn without replacement ----------------------------


def test_sample_children_is_drawing_without_replacement():
    """Ordered pairs drawn by the Gumbel-top-2 rule over many rounds follow
    q(x1) q(x2) / (1 - q(x1)), q = softmax(z / T) (chi-square over all 20 ordered pairs)."""
    V, T, n = 5, 0.8, 12000
    z = np.array([0.3, -1.0, 1.2, 0.0, 0.7], dtype=np.float32)
    q = O.softmax64(z, T)
    cnt = np.zeros((V, V))
    for rnd in range(n):
        ids, _ = O.sample_children(z, T, 2, 5, rnd, 1, 3)
        cnt[ids[0], ids[1]] += 1
    exp = np.array([[q[a] * q[b] / (1 - q[a]) if a != b else 0 for b in range(V)] for a in range(V)]) * n
    m = exp > 0
    chi = ((cnt[m] - exp[m]) ** 2 / exp[m]).sum()
    from scipy.stats import chi2 as C
    assert C.sf(chi, m.sum() - 1) > 1e-3, chi
    assert np.all(cnt[~m] == 0)


def test_sample_children_values_and_order():
    rng = np.random.default_rng(2)
    z = rng.normal(size=300).astype(np.float32) * 3
    ids, zs = O.sample_children(z, 0.7, 8, 11, 4, 0, 17)
    assert len(set(ids.tolist())) == 8
    invT = np.float32(1) / np.float32(0.7)
    np.testing.assert_array_equal(zs, (z[ids] * invT).astype(np.float32))
    g = O.draft_gumbel(11, 4, 0, 17, np.arange(300))
    v = ((z * invT).astype(np.float32) + g).astype(np.float32)
    assert np.all(np.diff(v[ids].astype(np.float64)) <= 0)          # drawn best first
    assert v[ids[-1]] >= np.sort(v)[-8]                              # and they are the 8 best
    # the drafter's stream is not the verifier's
    assert not np.array_equal(g, O.gumbel(11, 4, 0, 17, np.arange(300)))


def test_expand_tree_scores_keep_sibling_prefixes():
    """With children listed in draw order (values not sorted), a child's score never exceeds
    an earlier sibling's; with a sorted top-K list the scores are the plain cumulative ones."""
    vals = {0: [-0.5, -0.1, -2.0, -0.3], 1: [-1.0, -3.0, -0.2, -0.4]}

    def evaluate(t, nodes):
        out = []
        for nd in nodes:
            v = np.array(vals[min(t, 1)], dtype=np.float32)
            out.append({"topk_ids": np.arange(4) + 10 * t, "topk_vals": v, "lse": np.float32(0.0)})
        return out
    tr = O.expand_tree(3, 4, 2, 12, 7, evaluate)
    by_parent = {}
    for c in tr["cands"]:
        by_parent.setdefault((c["parent_slot"], c["depth"]), []).append(float(c["score"]))
    for sc in by_parent.values():
        assert all(b <= a for a, b in zip(sc, sc[1:]))
    root_kids = by_parent[(0, 1)]
    assert root_kids == [-0.5, -0.5, -2.0, -2.0]

    def evaluate_sorted(t, nodes):
        return [{"topk_ids": np.arange(4), "topk_vals": np.array([-0.1, -0.3, -0.5, -2.0], np.float32),
                 "lse": np.float32(0.0)} for _ in nodes]
    tr = O.expand_tree(2, 4, 2, 8, 7, evaluate_sorted)
    assert [float(c["score"]) for c in tr["cands"][:4]] == [float(np.float32(x)) for x in (-0.1, -0.3, -0.5, -2.0)]
