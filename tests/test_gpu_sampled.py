"""GPU parity of eagle3_accept_sampled (acceptance of sampled candidates) against the oracle's
accept_sampled: accepted lengths, paths, output tokens and bonus tokens must be equal (integer
results; both sides take every decision in float64), over many rounds (fresh uniforms and
Gumbel noise), trees from chains to wide stars and random trees, ragged and full
vocabularies, bf16 and fp32 logits, and the edge cases (empty request, a node without a draft
row, repeated and out-of-vocabulary children, more children than max_children, every token the
drafter can propose rejected, a child the drafter gives probability zero)."""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import capi, synth
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"
KEYS = ("accept_len", "path", "out_tokens", "bonus")


def max_kids(trees):
    m = 1
    for t in trees:
        cnt = {}
        for p in t[1:]:
            cnt[p] = cnt.get(p, 0) + 1
        m = max([m] + list(cnt.values()))
    return m


def tree_depth(trees):
    best = 0
    for t in trees:
        d = [0] * len(t)
        for j in range(1, len(t)):
            d[j] = d[t[j]] + 1
        best = max(best, max(d))
    return best


SYNC = 32      # a partial handed between workgroups was not seen within the bounded wait


def gpu_run(d, temp, seed, rnd, max_depth, maxc, status=None):
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = capi.eagle3_accept_sampled(d["cu_nodes"], d["tokens"], d["parents"], d["logits"],
                                     d["draft_logits"], d["draft_row"], temp, seed, rnd, max_depth,
                                     maxc, dev_status=status)
    torch.cuda.synchronize()
    assert not int(status.item()) & SYNC
    return [out[k].cpu().numpy() for k in KEYS]


def oracle_run(d, temp, seed, rnd, max_depth, maxc):
    c = lambda k: d[k].cpu().numpy()
    return O.accept_sampled(c("cu_nodes"), c("tokens"), c("parents"), d["logits"].float().cpu(),
                            d["draft_logits"].float().cpu(), c("draft_row"), temp, seed, rnd,
                            max_depth, max_children=maxc)


def compare(d, temp, seed, rounds, max_depth, maxc, status=None):
    lens = []
    for rnd in rounds:
        print(f"round {rnd}", flush=True)
        got = gpu_run(d, temp, seed, rnd, max_depth, maxc, status)
        ref = oracle_run(d, temp, seed, rnd, max_depth, maxc)
        for k, g, r in zip(KEYS, got, ref):
            assert np.array_equal(g, r), (k, rnd, g, r)
        lens += list(got[0])
    return np.array(lens)


SMALL = [synth.full_tree(3, 3), synth.chain_tree(5), synth.star_tree(12)]


@pytest.mark.parametrize("V,dt,noise,temp", [
    (1003, torch.float32, 3.0, 0.7),       # one ragged chunk, scalar loads, many rejections
    (9000, torch.bfloat16, 1.0, 1.0),      # three chunks, the last ragged
    (9000, torch.float32, 0.3, 1.3),       # mostly kept
], ids=["v1003_f32_noisy", "v9000_bf16", "v9000_f32_close"])
def test_small_trees_match_oracle(V, dt, noise, temp):
    need_gpu()
    d = synth.sampled_tree_inputs(SMALL, V, seed=11, dtype=dt, device=DEV, target_noise=noise)
    lens = compare(d, temp, 1234, range(10), tree_depth(SMALL), max_kids(SMALL))
    assert lens.min() < lens.max()          # the rounds reach different depths


def test_random_trees_full_vocabulary():
    """Random 60-node trees of depth 6 over the Llama-3 vocabulary (128256), bf16."""
    need_gpu()
    trees = [synth.random_tree(60, 6, seed=s) for s in (3, 4)]
    d = synth.sampled_tree_inputs(trees, 128256, seed=21, device=DEV, target_noise=2.0)
    compare(d, 1.0, 77, range(4), tree_depth(trees), max_kids(trees))


def test_batch16_full_vocabulary():
    """Sixteen 48-node trees (the batched serving shape) at V = 128256, bf16."""
    need_gpu()
    trees = [synth.random_tree(48, 6, seed=100 + s) for s in range(16)]
    d = synth.sampled_tree_inputs(trees, 128256, seed=31, device=DEV, target_noise=1.0)
    compare(d, 0.8, 5, range(2), tree_depth(trees), max_kids(trees))


def test_equal_distributions_keep_every_first_child():
    """Target logits equal to the draft logits: p / q = 1 at every candidate, so each node
    keeps its first child and the path is the first-child chain."""
    need_gpu()
    trees = [synth.full_tree(3, 3), synth.random_tree(30, 5, seed=9)]
    d = synth.sampled_tree_inputs(trees, 5000, seed=41, dtype=torch.float32, device=DEV, target_noise=0.0)
    for rnd in range(3):
        acc, path, _, _ = gpu_run(d, 1.0, 3, rnd, tree_depth(trees), max_kids(trees))
        for b, t in enumerate(trees):
            i, chain = 0, [0]
            while i in t[1:]:
                i = t.index(i, 1)
                chain.append(i)
            assert acc[b] == len(chain) - 1
            assert list(path[b, :len(chain)]) == chain


def test_edge_cases_match_oracle():
    """An empty request; a node with children but no draft row (flagged, draws from p); repeated
    and out-of-vocabulary children (flagged, skipped); a star tested with max_children = 2."""
    need_gpu()
    trees = [synth.star_tree(6), synth.full_tree(2, 2), synth.star_tree(9)]
    d = synth.sampled_tree_inputs(trees, 3000, seed=51, dtype=torch.float32, device=DEV, target_noise=3.0)
    cu = d["cu_nodes"].cpu().tolist()
    # insert an empty request after the first
    d["cu_nodes"] = torch.tensor([cu[0], cu[1], cu[1], cu[2], cu[3]], dtype=torch.int32, device=DEV)
    tok = d["tokens"].cpu()
    tok[2] = tok[1]                   # star 0: children 1 and 2 share a token
    tok[4] = 3000 + 5                 # star 0: child 4 outside the vocabulary
    d["tokens"] = tok.to(DEV)
    row = d["draft_row"].cpu()
    row[cu[1] + 1] = -1               # full tree: node 1 has children but no draft row
    d["draft_row"] = row.to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    for maxc in (8, 2):
        compare(d, 0.9, 8, range(6), 2, maxc, status)
    st = int(status.item())
    assert st & 16 and st & 4


def test_every_proposable_token_rejected():
    """A node whose drafter gives probability zero to all but three tokens, with children
    [three positive tokens, then zero-probability ones], and a target concentrated elsewhere:
    once the three are rejected nothing is left to test and the token is drawn from the
    residual.  A second request's first child has draft probability zero: it is kept."""
    need_gpu()
    V = 8
    trees = [[-1, 0, 0, 0, 0, 0], [-1, 0]]
    T = 8
    neg = float("-inf")
    zq = torch.tensor([[0.0, 0.2, 0.4, neg, neg, neg, neg, neg],
                       [0.0, 0.0, neg, 1.0, 1.0, 1.0, 1.0, 1.0]])
    z = torch.full((T, V), -2.0)
    z[0, 5:] = 3.0                                   # target mass on tokens 5..7
    z[6] = torch.linspace(0, 1, V)
    d = {"cu_nodes": torch.tensor([0, 6, 8], dtype=torch.int32),
         "tokens": torch.tensor([0, 0, 1, 2, 3, 4, 0, 2], dtype=torch.int32),
         "parents": torch.tensor([p for t in trees for p in t], dtype=torch.int32),
         "logits": z, "draft_logits": zq,
         "draft_row": torch.tensor([0, -1, -1, -1, -1, -1, 1, -1], dtype=torch.int32)}
    # request 1's only child has token 2, where its drafter's probability is zero
    d = {k: v.to(DEV) for k, v in d.items()}
    draws = set()
    for rnd in range(12):
        got = gpu_run(d, 1.0, 2, rnd, 1, 8)
        ref = oracle_run(d, 1.0, 2, rnd, 1, 8)
        for k, g, r in zip(KEYS, got, ref):
            assert np.array_equal(g, r), (k, rnd, g, r)
        assert got[0][1] == 1 and got[2][1][0] == 2  # the zero-probability child is kept
        draws.add(int(got[3][0]))
    assert draws & {5, 6, 7}


@pytest.mark.parametrize("shape_name,B", [("llama8b", 1), ("llama70b", 4)])
def test_bench_configurations(shape_name, B):
    """The inputs the benchmark times (random 61-node trees of depth 6 at the 8B and 70B
    shapes, V = 128256 bf16, T = 1, at most 10 children tested per node), through the same
    entry point, equal to the oracle's walk over several rounds."""
    need_gpu()
    sh = synth.LLAMA8B if shape_name == "llama8b" else synth.LLAMA70B
    trees = [synth.random_tree(61, sh.depth, 4400 + i) for i in range(B)]
    d = synth.sampled_tree_inputs(trees, sh.V, seed=970, device=DEV, target_noise=1.0)
    compare(d, 1.0, 7, range(3), sh.depth, 10)


def test_vocabulary_beyond_64_chunks():
    """V = 300000 (74 chunks of 4096 per node, more than one wave of partials per node) with a
    ragged last chunk: the per-node combines loop over the chunks."""
    need_gpu()
    trees = [synth.full_tree(2, 2), synth.star_tree(5)]
    d = synth.sampled_tree_inputs(trees, 300000, seed=61, device=DEV, target_noise=2.0)
    compare(d, 1.0, 13, range(3), tree_depth(trees), max_kids(trees))


def test_accept_sampled_chi_square_on_gpu():
    """Losslessness of the sampled-candidate rule on the GPU, 1e6 draws: two-level trees whose
    root has 3 children drawn without replacement from its draft distribution q_root and each
    child 2 of its own (fresh draws per request and call, Gumbel-top-k on the host); target and
    draft logits depend on the token path.  The first output token must follow
    p(. | root) = softmax(z_root / T), and the second, given that the first was the kept child
    a, p(. | root, a) (chi-square p > 0.01 for each of the two tables)."""
    need_gpu()
    from scipy import stats
    from tests.test_oracle_sampled import _path_logits
    V, K1, K2, T, B, calls = 6, 3, 2, 0.8, 100_000, 10
    zt_root, zq_root = _path_logits([], V, 7), _path_logits([], V, 8)
    zt1 = np.stack([_path_logits([x], V, 7) for x in range(V)])          # target at child x
    zq1 = np.stack([_path_logits([x], V, 8) for x in range(V)])          # draft at child x
    zt2 = np.stack([[_path_logits([x, y], V, 7) for y in range(V)] for x in range(V)])
    lq_root = np.log(O.softmax64(zq_root, T))
    lq1 = np.log(np.stack([O.softmax64(zq1[x], T) for x in range(V)]))
    n = 1 + K1 + K1 * K2
    par = [-1] + [0] * K1 + [1 + a for a in range(K1) for _ in range(K2)]
    rng = np.random.default_rng(2026)
    first, pair = np.zeros(V), np.zeros((V, V))
    for call in range(calls):
        g = rng.gumbel(size=(B, V))
        c1 = np.argsort(-(lq_root[None, :] + g), axis=1)[:, :K1]                        # [B, K1]
        g2 = rng.gumbel(size=(B, K1, V))
        c2 = np.argsort(-(lq1[c1] + g2), axis=2)[:, :, :K2]                              # [B, K1, K2]
        tok = np.concatenate([np.zeros((B, 1), np.int64), c1, c2.reshape(B, -1)], axis=1)
        tgt = np.concatenate([np.broadcast_to(zt_root, (B, 1, V)), zt1[c1],
                              zt2[np.repeat(c1, K2, axis=1), c2.reshape(B, -1)]], axis=1)
        drf = np.concatenate([np.broadcast_to(zq_root, (B, 1, V)), zq1[c1]], axis=1)      # [B, 4, V]
        drow = np.full((B, n), -1, np.int64)
        drow[:, :1 + K1] = np.arange(B)[:, None] * (1 + K1) + np.arange(1 + K1)[None, :]
        d = {"cu_nodes": torch.arange(0, (B + 1) * n, n, dtype=torch.int32, device=DEV),
             "tokens": torch.tensor(tok.reshape(-1), dtype=torch.int32, device=DEV),
             "parents": torch.tensor(par * B, dtype=torch.int32, device=DEV),
             "logits": torch.tensor(tgt.reshape(-1, V), dtype=torch.float32, device=DEV),
             "draft_logits": torch.tensor(drf.reshape(-1, V), dtype=torch.float32, device=DEV),
             "draft_row": torch.tensor(drow.reshape(-1), dtype=torch.int32, device=DEV)}
        acc, path, outt, bonus = gpu_run(d, T, 4242, call, 2, K1)
        first += np.bincount(outt[:, 0], minlength=V)
        went = acc >= 1
        np.add.at(pair, (outt[went, 0], outt[went, 1]), 1)
        if call == 0:       # the GPU walk equals the oracle's on the first requests of this call
            m = 3
            o = O.accept_sampled(np.arange(0, (m + 1) * n, n), tok[:m].reshape(-1), np.array(par * m),
                                 tgt[:m].reshape(-1, V), drf[:m].reshape(-1, V), drow[:m].reshape(-1),
                                 T, 4242, call, 2, max_children=K1)
            for got, ref in zip((acc, path, outt, bonus), o):
                assert np.array_equal(got[:m], ref)
    p1 = O.softmax64(zt_root, T)
    assert first.sum() == B * calls
    assert stats.chisquare(first, p1 * first.sum()).pvalue > 0.01
    chi, dof = 0.0, 0
    for a in range(V):
        na = pair[a].sum()
        if na < 1000:
            continue
        e = na * O.softmax64(zt1[a], T)
        keep = e >= 5
        o_, e_ = pair[a][keep], e[keep] / e[keep].sum() * pair[a][keep].sum()
        chi += ((o_ - e_) ** 2 / e_).sum()
        dof += int(keep.sum()) - 1
    assert pair.sum() > 200_000 and dof >= 10
    assert stats.chi2.sf(chi, dof) > 0.01, (chi, dof)
