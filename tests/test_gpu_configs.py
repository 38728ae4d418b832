"""GPU parity at the full sizes of the batched, 70B-shaped and long-context workloads, through
the C-ABI.  The oracle recomputes sampled requests (attention) or every node (masks,
acceptance); the bars are those of the other parity tests: index outputs bit-exact, floats
within 2e-2 relative in bf16."""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import capi, synth
from tests.gpu_util import TOL, lse_err, need_gpu, np32, rel_err, u64

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def verify_case(shape, trees, prefix, seed):
    vi = synth.verify_inputs(shape, trees, prefix, seed=seed, device=DEV, with_logits=False)
    maxn = max(len(t) for t in trees)
    mk = capi.eagle3_build_tree_mask(vi["cu_nodes"], vi["parents"], vi["cu_prefix"], max_nodes=maxn)
    return vi, mk, maxn


def check_mask(vi, mk, trees, prefix):
    cu = [0]
    for t in trees:
        cu.append(cu[-1] + len(t))
    cup = [0]
    for p in prefix:
        cup.append(cup[-1] + p)
    om, od, op, ok = O.build_tree_mask([p for t in trees for p in t], cu, cup)
    assert ok
    assert np.array_equal(u64(mk["mask"]), om)
    assert np.array_equal(mk["depth"].cpu().numpy(), od)
    assert np.array_equal(mk["pos"].cpu().numpy(), op)


def check_attention_requests(vi, mk, out, requests, scale):
    """Oracle attention of the sampled requests alone (their slices of every input)."""
    cu = vi["cu_nodes"].tolist()
    cup = vi["cu_prefix"].tolist()
    mask = u64(mk["mask"])
    for b in requests:
        n0, n1, p0, p1 = cu[b], cu[b + 1], cup[b], cup[b + 1]
        o_ref, l_ref = O.tree_attention(vi["q"][n0:n1].cpu(), vi["k_tree"][n0:n1].cpu(),
                                        vi["v_tree"][n0:n1].cpu(), [0, n1 - n0], mask[n0:n1],
                                        vi["kpre"][p0:p1].cpu(), vi["vpre"][p0:p1].cpu(),
                                        [0, p1 - p0], scale)
        assert rel_err(np32(out["o"][n0:n1]), o_ref) <= TOL[BF], b
        assert lse_err(np32(out["lse"][n0:n1]), l_ref) <= TOL[BF], b


def run_attention(vi, mk, maxn, prefix, scale, partials=False):
    out = capi.eagle3_tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], vi["cu_nodes"], maxn,
                                     mk["mask"], vi["kpre"], vi["vpre"], vi["cu_prefix"], max(prefix),
                                     scale, partials=partials, merged=True)
    torch.cuda.synchronize()
    return out


def check_accept(vi, mk, trees, logits, temperature, seed, rnd, max_depth):
    par = [p for t in trees for p in t]
    out = capi.eagle3_accept(vi["cu_nodes"], vi["tokens"], vi["parents"], mk["mask"], logits,
                             temperature, seed=seed, round=rnd, max_depth=max_depth)
    acc, path, outt, bonus = O.accept(vi["cu_nodes"].tolist(), vi["tokens"].tolist(), par,
                                      logits.cpu(), temperature, seed, rnd, max_depth)
    assert np.array_equal(out["accept_len"].cpu().numpy(), acc)
    assert np.array_equal(out["path"].cpu().numpy(), path)
    assert np.array_equal(out["out_tokens"].cpu().numpy(), outt)
    assert np.array_equal(out["bonus"].cpu().numpy(), bonus)
    return acc


def planted_logits(shape, vi, trees, seed):
    """N(0, 1) target logits with one planted root-to-node path per request (so that the
    accepted length is not trivially 0)."""
    logits = synth.normal((vi["T"], shape.V), 1.0, seed, BF, "cpu")
    tok = vi["tokens"].cpu()
    n0 = 0
    for t in trees:
        depth = O.build_tree_mask(t, [0, len(t)], [0, 0])[1]
        end = int(np.argmax(depth))          # the first deepest node
        synth.plant_path(logits, tok, t, n0, end)
        n0 += len(t)
    return logits.to(DEV)


def test_batch16_ragged_verify_full_size():
    """16 requests, prefixes uniform in [512, 4096], random trees of <= 48 nodes (depth <= 6):
    masks of every request bit-exact, attention of 4 sampled requests, greedy acceptance of
    every request bit-exact."""
    need_gpu()
    shape = synth.BATCH16
    prefix = synth.prefix_lengths(shape, seed=31)
    rng = np.random.default_rng(31)
    trees = [synth.random_tree(int(rng.integers(1, shape.verify_max_nodes + 1)), shape.verify_max_depth,
                               3100 + i) for i in range(shape.B)]
    vi, mk, maxn = verify_case(shape, trees, prefix, seed=32)
    check_mask(vi, mk, trees, prefix)
    scale = float(np.float32(shape.Dh ** -0.5))
    out = run_attention(vi, mk, maxn, prefix, scale)
    check_attention_requests(vi, mk, out, [0, 5, 10, 15], scale)
    logits = planted_logits(shape, vi, trees, seed=33)
    acc = check_accept(vi, mk, trees, logits, 0.0, 0, 0, shape.verify_max_depth)
    assert acc.max() >= 1


def test_llama70b_verify_full_size():
    """4 requests x 60-node trees over 8192-token prefixes at the 64 q / 8 kv head shape:
    masks bit-exact, attention of requests 0 and 3, stochastic acceptance at T = 0.7 with a
    fixed seed bit-exact over the full 128256-token vocabulary."""
    need_gpu()
    shape = synth.LLAMA70B
    prefix = synth.prefix_lengths(shape, seed=41)
    trees = [synth.random_tree(60, shape.depth, 4100 + i) for i in range(shape.B)]
    vi, mk, maxn = verify_case(shape, trees, prefix, seed=42)
    check_mask(vi, mk, trees, prefix)
    scale = float(np.float32(shape.Dh ** -0.5))
    out = run_attention(vi, mk, maxn, prefix, scale)
    check_attention_requests(vi, mk, out, [0, 3], scale)
    logits = planted_logits(shape, vi, trees, seed=43)
    for rnd in (0, 1):
        check_accept(vi, mk, trees, logits, shape.temperature, 0x70B0070B, rnd, shape.depth)


def test_longctx_branch_merge_full_size():
    """A 7-step branch after a 65536-token prefix: the fused output equals one softmax over
    [prefix; branch ancestors] for every row, and folding the branch partial into the merged
    main partial (a second LSE merge) gives the same result."""
    need_gpu()
    shape = synth.LONGCTX
    prefix = [65536]
    trees = [synth.chain_tree(shape.branch)]
    vi, mk, maxn = verify_case(shape, trees, prefix, seed=52)
    scale = float(np.float32(shape.Dh ** -0.5))
    out = run_attention(vi, mk, maxn, prefix, scale, partials=True)
    check_attention_requests(vi, mk, out, [0], scale)
    S = out["splits"]
    rows = vi["T"] * shape.Hq
    main = capi.eagle3_lse_merge(out["o_part"][:S].reshape(S, rows, shape.Dh),
                                 out["lse_part"][:S].reshape(S, rows))
    o2 = torch.stack([main["o"], out["o_part"][S].reshape(rows, shape.Dh)])
    l2 = torch.stack([main["lse"], out["lse_part"][S].reshape(rows)])
    fused = capi.eagle3_lse_merge(o2, l2, out_dtype=BF)
    torch.cuda.synchronize()
    # the fused bf16 output equals the one-call merged output up to rounding of the extra stage
    assert rel_err(np32(fused["o"]), np32(out["o"].reshape(rows, shape.Dh))) <= TOL[BF]
    assert lse_err(np32(fused["lse"]), np32(out["lse"].reshape(rows))) <= 1e-5
