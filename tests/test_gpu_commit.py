"""GPU parity of the step after acceptance, through the C-ABI: eagle3_commit_kv against the
oracle's commit (bit-exact: a copy), and eagle3_drafter_catchup against the oracle's
catch-up (fused features, keys with RoPE and values; within 1e-4 (fp32) or 2e-2 (bf16)
relative), from a few rows to a 2048-token prompt (sampled rows), plus the device-side
checks (flags raised, offending rows skipped)."""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import capi, synth
from tests.gpu_util import TOL, need_gpu, np32, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _commit_case(dt, seed):
    rng = np.random.default_rng(seed)
    sizes = [61, 1, 17, 40]
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T, Hkv, Dh, D = int(cu[-1]), 8, 128, 6
    path = np.full((len(sizes), D + 1), -1, dtype=np.int32)
    acc = np.zeros(len(sizes), dtype=np.int32)
    for b, n in enumerate(sizes):
        a = int(rng.integers(0, min(n, D + 1)))
        acc[b] = a
        path[b, 0] = 0
        if a:
            path[b, 1:a + 1] = np.sort(rng.choice(np.arange(1, n), a, replace=False))
    dst = np.array([0, 100, 7, 300], dtype=np.int32)
    rows = 320
    k_tree = synth.normal((T, Hkv, Dh), 1.0, seed, dt, DEV)
    v_tree = synth.normal((T, Hkv, Dh), 1.0, seed + 1, dt, DEV)
    k_cache = synth.normal((rows, Hkv, Dh), 1.0, seed + 2, dt, DEV)
    v_cache = synth.normal((rows, Hkv, Dh), 1.0, seed + 3, dt, DEV)
    t = lambda x: torch.as_tensor(x, device=DEV)
    return cu, path, acc, dst, k_tree, v_tree, k_cache, v_cache, t


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_commit_matches_oracle(dt):
    need_gpu()
    cu, path, acc, dst, k_tree, v_tree, k_cache, v_cache, t = _commit_case(dt, 5)
    kref, vref = O.commit_kv(cu, path, acc, np32(k_tree), np32(v_tree), dst, np32(k_cache), np32(v_cache))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    capi.eagle3_commit_kv(t(cu), t(path), t(acc), k_tree, v_tree, t(dst), k_cache, v_cache, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(np32(k_cache), kref)
    assert np.array_equal(np32(v_cache), vref)


def test_commit_flags_bad_entries():
    """A path node outside its request and a destination outside the cache are flagged and
    skipped; the other rows are still committed."""
    need_gpu()
    dt = torch.bfloat16
    cu, path, acc, dst, k_tree, v_tree, k_cache, v_cache, t = _commit_case(dt, 9)
    acc[0] = max(acc[0], 1)
    path[0, 1] = 500                         # node outside request 0 (61 nodes)
    acc[2] = 2
    path[2, 1], path[2, 2] = 1, 2
    dst[2] = 319                             # rows 319, 320, 321: the last two are outside
    k0 = np32(k_cache).copy()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    capi.eagle3_commit_kv(t(cu), t(path), t(acc), k_tree, v_tree, t(dst), k_cache, v_cache, dev_status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st & 8 and st & 16
    got = np32(k_cache)
    np.testing.assert_array_equal(got[0], np32(k_tree)[0])           # request 0 root committed
    for i in range(2, acc[0] + 1):                                    # its valid later rows too
        np.testing.assert_array_equal(got[i], np32(k_tree)[cu[0] + path[0, i]])
    np.testing.assert_array_equal(got[1], k0[1])                      # the bad node's row untouched
    np.testing.assert_array_equal(got[319], np32(k_tree)[cu[2]])     # in range: committed
    for b in (1, 3):
        for i in range(acc[b] + 1):
            np.testing.assert_array_equal(got[dst[b] + i], np32(k_tree)[cu[b] + path[b, i]])


def _oracle_drafter(w, shape, tokens):
    """Oracle drafter restricted to what the catch-up reads: the embedding rows of `tokens`
    (ids remapped), W_f, W_qkv and the two input norms (the later layers are not used)."""
    uniq, inv = np.unique(np.asarray(tokens), return_inverse=True)
    cpu = lambda x: x.float().cpu()
    small = torch.zeros((1, 1))
    wd = {"embed": cpu(w["embed"][torch.as_tensor(uniq, device=w["embed"].device)]),
          "w_fuse": cpu(w["w_fuse"]), "w_qkv": cpu(w["w_qkv"]), "g_embed": cpu(w["g_embed"]),
          "g_feat": cpu(w["g_feat"]), "g_mlp": cpu(w["g_mlp"]), "g_final": cpu(w["g_final"]),
          "w_o": small, "w_gate_up": small, "w_down": small, "w_lm": small}
    return O.Drafter(wd, shape.Hq, shape.Hkv, shape.Dh), inv


def _catchup_run(shape, n, seed, rows_checked=None):
    w = synth.drafter_weights(shape, seed=seed, device=DEV)
    dt = w["embed"].dtype
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    h = [synth.normal((n, shape.d), 1.0, seed + 10 + i, dt, DEV) for i in range(3)]
    tok = synth.uniform_int(n, shape.V, seed + 20, DEV).to(torch.int32)
    pos = (torch.arange(n, device=DEV, dtype=torch.int32) * 7 + 3) % 65536
    cache_rows = n + 16
    # destinations out of row order
    dst = torch.as_tensor(np.random.default_rng(seed).permutation(cache_rows)[:n].astype(np.int32), device=DEV)
    kc = torch.full((cache_rows, shape.Hkv, shape.Dh), 7.0, dtype=dt, device=DEV)
    vc = torch.full((cache_rows, shape.Hkv, shape.Dh), 7.0, dtype=dt, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = capi.eagle3_drafter_catchup(dr, tok, pos, *h, dst, kc, vc, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    sel = np.arange(n) if rows_checked is None else np.sort(
        np.random.default_rng(seed).choice(n, rows_checked, replace=False))
    tsel = tok.cpu().numpy()[sel]
    odr, inv = _oracle_drafter(w, shape, tsel)
    hs = [np32(x)[sel] for x in h]
    gref, kref, vref = O.drafter_catchup(odr, inv, *hs, pos.cpu().numpy()[sel])
    d_sel = dst.cpu().numpy()[sel]
    tol = TOL[dt]
    assert rel_err(np32(g)[sel], gref) <= tol
    assert rel_err(np32(kc)[d_sel], kref) <= tol
    assert rel_err(np32(vc)[d_sel], vref) <= tol
    untouched = np.setdiff1d(np.arange(cache_rows), dst.cpu().numpy())
    assert np.all(np32(kc)[untouched] == 7.0) and np.all(np32(vc)[untouched] == 7.0)
    return w, dr


@pytest.mark.parametrize("shape,n,rows", [
    (synth.TINY, 7, None),             # fp32, a round's accepted path (register kernel)
    (synth.TINY, 160, 24),             # fp32, the largest fp32 catch-up
    (synth.LLAMA8B, 7, None),          # bf16 8B shapes, a round's accepted path (LDS ring)
    (synth.LLAMA8B, 100, 16),          # bf16, register-stationary kernel
    (synth.LLAMA8B, 2048, 24),         # bf16, a 2048-token prompt: matrix-core tiles
], ids=["tiny_7", "tiny_160", "8b_7", "8b_100", "8b_prompt_2048"])
def test_catchup_matches_oracle(shape, n, rows):
    need_gpu()
    _catchup_run(shape, n, 31, rows)


def test_catchup_feature_is_the_draft_roots():
    """One catch-up row with a request's root token and features computes the same fused
    feature as the draft round's root, bit for bit (same GEMM plan, same summation)."""
    need_gpu()
    shape = synth.TINY
    w = synth.drafter_weights(shape, seed=3, device=DEV)
    di = synth.draft_inputs(shape, seed=4, device=DEV, prefix=[40])
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    tree = capi.Eagle3TreeCfg(depth=shape.depth, topk=shape.topk, width=shape.width, n_nodes=shape.n_nodes)
    out = capi.eagle3_draft_expand(dr, tree, di["h_low"], di["h_mid"], di["h_high"], di["root_tok"],
                                   di["kpre"], di["vpre"], di["cu_prefix"], 40, debug=True)
    kc = torch.zeros((4, shape.Hkv, shape.Dh), dtype=torch.float32, device=DEV)
    g = capi.eagle3_drafter_catchup(dr, di["root_tok"].to(torch.int32), torch.tensor([40], dtype=torch.int32, device=DEV),
                                    di["h_low"], di["h_mid"], di["h_high"],
                                    torch.tensor([2], dtype=torch.int32, device=DEV), kc, kc.clone())
    torch.cuda.synchronize()
    assert torch.equal(g, out["debug"]["g"])


def test_catchup_flags_bad_token_and_row():
    need_gpu()
    shape = synth.TINY
    w = synth.drafter_weights(shape, seed=3, device=DEV)
    dr = capi.make_drafter(w, shape.Hq, shape.Hkv, shape.Dh)
    h = [synth.normal((3, shape.d), 1.0, 50 + i, torch.float32, DEV) for i in range(3)]
    tok = torch.tensor([5, shape.V + 3, 9], dtype=torch.int32, device=DEV)
    pos = torch.tensor([1, 2, 3], dtype=torch.int32, device=DEV)
    dst = torch.tensor([0, 1, 99], dtype=torch.int32, device=DEV)
    kc = torch.full((4, shape.Hkv, shape.Dh), 7.0, device=DEV)
    vc = kc.clone()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    capi.eagle3_drafter_catchup(dr, tok, pos, *h, dst, kc, vc, dev_status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st & 4 and st & 16
    assert torch.all(kc[2:] == 7.0) and torch.all(vc[2:] == 7.0)   # row 99 skipped
    assert not torch.all(kc[1] == 7.0)                               # clamped token still written
