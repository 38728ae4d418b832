"""Pins for the oracle's commit of the accepted path's KV and its drafter catch-up over
committed positions (the step after acceptance)."""
import json
import os

import numpy as np
import torch
import torch.nn.functional as Fnn

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
SMALL = synth.scaled(synth.TINY, d=32, Hq=4, Hkv=2, Dh=8, F=48, V=50)


def test_commit_golden():
    g = json.load(open(os.path.join(HERE, "golden", "commit_kv.json")))
    T = g["cu_nodes"][-1]
    k_tree = np.array([[10 * r, 10 * r + 1] for r in range(T)], dtype=np.float64)[:, None, :]
    v_tree = -k_tree
    kc = np.full((g["cache_rows"], 1, 2), g["fill"], dtype=np.float64)
    kc2, vc2 = O.commit_kv(g["cu_nodes"], g["path"], g["accept_len"], k_tree, v_tree,
                           g["dst_row"], kc, kc.copy())
    np.testing.assert_array_equal(kc2[:, 0, :], np.array(g["expect_k"], dtype=np.float64))
    np.testing.assert_array_equal(vc2[:, 0, :], np.array(g["expect_v"], dtype=np.float64))


def test_commit_properties():
    """Random trees: committed rows are the path's tree rows in path order, every other cache
    row is unchanged, accept_len 0 commits the root alone, the inputs are not modified."""
    rng = np.random.default_rng(3)
    sizes = [7, 1, 12, 5]
    cu = np.concatenate([[0], np.cumsum(sizes)])
    T = int(cu[-1])
    k_tree = rng.standard_normal((T, 2, 4))
    v_tree = rng.standard_normal((T, 2, 4))
    D = 4
    path = np.full((len(sizes), D + 1), -1)
    acc = np.zeros(len(sizes), dtype=np.int64)
    for b, n in enumerate(sizes):
        a = int(rng.integers(0, min(n, D + 1)))
        acc[b] = a
        path[b, 0] = 0
        path[b, 1:a + 1] = rng.choice(np.arange(1, n), a, replace=False) if a else []
    dst = np.array([0, 9, 20, 40])
    kc = rng.standard_normal((50, 2, 4))
    vc = rng.standard_normal((50, 2, 4))
    k0, v0, kc0 = k_tree.copy(), v_tree.copy(), kc.copy()
    kn, vn = O.commit_kv(cu, path, acc, k_tree, v_tree, dst, kc, vc)
    touched = set()
    for b in range(len(sizes)):
        for i in range(acc[b] + 1):
            r = dst[b] + i
            touched.add(r)
            np.testing.assert_array_equal(kn[r], k_tree[cu[b] + path[b, i]])
            np.testing.assert_array_equal(vn[r], v_tree[cu[b] + path[b, i]])
    for r in range(50):
        if r not in touched:
            np.testing.assert_array_equal(kn[r], kc[r])
            np.testing.assert_array_equal(vn[r], vc[r])
    assert acc[1] == 0 and np.array_equal(kn[9], k_tree[cu[1]])
    np.testing.assert_array_equal(k_tree, k0)
    np.testing.assert_array_equal(kc, kc0)


def _catchup_inputs(n, seed):
    w = synth.drafter_weights(SMALL, seed=seed)
    dr = O.Drafter(w, SMALL.Hq, SMALL.Hkv, SMALL.Dh)
    rng = np.random.default_rng(seed)
    h = [rng.standard_normal((n, SMALL.d)).astype(np.float32) for _ in range(3)]
    tok = rng.integers(0, SMALL.V, n)
    pos = rng.integers(0, 3000, n)
    return w, dr, h, tok, pos


def textbook_kv(w, shape, tok, g, pos, eps=1e-5, theta=500000.0):
    """Key and value of one decoder-layer input written from the layer's definition with
    torch: RMSNorm from torch.nn.functional, RoPE as a complex rotation of the pairs
    (x_i, x_{i+Dh/2}) by pos * theta^(-2i/Dh)."""
    d, Hq, Hkv, Dh = shape.d, shape.Hq, shape.Hkv, shape.Dh
    t64 = lambda x: torch.as_tensor(np.asarray(x, dtype=np.float64))
    e = t64(w["embed"].float().numpy())[torch.as_tensor(tok, dtype=torch.long)]
    u = torch.cat([Fnn.rms_norm(e, (d,), t64(w["g_embed"].float().numpy()), eps),
                   Fnn.rms_norm(t64(g), (d,), t64(w["g_feat"].float().numpy()), eps)], dim=-1)
    wq = t64(w["w_qkv"].float().numpy())
    k = (u @ wq[Hq * Dh:(Hq + Hkv) * Dh].T).reshape(-1, Hkv, Dh)
    v = (u @ wq[(Hq + Hkv) * Dh:].T).reshape(-1, Hkv, Dh)
    half = Dh // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / Dh)
    ang = t64(pos)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    kc = torch.complex(k[..., :half], k[..., half:]) * rot
    k = torch.cat([kc.real, kc.imag], dim=-1)
    return k.numpy(), v.numpy()


def test_catchup_against_textbook_layer():
    w, dr, h, tok, pos = _catchup_inputs(6, 11)
    g, k, v = O.drafter_catchup(dr, tok, *h, pos)
    gref = np.concatenate([x.astype(np.float64) for x in h], axis=1) @ O.f64(w["w_fuse"]).T
    np.testing.assert_allclose(g, gref, rtol=1e-12, atol=1e-12)
    kr, vr = textbook_kv(w, SMALL, tok, gref, pos)
    np.testing.assert_allclose(k, kr, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(v, vr, rtol=1e-10, atol=1e-12)


def test_catchup_row_is_a_draft_root():
    """A catch-up row is the drafter's first-step input: it equals the root slot of a
    one-step draft round with the row's token, features and prefix length = position."""
    w, dr, h, tok, pos = _catchup_inputs(4, 12)
    pos = np.array([0, 3, 17, 5])
    g, k, v = O.drafter_catchup(dr, tok, *h, pos)
    rng = np.random.default_rng(1)
    for r in range(4):
        P = int(pos[r])
        kpre = rng.standard_normal((P, SMALL.Hkv, SMALL.Dh))
        res = O.draft_round(dr, 1, 2, 1, 2, h[0][r:r + 1], h[1][r:r + 1], h[2][r:r + 1],
                            [int(tok[r])], kpre, kpre, [P])[0]
        np.testing.assert_allclose(res["g"], g[r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["store"][0]["k"], k[r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["store"][0]["v"], v[r], rtol=1e-12, atol=1e-12)


def test_catchup_rows_independent_and_positions():
    """Rows do not interact (a permutation of rows permutes the outputs), the value does not
    depend on the position, and moving a row by delta positions rotates each key pair by
    delta * theta^(-2i/Dh) (relative-position property of RoPE)."""
    w, dr, h, tok, pos = _catchup_inputs(5, 13)
    g, k, v = O.drafter_catchup(dr, tok, *h, pos)
    perm = np.array([3, 0, 4, 2, 1])
    g2, k2, v2 = O.drafter_catchup(dr, tok[perm], *[x[perm] for x in h], pos[perm])
    np.testing.assert_allclose(k2, k[perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g2, g[perm], rtol=1e-12, atol=1e-12)
    delta = 37
    _, k3, v3 = O.drafter_catchup(dr, tok, *h, pos + delta)
    np.testing.assert_allclose(v3, v, rtol=1e-12, atol=1e-12)
    half = SMALL.Dh // 2
    ang = delta * 500000.0 ** (-2.0 * np.arange(half) / SMALL.Dh)
    c, s = np.cos(ang), np.sin(ang)
    rot = np.concatenate([k[..., :half] * c - k[..., half:] * s, k[..., :half] * s + k[..., half:] * c], -1)
    np.testing.assert_allclose(k3, rot, rtol=1e-9, atol=1e-10)
