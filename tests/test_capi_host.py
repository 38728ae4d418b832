"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every symbol
that include/eagle3.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from speculative_decoding_round_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "eagle3.h")).read()
    return sorted(set(re.findall(r"EAGLE3_API\s+[\w\s\*]+?\b(eagle3_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(capi.LIB_PATH):
        pytest.skip("libeagle3.so not built")
    return capi.lib()


def test_header_declares_the_five_entry_points():
    fns = header_functions()
    for f in ("eagle3_draft_expand", "eagle3_build_tree_mask", "eagle3_tree_attention",
              "eagle3_lse_merge", "eagle3_accept"):
        assert f in fns


def test_every_declared_symbol_is_exported(lib):
    for f in header_functions():
        assert hasattr(lib, f), f
        assert f in capi.EXPORTS, f"binding lacks {f}"


def test_internal_symbols_hidden():
    out = os.popen(f"nm -D --defined-only {capi.LIB_PATH}").read()
    text = [ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"]
    assert text and all(n.startswith("eagle3_") or n in ("_init", "_fini") for n in text), text


def test_abi_and_status_strings(lib):
    assert capi.abi_version() == 1
    for code in (0, -1, -2, -3, -4):
        assert lib.eagle3_status_string(code)
    assert b"unknown" in lib.eagle3_status_string(7)


def test_host_validation_rejects_before_launch(lib):
    L = lib
    # tree mask: no requests / null pointers / too many nodes for the mask
    assert L.eagle3_build_tree_mask(0, 1, None, None, None, 1, None, 1, None, None, None, None) == -1
    assert L.eagle3_build_tree_mask(1, 3, None, None, None, 3, None, 1, None, None, None, None) == -1
    assert L.eagle3_build_tree_mask(1, 3, 8, 8, None, 65, 8, 1, None, None, None, None) == -1
    assert L.eagle3_build_tree_mask(1, 3, 8, 8, None, 3, 8, 5, None, None, None, None) == -2
    # attention: bad head dim, bad dtype, GQA mismatch, non-positive scale
    args = [1, 4, 8, 2, 96, 1, 8, 8, 8, 8, 4, 8, 1, None, None, None, 0, 0.1, 0,
            8, 8, None, None, None, 0, None]
    assert L.eagle3_tree_attention(*args) == -2
    args[4] = 128
    args[5] = 7
    assert L.eagle3_tree_attention(*args) == -1
    args[5] = 1
    args[3] = 3
    assert L.eagle3_tree_attention(*args) == -1
    args[3] = 2
    args[17] = 0.0
    assert L.eagle3_tree_attention(*args) == -1
    args[17] = 0.1
    args[19] = None    # neither partial outputs nor merged output
    assert L.eagle3_tree_attention(*args) == -1
    # merge
    assert L.eagle3_lse_merge(0, 4, 8, 8, 8, 0, 8, None, None) == -1
    assert L.eagle3_lse_merge(2, 4, 6, 8, 8, 0, 8, None, None) == -1
    assert L.eagle3_lse_merge(2, 4, 8, 16, 16, 0, 24, None, None) == -1   # output not 16-byte aligned
    # accept: workspace too small, negative temperature
    assert L.eagle3_accept(1, 3, 8, 8, 8, 8, 1, 8, 100, 1, 0.0, 0, 0, 2, 8, 8, 8, 8, None, 0, None) == -3
    assert L.eagle3_accept(1, 3, 8, 8, 8, 8, 1, 8, 100, 1, -1.0, 0, 0, 2, 8, 8, 8, 8, 8, 1 << 20, None) == -1
    assert L.eagle3_accept_workspace_size(3, 100) > 0


def test_draft_validation_and_workspace(lib):
    from speculative_decoding_round_amd.capi import Eagle3Drafter, Eagle3TreeCfg
    w = Eagle3Drafter(d=4096, n_heads_q=32, n_heads_kv=8, head_dim=128, ffn=14336, vocab=128256,
                      dtype=1, eps=1e-5, rope_theta=5e5)
    for k in capi.WEIGHT_KEYS:
        setattr(w, k, 256)
    t = Eagle3TreeCfg(depth=6, topk=10, width=10, n_nodes=60)
    ws = lib.eagle3_draft_expand_workspace_size(ctypes.byref(w), ctypes.byref(t), 1, 2048)
    assert 0 < ws < 512 << 20
    t8 = Eagle3TreeCfg(depth=8, topk=10, width=10, n_nodes=60)       # 71 slots: two mask words
    assert lib.eagle3_draft_expand_workspace_size(ctypes.byref(w), ctypes.byref(t8), 1, 2048) > ws
    t_bad = Eagle3TreeCfg(depth=18, topk=1, width=16, n_nodes=60)    # 273 slots > 256
    assert lib.eagle3_draft_expand_workspace_size(ctypes.byref(w), ctypes.byref(t_bad), 1, 2048) == 0
    st = lib.eagle3_draft_expand(ctypes.byref(w), ctypes.byref(t_bad), 1, 256, 256, 256, 256, 256, 256,
                                 256, 2048, 256, 256, 256, 256, 256, None, 256, 1 << 30, None)
    assert st == -2
    st = lib.eagle3_draft_expand(ctypes.byref(w), ctypes.byref(t), 1, 256, 256, 256, 256, 256, 256,
                                 256, 2048, 256, 256, 256, 256, 256, None, 256, 16, None)
    assert st == -3
    st = lib.eagle3_draft_expand(ctypes.byref(w), ctypes.byref(t), 1, 264, 256, 256, 256, 256, 256,
                                 256, 2048, 256, 256, 256, 256, 256, None, 256, 1 << 30, None)
    assert st == -1   # misaligned h_low
    w.head_dim = 80
    assert lib.eagle3_draft_expand_workspace_size(ctypes.byref(w), ctypes.byref(t), 1, 2048) == 0


def test_draft_workspace_is_a_function_of_the_shapes(lib):
    """The workspace size (and so every launch plan behind it) depends on the shapes alone:
    the same shapes give the same size whatever was computed before and whatever the
    weight addresses are.  Covers the fp32 path, bf16 with few rows (LDS-ring GEMMs) and bf16
    with 160 rows (register-stationary GEMMs)."""
    from speculative_decoding_round_amd.capi import Eagle3Drafter, Eagle3TreeCfg

    def size(d, hq, hkv, dh, f, v, dt, b, tree, prefix, base):
        w = Eagle3Drafter(d=d, n_heads_q=hq, n_heads_kv=hkv, head_dim=dh, ffn=f, vocab=v, dtype=dt,
                          eps=1e-5, rope_theta=5e5)
        for i, k in enumerate(capi.WEIGHT_KEYS):
            setattr(w, k, base + 4096 * i)
        t = Eagle3TreeCfg(*tree)
        return lib.eagle3_draft_expand_workspace_size(ctypes.byref(w), ctypes.byref(t), b, prefix)

    shapes = [(256, 4, 4, 64, 1024, 1024, 0, 1, (3, 2, 4, 14), 128),
              (4096, 32, 8, 128, 14336, 128256, 1, 1, (6, 10, 10, 60), 2048),
              (4096, 32, 8, 128, 14336, 128256, 1, 16, (6, 10, 10, 48), 4096),
              (512, 8, 8, 64, 1536, 8192, 0, 2, (4, 5, 6, 20), 513)]
    first = [size(*s, base=1 << 20) for s in shapes]
    assert all(x > 0 for x in first)
    for rep in range(3):
        again = [size(*s, base=(1 << 40) + rep * (1 << 24)) for s in reversed(shapes)][::-1]
        assert again == first


def test_linear_validation(lib):
    """Host-side checks of eagle3_linear, before anything is launched."""
    P = 1 << 12
    assert lib.eagle3_linear(0, 8, 8, 1, P, 8, P, P, None, 0, None) == -1          # M = 0
    assert lib.eagle3_linear(4, 8, 8, 1, P, 4, P, P, None, 0, None) == -1          # ldx < K
    assert lib.eagle3_linear(4, 6, 8, 1, P, 8, P, P, None, 0, None) == -2          # N % 4
    assert lib.eagle3_linear(200, 8, 8, 1, P, 8, P, P, None, 0, None) == -2        # tiled needs K % 64
    assert lib.eagle3_linear(256, 8, 40, 1, P, 40, P, P, None, 0, None) == -2      # tiled needs K % 64
    assert lib.eagle3_linear(256, 8, 64, 0, P, 64, P, P, None, 0, None) == -2      # tiled is bf16 only
    assert lib.eagle3_linear(4, 8, 8, 1, P + 8, 8, P, P, None, 0, None) == -1      # misaligned X
    need = lib.eagle3_linear_workspace_size(10, 4096, 4096, 1)
    assert need > 0 and lib.eagle3_linear_workspace_size(2048, 6144, 8192, 1) == 0
    # tiles: 192 output tiles of 256 x 256 keep the k-range whole; 96 tiles (fewer than half
    # the compute units) split it in two, one fp32 partial [M, N] per split
    assert lib.eagle3_linear_workspace_size(1024, 6144, 8192, 1) == 2 * 1024 * 6144 * 4
    assert lib.eagle3_linear(10, 4096, 4096, 1, P, 4096, P, P, None, 0, None) == -3  # no workspace


def test_commit_and_catchup_validation(lib):
    """Host-side checks of eagle3_commit_kv and eagle3_drafter_catchup."""
    P = 1 << 12
    # commit: B, Hkv, Dh, dtype, path_stride, cu_nodes, path, accept_len, k_tree, v_tree,
    # dst_row, cache_rows, k_cache, v_cache, dev_status, stream
    args = [2, 8, 128, 1, 7, P, P, P, P, P, P, 100, P, P, None, None]
    bad = list(args); bad[0] = 0
    assert lib.eagle3_commit_kv(*bad) == -1                       # no request
    bad = list(args); bad[3] = 5
    assert lib.eagle3_commit_kv(*bad) == -1                       # dtype
    bad = list(args); bad[1] = 1; bad[2] = 3
    assert lib.eagle3_commit_kv(*bad) == -1                       # row of 6 bytes: not 16-aligned
    bad = list(args); bad[12] = P + 4
    assert lib.eagle3_commit_kv(*bad) == -1                       # misaligned cache
    bad = list(args); bad[6] = None
    assert lib.eagle3_commit_kv(*bad) == -1                       # null path
    assert lib.eagle3_drafter_catchup_workspace_size(None, 4) == 0
    assert lib.eagle3_drafter_catchup(None, 4, P, P, P, P, P, P, 10, P, P, None, None, P, 1 << 20,
                                      None) == -1


def test_accept_sampled_validation(lib):
    """Host-side checks of eagle3_accept_sampled, before anything is launched."""
    P = 1 << 12
    # B, T, cu, tokens, parents, logits, V, dtype, draft_logits, draft_dtype, R, draft_row,
    # max_children, temperature, seed, round, max_depth, accept_len, path, out_tokens, bonus,
    # dev_status, workspace, workspace_bytes, stream
    ws = lib.eagle3_accept_sampled_workspace_size(60, 128256, 10)
    assert ws > 0
    assert lib.eagle3_accept_sampled_workspace_size(60, 128256, 65) == 0     # max_children > 64
    assert lib.eagle3_accept_sampled_workspace_size(60, 128256, 16) > ws
    args = [1, 60, P, P, P, P, 128256, 1, P, 1, 30, P, 10, 0.8, 1, 2, 6, P, P, P, P, None, P, ws, None]

    def call(**kw):
        a = list(args)
        names = {"B": 0, "T": 1, "dtype": 7, "R": 10, "draft": 8, "maxc": 12, "temp": 13, "depth": 16,
                 "ws": 22, "wsb": 23}
        for k, v in kw.items():
            a[names[k]] = v
        return lib.eagle3_accept_sampled(*a)

    assert call(B=0) == -1
    assert call(dtype=3) == -1
    assert call(temp=0.0) == -1                  # sampled acceptance needs T > 0
    assert call(temp=float("inf")) == -1
    assert call(depth=-1) == -1
    assert call(R=-1) == -1
    assert call(draft=None) == -1                # rows declared but no pointer
    assert call(maxc=0) == -2
    assert call(maxc=65) == -2
    assert call(ws=None) == -3
    assert call(wsb=ws - 1) == -3


def test_draft_sampled_validation(lib):
    """Host-side checks of eagle3_draft_expand_sampled: temperature, the required outputs."""
    from speculative_decoding_round_amd.capi import Eagle3Drafter, Eagle3TreeCfg
    w = Eagle3Drafter(d=4096, n_heads_q=32, n_heads_kv=8, head_dim=128, ffn=14336, vocab=128256,
                      dtype=1, eps=1e-5, rope_theta=5e5)
    for k in capi.WEIGHT_KEYS:
        setattr(w, k, 256)
    t = Eagle3TreeCfg(depth=6, topk=10, width=10, n_nodes=60)
    P = 256

    def call(temp=0.8, logits=P, rows=P, ws_bytes=1 << 30):
        return lib.eagle3_draft_expand_sampled(ctypes.byref(w), ctypes.byref(t), 1, temp, 1, 2, P, P, P, P, P,
                                               P, P, 2048, P, P, P, P, P, logits, rows, None, P, ws_bytes, None)
    assert call(temp=0.0) == -1
    assert call(temp=float("inf")) == -1
    assert call(logits=None) == -1
    assert call(logits=P + 4) == -1            # slot logits must be 16-byte aligned
    assert call(rows=None) == -1
    assert call(ws_bytes=16) == -3


def test_binding_refuses_mismatched_caches():
    """The commit and catch-up kernels bound their writes by k_cache's row count: the binding
    refuses caches whose row shape differs from what is written, or whose V cache has a
    different shape from the K cache (either would be an out-of-bounds device write)."""
    import torch
    k = torch.empty((10, 8, 128))
    capi._cache_pair(k, torch.empty((10, 8, 128)), (8, 128))
    with pytest.raises(ValueError):
        capi._cache_pair(k, torch.empty((9, 8, 128)), (8, 128))     # shorter V cache
    with pytest.raises(ValueError):
        capi._cache_pair(k, torch.empty((10, 8, 64)), (8, 128))     # V row of another shape
    with pytest.raises(ValueError):
        capi._cache_pair(torch.empty((10, 4, 128)), torch.empty((10, 4, 128)), (8, 128))
    with pytest.raises(ValueError):
        capi._cache_pair(torch.empty((10, 1024)), torch.empty((10, 1024)), (8, 128))
    with pytest.raises(ValueError):
        capi._cache_pair(torch.empty((10, 8, 256))[:, :, :128], torch.empty((10, 8, 128)), (8, 128))


def test_binding_refuses_mismatched_shapes():
    """The library sees raw pointers: every binding checks, on the host and before any device
    check, that the tensors it passes have the shapes its size arguments imply (a smaller
    tensor would be read or written out of bounds on the device).  CPU tensors suffice: the
    shape check comes first."""
    import torch
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="w has shape"):
        capi.eagle3_linear(torch.empty((4, 64), dtype=bf), torch.empty((8, 32), dtype=bf))
    with pytest.raises(ValueError, match="out has shape"):
        capi.eagle3_linear(torch.empty((4, 64), dtype=bf), torch.empty((8, 64), dtype=bf),
                           out=torch.empty((4, 7)))
    T, Hq, Hkv, Dh = 6, 8, 2, 64
    q = torch.empty((T, Hq, Dh), dtype=bf)
    kt = torch.empty((T, Hkv, Dh), dtype=bf)
    cu = torch.tensor([0, T], dtype=torch.int32)
    mask = torch.empty((T, 1), dtype=torch.uint64)
    kp = torch.empty((40, Hkv, Dh), dtype=bf)
    with pytest.raises(ValueError, match="k_tree has 5 rows"):
        capi.eagle3_tree_attention(q, kt[:5], kt[:5], cu, T, mask, kp, kp, cu, 40, 0.125)
    with pytest.raises(ValueError, match="differs"):
        capi.eagle3_tree_attention(q, kt, kt[:, :, :32], cu, T, mask, kp, kp, cu, 40, 0.125)
    with pytest.raises(ValueError, match="mask"):
        capi.eagle3_tree_attention(q, kt, kt, cu, T, mask[:4], kp, kp, cu, 40, 0.125)
    with pytest.raises(ValueError, match="kpre has shape"):
        capi.eagle3_tree_attention(q, kt, kt, cu, T, mask, kp[:, :1], kp[:, :1], cu, 40, 0.125)
    with pytest.raises(ValueError, match="multiple"):
        capi.eagle3_tree_attention(q, torch.empty((T, 3, Dh), dtype=bf), torch.empty((T, 3, Dh), dtype=bf),
                                   cu, T, mask, kp, kp, cu, 40, 0.125)
    with pytest.raises(ValueError, match="lse_part has shape"):
        capi.eagle3_lse_merge(torch.empty((3, 10, 64)), torch.empty((3, 9)))
    logits = torch.empty((T, 100), dtype=bf)
    tok = torch.empty((T,), dtype=torch.int32)
    with pytest.raises(ValueError, match="one entry per logits row"):
        capi.eagle3_accept(cu, tok[:5], tok, mask, logits, 1.0, 0, 0, 3)
    with pytest.raises(ValueError, match="path has shape"):
        capi.eagle3_accept(cu, tok, tok, mask, logits, 1.0, 0, 0, 3,
                           out={"path": torch.empty((1, 3), dtype=torch.int32)})
    with pytest.raises(ValueError, match="draft_row"):
        capi.eagle3_accept_sampled(cu, tok, tok, logits, logits, tok[:2], 1.0, 0, 0, 3, 4)
    with pytest.raises(ValueError, match="dst_row has shape"):
        capi.eagle3_commit_kv(cu, torch.empty((1, 4), dtype=torch.int32), torch.empty((1,), dtype=torch.int32),
                              kt, kt, torch.empty((2,), dtype=torch.int32), kp, kp)
    L = 32
    with pytest.raises(ValueError, match="v has shape"):
        capi.eagle3_causal_attention(torch.empty((L, Hq, Dh), dtype=bf), torch.empty((L, Hkv, Dh), dtype=bf),
                                     torch.empty((L - 1, Hkv, Dh), dtype=bf), 0.125)
    with pytest.raises(ValueError, match="vb has shape"):
        capi.eagle3_branch_attention(torch.empty((L, Hq, Dh), dtype=bf), torch.empty((3, L, Hkv, Dh), dtype=bf),
                                     torch.empty((2, L, Hkv, Dh), dtype=bf), 0.125)
    with pytest.raises(ValueError, match="parents has"):
        capi.eagle3_build_tree_mask(cu, tok[:3], None, T, T=T)


def test_make_drafter_checks_weight_shapes():
    """make_drafter refuses weights whose shapes disagree with the layer the struct describes."""
    import torch
    d, Hq, Hkv, Dh, F, V = 64, 4, 2, 16, 96, 50
    w = {"embed": (V, d), "w_fuse": (d, 3 * d), "g_embed": (d,), "g_feat": (d,), "g_mlp": (d,),
         "g_final": (d,), "w_qkv": ((Hq + 2 * Hkv) * Dh, 2 * d), "w_o": (d, Hq * Dh),
         "w_gate_up": (2 * F, d), "w_down": (d, F), "w_lm": (V, d)}
    weights = {k: torch.empty(v) for k, v in w.items()}
    weights["w_qkv"] = torch.empty(((Hq + 2 * Hkv) * Dh, d))   # half the input width
    with pytest.raises(ValueError, match="w_qkv has shape"):
        capi.make_drafter(weights, Hq, Hkv, Dh)
    weights = {k: torch.empty(v) for k, v in w.items()}
    with pytest.raises(ValueError, match="multiple"):
        capi.make_drafter(weights, Hq, 3, Dh)


def test_accept_noalloc_host_validation(lib):
    """eagle3_accept_noalloc rejects a winner list larger than its fixed scratch array (and
    bad arguments) on the host, before any device call."""
    P = 1 << 12
    n_max = lib.eagle3_accept_noalloc_max_entries()
    assert n_max == (1 << 20) // 8 - 64
    V = 128256
    T_ok = n_max // 32
    T_big = T_ok + 1
    # B, T, cu_nodes, tokens, parents, mask, W64, logits, V, dtype, temperature, seed, round,
    # max_depth, accept_len, path, out_tokens, bonus, stream
    args = [1, T_big, P, P, P, P, 1, P, V, 1, 0.0, 0, 0, 6, P, P, P, P, None]
    assert lib.eagle3_accept_noalloc(*args) == -2                 # over the scratch array
    bad = list(args); bad[1] = 0
    assert lib.eagle3_accept_noalloc(*bad) == -1                  # T < B
    bad = list(args); bad[6] = 5
    assert lib.eagle3_accept_noalloc(*bad) == -2                  # W64 > 4
    bad = list(args); bad[10] = -1.0
    assert lib.eagle3_accept_noalloc(*bad) == -1                  # negative temperature
    bad = list(args); bad[2] = None
    assert lib.eagle3_accept_noalloc(*bad) == -1                  # null cu_nodes
