"""ctypes binding over libeagle3.so's C-ABI (include/eagle3.h).

Argument marshalling only: every function checks tensor dtype, device and contiguity,
allocates outputs and the device workspace with torch when the caller does not pass them,
and hands raw device pointers plus the current HIP stream to the library.  No compute step
runs here.  If the library is missing this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeagle3.so")

EAGLE3_OK, EAGLE3_EINVAL, EAGLE3_EUNSUPPORTED, EAGLE3_EWORKSPACE, EAGLE3_EHIP = 0, -1, -2, -3, -4
EAGLE3_F32, EAGLE3_BF16 = 0, 1

c_int, c_float, c_size_t, c_void_p, c_uint64, c_double = (
    ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_double)
c_char_p = ctypes.c_char_p


class Eagle3Drafter(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_heads_q", ctypes.c_int32), ("n_heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("eps", c_float), ("rope_theta", c_float),
                ("embed", c_void_p), ("w_fuse", c_void_p), ("g_embed", c_void_p),
                ("g_feat", c_void_p), ("g_mlp", c_void_p), ("g_final", c_void_p),
                ("w_qkv", c_void_p), ("w_o", c_void_p), ("w_gate_up", c_void_p),
                ("w_down", c_void_p), ("w_lm", c_void_p)]


class Eagle3TreeCfg(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_int32), ("topk", ctypes.c_int32), ("width", ctypes.c_int32),
                ("n_nodes", ctypes.c_int32)]


class Eagle3DraftDebug(ctypes.Structure):
    _fields_ = [("g", c_void_p), ("slot_token", c_void_p), ("slot_parent", c_void_p),
                ("slot_a", c_void_p), ("slot_topk_id", c_void_p), ("slot_topk_val", c_void_p),
                ("slot_lse", c_void_p), ("slot_logits", c_void_p)]


class Eagle3BudgetParams(ctypes.Structure):
    _fields_ = [("n_levels", ctypes.c_int32), ("levels", Eagle3TreeCfg * 16),
                ("start_level", ctypes.c_int32), ("cooldown", ctypes.c_int32),
                ("window", ctypes.c_int32), ("low_frac", c_float), ("high_frac", c_float),
                ("max_cv", c_float), ("draft_share_max", c_float), ("verify_ms_max", c_float),
                ("revert_drop", c_float)]


class Eagle3BudgetState(ctypes.Structure):
    _fields_ = [("level", ctypes.c_int32), ("since", ctypes.c_int32), ("block", ctypes.c_int32),
                ("check", ctypes.c_int32), ("count", ctypes.c_int32), ("head", ctypes.c_int32),
                ("g_before", c_double), ("committed", c_double * 256), ("draft_ms", c_double * 256),
                ("verify_ms", c_double * 256)]


EXPORTS = {
    "eagle3_abi_version": (c_int, []),
    "eagle3_status_string": (c_char_p, [c_int]),
    "eagle3_draft_expand_workspace_size": (c_size_t, [c_void_p, c_void_p, c_int, c_int]),
    "eagle3_draft_expand": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_size_t, c_void_p]),
    "eagle3_draft_expand_sampled": (c_int, [c_void_p, c_void_p, c_int, c_float, c_uint64, c_uint64,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                            c_void_p]),
    "eagle3_build_tree_mask": (c_int, [c_int, c_int, c_void_p, c_void_p, c_void_p, c_int,
                                       c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "eagle3_tree_attention_num_splits": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "eagle3_tree_attention_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int,
                                                        c_int, c_int]),
    "eagle3_tree_attention": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int,
                                      c_void_p, c_void_p, c_void_p, c_int, c_float, c_int,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p]),
    "eagle3_lse_merge": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p,
                                 c_void_p, c_void_p]),
    "eagle3_causal_attention": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                        c_float, c_void_p, c_void_p, c_void_p]),
    "eagle3_branch_attention": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                        c_void_p, c_float, c_void_p, c_void_p, c_void_p]),
    "eagle3_linear_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "eagle3_linear": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                              c_size_t, c_void_p]),
    "eagle3_commit_kv": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, ctypes.c_int64, c_void_p, c_void_p,
                                 c_void_p, c_void_p]),
    "eagle3_drafter_catchup_workspace_size": (c_size_t, [c_void_p, c_int]),
    "eagle3_drafter_catchup": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, ctypes.c_int64, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "eagle3_accept_workspace_size": (c_size_t, [c_int, c_int]),
    "eagle3_accept": (c_int, [c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                              c_void_p, c_int, c_int, c_float, c_uint64, c_uint64, c_int,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                              c_void_p]),
    "eagle3_accept_noalloc_max_entries": (c_size_t, []),
    "eagle3_accept_noalloc": (c_int, [c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                      c_void_p, c_int, c_int, c_float, c_uint64, c_uint64, c_int,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "eagle3_accept_sampled_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "eagle3_accept_sampled": (c_int, [c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                      c_int, c_void_p, c_int, c_int, c_void_p, c_int, c_float,
                                      c_uint64, c_uint64, c_int, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "eagle3_budget_init": (c_int, [c_void_p, c_void_p]),
    "eagle3_budget_update": (c_int, [c_void_p, c_void_p, ctypes.c_int32, c_float, c_float, c_void_p]),
    "eagle3_profile_enable": (c_int, [c_int, c_char_p]),
    "eagle3_profile_reset": (c_int, []),
    "eagle3_profile_read": (c_int, [c_char_p, ctypes.POINTER(c_double), ctypes.POINTER(c_int)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libeagle3.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m speculative_decoding_round_amd.build_lib`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class Eagle3Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().eagle3_status_string(status).decode()
        super().__init__(f"{fn} returned {status}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != EAGLE3_OK:
        raise Eagle3Error(fn, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shape(t, name: str, *dims) -> None:
    """Raise unless `t` has len(dims) dimensions matching `dims` (None matches any extent).
    The library sees raw pointers only: a tensor smaller than the layout the arguments imply
    would be read or written out of bounds on the device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dim() != len(dims) or any(d is not None and t.shape[i] != d for i, d in enumerate(dims)):
        want = ", ".join("*" if d is None else str(d) for d in dims)
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [{want}]")


def _out_shapes(out: Optional[dict], shapes: dict) -> None:
    """Caller-provided outputs must have the shapes the call writes."""
    if out is None:
        return
    for k, dims in shapes.items():
        if out.get(k) is not None:
            _shape(out[k], k, *dims)


def _kv_pair(k, v, Hkv: int, Dh: int, kname: str, vname: str) -> None:
    _shape(k, kname, None, Hkv, Dh)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"{vname} shape {tuple(v.shape)} differs from {kname} {tuple(k.shape)}")


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return EAGLE3_F32
    if dt == torch.bfloat16:
        return EAGLE3_BF16
    raise ValueError(f"unsupported element type {dt}")


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def abi_version() -> int:
    return lib().eagle3_abi_version()


# ---------------------------------------------------------------------------------------
# Drafter
# ---------------------------------------------------------------------------------------

WEIGHT_KEYS = ("embed", "w_fuse", "g_embed", "g_feat", "g_mlp", "g_final", "w_qkv", "w_o",
               "w_gate_up", "w_down", "w_lm")


def make_drafter(weights: dict, n_heads_q: int, n_heads_kv: int, head_dim: int,
                 eps: float = 1e-5, rope_theta: float = 500000.0) -> Eagle3Drafter:
    """Describe device-resident drafter weights (layouts as in include/eagle3.h).  The
    returned struct holds raw pointers: keep `weights` alive while it is used."""
    dt = weights["embed"].dtype
    V, d = weights["embed"].shape
    F = weights["w_down"].shape[1]
    if n_heads_kv <= 0 or n_heads_q % n_heads_kv:
        raise ValueError("n_heads_q must be a positive multiple of n_heads_kv")
    dims = {"embed": (V, d), "w_fuse": (d, 3 * d), "g_embed": (d,), "g_feat": (d,), "g_mlp": (d,),
            "g_final": (d,), "w_qkv": ((n_heads_q + 2 * n_heads_kv) * head_dim, 2 * d),
            "w_o": (d, n_heads_q * head_dim), "w_gate_up": (2 * F, d), "w_down": (d, F), "w_lm": (V, d)}
    for k in WEIGHT_KEYS:
        _shape(weights[k], k, *dims[k])
    for k in WEIGHT_KEYS:
        _dev(weights[k], k, dt)
    s = Eagle3Drafter(d=d, n_heads_q=n_heads_q, n_heads_kv=n_heads_kv, head_dim=head_dim, ffn=F,
                      vocab=V, dtype=dtype_code(dt), eps=eps, rope_theta=rope_theta)
    for k in WEIGHT_KEYS:
        setattr(s, k, weights[k].data_ptr())
    return s


def _draft_inputs(drafter: Eagle3Drafter, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix) -> int:
    B = h_low.shape[0] if isinstance(h_low, torch.Tensor) and h_low.dim() == 2 else -1
    for n, t in (("h_low", h_low), ("h_mid", h_mid), ("h_high", h_high)):
        _shape(t, n, B, drafter.d)
    _shape(root_tok, "root_tok", B)
    _shape(cu_prefix, "cu_prefix", B + 1)
    _kv_pair(kpre, vpre, drafter.n_heads_kv, drafter.head_dim, "kpre", "vpre")
    return B


def eagle3_draft_expand_workspace_size(drafter: Eagle3Drafter, tree: Eagle3TreeCfg, B: int,
                                       max_prefix: int) -> int:
    return lib().eagle3_draft_expand_workspace_size(ctypes.byref(drafter), ctypes.byref(tree), B,
                                                    max_prefix)


def eagle3_draft_expand(drafter: Eagle3Drafter, tree: Eagle3TreeCfg, h_low, h_mid, h_high,
                        root_tok, kpre, vpre, cu_prefix, max_prefix: int, debug: bool = False,
                        debug_logits: bool = False, workspace: Optional[torch.Tensor] = None,
                        out: Optional[dict] = None, stream=None) -> dict:
    """One draft-tree round.  Returns dict(tokens, parents, depth, score, n_nodes[, debug]).
    kpre, vpre [rows, Hkv, Dh] must hold every row that cu_prefix (device) names."""
    B = _draft_inputs(drafter, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix)
    dev = h_low.device
    dt = h_low.dtype
    for n, t in (("h_low", h_low), ("h_mid", h_mid), ("h_high", h_high), ("kpre", kpre),
                 ("vpre", vpre)):
        _dev(t, n, dt)
    _dev(root_tok, "root_tok", torch.int32)
    _dev(cu_prefix, "cu_prefix", torch.int32)
    N1 = tree.n_nodes + 1
    _out_shapes(out, {"tokens": (B, N1), "parents": (B, N1), "depth": (B, N1), "score": (B, N1),
                      "n_nodes": (B,)})
    if out is None:
        out = {
            "tokens": torch.empty((B, N1), dtype=torch.int32, device=dev),
            "parents": torch.empty((B, N1), dtype=torch.int32, device=dev),
            "depth": torch.empty((B, N1), dtype=torch.int32, device=dev),
            "score": torch.empty((B, N1), dtype=torch.float32, device=dev),
            "n_nodes": torch.empty((B,), dtype=torch.int32, device=dev),
        }
    dbg_struct = None
    if debug:
        S = 1 + (tree.depth - 1) * tree.width
        K, d, V = tree.topk, drafter.d, drafter.vocab
        dbg = {
            "g": torch.empty((B, d), dtype=torch.float32, device=dev),
            "slot_token": torch.empty((B, S), dtype=torch.int32, device=dev),
            "slot_parent": torch.empty((B, S), dtype=torch.int32, device=dev),
            "slot_a": torch.zeros((B, S, d), dtype=torch.float32, device=dev),
            "slot_topk_id": torch.full((B, S, K), -1, dtype=torch.int32, device=dev),
            "slot_topk_val": torch.zeros((B, S, K), dtype=torch.float32, device=dev),
            "slot_lse": torch.zeros((B, S), dtype=torch.float32, device=dev),
        }
        if debug_logits:
            dbg["slot_logits"] = torch.zeros((B, S, V), dtype=torch.float32, device=dev)
        dbg_struct = Eagle3DraftDebug(**{k: v.data_ptr() for k, v in dbg.items()})
        out["debug"] = dbg
    if workspace is None:
        workspace = _workspace(eagle3_draft_expand_workspace_size(drafter, tree, B, max_prefix), dev)
    st = lib().eagle3_draft_expand(
        ctypes.byref(drafter), ctypes.byref(tree), B, h_low.data_ptr(), h_mid.data_ptr(),
        h_high.data_ptr(), root_tok.data_ptr(), kpre.data_ptr(), vpre.data_ptr(),
        cu_prefix.data_ptr(), int(max_prefix), out["tokens"].data_ptr(), out["parents"].data_ptr(),
        out["depth"].data_ptr(), out["score"].data_ptr(), out["n_nodes"].data_ptr(),
        ctypes.byref(dbg_struct) if dbg_struct is not None else None,
        workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check("eagle3_draft_expand", st)
    return out


def eagle3_draft_expand_sampled(drafter: Eagle3Drafter, tree: Eagle3TreeCfg, temperature: float,
                                seed: int, round: int, h_low, h_mid, h_high, root_tok, kpre, vpre,
                                cu_prefix, max_prefix: int, debug: bool = False,
                                workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                                stream=None) -> dict:
    """The draft-tree round with sampled candidates.  Returns dict(tokens, parents, depth, score,
    n_nodes, slot_logits [B, S, V] fp32, draft_row [B, N+1] (row of slot_logits viewed as
    [B*S, V] at each node, -1 when the node was not evaluated)[, debug])."""
    B = _draft_inputs(drafter, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix)
    dev = h_low.device
    dt = h_low.dtype
    for n, t in (("h_low", h_low), ("h_mid", h_mid), ("h_high", h_high), ("kpre", kpre),
                 ("vpre", vpre)):
        _dev(t, n, dt)
    _dev(root_tok, "root_tok", torch.int32)
    _dev(cu_prefix, "cu_prefix", torch.int32)
    N1 = tree.n_nodes + 1
    S = 1 + (tree.depth - 1) * tree.width
    _out_shapes(out, {"tokens": (B, N1), "parents": (B, N1), "depth": (B, N1), "score": (B, N1),
                      "n_nodes": (B,), "slot_logits": (B, S, drafter.vocab), "draft_row": (B, N1)})
    if out is None:
        out = {
            "tokens": torch.empty((B, N1), dtype=torch.int32, device=dev),
            "parents": torch.empty((B, N1), dtype=torch.int32, device=dev),
            "depth": torch.empty((B, N1), dtype=torch.int32, device=dev),
            "score": torch.empty((B, N1), dtype=torch.float32, device=dev),
            "n_nodes": torch.empty((B,), dtype=torch.int32, device=dev),
            "slot_logits": torch.zeros((B, S, drafter.vocab), dtype=torch.float32, device=dev),
            "draft_row": torch.empty((B, N1), dtype=torch.int32, device=dev),
        }
    dbg_struct = None
    if debug:
        K, d = tree.topk, drafter.d
        dbg = {
            "g": torch.empty((B, d), dtype=torch.float32, device=dev),
            "slot_token": torch.empty((B, S), dtype=torch.int32, device=dev),
            "slot_parent": torch.empty((B, S), dtype=torch.int32, device=dev),
            "slot_a": torch.zeros((B, S, d), dtype=torch.float32, device=dev),
            "slot_topk_id": torch.full((B, S, K), -1, dtype=torch.int32, device=dev),
            "slot_topk_val": torch.zeros((B, S, K), dtype=torch.float32, device=dev),
            "slot_lse": torch.zeros((B, S), dtype=torch.float32, device=dev),
        }
        dbg_struct = Eagle3DraftDebug(**{k: v.data_ptr() for k, v in dbg.items()})
        dbg["slot_logits"] = out["slot_logits"]
        out["debug"] = dbg
    if workspace is None:
        workspace = _workspace(eagle3_draft_expand_workspace_size(drafter, tree, B, max_prefix), dev)
    st = lib().eagle3_draft_expand_sampled(
        ctypes.byref(drafter), ctypes.byref(tree), B, float(temperature), int(seed) & (2**64 - 1),
        int(round) & (2**64 - 1), h_low.data_ptr(), h_mid.data_ptr(), h_high.data_ptr(),
        root_tok.data_ptr(), kpre.data_ptr(), vpre.data_ptr(), cu_prefix.data_ptr(), int(max_prefix),
        out["tokens"].data_ptr(), out["parents"].data_ptr(), out["depth"].data_ptr(),
        out["score"].data_ptr(), out["n_nodes"].data_ptr(), out["slot_logits"].data_ptr(),
        out["draft_row"].data_ptr(), ctypes.byref(dbg_struct) if dbg_struct is not None else None,
        workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check("eagle3_draft_expand_sampled", st)
    return out


# ---------------------------------------------------------------------------------------
# Verify side
# ---------------------------------------------------------------------------------------


def eagle3_build_tree_mask(cu_nodes, parents, cu_prefix, max_nodes: int, W64: int = 1,
                           T: Optional[int] = None, dev_status: Optional[torch.Tensor] = None,
                           out: Optional[dict] = None, stream=None) -> dict:
    _shape(cu_nodes, "cu_nodes", None)
    _shape(parents, "parents", None)
    B = cu_nodes.numel() - 1
    T = parents.numel() if T is None else T
    if parents.numel() < T:
        raise ValueError(f"parents has {parents.numel()} entries, fewer than T = {T}")
    if cu_prefix is not None:
        _shape(cu_prefix, "cu_prefix", B + 1)
    _out_shapes(out, {"mask": (T, W64), "depth": (T,), "pos": (T,)})
    _dev(cu_nodes, "cu_nodes", torch.int32)
    _dev(parents, "parents", torch.int32)
    if cu_prefix is not None:
        _dev(cu_prefix, "cu_prefix", torch.int32)
    dev = parents.device
    if out is None:
        out = {"mask": torch.empty((T, W64), dtype=torch.uint64, device=dev),
               "depth": torch.empty((T,), dtype=torch.int32, device=dev),
               "pos": torch.empty((T,), dtype=torch.int32, device=dev)}
    st = lib().eagle3_build_tree_mask(B, T, cu_nodes.data_ptr(), parents.data_ptr(),
                                      _ptr(cu_prefix), int(max_nodes), out["mask"].data_ptr(), W64,
                                      _ptr(out.get("depth")), _ptr(out.get("pos")), _ptr(dev_status),
                                      _stream(stream))
    _check("eagle3_build_tree_mask", st)
    return out


def eagle3_tree_attention_num_splits(B: int, Hq: int, Hkv: int, max_nodes: int, max_prefix: int,
                                     n_splits: int = 0) -> int:
    s = lib().eagle3_tree_attention_num_splits(B, Hq, Hkv, max_nodes, max_prefix, n_splits)
    if s < 1:
        raise Eagle3Error("eagle3_tree_attention_num_splits", s)
    return s


def eagle3_tree_attention(q, k_tree, v_tree, cu_nodes, max_nodes: int, mask, kpre, vpre,
                          cu_prefix, max_prefix: int, scale: float, n_splits: int = 0,
                          partials: bool = False, merged: bool = True,
                          workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                          stream=None) -> dict:
    """Tree attention.  partials=True returns o_part/lse_part; merged=True returns o/lse.
    kpre, vpre [rows, Hkv, Dh] must hold every row that cu_prefix (device) names."""
    _shape(q, "q", None, None, None)
    T, Hq, Dh = q.shape
    Hkv = k_tree.shape[1] if isinstance(k_tree, torch.Tensor) and k_tree.dim() == 3 else -1
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError("k_tree must be [T, Hkv, Dh] with Hq a multiple of Hkv")
    _kv_pair(k_tree, v_tree, Hkv, Dh, "k_tree", "v_tree")
    if k_tree.shape[0] != T:
        raise ValueError(f"k_tree has {k_tree.shape[0]} rows, q has {T}")
    if not isinstance(mask, torch.Tensor) or mask.dim() not in (1, 2) or mask.shape[0] != T:
        raise ValueError(f"mask must be [T, W64] or [T] with T = {T} rows")
    if max_prefix > 0:
        _kv_pair(kpre, vpre, Hkv, Dh, "kpre", "vpre")
        _shape(cu_prefix, "cu_prefix", cu_nodes.numel())
    dt = q.dtype
    for n, t in (("q", q), ("k_tree", k_tree), ("v_tree", v_tree)):
        _dev(t, n, dt)
    _dev(cu_nodes, "cu_nodes", torch.int32)
    _dev(mask, "mask", torch.uint64)
    if max_prefix > 0:
        _dev(kpre, "kpre", dt)
        _dev(vpre, "vpre", dt)
        _dev(cu_prefix, "cu_prefix", torch.int32)
    B = cu_nodes.numel() - 1
    W64 = mask.shape[1] if mask.dim() == 2 else 1
    S = eagle3_tree_attention_num_splits(B, Hq, Hkv, max_nodes, max_prefix, n_splits)
    dev = q.device
    _out_shapes(out, {"o_part": (S + 1, T, Hq, Dh), "lse_part": (S + 1, T, Hq), "o": (T, Hq, Dh),
                      "lse": (T, Hq)})
    if out is None:
        out = {}
        if partials:
            out["o_part"] = torch.empty((S + 1, T, Hq, Dh), dtype=torch.float32, device=dev)
            out["lse_part"] = torch.empty((S + 1, T, Hq), dtype=torch.float32, device=dev)
        if merged:
            out["o"] = torch.empty((T, Hq, Dh), dtype=dt, device=dev)
            out["lse"] = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if workspace is None and "o_part" not in out:
        workspace = _workspace(lib().eagle3_tree_attention_workspace_size(
            B, T, Hq, Hkv, Dh, max_nodes, max_prefix, n_splits), dev)
    st = lib().eagle3_tree_attention(
        B, T, Hq, Hkv, Dh, dtype_code(dt), q.data_ptr(), k_tree.data_ptr(), v_tree.data_ptr(),
        cu_nodes.data_ptr(), int(max_nodes), mask.data_ptr(), W64, _ptr(kpre), _ptr(vpre),
        _ptr(cu_prefix), int(max_prefix), float(scale), int(n_splits), _ptr(out.get("o_part")),
        _ptr(out.get("lse_part")), _ptr(out.get("o")), _ptr(out.get("lse")), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream))
    _check("eagle3_tree_attention", st)
    out["splits"] = S
    return out


def eagle3_lse_merge(o_part, lse_part, out_dtype=torch.float32, out: Optional[dict] = None,
                     stream=None) -> dict:
    """o_part [S, rows, Dh] fp32, lse_part [S, rows] fp32 -> dict(o [rows, Dh], lse [rows])."""
    _shape(o_part, "o_part", None, None, None)
    S, rows, Dh = o_part.shape
    _shape(lse_part, "lse_part", S, rows)
    _dev(o_part, "o_part", torch.float32)
    _dev(lse_part, "lse_part", torch.float32)
    _out_shapes(out, {"o": (rows, Dh), "lse": (rows,)})
    if out is None:
        out = {"o": torch.empty((rows, Dh), dtype=out_dtype, device=o_part.device),
               "lse": torch.empty((rows,), dtype=torch.float32, device=o_part.device)}
    st = lib().eagle3_lse_merge(S, rows, Dh, o_part.data_ptr(), lse_part.data_ptr(),
                                dtype_code(out["o"].dtype), out["o"].data_ptr(), _ptr(out.get("lse")),
                                _stream(stream))
    _check("eagle3_lse_merge", st)
    return out


def _accept_inputs(cu_nodes, tokens, parents, mask, logits, max_depth: int, out: Optional[dict]):
    _shape(logits, "logits", None, None)
    T = logits.shape[0]
    _shape(cu_nodes, "cu_nodes", None)
    B = cu_nodes.numel() - 1
    if tokens.numel() != T or parents.numel() != T:
        raise ValueError(f"tokens and parents need one entry per logits row ({T})")
    if mask is not None and (not isinstance(mask, torch.Tensor) or mask.dim() not in (1, 2) or mask.shape[0] != T):
        raise ValueError(f"mask must be [T, W64] or [T] with T = {T} rows")
    if max_depth < 0:
        raise ValueError("max_depth must be >= 0")
    _out_shapes(out, {"accept_len": (B,), "path": (B, max_depth + 1), "out_tokens": (B, max_depth + 1),
                      "bonus": (B,)})


def eagle3_accept(cu_nodes, tokens, parents, mask, logits, temperature: float, seed: int,
                  round: int, max_depth: int, workspace: Optional[torch.Tensor] = None,
                  out: Optional[dict] = None, stream=None) -> dict:
    _accept_inputs(cu_nodes, tokens, parents, mask, logits, max_depth, out)
    _dev(cu_nodes, "cu_nodes", torch.int32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parents, "parents", torch.int32)
    _dev(mask, "mask", torch.uint64)
    _dev(logits, "logits")
    B = cu_nodes.numel() - 1
    T, V = logits.shape
    W64 = mask.shape[1] if mask.dim() == 2 else 1
    dev = logits.device
    if out is None:
        out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
               "path": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty((B,), dtype=torch.int32, device=dev)}
    if workspace is None:
        workspace = _workspace(lib().eagle3_accept_workspace_size(T, V), dev)
    st = lib().eagle3_accept(B, T, cu_nodes.data_ptr(), tokens.data_ptr(), parents.data_ptr(),
                             mask.data_ptr(), W64, logits.data_ptr(), V, dtype_code(logits.dtype),
                             float(temperature), int(seed) & (2**64 - 1), int(round) & (2**64 - 1),
                             int(max_depth), out["accept_len"].data_ptr(), out["path"].data_ptr(),
                             out["out_tokens"].data_ptr(), out["bonus"].data_ptr(),
                             workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check("eagle3_accept", st)
    return out


def eagle3_accept_noalloc(cu_nodes, tokens, parents, mask, logits, temperature: float, seed: int,
                          round: int, max_depth: int, out: Optional[dict] = None, stream=None) -> dict:
    """eagle3_accept without a workspace (the library's fixed per-GPU scratch array); for
    callers that cannot allocate.  Pass `out` to allocate nothing here either."""
    _accept_inputs(cu_nodes, tokens, parents, mask, logits, max_depth, out)
    _dev(cu_nodes, "cu_nodes", torch.int32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parents, "parents", torch.int32)
    _dev(mask, "mask", torch.uint64)
    _dev(logits, "logits")
    B = cu_nodes.numel() - 1
    T, V = logits.shape
    W64 = mask.shape[1] if mask.dim() == 2 else 1
    dev = logits.device
    if out is None:
        out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
               "path": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty((B,), dtype=torch.int32, device=dev)}
    st = lib().eagle3_accept_noalloc(B, T, cu_nodes.data_ptr(), tokens.data_ptr(), parents.data_ptr(),
                                     mask.data_ptr(), W64, logits.data_ptr(), V, dtype_code(logits.dtype),
                                     float(temperature), int(seed) & (2**64 - 1), int(round) & (2**64 - 1),
                                     int(max_depth), out["accept_len"].data_ptr(), out["path"].data_ptr(),
                                     out["out_tokens"].data_ptr(), out["bonus"].data_ptr(), _stream(stream))
    _check("eagle3_accept_noalloc", st)
    return out


def eagle3_accept_sampled(cu_nodes, tokens, parents, logits, draft_logits, draft_row,
                          temperature: float, seed: int, round: int, max_depth: int,
                          max_children: int, dev_status: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                          stream=None) -> dict:
    """Acceptance of sampled candidates: draft_logits [R, V] holds the drafter's logits, and
    draft_row[i] names the row of node i (-1 for a node without children)."""
    _accept_inputs(cu_nodes, tokens, parents, None, logits, max_depth, out)
    if draft_row.numel() != logits.shape[0]:
        raise ValueError("draft_row needs one entry per logits row")
    _dev(cu_nodes, "cu_nodes", torch.int32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parents, "parents", torch.int32)
    _dev(draft_row, "draft_row", torch.int32)
    _dev(logits, "logits")
    B = cu_nodes.numel() - 1
    T, V = logits.shape
    dev = logits.device
    R = 0 if draft_logits is None else draft_logits.shape[0]
    if draft_logits is not None:
        _dev(draft_logits, "draft_logits")
        if draft_logits.shape[1] != V:
            raise ValueError("draft_logits must have the target's vocabulary")
    if out is None:
        out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
               "path": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty((B,), dtype=torch.int32, device=dev)}
    if workspace is None:
        workspace = _workspace(lib().eagle3_accept_sampled_workspace_size(T, V, int(max_children)), dev)
    st = lib().eagle3_accept_sampled(
        B, T, cu_nodes.data_ptr(), tokens.data_ptr(), parents.data_ptr(), logits.data_ptr(), V,
        dtype_code(logits.dtype), None if draft_logits is None else draft_logits.data_ptr(),
        dtype_code(logits.dtype if draft_logits is None else draft_logits.dtype), R,
        draft_row.data_ptr(), int(max_children), float(temperature), int(seed) & (2**64 - 1),
        int(round) & (2**64 - 1), int(max_depth), out["accept_len"].data_ptr(), out["path"].data_ptr(),
        out["out_tokens"].data_ptr(), out["bonus"].data_ptr(),
        None if dev_status is None else dev_status.data_ptr(), workspace.data_ptr(), workspace.numel(),
        _stream(stream))
    _check("eagle3_accept_sampled", st)
    return out


# ---------------------------------------------------------------------------------------
# After acceptance: commit and drafter catch-up
# ---------------------------------------------------------------------------------------


def _cache_pair(k_cache, v_cache, row_shape) -> None:
    """The kernels bound their writes by k_cache's row count alone: both caches must be
    [rows, Hkv, Dh] with the same rows and the (Hkv, Dh) of what is written into them."""
    if k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != tuple(row_shape):
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} is not [rows, {row_shape[0]}, {row_shape[1]}]")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} differs from k_cache {tuple(k_cache.shape)}")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("k_cache and v_cache must be contiguous")


def eagle3_commit_kv(cu_nodes, path, accept_len, k_tree, v_tree, dst_row, k_cache, v_cache,
                     dev_status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Copy the accepted path's tree K/V rows (path [B, path_stride] from eagle3_accept) into
    the caches at rows dst_row[b] + i, in place."""
    _shape(cu_nodes, "cu_nodes", None)
    B = cu_nodes.numel() - 1
    _shape(path, "path", B, None)
    _shape(accept_len, "accept_len", B)
    _shape(dst_row, "dst_row", B)
    for n, t in (("cu_nodes", cu_nodes), ("path", path), ("accept_len", accept_len),
                 ("dst_row", dst_row)):
        _dev(t, n, torch.int32)
    dt = k_tree.dtype
    for n, t in (("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, n, dt)
    B = cu_nodes.numel() - 1
    _, Hkv, Dh = k_tree.shape
    if tuple(v_tree.shape) != tuple(k_tree.shape):
        raise ValueError(f"v_tree shape {tuple(v_tree.shape)} differs from k_tree {tuple(k_tree.shape)}")
    _cache_pair(k_cache, v_cache, (Hkv, Dh))
    st = lib().eagle3_commit_kv(B, Hkv, Dh, dtype_code(dt), path.shape[1], cu_nodes.data_ptr(),
                                path.data_ptr(), accept_len.data_ptr(), k_tree.data_ptr(),
                                v_tree.data_ptr(), dst_row.data_ptr(), k_cache.shape[0],
                                k_cache.data_ptr(), v_cache.data_ptr(), _ptr(dev_status), _stream(stream))
    _check("eagle3_commit_kv", st)


def eagle3_drafter_catchup_workspace_size(drafter: Eagle3Drafter, n: int) -> int:
    return lib().eagle3_drafter_catchup_workspace_size(ctypes.byref(drafter), n)


def eagle3_drafter_catchup(drafter: Eagle3Drafter, tokens, pos, h_low, h_mid, h_high, dst_row,
                           k_cache, v_cache, g_out: Optional[torch.Tensor] = None,
                           dev_status: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Drafter keys/values of committed positions (rows) into the drafter prefix caches at
    dst_row, from the real target features; returns the fused features g [n, d] (fp32)."""
    _shape(tokens, "tokens", None)
    n_rows = tokens.numel()
    for n, t in (("pos", pos), ("dst_row", dst_row)):
        _shape(t, n, n_rows)
    for n, t in (("h_low", h_low), ("h_mid", h_mid), ("h_high", h_high)):
        _shape(t, n, n_rows, drafter.d)
    if g_out is not None:
        _shape(g_out, "g_out", n_rows, drafter.d)
    for n, t in (("tokens", tokens), ("pos", pos), ("dst_row", dst_row)):
        _dev(t, n, torch.int32)
    dt = h_low.dtype
    for n, t in (("h_low", h_low), ("h_mid", h_mid), ("h_high", h_high), ("k_cache", k_cache),
                 ("v_cache", v_cache)):
        _dev(t, n, dt)
    n_rows = tokens.numel()
    _cache_pair(k_cache, v_cache, (drafter.n_heads_kv, drafter.head_dim))
    if g_out is None:
        g_out = torch.empty((n_rows, drafter.d), dtype=torch.float32, device=h_low.device)
    _dev(g_out, "g_out", torch.float32)
    if workspace is None:
        workspace = _workspace(eagle3_drafter_catchup_workspace_size(drafter, n_rows), h_low.device)
    st = lib().eagle3_drafter_catchup(ctypes.byref(drafter), n_rows, tokens.data_ptr(), pos.data_ptr(),
                                      h_low.data_ptr(), h_mid.data_ptr(), h_high.data_ptr(),
                                      dst_row.data_ptr(), k_cache.shape[0], k_cache.data_ptr(),
                                      v_cache.data_ptr(), g_out.data_ptr(), _ptr(dev_status),
                                      workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check("eagle3_drafter_catchup", st)
    return g_out


# ---------------------------------------------------------------------------------------
# Training form of the long-context shape (every position a query)
# ---------------------------------------------------------------------------------------


def eagle3_causal_attention(q, k, v, scale: float, o: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, stream=None):
    """Main causal attention of every position: q [L, Hq, Dh], k, v [L, Hkv, Dh] (bf16).
    Returns (o [L, Hq, Dh] fp32, lse [L, Hq] fp32)."""
    _shape(q, "q", None, None, None)
    L, Hq, Dh = q.shape
    Hkv = k.shape[1] if isinstance(k, torch.Tensor) and k.dim() == 3 else -1
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError("k must be [L, Hkv, Dh] with Hq a multiple of Hkv")
    _shape(k, "k", L, Hkv, Dh)
    _shape(v, "v", L, Hkv, Dh)
    for n, t in (("o", o), ("lse", lse)):
        if t is not None:
            _shape(t, n, *((L, Hq, Dh) if n == "o" else (L, Hq)))
    dt = q.dtype
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, n, dt)
    if o is None:
        o = torch.empty((L, Hq, Dh), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((L, Hq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    st = lib().eagle3_causal_attention(L, Hq, Hkv, Dh, dtype_code(dt), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       float(scale), o.data_ptr(), lse.data_ptr(), _stream(stream))
    _check("eagle3_causal_attention", st)
    return o, lse


def eagle3_branch_attention(q, kb, vb, scale: float, o: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, stream=None):
    """Per-position branch attention: q [L, Hq, Dh], kb, vb [n_steps, L, Hkv, Dh].
    Returns (o [L, Hq, Dh] fp32, lse [L, Hq] fp32)."""
    _shape(q, "q", None, None, None)
    L, Hq, Dh = q.shape
    _shape(kb, "kb", None, L, None, Dh)
    n_steps, _, Hkv, _ = kb.shape
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError("kb must be [n_steps, L, Hkv, Dh] with Hq a multiple of Hkv")
    _shape(vb, "vb", n_steps, L, Hkv, Dh)
    for n, t in (("o", o), ("lse", lse)):
        if t is not None:
            _shape(t, n, *((L, Hq, Dh) if n == "o" else (L, Hq)))
    dt = q.dtype
    for n, t in (("q", q), ("kb", kb), ("vb", vb)):
        _dev(t, n, dt)
    if o is None:
        o = torch.empty((L, Hq, Dh), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((L, Hq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    st = lib().eagle3_branch_attention(L, n_steps, Hq, Hkv, Dh, dtype_code(dt), q.data_ptr(), kb.data_ptr(),
                                       vb.data_ptr(), float(scale), o.data_ptr(), lse.data_ptr(), _stream(stream))
    _check("eagle3_branch_attention", st)
    return o, lse


# ---------------------------------------------------------------------------------------
# Projections' GEMM
# ---------------------------------------------------------------------------------------


def eagle3_linear(x, w, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Y = X W^T in fp32 through the drafter's GEMM kernels; x [M, K], w [N, K] (same dtype)."""
    _shape(x, "x", None, None)
    _shape(w, "w", None, x.shape[1])
    if out is not None:
        _shape(out, "out", x.shape[0], w.shape[0])
    _dev(w, "w")
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dim() == 2 and x.stride(1) == 1):
        raise ValueError("x must be a 2-D device tensor with unit column stride")
    if x.dtype != w.dtype:
        raise ValueError("x and w must have the same dtype")
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    dt = dtype_code(x.dtype)
    need = lib().eagle3_linear_workspace_size(M, N, K, dt)
    if workspace is None and need > 0:
        workspace = _workspace(need, x.device)
    st = lib().eagle3_linear(M, N, K, dt, x.data_ptr(), x.stride(0), w.data_ptr(), out.data_ptr(),
                             _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    _check("eagle3_linear", st)
    return out


# ---------------------------------------------------------------------------------------
# Speculative-budget controller (host)
# ---------------------------------------------------------------------------------------


class BudgetController:
    """Host-side budget controller over the library's state machine (eagle3_budget_*).
    levels: sequence of (depth, topk, width, n_nodes) in increasing size."""

    def __init__(self, levels, start: int, cooldown: int, window: int, low_frac: float,
                 high_frac: float, max_cv: float, draft_share_max: float, verify_ms_max: float,
                 revert_drop: float):
        p = Eagle3BudgetParams(n_levels=len(levels), start_level=start, cooldown=cooldown,
                               window=window, low_frac=low_frac, high_frac=high_frac, max_cv=max_cv,
                               draft_share_max=draft_share_max, verify_ms_max=verify_ms_max,
                               revert_drop=revert_drop)
        for i, (d, k, w, n) in enumerate(levels):
            p.levels[i] = Eagle3TreeCfg(depth=d, topk=k, width=w, n_nodes=n)
        self.params = p
        self.state = Eagle3BudgetState()
        _check("eagle3_budget_init", lib().eagle3_budget_init(ctypes.byref(p), ctypes.byref(self.state)))

    def update(self, accept_len: int, draft_ms: float, verify_ms: float):
        """Report one round; returns (level, Eagle3TreeCfg) for the next round."""
        t = Eagle3TreeCfg()
        lv = lib().eagle3_budget_update(ctypes.byref(self.params), ctypes.byref(self.state), int(accept_len),
                                        float(draft_ms), float(verify_ms), ctypes.byref(t))
        _check("eagle3_budget_update", min(lv, 0))
        return lv, t


# ---------------------------------------------------------------------------------------
# Launch timing
# ---------------------------------------------------------------------------------------


def eagle3_profile_enable(on: bool = True, only_kernel: Optional[str] = None) -> None:
    """Time the library's launches (only those named `only_kernel` if given)."""
    name = only_kernel.encode() if only_kernel else None
    _check("eagle3_profile_enable", lib().eagle3_profile_enable(1 if on else 0, name))


def eagle3_profile_reset() -> None:
    _check("eagle3_profile_reset", lib().eagle3_profile_reset())


def eagle3_profile_read(kernel: str):
    """(total milliseconds, launches) recorded for one kernel name."""
    ms = c_double(0.0)
    n = c_int(0)
    _check("eagle3_profile_read", lib().eagle3_profile_read(kernel.encode(), ctypes.byref(ms),
                                                            ctypes.byref(n)))
    return ms.value, n.value
