"""Benchmark: one EAGLE-3 draft-tree round + one tree-verification round per step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama70b]

A step runs the whole hot path on one stream through the C-ABI:
  eagle3_draft_expand -> eagle3_build_tree_mask -> eagle3_tree_attention (partials)
  -> eagle3_lse_merge -> eagle3_accept.
The default workload is the largest one that fits one GPU: a Llama-3.1-70B-shaped drafter
(d 8192, 64 / 8 heads of 128, FFN 28672, vocabulary 128256, fusion 24576 -> 8192), batch 4,
8192-token prefixes, 60-node trees of depth 6 (K = W = 10), acceptance at T = 0.7.  Inputs
are seeded synthetic tensors already resident in HBM (random-init weights, Gaussian features
and KV); the verify layer's Q/K/V and the target logits (the drafter's own logits plus
noise) are given, untimed.  The whole rounds of the 8B-shaped and batch-16 workloads are
reported as extra fields.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tree tokens/sec per draft+verify round; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama70b", choices=["llama8b", "batch16", "llama70b", "tiny"])
    ap.add_argument("--no-other-rounds", action="store_true",
                    help="skip the whole rounds of the other workloads (extra fields)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ops", action="store_true", help="skip the per-op roofline measurements")
    ap.add_argument("--only-ops", action="store_true",
                    help="measure only the per-op rooflines (no round, no CPU baseline)")
    ap.add_argument("--ops", default=",".join(OP_KEYS),
                    help="comma-separated per-op measurements to run")
    ap.add_argument("--kernel", default="gemm_lm_head",
                    help="kernel timed for the roofline (gemm_lm_head: the depth steps' LM head)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (for scaling HBM byte "
                         "counters against a kernel of known traffic)")
    return ap.parse_args()


class Round:
    """Preallocated buffers for one draft + verify round.

    Per-round inputs (the drafter's prefix KV, the verify layer's Q/K/V and prefix KV, the
    target logits) exist in `ncopy` identical copies at different addresses, and round r reads
    copy r % ncopy, so that together they exceed the 256 MB Infinity Cache twice and every
    round reads them from HBM, as a serving loop over fresh requests would.

    Target logits (harness, untimed): one draft round is run with per-slot logits kept; at
    every drafted node the drafter evaluated, Z_t = Z_d + N(0, noise^2) (the workloads'
    "target logits correlated with the draft logits"); at a leaf the drafter never evaluated
    (it only decides the bonus token) a fresh N(0, 1) row.  The batch-16 workload instead takes
    N(0, 1) rows with one planted path per request (a uniform length 0..depth, a random node at
    that depth, each edge's child token raised above its parent row's maximum)."""

    def __init__(self, shape, dev, seed=1234, rotate=True, targets=True):
        import torch
        from speculative_decoding_round_amd import capi, synth
        self.shape = shape
        self.capi = capi
        self.B = shape.B
        self.prefix = synth.prefix_lengths(shape, seed)
        self.w = synth.drafter_weights(shape, seed=seed, device=dev)
        di = synth.draft_inputs(shape, seed=seed + 1, device=dev, prefix=self.prefix)
        self.drafter = capi.make_drafter(self.w, shape.Hq, shape.Hkv, shape.Dh)
        self.tree = capi.Eagle3TreeCfg(depth=shape.depth, topk=shape.topk, width=shape.width,
                                       n_nodes=shape.n_nodes)
        self.max_prefix = max(self.prefix)
        n1 = shape.n_nodes + 1
        self.n1 = n1
        self.T = self.B * n1
        ws = capi.eagle3_draft_expand_workspace_size(self.drafter, self.tree, self.B, self.max_prefix)
        self.ws_draft = torch.empty(ws, dtype=torch.uint8, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.draft_out = {"tokens": torch.empty((self.B, n1), **i32),
                          "parents": torch.empty((self.B, n1), **i32),
                          "depth": torch.empty((self.B, n1), **i32),
                          "score": torch.empty((self.B, n1), dtype=torch.float32, device=dev),
                          "n_nodes": torch.empty((self.B,), **i32)}
        # verify layer: queries and tree K/V for every node, its own prefix KV, target logits
        trees = [[-1] + [0] * (n1 - 1)] * self.B        # shapes only; topology comes from the draft
        vi = synth.verify_inputs(shape, trees, self.prefix, seed=seed + 2, device=dev)
        self.cu_nodes = torch.arange(0, self.T + 1, n1, **i32)
        self.mask_out = {"mask": torch.empty((self.T, 1), dtype=torch.uint64, device=dev),
                         "depth": torch.empty((self.T,), **i32), "pos": torch.empty((self.T,), **i32)}
        self.S = capi.eagle3_tree_attention_num_splits(self.B, shape.Hq, shape.Hkv, n1, self.max_prefix, 0)
        Hq, Dh = shape.Hq, shape.Dh
        f32 = dict(dtype=torch.float32, device=dev)
        self.att_out = {"o_part": torch.empty((self.S + 1, self.T, Hq, Dh), **f32),
                        "lse_part": torch.empty((self.S + 1, self.T, Hq), **f32)}
        self.merge_out = {"o": torch.empty((self.T * Hq, Dh), dtype=synth.torch_dtype(shape), device=dev),
                          "lse": torch.empty((self.T * Hq,), **f32)}
        self.ws_acc = torch.empty(capi.lib().eagle3_accept_workspace_size(self.T, shape.V),
                                  dtype=torch.uint8, device=dev)
        D = shape.depth
        self.acc_out = {"accept_len": torch.empty((self.B,), **i32),
                        "path": torch.empty((self.B, D + 1), **i32),
                        "out_tokens": torch.empty((self.B, D + 1), **i32),
                        "bonus": torch.empty((self.B,), **i32)}
        self.scale = float(1.0 / math.sqrt(Dh))
        self.round = 0
        self.di, self.vi = di, vi
        if targets:
            vi["logits"] = self.target_logits(seed + 3)
        per_round = sum(t.numel() * t.element_size() for t in (di["kpre"], di["vpre"]))
        per_round += sum(vi[k].numel() * vi[k].element_size()
                         for k in ("q", "k_tree", "v_tree", "kpre", "vpre", "logits"))
        self.per_round_input_bytes = per_round
        self.ncopy = _copies(per_round) if rotate else 1
        dk, vk = ("kpre", "vpre"), ("q", "k_tree", "v_tree", "kpre", "vpre", "logits")
        self.di_c = [di] + [dict(di, **{k: di[k].clone() for k in dk}) for _ in range(self.ncopy - 1)]
        self.vi_c = [vi] + [dict(vi, **{k: vi[k].clone() for k in vk}) for _ in range(self.ncopy - 1)]

    def target_logits(self, seed):
        """Target logits [T, V] for the drafted trees (see the class docstring)."""
        import torch
        from speculative_decoding_round_amd import synth
        s, c, di = self.shape, self.capi, self.di
        out = c.eagle3_draft_expand(self.drafter, self.tree, di["h_low"], di["h_mid"], di["h_high"],
                                    di["root_tok"], di["kpre"], di["vpre"], di["cu_prefix"],
                                    self.max_prefix, debug=True, debug_logits=True)
        torch.cuda.synchronize()
        tok, par = out["tokens"].cpu(), out["parents"].cpu()
        dbg = out["debug"]
        st, sp = dbg["slot_token"].cpu(), dbg["slot_parent"].cpu()
        g = torch.Generator(device="cpu").manual_seed(seed)
        rows = []
        for b in range(self.B):
            slot_of = {0: 0}
            for i in range(1, self.n1):
                ps = slot_of.get(int(par[b, i]), -1)
                hit = ((sp[b] == ps) & (st[b] == tok[b, i])).nonzero() if ps >= 0 else []
                slot_of[i] = int(hit[0]) if len(hit) else -1
            for i in range(self.n1):
                z = torch.randn(s.V, generator=g)
                if s.verify_tree != "random" and slot_of[i] >= 0:
                    z = dbg["slot_logits"][b, slot_of[i]].cpu() + s.noise * z
                rows.append(z)
        z = torch.stack(rows)
        if s.verify_tree == "random":
            dep = out["depth"].cpu()
            for b in range(self.B):
                L = int(torch.randint(0, s.depth + 1, (1,), generator=g))
                cand = [i for i in range(self.n1) if int(dep[b, i]) == L] or [0]
                end = cand[int(torch.randint(0, len(cand), (1,), generator=g))]
                synth.plant_path(z, tok.view(-1), par[b].tolist(), b * self.n1, end)
        self.draft_tokens = tok
        self.draft_parents = par
        return z.to(synth.torch_dtype(s)).to(self.di["kpre"].device)

    def step(self):
        c, s = self.capi, self.shape
        di, vi = self.di_c[self.round % self.ncopy], self.vi_c[self.round % self.ncopy]
        out = c.eagle3_draft_expand(self.drafter, self.tree, di["h_low"], di["h_mid"], di["h_high"],
                                    di["root_tok"], di["kpre"], di["vpre"], di["cu_prefix"],
                                    self.max_prefix, workspace=self.ws_draft, out=self.draft_out)
        parents = out["parents"].view(-1)
        tokens = out["tokens"].view(-1)
        mk = c.eagle3_build_tree_mask(self.cu_nodes, parents, vi["cu_prefix"], self.n1,
                                      out=self.mask_out)
        att = c.eagle3_tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], self.cu_nodes, self.n1,
                                      mk["mask"], vi["kpre"], vi["vpre"], vi["cu_prefix"],
                                      self.max_prefix, self.scale, out=self.att_out)
        T, Hq, Dh = self.T, s.Hq, s.Dh
        c.eagle3_lse_merge(att["o_part"].view(self.S + 1, T * Hq, Dh),
                           att["lse_part"].view(self.S + 1, T * Hq), out=self.merge_out)
        c.eagle3_accept(self.cu_nodes, tokens, parents, mk["mask"], vi["logits"], s.temperature,
                        seed=20260101, round=self.round, max_depth=s.depth, workspace=self.ws_acc,
                        out=self.acc_out)
        self.round += 1

    def mean_accept_len(self, rounds=32):
        """Mean accept length per request over `rounds` further rounds (each round draws its
        own Gumbel noise at T > 0; greedy rounds repeat)."""
        import torch
        hist = torch.empty((rounds, self.B), dtype=torch.int32, device=self.acc_out["accept_len"].device)
        for r in range(rounds):
            self.step()
            hist[r].copy_(self.acc_out["accept_len"])
        return float(hist.float().mean().item())


def recorded(name: str, field: str):
    """A figure stored under profiles/<name>.txt by profsum (rocprofv3 counters), or None if
    it is missing or was measured on a different source of the kernel."""
    from speculative_decoding_round_amd import profsum
    path = os.path.join(ROOT, "profiles", f"{name}.txt")
    if not os.path.exists(path):
        return None
    kv = dict(line.split(": ", 1) for line in open(path).read().splitlines() if ": " in line)
    if kv.get("source_sha256_16") != profsum.source_hash(profsum.sources_for(kv.get("kernel", ""))):
        return None
    return int(kv[field]) if field in kv else None


def recorded_traffic(workload: str):
    """HBM bytes per LM-head launch measured by rocprofv3 counters (profiles/)."""
    return recorded(f"gemm_lm_head_{workload}_traffic", "traffic_bytes_per_launch")


# counters stored per op (profiles/<name>.txt): HBM traffic per launch, VALU instructions
OP_PROFILES = {"attn_longctx": "tree_attention_longctx_traffic", "merge": "lse_merge_longctx_training_traffic",
               "accept_greedy": "accept_scan_llama8b_greedy_traffic"}
VALU_PROFILE = {"accept_t07": "accept_scan_llama70b_t07_valu"}
# VALU lane-instructions per second at the published fp32 vector peak (157.3 TFLOP/s, two
# flops per FMA lane-instruction): 256 CUs x 128 lanes x 2.4 GHz.  Quarter-rate instructions
# (64-bit integer multiply-add, reciprocal, the division helpers) take four issue slots, so a
# mix with them stays below this.
VALU_PEAK_LANE_INSTR = 157.3e12 / 2


def lm_head_bytes(shape, M):
    """Algorithmic HBM bytes of one LM-head launch: weights once, the M input rows, the M
    logit rows written in fp32."""
    es = 4 if shape.dtype == "f32" else 2
    return shape.V * shape.d * es + M * shape.d * es + M * shape.V * 4


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(rnd: Round, repeats: int = 3):
    """Time the oracle (as written, untuned) on a bounded sample of the same workload: the
    whole draft + verify round of request 0 alone (its prefix, the same drafter shapes, tree
    budget, verify splits and acceptance rule), median of `repeats` runs on the host cores,
    then one run on one core.  Scaled to verified tree tokens per second."""
    import numpy as np
    import torch
    from oracle import eagle3_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    s = rnd.shape
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    w = {k: v.cpu() for k, v in rnd.w.items()}
    di = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in rnd.di.items()}
    drafter = O.Drafter(w, s.Hq, s.Hkv, s.Dh)                 # fp64 upcast: not timed
    n1, P = rnd.n1, rnd.prefix[0]
    vi = {k: rnd.vi[k][:n1].cpu() for k in ("q", "k_tree", "v_tree", "logits")}
    vi["kpre"] = rnd.vi["kpre"][:P].cpu()
    vi["vpre"] = rnd.vi["vpre"][:P].cpu()
    S = rnd.S

    def one_round():
        t0 = time.perf_counter()
        res = O.draft_round(drafter, s.depth, s.topk, s.width, s.n_nodes, di["h_low"][:1], di["h_mid"][:1],
                            di["h_high"][:1], di["root_tok"][:1], di["kpre"][:P], di["vpre"][:P], [P])[0]
        n = len(res["parents"])
        parents = res["parents"] + [0] * (n1 - n)
        tokens = res["tokens"] + [0] * (n1 - n)
        cu, cup = [0, n1], [0, P]
        mask, _, _, _ = O.build_tree_mask(parents, cu, cup)
        o_parts, l_parts = [], []
        for sp in range(S + 1):
            def filt(b, Pb, sp=sp):
                keep = np.zeros(Pb, dtype=bool)
                if sp < S:
                    ch = (-(-Pb // S) + 127) // 128 * 128
                    keep[min(Pb, sp * ch):min(Pb, sp * ch + ch)] = True
                return keep, np.full(n1, sp == S)
            o, l = O.tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], cu, mask, vi["kpre"], vi["vpre"],
                                    cup, rnd.scale, key_filter=filt)
            o_parts.append(o.reshape(-1, s.Dh))
            l_parts.append(l.reshape(-1))
        O.lse_merge(np.stack(o_parts), np.stack(l_parts))
        O.accept(cu, tokens, parents, vi["logits"], s.temperature, 20260101, 0, s.depth)
        return time.perf_counter() - t0, n - 1

    times = []
    for _ in range(repeats):
        dt, verified = one_round()
        times.append(dt)
    med = float(np.median(times))
    out = {"value": verified / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"request 0 of the workload alone: one draft + verify round ({verified} verified tree "
                     f"tokens, prefix {P}), float64 numpy oracle, median of {repeats} runs "
                     f"({', '.join(f'{t:.2f}' for t in times)} s)",
           "seconds_median": round(med, 3), "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
           "affinity_cpus": len(os.sched_getaffinity(0))}
    with threadpool_limits(limits=1):
        dt1, v1 = one_round()
    out["single_core"] = {"value": v1 / dt1, "seconds": round(dt1, 2), "cores": 1}
    return out


# ---------------------------------------------------------------------------------------
# Per-op rooflines.  Each op is one library call on the shapes of the other workloads,
# timed by the library's HIP event pair on the launch stream (eagle3_profile_*), over
# `reps` launches that cycle through enough input copies that the reads miss the 256 MB
# Infinity Cache.  `bytes` / `flops` are algorithmic: what the method itself must read and
# write (or multiply-add), never the split partials the kernels add.
# ---------------------------------------------------------------------------------------
MFMA_BF16_PEAK_TFLOPS = 2500.0
INFINITY_CACHE_BYTES = 256 << 20


def _copies(nbytes: int, want: int = 2) -> int:
    """Enough rotating copies of an nbytes working set to exceed the Infinity Cache twice."""
    return max(want, -(-2 * INFINITY_CACHE_BYTES // max(nbytes, 1)))


def _time_b2b(fn, reps: int) -> float:
    """Average device time (us) of one call of fn, over reps calls run back to back: a device
    spin long enough for the host to enqueue every call holds the stream, one event pair on
    the launch stream brackets the calls, so the time is the kernels' own (plus the
    dispatch gaps between them), not the host's enqueue latency or per-launch events."""
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)          # several ms at the shader clock
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def _entry(op, workload, kernel, us, bound, bytes_=None, flops=None, **extra):
    e = {"op": op, "workload": workload, "kernel": kernel, "bound": bound,
         "avg_launch_us": round(us, 2)}
    if bytes_ is not None:
        gbs = bytes_ / (us * 1e-6) / 1e9
        e.update({"algorithmic_bytes": int(bytes_), "achieved_gbs": round(gbs, 1),
                  "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    if flops is not None:
        tfs = flops / (us * 1e-6) / 1e12
        e.update({"algorithmic_flops": int(flops), "achieved_tflops": round(tfs, 1),
                  "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)})
    if bound == "hbm":
        e.update({"achieved": e["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": e["hbm_frac"]})
    elif bound == "mfma":
        e.update({"achieved": e["achieved_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": e["mfma_frac"]})
    e.update(extra)
    return e


def _tree_depths(parents):
    dep = []
    for p in parents:
        dep.append(0 if p < 0 else dep[p] + 1)
    return dep


def attention_op(capi, synth, shape, trees, prefix, bound, reps=20, seed=500):
    """Verify tree attention (the partial-producing kernel alone) on one workload."""
    import numpy as np
    import torch
    dev = "cuda:0"
    vi = synth.verify_inputs(shape, trees, prefix, seed=seed, device=dev, with_logits=False)
    maxn = max(len(t) for t in trees)
    mk = capi.eagle3_build_tree_mask(vi["cu_nodes"], vi["parents"], vi["cu_prefix"], max_nodes=maxn)
    es = 2
    kv_bytes = sum(prefix) * shape.Hkv * shape.Dh * 2 * es
    ncopy = _copies(kv_bytes)
    kp = [vi["kpre"]] + [synth.normal(tuple(vi["kpre"].shape), 1.0, seed + 10 + c, vi["kpre"].dtype, dev)
                         for c in range(ncopy - 1)]
    vp = [vi["vpre"]] + [synth.normal(tuple(vi["vpre"].shape), 1.0, seed + 50 + c, vi["vpre"].dtype, dev)
                         for c in range(ncopy - 1)]
    S = capi.eagle3_tree_attention_num_splits(len(trees), shape.Hq, shape.Hkv, maxn, max(prefix), 0)
    T = vi["T"]
    part = {"o_part": torch.empty((S + 1, T, shape.Hq, shape.Dh), dtype=torch.float32, device=dev),
            "lse_part": torch.empty((S + 1, T, shape.Hq), dtype=torch.float32, device=dev)}
    scale = float(1.0 / math.sqrt(shape.Dh))

    def run(i):
        capi.eagle3_tree_attention(vi["q"], vi["k_tree"], vi["v_tree"], vi["cu_nodes"], maxn, mk["mask"],
                                   kp[i % ncopy], vp[i % ncopy], vi["cu_prefix"], max(prefix), scale,
                                   out=part)
    us = _time_b2b(run, reps)
    n_nodes = [len(t) for t in trees]
    tree_bytes = T * shape.Hkv * shape.Dh * 2 * es
    q_bytes = T * shape.Hq * shape.Dh * es
    out_bytes = T * shape.Hq * (shape.Dh * es + 4)
    flops = 0
    for t, P in zip(trees, prefix):
        anc = [d + 1 for d in _tree_depths(t)]          # ancestors-or-self of each node
        flops += shape.Hq * 4 * shape.Dh * (len(t) * P + sum(anc))
    rows_per_kv = max(n_nodes) * shape.Hq // shape.Hkv
    return _entry("tree_attention", shape.name, "k_tree_attn_dma", us, bound,
                  bytes_=kv_bytes + tree_bytes + q_bytes + out_bytes, flops=flops,
                  splits=S, rows_per_kv_head=rows_per_kv, prefix_tokens=sum(prefix),
                  rotating_copies=ncopy)


OP_KEYS = ("attn_longctx", "attn_batch16", "attn_70b", "attn_8b", "merge", "accept_greedy", "accept_t07",
           "accept_sampled", "draft_sampled", "gemm_sweep", "catchup", "commit", "tree_budgets", "usp")


def sampled_accept_ops(capi, synth, reps):
    """Acceptance of sampled candidates (eagle3_accept_sampled) at the 8B shape (one random
    61-node tree of depth 6) and the 70B shape (four), V = 128256 bf16 target and draft logits,
    at most 10 children tested per node, T = 1.  Draft rows are hot-boosted N(0, 1) rows whose
    children are hot tokens; target rows are the draft rows plus N(0, 1) (about half the
    candidates kept).  Algorithmic bytes: every target row and every draft row read once."""
    import numpy as np
    import torch
    dev = "cuda:0"
    out = []
    for key, sh, B in (("accept_sampled_8b", synth.LLAMA8B, 1), ("accept_sampled_70b", synth.LLAMA70B, 4)):
        trees = [synth.random_tree(61, sh.depth, 4400 + i) for i in range(B)]
        d = synth.sampled_tree_inputs(trees, sh.V, seed=970, device=dev, target_noise=1.0)
        T, V, R = d["T"], sh.V, d["draft_logits"].shape[0]
        nbytes = (T + R) * V * 2
        ncopy = _copies(nbytes)
        zs = [d["logits"]] + [d["logits"] + synth.normal((T, V), 0.05, 980 + c, torch.bfloat16, dev)
                              for c in range(ncopy - 1)]
        qs = [d["draft_logits"]] + [d["draft_logits"] + synth.normal((R, V), 0.05, 990 + c, torch.bfloat16, dev)
                                    for c in range(ncopy - 1)]
        maxc = 10
        ws = torch.empty(capi.lib().eagle3_accept_sampled_workspace_size(T, V, maxc), dtype=torch.uint8, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        ao = {"accept_len": torch.empty((B,), **i32), "path": torch.empty((B, sh.depth + 1), **i32),
              "out_tokens": torch.empty((B, sh.depth + 1), **i32), "bonus": torch.empty((B,), **i32)}

        def run(i, d=d, zs=zs, qs=qs, ws=ws, ao=ao, sh=sh):
            capi.eagle3_accept_sampled(d["cu_nodes"], d["tokens"], d["parents"], zs[i % len(zs)],
                                       qs[i % len(qs)], d["draft_row"], 1.0, 7, i, sh.depth, maxc,
                                       workspace=ws, out=ao)
        us = _time_b2b(run, reps)
        lens = []
        for i in range(16):
            run(i)
            lens += ao["accept_len"].cpu().tolist()
        out.append(dict(key=key, **_entry("accept (sampled candidates, T=1)",
                                          f"{sh.name}: {T} nodes ({R} with children) x {V} logits",
                                          "k_samp_clear + k_samp_stats + k_samp_npass x 9 + k_samp_walk + k_samp_draw",
                                          us, "latency", bytes_=nbytes, rotating_copies=ncopy, launches=13,
                                          mean_accept_len=round(float(np.mean(lens)), 2))))
        del zs, qs
    return out


def sampled_draft_ops(steps=10):
    """The draft-tree round at the 8B shape (D = 6, K = W = 10, N = 60) with top-K children and
    with sampled children (eagle3_draft_expand_sampled, T = 1: Gumbel noise on every logit of
    the LM head, and every slot's logits kept for the verifier).  Both stream the fusion weights
    once and the layer and LM-head weights at every depth step (HBM-bound)."""
    import torch
    from speculative_decoding_round_amd import capi, synth
    dev = "cuda:0"
    shape = synth.LLAMA8B
    rnd = Round(shape, dev)
    di = rnd.di
    S = 1 + (shape.depth - 1) * shape.width
    so = dict(rnd.draft_out)
    so["slot_logits"] = torch.empty((rnd.B, S, shape.V), dtype=torch.float32, device=dev)
    so["draft_row"] = torch.empty((rnd.B, rnd.n1), dtype=torch.int32, device=dev)

    def det(i):
        capi.eagle3_draft_expand(rnd.drafter, rnd.tree, di["h_low"], di["h_mid"], di["h_high"], di["root_tok"],
                                 di["kpre"], di["vpre"], di["cu_prefix"], rnd.max_prefix, workspace=rnd.ws_draft,
                                 out=rnd.draft_out)

    def smp(i):
        capi.eagle3_draft_expand_sampled(rnd.drafter, rnd.tree, 1.0, 7, i, di["h_low"], di["h_mid"], di["h_high"],
                                         di["root_tok"], di["kpre"], di["vpre"], di["cu_prefix"], rnd.max_prefix,
                                         workspace=rnd.ws_draft, out=so)
    d, F, V, D = shape.d, shape.F, shape.V, shape.depth
    nqkv = (shape.Hq + 2 * shape.Hkv) * shape.Dh
    wbytes = 2 * (3 * d * d + D * (2 * d * nqkv + shape.Hq * shape.Dh * d + 3 * d * F + V * d))
    out = []
    for name, fn in (("draft round (top-K children)", det), ("draft round (sampled children, T=1)", smp)):
        us = _time_b2b(fn, steps)
        out.append(dict(key="draft_sampled", **_entry(name, "llama8b_bf16 D=6 K=10 W=10 N=60", "whole draft round",
                                                      us, "hbm", bytes_=wbytes)))
    del rnd, so
    torch.cuda.empty_cache()
    return out


def round_distribution(rnd: "Round", n: int) -> dict:
    """Per-round device times over n more rounds (an event between consecutive rounds on the
    launch stream): median, p10, p90 in ms."""
    import numpy as np
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(n):
        rnd.step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n)])
    return {"rounds": n, "median": round(float(np.median(t)), 4), "p10": round(float(np.percentile(t, 10)), 4),
            "p90": round(float(np.percentile(t, 90)), 4)}


def measured_ceilings() -> dict:
    """What this part reaches outside the library, for scale: a 1 GiB device-to-device copy
    (torch's copy kernel; read + write bytes over time) and an 8192^3 bf16 matrix product
    (torch.matmul, i.e. the vendor GEMM library) against the published peaks."""
    import torch
    dev = "cuda:0"
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    us_copy = _time_b2b(lambda i: dst.copy_(src), 10)
    del src, dst
    m = 8192
    a = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    b = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    c = torch.empty((m, m), dtype=torch.bfloat16, device=dev)
    us_mm = _time_b2b(lambda i: torch.matmul(a, b, out=c), 10)
    del a, b, c
    torch.cuda.empty_cache()
    copy_gbs = 2 * n / (us_copy * 1e-6) / 1e9
    tflops = 2 * m ** 3 / (us_mm * 1e-6) / 1e12
    return {"copy_1gib_gbs": round(copy_gbs, 1), "copy_frac": round(copy_gbs / HBM_PEAK_GBS, 4),
            "gemm_bf16_8192_tflops": round(tflops, 1), "gemm_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}


def gemm_sweep(capi, synth, reps):
    """The drafter projections' GEMM (eagle3_linear) over the number of rows: at the QKV
    shape (N = 6144, K = 8192) for M = 1 .. 8192, at M = 2048 (a prompt's worth of rows) for
    the MLP-down and LM-head shapes, and at the depth-step rows of the 70B-shaped (40) and
    batch-16 (160) rounds.  Up to 160 rows are bound by streaming W (HBM), many rows by the
    matrix cores (bf16 MFMA)."""
    import torch
    dev = "cuda:0"
    out = []
    cases = [(m, 6144, 8192, "QKV") for m in (1, 10, 160, 1024, 2048, 8192)]
    cases += [(2048, 4096, 12288, "feature fusion"), (2048, 4096, 14336, "MLP down"),
              (2048, 128256, 4096, "LM head")]
    # the depth steps' rows of the 70B-shaped (4 x 10 = 40) and batch-16 (16 x 10 = 160)
    # rounds at their projections' shapes (gate/up as a plain product of both halves)
    cases += [(40, 10240, 16384, "70B QKV"), (40, 57344, 8192, "70B gate/up"), (40, 8192, 28672, "70B MLP down"),
              (40, 8192, 8192, "70B O"), (40, 128256, 8192, "70B LM head"),
              (160, 28672, 4096, "8B gate/up"), (160, 4096, 14336, "8B MLP down"), (160, 128256, 4096, "8B LM head")]
    for M, N, K, name in cases:
        wbytes = N * K * 2
        ncopy = _copies(wbytes) if M <= 160 else 1
        ws = [synth.normal((N, K), K ** -0.5, 70 + c, torch.bfloat16, dev) for c in range(ncopy)]
        x = synth.normal((M, K), 1.0, 71, torch.bfloat16, dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        need = capi.lib().eagle3_linear_workspace_size(M, N, K, capi.EAGLE3_BF16)
        wk = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

        def run(i, ws=ws, x=x, y=y, wk=wk):
            capi.eagle3_linear(x, ws[i % len(ws)], out=y, workspace=wk)
        us = _time_b2b(run, reps if M <= 2048 else max(4, reps // 4))
        bound = "hbm" if M <= 160 else "mfma"
        e = _entry(f"linear ({name})", f"M={M} N={N} K={K} bf16", "k_gemm_ring" if M <= 32 else
                   ("k_gemm_wide" if M <= 160 else "k_gemm_tile"), us, bound,
                   bytes_=wbytes + M * K * 2 + M * N * 4, flops=2 * M * N * K)
        out.append(dict(key="gemm_sweep", **e))
        del ws, x, y, wk
    return out


def catchup_ops(capi, synth, reps):
    """The step after acceptance at the 8B shapes: drafter catch-up over a 2048-token prompt
    (fusion 12288 -> 4096 and the K/V rows of the QKV projection, 8192 -> 2048, on the matrix
    cores) and over one round's committed path (accept_len + 1 = 7 rows, streaming the same
    weights), and the commit of a 7-node path (8 KV heads x 128, bf16)."""
    import torch
    dev = "cuda:0"
    shape = synth.LLAMA8B
    d, Hkv, Dh = shape.d, shape.Hkv, shape.Dh
    nkv = 2 * Hkv * Dh
    out = []
    w = synth.drafter_weights(shape, seed=81, device=dev)
    wbytes = (3 * d * d + 2 * d * nkv) * 2
    # rotating copies of the two weights the catch-up streams, so the 7-row case reads HBM
    drs, keep = [], []
    for c in range(_copies(wbytes)):
        wc = dict(w)
        if c:
            wc["w_fuse"] = w["w_fuse"].clone()
            wc["w_qkv"] = w["w_qkv"].clone()
            keep.append(wc)
        drs.append(capi.make_drafter(wc, shape.Hq, shape.Hkv, shape.Dh))
    for n, bound in ((2048, "mfma"), (7, "hbm")):
        h = [synth.normal((n, d), 1.0, 90 + i, torch.bfloat16, dev) for i in range(3)]
        tok = synth.uniform_int(n, shape.V, 93, dev).to(torch.int32)
        pos = torch.arange(n, device=dev, dtype=torch.int32)
        dst = torch.arange(n, device=dev, dtype=torch.int32)
        kc = torch.empty((n, Hkv, Dh), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        g = torch.empty((n, d), dtype=torch.float32, device=dev)
        ws = torch.empty(max(capi.eagle3_drafter_catchup_workspace_size(drs[0], n), 256), dtype=torch.uint8,
                         device=dev)

        def run(i, h=h, tok=tok, pos=pos, dst=dst, kc=kc, vc=vc, g=g, ws=ws):
            capi.eagle3_drafter_catchup(drs[i % len(drs)], tok, pos, *h, dst, kc, vc, g_out=g, workspace=ws)
        us = _time_b2b(run, reps)
        flops = 2 * n * (3 * d * d + 2 * d * nkv)
        byts = wbytes + n * (3 * d * 2 + 4 * d + 2 * nkv) + n * d * 2
        e = _entry("drafter catch-up", f"8B shapes, {n} committed positions",
                   "k_gemm_tile + prep + rope" if n > 160 else "k_gemm_ring + prep + rope", us, bound,
                   bytes_=byts, flops=flops)
        out.append(dict(key="catchup", **e))
        del h, kc, vc, g, ws
    del w, keep, drs
    return out


def commit_ops(capi, synth, reps):
    import torch
    dev = "cuda:0"
    T, Hkv, Dh, D = 61, 8, 128, 6
    k_tree = synth.normal((T, Hkv, Dh), 1.0, 1, torch.bfloat16, dev)
    v_tree = synth.normal((T, Hkv, Dh), 1.0, 2, torch.bfloat16, dev)
    kc = torch.zeros((4096, Hkv, Dh), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    path = torch.tensor([[0, 1, 11, 21, 31, 41, 51]], dtype=torch.int32, device=dev)
    acc = torch.tensor([D], dtype=torch.int32, device=dev)
    dst = torch.tensor([2048], dtype=torch.int32, device=dev)

    def run(i):
        capi.eagle3_commit_kv(cu, path, acc, k_tree, v_tree, dst, kc, vc)
    us = _time_b2b(run, reps)
    byts = 2 * 2 * (D + 1) * Hkv * Dh * 2
    return [dict(key="commit", **_entry("commit accepted KV", "7-node path, 8 KV heads x 128, bf16",
                                        "k_commit_kv", us, "latency", bytes_=byts))]


def tree_budget_ops(steps=10):
    """Whole rounds at the 8B shapes for other tree budgets: EAGLE-2's depth 6 and EAGLE-3's
    depth 8 at 60, 50 and 48 kept nodes (K = W = 10).  The round streams the fusion weights
    once and the layer and LM-head weights at every depth step (HBM-bound)."""
    import torch
    from speculative_decoding_round_amd import synth
    dev = "cuda:0"
    out = []
    for D, N in ((6, 60), (8, 60), (8, 50), (8, 48)):
        shape = synth.scaled(synth.LLAMA8B, depth=D, n_nodes=N)
        rnd = Round(shape, dev)
        for _ in range(3):
            rnd.step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            rnd.step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        n_ver = int(rnd.draft_out["n_nodes"].sum().item()) - rnd.B
        d, F, V = shape.d, shape.F, shape.V
        nqkv = (shape.Hq + 2 * shape.Hkv) * shape.Dh
        wbytes = 2 * (3 * d * d + D * (2 * d * nqkv + shape.Hq * shape.Dh * d + 3 * d * F + V * d))
        e = _entry("draft + verify round", f"llama8b_bf16 D={D} K=10 W=10 N={N}", "whole round", ms * 1e3,
                   "hbm", bytes_=wbytes, verified_tokens_per_s=round(n_ver / (ms / 1e3), 1),
                   verified_nodes=n_ver)
        out.append(dict(key="tree_budgets", **e))
        del rnd
        torch.cuda.empty_cache()
    return out


def usp_ops(capi, synth, reps):
    """The long-context shape's training form at 65536 positions, 32 query / 8 KV heads of
    128, bf16: the causal main attention (4 * Dh flops per (row, visible key): 35.2 TFLOP,
    matrix-core bound) and the 7-step per-position branch (reads q and the branch K/V,
    writes the fp32 output: HBM-bound).  The fusion is the `merge` op at the same scale."""
    import torch
    dev = "cuda:0"
    L, Hq, Hkv, Dh, steps = 65536, 32, 8, 128, 7
    q = synth.normal((L, Hq, Dh), 1.0, 1, torch.bfloat16, dev)
    k = synth.normal((L, Hkv, Dh), 1.0, 2, torch.bfloat16, dev)
    v = synth.normal((L, Hkv, Dh), 1.0, 3, torch.bfloat16, dev)
    o = torch.empty((L, Hq, Dh), dtype=torch.float32, device=dev)
    lse = torch.empty((L, Hq), dtype=torch.float32, device=dev)
    sc = Dh ** -0.5
    us = _time_b2b(lambda i: capi.eagle3_causal_attention(q, k, v, sc, o=o, lse=lse), max(2, reps // 5))
    flops = 4 * Dh * Hq * L * (L + 1) // 2
    out = [dict(key="usp", **_entry("causal attention (main)", f"L={L}, {Hq}/{Hkv} heads x {Dh}, bf16",
                                    "k_tree_attn_dma (causal)", us, "mfma", flops=flops))]
    del k, v
    kb = synth.normal((steps, L, Hkv, Dh), 1.0, 4, torch.bfloat16, dev)
    vb = synth.normal((steps, L, Hkv, Dh), 1.0, 5, torch.bfloat16, dev)
    us = _time_b2b(lambda i: capi.eagle3_branch_attention(q, kb, vb, sc, o=o, lse=lse), reps)
    byts = L * Hq * Dh * 2 + 2 * steps * L * Hkv * Dh * 2 + L * Hq * (Dh + 1) * 4
    out.append(dict(key="usp", **_entry("branch attention", f"L={L}, {steps} steps, {Hq}/{Hkv} heads x {Dh}",
                                        "k_branch_attn", us, "hbm", bytes_=byts)))
    return out


def op_rooflines(reps=20, keys=OP_KEYS):
    import numpy as np
    import torch
    from speculative_decoding_round_amd import capi, synth
    dev = "cuda:0"
    ops = []
    if "attn_longctx" in keys:
        # long-context branch: 7 chain queries over a 65536-token prefix (HBM-bound)
        sh = synth.LONGCTX
        e = attention_op(capi, synth, sh, [synth.chain_tree(sh.branch)], [65536], "hbm", reps)
        ops.append(dict(key="attn_longctx", **e))
    if "attn_batch16" in keys:
        # batched serving: 16 random trees of <= 48 nodes, prefixes uniform in [512, 4096] (HBM-bound)
        sh = synth.BATCH16
        prefix = synth.prefix_lengths(sh, seed=31)
        rng = np.random.default_rng(31)
        trees = [synth.random_tree(int(rng.integers(1, sh.verify_max_nodes + 1)), sh.verify_max_depth, 3100 + i)
                 for i in range(sh.B)]
        ops.append(dict(key="attn_batch16", **attention_op(capi, synth, sh, trees, prefix, "hbm", reps)))
    if "attn_70b" in keys:
        # 70B-shaped verify: 4 x (root + 60 nodes), 488 query rows per KV head (MFMA-bound)
        sh = synth.LLAMA70B
        trees = [synth.random_tree(61, sh.depth, 4100 + i) for i in range(sh.B)]
        ops.append(dict(key="attn_70b", **attention_op(capi, synth, sh, trees, synth.prefix_lengths(sh, 41),
                                                        "mfma", reps)))
    if "attn_8b" in keys:
        # 8B-shaped verify (60-node tree over 2048 keys): latency-sized, reported for both bounds
        sh = synth.LLAMA8B
        ops.append(dict(key="attn_8b", **attention_op(capi, synth, sh, [synth.random_tree(61, sh.depth, 4200)],
                                                       [2048], "hbm", reps)))
    if "merge" in keys:
        # LSE merge at the long-context training scale: two partials of 65536 x 32 rows
        rows, Dh = 65536 * 32, 128
        o_part = synth.normal((2, rows, Dh), 1.0, 900, torch.float32, dev)
        lse_part = synth.normal((2, rows), 1.0, 901, torch.float32, dev)
        mo = {"o": torch.empty((rows, Dh), dtype=torch.bfloat16, device=dev),
              "lse": torch.empty((rows,), dtype=torch.float32, device=dev)}
        us = _time_b2b(lambda i: capi.eagle3_lse_merge(o_part, lse_part, out=mo), reps)
        ops.append(dict(key="merge", **_entry("lse_merge", "2 partials x 65536 positions x 32 heads x 128 "
                                              "(fp32 -> bf16)", "k_lse_merge_rows", us, "hbm",
                                              bytes_=2 * rows * (Dh + 1) * 4 + rows * (Dh * 2 + 4))))
        del o_part, lse_part, mo
    # acceptance: greedy at the 8B shape (61 nodes x 128256 bf16 logits), T = 0.7 at the 70B
    # shape (4 x 61 nodes)
    for key, sh, B, temp in (("accept_greedy", synth.LLAMA8B, 1, 0.0), ("accept_t07", synth.LLAMA70B, 4, 0.7)):
        if key not in keys:
            continue
        trees = [synth.random_tree(61, sh.depth, 4300 + i) for i in range(B)]
        vi = synth.verify_inputs(sh, trees, [0] * B, seed=950, device=dev, with_logits=False)
        mk = capi.eagle3_build_tree_mask(vi["cu_nodes"], vi["parents"], None, max_nodes=61)
        T, V = vi["T"], sh.V
        lbytes = T * V * 2
        ncopy = _copies(lbytes)
        logits = [synth.normal((T, V), 1.0, 960 + c, torch.bfloat16, dev) for c in range(ncopy)]
        ws = torch.empty(capi.lib().eagle3_accept_workspace_size(T, V), dtype=torch.uint8, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        ao = {"accept_len": torch.empty((B,), **i32), "path": torch.empty((B, sh.depth + 1), **i32),
              "out_tokens": torch.empty((B, sh.depth + 1), **i32), "bonus": torch.empty((B,), **i32)}

        def run(i, vi=vi, mk=mk, logits=logits, ws=ws, ao=ao, temp=temp, sh=sh):
            capi.eagle3_accept(vi["cu_nodes"], vi["tokens"], vi["parents"], mk["mask"], logits[i % len(logits)],
                               temp, seed=7, round=i, max_depth=sh.depth, workspace=ws, out=ao)
        us = _time_b2b(run, reps)
        name = "greedy" if temp == 0 else f"T={temp}"
        ops.append(dict(key=key, **_entry(f"accept ({name})", f"{sh.name}: {T} nodes x {V} logits",
                                          "k_accept_scan + k_accept_path", us, "hbm", bytes_=lbytes,
                                          rotating_copies=ncopy,
                                          logits_per_s=round(T * V / (us * 1e-6) / 1e9, 2))))
        del logits
    if "accept_sampled" in keys:
        ops += sampled_accept_ops(capi, synth, reps)
    if "draft_sampled" in keys:
        ops += sampled_draft_ops()
    if "gemm_sweep" in keys:
        ops += gemm_sweep(capi, synth, reps)
    if "catchup" in keys:
        ops += catchup_ops(capi, synth, reps)
    if "commit" in keys:
        ops += commit_ops(capi, synth, reps)
    if "tree_budgets" in keys:
        ops += tree_budget_ops()
    if "usp" in keys:
        ops += usp_ops(capi, synth, reps)
    torch.cuda.empty_cache()
    for o in ops:
        if o["key"] in OP_PROFILES:
            o["traffic"] = recorded(OP_PROFILES[o["key"]], "traffic_bytes_per_launch")
        if o["key"] in VALU_PROFILE:
            n = recorded(VALU_PROFILE[o["key"]], "sq_insts_valu_per_launch")
            if n is not None:
                # the scan is bound by its arithmetic (Philox + two float32 logs per logit); the
                # time covers the whole call (scan and path kernels), the count the scan alone
                ach = n * 64 / (o["avg_launch_us"] * 1e-6)
                o.update({"bound": "alu", "achieved": round(ach / 1e12, 2), "peak": round(VALU_PEAK_LANE_INSTR / 1e12, 2),
                          "unit": "T VALU lane-instr/s", "frac": round(ach / VALU_PEAK_LANE_INSTR, 4),
                          "valu_wave_instr_per_launch": n})
    return ops


def gemm_rooflines(rnd: "Round", steps: int):
    """Per-projection GEMM times inside the round (every launch timed by its event pair)."""
    import torch
    capi, s = rnd.capi, rnd.shape
    capi.eagle3_profile_reset()
    capi.eagle3_profile_enable(True)
    for _ in range(steps):
        rnd.step()
    torch.cuda.synchronize()
    capi.eagle3_profile_enable(False)
    es = 2 if s.dtype == "bf16" else 4
    d, F, V = s.d, s.F, s.V
    nqkv = (s.Hq + 2 * s.Hkv) * s.Dh
    rows = [s.B] + [s.B * s.width] * (s.depth - 1)
    avg_m = sum(rows) / len(rows)
    # weights once + activations in (dtype) + outputs (fp32 partial sums once, or dtype for
    # the SiLU product), at the average row count of the round's steps
    spec = {
        "gemm_fuse": (d * 3 * d, s.B, 3 * d, d, 4),
        "gemm_qkv": (nqkv * 2 * d, avg_m, 2 * d, nqkv, 4),
        "gemm_o": (d * s.Hq * s.Dh, avg_m, s.Hq * s.Dh, d, 4),
        "gemm_gate_up": (2 * F * d, avg_m, d, F, es),
        "gemm_down": (d * F, avg_m, F, d, 4),
        "gemm_lm_head": (V * d, s.B * s.width, d, V, 4),       # depth steps: B * W rows
        "gemm_lm_head_root": (V * d, s.B, d, V, 4),            # the root step: B rows
    }
    def kernel_for(ms_rows):
        """The bf16 weight-streaming kernels that run these row counts: the LDS ring up to 32
        rows, the wide kernel up to 160."""
        names = []
        for r in ms_rows:
            k = "k_gemm_ring" if r <= 32 else "k_gemm_wide"
            if k not in names:
                names.append(k)
        return " / ".join(names)

    root, deep = [s.B], [s.B * s.width]
    launched = {"gemm_fuse": root, "gemm_lm_head": deep, "gemm_lm_head_root": root}
    out = []
    for tag, (wn, m, kin, nout, oes) in spec.items():
        ms, n = capi.eagle3_profile_read(tag)
        if n == 0:
            continue
        us = ms / n * 1e3
        b = wn * es + m * kin * es + m * nout * oes
        out.append(_entry(tag, s.name, kernel_for(launched.get(tag, root + deep)), us, "hbm", bytes_=b,
                          launches=n))
    capi.eagle3_profile_reset()
    return out


def round_summary(shape, steps, warmup, dev):
    """A whole round of another workload, as extra fields of the line: device time per round
    over `steps` rounds (HIP events), verified tree tokens per second, mean accept length."""
    import torch
    rnd = Round(shape, dev)
    for _ in range(warmup):
        rnd.step()
    torch.cuda.synchronize()
    n_ver = int(rnd.draft_out["n_nodes"].sum().item()) - rnd.B
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        rnd.step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    out = {"workload": workload_name(rnd), "value": round(n_ver / (ms / 1e3), 2), "unit": "tokens/s",
           "ms_per_step": round(ms, 4), "verified_nodes_per_round": n_ver, "steps": steps,
           "mean_accept_len": round(rnd.mean_accept_len(), 3), "temperature": shape.temperature,
           "rotating_input_copies": rnd.ncopy}
    del rnd
    torch.cuda.empty_cache()
    return out


def workload_name(rnd) -> str:
    s = rnd.shape
    pre = f"prefix {rnd.max_prefix}" if len(set(rnd.prefix)) == 1 else \
        f"prefixes {min(rnd.prefix)}..{max(rnd.prefix)}"
    return (f"{s.name}: batch {s.B}, draft tree D={s.depth} K={s.topk} W={s.width} N={s.n_nodes}, "
            f"verify over {pre}, {'greedy' if s.temperature == 0 else f'T={s.temperature}'} acceptance")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from speculative_decoding_round_amd import capi, synth
    dev = "cuda:0"
    keys = tuple(k for k in args.ops.split(",") if k)
    if args.only_ops:
        out = {"ops": op_rooflines(keys=keys)}
        if args.copy_calibration_mb > 0:
            n = args.copy_calibration_mb << 20
            src = torch.empty(n, dtype=torch.uint8, device=dev)
            dst = torch.empty(n, dtype=torch.uint8, device=dev)
            dst.copy_(src)
            torch.cuda.synchronize()
            out["copy_calibration_bytes"] = n
        print(json.dumps(out), flush=True)
        return
    shapes = {"llama8b": synth.LLAMA8B, "batch16": synth.BATCH16, "llama70b": synth.LLAMA70B,
              "tiny": synth.TINY}
    shape = shapes[args.workload]
    rnd = Round(shape, dev)
    for _ in range(args.warmup):
        rnd.step()
    torch.cuda.synchronize()
    n_verified = int(rnd.draft_out["n_nodes"].sum().item()) - rnd.B

    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def timed(kernel_events: bool):
        # kernel_events: the library records a HIP event pair on the launch stream around
        # every launch of args.kernel
        capi.eagle3_profile_reset()
        capi.eagle3_profile_enable(kernel_events, only_kernel=args.kernel)
        torch.cuda.synchronize()
        ev0.record(stream)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            rnd.step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        capi.eagle3_profile_enable(False)
        k_ms, k_n = capi.eagle3_profile_read(args.kernel)
        capi.eagle3_profile_reset()
        return ev0.elapsed_time(ev1) / args.steps, wall, k_ms, k_n

    # the throughput pass carries no per-kernel events; a second pass of the same K steps
    # times the roofline kernel's launches
    ms, wall, _, _ = timed(False)
    ms_ev, _, k_ms, k_n = timed(True)

    value = n_verified / (ms / 1e3)
    # the LM head of the depth steps (B * W rows; the root step's launch is tagged apart)
    lm_rows = shape.B * shape.width if args.kernel == "gemm_lm_head" else shape.B
    bytes_lm = lm_head_bytes(shape, lm_rows)
    k_avg_ms = k_ms / max(k_n, 1)
    achieved = bytes_lm / (k_avg_ms / 1e3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random-init drafter weights, Gaussian features and KV; target logits "
                "= draft logits + noise at the drafted nodes)",
        "config": {"workload": workload_name(rnd),
                   "batch": shape.B, "d": shape.d, "heads": [shape.Hq, shape.Hkv, shape.Dh],
                   "ffn": shape.F, "vocab": shape.V, "prefix": rnd.prefix if shape.B <= 4 else "ragged",
                   "verified_nodes_per_round": n_verified, "temperature": shape.temperature,
                   "target_logit_noise": shape.noise, "rotating_input_copies": rnd.ncopy,
                   "per_round_input_bytes": rnd.per_round_input_bytes},
        "roofline": {"kernel": f"{args.kernel} ({lm_rows} rows per launch)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(args.workload), "avg_launch_us": round(k_avg_ms * 1e3, 2),
                     "launches": k_n, "algorithmic_bytes_per_launch": int(bytes_lm)},
        "wall_s_timed": round(wall, 3),
        "ms_per_step_with_kernel_events": round(ms_ev, 4),
    }
    line["mean_accept_len"] = round(rnd.mean_accept_len(), 3)
    if not args.no_ops:
        line["gemms"] = gemm_rooflines(rnd, args.steps)
        line["round_ms"] = round_distribution(rnd, 100)
        line["ceilings"] = measured_ceilings()
    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(rnd)
    del rnd
    torch.cuda.empty_cache()
    if not args.no_other_rounds:
        line["other_rounds"] = [round_summary(shapes[w], args.steps, args.warmup, dev)
                                for w in ("llama8b", "batch16", "llama70b") if w != args.workload]
    if not args.no_ops:
        line["ops"] = op_rooflines(keys=keys)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
