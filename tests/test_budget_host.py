"""The library's speculative-budget controller (host code, no GPU) against the oracle's:
identical level sequences on random traces and on traces that walk the ladder, and
argument validation."""
import ctypes

import numpy as np
import pytest

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import capi

LEVELS = [(3, 4, 4, 16), (4, 8, 8, 32), (6, 10, 10, 60), (8, 10, 10, 60)]


def pair(**kw):
    p = dict(start=2, cooldown=8, window=16, low_frac=0.25, high_frac=0.5, max_cv=0.35,
             draft_share_max=0.75, verify_ms_max=1.0, revert_drop=0.05)
    p.update(kw)
    lib_c = capi.BudgetController(LEVELS, **p)
    ora = O.BudgetController(len(LEVELS), [l[0] for l in LEVELS], **p)
    return lib_c, ora


@pytest.mark.parametrize("seed", range(6))
def test_matches_oracle_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    kw = dict(start=int(rng.integers(0, 4)), cooldown=int(rng.integers(1, 12)),
              window=int(rng.integers(1, 40)), verify_ms_max=float(np.float32(rng.uniform(0.2, 2.0))))
    c, o = pair(**kw)
    for r in range(1500):
        # regimes that change every 100 rounds: acceptance level and spread, cost split
        reg = np.random.default_rng(seed * 1000 + r // 100)
        hi, spread = int(reg.integers(0, 9)), int(reg.integers(0, 3))
        a = int(np.clip(hi + rng.integers(-spread, spread + 1), 0, 8))
        d = np.float32(rng.uniform(0.05, 1.5) * reg.uniform(0.2, 2))
        v = np.float32(rng.uniform(0.05, 1.5))
        lc, t = c.update(a, d, v)
        lo = o.update(a, float(d), float(v))
        assert lc == lo, (seed, r)
        assert (t.depth, t.topk, t.width, t.n_nodes) == LEVELS[lc]


def test_walks_the_ladder_like_the_oracle():
    c, o = pair(start=0)
    seq_c, seq_o = [], []
    for r in range(300):
        L = c.state.level
        a = LEVELS[L][0] if r < 150 else 0          # full acceptance, then none
        lat = np.float32(0.2 + 0.05 * L)
        seq_c.append(c.update(a, lat, np.float32(0.3))[0])
        seq_o.append(o.update(a, float(lat), float(np.float32(0.3))))
    assert seq_c == seq_o
    assert max(seq_c) == 3 and seq_c[-1] == 0


def test_validation():
    lib = capi.lib()
    p = capi.Eagle3BudgetParams(n_levels=0, start_level=0, cooldown=1, window=4)
    s = capi.Eagle3BudgetState()
    assert lib.eagle3_budget_init(ctypes.byref(p), ctypes.byref(s)) == -1      # no levels
    p.n_levels = 2
    p.levels[0] = capi.Eagle3TreeCfg(depth=3, topk=2, width=2, n_nodes=6)
    p.levels[1] = capi.Eagle3TreeCfg(depth=0, topk=2, width=2, n_nodes=6)
    assert lib.eagle3_budget_init(ctypes.byref(p), ctypes.byref(s)) == -1      # bad tree
    p.levels[1] = capi.Eagle3TreeCfg(depth=4, topk=2, width=2, n_nodes=8)
    p.window = 300
    assert lib.eagle3_budget_init(ctypes.byref(p), ctypes.byref(s)) == -1      # window too long
    p.window = 4
    p.low_frac = float("nan")
    assert lib.eagle3_budget_init(ctypes.byref(p), ctypes.byref(s)) == -1      # not a number
    p.low_frac = 0.25
    assert lib.eagle3_budget_init(ctypes.byref(p), ctypes.byref(s)) == 0
    assert lib.eagle3_budget_update(ctypes.byref(p), ctypes.byref(s), -1, 0.1, 0.1, None) == -1
    assert lib.eagle3_budget_update(ctypes.byref(p), ctypes.byref(s), 1, -0.1, 0.1, None) == -1
    assert lib.eagle3_budget_update(ctypes.byref(p), ctypes.byref(s), 1, 0.1, 0.1, None) == 0
