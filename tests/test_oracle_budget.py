"""Pins for the oracle's speculative-budget controller ([P5] 执行控制器): the behaviours the
page asks for (lower on low acceptance or costly drafting, raise cautiously when acceptance
is stable and verification has room, bounded, cooled down, falling back instead of
oscillating), plus a short trace whose decisions are worked out by hand."""
import numpy as np

from oracle import eagle3_oracle as O

DEPTHS = [3, 4, 6, 8]          # a ladder of four tree budgets


def ctl(**kw):
    p = dict(n_levels=4, depths=DEPTHS, start=2, cooldown=8, window=16, low_frac=0.25,
             high_frac=0.5, max_cv=0.35, draft_share_max=0.75, verify_ms_max=1.0, revert_drop=0.05)
    p.update(kw)
    return O.BudgetController(**p)


def run(c, trace):
    return [c.update(*t) for t in trace]


def changes(levels, start):
    prev, out = start, []
    for r, l in enumerate(levels):
        if l != prev:
            out.append((r, prev, l))
        prev = l
    return out


def test_low_acceptance_walks_down_to_the_floor():
    c = ctl()
    lv = run(c, [(0, 1.0, 0.5)] * 80)          # one token per round: frac = 1/7 at depth 6
    ch = changes(lv, 2)
    assert [(a, b) for _, a, b in ch] == [(2, 1), (1, 0)]
    assert ch[0][0] == 15 and ch[1][0] == 31   # a full window (16 rounds) at each level
    assert lv[-1] == 0


def test_costly_drafting_lowers_the_budget():
    c = ctl()
    lv = run(c, [(6, 4.0, 0.5)] * 40)          # every node accepted, but drafting is 89% of the round
    assert changes(lv, 2)[0][1:] == (2, 1)


def test_stable_high_acceptance_with_room_climbs_to_the_top():
    c = ctl(start=0)
    trace, lv = [], []
    for r in range(200):
        L = c.level
        a = DEPTHS[L]                            # the whole path accepted
        lv.append(c.update(a, 0.2 + 0.05 * L, 0.3))
    assert lv[-1] == 3
    ch = changes(lv, 0)
    assert [(a, b) for _, a, b in ch] == [(0, 1), (1, 2), (2, 3)]
    assert all(r2 - r1 >= 16 for (r1, _, _), (r2, _, _) in zip(ch, ch[1:]))


def test_noisy_acceptance_never_raises():
    """Committed tokens alternating 1, 5 (mean 3 of 5, coefficient of variation 2/3): high
    on average but unstable, so the budget is never raised (nor lowered)."""
    c = ctl(start=1)
    lv = run(c, [(0 if r % 2 else 4, 0.2, 0.3) for r in range(300)])
    assert lv == [1] * 300


def test_no_room_in_verification_never_raises():
    c = ctl(start=1)
    lv = run(c, [(4, 0.2, 1.5)] * 200)          # verify time over the cap
    assert lv == [1] * 200


def test_a_raise_that_costs_goodput_is_reverted_and_blocked():
    c = ctl(start=1, cooldown=4, window=8)
    lv = []
    for r in range(120):
        L = c.level
        a = DEPTHS[L]
        lat = 0.5 if L <= 1 else 2.0             # level 2 is four times as slow
        lv.append(c.update(a, 0.1 * lat, 0.9 * lat))
    ch = changes(lv, 1)
    assert ch[0][1:] == (1, 2) and ch[1][1:] == (2, 1)          # raise, then revert
    assert ch[1][0] - ch[0][0] == 8                               # after one full window
    if len(ch) > 2:                                               # blocked for 4 * cooldown
        assert ch[2][0] - ch[1][0] >= 16


def test_bounds_and_spacing_under_random_traces():
    rng = np.random.default_rng(7)
    for seed in range(5):
        c = ctl(start=int(rng.integers(0, 4)), cooldown=int(rng.integers(1, 10)),
                window=int(rng.integers(1, 12)))
        start = c.level
        lv = run(c, [(int(rng.integers(0, 9)), float(rng.uniform(0.05, 2)), float(rng.uniform(0.05, 2)))
                     for _ in range(400)])
        assert all(0 <= l <= 3 for l in lv)
        ch = changes(lv, start)
        assert all(abs(b - a) == 1 for _, a, b in ch)
        gap = max(c.window, c.cooldown)
        assert all(r2 - r1 >= gap for (r1, _, _), (r2, _, _) in zip(ch, ch[1:]))


def test_hand_worked_trace():
    """window 2, cooldown 2, depths [3, 4, 6, 8], start at level 1 (depth 4, frac = c / 5).
    round 0: (4, 0.1, 0.3)  window not full                      -> 1
    round 1: (4, 0.1, 0.3)  c = [5, 5], frac 1, cv 0, verify 0.3 -> raise to 2, goodput 5/0.4
    round 2: (6, 0.1, 0.3)  window cleared, not full             -> 2
    round 3: (6, 0.3, 0.5)  c = [7, 7], goodput 7/0.6 = 11.67 < 12.5 * 0.95 = 11.875 -> revert to 1
    round 4: (4, 0.1, 0.3)  -> 1;  round 5: (4, 0.1, 0.3): frac 1 but raises blocked (8 rounds) -> 1
    round 6: (0, 0.1, 0.3)  -> 1;  round 7: (0, 0.1, 0.3): c = [1, 1], frac 0.2 < 0.25 -> lower to 0"""
    c = ctl(start=1, cooldown=2, window=2)
    trace = [(4, 0.1, 0.3), (4, 0.1, 0.3), (6, 0.1, 0.3), (6, 0.3, 0.5), (4, 0.1, 0.3), (4, 0.1, 0.3),
             (0, 0.1, 0.3), (0, 0.1, 0.3)]
    assert run(c, trace) == [1, 2, 2, 1, 1, 1, 1, 0]
