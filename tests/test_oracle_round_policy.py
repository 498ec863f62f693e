"""Pins for the oracle's round statistics and adaptive draft length.

The values come from the pages' own numbers (the 0.85 / 0.60 rule applied
literally in floating point), the exact law of a round found by exhaustive
enumeration, the verification oracle's own stop paths, hand-worked sequences
and brute force.  Planted mistakes at the end must each fail one of them.
"""

import os
import types
from fractions import Fraction as F

import numpy as np
import pytest

import oracle as O
import oracle.round_policy as RP
from tests.test_oracle_pins import _exhaustive_round

# ---------------------------------------------------------------------------
# Accepted drafts of a round, against the stop path the verifier reports
# ---------------------------------------------------------------------------


def _random_verify(R, seed, eos_id):
    rng = np.random.default_rng(seed)
    B, K, V = 400, 5, 6
    tgt = rng.normal(0, 1.5, size=(B, K + 1, V))
    dft = tgt[:, :K] + rng.normal(0, 0.8, size=(B, K, V))
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    dl = rng.integers(0, K + 1, size=B).astype(np.int32)
    dl[::37] = -1                                  # invalid draft_len: a failed round
    u = rng.random((B, K)).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    return R.verify(tgt, dft, toks, dl, u, uf, 1.0, eos_id=eos_id, dtype="f64"), toks, dl


def _want_accepted(res, b):
    n, path = int(res["n_emitted"][b]), int(res["path"][b])
    return {O.PATH_ERROR: -1, O.PATH_EOS: n}.get(path, n - 1)


@pytest.mark.parametrize("eos_id", [-1, 2])
def test_drafts_accepted_follows_the_stop_path(eos_id, rp=None):
    # tbxsx.cn "4. 实现逻辑" feeds the monitor the round's accepted count; the
    # verifier's path tells which emitted tokens are accepted drafts: all but
    # the last after a rejection or a full acceptance, all after an EOS stop.
    rp = rp or RP
    res, toks, dl = _random_verify(O, 13 + eos_id, eos_id)
    paths = set(res["path"].tolist())
    assert {O.PATH_REJECT, O.PATH_BONUS, O.PATH_ERROR} <= paths
    if eos_id >= 0:
        assert O.PATH_EOS in paths
    acc, tot = rp.round_stats(toks, dl, res["out_tokens"], res["n_emitted"])
    for b in range(len(dl)):
        assert acc[b] == _want_accepted(res, b), b
    ok = res["path"] != O.PATH_ERROR
    assert tot["requests"] == ok.sum() and tot["errors"] == (~ok).sum()
    assert tot["drafted"] == dl[ok].sum() and tot["emitted"] == res["n_emitted"][ok].sum()
    assert tot["eos_stops"] == (res["path"] == O.PATH_EOS).sum()
    assert tot["full_accepts"] == (res["path"] == O.PATH_BONUS).sum()
    assert tot["rejections"] == (res["path"] == O.PATH_REJECT).sum()
    assert tot["accepted"] == sum(_want_accepted(res, b) for b in np.nonzero(ok)[0])


def test_round_stats_bookkeeping():
    # Hand-built outputs: a rejection at 1, a full acceptance, an EOS stop at 0,
    # a round with nothing drafted and a failed round.
    toks = np.array([[4, 5, 6], [4, 5, 6], [9, 5, 6], [1, 1, 1], [1, 2, 3]])
    dl = np.array([3, 2, 3, 0, 3])
    out = np.array([[4, 7, -1, -1], [4, 5, 8, -1], [9, -1, -1, -1], [3, -1, -1, -1],
                    [-1, -1, -1, -1]])
    n = np.array([2, 3, 1, 1, -1])
    acc, tot = RP.round_stats(toks, dl, out, n)
    assert list(acc) == [1, 2, 1, 0, -1]
    assert tot == {"requests": 4, "errors": 1, "drafted": 8, "accepted": 4, "emitted": 7,
                   "eos_stops": 1, "full_accepts": 2, "rejections": 1}


# ---------------------------------------------------------------------------
# E[N] with a rate per position, against the exact law of a round
# ---------------------------------------------------------------------------


def test_expected_tokens_equal_rates_is_the_pages_sum():
    # nickwang.xyz "好草稿也要算得便宜": equal rates give 1 + a + ... + a^gamma,
    # whose printed values the other pins hold.
    for a in (0.0, 0.3, 0.8, 1.0):
        for g in range(6):
            want = sum(a ** j for j in range(g + 1))
            assert abs(RP.expected_tokens_given_rates([a] * g) - want) < 1e-12


@pytest.mark.parametrize("draft_len", [1, 2])
def test_expected_tokens_given_rates_is_the_exact_round_mean(draft_len):
    # Rows that do not depend on the prefix: positions accept independently,
    # each with its own sum_x min(p, q).  The exhaustive law of O.verify gives
    # the mean emitted tokens and accepted drafts exactly.
    p_rows = [np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.6, 0.3]), np.array([0.25, 0.25, 0.5])]
    q_rows = [np.array([0.6, 0.1, 0.3]), np.array([0.3, 0.3, 0.4])]
    res = _exhaustive_round(p_rows, q_rows, draft_len=draft_len, with_drafts=True)
    beta = [O.acceptance_rate(p_rows[k], q_rows[k]) for k in range(draft_len)]
    e = RP.expected_tokens_given_rates(beta)
    mean_n = sum(w * n for w, _, n, _ in res)
    mean_acc = sum(w * RP.drafts_accepted(x, draft_len, o, n) for w, o, n, x in res)
    assert abs(mean_n - e) < 1e-12
    assert abs(mean_acc - (e - 1)) < 1e-12
    assert abs(e - (1 + 0.8 + (0.8 * 0.7 if draft_len == 2 else 0))) < 1e-12


def test_expected_tokens_brute_force_patterns():
    # Enumerate every accept / reject pattern of independent positions.
    rng = np.random.default_rng(4)
    for _ in range(50):
        g = int(rng.integers(0, 7))
        rates = rng.random(g)
        e = 0.0
        for pat in range(1 << g):
            w, lead = 1.0, 0
            bits = [(pat >> k) & 1 for k in range(g)]
            for k, bit in enumerate(bits):
                w *= rates[k] if bit else 1 - rates[k]
            while lead < g and bits[lead]:
                lead += 1
            e += w * (lead + 1)
        assert abs(RP.expected_tokens_given_rates(rates) - e) < 1e-12


def test_expected_tokens_per_request():
    beta = np.array([[0.5, 0.25, -1.0], [0.5, -1.0, -1.0], [1.0, 1.0, 1.0], [0.1, 0.2, 0.3]],
                    dtype=np.float32)
    got = RP.expected_tokens_per_request(beta, [2, 2, 3, -1])
    assert got.dtype == np.float32
    assert list(got) == [1 + 0.5 + 0.125, -1.0, 4.0, -1.0]
    assert list(RP.expected_tokens_per_request(beta, [0, 1, 4, 3])) == [1.0, 1.5, -1.0,
                                                                       np.float32(1 + 0.1 + 0.02
                                                                                  + 0.006)]


# ---------------------------------------------------------------------------
# The adaptive draft length of tbxsx.cn "4. 实现逻辑"
# ---------------------------------------------------------------------------


def _page_rule(rate, k, max_k):
    # The rule as printed: float comparisons with 0.85 and 0.60.
    if rate > 0.85:
        return min(max_k, k + 1)
    if rate < 0.60:
        return max(1, k - 1)
    return k


def test_rational_thresholds_match_the_printed_rule():
    # For every count up to 512 the exact thresholds decide as the printed
    # floating-point rule does (17/20 and 3/5 themselves included).
    for d in range(1, 513):
        for a in range(d + 1):
            for k, mk in ((1, 8), (4, 8), (8, 8)):
                assert RP.next_draft_length(a, d, k, mk) == _page_rule(a / d, k, mk), (a, d, k)


def test_thresholds_at_and_around_the_edges():
    assert RP.next_draft_length(17, 20, 4, 8) == 4 and RP.next_draft_length(3, 5, 4, 8) == 4
    assert RP.next_draft_length(18, 20, 4, 8) == 5 and RP.next_draft_length(11, 20, 4, 8) == 3
    assert RP.next_draft_length(1, 1, 8, 8) == 8 and RP.next_draft_length(0, 1, 1, 8) == 1
    assert RP.next_draft_length(0, 0, 5, 8) == 5
    assert RP.next_draft_length(0, 0, 0, 8) == 1 and RP.next_draft_length(0, 0, 12, 8) == 8


def test_monitor_hand_worked_sequence():
    # window 3, max K 6, starting at K = 4; (accepted, drafted) per round.
    rounds = [(4, 4), (2, 5), (0, 5), (4, 4), (3, 3), (2, 2)]
    want_rate = [F(4, 4), F(6, 9), F(6, 14), F(6, 14), F(7, 12), F(9, 9)]
    want_k = [5, 5, 4, 3, 2, 3]
    m, k = RP.RateWindow(3), 4
    for (a, d), wr, wk in zip(rounds, want_rate, want_k):
        m.push(a, d)
        k = RP.next_draft_length(*m.totals(), k, 6)
        assert m.rate() == wr and k == wk


def test_monitor_is_a_ratio_of_sums():
    # (1 of 1) then (2 of 5): 3/6 lowers K; the mean of the two ratios (0.7)
    # would keep it.
    m = RP.RateWindow(2)
    m.push(1, 1)
    m.push(2, 5)
    assert m.rate() == F(1, 2)
    assert RP.next_draft_length(*m.totals(), 4, 8) == 3


def test_monitor_window_brute_force():
    rng = np.random.default_rng(9)
    for W in (1, 2, 5, 16):
        m = RP.RateWindow(W)
        hist = []
        for _ in range(60):
            d = int(rng.integers(0, 9))
            a = int(rng.integers(0, d + 1))
            hist.append((a, d))
            m.push(a, d)
            r = m.rate()
            last = hist[-W:]
            sd = sum(x[1] for x in last)
            assert r == (F(sum(x[0] for x in last), sd) if sd else None)


def test_monitor_round_batch():
    # Requests keep separate windows; a failed round adds nothing and keeps K
    # (clamped to [1, max_k]).
    mons = [RP.RateWindow(2) for _ in range(3)]
    toks = np.array([[1, 2, 3]] * 3)
    # request 0 accepts everything, 1 rejects at 0, 2 fails
    out = np.array([[1, 2, 3, 7], [5, -1, -1, -1], [-1, -1, -1, -1]])
    nxt, rate = RP.monitor_round(mons, toks, np.array([3, 3, 3]), out, np.array([4, 1, -1]),
                                 max_k=4)
    assert list(nxt) == [4, 2, 3] and list(rate) == [1.0, 0.0, -1.0]
    assert len(mons[2].counts) == 0
    out2 = np.array([[1, 2, 3, 7], [1, 2, 8, -1], [1, 9, -1, -1]])
    nxt, rate = RP.monitor_round(mons, toks, np.array([3, 2, 3]), out2,
                                 np.array([4, 3, 2]), max_k=4)
    # request 1: window (0 of 3), (2 of 2) -> 2/5 lowers 2 to 1
    assert list(nxt) == [4, 1, 2]
    assert rate[1] == 0.4 and rate[2] == float(F(1, 3))


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "round_policy.py")

MUTANTS = {
    "eos_stop_not_counted": ("        return n\n    return n - 1", "        return n - 1\n    return n - 1"),
    "correction_counted": ("    return n - 1\n\n\ndef round_stats", "    return n\n\n\ndef round_stats"),
    "raise_not_strict": ("RAISE_ABOVE.denominator * a > RAISE_ABOVE.numerator * d",
                         "RAISE_ABOVE.denominator * a >= RAISE_ABOVE.numerator * d"),
    "lower_not_strict": ("LOWER_BELOW.denominator * a < LOWER_BELOW.numerator * d",
                         "LOWER_BELOW.denominator * a <= LOWER_BELOW.numerator * d"),
    "thresholds_swapped": ("RAISE_ABOVE = Fraction(17, 20)", "RAISE_ABOVE = Fraction(3, 5)"),
    "window_off_by_one": ("[-self.window:]", "[-(self.window + 1):]"),
    "mean_of_ratios": ("return Fraction(a, d) if d > 0 else None",
                       "return (sum(Fraction(x, y) for x, y in self.counts if y) / "
                       "sum(1 for _, y in self.counts if y)) if d > 0 else None"),
    "last_round_only": ("return sum(c[0] for c in self.counts), sum(c[1] for c in self.counts)",
                        "return self.counts[-1] if self.counts else (0, 0)"),
    "failed_round_counted": ("        if acc[b] >= 0:\n            monitors[b].push",
                             "        if True:\n            monitors[b].push"),
    "expected_off_by_one": ("        run *= float(beta)\n        total += run",
                            "        total += run\n        run *= float(beta)"),
}

CHECKS = [
    lambda rp: test_drafts_accepted_follows_the_stop_path(2, rp),
    lambda rp: test_drafts_accepted_follows_the_stop_path(-1, rp),
]


def _mutant(old, new):
    with open(SRC, encoding="utf-8") as f:
        text = f.read()
    assert text.count(old) == 1, old
    mod = types.ModuleType("round_policy_mutant")
    exec(compile(text.replace(old, new), "round_policy_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    mod = _mutant(*MUTANTS[mutant])
    monkeypatch.setitem(globals(), "RP", mod)
    checks = [test_round_stats_bookkeeping, test_expected_tokens_equal_rates_is_the_pages_sum,
              lambda: test_expected_tokens_given_rates_is_the_exact_round_mean(2),
              test_rational_thresholds_match_the_printed_rule, test_thresholds_at_and_around_the_edges,
              test_monitor_hand_worked_sequence, test_monitor_is_a_ratio_of_sums,
              test_monitor_window_brute_force, test_monitor_round_batch] + \
        [lambda c=c: c(mod) for c in CHECKS]
    caught = 0
    for fn in checks:
        try:
            fn()
        except Exception:
            caught += 1
    assert caught, f"mutant {mutant} passes every pin"
