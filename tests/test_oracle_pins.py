"""Pins for the fp64 oracle against what the pages and the mathematics fix.

Each test names the page passage (title + section) it checks.  Nothing here
retypes an oracle formula to compare it with itself: values come from the
pages' printed output, exact rational arithmetic, closed forms, library
routines or brute force.
"""

import decimal
import json
import math
import os
from decimal import Decimal as D
from fractions import Fraction as F

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _fr(xs):
    return np.array([F(x) for x in xs], dtype=object)


# ---------------------------------------------------------------------------
# nickwang.xyz "推测解码：草稿、验证与实际加速", section "算完三个 token 的全部概率"
# ---------------------------------------------------------------------------

def test_worked_example_exact_fractions():
    g = _golden("nw_worked_example.json")
    p, q = _fr(g["p"]), _fr(g["q"])
    alpha = [O.accept_prob(p, q, x) for x in range(3)]
    assert alpha == [F(a) for a in g["alpha"]]
    accepted = np.array([q[x] * alpha[x] for x in range(3)], dtype=object)
    assert [float(a) for a in accepted] == g["accepted_mass_printed"]
    acc = sum(accepted)
    assert float(acc) == g["acceptance_printed"]
    r = O.residual(p, q)
    s_r = sum(r)
    assert s_r == 1 - acc                      # normaliser equals 1 - acceptance
    assert [float(x / s_r) for x in r] == g["residual_printed"]
    restored = accepted + (1 - acc) * (r / s_r)
    assert list(restored) == list(p)           # exact reconstruction
    assert [float(x) for x in restored] == g["reconstructed_printed"]


def _toy_logits(dtype=np.float64):
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.6, 0.1, 0.3])
    return np.log(p).astype(dtype), np.log(q).astype(dtype)


def _toy_call(draft, u, u_final, K=None, eos=-1, dtype="f64", draft_len=None):
    lp, lq = _toy_logits(np.float64 if dtype == "f64" else np.float32)
    K = len(draft) if K is None else K
    target = np.tile(lp, (1, K + 1, 1))
    dr = np.tile(lq, (1, K, 1))
    tokens = np.array([draft], dtype=np.int32)
    dl = np.array([len(draft) if draft_len is None else draft_len], dtype=np.int32)
    return O.verify(target, dr, tokens, dl, np.array([u], dtype=np.float32),
                    np.array([u_final], dtype=np.float32), 1.0, eos_id=eos, dtype=dtype)


@pytest.mark.parametrize("dtype,tol", [("f64", 1e-12), ("f32", 1e-6)])
def test_worked_example_replay(dtype, tol):
    g = _golden("nw_worked_example.json")["replay"]
    r = _toy_call(g["draft"], g["draws"], g["final_draw"], dtype=dtype)
    assert list(r["out_tokens"][0]) == g["emit_printed"] + [-1, -1]
    assert r["n_emitted"][0] == 2
    assert r["path"][0] == O.PATH_REJECT and r["stop_pos"][0] == 1
    a = r["alpha"][0]
    assert abs(a[0] - 5 / 6) < tol and abs(a[1] - 2 / 3) < tol and abs(a[2] - 1.0) < tol
    assert [f"{x:.3f}" for x in a[:2]] == g["thresholds_printed"]
    assert abs(r["residual_mass"][0] - 0.2) < tol
    assert r["flag_kind"][0] == O.FLAG_NONE


def test_worked_example_bonus_and_strict_cdf():
    # Same toy, every draft accepted: the bonus comes from p with the final draw
    # (the replay's else-branch).  p's CDF edges are 0.5 and 0.8; the strict
    # comparison of sample() puts an edge value into the next token.
    for uf, want in [(0.2, 0), (0.5, 1), (0.6, 1), (0.8, 2), (0.95, 2)]:
        r = _toy_call([0, 1], [0.1, 0.1], uf)
        assert r["path"][0] == O.PATH_BONUS
        assert list(r["out_tokens"][0]) == [0, 1, want]
        assert r["n_emitted"][0] == 3


def test_sample_semantics_exact():
    # sample(distribution, u) of the replay, with exact fractions.
    p = _fr(["1/2", "3/10", "1/5"])
    assert O.icdf(p, F(1, 5))[0] == 0
    assert O.icdf(p, F(1, 2))[0] == 1          # u equal to the running sum moves on
    assert O.icdf(p, F(4, 5))[0] == 2
    assert O.icdf(p, F(99, 100))[0] == 2
    resid = _fr(["0", "1", "0"])
    assert O.icdf(resid, F(1, 5))[0] == 1
    assert O.icdf(resid, F(0))[0] == 1         # zero-weight token 0 is never drawn


# ---------------------------------------------------------------------------
# Identities: acceptance rate and distribution preservation
# ---------------------------------------------------------------------------

def _rand_dist(rng, V, zero_frac=0.0):
    n = rng.integers(1, 50, size=V)
    n[rng.random(V) < zero_frac] = 0
    if n.sum() == 0:
        n[0] = 1
    tot = int(n.sum())
    return np.array([F(int(x), tot) for x in n], dtype=object)


def test_acceptance_rate_identity_exact():
    # nickwang.xyz "好草稿也要算得便宜": for a fixed prefix the acceptance rate
    # is sum_x min(p(x), q(x)).  The oracle's alpha, averaged under x ~ q, must
    # give exactly that, and the residual mass must be its complement.
    rng = np.random.default_rng(7)
    for _ in range(200):
        V = int(rng.integers(2, 7))
        p, q = _rand_dist(rng, V, 0.2), _rand_dist(rng, V, 0.2)
        rate = sum(q[x] * O.accept_prob(p, q, x) for x in range(V) if q[x] > 0)
        assert rate == sum(min(a, b) for a, b in zip(p, q))
        assert sum(O.residual(p, q)) == 1 - rate


def test_distribution_preservation_exact():
    # bowenzhou.top "深入推导": q*alpha + norm(max(p-q,0)) * (1 - sum q*alpha)
    # equals p pointwise; nickwang.xyz checks the same with fractions.
    rng = np.random.default_rng(11)
    for _ in range(200):
        V = int(rng.integers(2, 8))
        p, q = _rand_dist(rng, V, 0.3), _rand_dist(rng, V, 0.3)
        acc = [q[x] * O.accept_prob(p, q, x) if q[x] > 0 else F(0) for x in range(V)]
        rej = 1 - sum(acc)
        r = O.residual(p, q)
        if rej == 0:
            assert list(p) == list(q)
            continue
        final = [acc[x] + rej * r[x] / sum(r) for x in range(V)]
        assert final == list(p)


def test_equal_distributions_accept_everything():
    # nickwang.xyz "接受与拒绝怎样保住分布": p == q accepts every candidate, so
    # the correction branch (0/0) is never entered.
    rng = np.random.default_rng(3)
    p = _rand_dist(rng, 5)
    assert all(O.accept_prob(p, p, x) == 1 for x in range(5))
    assert sum(O.residual(p, p)) == 0


# ---------------------------------------------------------------------------
# Processed distribution: temperature, top-k, top-p
# ---------------------------------------------------------------------------

def test_two_token_closed_form():
    rng = np.random.default_rng(5)
    for _ in range(50):
        z = rng.normal(0, 3, size=2)
        T = float(rng.uniform(0.3, 2.0))
        P, _ = O.processed_distribution(z, T)
        want = 1.0 / (1.0 + math.exp(-(z[1] - z[0]) / T))
        assert abs(P[1] - want) < 1e-15 and abs(P.sum() - 1) < 1e-15


def test_softmax_matches_library():
    from scipy.special import softmax
    rng = np.random.default_rng(6)
    z = rng.normal(0, 3, size=1000)
    for T in (1.0, 0.7, 2.5):
        P, _ = O.processed_distribution(z, T)
        np.testing.assert_allclose(P, softmax(z / T), rtol=1e-12, atol=0)


def test_topk_brute_force_with_ties():
    # Keep every token whose logit is >= the k-th largest (ties kept): token v is
    # kept iff fewer than k logits are strictly larger than z[v].
    rng = np.random.default_rng(8)
    for _ in range(300):
        V = int(rng.integers(2, 12))
        z = rng.integers(-3, 4, size=V).astype(np.float64)   # many ties
        k = int(rng.integers(1, V + 2))
        P, info = O.processed_distribution(z, 1.0, top_k=k)
        kept = np.array([(z > z[v]).sum() < k for v in range(V)])
        assert np.array_equal(P > 0, kept), (z, k)
        ref = sorted(z, reverse=True)[k - 1] if k < V else -np.inf
        assert info["tau_k"] == ref


def test_topp_brute_force_over_thresholds():
    # The kept set is {z >= tau} for the largest logit value tau whose upper set
    # carries at least top_p of the (top-k renormalised) mass.
    rng = np.random.default_rng(9)
    checked = 0
    for _ in range(400):
        V = int(rng.integers(2, 10))
        z = np.round(rng.normal(0, 1.5, size=V), 1)
        k = int(rng.integers(0, V + 1))
        top_p = float(rng.uniform(0.05, 0.99))
        T = float(rng.uniform(0.5, 1.5))
        P, info = O.processed_distribution(z, T, top_k=k, top_p=top_p)
        if info["topp_margin"] < 1e-9:
            continue
        base = np.ones(V, dtype=bool)
        if 0 < k < V:
            base = np.array([(z > z[v]).sum() < k for v in range(V)])
        w = np.where(base, np.exp((z - z.max()) / T), 0.0)
        w /= w.sum()
        best = None
        for tau in sorted(set(z[base]), reverse=True):
            if w[z >= tau].sum() >= top_p:
                best = tau
                break
        kept = base & (z >= best)
        assert np.array_equal(P > 0, kept), (z, k, top_p)
        want = np.where(kept, np.exp((z - z.max()) / T), 0.0)
        np.testing.assert_allclose(P, want / want.sum(), rtol=1e-13, atol=1e-300)
        checked += 1
    assert checked > 300


def _exact_topp(z, T, k, top_p, prec=60):
    """The top-p cut of one row in 60-digit decimal arithmetic, by brute force.

    The top-k base set comes from counting strictly larger logits (ties kept),
    each weight exp((z - m) / T) is evaluated by decimal's own exp from the
    exact binary values of z, T and top_p, and the shares are accumulated in
    (logit descending, id ascending) order.  M is the first share reaching
    top_p; the margin is the distance of top_p from the nearer of the two
    shares around the cut, c_M and c_{M-1}.  Returns (tau_p, margin, order).
    """
    with decimal.localcontext() as ctx:
        ctx.prec = prec
        V = len(z)
        if 0 < k < V:
            idx = [v for v in range(V) if sum(1 for x in z if x > z[v]) < k]
        else:
            idx = list(range(V))
        m = max(D(float(z[v])) for v in idx)
        w = {v: ((D(float(z[v])) - m) / D(float(T))).exp() for v in idx}
        order = sorted(idx, key=lambda v: (-z[v], v))
        total = sum(w[v] for v in order)
        shares, run = [], D(0)
        for v in order:
            run += w[v]
            shares.append(run / total)
        tp = D(float(top_p))
        M = next(j for j, c in enumerate(shares) if c >= tp)
        margin = shares[M] - tp
        if M > 0:
            margin = min(margin, tp - shares[M - 1])
        return float(z[order[M]]), float(margin), order, shares


def test_topp_margin_exact_decimal():
    # The flag that guards the top-p cut measures how far top_p lies from the
    # shares on either side of the crossing token (the cumulative mass in
    # sorted order).  Checked against an exact-decimal brute force of the same
    # quantity: its value, and the kept set whenever the cut is not a near tie.
    rng = np.random.default_rng(31)
    lower_side = 0
    for _ in range(300):
        V = int(rng.integers(2, 10))
        z = np.round(rng.normal(0, 1.5, size=V), 1)
        k = int(rng.integers(0, V + 1))
        top_p = float(rng.uniform(0.05, 0.99))
        T = float(rng.uniform(0.5, 1.5))
        P, info = O.processed_distribution(z, T, top_k=k, top_p=top_p)
        tau, margin, order, shares = _exact_topp(z, T, k, top_p)
        assert abs(info["topp_margin"] - margin) <= 1e-14, (z, k, top_p, T)
        if margin > 1e-12:
            assert info["tau_p"] == tau
            base = np.ones(V, dtype=bool)
            if 0 < k < V:
                base = np.array([(z > z[v]).sum() < k for v in range(V)])
            assert np.array_equal(P > 0, base & (z >= tau))
        j = next(i for i, c in enumerate(shares) if c >= decimal.Decimal(top_p))
        lower_side += j > 0 and float(decimal.Decimal(top_p) - shares[j - 1]) < margin + 1e-15
    assert lower_side > 50          # the share below the cut decided the margin often


def _topp_flag_request(critical_pos, delta, reject0=False, bonus=False):
    """One request (K = 2, V = 6, T = 1, top-p only) whose target row
    ``critical_pos`` has a top-p cut exactly ``delta`` away from top_p.

    top_p is set to the exact share of that row's third token plus delta
    (so |margin| = |delta|); every other row's margin is checked (exactly) to
    be far larger.  Each draft token is its draft row's top token, which
    that row keeps; with ``reject0`` target row 0 gives draft token 0 a logit
    far below its others, so top-p drops it and position 0 rejects at
    u[0] = 0.5 (u is 0 elsewhere).
    """
    rng = np.random.default_rng(5)
    K, V = 2, 6
    t = np.round(rng.normal(0, 1.0, size=(1, K + 1, V)), 2)
    d = np.round(t[:, :K] + rng.normal(0, 0.5, size=(1, K, V)), 2)
    crit = np.array([2.0, 1.0, 0.5, 0.0, -1.0, -2.0])
    t[0, critical_pos] = crit
    if reject0:
        t[0, 0, int(np.argmax(d[0, 0]))] = t[0, 0].min() - 8.0
    _, _, _, shares = _exact_topp(crit, 1.0, 0, 0.5)
    top_p = float(shares[2]) + delta
    for k in range(K + 1):
        if k != critical_pos:
            assert abs(_exact_topp(t[0, k], 1.0, 0, top_p)[1]) > 1e-6
    for k in range(K):
        assert abs(_exact_topp(d[0, k], 1.0, 0, top_p)[1]) > 1e-6
    toks = np.array([[int(np.argmax(d[0, k])) for k in range(K)]], dtype=np.int32)
    if not bonus:
        # position 1 drafts a token the target row keeps (its top token)
        toks[0, 1] = int(np.argmax(t[0, 1]))
        d[0, 1, toks[0, 1]] = d[0, 1].max() + 1.0
    u = np.array([[0.5 if reject0 else 0.0, 0.0]], dtype=np.float32)
    return O.verify(t, d, toks, np.array([K], np.int32), u, np.array([0.37], np.float32), 1.0,
                    top_k=0, top_p=top_p, dtype="f64")


def test_topp_flag_marks_the_cut_inside_its_window():
    # A decided position whose target row has a top-p cut within 1e-10 of
    # top_p is flagged FLAG_TOPP at that position, on both sides of the
    # share; 4e-10 away it is not.
    for delta in (4e-11, -4e-11):
        r = _topp_flag_request(1, delta)
        assert r["flag_kind"][0] == O.FLAG_TOPP and r["flag_pos"][0] == 1, delta
        assert abs(r["topp_margin_rows"][0, 1] - abs(delta)) < 1e-15
    for delta in (4e-10, -4e-10):
        r = _topp_flag_request(1, delta)
        assert r["flag_kind"][0] == O.FLAG_NONE, delta


def test_topp_flag_on_the_bonus_row_and_not_past_the_stop():
    # Every draft accepted: the bonus row's cut is checked too (flag at n).
    r = _topp_flag_request(2, 3e-11, bonus=True)
    assert r["path"][0] == O.PATH_BONUS
    assert r["flag_kind"][0] == O.FLAG_TOPP and r["flag_pos"][0] == 2
    # A rejection at position 0 leaves position 1 undecided: its cut does not
    # matter, so it is not flagged.
    r = _topp_flag_request(1, 3e-11, reject0=True)
    assert r["path"][0] == O.PATH_REJECT and r["stop_pos"][0] == 0
    assert r["flag_kind"][0] == O.FLAG_NONE


def test_filters_off_is_unfiltered_bit_for_bit():
    rng = np.random.default_rng(10)
    z = rng.normal(0, 2, size=777)
    P0, _ = O.processed_distribution(z, 0.9)
    P1, _ = O.processed_distribution(z, 0.9, top_k=777, top_p=1.0)
    P2, _ = O.processed_distribution(z, 0.9, top_k=0, top_p=1.0)
    assert np.array_equal(P0, P1) and np.array_equal(P0, P2)


def test_icdf_matches_searchsorted():
    rng = np.random.default_rng(12)
    for _ in range(200):
        w = rng.random(int(rng.integers(1, 300))) * (rng.random() < 0.5 or 1)
        w[rng.random(w.size) < 0.3] = 0
        if w.sum() == 0:
            w[-1] = 1.0
        uu = float(rng.random())
        y, _ = O.icdf(w, uu)
        c = np.cumsum(w)
        assert y == int(np.searchsorted(c, uu * c[-1], side="right"))
        assert w[y] > 0


def test_bf16_widening():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3E80, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, 0.25, 3.140625]
    assert list(O.widen_row(bits, "bf16")) == want


# ---------------------------------------------------------------------------
# Whole-round law, exhaustively: every decision interval of every uniform
# ---------------------------------------------------------------------------

def _exhaustive_round(p_rows, q_rows, draft_len, T=1.0, with_drafts=False):
    """Exact output law of one request, found by running ``O.verify`` once per
    cell of the uniforms' decision partition, weighted by the cell's size.

    p_rows: K+1 target distributions, q_rows: K draft distributions (float64).
    Returns a list of (weight, out_tokens, n_emitted), with the drafted
    tokens appended to each tuple when ``with_drafts``.
    """
    K = len(q_rows)
    V = len(p_rows[0])
    lp = np.log(np.asarray(p_rows, dtype=np.float64))
    lq = np.log(np.asarray(q_rows, dtype=np.float64))
    # every CDF edge of every distribution a final draw may use
    edges = {0.0, 1.0}
    for k in range(K + 1):
        P = np.asarray(p_rows[k])
        edges.update(np.cumsum(P / P.sum()).tolist())
        if k < K:
            r = np.maximum(P - np.asarray(q_rows[k]), 0)
            if r.sum() > 0:
                edges.update(np.cumsum(r / r.sum()).tolist())
    edges = sorted(e for e in edges if 0.0 <= e <= 1.0)
    uf_cells = [((a + b) / 2, b - a) for a, b in zip(edges[:-1], edges[1:]) if b - a > 1e-9]

    combos_x = np.array(np.meshgrid(*[np.arange(V)] * K, indexing="ij")).reshape(K, -1).T
    rows = []
    for xs in combos_x:
        wx = np.prod([q_rows[k][xs[k]] for k in range(K)])
        if wx == 0:
            continue
        alphas = [min(1.0, p_rows[k][xs[k]] / q_rows[k][xs[k]]) for k in range(K)]
        cells_per_k = []
        for a in alphas:
            c = []
            if a > 0:
                c.append((a / 2, a))
            if a < 1:
                c.append(((a + 1) / 2, 1 - a))
            cells_per_k.append(c)
        for choice in np.ndindex(*[len(c) for c in cells_per_k]):
            us = [cells_per_k[k][choice[k]][0] for k in range(K)]
            wu = np.prod([cells_per_k[k][choice[k]][1] for k in range(K)])
            for ufm, wuf in uf_cells:
                rows.append((wx * wu * wuf, xs.copy(), us, ufm))
    B = len(rows)
    tgt = np.broadcast_to(lp, (B, K + 1, V)).copy()
    dft = np.broadcast_to(lq, (B, K, V)).copy()
    toks = np.array([r[1] for r in rows], dtype=np.int32)
    uu = np.array([r[2] for r in rows], dtype=np.float32)
    uf = np.array([r[3] for r in rows], dtype=np.float32)
    dl = np.full(B, draft_len, dtype=np.int32)
    res = O.verify(tgt, dft, toks, dl, uu, uf, T, dtype="f64")
    if with_drafts:
        return [(rows[i][0], res["out_tokens"][i], int(res["n_emitted"][i]), toks[i])
                for i in range(B)]
    return [(rows[i][0], res["out_tokens"][i], int(res["n_emitted"][i])) for i in range(B)]


def _law_checks(results, p_rows, q_rows, draft_len):
    W = sum(w for w, _, _ in results)
    assert abs(W - 1.0) < 1e-12
    # position j of the output, given the round reached it, follows p_j
    for j in range(draft_len + 1):
        reach = [(w, o) for w, o, n in results if n > j]
        mass = sum(w for w, _ in reach)
        if mass < 1e-12:
            continue
        emp = np.zeros(len(p_rows[0]))
        for w, o in reach:
            emp[o[j]] += w
        np.testing.assert_allclose(emp / mass, p_rows[j], atol=1e-9)
    # N follows the position-wise truncated geometric law
    beta = [np.minimum(p_rows[k], q_rows[k]).sum() for k in range(draft_len)]
    for n in range(1, draft_len + 2):
        got = sum(w for w, _, m in results if m == n)
        want = np.prod(beta[:n - 1]) * (1 - beta[n - 1] if n - 1 < draft_len else 1.0)
        assert abs(got - want) < 1e-9, (n, got, want)


def test_exhaustive_round_law_positionwise():
    # bowenzhou.top "深入推导" + nickwang.xyz "候选已知，验证才能并行": each output
    # position is distributed as that position's p; p_{K+1} supplies the bonus.
    p_rows = [np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.6, 0.3]), np.array([0.25, 0.25, 0.5])]
    q_rows = [np.array([0.6, 0.1, 0.3]), np.array([0.3, 0.3, 0.4])]
    res = _exhaustive_round(p_rows, q_rows, draft_len=2)
    _law_checks(res, p_rows, q_rows, 2)


def test_exhaustive_round_law_ragged_bonus_row():
    # With draft_len = 1 < K = 2 the bonus must come from target row 1.
    p_rows = [np.array([0.5, 0.3, 0.2]), np.array([0.1, 0.6, 0.3]), np.array([0.25, 0.25, 0.5])]
    q_rows = [np.array([0.6, 0.1, 0.3]), np.array([0.3, 0.3, 0.4])]
    res = _exhaustive_round(p_rows, q_rows, draft_len=1)
    _law_checks(res, p_rows, q_rows, 1)


@pytest.mark.parametrize("gamma", [3, 4])
def test_expected_tokens_exhaustive(gamma):
    # The toy of "算完三个 token 的全部概率" has acceptance exactly 0.8; with
    # gamma i.i.d. drafts the mean round length is the closed form of
    # "好草稿也要算得便宜" (3.3616 for gamma = 4) and of bowenzhou.top "参考答案"
    # (about 2.95 for gamma = 3).
    p, q = np.array([0.5, 0.3, 0.2]), np.array([0.6, 0.1, 0.3])
    res = _exhaustive_round([p] * (gamma + 1), [q] * gamma, draft_len=gamma)
    mean_n = sum(w * n for w, _, n in res)
    for case in _golden("expected_tokens_per_round.json")["cases"]:
        if case["alpha"] == 0.8 and case["gamma"] == gamma:
            assert round(mean_n, case["decimals"]) == case["tokens"]
    assert abs(mean_n - (1 - 0.8 ** (gamma + 1)) / (1 - 0.8)) < 1e-9


def test_expected_tokens_printed_values():
    for case in _golden("expected_tokens_per_round.json")["cases"]:
        e = O.expected_tokens_per_round(case["alpha"], case["gamma"])
        assert round(e, case["decimals"]) == case["tokens"]
        a, g = case["alpha"], case["gamma"]
        assert abs(e - (1 - a ** (g + 1)) / (1 - a)) < 1e-12


# ---------------------------------------------------------------------------
# EOS, p == q, draft_len == 0, errors, flags
# ---------------------------------------------------------------------------

def _random_call(rng, B=40, K=4, V=50, eos=-1, same=False, T=1.0):
    t = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    d = t[:, :K] if same else (t[:, :K] + rng.normal(0, 0.8, size=(B, K, V))).astype(np.float32)
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    dl = rng.integers(0, K + 1, size=B).astype(np.int32)
    u = rng.random((B, K)).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    return t, np.ascontiguousarray(d), toks, dl, u, uf, T


def test_eos_truncation_invariant():
    rng = np.random.default_rng(21)
    t, d, toks, dl, u, uf, T = _random_call(rng, B=200, V=6)
    base = O.verify(t, d, toks, dl, u, uf, T)
    for eos in range(6):
        r = O.verify(t, d, toks, dl, u, uf, T, eos_id=eos)
        for b in range(200):
            n0 = base["n_emitted"][b]
            seq = list(base["out_tokens"][b][:n0])
            if eos in seq:
                cut = seq.index(eos) + 1
                assert r["n_emitted"][b] == cut
                assert list(r["out_tokens"][b][:cut]) == seq[:cut]
                assert all(r["out_tokens"][b][cut:] == -1)
            else:
                assert r["n_emitted"][b] == n0
                assert np.array_equal(r["out_tokens"][b], base["out_tokens"][b])


def test_p_equals_q_always_bonus():
    rng = np.random.default_rng(22)
    t, d, toks, dl, u, uf, T = _random_call(rng, same=True)
    r = O.verify(t, d, toks, dl, u, uf, T)
    assert (r["path"] == O.PATH_BONUS).all()
    assert np.array_equal(r["n_emitted"], dl + 1)
    for b in range(len(dl)):
        assert np.all(r["alpha"][b, :dl[b]] == 1.0)


def test_draft_len_zero_is_bonus_from_row0():
    rng = np.random.default_rng(23)
    t, d, toks, dl, u, uf, T = _random_call(rng)
    dl[:] = 0
    r = O.verify(t, d, toks, dl, u, uf, T)
    assert (r["n_emitted"] == 1).all() and (r["path"] == O.PATH_BONUS).all()
    for b in range(len(dl)):
        w = np.exp(t[b, 0].astype(np.float64) - t[b, 0].max())
        c = np.cumsum(w)
        assert r["out_tokens"][b, 0] == np.searchsorted(c, float(uf[b]) * c[-1], side="right")


def test_error_requests_are_isolated():
    rng = np.random.default_rng(24)
    t, d, toks, dl, u, uf, T = _random_call(rng, B=8, V=30)
    dl[:] = 4
    good = O.verify(t, d, toks, dl, u, uf, T)
    dl2, toks2, u2, uf2, d2 = dl.copy(), toks.copy(), u.copy(), uf.copy(), d.copy()
    dl2[0] = 5                       # draft_len > K
    dl2[1] = -1                      # negative draft_len
    toks2[2, 3] = 30                 # token out of range
    u2[3, 1] = 1.0                   # uniform outside [0, 1)
    uf2[4] = np.nan                  # final uniform not a number
    d2[5, 2, toks2[5, 2]] = -np.inf  # q(x) == 0
    r = O.verify(t, d2, toks2, dl2, u2, uf2, T)
    for b in range(6):
        assert r["n_emitted"][b] == -1 and (r["out_tokens"][b] == -1).all()
    for b in (6, 7):
        assert r["n_emitted"][b] == good["n_emitted"][b]
        assert np.array_equal(r["out_tokens"][b], good["out_tokens"][b])


def test_topk_makes_unkept_draft_an_error_and_unkept_target_a_reject():
    V = 10
    z = np.arange(V, dtype=np.float32)
    t = np.tile(z, (1, 2, 1))
    d = np.tile(z[::-1].copy(), (1, 1, 1))
    # top-2 keeps {8, 9} in the target and {0, 1} in the draft.
    r = O.verify(t, d, np.array([[9]], np.int32), np.array([1], np.int32),
                 np.array([[0.0]], np.float32), np.array([0.5], np.float32), 1.0, top_k=2)
    assert r["n_emitted"][0] == -1                       # q(9) == 0 after top-k
    r = O.verify(t, d, np.array([[0]], np.int32), np.array([1], np.int32),
                 np.array([[0.0]], np.float32), np.array([0.5], np.float32), 1.0, top_k=2)
    assert r["alpha"][0, 0] == 0.0 and r["path"][0] == O.PATH_REJECT
    assert r["out_tokens"][0, 0] in (8, 9)               # correction from target's kept set


def test_flags_accept_and_cdf():
    # alpha = 5/6 at A; a draw within 1e-5 * alpha of it is flagged.
    r = _toy_call([0], [np.float32(5 / 6)], 0.3, dtype="f64")
    assert r["flag_kind"][0] == O.FLAG_ACCEPT and r["flag_pos"][0] == 0
    # bonus draw exactly on p's first CDF edge (0.5) is flagged as a CDF case.
    r = _toy_call([0], [0.1], 0.5, dtype="f64")
    assert r["path"][0] == O.PATH_BONUS and r["flag_kind"][0] == O.FLAG_CDF
    assert r["flag_pos"][0] == 1
    r = _toy_call([0], [0.1], 0.3, dtype="f64")
    assert r["flag_kind"][0] == O.FLAG_NONE


def test_strict_accept_never_takes_a_zero_probability_token():
    # Strict u < alpha (the replay's comparison): a draft the target gives
    # probability 0 is rejected even at u = 0.
    t = np.log(np.array([[[0.5, 0.5, 0.0], [0.2, 0.3, 0.5]]], dtype=np.float64))
    d = np.log(np.array([[[0.2, 0.3, 0.5]]], dtype=np.float64))
    r = O.verify(t, d, np.array([[2]], np.int32), np.array([1], np.int32),
                 np.array([[0.0]], np.float32), np.array([0.1], np.float32), 1.0, dtype="f64")
    assert r["alpha"][0, 0] == 0.0 and r["path"][0] == O.PATH_REJECT
    assert r["out_tokens"][0, 0] in (0, 1)


# ---------------------------------------------------------------------------
# nickwang.xyz "推测解码：草稿、验证与实际加速", section "好草稿也要算得便宜":
# the acceptance rate of a fixed prefix
# ---------------------------------------------------------------------------

def test_acceptance_rate_worked_example():
    # The three-token example of "算完三个 token 的全部概率" prints a total
    # acceptance rate of 0.8 (accepted mass 0.5 + 0.1 + 0.2).
    g = _golden("nw_worked_example.json")
    p, q = _fr(g["p"]), _fr(g["q"])
    assert O.acceptance_rate(p, q) == F(g["acceptance_printed"]).limit_denominator(1000)
    pf = np.array([float(x) for x in p]); qf = np.array([float(x) for x in q])
    assert abs(O.acceptance_rate(pf, qf) - g["acceptance_printed"]) < 1e-15


def test_acceptance_rate_is_one_minus_total_variation():
    # Closed form: for distributions p, q, sum min(p, q) = 1 - (1/2) sum |p - q|
    # (min(a, b) = (a + b - |a - b|) / 2 summed over x); hence symmetric, 1 for
    # p = q and 0 for disjoint supports.
    rng = np.random.default_rng(21)
    for _ in range(200):
        V = int(rng.integers(2, 8))
        p, q = _rand_dist(rng, V, 0.3), _rand_dist(rng, V, 0.3)
        tv = sum(abs(a - b) for a, b in zip(p, q)) / 2
        assert O.acceptance_rate(p, q) == 1 - tv
        assert O.acceptance_rate(q, p) == O.acceptance_rate(p, q)
        assert O.acceptance_rate(p, p) == 1
    a = _fr(["1/2", "1/2", "0", "0"])
    b = _fr(["0", "0", "1/4", "3/4"])
    assert O.acceptance_rate(a, b) == 0


@pytest.mark.parametrize("top_k,top_p", [(0, 1.0), (3, 1.0), (4, 0.8)])
def test_acceptance_rates_equal_expected_acceptance_per_position(top_k, top_p):
    # For every drafted position of a batch, beta equals the probability that
    # the verification accepts a token drawn from q there: sum_x q(x) alpha(x)
    # with the oracle's alpha on the same processed rows.  Positions at or
    # after draft_len, an out-of-range draft_len and a row with no finite
    # logit read -1.
    rng = np.random.default_rng(31 + top_k)
    B, K, V = 5, 3, 7
    target = rng.normal(0, 1.5, size=(B, K + 1, V)).astype(np.float32)
    draft = (target[:, :K] + rng.normal(0, 0.8, size=(B, K, V))).astype(np.float32)
    draft_len = np.array([3, 1, 0, 2, 9], dtype=np.int32)
    draft[3, 1, :] = -np.inf
    T = 0.9
    beta = O.acceptance_rates(target, draft, draft_len, T, top_k, top_p, "f32")
    for b in range(B):
        for k in range(K):
            nb = int(draft_len[b])
            if not 0 <= nb <= K or k >= nb or (b, k) == (3, 1):
                assert beta[b, k] == -1.0
                continue
            P, _ = O.processed_distribution(target[b, k].astype(np.float64), T, top_k, top_p)
            Q, _ = O.processed_distribution(draft[b, k].astype(np.float64), T, top_k, top_p)
            expect = sum(Q[x] * O.accept_prob(P, Q, x) for x in range(V) if Q[x] > 0)
            assert abs(beta[b, k] - expect) < 1e-12
