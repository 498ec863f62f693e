"""Round statistics and the adaptive draft length, written plainly.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing in the
product path imports it.  It shares no code with the HIP library.

Sources (page title and section):

* [TB] tbxsx.cn, "推测解码采样验证优化策略 —— 深度调研报告", section
  "4. 实现逻辑": after each round the decode loop hands the round's accepted
  and drafted counts to an acceptance-rate monitor that keeps a window of
  rounds, and the draft length K moves up by one (never above the maximum
  draft length) when the monitored rate exceeds 0.85 and down by one (never
  below 1) when it falls under 0.60.
* [NW] nickwang.xyz, "推测解码：草稿、验证与实际加速", section
  "好草稿也要算得便宜": E[N] = 1 + a + ... + a^gamma tokens per round when
  every position accepts independently with the same rate a; when the rate
  varies by position, the tokens a round really commits are what counts.
  Section "在相同负载和质量下比较" (its measurement table): keep the draft
  acceptance rate apart from the useful output.

Readings where the pages leave a step open:

* Accepted drafts of a round are the emitted tokens that are drafts the
  verifier accepted.  The correction after a rejection and the bonus after a
  full acceptance are emitted but are not accepted drafts; an accepted EOS
  that ends the round is one.  ([TB]'s loop passes len(accepted), which
  holds the correction; [NW]'s table asks the two to be kept apart.)
* The monitor's rate is the sum of accepted drafts over the sum of drafted
  positions in the request's last ``window`` rounds (a ratio of sums).  With
  no drafted position in the window the rate is undefined and K is kept.
* The thresholds are the exact rationals 17/20 and 3/5, compared strictly.
* In a batch every request is its own sequence with its own monitor; its
  current K is the draft_len of the round just verified, and the next one is
  kept within [1, max_K].  A round that failed verification adds nothing to
  the window.
"""

from fractions import Fraction

import numpy as np

RAISE_ABOVE = Fraction(17, 20)      # [TB] "4. 实现逻辑": 0.85
LOWER_BELOW = Fraction(3, 5)        # [TB] "4. 实现逻辑": 0.60

TOTAL_FIELDS = ("requests", "errors", "drafted", "accepted", "emitted", "eos_stops",
                "full_accepts", "rejections")


def drafts_accepted(draft_tokens, draft_len, out_tokens, n_emitted):
    """Accepted drafts of one request's round, or -1 for a failed round.

    The first n_emitted - 1 emitted tokens are accepted drafts.  The last one
    is an accepted draft only when the round ended on an accepted EOS: it is
    then a drafted position whose output is the draft itself.  A correction
    never repeats the rejected draft, since the residual max(p - q, 0) is zero
    at a token whose acceptance ratio p/q was below one ([NW]
    "接受与拒绝怎样保住分布", eq. r(x)), and a bonus lies past the drafts.
    """
    nb, n = int(draft_len), int(n_emitted)
    if nb < 0 or n < 1 or n > nb + 1:
        return -1
    last = n - 1
    if last < nb and int(out_tokens[last]) == int(draft_tokens[last]):
        return n
    return n - 1


def round_stats(draft_tokens, draft_len, out_tokens, n_emitted):
    """Per-request accepted drafts and batch totals of one verified round.

    draft_tokens [B][K], draft_len [B], out_tokens [B][K+1], n_emitted [B].
    Totals (``TOTAL_FIELDS``): valid requests, failed ones, drafted positions,
    accepted drafts, emitted tokens, rounds ended by an accepted EOS, rounds
    that accepted every draft (and so drew a bonus), and rounds that ended in
    a rejection.
    """
    B = len(draft_len)
    K = np.asarray(draft_tokens).shape[1] if B else 0
    acc = np.full(B, -1, dtype=np.int64)
    tot = dict.fromkeys(TOTAL_FIELDS, 0)
    for b in range(B):
        nb, n = int(draft_len[b]), int(n_emitted[b])
        a = drafts_accepted(draft_tokens[b], nb, out_tokens[b], n) if nb <= K else -1
        acc[b] = a
        if a < 0:
            tot["errors"] += 1
            continue
        tot["requests"] += 1
        tot["drafted"] += nb
        tot["accepted"] += a
        tot["emitted"] += n
        if a == n:
            tot["eos_stops"] += 1
        elif a == nb:
            tot["full_accepts"] += 1
        else:
            tot["rejections"] += 1
    return acc, tot


def expected_tokens_given_rates(rates):
    """E[N] of one round whose drafted positions accept independently with
    rates beta_0, beta_1, ...: 1 + beta_0 + beta_0 beta_1 + ... (the sum of
    [NW] "好草稿也要算得便宜" with a rate per position).  The j-th draft is
    emitted as accepted when positions 0..j all accept; the final 1 is the
    correction or bonus.  An EOS stop is not modelled.
    """
    total, run = 1.0, 1.0
    for beta in rates:
        run *= float(beta)
        total += run
    return total


def expected_tokens_per_request(beta, draft_len):
    """E[N] of every request of a batch from its rates beta [B][K] (float32,
    -1 where undefined) over its drafted positions, as float32; -1 where
    draft_len is outside [0, K] or a drafted position has no rate."""
    beta = np.asarray(beta, dtype=np.float32)
    B, K = beta.shape
    out = np.full(B, -1.0, dtype=np.float32)
    for b in range(B):
        nb = int(draft_len[b])
        if nb < 0 or nb > K:
            continue
        rates = beta[b, :nb].astype(np.float64)
        if np.all(rates >= 0.0):
            out[b] = np.float32(expected_tokens_given_rates(rates))
    return out


def next_draft_length(accepted, drafted, k, max_k):
    """The draft length after a window holding ``accepted`` of ``drafted``
    drafts ([TB] "4. 实现逻辑": one more when the rate is above 0.85, one
    fewer when it is below 0.60).

    The rate a/d is compared with 17/20 and 3/5 by cross-multiplying the
    integers (20a > 17d raises, 5a < 3d lowers), so no rounding enters.  An
    empty window (d = 0) leaves k as it is.  The result lies in [1, max_k].
    """
    a, d = int(accepted), int(drafted)
    step = 0
    if d > 0:
        if RAISE_ABOVE.denominator * a > RAISE_ABOVE.numerator * d:
            step = 1
        elif LOWER_BELOW.denominator * a < LOWER_BELOW.numerator * d:
            step = -1
    return min(max(int(k) + step, 1), int(max_k))


class RateWindow:
    """The (accepted, drafted) counts of a request's last ``window`` rounds;
    the monitored rate is their ratio of sums ([TB] "4. 实现逻辑" keeps such a
    window of rounds per sequence)."""

    def __init__(self, window):
        if window < 1:
            raise ValueError("window must be >= 1")
        self.window = int(window)
        self.counts = []

    def push(self, accepted, drafted):
        """Record one round, dropping the oldest beyond the window."""
        self.counts = (self.counts + [(int(accepted), int(drafted))])[-self.window:]

    def totals(self):
        return sum(c[0] for c in self.counts), sum(c[1] for c in self.counts)

    def rate(self):
        """The window's rate as a Fraction, or None with no drafted position."""
        a, d = self.totals()
        return Fraction(a, d) if d > 0 else None


def monitor_round(monitors, draft_tokens, draft_len, out_tokens, n_emitted, max_k):
    """One batched round of the adaptive draft length: each request's window
    takes its round (failed rounds add nothing), then the next draft_len is
    next_draft_length of the request's draft_len under the window's counts.

    Returns (next_draft_len [B] int, rate [B] float64 with -1 where it is
    undefined).
    """
    acc, _ = round_stats(draft_tokens, draft_len, out_tokens, n_emitted)
    B = len(draft_len)
    nxt = np.zeros(B, dtype=np.int64)
    rate = np.full(B, -1.0)
    for b in range(B):
        if acc[b] >= 0:
            monitors[b].push(acc[b], draft_len[b])
        r = monitors[b].rate()
        if r is not None:
            rate[b] = float(r)                 # correctly rounded to float64
        nxt[b] = next_draft_length(*monitors[b].totals(), int(draft_len[b]), max_k)
    return nxt, rate
