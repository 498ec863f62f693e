"""fp64 reference for one batched speculative-decoding verification call.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain numpy, float64,
one request at a time, no blocking or fusion beyond what the definitions say.

Citation labels: [TB] tbxsx.cn report "推测解码采样验证优化策略 —— 深度调研报告";
[NW] nickwang.xyz notes "推测解码：草稿、验证与实际加速"; [BZ] bowenzhou.top
notes "投机采样".

Readings taken where the pages are silent or disagree (each is also listed in
the design notes of the repository):

* Accept test is strict ``u < alpha`` ([NW] replay code) rather than the
  ``u <= alpha`` of the [TB] pseudo-code: with u in [0, 1) the strict test
  accepts with probability exactly alpha and never accepts a token with p = 0.
* A bonus token is drawn from the target row after the last draft when every
  draft is accepted ([NW] "候选已知，验证才能并行"; [BZ] n in [1, gamma+1]);
  the [TB] pseudo-code omits it.  With ragged draft lengths the bonus row is
  target row ``draft_len[b]``.
* One final uniform per request feeds whichever draw happens (residual or
  bonus), as in the [NW] replay; uniforms after the first rejection are unused.
* Inverse-CDF sampling walks token ids in ascending order and returns the
  first id whose running sum exceeds ``t = u * total`` (strict, [NW]
  ``sample()``).  If rounding leaves no such id, the last id with positive
  weight is returned instead of raising.
* Temperature divides the logits before both filters.  top-k keeps every
  logit >= the k-th largest (ties kept); top-p then acts on the renormalised
  top-k distribution, keeps the shortest prefix (by logit descending, id
  ascending) whose cumulative mass reaches top_p, including the crossing token
  and every logit tied with it.  The same procedure is applied separately to
  the target row and to the draft row ([NW] "接受与拒绝怎样保住分布": p and q are
  both the processed distributions actually used).
* EOS stops the round right after the first emitted EOS, whether it was an
  accepted draft or the drawn token; no bonus follows ([NW] "候选已知，
  验证才能并行" says EOS may end a round early).
* Precondition violations ([NW] replay asserts q(x) > 0 and 0 <= u < 1):
  draft_len outside [0, K], a draft token outside [0, V), q(x) == 0, a uniform
  outside [0, 1) or a row with no finite logit make the request an error:
  n_emitted = -1 and its out_tokens row stays -1.
* Flags mark decisions that a correct implementation with different rounding
  may legitimately take the other way: an accept test with
  |u - alpha| <= 1e-5 * alpha; a final draw whose t lies within 1e-10 * total
  of either edge of the chosen token's CDF interval; a top-p cut whose
  cumulative mass lies within 1e-10 of top_p.
"""

import numpy as np

ACCEPT_FLAG_REL = 1e-5
CDF_FLAG_REL = 1e-10
TOPP_FLAG_ABS = 1e-10

PATH_ERROR, PATH_REJECT, PATH_BONUS, PATH_EOS = -1, 0, 1, 2
FLAG_NONE, FLAG_ACCEPT, FLAG_CDF, FLAG_TOPP, FLAG_EMPTY_RESIDUAL = 0, 1, 2, 3, 4


def widen_row(row, dtype):
    """Widen one row of logits to float64 exactly.

    bf16 rows arrive as uint16 bit patterns (numpy has no bf16 type): the bits
    are the top half of the float32 with the same value.
    """
    if dtype == "bf16":
        bits = np.asarray(row, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(row).astype(np.float64)


def topk_threshold(z, k):
    """The k-th largest entry of z, counting repeated values; -inf when k is 0 or >= len(z)."""
    V = z.shape[0]
    if k <= 0 or k >= V:
        return -np.inf
    return float(np.partition(z, V - k)[V - k])


def processed_distribution(z, temperature, top_k=0, top_p=1.0):
    """Target or draft distribution after temperature, top-k and top-p.

    [TB] "4. 实现逻辑": softmax of logits / temperature.  [NW]
    "接受与拒绝怎样保住分布": p and q already include temperature, top-k and
    top-p.  Returns ``(P, info)``; ``P`` is None when no finite logit is left.
    ``info['topp_margin']`` is the distance of the top-p crossing from top_p.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    info = {"tau_k": -np.inf, "tau_p": -np.inf, "topp_margin": np.inf, "m": np.nan}
    kept = z > -np.inf
    tau_k = topk_threshold(z, top_k)
    info["tau_k"] = tau_k
    if tau_k > -np.inf:
        kept &= z >= tau_k
    if not kept.any():
        return None, info
    m = z[kept].max()
    info["m"] = m
    w = np.zeros(V, dtype=np.float64)
    w[kept] = np.exp((z[kept] - m) / temperature)
    if top_p < 1.0:
        idx = np.flatnonzero(kept)
        order = idx[np.lexsort((idx, -z[idx]))]      # logit descending, id ascending
        running = np.cumsum(w[order])
        c = running / running[-1]
        M = int(np.argmax(c >= top_p))               # first prefix reaching top_p
        tau_p = z[order[M]]
        margin = c[M] - top_p
        if M > 0:
            margin = min(margin, top_p - c[M - 1])
        kept &= z >= tau_p
        w[~kept] = 0.0
        info["tau_p"] = tau_p
        info["topp_margin"] = float(margin)
    info["kept"] = kept
    return w / w.sum(), info


def _one_like(v):
    return v * 0 + 1


def accept_prob(P, Q, x):
    """alpha(x) = min(1, p(x) / q(x)).

    [NW] "接受与拒绝怎样保住分布" eq. a(x); [TB] formula 1 (the minimum of one
    and the probability ratio); [BZ] "机制：起草-验证-接受".  Works on float
    arrays and on arrays of Fractions.  The caller guarantees q(x) > 0.
    """
    ratio = P[x] / Q[x]
    one = _one_like(ratio)
    return ratio if ratio < one else one


def residual(P, Q):
    """Unnormalised correction distribution max(p - q, 0).

    [NW] eq. r(x) (normalised by its own sum, which equals 1 - sum min(p, q));
    [TB] formula 4; [BZ] "深入推导".
    """
    diff = P - Q
    return np.maximum(diff, diff * 0)


def icdf(w, u):
    """Inverse-CDF draw from unnormalised weights w at a uniform u in [0, 1).

    [NW] ``sample()`` in "算完三个 token 的全部概率": walk ids in order and return
    the first whose running sum exceeds the draw.  Here the draw is scaled by
    the total, t = u * sum(w), so w need not be normalised.  Returns
    ``(y, margin)`` where margin is the distance of t from the nearer edge of
    y's interval, relative to the total.
    """
    C = np.cumsum(w)
    total = C[-1]
    t = u * total
    hit = t < C
    if hit.any():
        y = int(np.argmax(hit))
    else:                                            # rounding fall-through
        y = int(np.flatnonzero(np.asarray(w) > 0)[-1])
    lo = C[y - 1] if y > 0 else total * 0
    margin = min(t - lo, C[y] - t) / total
    return y, float(margin)


def acceptance_rate(P, Q):
    """beta = sum_x min(p(x), q(x)), the probability that a token drawn from
    q is accepted for a fixed prefix.

    [NW] "好草稿也要算得便宜" (the acceptance rate of a fixed prefix); the same
    page's worked example sums the directly accepted mass to 0.8.  Works on
    float arrays and on arrays of Fractions.
    """
    return np.minimum(P, Q).sum()


def acceptance_rates(target, draft, draft_len, temperature, top_k=0, top_p=1.0, dtype="f32"):
    """beta[b][k] = acceptance_rate(p_k, q_k) of every drafted position.

    p_k and q_k are the processed distributions of target row k and draft
    row k (the same ones verify() uses).  Positions at or after draft_len[b],
    requests whose draft_len lies outside [0, K], and positions whose target
    or draft row has no finite logit read -1.
    """
    B, K1, V = target.shape
    K = K1 - 1
    beta = np.full((B, K), -1.0)
    for b in range(B):
        nb = int(draft_len[b])
        if not 0 <= nb <= K:
            continue
        for k in range(nb):
            zt = widen_row(target[b, k], dtype)
            zd = widen_row(draft[b, k], dtype)
            if not (np.isfinite(zt).any() and np.isfinite(zd).any()):
                continue
            P, _ = processed_distribution(zt, temperature, top_k, top_p)
            Q, _ = processed_distribution(zd, temperature, top_k, top_p)
            if P is None or Q is None:
                continue
            beta[b, k] = float(acceptance_rate(P, Q))
    return beta


def expected_tokens_per_round(alpha, gamma):
    """E[N] = 1 + alpha + ... + alpha^gamma under i.i.d. acceptance.

    [NW] "好草稿也要算得便宜"; [BZ] "收益账" gives the same sum in closed form.
    """
    return sum(alpha ** j for j in range(gamma + 1))


def verify(target, draft, draft_tokens, draft_len, u, u_final, temperature,
           top_k=0, top_p=1.0, eos_id=-1, dtype="f32", requests=None):
    """One verification call, request by request.

    target: [B, K+1, V] logits; draft: [B, K, V]; bf16 tensors are given as
    uint16 bit patterns with ``dtype="bf16"``.  draft_tokens [B, K] and
    draft_len [B] are integers; u [B, K] and u_final [B] are float32 uniforms.
    ``requests`` restricts the work to some request ids (others are left with
    ``evaluated == False``).

    Target row k verifies draft token k; target row draft_len[b] supplies the
    bonus ([NW] "候选已知，验证才能并行").  The scan accepts left to right and
    stops at the first rejection, drawing the correction from
    max(p - q, 0) ([TB] ``_sampling_verification``; [NW] replay; [BZ]
    "机制：起草-验证-接受").
    """
    draft_tokens = np.asarray(draft_tokens)
    draft_len = np.asarray(draft_len)
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    u_final = np.asarray(u_final, dtype=np.float32).astype(np.float64)
    B = draft_tokens.shape[0]
    K = draft_tokens.shape[1]
    V = target.shape[2]
    T = float(temperature)

    res = {
        "out_tokens": np.full((B, K + 1), -1, dtype=np.int32),
        "n_emitted": np.full(B, -1, dtype=np.int32),
        "alpha": np.full((B, K), np.nan, dtype=np.float64),
        "residual_mass": np.zeros(B, dtype=np.float64),
        "stop_pos": np.full(B, -1, dtype=np.int32),
        "path": np.full(B, PATH_ERROR, dtype=np.int32),
        "flag_kind": np.zeros(B, dtype=np.int32),
        "flag_pos": np.full(B, -1, dtype=np.int32),
        "topp_margin_rows": np.full((B, 2 * K + 1), np.inf),
        "evaluated": np.zeros(B, dtype=bool),
    }
    reqs = range(B) if requests is None else requests
    for b in reqs:
        res["evaluated"][b] = True
        _verify_one(res, b, target, draft, draft_tokens, draft_len, u, u_final,
                    T, top_k, top_p, eos_id, dtype, K, V)
    return res


def _verify_one(res, b, target, draft, draft_tokens, draft_len, u, u_final,
                T, top_k, top_p, eos_id, dtype, K, V):
    nb = int(draft_len[b])
    uf = float(u_final[b])
    if not (0 <= nb <= K) or not (0.0 <= uf < 1.0):
        return
    P, Q = [], []
    for k in range(nb + 1):
        Pk, info = processed_distribution(widen_row(target[b, k], dtype), T, top_k, top_p)
        if Pk is None:
            return
        res["topp_margin_rows"][b, k] = info["topp_margin"]
        P.append(Pk)
    for k in range(nb):
        Qk, info = processed_distribution(widen_row(draft[b, k], dtype), T, top_k, top_p)
        if Qk is None:
            return
        res["topp_margin_rows"][b, K + 1 + k] = info["topp_margin"]
        Q.append(Qk)

    alphas = []
    for k in range(nb):
        x = int(draft_tokens[b, k])
        uk = u[b, k]
        if not (0 <= x < V) or not (0.0 <= uk < 1.0) or not Q[k][x] > 0.0:
            res["alpha"][b, :] = np.nan
            return
        alphas.append(float(accept_prob(P[k], Q[k], x)))
    res["alpha"][b, :nb] = alphas

    out = res["out_tokens"][b]
    stop = nb
    path = PATH_BONUS
    for k in range(nb):
        x = int(draft_tokens[b, k])
        if u[b, k] < alphas[k]:
            out[k] = x
            if x == eos_id:
                stop, path = k, PATH_EOS
                break
        else:
            stop, path = k, PATH_REJECT
            break

    flag_kind, flag_pos = FLAG_NONE, -1
    last_decided = min(stop, nb - 1)
    for k in range(last_decided + 1):
        topp_rows = (res["topp_margin_rows"][b, k], res["topp_margin_rows"][b, K + 1 + k])
        if min(topp_rows) < TOPP_FLAG_ABS:
            flag_kind, flag_pos = FLAG_TOPP, k
            break
        if abs(u[b, k] - alphas[k]) <= ACCEPT_FLAG_REL * alphas[k]:
            flag_kind, flag_pos = FLAG_ACCEPT, k
            break

    if path == PATH_REJECT:
        r = residual(P[stop], Q[stop])
        s_r = float(r.sum())
        res["residual_mass"][b] = s_r
        weights = r
        if not s_r > 0.0:                     # unreachable in exact arithmetic
            weights = P[stop]
            if flag_kind == FLAG_NONE:
                flag_kind, flag_pos = FLAG_EMPTY_RESIDUAL, stop
        y, margin = icdf(weights, uf)
        out[stop] = y
    elif path == PATH_BONUS:
        if flag_kind == FLAG_NONE and res["topp_margin_rows"][b, nb] < TOPP_FLAG_ABS:
            flag_kind, flag_pos = FLAG_TOPP, nb
        y, margin = icdf(P[nb], uf)
        out[nb] = y
    else:
        margin = np.inf
    if flag_kind == FLAG_NONE and margin < CDF_FLAG_REL:
        flag_kind, flag_pos = FLAG_CDF, stop

    res["n_emitted"][b] = stop + 1
    res["stop_pos"][b] = stop
    res["path"][b] = path
    res["flag_kind"][b] = flag_kind
    res["flag_pos"][b] = flag_pos
