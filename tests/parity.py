"""Compare the HIP path's outputs with the oracle's, request by request.

A request the oracle flags (see the oracle's module docstring) is compared
only on what stays certain: tokens before an uncertain accept test, or
everything but the drawn token when only the final draw is uncertain.
"""

import numpy as np

import oracle as O


def flag_ceiling(positions):
    """The most flagged requests one parity case may have: the flag budget of
    1e-4 of the verified positions, plus one.  An oracle that flags too much
    would otherwise let parity pass on the few decisions left to compare."""
    return 1 + int(1e-4 * positions)


def to_numpy(res):
    return {k: v.detach().cpu().numpy() for k, v in res.items()}


def compare(gpu, ora, K, alpha_tol=1e-5, mass_tol=1e-5, check_flags=True):
    """Return a report dict; ``report['mismatches']`` lists every failure.

    With ``check_flags`` more than flag_ceiling(positions) flagged requests
    is a failure too (cases that force near-ties on purpose turn it off)."""
    out_g, n_g = gpu["out_tokens"], gpu["n_emitted"]
    rep = {"requests": 0, "flagged": 0, "positions": 0, "mismatches": [], "flag_kinds": {},
           "max_alpha_err": 0.0, "max_mass_err": 0.0}
    for b in np.flatnonzero(ora["evaluated"]):
        rep["requests"] += 1
        n_o = int(ora["n_emitted"][b])
        row_o, row_g = ora["out_tokens"][b], out_g[b]
        if n_o == -1:
            if n_g[b] != -1 or not np.all(row_g == -1):
                rep["mismatches"].append((int(b), "error request", int(n_g[b]), row_g.tolist()))
            continue
        fk, fp = int(ora["flag_kind"][b]), int(ora["flag_pos"][b])
        stop = int(ora["stop_pos"][b])
        nb_used = int(np.sum(~np.isnan(ora["alpha"][b])))
        rep["positions"] += nb_used
        if fk != O.FLAG_NONE:
            rep["flagged"] += 1
            rep["flag_kinds"][fk] = rep["flag_kinds"].get(fk, 0) + 1
        if fk == O.FLAG_NONE:
            ok = n_g[b] == n_o and np.array_equal(row_g, row_o)
            if ok and "stop_pos" in gpu:
                ok = gpu["stop_pos"][b] == stop and gpu["path"][b] == ora["path"][b]
        elif fk in (O.FLAG_ACCEPT, O.FLAG_TOPP):
            ok = np.array_equal(row_g[:fp], row_o[:fp])
        else:                                   # only the final draw is uncertain
            keep = np.ones(K + 1, dtype=bool)
            keep[fp] = False
            ok = n_g[b] == n_o and np.array_equal(row_g[keep], row_o[keep])
        if not ok:
            rep["mismatches"].append((int(b), f"tokens (flag {fk}@{fp})", row_g.tolist(),
                                      row_o.tolist(), int(n_g[b]), n_o))
        if "accept_prob" in gpu:
            a_o = ora["alpha"][b, :nb_used]
            a_g = gpu["accept_prob"][b, :nb_used].astype(np.float64)
            margins = ora["topp_margin_rows"][b]
            use = np.array([min(margins[k], margins[K + 1 + k]) >= O.TOPP_FLAG_ABS
                            for k in range(nb_used)], dtype=bool)
            if use.any():
                err = float(np.max(np.abs(a_g[use] - a_o[use])))
                rep["max_alpha_err"] = max(rep["max_alpha_err"], err)
                if err > alpha_tol:
                    rep["mismatches"].append((int(b), "alpha", a_g.tolist(), a_o.tolist()))
            if ora["path"][b] == O.PATH_REJECT and gpu["path"][b] == O.PATH_REJECT \
                    and gpu["stop_pos"][b] == stop:
                err = abs(float(gpu["residual_mass"][b]) - float(ora["residual_mass"][b]))
                rep["max_mass_err"] = max(rep["max_mass_err"], err)
                if err > mass_tol:
                    rep["mismatches"].append((int(b), "residual mass", float(gpu["residual_mass"][b]),
                                              float(ora["residual_mass"][b])))
    if check_flags and rep["flagged"] > flag_ceiling(rep["positions"]):
        rep["mismatches"].append(("flag budget", rep["flagged"], rep["positions"],
                                  rep["flag_kinds"]))
    return rep
