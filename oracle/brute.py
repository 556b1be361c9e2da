"""Pure-Python second statement of the decode step, for tiny inputs only --
TEST INFRASTRUCTURE ONLY (same import rule as the rest of oracle/).

Each function reaches the same quantity as basiskv_ref by a different road,
so that a slip in either one (a dropped term, a transposed factor, a wrong
head or page index) makes the pins in tests/test_oracle.py disagree:

  route      projected queries (P q, Q q) dotted with the cached codes,
             instead of building the predicted Key;
  select     exhaustive search over all k-subsets for the valid top-k set
             with the smallest indices, instead of sorting;
  attend     explicit token loop with an unshifted softmax;
  compress   residual as k E - z_s (P E), instead of (k - z_s P) E;
  reconstruct  through the fused latent-to-output matrix B W_O, instead of
             decoding the Value first;
  rope       each pair's rotation as an explicit 2 x 2 matrix, applied to the
             query (transposed) instead of the Key: q . R(t) k = (R(t)^T q) . k.

Inputs are nested Python lists or numpy arrays of floats; all arithmetic is
Python float (IEEE double) in explicit loops.
"""

import itertools
import math


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def _matvec(m, v):
    """m: rows x cols (list of rows), v: cols -> rows."""
    return [_dot(row, v) for row in m]


def _vecmat(v, m):
    """v: rows, m: rows x cols -> cols."""
    cols = len(m[0])
    return [sum(v[i] * m[i][j] for i in range(len(v))) for j in range(cols)]


def route_page_scores(q_group, z, r, P_g, Q_g, rb, seq_len, page_size, n_pages_out):
    """Page scores via projected queries: logit = (P q)[:rb].z[:rb] + (Q q).r."""
    qz = [_matvec(P_g, list(qh)) for qh in q_group]  # each rb
    qr = [_matvec(Q_g, list(qh)) for qh in q_group]  # each rq
    scores = [-math.inf] * n_pages_out
    for t in range(seq_len):
        p = t // page_size
        if p >= n_pages_out:
            continue
        for h in range(len(q_group)):
            logit = _dot(qz[h], list(z[t][:rb])) + _dot(qr[h], list(r[t]))
            if logit > scores[p]:
                scores[p] = logit
    return scores


def select_pages(scores, n_pages, k):
    """Exhaustive top-k: among all subsets T of size min(k, n_pages) whose
    smallest score is >= the largest score outside T, the lexicographically
    smallest sorted index tuple; padded with -1."""
    m = min(k, n_pages)
    best = None
    for subset in itertools.combinations(range(n_pages), m):
        inside = min((scores[p] for p in subset), default=math.inf)
        outside = max((scores[p] for p in range(n_pages) if p not in subset), default=-math.inf)
        if inside >= outside:
            if best is None or subset < best:
                best = subset
    return list(best) + [-1] * (k - m)


def attend_group(q_group, kc, z, sel, seq_len, page_size, scale):
    """Explicit loop over the selected pages' valid tokens; softmax without a
    max shift (valid for the small logits of tiny tests)."""
    rv = len(z[0])
    out = []
    for qh in q_group:
        weights = []
        rows = []
        for p in sel:
            if p < 0:
                continue
            for t in range(p * page_size, min((p + 1) * page_size, seq_len)):
                weights.append(math.exp(scale * _dot(list(qh), list(kc[t]))))
                rows.append(list(z[t]))
        total = sum(weights)
        if total == 0.0:
            out.append([0.0] * rv)
            continue
        acc = [0.0] * rv
        for w, row in zip(weights, rows):
            for d in range(rv):
                acc[d] += (w / total) * row[d]
        out.append(acc)
    return out


def compress_token(k_vec, v_vec, A_g, P_g, E_g, rb, round_fn):
    """One token, one KV head: z = v A; r = k E - z_s[:rb] (P E)."""
    z = _vecmat(list(v_vec), A_g)
    z_s = [round_fn(x) for x in z]
    PE = [_vecmat(list(P_g[i]), E_g) for i in range(rb)]  # rb x rq
    kE = _vecmat(list(k_vec), E_g)
    # with r_b = 0 (a residual-only router) nothing is predicted from the latent
    zPE = _vecmat(z_s[:rb], PE) if rb > 0 else [0.0] * len(kE)
    r = [round_fn(a - b) for a, b in zip(kE, zPE)]
    return z_s, r


def reconstruct(u, Bf, W_O, group):
    """y = sum_h u_h M_h with the fused block M_h = Bf_{h//G} W_O[h*dh:(h+1)*dh]."""
    hq = len(u)
    dh = len(Bf[0][0])
    D = len(W_O[0])
    y = [0.0] * D
    for h in range(hq):
        Bg = Bf[h // group]
        block = [list(W_O[h * dh + d]) for d in range(dh)]
        M_h = [_vecmat(list(Bg[i]), block) for i in range(len(Bg))]  # rV x D
        contrib = _vecmat(list(u[h]), M_h)
        y = [a + b for a, b in zip(y, contrib)]
    return y


def attend_tokens(q_group, kc, z, tokens, scale):
    """Latent attention over an explicit token list (explicit loops, an
    unshifted softmax): for the recent-window pins, where the attended set is
    written as a per-token predicate instead of a list of pages."""
    G, rv = len(q_group), len(z[0])
    out = [[0.0] * rv for _ in range(G)]
    if not tokens:
        return out
    for h in range(G):
        w = [math.exp(scale * _dot(q_group[h], kc[t])) for t in tokens]
        tot = sum(w)
        for wi, t in zip(w, tokens):
            for d in range(rv):
                out[h][d] += wi / tot * z[t][d]
    return out


def rotate_pair_matrix(angle):
    """The 2 x 2 rotation [[cos, -sin], [sin, cos]] by ``angle``."""
    c, s = math.cos(angle), math.sin(angle)
    return [[c, -s], [s, c]]


def rope_unrotate_query(q, position, inv_freq):
    """R(t)^T q for a query q (list, dh) and a token position t: each pair
    (i, i + dh/2) multiplied by the transposed 2 x 2 rotation matrix."""
    half = len(q) // 2
    out = list(q)
    for i in range(half):
        m = rotate_pair_matrix(position * float(inv_freq[i]))
        a, b = q[i], q[i + half]
        out[i] = m[0][0] * a + m[1][0] * b
        out[i + half] = m[0][1] * a + m[1][1] * b
    return out


def route_page_scores_rope(q_group, z, r, P_g, Q_g, rb, seq_len, page_size, n_pages_out, inv_freq):
    """Page scores with RoPE via projected queries: for token t the query is
    turned back by t, R(t)^T q, and then projected onto the routing factors:
    logit = (P R(t)^T q)[:rb] . z[:rb] + (Q R(t)^T q) . r."""
    scores = [-math.inf] * n_pages_out
    for t in range(seq_len):
        p = t // page_size
        if p >= n_pages_out:
            continue
        for qh in q_group:
            qt = rope_unrotate_query(list(qh), t, inv_freq)
            logit = (_dot(_matvec(P_g, qt), list(z[t][:rb])) if rb else 0.0) + \
                (_dot(_matvec(Q_g, qt), list(r[t])) if len(r[t]) else 0.0)
            if logit > scores[p]:
                scores[p] = logit
    return scores


def attend_tokens_rope(q_group, kc, z, tokens, scale, inv_freq):
    """Latent attention over an explicit token list with RoPE: each query
    turned back by the token's position (R(t)^T q) and dotted with the
    pre-RoPE Key, explicit loops, an unshifted softmax."""
    G, rv = len(q_group), len(z[0])
    out = [[0.0] * rv for _ in range(G)]
    if not tokens:
        return out
    for h in range(G):
        w = [math.exp(scale * _dot(rope_unrotate_query(list(q_group[h]), t, inv_freq), kc[t]))
             for t in tokens]
        tot = sum(w)
        for wi, t in zip(w, tokens):
            for d in range(rv):
                out[h][d] += wi / tot * z[t][d]
    return out
