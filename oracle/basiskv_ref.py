"""float64 CPU oracle for one BasisKV decode step -- TEST INFRASTRUCTURE ONLY.

Source: "BasisKV: Value Latents for Communication and Key Routing"
(arXiv 2611.02583).  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the product path never does.

What is cached per token and per physical KV head (appendix Table 4):
  z  Value latent, width rV   (the full Value is not cached)
  r  Key residual code, width rq
  k  exact Key, width dh
Routing reads rb <= rV leading latent dims plus the rq residual dims of every
context token; selected attention reads all rV latent dims and the dh Key dims
of the selected tokens only (Table 4's two read columns).

Array conventions (all "logical", i.e. contiguous per sequence, no pages):
  q   [B, Hq, dh]            queries of the step
  z   [B, Hkv, T, rV]        latent cache
  r   [B, Hkv, T, rq]        residual cache
  kc  [B, Hkv, T, dh]        exact-Key cache
  A   [Hkv, dh, rV]          Value encoder  (z = v A)
  Bf  [Hkv, rV, dh]          Value decoder  (v_hat = z Bf)
  P   [Hkv, rb, dh]          latent -> Key predictor
  Q   [Hkv, rq, dh]          residual -> Key decoder
  E   [Hkv, dh, rq]          residual encoder
  W_O [Hq*dh, D]             output projection, y = concat_h(v_h) W_O
Query head h belongs to KV head h // G with G = Hq / Hkv.

Every value is float64.  Stored inputs are decoded exactly
(storage_to_f64); the only roundings are the ones the method itself performs
when it writes the cache (compress) and, optionally, the final output store.

Readings of points the pages leave open (each used below):
  R1 token -> page score: the maximum predicted logit over the page's valid
     tokens;  R2 the KV head's page score is also the maximum over its G query
     heads;  R3 query head h uses KV head h // G;  R4 routing logits are
     unscaled (top-k is invariant to a positive scale);  R5 attention scale is
     1/sqrt(dh) unless the caller passes another;  R6 the routing base is the
     leading rb latent dims;  R7 residual code r = (k - z_s[:rb] P) E with the
     stored (rounded) latent z_s;  R8 the softmax is normalised over the valid
     tokens of the selected pages only;  R9 ties in page score go to the lower
     page index, the selection is reported in ascending page order and padded
     with -1 when k exceeds the number of pages;  R10 a sequence with no valid
     token yields u = 0 and y = 0;  R11 a recent window of W tokens (the
     pages' adopted router: 64 recent tokens besides the routed budget) is
     taken page by page: the pages holding the last W valid tokens are always
     attended, and the top-k routed pages are chosen among the pages before
     them;  R12 an FP8 cache (appendix Table 13: E4M3) holds the OCP E4M3FN
     code of each value with no scale factor (scale 1): exponent bias 7,
     3 mantissa bits, largest finite magnitude 448, subnormal step 2**-9, no
     infinities; writes round to nearest even and saturate to +-448 instead
     of producing the NaN code;  R13 rotary position embedding (RoPE; the
     Figure 6 caption of the pages measures how well the latent explains
     the *pre-RoPE* Key): every cached state is pre-RoPE (latent, residual
     and exact Key), queries come already rotated at their own position, and
     both the predicted Key (routing) and the exact Key (attention) of the
     token at position t (its index in the sequence) are rotated to t before
     the dot product.  Rotation: rotate-half pairs (i, i + dh/2), angle
     t * w_i taken exactly, w_i the caller's float32 inverse frequencies
     (w_i = base**(-2i/dh) for the standard embedding).
"""

import math

import numpy as np

_STORAGES = ("f32", "bf16", "fp8", "f64")


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def storage_to_f64(a, storage):
    """Decode stored values to float64, exactly.

    ``storage`` is "f32" (float32 array), "bf16" (uint16 bit patterns: the
    upper half of an IEEE float32), "fp8" (uint8 E4M3FN codes, reading R12)
    or "f64" (no storage rounding; used by the exactness pins).
    """
    if storage == "f64":
        return np.asarray(a, dtype=np.float64)
    if storage == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if storage == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if storage == "fp8":
        return _e4m3_decode(np.asarray(a, dtype=np.uint8))
    raise ValueError(f"unknown storage {storage!r}")


def _e4m3_decode(codes):
    """E4M3FN code -> value (R12): sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent field 0 is subnormal (m * 2**-9); the two
    codes with every exponent and mantissa bit set are NaN."""
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def round_to_storage(x, storage):
    """Round float64 values to the storage format, round-to-nearest-even.

    Returns the rounded values as float64.  For bf16 (8 significant bits) the
    quantum of a value with frexp exponent e is 2**(e-8); dividing by it is
    exact, numpy's round() is round-half-even, and the smallest normal's
    quantum (2**-133) is kept below it (subnormals).  Values past the bf16
    range become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    if storage == "f64":
        return x.copy()
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)
    if storage == "fp8":
        return _round_e4m3(x)
    if storage != "bf16":
        raise ValueError(f"unknown storage {storage!r}")
    out = np.zeros_like(x)
    nz = x != 0
    xs = x[nz]
    _, e = np.frexp(xs)
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    rounded = np.round(xs / quantum) * quantum
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    rounded = np.where(np.abs(rounded) > bf16_max, np.copysign(np.inf, rounded), rounded)
    out[nz] = rounded
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def _round_e4m3(x):
    """Nearest E4M3FN value, ties to even, saturating at +-448 (R12).

    E4M3 carries 4 significant bits, so a value with frexp exponent e has the
    quantum 2**(e-4); below the smallest normal (2**-6, frexp exponent -5) the
    quantum stays 2**-9 (subnormals).  NaN stays NaN; +-inf saturates.
    """
    out = np.zeros_like(x)
    nz = (x != 0) & ~np.isnan(x)
    xs = np.clip(x[nz], -448.0, 448.0)
    _, e = np.frexp(xs)
    quantum = np.ldexp(1.0, np.maximum(e, -5) - 4)
    out[nz] = np.clip(np.round(xs / quantum) * quantum, -448.0, 448.0)
    out[np.isnan(x)] = np.nan
    out[x == 0] = x[x == 0]
    return out


# ---------------------------------------------------------------------------
# (a0) compression of new tokens into the cache
# ---------------------------------------------------------------------------

def compress_tokens(k_new, v_new, A, P, E, rb, storage):
    """Compress tokens' Keys and Values into the three cached states.

    BasisKV abstract: Values are stored only as a low-rank latent, and a
    Key-specific residual keeps the part of the Key that the latent cannot
    predict; appendix Table 4 lists the three per-token states (latent rV,
    residual rq, exact Key dh).

    k_new, v_new: [n, Hkv, dh] float64.  Returns (z_s, r_s, k_s), each
    [n, Hkv, width], already rounded to ``storage`` (z_s: rV, r_s: rq,
    k_s: dh).  Steps: z = v A_g; z_s = round(z); r = (k - z_s[:, :rb] P_g) E_g
    (reading R7); r_s = round(r); the exact Key is stored as given.
    """
    n, hkv, dh = k_new.shape
    z_s = np.empty((n, hkv, A.shape[2]))
    r_s = np.empty((n, hkv, E.shape[2]))
    for g in range(hkv):
        z_s[:, g, :] = round_to_storage(latent_code(v_new[:, g, :], A[g]), storage)
        r_s[:, g, :] = round_to_storage(residual_code(k_new[:, g, :], z_s[:, g, :], P[g], E[g], rb),
                                        storage)
    k_s = round_to_storage(k_new, storage)
    return z_s, r_s, k_s


def latent_code(v, A_g):
    """Unrounded Value latent z = v A_g of rows v [n, dh] (abstract: the Value
    is kept only as a low-rank latent)."""
    return v @ A_g


def residual_code(k, z_s, P_g, E_g, rb):
    """Unrounded residual code r = (k - z_s[:, :rb] P_g) E_g of rows k [n, dh]
    given their stored latents z_s [n, rV] (reading R7: the part of the Key the
    latent's leading rb dims do not predict, encoded with E_g)."""
    return (k - z_s[:, :rb] @ P_g) @ E_g


# ---------------------------------------------------------------------------
# rotary position embedding (reading R13)
# ---------------------------------------------------------------------------

def rope_rotate(x, positions, inv_freq):
    """Rows x [n, dh] rotated to their positions [n] (R13): for each pair
    (i, i + dh/2), angle phi = position * w_i (float64: exact for positions
    below 2**24 and float32 frequencies),
      x_i' = x_i cos(phi) - x_{i+dh/2} sin(phi),
      x_{i+dh/2}' = x_i sin(phi) + x_{i+dh/2} cos(phi).
    inv_freq None: no rotation."""
    x = np.asarray(x, dtype=np.float64)
    if inv_freq is None:
        return x
    half = x.shape[-1] // 2
    w = np.asarray(inv_freq, dtype=np.float32).astype(np.float64)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * w[None, :]
    c, s_ = np.cos(phi), np.sin(phi)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s_, lo * s_ + hi * c], axis=-1)


def rope_inverse_frequencies(head_dim, base):
    """Standard RoPE frequencies w_i = base**(-2i/dh) as float32."""
    return (float(base) ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)).astype(np.float32)


# ---------------------------------------------------------------------------
# (a1, a2) routing: predicted keys and page scores
# ---------------------------------------------------------------------------

def predicted_keys(z, r, P_g, Q_g, rb):
    """Predicted Keys of a token range for one KV head.

    BasisKV abstract and Figure 1 caption: the cached Value latent predicts
    part of the Key used for routing and the Key residual supplies the rest.
    k_hat_t = z_t[:rb] P_g + r_t Q_g, as an explicit dh-vector (reading R6).
    z: [T, rV], r: [T, rq]  ->  [T, dh].
    """
    return z[:, :rb] @ P_g + r @ Q_g


def route_page_scores(q_group, z, r, P_g, Q_g, rb, seq_len, page_size, n_pages_out,
                      inv_freq=None):
    """Page scores of one (sequence, KV head).

    BasisKV abstract: the predicted Key information decides which Key pages
    are read; Table 9's caption fixes the routing unit as a page of tokens.
    For every valid token t and query head h of the group, the routing logit
    is q_h . k_hat_t (unscaled, R4); a page's score is the maximum over its
    valid tokens and the group's heads (R1, R2).  Pages at or beyond
    ceil(seq_len / page_size) get -inf.  With inv_freq the predicted Key of
    token t is rotated to position t first (R13).  Returns [n_pages_out]
    float64.
    """
    scores = np.full(n_pages_out, -np.inf)
    if seq_len <= 0:
        return scores
    khat = predicted_keys(z[:seq_len], r[:seq_len], P_g, Q_g, rb)
    khat = rope_rotate(khat, np.arange(seq_len), inv_freq)
    logits = q_group @ khat.T  # [G, seq_len]
    n_pages = -(-seq_len // page_size)
    for p in range(min(n_pages, n_pages_out)):
        lo, hi = p * page_size, min((p + 1) * page_size, seq_len)
        scores[p] = logits[:, lo:hi].max()
    return scores


# ---------------------------------------------------------------------------
# (a3) page selection
# ---------------------------------------------------------------------------

def select_pages(scores, n_pages, k):
    """The k highest-scoring pages among the first n_pages, ascending.

    BasisKV abstract: only the selected pages' original Keys are fetched.
    Ties go to the lower page index and the result is padded with -1 when
    k > n_pages (reading R9).  Pure-Python ordering by (-score, index).
    """
    n_pages = max(0, int(n_pages))
    order = sorted(range(n_pages), key=lambda p: (-float(scores[p]), p))
    chosen = sorted(order[:k])
    return np.array(chosen + [-1] * (k - len(chosen)), dtype=np.int64)


def recent_window_first_page(seq_len, page_size, recent_tokens):
    """First page of the recent window (reading R11): the pages from here to
    the last valid page hold the last ``recent_tokens`` valid tokens and are
    attended whatever their score; routing picks among the pages before.
    Appendix Table 9 caption: the sparse routers keep 64 recent tokens beside
    the routed budget.  Without a window this is the number of valid pages."""
    L = max(0, int(seq_len))
    if recent_tokens <= 0:
        return -(-L // page_size)
    return max(0, L - int(recent_tokens)) // page_size


def selected_tokens(sel, seq_len, page_size):
    """Token positions covered by the selected pages (valid ones only)."""
    toks = []
    for p in sel:
        if p < 0:
            continue
        lo = p * page_size
        toks.extend(range(lo, min(lo + page_size, seq_len)))
    return np.array(toks, dtype=np.int64)


# ---------------------------------------------------------------------------
# (a4) exact attention over the selected pages, summed in latent space
# ---------------------------------------------------------------------------

def attend_group(q_group, kc, z, sel, seq_len, page_size, scale, inv_freq=None):
    """Latent attention output of one KV head's query group.

    BasisKV abstract: exact QK scores are computed from the original Keys of
    the selected pages; Figure 1 caption: the attention output is formed as a
    Value latent (the weighted sum runs over the cached latents, all rV
    dims, appendix Table 4 "selected attention").  For each head h:
    s_t = scale * q_h . k_t over the valid tokens of the selected pages,
    p = softmax(s) over those tokens only (R8), u_h = sum_t p_t z_t.
    q_group [G, dh], kc [T, dh], z [T, rV]  ->  [G, rV].
    """
    toks = selected_tokens(sel, seq_len, page_size)
    if toks.size == 0:
        return np.zeros((q_group.shape[0], z.shape[1]))
    keys = rope_rotate(kc[toks], toks, inv_freq)  # R13: each Key at its position
    s = scale * (q_group @ keys.T)  # [G, n]
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ z[toks]


def dense_attention(q_group, k, v, seq_len, scale):
    """Dense decode attention, the baseline the pages' Table 3 compares with:
    o_h = softmax(scale * q_h . k_t over the valid tokens) weighted sum of the
    Values v_t.  q_group [G, dh], k, v [T, dh] -> [G, dh]; zeros when the
    sequence is empty."""
    L = max(0, int(seq_len))
    if L == 0:
        return np.zeros((q_group.shape[0], v.shape[1]))
    s = scale * (q_group @ k[:L].T)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return (w / w.sum(axis=1, keepdims=True)) @ v[:L]


# ---------------------------------------------------------------------------
# (a5) reconstruction through the Value decoder and the output projection
# ---------------------------------------------------------------------------

def reconstruct(u, Bf, W_O, group):
    """Output of one sequence from the per-head latents.

    BasisKV abstract: Value compression is tied to the output projection;
    Figure 1 caption: the full output is rebuilt from the latents after they
    are exchanged.  Definition (unfused): v_h = u_h Bf_{h // G}, then
    y = concat_h(v_h) W_O.  u [Hq, rV], Bf [Hkv, rV, dh], W_O [Hq*dh, D].
    """
    hq = u.shape[0]
    v = np.stack([u[h] @ Bf[h // group] for h in range(hq)])  # [Hq, dh]
    return v.reshape(-1) @ W_O


# ---------------------------------------------------------------------------
# one decode step
# ---------------------------------------------------------------------------

def decode_step(q, z, r, kc, seq_lens, A, Bf, P, Q, E, W_O, *, rb, page_size,
                top_k, n_pages_out, storage, scale=None, k_new=None, v_new=None,
                store_output=True, recent_tokens=0, cache_storage=None, rope_inv_freq=None):
    """One decode step of one layer for a batch.

    Inputs are float64 (decode stored values with storage_to_f64 first);
    ``storage`` names the format of the output store ("f32", "bf16",
    "f64") and ``cache_storage`` (default: ``storage``) the one the cache is
    written in (also "fp8", R12).  If k_new / v_new ([B, Hkv, dh]) are given, the step first
    compresses that token into position seq_lens[b] - 1 of each sequence
    (a0); then it routes (a1, a2), selects (a3), attends (a4) and
    reconstructs (a5).  With recent_tokens > 0 the top-k pages are chosen
    before the recent window and the window's pages are attended as well
    (R11); ``sel`` holds the routed pages only.  With rope_inv_freq the
    cached Keys are pre-RoPE and rotated to their positions (R13).  Arrays
    z, r, kc are copied, not modified.

    Returns a dict: scores [B, Hkv, n_pages_out], sel [B, Hkv, top_k],
    u [B, Hq, rV], y [B, D] (float64, unrounded), y_stored (y rounded to
    ``storage`` when store_output), and z, r, kc (the caches after the
    append).
    """
    bsz, hq, dh = q.shape
    hkv = z.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    z = np.array(z, dtype=np.float64, copy=True)
    r = np.array(r, dtype=np.float64, copy=True)
    kc = np.array(kc, dtype=np.float64, copy=True)
    if k_new is not None:
        for b in range(bsz):
            pos = int(seq_lens[b]) - 1
            if pos < 0 or pos >= z.shape[2]:
                continue
            zs, rs, ks = compress_tokens(k_new[b:b + 1], v_new[b:b + 1], A, P, E, rb,
                                         cache_storage or storage)
            z[b, :, pos, :] = zs[0]
            r[b, :, pos, :] = rs[0]
            kc[b, :, pos, :] = ks[0]

    rv = z.shape[3]
    scores = np.full((bsz, hkv, n_pages_out), -np.inf)
    sel = np.full((bsz, hkv, top_k), -1, dtype=np.int64)
    u = np.zeros((bsz, hq, rv))
    y = np.zeros((bsz, W_O.shape[1]))
    for b in range(bsz):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        n_pages = -(-L // page_size)
        first_recent = recent_window_first_page(L, page_size, recent_tokens)
        recent = np.arange(first_recent, n_pages, dtype=np.int64)
        for g in range(hkv):
            qg = q[b, g * group:(g + 1) * group]
            scores[b, g] = route_page_scores(qg, z[b, g], r[b, g], P[g], Q[g], rb, L,
                                             page_size, n_pages_out, rope_inv_freq)
            sel[b, g] = select_pages(scores[b, g], first_recent, top_k)
            pages = np.concatenate([sel[b, g], recent])
            u[b, g * group:(g + 1) * group] = attend_group(qg, kc[b, g], z[b, g], pages,
                                                           L, page_size, scale, rope_inv_freq)
        y[b] = reconstruct(u[b], Bf, W_O, group)
    out = dict(scores=scores, sel=sel, u=u, y=y, z=z, r=r, kc=kc)
    if store_output:
        out["y_stored"] = round_to_storage(y, storage)
    return out
