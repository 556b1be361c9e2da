"""Seeded synthetic inputs for the decode path (queries, caches, factors).

This module only draws random numbers and shapes them into the workloads'
structure; it holds none of the method's steps (no compression, routing,
selection, attention or reconstruction).  Both the HIP path and the oracle
consume what it returns, as stored arrays: float32 for "f32" storage,
uint16 bf16 bit patterns for "bf16", uint8 E4M3FN codes for "fp8" (the
cache of an FP8 workload: z, r and the Keys; its other arrays are bf16).

Recipe (per workload, see configs.py):
  factors   P [Hkv, rb, dh] ~ N(0,1)/sqrt(rb), Q [Hkv, rq, dh] ~ N(0,1)/sqrt(rq),
            Bf [Hkv, rV, dh] ~ N(0,1)/sqrt(rV), W_O [Hq*dh, D] ~ N(0,1)/sqrt(Hq*dh)
            (fan-in scaling); encoders A = pinv(Bf_g), E = pinv(Q_g).
  queries   q ~ N(0, 1).
  latents   z ~ N(0, 1), times a per-token LogNormal(0, sigma) norm when
            sigma > 0; residual codes r ~ N(0, 1).
  keys      k = z[:rb] P + r Q + noise * N(0, 1); values (prefill / append)
            v = z Bf + noise * N(0, 1).
  planted   pages whose tokens' residual codes are shifted along Q_g qbar
            (qbar = mean query of the KV head's group), with a strength of
            about twice the largest unplanted logit expected by chance; a
            router without a residual (rq = 0) shifts the latent's routing
            dims z[:rb] along P_g qbar instead.  With rotary positions the
            cached Keys are pre-RoPE, so qbar is first turned back by each
            planted token's position.
  rope      (workloads with rope_theta > 0) the inverse frequencies
            base**(-2i/dh), i < dh/2, as float32: an input table of the
            step, like the factors.
Every tensor draws from its own numpy SeedSequence keyed by
(tensor id, sequence, KV head), so a smaller batch reproduces the leading
sequences of a larger one.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_ID = dict(q=1, z=2, zscale=3, r=4, knoise=5, vnoise=6, P=7, Q=8, B=9, W_O=10, plant=11,
           table=12, qstep=13, znew=14, rnew=15, kvnew=16, prefill=17)


def _rng(seed, *key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------------------
# storage conversion (generator side)
# ---------------------------------------------------------------------------

def to_storage(x, storage):
    """float64 -> stored array.  bf16: float32 bits rounded to the upper 16
    bits, nearest-even.  fp8: E4M3FN codes of the float32 value, nearest-even,
    saturated at +-448."""
    if storage == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if storage == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    if storage == "fp8":
        return _e4m3_codes(np.asarray(x, dtype=np.float32))
    if storage != "bf16":
        raise ValueError(storage)
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def _e4m3_codes(x32):
    """float32 -> E4M3FN codes: bias 7, 3 mantissa bits; |x| >= 2**-6 keeps
    the float32 exponent and rounds its 23-bit mantissa to 3 bits (carry into
    the exponent included), smaller magnitudes are multiples of 2**-9."""
    a = np.minimum(np.abs(x32), np.float32(448.0))
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + np.uint64(0x7FFFF) + ((bits >> np.uint64(20)) & np.uint64(1))) >> np.uint64(20)
    normal = ((bits >> np.uint64(3)) - np.uint64(120)) << np.uint64(3) | (bits & np.uint64(7))
    sub = np.rint(a.astype(np.float64) * 512.0).astype(np.uint64)
    code = np.where(a >= np.float32(2.0 ** -6), normal, sub).astype(np.uint8)
    return np.where(np.signbit(x32), code | np.uint8(0x80), code).astype(np.uint8)


def _e4m3_values(codes):
    c = codes.astype(np.int64)
    e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(c & 0x80, -mag, mag)


def from_storage(a, storage):
    if storage in ("f32", "f64"):
        return np.asarray(a, dtype=np.float64)
    if storage == "fp8":
        return _e4m3_values(np.asarray(a, dtype=np.uint8))
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def storage_dtype(storage):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "f64": np.float64}[storage]


# ---------------------------------------------------------------------------
# factors
# ---------------------------------------------------------------------------

def factors(wl, storage=None):
    """Seeded factor set of a workload, as stored arrays (dict)."""
    st = storage or wl.storage
    hkv, dh = wl.n_kv_heads, wl.head_dim
    P = np.stack([_rng(wl.seed, _ID["P"], g).standard_normal((wl.r_b, dh)) for g in range(hkv)])
    P /= math.sqrt(max(wl.r_b, 1))
    Q = np.stack([_rng(wl.seed, _ID["Q"], g).standard_normal((wl.r_q, dh)) for g in range(hkv)])
    Q /= math.sqrt(max(wl.r_q, 1))
    Bf = np.stack([_rng(wl.seed, _ID["B"], g).standard_normal((wl.r_v, dh)) for g in range(hkv)])
    Bf /= math.sqrt(wl.r_v)
    W_O = _rng(wl.seed, _ID["W_O"]).standard_normal((wl.n_q_heads * dh, wl.hidden))
    W_O /= math.sqrt(wl.n_q_heads * dh)
    A = np.stack([np.linalg.pinv(Bf[g]) for g in range(hkv)])   # [Hkv, dh, rV]
    E = np.stack([np.linalg.pinv(Q[g]) for g in range(hkv)])    # [Hkv, dh, rq]
    return dict(A=to_storage(A, st), Bf=to_storage(Bf, st), P=to_storage(P, st),
                Q=to_storage(Q, st), E=to_storage(E, st), W_O=to_storage(W_O, st))


# ---------------------------------------------------------------------------
# decode-step inputs (caches given directly)
# ---------------------------------------------------------------------------

def planted_pages(wl, b, n_pages):
    """Planted page indices of sequence b (sorted)."""
    n = min(wl.n_planted, n_pages)
    if n <= 0 or wl.planted == "none":
        return np.zeros(0, dtype=np.int64)
    if wl.planted == "even":
        return np.array([int((j + 0.5) * n_pages / n) for j in range(n)], dtype=np.int64)
    rng = _rng(wl.seed, _ID["plant"], b)
    return np.sort(rng.choice(n_pages, size=n, replace=False)).astype(np.int64)


def _latent_scale_sq(wl):
    s = wl.latent_norm_sigma
    return math.exp(2.0 * s * s) if s > 0 else 1.0


def rope_frequencies(wl):
    """The workload's RoPE inverse frequencies (float32 [dh/2]), or None."""
    if not wl.rope_theta:
        return None
    i = np.arange(0, wl.head_dim, 2, dtype=np.float64)
    return (float(wl.rope_theta) ** (-i / wl.head_dim)).astype(np.float32)


def _turn_back(x, pos, freqs):
    """x rotated by -pos * freqs in rotate-half pairs (i, i + dh/2): the
    direction a pre-RoPE Key at position pos must have to align with x."""
    half = x.shape[-1] // 2
    phi = pos * freqs.astype(np.float64)
    c, s = np.cos(phi), np.sin(phi)
    lo, hi = x[:half], x[half:]
    return np.concatenate([lo * c + hi * s, -lo * s + hi * c])


def _plant_shift(wl, qg_stored, Qg, T, st, pos=None):
    """Code shift for planted tokens of one KV head along Qg qbar (Qg: the
    residual decoder Q_g, or the predictor P_g when there is no residual);
    with RoPE, qbar turned back by the token's position pos first."""
    qbar = from_storage(qg_stored, st).mean(axis=0)
    freqs = rope_frequencies(wl)
    if freqs is not None and pos is not None:
        qbar = _turn_back(qbar, pos, freqs)
    w = Qg @ qbar
    nw = float(np.linalg.norm(w))
    if nw == 0.0:
        return np.zeros_like(w)
    expected_max = math.sqrt((_latent_scale_sq(wl) + 1.0) * wl.head_dim) * \
        math.sqrt(2.0 * math.log(max(2, T * wl.group)))
    gamma = 2.0 * expected_max / nw
    return gamma * w / nw


def _codes(wl, key, n):
    """Draw latent and residual codes of n tokens.  key = (b, g)."""
    z = _rng(wl.seed, _ID["z"], *key).standard_normal((n, wl.r_v))
    if wl.latent_norm_sigma > 0:
        s = _rng(wl.seed, _ID["zscale"], *key).lognormal(0.0, wl.latent_norm_sigma, size=n)
        z *= s[:, None]
    r = _rng(wl.seed, _ID["r"], *key).standard_normal((n, wl.r_q))
    return z, r


def decode_inputs(wl, *, batch=None, ctx=None, seq_lens=None, exact=False, storage=None,
                  cache_storage=None):
    """Inputs of one decode step of a decode workload.

    Returns a dict of stored arrays:
      q [B, Hq, dh]; z [B, Hkv, T, rV]; r [B, Hkv, T, rq]; kc [B, Hkv, T, dh];
      k_new, v_new [B, Hkv, dh] (the token the step appends at seq_len - 1);
      seq_lens [B] int32; planted: list of per-sequence page arrays; and the
      factor arrays (A, Bf, P, Q, E, W_O).
    ``exact`` removes the noise terms (keys and values become exact low-rank
    functions of the codes).  ``storage`` overrides the workload's format and
    ``cache_storage`` its cache format (z, r, kc; default: the workload's
    cache format, else ``storage``); the dict names both.
    """
    st = storage or wl.storage
    B = batch or wl.batch
    T = ctx or wl.ctx
    hkv, G, dh = wl.n_kv_heads, wl.group, wl.head_dim
    noise = 0.0 if exact else wl.noise
    fac = factors(wl, st)
    Pf, Qf, Bff = (from_storage(fac[k], st) for k in ("P", "Q", "Bf"))
    if seq_lens is None:
        seq_lens = np.full(B, T, dtype=np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)

    q = np.stack([_rng(wl.seed, _ID["q"], b).standard_normal((wl.n_q_heads, dh)) for b in range(B)])
    q_st = to_storage(q, st)

    sd = storage_dtype(st)
    cst = cache_storage or wl.cache_storage or st
    cd = storage_dtype(cst)
    z_st = np.empty((B, hkv, T, wl.r_v), dtype=cd)
    r_st = np.empty((B, hkv, T, wl.r_q), dtype=cd)
    k_st = np.empty((B, hkv, T, dh), dtype=cd)
    kn_st = np.empty((B, hkv, dh), dtype=sd)
    vn_st = np.empty((B, hkv, dh), dtype=sd)
    planted = [planted_pages(wl, b, -(-max(int(seq_lens[b]), 1) // wl.page_size)) for b in range(B)]

    def one(bg):
        b, g = bg
        z, r = _codes(wl, (b, g), T)
        shift = None
        plant_z = wl.r_q == 0  # no residual: plant through the latent's routing dims
        qgb = q_st[b, g * G:(g + 1) * G]
        Fg = Pf[g] if plant_z else Qf[g]
        if len(planted[b]):
            shift = _plant_shift(wl, qgb, Fg, T, st)
            for p in planted[b]:
                for t in range(p * wl.page_size, min((p + 1) * wl.page_size, T)):
                    sh = shift if not wl.rope_theta else _plant_shift(wl, qgb, Fg, T, st, pos=t)
                    if plant_z:
                        z[t, :wl.r_b] += sh
                    else:
                        r[t] += sh
        k = z[:, :wl.r_b] @ Pf[g] + r @ Qf[g]
        if noise:
            k += noise * _rng(wl.seed, _ID["knoise"], b, g).standard_normal((T, dh))
        z_st[b, g] = to_storage(z, cst)
        r_st[b, g] = to_storage(r, cst)
        k_st[b, g] = to_storage(k, cst)
        # the token appended by the step, at position seq_len - 1
        zn = _rng(wl.seed, _ID["znew"], b, g).standard_normal(wl.r_v)
        if wl.latent_norm_sigma > 0:
            zn *= _rng(wl.seed, _ID["znew"], b, g, 1).lognormal(0.0, wl.latent_norm_sigma)
        rn = _rng(wl.seed, _ID["rnew"], b, g).standard_normal(wl.r_q)
        last_page = (int(seq_lens[b]) - 1) // wl.page_size
        if shift is not None and wl.rope_theta:
            shift = _plant_shift(wl, qgb, Fg, T, st, pos=int(seq_lens[b]) - 1)
        if shift is not None and last_page in set(planted[b].tolist()):
            if plant_z:
                zn = zn.copy()
                zn[:wl.r_b] += shift
            else:
                rn = rn + shift
        kn = zn[:wl.r_b] @ Pf[g] + rn @ Qf[g]
        vn = zn @ Bff[g]
        if noise:
            nz = _rng(wl.seed, _ID["kvnew"], b, g).standard_normal((2, dh))
            kn = kn + noise * nz[0]
            vn = vn + noise * nz[1]
        kn_st[b, g] = to_storage(kn, st)
        vn_st[b, g] = to_storage(vn, st)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, [(b, g) for b in range(B) for g in range(hkv)]))

    out = dict(q=q_st, z=z_st, r=r_st, kc=k_st, k_new=kn_st, v_new=vn_st, seq_lens=seq_lens,
               planted=planted, storage=st, cache_storage=cst, rope_inv_freq=rope_frequencies(wl))
    out.update(fac)
    return out


# ---------------------------------------------------------------------------
# activations for compression (prefill and per-step append)
# ---------------------------------------------------------------------------

def kv_activations(wl, *, batch, tokens, stream, exact=False, storage=None):
    """Keys and Values of ``tokens`` new tokens per sequence, [B, T, Hkv, dh]
    stored, with the low-rank structure of the recipe (z, r ~ N(0,1)).
    ``stream`` separates independent draws (prefill, context, step i)."""
    st = storage or wl.storage
    hkv, dh = wl.n_kv_heads, wl.head_dim
    noise = 0.0 if exact else wl.noise
    fac = factors(wl, st)
    Pf, Qf, Bff = (from_storage(fac[k], st) for k in ("P", "Q", "Bf"))
    sd = storage_dtype(st)
    k_st = np.empty((batch, tokens, hkv, dh), dtype=sd)
    v_st = np.empty((batch, tokens, hkv, dh), dtype=sd)

    def one(bg):
        b, g = bg
        rng = _rng(wl.seed, _ID["prefill"], stream, b, g)
        z = rng.standard_normal((tokens, wl.r_v))
        r = rng.standard_normal((tokens, wl.r_q))
        k = z[:, :wl.r_b] @ Pf[g] + r @ Qf[g]
        v = z @ Bff[g]
        if noise:
            k += noise * rng.standard_normal((tokens, dh))
            v += noise * rng.standard_normal((tokens, dh))
        k_st[b, :, g, :] = to_storage(k, st)
        v_st[b, :, g, :] = to_storage(v, st)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, [(b, g) for b in range(batch) for g in range(hkv)]))
    return k_st, v_st


def step_queries(wl, *, batch, step, storage=None):
    """Queries of decode step ``step`` of the prefill+decode workload."""
    st = storage or wl.storage
    q = np.stack([_rng(wl.seed, _ID["qstep"], step, b).standard_normal((wl.n_q_heads, wl.head_dim))
                  for b in range(batch)])
    return to_storage(q, st)


# ---------------------------------------------------------------------------
# block tables
# ---------------------------------------------------------------------------

def block_table(n_seqs, max_pages, *, shuffle_seed=None):
    """Logical -> physical page map [n_seqs, max_pages] int32 over a pool of
    n_seqs * max_pages pages; a seeded permutation when shuffle_seed is set."""
    n = n_seqs * max_pages
    phys = np.arange(n, dtype=np.int64)
    if shuffle_seed is not None:
        phys = _rng(shuffle_seed, _ID["table"]).permutation(n)
    return phys.reshape(n_seqs, max_pages).astype(np.int32)
