"""Helpers of the GPU parity tests: the oracle's answer for chosen sequences of
a workload, and the comparison rules.

The oracle side calls only oracle/ on the generator's stored arrays (decoded
exactly to float64).  Nothing computed by the HIP library is ever an oracle
input, with one sanctioned exception: attention and reconstruction are also
re-run over the library's own page selection, since several selections are
correct when two page scores are within rounding of each other.

Tolerances (stated once, used by every GPU test):
  page scores  |gpu - ref| <= 1e-4 * max(|ref|, rms of the row's valid scores)
               (the float32 output bar; the kernel accumulates up to 144
               products in float32 after a 128-term float32 projection, whose
               worst-case error relative to a near-cancelling score exceeds
               1e-5)
  selection    bit-exact against the oracle's select applied to the library's
               own float32 scores (the integer decision taken in the kernel's
               precision), and the band rule against the oracle's scores: a
               page more than 1e-3 (relative) above the k-th score is chosen,
               one more than 1e-3 below it is not
  u            max |gpu - ref| / max |ref| <= 1e-4 per (sequence, head)
               (float32 arithmetic in both storage formats)
  y            max |gpu - ref| / max |ref| <= 1e-4 (float32) or 2e-2 (bf16)
               per sequence
  z, r codes   (the appended token's, and every prefilled token's) bf16 and
               E4M3 caches: every stored latent code is a valid rounding of
               the exact (float64) latent: the nearest-even value, in the
               cache format, of some point within TIE_RTOL[format] times the
               row's largest magnitude of it (float32 accumulation may land
               on either side of a rounding boundary; the band admits exactly
               those neighbours).  Every stored residual code is a valid
               rounding, under the same rule, of the exact residual formed
               from the library's OWN stored latent (reading R7: the residual
               is taken against the latent as stored).  The Key codes are
               bit-exact (one rounding of a bf16 input, or a copy).  float32
               caches: latent and residual within 1e-5 of the row maximum of
               those same exact values.  When a valid code differs from the
               oracle's, the oracle continues from the library's codes
               (several roundings are correct).
               TIE_RTOL: bf16 3e-5 -- the kernels' float32 orders, simulated
               in float32 on the host, err by at most 6e-6 of the row maximum
               (the prefill's residual, whose P E factor enters as bf16 hi +
               lo terms), while a residual formed from the unrounded latent
               moves by 6e-4 to 2e-3 of it and leaves the band on 8-28% of a
               token's elements (tests/test_parity_rules.py); E4M3 1e-4
               (its quantum is 16 times coarser).
  E4M3 pages   (BASISKV_BF16_FP8_E4M3: z, r and Key pages as E4M3 codes): the
               codes follow the rule above.  Scores, selection and u keep the
               bars above: every page is decoded exactly on both sides.
"""

import math

import numpy as np

from oracle import basiskv_ref as ref

SCORE_RTOL = 1e-4
BAND = 1e-3
U_RTOL = 1e-4
Y_RTOL = {"f32": 1e-4, "bf16": 2e-2}
CODE_RTOL = {"f32": 1e-5}
TIE_RTOL = {"bf16": 3e-5, "fp8": 1e-4}


def f64(a, storage):
    return ref.storage_to_f64(a, storage)


def oracle_sequence(wl, inp, b, *, top_k, append=True, sel_override=None, n_pages_out=None,
                    scale=None, recent_tokens=0, codes_override=None):
    """The oracle's decode step for sequence b of a workload's stored inputs.

    Returns scores [Hkv, NPout], sel [Hkv, k], u [Hq, rV], y [D], y_stored,
    the appended token's stored codes (z_new, r_new: [Hkv, w]; k_new) and
    its unrounded latent z_exact.  sel_override [Hkv, k] replaces the
    oracle's own selection for attention; codes_override (z, r as float64)
    replaces its appended latent and residual codes.  With a recent window
    the routed candidates are the pages before it (n_candidates) and its
    pages are attended as well.
    """
    st = inp["storage"]
    cst = inp.get("cache_storage", st)
    G, hkv, S = wl.group, wl.n_kv_heads, wl.page_size
    T = inp["z"].shape[2]
    if n_pages_out is None:
        n_pages_out = -(-T // S)
    if scale is None:
        scale = 1.0 / math.sqrt(wl.head_dim)
    L = int(inp["seq_lens"][b])
    fac = {k: f64(inp[k], st) for k in ("A", "Bf", "P", "Q", "E", "W_O")}
    q = f64(inp["q"][b], st)
    freqs = inp.get("rope_inv_freq")  # rotary positions (pre-RoPE caches), or None
    scores = np.full((hkv, n_pages_out), -np.inf)
    sel = np.full((hkv, top_k), -1, dtype=np.int64)
    u = np.zeros((wl.n_q_heads, wl.r_v))
    z_new = np.zeros((hkv, wl.r_v))
    r_new = np.zeros((hkv, wl.r_q))
    z_exact = np.zeros((hkv, wl.r_v))
    k_new = np.zeros((hkv, wl.head_dim))
    n_cand = ref.recent_window_first_page(L, S, recent_tokens)
    if L > 0:
        n_pages = -(-L // S)
        recent = np.arange(n_cand, n_pages, dtype=np.int64)
        if append:
            zs, rs, ks = ref.compress_tokens(f64(inp["k_new"][b:b + 1], st),
                                             f64(inp["v_new"][b:b + 1], st),
                                             fac["A"], fac["P"], fac["E"], wl.r_b, cst)
            z_new, r_new, k_new = zs[0], rs[0], ks[0]
            z_exact = np.stack([ref.latent_code(f64(inp["v_new"][b, g], st), fac["A"][g])
                                for g in range(hkv)])
            if codes_override is not None:
                z_new, r_new = codes_override
        for g in range(hkv):
            z = f64(inp["z"][b, g, :L], cst)
            r = f64(inp["r"][b, g, :L], cst)
            kc = f64(inp["kc"][b, g, :L], cst)
            if append:
                z[L - 1], r[L - 1], kc[L - 1] = z_new[g], r_new[g], k_new[g]
            qg = q[g * G:(g + 1) * G]
            scores[g] = ref.route_page_scores(qg, z, r, fac["P"][g], fac["Q"][g], wl.r_b, L, S,
                                              n_pages_out, freqs)
            sel[g] = ref.select_pages(scores[g], n_cand, top_k)
            use = sel[g] if sel_override is None else np.asarray(sel_override[g], dtype=np.int64)
            u[g * G:(g + 1) * G] = ref.attend_group(qg, kc, z, np.concatenate([use, recent]),
                                                    L, S, scale, freqs)
    y = ref.reconstruct(u, fac["Bf"], fac["W_O"], G) if L > 0 else np.zeros(wl.hidden)
    return dict(scores=scores, sel=sel, u=u, y=y, y_stored=ref.round_to_storage(y, st),
                z_new=z_new, r_new=r_new, k_new=k_new, z_exact=z_exact,
                n_pages=(-(-L // S) if L > 0 else 0), n_candidates=n_cand)


def rounding_valid(gpu_codes, exact, storage):
    """Mask of stored codes (bf16 bits or E4M3 codes) that are valid roundings
    of the float64 values ``exact`` (last axis = row): the nearest-even
    rounding, in ``storage``, of some value within TIE_RTOL[storage] *
    max|row| of the exact one.  Rounding is monotone and the band is an
    interval, so those roundings are exactly the representable values between
    the roundings of the band's two ends."""
    exact = np.asarray(exact, dtype=np.float64)
    g = ref.storage_to_f64(gpu_codes, storage)
    if exact.shape[-1] == 0:  # a zero-width row (no residual): nothing to check
        return np.ones(exact.shape, dtype=bool)
    tol = TIE_RTOL[storage] * np.abs(exact).max(axis=-1, keepdims=True)
    lo = ref.round_to_storage(exact - tol, storage)
    hi = ref.round_to_storage(exact + tol, storage)
    return (g >= lo) & (g <= hi)


def exact_residual(wl, inp, k_rows, z_stored):
    """Exact float64 residuals r = (k - z_s[:r_b] P_g) E_g of Key rows
    k_rows [Hkv, dh] (stored inputs) against the latents z_stored [Hkv, r_v]
    (float64) the library stored (reading R7)."""
    st = inp["storage"]
    P, E = f64(inp["P"], st), f64(inp["E"], st)
    return np.concatenate([ref.residual_code(k_rows[g][None], z_stored[g][None], P[g], E[g], wl.r_b)
                           for g in range(wl.n_kv_heads)])


def check_token_codes(wl, inp, b, want, gpu_z, gpu_r, gpu_k, where=""):
    """Appended codes of sequence b (rules in the module docstring), any cache
    format.  Returns (largest relative deviation of a code from the exact
    value, over z and r), and the library's latent and residual as float64
    when they differ from the oracle's (for codes_override), else None."""
    cst = inp.get("cache_storage", inp["storage"])
    st = inp["storage"]
    zg = f64(gpu_z, cst)
    k = f64(inp["k_new"][b], st)
    r_exact = exact_residual(wl, inp, k, zg)
    if cst == "f32":
        ez = rel_rows(zg, want["z_exact"])
        er = rel_rows(f64(gpu_r, cst), r_exact)
        assert ez.max() <= CODE_RTOL[cst], f"{where}: appended latent err {ez.max():.3g}"
        assert er.max() <= CODE_RTOL[cst], f"{where}: appended residual err {er.max():.3g}"
    else:
        ok_z = rounding_valid(gpu_z, want["z_exact"], cst)
        assert ok_z.all(), f"{where}: appended latent codes not a valid rounding at {np.argwhere(~ok_z)[:4]}"
        ok_r = rounding_valid(gpu_r, r_exact, cst)
        assert ok_r.all(), f"{where}: appended residual codes not a valid rounding at {np.argwhere(~ok_r)[:4]}"
    np.testing.assert_array_equal(f64(gpu_k, cst), want["k_new"], err_msg=f"{where}: appended Key codes")
    dev = max(float(rel_rows(zg, want["z_exact"]).max()), float(rel_rows(f64(gpu_r, cst), r_exact).max()))
    rg = f64(gpu_r, cst)
    if np.array_equal(zg, want["z_new"]) and np.array_equal(rg, want["r_new"]):
        return dev, None
    return dev, (zg, rg)


def check_scores(gpu, want, n_pages, where=""):
    """Page scores of one (sequence, KV head); returns the largest error as a
    fraction of SCORE_RTOL."""
    gpu = np.asarray(gpu, dtype=np.float64)
    assert np.all(np.isneginf(gpu[n_pages:])), f"{where}: pages past the sequence must be -inf"
    if n_pages == 0:
        return 0.0
    g, w = gpu[:n_pages], want[:n_pages]
    rms = math.sqrt(float(np.mean(w * w)))
    den = np.maximum(np.abs(w), rms)
    err = np.where(den > 0, np.abs(g - w) / np.where(den > 0, den, 1.0), np.abs(g - w))
    assert err.max() <= SCORE_RTOL, f"{where}: score rel err {err.max():.3g} at page {int(err.argmax())}"
    return float(err.max()) / SCORE_RTOL


def check_selection(gpu_sel, gpu_scores, want_scores, n_pages, top_k, where=""):
    """Selection of one (sequence, KV head): exact in the kernel's precision,
    and inside the band rule against the oracle's float64 scores."""
    gpu_sel = np.asarray(gpu_sel, dtype=np.int64)
    # 1. the integer decision over the library's own float32 scores
    exact = ref.select_pages(np.asarray(gpu_scores, dtype=np.float64), n_pages, top_k)
    np.testing.assert_array_equal(gpu_sel, exact, err_msg=f"{where}: selection over own scores")
    if n_pages <= top_k:
        return
    # 2. band rule against the oracle's scores
    w = want_scores[:n_pages]
    tau = np.sort(w)[::-1][top_k - 1]
    chosen = np.zeros(n_pages, dtype=bool)
    chosen[gpu_sel[gpu_sel >= 0]] = True
    rel = np.abs(w - tau) / np.maximum(np.maximum(np.abs(tau), np.abs(w)), 1e-300)
    must = (w > tau) & (rel > BAND)
    must_not = (w < tau) & (rel > BAND)
    assert np.all(chosen[must]), f"{where}: missed pages {np.nonzero(must & ~chosen)[0]}"
    assert not np.any(chosen[must_not]), f"{where}: extra pages {np.nonzero(must_not & chosen)[0]}"


def rel_rows(gpu, want):
    """max |gpu - want| / max |want| over the last axis, per leading index."""
    gpu = np.asarray(gpu, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if want.shape[-1] == 0:  # zero-width rows agree trivially
        return np.zeros(want.shape[:-1])
    num = np.abs(gpu - want).max(axis=-1)
    den = np.abs(want).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
