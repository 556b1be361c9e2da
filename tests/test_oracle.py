"""Pins of the float64 oracle against things other than itself (CPU only).

Each test ties one oracle function to brute force, a closed form, an
invariant or a library routine, so that a plausible slip (dropped term,
transposed factor, wrong head / page index, wrong softmax set, wrong tie
rule) fails at least one of them.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import basiskv_ref as ref
from oracle import brute
from sparse_decode_attention_latent_amd import synth
from sparse_decode_attention_latent_amd.configs import workload, Workload


def tiny_workload(**kw):
    base = dict(name="tiny-brute", storage="f64", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
                hidden=6, ctx=11, page_size=2, r_v=4, r_b=3, r_q=2, top_k=3, n_planted=0,
                planted="none", seed=77)
    base.update(kw)
    return Workload(**base)


def as64(inp, key):
    return ref.storage_to_f64(inp[key], inp["storage"])


def unpack(inp):
    names = ("q", "z", "r", "kc", "k_new", "v_new", "A", "Bf", "P", "Q", "E", "W_O")
    return {n: as64(inp, n) for n in names}


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_and_closed_forms():
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    x32[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130]
    mine = ref.round_to_storage(x32.astype(np.float64), "bf16")
    lib = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, lib)
    # halfway cases go to the even neighbour
    assert mine[0] == 1.0 and mine[1] == 1 + 2 ** -6 and mine[2] == -1.0


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    finite = ((bits.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    bits = bits[finite]
    mine = ref.storage_to_f64(bits, "bf16")
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, lib)


def _e4m3_values():
    """Every finite non-negative E4M3FN value with its code, enumerated from
    the format's fields (bias 7, 3 mantissa bits, exponent field 0 subnormal,
    code 0x7F reserved for NaN), written out independently of the oracle."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append((m / 8.0 * 2.0 ** -6) if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return vals


def _nearest_e4m3(x, vals):
    """Brute force: the nearest value in the table (ties to the even code),
    magnitudes past 448 saturated."""
    a = min(abs(x), 448.0)
    best = min(range(len(vals)), key=lambda c: (abs(vals[c] - a), c & 1))
    return math.copysign(vals[best], x)


def test_fp8_decode_matches_torch_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    mine = ref.storage_to_f64(codes, "fp8")
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, lib)  # NaN codes compare equal here too
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x38] == 1.0 and mine[0xB8] == -1.0
    assert mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9 and mine[0x07] == 7 * 2.0 ** -9
    np.testing.assert_array_equal(mine[:0x7F], _e4m3_values())


def test_fp8_rounding_matches_brute_nearest_and_torch():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-13, 10, 4000))
    x32 = (mag * np.where(rng.random(4000) < 0.5, -1, 1)).astype(np.float32)
    vals = _e4m3_values()
    # halfway cases, saturation, subnormal ties and zeros
    special = [1.0625, 1.1875, -1.0625, 1.5 * 2 ** -9, 0.5 * 2 ** -9, 2.5 * 2 ** -9,
               7.5 * 2 ** -9, 440.0, 448.0, 456.0, 464.0, 1000.0, -1e6, 0.0, 2 ** -12]
    x32[:len(special)] = special
    mine = ref.round_to_storage(x32.astype(np.float64), "fp8")
    want = np.array([_nearest_e4m3(float(v), vals) for v in x32])
    np.testing.assert_array_equal(mine, want)
    clamped = torch.from_numpy(np.clip(x32, -448, 448))
    lib = clamped.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, lib)
    assert mine[0] == 1.0 and mine[1] == 1.25 and mine[2] == -1.0
    assert mine[3] == 2 * 2.0 ** -9 and mine[4] == 0.0 and mine[5] == 2 * 2.0 ** -9
    assert mine[6] == 2.0 ** -6 and mine[8] == 448.0 and mine[10] == 448.0 and mine[12] == -448.0
    assert np.isnan(ref.round_to_storage(np.array([np.nan]), "fp8")[0])


def test_compress_into_fp8_cache_matches_brute():
    """The step's append with an FP8 cache: the latent is rounded to E4M3
    before the residual is formed from it (R7 with R12), the Key is stored
    rounded; every stored value is the brute-force nearest E4M3 value."""
    wl = tiny_workload(batch=2)
    inp = synth.decode_inputs(wl, seq_lens=np.array([11, 4]))
    d = unpack(inp)
    vals = _e4m3_values()

    def rnd(x):
        return _nearest_e4m3(float(x), vals)

    out = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], inp["seq_lens"], d["A"], d["Bf"], d["P"],
                          d["Q"], d["E"], d["W_O"], rb=wl.r_b, page_size=wl.page_size,
                          top_k=wl.top_k, n_pages_out=wl.max_pages, storage="f64",
                          cache_storage="fp8", k_new=d["k_new"] * 7.0, v_new=d["v_new"] * 7.0)
    for b, L in enumerate((11, 4)):
        for g in range(wl.n_kv_heads):
            zb, rb_ = brute.compress_token(d["k_new"][b, g] * 7.0, d["v_new"][b, g] * 7.0,
                                           d["A"][g].tolist(), d["P"][g].tolist(),
                                           d["E"][g].tolist(), wl.r_b, rnd)
            np.testing.assert_array_equal(out["z"][b, g, L - 1], zb)
            np.testing.assert_array_equal(out["r"][b, g, L - 1], rb_)
            np.testing.assert_array_equal(out["kc"][b, g, L - 1],
                                          [rnd(v) for v in d["k_new"][b, g] * 7.0])
        # rows other than the appended one are untouched
        np.testing.assert_array_equal(out["z"][b, :, :L - 1], d["z"][b, :, :L - 1])


# ---------------------------------------------------------------------------
# compression
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("storage", ["f64", "bf16"])
def test_compress_matches_brute(storage):
    wl = tiny_workload(storage=storage)
    fac = synth.factors(wl)
    A, P, E = (ref.storage_to_f64(fac[k], storage) for k in ("A", "P", "E"))
    rng = np.random.default_rng(5)
    k_new = ref.round_to_storage(rng.standard_normal((3, wl.n_kv_heads, wl.head_dim)), storage)
    v_new = ref.round_to_storage(rng.standard_normal((3, wl.n_kv_heads, wl.head_dim)), storage)
    z_s, r_s, k_s = ref.compress_tokens(k_new, v_new, A, P, E, wl.r_b, storage)
    np.testing.assert_array_equal(k_s, k_new)

    def rnd(x):
        return float(ref.round_to_storage(np.array([x]), storage)[0])

    for n in range(3):
        for g in range(wl.n_kv_heads):
            zb, rb_ = brute.compress_token(k_new[n, g], v_new[n, g], A[g].tolist(), P[g].tolist(),
                                           E[g].tolist(), wl.r_b, rnd)
            if storage == "f64":
                np.testing.assert_allclose(z_s[n, g], zb, rtol=0, atol=1e-12)
                np.testing.assert_allclose(r_s[n, g], rb_, rtol=0, atol=1e-12)
            else:
                # both orders agree to ~1e-16 before the bf16 store, so the stored
                # values are identical unless a value sits on a rounding tie
                # (none does for these seeded inputs)
                np.testing.assert_array_equal(z_s[n, g], zb)
                np.testing.assert_array_equal(r_s[n, g], rb_)


def test_compress_recovers_exact_codes():
    """With noise-free K, V and A = pinv(B), E = pinv(Q), the encoders give back
    the generating codes exactly (the latent/residual split of the abstract)."""
    wl = workload(0).with_(storage="f64", ctx=64, n_planted=0, planted="none")
    fac = synth.factors(wl)
    A, P, Q, E, Bf = (ref.storage_to_f64(fac[k], "f64") for k in ("A", "P", "Q", "E", "Bf"))
    rng = np.random.default_rng(3)
    n = 40
    z = rng.standard_normal((n, wl.n_kv_heads, wl.r_v))
    r = rng.standard_normal((n, wl.n_kv_heads, wl.r_q))
    k = np.einsum("ngi,gid->ngd", z[:, :, :wl.r_b], P) + np.einsum("ngj,gjd->ngd", r, Q)
    v = np.einsum("ngi,gid->ngd", z, Bf)
    z_s, r_s, _ = ref.compress_tokens(k, v, A, P, E, wl.r_b, "f64")
    np.testing.assert_allclose(z_s, z, rtol=0, atol=1e-10)
    np.testing.assert_allclose(r_s, r, rtol=0, atol=1e-10)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seq_len", [11, 10, 1])
def test_route_matches_projected_query_brute(seq_len):
    wl = tiny_workload()
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    G = wl.group
    n_out = wl.max_pages + 1
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            qg = d["q"][b, g * G:(g + 1) * G]
            mine = ref.route_page_scores(qg, d["z"][b, g], d["r"][b, g], d["P"][g], d["Q"][g],
                                         wl.r_b, seq_len, wl.page_size, n_out)
            other = brute.route_page_scores(qg.tolist(), d["z"][b, g].tolist(), d["r"][b, g].tolist(),
                                            d["P"][g].tolist(), d["Q"][g].tolist(), wl.r_b, seq_len,
                                            wl.page_size, n_out)
            np.testing.assert_allclose(mine, other, rtol=1e-12, atol=1e-12)
            n_pages = -(-seq_len // wl.page_size)
            assert np.all(np.isneginf(mine[n_pages:])) and np.all(np.isfinite(mine[:n_pages]))


def test_route_equals_exact_logits_when_keys_are_exact():
    """Noise-free keys are exactly z[:rb] P + r Q, so the predicted-key logit
    equals the true q.k logit; the page score is then the page's largest
    exact logit over the group (closed form)."""
    wl = workload(0).with_(storage="f64", ctx=300, batch=1)
    inp = synth.decode_inputs(wl, exact=True)
    d = unpack(inp)
    G, S = wl.group, wl.page_size
    L = 300
    for g in range(wl.n_kv_heads):
        qg = d["q"][0, g * G:(g + 1) * G]
        mine = ref.route_page_scores(qg, d["z"][0, g], d["r"][0, g], d["P"][g], d["Q"][g], wl.r_b,
                                     L, S, wl.max_pages)
        exact = torch.from_numpy(qg) @ torch.from_numpy(d["kc"][0, g, :L]).T
        n_pages = -(-L // S)
        want = [exact[:, p * S:min((p + 1) * S, L)].max().item() for p in range(n_pages)]
        np.testing.assert_allclose(mine[:n_pages], want, rtol=1e-10, atol=1e-9)


def test_route_uses_only_leading_rb_latent_dims():
    wl = tiny_workload(r_v=6, r_b=2)
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    qg = d["q"][0, :wl.group]
    base = ref.route_page_scores(qg, d["z"][0, 0], d["r"][0, 0], d["P"][0], d["Q"][0], wl.r_b, 11, 2, 6)
    z2 = d["z"][0, 0].copy()
    z2[:, wl.r_b:] += 100.0
    moved = ref.route_page_scores(qg, z2, d["r"][0, 0], d["P"][0], d["Q"][0], wl.r_b, 11, 2, 6)
    np.testing.assert_array_equal(base, moved)


# ---------------------------------------------------------------------------
# single-source routers (appendix Table 9: B16 routes from the latent's leading
# dims alone, R16 / R32 from the residual alone)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rb,rq", [(3, 0), (0, 2)])
def test_single_source_router_matches_brute(rb, rq):
    """Routing and compression with r_q = 0 or r_b = 0 agree with the brute
    force (projected queries; residual as k E - z_s (P E))."""
    wl = tiny_workload(r_b=rb, r_q=rq)
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    G, n_out = wl.group, wl.max_pages
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            qg = d["q"][b, g * G:(g + 1) * G]
            mine = ref.route_page_scores(qg, d["z"][b, g], d["r"][b, g], d["P"][g], d["Q"][g],
                                         wl.r_b, 11, wl.page_size, n_out)
            other = brute.route_page_scores(qg.tolist(), d["z"][b, g].tolist(), d["r"][b, g].tolist(),
                                            d["P"][g].tolist(), d["Q"][g].tolist(), wl.r_b, 11,
                                            wl.page_size, n_out)
            np.testing.assert_allclose(mine, other, rtol=1e-12, atol=1e-12)
    z_s, r_s, _ = ref.compress_tokens(d["k_new"], d["v_new"], d["A"], d["P"], d["E"], wl.r_b, "f64")
    assert r_s.shape[-1] == rq and z_s.shape[-1] == wl.r_v
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            zb, rb_ = brute.compress_token(d["k_new"][b, g], d["v_new"][b, g], d["A"][g].tolist(),
                                           d["P"][g].tolist(), d["E"][g].tolist(), wl.r_b, float)
            np.testing.assert_allclose(z_s[b, g], zb, rtol=0, atol=1e-12)
            np.testing.assert_allclose(r_s[b, g], rb_, rtol=0, atol=1e-12)


def test_b_only_router_is_the_full_router_with_zero_residual():
    """Special case: routing without a residual (r_q = 0) gives exactly the
    scores of the combined router whose residual codes are all zero, for any
    residual decoder."""
    wl = tiny_workload(r_q=0)
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    rng = np.random.default_rng(9)
    Q_any = rng.standard_normal((5, wl.head_dim))
    qg = d["q"][0, :wl.group]
    mine = ref.route_page_scores(qg, d["z"][0, 0], d["r"][0, 0], d["P"][0], d["Q"][0], wl.r_b,
                                 11, wl.page_size, wl.max_pages)
    full = ref.route_page_scores(qg, d["z"][0, 0], np.zeros((wl.ctx, 5)), d["P"][0], Q_any, wl.r_b,
                                 11, wl.page_size, wl.max_pages)
    np.testing.assert_array_equal(mine, full)


def test_r_only_residual_is_the_key_encoded():
    """With r_b = 0 nothing is predicted from the latent: the residual code is
    the Key through the residual encoder, r = k E (closed form), and a
    noise-free Key k = r Q (E = pinv(Q)) gives its code back exactly."""
    wl = workload("llama8b-ctx32k-r32-page4").with_(storage="f64")
    fac = synth.factors(wl)
    A, P, Q, E = (ref.storage_to_f64(fac[k], "f64") for k in ("A", "P", "Q", "E"))
    assert P.shape[1] == 0
    rng = np.random.default_rng(21)
    r = rng.standard_normal((30, wl.n_kv_heads, wl.r_q))
    k = np.einsum("ngj,gjd->ngd", r, Q)
    v = rng.standard_normal((30, wl.n_kv_heads, wl.head_dim))
    _, r_s, _ = ref.compress_tokens(k, v, A, P, E, 0, "f64")
    np.testing.assert_allclose(r_s, np.einsum("ngd,gdj->ngj", k, E), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r_s, r, rtol=0, atol=1e-10)


@pytest.mark.parametrize("name", ["llama8b-ctx32k-b16-page4", "llama8b-ctx32k-r16-page4"])
def test_single_source_route_equals_exact_logits_when_keys_are_exact(name):
    """Noise-free Keys are exactly the single source's prediction (z[:rb] P,
    or r Q), so the routing logits are the exact q.k logits."""
    wl = workload(name).with_(storage="f64", ctx=200, batch=1)
    inp = synth.decode_inputs(wl, exact=True)
    d = unpack(inp)
    G, S, L = wl.group, wl.page_size, 200
    for g in (0, wl.n_kv_heads - 1):
        qg = d["q"][0, g * G:(g + 1) * G]
        mine = ref.route_page_scores(qg, d["z"][0, g], d["r"][0, g], d["P"][g], d["Q"][g], wl.r_b,
                                     L, S, wl.max_pages)
        exact = qg @ d["kc"][0, g, :L].T
        n_pages = -(-L // S)
        want = [exact[:, p * S:min((p + 1) * S, L)].max() for p in range(n_pages)]
        np.testing.assert_allclose(mine[:n_pages], want, rtol=1e-10, atol=1e-9)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def test_select_matches_exhaustive_search_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 11))
        scores = rng.integers(-3, 4, size=n).astype(np.float64)  # many exact ties
        mine = ref.select_pages(scores, n, k)
        other = brute.select_pages(scores.tolist(), n, k)
        assert mine.tolist() == other, (scores, k)


def test_select_matches_stable_argsort():
    rng = np.random.default_rng(12)
    for n, k in [(128, 16), (1024, 128), (4096, 128), (100, 100), (37, 50)]:
        scores = rng.standard_normal(n)
        scores[::7] = scores[3]  # ties
        want = np.sort(np.argsort(-scores, kind="stable")[:k])
        want = np.concatenate([want, -np.ones(k - len(want), dtype=np.int64)])
        np.testing.assert_array_equal(ref.select_pages(scores, n, k), want)


def test_select_ignores_pages_past_n_pages():
    scores = np.array([1.0, 5.0, 3.0, 9.0, 8.0])
    np.testing.assert_array_equal(ref.select_pages(scores, 3, 2), [1, 2])
    np.testing.assert_array_equal(ref.select_pages(scores, 0, 2), [-1, -1])


# ---------------------------------------------------------------------------
# attention over the selected pages
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, mask=None):
    """torch's CPU scaled_dot_product_attention in float64 (scale 1/sqrt(dh)).
    q [G, dh] (the G heads act as a batch), k [n, dh], v [n, w], mask [n] bool."""
    G = q.shape[0]
    qt = torch.from_numpy(np.ascontiguousarray(q)).reshape(G, 1, 1, -1)
    kt = torch.from_numpy(np.ascontiguousarray(k)).reshape(1, 1, *k.shape).expand(G, 1, -1, -1).contiguous()
    vt = torch.from_numpy(np.ascontiguousarray(v)).reshape(1, 1, *v.shape).expand(G, 1, -1, -1).contiguous()
    m = None
    if mask is not None:
        m = torch.from_numpy(mask).reshape(1, 1, 1, -1).expand(G, 1, 1, -1).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    return out[:, 0, 0, :].numpy()


@pytest.mark.parametrize("L", [2048, 2041])
def test_attend_all_pages_equals_sdpa(L):
    """k >= number of pages: attention over every valid token (library routine),
    including a partial last page."""
    wl = workload(0).with_(storage="f64", batch=1)
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    G, S = wl.group, wl.page_size
    n_pages = -(-L // S)
    sel = np.arange(n_pages)
    for g in range(wl.n_kv_heads):
        qg = d["q"][0, g * G:(g + 1) * G]
        mine = ref.attend_group(qg, d["kc"][0, g], d["z"][0, g], sel, L, S, 1 / math.sqrt(wl.head_dim))
        want = _sdpa(qg, d["kc"][0, g, :L], d["z"][0, g, :L])
        np.testing.assert_allclose(mine, want, rtol=1e-10, atol=1e-12)


def test_attend_subset_matches_masked_sdpa_and_brute():
    wl = tiny_workload()
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    G, S, L = wl.group, wl.page_size, 11
    sel = np.array([0, 2, 5, -1])  # page 5 is the partial last page (token 10 only)
    scale = 0.37
    for g in range(wl.n_kv_heads):
        qg = d["q"][1, g * G:(g + 1) * G]
        mine = ref.attend_group(qg, d["kc"][1, g], d["z"][1, g], sel, L, S, scale)
        other = brute.attend_group(qg.tolist(), d["kc"][1, g].tolist(), d["z"][1, g].tolist(),
                                   sel.tolist(), L, S, scale)
        np.testing.assert_allclose(mine, other, rtol=1e-12, atol=1e-13)
        mask = np.zeros(L, dtype=bool)
        for p in (0, 2, 5):
            mask[p * S:min((p + 1) * S, L)] = True
        want = _sdpa(qg * scale * math.sqrt(wl.head_dim), d["kc"][1, g, :L], d["z"][1, g, :L], mask)
        np.testing.assert_allclose(mine, want, rtol=1e-10, atol=1e-12)


def test_attend_empty_selection_is_zero():
    wl = tiny_workload()
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    out = ref.attend_group(d["q"][0, :2], d["kc"][0, 0], d["z"][0, 0], np.array([-1, -1]), 11, 2, 0.5)
    np.testing.assert_array_equal(out, 0.0)


# ---------------------------------------------------------------------------
# reconstruction
# ---------------------------------------------------------------------------

def test_reconstruct_matches_fused_brute():
    wl = tiny_workload()
    fac = synth.factors(wl)
    Bf, W_O = ref.storage_to_f64(fac["Bf"], "f64"), ref.storage_to_f64(fac["W_O"], "f64")
    u = np.random.default_rng(4).standard_normal((wl.n_q_heads, wl.r_v))
    mine = ref.reconstruct(u, Bf, W_O, wl.group)
    other = brute.reconstruct(u.tolist(), Bf.tolist(), W_O.tolist(), wl.group)
    np.testing.assert_allclose(mine, other, rtol=1e-12, atol=1e-12)


def test_full_k_invariant_equals_dense_attention_through_W_O():
    """Exact factors and k = all pages: the latent path equals dense softmax
    attention over (K, V = z B) followed by W_O (the pages' Full-K reference
    with the same compressed Values)."""
    wl = workload(0).with_(storage="f64", batch=1, ctx=512)
    inp = synth.decode_inputs(wl, exact=True)
    d = unpack(inp)
    n_pages = wl.max_pages
    out = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], inp["seq_lens"], d["A"], d["Bf"], d["P"],
                          d["Q"], d["E"], d["W_O"], rb=wl.r_b, page_size=wl.page_size,
                          top_k=n_pages, n_pages_out=n_pages, storage="f64")
    G = wl.group
    heads = []
    for h in range(wl.n_q_heads):
        g = h // G
        v = d["z"][0, g] @ d["Bf"][g]
        heads.append(_sdpa(d["q"][0, h:h + 1], d["kc"][0, g], v)[0])
    y_dense = np.concatenate(heads) @ d["W_O"]
    np.testing.assert_allclose(out["y"][0], y_dense, rtol=1e-9, atol=1e-10)


def test_latent_identity_for_any_selection():
    """(sum_t p_t z_t) B W_O == attention over reconstructed values z B, on the
    selected tokens only, then W_O."""
    wl = workload(0).with_(storage="f64", batch=1, ctx=700)
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    L, S, G = 700, wl.page_size, wl.group
    rng = np.random.default_rng(9)
    sel = np.sort(rng.choice(-(-L // S), size=7, replace=False))
    u = np.zeros((wl.n_q_heads, wl.r_v))
    heads = []
    mask = np.zeros(L, dtype=bool)
    for p in sel:
        mask[p * S:min((p + 1) * S, L)] = True
    for g in range(wl.n_kv_heads):
        qg = d["q"][0, g * G:(g + 1) * G]
        u[g * G:(g + 1) * G] = ref.attend_group(qg, d["kc"][0, g], d["z"][0, g], sel, L, S,
                                                1 / math.sqrt(wl.head_dim))
    for h in range(wl.n_q_heads):
        g = h // G
        heads.append(_sdpa(d["q"][0, h:h + 1], d["kc"][0, g, :L], (d["z"][0, g] @ d["Bf"][g])[:L], mask)[0])
    np.testing.assert_allclose(ref.reconstruct(u, d["Bf"], d["W_O"], G),
                               np.concatenate(heads) @ d["W_O"], rtol=1e-10, atol=1e-11)


# ---------------------------------------------------------------------------
# a whole step, end to end against the brute-force statement
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seq_lens", [(11, 7), (0, 3), (1, 11)])
def test_decode_step_matches_brute_end_to_end(seq_lens):
    wl = tiny_workload()
    inp = synth.decode_inputs(wl, seq_lens=np.array(seq_lens))
    d = unpack(inp)
    G, S, k = wl.group, wl.page_size, wl.top_k
    out = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], inp["seq_lens"], d["A"], d["Bf"], d["P"],
                          d["Q"], d["E"], d["W_O"], rb=wl.r_b, page_size=S, top_k=k,
                          n_pages_out=wl.max_pages, storage="f64", k_new=d["k_new"], v_new=d["v_new"])
    scale = 1 / math.sqrt(wl.head_dim)
    for b in range(wl.batch):
        L = int(seq_lens[b])
        z, r, kc = d["z"][b].copy(), d["r"][b].copy(), d["kc"][b].copy()
        u = np.zeros((wl.n_q_heads, wl.r_v))
        if L > 0:
            for g in range(wl.n_kv_heads):
                zz, rr = brute.compress_token(d["k_new"][b, g], d["v_new"][b, g], d["A"][g].tolist(),
                                              d["P"][g].tolist(), d["E"][g].tolist(), wl.r_b, float)
                z[g, L - 1], r[g, L - 1], kc[g, L - 1] = zz, rr, d["k_new"][b, g]
        for g in range(wl.n_kv_heads):
            qg = d["q"][b, g * G:(g + 1) * G].tolist()
            sc = brute.route_page_scores(qg, z[g].tolist(), r[g].tolist(), d["P"][g].tolist(),
                                         d["Q"][g].tolist(), wl.r_b, L, S, wl.max_pages)
            np.testing.assert_allclose(out["scores"][b, g], sc, rtol=1e-11, atol=1e-11)
            n_pages = -(-L // S) if L > 0 else 0
            sel = brute.select_pages(sc, n_pages, k)
            assert out["sel"][b, g].tolist() == sel
            u[g * G:(g + 1) * G] = brute.attend_group(qg, kc[g].tolist(), z[g].tolist(), sel, L, S, scale)
        np.testing.assert_allclose(out["u"][b], u, rtol=1e-11, atol=1e-12)
        y = brute.reconstruct(u.tolist(), d["Bf"].tolist(), d["W_O"].tolist(), G)
        np.testing.assert_allclose(out["y"][b], y, rtol=1e-10, atol=1e-11)
        if L <= 0:
            np.testing.assert_array_equal(out["y"][b], 0.0)


# ---------------------------------------------------------------------------
# the recent window (appendix Table 9 caption: 64 recent tokens beside the
# routed budget; reading R11: whole pages holding the last W tokens)
# ---------------------------------------------------------------------------

def test_recent_window_first_page_closed_forms():
    f = ref.recent_window_first_page
    assert f(100, 4, 0) == 25 and f(101, 4, 0) == 26 and f(0, 4, 0) == 0
    assert f(100, 4, 64) == 9          # tokens 36..99 -> pages 9..24
    assert f(101, 4, 64) == 9          # tokens 37..100 -> pages 9..25
    assert f(40, 4, 64) == 0 and f(0, 4, 64) == 0
    assert f(65, 32, 64) == 0 and f(97, 32, 64) == 1


@pytest.mark.parametrize("seq_lens,recent", [([11, 7], 3), ([11, 6], 4), ([9, 11], 1), ([1, 0], 5)])
def test_recent_window_matches_token_predicate_brute(seq_lens, recent):
    """Routed pages are the top-k of the pages before the window (brute
    exhaustive search over that prefix) and the attention runs over the
    tokens t with page(t) routed or t >= first_recent_page * S (brute token
    loop)."""
    wl = tiny_workload()
    inp = synth.decode_inputs(wl, seq_lens=np.array(seq_lens))
    d = unpack(inp)
    G, S, k = wl.group, wl.page_size, wl.top_k
    out = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], inp["seq_lens"], d["A"], d["Bf"], d["P"],
                          d["Q"], d["E"], d["W_O"], rb=wl.r_b, page_size=S, top_k=k,
                          n_pages_out=wl.max_pages, storage="f64", recent_tokens=recent)
    scale = 1 / math.sqrt(wl.head_dim)
    for b in range(wl.batch):
        L = int(seq_lens[b])
        first = max(0, L - recent) // S          # written out again from the definition
        for g in range(wl.n_kv_heads):
            qg = d["q"][b, g * G:(g + 1) * G].tolist()
            sc = brute.route_page_scores(qg, d["z"][b, g].tolist(), d["r"][b, g].tolist(),
                                         d["P"][g].tolist(), d["Q"][g].tolist(), wl.r_b, L, S,
                                         wl.max_pages)
            sel = brute.select_pages(sc, first if L > 0 else 0, k)
            assert out["sel"][b, g].tolist() == sel
            toks = [t for t in range(L) if (t // S) in sel or t >= first * S]
            u = brute.attend_tokens(qg, d["kc"][b, g].tolist(), d["z"][b, g].tolist(), toks, scale)
            np.testing.assert_allclose(out["u"][b, g * G:(g + 1) * G], u, rtol=1e-11, atol=1e-12)


def test_recent_window_covering_everything_is_dense_attention():
    """A window at least as long as the sequence routes nothing and attends
    every token: the step equals dense softmax attention (torch SDPA)."""
    wl = tiny_workload(batch=1)
    inp = synth.decode_inputs(wl, seq_lens=np.array([11]))
    d = unpack(inp)
    out = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], inp["seq_lens"], d["A"], d["Bf"], d["P"],
                          d["Q"], d["E"], d["W_O"], rb=wl.r_b, page_size=wl.page_size,
                          top_k=wl.top_k, n_pages_out=wl.max_pages, storage="f64",
                          recent_tokens=11)
    assert (out["sel"] == -1).all()
    G = wl.group
    for g in range(wl.n_kv_heads):
        q = torch.from_numpy(d["q"][0, g * G:(g + 1) * G])[:, None, :]
        kk = torch.from_numpy(d["kc"][0, g])[None].expand(G, -1, -1)
        zz = torch.from_numpy(d["z"][0, g])[None].expand(G, -1, -1)
        want = torch.nn.functional.scaled_dot_product_attention(q, kk, zz)[:, 0].numpy()
        np.testing.assert_allclose(out["u"][0, g * G:(g + 1) * G], want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("L", [1, 7, 11])
def test_dense_attention_equals_sdpa(L):
    """The dense baseline's oracle against torch's scaled dot-product attention."""
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((4, 8)), rng.standard_normal((11, 8)), rng.standard_normal((11, 8))
    got = ref.dense_attention(q, k, v, L, 1 / math.sqrt(8))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None], torch.from_numpy(k[:L])[None].expand(4, -1, -1),
        torch.from_numpy(v[:L])[None].expand(4, -1, -1))[:, 0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    assert not ref.dense_attention(q, k, v, 0, 1.0).any()


# ---------------------------------------------------------------------------
# semantics of the synthetic workloads: planted pages are routed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("index,batch", [(0, 1), (1, 2), (2, 1), (3, 1), ("llama8b-ctx32k-b16-page4", 1),
                                         ("llama8b-ctx32k-r32-page4", 1),
                                         ("llama8b-ctx32k-b16r16-page4-rope", 1)])
def test_planted_pages_are_selected(index, batch):
    wl = workload(index).with_(batch=batch)
    inp = synth.decode_inputs(wl)
    st = inp["storage"]
    q, z, r = (ref.storage_to_f64(inp[k], st) for k in ("q", "z", "r"))
    P, Q = ref.storage_to_f64(inp["P"], st), ref.storage_to_f64(inp["Q"], st)
    G = wl.group
    for b in range(batch):
        planted = set(inp["planted"][b].tolist())
        assert len(planted) == wl.n_planted
        for g in range(wl.n_kv_heads):
            sc = ref.route_page_scores(q[b, g * G:(g + 1) * G], z[b, g], r[b, g], P[g], Q[g], wl.r_b,
                                       wl.ctx, wl.page_size, wl.max_pages, inp["rope_inv_freq"])
            sel = set(ref.select_pages(sc, wl.max_pages, wl.top_k).tolist())
            assert planted <= sel, (b, g, sorted(planted - sel))


# ---------------------------------------------------------------------------
# rotary position embedding (reading R13: cached states pre-RoPE, predicted and
# exact Keys rotated to their positions; the pages' Figure 6 caption)
# ---------------------------------------------------------------------------

def _freqs(dh, base=10000.0):
    return ref.rope_inverse_frequencies(dh, base)


def test_rope_frequencies_closed_form():
    w = _freqs(128, 500000.0)
    assert w.dtype == np.float32 and w.shape == (64,) and w[0] == 1.0
    np.testing.assert_allclose(w[1:], 500000.0 ** (-np.arange(2, 128, 2) / 128.0), rtol=1e-7)


def test_rope_rotation_matches_pair_matrix_brute():
    """q . R(t) k with the oracle's rotate-half rotation of k equals the brute
    force's transposed 2 x 2 matrices applied to q, (R(t)^T q) . k."""
    rng = np.random.default_rng(41)
    w = _freqs(16, 100.0)
    for t in (0, 1, 7, 1000, 131071):
        q, k = rng.standard_normal(16), rng.standard_normal(16)
        mine = q @ ref.rope_rotate(k[None], [t], w)[0]
        other = brute._dot(brute.rope_unrotate_query(q.tolist(), t, w), k.tolist())
        assert abs(mine - other) <= 1e-12 * max(1.0, abs(mine))


def test_rope_is_a_rotation_of_relative_position():
    """Norms are kept, and (R(s) q) . (R(t) k) = q . R(t - s) k."""
    rng = np.random.default_rng(42)
    w = _freqs(128, 500000.0)
    x = rng.standard_normal((5, 128))
    rx = ref.rope_rotate(x, [0, 3, 99, 4096, 70000], w)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for s_, t in ((5, 9), (1000, 37), (65536, 65539)):
        lhs = ref.rope_rotate(q[None], [s_], w)[0] @ ref.rope_rotate(k[None], [t], w)[0]
        rhs = q @ ref.rope_rotate(k[None], [t - s_], w)[0]
        assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))


def test_rope_with_zero_frequencies_is_the_unrotated_path():
    wl = tiny_workload()
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    zero = np.zeros(wl.head_dim // 2, dtype=np.float32)
    kw = dict(rb=wl.r_b, page_size=wl.page_size, top_k=wl.top_k, n_pages_out=wl.max_pages,
              storage="f64", k_new=d["k_new"], v_new=d["v_new"])
    base = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], inp["seq_lens"], d["A"], d["Bf"], d["P"],
                           d["Q"], d["E"], d["W_O"], **kw)
    rot = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], inp["seq_lens"], d["A"], d["Bf"], d["P"],
                          d["Q"], d["E"], d["W_O"], rope_inv_freq=zero, **kw)
    for key in ("scores", "sel", "u", "y"):
        np.testing.assert_array_equal(rot[key], base[key])


@pytest.mark.parametrize("rb,rq", [(3, 2), (3, 0), (0, 2)])
def test_rope_route_matches_projected_rotated_query_brute(rb, rq):
    """Rotated predicted Key . query = the projected-query route with the
    query turned back by each token's position (brute force, pure Python)."""
    wl = tiny_workload(r_b=rb, r_q=rq)
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    w = _freqs(wl.head_dim, 10.0)
    G = wl.group
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            qg = d["q"][b, g * G:(g + 1) * G]
            mine = ref.route_page_scores(qg, d["z"][b, g], d["r"][b, g], d["P"][g], d["Q"][g], rb, 11,
                                         wl.page_size, wl.max_pages, w)
            other = brute.route_page_scores_rope(qg.tolist(), d["z"][b, g].tolist(),
                                                 d["r"][b, g].tolist(), d["P"][g].tolist(),
                                                 d["Q"][g].tolist(), rb, 11, wl.page_size,
                                                 wl.max_pages, w)
            np.testing.assert_allclose(mine, other, rtol=1e-12, atol=1e-12)


def test_rope_attend_matches_sdpa_on_rotated_keys_and_brute():
    """Attention with RoPE = SDPA (library) on the Keys rotated to their
    positions, and = the brute force's turned-back queries."""
    wl = workload(0).with_(storage="f64", ctx=300, batch=1)
    inp = synth.decode_inputs(wl)
    d = unpack(inp)
    w = _freqs(wl.head_dim, 500000.0)
    G, S, L, scale = wl.group, wl.page_size, 290, 1 / math.sqrt(wl.head_dim)
    sel = np.array([0, 3, 7, 11, 18], dtype=np.int64)
    toks = ref.selected_tokens(sel, L, S)
    qg, kc, z = d["q"][0, :G], d["kc"][0, 0], d["z"][0, 0]
    mine = ref.attend_group(qg, kc, z, sel, L, S, scale, w)
    krot = ref.rope_rotate(kc[toks], toks, w)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qg)[None, :, None], torch.from_numpy(krot)[None, None].expand(1, G, -1, -1),
        torch.from_numpy(z[toks])[None, None].expand(1, G, -1, -1), scale=scale)[0, :, 0].numpy()
    np.testing.assert_allclose(mine, want, rtol=1e-12, atol=1e-12)
    small = tiny_workload()
    sinp = synth.decode_inputs(small)
    sd = unpack(sinp)
    sw = _freqs(small.head_dim, 10.0)
    qs = sd["q"][0, :small.group] * 0.3
    stoks = [0, 1, 4, 5, 8, 9]  # pages 0, 2, 4 of 2-token pages
    other = brute.attend_tokens_rope(qs.tolist(), sd["kc"][0, 0].tolist(), sd["z"][0, 0].tolist(),
                                     stoks, 0.5, sw)
    mine_s = ref.attend_group(qs, sd["kc"][0, 0], sd["z"][0, 0], np.array([0, 2, 4]), 10, 2, 0.5, sw)
    np.testing.assert_allclose(mine_s, other, rtol=1e-12, atol=1e-12)


def test_rope_full_k_invariant_equals_dense_rotated_attention():
    """Exact factors (V = z B, noise-free) and k = all pages: the RoPE decode
    step equals dense softmax attention over the rotated Keys and the Values,
    through W_O (the Full-K reference with positions)."""
    wl = workload(0).with_(storage="f64", ctx=200, batch=1, top_k=13)
    inp = synth.decode_inputs(wl, exact=True)
    d = unpack(inp)
    w = _freqs(wl.head_dim, 500000.0)
    L = 200
    out = ref.decode_step(d["q"], d["z"], d["r"], d["kc"], [L], d["A"], d["Bf"], d["P"], d["Q"],
                          d["E"], d["W_O"], rb=wl.r_b, page_size=wl.page_size, top_k=wl.top_k,
                          n_pages_out=wl.max_pages, storage="f64", rope_inv_freq=w)
    G, scale = wl.group, 1 / math.sqrt(wl.head_dim)
    heads = []
    for g in range(wl.n_kv_heads):
        v = d["z"][0, g, :L] @ d["Bf"][g]
        krot = ref.rope_rotate(d["kc"][0, g, :L], np.arange(L), w)
        heads.append(ref.dense_attention(d["q"][0, g * G:(g + 1) * G], krot, v, L, scale))
    y = np.concatenate(heads).reshape(-1) @ d["W_O"]
    np.testing.assert_allclose(out["y"][0], y, rtol=1e-10, atol=1e-10)
