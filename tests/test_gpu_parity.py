"""GPU parity of the whole decode path against the float64 oracle, through the
C ABI (libbasiskv.so on an MI355X).

Every case runs the library's calls (one-token append, query projection,
page scoring, top-k selection, sparse attention, reconstruction) on seeded
synthetic inputs and compares each stage with oracle/ under the rules in
tests/parity.py.  Every sequence is checked, at the workloads' full sizes
(the oracle recomputes each sequence completely) and in the small ragged
cases, which still span many pages, scoring tiles and attention splits.
"""

import math

import numpy as np
import pytest
import torch

from oracle import basiskv_ref as ref
from sparse_decode_attention_latent_amd import api, synth
from sparse_decode_attention_latent_amd.configs import workload
from sparse_decode_attention_latent_amd.runner import DecodeProblem, DenseProblem, PrefillProblem, to_device

import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def compare_step(wl, inp, prob, out, seqs):
    """Check scores, selection, u, y and the appended codes for sequences seqs."""
    st = inp["storage"]
    cst = inp.get("cache_storage", st)
    rw = prob.recent_tokens
    for b in seqs:
        kw = dict(top_k=prob.top_k, n_pages_out=prob.max_pages, recent_tokens=rw)
        want = parity.oracle_sequence(wl, inp, b, **kw)
        L = int(inp["seq_lens"][b])
        codes, code_dev = None, 0.0
        if L > 0:  # the appended token's stored codes first: the rest is computed from them
            zg, rg, kg = prob.token_codes(b, L - 1)
            code_dev, codes = parity.check_token_codes(wl, inp, b, want, zg, rg, kg, f"{wl.name} b={b}")
            if codes is not None:  # another valid rounding: continue from the library's
                want = parity.oracle_sequence(wl, inp, b, codes_override=codes, **kw)
        n_pages = want["n_candidates"]  # routed among the pages before any recent window
        score_frac = 0.0
        for g in range(wl.n_kv_heads):
            where = f"{wl.name} b={b} g={g}"
            score_frac = max(score_frac, parity.check_scores(out["scores"][b, g], want["scores"][g],
                                                             want["n_pages"], where))
            parity.check_selection(out["sel"][b, g], out["scores"][b, g], want["scores"][g], n_pages,
                                   prob.top_k, where)
        same_sel = np.array_equal(out["sel"][b], want["sel"])
        if not same_sel:  # several selections are correct: attend over the library's own
            want = parity.oracle_sequence(wl, inp, b, sel_override=out["sel"][b],
                                          codes_override=codes, **kw)
        eu = parity.rel_rows(out["u"][b], want["u"])
        assert eu.max() <= parity.U_RTOL, f"{wl.name} b={b}: u rel err {eu.max():.3g} head {eu.argmax()}"
        ey = parity.rel_rows(ref.storage_to_f64(out["y"][b], st), want["y"])
        assert ey <= parity.Y_RTOL[st], f"{wl.name} b={b}: y rel err {float(ey):.3g}"
        _say(f"  {wl.name} b={b} L={L} ok (sel {'=' if same_sel else 'band'}; scores at "
             f"{score_frac:.3f} of SCORE_RTOL; u {eu.max():.2e}; y {float(ey):.2e}; codes "
             f"{code_dev:.1e} from exact{'; library rounding' if codes is not None else ''})")


def run_case(wl, *, batch=None, ctx=None, seq_lens=None, seqs=None, top_k=None, shuffle_seed=12345,
             recent_tokens=None):
    _say(f"case {wl.name}: batch={batch or wl.batch} ctx={ctx or wl.ctx} seq_lens={seq_lens} "
         f"top_k={top_k or wl.top_k} recent={wl.recent_tokens if recent_tokens is None else recent_tokens}")
    inp = synth.decode_inputs(wl, batch=batch, ctx=ctx, seq_lens=seq_lens)
    prob = DecodeProblem(wl, inp, top_k=top_k, shuffle_seed=shuffle_seed,
                         recent_tokens=recent_tokens)
    prob.step(append=True)
    out = prob.outputs()
    B = inp["q"].shape[0]
    compare_step(wl, inp, prob, out, range(B) if seqs is None else seqs)
    return inp, prob, out


# ---------------------------------------------------------------------------
# the five workloads at their full sizes
# ---------------------------------------------------------------------------

def test_tiny_fp32_full():
    run_case(workload(0))


def test_llama8b_ctx4k_full():
    run_case(workload(1))


def test_llama8b_ctx32k_full():
    run_case(workload(2))


def test_qwen32b_ctx32k_full():
    run_case(workload(3))


def test_prefill_decode_128k_decode_step_full():
    # the decode step at the longest context of the prefill + decode workload
    run_case(workload(4))


@pytest.mark.parametrize("name", ["tiny-fp32", "llama8b-ctx4k", "llama8b-ctx32k", "qwen32b-ctx32k",
                                  "llama8b-prefill-decode-128k", "llama8b-ctx32k-b16r16-page4",
                                  "llama8b-ctx32k-fp8", "llama8b-ctx32k-b16r16-page4-fp8",
                                  "llama8b-ctx32k-b16-page4", "llama8b-ctx32k-r16-page4",
                                  "llama8b-ctx32k-r32-page4", "llama8b-ctx32k-b16r16-page4-rope",
                                  "llama8b-ctx32k-rope"])
def test_decode_step_full_size_every_sequence(name):
    """The call bench.py times, basiskv_decode_step, at the workload's full
    size and in the launch configuration the benchmark uses (the same seeded
    inputs, shuffled block table, top_k and workspace): every sequence against
    the oracle, then bit-identical to the library's four separate calls on the
    same problem."""
    wl = workload(name)
    _say(f"decode_step {name}: batch={wl.batch} ctx={wl.ctx} top_k={wl.top_k}")
    inp = synth.decode_inputs(wl)
    prob = DecodeProblem(wl, inp)
    prob.decode_step()
    got = prob.outputs()
    compare_step(wl, inp, prob, got, range(inp["q"].shape[0]))
    for t in (prob.page_scores, prob.u):
        t.fill_(float("nan"))
    prob.sel.fill_(-7)
    prob.y.fill_(0)
    prob.step(append=True)  # the same token appended again at the same position
    base = prob.outputs()
    for key in ("scores", "sel", "u", "y"):
        np.testing.assert_array_equal(got[key], base[key], err_msg=f"one call vs separate calls: {key}")


def test_prefill_decode_128k_sequence_steps():
    """Steps 0, 1, 2, 63 and 127 of the workload's 128 decode steps (context
    131072 - 127 + i, the step's own queries, the new token appended at the
    end), run in order on one cache: each checked against the oracle on the
    cache as the earlier checked steps left it."""
    wl = workload(4)
    inp = synth.decode_inputs(wl)
    st = inp["storage"]
    prob = DecodeProblem(wl, inp)
    L_last = int(inp["seq_lens"].max())
    B = inp["q"].shape[0]
    for i in (0, 1, 2, 63, 127):
        L = L_last - (wl.decode_steps - 1) + i
        q = synth.step_queries(wl, batch=B, step=i)
        prob.seq_lens.fill_(L)
        prob.start_pos.fill_(L - 1)
        prob.q.copy_(to_device(q, st))
        prob.decode_step()
        out = prob.outputs()
        step_inp = dict(inp, q=q, seq_lens=np.full(B, L, dtype=np.int32))
        _say(f"step {i}: ctx {L}")
        compare_step(wl, step_inp, prob, out, range(B))
        fac = {n: ref.storage_to_f64(inp[n], st) for n in ("A", "P", "E")}
        for b in range(B):  # the appended token stays in the cache for the later steps
            zs, rs, _ = ref.compress_tokens(ref.storage_to_f64(inp["k_new"][b:b + 1], st),
                                            ref.storage_to_f64(inp["v_new"][b:b + 1], st),
                                            fac["A"], fac["P"], fac["E"], wl.r_b, st)
            inp["z"][b, :, L - 1] = synth.to_storage(zs[0], st)
            inp["r"][b, :, L - 1] = synth.to_storage(rs[0], st)
            inp["kc"][b, :, L - 1] = inp["k_new"][b]


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_compress_prefill(storage):
    """(a0) compression of four 4096-token prompts (bf16 workload), and a
    ragged fp32 variant, on every token: Keys bit-exact; every latent code a
    valid rounding of the exact latent and every residual code a valid
    rounding of the exact residual formed from the library's own stored
    latent (reading R7; rules in tests/parity.py)."""
    wl = workload(4)
    B, T = (wl.prefill_batch, wl.prefill_tokens) if storage == "bf16" else (3, 1000)
    if storage == "f32":
        wl = wl.with_(storage="f32")
    _say(f"compress {storage}: B={B} T={T}")
    k, v = synth.kv_activations(wl, batch=B, tokens=T, stream=0)
    fac = synth.factors(wl)
    prob = PrefillProblem(wl, k, v, fac, storage=storage)
    prob.run()
    got = prob.logical()
    A, P, E = (ref.storage_to_f64(fac[n], storage) for n in ("A", "P", "E"))
    for b in range(B):
        kb, vb = ref.storage_to_f64(k[b], storage), ref.storage_to_f64(v[b], storage)  # [T, Hkv, dh]
        # pools are [B, Hkv, T, w]
        kg = ref.storage_to_f64(got["k"][b], storage)
        np.testing.assert_array_equal(kg, kb.transpose(1, 0, 2))
        flips, dev = 0, 0.0
        for g in range(wl.n_kv_heads):
            z_exact = ref.latent_code(vb[:, g], A[g])
            zgv = ref.storage_to_f64(got["z"][b, g], storage)
            r_exact = ref.residual_code(kb[:, g], zgv, P[g], E[g], wl.r_b)
            rgv = ref.storage_to_f64(got["r"][b, g], storage)
            if storage == "f32":
                ez, er = parity.rel_rows(zgv, z_exact), parity.rel_rows(rgv, r_exact)
                assert ez.max() <= parity.CODE_RTOL["f32"], f"b={b} g={g}: z err {ez.max():.3g}"
                assert er.max() <= parity.CODE_RTOL["f32"], f"b={b} g={g}: r err {er.max():.3g}"
            else:
                okz = parity.rounding_valid(got["z"][b, g], z_exact, storage)
                assert okz.all(), f"b={b} g={g}: latent codes not a valid rounding at {np.argwhere(~okz)[:4]}"
                okr = parity.rounding_valid(got["r"][b, g], r_exact, storage)
                assert okr.all(), f"b={b} g={g}: residual codes not a valid rounding at {np.argwhere(~okr)[:4]}"
                flips += int((zgv != ref.round_to_storage(z_exact, storage)).sum())
            dev = max(dev, float(parity.rel_rows(zgv, z_exact).max()),
                      float(parity.rel_rows(rgv, r_exact).max()))
        _say(f"  b={b}: codes within {dev:.2e} of the exact values (row-relative); latent codes "
             f"off the nearest-even rounding: {flips}")


# ---------------------------------------------------------------------------
# ragged and degenerate cases (every sequence checked)
# ---------------------------------------------------------------------------

def test_ragged_lengths_bf16():
    """Partial last pages, a sequence with fewer pages than top_k, a
    one-token sequence and an empty one, in the 8B shape."""
    run_case(workload(1), batch=6, ctx=1000, seq_lens=[1000, 999, 33, 1, 0, 517])


def test_ragged_lengths_fp32():
    run_case(workload(0), batch=3, ctx=2048, seq_lens=[2041, 16, 1234])


def test_top_k_at_least_all_pages():
    wl = workload(0)
    run_case(wl, batch=1, ctx=256, top_k=20)  # 16 pages < 20


@pytest.mark.parametrize("page_size", [4, 8, 16, 64])
def test_page_sizes(page_size):
    wl = workload(2).with_(page_size=page_size)
    run_case(wl, batch=2, ctx=3000, seq_lens=[3000, 2001], top_k=24)


@pytest.mark.parametrize("group", [1, 2, 8])
def test_group_sizes(group):
    wl = workload(1).with_(n_q_heads=8 * group)
    run_case(wl, batch=2, ctx=2048, seq_lens=[2048, 1500])


@pytest.mark.parametrize("rv,rq", [(32, 16), (128, 32)])
def test_latent_and_residual_widths(rv, rq):
    wl = workload(2).with_(r_v=rv, r_b=rv, r_q=rq)
    run_case(wl, batch=2, ctx=2048, seq_lens=[2048, 1111], top_k=16)


@pytest.mark.parametrize("wl_index,batch", [(1, 40), (0, 70)])
def test_large_batches(wl_index, batch):
    """Batches past one reconstruction workgroup's 32 (bf16) or 64 (float32)
    rows take several row-tile groups: every sequence checked, and the
    one-call step bit-identical to the separate calls."""
    wl = workload(wl_index)
    inp, prob, out = run_case(wl, batch=batch, ctx=256, top_k=2)
    prob.u.fill_(float("nan"))
    prob.y.fill_(0)
    prob.decode_step()
    got = prob.outputs()
    for key in ("scores", "sel", "u", "y"):
        np.testing.assert_array_equal(got[key], out[key], err_msg=key)


@pytest.mark.parametrize("wl_index", [0, 2, 3])
def test_reconstruct_from_a_plain_fused_matrix(wl_index):
    """A caller's plain fused matrix M = blockdiag(B) W_O, [n_q * r_v][hidden]
    (formed on the host in float64 from the seeded factors and rounded to the
    storage format), packed by basiskv_pack_output_matrix: the tiled copy holds
    the same values bit for bit, and the step run with it matches the oracle
    (whose reconstruction is the unfused u B W_O) and u M with the stored M."""
    wl = workload(wl_index)
    B = min(wl.batch, 4)
    inp = synth.decode_inputs(wl, batch=B, ctx=2048)
    st = inp["storage"]
    prob = DecodeProblem(wl, inp)
    Bf, W_O = ref.storage_to_f64(inp["Bf"], st), ref.storage_to_f64(inp["W_O"], st)
    dh, G = wl.head_dim, wl.group
    m_plain = np.concatenate([Bf[h // G] @ W_O[h * dh:(h + 1) * dh] for h in range(wl.n_q_heads)])
    m_stored = synth.to_storage(m_plain, st)
    packed = torch.empty_like(prob.M)
    api.pack_output_matrix(prob.dims, to_device(m_stored, st), packed)
    from sparse_decode_attention_latent_amd.runner import to_host_storage
    flat = to_host_storage(packed.reshape(-1), st)
    K = wl.n_q_heads * wl.r_v
    np.testing.assert_array_equal(untile_output_matrix(flat, wl.hidden, K, 2 if st == "bf16" else 4),
                                  m_stored.T)
    prob.M.copy_(packed)
    prob.step(append=True)
    out = prob.outputs()
    m64 = ref.storage_to_f64(m_stored, st)
    for b in range(B):
        y_ref = out["u"][b].reshape(-1) @ m64
        ey = parity.rel_rows(ref.storage_to_f64(out["y"][b], st), y_ref)
        assert ey <= (5e-3 if st == "bf16" else 1e-5), f"b={b}: y vs u M err {float(ey):.3g}"
    compare_step(wl, inp, prob, out, range(B))


# ---------------------------------------------------------------------------
# properties
# ---------------------------------------------------------------------------

def test_block_table_permutation_and_determinism_bit_exact():
    """A shuffled block table gives the same bits as the identity table, and a
    second run the same bits as the first (no atomics, fixed reduction order)."""
    wl = workload(2)
    inp = synth.decode_inputs(wl, batch=2, ctx=8192)
    outs = []
    for seed in (None, 99, 99):
        prob = DecodeProblem(wl, inp, top_k=64, shuffle_seed=seed)
        prob.step(append=True)
        outs.append(prob.outputs())
    for o in outs[1:]:
        for key in ("scores", "sel", "u", "y"):
            np.testing.assert_array_equal(o[key], outs[0][key], err_msg=key)


# ---------------------------------------------------------------------------
# the recent window and the pages' adopted router (appendix Tables 9 and 10:
# B16R16 routing, Page4, 2048 routed tokens plus 64 recent tokens, V96)
# ---------------------------------------------------------------------------

def test_recent_window_ragged():
    """Recent window of 64 tokens on 32-token pages (it may start mid-page),
    ragged lengths including sequences shorter than the window."""
    run_case(workload(1), batch=6, ctx=1000, seq_lens=[1000, 999, 33, 1, 0, 517],
             recent_tokens=64)


def test_recent_window_wider_than_some_sequences():
    run_case(workload(2), batch=4, ctx=4096, seq_lens=[4096, 300, 2, 1500], top_k=8,
             recent_tokens=400)


def test_adopted_router_b16r16_page4_full():
    """The adopted router workload at full size (8 x 32K, 8192 pages of 4
    tokens, 512 routed pages + 64 recent tokens), every sequence."""
    run_case(workload("llama8b-ctx32k-b16r16-page4"))


def test_adopted_router_ragged():
    wl = workload("llama8b-ctx32k-b16r16-page4")
    run_case(wl, batch=4, ctx=8192, seq_lens=[8192, 8191, 2100, 63])


def test_recent_window_one_call_step_equals_separate_calls():
    wl = workload(1)
    inp = synth.decode_inputs(wl, batch=3, ctx=4096, seq_lens=[4096, 3000, 70])
    prob = DecodeProblem(wl, inp, top_k=16, recent_tokens=64)
    prob.step_unfused(append=True)
    base = prob.outputs()
    prob.u.fill_(float("nan"))
    prob.decode_step()
    got = prob.outputs()
    for key in ("scores", "sel", "u", "y"):
        np.testing.assert_array_equal(got[key], base[key], err_msg=key)
    compare_step(wl, inp, prob, got, range(3))


# ---------------------------------------------------------------------------
# single-source routers (appendix Table 9: B16 from the latent's leading 16
# dims alone, R16 / R32 from the residual alone)
# ---------------------------------------------------------------------------

SINGLE_SOURCE = ("llama8b-ctx32k-b16-page4", "llama8b-ctx32k-r16-page4", "llama8b-ctx32k-r32-page4")


@pytest.mark.parametrize("name", SINGLE_SOURCE)
def test_single_source_router_ragged(name):
    run_case(workload(name), batch=4, ctx=4096, seq_lens=[4096, 4095, 700, 63])


@pytest.mark.parametrize("name", SINGLE_SOURCE)
@pytest.mark.parametrize("fmt", ["fp8", "f32", "page32"])
def test_single_source_router_formats(name, fmt):
    """E4M3 pages; float32 (latent width 64); 32-token pages without a recent
    window."""
    wl = workload(name)
    if fmt == "fp8":
        wl = wl.with_(cache_storage="fp8")
    elif fmt == "f32":
        wl = wl.with_(storage="f32", r_v=64)
    else:
        wl = wl.with_(page_size=32, recent_tokens=0)
    top_k = 64 if wl.page_size == 4 else 16
    run_case(wl, batch=2, ctx=2048, seq_lens=[2048, 999], top_k=top_k)


@pytest.mark.parametrize("rb,rq", [(16, 0), (0, 32)])
@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_compress_prefill_single_source(rb, rq, cache):
    """(a0) on the MFMA path without a residual (r_q = 0: latents only) and
    without latent prediction (r_b = 0: the residual is the Key through E),
    every token checked under the rounding rules of tests/parity.py."""
    wl = workload(4).with_(r_b=rb, r_q=rq, cache_storage="fp8" if cache == "fp8" else "")
    B, T = 2, 700
    k, v = synth.kv_activations(wl, batch=B, tokens=T, stream=5)
    fac = synth.factors(wl)
    prob = PrefillProblem(wl, k, v, fac, storage="bf16", cache_storage=cache)
    prob.run()
    got = prob.logical()
    A, P, E = (ref.storage_to_f64(fac[n], "bf16") for n in ("A", "P", "E"))
    for b in range(B):
        kb, vb = ref.storage_to_f64(k[b], "bf16"), ref.storage_to_f64(v[b], "bf16")
        np.testing.assert_array_equal(ref.storage_to_f64(got["k"][b], cache),
                                      ref.round_to_storage(kb, cache).transpose(1, 0, 2))
        assert got["r"][b].shape[-1] == rq
        for g in range(wl.n_kv_heads):
            okz = parity.rounding_valid(got["z"][b, g], ref.latent_code(vb[:, g], A[g]), cache)
            assert okz.all(), f"b={b} g={g}: latent codes"
            if rq:
                zgv = ref.storage_to_f64(got["z"][b, g], cache)
                r_exact = ref.residual_code(kb[:, g], zgv, P[g], E[g], rb)
                assert parity.rounding_valid(got["r"][b, g], r_exact, cache).all(), f"b={b} g={g}: residual"
    _say(f"  compress r_b={rb} r_q={rq} {cache}: every token valid")


# ---------------------------------------------------------------------------
# rotary position embedding: pre-RoPE caches, predicted and exact Keys rotated
# to their positions (the pages' Figure 6 caption; reading in oracle/basiskv_ref.py)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,cache", [
    ("llama8b-ctx32k-b16r16-page4-rope", "bf16"), ("llama8b-ctx32k-b16r16-page4-rope", "fp8"),
    ("llama8b-ctx32k-rope", "bf16"), ("llama8b-ctx32k-rope", "fp8"), ("qwen32b-rope", "bf16")])
def test_rope_ragged(name, cache):
    """Ragged lengths (a partial last page, a sequence shorter than one scoring
    tile, a one-token sequence) with positions up to 4095."""
    wl = workload(name) if name != "qwen32b-rope" else workload(3).with_(rope_theta=1000000.0)
    if cache == "fp8":
        wl = wl.with_(cache_storage="fp8")
    top_k = None if wl.page_size == 4 else 16
    run_case(wl, batch=4, ctx=4096, seq_lens=[4096, 4093, 50, 1], top_k=top_k)


@pytest.mark.parametrize("name", ["llama8b-ctx32k-b16r16-page4-rope", "llama8b-ctx32k-rope"])
def test_rope_separate_calls_equal_routing(name):
    """basiskv_score_pages_rope + basiskv_select_pages give route_pages'
    scores and selection bit for bit, and the rest of the step follows."""
    wl = workload(name)
    inp = synth.decode_inputs(wl, batch=3, ctx=4096, seq_lens=[4096, 2049, 31])
    prob = DecodeProblem(wl, inp)
    prob.step(append=True)
    a = prob.outputs()
    for t in (prob.page_scores, prob.u):
        t.fill_(float("nan"))
    prob.sel.fill_(-7)
    prob.step_unfused(append=False)
    b = prob.outputs()
    for key in ("scores", "sel", "u", "y"):
        np.testing.assert_array_equal(b[key], a[key], err_msg=key)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_rope_routing_first_layout(cache):
    """RoPE routing and attention over routing-first pages (the RoPE kernels
    read a page's routing dims and latent chunks through the pool geometry),
    ragged lengths, against the oracle."""
    wl = workload("llama8b-ctx32k-b16r16-page4-rope").with_(page_layout=1)
    if cache == "fp8":
        wl = wl.with_(cache_storage="fp8")
    run_case(wl, batch=3, ctx=4096, seq_lens=[4096, 2001, 9])


@pytest.mark.parametrize("batch,ctx,top_k", [(2, 32768, 4096), (1, 65536, 12500)])
def test_rope_long_split_plans(batch, ctx, top_k):
    """RoPE attention split plans beyond the benchmark's: three-block wavefronts
    with more splits than the position-free plan would take (top_k 4096), and
    splits of several rounds each (top_k 12500, over the split cap)."""
    wl = workload("llama8b-ctx32k-b16r16-page4-rope")
    lens = [ctx, ctx - 2767][:batch]
    run_case(wl, batch=batch, ctx=ctx, seq_lens=lens, top_k=top_k)


@pytest.mark.parametrize("page_size", [8, 16, 64])
def test_rope_page_sizes(page_size):
    """RoPE routing and attention at the other page sizes (pages per 64-token
    step 8, 4 and 1/2), ragged lengths."""
    wl = workload("llama8b-ctx32k-rope").with_(page_size=page_size)
    run_case(wl, batch=2, ctx=4096, seq_lens=[4096, 1500], top_k=4096 // page_size // 8)


def test_rope_long_positions():
    """Positions up to 131071: rotation angles of the highest frequency reach
    about 1.3e5 radians, where the turn count has to be reduced exactly."""
    wl = workload(4).with_(rope_theta=500000.0, n_planted=8, planted="random")
    run_case(wl, seq_lens=[131072, 98305])


def test_rope_zero_frequencies_equal_no_rope():
    """An all-zero frequency table rotates nothing: the RoPE kernels give the
    position-free kernels' selection, and their scores and u within the parity
    tolerances (the two sum in different orders)."""
    wl = workload("llama8b-ctx32k-b16r16-page4")
    inp = synth.decode_inputs(wl, batch=2, ctx=2048, seq_lens=[2048, 777])
    plain = DecodeProblem(wl, inp)
    plain.decode_step()
    a = plain.outputs()
    zero = DecodeProblem(wl, inp)
    zero.rope_inv_freq = torch.zeros(wl.head_dim // 2, dtype=torch.float32, device="cuda")
    zero.cache = api.make_cache(zero.z_pages, zero.r_pages, zero.k_pages, zero.block_table,
                                zero.seq_lens, zero.rope_inv_freq)
    zero.decode_step()
    b = zero.outputs()
    np.testing.assert_array_equal(b["sel"], a["sel"])
    np.testing.assert_allclose(b["scores"], a["scores"], rtol=parity.SCORE_RTOL, atol=0)
    np.testing.assert_allclose(b["u"], a["u"], rtol=0, atol=parity.U_RTOL * np.abs(a["u"]).max())


# ---------------------------------------------------------------------------
# the dense baseline (full-context Key and Value reads; the pages' Table 3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wl_index,seq_lens", [(2, [4096, 1000, 0, 33]), (3, [4096, 2047])])
def test_dense_attend_matches_oracle(wl_index, seq_lens):
    wl = workload(wl_index)
    B = len(seq_lens)
    inp = synth.decode_inputs(wl, batch=B, ctx=4096, seq_lens=seq_lens)
    st = inp["storage"]
    rng = np.random.default_rng(31)
    v = synth.to_storage(rng.standard_normal(inp["kc"].shape), st)
    prob = DecodeProblem(wl, inp)
    dense = DenseProblem(prob, v=v)
    dense.step()
    torch.cuda.synchronize()
    o = dense.o.double().cpu().numpy()
    y = ref.storage_to_f64(dense.y.view(torch.int16).cpu().numpy().view(np.uint16), st)
    q = ref.storage_to_f64(inp["q"], st)
    kc, vv = ref.storage_to_f64(inp["kc"], st), ref.storage_to_f64(v, st)
    W_O = ref.storage_to_f64(inp["W_O"], st)
    G, scale = wl.group, 1 / math.sqrt(wl.head_dim)
    for b, L in enumerate(seq_lens):
        want = np.concatenate([ref.dense_attention(q[b, g * G:(g + 1) * G], kc[b, g], vv[b, g], L, scale)
                               for g in range(wl.n_kv_heads)])
        eo = parity.rel_rows(o[b], want)
        assert eo.max() <= parity.U_RTOL, f"b={b}: o rel err {eo.max():.3g}"
        ey = parity.rel_rows(y[b], want.reshape(-1) @ W_O)
        assert ey <= parity.Y_RTOL[st], f"b={b}: y rel err {float(ey):.3g}"
        _say(f"  dense {wl.name} b={b} L={L}: o {eo.max():.2e} y {float(ey):.2e}")


@pytest.mark.parametrize("wl_index", [1, 2, 4])
def test_combined_calls_equal_the_separate_calls(wl_index):
    """route_pages gives the bits of project + score + select, and the
    whole-step call (compression and projection sharing one launch) the bits
    of the four separate calls, also when repeated on one workspace."""
    wl = workload(wl_index)
    inp = synth.decode_inputs(wl, batch=4, ctx=8192, seq_lens=[8192, 8000, 33, 4097])
    prob = DecodeProblem(wl, inp, top_k=16)
    prob.step_unfused(append=True)
    base = prob.outputs()
    for call in ("step", "decode_step", "decode_step", "step"):
        for t in (prob.page_scores, prob.u):
            t.fill_(float("nan"))
        prob.sel.fill_(-7)
        prob.y.fill_(0)
        getattr(prob, call)()
        got = prob.outputs()
        for key in ("scores", "sel", "u", "y"):
            np.testing.assert_array_equal(got[key], base[key], err_msg=f"{call} {key}")
    compare_step(wl, inp, prob, got, range(4))


@pytest.mark.parametrize("name", ["llama8b-ctx32k", "qwen32b-ctx32k", "llama8b-ctx32k-fp8"])
def test_step_new_token_scored_beside_the_scan(name):
    """With a long scan (8 sequences of 32K-token capacity: 200 MB of routing
    reads and more) the one-call step compresses and scores each sequence's
    new token in workgroups of its own inside the scoring launch, the scan
    leaves that token out, and the selection folds the token's score into
    its page's.  With the new tokens scaled up (8x, either sign) some of them
    hold their page's and their row's highest score: page scores, selection,
    u and y are still bit-identical to the separate calls (which append first
    and scan every token), and such a page is selected.  Ragged lengths: new
    tokens that open a page, fill one, or are a sequence's only token."""
    wl = workload(name)
    S = wl.page_size
    lens = [32768, 32768 - S + 1, 4096, S + 1, 1, 20000, S - 1, 2 * S]
    inp = synth.decode_inputs(wl, batch=8, ctx=32768, seq_lens=lens)
    decided = 0
    for sign in (8.0, -8.0):
        prob = DecodeProblem(wl, inp, top_k=16)
        prob.k_new.mul_(sign)
        prob.v_new.mul_(sign)
        _say(f"new token x{sign} {name}: seq_lens={lens}")
        prob.decode_step()
        got = prob.outputs()
        for t in (prob.page_scores, prob.u):
            t.fill_(float("nan"))
        prob.sel.fill_(-7)
        prob.y.fill_(0)
        prob.step_unfused(append=True)  # the same token appended again, then scanned with the rest
        base = prob.outputs()
        for key in ("scores", "sel", "u", "y"):
            np.testing.assert_array_equal(got[key], base[key], err_msg=f"x{sign} {key}")
        for b, L in enumerate(lens):
            npg = (L - 1) // wl.page_size  # the new token's page
            NP = -(-L // wl.page_size)
            for g in range(wl.n_kv_heads):
                row = got["scores"][b, g, :NP]
                if row[npg] == row.max():
                    decided += 1
                    assert npg in set(got["sel"][b, g].tolist()), (b, g)
    _say(f"  rows whose top page score is the new token's page: {decided}")
    assert decided > 0


def test_repeated_steps_reuse_the_workspace_bit_exact():
    """Steps that merge several attention splits (the merge counters return to
    zero after every call) give identical bits call after call."""
    wl = workload(2)
    inp = synth.decode_inputs(wl, batch=3, ctx=16384, seq_lens=[16384, 9000, 100])
    prob = DecodeProblem(wl, inp, top_k=128)
    outs = []
    for _ in range(4):
        prob.u.fill_(float("nan"))
        prob.step(append=True)
        outs.append(prob.outputs())
    for o in outs[1:]:
        for key in ("scores", "sel", "u", "y"):
            np.testing.assert_array_equal(o[key], outs[0][key], err_msg=key)
    compare_step(wl, inp, prob, outs[-1], range(3))


def _new_queries(prob, seed):
    """Seeded N(0, 1) queries of the problem's shape, written into prob.q."""
    gen = torch.Generator().manual_seed(seed)
    prob.q.copy_(torch.randn(tuple(prob.q.shape), generator=gen).to(prob.q.dtype))


def _separate_calls(prob):
    """The same step as the library's separate calls, after the one-call step
    (its new token appended again at the same position), as host arrays."""
    for t in (prob.page_scores, prob.u):
        t.fill_(float("nan"))
    prob.sel.fill_(-7)
    prob.y.fill_(0)
    prob.step(append=True)
    return prob.outputs()


@pytest.mark.parametrize("name", ["llama8b-ctx32k", "qwen32b-ctx32k", "llama8b-ctx32k-fp8"])
def test_decode_steps_with_new_queries_every_call(name):
    """One-call steps where the scoring launch projects the queries itself
    (long scans): three calls in a row, each with new queries, each
    bit-identical to the separate calls on the same queries -- a call that
    scored with an earlier call's projected queries would differ."""
    wl = workload(name)
    _say(f"decode_step, new queries per call, {name}: batch={wl.batch} ctx={wl.ctx}")
    inp = synth.decode_inputs(wl)
    prob = DecodeProblem(wl, inp)
    for i in range(3):
        _new_queries(prob, 100 + i)
        prob.decode_step()
        got = prob.outputs()
        base = _separate_calls(prob)
        for key in ("scores", "sel", "u", "y"):
            np.testing.assert_array_equal(got[key], base[key], err_msg=f"call {i}: {key}")


@pytest.mark.parametrize("name", ["llama8b-ctx32k", "qwen32b-ctx32k"])
def test_decode_step_graph_replays_with_new_queries(name):
    """The one-call step captured once in a HIP graph and replayed with new
    queries each time (eager work and synchronisations between replays): every
    replay bit-identical to the separate calls on its queries.  The step's
    epoch lives in device memory, so replays never take an earlier replay's
    projected queries for their own (4- and 8-head groups)."""
    wl = workload(name)
    _say(f"decode_step graph replays: batch={wl.batch} ctx={wl.ctx}")
    inp = synth.decode_inputs(wl)
    prob = DecodeProblem(wl, inp)
    prob.decode_step()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            prob.decode_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(3):
        _new_queries(prob, 200 + i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = prob.outputs()
        base = _separate_calls(prob)
        for key in ("scores", "sel", "u", "y"):
            np.testing.assert_array_equal(got[key], base[key], err_msg=f"replay {i}: {key}")


@pytest.mark.parametrize("page_size,ctx", [(8, 100000), (4, 80000), (4, 131072)])
def test_long_rows_selection(page_size, ctx):
    """Rows of 12500, 20000 and 32768 pages (the largest max_pages_per_seq the
    library takes): the selection runs as its own launch with 1024 threads per
    row; every sequence checked against the oracle."""
    wl = workload(0).with_(page_size=page_size)
    run_case(wl, batch=1, ctx=ctx, top_k=40)


def _crafted_rows(n_rows, n, rng):
    """Score rows that exercise every path of the selection: both signs (the
    value-bucket first digit), a tiny range with many ties, -inf entries, one
    value everywhere, two values, a range too wide for float32 (the bit-digit
    path), +0 / -0 ties, subnormal scores, and normal scores whose range is
    too small for a finite bucket scale (both back to the bit digits)."""
    rows = []
    for r in range(n_rows):
        kind = r % 10
        x = rng.standard_normal(n).astype(np.float32)
        if kind == 1:
            x = (1.0 + rng.integers(0, 50, n) * 2.0 ** -20).astype(np.float32)
        elif kind == 2:
            x[rng.choice(n, n // 10, replace=False)] = -np.inf
        elif kind == 3:
            x[:] = 0.25
        elif kind == 4:
            x = np.where(rng.random(n) < 0.3, 1.0, 0.0).astype(np.float32)
        elif kind == 5:
            x[rng.choice(n, 3, replace=False)] = np.float32([3e38, -3e38, 2e38])
        elif kind == 6:
            x = (x * 1e-30).astype(np.float32)
        elif kind == 7:
            x = np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)) + \
                np.where(rng.random(n) < 0.01, np.float32(1.0), np.float32(0.0))
        elif kind == 8:  # subnormal scores: a range whose 256 / range overflows
            x = (rng.integers(0, 40, n).astype(np.uint32)).view(np.float32).copy()
        elif kind == 9:  # normal scores a few units apart: range ~5e-37 < 256 / FLT_MAX
            base = np.float32(1e-30).view(np.uint32)
            x = (base + rng.integers(0, 6, n).astype(np.uint32)).view(np.float32).copy()
        rows.append(x.astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("max_pages,top_k", [(2048, 100), (8192, 512), (12000, 640)])
def test_select_crafted_rows_match_oracle(max_pages, top_k):
    """basiskv_select_pages on crafted score rows (rows of 2048 pages run on
    four wavefronts with bit digits; 8192 and 12000 on sixteen, starting with
    value buckets) is exactly the oracle's selection, including ragged
    sequence lengths and a recent window."""
    rng = np.random.default_rng(max_pages)
    B, hkv, S = 8, 2, 4
    scores = _crafted_rows(B * hkv, max_pages, rng).reshape(B, hkv, max_pages)
    seq_lens = np.array([max_pages * S - 3 * i * S - i for i in range(B)], dtype=np.int32)
    for recent in (0, 64):
        d = api.make_dims(batch=B, n_q_heads=4 * hkv, n_kv_heads=hkv, head_dim=128, hidden=256,
                          r_v=64, r_b=64, r_q=32, page_size=S, max_pages_per_seq=max_pages,
                          num_phys_pages=B * max_pages, dtype=api.BF16, recent_tokens=recent)
        sc = torch.from_numpy(scores).cuda()
        sl = torch.from_numpy(seq_lens).cuda()
        sel = torch.full((B, hkv, top_k), -7, dtype=torch.int32, device="cuda")
        api.select_pages(d, sc, sl, top_k, sel)
        got = sel.cpu().numpy()
        for b in range(B):
            n_cand = ref.recent_window_first_page(int(seq_lens[b]), S, recent)
            for g in range(hkv):
                want = ref.select_pages(scores[b, g].astype(np.float64), n_cand, top_k)
                np.testing.assert_array_equal(got[b, g], want, err_msg=f"b={b} g={g} recent={recent}")
    _say(f"  select {max_pages} pages, k={top_k}: all rows exact")


@pytest.mark.parametrize("wl_index,ctx", [(2, 4096), (4, 8192 * 8)])
def test_all_scores_tied_selects_lowest_pages(wl_index, ctx):
    """Zero queries make every page score 0: the k lowest page indices are
    selected (ties go to the lower index), through the fused and the
    separate selection paths."""
    wl = workload(wl_index)
    inp = synth.decode_inputs(wl, batch=2, ctx=ctx, seq_lens=[ctx, ctx - 100])
    inp["q"] = np.zeros_like(inp["q"])
    prob = DecodeProblem(wl, inp, top_k=24)
    prob.step(append=True)
    out = prob.outputs()
    S = wl.page_size
    for b, L in enumerate(inp["seq_lens"]):
        n_pages = -(-int(L) // S)
        assert np.all(out["scores"][b][:, :n_pages] == 0.0)
        for g in range(wl.n_kv_heads):
            np.testing.assert_array_equal(out["sel"][b, g], np.arange(24))
    compare_step(wl, inp, prob, out, range(2))


# ---------------------------------------------------------------------------
# FP8 E4M3 cache pages (appendix Table 13: BasisKV under an E4M3 KV cache);
# bf16 queries, factors, inputs and output; rules in tests/parity.py
# ---------------------------------------------------------------------------

FP8 = "llama8b-ctx32k-fp8"
FP8_ADOPTED = "llama8b-ctx32k-b16r16-page4-fp8"


def test_fp8_headline_full():
    run_case(workload(FP8))


def test_fp8_adopted_router_full():
    run_case(workload(FP8_ADOPTED))


def test_fp8_ragged_lengths():
    run_case(workload(FP8), batch=6, ctx=1000, seq_lens=[1000, 999, 33, 1, 0, 517], top_k=16)


def test_fp8_adopted_router_ragged():
    run_case(workload(FP8_ADOPTED), batch=4, ctx=8192, seq_lens=[8192, 8191, 2100, 63])


@pytest.mark.parametrize("wl_index", [1, 3])
def test_fp8_other_shapes(wl_index):
    """Latent 96 / residual 48, groups of 4 and of 8 (the 8-head group runs as
    two 4-head subgroups), E4M3 pages."""
    wl = workload(wl_index).with_(cache_storage="fp8")
    run_case(wl, batch=3, ctx=4096, seq_lens=[4096, 2500, 77], top_k=16)


@pytest.mark.parametrize("page_size", [4, 8, 16, 64])
def test_fp8_page_sizes(page_size):
    wl = workload(FP8).with_(page_size=page_size)
    run_case(wl, batch=2, ctx=3000, seq_lens=[3000, 2001], top_k=24)


@pytest.mark.parametrize("group", [1, 2, 8])
def test_fp8_group_sizes(group):
    wl = workload(1).with_(n_q_heads=8 * group, cache_storage="fp8")
    run_case(wl, batch=2, ctx=2048, seq_lens=[2048, 1500])


def test_fp8_recent_window_ragged():
    run_case(workload(FP8), batch=5, ctx=1000, seq_lens=[1000, 999, 33, 1, 517], top_k=8,
             recent_tokens=64)


def test_fp8_combined_calls_equal_the_separate_calls():
    wl = workload(FP8)
    inp = synth.decode_inputs(wl, batch=3, ctx=8192, seq_lens=[8192, 5000, 40])
    prob = DecodeProblem(wl, inp, top_k=32)
    prob.step_unfused(append=True)
    base = prob.outputs()
    prob.u.fill_(float("nan"))
    prob.decode_step()
    got = prob.outputs()
    for key in ("scores", "sel", "u", "y"):
        np.testing.assert_array_equal(got[key], base[key], err_msg=key)
    compare_step(wl, inp, prob, got, range(3))


def test_fp8_append_saturates():
    """A new token whose Key and Value are far beyond the E4M3 range: the
    stored codes saturate at +-448 (no NaN code), as the oracle's rounding."""
    wl = workload(FP8)
    inp = synth.decode_inputs(wl, batch=2, ctx=2048, seq_lens=[2048, 999])
    st = inp["storage"]
    for key in ("k_new", "v_new"):
        inp[key] = synth.to_storage(synth.from_storage(inp[key], st) * 2000.0, st)
    prob = DecodeProblem(wl, inp, top_k=16)
    prob.step(append=True)
    out = prob.outputs()
    for b, L in enumerate((2048, 999)):
        z, r, k = prob.token_codes(b, L - 1)
        assert not np.any((k & 0x7F) == 0x7F) and not np.any((z & 0x7F) == 0x7F)
        assert np.any(k == 0x7E) or np.any(k == 0xFE)
    compare_step(wl, inp, prob, out, range(2))


def test_fp8_compress_prefill():
    """(a0) compression of ragged prompts into E4M3 pages on the MFMA path:
    every Key code bit-exact, every latent and residual code a valid rounding
    (tests/parity.py), on every token."""
    wl = workload(4).with_(cache_storage="fp8")
    B, T = 3, 1000
    k, v = synth.kv_activations(wl, batch=B, tokens=T, stream=0)
    fac = synth.factors(wl)
    prob = PrefillProblem(wl, k, v, fac, storage="bf16", cache_storage="fp8")
    prob.run()
    got = prob.logical()
    A, P, E = (ref.storage_to_f64(fac[n], "bf16") for n in ("A", "P", "E"))
    flips = 0
    for b in range(B):
        kb, vb = ref.storage_to_f64(k[b], "bf16"), ref.storage_to_f64(v[b], "bf16")  # [T, Hkv, dh]
        zs, rs, ks = ref.compress_tokens(kb, vb, A, P, E, wl.r_b, "fp8")
        zg = got["z"][b].transpose(1, 0, 2)  # codes [T, Hkv, w]
        rg = got["r"][b].transpose(1, 0, 2)
        kg = got["k"][b].transpose(1, 0, 2)
        np.testing.assert_array_equal(ref.storage_to_f64(kg, "fp8"), ks)
        for g in range(wl.n_kv_heads):
            z_exact = ref.latent_code(vb[:, g], A[g])
            assert parity.rounding_valid(zg[:, g], z_exact, "fp8").all(), f"b={b} g={g}: latent codes"
            zgv = ref.storage_to_f64(zg[:, g], "fp8")
            r_exact = ref.residual_code(kb[:, g], zgv, P[g], E[g], wl.r_b)
            assert parity.rounding_valid(rg[:, g], r_exact, "fp8").all(), f"b={b} g={g}: residual codes"
        flips += int((ref.storage_to_f64(zg, "fp8") != zs).sum())
    _say(f"  fp8 compress: latent codes differing from the oracle's rounding: {flips}")


@pytest.mark.parametrize("seq_lens", [[4096, 1000, 0, 33]])
def test_fp8_dense_attend_matches_oracle(seq_lens):
    """The dense baseline over E4M3 Key and Value pages (Table 13's Full-K
    FP8 row's data format)."""
    wl = workload(FP8)
    B = len(seq_lens)
    inp = synth.decode_inputs(wl, batch=B, ctx=4096, seq_lens=seq_lens)
    rng = np.random.default_rng(37)
    v = synth.to_storage(rng.standard_normal(inp["kc"].shape), "fp8")
    prob = DecodeProblem(wl, inp)
    dense = DenseProblem(prob, v=v)
    dense.step()
    torch.cuda.synchronize()
    o = dense.o.double().cpu().numpy()
    y = ref.storage_to_f64(dense.y.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    q = ref.storage_to_f64(inp["q"], "bf16")
    kc, vv = ref.storage_to_f64(inp["kc"], "fp8"), ref.storage_to_f64(v, "fp8")
    W_O = ref.storage_to_f64(inp["W_O"], "bf16")
    G, scale = wl.group, 1 / math.sqrt(wl.head_dim)
    for b, L in enumerate(seq_lens):
        want = np.concatenate([ref.dense_attention(q[b, g * G:(g + 1) * G], kc[b, g], vv[b, g], L, scale)
                               for g in range(wl.n_kv_heads)])
        eo = parity.rel_rows(o[b], want)
        assert eo.max() <= parity.U_RTOL, f"b={b}: o rel err {eo.max():.3g}"
        ey = parity.rel_rows(y[b], want.reshape(-1) @ W_O)
        assert ey <= parity.Y_RTOL["bf16"], f"b={b}: y rel err {float(ey):.3g}"
        _say(f"  dense fp8 b={b} L={L}: o {eo.max():.2e} y {float(ey):.2e}")


# ---------------------------------------------------------------------------
# the routing-first page layout (latent and residual in one pool, each page's
# routing dims first): the same results, bit for bit, as the separate pools
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,batch,ctx,seq_lens,top_k", [
    ("llama8b-ctx32k", 3, 4096, [4096, 3000, 33], 16),
    ("llama8b-ctx32k-fp8", 3, 4096, [4096, 2222, 1], 16),
    ("llama8b-ctx32k-b16r16-page4", 3, 4096, [4096, 4095, 100], None),
    ("llama8b-ctx32k-b16r16-page4-fp8", 3, 4096, [4096, 1234, 65], None),
    ("qwen32b-ctx32k", 2, 4096, [4096, 777], 16),
    ("tiny-fp32", 2, 2048, [2048, 1000], None),
])
def test_routing_first_layout_matches_separate_pools(name, batch, ctx, seq_lens, top_k):
    wl = workload(name)
    _say(f"routing-first {name}: batch={batch} ctx={ctx} seq_lens={seq_lens}")
    inp = synth.decode_inputs(wl, batch=batch, ctx=ctx, seq_lens=seq_lens)
    outs, probs = [], []
    for lay in (api.LAYOUT_SEPARATE, api.LAYOUT_ROUTING_FIRST):
        prob = DecodeProblem(wl, inp, top_k=top_k, page_layout=lay)
        prob.step_unfused(append=True)
        a = prob.outputs()
        codes = [prob.token_codes(b, int(L) - 1) for b, L in enumerate(seq_lens) if L > 0]
        prob.u.fill_(float("nan"))
        prob.decode_step()  # the one-call step on the same (already appended) cache
        outs.append((a, codes, prob.outputs()))
        probs.append(prob)
    (a0, c0, d0), (a1, c1, d1) = outs
    for key in ("scores", "sel", "u", "y"):
        np.testing.assert_array_equal(a1[key], a0[key], err_msg=key)
        np.testing.assert_array_equal(d1[key], d0[key], err_msg="one-call " + key)
    for x, y in zip(c0, c1):
        for u, v in zip(x, y):
            np.testing.assert_array_equal(v, u)
    compare_step(wl, inp, probs[1], a1, range(batch))


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_routing_first_prefill_compress_matches_separate_pools(cache):
    wl = workload(4).with_(cache_storage=cache if cache == "fp8" else "")
    k, v = synth.kv_activations(wl, batch=2, tokens=700, stream=3)
    fac = synth.factors(wl)
    got = []
    for lay in (api.LAYOUT_SEPARATE, api.LAYOUT_ROUTING_FIRST):
        prob = PrefillProblem(wl, k, v, fac, storage="bf16", cache_storage=cache, page_layout=lay)
        prob.run()
        got.append(prob.logical())
    for key in ("z", "r", "k"):
        np.testing.assert_array_equal(got[1][key], got[0][key], err_msg=key)


def untile_output_matrix(flat, hidden, K, itemsize):
    """The documented tiled layout of the fused output matrix back to [hidden][K]."""
    kl = 16 // itemsize
    ks = 4 * kl
    n = np.arange(hidden)[:, None]
    k = np.arange(K)[None, :]
    idx = ((n // 16 * (K // ks) + k // ks) * 64 + (k % ks) // kl * 16 + n % 16) * kl + k % kl
    return flat[idx]


@pytest.mark.parametrize("wl_index", [0, 2, 3])
def test_fused_output_matrix_layout(wl_index):
    """basiskv_fuse_output_matrix writes M = (blockdiag(B) W_O)^T in the tiled
    layout the header documents (checked against numpy in float64)."""
    wl = workload(wl_index)
    inp = synth.decode_inputs(wl, batch=1, ctx=64)
    prob = DecodeProblem(wl, inp)
    st = inp["storage"]
    K = wl.n_q_heads * wl.r_v
    from sparse_decode_attention_latent_amd.runner import to_host_storage
    flat = ref.storage_to_f64(to_host_storage(prob.M.reshape(-1), st), st)
    got = untile_output_matrix(flat, wl.hidden, K, 2 if st == "bf16" else 4)
    Bf = ref.storage_to_f64(inp["Bf"], st)
    W_O = ref.storage_to_f64(inp["W_O"], st)
    want = np.zeros((wl.hidden, K))
    for h in range(wl.n_q_heads):
        blk = Bf[h // wl.group] @ W_O[h * wl.head_dim:(h + 1) * wl.head_dim]  # [r_v, hidden]
        want[:, h * wl.r_v:(h + 1) * wl.r_v] = blk.T
    tol = 1e-5 if st == "f32" else 8e-3
    err = np.abs(got - want).max() / np.abs(want).max()
    assert err <= tol, err
