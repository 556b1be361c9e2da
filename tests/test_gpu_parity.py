"""GPU parity of the whole decode path against the float64 oracle, through the
C ABI (libbasiskv.so on an MI355X).

Every case runs the library's calls (one-token append, query projection,
page scoring, top-k selection, sparse attention, reconstruction) on seeded
synthetic inputs and compares each stage with oracle/ under the rules in
tests/parity.py.  Full-size workloads are checked on sampled sequences (the
oracle recomputes those sequences completely); small ragged cases, which
still span many pages, scoring tiles and attention splits, are checked on
every sequence.
"""

import math

import numpy as np
import pytest
import torch

from oracle import basiskv_ref as ref
from sparse_decode_attention_latent_amd import api, synth
from sparse_decode_attention_latent_amd.configs import workload
from sparse_decode_attention_latent_amd.runner import DecodeProblem, PrefillProblem

import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def compare_step(wl, inp, prob, out, seqs):
    """Check scores, selection, u, y and the appended codes for sequences seqs."""
    st = inp["storage"]
    for b in seqs:
        want = parity.oracle_sequence(wl, inp, b, top_k=prob.top_k, n_pages_out=prob.max_pages)
        n_pages = want["n_pages"]
        for g in range(wl.n_kv_heads):
            where = f"{wl.name} b={b} g={g}"
            parity.check_scores(out["scores"][b, g], want["scores"][g], n_pages, where)
            parity.check_selection(out["sel"][b, g], out["scores"][b, g], want["scores"][g], n_pages,
                                   prob.top_k, where)
        same_sel = np.array_equal(out["sel"][b], want["sel"])
        if not same_sel:  # several selections are correct: attend over the library's own
            want = parity.oracle_sequence(wl, inp, b, top_k=prob.top_k, n_pages_out=prob.max_pages,
                                          sel_override=out["sel"][b])
        eu = parity.rel_rows(out["u"][b], want["u"])
        assert eu.max() <= parity.U_RTOL, f"{wl.name} b={b}: u rel err {eu.max():.3g} head {eu.argmax()}"
        ey = parity.rel_rows(ref.storage_to_f64(out["y"][b], st), want["y"])
        assert ey <= parity.Y_RTOL[st], f"{wl.name} b={b}: y rel err {float(ey):.3g}"
        L = int(inp["seq_lens"][b])
        if L > 0:
            zg, rg = prob.token_codes(b, L - 1)
            for name, gv, wv in (("z", zg, want["z_new"]), ("r", rg, want["r_new"])):
                e = parity.rel_rows(ref.storage_to_f64(gv, st), wv)
                assert e.max() <= parity.CODE_RTOL[st], f"{wl.name} b={b}: appended {name} err {e.max():.3g}"
        _say(f"  {wl.name} b={b} L={L} ok (sel {'=' if same_sel else 'band'}; u {eu.max():.2e}; y {float(ey):.2e})")


def run_case(wl, *, batch=None, ctx=None, seq_lens=None, seqs=None, top_k=None, shuffle_seed=12345):
    _say(f"case {wl.name}: batch={batch or wl.batch} ctx={ctx or wl.ctx} seq_lens={seq_lens} top_k={top_k or wl.top_k}")
    inp = synth.decode_inputs(wl, batch=batch, ctx=ctx, seq_lens=seq_lens)
    prob = DecodeProblem(wl, inp, top_k=top_k, shuffle_seed=shuffle_seed)
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


def test_llama8b_ctx32k_full_sampled():
    run_case(workload(2), seqs=(0, 3, 7))


def test_qwen32b_ctx32k_full_sampled():
    run_case(workload(3), seqs=(0, 3))


def test_prefill_decode_128k_decode_step_sampled():
    # the decode step at the longest context of the prefill + decode workload
    run_case(workload(4), seqs=(0, 1))


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_compress_prefill(storage):
    """(a0) compression of four 4096-token prompts (bf16 workload), and a
    ragged fp32 variant, against the oracle's encoders on every token."""
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
        zs, rs, ks = ref.compress_tokens(ref.storage_to_f64(k[b], storage), ref.storage_to_f64(v[b], storage),
                                         A, P, E, wl.r_b, storage)
        # oracle arrays are [T, Hkv, w]; pools are [B, Hkv, T, w]
        zg = ref.storage_to_f64(got["z"][b], storage).transpose(1, 0, 2)
        rg = ref.storage_to_f64(got["r"][b], storage).transpose(1, 0, 2)
        kg = ref.storage_to_f64(got["k"][b], storage).transpose(1, 0, 2)
        np.testing.assert_array_equal(kg, ks)
        ez, er = parity.rel_rows(zg, zs), parity.rel_rows(rg, rs)
        assert ez.max() <= parity.CODE_RTOL[storage], f"b={b} z err {ez.max():.3g}"
        assert er.max() <= parity.CODE_RTOL[storage], f"b={b} r err {er.max():.3g}"
        if storage == "bf16":
            zb, rbits = got["z"][b].transpose(1, 0, 2), got["r"][b].transpose(1, 0, 2)
            bad_z = parity.bf16_off_by_more_than_one_ulp(zb, zs)
            assert not bad_z.any(), f"b={b}: {int(bad_z.sum())} latent elements off by more than one unit"
            uz = parity.bf16_ulps(zb, zs)
            _say(f"  b={b}: z rel {ez.max():.2e}, one-unit flips {int((uz > 0).sum())}/{uz.size}; "
                 f"r rel {er.max():.2e}")


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


def test_reconstruct_largest_batch():
    wl = workload(1)
    run_case(wl, batch=32, ctx=256, top_k=2, seqs=(0, 17, 31))


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


def test_fused_route_call_equals_the_three_step_calls():
    wl = workload(1)
    inp = synth.decode_inputs(wl, batch=4, ctx=2048)
    prob = DecodeProblem(wl, inp)
    prob.step(append=True)
    base = prob.outputs()
    scores = torch.empty_like(prob.page_scores)
    sel = torch.empty_like(prob.sel)
    api.route_pages(prob.dims, prob.q, prob.fac["P"], prob.fac["Q"], prob.cache, prob.top_k, scores,
                    sel, prob.workspace)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scores.double().cpu().numpy(), base["scores"])
    np.testing.assert_array_equal(sel.cpu().numpy(), base["sel"])
