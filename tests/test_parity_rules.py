"""The GPU parity rules themselves, checked on the CPU (no GPU, no library).

The rounding band of tests/parity.py must (a) accept every code a correct
kernel can store -- float32 arithmetic in the kernels' orders, simulated
here in numpy float32 -- and (b) reject a plausible mistake: a residual
formed from the unrounded latent instead of the stored one (the reading R7
of the BasisKV abstract: the residual keeps what the *cached* latent cannot
predict), and a latent stored by truncation instead of round-to-nearest-even.
Mistakes are planted in oracle outputs, on the CPU.
"""

import numpy as np
import pytest

from oracle import basiskv_ref as ref
from sparse_decode_attention_latent_amd import synth
from sparse_decode_attention_latent_amd.configs import workload

import parity


def _bf16_bits(x64):
    """float64 values exactly representable in bf16 -> uint16 bits."""
    return (np.asarray(x64, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _truncate_bf16(x):
    """Round toward zero to bf16 (a wrong rounding mode), as float64."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


def _case(idx, tokens=400):
    wl = workload(idx)
    k, v = synth.kv_activations(wl, batch=1, tokens=tokens, stream=0)
    fac = synth.factors(wl)
    A, P, E = (ref.storage_to_f64(fac[n], "bf16") for n in ("A", "P", "E"))
    return wl, ref.storage_to_f64(k[0], "bf16"), ref.storage_to_f64(v[0], "bf16"), A, P, E


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_band_accepts_float32_kernel_orders(idx):
    """Latents as v A in float32, residuals as (k - z_s P) E (the decode
    append's order) and as k E - z_s (P E)_{hi+lo} (the prefill MFMA order,
    P E as two bf16 terms), each rounded to bf16: all inside the band."""
    wl, kb, vb, A, P, E = _case(idx)
    f = np.float32
    for g in range(wl.n_kv_heads):
        z_exact = vb[:, g] @ A[g]
        z32 = vb[:, g].astype(f) @ A[g].astype(f)
        zs = ref.round_to_storage(z32.astype(np.float64), "bf16")
        assert parity.rounding_valid(_bf16_bits(zs), z_exact, "bf16").all()
        r_exact = ref.residual_code(kb[:, g], zs, P[g], E[g], wl.r_b)
        x32 = kb[:, g].astype(f) - zs[:, :wl.r_b].astype(f) @ P[g].astype(f)
        r_append = ref.round_to_storage((x32 @ E[g].astype(f)).astype(np.float64), "bf16")
        pe = P[g].astype(f) @ E[g].astype(f)
        hi = ref.round_to_storage(pe.astype(np.float64), "bf16").astype(f)
        lo = ref.round_to_storage((pe - hi).astype(np.float64), "bf16").astype(f)
        zf = zs[:, :wl.r_b].astype(f)
        r_pre = kb[:, g].astype(f) @ E[g].astype(f) - (zf @ hi + zf @ lo)
        r_pre = ref.round_to_storage(r_pre.astype(np.float64), "bf16")
        for r in (r_append, r_pre):
            assert parity.rounding_valid(_bf16_bits(r), r_exact, "bf16").all()


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_band_rejects_residual_from_unrounded_latent(idx):
    """Planted mistake: r = (k - z[:r_b] P) E with the unrounded latent z.
    Every token (all KV heads together) has residual codes outside the band."""
    wl, kb, vb, A, P, E = _case(idx, tokens=200)
    outside = np.zeros(kb.shape[0], dtype=np.int64)
    for g in range(wl.n_kv_heads):
        z = vb[:, g] @ A[g]
        zs = ref.round_to_storage(z, "bf16")
        r_exact = ref.residual_code(kb[:, g], zs, P[g], E[g], wl.r_b)
        wrong = ref.round_to_storage(ref.residual_code(kb[:, g], z, P[g], E[g], wl.r_b), "bf16")
        outside += (~parity.rounding_valid(_bf16_bits(wrong), r_exact, "bf16")).sum(axis=1)
    assert outside.min() >= 1, f"{int((outside == 0).sum())} tokens would pass the R7 mistake"


@pytest.mark.parametrize("idx", [1, 2])
def test_band_rejects_truncated_latent(idx):
    """Planted mistake: the latent stored by truncation toward zero."""
    wl, kb, vb, A, P, E = _case(idx, tokens=100)
    for g in range(wl.n_kv_heads):
        z = vb[:, g] @ A[g]
        ok = parity.rounding_valid(_bf16_bits(_truncate_bf16(z)), z, "bf16")
        assert (~ok).sum(axis=1).min() >= 1


def test_band_admits_both_neighbours_only_near_a_tie():
    """A value 1e-6 (relative to its row) from a bf16 rounding boundary admits
    both neighbours; a value mid-way between boundaries admits only its
    nearest-even rounding."""
    lo, hi = 1.0, 1.0 + 2.0 ** -7          # adjacent bf16 values
    mid = (lo + hi) / 2                     # the tie point
    row = np.array([mid * (1 + 1e-6), lo + 2.0 ** -9])  # near the tie; a quarter step above lo
    got_lo = _bf16_bits(np.array([lo, lo]))
    got_hi = _bf16_bits(np.array([hi, hi]))
    ok_lo = parity.rounding_valid(got_lo, row, "bf16")
    ok_hi = parity.rounding_valid(got_hi, row, "bf16")
    assert ok_lo[0] and ok_hi[0]            # both neighbours of a near-tie
    assert ok_lo[1] and not ok_hi[1]        # only the nearest one otherwise


def test_check_token_codes_accepts_the_oracle_codes():
    """The oracle's own append (rounded to nearest even from float64) passes
    the appended-token check with no override, for bf16 and E4M3 caches."""
    for name in ("llama8b-ctx32k", "llama8b-ctx32k-fp8"):
        wl = workload(name)
        inp = synth.decode_inputs(wl, batch=1, ctx=128)
        want = parity.oracle_sequence(wl, inp, 0, top_k=2)
        cst = inp.get("cache_storage", inp["storage"])
        codes = {k: synth.to_storage(want[k], cst) for k in ("z_new", "r_new", "k_new")}
        dev, override = parity.check_token_codes(wl, inp, 0, want, codes["z_new"], codes["r_new"],
                                                 codes["k_new"], name)
        assert override is None and dev < 0.07
