"""basiskv_decode_step_static (the decode step with the library's own
scratch in place of a workspace, for callers that cannot allocate) against
basiskv_decode_step on the same problems: bit-identical scores, selection, u
and y, on two calls in a row, the second on a smaller problem (the scratch
keeps the first call's contents)."""

import numpy as np
import pytest

from sparse_decode_attention_latent_amd import api, synth
from sparse_decode_attention_latent_amd.configs import workload
from sparse_decode_attention_latent_amd.runner import DecodeProblem

pytestmark = pytest.mark.gpu

CASES = (  # (workload, batch, ctx, seq_lens, top_k): the second is smaller
    ("llama8b-ctx32k", 8, 16384, [16384, 9000, 100, 16384, 5000, 33, 1, 12000], 128),
    ("llama8b-ctx32k", 3, 4096, [4096, 1000, 77], 16),
)
# rotary positions (the RoPE kernels' split plan), and E4M3 routing-first pages
# of whole lines
CASES_ROPE = (
    ("llama8b-ctx32k-b16r16-page4-rope", 4, 8192, [8192, 5000, 63, 8191], None),
    ("llama8b-ctx32k-b16r16-page4-fp8", 2, 4096, [4096, 999], None),
)

# long scans with the projection inside the scoring launch, one after the
# other with other dims (the epoch and marks sit elsewhere in the scratch),
# then the first dims again
CASES_PROJ = (
    ("llama8b-ctx32k", 4, 32768, [32768, 20000, 4097, 31000], 128),
    ("llama8b-ctx32k", 8, 16384, [16384, 9000, 100, 16384, 5000, 33, 1, 12000], 128),
    ("llama8b-ctx32k", 4, 32768, [32768, 20000, 4097, 31000], 128),
)


def _static_step(prob):
    api.decode_step_static(prob.dims, prob.q, prob.k_new, prob.v_new, prob.start_pos,
                           prob.fac["A"], prob.fac["P"], prob.fac["Q"], prob.fac["E"], prob.M,
                           prob.cache, prob.top_k, prob.scale, prob.page_scores, prob.sel, prob.u,
                           prob.y)


def _clear(prob):
    for t in (prob.page_scores, prob.u):
        t.fill_(float("nan"))
    prob.sel.fill_(-7)
    prob.y.fill_(0)


@pytest.mark.parametrize("cases", [CASES, CASES_ROPE, CASES_PROJ],
                         ids=["separate-pools", "rope-routing-first", "projection-inside"])
def test_static_step_matches_the_workspace_step_twice(cases):
    for name, batch, ctx, seq_lens, top_k in cases:
        print(f"static step {name}: batch={batch} ctx={ctx} top_k={top_k}", flush=True)
        wl = workload(name)
        inp = synth.decode_inputs(wl, batch=batch, ctx=ctx, seq_lens=seq_lens)
        prob = DecodeProblem(wl, inp, top_k=top_k)
        assert api.workspace_bytes(prob.dims, prob.top_k) <= api.static_scratch_bytes()
        prob.decode_step()
        want = prob.outputs()
        _clear(prob)
        _static_step(prob)
        got = prob.outputs()
        for key in ("scores", "sel", "u", "y"):
            np.testing.assert_array_equal(got[key], want[key], err_msg=f"{name} b={batch}: {key}")
