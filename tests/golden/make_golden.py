"""Writes tests/golden/tiny_step_bf16.json: a tiny decode step (with a one-token
append, a partial last page and a short second sequence) and the oracle's
outputs for it.

Inputs are drawn here with numpy's default_rng and stored in bf16; expected
values come from oracle.basiskv_ref only.  Run from the repository root:
    python tests/golden/make_golden.py
"""

import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import basiskv_ref as ref  # noqa: E402

DIMS = dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, hidden=16, r_v=16, r_b=16, r_q=8,
            page_size=16, ctx=40, top_k=2)
SEQ_LENS = [40, 17]


def bf16_bits(x64):
    """RNE float64 -> bf16 bit patterns via the oracle's rounding."""
    r = ref.round_to_storage(x64, "bf16").astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def main():
    d = DIMS
    rng = np.random.default_rng(20261203)
    B, Hq, Hkv, dh, D = d["batch"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["hidden"]
    rv, rb, rq, T = d["r_v"], d["r_b"], d["r_q"], d["ctx"]
    arrays = dict(
        q=rng.standard_normal((B, Hq, dh)),
        z=rng.standard_normal((B, Hkv, T, rv)),
        r=rng.standard_normal((B, Hkv, T, rq)),
        kc=rng.standard_normal((B, Hkv, T, dh)) * 1.5,
        k_new=rng.standard_normal((B, Hkv, dh)),
        v_new=rng.standard_normal((B, Hkv, dh)),
        A=rng.standard_normal((Hkv, dh, rv)) / math.sqrt(dh),
        Bf=rng.standard_normal((Hkv, rv, dh)) / math.sqrt(rv),
        P=rng.standard_normal((Hkv, rb, dh)) / math.sqrt(rb),
        Q=rng.standard_normal((Hkv, rq, dh)) / math.sqrt(rq),
        E=rng.standard_normal((Hkv, dh, rq)) / math.sqrt(dh),
        W_O=rng.standard_normal((Hq * dh, D)) / math.sqrt(Hq * dh),
    )
    bits = {k: bf16_bits(v) for k, v in arrays.items()}
    f = {k: ref.storage_to_f64(v, "bf16") for k, v in bits.items()}
    n_pages_out = -(-T // d["page_size"])
    out = ref.decode_step(f["q"], f["z"], f["r"], f["kc"], np.array(SEQ_LENS), f["A"], f["Bf"],
                          f["P"], f["Q"], f["E"], f["W_O"], rb=rb, page_size=d["page_size"],
                          top_k=d["top_k"], n_pages_out=n_pages_out, storage="bf16",
                          k_new=f["k_new"], v_new=f["v_new"])
    doc = dict(
        description="tiny bf16 decode step with a one-token append; expected values from the "
                    "float64 oracle (oracle/basiskv_ref.py)",
        dims=d, seq_lens=SEQ_LENS, storage="bf16",
        inputs={k: v.tolist() for k, v in bits.items()},
        expected=dict(scores=[[[None if math.isinf(x) else x for x in row] for row in bg]
                              for bg in out["scores"].tolist()],
                      sel=out["sel"].tolist(), u=out["u"].tolist(), y=out["y"].tolist(),
                      y_stored=out["y_stored"].tolist()),
    )
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_step_bf16.json")
    with open(path, "w") as fh:
        json.dump(doc, fh, separators=(",", ":"))
    print("wrote", path)


if __name__ == "__main__":
    main()
