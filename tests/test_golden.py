"""Regression pin: the oracle reproduces the stored tiny decode step
(tests/golden/tiny_step_bf16.json, written by tests/golden/make_golden.py)."""

import json
import math
import os

import numpy as np

from oracle import basiskv_ref as ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_step_bf16.json")


def load_golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_oracle_reproduces_golden_step():
    doc = load_golden()
    d = doc["dims"]
    f = {k: ref.storage_to_f64(np.array(v, dtype=np.uint16), "bf16") for k, v in doc["inputs"].items()}
    out = ref.decode_step(f["q"], f["z"], f["r"], f["kc"], np.array(doc["seq_lens"]), f["A"], f["Bf"],
                          f["P"], f["Q"], f["E"], f["W_O"], rb=d["r_b"], page_size=d["page_size"],
                          top_k=d["top_k"], n_pages_out=-(-d["ctx"] // d["page_size"]), storage="bf16",
                          k_new=f["k_new"], v_new=f["v_new"])
    exp = doc["expected"]
    scores = np.array([[[-math.inf if x is None else x for x in row] for row in bg] for bg in exp["scores"]])
    np.testing.assert_allclose(out["scores"], scores, rtol=1e-13, atol=0)
    np.testing.assert_array_equal(out["sel"], np.array(exp["sel"]))
    np.testing.assert_allclose(out["u"], np.array(exp["u"]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["y"], np.array(exp["y"]), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(out["y_stored"], np.array(exp["y_stored"]))
