"""Host-side checks of the benchmark: the one-GPU guard and the algorithmic
byte model behind its roofline figures (BasisKV appendix Table 4: routing
reads r_b + r_q elements of every context token, selected attention
head_dim + r_v elements of every selected token)."""
import os
import subprocess
import sys

import pytest

from sparse_decode_attention_latent_amd import traffic

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=REPO, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no bench line


def _c2(**kw):
    base = dict(batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, hidden=4096, r_v=64,
                r_b=64, r_q=32, page_size=32, max_pages=1024, top_k=128, elem=2)
    base.update(kw)
    return traffic.StepShape(**base)


def test_byte_model_at_the_headline_shape():
    s = _c2()
    lens = [32768] * 8
    # the dominant terms, written out: every token's routing dims; every
    # selected token's Key and latent; the fused matrix once
    route = 8 * 8 * 32768 * (64 + 32) * 2
    attend = 8 * 8 * (128 * 32) * (128 + 64) * 2
    recon = 4096 * 32 * 64 * 2
    sb, ab, rb = traffic.score_bytes(s, lens), traffic.attend_bytes(s, lens), \
        traffic.reconstruct_bytes(s)
    # the small terms (queries, block table, scores, u, outputs) stay under 1%
    assert route <= sb <= route * 1.01
    assert attend <= ab <= attend * 1.01
    assert recon <= rb <= recon * 1.01
    parts = traffic.step_bytes(s, lens)
    assert parts["total"] == sum(v for k, v in parts.items() if k != "total")


def test_byte_model_e4m3_pages_and_short_rows():
    lens = [32768] * 8
    s8 = _c2(cache_elem=1)
    # one byte per cached element halves the two page-reading launches
    assert traffic.score_bytes(s8, lens) == pytest.approx(traffic.score_bytes(_c2(), lens) / 2,
                                                          rel=0.01)
    assert traffic.attend_bytes(s8, lens) == pytest.approx(traffic.attend_bytes(_c2(), lens) / 2,
                                                           rel=0.01)
    # a row shorter than the page budget reads only its valid tokens
    short = [100] + [32768] * 7
    full = traffic.attend_bytes(_c2(), lens)
    assert traffic.attend_bytes(_c2(), short) < full
    assert full - traffic.attend_bytes(_c2(), short) >= (4096 - 100) * 8 * 192 * 2 * 0.99
