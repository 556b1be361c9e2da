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


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(f'"{v}"' for v in r) + "\n")


def test_trace_summary_splits_passes_in_dispatch_order(tmp_path):
    # a one-call step (scan, attention), then the stage pass (opened by the
    # separate compression call), then a cold step opened by the flush's sum
    d = tmp_path / "kt"
    seq = [("bkv::route_scan_kernel<unsigned short, 4>(int*, int)", 10),
           ("bkv::attend_split_kernel<unsigned short>(float*)", 4),
           ("bkv::append_kernel<unsigned short>(int)", 2),
           ("bkv::route_scan_kernel<unsigned short, 4>(int*, int)", 8),
           ("at::native::reduce_kernel<512, 1>(float)", 30),
           ("bkv::route_scan_kernel<unsigned short, 4>(int*, int)", 12)]
    t, rows = 0, []
    for name, us in seq:
        rows.append((name, t, t + us * 1000))
        t += us * 1000 + 500
    _write_csv(str(d / "h" / "1" / "run_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    stats = {}
    for name, us in seq:
        stats.setdefault(name, []).append(us * 1000)
    _write_csv(str(d / "h" / "1" / "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"],
               [(n, len(v), sum(v), sum(v) / len(v), min(v), max(v)) for n, v in stats.items()])
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--trace-summary", str(d)],
                       capture_output=True, text=True, cwd=REPO, timeout=60)
    assert r.returncode == 0, r.stderr
    out = r.stdout
    assert "| `bkv::route_scan_kernel<unsigned short, 4>` | 3 | 10.00 | 8.00 | 12.00 |" in out
    assert "| `bkv::route_scan_kernel<unsigned short, 4>` | one-call steps | 1 | 10.00 |" in out
    assert "| `bkv::route_scan_kernel<unsigned short, 4>` | stage pass | 1 | 8.00 |" in out
    assert "| `bkv::route_scan_kernel<unsigned short, 4>` | after the stage pass | 1 | 12.00 |" in out
    assert "| `bkv::append_kernel<unsigned short>` | stage pass | 1 | 2.00 |" in out
    assert "reduce_kernel<512, 1>` | 1 |" in out  # listed overall, not split by pass


def test_mfma_summary_averages_per_dispatch(tmp_path):
    d = tmp_path / "mfma_llama8b-ctx32k"
    rows = [("void bkv::reconstruct_kernel<unsigned short, 1, true>(float)", "MfmaUtil", 1.0),
            ("bkv::reconstruct_kernel<unsigned short, 1, true>(float)", "MfmaUtil", 3.0),
            ("bkv::reconstruct_kernel<unsigned short, 1, true>(float)", "MfmaFlopsBF16", 2e9),
            ("bkv::reconstruct_kernel<unsigned short, 1, true>(float)", "MfmaFlopsBF16", 4e9),
            ("bkv::topk_select_kernel<4, 4>(int)", "MfmaUtil", 0.0),
            ("bkv::topk_select_kernel<4, 4>(int)", "MfmaFlopsBF16", 0.0)]
    _write_csv(str(d / "h" / "1" / "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--mfma-summary", str(d)],
                       capture_output=True, text=True, cwd=REPO, timeout=60)
    assert r.returncode == 0, r.stderr
    assert ("| llama8b-ctx32k | `bkv::reconstruct_kernel<unsigned short, 1, true>` | 2 | 2.00 | 3.000 |"
            in r.stdout)
    assert "topk_select" not in r.stdout  # no matrix instructions: not listed
