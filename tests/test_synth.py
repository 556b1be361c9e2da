"""The seeded generator: reproducibility, storage rounding, distributions,
planted-page placement and block tables (CPU only)."""

import math

import numpy as np
import torch

from sparse_decode_attention_latent_amd import layout, synth
from sparse_decode_attention_latent_amd.configs import WORKLOADS, workload


def test_same_seed_same_bits_and_batch_prefix():
    wl = workload(1).with_(ctx=256)
    a = synth.decode_inputs(wl, batch=3)
    b = synth.decode_inputs(wl, batch=3)
    c = synth.decode_inputs(wl, batch=2)
    for k in ("q", "z", "r", "kc", "k_new", "v_new", "A", "W_O"):
        np.testing.assert_array_equal(a[k], b[k])
    for k in ("q", "z", "r", "kc", "k_new", "v_new"):
        np.testing.assert_array_equal(a[k][:2], c[k])


def test_generator_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000) * 7
    mine = synth.to_storage(x, "bf16")
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, lib)


def test_distributions():
    wl = workload(2).with_(ctx=4096, batch=1)
    inp = synth.decode_inputs(wl)
    z = synth.from_storage(inp["z"], "bf16")
    r = synth.from_storage(inp["r"], "bf16")
    norms = np.linalg.norm(z[0, 0], axis=1) / math.sqrt(wl.r_v)
    # lognormal(0, 0.5) token scales: log-norm mean ~0, std ~0.5 (chi noise adds a little)
    assert abs(np.log(norms).mean()) < 0.05 and 0.45 < np.log(norms).std() < 0.6
    unplanted = np.ones(wl.ctx, dtype=bool)
    for p in inp["planted"][0]:
        unplanted[p * wl.page_size:(p + 1) * wl.page_size] = False
    rr = r[0, 0][unplanted]
    assert abs(rr.mean()) < 0.02 and abs(rr.std() - 1) < 0.02
    q = synth.from_storage(inp["q"], "bf16")
    assert abs(q.std() - 1) < 0.05


def test_planted_pages_placement():
    w0 = workload(0)
    np.testing.assert_array_equal(synth.planted_pages(w0, 0, 128), [16, 48, 80, 112])
    w2 = workload(2)
    p = synth.planted_pages(w2, 3, 1024)
    assert len(p) == 8 and len(set(p.tolist())) == 8 and p.min() >= 0 and p.max() < 1024
    assert synth.planted_pages(workload(4), 0, 4096).size == 0


def test_block_table_is_a_permutation():
    bt = synth.block_table(4, 9, shuffle_seed=3)
    assert sorted(bt.reshape(-1).tolist()) == list(range(36))
    assert not np.array_equal(bt, synth.block_table(4, 9))


def test_pack_unpack_roundtrip_both_storages():
    bt = synth.block_table(2, 4, shuffle_seed=1)
    for dt, w in ((np.uint16, 24), (np.float32, 12)):
        x = np.random.default_rng(2).integers(0, 1000, size=(2, 3, 61, w)).astype(dt)
        pool = layout.pack_pages(x, bt, 16, 8)
        assert pool.shape == (3, 8, w * x.itemsize // 16, 16, 16 // x.itemsize)
        np.testing.assert_array_equal(layout.unpack_pages(pool, bt, 16, 61), x)


def test_routing_first_pages_hold_routing_dims_first():
    """Routing-first pool: chunk order z[:r_b], r, z[r_b:] within each page; the
    scoring chunks of a token are the first (r_b + r_q) / CE of its page; the
    split recovers both caches.  Pages are whole 128-byte lines: 4-token pages
    with an odd chunk count carry one unused chunk."""
    rng = np.random.default_rng(5)
    for S in (16, 4):
        bt = synth.block_table(2, 40 // S + 1, shuffle_seed=4)
        for dt, rv, rb, rq in ((np.uint8, 96, 16, 16), (np.uint16, 64, 64, 32), (np.float32, 32, 16, 8),
                               (np.uint16, 96, 16, 16)):
            z = rng.integers(0, 200, size=(2, 2, 40, rv)).astype(dt)
            r = rng.integers(0, 200, size=(2, 2, 40, rq)).astype(dt)
            n_phys = 2 * bt.shape[1]
            pool = layout.pack_routing_first(z, r, rb, bt, S, n_phys)
            ce = 16 // np.dtype(dt).itemsize
            chunks = (rv + rq) // ce
            if S == 4 and chunks % 2:
                chunks += 1  # 64-byte chunk rows: an even count fills whole lines
            assert pool.shape == (2, n_phys, chunks, S, ce)
            assert (chunks * S * 16) % 128 == 0
            assert layout.routing_first_width(rv, rq, S, ce) == chunks * ce
            rows = layout.unpack_pages(pool, bt, S, 40)
            zz, rr = layout.split_routing_first(rows, rb, rq, rv)
            np.testing.assert_array_equal(zz, z)
            np.testing.assert_array_equal(rr, r)
            # token 17 of sequence 1, KV head 1: its page and slot, chunk by chunk
            phys, slot = bt[1, 17 // S], 17 % S
            page = pool[1, phys, :, slot, :].reshape(-1)
            np.testing.assert_array_equal(page[:rb], z[1, 1, 17, :rb])
            np.testing.assert_array_equal(page[rb:rb + rq], r[1, 1, 17])
            np.testing.assert_array_equal(page[rb + rq:rv + rq], z[1, 1, 17, rb:])
            assert not page[rv + rq:].any()  # the unused chunk


def test_workload_shapes():
    assert [w.name for w in WORKLOADS][2] == "llama8b-ctx32k"
    for w in WORKLOADS:
        assert w.n_q_heads % w.n_kv_heads == 0 and w.r_b <= w.r_v
        assert w.head_dim == 128
    assert workload(1).top_k == workload(1).max_pages // 8
    assert workload(3).top_k == workload(3).max_pages // 16
    assert workload(4).top_k == workload(4).max_pages // 32
