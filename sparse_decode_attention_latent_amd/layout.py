"""Host-side packing of logical caches into the library's paged pools.

Pool layout (declared in include/basiskv.h): one pool per cached state,
``[n_kv_heads][num_phys_pages][width / CE][page_size][CE]`` where CE is the
number of elements in 16 bytes (8 for bf16, 4 for float32).  Within a page,
the 16-byte chunk c of token t sits at ((c * page_size) + t) * 16 bytes, so
a wavefront whose lanes each take one token reads one contiguous
page_size * 16-byte run per chunk.  Logical page p of sequence b lives in
physical page block_table[b][p].

These helpers build test and benchmark inputs from the synthetic generator
and read pools back; they are numpy code on the host and are not part of
the decode path.
"""

import numpy as np


def chunk_elems(itemsize):
    return 16 // itemsize


def pack_pages(logical, block_table, page_size, num_phys_pages):
    """logical [B, Hkv, T, w] -> pool [Hkv, num_phys_pages, w/CE, S, CE]."""
    logical = np.asarray(logical)
    B, H, T, w = logical.shape
    ce = chunk_elems(logical.dtype.itemsize)
    assert w % ce == 0, "width must be a multiple of 16 bytes"
    n_pages = block_table.shape[1]
    assert T <= n_pages * page_size
    padded = np.zeros((B, H, n_pages * page_size, w), dtype=logical.dtype)
    padded[:, :, :T] = logical
    x = padded.reshape(B, H, n_pages, page_size, w // ce, ce).transpose(1, 0, 2, 4, 3, 5)
    pool = np.zeros((H, num_phys_pages, w // ce, page_size, ce), dtype=logical.dtype)
    flat = block_table.reshape(-1).astype(np.int64)
    ok = flat >= 0
    pool[:, flat[ok]] = x.reshape(H, B * n_pages, w // ce, page_size, ce)[:, ok]
    return pool


def unpack_pages(pool, block_table, page_size, T):
    """pool [Hkv, num_phys, w/CE, S, CE] -> logical [B, Hkv, T, w]."""
    pool = np.asarray(pool)
    H, _, nc, S, ce = pool.shape
    B, n_pages = block_table.shape
    x = pool[:, block_table.reshape(-1).astype(np.int64)]          # [H, B*NP, nc, S, ce]
    x = x.reshape(H, B, n_pages, nc, S, ce).transpose(1, 0, 2, 4, 3, 5)
    return x.reshape(B, H, n_pages * S, nc * ce)[:, :, :T]


def routing_first_width(r_v, r_q, page_size, ce):
    """Elements per token of a routing-first page: r_v + r_q, plus one unused
    chunk where needed to make the page whole 128-byte lines (4-token pages
    with an odd chunk count)."""
    chunks = (r_v + r_q) // ce
    unit = 1 if page_size * 16 >= 128 else 128 // (page_size * 16)
    return -(-chunks // unit) * unit * ce


def pack_routing_first(z, r, r_b, block_table, page_size, num_phys_pages):
    """Routing-first layout: logical z [B, Hkv, T, rV] and r [B, Hkv, T, rq]
    -> one pool [Hkv, num_phys_pages, width/CE, S, CE] whose page chunks are
    z[:r_b], then r, then z[r_b:] (r_b and rq whole chunks), then zeros up to
    routing_first_width."""
    z, r = np.asarray(z), np.asarray(r)
    ce = chunk_elems(z.dtype.itemsize)
    assert r_b % ce == 0 and r.shape[-1] % ce == 0
    width = routing_first_width(z.shape[-1], r.shape[-1], page_size, ce)
    pad = np.zeros(z.shape[:-1] + (width - z.shape[-1] - r.shape[-1],), dtype=z.dtype)
    rows = np.concatenate([z[..., :r_b], r, z[..., r_b:], pad], axis=-1)
    return pack_pages(rows, block_table, page_size, num_phys_pages)


def split_routing_first(rows, r_b, r_q, r_v):
    """Rows [..., width] in routing-first order -> (z [..., rV], r [..., rq])
    (any unused chunk past rV + rq is dropped)."""
    rows = np.asarray(rows)
    z = np.concatenate([rows[..., :r_b], rows[..., r_b + r_q:r_v + r_q]], axis=-1)
    return z, rows[..., r_b:r_b + r_q]
