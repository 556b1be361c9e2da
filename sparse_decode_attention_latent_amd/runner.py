"""A decode problem resident on the GPU, driven through the C ABI.

Builds the device state of one layer's decode step from stored host arrays
(queries, logical caches, factors) -- paged pools, block table, the fused
latent-to-output matrix (computed by the library), workspace and outputs --
and runs the step as the sequence of library calls:
    compress_prefill (one new token per sequence, optional)
    -> route_pages (project, score, select) -> sparse_attend -> reconstruct;
the three routing stages are also callable one by one.
PyTorch only allocates device memory and provides the stream.
"""

import math

import numpy as np
import torch

from . import api, layout, synth


def to_device(arr, storage, device="cuda"):
    """Stored numpy array (float32, uint16 bf16 bits or uint8 E4M3 codes) ->
    device tensor (E4M3 codes stay uint8: the library reads raw bytes)."""
    a = np.ascontiguousarray(arr)
    if storage == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def dims_dtype(storage, cache_storage):
    """The library's dims.dtype for activation and cache formats."""
    if cache_storage == "fp8":
        assert storage == "bf16", "E4M3 pages go with bf16 activations"
        return api.BF16_FP8
    assert cache_storage == storage
    return api.BF16 if storage == "bf16" else api.F32


def random_pool(shape, storage, gen, device):
    """Seeded N(0, 1) draws on the device in a storage format (timing-only
    state); E4M3 codes via torch's float8_e4m3fn cast."""
    if storage == "fp8":
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return x.to(torch.float8_e4m3fn).view(torch.uint8)
    tdt = torch.bfloat16 if storage == "bf16" else torch.float32
    return torch.randn(shape, generator=gen, device=device, dtype=tdt)


def to_host_storage(t, storage):
    """Device tensor -> stored numpy array (inverse of to_device)."""
    if storage == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DecodeProblem:
    """Device state for decode steps of one layer.

    inp: dict from synth.decode_inputs (stored arrays).  The pools hold
    ``max_pages`` pages per sequence, placed through a (by default shuffled)
    block table.
    """

    def __init__(self, wl, inp, *, top_k=None, shuffle_seed=12345, device="cuda",
                 max_pages=None, recent_tokens=None, device_random=None, page_layout=None):
        """device_random: None, or (batch, ctx, seed) for timing-only state whose
        pools, queries and new token are seeded N(0, 1) draws made on the device
        (inp then only supplies the factors); the selection is then arbitrary
        but valid, and no host copy of the caches exists."""
        self.wl = wl
        self.storage = inp["storage"]
        st = self.storage
        self.cache_storage = cst = inp.get("cache_storage") or wl.cache
        self.page_layout = wl.page_layout if page_layout is None else int(page_layout)
        rf = self.page_layout == api.LAYOUT_ROUTING_FIRST
        if device_random is None:
            q = inp["q"]
            B, Hq, dh = q.shape
            Hkv = inp["z"].shape[1]
            T = inp["z"].shape[2]
        else:
            B, T, seed = device_random
            Hq, dh, Hkv = wl.n_q_heads, wl.head_dim, wl.n_kv_heads
        S = wl.page_size
        self.top_k = int(top_k or wl.top_k)
        if recent_tokens is None:
            recent_tokens = wl.recent_tokens
        self.max_pages = int(max_pages or -(-T // S))
        self.num_phys = B * self.max_pages
        self.dims = api.make_dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=dh,
                                  hidden=wl.hidden, r_v=wl.r_v, r_b=wl.r_b, r_q=wl.r_q,
                                  page_size=S, max_pages_per_seq=self.max_pages,
                                  num_phys_pages=self.num_phys,
                                  dtype=dims_dtype(st, cst), recent_tokens=recent_tokens,
                                  page_layout=self.page_layout)
        self.recent_tokens = int(recent_tokens)
        self.block_table_host = synth.block_table(B, self.max_pages, shuffle_seed=shuffle_seed)
        dev = device
        self.block_table = torch.from_numpy(self.block_table_host).to(dev)
        self.fac = {k: to_device(inp[k], st, dev) for k in ("A", "Bf", "P", "Q", "E", "W_O")}
        if device_random is None:
            self.seq_lens_host = np.asarray(inp["seq_lens"], dtype=np.int32)
            pack = lambda a: to_device(layout.pack_pages(a, self.block_table_host, S, self.num_phys),
                                       cst, dev)
            if rf:  # latent and residual in one pool; no residual pool
                self.z_pages = to_device(layout.pack_routing_first(
                    inp["z"], inp["r"], wl.r_b, self.block_table_host, S, self.num_phys), cst, dev)
                self.r_pages = None
            else:
                self.z_pages, self.r_pages = pack(inp["z"]), pack(inp["r"])
            self.k_pages = pack(inp["kc"])
            self.q = to_device(q, st, dev)
            # appended token of the step: [B, 1, Hkv, dh], written at seq_len - 1
            self.k_new = to_device(inp["k_new"][:, None], st, dev)
            self.v_new = to_device(inp["v_new"][:, None], st, dev)
        else:
            self.seq_lens_host = np.full(B, T, dtype=np.int32)
            ce = {"fp8": 16, "bf16": 8}.get(cst, 4)
            gen = torch.Generator(device=dev)
            gen.manual_seed(seed)
            rnd = lambda *shape: random_pool(shape, st, gen, dev)
            pool = lambda w: random_pool((Hkv, self.num_phys, w // ce, S, ce), cst, gen, dev)
            if rf:
                self.z_pages = pool(layout.routing_first_width(wl.r_v, wl.r_q, S, ce))
                self.r_pages = None
            else:
                self.z_pages, self.r_pages = pool(wl.r_v), pool(wl.r_q)
            self.k_pages = pool(dh)
            self.q = rnd(B, Hq, dh)
            self.k_new, self.v_new = rnd(B, 1, Hkv, dh), rnd(B, 1, Hkv, dh)
        self.seq_lens = torch.from_numpy(self.seq_lens_host).to(dev)
        self.start_pos = (self.seq_lens - 1).to(torch.int32)
        freqs = synth.rope_frequencies(wl)  # rotary positions: pre-RoPE caches
        self.rope_inv_freq = None if freqs is None else torch.from_numpy(freqs).to(dev)
        self.cache = api.make_cache(self.z_pages, self.r_pages, self.k_pages, self.block_table,
                                    self.seq_lens, self.rope_inv_freq)
        tdt = torch.bfloat16 if st == "bf16" else torch.float32
        self.M = torch.empty((wl.hidden, Hq * wl.r_v), dtype=tdt, device=dev)
        api.fuse_output_matrix(self.dims, self.fac["Bf"], self.fac["W_O"], self.M)
        ws = api.workspace_bytes(self.dims, self.top_k)
        # zero-filled once: the attention call's merge counters live in it
        self.workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        self.q_proj = torch.empty((B, Hq, wl.r_b + wl.r_q), dtype=torch.float32, device=dev)
        self.page_scores = torch.empty((B, Hkv, self.max_pages), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, Hkv, self.top_k), dtype=torch.int32, device=dev)
        self.u = torch.empty((B, Hq, wl.r_v), dtype=torch.float32, device=dev)
        self.y = torch.empty((B, wl.hidden), dtype=tdt, device=dev)
        self.scale = 1.0 / math.sqrt(dh)

    # -- the steps of the path, one library call each -------------------------
    def append(self):
        api.compress_prefill(self.dims, self.k_new, self.v_new, self.start_pos, 1, self.fac["A"],
                             self.fac["P"], self.fac["E"], self.cache)

    def project(self):
        api.project_queries(self.dims, self.q, self.fac["P"], self.fac["Q"], self.q_proj)

    def score(self):
        if self.rope_inv_freq is not None:  # predicted Keys rotated: scored from the raw queries
            api.score_pages_rope(self.dims, self.q, self.fac["P"], self.fac["Q"], self.cache,
                                 self.page_scores)
        else:
            api.score_pages(self.dims, self.q_proj, self.cache, self.page_scores)

    def select(self):
        api.select_pages(self.dims, self.page_scores, self.seq_lens, self.top_k, self.sel)

    def route(self):
        """Projection, scoring and selection in one library call."""
        api.route_pages(self.dims, self.q, self.fac["P"], self.fac["Q"], self.cache, self.top_k,
                        self.page_scores, self.sel, self.workspace)

    def attend(self):
        api.sparse_attend(self.dims, self.q, self.cache, self.sel, self.top_k, self.scale, self.u,
                          self.workspace)

    def reconstruct(self):
        api.reconstruct(self.dims, self.u.view(self.u.shape[0], -1), self.M, self.y)

    def decode_step(self):
        """The whole step (append, route, attend, reconstruct) in one library call."""
        api.decode_step(self.dims, self.q, self.k_new, self.v_new, self.start_pos, self.fac["A"],
                        self.fac["P"], self.fac["Q"], self.fac["E"], self.M, self.cache, self.top_k,
                        self.scale, self.page_scores, self.sel, self.u,
                        self.y, self.workspace)

    def step(self, append=True):
        """One decode step: the library's four calls (the new token's append,
        routing, sparse attention, reconstruction)."""
        if append:
            self.append()
        self.route()
        self.attend()
        self.reconstruct()

    def step_unfused(self, append=True):
        """The same step with routing as its separate calls (three; with RoPE,
        no projection call: scoring takes the raw queries)."""
        if append:
            self.append()
        if self.rope_inv_freq is None:
            self.project()
        self.score()
        self.select()
        self.attend()
        self.reconstruct()

    def outputs(self):
        """Host copies: page_scores, sel, u (float64), y (stored form)."""
        torch.cuda.synchronize()
        return dict(scores=self.page_scores.double().cpu().numpy(),
                    sel=self.sel.cpu().numpy().astype(np.int64),
                    u=self.u.double().cpu().numpy(),
                    y=to_host_storage(self.y, self.storage))

    def token_codes(self, b, pos):
        """Stored latent, residual and Key of token ``pos`` of sequence b, read
        back from the pools: (z [Hkv, rV], r [Hkv, rq], k [Hkv, dh]) in the
        cache's stored form."""
        S = self.wl.page_size
        phys = int(self.block_table_host[b, pos // S])
        slot = pos % S

        def row(pool):
            t = pool[:, phys, :, slot, :].reshape(pool.shape[0], -1).contiguous()
            return to_host_storage(t, self.cache_storage)

        k = row(self.k_pages)
        if self.r_pages is None:  # routing-first: one pool
            z, r = layout.split_routing_first(row(self.z_pages), self.wl.r_b, self.wl.r_q,
                                              self.wl.r_v)
            return np.ascontiguousarray(z), np.ascontiguousarray(r), k
        return row(self.z_pages), row(self.r_pages), k


class DenseProblem:
    """The dense baseline beside a DecodeProblem: the same queries, Key pool,
    block table and sequence lengths, plus a Value pool of full head_dim
    Values, and the output projection W_O in the reconstruction's tiled
    layout (the fused matrix of an identity decoder).  Dense attention reads
    every valid token's Key and Value (the pages' Table 3 comparison).

    v: stored host Values [B, Hkv, T, dh] (for parity checks), or None for
    seeded random Values drawn on the device (for timing).
    """

    def __init__(self, prob, v=None, seed=0):
        wl, st, cst = prob.wl, prob.storage, prob.cache_storage
        d = prob.dims
        self.prob = prob
        self.dims = api.make_dims(batch=d.batch, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                                  head_dim=d.head_dim, hidden=d.hidden, r_v=d.head_dim,
                                  r_b=d.head_dim, r_q=d.r_q, page_size=d.page_size,
                                  max_pages_per_seq=d.max_pages_per_seq,
                                  num_phys_pages=d.num_phys_pages, dtype=d.dtype)
        dev = prob.q.device
        if v is not None:  # stored in the cache format, as the Key pool
            self.v_pages = to_device(layout.pack_pages(v, prob.block_table_host, wl.page_size,
                                                       prob.num_phys), cst, dev)
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(seed)
            self.v_pages = random_pool(tuple(prob.k_pages.shape), cst, g, dev)
        dh, hq, hkv = d.head_dim, d.n_q_heads, d.n_kv_heads
        eye = torch.eye(dh, dtype=prob.M.dtype, device=dev).expand(hkv, dh, dh).contiguous()
        self.M = torch.empty((wl.hidden, hq * dh), dtype=prob.M.dtype, device=dev)
        api.fuse_output_matrix(self.dims, eye, prob.fac["W_O"], self.M)
        self.workspace = torch.zeros(max(api.dense_workspace_bytes(self.dims), 256),
                                     dtype=torch.uint8, device=dev)
        self.o = torch.empty((d.batch, hq, dh), dtype=torch.float32, device=dev)
        self.y = torch.empty_like(prob.y)

    def attend(self):
        p = self.prob
        api.dense_attend(self.dims, p.q, p.k_pages, self.v_pages, p.block_table, p.seq_lens,
                         p.scale, self.o, self.workspace)

    def reconstruct(self):
        api.reconstruct(self.dims, self.o.view(self.o.shape[0], -1), self.M, self.y)

    def step(self):
        """Dense decode attention and the output projection: the dense step."""
        self.attend()
        self.reconstruct()


class PrefillProblem:
    """Compression of a batch of prompts into empty paged pools.

    k, v: stored host arrays [B, T, Hkv, dh]; fac: stored factor arrays (A, P,
    E).  Tokens of sequence b go to positions 0 .. T-1 through a (by default
    shuffled) block table.
    """

    def __init__(self, wl, k, v, fac, *, storage, cache_storage=None, shuffle_seed=54321,
                 device="cuda", page_layout=0):
        self.wl, self.storage = wl, storage
        self.cache_storage = cst = cache_storage or storage
        self.page_layout = int(page_layout)
        B, T, Hkv, dh = k.shape
        S = wl.page_size
        self.T = T
        self.max_pages = -(-T // S)
        self.num_phys = B * self.max_pages
        self.dims = api.make_dims(batch=B, n_q_heads=wl.n_q_heads, n_kv_heads=Hkv, head_dim=dh,
                                  hidden=wl.hidden, r_v=wl.r_v, r_b=wl.r_b, r_q=wl.r_q,
                                  page_size=S, max_pages_per_seq=self.max_pages,
                                  num_phys_pages=self.num_phys,
                                  dtype=dims_dtype(storage, cst), page_layout=self.page_layout)
        self.block_table_host = synth.block_table(B, self.max_pages, shuffle_seed=shuffle_seed)
        self.block_table = torch.from_numpy(self.block_table_host).to(device)
        self.seq_lens = torch.full((B,), T, dtype=torch.int32, device=device)
        self.start_pos = torch.zeros((B,), dtype=torch.int32, device=device)
        self.k = to_device(k, storage, device)
        self.v = to_device(v, storage, device)
        self.fac = {n: to_device(fac[n], storage, device) for n in ("A", "P", "E")}
        tdt = {"fp8": torch.uint8, "bf16": torch.bfloat16}.get(cst, torch.float32)
        ce = {"fp8": 16, "bf16": 8}.get(cst, 4)

        def pool(w):
            return torch.zeros((Hkv, self.num_phys, w // ce, S, ce), dtype=tdt, device=device)

        if self.page_layout == api.LAYOUT_ROUTING_FIRST:
            self.z_pages, self.r_pages = pool(layout.routing_first_width(wl.r_v, wl.r_q, S, ce)), None
        else:
            self.z_pages, self.r_pages = pool(wl.r_v), pool(wl.r_q)
        self.k_pages = pool(dh)
        self.cache = api.make_cache(self.z_pages, self.r_pages, self.k_pages, self.block_table,
                                    self.seq_lens)

    def run(self):
        api.compress_prefill(self.dims, self.k, self.v, self.start_pos, self.T, self.fac["A"],
                             self.fac["P"], self.fac["E"], self.cache)

    def logical(self):
        """Host copies of the pools as logical [B, Hkv, T, w] stored arrays."""
        torch.cuda.synchronize()
        def logical(t):
            return layout.unpack_pages(to_host_storage(t, self.cache_storage),
                                       self.block_table_host, self.wl.page_size, self.T)

        out = {"k": logical(self.k_pages)}
        if self.r_pages is None:  # routing-first: one pool
            out["z"], out["r"] = layout.split_routing_first(logical(self.z_pages), self.wl.r_b,
                                                            self.wl.r_q, self.wl.r_v)
        else:
            out["z"], out["r"] = logical(self.z_pages), logical(self.r_pages)
        return out
