"""The C-ABI library: it loads, exports every symbol the header declares, and
its host-side validation answers with the documented status codes before any
device work (no GPU needed: invalid calls return before any HIP call)."""

import ctypes
import os
import re

import pytest

from sparse_decode_attention_latent_amd import api
from sparse_decode_attention_latent_amd.configs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "basiskv.h")

needs_lib = pytest.mark.skipif(not os.path.exists(api.LIB_PATH), reason="libbasiskv.so not built")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(basiskv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert header_functions() == sorted(api.EXPORTED)


def test_dims_struct_matches_the_header():
    """The ctypes mirror of basiskv_dims has the header's fields, in order."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} basiskv_dims;", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [n for n, _ in api.Dims._fields_]
    assert ctypes.sizeof(api.Dims) == 4 * len(fields)


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(api.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


@needs_lib
def test_status_strings():
    lib = api.lib()
    for code in range(6):
        assert lib.basiskv_status_string(code)
    assert lib.basiskv_status_string(99) == b"unknown status"


def dims_of(wl, **over):
    kw = dict(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
              hidden=wl.hidden, r_v=wl.r_v, r_b=wl.r_b, r_q=wl.r_q, page_size=wl.page_size,
              max_pages_per_seq=wl.max_pages, num_phys_pages=wl.batch * wl.max_pages,
              dtype=(api.BF16_FP8 if wl.cache == "fp8" else
                     api.BF16 if wl.storage == "bf16" else api.F32))
    kw.update(over)
    return api.make_dims(**kw)


@needs_lib
def test_workspace_bytes():
    for wl in WORKLOADS:
        d = dims_of(wl)
        ws = api.workspace_bytes(d, wl.top_k)
        assert ws > 0 and ws % 256 == 0
        # covers the routing projections and the attention partials
        assert ws >= wl.batch * wl.n_q_heads * (wl.r_b + wl.r_q) * 4
    assert api.workspace_bytes(dims_of(WORKLOADS[2], n_q_heads=30), 8) == 0
    assert api.workspace_bytes(dims_of(WORKLOADS[2]), 0) == 0
    # a recent window adds its pages to every attention row: never less room
    wl = WORKLOADS[2]
    assert (api.workspace_bytes(dims_of(wl, recent_tokens=64), wl.top_k)
            >= api.workspace_bytes(dims_of(wl), wl.top_k))


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _cache(**kw):
    base = dict(z_pages=0x1000, r_pages=0x1000, k_pages=0x1000, block_table=0x1000, seq_lens=0x1000)
    base.update(kw)
    return api.Cache(**base)


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(n_q_heads=30), 2),          # Hq % Hkv != 0
    (dict(r_b=128), 2),               # r_b > r_v
    (dict(batch=0), 2),
    (dict(head_dim=64), 3),           # only 128 is built
    (dict(page_size=12), 3),
    (dict(r_q=36), 3),                # not a multiple of 16 bytes
    (dict(dtype=7), 3),
    (dict(max_pages_per_seq=40000), 3),
    (dict(recent_tokens=-1), 2),
    (dict(dtype=2, r_q=40), 3),       # E4M3 rows: widths must fill 16-byte chunks (16 codes)
    (dict(page_layout=2), 3),         # no such page layout
])
def test_dims_validation(over, code):
    lib = api.lib()
    d = dims_of(WORKLOADS[2], **over)
    c = _cache()
    assert lib.basiskv_project_queries(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.basiskv_score_pages(ctypes.byref(d), FAKE, ctypes.byref(c), FAKE, None) == code
    assert lib.basiskv_select_pages(ctypes.byref(d), FAKE, FAKE, 8, FAKE, None) == code
    assert lib.basiskv_reconstruct(ctypes.byref(d), FAKE, FAKE, FAKE, None) == code


@needs_lib
def test_null_and_shape_and_workspace_errors():
    lib = api.lib()
    d = dims_of(WORKLOADS[2])
    c = _cache()
    assert lib.basiskv_project_queries(None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.basiskv_project_queries(ctypes.byref(d), None, FAKE, FAKE, FAKE, None) == 1
    assert lib.basiskv_score_pages(ctypes.byref(d), FAKE, ctypes.byref(_cache(r_pages=None)), FAKE, None) == 1
    assert lib.basiskv_select_pages(ctypes.byref(d), FAKE, FAKE, 0, FAKE, None) == 2
    assert lib.basiskv_route_pages(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(c), 128, FAKE, FAKE,
                                   FAKE, 16, None) == 4
    assert lib.basiskv_route_pages(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(c), 128, FAKE, FAKE,
                                   None, 1 << 20, None) == 4
    assert lib.basiskv_sparse_attend(ctypes.byref(d), FAKE, ctypes.byref(c), FAKE, 128, 0.1, FAKE, FAKE,
                                     64, None) == 4
    assert lib.basiskv_sparse_attend(ctypes.byref(d), FAKE, ctypes.byref(_cache(k_pages=None)), FAKE, 128,
                                     0.1, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.basiskv_compress_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE,
                                        ctypes.byref(c), None) == 2
    assert lib.basiskv_compress_prefill(ctypes.byref(d), FAKE, FAKE, None, 1, FAKE, FAKE, FAKE,
                                        ctypes.byref(c), None) == 1
    assert lib.basiskv_fuse_output_matrix(ctypes.byref(d), FAKE, None, FAKE, None) == 1
    # the whole-step call: null, shape, workspace and batch checks (all return
    # before any launch)
    def step(dd, q=FAKE, top_k=128, ws=FAKE, ws_bytes=1 << 30):
        return lib.basiskv_decode_step(ctypes.byref(dd), q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, ctypes.byref(c), top_k, 0.1, FAKE, FAKE, FAKE,
                                       FAKE, ws, ws_bytes, None)
    assert step(d, q=None) == 1
    assert step(d, top_k=0) == 2
    assert step(d, ws_bytes=64) == 4
    assert step(d, ws=None) == 4
    # no batch limit: a batch of 40 gets past the size checks to the workspace check
    assert step(dims_of(WORKLOADS[2], batch=40), ws_bytes=64) == 4
    big = dims_of(WORKLOADS[2], batch=40)
    assert lib.basiskv_reconstruct(ctypes.byref(big), None, FAKE, FAKE, None) == 1


@needs_lib
def test_pack_output_matrix_validation():
    """basiskv_pack_output_matrix: null pointers, an in-place call, and sizes
    the tiled layout cannot hold are refused before any launch."""
    lib = api.lib()
    d = dims_of(WORKLOADS[2])
    assert lib.basiskv_pack_output_matrix(ctypes.byref(d), None, FAKE, None) == 1
    assert lib.basiskv_pack_output_matrix(ctypes.byref(d), FAKE, None, None) == 1
    assert lib.basiskv_pack_output_matrix(None, FAKE, FAKE, None) == 1
    assert lib.basiskv_pack_output_matrix(ctypes.byref(d), FAKE, FAKE, None) == 2  # in place
    other = ctypes.c_void_p(0x2000)
    assert lib.basiskv_pack_output_matrix(ctypes.byref(dims_of(WORKLOADS[2], hidden=4100)), FAKE,
                                          other, None) == 3   # hidden % 16 != 0
    assert lib.basiskv_pack_output_matrix(ctypes.byref(dims_of(WORKLOADS[2], n_q_heads=3, n_kv_heads=3,
                                                               r_v=8, r_b=8)), FAKE, other, None) == 3  # K = 24


@needs_lib
def test_fp8_cache_dims():
    """BASISKV_BF16_FP8_E4M3 (bf16 activations, E4M3 pages) is a valid dtype
    for the FP8 workloads; the workspace does not depend on the page format
    (it holds float32 partials and bf16 operand tiles)."""
    from sparse_decode_attention_latent_amd.configs import workload
    for name in ("llama8b-ctx32k-fp8", "llama8b-ctx32k-b16r16-page4-fp8"):
        wl = workload(name)
        d = dims_of(wl)
        assert d.dtype == api.BF16_FP8
        assert api.workspace_bytes(d, wl.top_k) == api.workspace_bytes(
            dims_of(wl, dtype=api.BF16), wl.top_k) > 0


@needs_lib
def test_routing_first_needs_no_residual_pool():
    """Routing-first: the residual lives in the latent pool, so a NULL r_pages
    passes validation and a NULL z_pages does not; with separate pools a NULL
    r_pages is an error.  (Only calls that fail validation are made here.)"""
    lib = api.lib()
    d_rf = dims_of(WORKLOADS[2], page_layout=api.LAYOUT_ROUTING_FIRST)
    d_sep = dims_of(WORKLOADS[2])
    no_r = _cache(r_pages=None)
    no_z = _cache(z_pages=None)
    assert lib.basiskv_score_pages(ctypes.byref(d_sep), FAKE, ctypes.byref(no_r), FAKE, None) == 1
    assert lib.basiskv_score_pages(ctypes.byref(d_rf), FAKE, ctypes.byref(no_z), FAKE, None) == 1
    # a workspace too small: the routing-first call gets past the pool checks to the workspace one
    assert lib.basiskv_route_pages(ctypes.byref(d_rf), FAKE, FAKE, FAKE, ctypes.byref(no_r), 8,
                                   FAKE, FAKE, FAKE, 16, None) == 4
    assert lib.basiskv_route_pages(ctypes.byref(d_sep), FAKE, FAKE, FAKE, ctypes.byref(no_r), 8,
                                   FAKE, FAKE, FAKE, 16, None) == 1


@needs_lib
def test_unsupported_variant_is_reported_before_launch():
    lib = api.lib()
    # group size 3 has no scoring / attention variant
    d = dims_of(WORKLOADS[2], n_q_heads=24)
    c = _cache()
    assert lib.basiskv_score_pages(ctypes.byref(d), FAKE, ctypes.byref(c), FAKE, None) == 3
    assert lib.basiskv_route_pages(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(c), 8, FAKE, FAKE,
                                   FAKE, 1 << 30, None) == 3
    assert lib.basiskv_sparse_attend(ctypes.byref(d), FAKE, ctypes.byref(c), FAKE, 8, 0.1, FAKE, FAKE,
                                     1 << 30, None) == 3


@needs_lib
def test_decode_step_static_validation():
    """The no-allocation decode step: the documented scratch size, and every
    host check -- including a problem whose workspace would not fit the
    library's scratch -- answered before any HIP call."""
    lib = api.lib()
    assert api.static_scratch_bytes() == 8 << 20
    c = _cache()

    def step(dd, q=FAKE, top_k=128):
        return lib.basiskv_decode_step_static(ctypes.byref(dd), q, FAKE, FAKE, FAKE, FAKE, FAKE,
                                              FAKE, FAKE, FAKE, ctypes.byref(c), top_k, 0.1, FAKE,
                                              FAKE, FAKE, FAKE, None)
    d = dims_of(WORKLOADS[2])
    assert step(d, q=None) == 1
    assert step(d, top_k=0) == 2
    assert step(dims_of(WORKLOADS[2], n_q_heads=30)) == 2
    big = dims_of(WORKLOADS[1], batch=512)
    assert api.workspace_bytes(big, 16) > api.static_scratch_bytes()
    assert step(big, top_k=16) == 4


@needs_lib
def test_single_source_router_dims():
    """r_b = 0 or r_q = 0 are valid (appendix Table 9's single-source
    routers), both zero is not; a factor the router does not use may be NULL
    (the calls below get past the pointer checks to the workspace check)."""
    lib = api.lib()
    both = dims_of(WORKLOADS[2], r_b=0, r_q=0)
    assert lib.basiskv_project_queries(ctypes.byref(both), FAKE, FAKE, FAKE, FAKE, None) == 2
    b_only = dims_of(WORKLOADS[2], r_b=16, r_q=0)  # the B16 router of Table 9
    r_only = dims_of(WORKLOADS[2], r_b=0)
    c_no_r = _cache(r_pages=None)
    # B-only: Q (and the residual pool) unused
    assert lib.basiskv_route_pages(ctypes.byref(b_only), FAKE, FAKE, None, ctypes.byref(c_no_r), 8,
                                   FAKE, FAKE, FAKE, 16, None) == 4
    assert lib.basiskv_route_pages(ctypes.byref(b_only), FAKE, None, None, ctypes.byref(c_no_r), 8,
                                   FAKE, FAKE, FAKE, 16, None) == 1
    # R-only: P unused, the residual pool and Q needed
    assert lib.basiskv_route_pages(ctypes.byref(r_only), FAKE, None, FAKE, ctypes.byref(_cache()), 8,
                                   FAKE, FAKE, FAKE, 16, None) == 4
    assert lib.basiskv_route_pages(ctypes.byref(r_only), FAKE, None, FAKE, ctypes.byref(c_no_r), 8,
                                   FAKE, FAKE, FAKE, 16, None) == 1
    assert lib.basiskv_compress_prefill(ctypes.byref(r_only), FAKE, FAKE, FAKE, 0, FAKE, None, FAKE,
                                        ctypes.byref(_cache()), None) == 2  # n_tokens checked after pointers
    assert lib.basiskv_compress_prefill(ctypes.byref(b_only), FAKE, FAKE, FAKE, 1, FAKE, None, None,
                                        ctypes.byref(c_no_r), None) == 1  # P needed when r_b > 0
    for d in (b_only, r_only):
        assert api.workspace_bytes(d, 16) > 0


@needs_lib
def test_rope_cache_support_is_reported_before_launch():
    """A cache with a RoPE frequency table: the scores-only call does not take
    positions (it returns UNSUPPORTED rather than unrotated scores); routing
    and the whole step accept bf16 and E4M3 pages and refuse float32 ones."""
    lib = api.lib()
    rope = _cache(rope_inv_freq=0x1000)
    d = dims_of(WORKLOADS[2])
    assert lib.basiskv_score_pages(ctypes.byref(d), FAKE, ctypes.byref(rope), FAKE, None) == 3
    assert lib.basiskv_score_pages(ctypes.byref(d), FAKE, ctypes.byref(_cache()), FAKE, None) != 3
    # the scores-only RoPE call: needs the table, P and Q; float32 pages unsupported
    assert lib.basiskv_score_pages_rope(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(_cache()),
                                        FAKE, None) == 1
    assert lib.basiskv_score_pages_rope(ctypes.byref(d), FAKE, None, FAKE, ctypes.byref(rope),
                                        FAKE, None) == 1
    assert lib.basiskv_score_pages_rope(ctypes.byref(dims_of(WORKLOADS[0])), FAKE, FAKE, FAKE,
                                        ctypes.byref(rope), FAKE, None) == 3
    assert lib.basiskv_score_pages_rope(ctypes.byref(dims_of(WORKLOADS[2], n_q_heads=24)), FAKE, FAKE,
                                        FAKE, ctypes.byref(rope), FAKE, None) == 3
    for dd, code in ((d, 4), (dims_of(WORKLOADS[2], dtype=api.BF16_FP8), 4), (dims_of(WORKLOADS[0]), 3)):
        assert lib.basiskv_route_pages(ctypes.byref(dd), FAKE, FAKE, FAKE, ctypes.byref(rope), 8,
                                       FAKE, FAKE, FAKE, 16, None) == code
        assert lib.basiskv_decode_step(ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, ctypes.byref(rope), 8, 0.1, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, 64, None) == code
