"""Thin Python binding of libbasiskv.so (include/basiskv.h).

Argument marshalling only: every function here checks nothing beyond what
ctypes needs, passes raw device pointers and the current HIP stream to the C
ABI, and raises BasisKVError on a non-OK status.  All computation runs in the
library's HIP kernels.  There is no fallback: if the library is missing this
module raises on first use.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbasiskv.so")

F32, BF16, BF16_FP8 = 0, 1, 2  # BF16_FP8: bf16 activations, E4M3 cache pages
LAYOUT_SEPARATE, LAYOUT_ROUTING_FIRST = 0, 1  # page layouts (include/basiskv.h)
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_UNSUPPORTED", 4: "ERR_WORKSPACE",
          5: "ERR_LAUNCH"}

EXPORTED = (
    "basiskv_status_string", "basiskv_workspace_bytes", "basiskv_compress_prefill",
    "basiskv_project_queries", "basiskv_score_pages", "basiskv_select_pages",
    "basiskv_route_pages", "basiskv_sparse_attend", "basiskv_reconstruct",
    "basiskv_decode_step", "basiskv_fuse_output_matrix", "basiskv_pack_output_matrix",
    "basiskv_dense_workspace_bytes", "basiskv_dense_attend", "basiskv_static_scratch_bytes",
    "basiskv_decode_step_static", "basiskv_score_pages_rope",
)


class BasisKVError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_lib().basiskv_status_string(status).decode()})")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "hidden", "r_v", "r_b", "r_q",
        "page_size", "max_pages_per_seq", "num_phys_pages", "dtype", "recent_tokens",
        "page_layout")]


class Cache(ctypes.Structure):
    _fields_ = [("z_pages", ctypes.c_void_p), ("r_pages", ctypes.c_void_p),
                ("k_pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("rope_inv_freq", ctypes.c_void_p)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_decode_attention_latent_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        DP, CP = ctypes.POINTER(Dims), ctypes.POINTER(Cache)
        sig = {
            "basiskv_status_string": (ctypes.c_char_p, [I32]),
            "basiskv_workspace_bytes": (SZ, [DP, I32]),
            "basiskv_compress_prefill": (I32, [DP, P, P, P, I32, P, P, P, CP, P]),
            "basiskv_project_queries": (I32, [DP, P, P, P, P, P]),
            "basiskv_score_pages": (I32, [DP, P, CP, P, P]),
            "basiskv_score_pages_rope": (I32, [DP, P, P, P, CP, P, P]),
            "basiskv_select_pages": (I32, [DP, P, P, I32, P, P]),
            "basiskv_route_pages": (I32, [DP, P, P, P, CP, I32, P, P, P, SZ, P]),
            "basiskv_sparse_attend": (I32, [DP, P, CP, P, I32, ctypes.c_float, P, P, SZ, P]),
            "basiskv_reconstruct": (I32, [DP, P, P, P, P]),
            "basiskv_decode_step": (I32, [DP, P, P, P, P, P, P, P, P, P, CP, I32, ctypes.c_float,
                                          P, P, P, P, P, SZ, P]),
            "basiskv_fuse_output_matrix": (I32, [DP, P, P, P, P]),
            "basiskv_pack_output_matrix": (I32, [DP, P, P, P]),
            "basiskv_dense_workspace_bytes": (SZ, [DP]),
            "basiskv_dense_attend": (I32, [DP, P, P, P, P, P, ctypes.c_float, P, P, SZ, P]),
            "basiskv_static_scratch_bytes": (SZ, []),
            "basiskv_decode_step_static": (I32, [DP, P, P, P, P, P, P, P, P, P, CP, I32,
                                                 ctypes.c_float, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    return _lib()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, where):
    if status != 0:
        raise BasisKVError(status, where)


def make_dims(*, batch, n_q_heads, n_kv_heads, head_dim, hidden, r_v, r_b, r_q, page_size,
              max_pages_per_seq, num_phys_pages, dtype, recent_tokens=0,
              page_layout=LAYOUT_SEPARATE):
    return Dims(batch, n_q_heads, n_kv_heads, head_dim, hidden, r_v, r_b, r_q, page_size,
                max_pages_per_seq, num_phys_pages, dtype, recent_tokens, page_layout)


def make_cache(z_pages, r_pages, k_pages, block_table, seq_lens, rope_inv_freq=None):
    p = lambda t: _ptr(t).value if t is not None else None
    return Cache(p(z_pages), p(r_pages), p(k_pages), p(block_table), p(seq_lens), p(rope_inv_freq))


def workspace_bytes(dims, top_k):
    return int(_lib().basiskv_workspace_bytes(ctypes.byref(dims), int(top_k)))


def compress_prefill(dims, k, v, start_pos, n_tokens, A, P, E, cache, stream=None):
    _check(_lib().basiskv_compress_prefill(ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(start_pos),
                                           int(n_tokens), _ptr(A), _ptr(P), _ptr(E),
                                           ctypes.byref(cache), _stream(stream)),
           "basiskv_compress_prefill")


def project_queries(dims, q, P, Q, q_proj, stream=None):
    _check(_lib().basiskv_project_queries(ctypes.byref(dims), _ptr(q), _ptr(P), _ptr(Q),
                                          _ptr(q_proj), _stream(stream)),
           "basiskv_project_queries")


def score_pages(dims, q_proj, cache, page_scores, stream=None):
    _check(_lib().basiskv_score_pages(ctypes.byref(dims), _ptr(q_proj), ctypes.byref(cache),
                                      _ptr(page_scores), _stream(stream)),
           "basiskv_score_pages")


def score_pages_rope(dims, q, P, Q, cache, page_scores, stream=None):
    _check(_lib().basiskv_score_pages_rope(ctypes.byref(dims), _ptr(q), _ptr(P), _ptr(Q),
                                           ctypes.byref(cache), _ptr(page_scores), _stream(stream)),
           "basiskv_score_pages_rope")


def select_pages(dims, page_scores, seq_lens, top_k, sel, stream=None):
    _check(_lib().basiskv_select_pages(ctypes.byref(dims), _ptr(page_scores), _ptr(seq_lens),
                                       int(top_k), _ptr(sel), _stream(stream)),
           "basiskv_select_pages")


def route_pages(dims, q, P, Q, cache, top_k, page_scores, sel, workspace, stream=None):
    _check(_lib().basiskv_route_pages(ctypes.byref(dims), _ptr(q), _ptr(P), _ptr(Q),
                                      ctypes.byref(cache), int(top_k), _ptr(page_scores), _ptr(sel),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)),
           "basiskv_route_pages")


def sparse_attend(dims, q, cache, sel, top_k, scale, u, workspace, stream=None):
    _check(_lib().basiskv_sparse_attend(ctypes.byref(dims), _ptr(q), ctypes.byref(cache), _ptr(sel),
                                        int(top_k), float(scale), _ptr(u), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)),
           "basiskv_sparse_attend")


def reconstruct(dims, u, M, y, stream=None):
    _check(_lib().basiskv_reconstruct(ctypes.byref(dims), _ptr(u), _ptr(M), _ptr(y),
                                      _stream(stream)),
           "basiskv_reconstruct")


def decode_step(dims, q, k_new, v_new, start_pos, A, P, Q, E, M, cache, top_k, scale,
                page_scores, sel, u, y, workspace, stream=None):
    _check(_lib().basiskv_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new),
                                      _ptr(start_pos), _ptr(A), _ptr(P), _ptr(Q), _ptr(E), _ptr(M),
                                      ctypes.byref(cache), int(top_k), float(scale),
                                      _ptr(page_scores), _ptr(sel), _ptr(u), _ptr(y),
                                      _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)),
           "basiskv_decode_step")


def fuse_output_matrix(dims, Bf, W_O, M, stream=None):
    _check(_lib().basiskv_fuse_output_matrix(ctypes.byref(dims), _ptr(Bf), _ptr(W_O), _ptr(M),
                                             _stream(stream)),
           "basiskv_fuse_output_matrix")


def pack_output_matrix(dims, M_plain, M, stream=None):
    """A plain fused matrix [n_q_heads * r_v][hidden] into the tiled layout."""
    _check(_lib().basiskv_pack_output_matrix(ctypes.byref(dims), _ptr(M_plain), _ptr(M),
                                             _stream(stream)),
           "basiskv_pack_output_matrix")


def dense_workspace_bytes(dims):
    return int(_lib().basiskv_dense_workspace_bytes(ctypes.byref(dims)))


def dense_attend(dims, q, k_pages, v_pages, block_table, seq_lens, scale, o, workspace,
                 stream=None):
    """Dense decode attention over every page (the baseline)."""
    _check(_lib().basiskv_dense_attend(ctypes.byref(dims), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                       _ptr(block_table), _ptr(seq_lens), float(scale), _ptr(o),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)),
           "basiskv_dense_attend")


def static_scratch_bytes():
    return int(_lib().basiskv_static_scratch_bytes())


def decode_step_static(dims, q, k_new, v_new, start_pos, A, P, Q, E, M, cache, top_k, scale,
                       page_scores, sel, u, y, stream=None):
    """basiskv_decode_step with the library's own scratch (no workspace)."""
    _check(_lib().basiskv_decode_step_static(ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new),
                                             _ptr(start_pos), _ptr(A), _ptr(P), _ptr(Q), _ptr(E),
                                             _ptr(M), ctypes.byref(cache), int(top_k), float(scale),
                                             _ptr(page_scores), _ptr(sel), _ptr(u), _ptr(y),
                                             _stream(stream)),
           "basiskv_decode_step_static")
