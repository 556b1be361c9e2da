"""Algorithmic HBM bytes of each decode-path kernel (host arithmetic only).

The byte model follows the per-token read widths of the BasisKV appendix
Table 4 ("Full-context routing" and "Selected attention" columns): routing
reads r_b latent dims plus r_q residual dims of every valid context token;
selected attention reads head_dim Key dims plus all r_v latent dims of every
valid token on the selected pages.  Reconstruction reads the fused matrix M
once.  Small terms (queries, projected queries, scores, selections, outputs)
are counted too, so a figure here is what one launch must move at minimum;
block-table reads are counted once per (sequence, page) touched.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class StepShape:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int
    r_v: int
    r_b: int
    r_q: int
    page_size: int
    max_pages: int
    top_k: int
    elem: int  # bytes per stored activation element: 2 (bf16) or 4 (float32)
    recent_tokens: int = 0  # recent window: its pages are attended besides the routed ones
    cache_elem: int = 0  # bytes per cached element (1 for E4M3 pages); 0: same as elem

    @property
    def ce(self):
        return self.cache_elem or self.elem


def _pages(seq_len, page_size):
    return -(-max(int(seq_len), 0) // page_size)


def append_bytes(s: StepShape):
    """compress_prefill with one token per sequence: read k, v and the three
    factors; write one z, r and Key row per (sequence, KV head)."""
    e = s.elem
    fac = s.n_kv_heads * s.head_dim * (s.r_v + s.r_b + s.r_q) * e
    io = s.batch * s.n_kv_heads * (2 * s.head_dim * e + (s.r_v + s.r_q + s.head_dim) * s.ce)
    return fac + io


def project_bytes(s: StepShape):
    e = s.elem
    return (s.batch * s.n_q_heads * s.head_dim * e
            + s.n_kv_heads * (s.r_b + s.r_q) * s.head_dim * e
            + s.batch * s.n_q_heads * (s.r_b + s.r_q) * 4)


def score_bytes(s: StepShape, seq_lens):
    """route_scan: (r_b + r_q) elements of every valid token, per KV head;
    plus projected queries, block-table entries and the page scores."""
    tok = sum(max(0, int(L)) for L in seq_lens)
    pages = sum(_pages(L, s.page_size) for L in seq_lens)
    stream = tok * s.n_kv_heads * (s.r_b + s.r_q) * s.ce
    small = (s.batch * s.n_q_heads * (s.r_b + s.r_q) * 4 + pages * 4
             + s.batch * s.n_kv_heads * s.max_pages * 4)
    return stream + small


def score_stream_bytes(s: StepShape, seq_lens):
    """The per-token latent + residual stream alone (Table 4 routing widths)."""
    tok = sum(max(0, int(L)) for L in seq_lens)
    return tok * s.n_kv_heads * (s.r_b + s.r_q) * s.ce


def select_bytes(s: StepShape, seq_lens):
    pages = sum(_pages(L, s.page_size) for L in seq_lens)
    return pages * s.n_kv_heads * 4 + s.batch * s.n_kv_heads * s.top_k * 4


def attend_bytes(s: StepShape, seq_lens):
    """attend: head_dim Key + r_v latent elements per selected token.  A
    sequence with more than top_k pages counts top_k full pages (exact when
    its last page is full or not selected); one with fewer counts its valid
    tokens; a recent window adds the valid tokens of its pages.  Plus queries,
    selection and the latent output u."""
    e = s.elem
    total = 0
    for L in seq_lens:
        L = max(0, int(L))
        n_pages = _pages(L, s.page_size)
        if s.recent_tokens > 0:  # the window's pages, then top_k (or fewer) full pages before it
            first = max(0, L - s.recent_tokens) // s.page_size
            toks = L - first * s.page_size + min(first, s.top_k) * s.page_size
        elif n_pages <= s.top_k:
            toks = L
        else:
            toks = s.top_k * s.page_size
        total += toks * s.n_kv_heads * (s.head_dim + s.r_v) * s.ce
    total += s.batch * s.n_q_heads * s.head_dim * e          # queries
    total += s.batch * s.n_kv_heads * s.top_k * 4            # selection
    total += s.batch * s.n_q_heads * s.r_v * 4               # u
    return total


def reconstruct_bytes(s: StepShape):
    e = s.elem
    return (s.hidden * s.n_q_heads * s.r_v * e + s.batch * s.n_q_heads * s.r_v * 4
            + s.batch * s.hidden * e)


def step_bytes(s: StepShape, seq_lens, append=True):
    """Per-launch algorithmic bytes of one decode step (keys: append, project,
    score, select, attend, reconstruct, total)."""
    parts = dict(project=project_bytes(s), score=score_bytes(s, seq_lens),
                 select=select_bytes(s, seq_lens), attend=attend_bytes(s, seq_lens),
                 reconstruct=reconstruct_bytes(s))
    if append:
        parts["append"] = append_bytes(s)
    parts["total"] = sum(parts.values())
    return parts


def prefill_bytes(batch, tokens, n_kv_heads, head_dim, r_v, r_b, r_q, elem, cache_elem=0):
    """compress_prefill of ``tokens`` tokens per sequence: read K and V and
    the three factors once; write one latent, residual and Key row per
    (token, KV head) (cache_elem bytes each; 0: elem)."""
    rows = batch * tokens * n_kv_heads
    fac = n_kv_heads * head_dim * (r_v + r_b + r_q) * elem
    return (rows * (2 * head_dim) * elem + fac
            + rows * (r_v + r_q + head_dim) * (cache_elem or elem))
