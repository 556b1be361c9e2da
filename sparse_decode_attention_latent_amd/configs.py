"""The five synthetic workloads the decode path is tested and measured on.

Shapes follow the models the BasisKV pages evaluate (Llama-3.1-8B:
32 query / 8 KV heads, head dim 128, hidden 4096; Qwen3-32B: 64 / 8, hidden
5120; page sizes of Table 10; latent widths V64 / V96 of Figure 3).  Values
are seeded and synthetic; no model weights or datasets are involved.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    storage: str            # "f32" or "bf16": q, caches, factors, output
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int
    ctx: int                # tokens per sequence at the (last) decode step
    page_size: int
    r_v: int                # Value-latent width
    r_b: int                # routing base width (leading latent dims)
    r_q: int                # Key-residual rank
    top_k: int              # pages kept per KV head
    n_planted: int = 0      # planted pages per sequence
    planted: str = "none"   # "even", "random" or "none"
    latent_norm_sigma: float = 0.0  # >0: per-token latent norms ~ LogNormal(0, sigma)
    noise: float = 0.05
    seed: int = 1000
    recent_tokens: int = 0  # recent window attended besides the routed pages
    cache_storage: str = ""  # "fp8": z, r and Key pages as E4M3 codes ("" = storage)
    page_layout: int = 0     # 1: routing-first pages (latent and residual in one pool)
    rope_theta: float = 0.0  # >0: rotary position embedding with this base (pre-RoPE caches)
    # prefill + decode workload only
    prefill_batch: int = 0
    prefill_tokens: int = 0
    decode_steps: int = 0

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_pages(self):
        return -(-self.ctx // self.page_size)

    @property
    def cache(self):
        """Format of the cached pages (z, r, Keys)."""
        return self.cache_storage or self.storage

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = (
    # 0: tiny fp32 single decode step
    Workload("tiny-fp32", "f32", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, hidden=1024,
             ctx=2048, page_size=16, r_v=64, r_b=64, r_q=32, top_k=16,
             n_planted=4, planted="even", seed=1000),
    # 1: Llama-3.1-8B-shaped layer, 4K context, top-k = 1/8 of the pages
    Workload("llama8b-ctx4k", "bf16", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128,
             hidden=4096, ctx=4096, page_size=32, r_v=96, r_b=96, r_q=48, top_k=16,
             n_planted=8, planted="even", seed=1001),
    # 2: Llama-3.1-8B-shaped layer, 32K context (the headline decode step)
    Workload("llama8b-ctx32k", "bf16", batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
             hidden=4096, ctx=32768, page_size=32, r_v=64, r_b=64, r_q=32, top_k=128,
             n_planted=8, planted="random", latent_norm_sigma=0.5, seed=1002),
    # 3: Qwen3-32B-shaped layer, 32K context, top-k = 1/16 of the pages
    Workload("qwen32b-ctx32k", "bf16", batch=4, n_q_heads=64, n_kv_heads=8, head_dim=128,
             hidden=5120, ctx=32768, page_size=32, r_v=96, r_b=96, r_q=48, top_k=64,
             n_planted=8, planted="random", latent_norm_sigma=0.5, seed=1003),
    # 4: Llama-3.1-8B-shaped prefill (4 x 4096 tokens) then 128 decode steps of
    #    batch 2 ending at 131072 tokens, top-k = 1/32 of the pages
    Workload("llama8b-prefill-decode-128k", "bf16", batch=2, n_q_heads=32, n_kv_heads=8,
             head_dim=128, hidden=4096, ctx=131072, page_size=32, r_v=64, r_b=64, r_q=32,
             top_k=128, seed=1004, prefill_batch=4, prefill_tokens=4096, decode_steps=128),
)

# Beyond the five: the pages' adopted router configuration (appendix Tables 9
# and 10: B16R16 routing, Page4, 2048 routed tokens plus 64 recent tokens,
# V96) on the 8B-shaped layer at c2's batch and context.
EXTRA_WORKLOADS = (
    Workload("llama8b-ctx32k-b16r16-page4", "bf16", batch=8, n_q_heads=32, n_kv_heads=8,
             head_dim=128, hidden=4096, ctx=32768, page_size=4, r_v=96, r_b=16, r_q=16,
             top_k=512, recent_tokens=64, n_planted=8, planted="random",
             latent_norm_sigma=0.5, seed=1005),
    # FP8 E4M3 caches (appendix Table 13: BasisKV B16R16 Page4 V96 under an
    # E4M3 KV cache): the headline 8B-shaped step and the adopted router with
    # latent, residual and Key pages stored as E4M3 codes, bf16 elsewhere.
    Workload("llama8b-ctx32k-fp8", "bf16", batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
             hidden=4096, ctx=32768, page_size=32, r_v=64, r_b=64, r_q=32, top_k=128,
             n_planted=8, planted="random", latent_norm_sigma=0.5, seed=1006,
             cache_storage="fp8"),
    # (routing-first pages: with E4M3 codes and 4-token pages a separate routing
    # chunk is a 64-byte run of a 128-byte line; the routing dims stored together
    # measured faster, 61.9 -> 59.0 us per step)
    Workload("llama8b-ctx32k-b16r16-page4-fp8", "bf16", batch=8, n_q_heads=32, n_kv_heads=8,
             head_dim=128, hidden=4096, ctx=32768, page_size=4, r_v=96, r_b=16, r_q=16,
             top_k=512, recent_tokens=64, n_planted=8, planted="random",
             latent_norm_sigma=0.5, seed=1007, cache_storage="fp8", page_layout=1),
)
# The single-source routers of the pages' router ablation (appendix Table 9,
# beside B16R16): B16 routes from the latent's leading 16 dims alone (no
# residual, r_q = 0); R16 and R32 from a residual of rank 16 or 32 alone
# (r_b = 0).  Same setting as the adopted router (Page4, 512 routed pages +
# 64 recent tokens, V96).
EXTRA_WORKLOADS = EXTRA_WORKLOADS + (
    EXTRA_WORKLOADS[0].with_(name="llama8b-ctx32k-b16-page4", r_b=16, r_q=0, seed=1008),
    EXTRA_WORKLOADS[0].with_(name="llama8b-ctx32k-r16-page4", r_b=0, r_q=16, seed=1009),
    EXTRA_WORKLOADS[0].with_(name="llama8b-ctx32k-r32-page4", r_b=0, r_q=32, seed=1010),
)
# Rotary position embedding on the predicted pre-RoPE Keys (the pages' Figure 6
# measures pre-RoPE Key predictability): the adopted router and the headline
# shape with positions, base 500000 (Llama-3.1's).
EXTRA_WORKLOADS = EXTRA_WORKLOADS + (
    EXTRA_WORKLOADS[0].with_(name="llama8b-ctx32k-b16r16-page4-rope", rope_theta=500000.0,
                             seed=1011),
    WORKLOADS[2].with_(name="llama8b-ctx32k-rope", rope_theta=500000.0, seed=1012),
)
# The other page layout of the same configurations: routing-first (each page's
# routing dims contiguous; include/basiskv.h) where separate pools are the
# default, separate pools for the E4M3 adopted router.
EXTRA_WORKLOADS = EXTRA_WORKLOADS + tuple(
    w.with_(name=w.name + "-routing-first", page_layout=1)
    for w in (WORKLOADS[2], EXTRA_WORKLOADS[0], EXTRA_WORKLOADS[1])) + (
    EXTRA_WORKLOADS[2].with_(name=EXTRA_WORKLOADS[2].name + "-separate", page_layout=0),)

HEADLINE = 2


def workload(index_or_name):
    if isinstance(index_or_name, int):
        return WORKLOADS[index_or_name]
    for w in WORKLOADS + EXTRA_WORKLOADS:
        if w.name == index_or_name:
            return w
    raise KeyError(index_or_name)
