"""The five decode workloads, as data.

Shapes follow DeepSeek-V3's attention configuration as the pages give it:
128 query heads, a 512-wide compressed latent c^KV and a 64-wide decoupled
RoPE key k^R per cached token (DeepSeek-V3 详解, yudonglee.me, §2.1 MLA;
DeepSeek-V3 architecture notes, deepseek.csdn.net, §2.1.3(D) and §3).
"""
from __future__ import annotations

import math

# (name) -> parameters.  "lens" is one of ("fixed", L), ("uniform", lo, hi) with
# inclusive bounds, or ("loguniform", lo, hi): L = floor(exp(U(ln lo, ln hi)))
# clamped to [lo, hi].  "layout" is "contiguous" ([B, cap, row] with no block
# table), "paged_shuffled" (a randomly permuted page pool) or "paged_sequential".
# "num_splits" is the number of work partitions of the whole batch (None: the
# library's hint for the GPU); the long-context workload's 64 splits per
# sequence are 4 x 64 = 256 partitions.
WORKLOADS = {
    "single_b1_l128": dict(
        batch=1, s_q=1, lens=("fixed", 128), layout="contiguous", q_std=1.0,
        cache="bf16", num_splits=1, unabsorbed=True,
        doc="Single-sequence decode, B=1, L=128, contiguous, q and cache ~N(0,1)"),
    "batched_b32_l1k_4k": dict(
        batch=32, s_q=1, lens=("uniform", 1024, 4096), layout="contiguous", q_std=1.0,
        cache="bf16", num_splits=None, unabsorbed=False,
        doc="Batched decode, B=32, L~U{1024..4096}, contiguous cache"),
    "paged_b64_l256_32k": dict(
        batch=64, s_q=1, lens=("loguniform", 256, 32768), layout="paged_shuffled",
        q_std=math.sqrt(0.5), cache="bf16", num_splits=None, unabsorbed=False,
        doc="Paged decode, B=64, page 64, shuffled table, L log-uniform [256, 32768], q~N(0,0.5)"),
    "mtp_b128_sq2_l4k_8k": dict(
        batch=128, s_q=2, lens=("uniform", 4096, 8192), layout="paged_shuffled", q_std=1.0,
        cache="bf16", num_splits=None, unabsorbed=False,
        doc="Two causal query tokens per sequence, B=128, L~U{4096..8192}, paged"),
    "fp8_b4_l128k": dict(
        batch=4, s_q=1, lens=("fixed", 131072), layout="paged_sequential", q_std=1.0,
        cache="fp8_e4m3", num_splits=256, unabsorbed=False,
        doc="Long-context decode, B=4, L=131072, e4m3 latent with 1x128 fp32 scales, bf16 RoPE part, "
            "64 splits of ~2048 rows per sequence (256 work partitions) + LSE combine"),
}

BLOCK_SIZE = 64          # rows per cache page
N_HEADS = 128            # n_h
D_LATENT = 512           # d_c
D_ROPE = 64              # d_h^R
D_HEAD = 128             # d_h (per-head width of the unabsorbed path)
D_ROW = D_LATENT + D_ROPE
SCALE = 1.0 / math.sqrt(D_HEAD + D_ROPE)   # 1/sqrt(d_h + d_h^R) = 1/sqrt(192)
TAIL_SENTINEL = 1.0e4    # value written into page slots past a sequence's end


def get_workload(name: str) -> dict:
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return dict(WORKLOADS[name], name=name)
