"""Seeded generators for the decode workloads.

Everything is drawn on the CPU from one ``torch.Generator`` in a fixed order:

  1. sequence lengths
  2. the page permutation (shuffled layouts only)
  3. the cache, drawn in fp32 chunk by chunk (``CACHE_CHUNK_PAGES`` pages per
     draw), then cast to bf16 or quantized to e4m3 with 1x128 block scales
  4. q_absorbed
  5. q_rope
  6. for the unabsorbed cross-check only: q^C, W^UK, W^UV (fp64)

The returned tensors are the exact bits both sides consume.  Nothing here
computes attention.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

from .configs import (BLOCK_SIZE, D_HEAD, D_LATENT, D_ROPE, D_ROW, N_HEADS, SCALE,
                      TAIL_SENTINEL, get_workload)

CACHE_CHUNK_PAGES = 1024
E4M3_MAX = 448.0   # largest finite OCP E4M3 value (the pages give E4M3's range as about 448)


@dataclass
class MlaInputs:
    """One decode batch.  Layout of ``cache``:

    * bf16 cache: ``cache`` is bf16 ``[num_pages, 64, 576]`` (512 latent || 64 rope).
    * fp8 cache: ``cache`` is uint8 e4m3 codes ``[num_pages, 64, 512]``,
      ``cache_scales`` fp32 ``[num_pages, 64, 4]`` (one per 128-wide block),
      ``cache_rope`` bf16 ``[num_pages, 64, 64]``.

    Row j of sequence b lives in page ``block_table[b, j // 64]`` slot ``j % 64``.
    For the contiguous layout ``block_table`` is None and page ``b * max_blocks + u``
    holds rows ``64u .. 64u+63`` of sequence b (``cache`` is then ``[B * max_blocks, 64, .]``,
    i.e. ``[B, max_blocks * 64, .]`` flattened).
    """
    name: str
    batch: int
    s_q: int
    seq_lens: torch.Tensor            # int32 [B]
    block_table: Optional[torch.Tensor]  # int32 [B, max_blocks] or None (contiguous)
    max_blocks: int
    cache_dtype: str                  # "bf16" or "fp8_e4m3"
    cache: torch.Tensor
    cache_scales: Optional[torch.Tensor]
    cache_rope: Optional[torch.Tensor]
    q_absorbed: torch.Tensor          # bf16 [B, S_q, 128, 512]
    q_rope: torch.Tensor              # bf16 [B, S_q, 128, 64]
    scale: float
    num_splits: Optional[int] = None
    extra: dict = field(default_factory=dict)

    @property
    def num_pages(self) -> int:
        return int(self.cache.shape[0])

    def total_rows(self) -> int:
        return int(self.seq_lens.to(torch.int64).sum())


def _draw_lens(spec, batch: int, g: torch.Generator) -> torch.Tensor:
    kind = spec[0]
    if kind == "fixed":
        return torch.full((batch,), int(spec[1]), dtype=torch.int32)
    if kind == "uniform":
        lo, hi = int(spec[1]), int(spec[2])
        return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64).to(torch.int32)
    if kind == "loguniform":
        lo, hi = int(spec[1]), int(spec[2])
        u = torch.rand((batch,), generator=g, dtype=torch.float64)
        lens = torch.floor(torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
        return lens.clamp(lo, hi).to(torch.int32)
    if kind == "explicit":
        return torch.tensor(list(spec[1]), dtype=torch.int32)
    raise ValueError(f"unknown length spec {spec!r}")


def quantize_e4m3_blocks(x: torch.Tensor, block: int = 128):
    """Quantize the last dim of fp32 ``x`` to OCP E4M3 with one fp32 scale per ``block`` values.

    scale = amax / 448 (an all-zero block gets scale 1); codes = RNE(x / scale)
    saturated to +-448.  Returns (uint8 codes, fp32 scales [..., n/block]).
    The fine-grained 1x128 scaling follows DeepSeek-V3 详解 (yudonglee.me), §4.2.
    """
    assert x.dtype == torch.float32 and x.shape[-1] % block == 0
    shp = x.shape
    xb = x.reshape(*shp[:-1], shp[-1] // block, block)
    amax = xb.abs().amax(dim=-1)
    scales = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (xb / scales.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(shp)
    return codes, scales.to(torch.float32)


def make_inputs(workload, seed: int = 0, **overrides) -> MlaInputs:
    """Build the seeded inputs of a workload (a name from WORKLOADS or a dict).

    ``overrides`` replace workload fields (e.g. ``batch=3, lens=("explicit", [5, 70, 129])``)
    so tests can draw small cases of the same recipe.
    """
    cfg = get_workload(workload) if isinstance(workload, str) else dict(workload)
    cfg.update(overrides)
    B, s_q = int(cfg["batch"]), int(cfg["s_q"])
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))

    seq_lens = _draw_lens(cfg["lens"], B, g)
    blocks_per_seq = [(int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE for L in seq_lens.tolist()]
    blocks_per_seq = [max(1, n) for n in blocks_per_seq]
    max_blocks = max(blocks_per_seq)
    layout = cfg["layout"]
    if layout == "contiguous":
        num_pages = B * max_blocks
        block_table = None
        page_of = [[b * max_blocks + u for u in range(blocks_per_seq[b])] for b in range(B)]
    else:
        num_pages = sum(blocks_per_seq)
        if layout == "paged_shuffled":
            perm = torch.randperm(num_pages, generator=g).to(torch.int32)
        elif layout == "paged_sequential":
            perm = torch.arange(num_pages, dtype=torch.int32)
        else:
            raise ValueError(f"unknown layout {layout!r}")
        block_table = torch.zeros((B, max_blocks), dtype=torch.int32)
        page_of = []
        off = 0
        for b in range(B):
            n = blocks_per_seq[b]
            block_table[b, :n] = perm[off:off + n]
            page_of.append(perm[off:off + n].tolist())
            off += n

    # page slots past each sequence's end get a large finite sentinel
    tail = []
    for b in range(B):
        L = int(seq_lens[b])
        for u, page in enumerate(page_of[b]):
            lo = L - u * BLOCK_SIZE
            if lo < BLOCK_SIZE:
                tail.append((page, max(0, lo)))
    if layout == "contiguous":
        for b in range(B):
            for u in range(blocks_per_seq[b], max_blocks):
                tail.append((b * max_blocks + u, 0))

    if cfg["cache"] not in ("bf16", "fp8_e4m3"):
        raise ValueError(f"unknown cache type {cfg['cache']!r} (bf16 or fp8_e4m3)")
    fp8 = cfg["cache"] == "fp8_e4m3"
    if fp8:
        cache = torch.empty((num_pages, BLOCK_SIZE, D_LATENT), dtype=torch.uint8)
        cache_scales = torch.empty((num_pages, BLOCK_SIZE, D_LATENT // 128), dtype=torch.float32)
        cache_rope = torch.empty((num_pages, BLOCK_SIZE, D_ROPE), dtype=torch.bfloat16)
    else:
        cache = torch.empty((num_pages, BLOCK_SIZE, D_ROW), dtype=torch.bfloat16)
        cache_scales = cache_rope = None
    tail_by_page = {}
    for page, lo in tail:
        tail_by_page[page] = min(lo, tail_by_page.get(page, BLOCK_SIZE))
    for p0 in range(0, num_pages, CACHE_CHUNK_PAGES):
        p1 = min(num_pages, p0 + CACHE_CHUNK_PAGES)
        x = torch.randn((p1 - p0, BLOCK_SIZE, D_ROW), generator=g, dtype=torch.float32)
        for page in range(p0, p1):
            lo = tail_by_page.get(page)
            if lo is not None and lo < BLOCK_SIZE:
                x[page - p0, lo:, :] = TAIL_SENTINEL
        if fp8:
            codes, sc = quantize_e4m3_blocks(x[..., :D_LATENT].contiguous())
            cache[p0:p1] = codes
            cache_scales[p0:p1] = sc
            cache_rope[p0:p1] = x[..., D_LATENT:].to(torch.bfloat16)
        else:
            cache[p0:p1] = x.to(torch.bfloat16)
        del x

    q_std = float(cfg.get("q_std", 1.0))
    q_absorbed = (torch.randn((B, s_q, N_HEADS, D_LATENT), generator=g, dtype=torch.float32) * q_std).to(torch.bfloat16)
    q_rope = (torch.randn((B, s_q, N_HEADS, D_ROPE), generator=g, dtype=torch.float32) * q_std).to(torch.bfloat16)

    extra = {}
    if cfg.get("unabsorbed"):
        # q^C per head, and per-head up-projections with variance 1/512
        extra["q_c"] = torch.randn((B, s_q, N_HEADS, D_HEAD), generator=g, dtype=torch.float64)
        w_std = math.sqrt(1.0 / D_LATENT)
        extra["W_UK"] = torch.randn((N_HEADS, D_HEAD, D_LATENT), generator=g, dtype=torch.float64) * w_std
        extra["W_UV"] = torch.randn((N_HEADS, D_HEAD, D_LATENT), generator=g, dtype=torch.float64) * w_std

    return MlaInputs(
        name=str(cfg.get("name", "custom")), batch=B, s_q=s_q, seq_lens=seq_lens,
        block_table=block_table, max_blocks=max_blocks, cache_dtype=("fp8_e4m3" if fp8 else "bf16"),
        cache=cache, cache_scales=cache_scales, cache_rope=cache_rope,
        q_absorbed=q_absorbed, q_rope=q_rope, scale=float(cfg.get("scale", SCALE)),
        num_splits=cfg.get("num_splits"), extra=extra)
