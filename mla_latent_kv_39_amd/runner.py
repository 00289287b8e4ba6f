"""One decode step on device-resident tensors: mla_decode then mla_combine.

Holds the output and partial buffers for a (batch, s_q, num_splits) shape so
that repeated steps allocate nothing.
"""
from __future__ import annotations

import torch

from .binding import LATENT_DIM, NUM_HEADS, mla_combine, mla_decode, mla_partial_out_bytes


class DecodeWorkspace:
    """Outputs (out_latent, lse) and split partials for one batch shape."""

    def __init__(self, batch: int, s_q: int, num_splits: int, device="cuda"):
        self.batch, self.s_q, self.num_splits = int(batch), int(s_q), int(num_splits)
        f32 = torch.float32
        self.out = torch.empty((batch, s_q, NUM_HEADS, LATENT_DIM), dtype=f32, device=device)
        self.lse = torch.empty((batch, s_q, NUM_HEADS), dtype=f32, device=device)
        if num_splits > 1:
            # fp16 partial blocks and their descales (layout in include/mla.h)
            self.partial_out = torch.empty((mla_partial_out_bytes(num_splits, s_q),), dtype=torch.uint8,
                                           device=device)
            self.partial_lse = torch.empty((num_splits, 2, s_q, NUM_HEADS), dtype=f32, device=device)
        else:
            self.partial_out = self.partial_lse = None


def decode_step(q_absorbed, q_rope, cache, block_table, seq_lens, scale, ws: DecodeWorkspace, stream=None):
    """Enqueue decode + combine; returns (out_latent, lse) views of the workspace."""
    mla_decode(q_absorbed, q_rope, cache, block_table, seq_lens, scale, ws.out, ws.lse, ws.partial_out,
               ws.partial_lse, stream=stream)
    mla_combine(ws.partial_out, ws.partial_lse, seq_lens, ws.out, ws.lse, stream=stream)
    return ws.out, ws.lse
