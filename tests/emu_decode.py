"""Run the generated decode kernels on the CPU emulator (tests/gcn_emu.py).

Host-side test infrastructure: builds the kernel argument block the library's
launcher builds, runs every workgroup of the launch, and merges the partials
of the sequences cut across partitions with the oracle's log-sum-exp merge,
so that the result can be compared with the oracle directly.
"""
from __future__ import annotations

import os
import struct
import sys

import numpy as np

import gcn_emu as E
from partial_format import partial_bytes, unpack

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "..", "mla_latent_kv_39_amd", "csrc"))
import gen_decode_gfx950 as G  # noqa: E402

N_HEADS, D_C = 128, 512


def emulate_decode(inp, num_splits, seed=0, text=None, fp8=None, hook=None):
    """The decode kernel's outputs for MlaInputs `inp`: (out, lse, part_out,
    part_lse) as written (partials unpacked to head/column order)."""
    fp8 = inp.cache_dtype == "fp8_e4m3" if fp8 is None else fp8
    if text is None:
        text = G.kernel(fp8)
    kname, lds = G.KNAME, G.LDS_BYTES
    G.configure(False)
    B, S = inp.batch, inp.s_q
    import torch
    mem = E.Memory()
    q_abs = mem.add(inp.q_absorbed.contiguous().view(torch.uint8).numpy())
    q_rope = mem.add(inp.q_rope.contiguous().view(torch.uint8).numpy())
    rows = mem.add(inp.cache.contiguous().view(torch.uint8).numpy())
    table = 0 if inp.block_table is None else mem.add(inp.block_table.numpy().astype(np.int32))
    lens = mem.add(inp.seq_lens.numpy().astype(np.int32))
    pout = mem.add(np.full(partial_bytes(num_splits, S), 0xFF, np.uint8))      # NaN until written
    plse = mem.add(np.full(num_splits * 2 * S * N_HEADS, np.nan, np.float32))
    out = mem.add(np.full(B * S * N_HEADS * D_C, np.nan, np.float32))
    lse = mem.add(np.full(B * S * N_HEADS, np.nan, np.float32))
    fsc = mem.add(inp.cache_scales.numpy()) if fp8 else 0
    fro = mem.add(inp.cache_rope.contiguous().view(torch.uint8).numpy()) if fp8 else 0
    lg = 0
    while (1 << lg) < num_splits:
        lg += 1
    scale_log2 = float(np.float32(inp.scale) * np.float32(1.4426950408889634))
    tok0 = 0
    while tok0 < S:   # token groups of 4, 2 and 1, one launch each (as the library's launcher)
        group = 4 if S - tok0 >= 4 else (2 if S - tok0 >= 2 else 1)
        hpb = 128 // group
        karg = struct.pack("<9Qf7i2Q2i", q_abs, q_rope, rows, table, lens, pout, plse, out, lse,
                           scale_log2, inp.max_blocks, B, num_splits, group, hpb, N_HEADS // hpb, lg, fsc, fro,
                           S, tok0)
        assert len(karg) == G.KARG_BYTES
        E.run_kernel(text, kname, lds, mem, karg, num_splits * (N_HEADS // hpb), seed=seed, hook=hook)
        tok0 += group
    f = lambda base, shape: mem.buffer(base).view(np.float32).reshape(shape).astype(np.float64)
    return (f(out, (B, S, N_HEADS, D_C)), f(lse, (B, S, N_HEADS)),
            unpack(mem.buffer(pout), num_splits, S),
            f(plse, (num_splits, 2, S, N_HEADS)))


def merged(inp, num_splits, out, lse, pout, plse, merge):
    """Final (out, lse): the kernel's own for sequences inside one partition,
    the merge of their partition shares (partition map of tests/partition_map.py)
    for the others."""
    from partition_map import partition_map
    lens = [int(x) for x in inp.seq_lens]
    _, owners = partition_map(lens, num_splits)
    out, lse = out.copy(), lse.copy()
    for b, own in enumerate(owners):
        if len(own) < 2:
            continue
        for s in range(inp.s_q):
            o, l = merge([pout[p, k, s] for p, k, _, _ in own], [plse[p, k, s] for p, k, _, _ in own])
            out[b, s], lse[b, s] = o, l
    return out, lse
