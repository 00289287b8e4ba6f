"""Staging of seeded inputs onto the GPU and comparison against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import mla_latent_kv_39_amd as mla
from mla_latent_kv_39_amd.runner import DecodeWorkspace, decode_step

OUT_TOL = 1e-2   # max-abs error on out_latent (bf16 inputs, fp32 accumulation)
LSE_TOL = 1e-3   # max-abs error on lse


class DeviceInputs:
    def __init__(self, inp, device="cuda"):
        self.inp = inp
        self.q_absorbed = inp.q_absorbed.to(device)
        self.q_rope = inp.q_rope.to(device)
        self.seq_lens = inp.seq_lens.to(device)
        self.block_table = None if inp.block_table is None else inp.block_table.to(device)
        if inp.cache_dtype == "bf16":
            self.cache = mla.LatentCache(mla.MLA_CACHE_BF16, inp.cache.to(device))
        else:
            self.cache = mla.LatentCache(mla.MLA_CACHE_FP8_E4M3, inp.cache.to(device),
                                         inp.cache_scales.to(device), inp.cache_rope.to(device))

    def run(self, num_splits: int, ws: DecodeWorkspace = None):
        inp = self.inp
        if ws is None:
            ws = DecodeWorkspace(inp.batch, inp.s_q, num_splits)
        out, lse = decode_step(self.q_absorbed, self.q_rope, self.cache, self.block_table, self.seq_lens,
                               inp.scale, ws)
        torch.cuda.synchronize()
        return out.cpu().double().numpy(), lse.cpu().double().numpy()


def compare(out, lse, ref_out, ref_lse, what="", out_tol=OUT_TOL):
    """Element-wise check against the oracle; -inf lse must match exactly."""
    assert np.all(np.isfinite(out)), f"{what}: non-finite out"
    neg = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), neg), f"{what}: -inf lse pattern differs"
    e_out = np.max(np.abs(out - ref_out)) if out.size else 0.0
    fin = ~neg
    e_lse = np.max(np.abs(lse[fin] - ref_lse[fin])) if fin.any() else 0.0
    assert e_out <= out_tol, f"{what}: max |out - oracle| = {e_out:.3e} > {out_tol}"
    assert e_lse <= LSE_TOL, f"{what}: max |lse - oracle| = {e_lse:.3e} > {LSE_TOL}"
    return e_out, e_lse


def pack_partial_out(po):
    """[splits, 2, s_q, 128, 512] partials in head/column order -> the library's
    partial_out bytes (fp16 values in lane order and their descales, the layout
    of include/mla.h) as a uint8 tensor."""
    import torch
    from partial_format import pack
    return torch.from_numpy(pack(po.double().numpy() if hasattr(po, "double") else po))

