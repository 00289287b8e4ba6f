"""The generated decode kernels, run instruction by instruction on the CPU
emulator (tests/gcn_emu.py), against the fp64 oracle.

These cover what the GPU parity tests cover (ragged pages, both cache
layouts, partitions that cut sequences, two query tokens, the restart path,
empty sequences, NaN in page tails, the e4m3 cache) on small inputs, and in
addition what a GPU run cannot show: every global and LDS access stays inside
its buffer (the emulator raises on any other), every register a memory
operation fills is read only after the wait that covers it, and the result
does not depend on the order in which the waves run between barriers.
"""
import numpy as np
import pytest
import torch

from mla_inputs import make_inputs
from oracle import mla_oracle as O

import emu_decode as ED

OUT_TOL, LSE_TOL = 1e-2, 1e-3


def _small(lens, s_q=1, layout="paged_shuffled", seed=0, cache="bf16"):
    return make_inputs(dict(batch=len(lens), s_q=s_q, lens=("explicit", list(lens)), layout=layout, q_std=1.0,
                            cache=cache, num_splits=None, unabsorbed=False, name="small"), seed=seed)


def _check(inp, splits, out_tol=OUT_TOL, seed=3, ref=None):
    out, lse, po, pl = ED.emulate_decode(inp, splits, seed=seed)
    out, lse = ED.merged(inp, splits, out, lse, po, pl, O.merge_partials)
    ref_out, ref_lse = O.mla_decode(inp) if ref is None else ref
    assert np.all(np.isfinite(out))
    neg = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), neg)
    e_out = np.max(np.abs(out - ref_out))
    e_lse = np.max(np.abs(lse[~neg] - ref_lse[~neg])) if (~neg).any() else 0.0
    print(f"[emu] {inp.cache_dtype} B={inp.batch} S_q={inp.s_q} splits={splits}: "
          f"max err out {e_out:.2e} lse {e_lse:.2e}")
    assert e_out <= out_tol
    assert e_lse <= LSE_TOL


@pytest.mark.parametrize("splits", [1, 4])
def test_bf16_paged_ragged(splits):
    _check(_small([1, 63, 64, 65, 130, 257], seed=1), splits)


def test_bf16_contiguous():
    _check(_small([100, 37], layout="contiguous", seed=2), 2)


@pytest.mark.parametrize("splits", [1, 2])
def test_bf16_two_query_tokens(splits):
    _check(_small([2, 65, 129], s_q=2, seed=3), splits)


def test_bf16_restart_path():
    # head 0 sees two rows whose score jumps ~300 log2 units past the first
    # rows' maximum: the lean sub-steps overflow and the segment restarts
    inp = _small([300], seed=6)
    for j in (150, 295):
        page = int(inp.block_table[0, j // 64])
        inp.cache[page, j % 64, 512:] = (inp.q_rope[0, 0, 0].float() * 48.0).to(torch.bfloat16)
    _check(inp, 1)


@pytest.mark.parametrize("s_q", [1, 2])
def test_bf16_empty_sequences_and_nan_tails(s_q):
    inp = _small([0, 1, 33, 70], s_q=s_q, seed=4)
    ref = O.mla_decode(inp)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        if L % 64:
            inp.cache[int(inp.block_table[b, (L - 1) // 64]), L % 64:, :] = float("nan")
    for splits in (1, 4):
        _check(inp, splits, ref=ref)


@pytest.mark.parametrize("cache,lens,splits", [("bf16", [4, 5, 66, 130], 1), ("bf16", [3, 70, 129, 200, 9], 8),
                                               ("fp8_e4m3", [3, 70, 129, 200], 4)])
def test_four_query_tokens(cache, lens, splits):
    # 128 heads x 4 tokens: four workgroups of 32 heads per partition (eight
    # partitions: the XCD-grouped workgroup order); the 3-row sequence leaves
    # token 0 with no row
    _check(_small(lens, s_q=4, seed=5, cache=cache), splits)


@pytest.mark.parametrize("cache,lens,s_q,splits", [("bf16", [3, 70, 129], 3, 4), ("fp8_e4m3", [7, 66, 200], 7, 2),
                                                    ("bf16", [8, 64, 65, 130], 8, 8)])
def test_token_groups(cache, lens, s_q, splits):
    # 3 = 2 + 1, 7 = 4 + 2 + 1, 8 = 4 + 4 tokens: one launch per group, each
    # writing its tokens' rows of the shared outputs and partials
    _check(_small(lens, s_q=s_q, seed=8, cache=cache), splits)


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3"])
def test_most_query_tokens(cache):
    # S_q = 64, the most a call takes: sixteen launches of four-token groups
    # writing their tokens' rows of the shared outputs and partials
    _check(_small([64, 70], s_q=64, seed=23, cache=cache), 2)


def test_bf16_result_independent_of_wave_order():
    inp = _small([65, 130, 200], seed=7)
    a = ED.emulate_decode(inp, 4, seed=1)
    b = ED.emulate_decode(inp, 4, seed=2)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


@pytest.mark.parametrize("lens,s_q,splits", [([100, 70], 1, 1), ([300, 70, 129, 1], 1, 4), ([200, 65], 2, 2)])
def test_fp8_cache(lens, s_q, splits):
    _check(_small(lens, s_q=s_q, seed=1, cache="fp8_e4m3"), splits)


@pytest.mark.parametrize("fast_chunks", [4, 1])
def test_bf16_partition_map_over_many_sequences(fast_chunks):
    # 66 sequences: two chunks of lengths, read from registers by the prologue
    # (4 chunks held) or in passes over memory (1 chunk held, batch too large)
    import gen_decode_gfx950 as G
    lens = [1 + (7 * i) % 5 for i in range(60)] + [70, 3, 130, 5, 64, 2]
    inp = _small(lens, seed=9)
    keep = G.FAST_LENS
    G.FAST_LENS = fast_chunks
    try:
        text = G.kernel(False)
    finally:
        G.FAST_LENS = keep
    out, lse, po, pl = ED.emulate_decode(inp, 4, seed=5, text=text)
    out, lse = ED.merged(inp, 4, out, lse, po, pl, O.merge_partials)
    ref_out, ref_lse = O.mla_decode(inp)
    assert np.max(np.abs(out - ref_out)) <= OUT_TOL
    assert np.max(np.abs(lse - ref_lse)) <= LSE_TOL


def test_fp8_restart_path():
    # as the bf16 case: two rows whose (bf16) k^R is 48 times head 0's q^R
    inp = _small([300], seed=6, cache="fp8_e4m3")
    for j in (150, 295):
        page = int(inp.block_table[0, j // 64])
        inp.cache_rope[page, j % 64] = (inp.q_rope[0, 0, 0].float() * 48.0).to(torch.bfloat16)
    _check(inp, 1)


def test_fp8_empty_sequences_and_nan_tails():
    # token 1 of the 33-row sequence gives one row 93% of its softmax: each
    # latent block is normalised by its own rounded weights, so the rounding of
    # P * scale to bf16 cannot move that row's share (0.0123 when the kernel
    # divided by the exact sum)
    inp = _small([0, 1, 33, 70], s_q=2, seed=4, cache="fp8_e4m3")
    ref = O.mla_decode(inp)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        if L % 64:
            page = int(inp.block_table[b, (L - 1) // 64])
            inp.cache[page, L % 64:, :] = 0x7F            # e4m3 NaN code
            inp.cache_scales[page, L % 64:, :] = float("nan")
            inp.cache_rope[page, L % 64:, :] = float("nan")
    for splits in (1, 4):
        _check(inp, splits, ref=ref)


def _run_tiny(body, lds=0):
    """A one-wave kernel: s[4:5] = a 4 KB buffer, v1 = 16 lane, v4..v7 = 1..4,
    then `body`."""
    import gcn_emu as E
    text = "k:\n" + "\n".join("\t" + ln for ln in [
        "s_load_dwordx2 s[4:5], s[0:1], 0x0", "s_waitcnt lgkmcnt(0)",
        "v_lshlrev_b32 v1, 4, v0", "v_mov_b32 v4, 1", "v_mov_b32 v5, 2", "v_mov_b32 v6, 3",
        "v_mov_b32 v7, 4", "s_nop 4"] + body + ["s_waitcnt vmcnt(0)", "s_endpgm"])
    mem = E.Memory()
    buf = mem.add(np.zeros(64 * 16 * 4, np.uint8))
    E.run_kernel(text, "k", lds, mem, np.array([buf], np.uint64).tobytes(), 1, nwaves=1)
    return mem.buffer(buf).view(np.uint32)


@pytest.mark.parametrize("case", ["store data", "sgpr address", "m0", "dpp", "trans", "dot"])
def test_emulator_flags_missing_wait_states(case):
    """Each wait-state rule the emulator checks faults when the wait is
    missing and passes with it: the kernels above are checked against them."""
    import gcn_emu as E
    bad, good, match = {
        "store data": (["global_store_dwordx4 v1, v[4:7], s[4:5]", "v_mov_b32 v5, 9"],
                       ["global_store_dwordx4 v1, v[4:7], s[4:5]", "s_nop 0", "v_mov_b32 v5, 9"], "store-data"),
        "sgpr address": (["v_mov_b32 v8, s4", "v_readfirstlane_b32 s6, v8", "s_mov_b32 s7, s5", "s_nop 2",
                          "global_store_dword v1, v5, s[6:7]"],
                         ["v_mov_b32 v8, s4", "v_readfirstlane_b32 s6, v8", "s_mov_b32 s7, s5", "s_nop 3",
                          "global_store_dword v1, v5, s[6:7]"], "as an address"),
        "m0": (["s_mov_b32 m0, 0", "global_load_lds_dwordx4 v1, s[4:5]"],
               ["s_mov_b32 m0, 0", "s_nop 0", "global_load_lds_dwordx4 v1, s[4:5]"], "M0"),
        "dpp": (["v_mov_b32 v2, 5", "s_nop 0", "v_add_u32_dpp v3, v2, v2 row_shr:1 row_mask:0xf bank_mask:0xf"],
                ["v_mov_b32 v2, 5", "s_nop 1", "v_add_u32_dpp v3, v2, v2 row_shr:1 row_mask:0xf bank_mask:0xf"],
                "DPP"),
        "trans": (["v_exp_f32 v2, v4", "v_add_f32 v3, v2, v2"],
                  ["v_exp_f32 v2, v4", "s_nop 0", "v_add_f32 v3, v2, v2"], "transcendental"),
        "dot": (["v_dot2_f32_bf16 v2, v4, v5, 0", "v_dot2_f32_bf16 v2, v6, v5, v2", "s_nop 1",
                 "v_add_f32 v3, v2, v2"],
                ["v_dot2_f32_bf16 v2, v4, v5, 0", "v_dot2_f32_bf16 v2, v6, v5, v2", "s_nop 2",
                 "v_add_f32 v3, v2, v2"], "DOT"),
    }[case]
    with pytest.raises(E.Fault, match=match):
        _run_tiny(bad, lds=16384)
    _run_tiny(good, lds=16384)
