"""Parity of the e4m3 latent-cache path (through the C ABI) with the fp64
oracle, which dequantizes exactly: c = e4m3(code) * scale per 128 latent
values, k^R in bf16 (DeepSeek-V3 详解 §4.2 fine-grained scaling).  The kernel
keeps the e4m3 values exact in the scores, rounds P * scale to bf16 for the
output and normalises each 128-wide latent block by the sum of its own rounded
weights, so the bf16 path's tolerances apply (1e-2 on out, 1e-3 on lse)."""
import pytest
import torch

from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _fp8(lens, s_q=1, layout="paged_shuffled", seed=0):
    return make_inputs(dict(batch=len(lens), s_q=s_q, lens=("explicit", list(lens)), layout=layout, q_std=1.0,
                            cache="fp8_e4m3", num_splits=None, unabsorbed=False, name="small_fp8"), seed=seed)


def _check(inp, splits, what):
    from gpu_helpers import DeviceInputs, compare
    assert inp.cache_dtype == "fp8_e4m3"
    print(f"[gpu] {what}: B={inp.batch} S_q={inp.s_q} lens={inp.seq_lens.tolist()[:8]} splits={splits}", flush=True)
    out, lse = DeviceInputs(inp).run(splits)
    ref_out, ref_lse = O.mla_decode(inp)
    e = compare(out, lse, ref_out, ref_lse, what)
    print(f"[gpu] {what}: max err out {e[0]:.2e} lse {e[1]:.2e}", flush=True)


@pytest.mark.parametrize("splits", [1, 4, 16])
def test_fp8_paged_ragged(splits):
    # head 102 of the 130-row sequence puts most of its weight on one row whose
    # |c| is 2.8: each latent block is normalised by the sum of its own rounded
    # weights, so the bf16 rounding of P * scale cannot move that row's share
    # (dividing by the exact sum gave 0.0106 here)
    inp = _fp8([1, 63, 64, 65, 130, 700, 257], seed=21)
    _check(inp, splits, f"fp8 ragged splits={splits}")


@pytest.mark.parametrize("splits", [1, 8])
def test_fp8_contiguous(splits):
    _check(_fp8([100, 1000, 37], layout="contiguous", seed=22), splits, f"fp8 contiguous splits={splits}")


@pytest.mark.parametrize("splits", [1, 4])
def test_fp8_two_query_tokens(splits):
    _check(_fp8([2, 3, 65, 129, 500], s_q=2, seed=23), splits, f"fp8 mtp splits={splits}")


@pytest.mark.parametrize("s_q,splits", [(3, 4), (6, 1)])
def test_fp8_token_groups(s_q, splits):
    _check(_fp8([s_q, 66, 129, 500], s_q=s_q, seed=27 + s_q), splits, f"fp8 s_q={s_q} splits={splits}")


def test_fp8_sequences_with_no_visible_row():
    _check(_fp8([0, 1, 70], s_q=2, seed=24), 4, "fp8 empty rows")


def test_fp8_nan_in_page_tails_never_reaches_output():
    from gpu_helpers import DeviceInputs, compare
    inp = _fp8([1, 63, 65, 200], seed=25)
    ref_out, ref_lse = O.mla_decode(inp)
    dev = DeviceInputs(inp)
    for b, L in enumerate(inp.seq_lens.tolist()):
        last = int(inp.block_table[b, (L - 1) // 64])
        if L % 64:
            dev.cache.rows[last, L % 64:, :] = 0x7F          # e4m3 NaN code
            dev.cache.scales[last, L % 64:, :] = float("nan")
            dev.cache.rope[last, L % 64:, :] = float("nan")
    print("[gpu] fp8 nan tails", flush=True)
    for splits in (1, 4):
        out, lse = dev.run(splits)
        e = compare(out, lse, ref_out, ref_lse, f"fp8 nan tails splits={splits}")
        print(f"[gpu] fp8 nan tails splits={splits}: max err out {e[0]:.2e} lse {e[1]:.2e}", flush=True)


@pytest.mark.parametrize("factor", [16.0, 48.0])
def test_fp8_large_spread_restart_path(factor):
    # rows whose (bf16) k^R is a large multiple of head 0's q^R: see the bf16 test
    inp = _fp8([300, 700], seed=26)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        for j in (L - 5, L // 2):
            page = int(inp.block_table[b, j // 64])
            inp.cache_rope[page, j % 64] = (inp.q_rope[b, 0, 0].float() * factor).to(torch.bfloat16)
    for splits in (1, 4):
        _check(inp, splits, f"fp8 large spread x{factor:g} splits={splits}")
