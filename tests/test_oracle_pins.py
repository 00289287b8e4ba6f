"""Pins that tie the fp64 oracle to facts fixed outside itself.

Each check is either a closed form, an independent library routine, an exact
algebraic identity, a brute-force loop on tiny inputs, or a number the pages
print (tests/golden/page_facts.json).  The mutation tests at the bottom plant
plausible mistakes in the oracle and require that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from mla_inputs import make_inputs, quantize_e4m3_blocks
from oracle import mla_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def small_inputs(lens, s_q=1, layout="paged_shuffled", cache="bf16", seed=3, q_std=1.0):
    return make_inputs(dict(batch=len(lens), s_q=s_q, lens=("explicit", list(lens)), layout=layout,
                            q_std=q_std, cache=cache, num_splits=None, unabsorbed=False, name="small"),
                       seed=seed)


# ----------------------------------------------------------------- page facts
def test_page_facts_golden():
    facts = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
    assert O.N_H == facts["n_heads"]["value"]
    assert O.D_C == facts["d_c"]["value"]
    assert O.D_H_R == facts["d_h_rope"]["value"]
    assert O.D_H == facts["d_h"]["value"]
    assert O.FP8_BLOCK == facts["fp8_block"]["value"]
    mla = O.mla_cache_values_per_token()
    mha = O.mha_cache_values_per_token()
    assert mla == facts["mla_values_per_token_layer"]["value"]
    assert mha == facts["mha_values_per_token_layer"]["value"]
    assert mha / mla >= facts["compression_factor_at_least"]["value"]
    assert abs(np.nanmax(O.e4m3_decode(np.arange(256))) - facts["e4m3_max_approx"]["value"]) < 1e-9
    kb = mla * 2 / 1024.0   # bf16 row
    assert abs(kb - facts["kv_bytes_per_token_layer_approx_kb"]["value"]) < 0.1


def test_scale_reading():
    # 1/sqrt(d_h + d_h^R) with d_h = 128 and d_h^R = 64
    assert O.default_scale() == pytest.approx(1.0 / math.sqrt(192.0), rel=0, abs=0)


# ------------------------------------------------------ a: uniform scores
@pytest.mark.parametrize("s_q", [1, 2])
def test_uniform_scores_give_latent_mean(s_q):
    inp = small_inputs([1, 7, 64, 65, 200], s_q=s_q)
    inp.q_absorbed.zero_()
    inp.q_rope.zero_()
    out, lse = O.mla_decode(inp)
    for b in range(inp.batch):
        for s in range(s_q):
            n = int(inp.seq_lens[b]) - s_q + s + 1
            if n <= 0:
                assert np.all(out[b, s] == 0) and np.all(np.isneginf(lse[b, s]))
                continue
            rows = O.sequence_rows(inp, b, n)
            mean = rows[:, :512].mean(axis=0)
            np.testing.assert_allclose(out[b, s], np.broadcast_to(mean, (128, 512)), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, s], math.log(n), rtol=0, atol=1e-12)


# -------------------------------------------------------- b: single row
def test_single_row_returns_that_latent():
    inp = small_inputs([1, 1, 2], s_q=1)
    out, lse = O.mla_decode(inp)
    for b in range(2):
        row = O.sequence_rows(inp, b, 1)[0]
        q = np.concatenate([inp.q_absorbed[b, 0].double().numpy(), inp.q_rope[b, 0].double().numpy()], axis=1)
        np.testing.assert_array_equal(out[b, 0], np.broadcast_to(row[:512], (128, 512)))
        np.testing.assert_allclose(lse[b, 0], inp.scale * (q @ row), rtol=1e-15, atol=1e-12)
    # MTP token 0 at seq_len 2 sees exactly one row
    mtp = small_inputs([2, 2], s_q=2)
    out2, _ = O.mla_decode(mtp)
    for b in range(2):
        row = O.sequence_rows(mtp, b, 1)[0]
        np.testing.assert_array_equal(out2[b, 0], np.broadcast_to(row[:512], (128, 512)))


# ------------------------------------------------------ c: associativity
def test_absorbed_equals_unabsorbed_per_head():
    inp = make_inputs("single_b1_l128", seed=0)
    q_c = inp.extra["q_c"][0, 0].numpy()
    W_UK = inp.extra["W_UK"].numpy()
    W_UV = inp.extra["W_UV"].numpy()
    n = int(inp.seq_lens[0])
    rows = O.sequence_rows(inp, 0, n)
    q_r = inp.q_rope[0, 0].double().numpy()
    q_abs = O.absorb_query(q_c, W_UK)                      # fp64, no bf16 rounding
    out_lat, lse_abs = O.attend_latent(np.concatenate([q_abs, q_r], axis=1), rows, inp.scale)
    o_abs = O.apply_output_absorption(out_lat, W_UV)
    o_ref, lse_ref, z_ref = O.unabsorbed_attention(q_c, q_r, rows[:, :512], rows[:, 512:], W_UK, W_UV, inp.scale)
    assert o_abs.shape == (128, 128)
    np.testing.assert_allclose(o_abs, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse_abs, lse_ref, rtol=1e-13, atol=1e-12)
    z_abs = inp.scale * (np.concatenate([q_abs, q_r], axis=1) @ rows.T)
    np.testing.assert_allclose(z_abs, z_ref, rtol=1e-11, atol=1e-11)
    # the scores are not trivially equal: they spread over several units
    assert z_ref.std() > 0.3


# ---------------------------------------------------- d: cache-size invariant
def test_cache_row_layout_invariant():
    inp = small_inputs([100, 64])
    assert inp.cache.shape[-1] == O.D_ROW == 576
    assert inp.cache.element_size() * O.D_ROW == 1152
    assert O.mha_cache_values_per_token() / O.mla_cache_values_per_token() == pytest.approx(32768 / 576)
    fp8 = small_inputs([100], cache="fp8_e4m3")
    per_row = (fp8.cache.shape[-1] * 1 + fp8.cache_scales.shape[-1] * 4 + fp8.cache_rope.shape[-1] * 2)
    assert per_row == 656


# ------------------------------------------------------ e: torch SDPA (fp64)
@pytest.mark.parametrize("s_q", [1, 2])
def test_oracle_matches_torch_sdpa(s_q):
    inp = small_inputs([3, 64, 130, 257], s_q=s_q, q_std=1.5)
    out, lse = O.mla_decode(inp)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        rows = torch.from_numpy(O.sequence_rows(inp, b, L))            # [L, 576]
        q = torch.cat([inp.q_absorbed[b].double(), inp.q_rope[b].double()], dim=-1)  # [S, H, 576]
        qh = q.permute(1, 0, 2).unsqueeze(0)                          # [1, H, S, 576]
        k = rows.unsqueeze(0).unsqueeze(0).expand(1, 128, L, 576)
        v = rows[:, :512].unsqueeze(0).unsqueeze(0).expand(1, 128, L, 512)
        pos = torch.arange(L)
        mask = torch.stack([pos < (L - s_q + s + 1) for s in range(s_q)])  # [S, L]
        ref = torch.nn.functional.scaled_dot_product_attention(qh, k, v, attn_mask=mask, scale=inp.scale)
        scores = inp.scale * torch.matmul(qh, k.transpose(-1, -2)).masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(scores, dim=-1)                     # [1, H, S]
        np.testing.assert_allclose(out[b], ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], ref_lse[0].permute(1, 0).numpy(), rtol=1e-13, atol=1e-12)


# -------------------------------------------------- f: split / merge identity
def test_split_merge_identity():
    rng = np.random.default_rng(7)
    inp = small_inputs([500])
    rows = O.sequence_rows(inp, 0, 500)
    q = np.concatenate([inp.q_absorbed[0, 0].double().numpy(), inp.q_rope[0, 0].double().numpy()], axis=1)
    full_out, full_lse = O.attend_latent(q, rows, inp.scale)
    for trial in range(5):
        k = int(rng.integers(1, 9))
        cuts = np.sort(rng.integers(0, 501, size=k - 1))
        bounds = [0, *cuts.tolist(), 500]                  # may contain empty ranges
        parts = [O.partial_over_range(q, rows, bounds[i], bounds[i + 1], inp.scale) for i in range(k)]
        outs = np.stack([p[0] for p in parts])
        lses = np.stack([p[1] for p in parts])
        m_out, m_lse = O.merge_partials(outs, lses)
        np.testing.assert_allclose(m_out, full_out, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(m_lse, full_lse, rtol=1e-14, atol=1e-13)
    # all splits empty -> out 0, lse -inf
    e_out, e_lse = O.merge_partials(np.zeros((3, 128, 512)), np.full((3, 128), -np.inf))
    assert np.all(e_out == 0) and np.all(np.isneginf(e_lse))


# --------------------------------------------------- g: brute force, tiny
def _brute(q_abs, q_r, rows, scale):
    """Pure-Python loops over heads, rows and dims."""
    H, n = len(q_abs), len(rows)
    outs, lses = [], []
    for h in range(H):
        z = []
        for j in range(n):
            acc = 0.0
            for k in range(512):
                acc += q_abs[h][k] * rows[j][k]
            for k in range(64):
                acc += q_r[h][k] * rows[j][512 + k]
            z.append(scale * acc)
        m = max(z)
        e = [math.exp(v - m) for v in z]
        s = sum(e)
        lses.append(m + math.log(s))
        outs.append([sum(e[j] / s * rows[j][k] for j in range(n)) for k in range(512)])
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("s_q", [1, 2])
def test_brute_force_tiny(s_q):
    inp = small_inputs([3, 8, 5], s_q=s_q, seed=11)
    heads = [0, 5, 77, 127]
    for b in range(inp.batch):
        for s in range(s_q):
            out, lse = O.decode_one(inp, b, s, heads=heads)
            n = int(inp.seq_lens[b]) - s_q + s + 1
            # gather rows through the table by hand, slot by slot
            rows = []
            for j in range(n):
                page = int(inp.block_table[b, j // 64])
                rows.append(inp.cache[page, j % 64].double().tolist())
            qa = inp.q_absorbed[b, s].double()[heads].tolist()
            qr = inp.q_rope[b, s].double()[heads].tolist()
            b_out, b_lse = _brute(qa, qr, rows, inp.scale)
            np.testing.assert_allclose(out, b_out, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse, b_lse, rtol=1e-13, atol=1e-13)


# ------------------------------ h: paged == contiguous, row permutation
def test_paged_equals_contiguous_and_row_permutation():
    paged = small_inputs([70, 130, 64], layout="paged_shuffled", seed=5)
    out_p, lse_p = O.mla_decode(paged)
    # rebuild the same logical rows as a contiguous [B, max_blocks*64, 576] cache
    cont = small_inputs([70, 130, 64], layout="contiguous", seed=5)
    B, mb = paged.batch, paged.max_blocks
    new = torch.empty((B * mb, 64, 576), dtype=torch.bfloat16)
    for b in range(B):
        for u in range(mb):
            new[b * mb + u] = paged.cache[int(paged.block_table[b, u])]
    cont.cache = new
    cont.q_absorbed = paged.q_absorbed.clone()
    cont.q_rope = paged.q_rope.clone()
    out_c, lse_c = O.mla_decode(cont)
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)
    # permuting rows inside a sequence (S_q = 1) leaves the result unchanged
    b = 1
    L = int(paged.seq_lens[b])
    rows = O.sequence_rows(paged, b, L)
    perm = np.random.default_rng(0).permutation(L)
    q = np.concatenate([paged.q_absorbed[b, 0].double().numpy(), paged.q_rope[b, 0].double().numpy()], axis=1)
    o1, l1 = O.attend_latent(q, rows, paged.scale)
    o2, l2 = O.attend_latent(q, rows[perm], paged.scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-13)


# ---------------------------------------------------- i: MTP consistency
def test_mtp_tokens_match_single_token_decode():
    mtp = small_inputs([5, 100, 129], s_q=2, seed=9)
    out2, lse2 = O.mla_decode(mtp)
    for s in range(2):
        single = small_inputs([5, 100, 129], s_q=1, seed=9)
        single.cache = mtp.cache
        single.block_table = mtp.block_table
        single.seq_lens = mtp.seq_lens - (1 - s)
        single.q_absorbed = mtp.q_absorbed[:, s:s + 1].clone()
        single.q_rope = mtp.q_rope[:, s:s + 1].clone()
        out1, lse1 = O.mla_decode(single)
        np.testing.assert_array_equal(out2[:, s], out1[:, 0])
        np.testing.assert_array_equal(lse2[:, s], lse1[:, 0])


# --------------------------------------------------------------- j: fp8
def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all((mine == ref) | both_nan)
    assert np.sum(np.isnan(mine)) == 2          # 0x7f and 0xff
    finite = mine[np.isfinite(mine)]
    assert finite.max() == 448.0 and finite.min() == -448.0
    # every finite e4m3 value is exact in bf16
    as_bf16 = torch.from_numpy(finite).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(as_bf16, finite)


def test_quantizer_error_saturation_zero_block():
    g = torch.Generator().manual_seed(1)
    x = torch.randn((64, 512), generator=g)
    x[3, :128] = 0.0          # a zero block
    x[5, 200] = 1e6           # an outlier affects only its own block
    codes, scales = quantize_e4m3_blocks(x)
    deq = O.dequantize_latent(codes.numpy(), scales.numpy())
    xs = x.double().numpy()
    assert scales[3, 0] == 1.0 and np.all(deq[3, :128] == 0)
    # relative error at most half an ulp of a 3-bit mantissa (2^-4) in the normal range
    s_rep = np.repeat(scales.double().numpy(), 128, axis=1)
    normal = np.abs(xs / s_rep) >= 2.0 ** -6
    rel = np.abs(deq - xs)[normal] / np.abs(xs)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-12
    # subnormal range: absolute error at most half the smallest step (2^-10) times the scale
    sub = ~normal
    assert np.all(np.abs(deq - xs)[sub] <= 2.0 ** -10 * s_rep[sub] + 1e-12)
    # the block max maps to exactly +-448
    assert np.isclose(np.abs(O.e4m3_decode(codes[5, 128:256].numpy())).max(), 448.0)
    # the outlier did not disturb the other blocks of its row
    np.testing.assert_array_equal(scales[5, [0, 2, 3]], (x[5].reshape(4, 128).abs().amax(1) / 448)[[0, 2, 3]])


def test_fp8_oracle_uses_dequantized_rows():
    inp = small_inputs([70], cache="fp8_e4m3", seed=2)
    rows = O.sequence_rows(inp, 0, 70)
    codes = inp.cache[0].numpy()
    sc = inp.cache_scales[0].numpy()
    for j in (0, 17, 63):
        for blk in range(4):
            for k in (0, 31, 127):
                c = blk * 128 + k
                assert rows[j, c] == O.e4m3_decode(codes[j, c]) * sc[j, blk]
    pages = [int(inp.block_table[0, u]) for u in range(2)]
    rope = np.concatenate([inp.cache_rope[p].double().numpy() for p in pages])[:70]
    np.testing.assert_array_equal(rows[:, 512:], rope)


# ------------------------------------------------ mutation sensitivity
def _mutant_checks():
    """Run a subset of pins; returns the names of those that failed."""
    failed = []
    for name, fn in [("sdpa", lambda: test_oracle_matches_torch_sdpa(2)),
                     ("uniform", lambda: test_uniform_scores_give_latent_mean(2)),
                     ("assoc", test_absorbed_equals_unabsorbed_per_head),
                     ("split", test_split_merge_identity),
                     ("mtp", test_mtp_tokens_match_single_token_decode),
                     ("e4m3", test_e4m3_decoder_matches_torch_all_codes),
                     ("fp8rows", test_fp8_oracle_uses_dequantized_rows),
                     ("rope", test_rope_closed_forms),
                     ("query", test_query_side_absorbs_and_rotates),
                     ("output", test_output_side_recovers_unabsorbed_values),
                     ("kvproj", test_kv_project_special_cases),
                     ("quant", test_e4m3_quantize_against_torch_and_edge_cases),
                     ("append", test_cache_append_writes_each_new_row_where_the_decode_reads_it)]:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def _bad_attend_scale(q_cat, rows, scale):
    return _orig_attend(q_cat, rows, 1.0 / math.sqrt(576.0))


def _bad_attend_no_rope(q_cat, rows, scale):
    q2 = q_cat.copy()
    q2[:, 512:] = 0
    return _orig_attend(q2, rows, scale)


def _bad_attend_v_rope(q_cat, rows, scale):
    out, lse = _orig_attend(q_cat, rows, scale)
    shifted = np.concatenate([rows[:, 64:576], rows[:, :64]], axis=1)
    out2, _ = _orig_attend(q_cat, shifted, scale)
    return out2 if rows.shape[0] > 0 else out, lse


def _bad_visible(seq_len, s_q, s):
    return max(0, int(seq_len) - int(s_q) + int(s))


def _bad_merge(outs, lses):
    outs = np.asarray(outs)
    return outs.mean(axis=0), np.asarray(lses).max(axis=0)


def _bad_e4m3(codes):
    return _orig_e4m3(codes) * 2.0


def _bad_rope_halves(x, pos, base=10000.0):
    # pairs (i, i + d/2) instead of (2i, 2i + 1)
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    perm = np.stack([np.arange(d // 2), np.arange(d // 2) + d // 2], axis=1).reshape(-1)
    inv = np.argsort(perm)
    return _orig_rope(x[..., perm], pos, base)[..., inv]


def _bad_rope_sign(x, pos, base=10000.0):
    return _orig_rope(x, -np.asarray(pos), base)


def _bad_positions(seq_lens, s_q):
    return _orig_positions(seq_lens, s_q) + 1


def _bad_nearest_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    vals, codes = O._e4m3_table()
    a = np.minimum(np.abs(v), 448.0)
    idx = np.searchsorted(vals, a, side="right") - 1
    out = codes[np.clip(idx, 0, len(codes) - 1)].astype(np.uint8)
    return (out | ((np.signbit(v)).astype(np.uint8) << 7)).astype(np.uint8)


def _bad_kv_swap(h, W_DKV, W_KR):
    kv = _orig_kv(h, W_DKV, W_KR)
    return np.concatenate([kv[..., 64:576], kv[..., :64]], axis=-1)


def _bad_output_transpose(out_latent, W_UV):
    return np.einsum("hdc,bshc->bshd", np.asarray(W_UV)[::-1], np.asarray(out_latent, dtype=np.float64))


_orig_attend = O.attend_latent
_orig_e4m3 = O.e4m3_decode
_orig_rope = O.rope
_orig_positions = O.token_positions
_orig_kv = O.kv_project


@pytest.mark.parametrize("target,mutant", [
    ("attend_latent", _bad_attend_scale),
    ("attend_latent", _bad_attend_no_rope),
    ("attend_latent", _bad_attend_v_rope),
    ("visible_rows", _bad_visible),
    ("merge_partials", _bad_merge),
    ("e4m3_decode", _bad_e4m3),
    ("rope", _bad_rope_halves),
    ("rope", _bad_rope_sign),
    ("token_positions", _bad_positions),
    ("e4m3_nearest", _bad_nearest_truncate),
    ("kv_project", _bad_kv_swap),
    ("output_side", _bad_output_transpose),
])
def test_pins_catch_planted_oracle_mistakes(monkeypatch, target, mutant):
    monkeypatch.setattr(O, target, mutant)
    failed = _mutant_checks()
    assert failed, f"no pin caught the planted mistake in {target} ({mutant.__name__})"


def test_input_generator_rejects_unknown_cache_type():
    import pytest
    from mla_inputs import make_inputs
    with pytest.raises(ValueError):
        make_inputs(dict(batch=1, s_q=1, lens=("explicit", [8]), layout="paged_shuffled", q_std=1.0,
                         cache="fp8", num_splits=None, unabsorbed=False, name="bad"), seed=0)


# ====================================== the next rows: absorption, RoPE, cache append
def test_rope_closed_forms():
    """RoPE of unit vectors gives cos/sin of pos * 10000^(-2i/64) in the pair
    (2i, 2i+1); position 0 is the identity; each pair keeps its length;
    rotations compose; scores depend only on the distance of the positions."""
    d = 64
    for i, p in ((0, 1), (1, 1), (5, 7), (31, 1000)):
        e = np.zeros(d)
        e[2 * i] = 1.0
        r = O.rope(e, p)
        th = 10000.0 ** (-2.0 * i / d)
        want = np.zeros(d)
        want[2 * i], want[2 * i + 1] = math.cos(p * th), math.sin(p * th)
        np.testing.assert_allclose(r, want, atol=1e-12)
        e2 = np.zeros(d)
        e2[2 * i + 1] = 1.0
        r2 = O.rope(e2, p)
        assert abs(r2[2 * i] + math.sin(p * th)) < 1e-12 and abs(r2[2 * i + 1] - math.cos(p * th)) < 1e-12
    rng = np.random.default_rng(0)
    x, k = rng.standard_normal(d), rng.standard_normal(d)
    np.testing.assert_array_equal(O.rope(x, 0), x)
    r = O.rope(x, 12345)
    np.testing.assert_allclose(r[0::2] ** 2 + r[1::2] ** 2, x[0::2] ** 2 + x[1::2] ** 2, rtol=1e-12)
    np.testing.assert_allclose(O.rope(O.rope(x, 300), 77), O.rope(x, 377), atol=1e-11)
    for t, j in ((10, 3), (5000, 4990), (7, 0)):
        np.testing.assert_allclose(O.rope(x, t) @ O.rope(k, j), O.rope(x, t - j) @ k, rtol=1e-10, atol=1e-10)
    # positions broadcast over leading dims
    xs = rng.standard_normal((3, 2, d))
    pos = np.array([[1, 2], [3, 4], [5, 6]])
    out = O.rope(xs, pos)
    np.testing.assert_allclose(out[2, 1], O.rope(xs[2, 1], 6), atol=1e-13)


def test_query_side_absorbs_and_rotates():
    """q_absorbed . c^KV equals the unabsorbed q^C . (W^UK c^KV) for every head
    ([P2] §2.1.3(B)); q_rope is q^R rotated to position seq_len - S_q + s, so
    its score against a key rotated to row j depends only on the distance."""
    rng = np.random.default_rng(1)
    B, S, H, dh, dc = 2, 2, 4, 128, 512
    q_c = rng.standard_normal((B, S, H, dh))
    q_r = rng.standard_normal((B, S, H, 64))
    W_UK = rng.standard_normal((H, dh, dc)) / math.sqrt(dc)
    lens = np.array([9, 300])
    q_abs, q_rot = O.query_side(q_c, q_r, W_UK, lens)
    c = rng.standard_normal(dc)
    for b in range(B):
        for s in range(S):
            for h in range(H):
                np.testing.assert_allclose(q_abs[b, s, h] @ c, q_c[b, s, h] @ (W_UK[h] @ c), rtol=1e-11, atol=1e-11)
    np.testing.assert_array_equal(O.token_positions(lens, S), [[7, 8], [298, 299]])
    k = rng.standard_normal(64)
    for b in range(B):
        for s in range(S):
            p = int(lens[b]) - S + s
            for j in (0, p // 2, p):
                np.testing.assert_allclose(q_rot[b, s, 1] @ O.rope(k, j), O.rope(q_r[b, s, 1], p - j) @ k,
                                           rtol=1e-10, atol=1e-10)


def test_output_side_recovers_unabsorbed_values():
    """o = W^UV_h out_latent equals the unabsorbed attention's per-head value
    output ([P2] §2.1.2): associativity on the output side."""
    inp = make_inputs("single_b1_l128", seed=0)
    q_c = inp.extra["q_c"][0, 0].numpy()
    W_UK, W_UV = inp.extra["W_UK"].numpy(), inp.extra["W_UV"].numpy()
    rows = O.sequence_rows(inp, 0, int(inp.seq_lens[0]))
    q_r = inp.q_rope[0, 0].double().numpy()
    q_abs = O.absorb_query(q_c, W_UK)
    out_lat, _ = O.attend_latent(np.concatenate([q_abs, q_r], axis=1), rows, inp.scale)
    o = O.output_side(out_lat[None, None], W_UV)[0, 0]
    o_ref, _, _ = O.unabsorbed_attention(q_c, q_r, rows[:, :512], rows[:, 512:], W_UK, W_UV, inp.scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)


def test_kv_project_special_cases():
    """Selection matrices pick the hidden state's own coordinates; the result
    equals torch's fp64 linear layers."""
    rng = np.random.default_rng(2)
    T, d = 5, 700
    h = rng.standard_normal((T, d))
    W_DKV = np.zeros((512, d))
    W_DKV[np.arange(512), np.arange(512)] = 1.0
    W_KR = np.zeros((64, d))
    W_KR[np.arange(64), 600 + np.arange(64)] = 1.0
    kv = O.kv_project(h, W_DKV, W_KR)
    np.testing.assert_array_equal(kv[:, :512], h[:, :512])
    np.testing.assert_array_equal(kv[:, 512:], h[:, 600:664])
    A, Bm = rng.standard_normal((512, d)), rng.standard_normal((64, d))
    kv = O.kv_project(h, A, Bm)
    ht = torch.from_numpy(h)
    ref = torch.cat([torch.nn.functional.linear(ht, torch.from_numpy(A)),
                     torch.nn.functional.linear(ht, torch.from_numpy(Bm))], dim=-1).numpy()
    np.testing.assert_allclose(kv, ref, rtol=1e-12, atol=1e-10)


def test_e4m3_quantize_against_torch_and_edge_cases():
    """Codes equal torch's float8_e4m3fn cast of the fp32 quotient (round to
    nearest even) wherever it is within range; every finite code is its own
    nearest value; midpoints go to the even code; values past 448 saturate;
    an all-zero block gets scale 1; the block's largest value maps to +-448."""
    g = torch.Generator().manual_seed(3)
    x = (torch.randn((16, 512), generator=g) * torch.logspace(-3, 3, 16)[:, None]).float()
    x[2, :128] = 0.0
    codes, scales = O.e4m3_quantize(x.numpy())
    q = (x.reshape(16, 4, 128) / torch.from_numpy(scales)[..., None]).float()
    ref = q.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(16, 512).numpy()
    np.testing.assert_array_equal(codes, ref)
    assert scales[2, 0] == 1.0 and np.all(codes[2, :128] == 0)
    amax = np.abs(x.numpy()).reshape(16, 4, 128).max(-1)
    np.testing.assert_array_equal(scales, np.where(amax > 0, amax / np.float32(448), 1.0).astype(np.float32))
    amax_idx = np.abs(x.numpy()).reshape(16, 4, 128).argmax(-1)
    for r in (0, 7, 15):
        for blk in range(4):
            assert O.e4m3_decode(codes[r, blk * 128 + amax_idx[r, blk]]) in (448.0, -448.0)
    # every finite code value is its own nearest; midpoints round to the even code
    all_codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(all_codes)
    fin = np.isfinite(vals) & ~((all_codes == 0x80))          # -0 maps back to +0's twin below
    np.testing.assert_array_equal(O.e4m3_nearest(vals[fin]), all_codes[fin])
    assert O.e4m3_nearest(np.array([-0.0]))[0] == 0x80
    pos_vals = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    mids = (pos_vals[:-1] + pos_vals[1:]) / 2
    got = O.e4m3_nearest(mids)
    assert np.all(got % 2 == 0)
    assert np.all(O.e4m3_nearest(np.array([449.0, 470.0, 1e9, -1e9])) == [0x7E, 0x7E, 0x7E, 0xFE])


def test_bf16_bits_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(O.to_bf16_bits(x), ref)


def test_cache_append_writes_each_new_row_where_the_decode_reads_it():
    """After cache_append the oracle's own row gather returns, at rows
    seq_len - S_q + s, [c^KV ; RoPE(k, row)] (bf16) or its e4m3 encoding;
    every other row is unchanged."""
    for cache_kind in ("bf16", "fp8_e4m3"):
        inp = small_inputs([70, 5, 130], s_q=2, cache=cache_kind, seed=4)
        rng = np.random.default_rng(5)
        kv = rng.standard_normal((3, 2, 576)).astype(np.float32)
        if cache_kind == "bf16":
            cache = {"rows": inp.cache.view(torch.int16).numpy().astype(np.uint16)}
        else:
            cache = {"rows": inp.cache.numpy(), "scales": inp.cache_scales.numpy(),
                     "rope": inp.cache_rope.view(torch.int16).numpy().astype(np.uint16)}
        before = [O.sequence_rows(inp, b, int(inp.seq_lens[b])) for b in range(3)]
        new = O.cache_append(kv, inp.seq_lens.numpy(), inp.block_table.numpy(), inp.max_blocks, cache)
        if cache_kind == "bf16":
            inp.cache = torch.from_numpy(new["rows"].astype(np.int16)).view(torch.bfloat16)
        else:
            inp.cache = torch.from_numpy(new["rows"])
            inp.cache_scales = torch.from_numpy(new["scales"])
            inp.cache_rope = torch.from_numpy(new["rope"].astype(np.int16)).view(torch.bfloat16)
        for b in range(3):
            L = int(inp.seq_lens[b])
            after = O.sequence_rows(inp, b, L)
            np.testing.assert_array_equal(after[:L - 2], before[b][:L - 2])
            for s in range(2):
                row = after[L - 2 + s]
                kr = O.rope(kv[b, s, 512:].astype(np.float64), L - 2 + s)
                np.testing.assert_allclose(row[512:], kr, rtol=2 ** -8, atol=1e-30)
                if cache_kind == "bf16":
                    np.testing.assert_allclose(row[:512], kv[b, s, :512], rtol=2 ** -8)
                else:
                    sc = np.abs(kv[b, s, :512]).reshape(4, 128).max(1) / 448
                    err = np.abs(row[:512] - kv[b, s, :512])
                    assert np.all(err <= np.maximum(2 ** -4 * np.abs(kv[b, s, :512]), np.repeat(sc, 128) * 2 ** -10)
                                  + 1e-12)
