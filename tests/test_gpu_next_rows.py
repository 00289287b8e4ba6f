"""Parity of the steps around the decode (query absorption + RoPE, output
absorption, KV projection, cache append) through the C ABI with the fp64
oracle, on seeded inputs spanning several 64-token tiles and a ragged tail,
and one chained attention step against the unabsorbed per-head form."""
import math

import numpy as np
import pytest
import torch

from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _small(lens, s_q=1, seed=0, cache="bf16", layout="paged_shuffled"):
    return make_inputs(dict(batch=len(lens), s_q=s_q, lens=("explicit", list(lens)), layout=layout, q_std=1.0,
                            cache=cache, num_splits=None, unabsorbed=False, name="next"), seed=seed)


@pytest.mark.parametrize("B,S,in_place", [(35, 2, False), (3, 1, False), (64, 4, False), (100, 3, True)])
def test_absorb_query_and_rope(B, S, in_place):
    """Up to 256 tokens one tile or two, each workgroup rotating one token's
    q^R; 300 tokens take three tiles and rotate the last 44 after them, with
    q_rope written over q_r (the documented in-place use)."""
    import mla_latent_kv_39_amd as mla
    g = torch.Generator().manual_seed(40 + B)
    q_c = torch.randn((B, S, 128, 128), generator=g).to(torch.bfloat16)
    q_r = torch.randn((B, S, 128, 64), generator=g).to(torch.bfloat16)
    W_UK = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    lens = torch.randint(S, 140000, (B,), generator=g, dtype=torch.int32)
    print(f"[gpu] absorb_query B={B} S={S} tokens={B * S} in_place={in_place}", flush=True)
    d = torch.device("cuda")
    q_abs = torch.full((B, S, 128, 512), float("nan"), dtype=torch.bfloat16, device=d)
    q_r_dev = q_r.to(d)
    q_rot = q_r_dev if in_place else torch.full((B, S, 128, 64), float("nan"), dtype=torch.bfloat16, device=d)
    mla.mla_absorb_query(q_c.to(d), q_r_dev, W_UK.transpose(1, 2).contiguous().to(d), lens.to(d), q_abs, q_rot)
    torch.cuda.synchronize()
    ref_abs, ref_rot = O.query_side(q_c.double().numpy(), q_r.double().numpy(), W_UK.double().numpy(), lens.numpy())
    got_abs, got_rot = q_abs.cpu().double().numpy(), q_rot.cpu().double().numpy()
    # one bf16 rounding of an fp32-accumulated sum: 2^-8 relative, plus the accumulation
    e_abs = np.abs(got_abs - ref_abs)
    assert np.all(e_abs <= 2.0 ** -8 * np.abs(ref_abs) + 1e-4), e_abs.max()
    e_rot = np.abs(got_rot - ref_rot)
    assert np.all(e_rot <= 2.0 ** -8 * np.abs(ref_rot) + 1e-6), e_rot.max()
    print(f"[gpu] absorb_query: max err q_absorbed {e_abs.max():.2e} q_rope {e_rot.max():.2e}", flush=True)


@pytest.mark.parametrize("B,S", [(35, 2), (1, 1), (128, 2), (150, 2)])
def test_absorb_output(B, S):
    import mla_latent_kv_39_amd as mla
    g = torch.Generator().manual_seed(50 + B)
    out_lat = (torch.randn((B, S, 128, 512), generator=g) * 0.3).float()
    W_UV = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    print(f"[gpu] absorb_output B={B} S={S}", flush=True)
    d = torch.device("cuda")
    vals = torch.full((B, S, 128, 128), float("nan"), device=d)
    mla.mla_absorb_output(out_lat.to(d), W_UV.to(d), vals)
    torch.cuda.synchronize()
    W = W_UV.double().numpy()
    ref = O.output_side(out_lat.double().numpy(), W)
    # out_latent enters the MFMAs rounded to bf16: each product is off by at most
    # 2^-8 of itself; fp32 accumulation adds ~1e-6
    bound = 2.0 ** -8 * np.einsum("hdc,bshc->bshd", np.abs(W), np.abs(out_lat.double().numpy())) + 1e-5
    err = np.abs(vals.cpu().double().numpy() - ref)
    assert np.all(err <= bound), (err / bound).max()
    print(f"[gpu] absorb_output: max err {err.max():.2e} (largest share of the bound {(err / bound).max():.2f})",
          flush=True)


@pytest.mark.parametrize("T,D", [(70, 7168), (256, 7168), (5, 128), (33, 640)])
def test_kv_project(T, D):
    import mla_latent_kv_39_amd as mla
    g = torch.Generator().manual_seed(60 + T)
    h = torch.randn((T, D), generator=g).to(torch.bfloat16)
    W = (torch.randn((576, D), generator=g) / math.sqrt(D)).to(torch.bfloat16)
    print(f"[gpu] kv_project T={T} d={D}", flush=True)
    d = torch.device("cuda")
    kv = torch.full((T, 576), float("nan"), device=d)
    mla.mla_kv_project(h.to(d), W.to(d), kv)
    torch.cuda.synchronize()
    Wd = W.double().numpy()
    ref = O.kv_project(h.double().numpy(), Wd[:512], Wd[512:])
    err = np.abs(kv.cpu().double().numpy() - ref)
    # exact bf16 products, fp32 accumulation over D terms
    bound = 1e-6 * (np.abs(h.double().numpy()) @ np.abs(Wd).T) + 1e-6
    assert np.all(err <= bound), (err / bound).max()
    print(f"[gpu] kv_project: max err {err.max():.2e}", flush=True)



@pytest.mark.parametrize("T,D,S", [(70, 7168, None), (256, 7168, None), (300, 7168, None), (256, 7168, 1),
                                   (256, 7168, 7), (5, 128, None), (33, 640, None)])
def test_kv_project_split(T, D, S):
    """K cut into S slices (None: the library's hint; 14 for 256 x 7168, 28 for
    70 tokens) against the oracle, two calls bit for bit (the partials are
    summed in slice order), and against the unsplit entry point within the
    same fp32 bound."""
    import mla_latent_kv_39_amd as mla
    S = S or mla.mla_kv_project_splits(T, D)
    g = torch.Generator().manual_seed(70 + T + S)
    h = torch.randn((T, D), generator=g).to(torch.bfloat16)
    W = (torch.randn((576, D), generator=g) / math.sqrt(D)).to(torch.bfloat16)
    print(f"[gpu] kv_project_split T={T} d={D} S={S}", flush=True)
    d = torch.device("cuda")
    hd, Wd_ = h.to(d), W.to(d)
    ws = torch.full((S, T, 576), float("nan"), device=d)
    kv = torch.full((T, 576), float("nan"), device=d)
    mla.mla_kv_project_split(hd, Wd_, kv, ws)
    kv2 = torch.full((T, 576), float("nan"), device=d)
    mla.mla_kv_project_split(hd, Wd_, kv2, ws)
    kv1 = torch.full((T, 576), float("nan"), device=d)
    mla.mla_kv_project(hd, Wd_, kv1)
    torch.cuda.synchronize()
    assert torch.equal(kv, kv2)
    Wd = W.double().numpy()
    ref = O.kv_project(h.double().numpy(), Wd[:512], Wd[512:])
    bound = 1e-6 * (np.abs(h.double().numpy()) @ np.abs(Wd).T) + 1e-6
    err = np.abs(kv.cpu().double().numpy() - ref)
    assert np.all(err <= bound), (err / bound).max()
    assert np.all(np.abs(kv.cpu().double().numpy() - kv1.cpu().double().numpy()) <= 2 * bound)
    print(f"[gpu] kv_project_split: max err {err.max():.2e}", flush=True)


def _cache_dict(inp):
    if inp.cache_dtype == "bf16":
        return {"rows": inp.cache.view(torch.int16).numpy().astype(np.uint16).copy()}
    return {"rows": inp.cache.numpy().copy(), "scales": inp.cache_scales.numpy().copy(),
            "rope": inp.cache_rope.view(torch.int16).numpy().astype(np.uint16).copy()}


@pytest.mark.parametrize("cache,layout", [("bf16", "paged_shuffled"), ("fp8_e4m3", "paged_shuffled"),
                                          ("bf16", "contiguous"), ("fp8_e4m3", "contiguous")])
def test_cache_append_bit_exact(cache, layout):
    """Every byte of the cache after the append equals the oracle's: the e4m3
    codes and scales and the bf16 latent bits (the same fp32 input, the same
    fp32 decisions on both sides), the rotated keys to within one bf16 unit;
    rows past the capacity and sequences shorter than S_q write nothing."""
    import mla_latent_kv_39_amd as mla
    from gpu_helpers import DeviceInputs
    S = 2
    lens = [1, 2, 63, 64, 65, 127, 128, 129, 700, 64 * 12]
    inp = _small(lens, s_q=S, seed=71, cache=cache, layout=layout)
    g = torch.Generator().manual_seed(72)
    kv = torch.randn((len(lens), S, 576), generator=g).float()
    kv[2, 0, :128] = 0.0                       # an all-zero block: scale 1, codes 0
    kv[3, 1, 130] = 1e4                        # one large value in its block
    kv[4, 0, 300] = -0.0
    print(f"[gpu] cache_append {cache} {layout} B={len(lens)} S={S}", flush=True)
    dev = DeviceInputs(inp)
    mla.mla_cache_append(kv.cuda(), dev.seq_lens, dev.block_table, dev.cache)
    torch.cuda.synchronize()
    ref = O.cache_append(kv.numpy(), inp.seq_lens.numpy(), None if inp.block_table is None else
                         inp.block_table.numpy(), inp.max_blocks, _cache_dict(inp))
    if cache == "bf16":
        got = dev.cache.rows.cpu().view(torch.int16).numpy().astype(np.uint16)
        np.testing.assert_array_equal(got[..., :512], ref["rows"][..., :512])
        kr_got, kr_ref = got[..., 512:], ref["rows"][..., 512:]
    else:
        np.testing.assert_array_equal(dev.cache.rows.cpu().numpy(), ref["rows"])
        np.testing.assert_array_equal(dev.cache.scales.cpu().numpy(), ref["scales"])
        kr_got = dev.cache.rope.cpu().view(torch.int16).numpy().astype(np.uint16)
        kr_ref = ref["rope"]
    diff = np.abs(kr_got.astype(np.int32) - kr_ref.astype(np.int32))
    assert diff.max() <= 1, diff.max()
    print(f"[gpu] cache_append {cache} {layout}: bit-exact latent part; rotated keys differ in "
          f"{int((diff > 0).sum())} of {diff.size} bf16 values by one unit", flush=True)


def test_attention_step_matches_unabsorbed_form():
    """kv_project -> cache_append -> absorb_query -> decode -> absorb_output
    on a small batch against the oracle's unabsorbed per-head attention over
    the same rows (the associativity of DeepSeek-V3 architecture notes
    §2.1.3(B), end to end)."""
    import mla_latent_kv_39_amd as mla
    from gpu_helpers import DeviceInputs
    from mla_latent_kv_39_amd.runner import DecodeWorkspace, decode_step
    B, S, D = 4, 2, 256
    lens = [70, 129, 300, 2]
    inp = _small(lens, s_q=S, seed=81)
    g = torch.Generator().manual_seed(82)
    h = torch.randn((B * S, D), generator=g).to(torch.bfloat16)
    W_kv = (torch.randn((576, D), generator=g) / math.sqrt(D)).to(torch.bfloat16)
    q_c = torch.randn((B, S, 128, 128), generator=g).to(torch.bfloat16)
    q_r = torch.randn((B, S, 128, 64), generator=g).to(torch.bfloat16)
    W_UK = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    W_UV = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    dev = DeviceInputs(inp)
    d = torch.device("cuda")
    kv = torch.empty((B * S, 576), device=d)
    mla.mla_kv_project(h.to(d), W_kv.to(d), kv)
    mla.mla_cache_append(kv.view(B, S, 576), dev.seq_lens, dev.block_table, dev.cache)
    q_abs = torch.empty((B, S, 128, 512), dtype=torch.bfloat16, device=d)
    q_rot = torch.empty((B, S, 128, 64), dtype=torch.bfloat16, device=d)
    mla.mla_absorb_query(q_c.to(d), q_r.to(d), W_UK.transpose(1, 2).contiguous().to(d), dev.seq_lens, q_abs, q_rot)
    ws = DecodeWorkspace(B, S, 8)
    out_lat, _ = decode_step(q_abs, q_rot, dev.cache, dev.block_table, dev.seq_lens, inp.scale, ws)
    vals = torch.empty((B, S, 128, 128), device=d)
    mla.mla_absorb_output(out_lat, W_UV.to(d), vals)
    torch.cuda.synchronize()
    # oracle: the same rows written by the oracle's own append of its own projection
    Wd = W_kv.double().numpy()
    kv_ref = O.kv_project(h.double().numpy(), Wd[:512], Wd[512:]).reshape(B, S, 576)
    new = O.cache_append(kv_ref.astype(np.float32), inp.seq_lens.numpy(), inp.block_table.numpy(), inp.max_blocks,
                         _cache_dict(inp))
    inp.cache = torch.from_numpy(new["rows"].astype(np.int16)).view(torch.bfloat16)
    q_abs_ref, q_rot_ref = O.query_side(q_c.double().numpy(), q_r.double().numpy(), W_UK.double().numpy(),
                                        inp.seq_lens.numpy())
    # tolerance: the decode's own 1e-2 on out_latent carried through W^UV_h
    # (rows of unit 2-norm: an uncorrelated elementwise error keeps its size)
    # plus the bf16 rounding of out_latent and q_absorbed on the way (2^-8 of
    # each value, relative): 1e-2 + 2^-7 |o|
    worst, share = 0.0, 0.0
    for b in range(B):
        for s in range(S):
            n = O.visible_rows(lens[b], S, s)
            rows = O.sequence_rows(inp, b, n)
            o_ref, _, _ = O.unabsorbed_attention(q_c[b, s].double().numpy(), q_rot_ref[b, s], rows[:, :512],
                                                 rows[:, 512:], W_UK.double().numpy(), W_UV.double().numpy(),
                                                 inp.scale)
            got = vals[b, s].cpu().double().numpy()
            if n == 0:
                assert np.all(got == 0)
                continue
            err = np.abs(got - o_ref)
            worst = max(worst, float(err.max()))
            share = max(share, float((err / (1e-2 + 2.0 ** -7 * np.abs(o_ref))).max()))
    assert share <= 1.0, (worst, share)
    print(f"[gpu] attention step vs unabsorbed per-head form: max err {worst:.2e} "
          f"(largest share of the bound {share:.2f})", flush=True)
