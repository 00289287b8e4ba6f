"""Decode steps captured in a HIP graph (the launches allocate, free and
clear nothing, so they can be captured): the prepared step and the no-alloc
entry point, each captured once and replayed several times with the query
changed in place and eager work in between; every replay must equal an eager
call on the same inputs bit for bit."""
import pytest
import torch

from mla_inputs import make_inputs

pytestmark = pytest.mark.gpu


def _inputs(cache, s_q, seed):
    return make_inputs(dict(batch=5, s_q=s_q, lens=("explicit", [5, 64, 200, 129, 333]), layout="paged_shuffled",
                            q_std=1.0, cache=cache, num_splits=None, unabsorbed=False, name="graph"), seed=seed)


@pytest.mark.parametrize("cache,s_q,splits", [("bf16", 1, 8), ("bf16", 2, 4), ("fp8_e4m3", 1, 16)])
def test_prepared_step_replays_like_eager(cache, s_q, splits):
    import mla_latent_kv_39_amd as mla
    from gpu_helpers import DeviceInputs
    from mla_latent_kv_39_amd.runner import DecodeWorkspace
    print(f"[gpu] graph of a prepared step: {cache} S_q={s_q} splits={splits}", flush=True)
    inp = _inputs(cache, s_q, 21)
    dev = DeviceInputs(inp)
    ws_g, ws_e = DecodeWorkspace(inp.batch, s_q, splits), DecodeWorkspace(inp.batch, s_q, splits)
    args = (dev.q_absorbed, dev.q_rope, dev.cache, dev.block_table, dev.seq_lens, inp.scale)
    step_g = mla.PreparedStep(*args, ws_g.out, ws_g.lse, ws_g.partial_out, ws_g.partial_lse)
    step_e = mla.PreparedStep(*args, ws_e.out, ws_e.lse, ws_e.partial_out, ws_e.partial_lse)
    step_g()                      # loads the code object before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_g()
    q0 = dev.q_absorbed.clone()
    for k in range(4):
        dev.q_absorbed.copy_(q0 * (1.0 - 0.2 * k))
        noise = torch.randn(1 << 20, device="cuda").sum()      # eager work between the replays
        graph.replay()
        step_e()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        assert torch.equal(ws_g.out, ws_e.out) and torch.equal(ws_g.lse, ws_e.lse), f"replay {k}"
    del graph


def test_noalloc_decode_replays_like_eager():
    import mla_latent_kv_39_amd as mla
    from gpu_helpers import DeviceInputs
    print("[gpu] graph of mla_decode_noalloc", flush=True)
    inp = _inputs("bf16", 2, 22)
    dev = DeviceInputs(inp)
    shape_o, shape_l = (inp.batch, 2, 128, 512), (inp.batch, 2, 128)
    out_g, lse_g = torch.empty(shape_o, device="cuda"), torch.empty(shape_l, device="cuda")
    out_e, lse_e = torch.empty(shape_o, device="cuda"), torch.empty(shape_l, device="cuda")
    args = (dev.q_absorbed, dev.q_rope, dev.cache, dev.block_table, dev.seq_lens, inp.scale)
    mla.mla_init(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mla.mla_decode_noalloc(*args, out_g, lse_g, 16)
    q0 = dev.q_absorbed.clone()
    for k in range(4):
        dev.q_absorbed.copy_(q0 * (1.0 + 0.3 * k))
        graph.replay()
        torch.cuda.synchronize()
        mla.mla_decode_noalloc(*args, out_e, lse_e, 16)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), f"replay {k}"
    del graph


def test_layer_kernels_replay_like_eager():
    """The kernels around the decode captured together (split KV projection,
    cache append into a bf16 cache, query absorption with RoPE, output
    absorption) and replayed with their inputs changed in place and eager
    work in between: every replay equals the same calls made eagerly."""
    import mla_latent_kv_39_amd as mla
    print("[gpu] graph of the kernels around the decode", flush=True)
    d = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(23)
    B, S, D = 4, 2, 7168
    T = B * S
    lens = torch.tensor([70, 130, 2, 64], dtype=torch.int32, device=d)
    table = torch.arange(B * 4, dtype=torch.int32, device=d).view(B, 4)
    h = torch.randn((T, D), generator=g).to(torch.bfloat16).to(d)
    w_kv = (torch.randn((576, D), generator=g) * D ** -0.5).to(torch.bfloat16).to(d)
    q_c = torch.randn((B, S, 128, 128), generator=g).to(torch.bfloat16).to(d)
    q_r = torch.randn((B, S, 128, 64), generator=g).to(torch.bfloat16).to(d)
    w_uk_t = (torch.randn((128, 512, 128), generator=g) * 512 ** -0.5).to(torch.bfloat16).to(d)
    out_lat = torch.randn((B, S, 128, 512), generator=g).to(d)
    w_uv = (torch.randn((128, 128, 512), generator=g) * 512 ** -0.5).to(torch.bfloat16).to(d)
    splits = mla.mla_kv_project_splits(T, D)

    def buffers():
        rows = torch.zeros((B * 4, 64, 576), dtype=torch.bfloat16, device=d)
        return dict(ws=torch.empty((splits, T, 576), device=d), kv=torch.empty((T, 576), device=d), rows=rows,
                    cache=mla.LatentCache(mla.MLA_CACHE_BF16, rows),
                    qa=torch.empty((B, S, 128, 512), dtype=torch.bfloat16, device=d),
                    qr=torch.empty((B, S, 128, 64), dtype=torch.bfloat16, device=d),
                    ov=torch.empty((B, S, 128, 128), device=d))

    def layer(o):
        mla.mla_kv_project_split(h, w_kv, o["kv"], o["ws"])
        mla.mla_cache_append(o["kv"].view(B, S, 576), lens, table, o["cache"])
        mla.mla_absorb_query(q_c, q_r, w_uk_t, lens, o["qa"], o["qr"])
        mla.mla_absorb_output(out_lat, w_uv, o["ov"])

    og, oe = buffers(), buffers()
    layer(og)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(og)
    h0, q0, o0 = h.clone(), q_c.clone(), out_lat.clone()
    for k in range(4):
        f = 1.0 - 0.2 * k
        h.copy_(h0 * f)
        q_c.copy_(q0 * f)
        out_lat.copy_(o0 * f)
        noise = torch.randn(1 << 20, device="cuda").sum()      # eager work between the replays
        graph.replay()
        layer(oe)
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        for key in ("kv", "rows", "qa", "qr", "ov"):
            assert torch.equal(og[key], oe[key]), f"replay {k}: {key}"
    del graph
