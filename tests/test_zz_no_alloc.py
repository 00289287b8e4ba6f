"""mla_decode_noalloc (decode + combine with the library's static scratch for
the split partials) against mla_decode + mla_combine with a caller workspace,
through the C ABI: two calls in a row, the second on a smaller input, so that
the scratch's leftover partials from the first call must not reach the second
result.  Both runs use the same kernels and partition map, so the outputs
agree bit for bit; each is also held to the oracle's tolerance."""
import numpy as np
import pytest
import torch

from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def _small(lens, s_q=1, seed=0, cache="bf16", layout="paged_shuffled"):
    return make_inputs(dict(batch=len(lens), s_q=s_q, lens=("explicit", list(lens)), layout=layout, q_std=1.0,
                            cache=cache, num_splits=None, unabsorbed=False, name="noalloc"), seed=seed)


def _both(inp, splits):
    import mla_latent_kv_39_amd as mla
    from gpu_helpers import DeviceInputs, compare
    print(f"[gpu] noalloc: B={inp.batch} S_q={inp.s_q} cache={inp.cache_dtype} splits={splits}", flush=True)
    dev = DeviceInputs(inp)
    out_ws, lse_ws = dev.run(splits)
    out = torch.full((inp.batch, inp.s_q, 128, 512), float("nan"), device="cuda")
    lse = torch.full((inp.batch, inp.s_q, 128), float("nan"), device="cuda")
    mla.mla_decode_noalloc(dev.q_absorbed, dev.q_rope, dev.cache, dev.block_table, dev.seq_lens, inp.scale, out,
                           lse, splits)
    torch.cuda.synchronize()
    out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.array_equal(out, out_ws) and np.array_equal(lse, lse_ws, equal_nan=False), "differs from mla_decode"
    ref_out, ref_lse = O.mla_decode(inp)
    e = compare(out, lse, ref_out, ref_lse, "noalloc")
    print(f"[gpu] noalloc: identical to the workspace path; max err out {e[0]:.2e} lse {e[1]:.2e}", flush=True)


def test_noalloc_matches_the_workspace_path_twice():
    import mla_latent_kv_39_amd as mla
    mla.mla_init(torch.cuda.current_device())
    _both(_small([1, 63, 64, 65, 130, 700, 257, 3000], s_q=2, seed=31), 128)     # fills the scratch: 128 x 2
    _both(_small([2, 65, 129], s_q=1, seed=32), 8)                               # smaller, right after
    _both(_small([33, 200, 129, 64], s_q=1, seed=33, cache="fp8_e4m3"), 16)
    _both(_small([100, 37, 640], s_q=4, seed=34, layout="contiguous"), 1)       # one partition: no scratch


def test_noalloc_rejects_requests_beyond_its_scratch():
    import mla_latent_kv_39_amd as mla
    from gpu_helpers import DeviceInputs
    inp = _small([65, 130], s_q=2, seed=35)
    dev = DeviceInputs(inp)
    out = torch.empty((2, 2, 128, 512), device="cuda")
    lse = torch.empty((2, 2, 128), device="cuda")
    with pytest.raises(mla.MlaError, match="static scratch") as e:
        mla.mla_decode_noalloc(dev.q_absorbed, dev.q_rope, dev.cache, dev.block_table, dev.seq_lens, inp.scale,
                               out, lse, 256)       # 256 x 2 tokens > 256
    assert e.value.status == 7
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_noalloc(dev.q_absorbed, dev.q_rope, dev.cache, dev.block_table, dev.seq_lens, inp.scale,
                               out, lse, 6)         # not a power of two
    assert e.value.status == 3
