"""The five decode workloads at full size, in the launch configuration bench.py times.

Sampled: the oracle computes the first, the last, the shortest and the
longest sequence's results one by one, all 128 heads, for every workload.
Full: every output of the four large workloads (about 20 s of host work in
all; measured max errors 3.4e-3, 2.2e-3, 3.7e-3 and 1.6e-4 on out, ~2e-6 on
lse).
"""
import numpy as np
import pytest
import torch

from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = [pytest.mark.gpu]


def _num_splits(inp):
    import mla_latent_kv_39_amd as mla
    if inp.num_splits:
        return int(inp.num_splits)
    return mla.mla_num_splits_hint(torch.cuda.current_device(), inp.batch, inp.s_q, inp.max_blocks)


@pytest.mark.parametrize("name", ["single_b1_l128", "batched_b32_l1k_4k", "paged_b64_l256_32k",
                                  "mtp_b128_sq2_l4k_8k", "fp8_b4_l128k"])
def test_workload_sampled_parity(name):
    from gpu_helpers import DeviceInputs, compare
    print(f"[gpu] workload {name}: generating inputs", flush=True)
    inp = make_inputs(name, seed=0)
    splits = _num_splits(inp)
    print(f"[gpu] workload {name}: B={inp.batch} rows={inp.total_rows()} splits={splits}", flush=True)
    dev = DeviceInputs(inp)
    out, lse = dev.run(splits)
    lens = inp.seq_lens.numpy()
    picks = sorted({0, inp.batch - 1, int(np.argmin(lens)), int(np.argmax(lens))})
    worst = (0.0, 0.0)
    for b in picks:
        for s in range(inp.s_q):
            ref_out, ref_lse = O.decode_one(inp, b, s)
            e = compare(out[b, s], lse[b, s], ref_out, ref_lse, f"{name} b={b} s={s}")
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    # properties that hold for every result: finite, lse finite, out inside the rows' range
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    print(f"[gpu] workload {name}: sampled max err out {worst[0]:.2e} lse {worst[1]:.2e}", flush=True)


@pytest.mark.parametrize("name,splits", [("batched_b32_l1k_4k", None), ("paged_b64_l256_32k", None),
                                         ("mtp_b128_sq2_l4k_8k", None), ("fp8_b4_l128k", None),
                                         ("fp8_b4_l128k", 64)])
def test_workload_full_parity(name, splits):
    """Every output of the four large workloads, all sequences, query tokens
    and heads, against the oracle (seconds of host work each), in bench.py's
    launch (the workload's partition count, else the library's hint); the
    long-context e4m3 workload also with 16 partitions per sequence."""
    from gpu_helpers import DeviceInputs, compare
    print(f"[gpu] workload {name} (full): generating inputs", flush=True)
    inp = make_inputs(name, seed=0)
    splits = splits or _num_splits(inp)
    print(f"[gpu] workload {name} (full): splits={splits}", flush=True)
    out, lse = DeviceInputs(inp).run(splits)
    print(f"[gpu] workload {name} (full): oracle over {inp.batch} sequences", flush=True)
    ref_out, ref_lse = O.mla_decode(inp)
    e = compare(out, lse, ref_out, ref_lse, f"{name} full")
    print(f"[gpu] workload {name} (full): max err out {e[0]:.2e} lse {e[1]:.2e}", flush=True)
