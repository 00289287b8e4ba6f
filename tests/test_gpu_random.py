"""Seeded random decode requests through the C ABI against the fp64 oracle.

Each case draws its own shape: batch 1..40, 1..6 query tokens, lengths from 0
to 900 with page-border values (0, 1, 63, 64, 65, 128) mixed in, contiguous,
sequential or shuffled pages, a bf16 or e4m3 cache, query spread 0.3..2 and a
power-of-two partition count up to 128 — combinations the directed tests do
not enumerate.  Every output element is compared at the usual bounds."""
import random

import numpy as np
import pytest

from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

EDGE = [0, 1, 63, 64, 65, 128]


def _case(seed):
    r = random.Random(1000 + seed)
    B = r.randint(1, 40)
    s_q = r.choice([1, 1, 2, 2, 3, 4, 5, 6])
    lens = [r.choice(EDGE) if r.random() < 0.3 else r.randint(0, 900) for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 1
    cfg = dict(batch=B, s_q=s_q, lens=("explicit", lens),
               layout=r.choice(["contiguous", "paged_sequential", "paged_shuffled"]),
               q_std=r.choice([0.3, 0.7, 1.0, 1.5, 2.0]), cache=r.choice(["bf16", "bf16", "fp8_e4m3"]),
               num_splits=None, unabsorbed=False, name=f"random{seed}")
    splits = 1 << r.randint(0, 7)
    return make_inputs(cfg, seed=seed), splits


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_request(seed):
    from gpu_helpers import DeviceInputs, compare, OUT_TOL
    inp, splits = _case(seed)
    what = (f"random {seed}: B={inp.batch} S_q={inp.s_q} {inp.cache_dtype} "
            f"{'contiguous' if inp.block_table is None else 'paged'} splits={splits} "
            f"lens={inp.seq_lens.tolist()[:6]}")
    print(f"[gpu] {what}", flush=True)
    out, lse = DeviceInputs(inp).run(splits)
    ref_out, ref_lse = O.mla_decode(inp)
    e = compare(out, lse, ref_out, ref_lse, what, out_tol=OUT_TOL)
    assert np.all(np.isfinite(out))
    print(f"[gpu] {what}: max err out {e[0]:.2e} lse {e[1]:.2e}", flush=True)
