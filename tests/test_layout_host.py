"""Host-side checks of the partial_out layout helper the GPU tests use to feed
mla_combine: it must place each value where include/mla.h says."""
import numpy as np
import torch

from gpu_helpers import pack_partial_out


def test_pack_partial_out_matches_documented_offsets():
    rng = np.random.default_rng(3)
    po = torch.from_numpy(rng.standard_normal((2, 2, 2, 128, 512)).astype(np.float32))
    packed = pack_partial_out(po)
    assert packed.shape == (2, 2, 2, 128 * 512)
    for _ in range(2000):
        n, k, s = (int(x) for x in rng.integers(0, 2, 3))
        j, a, r = int(rng.integers(4)), int(rng.integers(2)), int(rng.integers(16))
        c, g, i = int(rng.integers(32)), int(rng.integers(4)), int(rng.integers(4))
        off = 16384 * j + 4 * (64 * (32 * a + c) + 16 * g + r) + i
        assert packed[n, k, s, off] == po[n, k, s, 32 * j + 16 * a + r, 16 * c + 4 * g + i]


def test_pack_partial_out_is_a_permutation():
    po = torch.arange(128 * 512, dtype=torch.float32).reshape(1, 1, 1, 128, 512)
    packed = pack_partial_out(po).flatten()
    assert torch.equal(torch.sort(packed).values, po.flatten())
