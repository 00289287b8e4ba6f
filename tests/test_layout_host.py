"""Host-side checks of the partial_out format helpers the tests use to feed
mla_combine and to read the emulated kernels' partials: values and descales
must sit where include/mla.h says, and the round trip keeps 11 bits."""
import numpy as np
import torch

from gpu_helpers import pack_partial_out
from partial_format import BLOCK_BYTES, partial_bytes, unpack


def _partials(seed, shape=(2, 2, 2)):
    rng = np.random.default_rng(seed)
    po = rng.standard_normal(shape + (128, 512)) * np.exp(3 * rng.standard_normal(shape + (128, 1)))
    po[0, 0, 0, 7] = 0.0                       # a row that saw nothing
    po[0, 1, 0, 9, :128] *= 1e-30              # a quarter far below the others
    return po


def test_pack_partial_out_matches_documented_offsets():
    rng = np.random.default_rng(3)
    po = _partials(3)
    packed = pack_partial_out(torch.from_numpy(po)).numpy()
    assert packed.dtype == np.uint8 and packed.size == partial_bytes(2, 2)
    nb = 8
    vals = packed[:nb * BLOCK_BYTES].view(np.float16)
    desc = packed[nb * BLOCK_BYTES:].view(np.float32)
    flat = po.reshape(nb, 128, 512)
    for _ in range(3000):
        blk = int(rng.integers(nb))
        j, a, r = int(rng.integers(4)), int(rng.integers(2)), int(rng.integers(16))
        c, g, i = int(rng.integers(32)), int(rng.integers(4)), int(rng.integers(4))
        head, col, q = 32 * j + 16 * a + r, 16 * c + 4 * g + i, c // 8
        d = float(desc[512 * blk + 128 * q + 32 * j + 2 * r + a])
        x = float(vals[65536 * blk + 16384 * j + 8 * (64 * c + 16 * g + r) + 4 * a + i]) * d
        m = np.abs(flat[blk, head, 128 * q:128 * q + 128]).max()
        assert d == 2.0 ** np.round(np.log2(d))                          # a power of two
        # largest |value| in [2^14, 2^15) d, d no smaller than 2^-90 (rows of (nearly) zeros)
        assert (2.0 ** 14 <= m / d < 2.0 ** 15) if m >= 2.0 ** -76 else (d == 2.0 ** -90)
        assert abs(x - flat[blk, head, col]) <= 2.0 ** -11 * m


def test_partial_round_trip_keeps_eleven_bits():
    po = _partials(4)
    back = unpack(pack_partial_out(torch.from_numpy(po)).numpy(), 2, 2)
    m = np.abs(po).reshape(2, 2, 2, 128, 4, 128).max(axis=5, keepdims=True)
    err = np.abs(back - po).reshape(2, 2, 2, 128, 4, 128)
    assert np.all(err <= 2.0 ** -11 * m)
    assert np.all(back[0, 0, 0, 7] == 0)


# ------------------------------------------------------- partition map
def test_partition_map_covers_every_unit_once():
    """Every unit of every sequence belongs to exactly one partition; the
    units of a partition are consecutive; slot 1 only for a sequence that
    starts inside the partition."""
    import random
    from partition_map import partition_map, units_of_len
    rng = random.Random(0)
    for _ in range(200):
        lens = [rng.choice([0, 1, 63, 64, 65, rng.randint(1, 5000)]) for _ in range(rng.randint(1, 40))]
        parts = 2 ** rng.randint(0, 9)
        ranges, owners = partition_map(lens, parts)
        total = sum(units_of_len(L) for L in lens)
        assert ranges[0][0] == 0 and ranges[-1][1] == total
        for (a0, b0), (a1, b1) in zip(ranges, ranges[1:]):
            assert a0 <= b0 == a1 <= b1
        u0 = 0
        for b, own in enumerate(owners):
            n = units_of_len(lens[b])
            covered = sorted((lo, hi) for _, _, lo, hi in own)
            assert covered[0][0] == u0 and covered[-1][1] == u0 + n
            assert all(x[1] == y[0] for x, y in zip(covered, covered[1:]))
            for p, slot, lo, hi in own:
                assert slot == (1 if u0 > ranges[p][0] else 0)
            u0 += n


def test_partition_map_weighs_sequence_boundaries():
    """A partition that holds more sequences gets fewer units: the cost
    units + SEG_WEIGHT x (sequences it touches) varies across partitions by
    at most about one sequence's weight, where equal unit counts would let it
    vary by several."""
    from partition_map import partition_map, SEG_WEIGHT
    lens = [64 * 7] * 12 + [64 * 3] * 20
    parts = 16
    ranges, owners = partition_map(lens, parts)
    cost = []
    for p, (ua, ub) in enumerate(ranges):
        seqs = sum(1 for own in owners if any(q == p for q, *_ in own))
        cost.append((ub - ua) + SEG_WEIGHT * seqs)
    assert max(cost) - min(cost) <= 2 * SEG_WEIGHT + 1


def test_partition_weight_is_the_same_everywhere():
    """The decode kernels (generator), the combine kernel (header) and this
    reference use one sequence weight."""
    import os
    import re
    import sys
    import partition_map
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, os.path.join(root, "mla_latent_kv_39_amd", "csrc"))
    import gen_decode_gfx950 as G
    hdr = open(os.path.join(root, "mla_latent_kv_39_amd", "csrc", "mla_schedule.h")).read()
    assert int(re.search(r"kSegWeight = (\d+);", hdr).group(1)) == G.SEG_WEIGHT == partition_map.SEG_WEIGHT
