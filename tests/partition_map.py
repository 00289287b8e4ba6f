"""The work partition map of mla_decode / mla_combine, written out plainly
(host-side test helper, the description in include/mla.h).

The rows of the batch are cut into 64-row units (pages), sequence after
sequence; sequence b has n_b = max(1, ceil(len_b / 64)) units.  Every
sequence also weighs SEG_WEIGHT units of fixed cost, placed before its pages:
unit j of sequence b has the weighted position u0_b + (b + 1) SEG_WEIGHT + j
(u0_b = units of the sequences before b).  Partition p of P (a power of two)
takes the units whose positions fall in [A_p, A_{p+1}), A_p = floor(p W / P),
W = total units + batch SEG_WEIGHT.  A partition's units are consecutive; it
writes partial slot 0 for the sequence it starts in (or whose first unit is
its first unit) and slot 1 for the one it ends in.
"""
SEG_WEIGHT = 3


def units_of_len(n):
    return max(1, (int(n) + 63) >> 6)


def partition_map(lens, parts):
    """-> (unit range [ua, ub) of every partition, and for every sequence the
    list of (partition, slot, first unit, end unit) holding its units)."""
    n = [units_of_len(L) for L in lens]
    u0 = [sum(n[:b]) for b in range(len(n))]
    W = sum(n) + len(n) * SEG_WEIGHT
    A = [(p * W) // parts for p in range(parts + 1)]

    def before(x):
        return sum(min(max(x - (u0[b] + (b + 1) * SEG_WEIGHT), 0), n[b]) for b in range(len(n)))

    ranges = [(before(A[p]), before(A[p + 1])) for p in range(parts)]
    owners = []
    for b in range(len(n)):
        lo_b, hi_b = u0[b], u0[b] + n[b]
        own = []
        for p, (ua, ub) in enumerate(ranges):
            lo, hi = max(ua, lo_b), min(ub, hi_b)
            if lo < hi:
                own.append((p, 0 if lo_b <= ua else 1, lo, hi))
        owners.append(own)
    return ranges, owners
