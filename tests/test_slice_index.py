"""The shard-slice index of the standalone apply kernel (host check
of its arithmetic, CPU only).

For a sharded matrix the kernel finds the slice of flattened element e as
k = int(e * (1.0 / slice)) followed by one correction, k += ((k + 1) * slice
<= e), instead of a 64-bit integer division.  IEEE-754 double multiplication
and division are correctly rounded on the host as on the device, so this
brute-forces the claim that the result always equals e // slice over the
accepted range (numel <= 2^34, slices of at least 8 elements) at the points
where a rounding error would show: around every multiple of slice.
"""

import numpy as np


def slice_index(e, slice_len):
    inv = 1.0 / float(slice_len)
    k = int(float(e) * inv)
    if (k + 1) * slice_len <= e:
        k += 1
    return k


def test_slice_index_equals_integer_division():
    rng = np.random.default_rng(5)
    lens = [8, 16, 24, 136, 4096, 2 ** 20 + 8, 2 ** 26 - 8, 2 ** 30, 2 ** 31 - 8, 2 ** 33]
    lens += [int(v) * 8 for v in rng.integers(1, 2 ** 28, size=40)]
    checked = 0
    for s in lens:
        shards = (2 ** 34) // s
        ks = {0, 1, 2, shards - 1, shards} | {int(v) for v in rng.integers(0, shards + 1, size=200)}
        for k in ks:
            for e in (k * s - 1, k * s, k * s + 1, k * s + s // 2, k * s + s - 1):
                if 0 <= e < 2 ** 34:
                    assert slice_index(e, s) == e // s, (e, s)
                    checked += 1
    assert checked > 10000
