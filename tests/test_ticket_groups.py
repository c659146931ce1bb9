"""The two-level ticket of the grid reduction (csrc/ecc_device.hpp, grid_reduce),
restated on the host: for launches of more than 64 workgroups, workgroup b
counts into group ticket b // gs with gs = ceil(N / 32); the workgroup that
completes its group counts into the main ticket, and the one that completes
that holds every contribution.  The arithmetic must put every workgroup in
exactly one group, use at most 32 group lines, and elect exactly one last
workgroup, the last to arrive, whatever the arrival order."""

import numpy as np
import pytest

GROUPS = 32


def groups(n):
    gs = (n + GROUPS - 1) // GROUPS
    ng = (n + gs - 1) // gs
    return gs, ng


def elect(n, order):
    gs, ng = groups(n)
    count = [0] * ng
    main = 0
    last = []
    for b in order:
        g = b // gs
        gsize = min(gs, n - g * gs)
        p = count[g]
        count[g] += 1
        if p == gsize - 1:
            count[g] = 0  # the group's last resets its line
            q = main
            main += 1
            if q == ng - 1:
                last.append(b)
                main = 0
    return last, count, main


@pytest.mark.parametrize("n", [65, 66, 96, 97, 127, 128, 129, 511, 512, 768, 1000, 1023, 1024, 1025, 4096,
                               16383, 16384, 65535])
def test_groups_cover_every_workgroup_once(n):
    gs, ng = groups(n)
    assert 1 <= ng <= GROUPS
    sizes = [min(gs, n - g * gs) for g in range(ng)]
    assert all(s >= 1 for s in sizes) and sum(sizes) == n
    assert max(b // gs for b in range(n)) == ng - 1


@pytest.mark.parametrize("n", [65, 97, 1000, 1024, 3001])
def test_exactly_one_last_and_lines_left_zero(n):
    rng = np.random.default_rng(n)
    for order in (range(n), range(n - 1, -1, -1), rng.permutation(n), rng.permutation(n)):
        order = list(order)
        last, count, main = elect(n, order)
        assert last == [order[-1]]
        assert all(c == 0 for c in count) and main == 0
