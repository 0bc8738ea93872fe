"""Host model of the single-pass quantize's two-level grid barrier: the
counter arithmetic of fused_arrive_wait / fused_last_to_finish
(bit_block_scaled_nvfp4_amd/csrc/quantize.hip) replayed over calls with
different grid sizes and random arrival orders.  The release must come
exactly with the last arrival of each call, the finish count must pick the
last workgroup, and every counter must be back at zero after each call --
which the earlier rule (counters that only grow, tested modulo the slot
size) did not give once grid sizes changed between calls."""
import random

import pytest


class Ctrl:
    def __init__(self):
        self.arrive = [0] * 8
        self.fin = [0] * 8
        self.top = 0
        self.top_fin = 0
        self.release = 0


def per_slot(grid, slot):
    return grid // 8 + (1 if slot < grid % 8 else 0)


def arrive(c: Ctrl, grid: int, bid: int, e: int) -> bool:
    """One workgroup's arrival; True if it published the release."""
    slot = bid & 7
    old = c.arrive[slot]
    c.arrive[slot] += 1
    if old + 1 == per_slot(grid, slot):
        c.arrive[slot] = 0
        t = c.top
        c.top += 1
        if t + 1 == min(grid, 8):
            c.top = 0
            c.release = e + 1
            return True
    return False


def finish(c: Ctrl, grid: int, bid: int) -> bool:
    slot = bid & 7
    old = c.fin[slot]
    c.fin[slot] += 1
    if old + 1 != per_slot(grid, slot):
        return False
    c.fin[slot] = 0
    t = c.top_fin
    c.top_fin += 1
    if t + 1 != min(grid, 8):
        return False
    c.top_fin = 0
    return True


def old_rule_arrive(c: Ctrl, grid: int, bid: int, e: int) -> bool:
    slot = bid & 7
    old = c.arrive[slot]
    c.arrive[slot] += 1
    if (old + 1) % per_slot(grid, slot) == 0:
        t = c.top
        c.top += 1
        if (t + 1) % min(grid, 8) == 0:
            c.release = e + 1
            return True
    return False


@pytest.mark.parametrize("seed", range(20))
def test_release_with_the_last_arrival_for_mixed_grids(seed):
    rng = random.Random(seed)
    c = Ctrl()
    for call in range(40):
        grid = rng.choice([1, 2, 3, 4, 7, 8, 9, 15, 16, 31, 64, 100, 255, 256])
        e = c.release
        order = list(range(grid))
        rng.shuffle(order)
        for n, bid in enumerate(order):
            published = arrive(c, grid, bid, e)
            assert published == (n == grid - 1), (call, grid, n)
        assert c.release == e + 1
        assert c.arrive == [0] * 8 and c.top == 0
        order = list(range(grid))
        rng.shuffle(order)
        lasts = [finish(c, grid, bid) for bid in order]
        assert lasts == [False] * (grid - 1) + [True]
        assert c.fin == [0] * 8 and c.top_fin == 0


def test_old_rule_released_early_after_a_smaller_grid():
    """The case the reset fixes: a 4-workgroup call, then 256 workgroups in
    index order, then 256 workgroups in reverse order (the data-holding low
    indices last) on the same counters."""
    c = Ctrl()
    early = False
    for grid, order in [(4, range(4)), (256, range(256)), (256, range(255, -1, -1))]:
        e = c.release
        order = list(order)
        for n, bid in enumerate(order):
            if old_rule_arrive(c, grid, bid, e) and n != grid - 1:
                early = True
    assert early
