"""The recomputing kernels' division of rows among workgroups, restated on the
CPU: every grid size and weight must tile the row sequence exactly once.

The device computes, per workgroup (ssim_fused.hpp, fused_share, with
logical_block from ssim_device.hpp):
    lb = (b mod 8) * G/8 + b div 8            (G a multiple of 8; else lb = b)
    equal shares:    [lb * T / G, (lb + 1) * T / G)
    weighted shares: in each XCD's run of m = G/8 workgroups the first h = m/2
                     weigh first_w, the rest 100; share = the run's cumulative
                     weight scaled to T / 8 per run.
The host (ssim_api.hip) asks for weighted shares only for a grid of exactly two
workgroups per CU.  Integer division is floor division on non-negative values,
as in C.
"""
import pytest


def logical_block(b, G):
    return (b & 7) * (G >> 3) + (b >> 3) if G % 8 == 0 else b


def share(lb, G, total, first_w):
    if first_w == 100 or G % 8 != 0:
        return lb * total // G, (lb + 1) * total // G
    m = G // 8
    h = m // 2
    x, k = divmod(lb, m)

    def cum(kk):
        return first_w * min(kk, h) + 100 * max(kk - h, 0)

    per = cum(m)
    return (x * per + cum(k)) * total // (8 * per), (x * per + cum(k + 1)) * total // (8 * per)


GRIDS = [1, 2, 7, 8, 16, 24, 64, 250, 256, 264, 512, 520, 1024]
TOTALS = [0, 1, 7, 21, 1099, 27500, 854_560]


@pytest.mark.parametrize("first_w", [100, 135, 170, 190])
@pytest.mark.parametrize("G", GRIDS)
def test_shares_tile_the_sequence_once(G, first_w):
    lbs = [logical_block(b, G) for b in range(G)]
    assert sorted(lbs) == list(range(G))
    for total in TOTALS:
        spans = [share(lb, G, total, first_w) for lb in range(G)]
        assert spans[0][0] == 0 and spans[-1][1] == total
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a0 <= a1 == b0 <= b1


@pytest.mark.parametrize("first_w", [135, 170, 190])
def test_first_dispatched_workgroups_take_the_weighted_share(first_w):
    """With two workgroups per CU on 256 CUs, ids below G/2 (the first
    dispatched onto each CU) get first_w / 100 times the share of the others,
    to within the rounding of the integer division."""
    G = 512
    total = 854_560  # the 8 x 3 x 2160 x 3840 batch's sequence
    for b in range(G):
        lb = logical_block(b, G)
        v0, v1 = share(lb, G, total, first_w)
        m, h = G // 8, G // 16
        expect = total / 8 * (first_w if lb % m < h else 100) / (first_w * h + 100 * (m - h))
        assert abs((v1 - v0) - expect) <= 1
        assert (lb % m < h) == (b < G // 2)
