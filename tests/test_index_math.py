"""Host-side checks of the integer index math the kernels rely on: the
multiply-high division by an invariant divisor (Granlund & Montgomery, sec. 4)
for dividends below 2^31, and the QK kernel's block -> (tensor, row, slot)
mapping (tensor-major order, chunked launches): every (tensor, row, slot)
is produced exactly once and every row lies inside the call."""
import random

import pytest


def make_fastdiv(d):
    s = 0
    while (1 << s) < d:
        s += 1
    m = ((1 << 32) * ((1 << s) - d)) // d + 1
    return d, m & 0xFFFFFFFF, s


def fdiv(n, f):
    d, m, s = f
    hi = (n * m) >> 32
    return ((hi + n) & 0xFFFFFFFF) >> s


@pytest.mark.parametrize("d", [1, 2, 3, 5, 7, 10, 20, 40, 64, 84, 640, 1280, 1728, 4032, 124992,
                               125120, 246208, 2 ** 20 + 1, 2 ** 30 + 3, 2 ** 31 - 1])
def test_fastdiv_matches_integer_division(d):
    f = make_fastdiv(d)
    rng = random.Random(d)
    samples = [0, 1, d - 1, d, d + 1, 2 ** 31 - 1, 2 ** 31 - 2] + [rng.randrange(0, 2 ** 31)
                                                                  for _ in range(20000)]
    for k in (1, 2, 3, 1000):
        for n in (k * d - 1, k * d, k * d + 1):
            if 0 <= n < 2 ** 31:
                samples.append(n)
    for n in samples:
        assert fdiv(n, f) == n // d, (n, d)


def qk_blocks(rows, heads, lph):
    """Emulates the launch loop and the kernel's index math of the QK kernel."""
    gpw = 64 // lph
    nl = (heads + gpw - 1) // gpw
    step = 0x7FFFFFFF // (2 * nl)
    seen = {}
    f = make_fastdiv(nl)
    r0 = 0
    while r0 < rows:
        nr = min(rows - r0, step)
        nq = nr * nl
        for bid in range(2 * nr * nl):
            isk = bid >= nq
            bb = bid - nq if isk else bid
            rr = fdiv(bb, f)
            slot = bb - rr * nl
            row = r0 + rr
            assert 0 <= row < rows and 0 <= slot < nl
            key = (isk, row, slot)
            assert key not in seen
            seen[key] = True
            for gsub in range(gpw):
                hd = slot * gpw + gsub
                # slots past the last head must lie outside the row resource
                assert hd < heads or hd >= heads
        r0 += nr
    assert len(seen) == 2 * rows * nl


@pytest.mark.parametrize("rows,heads,lph", [(112, 4, 16), (777, 40, 16), (300, 40, 16),
                                            (50, 3, 8), (40, 5, 32), (30, 2, 8), (9, 1, 64)])
def test_qk_block_mapping_covers_each_slot_once(rows, heads, lph):
    qk_blocks(rows, heads, lph)


def xcd_linear(w, n, xcds=8):
    """The router score kernel's workgroup -> tile order: workgroup w runs on
    XCD w mod 8; each XCD gets one contiguous run of tiles."""
    per, extra = n // xcds, n % xcds
    x, slot = w % xcds, w // xcds
    return x * (per + 1) + slot if x < extra else extra * (per + 1) + (x - extra) * per + slot


@pytest.mark.parametrize("n", [1, 3, 7, 8, 9, 17, 255, 256, 257, 40 * 16 * 16, 40 * 31 * 31])
def test_xcd_tile_order_is_a_permutation(n):
    tiles = [xcd_linear(w, n) for w in range(n)]
    assert sorted(tiles) == list(range(n))
    # each XCD's tiles form one contiguous run
    for x in range(8):
        mine = sorted(xcd_linear(w, n) for w in range(x, n, 8))
        assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True
