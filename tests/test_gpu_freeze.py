"""GPU parity of Freeze for anchor layouts that reach every path of the quantizing kernel's
slot-to-position lookup (HyQuant paper Alg. 4: every candidate position that is not an anchor
is quantized, in ascending order).

Slot s holds position s + c(s), c(s) the number of anchors a_i with a_i - i <= s.  The kernel
finds c for a tile's first slot with a 64-way search and counts the tile's other slots in a
window of the next 64 anchors; a tile whose slot range holds more anchors than that window
(a run of 64 or more consecutive anchor positions inside it) takes a per-slot binary search.
Layouts: long consecutive runs (the per-slot path), runs at the very start and end of the
candidate prefix, every other position, isolated anchors, and anchors exactly filling whole
tiles.  Bar: codes, fp16 scale and minimum, slot positions and the bf16 stores bit-exact
against the oracle's cache; one decode step within the decode bar."""
import numpy as np
import pytest

from tests.test_gpu_decode import Pair

pytestmark = pytest.mark.gpu


def _runs(lengths, P, rng, k):
    """k positions made of consecutive runs of the given lengths at random places, topped up
    with isolated positions."""
    taken = np.zeros(P, bool)
    for n in lengths:
        for _ in range(100):
            s = int(rng.integers(0, max(1, P - n)))
            if not taken[s:s + n].any():
                taken[s:s + n] = True
                break
    free = np.flatnonzero(~taken)
    extra = k - int(taken.sum())
    if extra > 0:
        taken[rng.choice(free, extra, replace=False)] = True
    A = np.flatnonzero(taken)
    return A[:k]


LAYOUTS = {
    # runs of 70, 100 and 200 consecutive anchors: tiles whose range holds more than 64
    "long_runs": lambda b, h, k, P: _runs([70, 100, 200], P, np.random.default_rng(11 + 7 * b + h), k),
    # the first k positions, then the last k positions of the candidate prefix
    "prefix": lambda b, h, k, P: np.arange(k),
    "suffix": lambda b, h, k, P: np.arange(P - k, P),
    # every other position from a random start
    "alternate": lambda b, h, k, P: (np.random.default_rng(5 + b).integers(0, P - 2 * k) + 2 * np.arange(k)),
    # 32-aligned blocks of 32 anchors (whole tiles of anchors between quantized tiles)
    "tile_blocks": lambda b, h, k, P: np.sort(np.concatenate(
        [64 * i + np.arange(32) for i in range(k // 32)] + [P - 1 - np.arange(k - 32 * (k // 32))])),
}


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("bits,bits_v", [(4, 4), (4, 2)])
def test_freeze_anchor_layouts(layout, bits, bits_v):
    print(f"[case] freeze anchor layout {layout} bits {bits}/{bits_v}", flush=True)
    p = Pair(9500 + len(layout), 2, 2, 4, 4200, n_steps=1, pct=10, bits=bits, bits_v=bits_v,
             anchor_layout=LAYOUTS[layout])
    p.codes_check()
    q = p.append()
    p.decode_check(q)


def test_freeze_more_anchors_than_one_window():
    """20% anchors in one run of 800 positions: many consecutive tiles take the per-slot path."""
    print("[case] freeze 800-anchor run", flush=True)
    p = Pair(9600, 1, 2, 4, 4200, n_steps=1, pct=20, anchor_layout=lambda b, h, k, P: _runs(
        [800], P, np.random.default_rng(3 + h), k))
    p.codes_check()
    q = p.append()
    p.decode_check(q)
