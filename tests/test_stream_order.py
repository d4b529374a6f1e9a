"""Pins the test-side definition of the weight-streaming layout (tests/_layout.py)."""

import numpy as np

from tests._layout import stream_order


def test_stream_order_matches_the_offset_formula():
    """The axis permutation against the offset formula in a plain loop (2 x 3 fragment blocks)."""
    rng = np.random.default_rng(3)
    wq = rng.integers(0, 256, size=(32, 384), dtype=np.uint8)
    got = stream_order(wq).ravel()
    Kb = 3
    for f in range(2):
        for kb in range(Kb):
            for h in range(2):
                for lane in range(64):
                    g, r = lane // 16, lane % 16
                    for b in range(16):
                        assert got[((f * Kb + kb) * 2 + h) * 1024 + 16 * lane + b] == \
                            wq[16 * f + r, 128 * kb + 32 * g + 16 * h + b]


def test_stream_order_is_a_permutation():
    wq = np.arange(64 * 256, dtype=np.int64).reshape(64, 256)
    got = stream_order(wq)
    assert sorted(got.ravel().tolist()) == list(range(64 * 256))
