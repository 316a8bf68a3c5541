"""The error metrics the parity tests use: the all-blocks-at-once forms agree
with the block-by-block definition (CPU only)."""

import numpy as np

from helpers import block_rel_err, state_rel_err


def _loop_block(x, ref, off):
    worst = 0.0
    for b in range(len(off) - 1):
        for h in range(ref.shape[1]):
            sl = slice(off[b], off[b + 1])
            d = np.max(np.abs(x[sl, h] - ref[sl, h]))
            den = np.max(np.abs(ref[sl, h]))
            worst = max(worst, d / den if den > 0 else d)
    return worst


def test_block_rel_err_vectorised_matches_definition():
    rng = np.random.default_rng(0)
    off = np.array([0, 5, 6, 40, 64], np.int32)
    ref = rng.standard_normal((64, 3, 8))
    x = ref + 1e-3 * rng.standard_normal(ref.shape)
    x[37, 2, 5] += 0.5  # one planted outlier in block (2, 2)
    ref[5] = 0.0        # a block whose reference is all zero (absolute error)
    x[5] = 1e-7
    all_units = [(b, h) for b in range(4) for h in range(3)]
    want = _loop_block(x, ref, off)
    assert block_rel_err(x, ref, off) == want
    assert block_rel_err(x, ref, off, all_units) == want
    assert block_rel_err(x, ref, off) > 0.1


def test_state_rel_err_vectorised_matches_definition():
    rng = np.random.default_rng(1)
    slot = np.array([3, 0, 2], np.int32)
    ref = rng.standard_normal((3, 2, 4, 4))
    pool = np.zeros((4, 2, 4, 4), np.float32)
    pool[slot] = ref + 1e-4
    pool[2, 1, 3, 3] += 1.0
    units = [(b, h) for b in range(3) for h in range(2)]
    fast = state_rel_err(pool, ref, slot, units)
    slow = max(state_rel_err(pool, ref, slot, [u]) for u in units)
    assert fast == slow and fast > 0.1
