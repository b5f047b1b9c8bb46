"""Pin of the fixed summation order of the step's row dot products.

The pages leave the order of the fp32 sums u = S'.k and o = S.q open; the
library fixes one so that the GPU and the oracle agree bit for bit (the
arithmetic contract of include/lsq.h): the columns in consecutive blocks of
32, a chain of fused multiply-adds from zero inside a block, then the block
sums added in adjacent pairs, level by level.

The expected values are computed here without the oracle, in exact
arithmetic: codes are integers in [-7, 7] and q lies in [0.5, 1) (24
significant bits), so every product and every partial sum of a block is a
multiple of 2^-24 below 2^11, exact in float64; rounding that exact value to
fp32 is the fp32 fused multiply-add.  The block sums are added with numpy's
fp32 addition (IEEE, round to nearest even).  With beta = 0, alpha = 1 and
unit scales, the step's output is exactly the dot product of each code row
with q.  The same data summed in two other plausible orders (one chain over
the row; the block sums added left to right) gives different fp32 results on
some rows, so the pin tells the orders apart.
"""
import numpy as np

import oracle
from oracle import OracleConfig

DK, DV = 128, 96


def _fma32(a, b, c):
    return np.float32(np.float64(a) * np.float64(b) + np.float64(c))


def _blocks(row, q, size=32):
    out = []
    for c0 in range(0, len(row), size):
        p = np.float32(0.0)
        for c in range(c0, min(c0 + size, len(row))):
            p = _fma32(row[c], q[c], p)
        out.append(p)
    return out


def blocked_pairwise(row, q):
    parts = _blocks(row, q)
    while len(parts) > 1:
        nxt = [np.float32(parts[i] + parts[i + 1]) for i in range(0, len(parts) - 1, 2)]
        if len(parts) % 2:
            nxt.append(parts[-1])
        parts = nxt
    return parts[0]


def one_chain(row, q):
    return _blocks(row, q, size=len(row))[0]


def blocked_left_to_right(row, q):
    parts = _blocks(row, q)
    s = parts[0]
    for p in parts[1:]:
        s = np.float32(s + p)
    return s


def _data(seed=5):
    rng = np.random.default_rng(seed)
    C = rng.integers(-7, 8, (DV, DK)).astype(np.int8)
    mant = rng.integers(0, 1 << 23, DK)
    q = ((1.0 + mant / float(1 << 23)) / 2.0 * rng.choice([-1.0, 1.0], DK)).astype(np.float32)
    return C, q


def _oracle_readout(C, q):
    cfg = OracleConfig(batch=1, heads=1, dk=DK, dv=DV, bits=4, group=32,
                       policy=oracle.POLICY_PERSISTENT, rounding=oracle.ROUND_RNE, delta=0,
                       decay=oracle.DECAY_SCALAR)
    st = oracle.zero_state(cfg)
    st.codes[0] = C
    st.scales[0] = 1.0
    k = np.zeros((1, DK), np.float32)
    v = np.zeros((1, DV), np.float32)
    o, _ = oracle.step(cfg, st, q.reshape(1, DK), k, v, np.ones(1, np.float32),
                       np.zeros(1, np.float32))
    return o[0]


def test_readout_follows_the_blocked_pairwise_order():
    C, q = _data()
    got = _oracle_readout(C, q)
    want = np.array([blocked_pairwise(C[r], q) for r in range(DV)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        np.argwhere(got != want)[:4].ravel().tolist()


def test_the_orders_differ_on_this_data():
    """The pin above discriminates: the other orders round differently on some rows."""
    C, q = _data()
    a = np.array([blocked_pairwise(C[r], q) for r in range(DV)], np.float32)
    b = np.array([one_chain(C[r], q) for r in range(DV)], np.float32)
    c = np.array([blocked_left_to_right(C[r], q) for r in range(DV)], np.float32)
    assert (a != b).sum() >= 5
    assert (a != c).sum() >= 5
