"""Pins of the block-copy oracle (no GPU).

The operation has a plain definition (block dst of each destination pool
becomes a bit copy of block src), so the oracle is that definition; it is
pinned here by an element-by-element walk over the flat byte images of the
pools (which fixes the block axis and the pool pairing), by round trips, and by
its preconditions."""
import numpy as np
import pytest

import oracle.blocks as B


def _pools(rng, n_blocks, dtypes=((np.uint16, (2, 16, 8)), (np.int8, (2, 16, 8)),
                                  (np.float32, (2, 16)))):
    return [rng.integers(0, 2**15, size=(n_blocks,) + shp).astype(dt) for dt, shp in dtypes]


def _byte_walk(src_pools, dst_pools, pairs):
    """Byte by byte over flat images: block b of a pool with block size S bytes
    is bytes b*S .. b*S + S - 1."""
    out = []
    for s, d in zip(src_pools, dst_pools):
        sb = bytearray(s.tobytes())
        db = bytearray(d.tobytes())
        S = s.nbytes // s.shape[0]
        for src, dst in pairs:
            for i in range(S):
                db[dst * S + i] = sb[src * S + i]
        out.append(bytes(db))
    return out


def test_copy_matches_a_byte_walk():
    rng = np.random.default_rng(1)
    pools = _pools(rng, 9)
    pairs = [(0, 5), (3, 8), (2, 6)]
    got = B.copy_blocks(pools, pools, pairs)
    want = _byte_walk(pools, pools, pairs)
    for g, w in zip(got, want):
        assert g.tobytes() == w


def test_swap_out_and_in_round_trip():
    rng = np.random.default_rng(2)
    dev = _pools(rng, 12)
    host = [np.zeros((5,) + p.shape[1:], p.dtype) for p in dev]
    out_pairs = [(7, 0), (2, 1), (11, 4)]
    host2 = B.copy_blocks(dev, host, out_pairs)
    want = _byte_walk(dev, host, out_pairs)
    for g, w in zip(host2, want):
        assert g.tobytes() == w
    back = B.copy_blocks(host2, [np.zeros_like(p) for p in dev], [(0, 3), (1, 9), (4, 10)])
    for p, b in zip(dev, back):
        assert np.array_equal(b[3], p[7]) and np.array_equal(b[9], p[2])
        assert np.array_equal(b[10], p[11])


def test_only_destinations_change():
    rng = np.random.default_rng(3)
    pools = _pools(rng, 10)
    got = B.copy_blocks(pools, pools, [(1, 4), (9, 0)])
    for g, p in zip(got, pools):
        for b in range(10):
            if b not in (4, 0):
                assert np.array_equal(g[b], p[b])


def test_preconditions():
    rng = np.random.default_rng(4)
    pools = _pools(rng, 6)
    with pytest.raises(ValueError):
        B.copy_blocks(pools, pools, [(0, 6)])
    with pytest.raises(ValueError):
        B.copy_blocks(pools, pools, [(0, 2), (1, 2)])
    with pytest.raises(ValueError):
        B.copy_blocks(pools, pools, [(0, 2), (2, 3)])  # block 2 read and written
    other = [np.zeros_like(p) for p in pools]
    B.copy_blocks(pools, other, [(0, 2), (2, 3)])      # fine across pool sets


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_mutation_wrong_axis_is_caught():
    """A copy along the wrong axis (the head axis instead of the block axis)."""
    def bad(src_pools, dst_pools, pairs):
        out = [np.array(d, copy=True) for d in dst_pools]
        for s, d in pairs:
            for sp, o in zip(src_pools, out):
                if o.ndim > 1 and o.shape[1] > max(s, d):
                    o[:, d] = sp[:, s]
        return out
    rng = np.random.default_rng(5)
    pools = _pools(rng, 9)

    def check(copy):
        pairs = [(0, 1)]
        for g, w in zip(copy(pools, pools, pairs), _byte_walk(pools, pools, pairs)):
            assert g.tobytes() == w
    check(B.copy_blocks)
    assert _fails(lambda: check(bad))
