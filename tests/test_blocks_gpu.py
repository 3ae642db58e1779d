"""Parity of copy_blocks / swap_blocks (HIP path through the C ABI) with the CPU
oracle: block copies are byte copies, so the pools must match bit for bit.

The pools hold random bytes (NaN patterns included).  Shapes cover blocks of
one 32 KiB slice, of several slices (128 KiB) and of less than one wave's
loads (the 128-byte scale blocks of an INT8 cache), and pool sets of 2 and 4
pools.  Swaps go to and from pinned host memory.  The last test runs the copy
on write of a shared, partly filled block, then the appends and the decode of
the two sequences, against the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle.attention as O
import oracle.blocks as OB
from gpu_run import max_err
from paged_kv_cache_274_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# name -> (n_blocks, [(dtype, block shape), ...])
POOL_SETS = {
    "bf16-kv-8x128": (40, [(torch.bfloat16, (8, 16, 128))] * 2),
    "bf16-kv-32x128": (12, [(torch.bfloat16, (32, 16, 128))] * 2),
    "f32-kv-2x64": (20, [(torch.float32, (2, 16, 64))] * 2),
    "int8-kv-2x64+scales": (24, [(torch.int8, (2, 16, 64))] * 2 + [(torch.float32, (2, 16))] * 2),
}


def _random_pools(n_blocks, spec, gen):
    """Pools of random bytes, viewed as their dtype (bit patterns of any kind)."""
    out = []
    for dt, shp in spec:
        nbytes = n_blocks * int(np.prod(shp)) * torch.empty((), dtype=dt).element_size()
        raw = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen)
        out.append(raw.view(dt).reshape((n_blocks,) + shp))
    return out


def _np(t: torch.Tensor) -> np.ndarray:
    """Bit-preserving NumPy view (bf16 as uint16)."""
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def _same_bits(got: torch.Tensor, ref: np.ndarray):
    assert _np(got.contiguous()).tobytes() == np.ascontiguousarray(ref).tobytes()


def _pairs_within(rng, n_blocks, n):
    """n pairs with distinct destinations and no block both read and written."""
    perm = rng.permutation(n_blocks)
    dst = perm[:n]
    src = rng.choice(perm[n:], size=n, replace=True)
    return np.stack([src, dst], axis=1).astype(np.int32)


@pytest.mark.parametrize("name", sorted(POOL_SETS))
def test_copy_blocks_matches_oracle(name):
    n_blocks, spec = POOL_SETS[name]
    gen = torch.Generator().manual_seed(sorted(POOL_SETS).index(name) + 100)
    rng = np.random.default_rng(11)
    pools = _random_pools(n_blocks, spec, gen)
    pairs = _pairs_within(rng, n_blocks, n_blocks // 3)
    dev = [p.to(DEV) for p in pools]
    ops.copy_blocks(dev, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    ref = OB.copy_blocks([_np(p) for p in pools], [_np(p) for p in pools], pairs)
    for g, r in zip(dev, ref):
        _same_bits(g.cpu(), r)


def test_copy_blocks_many_pairs_and_repeated_sources():
    """2000 pairs in one launch; one source copied to many destinations."""
    n_blocks = 4200
    gen = torch.Generator().manual_seed(3)
    pools = _random_pools(n_blocks, [(torch.bfloat16, (2, 16, 64))] * 2, gen)
    rng = np.random.default_rng(12)
    pairs = _pairs_within(rng, n_blocks, 2000)
    pairs[:50, 0] = pairs[0, 0]
    dev = [p.to(DEV) for p in pools]
    ops.copy_blocks(dev, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    ref = OB.copy_blocks([_np(p) for p in pools], [_np(p) for p in pools], pairs)
    for g, r in zip(dev, ref):
        _same_bits(g.cpu(), r)


def test_copy_blocks_skips_pairs_out_of_range():
    """Pairs naming a block outside the pool are not copied (the kernel's bounds
    check); the valid ones are."""
    n_blocks = 10
    gen = torch.Generator().manual_seed(4)
    pools = _random_pools(n_blocks, [(torch.bfloat16, (2, 16, 128))] * 2, gen)
    pairs = np.array([[0, 5], [-1, 6], [1, n_blocks], [n_blocks, 7], [2, -3], [3, 8]], np.int32)
    dev = [p.to(DEV) for p in pools]
    ops.copy_blocks(dev, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    ref = OB.copy_blocks([_np(p) for p in pools], [_np(p) for p in pools], [(0, 5), (3, 8)])
    for g, r in zip(dev, ref):
        _same_bits(g.cpu(), r)


def test_copy_blocks_empty_mapping_changes_nothing():
    gen = torch.Generator().manual_seed(5)
    pools = _random_pools(6, [(torch.bfloat16, (2, 16, 64))] * 2, gen)
    dev = [p.to(DEV) for p in pools]
    ops.copy_blocks(dev, torch.zeros((0, 2), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    for g, p in zip(dev, pools):
        assert torch.equal(g.cpu().view(torch.int16), p.view(torch.int16))


@pytest.mark.parametrize("name", ["bf16-kv-8x128", "int8-kv-2x64+scales", "bf16-kv-32x128"])
def test_swap_out_and_in_through_pinned_host_pools(name):
    """Swap a sequence's blocks out to a pinned host pool set, clobber the device
    blocks, swap them back in to other device blocks; both steps match the
    oracle bit for bit."""
    n_blocks, spec = POOL_SETS[name]
    gen = torch.Generator().manual_seed(6)
    pools = _random_pools(n_blocks, spec, gen)
    n_host = 7
    host = [torch.zeros((n_host,) + p.shape[1:], dtype=p.dtype).pin_memory() for p in pools]
    rng = np.random.default_rng(13)
    out_pairs = np.stack([rng.choice(n_blocks, 5, replace=False),
                          rng.choice(n_host, 5, replace=False)], axis=1).astype(np.int32)
    dev = [p.to(DEV) for p in pools]
    ops.swap_blocks(dev, host, torch.from_numpy(out_pairs).to(DEV))
    torch.cuda.synchronize()
    host_ref = OB.copy_blocks([_np(p) for p in pools], [_np(h) for h in host], out_pairs)
    for h, r in zip(host, host_ref):
        _same_bits(h, r)

    clobber = _random_pools(n_blocks, spec, gen)
    dev = [c.to(DEV) for c in clobber]
    in_pairs = np.stack([out_pairs[:, 1], rng.choice(n_blocks, 5, replace=False)],
                        axis=1).astype(np.int32)
    pinned_pairs = torch.from_numpy(in_pairs).pin_memory()   # the mapping may live on the host
    ops.swap_blocks(host, dev, pinned_pairs)
    torch.cuda.synchronize()
    dev_ref = OB.copy_blocks([_np(h) for h in host], [_np(c) for c in clobber], in_pairs)
    for g, r in zip(dev, dev_ref):
        _same_bits(g.cpu(), r)
    for g, p in zip(dev, pools):   # the round trip brought back the original blocks
        for (s, _), (_, d) in zip(out_pairs, in_pairs):
            assert _np(g[int(d)].cpu()).tobytes() == _np(p[int(s)]).tobytes()


def test_swap_rejects_pageable_host_memory():
    """A pool the GPU cannot reach is refused before anything is enqueued."""
    dev = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    pageable = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device=DEV)
    L = ops.lib()
    src = (ctypes.c_void_p * 1)(dev.data_ptr())
    dst = (ctypes.c_void_p * 1)(pageable.data_ptr())
    bb = (ctypes.c_int64 * 1)(2 * 16 * 64 * 2)
    assert L.swap_blocks(src, dst, bb, 1, 4, 4, pairs.data_ptr(), 1, None) == 1
    torch.cuda.synchronize()


def test_copy_on_write_then_append_and_decode():
    """Two sequences share every block of a 40-token context (the last block
    holds 8 tokens).  Before each appends its own next token, the second one
    copies the shared last block to a free block and points its table there.
    Pools must match the oracle bit for bit and both decodes within 2e-2; the
    shared full blocks stay shared."""
    h_q, h_kv, d, n_blocks, L = 8, 2, 128, 12, 40
    rng = np.random.default_rng(14)
    draw = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(
        torch.bfloat16)
    kc, vc = draw(n_blocks, h_kv, 16, d), draw(n_blocks, h_kv, 16, d)
    shared = [7, 2, 10]
    cow_to = 4
    tables = torch.tensor([shared, [7, 2, cow_to]], dtype=torch.int32)
    k_new, v_new, q = draw(2, h_kv, d), draw(2, h_kv, d), draw(2, h_q, d)
    slots = torch.tensor([10 * 16 + 8, cow_to * 16 + 8], dtype=torch.int64)
    lens = torch.tensor([L + 1, L + 1], dtype=torch.int32)
    scale = 1.0 / np.sqrt(d)

    kd, vd = kc.to(DEV), vc.to(DEV)
    ops.copy_blocks([kd, vd], torch.tensor([[10, cow_to]], dtype=torch.int32, device=DEV))
    ops.kv_append(k_new.to(DEV), v_new.to(DEV), slots.to(DEV), kd, vd)
    out = ops.paged_decode_attention(q.to(DEV), kd, vd, tables.to(DEV), lens.to(DEV), L + 1,
                                     scale=scale)
    torch.cuda.synchronize()

    f64 = lambda t: t.to(torch.float64).numpy()
    k_ref, v_ref = OB.copy_blocks([f64(kc), f64(vc)], [f64(kc), f64(vc)], [(10, cow_to)])
    k_ref, v_ref = O.kv_append(f64(k_new), f64(v_new), slots.numpy(), k_ref, v_ref)
    ref = O.decode(f64(q), k_ref, v_ref, tables.numpy(), lens.numpy(), scale)
    assert np.array_equal(f64(kd.cpu()), k_ref) and np.array_equal(f64(vd.cpu()), v_ref)
    err = max_err(out.cpu(), ref)
    print(f"copy-on-write decode max|err| = {err:.3e}")
    assert err <= 2e-2
    # the two sequences now differ only in their newest token
    assert not np.allclose(ref[0], ref[1])


def test_binding_rejects_malformed_pool_sets():
    """Argument errors of the bindings are raised before any launch."""
    a = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((9, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        ops.copy_blocks([a, b], pairs)                          # block counts differ
    with pytest.raises(ValueError):
        ops.copy_blocks([a], pairs.to(torch.int64))             # pairs must be int32
    with pytest.raises(ValueError):
        ops.copy_blocks([a], pairs.reshape(2))                  # pairs must be [n, 2]
    with pytest.raises(ValueError):
        ops.copy_blocks([a] * 9, pairs)                         # at most 8 pools
    with pytest.raises(ValueError):
        ops.copy_blocks([a.cpu()], pairs)                       # pageable host pool
    h = torch.zeros((4, 2, 16, 32), dtype=torch.bfloat16).pin_memory()
    with pytest.raises(ValueError):
        ops.swap_blocks([a], [h], pairs)                        # block shapes differ
    with pytest.raises(ValueError):
        ops.swap_blocks([a, a], [b], pairs)                     # set sizes differ
    with pytest.raises(ops.PkvError):
        ops.swap_blocks([a], [a], pairs)                        # a pool onto itself
    torch.cuda.synchronize()
