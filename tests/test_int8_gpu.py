"""Parity of the INT8 KV cache (HIP path through the C ABI) with the CPU oracle.

kv_append_int8 must match the oracle's codes and scales bit for bit (the codes
are integers decided in float32 by both sides, with the same division and the
same rounding).  Decode over the INT8 cache must be within 2e-2 of the float64
oracle's attention over the dequantised cache, like the bf16 decode: the
queries are bf16 and each softmax weight times its V scale is rounded to bf16
once.  Scales of unused slots are NaN, so an unmasked read shows up.
"""
import numpy as np
import pytest
import torch

import oracle.quant as Q
import pins
from gpu_run import bits, max_err
from paged_kv_cache_274_amd import ops
from paged_kv_cache_274_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


def _f32(t: torch.Tensor) -> np.ndarray:
    return t.float().numpy()


def _append(w, pools, slots=None):
    """GPU and oracle append of the workload's new tokens; returns both pool sets."""
    slots = w.slot_mapping if slots is None else slots
    g = [t.to(DEV) for t in (pools.k_codes, pools.v_codes, pools.k_scales, pools.v_scales)]
    ops.kv_append_int8(w.k_new.to(DEV), w.v_new.to(DEV), slots.to(DEV), *g)
    torch.cuda.synchronize()
    got = [t.cpu() for t in g]
    ref = Q.kv_append_int8(_f32(w.k_new), _f32(w.v_new), slots.numpy(), pools.k_codes.numpy(),
                           pools.v_codes.numpy(), pools.k_scales.numpy(), pools.v_scales.numpy())
    return got, ref


def _check_append_exact(got, ref):
    for g, r in zip(got, ref):
        r = torch.from_numpy(np.ascontiguousarray(r))
        if g.dtype == torch.int8:
            assert torch.equal(g, r)
        else:
            assert torch.equal(torch.isnan(g), torch.isnan(r))
            assert torch.equal(g.view(torch.int32), r.view(torch.int32))


def _decode(w, pools_dev, splits=0, lens=None):
    lens = w.dec_context_lens if lens is None else lens
    out = ops.paged_decode_attention_int8(
        w.dec_q.to(DEV), *pools_dev, w.dec_block_tables.to(DEV), lens.to(DEV),
        max(int(lens.max()), 0) if len(lens) else 0, scale=w.scale, num_splits=splits)
    return out.cpu()


def _oracle_decode(w, ref, lens=None):
    lens = w.dec_context_lens if lens is None else lens
    return Q.decode_int8(pins.np64(w.dec_q), *ref, w.dec_block_tables.numpy(), lens.numpy(),
                         w.scale)


# ----------------------------------------------------------------------------- append

@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("d,h_kv", [(64, 2), (128, 8), (128, 1), (64, 4)])
def test_append_int8_bit_exact(src, d, h_kv):
    rng = np.random.default_rng(300 + d + h_kv)
    lens = [1, 16, 17, 40, 100, 33, 64]
    w = W.build("app8", rng, dtype=src, h_q=h_kv * 2, h_kv=h_kv, d=d, decode_lens=lens,
                free_frac=0.3, poison=True)
    # rows that decide the rounding rule: max 127 then exact ties; an all-zero
    # row (the 1e-8 floor); a huge and a tiny row
    k_new = w.k_new.clone()
    k_new[0, 0, :6] = torch.tensor([127.0, 1.5, 2.5, -0.5, -3.5, 126.5])
    k_new[0, 0, 6:] = 0.0
    k_new[1, 0] = 0.0
    k_new[2, 0] *= 3000.0
    k_new[3, 0] *= 1e-6
    w.k_new = k_new
    slots = w.slot_mapping.clone()
    slots[4] = -1  # padding: nothing written for that token
    pools = W.int8_pools(w, seed=7, poison=True)
    got, ref = _append(w, pools, slots)
    _check_append_exact(got, ref)


# ----------------------------------------------------------------------------- decode

DECODE_GRID8 = [
    # d, h_q, h_kv
    (64, 4, 4), (64, 14, 2), (128, 32, 8), (128, 6, 2), (64, 40, 8), (128, 16, 1), (64, 12, 4),
    (128, 8, 1),
]


@pytest.mark.parametrize("d,h_q,h_kv", DECODE_GRID8)
@pytest.mark.parametrize("splits", [0, 1, 13, 300])
def test_decode_int8_grid(d, h_q, h_kv, splits):
    rng = np.random.default_rng(2000 + d + h_q * 7 + h_kv)
    lens = [1, 15, 16, 17, 63, 64, 65, 200, 333, 700]
    w = W.build("grid8", rng, dtype="bf16", h_q=h_q, h_kv=h_kv, d=d, decode_lens=lens,
                free_frac=0.2, max_blocks_per_seq=50, poison=True)
    pools = W.int8_pools(w, seed=11, poison=True)
    got, ref = _append(w, pools)
    _check_append_exact(got, ref)
    out = _decode(w, [t.to(DEV) for t in got], splits)
    err = max_err(out, _oracle_decode(w, ref))
    assert err <= TOL, f"int8 decode max|err| {err}"


@pytest.mark.parametrize("d,h_q,h_kv", [(64, 14, 2), (128, 16, 1)])
def test_decode_int8_large_batch_keeps_wide_chunks(d, h_q, h_kv):
    """Large batches keep chunks of up to 8 heads per wave (the grid above is
    small enough for 4-head chunks); the INT8 decode matches the oracle there
    too."""
    rng = np.random.default_rng(4000 + h_q + d)
    lens = [int(x) for x in rng.integers(1000, 4096, size=64, endpoint=True)]
    g = h_q // h_kv
    assert 64 * h_kv * -(-g // 4) * -(-max(lens) // 16) > 2048 * 16   # above the small-line rule
    w = W.build("wide8", rng, dtype="bf16", h_q=h_q, h_kv=h_kv, d=d, decode_lens=lens,
                free_frac=0.05, poison=True)
    pools = W.int8_pools(w, seed=12, poison=True)
    got, ref = _append(w, pools)
    _check_append_exact(got, ref)
    out = _decode(w, [t.to(DEV) for t in got])
    err = max_err(out, _oracle_decode(w, ref))
    assert err <= TOL, f"int8 decode max|err| {err}"


@pytest.mark.parametrize("k", [3, 5])
def test_decode_int8_configs(k):
    """The decode legs of configs 3 and 5 with an INT8 cache, full size."""
    w = W.config(k, poison=True)
    pools = W.int8_pools(w, seed=100 + k, poison=True)
    got, ref = _append(w, pools)
    _check_append_exact(got, ref)
    out = _decode(w, [t.to(DEV) for t in got])
    err = max_err(out, _oracle_decode(w, ref))
    print(f"config {k} int8: decode max|err| = {err:.3g}")
    assert err <= TOL


def test_decode_int8_zero_length_and_split_agreement():
    rng = np.random.default_rng(12)
    w = W.build("z8", rng, dtype="bf16", h_q=8, h_kv=2, d=128, decode_lens=[1, 40, 1, 2000],
                free_frac=0.5, poison=True)
    pools = W.int8_pools(w, seed=13, poison=True)
    got, ref = _append(w, pools)
    dev = [t.to(DEV) for t in got]
    lens0 = torch.tensor([0, 40, 0, 2000], dtype=torch.int32)
    # also with one range, where no second pass runs: the first pass zero-fills
    for splits in (0, 1):
        out = _decode(w, dev, splits, lens0)
        assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[2]) == 0
        assert max_err(out, _oracle_decode(w, ref, lens0)) <= TOL
    a = _decode(w, dev, 1)
    for splits in (2, 7, 64, 0):
        assert max_err(_decode(w, dev, splits), a.double().numpy()) <= TOL
    # one wave per sequence reduces in a fixed order: repeatable bit for bit
    assert torch.equal(bits(a), bits(_decode(w, dev, 1)))


@pytest.mark.parametrize("q_mag", [1e-8, 1e-6, 1.0, 3e5])
def test_decode_int8_query_magnitudes(q_mag):
    """The INT8 decode forms K products in f16 from q scaled by a power of two
    per piece; queries far outside f16's range (3e5, or 1e-6 and 1e-8 where f16
    would flush them) must still match the oracle.  The softmax scale is divided
    by the magnitude, so the scores keep the spread of |q| ~ 1 instead of
    collapsing to a one-hot (3e5) or uniform (1e-8) softmax that would hide
    score errors."""
    rng = np.random.default_rng(4100)
    w = W.build("qmag", rng, dtype="bf16", h_q=16, h_kv=4, d=128,
                decode_lens=[1, 17, 300, 1000, 2500], free_frac=0.2, poison=True)
    w.dec_q = (w.dec_q.float() * q_mag).to(torch.bfloat16)
    w.scale = float(np.float32(w.scale / q_mag))  # the kernel takes a float32 scale
    pools = W.int8_pools(w, seed=13, poison=True)
    got, ref = _append(w, pools)
    _check_append_exact(got, ref)
    for splits in (0, 7):
        out = _decode(w, [t.to(DEV) for t in got], splits)
        err = max_err(out, _oracle_decode(w, ref))
        print(f"|q| ~ {q_mag:g}, splits {splits}: max|err| {err:.3e}")
        assert err <= TOL, f"int8 decode max|err| {err} at |q| ~ {q_mag}"


def test_decode_int8_offset_queries():
    """Queries 50 + N(0, 1): every component has the same sign, so the biased
    f16 products q . (1152 + c) and the subtracted 1152 * sum(q) nearly cancel;
    the scores must still match the oracle's.  The scale is divided by 50 to
    keep the softmax from collapsing to one key."""
    rng = np.random.default_rng(4101)
    w = W.build("qoff", rng, dtype="bf16", h_q=16, h_kv=4, d=128,
                decode_lens=[1, 17, 300, 1000, 2500], free_frac=0.2, poison=True)
    w.dec_q = (w.dec_q.float() + 50.0).to(torch.bfloat16)
    w.scale = float(np.float32(w.scale / 50.0))
    pools = W.int8_pools(w, seed=14, poison=True)
    got, ref = _append(w, pools)
    _check_append_exact(got, ref)
    for splits in (0, 7):
        out = _decode(w, [t.to(DEV) for t in got], splits)
        err = max_err(out, _oracle_decode(w, ref))
        print(f"q = 50 + N(0,1), splits {splits}: max|err| {err:.3e}")
        assert err <= TOL, f"int8 decode max|err| {err} with offset queries"


def _term_err(got: torch.Tensor, ref: np.ndarray, ref_abs: np.ndarray) -> float:
    """Largest error over max(1, attention over |V|): each output is a weighted
    sum whose terms can cancel, and rounding each weight to bf16 errs by up to
    2^-9 of that term, so the error scales with the sum of the terms'
    magnitudes, not with the (possibly cancelled) result."""
    g = got.to(torch.float64).numpy()
    assert not np.isnan(g).any(), "NaN in GPU output"
    return float((np.abs(g - ref) / np.maximum(1.0, ref_abs)).max()) if g.size else 0.0


@pytest.mark.parametrize("wide_k", [False, True])
def test_int8_wide_scales(wide_k):
    """V scales drawn log-uniformly over [1e-4, 10] (and K scales too with
    wide_k), unused slots' scales NaN: decode and prefill over the cache.  The
    outputs reach a few hundred, and with random-sign codes a sum of large
    terms can cancel to near zero, so the bound is 2e-2 times max(1, the
    oracle's attention over |V|): in decode and prefill alike each softmax
    weight times its token's V scale is rounded to bf16 once, an error of at
    most 2^-9 of its term."""
    rng = np.random.default_rng(4200 + wide_k)
    w = W.build("wide", rng, dtype="bf16", h_q=32, h_kv=8, d=128,
                decode_lens=[1, 17, 300, 1000, 2500], prefill=[(700, 300), (90, 33)],
                free_frac=0.2, poison=True)
    pools = W.int8_pools(w, seed=15, poison=True)

    def wide(t: torch.Tensor) -> torch.Tensor:
        x = t.numpy().copy()
        nan = np.isnan(x)
        x = (10.0 ** rng.uniform(-4.0, 1.0, size=x.shape)).astype(np.float32)
        x[nan] = np.nan
        return torch.from_numpy(x)

    pools.v_scales = wide(pools.v_scales)
    if wide_k:
        pools.k_scales = wide(pools.k_scales)
    got, ref = _append(w, pools)
    _check_append_exact(got, ref)
    dev = [t.to(DEV) for t in got]
    kq, vq, ks, vs = ref
    ref_abs = (kq, np.abs(vq), ks, vs)
    o_dec, a_dec = _oracle_decode(w, ref), _oracle_decode(w, ref_abs)
    e_dec = max(_term_err(_decode(w, dev, splits), o_dec, a_dec) for splits in (0, 7))
    e_pre = _term_err(_prefill(w, dev), _oracle_prefill(w, ref), _oracle_prefill(w, ref_abs))
    print(f"wide scales (K too: {wide_k}): decode {e_dec:.3e}, prefill {e_pre:.3e} "
          "(over attention of |V|)")
    assert e_dec <= 2e-2 and e_pre <= 2e-2


# ----------------------------------------------------------------------------- prefill

def _prefill(w, pools_dev):
    out = ops.paged_prefill_attention_int8(
        w.pre_q.to(DEV), w.pre_cu_seqlens.to(DEV), *pools_dev, w.pre_block_tables.to(DEV),
        w.pre_context_lens.to(DEV), w.pre_max_q_len, scale=w.scale)
    return out.cpu()


def _oracle_prefill(w, ref):
    return Q.prefill_int8(pins.np64(w.pre_q), w.pre_cu_seqlens.numpy(), *ref,
                          w.pre_block_tables.numpy(), w.pre_context_lens.numpy(), w.scale)


PREFILL8 = [
    # name, d, h_q, h_kv, [(context, n_new)]
    ("config-5 prompts", 64, 14, 2, [(512, 512)] * 4),
    ("chunks cut mid-tile", 128, 32, 8, [(1500, 300), (700, 700), (90, 33), (17, 16)]),
    ("gqa 8, ragged", 128, 8, 1, [(150, 150), (260, 130), (1, 1)]),
    ("d 64, long chunk", 64, 16, 2, [(2100, 1000), (48, 48)]),
]


@pytest.mark.parametrize("name,d,h_q,h_kv,seqs", PREFILL8, ids=[p[0] for p in PREFILL8])
def test_prefill_int8_matches_oracle(name, d, h_q, h_kv, seqs):
    """Causal chunked prefill over the INT8 cache (appended this step by
    kv_append_int8; unused slots' scales NaN) against the oracle's prefill over
    the dequantised cache."""
    rng = np.random.default_rng(400 + d + h_q + len(seqs))
    w = W.build("pre8", rng, dtype="bf16", h_q=h_q, h_kv=h_kv, d=d, prefill=seqs,
                free_frac=0.2, poison=True)
    p8 = W.int8_pools(w, seed=41, poison=True)
    got, ref = _append(w, p8)
    _check_append_exact(got, ref)
    out = _prefill(w, [t.to(DEV) for t in got])
    err = max_err(out, _oracle_prefill(w, ref))
    print(f"int8 prefill {name}: max|err| {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("n_s", [2, 4, 5])
def test_verify_over_int8_cache(n_s):
    """Multi-token decode (the n_s newest tokens of each sequence, decode-shaped
    contexts) over the INT8 cache; the last row equals the one-token INT8
    decode of the same context."""
    rng = np.random.default_rng(450 + n_s)
    lens = [int(x) for x in rng.integers(128, 4096, size=12, endpoint=True)] + [n_s, 16 + n_s]
    w = W.build("verify8", rng, dtype="bf16", h_q=32, h_kv=8, d=128,
                prefill=[(L, n_s) for L in lens], free_frac=0.1, poison=True)
    p8 = W.int8_pools(w, seed=42, poison=True)
    got, ref = _append(w, p8)
    dev = [t.to(DEV) for t in got]
    out = _prefill(w, dev)
    err = max_err(out, _oracle_prefill(w, ref))
    last = w.pre_cu_seqlens[1:].long() - 1
    one = ops.paged_decode_attention_int8(w.pre_q[last].to(DEV), *dev,
                                          w.pre_block_tables.to(DEV),
                                          w.pre_context_lens.to(DEV), max(lens),
                                          scale=w.scale).cpu()
    print(f"int8 verify n_s={n_s}: max|err| {err:.3e}")
    assert err <= TOL
    assert max_err(out[last], one.double().numpy()) <= TOL


@pytest.mark.parametrize("S", [40, 300])
def test_prefill_int8_beyond_one_round(S):
    """Grids of more workgroups than the chip holds: sequence planes taken
    longest context first (S <= 256) or in index order (S = 300)."""
    rng = np.random.default_rng(470 + S)
    lens = [max(3, int(x)) for x in rng.integers(3, 1500, size=S)]
    w = W.build("many8", rng, dtype="bf16", h_q=16, h_kv=8, d=128,
                prefill=[(L, 3) for L in lens], free_frac=0.05, poison=True)
    p8 = W.int8_pools(w, seed=43, poison=True)
    got, ref = _append(w, p8)
    out = _prefill(w, [t.to(DEV) for t in got])
    err = max_err(out, _oracle_prefill(w, ref))
    print(f"int8 prefill, {S} sequences: max|err| {err:.3e}")
    assert err <= TOL
