"""Pins of the INT8 KV-cache oracle (no GPU).

The pages give the quantiser as a formula, s = max|x| / 127, x_q = round(x / s),
x_hat = s * x_q (LLM Inference Server page, "Required Mathematical Concepts"),
and print a reference INT8 layer whose details (float32 values, the 1e-8 floor
on the maximum, PyTorch's round-half-to-even) the oracle follows.  They print no
worked numeric example, so the oracle is pinned by:

* hand-derived rows whose quotients x / s are exact, including ties, so that the
  rounding rule is decided by the example (worked out below, not computed by
  the code under test);
* properties the formula implies: the largest |x| maps to +-127, the error
  |x - s x_q| is at most s / 2, the codes are monotone in x, a power-of-two
  rescaling of a row leaves its codes unchanged, negation negates them, and
  each (token, head) row is scaled on its own;
* a brute force in exact rational arithmetic, with IEEE float32 rounding done
  explicitly, on random rows;
* for attention over the cache: exactly representable caches (where int8
  decode must equal plain decode), a pure-Python brute force over s * x_q, and
  physical-block permutation;
* mutation tests that plant one plausible mistake at a time and require a pin
  to fail.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle.attention as A
import oracle.quant as Q
import pins


# ----------------------------------------------------------------------------- worked rows

# Row with max |x| = 127, so s = 127 / 127 = 1 exactly and x / s = x:
#   127 -> 127; 1.5 -> 2 (tie, even); 2.5 -> 2 (tie, even); -0.5 -> -0 (tie, even);
#   -3.5 -> -4 (tie, even); 0.49999997 -> 0; -127 -> -127.
ROW_S1 = [127.0, 1.5, 2.5, -0.5, -3.5, 0.49999997, -127.0]
CODES_S1 = [127, 2, 2, 0, -4, 0, -127]
# Row with max |x| = 254, so s = 2 exactly: x / s = 127, 1.5, 2.5, -0.5, -3.5.
ROW_S2 = [254.0, 3.0, 5.0, -1.0, -7.0]
CODES_S2 = [127, 2, 2, 0, -4]


def _check_worked(quantize_row):
    c, s = quantize_row(np.array(ROW_S1, dtype=np.float32))
    assert s == np.float32(1.0) and c.tolist() == CODES_S1
    c, s = quantize_row(np.array(ROW_S2, dtype=np.float32))
    assert s == np.float32(2.0) and c.tolist() == CODES_S2


def test_worked_rows():
    _check_worked(Q.quantize_row)


def test_zero_row_gets_zero_codes_and_the_floor_scale():
    c, s = Q.quantize_row(np.zeros(16, dtype=np.float32))
    assert c.tolist() == [0] * 16
    assert s == np.float32(np.float32(1e-8) / np.float32(127.0))
    assert np.array_equal(Q.dequantize(c[None], np.array([s])), np.zeros((1, 16)))


# ----------------------------------------------------------------------------- properties

def _rows(seed, n=200, d=64):
    rng = np.random.default_rng(seed)
    mags = 10.0 ** rng.uniform(-6, 4, size=(n, 1))
    rows = (rng.standard_normal((n, d)) * mags).astype(np.float32)
    rows[::7, 3] = 0.0
    return rows


def _check_properties(quantize_row, seed=1):
    for x in _rows(seed):
        c, s = quantize_row(x)
        assert c.dtype == np.int8 and np.abs(c.astype(int)).max() <= 127
        i = int(np.argmax(np.abs(x)))
        assert abs(int(c[i])) == 127 and np.sign(c[i]) == np.sign(x[i])
        # |x - s x_q| <= s / 2 (plus the float32 rounding of s and of x / s)
        err = np.abs(x.astype(np.float64) - float(s) * c.astype(np.float64))
        assert err.max() <= 0.5 * float(s) * (1 + 1e-6) + 1e-45
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(c[order].astype(int)) >= 0)
        c2, s2 = quantize_row(x * np.float32(4.0))
        assert np.array_equal(c2, c) and s2 == np.float32(4.0) * s
        c3, s3 = quantize_row(-x)
        assert np.array_equal(c3.astype(int), -c.astype(int)) and s3 == s


def test_properties():
    _check_properties(Q.quantize_row)


def _check_per_head_rows(kv_append_int8):
    """Two KV heads of very different magnitude: each head row is scaled on its own."""
    d = 8
    k = np.zeros((1, 2, d), dtype=np.float32)
    k[0, 0] = np.linspace(-1, 1, d)
    k[0, 1] = np.linspace(-1000, 500, d)
    kq, vq, ks, vs = kv_append_int8(k, k, np.array([5]), np.zeros((1, 2, 16, d), np.int8),
                                    np.zeros((1, 2, 16, d), np.int8),
                                    np.zeros((1, 2, 16), np.float32), np.zeros((1, 2, 16), np.float32))
    assert ks[0, 0, 5] == np.float32(np.float32(1.0) / np.float32(127.0))
    assert ks[0, 1, 5] == np.float32(np.float32(1000.0) / np.float32(127.0))
    assert abs(int(kq[0, 0, 5, 0])) == 127 and abs(int(kq[0, 1, 5, 0])) == 127


def test_each_token_head_row_has_its_own_scale():
    _check_per_head_rows(Q.kv_append_int8)


# ----------------------------------------------------------------------------- exact brute force

def _round_f32(r: Fraction) -> Fraction:
    """r rounded to the nearest float32 (ties to even), normal range only."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (e - 23)  # spacing of float32 numbers in [2^e, 2^(e+1))
    m = a / step
    return sign * round(m) * step  # round(Fraction) rounds ties to even


def _brute_quantize(x):
    """The pages' steps in exact arithmetic with explicit float32 roundings."""
    xs = [Fraction(float(v)) for v in np.asarray(x, dtype=np.float32)]
    amax = max(abs(v) for v in xs)
    amax = max(amax, Fraction(float(np.float32(1e-8))))
    s = _round_f32(amax / 127)
    codes = [int(round(_round_f32(v / s))) for v in xs]
    return codes, s


def test_brute_force_exact_arithmetic():
    rows = _rows(2, n=60, d=32)
    # rows built to land exactly on ties after the float32 division
    rows[0, :6] = [127.0, 0.5, 1.5, -2.5, 3.5, 126.5]
    rows[1, :4] = [-63.5, 31.75, 0.25, 10.0]
    for x in rows:
        codes, s = Q.quantize_row(x)
        bc, bs = _brute_quantize(x)
        assert Fraction(float(s)) == bs
        assert codes.astype(int).tolist() == bc


# ----------------------------------------------------------------------------- attention over the cache

def _random_int8_cache(rng, n_blocks, h_kv, d):
    kq = rng.integers(-127, 128, size=(n_blocks, h_kv, 16, d)).astype(np.int8)
    vq = rng.integers(-127, 128, size=(n_blocks, h_kv, 16, d)).astype(np.int8)
    ks = rng.uniform(0.005, 0.03, size=(n_blocks, h_kv, 16)).astype(np.float32)
    vs = rng.uniform(0.005, 0.03, size=(n_blocks, h_kv, 16)).astype(np.float32)
    return kq, vq, ks, vs


def test_exactly_representable_cache_decodes_like_the_plain_cache():
    """Rows of integers with max |x| = 127 quantise to themselves with s = 1, so
    int8 decode must equal plain decode on the same values, bit for bit."""
    rng = np.random.default_rng(3)
    h_kv, d, nb = 2, 16, 6
    kf = rng.integers(-126, 127, size=(nb, h_kv, 16, d)).astype(np.float32)
    vf = rng.integers(-126, 127, size=(nb, h_kv, 16, d)).astype(np.float32)
    kf[..., 0] = 127.0
    vf[..., 1] = -127.0
    kq = np.zeros(kf.shape, np.int8)
    vq = np.zeros(vf.shape, np.int8)
    ks = np.zeros(kf.shape[:3], np.float32)
    vs = np.zeros(vf.shape[:3], np.float32)
    for idx in np.ndindex(*kf.shape[:3]):
        kq[idx], ks[idx] = Q.quantize_row(kf[idx])
        vq[idx], vs[idx] = Q.quantize_row(vf[idx])
    assert np.all(ks == 1) and np.all(vs == 1)
    assert np.array_equal(kq.astype(np.float32), kf) and np.array_equal(vq.astype(np.float32), vf)
    q = rng.standard_normal((2, 4, d)) * 0.05
    tables = np.array([[3, 1, 5], [0, 2, 4]], dtype=np.int32)
    lens = np.array([40, 33])
    assert np.array_equal(Q.decode_int8(q, kq, vq, ks, vs, tables, lens, 0.25),
                          A.decode(q, kf, vf, tables, lens, 0.25))


def _brute_decode_int8(q, kq, vq, ks, vs, tables, lens, scale):
    """Pure-Python decode over s * x_q, element by element."""
    kd = [[[[float(ks[b, h, o]) * int(kq[b, h, o, c]) for c in range(kq.shape[3])]
            for o in range(16)] for h in range(kq.shape[1])] for b in range(kq.shape[0])]
    vd = [[[[float(vs[b, h, o]) * int(vq[b, h, o, c]) for c in range(vq.shape[3])]
            for o in range(16)] for h in range(vq.shape[1])] for b in range(vq.shape[0])]
    return pins.brute_decode(q, np.array(kd), np.array(vd), tables, lens, scale)


def test_decode_int8_matches_brute_force():
    rng = np.random.default_rng(4)
    kq, vq, ks, vs = _random_int8_cache(rng, 7, 2, 8)
    q = rng.standard_normal((3, 6, 8))
    tables = np.array([[6, 0, 3], [2, 5, 1], [4, 0, 0]], dtype=np.int32)
    lens = np.array([37, 48, 5])
    got = Q.decode_int8(q, kq, vq, ks, vs, tables, lens, 0.3)
    ref = _brute_decode_int8(q, kq, vq, ks, vs, tables, lens, 0.3)
    assert np.abs(got - ref).max() <= 1e-12


def test_decode_int8_block_permutation():
    rng = np.random.default_rng(5)
    kq, vq, ks, vs = _random_int8_cache(rng, 6, 2, 8)
    q = rng.standard_normal((2, 4, 8))
    tables = np.array([[0, 1, 2], [3, 4, 5]], dtype=np.int32)
    lens = np.array([40, 35])
    perm = rng.permutation(6)  # new block i holds old block perm[i] (codes and scales)
    inv = np.argsort(perm)     # so old block j is new block inv[j]
    new_tables = inv[tables].astype(np.int32)
    a = Q.decode_int8(q, kq, vq, ks, vs, tables, lens, 0.2)
    b = Q.decode_int8(q, kq[perm], vq[perm], ks[perm], vs[perm], new_tables, lens, 0.2)
    assert np.array_equal(a, b)


def _integer_cache(rng, nb, h_kv, d):
    """Integer rows with max |x| = 127: they quantise to themselves with s = 1."""
    kf = rng.integers(-126, 127, size=(nb, h_kv, 16, d)).astype(np.float32)
    vf = rng.integers(-126, 127, size=(nb, h_kv, 16, d)).astype(np.float32)
    kf[..., 2] = -127.0
    vf[..., 0] = 127.0
    kq = np.zeros(kf.shape, np.int8)
    vq = np.zeros(vf.shape, np.int8)
    ks = np.zeros(kf.shape[:3], np.float32)
    vs = np.zeros(vf.shape[:3], np.float32)
    for idx in np.ndindex(*kf.shape[:3]):
        kq[idx], ks[idx] = Q.quantize_row(kf[idx])
        vq[idx], vs[idx] = Q.quantize_row(vf[idx])
    assert np.all(ks == 1) and np.all(vs == 1)
    return kf, vf, kq, vq, ks, vs


def test_exactly_representable_cache_prefills_like_the_plain_cache():
    """Chunked prefill (a 20-token chunk at the end of a 45-token context, a
    whole 30-token prompt) over an integer cache with s = 1 equals the plain
    prefill of the same values, bit for bit."""
    rng = np.random.default_rng(13)
    kf, vf, kq, vq, ks, vs = _integer_cache(rng, 7, 2, 16)
    q = rng.standard_normal((50, 6, 16)) * 0.05
    cu = np.array([0, 20, 50], np.int32)
    tables = np.array([[4, 0, 6], [1, 3, 5]], dtype=np.int32)
    lens = np.array([45, 30])
    assert np.array_equal(Q.prefill_int8(q, cu, kq, vq, ks, vs, tables, lens, 0.25),
                          A.prefill(q, cu, kf, vf, tables, lens, 0.25))


def _brute_prefill_int8(q, cu, kq, vq, ks, vs, tables, lens, scale):
    """Pure-Python prefill over s * x_q, element by element."""
    kd = [[[[float(ks[b, h, o]) * int(kq[b, h, o, c]) for c in range(kq.shape[3])]
            for o in range(16)] for h in range(kq.shape[1])] for b in range(kq.shape[0])]
    vd = [[[[float(vs[b, h, o]) * int(vq[b, h, o, c]) for c in range(vq.shape[3])]
            for o in range(16)] for h in range(vq.shape[1])] for b in range(vq.shape[0])]
    return pins.brute_prefill(q, cu, np.array(kd), np.array(vd), tables, lens, scale)


def _check_prefill_int8_brute(prefill_int8):
    rng = np.random.default_rng(14)
    kq, vq, ks, vs = _random_int8_cache(rng, 7, 2, 8)
    q = rng.standard_normal((27, 4, 8))
    cu = np.array([0, 17, 20, 27], np.int32)
    tables = np.array([[6, 0, 3], [2, 5, 1], [4, 0, 0]], dtype=np.int32)
    lens = np.array([37, 20, 7])
    got = prefill_int8(q, cu, kq, vq, ks, vs, tables, lens, 0.3)
    ref = _brute_prefill_int8(q, cu, kq, vq, ks, vs, tables, lens, 0.3)
    assert np.abs(got - ref).max() <= 1e-12


def test_prefill_int8_matches_brute_force():
    _check_prefill_int8_brute(Q.prefill_int8)


def test_prefill_int8_last_row_is_decode():
    """The last query row of a prefill is the decode of that token over the
    same cache (cached equals recomputed, LLM Inference Server page, Stage 1)."""
    rng = np.random.default_rng(15)
    kq, vq, ks, vs = _random_int8_cache(rng, 6, 2, 8)
    q = rng.standard_normal((9, 4, 8))
    tables = np.array([[5, 2, 0]], dtype=np.int32)
    lens = np.array([41])
    pre = Q.prefill_int8(q, np.array([0, 9], np.int32), kq, vq, ks, vs, tables, lens, 0.2)
    dec = Q.decode_int8(q[-1:], kq, vq, ks, vs, tables, lens, 0.2)
    assert np.abs(pre[-1] - dec[0]).max() <= 1e-13


def test_mutation_scale_on_the_wrong_axis_is_caught(monkeypatch):
    """A dequantisation that takes the scale along the channel axis (scale of
    slot c % 16 for channel c) instead of one scale per token row fails the
    brute-force pin."""
    def wrong_axis(codes, scales):
        c = np.asarray(codes, dtype=np.float64)
        s = np.asarray(scales, dtype=np.float64)
        ch = np.arange(c.shape[-1]) % 16
        return c * s[..., ch][..., None, :]
    monkeypatch.setattr(Q, "dequantize", wrong_axis)
    assert _fails(_check_prefill_int8_brute, Q.prefill_int8)


def test_kv_append_int8_writes_only_the_named_slots():
    rng = np.random.default_rng(6)
    kq, vq, ks, vs = _random_int8_cache(rng, 4, 2, 8)
    k_new = rng.standard_normal((3, 2, 8)).astype(np.float32)
    v_new = rng.standard_normal((3, 2, 8)).astype(np.float32)
    slots = np.array([17, -1, 63])
    nk, nv, nks, nvs = Q.kv_append_int8(k_new, v_new, slots, kq, vq, ks, vs)
    written = {(1, 1): 0, (3, 15): 2}
    for blk in range(4):
        for off in range(16):
            if (blk, off) in written:
                i = written[(blk, off)]
                for h in range(2):
                    c, s = Q.quantize_row(k_new[i, h])
                    assert np.array_equal(nk[blk, h, off], c) and nks[blk, h, off] == s
                    c, s = Q.quantize_row(v_new[i, h])
                    assert np.array_equal(nv[blk, h, off], c) and nvs[blk, h, off] == s
            else:
                assert np.array_equal(nk[blk, :, off], kq[blk, :, off])
                assert np.array_equal(nvs[blk, :, off], vs[blk, :, off])
    with pytest.raises(ValueError):
        Q.kv_append_int8(k_new, v_new, np.array([5, 5, -1]), kq, vq, ks, vs)


# ----------------------------------------------------------------------------- mutations

def _q_half_away(row):
    x = np.asarray(row, dtype=np.float32)
    s = Q.absmax_scale(x)
    return (np.sign(x / s) * np.floor(np.abs(x / s) + np.float32(0.5))).astype(np.int8), s


def _q_div128(row):
    x = np.asarray(row, dtype=np.float32)
    s = np.float32(np.maximum(np.abs(x).max(), Q.AMAX_FLOOR) / np.float32(128.0))
    return np.rint(x / s).astype(np.int8), s


def _q_truncate(row):
    x = np.asarray(row, dtype=np.float32)
    s = Q.absmax_scale(x)
    return np.trunc(x / s).astype(np.int8), s


def _q_no_floor(row):
    x = np.asarray(row, dtype=np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        s = np.float32(np.abs(x).max() / np.float32(127.0))
        return np.nan_to_num(np.rint(x / s)).astype(np.int8), s


def _append_per_token(k_new, v_new, slots, kq, vq, ks, vs):
    """Mistake: one scale over all KV heads of a token."""
    kq, vq, ks, vs = (np.array(a, copy=True) for a in (kq, vq, ks, vs))
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        blk, off = divmod(int(sl), 16)
        for src, codes, scales in ((k_new[i], kq, ks), (v_new[i], vq, vs)):
            s = Q.absmax_scale(np.asarray(src).reshape(-1))
            for h in range(codes.shape[1]):
                codes[blk, h, off] = np.rint(np.asarray(src[h], np.float32) / s).astype(np.int8)
                scales[blk, h, off] = s
    return kq, vq, ks, vs


def _fails(check, *args):
    try:
        check(*args)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("bad", [_q_half_away, _q_div128, _q_truncate], ids=lambda f: f.__name__)
def test_mutations_of_the_rounding_or_divisor_are_caught(bad):
    assert _fails(_check_worked, bad) or _fails(_check_properties, bad)


def test_mutation_without_the_floor_is_caught():
    def zero_row(quantize_row):
        c, s = quantize_row(np.zeros(8, dtype=np.float32))
        assert s > 0 and c.tolist() == [0] * 8
    zero_row(Q.quantize_row)
    assert _fails(zero_row, _q_no_floor)


def test_mutation_one_scale_per_token_is_caught():
    assert _fails(_check_per_head_rows, _append_per_token)
