"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every pool is NaN-poisoned outside the slots that hold context tokens, so any
read the kernels fail to mask shows up as NaN.  kv_append must be bit-exact;
attention outputs must be within 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs) of
the float64 oracle, element by element.
"""
import numpy as np
import pytest
import torch

import oracle.attention as O
import pins
from gpu_run import TOL, bits, max_err, run
from paged_kv_cache_274_amd import ops
from paged_kv_cache_274_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check_append(w, res):
    kc_ref, vc_ref = pins.appended_pools(w)
    for got, ref in ((res.k_cache, kc_ref), (res.v_cache, vc_ref)):
        exp = torch.from_numpy(ref).to(w.dtype)
        nan_g, nan_e = torch.isnan(got), torch.isnan(exp)
        assert torch.equal(nan_g, nan_e)
        assert torch.equal(bits(got)[~nan_g], bits(exp)[~nan_e])
    return kc_ref, vc_ref


def check_decode(w, res, kc_ref, vc_ref):
    ref = pins.oracle_decode(w, kc_ref, vc_ref)
    err = max_err(res.decode, ref)
    assert err <= TOL[w.dtype], f"decode max|err| {err}"
    return err


def check_prefill(w, res, kc_ref, vc_ref):
    ref = pins.oracle_prefill(w, kc_ref, vc_ref)
    err = max_err(res.prefill, ref)
    assert err <= TOL[w.dtype], f"prefill max|err| {err}"
    return err


# ----------------------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_config_parity(k):
    """Append (bit-exact), then decode and prefill, in the launch configuration the bench uses."""
    w = W.config(k, poison=True)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    if w.B:
        err = check_decode(w, res, kc_ref, vc_ref)
        print(f"config {k}: decode max|err| = {err:.3g}")
    if w.S:
        err = check_prefill(w, res, kc_ref, vc_ref)
        print(f"config {k}: prefill max|err| = {err:.3g}")


# ----------------------------------------------------------------------------- decode coverage

DECODE_GRID = [
    # dtype, d, h_q, h_kv
    ("f32", 64, 4, 2), ("f32", 128, 8, 8), ("f32", 64, 16, 2), ("f32", 128, 24, 4),
    ("bf16", 64, 4, 4), ("bf16", 64, 14, 2), ("bf16", 128, 32, 8), ("bf16", 128, 6, 2),
    ("bf16", 64, 40, 8), ("bf16", 128, 16, 1), ("bf16", 64, 12, 4), ("bf16", 128, 8, 1),
]


@pytest.mark.parametrize("dtype,d,h_q,h_kv", [("bf16", 64, 14, 2), ("f32", 64, 16, 2),
                                              ("bf16", 128, 16, 1)])
def test_decode_large_batch_keeps_wide_chunks(dtype, d, h_q, h_kv):
    """Small lines split a GQA group of more than 4 heads into chunks of at
    most 4 (the grid above); large ones keep chunks of up to 8 heads per wave.
    These batches are large enough for the wide chunks, and match the oracle."""
    rng = np.random.default_rng(3000 + h_q + d)
    lens = [int(x) for x in rng.integers(1000, 4096, size=64, endpoint=True)]
    g = h_q // h_kv
    assert 64 * h_kv * -(-g // 4) * -(-max(lens) // 16) > 2048 * 16   # above the small-line rule
    w = W.build("wide", rng, dtype=dtype, h_q=h_q, h_kv=h_kv, d=d, decode_lens=lens,
                free_frac=0.05, poison=True)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    check_decode(w, res, kc_ref, vc_ref)


@pytest.mark.parametrize("dtype,d,h_q,h_kv", DECODE_GRID)
@pytest.mark.parametrize("splits", [0, 1, 13, 300])
def test_decode_grid(dtype, d, h_q, h_kv, splits):
    rng = np.random.default_rng(1000 + d + h_q * 7 + h_kv)
    lens = [1, 15, 16, 17, 63, 64, 65, 200, 333, 700]
    w = W.build("grid", rng, dtype=dtype, h_q=h_q, h_kv=h_kv, d=d, decode_lens=lens,
                free_frac=0.2, max_blocks_per_seq=50, poison=True)
    res = run(w, DEV, num_splits=splits)
    kc_ref, vc_ref = check_append(w, res)
    check_decode(w, res, kc_ref, vc_ref)


def test_decode_zero_length_and_single_token():
    rng = np.random.default_rng(5)
    w = W.build("edge", rng, dtype="bf16", h_q=8, h_kv=2, d=128, decode_lens=[1, 40, 1],
                free_frac=0.5, poison=True)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    check_decode(w, res, kc_ref, vc_ref)
    # one token: the output is that token's V row exactly (weight 1)
    for b in (0, 2):
        g = w.h_q // w.h_kv
        for h in range(w.h_q):
            assert torch.equal(bits(res.decode[b, h]), bits(w.v_new[b, h // g]))
    # context length 0 gives zeros
    kc = res.k_cache.to(DEV)
    vc = res.v_cache.to(DEV)
    lens0 = torch.tensor([0, 40, 0], dtype=torch.int32)
    ref = O.decode(pins.np64(w.dec_q), kc_ref, vc_ref, w.dec_block_tables.numpy(), lens0.numpy(), w.scale)
    # with one range no second pass runs: the first pass zero-fills and stores
    for splits in (0, 1):
        out = ops.paged_decode_attention(w.dec_q.to(DEV), kc, vc, w.dec_block_tables.to(DEV),
                                         lens0.to(DEV), 40, scale=w.scale, num_splits=splits).cpu()
        assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[2]) == 0
        assert max_err(out, ref) <= TOL[w.dtype]


@pytest.mark.parametrize("splits", [1, 2, 3, 17, 64, 500, 2048, 5000])
def test_decode_split_invariance(splits):
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 3000, size=12)
    w = W.build("pinv", rng, dtype="bf16", h_q=32, h_kv=8, d=128, decode_lens=lens,
                free_frac=0.1, poison=True)
    res = run(w, DEV, num_splits=splits)
    kc_ref, vc_ref = check_append(w, res)
    check_decode(w, res, kc_ref, vc_ref)


def test_decode_workspace_reused_across_shapes():
    """One workspace serves calls of different shapes in turn, whatever an
    earlier call left in it: results are bit-identical to calls on fresh
    workspaces."""
    shapes = [("bf16", 32, 8, 128, [int(x) for x in np.random.default_rng(3).integers(1, 3000, 40)]),
              ("bf16", 14, 2, 64, [int(x) for x in np.random.default_rng(4).integers(1, 2000, 60)]),
              ("f32", 8, 2, 64, [5, 700, 1200])]
    runs = []
    for i, (dt, h_q, h_kv, d, lens) in enumerate(shapes):
        w = W.build("reuse", np.random.default_rng(60 + i), dtype=dt, h_q=h_q, h_kv=h_kv, d=d,
                    decode_lens=lens, free_frac=0.1, poison=True)
        kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
        ops.kv_append(w.k_new.to(DEV), w.v_new.to(DEV), w.slot_mapping.to(DEV), kc, vc)
        runs.append((w, kc, vc, w.dec_q.to(DEV), w.dec_block_tables.to(DEV),
                     w.dec_context_lens.to(DEV)))
    size = max(ops.decode_workspace_bytes(w.B, w.h_q, w.h_kv, w.d, w.dec_max_context_len, w.dtype)
               for w, *_ in runs)
    shared = torch.full((size,), 0xA5, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        for w, kc, vc, q, tbl, lens in runs:
            fresh = ops.paged_decode_attention(q, kc, vc, tbl, lens, w.dec_max_context_len,
                                               scale=w.scale)
            again = ops.paged_decode_attention(q, kc, vc, tbl, lens, w.dec_max_context_len,
                                               scale=w.scale, workspace=shared)
            torch.cuda.synchronize()
            assert torch.equal(bits(fresh.cpu()), bits(again.cpu())), (w.h_q, w.d, rep)


CURSOR_MIXES = [
    # name, lens, h_q, h_kv, d
    ("many short", [int(x) for x in np.random.default_rng(41).integers(1, 40, size=300)], 8, 2, 64),
    ("zeros between", [0, 500, 0, 0, 17, 3000, 0, 1, 0], 32, 8, 128),
    ("one long", [30000], 32, 8, 128),
    ("one long, one head", [20011], 4, 1, 64),
    ("fewer blocks than groups", [5, 3], 8, 1, 128),
]


@pytest.mark.parametrize("name,lens,h_q,h_kv,d", CURSOR_MIXES, ids=[m[0] for m in CURSOR_MIXES])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_automatic_split_length_mixes(name, lens, h_q, h_kv, d, dtype):
    """The automatic split on length mixes that stress its bookkeeping: many
    segments per wave, empty sequences, a segment spread over every wave (more
    than 64 pieces to merge), and fewer blocks than waves."""
    rng = np.random.default_rng(sum(lens) % 1000 + h_q)
    # a decode step appends one token, so the workload has length >= 1; the
    # zero-length sequences are given to a second decode call directly
    w = W.build("mix", rng, dtype=dtype, h_q=h_q, h_kv=h_kv, d=d,
                decode_lens=[max(1, L) for L in lens], free_frac=0.1, poison=True)
    res = run(w, DEV, num_splits=0)
    kc_ref, vc_ref = check_append(w, res)
    check_decode(w, res, kc_ref, vc_ref)
    if 0 in lens:
        lz = torch.tensor(lens, dtype=torch.int32)
        out = ops.paged_decode_attention(w.dec_q.to(DEV), res.k_cache.to(DEV),
                                         res.v_cache.to(DEV), w.dec_block_tables.to(DEV),
                                         lz.to(DEV), max(lens), scale=w.scale).cpu()
        ref = O.decode(pins.np64(w.dec_q), kc_ref, vc_ref, w.dec_block_tables.numpy(),
                       lz.numpy(), w.scale)
        assert max_err(out, ref) <= TOL[w.dtype]
        for b, L in enumerate(lens):
            if L == 0:
                assert torch.count_nonzero(out[b]) == 0


def _pool_from_logical(Ks, Vs, seed, dtype, extra=5, prefix_share=0):
    kc, vc, t = pins.page(Ks, Vs, np.random.default_rng(seed), extra_blocks=extra,
                          prefix_share=prefix_share)
    return (torch.from_numpy(kc).to(dtype), torch.from_numpy(vc).to(dtype),
            torch.from_numpy(t))


def _decode_gpu(q, kc, vc, t, lens, splits, scale):
    out = ops.paged_decode_attention(q.to(DEV), kc.to(DEV), vc.to(DEV), t.to(DEV),
                                     torch.tensor(lens, dtype=torch.int32).to(DEV), max(lens),
                                     scale=scale, num_splits=splits)
    return out.cpu()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_block_permutation_bit_exact(dtype):
    """Reduction order depends only on logical token positions, so moving blocks
    to other physical ids changes no bit of the output."""
    rng = np.random.default_rng(8)
    lens = [700, 33, 1500, 16, 257]
    Ks = [rng.standard_normal((L, 4, 64)) for L in lens]
    Vs = [rng.standard_normal((L, 4, 64)) for L in lens]
    q = torch.from_numpy(rng.standard_normal((len(lens), 16, 64))).to(dtype)
    a = _pool_from_logical(Ks, Vs, 1, dtype)
    b = _pool_from_logical(Ks, Vs, 2, dtype, extra=40)
    assert not torch.equal(a[2], b[2])
    oa = _decode_gpu(q, *a, lens, 128, 0.125)
    ob = _decode_gpu(q, *b, lens, 128, 0.125)
    assert torch.equal(bits(oa), bits(ob))
    ref = O.decode(q.double().numpy(), a[0].double().numpy(), a[1].double().numpy(),
                   a[2].numpy(), lens, 0.125)
    assert max_err(oa, ref) <= TOL[dtype]


def test_decode_prefix_sharing_and_batch_invariance():
    """Shared prefix blocks give the same bits as private copies (same work
    layout).  Batched equals single: bit-exact when each sequence is reduced by
    one wave (num_splits=1), within tolerance for any split, since the split of
    a sequence across waves depends on the rest of the batch."""
    rng = np.random.default_rng(9)
    P_blocks = 13
    pk = rng.standard_normal((P_blocks * 16, 8, 128))
    pv = rng.standard_normal((P_blocks * 16, 8, 128))
    lens = [1000, 600, 2049, 208 + 1]
    Ks = [np.concatenate([pk, rng.standard_normal((L - 208, 8, 128))]) for L in lens]
    Vs = [np.concatenate([pv, rng.standard_normal((L - 208, 8, 128))]) for L in lens]
    q = torch.from_numpy(rng.standard_normal((len(lens), 32, 128))).to(torch.bfloat16)
    shared = _pool_from_logical(Ks, Vs, 3, torch.bfloat16, prefix_share=P_blocks)
    private = _pool_from_logical(Ks, Vs, 4, torch.bfloat16)
    assert torch.equal(shared[2][1:, :P_blocks], shared[2][:1, :P_blocks].expand(3, -1))
    scale = 0.0883883476
    ref = O.decode(q.double().numpy(), shared[0].double().numpy(), shared[1].double().numpy(),
                   shared[2].numpy(), lens, scale)
    for splits in (0, 1, 256):
        o_sh = _decode_gpu(q, *shared, lens, splits, scale)
        o_pr = _decode_gpu(q, *private, lens, splits, scale)
        assert torch.equal(bits(o_sh), bits(o_pr))
        assert max_err(o_sh, ref) <= 2e-2
        for b in range(len(lens)):
            one = _decode_gpu(q[b:b + 1], shared[0], shared[1], shared[2][b:b + 1], [lens[b]],
                              splits, scale)
            if splits == 1:
                assert torch.equal(bits(one[0]), bits(o_sh[b]))
            assert max_err(one, ref[b:b + 1]) <= 2e-2


# ----------------------------------------------------------------------------- prefill coverage

PREFILL_GRID = [
    # d, h_q, h_kv, [(context, n_new)]
    (64, 14, 2, [(512, 512), (100, 100), (37, 5), (300, 1)]),
    (64, 4, 4, [(33, 33), (64, 64), (129, 64), (17, 16)]),
    (128, 32, 8, [(200, 200), (96, 31), (1, 1)]),
    (128, 8, 1, [(150, 150), (260, 130)]),
    (64, 16, 2, [(1000, 200), (48, 48)]),
    (128, 6, 3, [(70, 70), (33, 2)]),
    # many 64-key tiles, ragged context tails, chunks that start mid-tile
    (128, 32, 8, [(3000, 700), (2049, 2049)]),
    (64, 14, 2, [(4096, 64), (777, 777), (1, 1)]),
    # a chunk whose rows straddle key 64 in a small grid: the second key group
    # starts at tile 1, wholly past some rows' positions
    (64, 14, 2, [(100, 60)]),
    (64, 16, 2, [(90, 50), (70, 70)]),
]


@pytest.mark.parametrize("d,h_q,h_kv,seqs", PREFILL_GRID)
def test_prefill_grid(d, h_q, h_kv, seqs):
    rng = np.random.default_rng(2000 + d + h_q + h_kv)
    w = W.build("pgrid", rng, dtype="bf16", h_q=h_q, h_kv=h_kv, d=d, prefill=seqs,
                free_frac=0.2, poison=True)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    check_prefill(w, res, kc_ref, vc_ref)


# Grids of at least one workgroup of 256 packed rows per compute unit, which
# take the 8-wave kernel (wave pairs alternating matrix and softmax phases):
# GQA 1, 2, 4, 7, 8; whole prompts, chunks starting mid-tile, ragged lengths.
PREFILL_EIGHT_WAVE = [
    # d, h_q, h_kv, [(context, n_new)], scale (None: 1/sqrt(d))
    (128, 16, 16, [(1024, 1024), (2000, 700), (900, 900), (1000, 1000)], None),
    (128, 64, 8, [(300, 300), (1200, 511)], None),
    (64, 14, 2, [(600, 600)] * 4 + [(1800, 600)] * 4, None),
    (128, 32, 8, [(3000, 260), (700, 700), (1500, 1000), (2048, 1000)], None),
    (64, 8, 4, [(513, 513)] * 16, None),
    (128, 32, 8, [(1100, 1024), (1024, 1024), (640, 640), (2000, 333)], -0.2),
    (128, 32, 8, [(1100, 1024), (1024, 1024), (640, 640), (2000, 333)], 1.0),
]


@pytest.mark.parametrize("d,h_q,h_kv,seqs,scale", PREFILL_EIGHT_WAVE)
def test_prefill_eight_wave_grid(d, h_q, h_kv, seqs, scale):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = max(n for _, n in seqs) * (h_q // h_kv)
    assert rows >= 256 and -(-rows // 256) * h_kv * len(seqs) >= cus, "not the 8-wave launch"
    rng = np.random.default_rng(2200 + d + h_q + h_kv + len(seqs))
    w = W.build("pp", rng, dtype="bf16", h_q=h_q, h_kv=h_kv, d=d, prefill=seqs,
                free_frac=0.1, poison=True, scale=scale)
    res = run(w, DEV, do_decode=False)
    kc_ref, vc_ref = check_append(w, res)
    # The bf16 output rounding is relative (half an ulp, 2^-9 |o|): with scale
    # 1.0 the softmax is nearly one-hot and outputs reach |o| ~ 4.8, where half
    # an ulp is 1/64, so the bound is taken relative to max(1, |o|).
    ref = pins.oracle_prefill(w, kc_ref, vc_ref)
    got = res.prefill.double().numpy()
    err = float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max())
    print(f"eight-wave prefill {d}/{h_q}/{h_kv} scale {scale}: max|err|/max(1,|ref|) {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("d,h_q,h_kv,seqs", [
    (128, 32, 8, [(512, 512)] * 16),
    (64, 14, 2, [(512, 512)] * 40),
    (128, 32, 8, [(1500, 300)] * 8 + [(1300, 301)] * 8),   # chunks starting mid-tile
])
def test_prefill_full_prompts_many_rounds(d, h_q, h_kv, seqs):
    """Whole and chunked prompts on grids of several rounds of the chip (the
    8-wave kernel, sequence planes longest context first)."""
    rng = np.random.default_rng(2100 + d + len(seqs))
    w = W.build("rb2", rng, dtype="bf16", h_q=h_q, h_kv=h_kv, d=d, prefill=seqs,
                free_frac=0.1, poison=True)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    check_prefill(w, res, kc_ref, vc_ref)


@pytest.mark.parametrize("shape", [(32, 8, 128), (14, 2, 64)])
def test_prefill_long_prompts_sampled(shape):
    """The bench's long-prompt workload (4 causal prompts of 4096 tokens) in
    the launch the bench times, checked on sampled query rows: row p of a
    prompt is the oracle's prefill of that one query at position p over keys
    0..p."""
    w = W.long_prefill(*shape)
    res = run(w, DEV, do_decode=False)
    kc_ref, vc_ref = O.kv_append(pins.np64(w.k_new), pins.np64(w.v_new), w.slot_mapping.numpy(),
                                 pins.np64(w.k_cache), pins.np64(w.v_cache))
    rng = np.random.default_rng(9)
    err = 0.0
    for s in range(w.S):
        for p in [0, 1, 63, 64, 127, 2048, 4094, 4095] + [int(x) for x in rng.integers(0, 4096, 3)]:
            r = int(w.pre_cu_seqlens[s]) + p
            ref = O.prefill(pins.np64(w.pre_q[r:r + 1]), np.array([0, 1], np.int32), kc_ref,
                            vc_ref, w.pre_block_tables[s:s + 1].numpy(),
                            np.array([p + 1], np.int32), w.scale)
            err = max(err, max_err(res.prefill[r:r + 1], ref))
    print(f"long prompts {shape}: sampled max|err| {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("n_s", [2, 4, 5])
def test_multi_token_decode_verify(n_s):
    """Multi-token decode (a speculative verify step: the n_s newest tokens of
    each sequence attend causally over its whole cache) runs as chunked prefill
    with tiny n_s, on decode-shaped contexts; its last row equals a one-token
    decode over the same context."""
    rng = np.random.default_rng(40 + n_s)
    lens = [int(x) for x in rng.integers(128, 4096, size=12, endpoint=True)] + [n_s, 16 + n_s]
    w = W.build("verify", rng, dtype="bf16", h_q=32, h_kv=8, d=128,
                prefill=[(L, n_s) for L in lens], free_frac=0.1, poison=True)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    check_prefill(w, res, kc_ref, vc_ref)
    last = w.pre_cu_seqlens[1:].long() - 1
    q_last = w.pre_q[last]
    one = ops.paged_decode_attention(q_last.to(DEV), res.k_cache.to(DEV), res.v_cache.to(DEV),
                                     w.pre_block_tables.to(DEV), w.pre_context_lens.to(DEV),
                                     max(lens), scale=w.scale).cpu()
    assert max_err(res.prefill[last], one.double().numpy()) <= 2e-2


@pytest.mark.parametrize("S,n_s,lens_of", [
    (40, 3, lambda rng, S: rng.integers(4, 1500, size=S)),
    (200, 2, lambda rng, S: rng.integers(1, 40, size=S) * 7),     # many equal lengths
    (300, 2, lambda rng, S: rng.integers(3, 200, size=S))])
def test_prefill_grid_beyond_one_round(S, n_s, lens_of):
    """Grids with more workgroups than the chip holds at once take their
    sequence planes longest context first (ties by index; S <= 256), so the
    sequence a workgroup serves is not its plane index; with S > 256 the
    index order stays.  Every row matches the oracle either way."""
    rng = np.random.default_rng(500 + S)
    lens = [max(int(x), n_s) for x in lens_of(rng, S)]
    w = W.build("many", rng, dtype="bf16", h_q=16, h_kv=8, d=128,
                prefill=[(L, n_s) for L in lens], free_frac=0.05, poison=True)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    check_prefill(w, res, kc_ref, vc_ref)


@pytest.mark.parametrize("scale", [-0.2, 1.0])
def test_negative_and_large_scale(scale):
    """Any finite scale: a negative one reverses the ranking of the keys, a
    large one makes the softmax nearly one-hot (decode and prefill)."""
    rng = np.random.default_rng(77)
    w = W.build("scale", rng, dtype="bf16", h_q=8, h_kv=2, d=128, decode_lens=[300, 17, 1000],
                prefill=[(257, 100), (64, 64)], free_frac=0.2, poison=True, scale=scale)
    res = run(w, DEV)
    kc_ref, vc_ref = check_append(w, res)
    check_decode(w, res, kc_ref, vc_ref)
    check_prefill(w, res, kc_ref, vc_ref)


def test_prefill_chunked_equals_whole_and_decode():
    """A prompt prefilled in two chunks gives the rows of the whole-prompt
    prefill, and its last row matches decode of the last token."""
    rng = np.random.default_rng(31)
    L, cut = 300, 123
    whole = W.build("whole", rng, dtype="bf16", h_q=14, h_kv=2, d=64, prefill=[(L, L)],
                    free_frac=0.2, poison=True)
    res = run(whole, DEV)
    kc = res.k_cache.to(DEV)
    vc = res.v_cache.to(DEV)
    t = whole.pre_block_tables.to(DEV)
    q = whole.pre_q.to(DEV)
    first = ops.paged_prefill_attention(q[:cut].contiguous(), torch.tensor([0, cut], dtype=torch.int32).to(DEV),
                                        kc, vc, t, torch.tensor([cut], dtype=torch.int32).to(DEV), cut,
                                        scale=whole.scale)
    second = ops.paged_prefill_attention(q[cut:].contiguous(), torch.tensor([0, L - cut], dtype=torch.int32).to(DEV),
                                         kc, vc, t, torch.tensor([L], dtype=torch.int32).to(DEV), L - cut,
                                         scale=whole.scale)
    dec = ops.paged_decode_attention(q[L - 1:].contiguous(), kc, vc, t,
                                     torch.tensor([L], dtype=torch.int32).to(DEV), L, scale=whole.scale)
    chunked = torch.cat([first, second]).cpu()
    ref = pins.oracle_prefill(whole, *pins.appended_pools(whole))
    assert max_err(chunked, ref) <= 2e-2
    assert max_err(dec.cpu(), ref[L - 1:]) <= 2e-2
    diff = (chunked.float() - res.prefill.float()).abs().max().item()
    assert diff <= 2e-2


def test_prefill_fp32_is_unsupported():
    w = pins.tiny_workload(3, prefill=((20, 20),), d=64)
    with pytest.raises(ops.PkvError) as e:
        run(w, DEV)
    assert e.value.status == 2


# ----------------------------------------------------------------------------- append coverage

def test_append_skips_negative_slots_and_keeps_other_bits():
    rng = np.random.default_rng(12)
    n_blocks, h_kv, d = 10, 2, 128
    kc = torch.from_numpy(rng.standard_normal((n_blocks, h_kv, 16, d)).astype(np.float32)).to(torch.bfloat16)
    vc = kc.clone() * 2
    slots = torch.tensor([0, 15, 16, -1, 159, 77, -5], dtype=torch.int64)
    kn = torch.from_numpy(rng.standard_normal((7, h_kv, d)).astype(np.float32)).to(torch.bfloat16)
    vn = kn * 3
    gk, gv = kc.to(DEV), vc.to(DEV)
    ops.kv_append(kn.to(DEV), vn.to(DEV), slots.to(DEV), gk, gv)
    ko, vo = O.kv_append(kn.double().numpy(), vn.double().numpy(), slots.numpy(),
                         kc.double().numpy(), vc.double().numpy())
    assert torch.equal(bits(gk.cpu()), bits(torch.from_numpy(ko).to(torch.bfloat16)))
    assert torch.equal(bits(gv.cpu()), bits(torch.from_numpy(vo).to(torch.bfloat16)))


def test_bound_calls_match_the_checked_calls():
    """The pre-bound launches the bench times (bind_kv_append, bind_decode,
    bind_prefill) give bit for bit what the checked calls give."""
    w = W.config(5, poison=True)
    dev = DEV
    pools = [(w.k_cache.to(dev), w.v_cache.to(dev)) for _ in range(2)]
    k_new, v_new, slots = w.k_new.to(dev), w.v_new.to(dev), w.slot_mapping.to(dev)
    q, tbl, lens = w.dec_q.to(dev), w.dec_block_tables.to(dev), w.dec_context_lens.to(dev)
    ops.kv_append(k_new, v_new, slots, *pools[0])
    ops.bind_kv_append(k_new, v_new, slots, *pools[1])()
    ws = torch.zeros(ops.decode_workspace_bytes(w.B, w.h_q, w.h_kv, w.d, w.dec_max_context_len),
                     dtype=torch.uint8, device=dev)
    out_a = ops.paged_decode_attention(q, *pools[0], tbl, lens, w.dec_max_context_len,
                                       scale=w.scale)
    out_b = torch.empty_like(q)
    dec = ops.bind_decode(q, *pools[1], tbl, lens, w.dec_max_context_len, out_b, ws,
                          scale=w.scale)
    out_b.zero_()
    dec()
    pre_a = ops.paged_prefill_attention(w.pre_q.to(dev), w.pre_cu_seqlens.to(dev), *pools[0],
                                        w.pre_block_tables.to(dev), w.pre_context_lens.to(dev),
                                        w.pre_max_q_len, scale=w.scale)
    pre_b = ops.bind_prefill(w.pre_q.to(dev), w.pre_cu_seqlens.to(dev), *pools[1],
                             w.pre_block_tables.to(dev), w.pre_context_lens.to(dev),
                             w.pre_max_q_len, scale=w.scale)()
    torch.cuda.synchronize()
    for a, b in zip(pools[0], pools[1]):
        assert torch.equal(bits(a.cpu()), bits(b.cpu()))
    assert torch.equal(bits(out_a.cpu()), bits(out_b.cpu()))
    assert torch.equal(bits(pre_a.cpu()), bits(pre_b.cpu()))
