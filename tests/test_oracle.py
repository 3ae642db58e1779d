"""Pins of the CPU oracle (no GPU): brute force, a library special case, closed
forms and the invariants the pages state.  The mutation tests plant one
plausible mistake at a time in an oracle helper and require a pin to fail."""
import numpy as np
import pytest

import oracle.attention as O
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_brute_decode_gqa7():
    pins.check_brute_decode(seed=21, dec_lens=(3, 18, 49), h_q=14, h_kv=2, d=4)


def test_brute_prefill_chunked_many():
    pins.check_brute_prefill(seed=22, prefill=((33, 33), (50, 17), (17, 1), (1, 1)), h_q=4, h_kv=4, d=4)


def test_zero_context_gives_zeros():
    w = pins.tiny_workload(23, dec_lens=(5,))
    kc, vc = pins.appended_pools(w)
    out = O.decode(pins.np64(w.dec_q), kc, vc, w.dec_block_tables.numpy(), np.array([0]), w.scale)
    assert np.array_equal(out, np.zeros_like(out))


def test_config1_matches_brute_and_has_block_boundary():
    w = pins.W.config(1)
    # context 17: the appended token is the first slot of its sequence's second block
    assert sorted(w.dec_context_lens.tolist()) == [17, 40]
    assert int(w.slot_mapping[0]) % 16 == 0
    assert w.n_blocks == 16


def _bad_kv_head_of(h, h_q, h_kv):
    return h % h_kv


def _bad_slot_to_block(slot):
    return (slot + 1) // 16, (slot + 1) % 16


def _bad_key_limit_exclusive(L, n, i):
    return L - n + i


def _bad_key_limit_topleft(L, n, i):
    return i + 1


def _bad_gather_offset(cache, table_row, L):
    h_kv, d = cache.shape[1], cache.shape[3]
    out = np.empty((L, h_kv, d))
    for t in range(L):
        out[t] = cache[int(table_row[t % 16 if t % 16 < len(table_row) else 0]), :, t // 16 % 16, :]
    return out


def _bad_gather_shift(cache, table_row, L):
    h_kv, d = cache.shape[1], cache.shape[3]
    out = np.empty((L, h_kv, d))
    for t in range(L):
        out[t] = cache[int(table_row[(t + 1) // 16]) if (t + 1) // 16 < len(table_row) else 0, :, (t + 1) % 16, :]
    return out


def _bad_scores_noscale(keys, queries, scale):
    return queries @ keys.T


def _bad_scores_transposed(keys, queries, scale):
    return scale * (queries[:, ::-1] @ keys.T)


def _bad_softmax_unnormalised(scores, values):
    if scores.shape[0] == 0:
        return np.zeros(values.shape[1])
    return np.exp(scores - scores.max()) @ values


def _bad_softmax_mean(scores, values):
    if scores.shape[0] == 0:
        return np.zeros(values.shape[1])
    w = np.exp(scores - scores.max())
    return (w @ values) / len(w)


def _bad_softmax_negated(scores, values):
    if scores.shape[0] == 0:
        return np.zeros(values.shape[1])
    w = np.exp(-(scores - scores.min()))
    return (w @ values) / w.sum()


MUTANTS = {
    "gqa-modulo": ("kv_head_of", _bad_kv_head_of),
    "slot-off-by-one": ("slot_to_block", _bad_slot_to_block),
    "causal-exclusive": ("key_limit", _bad_key_limit_exclusive),
    "causal-top-left": ("key_limit", _bad_key_limit_topleft),
    "gather-swapped-index": ("gather_sequence", _bad_gather_offset),
    "gather-shifted": ("gather_sequence", _bad_gather_shift),
    "scores-no-scale": ("dot_scores", _bad_scores_noscale),
    "scores-transposed-operand": ("dot_scores", _bad_scores_transposed),
    "softmax-unnormalised": ("softmax_weighted_sum", _bad_softmax_unnormalised),
    "softmax-mean": ("softmax_weighted_sum", _bad_softmax_mean),
    "softmax-sign": ("softmax_weighted_sum", _bad_softmax_negated),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(O, attr, bad)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
