"""CPU pins of the schedule-independent bound on the 8-bit attention (tests/q8_bound.py): the oracle's
blocked online attention_q8 (lazy reference max, E4M3 probabilities on the 224 scale) satisfies it at
ordinary and at large score spreads, and the same schedule with one planted mistake -- the output not
rescaled when the reference max moves, or the probabilities normalised by their unrounded sum with a
2x error on one block -- does not, so the GPU check built on it can see such mistakes."""
import math

import numpy as np
import pytest

import oracle as O
from tests.q8_bound import exact_on_quantized


def _online(q, k, v, skip_rescale=False, bad_block=None):
    """The oracle's schedule written out for one head, with optional planted mistakes."""
    qc, qa = O.q8_quantize_q(q)
    kc, ka = O.q8_quantize_k(k)
    vc, va = O.fp8_quantize_v(v)
    vh = vc * (va / O.E4M3_MAX)[None, :]
    S, blk = k.shape[0], O.Q8_KEY_BLOCK
    m = np.full(q.shape[0], -np.inf)
    o = np.zeros((q.shape[0], 128))
    lsum = np.zeros(q.shape[0])
    for t in range((S + blk - 1) // blk):
        ks = slice(t * blk, min((t + 1) * blk, S))
        s = (qc @ kc[ks].T) * (qa / 127.0)[:, None] * (ka[t] / 127.0) / math.sqrt(128.0)
        mx = s.max(axis=1)
        with np.errstate(invalid="ignore"):
            move = ~np.isfinite(m) | ((mx - m) / math.log(2.0) > 1.0)
        m_new = np.where(move, mx, m)
        alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        p = O.e4m3_round(np.exp(s - m_new[:, None]) * O.Q8_P_SCALE) / O.Q8_P_SCALE
        if bad_block == t:
            p = 2.0 * p
        o = (o if skip_rescale else o * alpha[:, None]) + p @ vh[ks]
        lsum = lsum * alpha + p.sum(axis=1) / (2.0 if bad_block == t else 1.0)
        m = m_new
    return o / lsum[:, None]


def _inputs(seed, amp, S=300, rows=40):
    rng = np.random.default_rng(seed)
    q = O.bf16_round(rng.standard_normal((rows, 128)) * amp)
    k = O.bf16_round(rng.standard_normal((S, 128)) * amp)
    v = O.bf16_round(rng.standard_normal((S, 128)))
    return q, k, v


@pytest.mark.parametrize("amp", [1.0, 4.0])
def test_oracle_attention_q8_within_bound(amp):
    q, k, v = _inputs(7, amp)
    ref, bound = exact_on_quantized(q, k, v)
    got = O.attention_q8(q, k, v, 1, 128)
    assert np.all(np.abs(got - ref) <= bound)
    # the schedule written out here is the oracle's
    np.testing.assert_allclose(_online(q, k, v), got, rtol=1e-12, atol=1e-12)


def test_planted_schedule_mistakes_break_bound():
    q, k, v = _inputs(8, 4.0)                     # large spread: the reference max moves often
    ref, bound = exact_on_quantized(q, k, v)
    for kw in ({"skip_rescale": True}, {"bad_block": 2}):
        got = _online(q, k, v, **kw)
        assert np.any(np.abs(got - ref) > bound), kw
