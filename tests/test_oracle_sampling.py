"""Pins of the oracle's sampling at temperature > 0 (CPU only).

* Philox4x64-10 equals numpy's implementation of the same generator (numpy
  advances the counter before each block).
* The uniforms are the stated 24-bit grid in (0, 1).
* Gumbel-max draws follow softmax(l / T) (chi-square over many counters).
* One speculative position -- draft from q, accept with probability
  min(1, p/q), else a residual draw -- emits tokens distributed as p, the
  property that makes the verify lossless (chi-square); the closed form of
  the rule gives p exactly.
* As T -> 0, sampled AR and sampled self-speculation reduce to greedy AR.
"""
import numpy as np
import pytest
from scipy import stats

import oracle as O
import workloads as W
from oracle import sampling as SP

TINY = W.SHAPES["tiny"]


def test_philox_matches_numpy():
    for seed in (0, 99, 2 ** 63 + 5):
        for ctr in ([4, 77, 3, 2], [0, 0, 0, 0], [2 ** 64 - 2, 1, 2, 3]):
            g = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array([seed, 0], dtype=np.uint64))
            raw = [int(x) for x in g.random_raw(4)]
            nxt = [(ctr[0] + 1) % 2 ** 64] + ctr[1:]
            assert raw == SP.philox4x64_10(nxt, (seed, 0))
    arr = SP.philox_block_array(np.arange(9), 1234, 5, SP.PURPOSE_RESIDUAL, 42)
    for i in range(9):
        assert [int(x) for x in arr[i]] == SP.philox4x64_10((i, 1234, 5, SP.PURPOSE_RESIDUAL), (42, 0))


def test_uniform24_grid():
    x = np.array([0, 2 ** 40 - 1, 2 ** 64 - 1, 12345 << 40], dtype=np.uint64)
    u = SP.uniform24(x)
    np.testing.assert_array_equal(u, [0.5 * 2 ** -24, 0.5 * 2 ** -24, 1 - 0.5 * 2 ** -24, (12345 + 0.5) * 2 ** -24])
    v = SP.uniform24(SP.philox_block_array(np.arange(5000), 3, 1, 1, 7).reshape(-1))
    assert v.min() > 0 and v.max() < 1 and abs(v.mean() - 0.5) < 0.01
    np.testing.assert_array_equal((v * 2 ** 24 - 0.5) % 1, 0)


def _chi2_p(counts, probs):
    exp = probs * counts.sum()
    return stats.chisquare(counts, exp).pvalue


def test_gumbel_max_follows_softmax():
    logits = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4, 5.0])     # id 6 plays MASK
    mask, T = 6, 0.7
    p = np.exp(SP.log_softmax_T(logits, T, mask))
    assert p[mask] == 0
    counts = np.zeros(7)
    for pos in range(10000):
        s = SP.sample_row(logits, T, seed=11, seq=0, position=pos, purpose=SP.PURPOSE_SAMPLE, mask_id=mask)
        counts[s.tok] += 1
        assert abs(s.logp - np.log(p[s.tok])) < 1e-12
    assert counts[mask] == 0
    assert _chi2_p(counts[:6], p[:6]) > 1e-3


def test_speculative_position_is_lossless():
    rng = np.random.default_rng(3)
    V, mask, T = 8, 7, 0.9
    pl, ql = rng.normal(size=V) * 1.5, rng.normal(size=V) * 1.5
    p = np.exp(SP.log_softmax_T(pl, T, mask))
    q = np.exp(SP.log_softmax_T(ql, T, mask))
    # closed form of the rule: accept d with min(1, p/q), else draw from max(0, p - q)
    acc = np.minimum(q, p)
    resid = np.maximum(p - q, 0)
    np.testing.assert_allclose(acc + (1 - acc.sum()) * resid / resid.sum(), p, rtol=0, atol=1e-15)
    # the implementation, over many counters
    counts, drafts = np.zeros(V), np.zeros(V)
    for pos in range(12000):
        d = SP.sample_row(ql, T, 5, 1, pos, SP.PURPOSE_DRAFT, mask)
        drafts[d.tok] += 1
        ok, _ = SP.accept_draft(float(np.log(p[d.tok])), d.logp, 5, 1, pos)
        tok = d.tok if ok else SP.residual_sample(pl, ql, T, 5, 1, pos, mask).tok
        counts[tok] += 1
    assert counts[mask] == 0
    assert _chi2_p(counts[:7], p[:7]) > 1e-3
    # the same test rejects the drafts themselves (it can tell q from p)
    assert _chi2_p(drafts[:7], p[:7]) < 1e-9


@pytest.fixture(scope="module")
def tiny():
    return O.OracleModel(TINY, W.make_weights(TINY, seed=0), row_independent=True)


def test_temperature_to_zero_is_greedy(tiny):
    p = W.prompt_ids(TINY, 16, seed=0)
    g = O.generate_ar(tiny, p, 40)
    assert O.generate_ar_sample(tiny, p, 40, 1e-6, 7).tokens == g.tokens
    assert O.generate_selfspec_sample(tiny, p, 40, 8, 1e-6, 7).tokens == g.tokens


def test_sampled_streams_depend_on_the_seed(tiny):
    p = W.prompt_ids(TINY, 16, seed=0)
    a = O.generate_selfspec_sample(tiny, p, 40, 8, 0.8, 1)
    b = O.generate_selfspec_sample(tiny, p, 40, 8, 0.8, 1)
    c = O.generate_selfspec_sample(tiny, p, 40, 8, 0.8, 2)
    assert a.tokens == b.tokens and a.tokens != c.tokens
    assert all(1 <= L <= 8 for L in a.accept_lengths)
