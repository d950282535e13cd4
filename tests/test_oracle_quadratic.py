"""Pins of the oracle's quadratic self-speculation (CPU only).

The pages name the variant and give its tokens-per-forward figure but no
algorithm; the oracle's reading is one forward that verifies the block
causally and drafts a candidate next block for every accept length.  What
pins that reading's arithmetic:

* The masked forward with the block-attention visibility is the plain block
  forward, bit for bit (row-independent oracle): the general routine reduces
  to the pinned one.
* The verify rows of a quadratic forward equal a plain ``verify_block``, bit
  for bit.
* Candidate k equals, bit for bit, the bidirectional forward of [MASK x B]
  after committing block rows 0..k through a causal forward: the mask, the
  positions and the prefix of every candidate are checked against a separate
  computation.
* The stream equals greedy AR (the temperature-0 identity of
  self-speculation), for several block sizes, and each cycle costs one
  forward.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W

TINY = W.SHAPES["tiny"]


@pytest.fixture(scope="module")
def tiny():
    return O.OracleModel(TINY, W.make_weights(TINY, seed=0), row_independent=True)


def test_masked_attention_reduces_to_block_attention():
    rng = np.random.default_rng(5)
    n, T, Hq, Hkv, hd = 7, 5, 4, 2, 16
    q = rng.normal(size=(T, Hq, hd))
    K, V = rng.normal(size=(n + T, Hkv, hd)), rng.normal(size=(n + T, Hkv, hd))
    for mode in (O.CAUSAL, O.BIDIR):
        vis = O.visible(n, T, mode)
        for ri in (False, True):
            np.testing.assert_array_equal(O.attention_masked(q, K, V, vis, ri), O.attention(q, K, V, n, mode, ri))
    # a row that sees a single key returns that key's value
    vis = np.zeros((T, n + T), dtype=bool)
    vis[np.arange(T), 3 + np.arange(T)] = True
    o = O.attention_masked(q, K, V, vis)
    for i in range(T):
        np.testing.assert_allclose(o[i, 0], V[3 + i, 0], rtol=0, atol=1e-15)


def test_forward_masked_reduces_to_forward(tiny):
    p = W.prompt_ids(TINY, 16, seed=0)
    for mode in (O.CAUSAL, O.BIDIR):
        a, b = tiny.new_cache(), tiny.new_cache()
        tiny.forward(a, p, O.CAUSAL)
        tiny.forward(b, p, O.CAUSAL)
        a.n = b.n = len(p)
        blk = W.prompt_ids(TINY, 8, seed=1)
        want = tiny.forward(a, blk, mode)
        got = tiny.forward_masked(b, blk, len(p) + np.arange(8), O.visible(len(p), 8, mode), n_write=8)
        np.testing.assert_array_equal(got, want)
        for l in range(TINY.n_layers):
            np.testing.assert_array_equal(a.K[l][:24], b.K[l][:24])
            np.testing.assert_array_equal(a.V[l][:24], b.V[l][:24])


def _state(tiny, prompt, B):
    sess = O.OracleSession(tiny)
    first = sess.prefill(0, prompt)
    blk, _ = sess.draft_block(0, int(first.tok[0]), B)
    return sess, blk


@pytest.mark.parametrize("B", [8, 5])
def test_quadratic_rows_equal_separate_forwards(tiny, B):
    prompt = W.prompt_ids(TINY, 16, seed=0)
    sess, blk = _state(tiny, prompt, B)
    a, L, nxt, vsel, cands = sess.verify_block_quadratic(0, blk)
    assert sorted(cands) == list(range(B))
    # the verify rows: a plain verify_block
    ref, _ = _state(tiny, prompt, B)
    ra, rL, rsel = ref.verify_block(0, blk)
    np.testing.assert_array_equal(vsel.logits, rsel.logits)
    assert L == rL and np.array_equal(a, ra)
    # candidate k: commit block rows 0..k causally, then a bidirectional [MASK x B]
    for k in range(B):
        ref, _ = _state(tiny, prompt, B)
        ref.verify_block(0, blk)
        ref.commit_kv(0, k + 1)
        c = ref._cache(0)
        want = tiny.forward(c, np.full(B, TINY.mask_id), O.BIDIR)
        np.testing.assert_array_equal(cands[k].logits, want)
        assert nxt[k, 0] == a[k]
        np.testing.assert_array_equal(nxt[k, 1:], np.argmax(np.where(np.arange(TINY.vocab) == TINY.mask_id,
                                                                     -np.inf, want[1:]), axis=1))
    # a subset of candidates gives the same rows
    _, _, nxt2, _, c2 = _state(tiny, prompt, B)[0].verify_block_quadratic(0, blk, candidates=[B - 1, 0])
    assert sorted(c2) == [0, B - 1]
    for k in (0, B - 1):
        np.testing.assert_array_equal(c2[k].logits, cands[k].logits)
        np.testing.assert_array_equal(nxt2[k], nxt[k])
    assert (nxt2[1:B - 1] == -1).all()


@pytest.mark.parametrize("B", [8, 4, 13])
def test_quadratic_equals_greedy_ar(tiny, B):
    p = W.prompt_ids(TINY, 16, seed=0)
    ar = O.generate_ar(tiny, p, 64)
    q = O.generate_selfspec_quadratic(tiny, p, 64, B)
    assert q.tokens == ar.tokens
    assert q.forwards == 1 + len(q.accept_lengths)       # one draft forward, then one per cycle
    assert all(1 <= L <= B for L in q.accept_lengths)
    lin = O.generate_selfspec(tiny, p, 64, B)
    assert q.tpf > lin.tpf                                  # no draft forward per cycle


def test_quadratic_forced_schedule(tiny):
    """Forced accept lengths take the candidate of the forced length: the
    stream is the block's first L tokens then a_{L-1}, and the next block is
    that candidate's."""
    p = W.prompt_ids(TINY, 16, seed=0)
    B = 8
    forced = [3, 8, 1, 5, 2, 7]
    q = O.generate_selfspec_quadratic(tiny, p, 1 + sum(forced), B, forced=forced)
    assert q.accept_lengths == forced
    sess, blk = _state(tiny, p, B)
    toks = [int(blk[0])]
    for L in forced:
        a, _, nxt, _, _ = sess.verify_block_quadratic(0, blk)
        sess.commit_kv(0, L)
        toks += [int(t) for t in blk[1:L]] + [int(a[L - 1])]
        blk = nxt[L - 1]
        assert blk[0] == a[L - 1]
    assert q.tokens == toks
