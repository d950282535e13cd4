"""Pins of the oracle's decoding modes (CPU only).

The pages fix one exact identity: self-speculation at temperature 0 emits the
greedy AR stream token for token (fintech-frontier-insights, self-speculation
bullet and accuracy list).  The rest is pinned by special cases of the rules
and by brute force.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W

TINY = W.SHAPES["tiny"]


@pytest.fixture(scope="module")
def tiny():
    w = W.make_weights(TINY, seed=0)
    return O.OracleModel(TINY, w, row_independent=True)


@pytest.fixture(scope="module")
def prompt():
    return W.prompt_ids(TINY, 16, seed=0)


@pytest.fixture(scope="module")
def ar64(tiny, prompt):
    return O.generate_ar(tiny, prompt, 64)


# -- I1: self-spec == AR ---------------------------------------------------------
@pytest.mark.parametrize("B", [8, 2, 5, 16])
def test_selfspec_equals_ar(tiny, prompt, ar64, B):
    ss = O.generate_selfspec(tiny, prompt, 64, B)
    assert ss.tokens == ar64.tokens
    assert all(1 <= L <= B for L in ss.accept_lengths)


def test_selfspec_equals_ar_second_seed():
    w = W.make_weights(TINY, seed=11, gains="random")
    m = O.OracleModel(TINY, w, row_independent=True)
    p = W.prompt_ids(TINY, 9, seed=11)
    assert O.generate_selfspec(m, p, 40, 8).tokens == O.generate_ar(m, p, 40).tokens


# -- I2 perfect draft, I3 planted mismatch, I4 B = 1 ------------------------------------
def test_perfect_draft_accepts_whole_block(tiny, prompt, ar64):
    B = 8
    sess = O.OracleSession(tiny, keep_logits=False)
    y = ar64.tokens
    first = sess.prefill(0, prompt)
    assert int(first.tok[0]) == y[0]
    emitted = [y[0]]
    for _ in range(4):
        t = len(emitted)
        block = np.array(y[t - 1: t - 1 + B], dtype=np.int32)   # [anchor, the true continuation]
        a, L, _ = sess.verify_block(0, block)
        assert L == B
        np.testing.assert_array_equal(a[:-1], block[1:])
        sess.commit_kv(0, L)
        emitted += list(block[1:]) + [int(a[-1])]
    assert emitted == y[: len(emitted)]


@pytest.mark.parametrize("j", [1, 2, 5, 7])
def test_planted_mismatch_sets_accept_length(tiny, prompt, ar64, j):
    B = 8
    sess = O.OracleSession(tiny, keep_logits=False)
    sess.prefill(0, prompt)
    block = np.array(ar64.tokens[:B], dtype=np.int32)
    block[j] = (block[j] + 1) % (TINY.vocab - 1)
    _, L, _ = sess.verify_block(0, block)
    assert L == j


def test_block_of_one_is_ar(tiny, prompt, ar64):
    ss = O.generate_selfspec(tiny, prompt, 30, 1)
    assert ss.tokens == ar64.tokens[:30] and set(ss.accept_lengths) == {1}


def test_accept_length_brute_force():
    r = np.random.default_rng(0)
    for _ in range(500):
        B = int(r.integers(1, 12))
        blk = r.integers(0, 3, B)
        a = r.integers(0, 3, B)
        L = 1
        for k in range(B - 1, 0, -1):               # largest k whose whole prefix matches
            if all(blk[j] == a[j - 1] for j in range(1, k + 1)):
                L = k + 1
                break
        assert O.accept_length(blk, a) == L


# -- the forced schedule -------------------------------------------------------------
def test_forced_schedule(tiny, prompt):
    sched = W.forced_accept_schedule(40, 8, seed=0)
    assert sched.min() >= 1 and sched.max() <= 8
    r = O.generate_selfspec(tiny, prompt, 64, 8, forced=sched)
    assert r.accept_lengths == list(sched[: len(r.accept_lengths)])
    assert sum(r.accept_lengths[:-1]) + 1 < 64 <= sum(r.accept_lengths) + 1
    big = W.forced_accept_schedule(100000, 32, seed=0)
    assert set(np.unique(big)) == set(range(1, 33)) and abs(big.mean() - 16.5) < 0.1


# -- unmask rule ---------------------------------------------------------------------
def _unmask_brute(block, tok, conf, tau, force, mask):
    out = list(block)
    masked = [i for i in range(len(block)) if block[i] == mask]
    if not masked:
        return out, 0
    chosen = set()
    if force:
        chosen = set(masked)
    else:
        best = masked[0]
        for i in masked:
            if conf[i] > conf[best]:
                best = i
        chosen.add(best)
        for i in masked:
            if conf[i] > tau:
                chosen.add(i)
    for i in chosen:
        out[i] = tok[i]
    return out, len(masked) - len(chosen)


def test_unmask_rule_brute_force():
    r = np.random.default_rng(1)
    mask = 99
    for _ in range(2000):
        B = int(r.integers(1, 10))
        block = np.where(r.random(B) < 0.6, mask, r.integers(0, 99, B)).astype(np.int32)
        tok = r.integers(0, 99, B).astype(np.int32)
        conf = np.round(r.random(B), 1)                   # many exact ties
        tau = float(r.choice([0.0, 0.3, 0.5, 0.9, 1.0, 1.5]))
        force = bool(r.random() < 0.2)
        got, _, left = O.unmask_rule(block, tok, conf, tau, force, mask)
        exp, eleft = _unmask_brute(block, tok, conf, tau, force, mask)
        assert list(got) == exp and left == eleft


# -- I5: threshold special cases, step bounds ---------------------------------------------
def test_tau_above_one_unmasks_one_per_step(tiny, prompt):
    r = O.generate_diffusion(tiny, prompt, 16, 8, tau=1.01)
    assert r.steps_per_block == [8, 8]


def test_tau_zero_equals_one_shot_fill(tiny, prompt):
    sess = O.OracleSession(tiny)
    sess.prefill(0, prompt)
    blk = np.full(8, TINY.mask_id, dtype=np.int32)
    new, U, left, sel = sess.diffuse_step(0, blk, 0.0, False)
    assert left == 0 and len(U) == 8
    np.testing.assert_array_equal(new, sel.tok)          # every row's argmax at once
    # the same fill happens with any tau below the smallest possible max-confidence 1/(V-1)
    new2, _, left2, _ = sess.diffuse_step(0, blk, 0.999 / (TINY.vocab - 1), False)
    assert left2 == 0 and np.array_equal(new, new2)


@pytest.mark.parametrize("tau,S", [(0.9, None), (0.9, 3), (0.0045, None), (0.0045, 2), (0.0, 5)])
def test_step_count_bounds(tiny, prompt, tau, S):
    r = O.generate_diffusion(tiny, prompt, 24, 8, tau=tau, max_steps=S)
    for s in r.steps_per_block:
        assert 1 <= s <= min(8, S or 8)
    assert len(r.tokens) == 24 and TINY.mask_id not in r.tokens


def test_step_cap_forces_all():
    mask = 9
    block = np.full(6, mask, dtype=np.int32)
    tok = np.arange(6, dtype=np.int32)
    conf = np.full(6, 0.01)
    new, U, left = O.unmask_rule(block, tok, conf, 0.9, True, mask)
    assert left == 0 and list(new) == list(range(6))


# -- revision (remasking) variant of diffusion ---------------------------------------------
def test_revise_rule_planted():
    mask = 9
    block = np.array([3, mask, 5, 5, 7, 1], dtype=np.int32)
    tok = np.array([4, 2, 5, 6, 8, 0], dtype=np.int32)
    conf = np.array([0.95, 0.99, 0.99, 0.5, 0.95, 0.9], dtype=np.float64)
    # position 0: differs, conf 0.95 > 0.9 -> revised; 1: masked (never revised); 2: same token;
    # 3: differs but conf 0.5; 4: differs, 0.95 -> revised; 5: differs, conf exactly tau (strict >) -> kept
    new, R = O.revise_rule(block, tok, conf, 0.9, mask)
    assert list(R) == [0, 4]
    assert list(new) == [4, mask, 5, 5, 8, 1]
    new1, R1 = O.revise_rule(block, tok, np.ones(6), 1.0, mask)     # conf <= 1: tau 1 revises nothing
    assert len(R1) == 0 and list(new1) == list(block)


def test_revise_rule_brute_force():
    r = np.random.default_rng(2)
    mask = 99
    for _ in range(2000):
        B = int(r.integers(1, 10))
        block = np.where(r.random(B) < 0.4, mask, r.integers(0, 6, B)).astype(np.int32)
        tok = r.integers(0, 6, B).astype(np.int32)                # small alphabet: many equal tokens
        conf = np.round(r.random(B), 1)
        tau = float(r.choice([0.0, 0.3, 0.5, 0.9, 1.0]))
        got, R = O.revise_rule(block, tok, conf, tau, mask)
        exp = list(block)
        rev = []
        for i in range(B):
            if block[i] != mask and tok[i] != block[i] and conf[i] > tau:
                exp[i] = tok[i]
                rev.append(i)
        assert list(got) == exp and list(R) == rev


def test_diffuse_step_revise_decides_on_the_block_before_the_step(tiny, prompt):
    """Masked positions follow the unmask rule, written ones the revise rule,
    both from the same forward; with tau_revise >= 1 it is the plain step."""
    sess = O.OracleSession(tiny)
    sess.prefill(0, prompt)
    blk = np.full(8, TINY.mask_id, dtype=np.int32)
    blk[[1, 4, 6]] = [3, 17, 200]
    new_p, U_p, left_p, sel_p = sess.diffuse_step(0, blk, 0.0045, False)
    new_1, U_1, R_1, left_1, sel_1 = sess.diffuse_step_revise(0, blk, 0.0045, 1.0, False)
    assert len(R_1) == 0 and np.array_equal(new_p, new_1) and left_p == left_1
    np.testing.assert_array_equal(sel_p.logits, sel_1.logits)
    new, U, R, left, sel = sess.diffuse_step_revise(0, blk, 0.0045, 0.0, False)
    assert set(R) == {i for i in (1, 4, 6) if sel.tok[i] != blk[i]} and len(R) > 0
    for i in range(8):
        if blk[i] == TINY.mask_id:
            assert new[i] == new_p[i]                          # unmask rule untouched
        else:
            assert new[i] == (sel.tok[i] if i in R else blk[i])


def test_diffusion_with_revision(tiny, prompt):
    plain = O.generate_diffusion(tiny, prompt, 24, 8, tau=0.0045)
    off = O.generate_diffusion(tiny, prompt, 24, 8, tau=0.0045, tau_revise=1.0)
    assert off.tokens == plain.tokens and off.revisions == [0, 0, 0]
    on = O.generate_diffusion(tiny, prompt, 24, 8, tau=1.01, tau_revise=0.0)   # one unmask per step
    assert sum(on.revisions) > 0 and on.steps_per_block == [8, 8, 8]
    assert len(on.tokens) == 24 and TINY.mask_id not in on.tokens
    for s in on.steps_per_block:
        assert 1 <= s <= 8


# -- I6: committed cache equals a fresh prefill -------------------------------------------
def test_commit_equals_fresh_prefill(tiny, prompt):
    sess = O.OracleSession(tiny, keep_logits=False)
    g = int(sess.prefill(0, prompt).tok[0])
    sched = [3, 1, 8, 5]
    committed = list(prompt)
    for L in sched:
        blk, _ = sess.draft_block(0, g, 8)
        a, _, _ = sess.verify_block(0, blk)
        sess.commit_kv(0, L)
        committed += [int(t) for t in blk[:L]]
        g = int(a[L - 1])
    c = sess.caches[0]
    assert c.n == len(committed)
    fresh = tiny.new_cache()
    tiny.forward(fresh, committed, O.CAUSAL)
    for l in range(TINY.n_layers):
        np.testing.assert_array_equal(c.K[l][: c.n], fresh.K[l][: c.n])
        np.testing.assert_array_equal(c.V[l][: c.n], fresh.V[l][: c.n])


def test_diffusion_batch_is_per_sequence(tiny):
    prompts = [W.prompt_ids(TINY, n, seed=0, index=i) for i, n in enumerate([5, 12, 9])]
    batch = O.generate_diffusion_batch(tiny, prompts, 16, 8, 0.9, 3)
    for i, p in enumerate(prompts):
        assert batch[i].tokens == O.generate_diffusion(tiny, p, 16, 8, 0.9, 3).tokens


def test_golden_tiny_streams_current(tiny, prompt):
    """The stored tiny-config streams (written by tests/golden/make_golden.py
    from the oracle) are what the oracle produces now."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_streams.json")))
    assert g["prompt"] == [int(t) for t in prompt]
    assert O.generate_ar(tiny, prompt, 64).tokens == g["ar"] == g["selfspec"]
    assert O.generate_diffusion(tiny, prompt, 64, 8, 0.9).tokens == g["diffusion"]
