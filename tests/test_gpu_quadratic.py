"""GPU parity of quadratic self-speculation (``sdm_verify_block_quadratic``:
one forward of B + B^2 rows verifies the block and drafts a candidate next
block for every accept length) against the oracle.

* tiny float32 decoder (B = 8, 5, 13): whole token streams, natural and
  forced, equal the oracle's; call by call every row's logits agree within
  1e-4 and the next blocks are the oracle's.
* small bf16 decoder (2 layers, d 256, B = 32: 1056 rows, pages straddled by
  the block): lockstep cycles, logits within 2e-2, next-block tokens equal
  except near-ties; the GPU quadratic stream equals the GPU AR stream
  exactly, because its verify rows are computed as the linear verify's.
* 8B shape in the benchmark's quadratic launch configuration: one cycle, the
  verify rows and three sampled candidates against the oracle.
* 4-bit weights: one lockstep cycle.
* Argument and state errors change nothing.

Near-tie exemptions follow the lockstep rules: a token may differ only where
the oracle's top-2 margin is below max(1e-3, 2 x the row's logit deviation).
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from lockstep import Report, accept_exempt, tokens_agree

pytestmark = pytest.mark.gpu
DEV = "cuda"
TINY = W.SHAPES["tiny"]
SMALL = W.ModelShape("small-bf16", 2, 256, 4, 2, 128, 512, 1024, "bf16")


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _quad_lockstep(gm, sess, seq, blk, B, rep, lg, L_forced=None, cands=None):
    """One quadratic forward on both sides from the same block; compares the
    verify rows, the accept length and the listed candidates (all when None).
    Commits L on both sides and returns (the oracle's next block, L)."""
    ar = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    nx = torch.full((B, B), -7, dtype=torch.int32, device=DEV)
    gm.verify_block_quadratic(seq, _i32(blk), B, ar, acc, nx, lg)
    oa, oL, onx, vsel, csel = sess.verify_block_quadratic(0, blk, candidates=cands)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:B], vsel.logits)
    gar = ar.cpu().numpy()
    assert tokens_agree(gar, vsel, range(B), rep, eps), rep.notes
    gL = int(acc.item())
    if gL != oL:
        assert accept_exempt(vsel, gL, oL, rep), rep.notes
        rep.resync()
    gnx = nx.cpu().numpy()
    assert np.array_equal(gnx[:, 0], gar)          # row k starts with the GPU's own a_k
    for k, cs in csel.items():
        ceps = rep.logits(lg[B * (1 + k):B * (2 + k)], cs.logits)
        assert tokens_agree(np.r_[0, gnx[k, 1:]], cs, range(1, B), rep, ceps), (k, rep.notes)
    L = oL if L_forced is None else L_forced
    gm.commit_kv(seq, L)
    sess.commit_kv(0, L)
    return onx[L - 1].copy(), L


# -- tiny float32 --------------------------------------------------------------
@pytest.fixture(scope="module")
def tiny_gm():
    from self_speculative_amd.model import Model
    m = Model(TINY, W.make_weights(TINY, seed=0), max_seqs=8, max_block=16, max_context=512, max_rows=272)
    yield m
    m.close()


@pytest.fixture(scope="module")
def tiny_om():
    return O.OracleModel(TINY, W.make_weights(TINY, seed=0), row_independent=True)


@pytest.mark.parametrize("B", [8, 5, 13])
def test_tiny_quadratic_streams(tiny_gm, tiny_om, B):
    from self_speculative_amd import decode as D
    p = W.prompt_ids(TINY, 16, seed=0)
    print(f"tiny quadratic streams B={B}", flush=True)
    tiny_gm.seq_reset(0)
    g = D.generate_selfspec_quadratic(tiny_gm, p, 64, B, seq=0)
    o = O.generate_selfspec_quadratic(tiny_om, p, 64, B)
    assert g.tokens == o.tokens and g.accept_lengths == o.accept_lengths
    assert g.tokens == O.generate_ar(tiny_om, p, 64).tokens
    forced = [int(x) for x in np.random.default_rng(B).integers(1, B + 1, size=64)]
    tiny_gm.seq_reset(1)
    gf = D.generate_selfspec_quadratic(tiny_gm, p, 64, B, forced=forced, seq=1)
    of = O.generate_selfspec_quadratic(tiny_om, p, 64, B, forced=forced)
    assert gf.tokens == of.tokens and gf.accept_lengths == of.accept_lengths


def test_tiny_quadratic_extreme_blocks(tiny_om):
    """The smallest block (B = 2) and the largest (B = 63: 64 slots, 4032-row
    forwards): streams equal the oracle's, natural and forced."""
    from self_speculative_amd import decode as D
    from self_speculative_amd.model import Model
    m = Model(TINY, W.make_weights(TINY, seed=0), max_seqs=2, max_block=63, max_context=512, max_rows=63 * 64)
    try:
        p = W.prompt_ids(TINY, 16, seed=0)
        for B, n, forced in ((2, 24, [2, 1, 2, 2, 1, 2]), (63, 6, [63, 1, 40])):
            print(f"tiny quadratic B={B}", flush=True)
            m.seq_reset(0)
            g = D.generate_selfspec_quadratic(m, p, n, B, seq=0)
            o = O.generate_selfspec_quadratic(tiny_om, p, n, B)
            assert g.tokens == o.tokens and g.accept_lengths == o.accept_lengths, B
            m.seq_reset(1)
            nf = 1 + sum(forced)
            gf = D.generate_selfspec_quadratic(m, p, nf, B, forced=forced, seq=1)
            of = O.generate_selfspec_quadratic(tiny_om, p, nf, B, forced=forced)
            assert gf.tokens == of.tokens, B
    finally:
        m.close()


def test_tiny_quadratic_lockstep_rows(tiny_gm, tiny_om):
    B = 8
    seq = 2
    tiny_gm.seq_reset(seq)
    p = W.prompt_ids(TINY, 61, seed=3)                 # the blocks straddle the first page boundary
    sess = O.OracleSession(tiny_om)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    tiny_gm.prefill(seq, _i32(p), nxt)
    g = int(sess.prefill(0, p).tok[0])
    assert int(nxt.item()) == g
    blk = torch.empty(B, dtype=torch.int32, device=DEV)
    tiny_gm.draft_block(seq, _i32([g]), B, blk)
    oblk, _ = sess.draft_block(0, g, B)
    assert np.array_equal(blk.cpu().numpy(), oblk)
    rep = Report()
    lg = torch.empty((B * (B + 1), TINY.vocab), dtype=torch.float32, device=DEV)
    for cyc, L in enumerate([None, 8, 1, 3, None]):
        print(f"tiny quadratic lockstep cycle {cyc}", flush=True)
        oblk, _ = _quad_lockstep(tiny_gm, sess, seq, oblk, B, rep, lg, L)
    print(f"tiny quadratic: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= 1e-4 and rep.exempt == 0 and rep.resyncs == 0


# -- small bf16 ----------------------------------------------------------------
@pytest.fixture(scope="module")
def small_w():
    return W.make_weights(SMALL, seed=21, gains="random")


@pytest.fixture(scope="module")
def small_gm(small_w):
    from self_speculative_amd.model import Model
    m = Model(SMALL, small_w, max_seqs=4, max_block=32, max_context=1024, max_rows=1056)
    yield m
    m.close()


def test_bf16_quadratic_lockstep(small_gm, small_w):
    B = 32
    seq = 0
    small_gm.seq_reset(seq)
    sess = O.OracleSession(O.OracleModel(SMALL, small_w))
    p = W.prompt_ids(SMALL, 150, seed=22)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    rep = Report()
    lg = torch.empty((B * (B + 1), SMALL.vocab), dtype=torch.float32, device=DEV)
    small_gm.prefill(seq, _i32(p), nxt, lg[:1])
    ref = sess.prefill(0, p)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:1], ref.logits)
    assert tokens_agree(nxt.cpu().numpy(), ref, [0], rep, eps), rep.notes
    g = int(ref.tok[0])
    blk = torch.empty(B, dtype=torch.int32, device=DEV)
    small_gm.draft_block(seq, _i32([g]), B, blk, lg[:B])
    oblk, dsel = sess.draft_block(0, g, B)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:B], dsel.logits)
    assert tokens_agree(np.r_[0, blk.cpu().numpy()[1:]], dsel, range(1, B), rep, eps), rep.notes
    for cyc, L in enumerate([None, 32, 17, 1]):
        print(f"bf16 quadratic lockstep cycle {cyc}", flush=True)
        oblk, _ = _quad_lockstep(small_gm, sess, seq, oblk, B, rep, lg, L)
    print(f"bf16 quadratic: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= 2e-2


def test_bf16_quadratic_largest_block_lockstep(small_w):
    """B = 63: 64 slots and 4032-row forwards (32 activation groups of the
    many-row GEMMs, four placement bands) in lockstep with the oracle."""
    from self_speculative_amd.model import Model
    B = 63
    m = Model(SMALL, small_w, max_seqs=1, max_block=B, max_context=512, max_rows=B * (B + 1))
    try:
        sess = O.OracleSession(O.OracleModel(SMALL, small_w))
        p = W.prompt_ids(SMALL, 70, seed=26)
        nxt = torch.empty(1, dtype=torch.int32, device=DEV)
        m.prefill(0, _i32(p), nxt)
        g = int(sess.prefill(0, p).tok[0])
        blk = torch.empty(B, dtype=torch.int32, device=DEV)
        m.draft_block(0, _i32([g]), B, blk)
        oblk, _ = sess.draft_block(0, g, B)
        rep = Report()
        lg = torch.empty((B * (B + 1), SMALL.vocab), dtype=torch.float32, device=DEV)
        for cyc, L in enumerate([None, 63]):
            print(f"bf16 quadratic B=63 cycle {cyc}", flush=True)
            oblk, _ = _quad_lockstep(m, sess, 0, oblk, B, rep, lg, L)
        print(f"bf16 quadratic B=63: {rep.summary()}", flush=True)
        rep.assert_strict()
        assert rep.max_logit_err <= 2e-2
    finally:
        m.close()


def test_bf16_quadratic_equals_ar_on_gpu(small_gm):
    from self_speculative_amd import decode as D
    p = W.prompt_ids(SMALL, 77, seed=23)
    small_gm.seq_reset(1)
    small_gm.seq_reset(2)
    print("bf16 gpu quadratic vs gpu AR", flush=True)
    ar = D.generate_ar(small_gm, p, 120, seq=1)
    for B in (32, 7):
        small_gm.seq_reset(2)
        q = D.generate_selfspec_quadratic(small_gm, p, 120, B, seq=2)
        assert q.tokens == ar.tokens, B


def test_bf16_quadratic_verify_rows_equal_linear_verify(small_gm):
    """The verify rows of the quadratic forward are the linear verify's, bit
    for bit (logits and outputs), for any block."""
    B = 32
    p = W.prompt_ids(SMALL, 90, seed=24)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    blk = _i32(W.prompt_ids(SMALL, B, seed=25))
    outs = []
    for quad in (False, True):
        small_gm.seq_reset(3)
        small_gm.prefill(3, _i32(p), nxt)
        ar = torch.empty(B, dtype=torch.int32, device=DEV)
        acc = torch.empty(1, dtype=torch.int32, device=DEV)
        lg = torch.empty((B * (B + 1), SMALL.vocab), dtype=torch.float32, device=DEV)
        if quad:
            nx = torch.empty((B, B), dtype=torch.int32, device=DEV)
            small_gm.verify_block_quadratic(3, blk, B, ar, acc, nx, lg)
        else:
            small_gm.verify_block([3], blk, B, ar, acc, lg[:B])
        torch.cuda.synchronize()
        outs.append((ar.cpu().numpy(), int(acc.item()), lg[:B].cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


def test_quadratic_error_paths(small_gm):
    from self_speculative_amd._lib import SDM_ERR_ARG, SDM_ERR_CAPACITY, SDM_ERR_STATE, SdmError
    m = small_gm
    B = 8
    ar = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    nx = torch.empty((B, B), dtype=torch.int32, device=DEV)
    blk = _i32(np.arange(B))
    m.seq_reset(0)

    def expect(status, fn):
        with pytest.raises(SdmError) as e:
            fn()
        assert e.value.status == status

    expect(SDM_ERR_STATE, lambda: m.verify_block_quadratic(0, blk, B, ar, acc, nx))    # no prompt
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    m.prefill(0, _i32([5, 6, 7]), nxt)
    expect(SDM_ERR_ARG, lambda: m.verify_block_quadratic(0, blk, 1, ar, acc, nx))      # B < 2
    expect(SDM_ERR_ARG, lambda: m.verify_block_quadratic(0, blk, 33, ar, acc, nx))     # above max_block
    expect(SDM_ERR_ARG, lambda: m.verify_block_quadratic(0, nx.view(-1)[3:], B, ar, acc, nx))  # overlap
    expect(SDM_ERR_STATE, lambda: m.commit_kv(0, 1))                                   # nothing verified
    assert m.seq_length(0) == 3
    m.verify_block_quadratic(0, blk, B, ar, acc, nx)
    expect(SDM_ERR_ARG, lambda: m.commit_kv(0, B + 1))
    m.commit_kv(0, B)
    assert m.seq_length(0) == 3 + B
    torch.cuda.synchronize()


def test_quadratic_capacity_errors(small_w):
    from self_speculative_amd._lib import SDM_ERR_CAPACITY, SdmError
    from self_speculative_amd.model import Model
    m = Model(SMALL, small_w, max_seqs=1, max_block=32, max_context=128, max_rows=96)
    try:
        nxt = torch.empty(1, dtype=torch.int32, device=DEV)
        m.prefill(0, _i32(np.arange(110)), nxt)
        B = 9                                          # 9 * 10 = 90 rows fit max_rows 96
        ar = torch.empty(B + 1, dtype=torch.int32, device=DEV)
        acc = torch.empty(1, dtype=torch.int32, device=DEV)
        nx = torch.empty((B + 1, B + 1), dtype=torch.int32, device=DEV)
        blk = _i32(np.arange(B + 1))
        with pytest.raises(SdmError) as e:            # 10 * 11 rows > max_rows
            m.verify_block_quadratic(0, blk, B + 1, ar, acc, nx)
        assert e.value.status == SDM_ERR_CAPACITY
        m.verify_block_quadratic(0, blk, B, ar, acc, nx)   # candidates reach position 127 < 128
        m.commit_kv(0, B)
        with pytest.raises(SdmError) as e:            # 119 + 2 * 9 > max_context
            m.verify_block_quadratic(0, blk, B, ar, acc, nx)
        assert e.value.status == SDM_ERR_CAPACITY
        m.verify_block([0], blk, B, ar, acc)           # a linear verify still fits
        torch.cuda.synchronize()
    finally:
        m.close()


# -- 4-bit weights -----------------------------------------------------------------
def test_w4_quadratic_lockstep():
    from self_speculative_amd.model import Model
    w = W.make_w4_weights(SMALL, seed=41, gains="random")
    B = 16
    gm = Model(SMALL, w, max_seqs=1, max_block=B, max_context=512, max_rows=B * (B + 1))
    try:
        sess = O.OracleSession(O.OracleModel(SMALL, w))
        p = W.prompt_ids(SMALL, 100, seed=42)
        nxt = torch.empty(1, dtype=torch.int32, device=DEV)
        gm.prefill(0, _i32(p), nxt)
        g = int(sess.prefill(0, p).tok[0])
        blk = torch.empty(B, dtype=torch.int32, device=DEV)
        gm.draft_block(0, _i32([g]), B, blk)
        oblk, _ = sess.draft_block(0, g, B)
        rep = Report()
        lg = torch.empty((B * (B + 1), SMALL.vocab), dtype=torch.float32, device=DEV)
        for cyc, L in enumerate([None, 16, 5]):
            print(f"w4 quadratic lockstep cycle {cyc}", flush=True)
            oblk, _ = _quad_lockstep(gm, sess, 0, oblk, B, rep, lg, L)
        print(f"w4 quadratic: {rep.summary()}", flush=True)
        rep.assert_strict()
        assert rep.max_logit_err <= 2e-2
    finally:
        gm.close()


# -- 8B ------------------------------------------------------------------------------
def test_8b_quadratic_configuration_cycle():
    from self_speculative_amd.model import Model
    s = W.SHAPES["8b"]
    B = 32
    print("8b quadratic: drawing weights", flush=True)
    w = W.make_weights(s, seed=0)
    prompt = W.prompt_ids(s, 1024, seed=0)
    gm = Model(s, w, max_seqs=1, max_block=B, max_context=4096, max_rows=B * (B + 1))
    om = O.OracleModel(s, w)
    sess = O.OracleSession(om)
    rep = Report()
    lg = torch.empty((B * (B + 1), s.vocab), dtype=torch.float32, device=DEV)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    print("8b quadratic: prefill 1024 (gpu, then oracle)", flush=True)
    gm.prefill(0, _i32(prompt), nxt, lg[:1])
    ref = sess.prefill(0, prompt)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:1], ref.logits)
    assert tokens_agree(nxt.cpu().numpy(), ref, [0], rep, eps), rep.notes
    g = int(ref.tok[0])
    print("8b quadratic: draft", flush=True)
    blk = torch.empty(B, dtype=torch.int32, device=DEV)
    gm.draft_block(0, _i32([g]), B, blk, lg[:B])
    oblk, dsel = sess.draft_block(0, g, B)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:B], dsel.logits)
    assert tokens_agree(np.r_[0, blk.cpu().numpy()[1:]], dsel, range(1, B), rep, eps), rep.notes
    print("8b quadratic: cycle (candidates 0, 15, 31 in the oracle)", flush=True)
    _quad_lockstep(gm, sess, 0, oblk, B, rep, lg, L_forced=16, cands=[0, 15, 31])
    print(f"8b quadratic: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= 2e-2
    gm.close()
    del om, sess, w
    gc.collect()
