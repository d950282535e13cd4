"""GPU parity on the tiny float32 decoder (2 layers, d 64, 4/2 heads of 16,
FFN 256, vocab 256, MASK 255): token streams of every mode equal the
oracle's, logits agree within 1e-4 call by call."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

TINY = W.SHAPES["tiny"]
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_streams.json")))


@pytest.fixture(scope="module")
def gm():
    from self_speculative_amd.model import Model
    w = W.make_weights(TINY, seed=0)
    m = Model(TINY, w, max_seqs=8, max_block=16, max_context=512, max_rows=64)
    yield m
    m.close()


@pytest.fixture(scope="module")
def om():
    return O.OracleModel(TINY, W.make_weights(TINY, seed=0), row_independent=True)


def _fresh(gm, seq):
    gm.seq_reset(seq)
    return seq


def test_tiny_streams_equal_golden(gm):
    from self_speculative_amd import decode as D
    p = np.array(GOLD["prompt"], dtype=np.int32)
    print("tiny: AR / self-spec / forced / diffusion streams", flush=True)
    assert D.generate_ar(gm, p, 64, seq=_fresh(gm, 0)).tokens == GOLD["ar"]
    ss = D.generate_selfspec(gm, p, 64, 8, seq=_fresh(gm, 1))
    assert ss.tokens == GOLD["selfspec"] and ss.accept_lengths == GOLD["selfspec_accept"]
    fs = D.generate_selfspec(gm, p, 64, 8, forced=GOLD["forced_schedule"], seq=_fresh(gm, 2))
    assert fs.tokens == GOLD["forced"] and fs.accept_lengths == GOLD["forced_accept"]
    df = D.generate_diffusion(gm, p, 64, 8, 0.9, seq=_fresh(gm, 3))
    assert df.tokens == GOLD["diffusion"] and df.steps_per_block == GOLD["diffusion_steps"]


@pytest.mark.parametrize("tau,S", [(1.01, None), (0.0045, 3)])
def test_tiny_diffusion_with_revision(gm, om, tau, S):
    """The revision variant: every written position whose argmax differs is
    rewritten (tau_revise 0), so only argmax decisions are involved."""
    from self_speculative_amd import decode as D
    p = W.prompt_ids(TINY, 13, seed=6)
    print(f"tiny diffusion with revision tau={tau} S={S}", flush=True)
    g = D.generate_diffusion(gm, p, 32, 8, tau, S, seq=_fresh(gm, 5), tau_revise=0.0)
    o = O.generate_diffusion(om, p, 32, 8, tau, S, tau_revise=0.0)
    assert g.tokens == o.tokens and g.steps_per_block == o.steps_per_block
    if tau > 1:
        assert sum(o.revisions) > 0


def test_tiny_revise_step_counts(gm, om):
    """Step by step: blocks and the per-sequence revise counts equal the oracle's."""
    seq = _fresh(gm, 6)
    p = W.prompt_ids(TINY, 9, seed=7)
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    gm.prefill(seq, torch.as_tensor(p, device="cuda"), nxt)
    sess = O.OracleSession(om)
    sess.prefill(0, p)
    blk = np.full(8, TINY.mask_id, dtype=np.int32)
    blk[[2, 5]] = [11, 40]                               # written positions the step may revise
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    nr = torch.empty(1, dtype=torch.int32, device="cuda")
    # tau_revise far from the tiny model's confidences (about 1/256): this test has no exemptions
    for step, (tau, taur) in enumerate([(1.01, 0.0), (0.0045, 0.5), (1.01, 2.0), (0.9, 0.0)]):
        print(f"tiny revise step {step}", flush=True)
        g = torch.as_tensor(blk, device="cuda")
        gm.diffuse_step_revise([seq], g, 8, tau, taur, False, nm, nr)
        new, U, R, left, sel = sess.diffuse_step_revise(0, blk, tau, taur, False)
        torch.cuda.synchronize()
        assert g.cpu().tolist() == new.tolist()
        assert int(nm.item()) == left and int(nr.item()) == len(R)
        blk = new


@pytest.mark.parametrize("tau,S", [(1.01, None), (0.0, None), (0.0045, 3), (0.9, 4)])
def test_tiny_diffusion_thresholds(gm, om, tau, S):
    from self_speculative_amd import decode as D
    p = W.prompt_ids(TINY, 11, seed=5)
    print(f"tiny diffusion tau={tau} S={S}", flush=True)
    g = D.generate_diffusion(gm, p, 32, 8, tau, S, seq=_fresh(gm, 4))
    o = O.generate_diffusion(om, p, 32, 8, tau, S)
    assert g.tokens == o.tokens and g.steps_per_block == o.steps_per_block


def test_tiny_lockstep_logits(gm, om):
    """Every call's logits within 1e-4 of the oracle's (float32 bar)."""
    dev = "cuda"
    seq = _fresh(gm, 5)
    p = W.prompt_ids(TINY, 21, seed=6)
    sess = O.OracleSession(om)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    lg = torch.empty((16, TINY.vocab), dtype=torch.float32, device=dev)
    gm.prefill(seq, torch.as_tensor(p, device=dev), nxt, lg[:1])
    ref = sess.prefill(0, p)
    torch.cuda.synchronize()
    assert int(nxt.item()) == int(ref.tok[0])
    np.testing.assert_allclose(lg[:1].cpu().numpy(), ref.logits, atol=1e-4, rtol=0)
    g = int(nxt.item())
    blk = torch.empty(8, dtype=torch.int32, device=dev)
    ar = torch.empty(8, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    anchor = torch.tensor([g], dtype=torch.int32, device=dev)
    for cyc in range(3):
        print(f"tiny lockstep cycle {cyc}", flush=True)
        gm.draft_block(seq, anchor, 8, blk, lg[:8])
        oblk, osel = sess.draft_block(0, g, 8)
        torch.cuda.synchronize()
        np.testing.assert_allclose(lg[:8].cpu().numpy(), osel.logits, atol=1e-4, rtol=0)
        assert blk.cpu().tolist() == oblk.tolist()
        gm.verify_block([seq], blk, 8, ar, acc, lg[:8])
        oa, oL, vsel = sess.verify_block(0, oblk)
        torch.cuda.synchronize()
        np.testing.assert_allclose(lg[:8].cpu().numpy(), vsel.logits, atol=1e-4, rtol=0)
        assert ar.cpu().tolist() == oa.tolist() and int(acc.item()) == oL
        L = [3, 8, 1][cyc]                       # forced commits exercise every slot
        gm.commit_kv(seq, L)
        sess.commit_kv(0, L)
        g = int(oa[L - 1])
        anchor.fill_(g)
    tok = torch.tensor([g], dtype=torch.int32, device=dev)
    gm.decode_ar(seq, tok, nxt, lg[:1])
    r = sess.decode_ar(0, g)
    torch.cuda.synchronize()
    np.testing.assert_allclose(lg[:1].cpu().numpy(), r.logits, atol=1e-4, rtol=0)
    assert gm.seq_length(seq) == sess.committed(0)


def test_tiny_batch_diffusion_matches_single(gm, om):
    """Three sequences with different prompt lengths in lockstep equal the
    oracle run of each sequence alone."""
    from self_speculative_amd import decode as D
    prompts = [W.prompt_ids(TINY, n, seed=7, index=i) for i, n in enumerate([5, 30, 17])]
    seqs = [_fresh(gm, 5 + i) for i in range(3)]
    print("tiny batch diffusion", flush=True)
    outs = D.generate_diffusion_batch(gm, prompts, 24, 8, 0.0045, 4, seqs)
    for i, p in enumerate(prompts):
        o = O.generate_diffusion(om, p, 24, 8, 0.0045, 4)
        assert outs[i].tokens == o.tokens and outs[i].steps_per_block == o.steps_per_block


def test_tiny_vocab_reduction_planted_tie_and_mask_maximum():
    """The LM head gets a later row b copying the draft's most frequent argmax
    row a, and a MASK row 1.25 x row a.  On rows whose best non-MASK id is a
    (with a positive logit) MASK holds the largest logit and b ties a exactly:
    the selection must still return a -- MASK is excluded and a tie goes to the
    lowest id -- on the GPU as in the oracle, with matching confidence."""
    from self_speculative_amd.model import Model
    mask, B = TINY.mask_id, 8
    w = W.make_weights(TINY, seed=0)
    p = W.prompt_ids(TINY, 12, seed=8)
    sess = O.OracleSession(O.OracleModel(TINY, w))
    g = int(sess.prefill(0, p).tok[0])
    _, sel0 = sess.draft_block(0, g, B)
    vals, counts = np.unique(sel0.tok[1:], return_counts=True)
    order = [int(v) for v in vals[np.argsort(-counts, kind="stable")] if int(v) + 1 < mask]
    a = order[0]
    b = a + 1
    w2 = dict(w)
    lm = w["lm_head"].copy()
    lm[b] = lm[a]
    lm[mask] = 1.25 * lm[a]
    w2["lm_head"] = lm
    sess = O.OracleSession(O.OracleModel(TINY, w2))
    assert int(sess.prefill(0, p).tok[0]) == g
    oblk, osel = sess.draft_block(0, g, B)
    planted = [r for r in range(1, B) if osel.tok[r] == a and osel.logits[r, a] > 0]
    assert planted, "the plant must reach at least one row"
    for r in planted:
        lg = osel.logits[r]
        assert lg[mask] > lg[a] == lg[b] and lg[a] == np.delete(lg, mask).max()
    m = Model(TINY, w2, max_seqs=2, max_block=B, max_context=128, max_rows=32)
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    m.prefill(0, torch.as_tensor(p, dtype=torch.int32, device="cuda"), nxt)
    blk = torch.empty(B, dtype=torch.int32, device="cuda")
    m.draft_block(0, nxt, B, blk)
    conf = torch.empty(B, dtype=torch.float32, device="cuda")
    m.row_stats(conf=conf)
    torch.cuda.synchronize()
    assert int(nxt.item()) == g
    got = blk.cpu().numpy()
    print(f"tiny planted selection: a={a} b={b} rows {planted}", flush=True)
    np.testing.assert_array_equal(got, oblk)
    np.testing.assert_allclose(conf.cpu().numpy()[1:], osel.conf[1:], rtol=1e-4)
    m.close()
