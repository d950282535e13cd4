"""GPU parity of the 4-bit weight path (w4a16: group-wise int4 codes, one bf16
scale per output row and 128 inputs) against the oracle, which dequantizes
exactly and multiplies in float64.

* A small shape (2 layers, d 256, 4 q / 2 KV heads of 128, FFN 512, vocab
  1024) in lockstep call by call: prefill in 96-row chunks (the many-row GEMM
  configuration), self-speculation, AR, block diffusion.
* Exact properties of the GPU path: self-speculation emits the GPU AR stream
  token for token, and a batch of sequences gives each the same bits as
  running it alone.
* The 8B shape in the benchmark's launch configuration and the 14B width
  (2 layers), whose GEMM configurations (tiles per workgroup, K splits) are
  those of the full models.

The bar is the bf16 path's: logits within 2e-2 max-abs; token, accept and
unmask decisions equal except where the oracle's own decision is a near-tie
(top-2 margin, or distance to the threshold, below 1e-3).
"""
import gc

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from lockstep import Report, accept_exempt, tokens_agree, unmask_exempt

pytestmark = pytest.mark.gpu

SHAPE = W.ModelShape("small-bf16", 2, 256, 4, 2, 128, 512, 1024, "bf16")
B = 32
DEV = "cuda"
LOGIT_TOL = 2e-2


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


@pytest.fixture(scope="module")
def weights():
    return W.make_w4_weights(SHAPE, seed=41, gains="random")


@pytest.fixture(scope="module")
def gm(weights):
    from self_speculative_amd.model import Model
    m = Model(SHAPE, weights, max_seqs=8, max_block=B, max_context=1024, max_rows=96)
    assert m.w4
    yield m
    m.close()


@pytest.fixture(scope="module")
def om(weights):
    return O.OracleModel(SHAPE, weights)


def _cycle(gm, sess, seq, g, L_forced, rep, lg):
    blk = torch.empty(B, dtype=torch.int32, device=DEV)
    ar = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.draft_block(seq, _i32([g]), B, blk, lg)
    oblk, osel = sess.draft_block(0, g, B)
    torch.cuda.synchronize()
    eps = rep.logits(lg, osel.logits)
    gb = blk.cpu().numpy()
    assert gb[0] == g
    assert tokens_agree(np.r_[0, gb[1:]], osel, range(1, B), rep, eps), rep.notes
    if not np.array_equal(gb, oblk):
        rep.resync()
        blk.copy_(_i32(oblk))
    gm.verify_block([seq], blk, B, ar, acc, lg)
    oa, oL, vsel = sess.verify_block(0, oblk)
    torch.cuda.synchronize()
    eps = rep.logits(lg, vsel.logits)
    assert tokens_agree(ar.cpu().numpy(), vsel, range(B), rep, eps), rep.notes
    gL = int(acc.item())
    if gL != oL:
        assert accept_exempt(vsel, gL, oL, rep), rep.notes
        rep.resync()
    L = oL if L_forced is None else L_forced
    gm.commit_kv(seq, L)
    sess.commit_kv(0, L)
    return int(oa[L - 1])


def _ar(gm, sess, seq, g, rep, lg, nxt):
    gm.decode_ar(seq, _i32([g]), nxt, lg[:1])
    r = sess.decode_ar(0, g)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:1], r.logits)
    assert tokens_agree(nxt.cpu().numpy(), r, [0], rep, eps), rep.notes
    return int(r.tok[0])


def test_w4_lockstep_selfspec_and_ar(gm, om):
    seq = 0
    gm.seq_reset(seq)
    rep = Report()
    p = W.prompt_ids(SHAPE, 200, seed=42)          # prefill chunks of 96, 96 and 8 rows
    sess = O.OracleSession(om)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    print("w4 lockstep: prefill", flush=True)
    gm.prefill(seq, _i32(p), nxt, lg[:1])
    ref = sess.prefill(0, p)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:1], ref.logits)
    assert tokens_agree(nxt.cpu().numpy(), ref, [0], rep, eps), rep.notes
    g = int(ref.tok[0])
    for cyc, L in enumerate([None, 17, 32, 1]):
        print(f"w4 lockstep: cycle {cyc}", flush=True)
        g = _cycle(gm, sess, seq, g, L, rep, lg)
    for step in range(3):
        print(f"w4 lockstep: AR step {step}", flush=True)
        g = _ar(gm, sess, seq, g, rep, lg, nxt)
    print(f"w4 lockstep: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= LOGIT_TOL


def test_w4_lockstep_diffusion(gm, om):
    seq = 1
    gm.seq_reset(seq)
    rep = Report()
    p = W.prompt_ids(SHAPE, 70, seed=43)
    sess = O.OracleSession(om)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.prefill(seq, _i32(p), nxt)
    sess.prefill(0, p)
    lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    nm = torch.empty(1, dtype=torch.int32, device=DEV)
    blk = np.full(B, SHAPE.mask_id, dtype=np.int32)
    taus = [0.9, 0.0012, 0.0012, 0.9]
    for s, tau in enumerate(taus):
        force = s == len(taus) - 1
        print(f"w4 diffuse step {s} tau={tau} force={force}", flush=True)
        gblk = _i32(blk)
        gm.diffuse_step([seq], gblk, B, tau, force, nm, None, lg)
        new, U, left, sel = sess.diffuse_step(0, blk, tau, force)
        torch.cuda.synchronize()
        eps = rep.logits(lg, sel.logits)
        got = gblk.cpu().numpy()
        if not np.array_equal(got, new):
            assert unmask_exempt(blk, sel, tau, SHAPE.mask_id, eps), (got, new)
            rep.exempt += 1
            rep.resync()
        else:
            assert int(nm.item()) == left
        blk = new
    assert (blk != SHAPE.mask_id).all()
    print(f"w4 diffusion lockstep: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= LOGIT_TOL


def test_w4_selfspec_equals_ar_on_gpu(gm):
    from self_speculative_amd import decode as D
    p = W.prompt_ids(SHAPE, 50, seed=44)
    gm.seq_reset(2)
    gm.seq_reset(3)
    print("w4 gpu self-spec vs gpu AR", flush=True)
    ar = D.generate_ar(gm, p, 100, seq=2)
    ss = D.generate_selfspec(gm, p, 100, B, seq=3)
    assert ss.tokens == ar.tokens


def test_w4_short_blocks_bit_identical(gm):
    """Launches of fewer than 32 rows load only their rows' activation lanes:
    causal blocks of 1, 7 and 31 tokens and the one-row AR step give each row
    the bits of the same row in a full 32-row block."""
    p = W.prompt_ids(SHAPE, 45, seed=46)
    toks = W.prompt_ids(SHAPE, B, seed=47)
    gm.seq_reset(5)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.prefill(5, _i32(p), nxt)
    full = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    a = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    print("w4 full 32-row causal block", flush=True)
    gm.verify_block([5], _i32(toks), B, a, acc, full)
    torch.cuda.synchronize()
    ref = full.cpu().numpy()
    for b in (1, 7, 31):
        print(f"w4 causal block of {b} rows", flush=True)
        lg = torch.empty((b, SHAPE.vocab), dtype=torch.float32, device=DEV)
        gm.verify_block([5], _i32(toks[:b]), b, a[:b], acc, lg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lg.cpu().numpy(), ref[:b])
    print("w4 one-row AR step", flush=True)
    lg = torch.empty((1, SHAPE.vocab), dtype=torch.float32, device=DEV)
    gm.decode_ar(5, _i32([toks[0]]), nxt, lg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lg.cpu().numpy(), ref[:1])


def test_w4_batch_independence(gm):
    """Three sequences in one 96-row forward (the many-row 4-bit GEMM) give
    each the bits of its own 32-row forward."""
    prompts = [W.prompt_ids(SHAPE, n, seed=45, index=i) for i, n in enumerate([33, 90, 64])]
    seqs = [5, 6, 7]
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    outs = {}
    for mode in ("batch", "single"):
        for s, p in zip(seqs, prompts):
            gm.seq_reset(s)
            gm.prefill(s, _i32(p), nxt)
        blk = torch.full((3, B), SHAPE.mask_id, dtype=torch.int32, device=DEV)
        blk[:, 0] = 7
        nm = torch.empty(3, dtype=torch.int32, device=DEV)
        lg = torch.empty((3 * B, SHAPE.vocab), dtype=torch.float32, device=DEV)
        print(f"w4 batch independence: {mode}", flush=True)
        if mode == "batch":
            gm.diffuse_step(seqs, blk, B, 0.0012, False, nm, None, lg)
        else:
            for i, s in enumerate(seqs):
                b1 = blk[i:i + 1].clone()
                gm.diffuse_step([s], b1, B, 0.0012, False, nm[i:i + 1], None, lg[i * B:(i + 1) * B])
                blk[i:i + 1] = b1
        torch.cuda.synchronize()
        outs[mode] = (blk.cpu().numpy(), lg.cpu().numpy())
    for a, b in zip(outs["batch"], outs["single"]):
        np.testing.assert_array_equal(a, b)


def test_w4_8b_bench_configuration_lockstep():
    from self_speculative_amd.model import Model
    s = W.SHAPES["8b"]
    print("w4 8b: drawing weights", flush=True)
    w = W.make_w4_weights(s, seed=0)
    prompt = W.prompt_ids(s, 1024, seed=0)
    gm = Model(s, w, max_seqs=1, max_block=B, max_context=2048, max_rows=128)
    om = O.OracleModel(s, w)
    sess = O.OracleSession(om)
    rep = Report()
    lg = torch.empty((B, s.vocab), dtype=torch.float32, device=DEV)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    print("w4 8b: prefill 1024 (gpu, then oracle)", flush=True)
    gm.prefill(0, _i32(prompt), nxt, lg[:1])
    ref = sess.prefill(0, prompt)
    torch.cuda.synchronize()
    eps = rep.logits(lg[:1], ref.logits)
    assert tokens_agree(nxt.cpu().numpy(), ref, [0], rep, eps), rep.notes
    g = int(ref.tok[0])
    print("w4 8b: self-spec cycle", flush=True)
    g = _cycle(gm, sess, 0, g, 29, rep, lg)
    print("w4 8b: AR step", flush=True)
    _ar(gm, sess, 0, g, rep, lg, nxt)
    print(f"w4 8b lockstep: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= LOGIT_TOL
    gm.close()
    del om, sess, w
    gc.collect()


def test_w4_14b_width_two_layers_lockstep():
    from self_speculative_amd.model import Model
    s = W.SHAPES["14b"].with_layers(2)
    print("w4 14b-width: drawing weights", flush=True)
    w = W.make_w4_weights(s, seed=3)
    gm = Model(s, w, max_seqs=2, max_block=B, max_context=1024, max_rows=64)
    om = O.OracleModel(s, w)
    rep = Report()
    lg = torch.empty((B, s.vocab), dtype=torch.float32, device=DEV)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    for seq, n in enumerate([300, 517]):
        sess = O.OracleSession(om)
        p = W.prompt_ids(s, n, seed=3, index=seq)
        print(f"w4 14b-width: sequence {seq} prefill {n}", flush=True)
        gm.prefill(seq, _i32(p), nxt, lg[:1])
        ref = sess.prefill(0, p)
        torch.cuda.synchronize()
        eps = rep.logits(lg[:1], ref.logits)
        assert tokens_agree(nxt.cpu().numpy(), ref, [0], rep, eps), rep.notes
        print(f"w4 14b-width: sequence {seq} cycle", flush=True)
        _cycle(gm, sess, seq, int(ref.tok[0]), None, rep, lg)
    print(f"w4 14b-width lockstep: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= LOGIT_TOL
    gm.close()
