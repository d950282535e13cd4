"""GPU parity of the bf16 decoder path on a small shape (2 layers, d 256,
4 q / 2 KV heads of 128, FFN 512, vocab 1024, MASK 1023): lockstep against the
oracle call by call, plus the exact properties of the GPU path itself."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from lockstep import Report, accept_exempt, tokens_agree

pytestmark = pytest.mark.gpu

SHAPE = W.ModelShape("small-bf16", 2, 256, 4, 2, 128, 512, 1024, "bf16")
B = 32
DEV = "cuda"


@pytest.fixture(scope="module")
def weights():
    return W.make_weights(SHAPE, seed=21, gains="random")


@pytest.fixture(scope="module")
def gm(weights):
    from self_speculative_amd.model import Model
    m = Model(SHAPE, weights, max_seqs=8, max_block=B, max_context=1024, max_rows=96)
    yield m
    m.close()


@pytest.fixture(scope="module")
def om(weights):
    return O.OracleModel(SHAPE, weights)


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def test_bf16_lockstep_selfspec_and_ar(gm, om):
    """prefill (several chunks) -> 4 self-spec cycles -> 3 AR steps."""
    seq = 0
    gm.seq_reset(seq)
    rep = Report()
    p = W.prompt_ids(SHAPE, 200, seed=22)          # 3 prefill chunks of <= 96 rows
    sess = O.OracleSession(om)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    print("bf16 lockstep: prefill", flush=True)
    gm.prefill(seq, _i32(p), nxt, lg[:1])
    ref = sess.prefill(0, p)
    torch.cuda.synchronize()
    rep.logits(lg[:1], ref.logits)
    assert tokens_agree(nxt.cpu().numpy(), ref, [0], rep), rep.notes
    g = int(ref.tok[0])
    blk = torch.empty(B, dtype=torch.int32, device=DEV)
    ar = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    for cyc in range(4):
        print(f"bf16 lockstep: cycle {cyc}", flush=True)
        anchor = _i32([g])
        gm.draft_block(seq, anchor, B, blk, lg)
        oblk, osel = sess.draft_block(0, g, B)
        torch.cuda.synchronize()
        rep.logits(lg, osel.logits)
        gblk = blk.cpu().numpy()
        assert tokens_agree(np.r_[0, gblk[1:]], osel, range(1, B), rep), rep.notes
        if not np.array_equal(gblk, oblk):
            rep.resync()
            blk.copy_(_i32(oblk))
        gm.verify_block([seq], blk, B, ar, acc, lg)
        oa, oL, vsel = sess.verify_block(0, oblk)
        torch.cuda.synchronize()
        rep.logits(lg, vsel.logits)
        assert tokens_agree(ar.cpu().numpy(), vsel, range(B), rep), rep.notes
        gL = int(acc.item())
        if gL != oL:
            assert accept_exempt(vsel, gL, oL, rep), rep.notes
            rep.resync()
        L = [oL, 17, 32, 1][cyc]                  # natural L first, then forced lengths
        gm.commit_kv(seq, L)
        sess.commit_kv(0, L)
        g = int(oa[L - 1])
    for step in range(3):
        gm.decode_ar(seq, _i32([g]), nxt, lg[:1])
        r = sess.decode_ar(0, g)
        torch.cuda.synchronize()
        rep.logits(lg[:1], r.logits)
        assert tokens_agree(nxt.cpu().numpy(), r, [0], rep), rep.notes
        g = int(r.tok[0])
    print(f"bf16 lockstep: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= 2e-2


def test_bf16_lockstep_diffusion(gm, om):
    seq = 1
    gm.seq_reset(seq)
    rep = Report()
    p = W.prompt_ids(SHAPE, 70, seed=23)
    sess = O.OracleSession(om)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.prefill(seq, _i32(p), nxt)
    sess.prefill(0, p)
    lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    conf = torch.empty(B, dtype=torch.float32, device=DEV)
    nm = torch.empty(1, dtype=torch.int32, device=DEV)
    blk = np.full(B, SHAPE.mask_id, dtype=np.int32)
    taus = [0.9, 0.9, 0.0012, 0.9]                  # random weights: conf ~ 1/V; 0.0012 unmasks several
    for s, tau in enumerate(taus):
        force = s == len(taus) - 1
        print(f"bf16 diffuse step {s} tau={tau} force={force}", flush=True)
        gblk = _i32(blk)
        gm.diffuse_step([seq], gblk, B, tau, force, nm, conf, lg)
        new, U, left, sel = sess.diffuse_step(0, blk, tau, force)
        torch.cuda.synchronize()
        err = rep.logits(lg, sel.logits)
        # conf = 1 / sum exp(l - max): per row |d ln conf| <= 2 max|d logit|
        assert np.all(np.abs(np.log(conf.cpu().numpy()) - np.log(sel.conf)) <= 2 * err + 1e-6)
        got = gblk.cpu().numpy()
        if not np.array_equal(got, new):
            from lockstep import unmask_exempt
            assert unmask_exempt(blk, sel, tau, SHAPE.mask_id), (got, new)
            rep.exempt += 1
            rep.resync()
        else:
            assert int(nm.item()) == left
        blk = new
    assert (blk != SHAPE.mask_id).all()
    ar = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.verify_block([seq], _i32(blk), B, ar, acc, lg)
    sess.verify_block(0, blk)
    gm.commit_kv(seq, B)
    sess.commit_kv(0, B)
    print(f"bf16 diffusion lockstep: {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= 2e-2


def test_bf16_lockstep_diffusion_with_revision(gm, om):
    """Revision variant in lockstep: masked positions by the unmask rule,
    written ones rewritten to a differing argmax whose conf clears tau_revise."""
    seq = 1
    gm.seq_reset(seq)
    rep = Report()
    p = W.prompt_ids(SHAPE, 70, seed=28)
    sess = O.OracleSession(om)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.prefill(seq, _i32(p), nxt)
    sess.prefill(0, p)
    lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    nm = torch.empty(1, dtype=torch.int32, device=DEV)
    nr = torch.empty(1, dtype=torch.int32, device=DEV)
    blk = np.full(B, SHAPE.mask_id, dtype=np.int32)
    blk[:6] = W.prompt_ids(SHAPE, 6, seed=29)
    revised = 0
    for s, (tau, taur) in enumerate([(0.9, 0.0), (0.0012, 0.0), (0.9, 0.0011), (0.9, 0.0)]):
        force = s == 3
        print(f"bf16 revise step {s} tau={tau} tau_revise={taur} force={force}", flush=True)
        gblk = _i32(blk)
        gm.diffuse_step_revise([seq], gblk, B, tau, taur, force, nm, nr, None, lg)
        new, U, R, left, sel = sess.diffuse_step_revise(0, blk, tau, taur, force)
        torch.cuda.synchronize()
        eps = rep.logits(lg, sel.logits)
        got = gblk.cpu().numpy()
        if not np.array_equal(got, new):
            from lockstep import revise_exempt, unmask_exempt
            diff = np.nonzero(got != new)[0]
            masked = blk == SHAPE.mask_id
            assert (not masked[diff].all() or unmask_exempt(blk, sel, tau, SHAPE.mask_id, eps)), (got, new)
            assert revise_exempt(blk, sel, taur, SHAPE.mask_id, eps, diff[~masked[diff]]), (got, new)
            rep.exempt += 1
            rep.resync()
        else:
            assert int(nm.item()) == left and int(nr.item()) == len(R)
        revised += len(R)
        blk = new
    assert (blk != SHAPE.mask_id).all() and revised > 0
    print(f"bf16 revision lockstep: revised {revised}, {rep.summary()}", flush=True)
    rep.assert_strict()
    assert rep.max_logit_err <= 2e-2


def test_bf16_revise_disabled_equals_plain_step(gm):
    p = W.prompt_ids(SHAPE, 40, seed=30)
    outs = []
    for variant in ("plain", "revise_off"):
        gm.seq_reset(2)
        nxt = torch.empty(1, dtype=torch.int32, device=DEV)
        gm.prefill(2, _i32(p), nxt)
        blk = torch.full((1, B), SHAPE.mask_id, dtype=torch.int32, device=DEV)
        blk[0, :4] = 5
        nm = torch.empty(1, dtype=torch.int32, device=DEV)
        conf = torch.empty(B, dtype=torch.float32, device=DEV)
        lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
        print(f"bf16 diffuse step {variant}", flush=True)
        if variant == "plain":
            gm.diffuse_step([2], blk, B, 0.0012, False, nm, conf, lg)
        else:
            gm.diffuse_step_revise([2], blk, B, 0.0012, 1.0, False, nm, None, conf, lg)
        torch.cuda.synchronize()
        outs.append((blk.cpu().numpy(), nm.cpu().numpy(), conf.cpu().numpy(), lg.cpu().numpy()))
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_bf16_selfspec_equals_ar_on_gpu(gm):
    """The GPU path is row-independent: a causal block forward reproduces the
    one-row AR forward bit for bit, so self-spec emits exactly the AR stream."""
    from self_speculative_amd import decode as D
    p = W.prompt_ids(SHAPE, 50, seed=24)
    gm.seq_reset(2)
    gm.seq_reset(3)
    print("bf16 gpu self-spec vs gpu AR", flush=True)
    ar = D.generate_ar(gm, p, 100, seq=2)
    ss = D.generate_selfspec(gm, p, 100, B, seq=3)
    assert ss.tokens == ar.tokens


def test_bf16_short_blocks_bit_identical(gm):
    """Launches of fewer than 32 rows load only their rows' activation lanes:
    causal blocks of 1, 7 and 31 tokens and the one-row AR step give each row
    the bits of the same row in a full 32-row block."""
    p = W.prompt_ids(SHAPE, 45, seed=26)
    toks = W.prompt_ids(SHAPE, B, seed=27)
    gm.seq_reset(5)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.prefill(5, _i32(p), nxt)
    full = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    a = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    print("bf16 full 32-row causal block", flush=True)
    gm.verify_block([5], _i32(toks), B, a, acc, full)
    torch.cuda.synchronize()
    ref = full.cpu().numpy()
    for b in (1, 7, 31):
        print(f"bf16 causal block of {b} rows", flush=True)
        lg = torch.empty((b, SHAPE.vocab), dtype=torch.float32, device=DEV)
        gm.verify_block([5], _i32(toks[:b]), b, a[:b], acc, lg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lg.cpu().numpy(), ref[:b])
    print("bf16 one-row AR step", flush=True)
    lg = torch.empty((1, SHAPE.vocab), dtype=torch.float32, device=DEV)
    gm.decode_ar(5, _i32([toks[0]]), nxt, lg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lg.cpu().numpy(), ref[:1])


def test_bf16_perfect_draft_and_planted_mismatch(gm):
    from self_speculative_amd import decode as D
    p = W.prompt_ids(SHAPE, 40, seed=25)
    gm.seq_reset(4)
    ar = D.generate_ar(gm, p, 2 * B + 2, seq=4).tokens
    for j in (None, 1, 9, 31):
        gm.seq_reset(4)
        print(f"bf16 verify with planted mismatch at {j}", flush=True)
        nxt = torch.empty(1, dtype=torch.int32, device=DEV)
        gm.prefill(4, _i32(p), nxt)
        block = np.array(ar[:B], dtype=np.int32)
        if j is not None:
            block[j] = (block[j] + 1) % (SHAPE.vocab - 1)
        a = torch.empty(B, dtype=torch.int32, device=DEV)
        acc = torch.empty(1, dtype=torch.int32, device=DEV)
        gm.verify_block([4], _i32(block), B, a, acc)
        torch.cuda.synchronize()
        assert int(acc.item()) == (B if j is None else j)
        if j is None:
            assert a.cpu().tolist()[:-1] == ar[1:B]


def test_bf16_batch_independence(gm):
    """Rows of one sequence do not depend on what else is in the batch."""
    prompts = [W.prompt_ids(SHAPE, n, seed=26, index=i) for i, n in enumerate([33, 90, 64])]
    seqs = [5, 6, 7]
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    outs = {}
    for mode in ("batch", "single"):
        for s, p in zip(seqs, prompts):
            gm.seq_reset(s)
            gm.prefill(s, _i32(p), nxt)
        blk = torch.full((3, B), SHAPE.mask_id, dtype=torch.int32, device=DEV)
        blk[:, 0] = 7
        conf = torch.empty((3, B), dtype=torch.float32, device=DEV)
        nm = torch.empty(3, dtype=torch.int32, device=DEV)
        lg = torch.empty((3 * B, SHAPE.vocab), dtype=torch.float32, device=DEV)
        print(f"bf16 batch independence: {mode}", flush=True)
        if mode == "batch":
            gm.diffuse_step(seqs, blk, B, 0.0012, False, nm, conf, lg)
        else:
            for i, s in enumerate(seqs):
                b1 = blk[i:i + 1].clone()
                gm.diffuse_step([s], b1, B, 0.0012, False, nm[i:i + 1], conf[i:i + 1], lg[i * B:(i + 1) * B])
                blk[i:i + 1] = b1
        torch.cuda.synchronize()
        outs[mode] = (blk.cpu().numpy(), conf.cpu().numpy(), lg.cpu().numpy())
    for a, b in zip(outs["batch"], outs["single"]):
        np.testing.assert_array_equal(a, b)


def test_bf16_staged_attention_matches_tile_parallel(weights, om):
    """A batch with enough (split, KV head) pairs runs attention with each
    256-key split staged once in LDS; alone, each sequence runs the
    tile-parallel shape.  Both must give the same bits, and the oracle's
    logits within the bar."""
    from self_speculative_amd.model import Model
    lens = [1900 + 37 * i for i in range(16)]           # 8+ splits x 2 KV heads x 16 = 256+ pairs
    m = Model(SHAPE, weights, max_seqs=16, max_block=B, max_context=2560, max_rows=16 * B)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    prompts = [W.prompt_ids(SHAPE, n, seed=31, index=i) for i, n in enumerate(lens)]
    for i, p in enumerate(prompts):
        m.prefill(i, _i32(p), nxt)
    seqs = list(range(16))
    blk = torch.full((16, B), SHAPE.mask_id, dtype=torch.int32, device=DEV)
    nm = torch.empty(16, dtype=torch.int32, device=DEV)
    lg = torch.empty((16 * B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    print("bf16 staged attention: batch of 16", flush=True)
    m.diffuse_step(seqs, blk, B, 0.9, False, nm, None, lg)
    torch.cuda.synchronize()
    batch = lg.cpu().numpy()
    for i in (0, 9, 15):
        print(f"bf16 staged attention: sequence {i} alone", flush=True)
        b1 = torch.full((1, B), SHAPE.mask_id, dtype=torch.int32, device=DEV)
        l1 = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
        m.diffuse_step([i], b1, B, 0.9, False, nm[:1], None, l1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(l1.cpu().numpy(), batch[i * B:(i + 1) * B])
    sess = O.OracleSession(om)
    sess.prefill(0, prompts[15])
    _, _, _, sel = sess.diffuse_step(0, np.full(B, SHAPE.mask_id, dtype=np.int32), 0.9, False)
    assert np.abs(batch[15 * B:] - sel.logits).max() <= 2e-2
    m.close()


def test_bf16_streamed_attention_matches_tile_parallel(weights):
    """A batch with at least 512 (split, KV head) pairs streams runs of splits
    through LDS; alone, each sequence runs the tile-parallel shape.  Both must
    give the same bits."""
    from self_speculative_amd.model import Model
    lens = [3900 + 37 * i for i in range(16)]           # 16+ splits x 2 KV heads x 16 = 512+ pairs
    m = Model(SHAPE, weights, max_seqs=16, max_block=B, max_context=4608, max_rows=16 * B)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    for i, n in enumerate(lens):
        m.prefill(i, _i32(W.prompt_ids(SHAPE, n, seed=33, index=i)), nxt)
    seqs = list(range(16))
    blk = torch.full((16, B), SHAPE.mask_id, dtype=torch.int32, device=DEV)
    nm = torch.empty(16, dtype=torch.int32, device=DEV)
    lg = torch.empty((16 * B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    print("bf16 streamed attention: batch of 16", flush=True)
    m.diffuse_step(seqs, blk, B, 0.9, False, nm, None, lg)
    torch.cuda.synchronize()
    batch = lg.cpu().numpy()
    for i in (0, 7, 15):
        print(f"bf16 streamed attention: sequence {i} alone", flush=True)
        b1 = torch.full((1, B), SHAPE.mask_id, dtype=torch.int32, device=DEV)
        l1 = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
        m.diffuse_step([i], b1, B, 0.9, False, nm[:1], None, l1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(l1.cpu().numpy(), batch[i * B:(i + 1) * B])
    m.close()


def test_bf16_decode_forward_repeatable(weights):
    """The same 32-row forward, repeated, gives the same bits every time (one
    sequence of 1900 keys: 8 attention splits per KV head, split-K GEMMs):
    nothing in the decode path depends on which workgroup finishes first."""
    from self_speculative_amd.model import Model
    m = Model(SHAPE, weights, max_seqs=1, max_block=B, max_context=2048, max_rows=B)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    m.prefill(0, _i32(W.prompt_ids(SHAPE, 1900, seed=35)), nxt)
    blk = torch.empty(B, dtype=torch.int32, device=DEV)
    lg = torch.empty((B, SHAPE.vocab), dtype=torch.float32, device=DEV)
    m.draft_block(0, nxt, B, blk, lg)
    torch.cuda.synchronize()
    ref = lg.clone()
    for r in range(40):
        m.draft_block(0, nxt, B, blk, lg)
        torch.cuda.synchronize()
        assert torch.equal(lg, ref), r
    m.close()


def test_bf16_prefill_chunking_bit_identical(weights):
    """A 2000-token prompt prefilled in one 2000-row chunk (125 query tiles:
    attention runs the staged shape in groups of four query tiles) and in
    128-row chunks (the tile-parallel shape) gives the same last-row logits
    and next token, and the same AR steps after it."""
    from self_speculative_amd.model import Model
    p = W.prompt_ids(SHAPE, 2000, seed=34)
    outs = []
    for rows in (2000, 128):
        print(f"bf16 prefill chunking: {rows}-row chunks", flush=True)
        m = Model(SHAPE, weights, max_seqs=1, max_block=B, max_context=2048, max_rows=rows)
        toks = torch.empty(5, dtype=torch.int32, device=DEV)
        lg = torch.empty((5, SHAPE.vocab), dtype=torch.float32, device=DEV)
        m.prefill(0, _i32(p), toks[0:1], lg[0:1])
        for t in range(1, 5):
            m.decode_ar(0, toks[t - 1:t], toks[t:t + 1], lg[t:t + 1])
        torch.cuda.synchronize()
        outs.append((toks.cpu().numpy(), lg.cpu().numpy()))
        m.close()
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_bf16_shuffled_pages_bit_identical(weights):
    from self_speculative_amd.model import Model
    from self_speculative_amd import decode as D
    p = W.prompt_ids(SHAPE, 150, seed=27)
    res = []
    for shuffle in (False, True):
        m = Model(SHAPE, weights, max_seqs=2, max_block=B, max_context=512, max_rows=64, n_pages=40)
        if shuffle:
            m.shuffle_free_pages(1234)
        print(f"bf16 paged layout shuffle={shuffle}", flush=True)
        res.append(D.generate_selfspec(m, p, 70, B, forced=[5, 32, 9, 20, 3], seq=1).tokens)
        m.close()
    assert res[0] == res[1]


def test_bf16_error_paths(gm):
    from self_speculative_amd._lib import SdmError, SDM_ERR_STATE, SDM_ERR_ARG, SDM_ERR_CAPACITY
    gm.seq_reset(0)
    with pytest.raises(SdmError) as e:
        gm.commit_kv(0, 1)                          # nothing verified
    assert e.value.status == SDM_ERR_STATE
    blk = torch.zeros(B, dtype=torch.int32, device=DEV)
    a = torch.empty(B, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    with pytest.raises(SdmError) as e:
        gm.verify_block([0], blk, B, a, acc)        # no prompt yet
    assert e.value.status == SDM_ERR_STATE
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.prefill(0, _i32([1, 2, 3]), nxt)
    with pytest.raises(SdmError) as e:
        gm.prefill(0, _i32([1, 2, 3]), nxt)         # not empty
    assert e.value.status == SDM_ERR_STATE
    with pytest.raises(SdmError) as e:
        gm.verify_block([0], blk, B + 1, a, acc)    # block above max_block
    assert e.value.status == SDM_ERR_ARG
    gm.verify_block([0], blk, 8, a, acc)
    with pytest.raises(SdmError) as e:
        gm.commit_kv(0, 9)                          # more than verified
    assert e.value.status == SDM_ERR_ARG
    assert gm.seq_length(0) == 3                    # failed calls changed nothing
    gm.commit_kv(0, 8)
    assert gm.seq_length(0) == 11
    with pytest.raises(SdmError) as e:
        gm.verify_block([99], blk, 8, a, acc)
    assert e.value.status == SDM_ERR_CAPACITY
    torch.cuda.synchronize()
