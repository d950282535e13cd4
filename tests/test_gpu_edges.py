"""GPU edge cases of the hot path, on the tiny float32 decoder, where the GPU
streams equal the oracle's exactly.

* A one-token prompt in every mode.
* Block size 1: self-speculation is AR (the oracle's invariant I4, on the
  GPU).
* The context limit reached exactly: the last position that fits is
  decoded (AR, a linear block and a quadratic block that end at
  max_context); the next call fails with SDM_ERR_CAPACITY and changes
  nothing.
* An empty prompt is rejected.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu
TINY = W.SHAPES["tiny"]
DEV = "cuda"


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


@pytest.fixture(scope="module")
def om():
    return O.OracleModel(TINY, W.make_weights(TINY, seed=0), row_independent=True)


@pytest.fixture(scope="module")
def gm():
    from self_speculative_amd.model import Model
    m = Model(TINY, W.make_weights(TINY, seed=0), max_seqs=6, max_block=32, max_context=64, max_rows=272)
    yield m
    m.close()


def test_one_token_prompt_every_mode(gm, om):
    from self_speculative_amd import decode as D
    p = W.prompt_ids(TINY, 1, seed=5)
    print("edges: one-token prompt", flush=True)
    for s in range(4):
        gm.seq_reset(s)
    ar = D.generate_ar(gm, p, 12, seq=0)
    assert ar.tokens == O.generate_ar(om, p, 12).tokens
    assert D.generate_selfspec(gm, p, 12, 8, seq=1).tokens == ar.tokens
    assert D.generate_diffusion(gm, p, 16, 8, 0.9, seq=2).tokens == O.generate_diffusion(om, p, 16, 8, 0.9).tokens
    assert D.generate_selfspec_quadratic(gm, p, 12, 4, seq=3).tokens == ar.tokens


def test_block_of_one_is_ar(gm):
    from self_speculative_amd import decode as D
    p = W.prompt_ids(TINY, 9, seed=6)
    print("edges: block of one", flush=True)
    gm.seq_reset(0)
    gm.seq_reset(1)
    ar = D.generate_ar(gm, p, 20, seq=0)
    ss = D.generate_selfspec(gm, p, 20, 1, seq=1)
    assert ss.tokens == ar.tokens and set(ss.accept_lengths) == {1}


def test_context_limit_reached_exactly(gm, om):
    from self_speculative_amd._lib import SDM_ERR_CAPACITY, SdmError
    print("edges: context limit", flush=True)
    # AR: prompt 40, then positions 40..63 are decoded; position 64 does not fit
    gm.seq_reset(0)
    p = W.prompt_ids(TINY, 40, seed=7)
    out = torch.empty(26, dtype=torch.int32, device=DEV)
    gm.prefill(0, _i32(p), out[0:1])
    base = out.data_ptr()
    for t in range(1, 25):
        gm.decode_ar(0, base + 4 * (t - 1), base + 4 * t)
    assert gm.seq_length(0) == 64
    with pytest.raises(SdmError) as e:
        gm.decode_ar(0, base + 4 * 24, base + 4 * 25)
    assert e.value.status == SDM_ERR_CAPACITY and gm.seq_length(0) == 64
    torch.cuda.synchronize()
    assert out[:25].cpu().tolist() == O.generate_ar(om, p, 25).tokens
    # a linear block that ends at position 63, then one that would not fit
    gm.seq_reset(1)
    p = W.prompt_ids(TINY, 32, seed=8)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.prefill(1, _i32(p), nxt)
    blk = torch.empty(32, dtype=torch.int32, device=DEV)
    ar = torch.empty(32, dtype=torch.int32, device=DEV)
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    gm.draft_block(1, nxt, 32, blk)
    gm.verify_block([1], blk, 32, ar, acc)
    gm.commit_kv(1, 1)
    with pytest.raises(SdmError) as e:
        gm.draft_block(1, ar, 32, blk)
    assert e.value.status == SDM_ERR_CAPACITY and gm.seq_length(1) == 33
    # a quadratic block whose last candidate ends at position 63, then one that would not fit
    gm.seq_reset(2)
    gm.prefill(2, _i32(p), nxt)
    gm.draft_block(2, nxt, 16, blk[:16])
    nx = torch.empty((16, 16), dtype=torch.int32, device=DEV)
    gm.verify_block_quadratic(2, blk[:16], 16, ar[:16], acc, nx)
    gm.commit_kv(2, 1)
    nx2 = torch.empty((16, 16), dtype=torch.int32, device=DEV)
    with pytest.raises(SdmError) as e:
        gm.verify_block_quadratic(2, nx[0], 16, ar[:16], acc, nx2)
    assert e.value.status == SDM_ERR_CAPACITY and gm.seq_length(2) == 33
    torch.cuda.synchronize()


def test_empty_prompt_rejected(gm):
    from self_speculative_amd._lib import SDM_ERR_ARG, SdmError
    gm.seq_reset(4)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    with pytest.raises(SdmError) as e:
        gm.prefill(4, torch.empty(0, dtype=torch.int32, device=DEV), nxt)
    assert e.value.status == SDM_ERR_ARG and gm.seq_length(4) == 0
