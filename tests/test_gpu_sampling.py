"""GPU parity of sampling at temperature > 0 (Philox4x64-10 draws, Gumbel-max
rows, the rejection-sampling verify) against the oracle's implementation of
the same definitions.

Both sides draw the same random numbers, so a run is deterministic: the GPU
must emit the oracle's tokens and accept lengths exactly.  fp32 against
float64 can flip only a decision closer to its boundary than the arithmetic
error, so each test takes the first seed whose every decision (Gumbel gaps,
|ln u - ln p/q|) clears a margin well above that error, then requires equal
streams.  The distributional properties (softmax frequencies, lossless
verify, the T -> 0 limit) are pinned on the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
TINY = W.SHAPES["tiny"]
SMALL = W.ModelShape("small-bf16", 2, 256, 4, 2, 128, 512, 1024, "bf16")


def _pick_seed(run, bar, seeds=range(1, 40)):
    for seed in seeds:
        r = run(seed)
        if min(r.margins) > bar:
            return seed, r
    pytest.fail(f"no seed with every decision margin above {bar}")


@pytest.fixture(scope="module")
def tiny():
    from self_speculative_amd.model import Model
    w = W.make_weights(TINY, seed=0)
    m = Model(TINY, w, max_seqs=4, max_block=8, max_context=512, max_rows=64)
    yield m, O.OracleModel(TINY, w, row_independent=True)
    m.close()


@pytest.fixture(scope="module")
def small():
    from self_speculative_amd.model import Model
    w = W.make_weights(SMALL, seed=21, gains="random")
    m = Model(SMALL, w, max_seqs=4, max_block=32, max_context=1024, max_rows=96)
    yield m, O.OracleModel(SMALL, w)
    m.close()


@pytest.mark.parametrize("T", [0.8, 2.0])
def test_tiny_ar_sample_stream(tiny, T):
    from self_speculative_amd import decode as D
    gm, om = tiny
    p = W.prompt_ids(TINY, 16, seed=0)
    seed, ref = _pick_seed(lambda s: O.generate_ar_sample(om, p, 48, T, s), 1e-4)
    print(f"tiny AR sample T={T} seed={seed}", flush=True)
    gm.seq_reset(0)
    g = D.generate_ar_sample(gm, p, 48, T, seed, seq=0)
    assert g.tokens == ref.tokens


@pytest.mark.parametrize("T,B", [(0.8, 8), (1.5, 4)])
def test_tiny_selfspec_sample_stream(tiny, T, B):
    from self_speculative_amd import decode as D
    gm, om = tiny
    p = W.prompt_ids(TINY, 16, seed=1)
    seed, ref = _pick_seed(lambda s: O.generate_selfspec_sample(om, p, 48, B, T, s, seq=1), 1e-4)
    print(f"tiny self-spec sample T={T} B={B} seed={seed}: oracle accepts {ref.accept_lengths}", flush=True)
    gm.seq_reset(1)
    g = D.generate_selfspec_sample(gm, p, 48, B, T, seed, seq=1)
    assert g.tokens == ref.tokens and g.accept_lengths == ref.accept_lengths
    assert min(ref.accept_lengths) < B                          # the residual path ran


def test_tiny_low_temperature_is_greedy(tiny):
    """T -> 0: sampled self-speculation emits the greedy AR stream (GPU)."""
    from self_speculative_amd import decode as D
    gm, om = tiny
    p = W.prompt_ids(TINY, 16, seed=2)
    gm.seq_reset(2)
    greedy = D.generate_ar(gm, p, 40, seq=2).tokens
    gm.seq_reset(2)
    print("tiny self-spec sample T=1e-4", flush=True)
    assert D.generate_selfspec_sample(gm, p, 40, 8, 1e-4, 5, seq=2).tokens == greedy


def test_small_bf16_selfspec_sample_stream(small):
    from self_speculative_amd import decode as D
    gm, om = small
    p = W.prompt_ids(SMALL, 70, seed=3)
    seed, ref = _pick_seed(lambda s: O.generate_selfspec_sample(om, p, 80, 32, 1.0, s), 2e-3, range(1, 12))
    print(f"small bf16 self-spec sample seed={seed}: oracle accepts {ref.accept_lengths}", flush=True)
    gm.seq_reset(0)
    g = D.generate_selfspec_sample(gm, p, 80, 32, 1.0, seed, seq=0)
    assert g.tokens == ref.tokens and g.accept_lengths == ref.accept_lengths


def test_sampling_argument_errors(small):
    from self_speculative_amd._lib import SdmError, SDM_ERR_ARG
    gm, _ = small
    gm.seq_reset(3)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    toks = torch.as_tensor(W.prompt_ids(SMALL, 10, seed=4), device=DEV)
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(SdmError) as e:
            gm.prefill_sample(3, toks, T, 1, nxt)
        assert e.value.status == SDM_ERR_ARG
    assert gm.seq_length(3) == 0                            # nothing ran


def test_w4_selfspec_sample_stream():
    """Sampling on a model with 4-bit decoder weights (the two extensions together)."""
    from self_speculative_amd import decode as D
    from self_speculative_amd.model import Model
    w = W.make_w4_weights(SMALL, seed=41, gains="random")
    om = O.OracleModel(SMALL, w)
    gm = Model(SMALL, w, max_seqs=1, max_block=16, max_context=512, max_rows=64)
    p = W.prompt_ids(SMALL, 50, seed=9)
    seed, ref = _pick_seed(lambda s: O.generate_selfspec_sample(om, p, 60, 16, 0.9, s), 2e-3, range(1, 12))
    print(f"w4 self-spec sample seed={seed}: oracle accepts {ref.accept_lengths}", flush=True)
    g = D.generate_selfspec_sample(gm, p, 60, 16, 0.9, seed, seq=0)
    gm.close()
    assert g.tokens == ref.tokens and g.accept_lengths == ref.accept_lengths


def test_sampled_tie_goes_to_the_lowest_id():
    """An exact tie of perturbed scores is resolved to the lowest id whatever
    thread scans it.  A row's ids are scanned in 4-id chunks handed to the
    threads round robin, so ids 4..7 (thread 1's first chunk) are lower than
    ids 1024..1027 (thread 0's second chunk of the same part).  LM-head rows 4
    and 1024 are set to 4096 x the row of the greedy token: both logits are
    then exactly 4096 x its logit (a power of two scales every product), and
    at T = 1e-6 a perturbed score above 4e8 absorbs the Gumbel noise
    (|g| < 18, below half a unit in the last place), so the two scores tie
    exactly in fp32.  The float64 oracle sees no tie there (its sum keeps the noise), so
    the rule itself is the reference."""
    from self_speculative_amd.model import Model
    s = W.ModelShape("tie-bf16", 1, 128, 1, 1, 128, 256, 151936, "bf16")
    w = W.make_weights(s, seed=5)
    p = torch.as_tensor(W.prompt_ids(s, 9, seed=5), device=DEV)
    nxt = torch.empty(1, dtype=torch.int32, device=DEV)
    lg = torch.empty((1, s.vocab), dtype=torch.float32, device=DEV)
    m = Model(s, w, max_seqs=1, max_block=8, max_context=64, max_rows=16)
    m.prefill(0, p, nxt, lg)
    torch.cuda.synchronize()
    j = int(nxt.item())
    top = float(lg[0, j].item())
    m.close()
    assert top > 0.1
    row = W.f32_from_bf16_bits(w["lm_head"][j]) * np.float32(4096.0)
    lo, hi = 4, 1024
    for planted, expect in (((hi,), hi), ((lo, hi), lo)):
        w2 = dict(w)
        w2["lm_head"] = w["lm_head"].copy()
        for v in planted:
            w2["lm_head"][v] = W.bf16_bits_from_f32(row)
        m = Model(s, w2, max_seqs=1, max_block=8, max_context=64, max_rows=16)
        for seed in (1, 2, 3):
            m.seq_reset(0)
            m.prefill_sample(0, p, 1e-6, seed, nxt)
            torch.cuda.synchronize()
            assert int(nxt.item()) == expect, (planted, seed, int(nxt.item()))
        m.close()
