"""Pins of the oracle's building blocks against closed forms, library routines
and brute force (CPU only)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W

rng = np.random.default_rng(1234)


# -- bf16 rounding ---------------------------------------------------------------
def test_bf16_round_matches_torch_on_float32_inputs():
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),        # subnormal range
        np.float32([0.0, -0.0, 1.0, -2.5, 3.0e38, 1.17549435e-38]),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even_closed_form():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert O.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert O.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert O.bf16_round(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)
    # values already on the bf16 grid are fixed points
    g = O.decode_bf16_bits(np.arange(0, 0x7F80, 7, dtype=np.uint16))
    np.testing.assert_array_equal(O.bf16_round(g), g)


def test_generator_bf16_bits_match_torch_and_oracle_decode():
    x = rng.standard_normal(5000).astype(np.float32)
    bits = W.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    np.testing.assert_array_equal(O.decode_bf16_bits(bits), O.bf16_round(x.astype(np.float64)))


# -- norms and activations -----------------------------------------------------------
def test_rms_normalize_matches_torch_rms_norm():
    h = rng.standard_normal((7, 96)) * 3.0
    ref = F.rms_norm(torch.from_numpy(h), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_normalize(h, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_rms_normalize_closed_form():
    # a constant row c normalises to c / sqrt(c^2 + eps)
    out = O.rms_normalize(np.full((1, 8), 2.0), 1e-6)
    np.testing.assert_allclose(out, 2.0 / math.sqrt(4.0 + 1e-6), rtol=1e-15)


def test_silu_matches_torch():
    x = rng.standard_normal(1000) * 6
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-15)
    assert O.silu(np.array([0.0]))[0] == 0.0


# -- RoPE ------------------------------------------------------------------------------
def _hf_rope(x, positions, base):
    """transformers' Llama rotate-half RoPE (a third-party implementation)."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    T, H, hd = x.shape
    cfg = LlamaConfig(hidden_size=H * hd, num_attention_heads=H, head_dim=hd, rope_theta=base,
                      max_position_embeddings=1 << 16)
    emb = LlamaRotaryEmbedding(cfg)
    xt = torch.from_numpy(x).permute(1, 0, 2)[None]                        # [1, H, T, hd]
    pos = torch.from_numpy(np.asarray(positions))[None]
    cos, sin = emb(xt, pos)
    q, _ = apply_rotary_pos_emb(xt, xt, cos.double(), sin.double())
    return q[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hd", [16, 128])
def test_rope_matches_transformers_llama(hd):
    x = rng.standard_normal((5, 3, hd))
    pos = np.array([0, 1, 17, 1000, 30000])
    cos, sin = O.rope_tables(pos, hd, 10000.0)
    ours = O.apply_rope(x, cos, sin)
    ref = _hf_rope(x, pos, 10000.0)
    # transformers takes cos/sin in float32 as well; residual difference is the
    # float32 evaluation of the angle at large positions.
    np.testing.assert_allclose(ours, ref, rtol=0, atol=2e-3 * np.abs(x).max())
    np.testing.assert_allclose(ours[:3], ref[:3], rtol=0, atol=1e-6)


def test_rope_invariants():
    hd = 16
    x = rng.standard_normal((1, 2, hd))
    c0, s0 = O.rope_tables(np.array([0]), hd, 10000.0)
    np.testing.assert_array_equal(O.apply_rope(x, c0, s0), x)              # position 0: identity
    c, s = O.rope_tables(np.array([123]), hd, 10000.0)
    r = O.apply_rope(x, c, s)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-7)
    # q(m).k(n) depends only on m - n
    q, k = rng.standard_normal((1, 1, hd)), rng.standard_normal((1, 1, hd))

    def score(m, n):
        cm, sm = O.rope_tables(np.array([m]), hd, 10000.0)
        cn, sn = O.rope_tables(np.array([n]), hd, 10000.0)
        return float((O.apply_rope(q, cm, sm) * O.apply_rope(k, cn, sn)).sum())
    assert abs(score(10, 3) - score(107, 100)) < 1e-6
    assert abs(score(5, 5) - float((q * k).sum())) < 1e-6


def test_rope_complex_closed_form():
    # pairing (t, t+hd/2) rotated by p * base^(-2t/hd) is multiplication of
    # x_t + i x_{t+hd/2} by exp(i p base^(-2t/hd)); frequencies at t = 0 and the
    # last pair are 1 and base^(-(hd-2)/hd).
    hd, p = 8, 7
    x = rng.standard_normal((1, 1, hd))
    c, s = O.rope_tables(np.array([p]), hd, 10000.0)
    r = O.apply_rope(x, c, s)
    z = x[0, 0, :4] + 1j * x[0, 0, 4:]
    freqs = np.array([1.0, 10000.0 ** -0.25, 10000.0 ** -0.5, 10000.0 ** -0.75])
    w = z * np.exp(1j * p * freqs)
    np.testing.assert_allclose(r[0, 0], np.concatenate([w.real, w.imag]), atol=1e-6)


# -- attention ------------------------------------------------------------------------
def _brute_mask(n, T, bidir):
    m = np.zeros((T, n + T), dtype=bool)
    for i in range(T):
        for j in range(n + T):
            if j < n:
                m[i, j] = True
            elif bidir:
                m[i, j] = True
            else:
                m[i, j] = (j - n) <= i
    return m


@pytest.mark.parametrize("n,T", [(0, 1), (0, 5), (3, 1), (9, 4), (17, 8)])
@pytest.mark.parametrize("mode", [O.CAUSAL, O.BIDIR])
def test_visible_matches_brute_force(n, T, mode):
    np.testing.assert_array_equal(O.visible(n, T, mode), _brute_mask(n, T, mode == O.BIDIR))


def _sdpa_ref(q, K, V, n, bidir):
    """torch SDPA with an explicit boolean mask and repeat_interleave'd KV heads."""
    T, Hq, hd = q.shape
    G = Hq // K.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
    mask = torch.from_numpy(_brute_mask(n, T, bidir))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("n,T,Hq,Hkv,hd", [(0, 4, 4, 2, 16), (13, 8, 4, 2, 16), (64, 32, 8, 2, 32),
                                          (5, 3, 6, 3, 8), (7, 5, 4, 4, 16)])
@pytest.mark.parametrize("mode", [O.CAUSAL, O.BIDIR])
@pytest.mark.parametrize("row_ind", [False, True])
def test_attention_matches_sdpa(n, T, Hq, Hkv, hd, mode, row_ind):
    q = rng.standard_normal((T, Hq, hd))
    K = rng.standard_normal((n + T, Hkv, hd))
    V = rng.standard_normal((n + T, Hkv, hd))
    ours = O.attention(q, K, V, n, mode, row_independent=row_ind)
    np.testing.assert_allclose(ours, _sdpa_ref(q, K, V, n, mode == O.BIDIR), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    Hq, Hkv, hd = 4, 2, 16
    q1 = rng.standard_normal((1, Hq, hd))
    K = rng.standard_normal((10, Hkv, hd))
    V = rng.standard_normal((10, Hkv, hd))
    # B = 1: bidirectional equals causal
    np.testing.assert_array_equal(O.attention(q1, K, V, 9, O.BIDIR), O.attention(q1, K, V, 9, O.CAUSAL))
    # last block row sees the same keys under both masks
    q = rng.standard_normal((6, Hq, hd))
    a = O.attention(q, K, V, 4, O.BIDIR)
    b = O.attention(q, K, V, 4, O.CAUSAL)
    np.testing.assert_allclose(a[-1], b[-1], rtol=1e-13)
    assert np.abs(a[0] - b[0]).max() > 1e-3
    # n = 0 bidirectional is full attention: a single softmax over all keys
    qq = rng.standard_normal((10, Hq, hd))
    full = O.attention(qq, K, V, 0, O.BIDIR)
    s = np.einsum("thd,jhd->thj", qq, np.repeat(K, 2, axis=1)) / 4.0
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    np.testing.assert_allclose(full, np.einsum("thj,jhd->thd", p, np.repeat(V, 2, axis=1)), rtol=1e-12)


# -- row selection ----------------------------------------------------------------------
def test_select_rows_matches_numpy_routines():
    V, mask = 300, 299
    l = rng.standard_normal((40, V)) * 2
    l[3, mask] = 100.0                       # planted maximum on the MASK column
    l[5, [10, 20]] = l[5].max() + 1.0        # planted tie: lowest id wins
    l[7, [250, 11, 12]] = 50.0
    tok, conf, margin = O.select_rows(l, mask)
    ll = l.copy()
    ll[:, mask] = -np.inf
    np.testing.assert_array_equal(tok, np.argmax(ll, axis=1))
    assert tok[3] != mask and tok[5] == 10 and tok[7] == 11
    from scipy.special import logsumexp
    np.testing.assert_allclose(np.log(conf), ll.max(1) - logsumexp(ll, axis=1), rtol=1e-12, atol=1e-12)
    top2 = -np.partition(-ll, 1, axis=1)[:, :2]
    np.testing.assert_allclose(margin, top2[:, 0] - top2[:, 1], rtol=0, atol=0)
    assert margin[5] == 0.0 and margin[7] == 0.0


def test_select_rows_uniform_and_onehot():
    l = np.zeros((1, 11))
    tok, conf, margin = O.select_rows(l, 10)
    assert tok[0] == 0 and abs(conf[0] - 0.1) < 1e-15 and margin[0] == 0
    l = np.full((1, 11), -1e9)
    l[0, 4] = 0.0
    tok, conf, margin = O.select_rows(l, 10)
    assert tok[0] == 4 and conf[0] == 1.0
