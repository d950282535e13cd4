"""Whole-forward pins of the oracle (CPU only).

* CAUSAL mode on a float shape equals transformers' Llama decoder (pre-norm
  RMSNorm, rotate-half RoPE, SwiGLU, GQA, no biases, untied head) loaded with
  the same weights -- a third-party implementation of the same architecture.
* BIDIR mode equals an independent torch composition (F.linear, SDPA with an
  explicit mask, F.rms_norm, F.silu, complex-number RoPE).
* On a bf16 shape, the oracle's rounding points equal the same composition
  with torch's own bf16 casts at those points: a single bf16 cast for k and v
  (the KV cache), a two-term cast (hi, then the residual) for the activations
  handed between kernels.  Moving either kind of point to the other rounding
  is detected.
"""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W

TINY = W.SHAPES["tiny"]
SMALL_BF16 = W.ModelShape("small-bf16", 2, 128, 4, 2, 32, 256, 512, "bf16")


def _f64(shape, w, name):
    a = w[name]
    if shape.dtype == "bf16":
        return torch.from_numpy(O.decode_bf16_bits(a))
    return torch.from_numpy(a.astype(np.float64))


def _llama(shape, w):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.d_model, intermediate_size=shape.ffn_dim,
                      num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_q_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rms_norm_eps=shape.rms_eps, rope_theta=shape.rope_base, tie_word_embeddings=False,
                      attention_bias=False, mlp_bias=False, max_position_embeddings=4096)
    cfg._attn_implementation = "eager"
    m = LlamaForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": _f64(shape, w, "embed"), "model.norm.weight": _f64(shape, w, "final_norm"),
          "lm_head.weight": _f64(shape, w, "lm_head")}
    for l in range(shape.n_layers):
        p, q = f"layers.{l}.", f"model.layers.{l}."
        qkv = _f64(shape, w, p + "w_qkv")
        sd[q + "self_attn.q_proj.weight"] = qkv[: shape.q_dim]
        sd[q + "self_attn.k_proj.weight"] = qkv[shape.q_dim: shape.q_dim + shape.kv_dim]
        sd[q + "self_attn.v_proj.weight"] = qkv[shape.q_dim + shape.kv_dim:]
        sd[q + "self_attn.o_proj.weight"] = _f64(shape, w, p + "w_o")
        sd[q + "mlp.gate_proj.weight"] = _f64(shape, w, p + "w_gate")
        sd[q + "mlp.up_proj.weight"] = _f64(shape, w, p + "w_up")
        sd[q + "mlp.down_proj.weight"] = _f64(shape, w, p + "w_down")
        sd[q + "input_layernorm.weight"] = _f64(shape, w, p + "attn_norm")
        sd[q + "post_attention_layernorm.weight"] = _f64(shape, w, p + "ffn_norm")
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in k for k in missing), (missing, unexpected)
    return m


@pytest.mark.parametrize("row_ind", [False, True])
def test_causal_forward_equals_transformers_llama(row_ind):
    w = W.make_weights(TINY, seed=3, gains="random")
    m = O.OracleModel(TINY, w, row_independent=row_ind)
    toks = W.prompt_ids(TINY, 21, seed=3)
    ours = m.forward(m.new_cache(), toks, O.CAUSAL)
    with torch.no_grad():
        ref = _llama(TINY, w)(torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    # transformers evaluates the RoPE angle and cos/sin in float32, the oracle
    # takes the angle in float64 and rounds cos/sin to float32: ~1e-7 relative.
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def test_causal_forward_with_cache_equals_transformers_llama():
    """Prefill 13 tokens, then an 8-token causal block on top of the cache."""
    w = W.make_weights(TINY, seed=4, gains="random")
    m = O.OracleModel(TINY, w)
    toks = W.prompt_ids(TINY, 21, seed=4)
    c = m.new_cache()
    m.forward(c, toks[:13], O.CAUSAL)
    c.n = 13
    ours = m.forward(c, toks[13:], O.CAUSAL)
    with torch.no_grad():
        ref = _llama(TINY, w)(torch.from_numpy(toks.astype(np.int64))[None]).logits[0, 13:].numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def _torch_forward(shape, w, prefix, block, bidir, rnd, rnd_kv=None):
    """Independent composition: whole sequence prefix+block in one pass, with
    the block's mask rule built by loops; rnd(x) is the storage rounding of the
    activations, rnd_kv(x) that of k and v (default: rnd)."""
    rnd_kv = rnd if rnd_kv is None else rnd_kv
    d, hd, Hq, Hkv = shape.d_model, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    toks = np.concatenate([prefix, block]).astype(np.int64)
    n, T = len(prefix), len(block)
    S = n + T
    mask = torch.zeros(S, S, dtype=torch.bool)
    for i in range(S):
        for j in range(S):
            if i < n:
                mask[i, j] = j <= i
            else:
                mask[i, j] = j < n or bidir or j <= i
    half = hd // 2
    pos = torch.arange(S, dtype=torch.float64)
    freqs = torch.tensor([shape.rope_base ** (-2.0 * t / hd) for t in range(half)], dtype=torch.float64)
    ang = pos[:, None] * freqs[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)
    rot = torch.complex(rot.real.float().double(), rot.imag.float().double())[:, None, :]

    def rope(x):                                   # x [S, H, hd]
        z = torch.complex(x[..., :half], x[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    h = _f64(shape, w, "embed")[toks]
    for l in range(shape.n_layers):
        p = f"layers.{l}."
        qkv = _f64(shape, w, p + "w_qkv")
        a = rnd(F.rms_norm(h, (d,), eps=shape.rms_eps) * _f64(shape, w, p + "attn_norm"))
        q = rnd(rope(F.linear(a, qkv[: shape.q_dim]).view(S, Hq, hd)))
        k = rnd_kv(rope(F.linear(a, qkv[shape.q_dim: shape.q_dim + shape.kv_dim]).view(S, Hkv, hd)))
        v = rnd_kv(F.linear(a, qkv[shape.q_dim + shape.kv_dim:]).view(S, Hkv, hd))
        G = Hq // Hkv
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1).repeat_interleave(G, 0),
                                           v.transpose(0, 1).repeat_interleave(G, 0), attn_mask=mask)
        h = h + F.linear(rnd(o.transpose(0, 1).reshape(S, Hq * hd)), _f64(shape, w, p + "w_o"))
        b = rnd(F.rms_norm(h, (d,), eps=shape.rms_eps) * _f64(shape, w, p + "ffn_norm"))
        u = rnd(F.silu(F.linear(b, _f64(shape, w, p + "w_gate"))) * F.linear(b, _f64(shape, w, p + "w_up")))
        h = h + F.linear(u, _f64(shape, w, p + "w_down"))
    z = rnd(F.rms_norm(h, (d,), eps=shape.rms_eps) * _f64(shape, w, "final_norm"))
    return F.linear(z, _f64(shape, w, "lm_head"))[n:].numpy()


@pytest.mark.parametrize("mode", [O.BIDIR, O.CAUSAL])
@pytest.mark.parametrize("n", [0, 11])
def test_block_forward_equals_torch_composition_float(mode, n):
    w = W.make_weights(TINY, seed=5, gains="random")
    m = O.OracleModel(TINY, w)
    toks = W.prompt_ids(TINY, n + 8, seed=5)
    toks[n + 3] = TINY.mask_id                      # MASK ids are ordinary embeddings in the forward
    c = m.new_cache()
    if n:
        m.forward(c, toks[:n], O.CAUSAL)
        c.n = n
    ours = m.forward(c, toks[n:], mode)
    ref = _torch_forward(TINY, w, toks[:n], toks[n:], mode == O.BIDIR, lambda x: x)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-10 * np.abs(ref).max())


@pytest.mark.parametrize("mode", [O.BIDIR, O.CAUSAL])
def test_block_forward_bf16_rounding_points(mode):
    """bf16 shape: rounding at the storage points, torch's own bf16 cast."""
    w = W.make_weights(SMALL_BF16, seed=6, gains="random")
    m = O.OracleModel(SMALL_BF16, w)
    toks = W.prompt_ids(SMALL_BF16, 19, seed=6)
    c = m.new_cache()
    m.forward(c, toks[:11], O.CAUSAL)
    c.n = 11
    ours = m.forward(c, toks[11:], mode)
    one = lambda x: x.to(torch.bfloat16).to(torch.float64)

    def two(x):
        hi = one(x)
        return hi + one(x - hi)

    bidir = mode == O.BIDIR
    ref = _torch_forward(SMALL_BF16, w, toks[:11], toks[11:], bidir, two, one)
    scale = np.abs(ref).max()
    # torch casts float64 -> bf16 through float32 (double rounding): a value
    # within float32 resolution of a bf16 midpoint could land one step away.
    tol = 2e-5 * scale
    assert np.abs(ref - ours).max() <= tol
    # each rounding point is visible: none at all, single bf16 for the
    # activations too, no KV rounding, or no activation rounding all move the
    # logits by far more (the last through k/v roundings that flip)
    ident = lambda x: x
    for act, kv in ((ident, ident), (one, one), (two, ident), (ident, one)):
        other = _torch_forward(SMALL_BF16, w, toks[:11], toks[11:], bidir, act, kv)
        assert np.abs(other - ours).max() > 10 * tol


def test_row_independent_equals_batched():
    w = W.make_weights(TINY, seed=7, gains="random")
    toks = W.prompt_ids(TINY, 24, seed=7)
    outs = []
    for ri in (False, True):
        m = O.OracleModel(TINY, w, row_independent=ri)
        c = m.new_cache()
        m.forward(c, toks[:16], O.CAUSAL)
        c.n = 16
        outs.append(m.forward(c, toks[16:], O.BIDIR))
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-12)


def test_kv_written_to_pending_rows_only():
    w = W.make_weights(TINY, seed=8)
    m = O.OracleModel(TINY, w)
    c = m.new_cache(64)
    toks = W.prompt_ids(TINY, 10, seed=8)
    m.forward(c, toks, O.CAUSAL)
    assert c.n == 0                                          # forward never commits
    assert np.abs(c.K[0][:10]).max() > 0 and np.abs(c.K[0][10:]).max() == 0


def test_generator_is_chunk_and_thread_independent():
    s = W.ModelShape("gen", 1, 64, 2, 1, 32, 128, 5000, "bf16")
    a = W.make_weights(s, seed=9, threads=1)
    b = W.make_weights(s, seed=9, threads=8)
    c = W.make_weights(s, seed=9, only=["lm_head"])
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_array_equal(a["lm_head"], c["lm_head"])
    vals = O.decode_bf16_bits(a["lm_head"])
    assert abs(vals.std() - 0.02) < 5e-4 and abs(vals.mean()) < 5e-4
    d = W.make_weights(s, seed=10, only=["lm_head"])
    assert not np.array_equal(a["lm_head"], d["lm_head"])
    p = W.prompt_ids(W.SHAPES["8b"], 100000, seed=0)
    assert p.min() >= 0 and p.max() == W.SHAPES["8b"].vocab - 2
