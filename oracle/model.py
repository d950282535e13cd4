"""CPU oracle of the block-wise decoding forward -- TEST INFRASTRUCTURE ONLY.

Only tests, the package's ``smoke()`` check and the benchmark's CPU-baseline
leg may import this module.  The product path never calls it.  It shares no
code with the HIP library: it imports only numpy and the seeded input module.

What it computes
----------------
One random-init decoder serves all three decoding modes; only the attention
mask and the token-selection rule change (Nemotron-Labs-Diffusion pages:
ai-feeds "inference: three modes", fintech-frontier-insights "three generation
modes": the same checkpoint switches modes without retraining).  Attention is
block-wise: the cached prefix is visible to every block row, and inside the
block rows see each other bidirectionally when drafting/denoising and causally
when verifying or decoding AR (fintech-frontier-insights, training route: the
Efficient-DLM block-wise attention; ai-feeds "training": one attention pattern
serves both paradigms with no extra parameters).

The forward, written out (pre-norm decoder, no biases, untied LM head):

    h      = E[x]                                   residual stream, float
    for each layer:
      a    = A(rms(h) * g1)
      q    = A(rope(a Wq^T, p)),  k = R(rope(a Wk^T, p)),  v = R(a Wv^T)
      o    = softmax over visible keys of (q . k / sqrt(hd)) applied to v
      h    = h + A(o) Wo^T
      b    = A(rms(h) * g2)
      u    = A(silu(b Wg^T) * (b Wu^T))
      h    = h + u Wd^T
    logits = A(rms(h) * gf) Wlm^T

with rms(h) = h / sqrt(mean(h^2) + eps), silu(x) = x / (1 + exp(-x)), key j
visible to block row i (absolute positions, block starts at n) iff j < n, or
j is in the block and (bidirectional, or j <= n + i); query head h uses KV
head floor(h * Hkv / Hq); rope rotates the pairs (t, t + hd/2) by the angle
p * base^(-2t/hd), the angle taken in float64 and cos/sin rounded to float32.

Storage precision of a bf16 shape.  R() is the rounding to bf16 (nearest,
ties to even): the weights and k/v after RoPE -- the paged KV cache -- are
bf16.  A() is the rounding of an activation that one kernel hands to the next
(the normalised activations, q, the attention output, the SwiGLU product) to a
two-term bf16 expansion, hi = R(x), lo = R(x - hi), value hi + lo: about 16
significant bits, which the bf16 matrix units consume as two products.  The
residual stream and the logits stay wide.  For float32 shapes R() and A() are
the identity.  Arithmetic between rounding points is float64 by default.

Row selection on a logits row (MASK excluded everywhere): tok = smallest id
reaching the max, conf = 1 / sum_v exp(l_v - max), margin = max minus the
largest logit over ids other than tok.

Readings of points the pages leave open are listed in the repository's design
notes; the ones that shape this file: MASK = V-1 is excluded from softmax and
argmax in every mode; eps 1e-6; RoPE base 10000, rotate-half pairing; norm
gains are per-feature multipliers applied after the normalisation.

Row independence.  With ``row_independent=True`` each block row is pushed
through every matmul, norm and attention by the same per-row routine that a
one-row (AR) forward uses, so a causal block forward reproduces the AR
forward bit for bit.  This is what makes "self-speculation at temperature 0
equals greedy AR" (fintech-frontier-insights, "three generation modes",
self-speculation bullet, and its accuracy list) an exact, checkable identity.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

CAUSAL = 0
BIDIR = 1


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round each value to the nearest bf16 number (ties to even), keep dtype.

    bf16 keeps 8 significant bits and float32's exponent range; below 2^-126
    the spacing stays 2^-133 (subnormals).  Done in float64 arithmetic, which
    represents x / quantum exactly for every finite input here.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                  # x = m * 2^e, |m| in [0.5, 1)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)          # spacing of bf16 numbers near x
    with np.errstate(invalid="ignore"):
        r = np.rint(x / q) * q                          # rint: half to even
    return np.where(x == 0, x, r)


def bf16_pair_round(x: np.ndarray) -> np.ndarray:
    """x rounded to a two-term bf16 expansion: hi = bf16(x), lo = bf16(x - hi),
    returned as the float64 value hi + lo (exact: both terms are bf16 numbers
    within 2^-8 of each other's scale)."""
    x = np.asarray(x, dtype=np.float64)
    hi = bf16_round(x)
    return hi + bf16_round(x - hi)


def decode_bf16_bits(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact float64 values."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


INT4_GROUP = 128  # input columns sharing one scale


def int4_codes(codes: np.ndarray) -> np.ndarray:
    """Unpack 4-bit weight codes.  ``codes`` is uint8 [rows, cols/2]; byte j of
    a row holds column 2j in its low nibble and column 2j+1 in its high nibble,
    each a two's-complement integer in [-8, 7].  Returns int64 [rows, cols]."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    q = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int64)
    q[:, 0::2] = b & 15
    q[:, 1::2] = b >> 4
    return np.where(q >= 8, q - 16, q)


def dequant_int4(codes: np.ndarray, scale_bits: np.ndarray, group: int = INT4_GROUP) -> np.ndarray:
    """Weight-only 4-bit matrix (the w4a16 format of the DGX Spark row of
    fintech-frontier-insights' hardware table, read as group-wise int4 with one
    bf16 scale per output row and group of ``group`` input columns):
    w[r, c] = s[r, c // group] * q[r, c], exact in float64.  ``scale_bits`` is
    uint16 bf16 bits [rows, cols / group]."""
    q = int4_codes(codes)
    s = decode_bf16_bits(scale_bits)
    return q * np.repeat(s, group, axis=1)


def rms_normalize(h: np.ndarray, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) along the last axis."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope_tables(positions: np.ndarray, head_dim: int, base: float):
    """cos, sin of p * base^(-2t/hd) for t < hd/2: angle in float64, values
    rounded to float32 (then widened back)."""
    t = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * t / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return (np.cos(ang).astype(np.float32).astype(np.float64),
            np.sin(ang).astype(np.float32).astype(np.float64))


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (t, t + hd/2) of x [T, H, hd] by the per-row angles."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def visible(n: int, T: int, mode: int) -> np.ndarray:
    """Boolean [T, n+T]: key j visible to block row i (block at n..n+T-1)."""
    i = np.arange(T)[:, None]
    j = np.arange(n + T)[None, :]
    in_block = j >= n
    return (~in_block) | (mode == BIDIR) | (j <= n + i)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, n: int, mode: int,
              row_independent: bool = False) -> np.ndarray:
    """Block attention.  q [T, Hq, hd]; K, V [n+T, Hkv, hd] (prefix then block).

    Returns o [T, Hq, hd].  Softmax scale 1/sqrt(hd).  Masked keys are left out
    of the softmax entirely (equivalent to a -inf score).
    """
    T, Hq, hd = q.shape
    Hkv = K.shape[1]
    scale = 1.0 / math.sqrt(hd)
    vis = visible(n, T, mode)
    o = np.empty_like(q)
    for h in range(Hq):
        kvh = (h * Hkv) // Hq
        if row_independent:
            for i in range(T):
                keys = np.nonzero(vis[i])[0]
                kk, vv = K[keys, kvh], V[keys, kvh]
                s = (kk @ q[i, h]) * scale
                p = np.exp(s - s.max())
                o[i, h] = (p @ vv) / p.sum()
        else:
            s = (q[:, h] @ K[:, kvh].T) * scale
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            o[:, h] = (p @ V[:, kvh]) / p.sum(axis=1, keepdims=True)
    return o


def attention_masked(q: np.ndarray, K: np.ndarray, V: np.ndarray, vis: np.ndarray,
                     row_independent: bool = False) -> np.ndarray:
    """Attention under an explicit visibility.  q [T, Hq, hd]; K, V [nk, Hkv,
    hd]; vis boolean [T, nk] (row i sees key j iff vis[i, j]).  Returns o [T,
    Hq, hd]; invisible keys are left out of the softmax."""
    T, Hq, hd = q.shape
    Hkv = K.shape[1]
    scale = 1.0 / math.sqrt(hd)
    o = np.empty_like(q)
    for h in range(Hq):
        kvh = (h * Hkv) // Hq
        if row_independent:
            for i in range(T):
                keys = np.nonzero(vis[i])[0]
                s = (K[keys, kvh] @ q[i, h]) * scale
                p = np.exp(s - s.max())
                o[i, h] = (p @ V[keys, kvh]) / p.sum()
        else:
            s = np.where(vis, (q[:, h] @ K[:, kvh].T) * scale, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o[:, h] = (p @ V[:, kvh]) / p.sum(axis=1, keepdims=True)
    return o


def select_rows(logits: np.ndarray, mask_id: int):
    """Per-row (tok, conf, margin) with MASK excluded.  logits [T, V]."""
    l = np.array(logits, dtype=np.float64, copy=True)
    l[:, mask_id] = -np.inf
    tok = np.argmax(l, axis=1)                      # first (lowest) id on ties
    mx = l[np.arange(l.shape[0]), tok]
    conf = 1.0 / np.exp(l - mx[:, None]).sum(axis=1)
    l2 = l.copy()
    l2[np.arange(l.shape[0]), tok] = -np.inf
    margin = mx - l2.max(axis=1)
    return tok.astype(np.int32), conf, margin


@dataclass
class LayerWeights:
    attn_norm: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    ffn_norm: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray


class KVCache:
    """Per-layer K/V rows by absolute position, plus the committed length."""

    def __init__(self, n_layers: int, capacity: int, n_kv_heads: int, head_dim: int, dtype=np.float64):
        self.K = [np.zeros((capacity, n_kv_heads, head_dim), dtype) for _ in range(n_layers)]
        self.V = [np.zeros((capacity, n_kv_heads, head_dim), dtype) for _ in range(n_layers)]
        self.n = 0

    @property
    def capacity(self) -> int:
        return self.K[0].shape[0]

    def ensure(self, need: int):
        if need <= self.capacity:
            return
        cap = max(need, 2 * self.capacity)
        for lst in (self.K, self.V):
            for l, a in enumerate(lst):
                b = np.zeros((cap,) + a.shape[1:], a.dtype)
                b[: a.shape[0]] = a
                lst[l] = b


class OracleModel:
    """The decoder as a pure function of (weights, tokens, positions, cache, mode).

    ``weights`` is the dict produced by ``workloads.make_weights`` (float32
    arrays, or uint16 bf16 bits for bf16 shapes) or by
    ``workloads.make_w4_weights`` (the decoder's linear layers as 4-bit codes
    ``<name>.codes`` plus bf16 scales ``<name>.scales``; they are dequantized
    exactly, then used as any other weight).  Layer weights are widened to
    ``dtype`` lazily; ``cache_layers`` keeps them widened between forwards.
    """

    def __init__(self, shape, weights: Dict[str, np.ndarray], dtype=np.float64,
                 row_independent: bool = False, cache_layers: bool = True):
        self.shape = shape
        self.bf16 = shape.dtype == "bf16"
        self.dtype = dtype
        self.row_independent = row_independent
        self.cache_layers = cache_layers
        self._raw = weights
        self._layers: Dict[int, LayerWeights] = {}
        self.embed_raw = weights["embed"]
        self.final_norm = self._widen(weights["final_norm"])
        self._lm_head: Optional[np.ndarray] = None

    # -- weights -----------------------------------------------------------
    def _widen(self, a: np.ndarray) -> np.ndarray:
        if self.bf16:
            return decode_bf16_bits(a).astype(self.dtype, copy=False)
        return np.asarray(a).astype(self.dtype)

    def R(self, x: np.ndarray) -> np.ndarray:
        """bf16 storage (the KV cache)."""
        return bf16_round(x).astype(self.dtype, copy=False) if self.bf16 else x

    def A(self, x: np.ndarray) -> np.ndarray:
        """Two-term bf16 storage of an activation handed between kernels."""
        return bf16_pair_round(x).astype(self.dtype, copy=False) if self.bf16 else x

    def _matrix(self, name: str) -> np.ndarray:
        """A weight matrix [out, in]: 4-bit codes are dequantized, bf16 widened."""
        w = self._raw
        if name + ".codes" in w:
            return dequant_int4(w[name + ".codes"], w[name + ".scales"]).astype(self.dtype, copy=False)
        return self._widen(w[name])

    def layer(self, l: int) -> LayerWeights:
        if l in self._layers:
            return self._layers[l]
        s, w, p = self.shape, self._raw, f"layers.{l}."
        qkv = self._matrix(p + "w_qkv")
        lw = LayerWeights(
            attn_norm=self._widen(w[p + "attn_norm"]),
            wq=qkv[: s.q_dim], wk=qkv[s.q_dim: s.q_dim + s.kv_dim], wv=qkv[s.q_dim + s.kv_dim:],
            wo=self._matrix(p + "w_o"),
            ffn_norm=self._widen(w[p + "ffn_norm"]),
            wg=self._matrix(p + "w_gate"), wu=self._matrix(p + "w_up"),
            wd=self._matrix(p + "w_down"),
        )
        if self.cache_layers:
            self._layers[l] = lw
        return lw

    def lm_head(self) -> np.ndarray:
        if self._lm_head is not None:
            return self._lm_head
        w = self._widen(self._raw["lm_head"])
        if self.cache_layers:
            self._lm_head = w
        return w

    def embed_rows(self, tokens: np.ndarray) -> np.ndarray:
        return self._widen(self.embed_raw[np.asarray(tokens)])

    # -- building blocks -------------------------------------------------------
    def _mm(self, x: np.ndarray, w: np.ndarray) -> np.ndarray:
        """x [T, in] times W^T for W [out, in]."""
        if self.row_independent:
            return np.stack([w @ x[i] for i in range(x.shape[0])])
        return x @ w.T

    def _norm(self, h: np.ndarray, g: np.ndarray) -> np.ndarray:
        eps = self.shape.rms_eps
        if self.row_independent:
            return np.stack([rms_normalize(h[i], eps) for i in range(h.shape[0])]) * g
        return rms_normalize(h, eps) * g

    # -- the forward -----------------------------------------------------------
    def forward(self, cache: KVCache, tokens: Sequence[int], mode: int,
                logits_rows: Optional[Sequence[int]] = None) -> np.ndarray:
        """Run the block [tokens] at positions cache.n .. cache.n+T-1.

        K/V of the block are written to the cache's pending rows n..n+T-1 (the
        committed length is not changed).  Returns logits [T, V] (or only the
        rows listed in ``logits_rows``).
        """
        s = self.shape
        tokens = np.asarray(tokens, dtype=np.int64)
        T, n = len(tokens), cache.n
        cache.ensure(n + T)
        pos = np.arange(n, n + T)
        cos, sin = rope_tables(pos, s.head_dim, s.rope_base)
        h = self.embed_rows(tokens)
        for l in range(s.n_layers):
            w = self.layer(l)
            a = self.A(self._norm(h, w.attn_norm))
            q = self.A(apply_rope(self._mm(a, w.wq).reshape(T, s.n_q_heads, s.head_dim), cos, sin))
            k = self.R(apply_rope(self._mm(a, w.wk).reshape(T, s.n_kv_heads, s.head_dim), cos, sin))
            v = self.R(self._mm(a, w.wv).reshape(T, s.n_kv_heads, s.head_dim))
            cache.K[l][n:n + T] = k
            cache.V[l][n:n + T] = v
            o = attention(q, cache.K[l][: n + T], cache.V[l][: n + T], n, mode, self.row_independent)
            h = h + self._mm(self.A(o.reshape(T, s.q_dim)), w.wo)
            b = self.A(self._norm(h, w.ffn_norm))
            u = self.A(silu(self._mm(b, w.wg)) * self._mm(b, w.wu))
            h = h + self._mm(u, w.wd)
        if logits_rows is not None:
            h = h[np.asarray(logits_rows)]
        z = self.A(self._norm(h, self.final_norm))
        return self._mm(z, self.lm_head())

    def forward_masked(self, cache: KVCache, tokens: Sequence[int], positions: Sequence[int],
                       vis: np.ndarray, n_write: int) -> np.ndarray:
        """Rows at arbitrary positions under an explicit visibility.

        The keys are the committed prefix 0..n-1 followed by the T rows of
        this call in row order; ``vis`` [T, n+T] says which of them each row
        sees.  RoPE uses ``positions``.  The K/V of the first ``n_write`` rows
        go to the cache's pending rows n..n+n_write-1 (the committed length
        is not changed); the other rows' K/V live only inside this call.
        Returns logits [T, V]."""
        s = self.shape
        tokens = np.asarray(tokens, dtype=np.int64)
        pos = np.asarray(positions, dtype=np.int64)
        T, n = len(tokens), cache.n
        vis = np.asarray(vis, dtype=bool)
        assert vis.shape == (T, n + T) and pos.shape == (T,)
        cache.ensure(n + n_write)
        cos, sin = rope_tables(pos, s.head_dim, s.rope_base)
        h = self.embed_rows(tokens)
        for l in range(s.n_layers):
            w = self.layer(l)
            a = self.A(self._norm(h, w.attn_norm))
            q = self.A(apply_rope(self._mm(a, w.wq).reshape(T, s.n_q_heads, s.head_dim), cos, sin))
            k = self.R(apply_rope(self._mm(a, w.wk).reshape(T, s.n_kv_heads, s.head_dim), cos, sin))
            v = self.R(self._mm(a, w.wv).reshape(T, s.n_kv_heads, s.head_dim))
            cache.K[l][n:n + n_write] = k[:n_write]
            cache.V[l][n:n + n_write] = v[:n_write]
            K = np.concatenate([cache.K[l][:n], k])
            V = np.concatenate([cache.V[l][:n], v])
            o = attention_masked(q, K, V, vis, self.row_independent)
            h = h + self._mm(self.A(o.reshape(T, s.q_dim)), w.wo)
            b = self.A(self._norm(h, w.ffn_norm))
            u = self.A(silu(self._mm(b, w.wg)) * self._mm(b, w.wu))
            h = h + self._mm(u, w.wd)
        z = self.A(self._norm(h, self.final_norm))
        return self._mm(z, self.lm_head())

    def new_cache(self, capacity: int = 64) -> KVCache:
        s = self.shape
        return KVCache(s.n_layers, capacity, s.n_kv_heads, s.head_dim, self.dtype)
