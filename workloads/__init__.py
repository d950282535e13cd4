"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds only shapes and random draws: model shapes, random-init
weights, prompt ids, forced accept-length schedules, prompt-length mixes and
attention-op operands.  It contains none of the decoding method's arithmetic,
and imports neither the oracle nor the HIP package.

The shapes follow the workloads described on the pages: the 3B/8B/14B model
family of "Nemotron-Labs-Diffusion: A Tri-Mode Language Model ..." (hotpaper.ai
abstract; fintech-frontier-insights "open source and ecosystem" list of 3B,
8B, 14B sizes), decoded with 32-token blocks (fintech-frontier-insights, "three
generation modes", diffusion-mode bullet).  The trained checkpoints are not
available, so random-init weights N(0, 0.02^2) at those shapes stand in; the
pages' SPEED-Bench prompts are not available either, so uniform random ids of
the stated lengths stand in for them.

Random streams.  Every tensor is drawn from numpy's PCG64 seeded by
``SeedSequence(entropy=seed, spawn_key=(stream, index, chunk))``, so the value
of any tensor does not depend on which other tensors were drawn, in which
order, or on how many threads drew them.

Weight storage.  Matrices are produced in "out-major" layout ``[out, in]``
(row ``o`` holds the input weights of output feature ``o``; ``y = x @ W.T``).
For bf16 shapes the draw is made in float32 and rounded to the nearest bf16
(ties to even); the result is returned as the raw uint16 bit patterns, which
is exactly what the GPU stores.  float32 shapes return float32 arrays.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "ModelShape", "SHAPES", "weight_specs", "make_weights", "make_w4_weights", "INT4_LINEARS", "prompt_ids",
    "forced_accept_schedule", "prompt_lengths", "attention_op_inputs",
    "bf16_bits_from_f32", "f32_from_bf16_bits", "STREAM_WEIGHTS",
]

# Independent random streams (the first spawn-key component).
STREAM_WEIGHTS = 0
STREAM_PROMPT = 1
STREAM_FORCED_L = 2
STREAM_PROMPT_LENGTHS = 3
STREAM_ATTN_OP = 4
STREAM_GAINS = 5
STREAM_W4 = 6

# Decoder matrices stored as 4-bit codes by make_w4_weights (embedding and LM
# head stay bf16).
INT4_LINEARS = ("w_qkv", "w_o", "w_gate", "w_up", "w_down")
W4_GROUP = 128  # input columns per bf16 scale

_CHUNK = 1 << 24  # elements per independently seeded chunk of a large tensor


@dataclass(frozen=True)
class ModelShape:
    """Decoder shape.  ``mask_id`` is the reserved MASK token (the last id)."""
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    dtype: str  # "f32" or "bf16"
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    init_std: float = 0.02

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim

    def with_layers(self, n_layers: int) -> "ModelShape":
        return replace(self, name=f"{self.name}-L{n_layers}", n_layers=n_layers)


SHAPES: Dict[str, ModelShape] = {
    # Tiny fp32 decoder: 2 layers, d 64, 4/2 heads of 16, FFN 256, vocab 256.
    "tiny": ModelShape("tiny", 2, 64, 4, 2, 16, 256, 256, "f32"),
    "3b": ModelShape("3b", 28, 3072, 24, 8, 128, 8192, 151936, "bf16"),
    "8b": ModelShape("8b", 36, 4096, 32, 8, 128, 12288, 151936, "bf16"),
    "14b": ModelShape("14b", 40, 5120, 40, 8, 128, 17408, 151936, "bf16"),
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Used only to store the drawn inputs in the precision the GPU keeps them in.
    Inputs here are finite, so no NaN special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weight_specs(shape: ModelShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) of every weight tensor, in a fixed order.

    kind is "matrix" (drawn N(0, std^2)) or "gain" (RMSNorm gain, ones).
    """
    d, F = shape.d_model, shape.ffn_dim
    specs: List[Tuple[str, Tuple[int, ...], str]] = [("embed", (shape.vocab, d), "matrix")]
    for l in range(shape.n_layers):
        specs += [
            (f"layers.{l}.attn_norm", (d,), "gain"),
            (f"layers.{l}.w_qkv", (shape.qkv_dim, d), "matrix"),
            (f"layers.{l}.w_o", (d, shape.q_dim), "matrix"),
            (f"layers.{l}.ffn_norm", (d,), "gain"),
            (f"layers.{l}.w_gate", (F, d), "matrix"),
            (f"layers.{l}.w_up", (F, d), "matrix"),
            (f"layers.{l}.w_down", (d, F), "matrix"),
        ]
    specs += [("final_norm", (d,), "gain"), ("lm_head", (shape.vocab, d), "matrix")]
    return specs


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key))))


def _fill_chunk(out: np.ndarray, seed: int, key: Tuple[int, ...], std: float, bf16: bool, start: int, stop: int):
    g = _rng(seed, *key)
    x = g.standard_normal(stop - start, dtype=np.float32)
    x *= np.float32(std)
    if bf16:
        out[start:stop] = bf16_bits_from_f32(x)
    else:
        out[start:stop] = x


def make_weights(shape: ModelShape, seed: int = 0, gains: str = "ones",
                 threads: int | None = None, only: List[str] | None = None) -> Dict[str, np.ndarray]:
    """Draw every weight tensor of ``shape``.

    gains: "ones" (the model's init) or "random" (1 + N(0, 0.1^2), used by tests
    so that a dropped gain cannot go unnoticed).
    only: optional list of tensor names to draw (others are skipped).
    Returns float32 arrays for f32 shapes, uint16 bf16 bit arrays for bf16.
    """
    bf16 = shape.dtype == "bf16"
    threads = threads or min(16, os.cpu_count() or 1)
    out: Dict[str, np.ndarray] = {}
    jobs = []
    for idx, (name, shp, kind) in enumerate(weight_specs(shape)):
        if only is not None and name not in only:
            continue
        n = int(np.prod(shp))
        if kind == "gain":
            if gains == "ones":
                g = np.ones(n, dtype=np.float32)
            else:
                g = (1.0 + 0.1 * _rng(seed, STREAM_GAINS, idx).standard_normal(n)).astype(np.float32)
            out[name] = (bf16_bits_from_f32(g) if bf16 else g).reshape(shp)
            continue
        buf = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
        for c, start in enumerate(range(0, n, _CHUNK)):
            jobs.append((buf, (STREAM_WEIGHTS, idx, c), start, min(n, start + _CHUNK)))
        out[name] = buf.reshape(shp)
    if jobs:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda j: _fill_chunk(j[0], seed, j[1], shape.init_std, bf16, j[2], j[3]), jobs))
    return out


def _fill_w4_rows(codes: np.ndarray, scales: np.ndarray, seed: int, key: Tuple[int, ...], r0: int, r1: int):
    g = _rng(seed, *key)
    cols = codes.shape[1] * 2
    z = g.standard_normal((r1 - r0, cols), dtype=np.float32)
    q = np.clip(np.rint(z * np.float32(2.5)), -8, 7).astype(np.int8).view(np.uint8)
    codes[r0:r1] = (q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)
    sc = g.uniform(0.8, 1.25, size=(r1 - r0, cols // W4_GROUP)).astype(np.float32) * np.float32(0.008)
    scales[r0:r1] = bf16_bits_from_f32(sc)


def make_w4_weights(shape: ModelShape, seed: int = 0, gains: str = "ones",
                    threads: int | None = None) -> Dict[str, np.ndarray]:
    """Weights of a bf16 shape whose decoder matrices are 4-bit.

    The embedding, the LM head and the gains are those of ``make_weights``.
    Each matrix named in INT4_LINEARS, [out, in], becomes ``<name>.codes``,
    uint8 [out, in/2] (column 2j in the low nibble of byte j, 2j+1 in the high
    nibble, two's complement), and ``<name>.scales``, uint16 bf16 bits
    [out, in/128].  Both are drawn directly: codes are a standard normal times
    2.5, rounded and clipped to [-8, 7] (the bell shape of rounded Gaussian
    weights), scales 0.008 * U(0.8, 1.25), so the weights' spread is about
    0.02 as in the bf16 draw.
    """
    if shape.dtype != "bf16":
        raise ValueError("4-bit weights need a bf16 shape")
    specs = weight_specs(shape)
    is_lin = lambda name: name.startswith("layers.") and name.split(".")[-1] in INT4_LINEARS
    out = make_weights(shape, seed, gains, threads, only=[n for n, _, _ in specs if not is_lin(n)])
    threads = threads or min(16, os.cpu_count() or 1)
    jobs = []
    for idx, (name, shp, _) in enumerate(specs):
        if not is_lin(name):
            continue
        rows, cols = shp
        if cols % W4_GROUP:
            raise ValueError(f"{name}: {cols} input columns is not a multiple of {W4_GROUP}")
        codes = np.empty((rows, cols // 2), dtype=np.uint8)
        scales = np.empty((rows, cols // W4_GROUP), dtype=np.uint16)
        step = max(1, _CHUNK // cols)
        for c, r0 in enumerate(range(0, rows, step)):
            jobs.append((codes, scales, (STREAM_W4, idx, c), r0, min(rows, r0 + step)))
        out[name + ".codes"] = codes
        out[name + ".scales"] = scales
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda j: _fill_w4_rows(j[0], j[1], seed, j[2], j[3], j[4]), jobs))
    return out


def prompt_ids(shape: ModelShape, length: int, seed: int = 0, index: int = 0) -> np.ndarray:
    """``length`` prompt ids uniform over {0 .. V-2} (MASK = V-1 never appears)."""
    return _rng(seed, STREAM_PROMPT, index).integers(0, shape.vocab - 1, size=length, dtype=np.int64).astype(np.int32)


def forced_accept_schedule(n_cycles: int, block: int, seed: int = 0) -> np.ndarray:
    """Accept lengths drawn uniform over {1 .. block}, one per self-spec cycle."""
    return _rng(seed, STREAM_FORCED_L).integers(1, block + 1, size=n_cycles, dtype=np.int64).astype(np.int32)


def prompt_lengths(n_seq: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Per-sequence prompt lengths uniform over {lo .. hi}."""
    return _rng(seed, STREAM_PROMPT_LENGTHS).integers(lo, hi + 1, size=n_seq, dtype=np.int64).astype(np.int32)


def attention_op_inputs(prefix: int, block: int = 32, n_q_heads: int = 32, n_kv_heads: int = 8,
                        head_dim: int = 128, seed: int = 0, bf16: bool = True):
    """Standalone attention-op operands, entries N(0, 1).

    Returns (q [block, Hq, hd], k [prefix+block, Hkv, hd], v [prefix+block, Hkv, hd]),
    as uint16 bf16 bits when ``bf16`` else float32.
    """
    g = _rng(seed, STREAM_ATTN_OP, prefix, block)
    n = prefix + block
    q = g.standard_normal((block, n_q_heads, head_dim), dtype=np.float32)
    k = g.standard_normal((n, n_kv_heads, head_dim), dtype=np.float32)
    v = g.standard_normal((n, n_kv_heads, head_dim), dtype=np.float32)
    if bf16:
        return bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    return q, k, v
