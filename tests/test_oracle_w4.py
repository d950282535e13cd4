"""Pins of the oracle's 4-bit weight format (CPU only).

The format (a reading: the pages name only "w4a16" for the DGX Spark row of
fintech-frontier-insights' hardware table) is group-wise int4: two
two's-complement codes per byte, the even column in the low nibble, and one
bf16 scale per output row and group of input columns; the weight is
scale * code, exactly.

* A worked example with the expected weights written out by hand.
* Matrix products against a brute-force loop over bytes and nibbles that
  decodes the scales through ``struct``.
* A special case that reduces to the pinned bf16 model: with power-of-two
  scales every weight scale * code is a bf16 number, so the 4-bit model must
  give exactly the bf16 model's logits; with general scales it must not equal
  the model whose weights were rounded to bf16 (the dequantization is exact).
* The generator: deterministic, thread-independent, codes in [-8, 7].
"""
import struct

import numpy as np
import pytest

import oracle as O
import workloads as W

SMALL = W.ModelShape("small-bf16-w4", 2, 256, 4, 2, 128, 512, 1024, "bf16")


def _bf16(v: float) -> int:
    """bf16 bits of a float that is a bf16 number."""
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    assert b & 0xFFFF == 0, v
    return b >> 16


def test_worked_example_nibbles_sign_and_scale():
    codes = np.array([[0x8F, 0x71], [0x00, 0xF7]], dtype=np.uint8)
    scales = np.array([[_bf16(0.5), _bf16(3.0)], [_bf16(1.0), _bf16(-0.25)]], dtype=np.uint16)
    # row 0: bytes 0x8F -> (-1, -8), 0x71 -> (1, 7); row 1: 0x00 -> (0, 0), 0xF7 -> (7, -1)
    np.testing.assert_array_equal(O.int4_codes(codes), [[-1, -8, 1, 7], [0, 0, 7, -1]])
    w = O.dequant_int4(codes, scales, group=2)
    np.testing.assert_array_equal(w, [[-0.5, -4.0, 3.0, 21.0], [0.0, 0.0, -1.75, 0.25]])


def test_matmul_against_byte_loop():
    rng = np.random.default_rng(0)
    rows, cols, g = 5, 256, 128
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = W.bf16_bits_from_f32(rng.uniform(-0.02, 0.02, size=(rows, cols // g)).astype(np.float32))
    x = rng.standard_normal((3, cols))
    ours = x @ O.dequant_int4(codes, scales, g).T
    ref = np.zeros((3, rows))
    for r in range(rows):
        for c in range(cols):
            byte = int(codes[r, c // 2])
            nib = (byte >> (4 * (c % 2))) & 0xF
            q = nib - 16 if nib & 0x8 else nib
            s = struct.unpack("<f", struct.pack("<I", int(scales[r, c // g]) << 16))[0]
            ref[:, r] += s * q * x[:, c]
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def _pack_int4(q: np.ndarray) -> np.ndarray:
    u = (q & 15).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def _w4_and_bf16_twin(seed, scale_of):
    """A 4-bit weight dict and the bf16 dict with weights bf16(scale * code)."""
    rng = np.random.default_rng(seed)
    base = W.make_weights(SMALL, seed=seed, gains="random")
    w4 = {k: v for k, v in base.items() if k.split(".")[-1] not in W.INT4_LINEARS}
    wb = dict(w4)
    for l in range(SMALL.n_layers):
        for name in W.INT4_LINEARS:
            key = f"layers.{l}.{name}"
            rows, cols = base[key].shape
            q = rng.integers(-8, 8, size=(rows, cols))
            s = scale_of(rng, rows, cols // 128)
            w4[key + ".codes"] = _pack_int4(q)
            w4[key + ".scales"] = W.bf16_bits_from_f32(s)
            wf = np.repeat(s.astype(np.float64), 128, axis=1) * q
            wb[key] = W.bf16_bits_from_f32(wf.astype(np.float32))
    return w4, wb


def _logits(w, toks):
    m = O.OracleModel(SMALL, w)
    c = m.new_cache()
    m.forward(c, toks[:13], O.CAUSAL)
    c.n = 13
    return m.forward(c, toks[13:], O.BIDIR)


def test_power_of_two_scales_reduce_to_bf16_model():
    pow2 = lambda rng, r, g: np.ldexp(1.0, rng.integers(-9, -5, size=(r, g))).astype(np.float32)
    w4, wb = _w4_and_bf16_twin(1, pow2)
    toks = W.prompt_ids(SMALL, 21, seed=1)
    np.testing.assert_array_equal(_logits(w4, toks), _logits(wb, toks))


def test_dequantization_is_not_rounded_to_bf16():
    general = lambda rng, r, g: rng.uniform(0.0064, 0.01, size=(r, g)).astype(np.float32)
    w4, wb = _w4_and_bf16_twin(2, general)
    toks = W.prompt_ids(SMALL, 21, seed=2)
    a, b = _logits(w4, toks), _logits(wb, toks)
    assert np.abs(a - b).max() > 1e-4 * np.abs(a).max()


def test_generator_w4():
    a = W.make_w4_weights(SMALL, seed=4, threads=1)
    b = W.make_w4_weights(SMALL, seed=4, threads=8)
    assert set(a) == set(b)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    full = W.make_weights(SMALL, seed=4)
    np.testing.assert_array_equal(a["lm_head"], full["lm_head"])
    np.testing.assert_array_equal(a["embed"], full["embed"])
    assert "layers.0.w_qkv" not in a
    codes, scales = a["layers.1.w_down.codes"], a["layers.1.w_down.scales"]
    assert codes.shape == (SMALL.d_model, SMALL.ffn_dim // 2) and scales.shape == (SMALL.d_model, SMALL.ffn_dim // 128)
    q = O.int4_codes(codes)
    assert q.min() == -8 and q.max() == 7
    s = O.decode_bf16_bits(scales)
    assert s.min() >= 0.0064 * 0.99 and s.max() <= 0.01 * 1.01
    w = O.dequant_int4(codes, scales)
    assert abs(w.std() - 0.02) < 2e-3 and abs(w.mean()) < 1e-3
    c = W.make_w4_weights(SMALL, seed=5)
    assert not np.array_equal(c["layers.1.w_down.codes"], codes)
    with pytest.raises(ValueError):
        W.make_w4_weights(W.SHAPES["tiny"])
