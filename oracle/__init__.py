"""CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow NumPy (float64) implementation of the block-wise decoding
forward and its three modes.  Only ``tests/``, the package's ``smoke()`` check
and the benchmark's CPU-baseline leg may import it; the HIP product path never
does, and the two share no code (the only common module is ``workloads``,
which holds seeded input draws and no arithmetic of the method).

Parity pins: every function here is checked by the ``-m "not gpu"`` tests
against closed forms, library special cases, brute force and the pages'
temperature-0 invariant.  The diffusion trajectory beyond the per-step
selection rule has no independent pin ("parity unpinned": the pages print no
worked example); the per-step rule itself is pinned.  Quadratic
self-speculation is a reading (the pages name it without an algorithm); its
arithmetic is pinned against separate forwards and the greedy-AR identity.
"""
from .model import (BIDIR, CAUSAL, INT4_GROUP, KVCache, OracleModel, apply_rope, attention, attention_masked,
                    bf16_pair_round,
                    bf16_round, decode_bf16_bits, dequant_int4, int4_codes, rms_normalize, rope_tables, select_rows,
                    silu, visible)
from .modes import (GenResult, OracleSession, RowSel, accept_length, generate_ar, generate_ar_sample,
                    generate_diffusion, generate_diffusion_batch, generate_selfspec, generate_selfspec_quadratic,
                    generate_selfspec_sample,
                    revise_rule, unmask_rule)
from . import sampling
