"""The C-ABI library loads on a machine without a GPU, exports every call the
header declares, and validates configurations before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")


@pytest.fixture(scope="module")
def lib():
    from self_speculative_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        from self_speculative_amd.build import build
        build()
    return L.lib()


def declared_calls():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_calls()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    from self_speculative_amd._lib import SIGNATURES
    assert set(SIGNATURES) == set(names)


def _cfg(**kw):
    import workloads as W
    from self_speculative_amd.model import make_config
    c = make_config(W.SHAPES["8b"], max_seqs=1, max_block=32, max_context=4096, max_rows=32)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_config_validation(lib):
    from self_speculative_amd import _lib as L
    good = _cfg()
    ws = lib.sdm_workspace_bytes(ctypes.byref(good))
    assert ws > 0
    # one KV page of the 8B shape: 36 layers x (K, V) x 8 heads x 64 positions x 128 dims x 2 bytes
    assert lib.sdm_kv_page_bytes(ctypes.byref(good)) == 36 * 2 * 8 * 64 * 128 * 2
    assert lib.sdm_packed_bytes(ctypes.byref(good), 4096, 4096) == 4096 * 4096 * 2
    for bad in (dict(head_dim=64), dict(n_q_heads=30), dict(page_tokens=32), dict(mask_id=151936),
                dict(dtype=7), dict(max_block=64), dict(vocab=151935)):
        c = _cfg(**bad)
        assert lib.sdm_workspace_bytes(ctypes.byref(c)) == 0, bad
        assert lib.sdm_last_error().decode()


def test_calls_reject_bad_arguments_without_a_device(lib):
    from self_speculative_amd import _lib as L
    c = _cfg()
    # argument checks run before any HIP call
    assert lib.sdm_pack_matrix(ctypes.byref(c), 9, 1, None, 1, 32, 32, None) == L.SDM_ERR_ARG
    assert lib.sdm_pack_matrix(ctypes.byref(c), 0, None, None, 1, 32, 32, None) == L.SDM_ERR_ARG
    assert lib.sdm_pack_matrix(ctypes.byref(c), 0, 1, None, 1, 31, 32, None) == L.SDM_ERR_UNSUPPORTED
    out = ctypes.c_void_p()
    assert lib.sdm_init_model(ctypes.byref(c), None, None, 1, None, 0, None, ctypes.byref(out)) == L.SDM_ERR_ARG
    assert lib.sdm_prefill(None, 0, None, 1, None, None) == L.SDM_ERR_ARG
    assert lib.sdm_commit_kv(None, 0, 1) == L.SDM_ERR_ARG
    assert lib.sdm_attention(32, 8, 64, 1, 1, 1, 0, 1, 0, 1, 1, 1 << 20, None) == L.SDM_ERR_UNSUPPORTED
    assert lib.sdm_attn_workspace_bytes(32, 8, 128, 32, 4128) > 0
    assert lib.sdm_attn_pool_bytes(8, 128, 10) == 10 * 2 * 8 * 64 * 128 * 2


def test_int4_weight_format_config_and_sizes(lib):
    from self_speculative_amd import _lib as L
    c = _cfg(weight_format=L.SDM_WEIGHTS_INT4)
    assert lib.sdm_workspace_bytes(ctypes.byref(c)) > 0
    # codes: 4096 x 4096 / 2 bytes; scales: 4096 rows x 32 groups x 2 bytes
    assert lib.sdm_packed_bytes_int4(ctypes.byref(c), 4096, 4096) == 4096 * 2048 + 4096 * 32 * 2
    # 6144 x 4096 QKV, 2 x 12288 gate/up rows
    assert lib.sdm_packed_bytes_int4(ctypes.byref(c), 6144, 4096) == 6144 * 2048 + 6144 * 32 * 2
    assert lib.sdm_packed_bytes_int4(ctypes.byref(c), 24576, 4096) == 24576 * 2048 + 24576 * 32 * 2
    assert lib.sdm_packed_bytes_int4(ctypes.byref(c), 4096, 4000) == 0
    assert lib.sdm_packed_bytes_int4(ctypes.byref(c), 4016, 4096) == 0
    for bad in (dict(weight_format=2), dict(weight_format=L.SDM_WEIGHTS_INT4, dtype=L.SDM_F32, head_dim=64),
                dict(weight_format=L.SDM_WEIGHTS_INT4, d_model=4096 + 32)):
        b = _cfg(**bad)
        assert lib.sdm_workspace_bytes(ctypes.byref(b)) == 0, bad
        assert lib.sdm_last_error().decode()
    # packing arguments are checked before any HIP call
    pk = lib.sdm_pack_matrix_int4
    assert pk(ctypes.byref(c), 9, 4, 4, None, None, 4, 32, 128, None) == L.SDM_ERR_ARG
    assert pk(ctypes.byref(c), 0, None, 4, None, None, 4, 32, 128, None) == L.SDM_ERR_ARG
    assert pk(ctypes.byref(c), 2, 4, 4, None, 4, 4, 32, 128, None) == L.SDM_ERR_ARG
    assert pk(ctypes.byref(c), 0, 4, 4, None, None, 4, 32, 100, None) == L.SDM_ERR_UNSUPPORTED
    assert pk(ctypes.byref(c), 0, 4, 4, None, None, 4, 31, 128, None) == L.SDM_ERR_UNSUPPORTED
    assert pk(ctypes.byref(c), 0, 6, 4, None, None, 4, 32, 128, None) == L.SDM_ERR_ARG
    f32 = _cfg(dtype=L.SDM_F32, head_dim=64, n_q_heads=32, n_kv_heads=8)
    assert pk(ctypes.byref(f32), 0, 4, 4, None, None, 4, 32, 128, None) == L.SDM_ERR_UNSUPPORTED


def test_product_path_does_not_import_the_oracle():
    """The package's sources never reference the oracle (it is test-only)."""
    pkg = os.path.join(ROOT, "self_speculative_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f
