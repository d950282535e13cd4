"""The allocation-free attention entry point (sdm_attention_noalloc, partials
in the library's per-device scratch array) gives, bit for bit, what the
workspace entry point (sdm_attention) gives on the same inputs: two calls in a
row, the second on a smaller input, each against its own workspace call; a
request beyond the scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

HQ, HKV, HD = 32, 8, 128
DEV = "cuda"


def _inputs(lib, L, P, T, seed):
    q, k, v = W.attention_op_inputs(P, T, HQ, HKV, HD, seed=seed)
    nkeys = P + T
    n_pages = (nkeys + 63) // 64
    pages = torch.as_tensor(np.random.default_rng(seed).permutation(n_pages + 3)[:n_pages].astype(np.int32),
                            device=DEV)
    pool = torch.zeros(lib.sdm_attn_pool_bytes(HKV, HD, n_pages + 3), dtype=torch.uint8, device=DEV)
    tq, tk, tv = (torch.from_numpy(a.view(np.int16)).to(DEV) for a in (q, k, v))
    st = torch.cuda.current_stream().cuda_stream
    L.check(lib.sdm_attn_pack_kv(HKV, HD, tk.data_ptr(), tv.data_ptr(), nkeys, pages.data_ptr(), pool.data_ptr(), st))
    return tq, pool, pages


def test_noalloc_attention_equals_workspace_entry():
    from self_speculative_amd import _lib as L
    lib = L.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert lib.sdm_attention_scratch_max_bytes() == 16 << 20
    # the second call is smaller: fewer keys, fewer rows, the other mask
    for P, T, mode in ((7000, 32, L.SDM_BIDIR), (1500, 9, L.SDM_CAUSAL)):
        tq, pool, pages = _inputs(lib, L, P, T, seed=P)
        wsb = lib.sdm_attn_workspace_bytes(HQ, HKV, HD, T, P + T)
        assert wsb <= lib.sdm_attention_scratch_max_bytes()
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        ref = torch.empty((T, HQ, HD), dtype=torch.int16, device=DEV)
        out = torch.full((T, HQ, HD), -1, dtype=torch.int16, device=DEV)
        L.check(lib.sdm_attention(HQ, HKV, HD, tq.data_ptr(), pool.data_ptr(), pages.data_ptr(), P, T, mode,
                                  ref.data_ptr(), ws.data_ptr(), wsb, st))
        L.check(lib.sdm_attention_noalloc(HQ, HKV, HD, tq.data_ptr(), pool.data_ptr(), pages.data_ptr(), P, T, mode,
                                          out.data_ptr(), st))
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (P, T, mode)


def test_noalloc_attention_rejects_oversized_request():
    from self_speculative_amd import _lib as L
    lib = L.lib()
    st = torch.cuda.current_stream().cuda_stream
    P, T = 8000, 32                                    # 32 splits: partials above 16 MiB
    assert lib.sdm_attn_workspace_bytes(HQ, HKV, HD, T, P + T) > lib.sdm_attention_scratch_max_bytes()
    tq, pool, pages = _inputs(lib, L, P, T, seed=3)
    out = torch.full((T, HQ, HD), -1, dtype=torch.int16, device=DEV)
    with pytest.raises(L.SdmError) as e:
        L.check(lib.sdm_attention_noalloc(HQ, HKV, HD, tq.data_ptr(), pool.data_ptr(), pages.data_ptr(), P, T,
                                          L.SDM_BIDIR, out.data_ptr(), st))
    assert e.value.status == L.SDM_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((out == -1).all())                     # nothing ran
