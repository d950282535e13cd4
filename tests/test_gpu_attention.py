"""GPU parity of the standalone block attention op (bf16, 32 q heads / 8 KV
heads, head_dim 128, 32 block rows over a paged prefix) against the oracle's
float64 attention on the same bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

HQ, HKV, HD = 32, 8, 128


def run_gpu(q, k, v, n, T, mode, page_perm_seed=None, hq=HQ, hkv=HKV):
    from self_speculative_amd import _lib as L
    lib = L.lib()
    dev = "cuda"
    nkeys = n + T
    n_pages = (nkeys + 63) // 64
    pages = np.arange(n_pages, dtype=np.int32)
    pool_pages = n_pages
    if page_perm_seed is not None:
        pool_pages = n_pages + 7
        pages = np.random.default_rng(page_perm_seed).permutation(pool_pages)[:n_pages].astype(np.int32)
    pool = torch.zeros(lib.sdm_attn_pool_bytes(hkv, HD, pool_pages), dtype=torch.uint8, device=dev)
    dpages = torch.as_tensor(pages, device=dev)
    tq = torch.from_numpy(q.view(np.int16)).to(dev)
    tk = torch.from_numpy(k.view(np.int16)).to(dev)
    tv = torch.from_numpy(v.view(np.int16)).to(dev)
    st = torch.cuda.current_stream().cuda_stream
    L.check(lib.sdm_attn_pack_kv(hkv, HD, tk.data_ptr(), tv.data_ptr(), nkeys, dpages.data_ptr(), pool.data_ptr(), st))
    wsb = lib.sdm_attn_workspace_bytes(hq, hkv, HD, T, nkeys)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((T, hq, HD), dtype=torch.int16, device=dev)
    L.check(lib.sdm_attention(hq, hkv, HD, tq.data_ptr(), pool.data_ptr(), dpages.data_ptr(), n, T, mode,
                              out.data_ptr(), ws.data_ptr(), wsb, st))
    torch.cuda.synchronize()
    return O.decode_bf16_bits(out.cpu().numpy().view(np.uint16))


def oracle_attn(q, k, v, n, mode):
    return O.attention(O.decode_bf16_bits(q), O.decode_bf16_bits(k), O.decode_bf16_bits(v), n, mode)


def check_close(gpu, ref):
    err = np.abs(gpu - ref)
    scale = np.abs(ref).max()
    assert err.max() <= 2e-2 and err.max() <= 1e-2 * scale, (err.max(), scale)
    # the GPU stores o in bf16: every element within one bf16 spacing of the
    # oracle, plus the fp32 accumulation error of P.V with P kept to ~2^-16
    # (absolute, visible where a row with few keys cancels to near zero)
    assert np.all(err <= np.abs(ref) * 2.0 ** -7 + 1e-4), err.max()


@pytest.mark.parametrize("P", [512, 4096, 32768])
@pytest.mark.parametrize("mode", [O.BIDIR, O.CAUSAL])
def test_attention_op_prefix_lengths(P, mode):
    print(f"attention op P={P} mode={mode}", flush=True)
    q, k, v = W.attention_op_inputs(P, 32, HQ, HKV, HD, seed=0)
    check_close(run_gpu(q, k, v, P, 32, mode), oracle_attn(q, k, v, P, mode))


@pytest.mark.parametrize("P,T", [(0, 32), (0, 1), (1000, 32), (1000, 7), (63, 1), (64, 32), (95, 32), (3000, 1)])
@pytest.mark.parametrize("mode", [O.BIDIR, O.CAUSAL])
def test_attention_op_edges(P, T, mode):
    print(f"attention op edge P={P} T={T} mode={mode}", flush=True)
    q, k, v = W.attention_op_inputs(P, T, HQ, HKV, HD, seed=1)
    check_close(run_gpu(q, k, v, P, T, mode), oracle_attn(q, k, v, P, mode))


@pytest.mark.parametrize("hq,hkv", [(24, 8), (40, 8), (4, 4)])
def test_attention_op_group_sizes(hq, hkv):
    print(f"attention op heads {hq}/{hkv}", flush=True)
    q, k, v = W.attention_op_inputs(700, 32, hq, hkv, HD, seed=2)
    for mode in (O.BIDIR, O.CAUSAL):
        check_close(run_gpu(q, k, v, 700, 32, mode, hq=hq, hkv=hkv), oracle_attn(q, k, v, 700, mode))


def test_attention_op_shuffled_pages_bit_identical():
    print("attention op shuffled page table", flush=True)
    q, k, v = W.attention_op_inputs(1500, 32, HQ, HKV, HD, seed=3)
    a = run_gpu(q, k, v, 1500, 32, O.CAUSAL)
    b = run_gpu(q, k, v, 1500, 32, O.CAUSAL, page_perm_seed=11)
    np.testing.assert_array_equal(a, b)


def test_attention_op_row_independence():
    """The last block row sees the same keys in both masks -> identical bits;
    a causal row equals the same row computed as a one-row block."""
    print("attention op row independence", flush=True)
    P = 2000
    q, k, v = W.attention_op_inputs(P, 32, HQ, HKV, HD, seed=4)
    bi = run_gpu(q, k, v, P, 32, O.BIDIR)
    ca = run_gpu(q, k, v, P, 32, O.CAUSAL)
    np.testing.assert_array_equal(bi[31], ca[31])
    for i in (0, 5, 31):
        one = run_gpu(q[i:i + 1], k[: P + i + 1], v[: P + i + 1], P + i, 1, O.CAUSAL)
        np.testing.assert_array_equal(one[0], ca[i])


def test_attention_op_staged_with_remainder_tile():
    """40 q / 8 KV heads (five query tiles per KV head) over a prefix long
    enough for the staged shape: four tiles a group run over the staged
    pages and the fifth is folded in page by page (each wave one page
    state, merged in LDS).  Parity with the oracle, and the fifth tile's
    rows bit-equal to the same rows computed as one-row blocks (where all
    five heads share one staged tile)."""
    P = 8300
    print(f"attention op heads 40/8, P={P} (staged + remainder tile)", flush=True)
    q, k, v = W.attention_op_inputs(P, 32, 40, 8, HD, seed=5)
    ca = run_gpu(q, k, v, P, 32, O.CAUSAL, hq=40, hkv=8)
    check_close(ca, oracle_attn(q, k, v, P, O.CAUSAL))
    check_close(run_gpu(q, k, v, P, 32, O.BIDIR, hq=40, hkv=8), oracle_attn(q, k, v, P, O.BIDIR))
    for i in (0, 17, 31):
        one = run_gpu(q[i:i + 1], k[: P + i + 1], v[: P + i + 1], P + i, 1, O.CAUSAL, hq=40, hkv=8)
        np.testing.assert_array_equal(one[0], ca[i])
