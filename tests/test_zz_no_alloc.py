"""The decode entry point that allocates nothing (kvarn_decode_attention_noalloc, fixed device
scratch) against kvarn_decode_attention with a caller workspace, through the C ABI: two calls
in a row on one GPU, the second with a smaller input, so the second reads a scratch that
still holds the first call's partials."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_tile_amd import synth
from tests import kvarn_testlib as T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def _cache(K, params, seed, lens, hq, hkv):
    """A paged cache of the given prompt lengths (permuted pages), its staging tiles filled
    with the tokens past the last full page, and one query per sequence."""
    w = synth.batched_paged(device="cpu", seed=seed, lens=list(lens), steps=1)
    dev = torch.device("cuda:0")
    # keep hkv heads of the generated 8
    k_src = w.k_src[:, :hkv].contiguous().to(dev)
    v_src = w.v_src[:, :hkv].contiguous().to(dev)
    kp = K.new_pool(w.num_pages, hkv, K.KIND_K, params=params)
    vp = K.new_pool(w.num_pages, hkv, K.KIND_V, params=params)
    K.quantize_kv_tiles(params, k_src, v_src, w.tile_src_token.to(dev), w.tile_dst_page.to(dev),
                        kp, vp)
    B = len(lens)
    kt = torch.zeros((B, hkv, 128, 128), dtype=torch.float16, device=dev)
    vt = torch.zeros_like(kt)
    g = torch.Generator().manual_seed(seed)
    for b, L in enumerate(lens):
        n = L % 128
        if n:
            kt[b, :, :n] = torch.randn((hkv, n, 128), generator=g).to(torch.float16).to(dev)
            vt[b, :, :n] = torch.randn((hkv, n, 128), generator=g).to(torch.float16).to(dev)
    q = torch.randn((B, hq, 128), generator=g).to(torch.float16).to(dev)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    return q, kp, vp, w.block_table.to(dev), seq_lens, kt, vt


def _check_pair(K, params, q, kp, vp, bt, seq_lens, kt, vt, max_len, G, what):
    ref = K.decode_attention(params, q, kp, vp, bt, seq_lens, max_len, k_tail=kt, v_tail=vt)
    out = torch.full_like(q, float("nan"))
    got = K.decode_attention_noalloc(params, q, kp, vp, bt, seq_lens, max_len, k_tail=kt,
                                     v_tail=vt, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    diff = (got.float() - ref.float()).abs().max().item()
    print(f"{what}: max |noalloc - workspace| = {diff:.3e}", flush=True)
    # same kernels, same grid: the outputs agree bit for bit
    assert torch.equal(got, ref), what
    # and both meet the attention bar against the oracle on a few rows
    rows = [(0, 0), (q.shape[0] - 1, kp.shape[1] - 1)]
    err = T.check_decode(q, got, kp, vp, bt, seq_lens, G, rows=rows, k_tail=kt, v_tail=vt)
    print(f"{what}: oracle rows max rel err {err:.2e}", flush=True)


def test_noalloc_two_calls_second_smaller(K):
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    cap = K.decode_noalloc_max_workspace_bytes()
    # call 1: 6 ragged sequences (balanced layout, partials in most of the scratch it uses)
    lens1 = [4096 + 37, 1000, 128, 8192, 3000 + 127, 257]
    hq, hkv = 32, 4
    need1 = K.decode_workspace_bytes(params, len(lens1), hq, hkv, max(lens1))
    assert 0 < need1 <= cap
    print(f"call 1: {len(lens1)} sequences, workspace {need1} B of {cap}", flush=True)
    c1 = _cache(K, params, 21, lens1, hq, hkv)
    _check_pair(K, params, *c1, max(lens1), hq // hkv, "call 1")
    # call 2: one shorter sequence (split layout, fewer bytes): the scratch still holds call
    # 1's partials
    lens2 = [2048 + 5]
    hq2, hkv2 = 16, 2
    need2 = K.decode_workspace_bytes(params, 1, hq2, hkv2, lens2[0])
    assert need2 < need1
    print(f"call 2: 1 sequence, workspace {need2} B", flush=True)
    c2 = _cache(K, params, 22, lens2, hq2, hkv2)
    _check_pair(K, params, *c2, lens2[0], hq2 // hkv2, "call 2")
