"""GPU parity of the kvarn_k2v2_g128 preset (2-bit keys per channel, 2-bit values per token;
the pages give 2-bit results, README intro and the hypho page's "core finding"): the quantizer
against the oracle with 2-bit keys, the 2-bit key record read back by the oracle's unpacker,
decode, chunk write and multi-query read through the C ABI."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_tile_amd import synth
from oracle import kvarn_oracle as O
from tests import kvarn_testlib as T
from tests.test_gpu_parity import _build_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("n_iters", [0, 1, 8])
def test_k2_quantize_against_oracle(K, n_iters):
    n, hkv = 12, 3
    tiles, kinds = synth.tile_batch(n * hkv, "cpu", seed=60 + n_iters, return_kinds=True)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    tok = torch.arange(n, dtype=torch.int64) * 128
    page = torch.randperm(n, generator=torch.Generator().manual_seed(61)).to(torch.int32)
    params = K.params_from_dtype("kvarn_k2v2_g128", n_iters)
    kp = K.new_pool(n, hkv, O.KIND_K, params=params)
    vp = K.new_pool(n, hkv, O.KIND_V, params=params)
    assert kp.shape[2] == O.K2_RECORD_BYTES
    K.quantize_kv_tiles(params, src.cuda(), src.cuda(), tok.cuda(), page.cuda(), kp, vp)
    torch.cuda.synchronize()
    x16 = tiles.view(n, hkv, 128, 128).numpy()
    for kind, pool in ((O.KIND_K, kp), (O.KIND_V, vp)):
        st = T.QuantStats()
        for h in range(hkv):
            recs = T.records_of(pool, page.tolist(), h)
            T.check_quantized_tiles(x16[:, h], recs, kind, n_iters, st,
                                    k_bits=2)
        say(f"k2v2 N={n_iters} kind={kind}: {st}")
        T.assert_rate(st)


def test_k2_dequantize_tiles(K):
    n, hkv = 6, 2
    tiles = synth.tile_batch(n * hkv, "cpu", seed=70)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    params = K.params_from_dtype("kvarn_k2v2_g128", 8)
    kp = K.new_pool(n, hkv, O.KIND_K, params=params)
    K.quantize_tiles(params, O.KIND_K, src.cuda(), (torch.arange(n, dtype=torch.int64) * 128).cuda(),
                     torch.arange(n, dtype=torch.int32).cuda(), kp)
    out = K.dequantize_tiles(params, O.KIND_K, kp, torch.arange(n, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for h in range(hkv):
        for i, rec in enumerate(T.records_of(kp, range(n), h)):
            d = O.unpack_k2_record(rec)
            ref = O.dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], O.KIND_K).T
            ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(got[i, h] - ref) <= 0.5 * ulp + 1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("G,hkv", [(8, 2), (1, 4)])
def test_k2_decode_ragged(K, G, hkv):
    lens = [0, 1, 127, 128, 129, 300, 1000, 1024 + 77]
    params = K.params_from_dtype("kvarn_k2v2_g128", 8)
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=80 + G)
    assert kp.shape[2] == O.K2_RECORD_BYTES
    q = torch.randn((len(lens), G * hkv, 128), generator=torch.Generator().manual_seed(81)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
    say(f"k2v2 decode G={G}: max rel err {err:.3e}")


def test_k2_write_and_chunk_attention(K):
    from tests.test_gpu_chunk import _reference_rows
    from tests.test_gpu_write import _chunk, _extend_block_table
    lens, lens_new = [5, 200, 0], [300, 56, 260]
    hkv, G = 2, 8
    params = K.params_from_dtype("kvarn_k2v2_g128", 8)
    kp, vp, bt, kt, vt, sl, free = _build_cache(K, params, lens, hkv, seed=90, spare=4,
                                                width=max((L + n) // 128 for L, n in zip(lens, lens_new)) + 2)
    bt = _extend_block_table(bt, lens, lens_new, free)
    kn, vn, cu = _chunk(lens_new, hkv, seed=91)
    kt0 = kt.clone()
    K.write_tokens(params, kn, vn, cu, sl, kt, vt, bt, kp, vp)
    torch.cuda.synchronize()
    # completed pages equal kvarn_quantize_tiles of the same tokens
    cu_h, bt_h = cu.cpu().numpy(), bt.cpu().numpy()
    for b, (L, n) in enumerate(zip(lens, lens_new)):
        for t in range(L // 128, (L + n) // 128):
            tile = torch.stack([kt0[b, :, a - 128 * t] if a < L else kn[int(cu_h[b]) + a - L]
                                for a in range(128 * t, 128 * t + 128)])
            ref = K.new_pool(1, hkv, O.KIND_K, params=params)
            K.quantize_tiles(params, O.KIND_K, tile.contiguous(),
                             torch.zeros(1, dtype=torch.int64, device="cuda"),
                             torch.zeros(1, dtype=torch.int32, device="cuda"), ref)
            torch.cuda.synchronize()
            assert torch.equal(kp[int(bt_h[b, t])], ref[0]), (b, t)
    sl2 = sl + torch.tensor(lens_new, dtype=torch.int32, device="cuda")
    total_q = sum(lens_new)
    q = torch.randn((total_q, hkv * G, 128), generator=torch.Generator().manual_seed(92)).to(torch.float16).cuda()
    out = K.chunk_attention(params, q, cu, kp, vp, bt, sl2, int(sl2.max().item()), kt, vt)
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(93).choice(total_q, 24, replace=False).tolist()) | {0, total_q - 1})
    ref = _reference_rows(q, cu, kp, vp, bt, kt, vt, sl2, G, rows)
    o = out.cpu().numpy().astype(np.float64)
    worst = max(T.assert_rows_close(o[r, hq], want, f"row {r} head {hq}") for (r, hq), want in ref.items())
    say(f"k2v2 write + chunk attention: {len(rows)} rows, max rel err {worst:.2e}")
