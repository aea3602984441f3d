"""GPU parity of the kvarn_k4v4_g128 preset (4-bit keys per channel, 4-bit values per token):
a wider-value member of the kvarn_k<K>v<V>_g<G> family, whose released member the README's
preset paragraph (after the four stages) presents as one choice of key and value widths. The
quantizer against the oracle with 4-bit values, the 4-bit value record read back by the
oracle's unpacker, decode, appends, chunk write and multi-query read through the C ABI."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_tile_amd import synth
from oracle import kvarn_oracle as O
from tests import kvarn_testlib as T
from tests.test_gpu_parity import _build_cache

pytestmark = pytest.mark.gpu

PRESET = "kvarn_k4v4_g128"


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("n_iters", [0, 1, 8])
def test_v4_quantize_against_oracle(K, n_iters):
    n, hkv = 12, 3
    tiles, kinds = synth.tile_batch(n * hkv, "cpu", seed=200 + n_iters, return_kinds=True)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    tok = torch.arange(n, dtype=torch.int64) * 128
    page = torch.randperm(n, generator=torch.Generator().manual_seed(201)).to(torch.int32)
    params = K.params_from_dtype(PRESET, n_iters)
    kp = K.new_pool(n, hkv, O.KIND_K, params=params)
    vp = K.new_pool(n, hkv, O.KIND_V, params=params)
    assert vp.shape[2] == O.V4_RECORD_BYTES and kp.shape[2] == O.K_RECORD_BYTES
    K.quantize_kv_tiles(params, src.cuda(), src.cuda(), tok.cuda(), page.cuda(), kp, vp)
    torch.cuda.synchronize()
    x16 = tiles.view(n, hkv, 128, 128).numpy()
    for kind, pool in ((O.KIND_K, kp), (O.KIND_V, vp)):
        st = T.QuantStats()
        for h in range(hkv):
            recs = T.records_of(pool, page.tolist(), h)
            T.check_quantized_tiles(x16[:, h], recs, kind, n_iters, st,
                                    k_bits=4, v_bits=4)
        say(f"k4v4 N={n_iters} kind={kind}: {st}")
        T.assert_rate(st)


def test_v4_single_kind_equals_pair(K):
    """kvarn_quantize_tiles of the values alone writes the same records as the K+V launch."""
    n, hkv = 5, 2
    tiles = synth.tile_batch(n * hkv, "cpu", seed=210)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous().cuda()
    tok = (torch.arange(n, dtype=torch.int64) * 128).cuda()
    page = torch.arange(n, dtype=torch.int32).cuda()
    params = K.params_from_dtype(PRESET, 8)
    kp = K.new_pool(n, hkv, O.KIND_K, params=params)
    vp = K.new_pool(n, hkv, O.KIND_V, params=params)
    vp1 = K.new_pool(n, hkv, O.KIND_V, params=params)
    K.quantize_kv_tiles(params, src, src, tok, page, kp, vp)
    K.quantize_tiles(params, O.KIND_V, src, tok, page, vp1)
    torch.cuda.synchronize()
    assert torch.equal(vp, vp1)


def test_v4_dequantize_tiles(K):
    n, hkv = 6, 2
    tiles = synth.tile_batch(n * hkv, "cpu", seed=220)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    params = K.params_from_dtype(PRESET, 8)
    vp = K.new_pool(n, hkv, O.KIND_V, params=params)
    K.quantize_tiles(params, O.KIND_V, src.cuda(), (torch.arange(n, dtype=torch.int64) * 128).cuda(),
                     torch.arange(n, dtype=torch.int32).cuda(), vp)
    out = K.dequantize_tiles(params, O.KIND_V, vp, torch.arange(n, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for h in range(hkv):
        for i, rec in enumerate(T.records_of(vp, range(n), h)):
            d = O.unpack_v4_record(rec)
            ref = O.dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], O.KIND_V).T
            ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(got[i, h] - ref) <= 0.5 * ulp + 1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("G,hkv", [(8, 2), (1, 4)])
def test_v4_decode_ragged(K, G, hkv):
    lens = [0, 1, 127, 128, 129, 300, 1000, 1024 + 77]
    params = K.params_from_dtype(PRESET, 8)
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=230 + G)
    assert vp.shape[2] == O.V4_RECORD_BYTES
    q = torch.randn((len(lens), G * hkv, 128), generator=torch.Generator().manual_seed(231)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
    say(f"k4v4 decode G={G}: max rel err {err:.3e}")


def test_v4_decode_long(K):
    """One long sequence (several splits, every wave several pages) and a short one."""
    lens = [64 * 128 + 50, 3 * 128]
    hkv, G = 2, 8
    params = K.params_from_dtype(PRESET, 8)
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=240)
    q = torch.randn((len(lens), G * hkv, 128), generator=torch.Generator().manual_seed(241)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
    say(f"k4v4 decode, {lens}: max rel err {err:.3e}")


def test_v4_write_appends_and_chunk_attention(K):
    from tests.test_gpu_chunk import _reference_rows
    from tests.test_gpu_write import _chunk, _extend_block_table
    lens, lens_new = [5, 200, 0], [300, 56, 260]
    hkv, G = 2, 8
    params = K.params_from_dtype(PRESET, 8)
    kp, vp, bt, kt, vt, sl, free = _build_cache(K, params, lens, hkv, seed=250, spare=4,
                                                width=max((L + n) // 128 for L, n in zip(lens, lens_new)) + 2)
    bt = _extend_block_table(bt, lens, lens_new, free)
    kn, vn, cu = _chunk(lens_new, hkv, seed=251)
    # the same tokens one append at a time, into copies
    kpb, vpb, ktb, vtb = kp.clone(), vp.clone(), kt.clone(), vt.clone()
    cu_h = cu.cpu().numpy()
    last = kn.shape[0] - 1
    for i in range(max(lens_new)):
        sl_i = torch.tensor([L + i if i < n else -1 for L, n in zip(lens, lens_new)],
                            dtype=torch.int32, device="cuda")
        rows = torch.tensor([min(int(cu_h[b]) + min(i, max(n - 1, 0)), last)
                             for b, n in enumerate(lens_new)], dtype=torch.long, device="cuda")
        K.append_tokens(params, kn[rows].contiguous(), vn[rows].contiguous(), sl_i, ktb, vtb, bt,
                        kpb, vpb)
    vt0 = vt.clone()
    K.write_tokens(params, kn, vn, cu, sl, kt, vt, bt, kp, vp)
    torch.cuda.synchronize()
    assert torch.equal(kp, kpb) and torch.equal(vp, vpb), "chunk write and appends differ"
    # completed value pages equal kvarn_quantize_tiles of the same tokens
    bt_h = bt.cpu().numpy()
    for b, (L, n) in enumerate(zip(lens, lens_new)):
        for t in range(L // 128, (L + n) // 128):
            tile = torch.stack([vt0[b, :, a - 128 * t] if a < L else vn[int(cu_h[b]) + a - L]
                                for a in range(128 * t, 128 * t + 128)])
            ref = K.new_pool(1, hkv, O.KIND_V, params=params)
            K.quantize_tiles(params, O.KIND_V, tile.contiguous(),
                             torch.zeros(1, dtype=torch.int64, device="cuda"),
                             torch.zeros(1, dtype=torch.int32, device="cuda"), ref)
            torch.cuda.synchronize()
            assert torch.equal(vp[int(bt_h[b, t])], ref[0]), (b, t)
    sl2 = sl + torch.tensor(lens_new, dtype=torch.int32, device="cuda")
    total_q = sum(lens_new)
    q = torch.randn((total_q, hkv * G, 128), generator=torch.Generator().manual_seed(252)).to(torch.float16).cuda()
    out = K.chunk_attention(params, q, cu, kp, vp, bt, sl2, int(sl2.max().item()), kt, vt)
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(253).choice(total_q, 24, replace=False).tolist()) | {0, total_q - 1})
    ref = _reference_rows(q, cu, kp, vp, bt, kt, vt, sl2, G, rows)
    o = out.cpu().numpy().astype(np.float64)
    worst = max(T.assert_rows_close(o[r, hq], want, f"row {r} head {hq}") for (r, hq), want in ref.items())
    say(f"k4v4 write + appends + chunk attention: {len(rows)} rows, max rel err {worst:.2e}")
