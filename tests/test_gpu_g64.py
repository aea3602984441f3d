"""GPU parity of group size 64 (presets kvarn_k*v*_g64: keys in two 64-token groups per
channel, values in two 64-channel groups per token, each with its own scale and zero) for
every preset and both record formats: the quantizer against the oracle's group-64 quantizer,
the records read back by the oracle's unpacker, dequantize, decode (split and balanced
layouts), appends, chunk write and multi-query read through the C ABI."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_tile_amd import synth
from oracle import kvarn_oracle as O
from tests import kvarn_testlib as T
from tests.test_gpu_parity import _build_cache

pytestmark = pytest.mark.gpu

PRESETS = [("kvarn_k4v2_g64", 4, 2), ("kvarn_k2v2_g64", 2, 2), ("kvarn_k4v4_g64", 4, 4)]


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def say(*a):
    print(*a, flush=True)


def _params(K, preset, fmt, n_iters=8):
    p = K.params_from_dtype(preset, n_iters, format=fmt)
    assert p.group == 64
    return p


@pytest.mark.parametrize("preset,kb,vb", PRESETS)
@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("n_iters", [0, 1, 8])
def test_g64_quantize_against_oracle(K, preset, kb, vb, fmt, n_iters):
    n, hkv = 12, 3
    tiles, kinds = synth.tile_batch(n * hkv, "cpu", seed=400 + n_iters, return_kinds=True)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    tok = torch.arange(n, dtype=torch.int64) * 128
    page = torch.randperm(n, generator=torch.Generator().manual_seed(401)).to(torch.int32)
    params = _params(K, preset, fmt, n_iters)
    say(f"g64 quantize {preset} fmt={fmt} N={n_iters}")
    kp = K.new_pool(n, hkv, O.KIND_K, params=params)
    vp = K.new_pool(n, hkv, O.KIND_V, params=params)
    assert kp.shape[2] == O.record_bytes(O.KIND_K, kb, vb, fmt, 64)
    assert vp.shape[2] == O.record_bytes(O.KIND_V, kb, vb, fmt, 64)
    K.quantize_kv_tiles(params, src.cuda(), src.cuda(), tok.cuda(), page.cuda(), kp, vp)
    torch.cuda.synchronize()
    x16 = tiles.view(n, hkv, 128, 128).numpy()
    for kind, pool in ((O.KIND_K, kp), (O.KIND_V, vp)):
        st = T.QuantStats()
        for h in range(hkv):
            T.check_quantized_tiles(x16[:, h], T.records_of(pool, page.tolist(), h), kind,
                                    n_iters, st, k_bits=kb, v_bits=vb, fmt=fmt, group=64)
        say(f"g64 {preset} fmt={fmt} N={n_iters} kind={kind}: {st}")
        T.assert_rate(st)


@pytest.mark.parametrize("preset,kb,vb", PRESETS)
@pytest.mark.parametrize("fmt", [1, 2])
def test_g64_single_kind_and_dequantize(K, preset, kb, vb, fmt):
    """The per-kind launch writes the records of the K+V launch, and the dequantize kernel
    reads them back as the oracle does."""
    n, hkv = 5, 2
    tiles = synth.tile_batch(n * hkv, "cpu", seed=410)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous().cuda()
    tok = (torch.arange(n, dtype=torch.int64) * 128).cuda()
    page = torch.arange(n, dtype=torch.int32).cuda()
    params = _params(K, preset, fmt)
    say(f"g64 single kind + dequantize {preset} fmt={fmt}")
    kp = K.new_pool(n, hkv, O.KIND_K, params=params)
    vp = K.new_pool(n, hkv, O.KIND_V, params=params)
    K.quantize_kv_tiles(params, src, src, tok, page, kp, vp)
    for kind, pool in ((O.KIND_K, kp), (O.KIND_V, vp)):
        one = K.new_pool(n, hkv, kind, params=params)
        K.quantize_tiles(params, kind, src, tok, page, one)
        torch.cuda.synchronize()
        assert torch.equal(one, pool), kind
        out = K.dequantize_tiles(params, kind, pool, page)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        for h in range(hkv):
            for i, rec in enumerate(T.records_of(pool, range(n), h)):
                d = O.unpack_record(rec, kind, kb, vb, fmt=fmt, group=64)
                ref = O.dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], kind,
                                         group=64).T
                ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
                assert np.all(np.abs(got[i, h] - ref) <= 0.5 * ulp + 1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("preset,kb,vb", PRESETS)
@pytest.mark.parametrize("fmt", [1, 2])
def test_g64_decode_ragged(K, preset, kb, vb, fmt):
    """Ragged lengths (balanced layout, several sequences) with staging tails."""
    lens = [0, 1, 127, 128, 129, 300, 1000, 1024 + 77]
    hkv, G = 2, 8
    params = _params(K, preset, fmt)
    say(f"g64 decode ragged {preset} fmt={fmt}")
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=420)
    assert T.group_of(kp) == 64 and T.format_of(kp) == fmt
    q = torch.randn((len(lens), G * hkv, 128), generator=torch.Generator().manual_seed(421)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
    say(f"g64 {preset} fmt={fmt} decode: max rel err {err:.3e}")


@pytest.mark.parametrize("preset,kb,vb", PRESETS)
def test_g64_decode_long_one_sequence(K, preset, kb, vb):
    """One long sequence (split layout, several splits of several pages), GQA group 1 too."""
    lens = [64 * 128 + 50]
    for hkv, G in ((2, 8), (4, 1)):
        params = _params(K, preset, 1)
        say(f"g64 decode long {preset} hkv={hkv} G={G}")
        kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=430 + G)
        q = torch.randn((1, G * hkv, 128), generator=torch.Generator().manual_seed(431)).to(torch.float16).cuda()
        out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt)
        torch.cuda.synchronize()
        err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
        say(f"g64 {preset} decode, {lens}, G={G}: max rel err {err:.3e}")


@pytest.mark.parametrize("preset,kb,vb,fmt", [p + (1,) for p in PRESETS] + [PRESETS[0] + (2,)])
def test_g64_write_appends_and_chunk_attention(K, preset, kb, vb, fmt):
    from tests.test_gpu_chunk import _reference_rows
    from tests.test_gpu_write import _chunk, _extend_block_table
    lens, lens_new = [5, 200, 0], [300, 56, 260]
    hkv, G = 2, 8
    params = _params(K, preset, fmt)
    say(f"g64 write + appends + chunk attention {preset} fmt={fmt}")
    kp, vp, bt, kt, vt, sl, free = _build_cache(K, params, lens, hkv, seed=440, spare=4,
                                                width=max((L + n) // 128 for L, n in zip(lens, lens_new)) + 2)
    bt = _extend_block_table(bt, lens, lens_new, free)
    kn, vn, cu = _chunk(lens_new, hkv, seed=441)
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
    K.write_tokens(params, kn, vn, cu, sl, kt, vt, bt, kp, vp)
    torch.cuda.synchronize()
    assert torch.equal(kp, kpb) and torch.equal(vp, vpb), "chunk write and appends differ"
    sl2 = sl + torch.tensor(lens_new, dtype=torch.int32, device="cuda")
    total_q = sum(lens_new)
    q = torch.randn((total_q, hkv * G, 128), generator=torch.Generator().manual_seed(442)).to(torch.float16).cuda()
    out = K.chunk_attention(params, q, cu, kp, vp, bt, sl2, int(sl2.max().item()), kt, vt)
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(443).choice(total_q, 24, replace=False).tolist()) | {0, total_q - 1})
    ref = _reference_rows(q, cu, kp, vp, bt, kt, vt, sl2, G, rows)
    o = out.cpu().numpy().astype(np.float64)
    worst = max(T.assert_rows_close(o[r, hq], want, f"row {r} head {hq}") for (r, hq), want in ref.items())
    say(f"g64 {preset} fmt={fmt} write + appends + chunk attention: {len(rows)} rows, max rel err {worst:.2e}")
