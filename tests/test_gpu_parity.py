"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, small shapes
that span several tiles, ragged tails and the degenerate cases."""
import numpy as np
import pytest
import torch

from oracle import kvarn_oracle as O
from kv_cache_quantization_tile_amd import synth
from tests import kvarn_testlib as T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def say(*a):
    print(*a, flush=True)


def _quantize(K, params, kind, src, tile_tok, tile_page, num_pages):
    hkv = src.shape[1]
    pool = K.new_pool(num_pages, hkv, kind, params=params)
    K.quantize_tiles(params, kind, src, tile_tok, tile_page, pool)
    torch.cuda.synchronize()
    return pool


def _tiles_from_src(src_cpu: torch.Tensor, tile_tok, head):
    """[n, 128 tok, 128 ch] numpy float16 tiles of one head."""
    return np.stack([src_cpu[t:t + 128, head, :].numpy() for t in tile_tok])


# ----------------------------------------------------------------------------- quantize


@pytest.mark.parametrize("kind", [O.KIND_K, O.KIND_V])
def test_quantize_single_tile(K, kind):
    w = synth.single_tile("cpu")
    say(f"single tile kind={kind} iters={w.n_iters}")
    params = K.params_from_dtype("kvarn_k4v2_g128", w.n_iters)
    src = (w.k_src if kind == O.KIND_K else w.v_src).cuda()
    pool = _quantize(K, params, kind, src, w.tile_src_token.cuda(), w.tile_dst_page.cuda(), 1)
    st = T.check_quantized_tiles(_tiles_from_src(src.cpu(), [0], 0), T.records_of(pool, [0], 0), kind, w.n_iters)
    say(st)
    T.assert_rate(st)


@pytest.mark.parametrize("n_iters", [0, 1, 2, 8])
@pytest.mark.parametrize("kind", [O.KIND_K, O.KIND_V])
def test_quantize_mixed_tiles_strided(K, kind, n_iters):
    """36 tiles of mixed distributions (normal, t(3), outlier channels, offset-dominated,
    large), spread over 3 KV heads of a token-major stream, written to permuted pages. Every
    tile is held to L1-L3; only the offset-dominated groups (the rotated DC channel of the
    offset tiles) compare codes through L2 and the reconstruction bound."""
    n, hkv = 12, 3
    tiles, kinds = synth.tile_batch(n * hkv, "cpu", seed=20 + n_iters, return_kinds=True)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    g = torch.Generator().manual_seed(5)
    order = torch.randperm(n, generator=g)
    tile_tok = (order * 128).to(torch.int64)
    pages = torch.randperm(n + 4, generator=g)[:n].to(torch.int32)
    say(f"mixed tiles kind={kind} iters={n_iters} n={n} hkv={hkv}")
    params = K.params_from_dtype("kvarn_k4v2_g128", n_iters)
    pool = _quantize(K, params, kind, src.cuda(), tile_tok.cuda(), pages.cuda(), n + 4)
    st = T.QuantStats()
    for h in range(hkv):
        x = _tiles_from_src(src, tile_tok.tolist(), h)
        T.check_quantized_tiles(x, T.records_of(pool, pages.tolist(), h), kind, n_iters, st)
    say(st)
    T.assert_rate(st)


@pytest.mark.parametrize("kind", [O.KIND_K, O.KIND_V])
@pytest.mark.parametrize("preset,fmt", [("kvarn_k4v2_g128", 1), ("kvarn_k4v2_g64", 1),
                                        ("kvarn_k4v4_g64", 2)])
def test_quantize_degenerate_tiles(K, kind, preset, fmt):
    """Zero tile, constant tile, one non-zero token, one non-zero channel, all tokens equal,
    tiny and huge magnitudes, heavy tails, and a constant offset whose noise sits below float16
    resolution (its rotated DC channel is offset-dominated; at one iteration its normalized
    values exceed the float16 range, so its zero saturates at 65504); also with group 64, where
    a non-zero token or channel sits in one half only. The offset tile's input takes only a few
    float16 values, so its normalized values repeat and the oracle itself puts many code values
    on rounding ties (group 64, N = 8: 869 of its 16,384 value codes within 2e-4 of a
    half-level): the L3 rate here counts the mismatches outside the tie band, and the codes at
    ties are held to L2."""
    rng = np.random.default_rng(3)
    tiles = np.zeros((9, 128, 128), np.float32)       # [tile, token, channel]
    tiles[1] = 2.5
    tiles[2, 17] = rng.standard_normal(128)
    tiles[3, :, 5] = rng.standard_normal(128)
    tiles[4] = rng.standard_normal(128)[None, :]
    tiles[5] = rng.standard_normal((128, 128)) * 1e-3
    tiles[6] = rng.standard_normal((128, 128)) * 3000
    tiles[7] = rng.standard_t(2.5, (128, 128))
    tiles[8] = 5.0 + 1e-3 * rng.standard_normal((128, 128))
    x16 = tiles.astype(np.float16)
    n = x16.shape[0]
    src = torch.from_numpy(x16).reshape(n * 128, 1, 128)
    tok = torch.arange(n, dtype=torch.int64) * 128
    st = T.QuantStats()
    for iters in (1, 8):
        say(f"degenerate tiles kind={kind} iters={iters} {preset} fmt={fmt}")
        params = K.params_from_dtype(preset, iters, format=fmt)
        pool = _quantize(K, params, kind, src.cuda(), tok.cuda(), torch.arange(n, dtype=torch.int32).cuda(), n)
        T.check_quantized_tiles(x16, T.records_of(pool, range(n), 0), kind, iters, st,
                                k_bits=params.k_bits, v_bits=params.v_bits, fmt=fmt,
                                group=params.group)
    say(st)
    T.assert_rate(st, ties_apart=True)


@pytest.mark.parametrize("kind", [O.KIND_K, O.KIND_V])
def test_quantize_float16_range_ends(K, kind):
    """Inputs at both ends of the float16 range: every value a float16 subnormal (~2e-6),
    subnormals with a few outliers 1000x larger, values up to +-60000 near the float16
    maximum, and a tile whose first half is subnormal and second half near the maximum."""
    rng = np.random.default_rng(8)
    tiles = np.zeros((4, 128, 128), np.float32)
    tiles[0] = rng.standard_normal((128, 128)) * 2e-6
    tiles[1] = rng.standard_normal((128, 128)) * 2e-6
    tiles[1][rng.random((128, 128)) < 0.01] *= 1000.0
    tiles[2] = np.clip(rng.standard_normal((128, 128)) * 2e4, -60000, 60000)
    tiles[3, :64] = rng.standard_normal((64, 128)) * 2e-6
    tiles[3, 64:] = np.clip(rng.standard_normal((64, 128)) * 2e4, -60000, 60000)
    x16 = tiles.astype(np.float16)
    assert np.isfinite(x16).all() and np.abs(x16[0]).max() < 6.1e-5   # tile 0 all subnormal
    n = x16.shape[0]
    src = torch.from_numpy(x16).reshape(n * 128, 1, 128)
    tok = torch.arange(n, dtype=torch.int64) * 128
    st = T.QuantStats()
    for iters in (1, 8):
        say(f"float16 range ends kind={kind} iters={iters}")
        params = K.params_from_dtype("kvarn_k4v2_g128", iters)
        pool = _quantize(K, params, kind, src.cuda(), tok.cuda(), torch.arange(n, dtype=torch.int32).cuda(), n)
        T.check_quantized_tiles(x16, T.records_of(pool, range(n), 0), kind, iters, st)
    say(st)
    T.assert_rate(st, ties_apart=True)


def test_saturated_zero_page_decodes_finite(K):
    """A near-constant tile (5 + 1e-3 noise) at one iteration normalizes its rotated DC channel
    to ~1.9e5, beyond float16: both sides store that key channel's zero saturated at 65504
    (codes at 15), the record stays finite, and a decode over the page matches the oracle
    reading the same record."""
    rng = np.random.default_rng(7)
    x16 = (5 + 1e-3 * rng.standard_normal((128, 128))).astype(np.float16)   # [token, channel]
    src = torch.from_numpy(x16).reshape(128, 1, 128).cuda()
    tok = torch.zeros(1, dtype=torch.int64, device="cuda")
    page = torch.zeros(1, dtype=torch.int32, device="cuda")
    params = K.params_from_dtype("kvarn_k4v2_g128", 1)
    say("saturated zero: near-constant tile at 1 iteration")
    kp = _quantize(K, params, O.KIND_K, src, tok, page, 1)
    vp = _quantize(K, params, O.KIND_V, src, tok, page, 1)
    g = O.unpack_k_record(T.records_of(kp, [0], 0)[0])
    assert g["zero"][0] == np.float16(65504) and np.all(g["codes"][0] == 15)
    for kind, pool in ((O.KIND_K, kp), (O.KIND_V, vp)):
        st = T.check_quantized_tiles(x16[None], T.records_of(pool, [0], 0), kind, 1)
        T.assert_rate(st)
    q = torch.from_numpy(rng.standard_normal((1, 8, 128)).astype(np.float16)).cuda()
    lens = torch.tensor([128], dtype=torch.int32, device="cuda")
    bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    out = K.decode_attention(params, q, kp, vp, bt, lens, 128)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    err = T.check_decode(q, out, kp, vp, bt, lens, 8)
    say(f"  decode over the saturated page: max rel err {err:.2e}")


def test_quantize_skips_out_of_range(K):
    w = synth.single_tile("cpu")
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    src = w.k_src.cuda()
    pool = torch.full((3, 1, 9216), 0xAB, dtype=torch.uint8, device="cuda")
    tok = torch.tensor([0, 1, -5, 0, 0], dtype=torch.int64, device="cuda")     # 1: past the end
    page = torch.tensor([0, 1, 2, 3, -1], dtype=torch.int32, device="cuda")    # 3, -1: outside
    say("quantize bounds: skipped tiles leave the pool untouched")
    K.quantize_tiles(params, O.KIND_K, src, tok, page, pool)
    torch.cuda.synchronize()
    p = pool.cpu()
    assert not torch.all(p[0] == 0xAB)
    assert torch.all(p[1] == 0xAB) and torch.all(p[2] == 0xAB)


def test_quantize_deterministic(K):
    tiles = synth.tile_batch(16, "cpu", seed=9)
    src = tiles.reshape(16 * 128, 1, 128).cuda()
    tok = (torch.arange(16, dtype=torch.int64) * 128).cuda()
    page = torch.arange(16, dtype=torch.int32).cuda()
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    say("quantize determinism")
    for kind in (O.KIND_K, O.KIND_V):
        a = _quantize(K, params, kind, src, tok, page, 16)
        b = _quantize(K, params, kind, src, tok, page, 16)
        assert torch.equal(a, b)


def test_quantize_kv_matches_separate_launches(K):
    """The one-launch K+V entry point writes exactly the records of the two per-kind calls
    (same kernels), on mixed tiles over 2 heads with permuted pages; the oracle then checks
    the records of the combined call."""
    n, hkv = 10, 2
    tk, kinds = synth.tile_batch(n * hkv, "cpu", seed=31, return_kinds=True)
    tv = synth.tile_batch(n * hkv, "cpu", seed=32)
    mk = lambda t: t.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    ksrc, vsrc = mk(tk), mk(tv)
    g = torch.Generator().manual_seed(6)
    order = torch.randperm(n, generator=g)
    tok = (order * 128).to(torch.int64)
    pages = torch.randperm(n + 3, generator=g)[:n].to(torch.int32)
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    say(f"quantize_kv_tiles n={n} hkv={hkv}")
    kp, vp = K.new_pool(n + 3, hkv, O.KIND_K, params=params), K.new_pool(n + 3, hkv, O.KIND_V, params=params)
    K.quantize_kv_tiles(params, ksrc.cuda(), vsrc.cuda(), tok.cuda(), pages.cuda(), kp, vp)
    kref = _quantize(K, params, O.KIND_K, ksrc.cuda(), tok.cuda(), pages.cuda(), n + 3)
    vref = _quantize(K, params, O.KIND_V, vsrc.cuda(), tok.cuda(), pages.cuda(), n + 3)
    assert torch.equal(kp, kref) and torch.equal(vp, vref)
    st = T.QuantStats()
    for h in range(hkv):
        T.check_quantized_tiles(_tiles_from_src(ksrc, tok.tolist(), h),
                                T.records_of(kp, pages.tolist(), h), O.KIND_K, 8, st)
    say(st)
    T.assert_rate(st)


@pytest.mark.parametrize("kind", [O.KIND_K, O.KIND_V])
def test_dequantize_tiles_matches_oracle(K, kind):
    """GPU records read back by kvarn_dequantize_tiles against the oracle's dequantization of
    the same records: each element within half a float16 ulp of the float64 value (the final
    rounding) plus 1e-5 of the tile's largest magnitude (float32 evaluation). Pages outside
    the pool leave their output tile untouched."""
    n, hkv = 8, 2
    tiles = synth.tile_batch(n * hkv, "cpu", seed=41)
    src = tiles.view(n, hkv, 128, 128).permute(0, 2, 1, 3).reshape(n * 128, hkv, 128).contiguous()
    tok = (torch.arange(n, dtype=torch.int64) * 128)
    pages = torch.randperm(n + 2, generator=torch.Generator().manual_seed(7))[:n].to(torch.int32)
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    say(f"dequantize kind={kind}")
    pool = _quantize(K, params, kind, src.cuda(), tok.cuda(), pages.cuda(), n + 2)
    read = torch.cat([pages, torch.tensor([n + 5, -1], dtype=torch.int32)])   # 2 outside
    out = torch.full((n + 2, hkv, 128, 128), 7.0, dtype=torch.float16, device="cuda")
    K.dequantize_tiles(params, kind, pool, read.cuda(), out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(got[n:] == 7.0)
    unpack = O.unpack_k_record if kind == O.KIND_K else O.unpack_v_record
    worst = 0.0
    for h in range(hkv):
        for i, rec in enumerate(T.records_of(pool, pages.tolist(), h)):
            d = unpack(rec)
            ref = O.dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], kind).T
            ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
            bound = 0.5 * ulp + 1e-5 * np.abs(ref).max()
            err = np.abs(got[i, h] - ref)
            assert np.all(err <= bound), (h, i, float((err / bound).max()))
            worst = max(worst, float((err / bound).max()))
    say(f"  worst error / bound {worst:.3f}")


# ----------------------------------------------------------------------------- decode


def _build_cache(K, params, lens, hkv, seed, spare=2, dist="normal", width=None):
    """Quantize random prompts of the given lengths into permuted pages; return the pools,
    block table, staging tails (holding each sequence's last L % 128 tokens) and lens."""
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    T_ = sum(lens)
    mk = (lambda s: torch.randn(s, generator=g)) if dist == "normal" else (
        lambda s: torch.randn(s, generator=g) * torch.exp(torch.randn((1, s[1], s[2]), generator=g)))
    k = mk((T_, hkv, 128)).to(torch.float16)
    v = mk((T_, hkv, 128)).to(torch.float16)
    n_pages = sum(L // 128 for L in lens) + spare * B
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    width = width or max(L // 128 for L in lens) + spare + 1
    bt = torch.full((B, width), -1, dtype=torch.int32)
    ktail = torch.zeros((B, hkv, 128, 128), dtype=torch.float16)
    vtail = torch.zeros((B, hkv, 128, 128), dtype=torch.float16)
    toks, pages, start, nxt = [], [], 0, 0
    for b, L in enumerate(lens):
        for p in range(L // 128):
            bt[b, p] = perm[nxt]
            toks.append(start + 128 * p)
            pages.append(int(perm[nxt]))
            nxt += 1
        r = L % 128
        if r:
            ktail[b, :, :r] = k[start + L - r:start + L].permute(1, 0, 2)
            vtail[b, :, :r] = v[start + L - r:start + L].permute(1, 0, 2)
        start += L
    kp = K.new_pool(n_pages, hkv, O.KIND_K, params=params)
    vp = K.new_pool(n_pages, hkv, O.KIND_V, params=params)
    if toks:
        tt = torch.tensor(toks, dtype=torch.int64).cuda()
        pp = torch.tensor(pages, dtype=torch.int32).cuda()
        K.quantize_tiles(params, O.KIND_K, k.cuda(), tt, pp, kp)
        K.quantize_tiles(params, O.KIND_V, v.cuda(), tt, pp, vp)
    free = [int(x) for x in perm[nxt:]]
    return kp, vp, bt.cuda(), ktail.cuda(), vtail.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), free


def test_decode_single_tile(K):
    w = synth.single_tile("cpu")
    params = K.params_from_dtype("kvarn_k4v2_g128", w.n_iters)
    say("decode single tile")
    kp = _quantize(K, params, O.KIND_K, w.k_src.cuda(), w.tile_src_token.cuda(), w.tile_dst_page.cuda(), 1)
    vp = _quantize(K, params, O.KIND_V, w.v_src.cuda(), w.tile_src_token.cuda(), w.tile_dst_page.cuda(), 1)
    q = w.extra["q0"].cuda()
    lens = torch.tensor([128], dtype=torch.int32).cuda()
    out = K.decode_attention(params, q, kp, vp, w.block_table.cuda(), lens, 128)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, w.block_table, lens, G=1)
    say(f"max rel err {err:.3e}")


@pytest.mark.parametrize("G,hkv", [(8, 2), (4, 3), (2, 1), (1, 4)])
def test_decode_ragged_gqa(K, G, hkv):
    lens = [0, 1, 127, 128, 129, 300, 1000, 1024 + 77]
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    say(f"decode ragged G={G} hkv={hkv} lens={lens}")
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=40 + G)
    q = torch.randn((len(lens), G * hkv, 128), generator=torch.Generator().manual_seed(1)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
    say(f"max rel err {err:.3e}")


@pytest.mark.parametrize("factor", [40.0, 1e-3])
@pytest.mark.parametrize("single", [False, True])
def test_decode_softmax_extremes(K, factor, single):
    """Softmax scales far from 1/sqrt(128): 40x (nearly one-hot attention, scores spanning
    hundreds of log2 units, most weights flushed to zero) and 1e-3x (nearly uniform weights,
    the output close to the mean of the values), over pages and staged tails, both layouts."""
    scale = factor / np.sqrt(128.0)
    lens = [128 * 3 + 77, 128 * 5, 200, 128 * 2 + 1] if not single else [128 * 6 + 45]
    hkv, G = 2, 4
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    say(f"decode softmax scale x{factor} single={single}")
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=70 + int(single))
    q = torch.randn((len(lens), G * hkv, 128), generator=torch.Generator().manual_seed(71)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt, softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt, softmax_scale=scale)
    say(f"max rel err {err:.3e}")


TAIL_LENS = [1, 31, 32, 33, 63, 64, 65, 96, 97, 127]


@pytest.mark.parametrize("G,hkv,single", [(8, 2, False), (4, 1, False), (1, 3, False),
                                          (8, 1, True), (2, 2, True)])
def test_decode_tail_lengths_across_wave_boundaries(K, G, hkv, single):
    """Staged tails of every length class of the staged-token attention (one to four waves
    of 32 tokens, each boundary from both sides), after two pages and alone; the staging rows
    past each tail hold NaN, so a key or value read there shows in the output. single: one
    sequence per call (the split layout), else all in one batch (the balanced layout)."""
    lens = [256 + t for t in TAIL_LENS] + [5, 100]
    params = K.params_from_dtype("kvarn_k4v2_g128", 4)
    say(f"decode tail lengths G={G} hkv={hkv} single={single}")
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=60 + 10 * G + hkv)
    for b, L in enumerate(lens):
        kt[b, :, L % 128:] = float("nan")
        vt[b, :, L % 128:] = float("nan")
    q = torch.randn((len(lens), G * hkv, 128), generator=torch.Generator().manual_seed(61)).to(torch.float16).cuda()
    if single:
        out = torch.empty((len(lens), G * hkv, 128), dtype=torch.float16, device="cuda")
        for b, L in enumerate(lens):
            out[b:b + 1] = K.decode_attention(params, q[b:b + 1], kp, vp, bt[b:b + 1], sl[b:b + 1], L,
                                              kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous())
    else:
        out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens), kt, vt)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
    say(f"max rel err {err:.3e}")


def test_decode_many_splits_and_max_seq_len_clamp(K):
    """Long enough for several splits; max_seq_len above every length (unused splits)."""
    lens = [128 * 37 + 5, 128 * 60, 128 * 3]
    params = K.params_from_dtype("kvarn_k4v2_g128", 4)
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, 2, seed=77, dist="scaled", width=81)
    q = torch.randn((3, 16, 128), generator=torch.Generator().manual_seed(2)).to(torch.float16).cuda()
    mx = 128 * 80
    say(f"decode splits={K.decode_num_splits(params, 3, 2, mx)} lens={lens}")
    out = K.decode_attention(params, q, kp, vp, bt, sl, mx, kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl, 8, k_tail=kt, v_tail=vt)
    say(f"max rel err {err:.3e}")


@pytest.mark.parametrize("preset,fmt,pages", [("kvarn_k4v2_g128", 1, 300), ("kvarn_k4v2_g128", 1, 256),
                                               ("kvarn_k4v4_g128", 1, 300), ("kvarn_k2v2_g64", 2, 300)])
def test_decode_one_sequence_several_pages_per_wave(K, preset, fmt, pages):
    """One sequence over 8 KV heads long enough for several pages per wave in one round of
    page waves (the split layout's page loop with its prefetch of the next page, at small
    size): 300 pages give waves with unequal page counts, 256 equal ones."""
    hkv, G = 8, 8
    lens = [128 * pages + 77]
    params = K.params_from_dtype(preset, 8, format=fmt)
    ns = K.decode_num_splits(params, 1, hkv, lens[0])
    assert hkv * ns * 4 <= 1024 and hkv * pages > 1024      # >= 2 pages per wave, one round
    say(f"decode one sequence, several pages per wave: {preset} fmt={fmt} pages={pages} splits={ns}")
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=90 + pages)
    q = torch.randn((1, G * hkv, 128), generator=torch.Generator().manual_seed(91)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, lens[0], kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, rows=[(0, 0), (0, 5)], k_tail=kt, v_tail=vt)
    say(f"max rel err {err:.3e}")


@pytest.mark.parametrize("B,hkv,G,hi", [(3, 1, 8, 260), (300, 1, 2, 700), (1024, 1, 1, 300),
                                        (1025, 1, 1, 300), (5, 2, 4, 128 * 500)])
def test_decode_balanced_layout(K, B, hkv, G, hi):
    """A decode of 2..1024 sequences gives every wave an equal share of all (sequence, KV
    head, page) entries, crossing sequence boundaries; 1025 sequences take the split layout.
    Cases: fewer pages than waves (3 sequences of at most 2 pages), several prefix entries per
    thread (300 and 1024 sequences, lengths from 0 to a few pages, some without a full page),
    and 5 long sequences (pages per wave above one segment). Every row is compared with the
    same sequence decoded alone (the split layout: same sums, another float32 order), sampled
    rows with the oracle."""
    gen = torch.Generator().manual_seed(900 + B)
    lens = torch.randint(0, hi + 1, (B,), generator=gen).tolist()
    lens[0], lens[-1] = 0, hi
    if B > 3:
        lens[1], lens[2] = 127, 128
    params = K.params_from_dtype("kvarn_k4v2_g128", 2)
    say(f"decode balanced layout B={B} hkv={hkv} G={G} pages={sum(L // 128 for L in lens)}")
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=910 + B)
    q = torch.randn((B, G * hkv, 128), generator=gen).to(torch.float16).cuda()
    mx = max(lens)
    out = K.decode_attention(params, q, kp, vp, bt, sl, mx, kt, vt)
    one = torch.empty_like(out)
    for b in range(B):
        one[b:b + 1] = K.decode_attention(params, q[b:b + 1].contiguous(), kp, vp,
                                          bt[b:b + 1].contiguous(), sl[b:b + 1], mx,
                                          kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous())
    torch.cuda.synchronize()
    of, sf = out.float(), one.float()
    empty = torch.tensor([L == 0 for L in lens]).cuda()
    assert torch.all(out[empty] == 0) and torch.all(one[empty] == 0)
    scale = sf.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    diff = float(((of - sf).abs() / scale).max())
    assert diff <= 2e-3, diff
    rng = np.random.default_rng(920 + B)
    pick, budget = [], 1200         # oracle pages (K and V records per KV head)
    for b in [B - 1] + rng.permutation(B).tolist():
        if len(pick) < 12 and b not in pick and lens[b] // 128 * hkv <= budget:
            pick.append(b)
            budget -= lens[b] // 128 * hkv
    err = T.check_decode(q, out, kp, vp, bt, sl, G, rows=[(b, g) for b in pick for g in range(hkv)],
                         k_tail=kt, v_tail=vt)
    say(f"  all rows vs one-sequence decodes: max rel diff {diff:.1e}; {len(pick)} sequences vs "
        f"the oracle: max rel err {err:.2e}")


def test_decode_balanced_random_shapes(K):
    """24 seeded shapes (2..40 sequences, 1..8 KV heads, groups 1..8, lengths 0..3000, pages
    out of the pool in a few block tables, with and without tails, 2 presets): the balanced
    layout's output equals each sequence decoded alone (split layout) within float32
    summation-order differences, and empty rows are zeros."""
    rng = np.random.default_rng(930)
    worst = 0.0
    for case in range(24):
        B = int(rng.integers(2, 41))
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        lens = rng.integers(0, 3001, size=B).tolist()
        preset = "kvarn_k4v2_g128" if case % 3 else "kvarn_k2v2_g128"
        params = K.params_from_dtype(preset, 1)
        kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=940 + case)
        if case % 4 == 1:                       # a few entries outside the pool
            bt = bt.cpu()
            for b in range(0, B, 3):
                if lens[b] >= 128:
                    bt[b, int(rng.integers(0, lens[b] // 128))] = kp.shape[0] + 5
            bt = bt.cuda()
        tails = case % 5 != 2
        q = torch.from_numpy(rng.standard_normal((B, G * hkv, 128))).to(torch.float16).cuda()
        mx = max(lens)
        args = (kt, vt) if tails else (None, None)
        out = K.decode_attention(params, q, kp, vp, bt, sl, mx, *args)
        one = torch.empty_like(out)
        for b in range(B):
            tb = (kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous()) if tails else (None, None)
            one[b:b + 1] = K.decode_attention(params, q[b:b + 1].contiguous(), kp, vp,
                                              bt[b:b + 1].contiguous(), sl[b:b + 1], mx, *tb)
        torch.cuda.synchronize()
        of, sf = out.float(), one.float()
        scale = sf.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
        diff = float(((of - sf).abs() / scale).max())
        assert diff <= 2e-3, (case, B, hkv, G, diff)
        zero_rows = (sf.abs().amax(dim=-1) == 0)
        assert torch.all(of[zero_rows] == 0), case
        worst = max(worst, diff)
    say(f"24 shapes: balanced layout vs one-sequence decodes, max rel diff {worst:.1e}")


def test_decode_without_tail_buffers(K):
    """NULL tails: tokens past the last full page are ignored."""
    lens = [128 * 5 + 40, 256]
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, 1, seed=5)
    q = torch.randn((2, 8, 128), generator=torch.Generator().manual_seed(3)).to(torch.float16).cuda()
    out = K.decode_attention(params, q, kp, vp, bt, sl, max(lens))
    torch.cuda.synchronize()
    full = torch.tensor([128 * 5, 256], dtype=torch.int32).cuda()
    T.check_decode(q, out, kp, vp, bt, full, 8)


def test_decode_skips_out_of_range_pages(K):
    """Block-table entries outside the pool are skipped: a sequence whose first page is -1,
    one with a page id past the pool in the middle, and one whose pages are all outside
    with no tail (its output is zeros); the others keep several splits' worth of pages."""
    lens = [128 * 9 + 17, 128 * 40 + 3, 128 * 4, 128 * 23]
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, 2, seed=61)
    n_pool = kp.shape[0]
    bt = bt.cpu()
    bt[0, 0] = -1
    bt[1, 17] = n_pool + 3
    bt[1, 30] = -7
    bt[2, :4] = torch.tensor([-1, n_pool, n_pool + 100, -2], dtype=torch.int32)
    bt = bt.cuda()
    kt[2].zero_()
    vt[2].zero_()
    q = torch.randn((4, 16, 128), generator=torch.Generator().manual_seed(6)).to(torch.float16).cuda()
    mx = max(lens)
    say(f"decode skipped pages: splits={K.decode_num_splits(params, 4, 2, mx)} lens={lens}")
    out = K.decode_attention(params, q, kp, vp, bt, sl, mx, kt, vt)
    torch.cuda.synchronize()
    assert torch.all(out[2] == 0)
    err = T.check_decode(q, out, kp, vp, bt, sl, 8, k_tail=kt, v_tail=vt)
    say(f"max rel err {err:.3e}")


def test_append_fill_and_decode(K):
    """Lengths 120 mod 128: appended tokens fill the staging tile after 8 steps, which is
    then quantized into a fresh page; decode is checked after every step, and the filled
    page must equal kvarn_quantize_tiles of the same 128 tokens bit for bit."""
    lens = [128 * 2 + 120, 120]
    hkv, G = 2, 8
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl, free = _build_cache(K, params, lens, hkv, seed=11)
    bt_cpu = bt.cpu()
    for b, L in enumerate(lens):  # reserve the page each sequence fills next
        bt_cpu[b, L // 128] = free[b]
    bt = bt_cpu.cuda()
    g = torch.Generator().manual_seed(12)
    for step in range(10):
        say(f"append step {step} lens={sl.tolist()}")
        kn = torch.randn((2, hkv, 128), generator=g).to(torch.float16).cuda()
        vn = torch.randn((2, hkv, 128), generator=g).to(torch.float16).cuda()
        q = torch.randn((2, hkv * G, 128), generator=g).to(torch.float16).cuda()
        pre = [kt.clone(), vt.clone()]
        K.append_tokens(params, kn, vn, sl, kt, vt, bt, kp, vp)
        filled = [b for b in range(2) if int(sl[b]) % 128 == 127]
        sl = sl + 1
        out = K.decode_attention(params, q, kp, vp, bt, sl, int(sl.max()), kt, vt)
        torch.cuda.synchronize()
        for b in filled:
            page = int(bt_cpu[b, (int(sl[b]) - 1) // 128])
            for kind, pool, stage, new in ((O.KIND_K, kp, pre[0], kn), (O.KIND_V, vp, pre[1], vn)):
                tile = stage[b].clone()
                tile[:, 127] = new[b]
                src = tile.permute(1, 0, 2).contiguous()          # [128 tok, hkv, 128]
                ref = K.new_pool(1, hkv, kind, params=params)
                K.quantize_tiles(params, kind, src, torch.zeros(1, dtype=torch.int64).cuda(),
                                 torch.zeros(1, dtype=torch.int32).cuda(), ref)
                torch.cuda.synchronize()
                assert torch.equal(pool[page], ref[0]), f"filled page b={b} kind={kind}"
        T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
