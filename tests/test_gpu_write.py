"""GPU tests of the chunk write path (kvarn_write_tokens): prefill chunks of ragged lengths
into caches at ragged lengths, checked against one-token appends (bit for bit), against
kvarn_quantize_tiles of the same 128 tokens (bit for bit), and through the decode against the
oracle."""
import numpy as np
import pytest
import torch

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


def _chunk(lens_new, hkv, seed):
    g = torch.Generator().manual_seed(seed)
    total = sum(lens_new)
    k = torch.randn((max(total, 1), hkv, 128), generator=g).to(torch.float16)
    v = (torch.randn((max(total, 1), hkv, 128), generator=g) * 2.0).to(torch.float16)
    cu = torch.tensor([0] + list(np.cumsum(lens_new)), dtype=torch.int32)
    return k.cuda(), v.cuda(), cu.cuda()


def _extend_block_table(bt, lens, lens_new, free):
    """Give every sequence the pages its chunk completes (from the spare pages)."""
    bt = bt.cpu().clone()
    it = iter(free)
    for b, (L, n) in enumerate(zip(lens, lens_new)):
        for t in range(L // 128, (L + n) // 128):
            if bt[b, t] < 0:
                bt[b, t] = next(it)
    return bt.cuda()


CASES = [
    # prompt lengths (cache before the chunk), chunk lengths
    ([0, 5, 127, 128, 200, 356, 0, 64], [1, 300, 1, 128, 56, 1000, 0, 64]),
    ([0, 0, 0], [128, 255, 1024 + 77]),
    ([250, 383], [262, 129]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_write_equals_appends(K, case):
    lens, lens_new = CASES[case]
    hkv = 2
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    say(f"write vs appends: lens {lens}, chunks {lens_new}")
    spare = max(lens_new) // 128 + 2
    c = _build_cache(K, params, lens, hkv, seed=90 + case, spare=spare,
                     width=max((L + n) // 128 for L, n in zip(lens, lens_new)) + 2)
    kp, vp, bt, kt, vt, sl, free = c
    bt = _extend_block_table(bt, lens, lens_new, free)
    kn, vn, cu = _chunk(lens_new, hkv, seed=7 + case)
    # A: one chunk write
    kpa, vpa, kta, vta = kp.clone(), vp.clone(), kt.clone(), vt.clone()
    K.write_tokens(params, kn, vn, cu, sl, kta, vta, bt, kpa, vpa)
    # B: the same tokens one append at a time (sequences already done pass L = -1)
    kpb, vpb, ktb, vtb = kp.clone(), vp.clone(), kt.clone(), vt.clone()
    cu_h = cu.cpu().numpy()
    for i in range(max(lens_new)):
        sl_i = torch.tensor([L + i if i < n else -1 for L, n in zip(lens, lens_new)],
                            dtype=torch.int32, device="cuda")
        last = kn.shape[0] - 1      # sequences already done read any valid row (skipped)
        rows = torch.tensor([min(int(cu_h[b]) + min(i, max(n - 1, 0)), last)
                             for b, n in enumerate(lens_new)], dtype=torch.long, device="cuda")
        K.append_tokens(params, kn[rows].contiguous(), vn[rows].contiguous(), sl_i, ktb, vtb, bt,
                        kpb, vpb)
    torch.cuda.synchronize()
    assert torch.equal(kpa, kpb) and torch.equal(vpa, vpb), "pages differ"
    for b, (L, n) in enumerate(zip(lens, lens_new)):
        # the valid staging rows (those of the partial last tile) agree; rows past the length
        # hold nothing the cache reads (the append loop leaves completed tiles' tokens there)
        r = (L + n) % 128
        assert torch.equal(kta[b, :, :r], ktb[b, :, :r]), f"staging b={b}"
        assert torch.equal(vta[b, :, :r], vtb[b, :, :r]), f"staging b={b}"
    n_pages = sum((L + n) // 128 - L // 128 for L, n in zip(lens, lens_new))
    say(f"  {n_pages} pages completed, pools and staging identical")


def test_write_pages_equal_quantize_tiles_and_decode(K):
    lens, lens_new = CASES[0]
    hkv, G = 2, 8
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    spare = max(lens_new) // 128 + 2
    kp, vp, bt, kt, vt, sl, free = _build_cache(K, params, lens, hkv, seed=120, spare=spare,
                                                width=max((L + n) // 128 for L, n in zip(lens, lens_new)) + 2)
    bt = _extend_block_table(bt, lens, lens_new, free)
    kn, vn, cu = _chunk(lens_new, hkv, seed=121)
    kt0, vt0 = kt.clone(), vt.clone()
    K.write_tokens(params, kn, vn, cu, sl, kt, vt, bt, kp, vp)
    torch.cuda.synchronize()
    cu_h, bt_h = cu.cpu().numpy(), bt.cpu().numpy()
    checked = 0
    for b, (L, n) in enumerate(zip(lens, lens_new)):
        for t in range(L // 128, (L + n) // 128):
            # the tile's 128 tokens: below L from the old staging, then from the chunk
            for kind, stage0, new, pool in ((O.KIND_K, kt0, kn, kp), (O.KIND_V, vt0, vn, vp)):
                tile = torch.stack([stage0[b, :, a - 128 * t] if a < L else new[int(cu_h[b]) + a - L]
                                    for a in range(128 * t, 128 * t + 128)])       # [128, hkv, 128]
                ref = K.new_pool(1, hkv, kind, params=params)
                K.quantize_tiles(params, kind, tile.contiguous(),
                                 torch.zeros(1, dtype=torch.int64, device="cuda"),
                                 torch.zeros(1, dtype=torch.int32, device="cuda"), ref)
                torch.cuda.synchronize()
                assert torch.equal(pool[int(bt_h[b, t])], ref[0]), (b, t, kind)
                checked += 1
        # staging: the chunk's tokens of the partial last tile, earlier rows untouched
        end = L + n
        first = max(L, end // 128 * 128)
        for a in range(first, end):
            assert torch.equal(kt[b, :, a % 128], kn[int(cu_h[b]) + a - L]), (b, a)
            assert torch.equal(vt[b, :, a % 128], vn[int(cu_h[b]) + a - L]), (b, a)
        if end // 128 == L // 128:       # chunk stayed inside the partial tile
            assert torch.equal(kt[b, :, :L % 128], kt0[b, :, :L % 128])
    say(f"write: {checked} completed page records equal kvarn_quantize_tiles")
    # decode over the written cache
    sl2 = sl + torch.tensor(lens_new, dtype=torch.int32, device="cuda")
    q = torch.randn((len(lens), hkv * G, 128), generator=torch.Generator().manual_seed(122)).to(torch.float16).cuda()
    mx = int(sl2.max().item())
    out = K.decode_attention(params, q, kp, vp, bt, sl2, mx, kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(q, out, kp, vp, bt, sl2, G, k_tail=kt, v_tail=vt)
    say(f"  decode after write: max rel err {err:.2e}")
