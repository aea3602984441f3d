"""Seeded sweep of decode and multi-query read configurations against the oracle: every
preset, group sizes that do and do not divide 8 (G in 1..8), one to three KV heads, ragged
lengths (empty, below one page, exact pages, partial tails) and ragged chunks. Each case
writes a chunk into a quantized cache (kvarn_write_tokens), then checks sampled rows of
kvarn_chunk_attention (the multi-row layout when a sequence has several rows) and every
sequence of kvarn_decode_attention."""
import numpy as np
import pytest
import torch

from tests import kvarn_testlib as T
from tests.test_gpu_chunk import _reference_rows
from tests.test_gpu_parity import _build_cache
from tests.test_gpu_write import _chunk, _extend_block_table

pytestmark = pytest.mark.gpu

PRESETS = ["kvarn_k4v2_g128", "kvarn_k2v2_g128", "kvarn_k4v4_g128"]


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def say(*a):
    print(*a, flush=True)


def _case(i):
    rng = np.random.default_rng(1000 + i)
    preset = PRESETS[i % len(PRESETS)]
    G = int(rng.choice([1, 2, 3, 4, 5, 7, 8]))
    hkv = int(rng.integers(1, 4))
    B = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.choice([0, 1, 64, 127, 128, 129, 255, 256, 300, 511, 700, 1100], B)]
    lens_new = [int(x) for x in rng.choice([0, 1, 2, 17, 64, 128, 130, 257], B)]
    if sum(lens_new) == 0:
        lens_new[0] = 5
    return preset, G, hkv, lens, lens_new


@pytest.mark.parametrize("i", range(12))
def test_sweep(K, i):
    preset, G, hkv, lens, lens_new = _case(i)
    say(f"case {i}: {preset} G={G} Hkv={hkv} lens {lens} + chunks {lens_new}")
    params = K.params_from_dtype(preset, 8)
    kp, vp, bt, kt, vt, sl, free = _build_cache(
        K, params, lens, hkv, seed=2000 + i, spare=max(lens_new) // 128 + 2,
        width=max((L + n) // 128 for L, n in zip(lens, lens_new)) + 2)
    bt = _extend_block_table(bt, lens, lens_new, free)
    kn, vn, cu = _chunk(lens_new, hkv, seed=3000 + i)
    K.write_tokens(params, kn, vn, cu, sl, kt, vt, bt, kp, vp)
    sl2 = sl + torch.tensor(lens_new, dtype=torch.int32, device="cuda")
    mx = int(sl2.max().item())
    gen = torch.Generator().manual_seed(4000 + i)
    # multi-query read of the chunk
    total_q = sum(lens_new)
    q = torch.randn((total_q, hkv * G, 128), generator=gen).to(torch.float16).cuda()
    out = K.chunk_attention(params, q, cu, kp, vp, bt, sl2, mx, kt, vt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5000 + i)
    cu_h = cu.cpu().numpy()
    rows = set(rng.choice(total_q, size=min(16, total_q), replace=False).tolist())
    for b in range(len(lens)):
        if lens_new[b]:
            rows |= {int(cu_h[b]), int(cu_h[b + 1]) - 1}
    ref = _reference_rows(q, cu, kp, vp, bt, kt, vt, sl2, G, sorted(rows))
    o = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for (r, hq), want in ref.items():
        worst = max(worst, T.assert_rows_close(o[r, hq], want, f"case {i} row {r} head {hq}"))
    # decode of one more query per sequence over the written cache
    qd = torch.randn((len(lens), hkv * G, 128), generator=gen).to(torch.float16).cuda()
    od = K.decode_attention(params, qd, kp, vp, bt, sl2, mx, kt, vt)
    torch.cuda.synchronize()
    err = T.check_decode(qd, od, kp, vp, bt, sl2, G, k_tail=kt, v_tail=vt)
    say(f"  chunk rows {len(rows)}: max rel err {worst:.2e}; decode {err:.2e}")
