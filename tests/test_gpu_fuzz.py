"""Seeded random shapes through the read paths, each case against the oracle: decode (both
work layouts: the balanced one for 2..1024 sequences, the split one for a single sequence)
over random presets, record formats, group sizes, GQA ratios and ragged lengths with staged
tails (NaN past every tail), and chunked multi-query reads over random chunk lengths. The
shapes stay small enough for the oracle to check every (sequence, KV head) row in seconds."""
import numpy as np
import pytest
import torch

from tests import kvarn_testlib as T
from tests.test_gpu_parity import _build_cache
from tests.test_gpu_chunk import _written_cache, _reference_rows

pytestmark = pytest.mark.gpu

PRESETS = ["kvarn_k4v2_g128", "kvarn_k2v2_g128", "kvarn_k4v4_g128",
           "kvarn_k4v2_g64", "kvarn_k2v2_g64", "kvarn_k4v4_g64"]


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def say(*a):
    print(*a, flush=True)


def _random_lens(rng, B):
    """Ragged lengths: empty, below one page, exact page multiples, tails on either side of
    the staged attention's 32-token wave boundaries, and a few pages plus any tail."""
    out = []
    for _ in range(B):
        kind = rng.integers(0, 5)
        if kind == 0:
            out.append(int(rng.choice([0, 1, 31, 32, 33, 127])))
        elif kind == 1:
            out.append(128 * int(rng.integers(1, 6)))
        elif kind == 2:
            out.append(128 * int(rng.integers(1, 6)) + int(rng.choice([1, 31, 32, 33, 63, 64, 65, 96, 97, 127])))
        else:
            out.append(int(rng.integers(0, 128 * 7)))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_shapes(K, seed):
    rng = np.random.default_rng(7000 + seed)
    preset = PRESETS[seed % len(PRESETS)]
    fmt = int(rng.integers(1, 3))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = 1 if seed % 4 == 3 else int(rng.integers(2, 25))
    lens = _random_lens(rng, B)
    if B == 1 and lens[0] < 128:
        lens[0] += 128 * 3
    params = K.params_from_dtype(preset, 8, format=fmt)
    say(f"fuzz decode seed={seed} {preset} fmt={fmt} B={B} hkv={hkv} G={G} lens={lens}")
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=7100 + seed)
    for b, L in enumerate(lens):
        kt[b, :, L % 128:] = float("nan")
        vt[b, :, L % 128:] = float("nan")
    q = torch.randn((B, G * hkv, 128), generator=torch.Generator().manual_seed(7200 + seed))
    q = q.to(torch.float16).cuda()
    # the host only knows an upper bound of the lengths: sometimes a loose one
    mx = max(lens) + (int(rng.integers(1, 300)) if seed % 3 == 0 else 0)
    mx = max(mx, 1)
    out = K.decode_attention(params, q, kp, vp, bt, sl, mx, kt, vt)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = T.check_decode(q, out, kp, vp, bt, sl, G, k_tail=kt, v_tail=vt)
    say(f"max rel err {err:.3e}")


@pytest.mark.parametrize("seed", range(6))
def test_chunk_random_shapes(K, seed):
    rng = np.random.default_rng(8000 + seed)
    preset = PRESETS[(seed * 5) % len(PRESETS)]
    fmt = int(rng.integers(1, 3))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([2, 4, 8]))
    B = int(rng.integers(1, 5))
    lens = [int(rng.choice([0, int(rng.integers(1, 128)), 128 * int(rng.integers(1, 4)),
                            int(rng.integers(1, 128 * 4))])) for _ in range(B)]
    lens_new = [int(rng.integers(1, 300)) for _ in range(B)]
    params = K.params_from_dtype(preset, 8, format=fmt)
    say(f"fuzz chunk seed={seed} {preset} fmt={fmt} hkv={hkv} G={G} lens={lens} + {lens_new}")
    kp, vp, bt, kt, vt, sl = _written_cache(K, params, lens, lens_new, hkv, seed=8100 + seed)
    total_q = sum(lens_new)
    cu_q = torch.tensor([0] + list(np.cumsum(lens_new)), dtype=torch.int32, device="cuda")
    q = torch.randn((total_q, hkv * G, 128), generator=torch.Generator().manual_seed(8200 + seed))
    q = q.to(torch.float16).cuda()
    out = K.chunk_attention(params, q, cu_q, kp, vp, bt, sl, int(sl.max().item()), kt, vt)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    cu = cu_q.cpu().numpy()
    rows = set(rng.choice(total_q, size=min(24, total_q), replace=False).tolist())
    for b in range(B):                       # first and last rows of every chunk
        rows |= {int(cu[b]), int(cu[b + 1]) - 1}
    ref = _reference_rows(q, cu_q, kp, vp, bt, kt, vt, sl, G, sorted(rows))
    o = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for (r, hq), want in ref.items():
        worst = max(worst, T.assert_rows_close(o[r, hq], want, f"row {r} head {hq}"))
    say(f"{len(ref)} rows, max rel err {worst:.3e}")
