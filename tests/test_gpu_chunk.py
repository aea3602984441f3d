"""GPU tests of the multi-query read path (kvarn_chunk_attention): after a chunk write, every
query row of the chunk against the oracle's causal attention over exactly the positions it may
see (dequantized pages, a causally cut page read up to its limit, raw staging), and one query
per sequence equal to kvarn_decode_attention (bit for bit where both take the split layout)."""
import numpy as np
import pytest
import torch

from oracle import kvarn_oracle as O
from tests import kvarn_testlib as T
from tests.test_gpu_parity import _build_cache
from tests.test_gpu_write import _chunk, _extend_block_table

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(128.0)


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def say(*a):
    print(*a, flush=True)


def _written_cache(K, params, lens, lens_new, hkv, seed):
    spare = max(lens_new) // 128 + 2
    kp, vp, bt, kt, vt, sl, free = _build_cache(
        K, params, lens, hkv, seed=seed, spare=spare,
        width=max((L + n) // 128 for L, n in zip(lens, lens_new)) + 2)
    bt = _extend_block_table(bt, lens, lens_new, free)
    kn, vn, cu = _chunk(lens_new, hkv, seed=seed + 1)
    K.write_tokens(params, kn, vn, cu, sl, kt, vt, bt, kp, vp)
    sl2 = sl + torch.tensor(lens_new, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    return kp, vp, bt, kt, vt, sl2


def _reference_rows(q, cu_q, kp, vp, bt, kt, vt, sl, G, rows_to_check, scale=SCALE):
    """Oracle causal attention (O.causal_attention) of the given query rows: the cache of
    sequence b in position order is its dequantized pages followed by the staged tokens of
    its partial last tile; row cu_q[b] + i sits at position C - n + i."""
    qh = q.cpu().numpy()
    cu = cu_q.cpu().numpy()
    bt_h, sl_h = bt.cpu().numpy(), sl.cpu().numpy()
    kt_h, vt_h = kt.cpu().numpy(), vt.cpu().numpy()
    hkv = kp.shape[1]
    cache = {}
    out = {}
    for r in rows_to_check:
        b = int(np.searchsorted(cu, r, side="right") - 1)
        C, n = int(sl_h[b]), int(cu[b + 1] - cu[b])
        pos = C - n + (r - int(cu[b]))
        for g in range(hkv):
            if (b, g) not in cache:
                pages = [int(p) for p in bt_h[b, :C // 128]]
                fm = T.format_of(kp)
                gs = T.group_of(kp)
                ks = [O.dequantize_k_record(x, T.key_bits_of(kp), fm, gs) for x in T.records_of(kp, pages, g)]
                vs = [O.dequantize_v_record(x, T.value_bits_of(vp), fm, gs) for x in T.records_of(vp, pages, g)]
                ks.append(kt_h[b, g, :C % 128].astype(np.float64))
                vs.append(vt_h[b, g, :C % 128].astype(np.float64))
                cache[(b, g)] = (np.concatenate(ks, 0), np.concatenate(vs, 0))
            kk, vv = cache[(b, g)]
            hqs = [g * G + hh for hh in range(G)]
            res = O.causal_attention(qh[r, hqs].astype(np.float64), [pos] * G, kk, vv, scale)
            for hh, hq in enumerate(hqs):
                out[(r, hq)] = res[hh]
    return out


@pytest.mark.parametrize("factor", [40.0, 1e-3])
def test_chunk_softmax_extremes(K, factor):
    """The multi-query read at softmax scales 40x and 1e-3x of 1/sqrt(128) (nearly one-hot
    and nearly uniform causal attention), rows against the oracle."""
    scale = factor * SCALE
    lens, lens_new = [130, 0, 300], [140, 70, 100]
    hkv, G = 2, 8
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl = _written_cache(K, params, lens, lens_new, hkv, seed=170 + int(factor))
    total_q = sum(lens_new)
    cu_q = torch.tensor([0] + list(np.cumsum(lens_new)), dtype=torch.int32, device="cuda")
    q = torch.randn((total_q, hkv * G, 128), generator=torch.Generator().manual_seed(171))
    q = q.to(torch.float16).cuda()
    say(f"chunk attention softmax scale x{factor}: {total_q} query rows")
    out = K.chunk_attention(params, q, cu_q, kp, vp, bt, sl, int(sl.max().item()), kt, vt,
                            softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(172)
    cu = cu_q.cpu().numpy()
    rows = set(rng.choice(total_q, size=32, replace=False).tolist())
    for b in range(len(lens)):
        rows |= {int(cu[b]), int(cu[b + 1]) - 1}
    ref = _reference_rows(q, cu_q, kp, vp, bt, kt, vt, sl, G, sorted(rows), scale=scale)
    o = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for (r, hq), want in ref.items():
        worst = max(worst, T.assert_rows_close(o[r, hq], want, f"row {r} head {hq}"))
    say(f"{len(ref)} rows, max rel err {worst:.3e}")


@pytest.mark.parametrize("case", [0, 1])
def test_chunk_rows_against_oracle(K, case):
    lens, lens_new = [([0, 5, 200, 356], [300, 130, 56, 400]), ([127, 640], [1, 260])][case]
    hkv, G = 2, 8
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl = _written_cache(K, params, lens, lens_new, hkv, seed=140 + case)
    total_q = sum(lens_new)
    cu_q = torch.tensor([0] + list(np.cumsum(lens_new)), dtype=torch.int32, device="cuda")
    q = torch.randn((total_q, hkv * G, 128), generator=torch.Generator().manual_seed(150 + case))
    q = q.to(torch.float16).cuda()
    mx = int(sl.max().item())
    say(f"chunk attention: lens {lens} + chunks {lens_new}, {total_q} query rows")
    out = K.chunk_attention(params, q, cu_q, kp, vp, bt, sl, mx, kt, vt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(160 + case)
    cu = cu_q.cpu().numpy()
    rows = set(rng.choice(total_q, size=min(48, total_q), replace=False).tolist())
    for b in range(len(lens)):                       # first and last rows of every chunk
        rows |= {int(cu[b]), int(cu[b + 1]) - 1}
    ref = _reference_rows(q, cu_q, kp, vp, bt, kt, vt, sl, G, sorted(rows))
    o = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for (r, hq), want in ref.items():
        worst = max(worst, T.assert_rows_close(o[r, hq], want, f"row {r} head {hq}"))
    say(f"  {len(rows)} rows x {hkv * G} heads, max rel err {worst:.2e}")


def test_one_query_per_sequence_equals_decode(K):
    lens, lens_new = [40, 300, 1000, 128], [88, 212, 1, 200]
    hkv, G = 2, 8
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl = _written_cache(K, params, lens, lens_new, hkv, seed=170)
    q = torch.randn((len(lens), hkv * G, 128), generator=torch.Generator().manual_seed(171))
    q = q.to(torch.float16).cuda()
    mx = int(sl.max().item())
    cu_q = torch.arange(len(lens) + 1, dtype=torch.int32, device="cuda")
    a = K.chunk_attention(params, q, cu_q, kp, vp, bt, sl, mx, kt, vt)
    d = K.decode_attention(params, q, kp, vp, bt, sl, mx, kt, vt)
    d1 = K.decode_attention(params, q[:1].contiguous(), kp, vp, bt[:1].contiguous(), sl[:1], mx,
                            kt[:1].contiguous(), vt[:1].contiguous())
    torch.cuda.synchronize()
    # a single sequence takes the decode's split layout, as the chunk read does: bit for bit
    assert torch.equal(a[:1], d1)
    # several sequences take the balanced layout: the same sums in another float32 order
    af, df = a.float(), d.float()
    scale = df.abs().amax(dim=-1, keepdim=True)
    err = float(((af - df).abs() / scale).max())
    assert err <= 2e-3, err
    say(f"one query per sequence: chunk attention == decode attention (1 sequence bit for bit, "
        f"{len(lens)} sequences max rel diff {err:.1e})")


def test_queries_below_position_zero_get_zeros(K):
    """More query rows than cached tokens: rows at negative positions output zeros."""
    lens, lens_new = [0], [3]
    hkv, G = 1, 8
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl = _written_cache(K, params, lens, lens_new, hkv, seed=180)
    q = torch.randn((5, G, 128), generator=torch.Generator().manual_seed(181)).to(torch.float16).cuda()
    cu_q = torch.tensor([0, 5], dtype=torch.int32, device="cuda")
    out = K.chunk_attention(params, q, cu_q, kp, vp, bt, sl, 3, kt, vt)
    torch.cuda.synchronize()
    assert torch.all(out[:2] == 0)
    ref = _reference_rows(q, cu_q, kp, vp, bt, kt, vt, sl, G, [2, 3, 4])
    o = out.cpu().numpy().astype(np.float64)
    for (r, hq), want in ref.items():
        T.assert_rows_close(o[r, hq], want, f"row {r} head {hq}")


def test_reads_are_deterministic(K):
    """Decode and multi-query read give identical bytes when run twice (no atomics, fixed
    split and merge order)."""
    lens, lens_new = [300, 1000, 0], [50, 130, 9]
    hkv, G = 2, 8
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl = _written_cache(K, params, lens, lens_new, hkv, seed=190)
    mx = int(sl.max().item())
    total_q = sum(lens_new)
    cu_q = torch.tensor([0] + list(np.cumsum(lens_new)), dtype=torch.int32, device="cuda")
    q = torch.randn((total_q, hkv * G, 128), generator=torch.Generator().manual_seed(191)).to(torch.float16).cuda()
    a1 = K.chunk_attention(params, q, cu_q, kp, vp, bt, sl, mx, kt, vt)
    a2 = K.chunk_attention(params, q, cu_q, kp, vp, bt, sl, mx, kt, vt)
    qd = q[:len(lens)].contiguous()
    d1 = K.decode_attention(params, qd, kp, vp, bt, sl, mx, kt, vt)
    d2 = K.decode_attention(params, qd, kp, vp, bt, sl, mx, kt, vt)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(d1, d2)
