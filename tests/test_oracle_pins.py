"""Pins of the CPU oracle to things other than itself (closed forms, invariants, library
routines, brute force, hand-derived byte patterns). CPU only."""
import json
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import kvarn_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _balanced_signs(rng, n=128):
    v = np.array([1.0] * (n // 2) + [-1.0] * (n // 2))
    rng.shuffle(v)
    return v


# ----------------------------------------------------------------------------- Hadamard


def test_hadamard_matches_library():
    assert np.array_equal(O.hadamard(128), scipy.linalg.hadamard(128) / np.sqrt(128))
    for n in (1, 2, 4, 16, 64):
        assert np.allclose(O.hadamard(n), scipy.linalg.hadamard(n) / np.sqrt(n), atol=0, rtol=0)


def test_hadamard_orthonormal_symmetric():
    h = O.hadamard(128)
    assert np.abs(h @ h.T - np.eye(128)).max() < 1e-12
    assert np.array_equal(h, h.T)


def test_rotation_preserves_scores():
    # README "How KVarN works" stage 2: the rotation is orthonormal so q.k is preserved.
    q, k = RNG.standard_normal(128), RNG.standard_normal((128, 50))
    h = O.hadamard(128)
    assert np.allclose((h @ q) @ (h @ k), q @ k, rtol=1e-12, atol=1e-12)
    x = RNG.standard_normal((3, 128, 128))
    assert np.allclose(O.rotate(x), np.einsum("ij,bjt->bit", scipy.linalg.hadamard(128) / np.sqrt(128), x))


# ----------------------------------------------------------------------------- Sinkhorn


@pytest.mark.parametrize("n_iters", [1, 2, 8])
def test_sinkhorn_closed_form_rank_one(n_iters):
    """X = diag(a) u w^T diag(b), u and w balanced +-1: after one column step s = sigma_a b,
    after one row step r = a / sigma_a with sigma_a = population std of a*u; later
    iterations change nothing (the normalized tile u w^T already has unit stds)."""
    rng = np.random.default_rng(7)
    a = rng.uniform(0.2, 5.0, 128)
    b = rng.uniform(0.2, 5.0, 128)
    u, w = _balanced_signs(rng), _balanced_signs(rng)
    xr = a[:, None] * np.outer(u, w) * b[None, :]
    sig_a = np.sqrt(np.mean((a * u) ** 2) - np.mean(a * u) ** 2)
    la, lb = O.sinkhorn_log(xr, n_iters)
    assert np.allclose(np.exp(lb), sig_a * b, rtol=1e-12)
    assert np.allclose(np.exp(la), a / sig_a, rtol=1e-12)


def test_sinkhorn_fixed_point_is_identity():
    rng = np.random.default_rng(8)
    y = np.outer(_balanced_signs(rng), _balanced_signs(rng))
    la, lb = O.sinkhorn_log(y, 8)
    assert np.array_equal(la, np.zeros(128)) and np.array_equal(lb, np.zeros(128))


@pytest.mark.parametrize("n_iters", [1, 3, 8])
def test_sinkhorn_last_row_step_gives_unit_row_std(n_iters):
    xr = O.rotate(RNG.standard_normal((4, 128, 128)) * RNG.lognormal(0, 1.5, (4, 128, 1)))
    la, lb = O.sinkhorn_log(xr, n_iters)
    y = xr * np.exp(-la)[..., :, None] * np.exp(-lb)[..., None, :]
    assert np.allclose(y.std(axis=-1), 1.0, rtol=1e-10)


def test_sinkhorn_converges_on_average():
    first, last = [], []
    for seed in range(6):
        rng = np.random.default_rng(100 + seed)
        x = rng.standard_t(3, (128, 128)) * rng.lognormal(0, 1.0, (128, 1)) * rng.lognormal(0, 1.0, (1, 128))
        hist = []
        O.sinkhorn_log(O.rotate(x), 8, history=hist)
        first.append(hist[1])
        last.append(hist[-1])
    assert np.mean(last) < np.mean(first)


def test_sinkhorn_zero_tile_is_skipped():
    la, lb = O.sinkhorn_log(np.zeros((128, 128)), 8)
    assert not la.any() and not lb.any()


def test_scale_by_power_of_two_moves_only_token_normalizer():
    x = RNG.standard_normal((128, 128)).astype(np.float16)
    a = O.quantize_tiles(x, O.KIND_K, 8)
    b = O.quantize_tiles((x.astype(np.float64) * 4.0).astype(np.float16), O.KIND_K, 8)
    assert np.array_equal(a["r"], b["r"])
    assert np.array_equal(a["s"].astype(np.float64) * 4.0, b["s"].astype(np.float64))
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["scale"], b["scale"]) and np.array_equal(a["zero"], b["zero"])


def test_token_permutation_equivariance():
    x = RNG.standard_normal((128, 128)).astype(np.float16)
    perm = RNG.permutation(128)
    for kind in (O.KIND_K, O.KIND_V):
        a = O.quantize_tiles(x, kind, 4)
        b = O.quantize_tiles(x[:, perm], kind, 4)
        assert np.array_equal(a["s"][perm], b["s"])
        assert np.array_equal(a["codes"][:, perm], b["codes"])
        assert np.allclose(a["r"].astype(float), b["r"].astype(float), rtol=2e-3)


def test_zero_iterations_is_plain_rotated_rtn():
    x = RNG.standard_normal((128, 128)).astype(np.float16)
    out = O.quantize_tiles(x, O.KIND_K, 0)
    assert np.all(out["r"] == 1) and np.all(out["s"] == 1)
    xr = scipy.linalg.hadamard(128) @ x.astype(np.float64) / np.sqrt(128)
    # per-channel min / max of the rotated tile are the zero point and range
    assert np.array_equal(out["zero"], xr.min(axis=1).astype(np.float16))
    assert np.array_equal(out["scale"], ((xr.max(axis=1) - xr.min(axis=1)) / 15).astype(np.float16))


# ----------------------------------------------------------------------------- RTN


@pytest.mark.parametrize("kind,bits", [(O.KIND_K, 4), (O.KIND_V, 2)])
def test_rtn_code_range_and_extremes(kind, bits):
    qmax = (1 << bits) - 1
    x = (RNG.standard_t(3, (6, 128, 128)) * 3).astype(np.float16)
    out = O.quantize_tiles(x, kind, 8)
    codes = out["codes"]
    assert codes.min() >= 0 and codes.max() <= qmax
    axis = -1 if kind == O.KIND_K else -2
    assert np.all(codes.min(axis=axis) == 0)
    assert np.all(codes.max(axis=axis) == qmax)


@pytest.mark.parametrize("kind,bits", [(O.KIND_K, 4), (O.KIND_V, 2)])
def test_rtn_error_bound(kind, bits):
    qmax = (1 << bits) - 1
    y = RNG.standard_normal((128, 128)) * RNG.lognormal(0, 1, (128, 1))
    axis = -1 if kind == O.KIND_K else -2
    codes, sc16, zr16, _ = O.rtn_asym(y, bits, axis)
    mn, mx = y.min(axis=axis), y.max(axis=axis)
    sc, zr = sc16.astype(np.float64), zr16.astype(np.float64)
    exp_ = (lambda v: v[:, None]) if kind == O.KIND_K else (lambda v: v[None, :])
    yhat = exp_(zr) + exp_(sc) * codes
    bound = exp_(sc) / 2 + np.abs(exp_(mn) - exp_(zr)) + qmax * np.abs(exp_((mx - mn) / qmax) - exp_(sc))
    assert np.all(np.abs(y - yhat) <= bound * (1 + 1e-12))


def test_rtn_groups_follow_kind():
    """K groups are channel rows, V groups are token columns (README stage 4)."""
    y = np.add.outer(np.arange(128.0), np.zeros(128)) + RNG.uniform(0, 1, (128, 128))
    _, sk, zk, _ = O.rtn_asym(y, 4, axis=-1)
    assert np.array_equal(zk, y.min(axis=1).astype(np.float16))
    _, sv, zv, _ = O.rtn_asym(y, 2, axis=-2)
    assert np.array_equal(zv, y.min(axis=0).astype(np.float16))


def test_rtn_exact_on_grid_and_constant_group():
    z, s = np.float16(-1.25), np.float16(0.125)
    k = RNG.integers(0, 16, (128, 128))
    k[:, 0], k[:, 1] = 0, 15
    y = float(z) + float(s) * k
    codes, sc, zr, _ = O.rtn_asym(y, 4, axis=-1)
    assert np.all(sc == s) and np.all(zr == z) and np.array_equal(codes, k)
    codes, sc, zr, _ = O.rtn_asym(np.full((128, 128), 3.0), 4, axis=-1)
    assert np.all(sc == 0) and np.all(codes == 0) and np.all(zr == 3.0)


def test_constant_and_zero_tiles():
    """A zero tile skips every normalizer update and codes to 0. A constant tile rotates
    into a single non-zero channel (row 0 of H X); it reconstructs to float16 accuracy."""
    for val in (0.0, 2.5):
        x = np.full((128, 128), val, dtype=np.float16)
        for kind in (O.KIND_K, O.KIND_V):
            out = O.quantize_tiles(x, kind, 8)
            if val == 0.0:
                assert np.all(out["codes"] == 0) and np.all(out["r"] == 1) and np.all(out["s"] == 1)
            else:
                assert np.all(out["codes"][1:] == 0)
            xh = O.dequantize_tiles(out["codes"], out["r"], out["s"], out["scale"], out["zero"], kind)
            assert np.allclose(xh, x.astype(np.float64), atol=3e-3 * max(val, 1))


def test_lossless_bookkeeping_reconstructs_input():
    """Without RTN, H (r s^T * Y) reproduces X exactly: pins the rotation and normalizers."""
    x = (RNG.standard_normal((128, 128)) * RNG.lognormal(0, 1, (128, 1))).astype(np.float16)
    out = O.quantize_tiles(x, O.KIND_K, 8, lossless=True)
    r, s = out["r"].astype(np.float64), out["s"].astype(np.float64)
    xh = O.hadamard() @ (r[:, None] * s[None, :] * out["y"])
    assert np.allclose(xh, x.astype(np.float64), rtol=0, atol=1e-12 * float(np.abs(x).max()))


def test_quantization_error_improves_over_plain_rtn():
    """Rotation + normalization lower the reconstruction error vs. RTN on the raw tile with
    outlier channels (README intro and stage 2/3: outliers spread, variance equalized)."""
    x = RNG.standard_normal((128, 128))
    x[RNG.choice(128, 4, replace=False), :] *= 20
    x16 = x.astype(np.float16)
    out = O.quantize_tiles(x16, O.KIND_K, 8)
    xh = O.dequantize_tiles(out["codes"], out["r"], out["s"], out["scale"], out["zero"], O.KIND_K)
    codes, sc, zr, _ = O.rtn_asym(x16.astype(np.float64), 4, axis=-1)
    plain = zr.astype(float)[:, None] + sc.astype(float)[:, None] * codes
    e_kvarn = np.linalg.norm(xh - x16)
    e_plain = np.linalg.norm(plain - x16)
    assert e_kvarn < e_plain


# ----------------------------------------------------------------------------- format


def _gold():
    with open(os.path.join(GOLD, "format_patterns.json")) as f:
        return json.load(f)


def _meta():
    return (np.full(128, 1.0, np.float16), np.full(128, 2.0, np.float16),
            np.full(128, 0.5, np.float16), np.full(128, -1.0, np.float16))


def _words(rec, n):
    return np.frombuffer(rec[:n], dtype="<u4")


def test_k_format_golden_patterns():
    g = _gold()
    c, t = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    w = _words(O.pack_k_record(c % 16, *_meta()), 8192).reshape(128, 16)
    assert np.all(w[:, 0::2] == int(g["k_codes_c_mod_16"]["word_even"], 16))
    assert np.all(w[:, 1::2] == int(g["k_codes_c_mod_16"]["word_odd"], 16))
    w = _words(O.pack_k_record(t % 16, *_meta()), 8192).reshape(128, 16)
    assert np.all(w == (np.arange(128)[:, None] % 16) * 0x11111111)
    rec = O.pack_k_record(t % 16, *_meta())
    m = g["metadata"]
    for i, key in enumerate(("r_bytes", "s_bytes", "scale_bytes", "zero_bytes")):
        seg = rec[8192 + 256 * i: 8192 + 256 * (i + 1)]
        assert seg == bytes.fromhex(m[key]) * 128


def test_v_format_golden_patterns():
    g = _gold()
    c, t = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    w = _words(O.pack_v_record(c % 4, *_meta()), 4096).reshape(128, 4, 2)
    assert np.all(w == (np.arange(128)[:, None, None] % 4) * 0x55555555)
    w = _words(O.pack_v_record(t // 32, *_meta()), 4096).reshape(128, 4, 2)
    assert np.all(w[:, :, 0] == int(g["v_codes_t_div_32"]["word_d0"], 16))
    assert np.all(w[:, :, 1] == int(g["v_codes_t_div_32"]["word_d1"], 16))
    w = _words(O.pack_v_record((t // 4) % 4, *_meta()), 4096).reshape(128, 4, 2)
    assert np.all(w == np.arange(4)[None, :, None] * 0x55555555)
    w = _words(O.pack_v_record(t % 4, *_meta()), 4096)
    assert np.all(w == int(g["v_codes_t_mod_4"]["word"], 16))
    rec = O.pack_v_record(t % 4, *_meta())
    assert rec[4096:4096 + 256] == bytes.fromhex(g["metadata"]["r_bytes"]) * 128
    assert rec[4096 + 768:] == bytes.fromhex(g["metadata"]["zero_bytes"]) * 128


def test_k2_format_byte_patterns():
    """2-bit key records: every bit of the crumb -> channel map against hand-derived words."""
    with open(os.path.join(GOLD, "format_k2_patterns.json")) as f:
        g = json.load(f)
    c = np.arange(128)[:, None] * np.ones((1, 128), dtype=np.int64)
    t = np.ones((128, 1), dtype=np.int64) * np.arange(128)[None, :]

    def words(codes):
        rec = O.pack_k2_record(codes.astype(np.uint8), *_meta())
        assert len(rec) == O.K2_RECORD_BYTES
        return np.frombuffer(rec[:4096], dtype="<u4").reshape(128, 4, 2)     # [t, g, d]

    assert np.all(words(c % 4) == int(g["k2_codes_c_mod_4"]["word"], 16))
    assert np.all(words((c // 4) % 2) == int(g["k2_codes_c_bit2"]["word"], 16))
    w = words((c // 8) % 4)
    assert np.all(w[:, :, 0] == int(g["k2_codes_c_div_8_mod_4"]["word_d0"], 16))
    assert np.all(w[:, :, 1] == int(g["k2_codes_c_div_8_mod_4"]["word_d1"], 16))
    w = words(c // 32)
    for gg in range(4):
        assert np.all(w[:, gg, :] == int(g["k2_codes_c_div_32"]["word_g"][gg], 16))
    w = words(t % 4)
    for tt in range(128):
        assert np.all(w[tt] == int(g["k2_codes_t_mod_4"]["word_t"][tt % 4], 16))


def test_v4_format_byte_patterns():
    """4-bit value records: every bit of the nibble -> token map against hand-derived words."""
    with open(os.path.join(GOLD, "format_v4_patterns.json")) as f:
        g = json.load(f)
    t = np.ones((128, 1), dtype=np.int64) * np.arange(128)[None, :]

    def words(codes):
        rec = O.pack_v4_record(codes.astype(np.uint8), *_meta())
        assert len(rec) == O.V4_RECORD_BYTES
        return np.frombuffer(rec[:8192], dtype="<u4").reshape(128, 4, 4)     # [c, g, m]

    assert np.all(words(t % 4) == int(g["v4_codes_t_mod_4"]["word"], 16))
    assert np.all(words((t // 16) % 2) == int(g["v4_codes_t_bit4"]["word"], 16))
    w = words((t // 4) % 4)
    for gg in range(4):
        assert np.all(w[:, gg, :] == int(g["v4_codes_t_div_4_mod_4"]["word_g"][gg], 16))
    w = words(t // 32)
    for m in range(4):
        assert np.all(w[:, :, m] == int(g["v4_codes_t_div_32"]["word_m"][m], 16))


def test_v4_nibble_map_is_a_permutation():
    toks = sorted(O.v4_nibble_token(g, m, q) for g in range(4) for m in range(4) for q in range(8))
    assert toks == list(range(128))


def test_k2_crumb_map_is_a_permutation():
    chans = sorted(O.k2_crumb_channel(g, d, p) for g in range(4) for d in range(2) for p in range(16))
    assert chans == list(range(128))


def test_pack_unpack_roundtrip():
    for bits, pack, unpack, size in ((4, O.pack_k_record, O.unpack_k_record, 9216),
                                     (2, O.pack_k2_record, O.unpack_k2_record, 5120),
                                     (4, O.pack_v4_record, O.unpack_v4_record, 9216),
                                     (2, O.pack_v_record, O.unpack_v_record, 5120)):
        codes = RNG.integers(0, 1 << bits, (128, 128)).astype(np.uint8)
        meta = [RNG.standard_normal(128).astype(np.float16) for _ in range(4)]
        rec = pack(codes, *meta)
        assert len(rec) == size
        d = unpack(rec)
        assert np.array_equal(d["codes"], codes)
        for key, m in zip(("r", "s", "scale", "zero"), meta):
            assert np.array_equal(d[key], m)


def test_v_crumb_map_is_a_permutation():
    toks = sorted(O.v_crumb_token(g, d, p) for g in range(4) for d in range(2) for p in range(16))
    assert toks == list(range(128))


def test_capacity_within_claimed_range():
    # README intro: 3-5x KV capacity vs FP16; format v1 stores K+V in 14336 B per 128 tokens.
    ratio = 2 * 128 * 128 * 2 / (O.K_RECORD_BYTES + O.V_RECORD_BYTES)
    assert 3.0 <= ratio <= 5.0


# ----------------------------------------------------------------------------- attention


def test_attention_matches_sdpa():
    q = RNG.standard_normal(128)
    k = RNG.standard_normal((300, 128))
    v = RNG.standard_normal((300, 128))
    sm = 1 / np.sqrt(128)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None], torch.tensor(k)[None, None], torch.tensor(v)[None, None],
        scale=sm)[0, 0, 0].numpy()
    assert np.allclose(O.attention(q, k, v, sm), ref, rtol=1e-12, atol=1e-13)


def test_split_merge_equals_single_pass():
    q = RNG.standard_normal(128)
    k = RNG.standard_normal((1000, 128)) * 3
    v = RNG.standard_normal((1000, 128))
    sm = 1 / np.sqrt(128)
    cuts = [0, 1, 128, 129, 500, 999, 1000]
    parts = [O.partial_attention(q, k[a:b], v[a:b], sm) for a, b in zip(cuts[:-1], cuts[1:])]
    m, l, acc = (np.array([p[i] for p in parts]) for i in range(3))
    assert np.allclose(O.merge_partials(m, l, acc), O.attention(q, k, v, sm), rtol=1e-12, atol=1e-13)


def _quantize_pages(xk, xv, n_iters=8):
    """xk, xv [n_pages, 128 tok, 128 ch] float16 -> lists of records."""
    kp, vp = [], []
    for i in range(xk.shape[0]):
        a = O.quantize_tiles(xk[i].T, O.KIND_K, n_iters)
        kp.append(O.pack_k_record(a["codes"], a["r"], a["s"], a["scale"], a["zero"]))
        b = O.quantize_tiles(xv[i].T, O.KIND_V, n_iters)
        vp.append(O.pack_v_record(b["codes"], b["r"], b["s"], b["scale"], b["zero"]))
    return kp, vp


def test_decode_row_equals_sdpa_on_dequantized_cache_with_gqa():
    """One sequence, 2 KV heads, 8 query heads (GQA 4): the oracle decode equals SDPA with
    repeat_interleave on the dequantized keys/values (+ raw fp16 tail)."""
    hkv, hq, pages, tail = 2, 8, 2, 37
    xk = RNG.standard_normal((hkv, pages, 128, 128)).astype(np.float16)
    xv = RNG.standard_normal((hkv, pages, 128, 128)).astype(np.float16)
    tk = RNG.standard_normal((hkv, tail, 128)).astype(np.float16)
    tv = RNG.standard_normal((hkv, tail, 128)).astype(np.float16)
    q = RNG.standard_normal((hq, 128)).astype(np.float16)
    recs = [_quantize_pages(xk[h], xv[h]) for h in range(hkv)]
    kfull = np.stack([np.concatenate([O.dequantize_k_record(r) for r in recs[h][0]] + [tk[h].astype(float)]) for h in range(hkv)])
    vfull = np.stack([np.concatenate([O.dequantize_v_record(r) for r in recs[h][1]] + [tv[h].astype(float)]) for h in range(hkv)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q.astype(float))[None, :, None],
        torch.tensor(kfull).repeat_interleave(hq // hkv, 0)[None],
        torch.tensor(vfull).repeat_interleave(hq // hkv, 0)[None], scale=1 / np.sqrt(128))[0, :, 0].numpy()
    for h in range(hq):
        g = h // (hq // hkv)
        o = O.decode_attention_row(q[h], recs[g][0], recs[g][1], tk[g], tv[g])
        assert np.allclose(o, ref[h], rtol=1e-11, atol=1e-12)


def test_rotated_space_decode_identity():
    """The read path's algebra: with q_rot = H q, per tile q'' = q_rot*r*scale (keys), the
    score is s_t (q''.code_t + q_rot.(r*zero)); values accumulate r * (sum_t p_t s_t
    (scale_t code_t + zero_t)); the output is H^T acc / l. Equal to dequantize-then-attend."""
    xk = RNG.standard_normal((3, 128, 128)).astype(np.float16)
    xv = RNG.standard_normal((3, 128, 128)).astype(np.float16)
    kp, vp = _quantize_pages(xk, xv)
    q = RNG.standard_normal(128).astype(np.float16).astype(np.float64)
    sm = 1 / np.sqrt(128)
    h = O.hadamard()
    q_rot = h @ q
    scores, contrib = [], []
    for kr, vr in zip(kp, vp):
        dk, dv = O.unpack_k_record(kr), O.unpack_v_record(vr)
        r, s, sc, zr = (dk[k_].astype(np.float64) for k_ in ("r", "s", "scale", "zero"))
        qpp = q_rot * r * sc
        scores.append(sm * s * (qpp @ dk["codes"] + q_rot @ (r * zr)))
        contrib.append(dv)
    z = np.concatenate(scores)
    p = np.exp(z - z.max())
    acc = np.zeros(128)
    for i, dv in enumerate(contrib):
        pt = p[128 * i: 128 * (i + 1)]
        r, s, sc, zr = (dv[k_].astype(np.float64) for k_ in ("r", "s", "scale", "zero"))
        acc += r * (dv["codes"] @ (pt * s * sc) + np.sum(pt * s * zr))
    o = h.T @ acc / p.sum()
    ref = O.decode_attention_row(q.astype(np.float16), kp, vp)
    assert np.allclose(o, ref, rtol=1e-11, atol=1e-12)


def test_quantized_attention_close_to_fp16_attention():
    """End-to-end sanity on a single tile: attention over the quantized cache stays close to
    exact attention (the method's accuracy claim, README intro; loose bound)."""
    xk = RNG.standard_normal((1, 128, 128)).astype(np.float16)
    xv = RNG.standard_normal((1, 128, 128)).astype(np.float16)
    kp, vp = _quantize_pages(xk, xv)
    q = RNG.standard_normal(128).astype(np.float16)
    exact = O.attention(q.astype(float), xk[0].astype(float), xv[0].astype(float), 1 / np.sqrt(128))
    approx = O.decode_attention_row(q, kp, vp)
    assert np.linalg.norm(approx - exact) < 0.5 * np.linalg.norm(exact) + 0.1


def test_population_std_is_exactly_zero_for_identical_values():
    """The std of identical values is 0 by definition, whatever the library's summation
    order; 0.1 (inexact in binary) repeated along either axis is the hard case."""
    y = np.full((128, 128), 0.1) * RNG.uniform(0.5, 2.0, (128, 1))
    assert np.all(O.population_std(y, axis=-1) == 0.0)
    assert np.all(O.population_std(y.T, axis=-2) == 0.0)
    z = RNG.standard_normal((128, 128))
    assert np.allclose(O.population_std(z, axis=-1), np.sqrt(np.mean((z - z.mean(-1, keepdims=True)) ** 2, -1)), rtol=1e-13)


# ----------------------------------------------------------------------------- rounding, clips


def test_rtn_rounds_half_to_even():
    """Values exactly on half-levels (scale 1, zero 0 exactly representable) round to the even
    code: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, ... (round-half-even; half-up would give 1, 2, 3 ...)."""
    half = np.arange(15) + 0.5
    row = np.concatenate([[0.0, 15.0], half, np.full(128 - 17, 7.0)])
    y = np.tile(row, (128, 1))                       # key groups = rows
    codes, sc, zr, u = O.rtn_asym(y, 4, axis=-1)
    assert np.all(sc == 1.0) and np.all(zr == 0.0)
    assert np.array_equal(u[0, 2:17], half)          # exact ties
    assert codes[0, 2:17].tolist() == [0, 2, 2, 4, 4, 6, 6, 8, 8, 10, 10, 12, 12, 14, 14]
    # 2-bit value groups (columns): scale 1 with the range [0, 3]
    col = np.concatenate([[0.0, 3.0, 0.5, 1.5, 2.5], np.full(123, 1.0)])
    codes, sc, zr, _ = O.rtn_asym(np.tile(col[:, None], (1, 128)), 2, axis=-2)
    assert np.all(sc == 1.0) and codes[2:5, 0].tolist() == [0, 2, 2]


def test_store_normalizer_clip_bounds():
    """Normalizers are clipped to the float16 normal range [2^-14, 65504], then rounded."""
    v = np.array([1e-9, 2.0 ** -14, 2.0 ** -14 * 0.75, 3.0, 65504.0, 65519.0, 1e6, 1e30])
    got = O.store_normalizer(np.log(v)).astype(np.float64)
    assert got.tolist() == [2.0 ** -14, 2.0 ** -14, 2.0 ** -14, 3.0, 65504.0, 65504.0, 65504.0,
                            65504.0]
    # driven past the lower bound by a real tile: tiny values leave every token std below
    # 2^-14, so s is stored at the bound and the codes still cover each group's range
    x = (RNG.standard_normal((128, 128)) * 2.0 ** -20).astype(np.float16)
    for kind in (O.KIND_K, O.KIND_V):
        out = O.quantize_tiles(x, kind, 8)
        assert np.all(out["s"] == np.float16(2.0 ** -14))
        axis = -1 if kind == O.KIND_K else -2
        assert np.all(out["codes"].max(axis=axis) == (15 if kind == O.KIND_K else 3))


def test_store_meta_saturates():
    """Scales and zeros round to float16 nearest-even and saturate to +-65504 (no inf)."""
    v = np.array([-1e9, -65520.0, -65504.0, -0.1, 0.0, 1.0 / 3, 65519.0, 65520.0, 2e5])
    got = O.store_meta(v).astype(np.float64)
    assert got.tolist() == [-65504.0, -65504.0, -65504.0, float(np.float16(-0.1)), 0.0,
                            float(np.float16(1.0 / 3)), 65504.0, 65504.0, 65504.0]


def test_overflowing_group_gives_finite_record_and_decode():
    """A near-constant tile (5 + 1e-3 noise) at one iteration: the rotated DC channel's
    normalized values reach ~1.9e5, beyond float16. Its zero saturates to 65504 and its codes
    clip at 15, so the record stays finite and a decode over it returns finite output."""
    rng = np.random.default_rng(7)
    x = (5 + 1e-3 * rng.standard_normal((128, 128))).astype(np.float16)
    out = O.quantize_tiles(x, O.KIND_K, 1)
    assert np.abs(out["y"]).max() > 65504
    for key in ("r", "s", "scale", "zero"):
        assert np.all(np.isfinite(out[key].astype(np.float64)))
    assert out["zero"][0] == np.float16(65504) and np.all(out["codes"][0] == 15)
    rec_k = O.pack_k_record(out["codes"], out["r"], out["s"], out["scale"], out["zero"])
    vo = O.quantize_tiles(x, O.KIND_V, 1)
    rec_v = O.pack_v_record(vo["codes"], vo["r"], vo["s"], vo["scale"], vo["zero"])
    o = O.decode_attention_row(rng.standard_normal(128).astype(np.float16), [rec_k], [rec_v])
    assert np.all(np.isfinite(o))


def test_causal_attention_matches_sdpa():
    """Causal rows against torch's scaled_dot_product_attention (float64) with a causal mask
    over the last n positions of the cache; a row before the cache start is zeros."""
    C, n = 300, 40
    q = RNG.standard_normal((n, 128))
    k = RNG.standard_normal((C, 128))
    v = RNG.standard_normal((C, 128))
    sm = 1 / np.sqrt(128)
    pos = np.arange(C - n, C)
    got = O.causal_attention(q, pos, k, v, sm)
    mask = torch.tensor(np.arange(C)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None], torch.tensor(k)[None, None], torch.tensor(v)[None, None],
        attn_mask=mask[None, None], scale=sm)[0, 0].numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)
    # square causal case (the chunk is the whole cache)
    got = O.causal_attention(q, np.arange(n), k[:n], v[:n], sm)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None], torch.tensor(k[:n])[None, None], torch.tensor(v[:n])[None, None],
        is_causal=True, scale=sm)[0, 0].numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert np.all(O.causal_attention(q[:2], [-1, -5], k, v, sm) == 0)


# ----------------------------------------------------------------------------- folded format


def test_folded_format_byte_patterns():
    """Format 2 metadata offsets and byte values, derived by hand (tests/golden)."""
    g = json.load(open(os.path.join(GOLD, "format_folded_patterns.json")))
    for case in g["cases"]:
        kind, kb, vb = case["kind"], case["k_bits"], case["v_bits"]
        bits = kb if kind == O.KIND_K else vb
        vec = {k: np.full(128, v, dtype=np.float16) for k, v in case["fill"].items()}
        for k, (i, v) in case["set"].items():
            vec[k][i] = v
        one = np.ones(128, dtype=np.float16)
        r16, s16 = (one, vec["first"]) if kind == O.KIND_K else (vec["first"], one)
        rec = O.pack_record(kind, np.zeros((128, 128), np.uint8), r16, s16, vec["scale"],
                            vec["zero"], kb, vb, fmt=2)
        assert len(rec) == case["record_bytes"] == O.record_bytes(kind, kb, vb, 2)
        assert O.record_layout(len(rec)) == (bits, 2)
        for off, lo, hi in case["bytes"]:
            assert (rec[off], rec[off + 1]) == (lo, hi), (case["kind"], off)


@pytest.mark.parametrize("kind,kb,vb", [(O.KIND_K, 4, 2), (O.KIND_V, 4, 2), (O.KIND_K, 2, 2),
                                        (O.KIND_V, 4, 4)])
def test_folded_format_roundtrip_and_fold_identity(kind, kb, vb):
    """Format 2 packs and unpacks losslessly (the folded-away normalizer reads back as 1), and
    folding changes the codes only at rounding ties: asymmetric round-to-nearest is invariant
    to a positive factor per group, so the folded codes equal the separate-format codes up
    to the float16 rounding of the folded scale and zero, and both reconstruct the tile with
    the same accuracy."""
    x = (RNG.standard_t(4, (8, 128, 128)) * RNG.lognormal(0, 1, (8, 128, 1))).astype(np.float16)
    a = O.quantize_tiles(x, kind, 8, k_bits=kb, v_bits=vb, fmt=1)
    b = O.quantize_tiles(x, kind, 8, k_bits=kb, v_bits=vb, fmt=2)
    gone = "r" if kind == O.KIND_K else "s"
    kept = "s" if kind == O.KIND_K else "r"
    assert np.all(b[gone] == 1) and np.array_equal(b[kept], a[kept])
    for i in range(x.shape[0]):
        rec = O.pack_record(kind, b["codes"][i], b["r"][i], b["s"][i], b["scale"][i],
                            b["zero"][i], kb, vb, fmt=2)
        d = O.unpack_record(rec, kind, kb, vb, fmt=2)
        for key in ("codes", "r", "s", "scale", "zero"):
            assert np.array_equal(d[key], b[key][i]), key
    diff = b["codes"].astype(int) - a["codes"].astype(int)
    assert np.abs(diff).max() <= 1 and np.count_nonzero(diff) <= 0.03 * diff.size
    # the differing codes sit at ties of the separate format: folded and separate scale and
    # zero differ by their float16 roundings (relative 2^-10 each), which moves the unrounded
    # code by at most 2^-10 (u + |zero| / scale)
    frac = np.abs(a["u"] - np.floor(a["u"]) - 0.5)
    grp = (lambda v: v[..., :, None]) if kind == O.KIND_K else (lambda v: v[..., None, :])
    with np.errstate(divide="ignore", invalid="ignore"):
        zs = np.abs(grp(a["zero"].astype(float))) / grp(a["scale"].astype(float))
    bound = 2.0 ** -10 * (np.abs(a["u"]) + np.broadcast_to(zs, a["u"].shape) + 1)
    assert np.all(frac[diff != 0] <= bound[diff != 0])
    ea = np.linalg.norm(O.dequantize_tiles(a["codes"], a["r"], a["s"], a["scale"], a["zero"], kind) - x)
    eb = np.linalg.norm(O.dequantize_tiles(b["codes"], b["r"], b["s"], b["scale"], b["zero"], kind) - x)
    assert abs(eb - ea) <= 0.02 * ea


# ----------------------------------------------------------------------------- group size 64


G64_PRESETS = [(O.KIND_K, 4, 2), (O.KIND_V, 4, 2), (O.KIND_K, 2, 2), (O.KIND_V, 4, 4)]


def test_g64_metadata_byte_patterns():
    """Group-64 metadata: vector order, offsets and float16 bit patterns derived by hand
    (tests/golden/format_g64_patterns.json), every preset width and both formats."""
    g = json.load(open(os.path.join(GOLD, "format_g64_patterns.json")))
    val = g["values"]
    r16, s16 = np.full(128, val["r"], np.float16), np.full(128, val["s"], np.float16)
    sc = np.stack([np.full(128, val["scale0"]), np.full(128, val["scale1"])]).astype(np.float16)
    zr = np.stack([np.full(128, val["zero0"]), np.full(128, val["zero1"])]).astype(np.float16)
    for case in g["cases"]:
        kind = O.KIND_K if case["kind"] == "K" else O.KIND_V
        kb, vb, fmt = case["k_bits"], case["v_bits"], case["fmt"]
        one = np.ones(128, np.float16)
        rr, ss = (r16, s16) if fmt == 1 else ((one, s16) if kind == O.KIND_K else (r16, one))
        rec = O.pack_record(kind, np.zeros((128, 128), np.uint8), rr, ss, sc, zr, kb, vb,
                            fmt=fmt, group=64)
        assert len(rec) == case["record_bytes"] == O.record_bytes(kind, kb, vb, fmt, 64)
        bits = kb if kind == O.KIND_K else vb
        assert O.record_layout(len(rec)) == (bits, fmt) and O.record_group(len(rec)) == 64
        meta = rec[case["code_bytes"]:]
        assert len(meta) == 256 * len(case["vectors"])
        for off, name, hexpat in case["vectors"]:
            word = int(hexpat, 16)
            want = bytes([word & 0xFF, word >> 8]) * 128
            assert meta[off:off + 256] == want, (case["kind"], fmt, name)


def test_g64_record_sizes_are_distinct():
    """Every (code width, format, group) record size is distinct, so a pool's record size
    names its layout: 4-bit 9216 / 8960 / 9728 / 9472, 2-bit 5120 / 4864 / 5632 / 5376."""
    sizes = {}
    for bits in (4, 2):
        for fmt in (1, 2):
            for grp in (128, 64):
                n = O.record_bytes(O.KIND_K, bits, 2, fmt, grp)
                assert n not in sizes
                sizes[n] = (bits, fmt, grp)
                assert O.record_layout(n) == (bits, fmt) and O.record_group(n) == grp
    assert sorted(sizes) == [4864, 5120, 5376, 5632, 8960, 9216, 9472, 9728]


@pytest.mark.parametrize("kind", [O.KIND_K, O.KIND_V])
def test_g64_dequantize_hand_values(kind):
    """Dequantization with two groups, values computed by hand: codes 1, r = 1, s = 2,
    scale 0.5 / 0.25 and zero -1 / -2 for halves 0 / 1, no rotation: x = r s (zero + scale)
    = 2 (-1 + 0.5) = -1 in half 0 and 2 (-2 + 0.25) = -3.5 in half 1 (tokens 64.. of every key
    channel; channels 64.. of every value token)."""
    codes = np.ones((128, 128), np.uint8)
    sc = np.stack([np.full(128, 0.5), np.full(128, 0.25)]).astype(np.float16)
    zr = np.stack([np.full(128, -1.0), np.full(128, -2.0)]).astype(np.float16)
    x = O.dequantize_tiles(codes, np.ones(128, np.float16), np.full(128, 2.0, np.float16), sc, zr,
                           kind, rotate_channels=False, group=64)       # [c, t]
    if kind == O.KIND_K:
        assert np.all(x[:, :64] == -1.0) and np.all(x[:, 64:] == -3.5)
    else:
        assert np.all(x[:64, :] == -1.0) and np.all(x[64:, :] == -3.5)


@pytest.mark.parametrize("axis", [-1, -2])
def test_g64_reduces_to_g128_when_halves_share_extremes(axis):
    """A special case that reduces to the 128-element groups: when each half of a group holds
    the group's minimum and its maximum, both halves get the full group's scale and zero, and
    every code equals the 128-element code."""
    y = RNG.normal(size=(4, 128, 128))
    yt = np.moveaxis(y, axis, -1)            # the group axis last (a view)
    mn, mx = yt.min(-1), yt.max(-1)
    for half in (0, 64):
        yt[..., half] = mn - 1.0
        yt[..., half + 1] = mx + 1.0
    c1, s1, z1, _ = O.rtn_asym(y, 4, axis, group=128)
    c2, s2, z2, _ = O.rtn_asym(y, 4, axis, group=64)
    assert np.array_equal(c1, c2)
    assert s2.shape == (4, 2, 128) and np.array_equal(s2[:, 0], s1) and np.array_equal(s2[:, 1], s1)
    assert np.array_equal(z2[:, 0], z1) and np.array_equal(z2[:, 1], z1)


@pytest.mark.parametrize("kind", [O.KIND_K, O.KIND_V])
def test_g64_rtn_error_bound_per_half(kind):
    """Every element is reconstructed within half a step of its own half's scale (plus the
    float16 roundings of that half's scale and zero): the halves are cut here by slicing,
    not by the oracle's reshape, so a swapped or shifted half fails the bound."""
    y = RNG.standard_t(3, (3, 128, 128)) * RNG.lognormal(0, 1, (3, 1, 128))
    bits = 4 if kind == O.KIND_K else 2
    axis = -1 if kind == O.KIND_K else -2
    codes, sc, zr, _ = O.rtn_asym(y, bits, axis, group=64)
    qmax = (1 << bits) - 1
    for h in (0, 1):
        sl = slice(64 * h, 64 * h + 64)
        yh = y[..., :, sl] if kind == O.KIND_K else y[..., sl, :]
        ch = codes[..., :, sl] if kind == O.KIND_K else codes[..., sl, :]
        s_h = sc[:, h].astype(np.float64)
        z_h = zr[:, h].astype(np.float64)
        mn, mx = yh.min(axis), yh.max(axis)
        e = lambda v: v[..., :, None] if kind == O.KIND_K else v[..., None, :]
        err = np.abs(yh - (e(z_h) + e(s_h) * ch))
        bound = 0.5 * s_h + qmax * np.abs(s_h - (mx - mn) / qmax) + np.abs(z_h - mn) + 1e-12
        assert np.all(err <= e(bound)), h


def test_g64_half_assignment_through_the_pipeline():
    """A rotated tile with one large entry at rotated channel 3, token 5 (built as X = H E, so
    that H X = E; H is its own inverse): after normalization that entry still dominates its
    groups, so with group 64 the key channel 3 scale of half 0 (tokens 0..63) and the value
    token 5 scale of half 0 (channels 0..63) are several times the other half's."""
    e = RNG.normal(size=(128, 128))
    e[3, 5] = 60.0
    x = (O.hadamard(128) @ e).astype(np.float16)
    k = O.quantize_tiles(x, O.KIND_K, 8, group=64)
    v = O.quantize_tiles(x, O.KIND_V, 8, group=64)
    sk = k["scale"].astype(np.float64)
    sv = v["scale"].astype(np.float64)
    assert sk[0, 3] > 3 * sk[1, 3]
    assert sv[0, 5] > 3 * sv[1, 5]
    # elsewhere the halves are alike (both a draw of the same distribution)
    others = np.delete(np.arange(128), [3])
    assert np.median(sk[0, others] / sk[1, others]) == pytest.approx(1.0, rel=0.2)


@pytest.mark.parametrize("kind,kb,vb", G64_PRESETS)
@pytest.mark.parametrize("fmt", [1, 2])
def test_g64_roundtrip_and_finer_error(kind, kb, vb, fmt):
    """Group-64 records pack and unpack losslessly, and the finer groups do not reconstruct
    worse than 128-element groups (their range is a subset of the full group's)."""
    x = (RNG.standard_t(4, (6, 128, 128)) * RNG.lognormal(0, 1, (6, 128, 1))).astype(np.float16)
    a = O.quantize_tiles(x, kind, 8, k_bits=kb, v_bits=vb, fmt=fmt, group=128)
    b = O.quantize_tiles(x, kind, 8, k_bits=kb, v_bits=vb, fmt=fmt, group=64)
    assert b["scale"].shape == (6, 2, 128) and np.array_equal(b["r"], a["r"])
    for i in range(x.shape[0]):
        rec = O.pack_record(kind, b["codes"][i], b["r"][i], b["s"][i], b["scale"][i],
                            b["zero"][i], kb, vb, fmt=fmt, group=64)
        assert len(rec) == O.record_bytes(kind, kb, vb, fmt, 64)
        d = O.unpack_record(rec, kind, kb, vb, fmt=fmt, group=64)
        for key in ("codes", "r", "s", "scale", "zero"):
            assert np.array_equal(d[key], b[key][i]), key
    xa = O.dequantize_tiles(a["codes"], a["r"], a["s"], a["scale"], a["zero"], kind)
    xb = O.dequantize_tiles(b["codes"], b["r"], b["s"], b["scale"], b["zero"], kind, group=64)
    assert np.linalg.norm(xb - x) <= np.linalg.norm(xa - x)
