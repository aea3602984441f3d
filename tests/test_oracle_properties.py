"""Property tests of the oracle over randomly drawn tiles (hypothesis; CPU). Each draws the
preset, the kind, the iteration count, a distribution and a magnitude, and checks what the
pages and the mathematics fix for every input, not one worked case:

  * codes lie in [0, 2^b - 1] for the kind's width (README "How KVarN works", stage 4);
  * every stored code is the nearest level of the stored grid, up to the float16 rounding of
    the group's scale and zero (asymmetric round-to-nearest, stage 4);
  * the page record of every preset round-trips through pack and unpack;
  * a power-of-two scaling of the tile moves only the per-token normalizer by that factor
    (the normalization divides it out; stage 3), codes and grids unchanged;
  * a permutation of the tile's tokens permutes the codes and per-token normalizers.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import kvarn_oracle as O

PRESETS = [(4, 2), (2, 2), (4, 4)]


def _tile(seed: int, dist: str, mag: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((128, 128))
    elif dist == "t3":
        x = rng.standard_t(3, (128, 128))
    elif dist == "outlier_channels":
        x = rng.standard_normal((128, 128)) * np.exp(rng.standard_normal((128, 1)))
        x[rng.choice(128, 3, replace=False)] *= 20.0
    else:   # uneven token scales
        x = rng.standard_normal((128, 128)) * np.exp(rng.standard_normal((1, 128)))
    return (x * 2.0 ** mag).astype(np.float16)          # channels x tokens


tiles = st.builds(_tile, st.integers(0, 2**31 - 1),
                  st.sampled_from(["normal", "t3", "outlier_channels", "uneven_tokens"]),
                  st.integers(-6, 6))
kinds = st.sampled_from([O.KIND_K, O.KIND_V])
presets = st.sampled_from(PRESETS)
iters = st.sampled_from([0, 1, 2, 8])


def _bits(kind, preset):
    return preset[0] if kind == O.KIND_K else preset[1]


@settings(max_examples=25, deadline=None)
@given(x=tiles, kind=kinds, preset=presets, n=iters)
def test_codes_are_the_nearest_level_of_the_stored_grid(x, kind, preset, n):
    out = O.quantize_tiles(x, kind, n, k_bits=preset[0], v_bits=preset[1])
    qmax = (1 << _bits(kind, preset)) - 1
    codes = out["codes"].astype(np.int64)
    assert codes.min() >= 0 and codes.max() <= qmax
    # the normalized tile against the stored grid: |y - (zero + scale code)| <= scale / 2,
    # widened only where the clip at the top level meets the float16-rounded range
    sc = out["scale"].astype(np.float64)
    zr = out["zero"].astype(np.float64)
    sc_b, zr_b = (sc[:, None], zr[:, None]) if kind == O.KIND_K else (sc[None, :], zr[None, :])
    y = out["y"]
    err = np.abs(y - (zr_b + sc_b * codes))
    top = np.abs(y - zr_b) > sc_b * (qmax - 0.5)
    ulp = lambda a: np.spacing(np.abs(a).astype(np.float16)).astype(np.float64)
    slack = np.where(top, qmax * ulp(sc_b) + ulp(zr_b), 0.0)
    assert np.all(err <= 0.5 * sc_b * (1 + 1e-9) + slack + 1e-12 * np.abs(y))


@settings(max_examples=15, deadline=None)
@given(x=tiles, kind=kinds, preset=presets, n=iters)
def test_page_record_round_trip(x, kind, preset, n):
    kb, vb = preset
    out = O.quantize_tiles(x, kind, n, k_bits=kb, v_bits=vb)
    rec = O.pack_record(kind, out["codes"], out["r"], out["s"], out["scale"], out["zero"],
                        k_bits=kb, v_bits=vb)
    back = O.unpack_record(rec, kind, kb, vb)
    for key in ("codes", "r", "s", "scale", "zero"):
        assert np.array_equal(back[key], out[key]), key


@settings(max_examples=15, deadline=None)
@given(x=tiles, kind=kinds, preset=presets, k=st.integers(-3, 3))
def test_power_of_two_scaling_moves_only_the_token_normalizer(x, kind, preset, k):
    kb, vb = preset
    a = O.quantize_tiles(x, kind, 8, k_bits=kb, v_bits=vb)
    xs = (x.astype(np.float64) * 2.0 ** k).astype(np.float16)
    if not np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** k):
        return    # the scaled tile left float16's exact range (subnormal or overflow)
    b = O.quantize_tiles(xs, kind, 8, k_bits=kb, v_bits=vb)
    sa = a["s"].astype(np.float64) * 2.0 ** k
    if not np.array_equal(sa.astype(np.float16).astype(np.float64), sa):
        return    # the scaled normalizer is not exact in float16
    assert np.array_equal(a["r"], b["r"])
    assert np.array_equal(sa, b["s"].astype(np.float64))
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["scale"], b["scale"]) and np.array_equal(a["zero"], b["zero"])


@settings(max_examples=10, deadline=None)
@given(x=tiles, kind=kinds, preset=presets, seed=st.integers(0, 2**31 - 1))
def test_token_permutation_permutes_codes_and_token_normalizers(x, kind, preset, seed):
    kb, vb = preset
    perm = np.random.default_rng(seed).permutation(128)
    a = O.quantize_tiles(x, kind, 4, k_bits=kb, v_bits=vb)
    b = O.quantize_tiles(x[:, perm], kind, 4, k_bits=kb, v_bits=vb)
    # the channel normalizer is a sum over tokens: reordering changes its last bits only
    assert np.allclose(a["r"].astype(float), b["r"].astype(float), rtol=2e-3)
    if np.array_equal(a["r"], b["r"]):
        assert np.array_equal(a["s"][perm], b["s"])
        assert np.array_equal(a["codes"][:, perm], b["codes"])
