"""Shared parity machinery for the GPU tests: the HIP path against the CPU oracle.

Criteria (tolerances stated for the method's output, checked element by element):
  L1 metadata: r, s within 1e-3 relative of the oracle's float16 values; scale within 1e-3
     relative and zero within 1e-3 * max(|zero|, scale), each widened by the relative r, s
     difference its group sees (scale and zero come from y = Xr / (r s) on each side's own
     stored r, s, so a 1-ulp normalizer flip carries over to them) and by the float32 bound
     on y that L2 uses (delta below): zero = min y moves by up to delta, scale = range / levels
     by up to 2 delta / levels. That term only matters for a group whose range is a tiny
     fraction of its values (e.g. the DC channel of a nearly constant tile).
  L2 conditional codes: codes re-derived by the oracle from its float64 rotated tile and the
     GPU's own stored r, s, scale, zero must equal the GPU codes, except where the unrounded
     code value lies within a tie band of a rounding boundary: TIE_BAND plus the float32
     rounding bound of the rotated value (32 ulp of the token's |x|_1 / sqrt(128)) divided by
     that element's step r_c s_t scale (float32 vs float64 evaluation). In units of y that
     bound is delta = 32 ulp(|x_t|_1 / sqrt(128)) / (r_c s_t).
  L3 unconditional codes: GPU codes differ from the oracle's in at most 1e-4 of all codes,
     each by exactly 1 (rounding ties, and cascades of a 1-ulp float16 metadata flip).
  Attention: per (sequence, query head) row, max|o_gpu - o_oracle| <= 2e-3 max|o_oracle|.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import kvarn_oracle as O

TIE_BAND = 1e-4
META_RTOL = 1e-3
CODE_MISMATCH_RATE = 1e-4
ATTN_RTOL = 2e-3


def records_of(pool: torch.Tensor, pages, head: int):
    """Host bytes of the records (page, head) for the given page ids."""
    sel = pool[torch.as_tensor(list(pages), dtype=torch.long, device=pool.device), head]
    arr = sel.cpu().numpy()
    return [arr[i].tobytes() for i in range(arr.shape[0])]


class QuantStats:
    def __init__(self):
        self.codes = 0
        self.l3_mismatch = 0
        self.l2_mismatch = 0
        self.meta_exact = 0
        self.meta_total = 0
        self.max_meta_rel = 0.0

    def rate(self):
        return self.l3_mismatch / max(self.codes, 1)

    def __repr__(self):
        return (f"codes={self.codes} L3 mismatches={self.l3_mismatch} ({self.rate():.2e}) "
                f"L2 outside-tie={self.l2_mismatch} meta exact {self.meta_exact}/{self.meta_total} "
                f"max meta rel {self.max_meta_rel:.2e}")


def reconstruction_error(x_ct: np.ndarray, d: dict, kind: int) -> float:
    xh = O.dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], kind)
    return float(np.linalg.norm(xh - x_ct))


def check_quantized_tiles(tiles_tc: np.ndarray, records, kind: int, n_iters: int,
                          stats: QuantStats | None = None, rate_exempt=(),
                          ill_conditioned=(), k_bits: int = 4, v_bits: int = 2) -> QuantStats:
    """tiles_tc: [n, 128 tokens, 128 channels] float16 (the source layout); records: the GPU
    page records of those tiles. Asserts L1 and L2, accumulates L3 statistics.

    Tiles listed in rate_exempt are ill-conditioned on purpose (values identical up to below
    float16 resolution, so a 1-ulp metadata difference moves many tied codes at once); they
    are held to L1, L2 and |code difference| <= 1 but kept out of the L3 rate.

    Tiles listed in ill_conditioned make the normalization itself ill-conditioned (a row that
    becomes constant up to ~1e-4 relative, where a float32 std cannot match a float64 one);
    they are held to L2 (codes correctly rounded for the stored metadata), finite metadata
    and a reconstruction error at most 5% above the oracle's."""
    stats = stats or QuantStats()
    x = np.ascontiguousarray(np.swapaxes(tiles_tc, -1, -2))  # channels x tokens
    ref = O.quantize_tiles(x, kind, n_iters, k_bits=k_bits, v_bits=v_bits)
    unpack = lambda rec: O.unpack_record(rec, kind, k_bits, v_bits)
    bits = k_bits if kind == O.KIND_K else v_bits
    qmax = (1 << bits) - 1
    for i, rec in enumerate(records):
        g = unpack(rec)
        if i in ill_conditioned:
            for key in ("r", "s", "scale", "zero"):
                assert np.all(np.isfinite(g[key].astype(np.float64))), (key, i)
            e_gpu = reconstruction_error(x[i].astype(np.float64), g, kind)
            e_ref = reconstruction_error(x[i].astype(np.float64), {k_: ref[k_][i] for k_ in ("codes", "r", "s", "scale", "zero")}, kind)
            assert e_gpu <= 1.05 * e_ref + 1e-6 * float(np.linalg.norm(x[i].astype(np.float64))), (i, e_gpu, e_ref)
        # ---- L1
        # scale and zero are float16 roundings of the range and minimum of y = Xr / (r s) taken
        # with each side's own stored r, s: a 1-ulp flip of those (allowed above) moves them by
        # the group's relative r, s differences, which are added to their tolerance, as is the
        # float32 evaluation bound on y (delta, the L2 band in units of y) over the group
        delta_g = _delta_group(x[i], ref["r"][i], ref["s"][i], kind)
        dev = {}
        for key in ("r", "s", "scale") if i not in ill_conditioned else ():
            a = g[key].astype(np.float64)
            b = ref[key][i].astype(np.float64)
            with np.errstate(invalid="ignore"):
                rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-30)
            # identical values match, including a float16 overflow to inf on both sides
            rel = np.where(a == b, 0.0, rel)
            dev[key] = rel
            stats.max_meta_rel = max(stats.max_meta_rel, float(rel.max()))
            if key != "scale":
                ok = rel <= META_RTOL
            else:   # absolute form, so that a zero-range group is held to 2 delta / levels
                with np.errstate(invalid="ignore"):
                    ok = (a == b) | (np.abs(a - b) <= (META_RTOL + 1.01 * _cascade(dev, kind)) * np.abs(b)
                                     + 1.01 * 2.0 * delta_g / qmax)
            assert np.all(ok), (key, i, float(rel.max()), _meta_report(g, ref, i))
            stats.meta_exact += int(np.sum(g[key] == ref[key][i]))
            stats.meta_total += 128
        if i not in ill_conditioned:
            za, zb = g["zero"].astype(np.float64), ref["zero"][i].astype(np.float64)
            zt = (META_RTOL * np.maximum(np.abs(zb), ref["scale"][i].astype(np.float64))
                  + 1.01 * (_cascade(dev, kind) * np.abs(zb) + delta_g) + 1e-30)
            with np.errstate(invalid="ignore"):
                zok = (za == zb) | (np.abs(za - zb) <= zt)
            assert np.all(zok), ("zero", i, za[~zok][:4], zb[~zok][:4], _meta_report(g, ref, i))
            stats.meta_exact += int(np.sum(g["zero"] == ref["zero"][i]))
            stats.meta_total += 128
        # ---- L2: the oracle's rounding step applied to the GPU's own metadata
        r, s = g["r"].astype(np.float64), g["s"].astype(np.float64)
        y = ref["xr"][i] / (r[:, None] * s[None, :])
        sc, zr = g["scale"].astype(np.float64), g["zero"].astype(np.float64)
        if kind == O.KIND_K:
            sc_b, zr_b = sc[:, None], zr[:, None]
        else:
            sc_b, zr_b = sc[None, :], zr[None, :]
        live = (sc_b > 0) & np.isfinite(zr_b) & np.isfinite(sc_b)
        with np.errstate(invalid="ignore", over="ignore"):
            u = np.where(live, (y - np.where(live, zr_b, 0.0)) / np.where(live, sc_b, 1.0), 0.0)
        re = np.clip(np.rint(u), 0, qmax)
        re = np.where(live, re, g["codes"])   # overflowed groups: compared at L3 only
        diff = re != g["codes"]
        if diff.any():
            frac = np.abs(u - np.floor(u) - 0.5)
            xscale = np.abs(x[i].astype(np.float64)).sum(axis=0)[None, :] / np.sqrt(128.0)
            step = r[:, None] * s[None, :] * np.where(sc_b > 0, sc_b, np.inf)
            band = TIE_BAND + 32 * 2.0 ** -24 * xscale / step
            near_tie = frac <= band
            outside = diff & ~near_tie
            stats.l2_mismatch += int(outside.sum())
            assert not outside.any(), (i, int(outside.sum()), u[outside][:5], g["codes"][outside][:5])
        # ---- L3
        if i in ill_conditioned:
            continue
        d = g["codes"].astype(int) - ref["codes"][i].astype(int)
        assert np.all(np.abs(d) <= 1), (i, int(np.abs(d).max()))
        if i not in rate_exempt:
            stats.l3_mismatch += int(np.count_nonzero(d))
            stats.codes += d.size
    return stats


def _delta_group(x_ct: np.ndarray, r16: np.ndarray, s16: np.ndarray, kind: int) -> np.ndarray:
    """Per group, the largest float32 evaluation bound on y = Xr / (r s) among its elements:
    32 ulp of the token's |x|_1 / sqrt(128) (the rotated value's bound), over r_c s_t. Keys:
    a group is a channel (max over tokens); values: a token (max over channels)."""
    xs = np.abs(x_ct.astype(np.float64)).sum(axis=0) / np.sqrt(128.0)       # per token
    rs = r16.astype(np.float64)[:, None] * s16.astype(np.float64)[None, :]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        d = 32 * 2.0 ** -24 * xs[None, :] / rs
    d = np.where(np.isfinite(d), d, 0.0)
    return d.max(axis=1) if kind == O.KIND_K else d.max(axis=0)


def _cascade(dev: dict, kind: int) -> np.ndarray:
    """Per group: relative r, s difference (GPU vs oracle) its elements can see. Keys: a
    group is a channel (its r, any token's s); values: a token (its s, any channel's r)."""
    dr, ds = dev["r"], dev["s"]
    return dr + ds.max() if kind == O.KIND_K else ds + dr.max()


def _meta_report(g: dict, ref: dict, i: int) -> str:
    out = []
    for key in ("r", "s", "scale", "zero"):
        a = g[key].astype(np.float64)
        b = ref[key][i].astype(np.float64)
        n = int(np.sum(a != b))
        out.append(f"{key}: {n} differ")
    return ", ".join(out)


def assert_rate(stats: QuantStats):
    assert stats.rate() <= CODE_MISMATCH_RATE, repr(stats)


def key_bits_of(k_pool) -> int:
    """Key code width of a pool, from its record size (9216 B: 4-bit, 5120 B: 2-bit)."""
    return 4 if k_pool.shape[2] == O.K_RECORD_BYTES else 2


def value_bits_of(v_pool) -> int:
    """Value code width of a pool, from its record size (5120 B: 2-bit, 9216 B: 4-bit)."""
    return 4 if v_pool.shape[2] == O.V4_RECORD_BYTES else 2


def oracle_rows(q: np.ndarray, hq_list, G: int, k_recs, v_recs, k_tail=None, v_tail=None,
                softmax_scale=1.0 / np.sqrt(128), k_bits: int = 4, v_bits: int = 2):
    """Oracle outputs for query heads hq_list (all sharing one KV head whose page records are
    k_recs / v_recs, plus float16 tails [n_tail, 128]). q: [Hq, 128] float16."""
    ks = [O.dequantize_k_record(r, k_bits) for r in k_recs]
    vs = [O.dequantize_v_record(r, v_bits) for r in v_recs]
    if k_tail is not None and len(k_tail):
        ks.append(np.asarray(k_tail, np.float16).astype(np.float64))
        vs.append(np.asarray(v_tail, np.float16).astype(np.float64))
    if not ks:
        return {hq: np.zeros(128) for hq in hq_list}
    k = np.concatenate(ks)
    v = np.concatenate(vs)
    return {hq: O.attention(q[hq].astype(np.float64), k, v, softmax_scale) for hq in hq_list}


def assert_rows_close(o_gpu: np.ndarray, o_ref: np.ndarray, what=""):
    ref16 = o_ref.astype(np.float16).astype(np.float64)
    denom = max(float(np.abs(ref16).max()), 1e-30)
    err = float(np.abs(o_gpu.astype(np.float64) - o_ref).max()) / denom
    assert err <= ATTN_RTOL, f"{what}: max-abs relative error {err:.3e}"
    return err


def check_decode(q_gpu, out_gpu, k_pool, v_pool, block_table, seq_lens, G, rows=None,
                 k_tail=None, v_tail=None, softmax_scale=1.0 / np.sqrt(128)):
    """Compare GPU decode output rows with the oracle, decoding the GPU-written pages with the
    oracle's own unpacker. rows: iterable of (b, g) KV-head rows to check (all by default).
    Returns the max relative error seen."""
    q = q_gpu.cpu().numpy()
    out = out_gpu.cpu().numpy()
    bt = block_table.cpu().numpy()
    lens = seq_lens.cpu().numpy()
    B, Hq = q.shape[0], q.shape[1]
    hkv = Hq // G
    if rows is None:
        rows = [(b, g) for b in range(B) for g in range(hkv)]
    kt = None if k_tail is None else k_tail.cpu().numpy()
    vt = None if v_tail is None else v_tail.cpu().numpy()
    worst = 0.0
    for b, g in rows:
        L = int(lens[b])
        nf = L // 128
        # pages outside the pool are skipped (they hold no keys)
        pages = [int(p) for p in bt[b, :nf] if 0 <= int(p) < k_pool.shape[0]]
        krec = records_of(k_pool, pages, g) if pages else []
        vrec = records_of(v_pool, pages, g) if pages else []
        tail_k = kt[b, g, :L % 128] if kt is not None else None
        tail_v = vt[b, g, :L % 128] if vt is not None else None
        hqs = list(range(g * G, (g + 1) * G))
        no_keys = not pages and (tail_k is None or tail_k.shape[0] == 0)
        ref = None if no_keys else oracle_rows(q[b], hqs, G, krec, vrec, tail_k, tail_v,
                                               softmax_scale, key_bits_of(k_pool),
                                               value_bits_of(v_pool))
        for hq in hqs:
            if no_keys:            # L = 0, or every page skipped and no tail: zeros
                assert np.all(out[b, hq] == 0), f"b={b} hq={hq}: expected zeros"
                continue
            worst = max(worst, assert_rows_close(out[b, hq], ref[hq], f"b={b} hq={hq} L={L}"))
    return worst
