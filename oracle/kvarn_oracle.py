"""Plain CPU oracle for the KVarN tile quantizer and the paged decode-attention read path.

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it. The HIP library never calls it
and shares no code, table or constant generator with it.

Everything here is float64 NumPy. The only roundings are the explicit float16 ones that
the stored format requires (normalizers, scales and zeros are float16 values in a page).

Sources (page titles; the pages hold no code, no worked example and no kernel):
  [README]  "huawei-csl/KVarN" README (Chinese translation on bittide.aicompass.dev),
            sections "Quick start" and "How KVarN works" (four stages).
  [README-ko] Korean translation of the same README (molayo1419.me), same sections.
  [hypho]   "KV-cache quantization finally production-ready? KVarN ..." (blog.hypho.cn),
            section "four-step pipeline".
  [icwork]  "Huawei open-sources KVarN" (ic.work), the preset description (4-bit keys,
            2-bit values, group/block size 128).

Readings taken where the pages are silent (all listed with reasons in the design notes):
  * tile = 128 channels (rows) x 128 tokens (columns);
  * H = natural-order Sylvester Hadamard / sqrt(128), no random signs;
  * one Sinkhorn iteration = a column (per-token) step then a row (per-channel) step;
  * "std" = population standard deviation (ddof=0), centred;
  * log-scales start at 0, accumulate additively, exp'd once at the end;
  * a zero / non-finite std skips that update;
  * normalizers rounded to float16 (clipped to [2^-14, 65504]) and the tile is quantized
    against the stored float16 values;
  * asymmetric RTN: zero = group min, scale = (max - min) / (2^b - 1), both stored float16
    (saturated to +-65504, as the normalizers are clipped to the float16 range),
    code = round-half-even((y - zero) / scale) clipped to [0, 2^b - 1]; scale 0 => code 0;
  * group size 64 (presets _g64, the finer setting of the pages' group-size knob): keys in
    two groups of 64 consecutive tokens per channel, values in two groups of 64 consecutive
    channels per token, each with its own scale and zero; normalization is unchanged.

Parity status: every function below is pinned by tests that do not re-type its formula
(closed forms, invariants, library routines, brute force, hand-derived byte patterns).
The exact normalizer values for general inputs are not printed on the pages; they are
fixed only by the readings above plus those pins.
"""
from __future__ import annotations

import numpy as np

TILE_TOKENS = 128
HEAD_DIM = 128
K_BITS = 4
V_BITS = 2
FP16_MIN_NORMAL = 2.0 ** -14
FP16_MAX = 65504.0

KIND_K = 0
KIND_V = 1

# ----------------------------------------------------------------------------- helpers


def to_fp16(x) -> np.ndarray:
    """Round float64 values to float16, nearest-even (NumPy converts directly from double)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def hadamard(n: int = HEAD_DIM) -> np.ndarray:
    """Normalized natural-order Sylvester Hadamard matrix, float64, n a power of two.

    [README] "How KVarN works", stage 2: the rotation along channels is a Hadamard rotation
    and is orthonormal. Built by the doubling recursion [[A, A], [A, -A]], then / sqrt(n).
    """
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


# ----------------------------------------------------------------------------- quantizer


def rotate(x: np.ndarray) -> np.ndarray:
    """Stage 2 ([README] "How KVarN works", stage 2): Xr = H @ X along the channel axis.

    x: [..., 128 channels, 128 tokens] float64.
    """
    return hadamard(x.shape[-2]) @ x


def _log_std_update(sigma: np.ndarray) -> np.ndarray:
    ok = np.isfinite(sigma) & (sigma > 0)
    return np.where(ok, np.log(np.where(ok, sigma, 1.0)), 0.0)


def population_std(y: np.ndarray, axis: int) -> np.ndarray:
    """Centred population standard deviation along `axis`; exactly 0 for a group of
    identical values (whatever the summation order of the library mean)."""
    sd = y.std(axis=axis)
    return np.where(y.max(axis=axis) == y.min(axis=axis), 0.0, sd)


def sinkhorn_log(xr: np.ndarray, n_iters: int, history: list | None = None):
    """Stage 3 ([README] "How KVarN works", stage 3; [README-ko] same stage; [hypho] step 3).

    Iterative variance normalization in log space, alternating a column (per-token) std
    normalization and a row (per-channel) std normalization.

    xr: [..., C, T] rotated tile. Returns (la [..., C], lb [..., T]) with r = exp(la) the
    per-channel normalizer and s = exp(lb) the per-token normalizer, so that the normalized
    tile is Y = xr / (r[:, None] * s[None, :]).

    If `history` is a list, the max |log column std| measured at the start of every column
    step is appended (a convergence diagnostic).
    """
    shape = xr.shape
    la = np.zeros(shape[:-1], dtype=np.float64)                 # log r, per channel
    lb = np.zeros(shape[:-2] + (shape[-1],), dtype=np.float64)  # log s, per token
    for _ in range(n_iters):
        # column step: every token column gets unit std over the channels
        y = xr * np.exp(-la)[..., :, None] * np.exp(-lb)[..., None, :]
        sig_t = population_std(y, axis=-2)
        if history is not None:
            history.append(float(np.max(np.abs(_log_std_update(sig_t)))))
        lb = lb + _log_std_update(sig_t)
        # row step: every channel row gets unit std over the tokens
        y = xr * np.exp(-la)[..., :, None] * np.exp(-lb)[..., None, :]
        sig_c = population_std(y, axis=-1)
        la = la + _log_std_update(sig_c)
    return la, lb


def store_normalizer(log_v: np.ndarray) -> np.ndarray:
    """exp of a log-normalizer, clipped to the float16 normal range and rounded to float16."""
    return to_fp16(np.clip(np.exp(log_v), FP16_MIN_NORMAL, FP16_MAX))


def store_meta(v: np.ndarray) -> np.ndarray:
    """A scale or zero point as stored: float16 round-to-nearest-even, saturated to the finite
    range [-65504, 65504] (the stored format holds float16 metadata, like the normalizers, and
    a finite input never yields an infinite record)."""
    return to_fp16(np.clip(v, -FP16_MAX, FP16_MAX))


def rtn_asym(y: np.ndarray, bits: int, axis: int, group: int = 128):
    """Stage 4 ([README] "How KVarN works", stage 4): asymmetric round-to-nearest.

    Groups run along `axis`: `group` consecutive elements of it that share the other indices
    (group = the axis length: one group per row or column; group 64: its two halves).
    Returns (codes uint8, scale16, zero16, u) where u is the unrounded code value in float64
    (kept for the analysis of rounding ties). scale16 and zero16 drop the group axis when it
    holds one group; with two groups (group 64) they are [..., 2, n] with the half first.
    """
    qmax = (1 << bits) - 1
    ax = axis % y.ndim
    ng = y.shape[ax] // group
    if ng * group != y.shape[ax]:
        raise ValueError("the group size must divide the axis")
    yg = y.reshape(y.shape[:ax] + (ng, group) + y.shape[ax + 1:])   # (half, element) at ax
    mn = yg.min(axis=ax + 1, keepdims=True)
    mx = yg.max(axis=ax + 1, keepdims=True)
    scale16 = store_meta((mx - mn) / qmax)
    zero16 = store_meta(mn)
    sc = scale16.astype(np.float64)
    zr = zero16.astype(np.float64)
    live = sc > 0
    u = np.where(live, (yg - zr) / np.where(live, sc, 1.0), 0.0)
    codes = np.clip(np.rint(u), 0, qmax).astype(np.uint8)
    codes = np.where(live, codes, 0).astype(np.uint8).reshape(y.shape)
    u = u.reshape(y.shape)
    scale16 = np.squeeze(scale16, ax + 1)
    zero16 = np.squeeze(zero16, ax + 1)
    if ng == 1:
        scale16, zero16 = np.squeeze(scale16, ax), np.squeeze(zero16, ax)
    elif ax == y.ndim - 1:          # [..., n, halves] -> [..., halves, n]
        scale16, zero16 = np.moveaxis(scale16, -1, -2), np.moveaxis(zero16, -1, -2)
    return codes, scale16, zero16, u


def quantize_tiles(x16: np.ndarray, kind: int, n_iters: int = 8, lossless: bool = False,
                   rotate_channels: bool = True, k_bits: int = 4, v_bits: int = 2,
                   fmt: int = 1, group: int = 128):
    """Quantize tiles end to end (stages 1-4 of [README] "How KVarN works").

    x16: [..., 128 channels, 128 tokens] float16 (stage 1: the raw tile, channels x tokens).
    kind: KIND_K (4-bit, one group per channel row) or KIND_V (2-bit, one group per token
    column) -- [README] stage 4 (keys per channel, values per token) and the preset
    kvarn_k4v2_g128 ([README] "Quick start"; [icwork] preset table: group size 128).

    Returns a dict with float16 r [...,128], s [...,128], scale [...,128], zero [...,128],
    uint8 codes [..., 128 c, 128 t], plus float64 'xr' (rotated tile), 'y' (normalized tile
    against the stored normalizers) and 'u' (unrounded codes).

    lossless=True stops after stage 3 and returns no codes (used to pin the bookkeeping).
    rotate_channels=False skips stage 2 (Xr = X): an ablation of the method, not the method.
    k_bits, v_bits: code widths of the preset (kvarn_k4v2_g128: 4, 2; kvarn_k2v2_g128: 2, 2;
    kvarn_k4v4_g128: 4, 4).
    fmt=2 is the folded record format: each group's own normalizer is folded into its scale
    and zero, so the round-to-nearest runs on Z = Xr / s (keys, groups = channels) or
    Z = Xr / r (values, groups = tokens) and the record stores only the other normalizer.
    Its dict then reports the folded-away normalizer as 1 (r for keys, s for values), 'scale'
    and 'zero' as the folded values and 'y' as Z, so that r s (zero + scale code) is still the
    reconstruction of Xr.
    group: elements per quantization group (the preset's _g<G>): 128 = one group per channel
    (keys) or token (values); 64 = keys in two 64-token groups per channel, values in two
    64-channel groups per token (a finer scale grid, the pages' group-size knob). With 64,
    'scale' and 'zero' are [..., 2, 128], half 0 first.
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if x.shape[-2:] != (HEAD_DIM, TILE_TOKENS):
        raise ValueError("tile must be 128 channels x 128 tokens")
    xr = rotate(x) if rotate_channels else x
    la, lb = sinkhorn_log(xr, n_iters)
    r16 = store_normalizer(la)
    s16 = store_normalizer(lb)
    y = xr / (r16.astype(np.float64)[..., :, None] * s16.astype(np.float64)[..., None, :])
    out = dict(r=r16, s=s16, xr=xr, y=y)
    if lossless:
        return out
    if kind not in (KIND_K, KIND_V):
        raise ValueError("kind must be KIND_K or KIND_V")
    if fmt == 2:
        # fold the group's normalizer: keys code Xr / s per channel, values Xr / r per token
        one = np.ones_like(r16)
        if kind == KIND_K:
            y = xr / s16.astype(np.float64)[..., None, :]
            out.update(r=one, y=y)
        else:
            y = xr / r16.astype(np.float64)[..., :, None]
            out.update(s=np.ones_like(s16), y=y)
    elif fmt != 1:
        raise ValueError("fmt must be 1 or 2")
    if group not in (128, 64):
        raise ValueError("group must be 128 or 64")
    if kind == KIND_K:
        codes, scale16, zero16, u = rtn_asym(y, k_bits, axis=-1, group=group)
    else:
        codes, scale16, zero16, u = rtn_asym(y, v_bits, axis=-2, group=group)
    out.update(codes=codes, scale=scale16, zero=zero16, u=u)
    return out


def dequantize_tiles(codes, r16, s16, scale16, zero16, kind: int,
                     rotate_channels: bool = True, group: int = 128) -> np.ndarray:
    """Inverse of quantize_tiles up to rounding: X_hat = H (r s^T * (zero + scale * code)).

    The scales are re-applied per channel for keys and per token for values
    ([README] "How KVarN works", stage 4); H is symmetric and its own inverse. With group 64
    the scale and zero are [..., 2, 128] and element (c, t) takes the half of t (keys) or of
    c (values). Returns float64 [..., 128 c, 128 t]. rotate_channels=False inverts a tile
    quantized without stage 2 (the ablation of quantize_tiles).
    """
    codes = np.asarray(codes, dtype=np.float64)
    sc = np.asarray(scale16, dtype=np.float64)
    zr = np.asarray(zero16, dtype=np.float64)
    if group == 128:
        sc_e = sc[..., :, None] if kind == KIND_K else sc[..., None, :]
        zr_e = zr[..., :, None] if kind == KIND_K else zr[..., None, :]
    elif group == 64:
        if kind == KIND_K:     # [..., half, c] -> [..., c, t]: token t takes half t // 64
            sc_e = np.repeat(np.swapaxes(sc, -1, -2), 64, axis=-1)
            zr_e = np.repeat(np.swapaxes(zr, -1, -2), 64, axis=-1)
        else:                  # [..., half, t] -> [..., c, t]: channel c takes half c // 64
            sc_e = np.repeat(sc, 64, axis=-2)
            zr_e = np.repeat(zr, 64, axis=-2)
    else:
        raise ValueError("group must be 128 or 64")
    yhat = zr_e + sc_e * codes
    r = np.asarray(r16, dtype=np.float64)
    s = np.asarray(s16, dtype=np.float64)
    xr_hat = r[..., :, None] * s[..., None, :] * yhat
    return hadamard(HEAD_DIM) @ xr_hat if rotate_channels else xr_hat


# ----------------------------------------------------------------------------- page format
# Format v1 of one page record (one 128-token tile of one KV head). Written here from the
# format specification, independently of the HIP packer.
#   K record, 9216 bytes: 8192 B of 4-bit codes, token-major: token t owns bytes
#     [64 t, 64 t + 64) as 16 little-endian 32-bit words; word j holds channels 8j..8j+7,
#     nibble p (bits 4p..4p+3) holding channel 8j + K_NIBBLE_CHANNEL[p].
#   V record, 5120 bytes: 4096 B of 2-bit codes, channel-major: channel c owns 8 words at
#     word index 8c + 2g + d (g in 0..3, d in 0..1); crumb p (bits 2p..2p+1) of that word
#     holds token v_crumb_token(g, d, p).
#   Then four float16[128] vectors: r (per channel), s (per token), scale, zero
#     (per channel for K, per token for V).

#   4-bit V record (preset kvarn_k4v4_g128), 9216 bytes: 8192 B of 4-bit codes, channel-major:
#     channel c owns the 16 words 16c + 4g + m (g, m in 0..3); nibble q (bits 4q..4q+3) of
#     word (c, g, m) holds token v4_nibble_token(g, m, q); then the metadata.
#   2-bit K record (preset kvarn_k2v2_g128), 5120 bytes: 4096 B of 2-bit codes, token-major:
#     token t owns bytes [32 t, 32 t + 32) as 8 words; word w = 2g + d (g in 0..3, d in 0..1)
#     holds channels 16 w .. 16 w + 15, crumb p (bits 2p..2p+1) = channel
#     k2_crumb_channel(g, d, p); then the metadata.

K_RECORD_BYTES = 9216
K2_RECORD_BYTES = 5120
V_RECORD_BYTES = 5120
V4_RECORD_BYTES = 9216
K_NIBBLE_CHANNEL = (0, 2, 4, 6, 1, 3, 5, 7)


def k2_crumb_channel(g: int, d: int, p: int) -> int:
    """Channel held by crumb p of word 2g + d of a token in a 2-bit K record: word 2g + d holds
    channels 32 g + 16 d .. + 15 (two groups of 8, hs = (p mod 8) div 4), crumb p of a group
    holding offset 2 (p mod 4) + p div 8."""
    hs, v, e = (p % 8) // 4, p % 4, p // 8
    return 32 * g + 8 * (2 * d + hs) + 2 * v + e


def v_crumb_token(g: int, d: int, p: int) -> int:
    """Token held by crumb p of word (g, d) of a channel in a V record."""
    i, half = (p, 0) if p < 8 else (p - 8, 1)
    step = 2 * d + i // 4
    slot = 2 * (i % 4) + half
    within = 4 * g + slot if slot < 4 else 12 + 4 * g + slot
    return 32 * step + within


def v4_nibble_token(g: int, m: int, q: int) -> int:
    """Token held by nibble q of word (g, m) of a channel in a 4-bit V record: the token that
    crumb 4 (m mod 2) + (q mod 4) + 8 (q div 4) of word (g, m div 2) holds in a 2-bit V record
    (the same token order, one code per nibble)."""
    return v_crumb_token(g, m // 2, 4 * (m % 2) + (q % 4) + 8 * (q // 4))


def _meta_bytes(r16, s16, scale16, zero16) -> bytes:
    """r, s, then the scale vectors and the zero vectors (one each for group 128; half 0 then
    half 1 for group 64), float16 little-endian."""
    parts = [np.asarray(r16, dtype="<f2").reshape(128), np.asarray(s16, dtype="<f2").reshape(128),
             np.asarray(scale16, dtype="<f2").reshape(-1), np.asarray(zero16, dtype="<f2").reshape(-1)]
    return b"".join(p.tobytes() for p in parts)


# Format 2 (folded) of the same records: the code bytes, then keys s, scale', zero' (per
# channel, of Z = Xr / s); values r, scale', zero' (per token, of Z = Xr / r). One float16[128]
# vector fewer.
# Group 64 (presets _g64): two scale and two zero vectors (half 0 = tokens 0..63 of a key
# channel / channels 0..63 of a value token, then half 1) in place of one each.
META_BYTES = {1: 1024, 2: 768}


def meta_bytes(fmt: int = 1, group: int = 128) -> int:
    """Metadata bytes of a record: 256 per float16[128] vector."""
    return 256 * ((2 if fmt == 1 else 1) + 2 * (128 // group))


def code_bytes(kind: int, k_bits: int = 4, v_bits: int = 2) -> int:
    bits = k_bits if kind == KIND_K else v_bits
    return 8192 if bits == 4 else 4096


def record_bytes(kind: int, k_bits: int = 4, v_bits: int = 2, fmt: int = 1, group: int = 128) -> int:
    return code_bytes(kind, k_bits, v_bits) + meta_bytes(fmt, group)


_LAYOUTS = {cb + meta_bytes(f, g): (bits, f, g) for bits, cb in ((4, 8192), (2, 4096))
            for f in (1, 2) for g in (128, 64)}


def record_layout(nbytes: int):
    """(code bits, format) of a record from its size: 9216 / 5120 bytes are format 1 with 4 /
    2-bit codes, 8960 / 4864 format 2; group 64 adds 512 bytes to either."""
    return _LAYOUTS[nbytes][:2]


def record_group(nbytes: int) -> int:
    """Group size (128 or 64) of a record from its size."""
    return _LAYOUTS[nbytes][2]


def fold_record(rec1: bytes, kind: int, group: int = 128) -> bytes:
    """Format-2 layout of a format-1 record whose folded-away normalizer is exactly 1 (the
    byte arrangement only: codes kept, the all-ones vector dropped)."""
    cb = len(rec1) - meta_bytes(1, group)
    m = np.frombuffer(rec1[cb:], dtype="<f2").reshape(-1, 128)
    drop = 0 if kind == KIND_K else 1
    assert np.all(m[drop] == 1.0)
    return rec1[:cb] + b"".join(m[k].tobytes() for k in range(m.shape[0]) if k != drop)


def pack_k_record(codes, r16, s16, scale16, zero16) -> bytes:
    codes = np.asarray(codes)
    assert codes.shape == (128, 128) and codes.max(initial=0) <= 15
    words = np.zeros((128, 16), dtype=np.uint32)
    for t in range(128):
        for j in range(16):
            w = 0
            for p in range(8):
                w |= int(codes[8 * j + K_NIBBLE_CHANNEL[p], t]) << (4 * p)
            words[t, j] = w
    return words.astype("<u4").tobytes() + _meta_bytes(r16, s16, scale16, zero16)


def pack_k2_record(codes, r16, s16, scale16, zero16) -> bytes:
    codes = np.asarray(codes)
    assert codes.shape == (128, 128) and codes.max(initial=0) <= 3
    words = np.zeros((128, 8), dtype=np.uint32)
    for t in range(128):
        for g in range(4):
            for d in range(2):
                w = 0
                for p in range(16):
                    w |= int(codes[k2_crumb_channel(g, d, p), t]) << (2 * p)
                words[t, 2 * g + d] = w
    return words.astype("<u4").tobytes() + _meta_bytes(r16, s16, scale16, zero16)


def pack_v_record(codes, r16, s16, scale16, zero16) -> bytes:
    codes = np.asarray(codes)
    assert codes.shape == (128, 128) and codes.max(initial=0) <= 3
    words = np.zeros(128 * 8, dtype=np.uint32)
    for c in range(128):
        for g in range(4):
            for d in range(2):
                w = 0
                for p in range(16):
                    w |= int(codes[c, v_crumb_token(g, d, p)]) << (2 * p)
                words[8 * c + 2 * g + d] = w
    return words.astype("<u4").tobytes() + _meta_bytes(r16, s16, scale16, zero16)


def pack_v4_record(codes, r16, s16, scale16, zero16) -> bytes:
    codes = np.asarray(codes)
    assert codes.shape == (128, 128) and codes.max(initial=0) <= 15
    words = np.zeros(128 * 16, dtype=np.uint32)
    for c in range(128):
        for g in range(4):
            for m in range(4):
                w = 0
                for q in range(8):
                    w |= int(codes[c, v4_nibble_token(g, m, q)]) << (4 * q)
                words[16 * c + 4 * g + m] = w
    return words.astype("<u4").tobytes() + _meta_bytes(r16, s16, scale16, zero16)


def _unpack_meta(buf: np.ndarray, off: int, group: int = 128):
    ng = 128 // group
    m = buf[off:off + meta_bytes(1, group)].view("<f2").reshape(2 + 2 * ng, 128)
    sc, zr = m[2:2 + ng].copy(), m[2 + ng:].copy()
    if ng == 1:
        sc, zr = sc[0], zr[0]
    return m[0].copy(), m[1].copy(), sc, zr


def unpack_k_record(rec, group: int = 128) -> dict:
    buf = np.frombuffer(bytes(rec), dtype=np.uint8)
    assert buf.size == 8192 + meta_bytes(1, group)
    words = buf[:8192].view("<u4").reshape(128, 16)
    codes = np.zeros((128, 128), dtype=np.uint8)
    for p in range(8):
        nib = (words >> np.uint32(4 * p)) & np.uint32(0xF)        # [t, j]
        for j in range(16):
            codes[8 * j + K_NIBBLE_CHANNEL[p], :] = nib[:, j]
    r, s, sc, zr = _unpack_meta(buf, 8192, group)
    return dict(codes=codes, r=r, s=s, scale=sc, zero=zr)


def unpack_k2_record(rec, group: int = 128) -> dict:
    buf = np.frombuffer(bytes(rec), dtype=np.uint8)
    assert buf.size == 4096 + meta_bytes(1, group)
    words = buf[:4096].view("<u4").reshape(128, 4, 2)                  # [t, g, d]
    codes = np.zeros((128, 128), dtype=np.uint8)
    for g in range(4):
        for d in range(2):
            for p in range(16):
                codes[k2_crumb_channel(g, d, p), :] = (words[:, g, d] >> np.uint32(2 * p)) & np.uint32(3)
    r, s, sc, zr = _unpack_meta(buf, 4096, group)
    return dict(codes=codes, r=r, s=s, scale=sc, zero=zr)


def unpack_v4_record(rec, group: int = 128) -> dict:
    buf = np.frombuffer(bytes(rec), dtype=np.uint8)
    assert buf.size == 8192 + meta_bytes(1, group)
    words = buf[:8192].view("<u4").reshape(128, 4, 4)                  # [c, g, m]
    codes = np.zeros((128, 128), dtype=np.uint8)
    for g in range(4):
        for m in range(4):
            for q in range(8):
                codes[:, v4_nibble_token(g, m, q)] = (words[:, g, m] >> np.uint32(4 * q)) & np.uint32(15)
    r, s, sc, zr = _unpack_meta(buf, 8192, group)
    return dict(codes=codes, r=r, s=s, scale=sc, zero=zr)


def unpack_record(rec, kind: int, k_bits: int = 4, v_bits: int = 2, fmt: int = 1,
                  group: int = 128) -> dict:
    """The record of `kind` for the preset with k_bits-bit keys and v_bits-bit values, in
    record format fmt (format 2 reports the folded-away normalizer as ones) and group size
    `group` (64: scale and zero are [2, 128])."""
    rec = bytes(rec)
    if fmt == 2:
        cb = code_bytes(kind, k_bits, v_bits)
        assert len(rec) == cb + meta_bytes(2, group)
        m = np.frombuffer(rec[cb:], dtype="<f2").reshape(-1, 128)
        ng = 128 // group
        one = np.ones(128, dtype=np.float16)
        r16, s16 = (one, m[0]) if kind == KIND_K else (m[0], one)
        rec = rec[:cb] + _meta_bytes(r16, s16, m[1:1 + ng], m[1 + ng:])
    if kind == KIND_V:
        return unpack_v_record(rec, group) if v_bits == 2 else unpack_v4_record(rec, group)
    return unpack_k_record(rec, group) if k_bits == 4 else unpack_k2_record(rec, group)


def pack_record(kind: int, codes, r16, s16, scale16, zero16, k_bits: int = 4,
                v_bits: int = 2, fmt: int = 1, group: int = 128) -> bytes:
    if kind == KIND_V:
        pack = pack_v_record if v_bits == 2 else pack_v4_record
    else:
        pack = pack_k_record if k_bits == 4 else pack_k2_record
    if np.asarray(scale16).size != 128 * (128 // group):
        raise ValueError("scale / zero do not match the group size")
    if fmt == 1:
        return pack(codes, r16, s16, scale16, zero16)
    if fmt != 2:
        raise ValueError("fmt must be 1 or 2")
    one = np.ones(128, dtype=np.float16)
    rec1 = pack(codes, one if kind == KIND_K else r16, s16 if kind == KIND_K else one,
                scale16, zero16)
    return fold_record(rec1, kind, group)


def unpack_v_record(rec, group: int = 128) -> dict:
    buf = np.frombuffer(bytes(rec), dtype=np.uint8)
    assert buf.size == 4096 + meta_bytes(1, group)
    words = buf[:4096].view("<u4").reshape(128, 4, 2)
    codes = np.zeros((128, 128), dtype=np.uint8)
    for g in range(4):
        for d in range(2):
            for p in range(16):
                codes[:, v_crumb_token(g, d, p)] = (words[:, g, d] >> np.uint32(2 * p)) & np.uint32(3)
    r, s, sc, zr = _unpack_meta(buf, 4096, group)
    return dict(codes=codes, r=r, s=s, scale=sc, zero=zr)


# ----------------------------------------------------------------------------- attention


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Single-query softmax attention in float64, written out from its definition.

    q: [128], k: [n, 128], v: [n, 128]. Returns o = sum_t p_t v_t with
    p = softmax(softmax_scale * k @ q).
    """
    z = softmax_scale * (np.asarray(k, np.float64) @ np.asarray(q, np.float64))
    z = z - z.max()
    p = np.exp(z)
    return (p / p.sum()) @ np.asarray(v, np.float64)


def dequantize_k_record(rec, k_bits: int = 4, fmt: int = 1, group: int = 128) -> np.ndarray:
    """Unpack one K page record and return the dequantized keys [128 tokens, 128 channels]."""
    d = unpack_record(rec, KIND_K, k_bits=k_bits, fmt=fmt, group=group)
    return dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], KIND_K,
                            group=group).T


def dequantize_v_record(rec, v_bits: int = 2, fmt: int = 1, group: int = 128) -> np.ndarray:
    d = unpack_record(rec, KIND_V, v_bits=v_bits, fmt=fmt, group=group)
    return dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], KIND_V,
                            group=group).T


def decode_attention_row(q_row, k_pages, v_pages, k_tail=None, v_tail=None,
                         softmax_scale: float = 1.0 / np.sqrt(HEAD_DIM), k_bits: int = 4,
                         v_bits: int = 2, fmt: int = 1, group: int = 128) -> np.ndarray:
    """Decode attention of one query row over one KV head's cache.

    k_pages / v_pages: lists of page records (bytes) of that KV head, in block-table order
    (the cache is read from quantized tiles, [README] intro: a native attention backend;
    scales re-applied on read, "How KVarN works" stage 4).
    k_tail / v_tail: [n_tail, 128] float16 tokens past the last full page (raw, exact).
    Returns float64 [128].
    """
    ks = [dequantize_k_record(p, k_bits, fmt, group) for p in k_pages]
    vs = [dequantize_v_record(p, v_bits, fmt, group) for p in v_pages]
    if k_tail is not None and len(k_tail):
        ks.append(np.asarray(k_tail, np.float16).astype(np.float64))
        vs.append(np.asarray(v_tail, np.float16).astype(np.float64))
    k = np.concatenate(ks, axis=0)
    v = np.concatenate(vs, axis=0)
    return attention(np.asarray(q_row, np.float16).astype(np.float64), k, v, softmax_scale)


def causal_attention(q_rows: np.ndarray, positions, k: np.ndarray, v: np.ndarray,
                     softmax_scale: float) -> np.ndarray:
    """Causal attention of several query rows over one cache (the read path of a prefill chunk
    or of draft tokens): row i sits at cache position positions[i] and attends to the keys at
    positions 0 .. positions[i], inclusive; a row at a negative position (before the cache
    starts) has no keys and returns zeros.

    q_rows: [n, 128]; k, v: [C, 128] (the cache in position order). Returns float64 [n, 128].
    """
    q_rows = np.asarray(q_rows, np.float64)
    out = np.zeros((q_rows.shape[0], np.asarray(v).shape[1]), dtype=np.float64)
    for i, p in enumerate(positions):
        if p < 0:
            continue
        out[i] = attention(q_rows[i], k[:p + 1], v[:p + 1], softmax_scale)
    return out


def merge_partials(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Combine partial softmax results of disjoint token ranges.

    Each part i holds its max score m_i, its sum l_i = sum exp(z - m_i) and its unnormalized
    output acc_i = sum exp(z - m_i) v. The result equals attention over the union.
    """
    m = np.asarray(m, np.float64)
    w = np.exp(m - m.max())
    return (w[:, None] * np.asarray(acc, np.float64)).sum(0) / (w * np.asarray(l, np.float64)).sum()


def partial_attention(q, k, v, softmax_scale):
    """(m, l, acc) of one token range, for merge_partials."""
    z = softmax_scale * (np.asarray(k, np.float64) @ np.asarray(q, np.float64))
    m = z.max()
    p = np.exp(z - m)
    return m, p.sum(), p @ np.asarray(v, np.float64)
