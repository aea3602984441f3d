"""The C ABI on the CPU: the library loads, exports every function include/kvarn.h declares,
and rejects bad arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

from kv_cache_quantization_tile_amd import kvarn as K

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kvarn.h")
OK, INVALID, UNSUP, WS = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(kvarn_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(K.lib, n), n
    assert set(names) == set(K.EXPORTED)


def test_versions_and_status_strings():
    assert K.lib.kvarn_abi_version() == 2
    assert K.lib.kvarn_format_version() == 2            # formats 1 (separate) and 2 (folded)
    for s in range(5):
        assert K.lib.kvarn_status_str(s).decode() == K.STATUS[s]
    assert K.lib.kvarn_status_str(99) == b"unknown status"


def test_params_from_dtype():
    p = K.params_from_dtype("kvarn_k4v2_g128", 8)
    assert (p.head_dim, p.tile_tokens, p.k_bits, p.v_bits, p.group, p.sinkhorn_iters, p.format) == (128, 128, 4, 2, 128, 8, 1)
    out = K.Params()
    for bad in ("", "fp8", "kvarn_k4v2", "kvarn_k4v2_g", "kvarn_kv2_g128", "kvarn_k4v2_g128x", "kvarn_k0v2_g128"):
        assert K.lib.kvarn_params_from_dtype(bad.encode(), 8, ctypes.byref(out)) == INVALID, bad
    p2 = K.params_from_dtype("kvarn_k2v2_g128", 4)
    assert (p2.k_bits, p2.v_bits, p2.group, p2.sinkhorn_iters) == (2, 2, 128, 4)
    p4 = K.params_from_dtype("kvarn_k4v4_g128", 8)
    assert (p4.k_bits, p4.v_bits, p4.group) == (4, 4, 128)
    for unsup in ("kvarn_k3v2_g128", "kvarn_k2v4_g128", "kvarn_k4v3_g128", "kvarn_k4v2_g32",
                  "kvarn_k4v2_g256", "kvarn_k2v4_g64"):
        assert K.lib.kvarn_params_from_dtype(unsup.encode(), 8, ctypes.byref(out)) == UNSUP, unsup
    for name, kb, vb in (("kvarn_k4v2_g64", 4, 2), ("kvarn_k2v2_g64", 2, 2), ("kvarn_k4v4_g64", 4, 4)):
        pg = K.params_from_dtype(name, 8)
        assert (pg.k_bits, pg.v_bits, pg.group) == (kb, vb, 64)
    assert K.lib.kvarn_params_from_dtype(b"kvarn_k4v2_g128", -1, ctypes.byref(out)) == INVALID
    assert K.lib.kvarn_params_from_dtype(b"kvarn_k4v2_g128", 65, ctypes.byref(out)) == INVALID
    assert K.lib.kvarn_params_from_dtype(None, 8, ctypes.byref(out)) == INVALID
    with pytest.raises(K.KvarnError):
        K.params_from_dtype("kvarn_k8v8_g128")


def test_page_bytes():
    p = K.params_from_dtype()
    assert K.page_bytes(p, K.KIND_K) == 9216 and K.page_bytes(p, K.KIND_V) == 5120
    assert K.page_bytes(p, 7) == 0
    p2 = K.params_from_dtype("kvarn_k2v2_g128")
    assert K.page_bytes(p2, K.KIND_K) == 5120 and K.page_bytes(p2, K.KIND_V) == 5120
    p4 = K.params_from_dtype("kvarn_k4v4_g128")
    assert K.page_bytes(p4, K.KIND_K) == 9216 and K.page_bytes(p4, K.KIND_V) == 9216
    bad = K.Params(128, 64, 4, 2, 128, 8, 1)
    assert K.lib.kvarn_params_check(ctypes.byref(bad)) == UNSUP
    assert K.page_bytes(bad, K.KIND_K) == 0
    # folded format: 3 metadata vectors instead of 4
    for preset, kb, vb in (("kvarn_k4v2_g128", 8960, 4864), ("kvarn_k2v2_g128", 4864, 4864),
                           ("kvarn_k4v4_g128", 8960, 8960)):
        pf = K.params_from_dtype(preset, 8, format=K.FORMAT_FOLDED)
        assert (K.page_bytes(pf, K.KIND_K), K.page_bytes(pf, K.KIND_V)) == (kb, vb)
    # group 64: two scale and two zero vectors instead of one each (+512 B), both formats
    for preset, kb, vb in (("kvarn_k4v2_g64", 9728, 5632), ("kvarn_k2v2_g64", 5632, 5632),
                           ("kvarn_k4v4_g64", 9728, 9728)):
        pg = K.params_from_dtype(preset, 8)
        assert (K.page_bytes(pg, K.KIND_K), K.page_bytes(pg, K.KIND_V)) == (kb, vb)
        pgf = K.params_from_dtype(preset, 8, format=K.FORMAT_FOLDED)
        assert (K.page_bytes(pgf, K.KIND_K), K.page_bytes(pgf, K.KIND_V)) == (kb - 256, vb - 256)
    for grp in (32, 96, 256, 0):
        pg = K.params_from_dtype()
        pg.group = grp
        assert K.lib.kvarn_params_check(ctypes.byref(pg)) == (INVALID if grp == 0 else UNSUP)
        assert K.page_bytes(pg, K.KIND_K) == 0
    for fmt in (0, 3, -1):
        pf = K.params_from_dtype()
        pf.format = fmt
        assert K.lib.kvarn_params_check(ctypes.byref(pf)) == INVALID
        assert K.page_bytes(pf, K.KIND_K) == 0
    with pytest.raises(K.KvarnError):
        K.params_from_dtype("kvarn_k4v2_g128", 8, format=3)


def _quant(p, **kw):
    a = dict(kind=0, src=FAKE, ts=1024, hs=128, ntok=4096, tok=FAKE, page=FAKE, n=1, hkv=8,
             pool=FAKE, npages=10)
    a.update(kw)
    return K.lib.kvarn_quantize_tiles(ctypes.byref(p), a["kind"], a["src"], a["ts"], a["hs"],
                                      a["ntok"], a["tok"], a["page"], a["n"], a["hkv"],
                                      a["pool"], a["npages"], None)


def test_quantize_validation():
    p = K.params_from_dtype()
    assert _quant(p, n=0) == OK                       # no-op, nothing enqueued
    assert _quant(p, src=None) == INVALID
    assert _quant(p, pool=None) == INVALID
    assert _quant(p, tok=None) == INVALID
    assert _quant(p, kind=2) == INVALID
    assert _quant(p, n=-1) == INVALID
    assert _quant(p, hkv=0) == INVALID
    assert _quant(p, ts=1023) == INVALID              # stride not a multiple of 8
    assert _quant(p, src=ctypes.c_void_p(0x10008)) == INVALID   # misaligned
    assert _quant(p, ntok=-1) == INVALID
    bad = K.Params(128, 128, 2, 4, 128, 8, 1)
    assert _quant(bad) == UNSUP
    assert K.lib.kvarn_quantize_tiles(None, 0, FAKE, 8, 8, 1, FAKE, FAKE, 1, 1, FAKE, 1, None) == INVALID


def _quant_kv(p, **kw):
    a = dict(ksrc=FAKE, vsrc=FAKE, ts=1024, hs=128, ntok=4096, tok=FAKE, page=FAKE, n=1, hkv=8,
             kpool=FAKE, vpool=FAKE, npages=10)
    a.update(kw)
    return K.lib.kvarn_quantize_kv_tiles(ctypes.byref(p), a["ksrc"], a["vsrc"], a["ts"], a["hs"],
                                         a["ntok"], a["tok"], a["page"], a["n"], a["hkv"],
                                         a["kpool"], a["vpool"], a["npages"], None)


def test_quantize_kv_validation():
    p = K.params_from_dtype()
    assert _quant_kv(p, n=0) == OK
    assert _quant_kv(p, ksrc=None) == INVALID
    assert _quant_kv(p, vsrc=None) == INVALID
    assert _quant_kv(p, vpool=None) == INVALID
    assert _quant_kv(p, page=None) == INVALID
    assert _quant_kv(p, n=-1) == INVALID
    assert _quant_kv(p, hkv=0) == INVALID
    assert _quant_kv(p, hs=100) == INVALID            # stride not a multiple of 8
    assert _quant_kv(p, vsrc=ctypes.c_void_p(0x10004)) == INVALID
    assert _quant_kv(p, kpool=ctypes.c_void_p(0x10008)) == INVALID
    assert _quant_kv(p, npages=-1) == INVALID
    assert _quant_kv(K.Params(128, 128, 2, 4, 128, 8, 1)) == UNSUP


def _dequant(p, **kw):
    a = dict(kind=0, pool=FAKE, npages=10, pages=FAKE, n=1, hkv=8, dst=FAKE)
    a.update(kw)
    return K.lib.kvarn_dequantize_tiles(ctypes.byref(p), a["kind"], a["pool"], a["npages"],
                                        a["pages"], a["n"], a["hkv"], a["dst"], None)


def test_dequantize_validation():
    p = K.params_from_dtype()
    assert _dequant(p, n=0) == OK
    assert _dequant(p, kind=3) == INVALID
    assert _dequant(p, pool=None) == INVALID
    assert _dequant(p, pages=None) == INVALID
    assert _dequant(p, dst=None) == INVALID
    assert _dequant(p, hkv=0) == INVALID
    assert _dequant(p, npages=-2) == INVALID
    assert _dequant(p, dst=ctypes.c_void_p(0x10002)) == INVALID
    assert _dequant(K.Params(128, 128, 2, 4, 128, 8, 1)) == UNSUP


def _write(p, **kw):
    a = dict(kn=FAKE, vn=FAKE, total=1000, cu=FAKE, mx=512, B=4, hkv=8, sl=FAKE, kt=FAKE, vt=FAKE,
             bt=FAKE, bts=64, kp=FAKE, vp=FAKE, npages=100)
    a.update(kw)
    return K.lib.kvarn_write_tokens(ctypes.byref(p), a["kn"], a["vn"], a["total"], a["cu"], a["mx"],
                                    a["B"], a["hkv"], a["sl"], a["kt"], a["vt"], a["bt"], a["bts"],
                                    a["kp"], a["vp"], a["npages"], None)


def test_write_tokens_validation():
    p = K.params_from_dtype()
    assert _write(p, B=0) == OK
    assert _write(p, mx=0) == OK
    assert _write(p, total=0) == OK
    assert _write(p, B=-1) == INVALID
    assert _write(p, mx=-1) == INVALID
    assert _write(p, total=-5) == INVALID
    assert _write(p, hkv=0) == INVALID
    assert _write(p, hkv=40000) == INVALID            # grid z = 2 * Hkv
    assert _write(p, bts=0) == INVALID
    assert _write(p, cu=None) == INVALID
    assert _write(p, vt=None) == INVALID
    assert _write(p, kn=ctypes.c_void_p(0x10004)) == INVALID
    assert _write(p, vp=ctypes.c_void_p(0x10008)) == INVALID
    assert _write(p, npages=-1) == INVALID
    assert _write(K.Params(128, 128, 2, 4, 128, 8, 1)) == UNSUP


def _decode(p, **kw):
    a = dict(q=FAKE, B=2, hq=64, hkv=8, kp=FAKE, vp=FAKE, npages=100, bt=FAKE, bts=200, sl=FAKE,
             mx=16384, kt=None, vt=None, scale=0.088, ws=FAKE, wsb=1 << 30, out=FAKE)
    a.update(kw)
    return K.lib.kvarn_decode_attention(ctypes.byref(p), a["q"], a["B"], a["hq"], a["hkv"], a["kp"],
                                        a["vp"], a["npages"], a["bt"], a["bts"], a["sl"], a["mx"],
                                        a["kt"], a["vt"], a["scale"], a["ws"], a["wsb"], a["out"], None)


def test_decode_validation():
    p = K.params_from_dtype()
    assert _decode(p, B=0) == OK
    assert _decode(p, hq=63) == INVALID               # not a multiple of hkv
    assert _decode(p, hq=128) == UNSUP                # 16 query heads per KV head
    assert _decode(p, B=70000) == UNSUP               # more sequences than merge grid rows
    assert _decode(p, B=40000, hq=65535, hkv=65535) == UNSUP   # B * Hkv above INT32_MAX
    assert _decode(p, q=None) == INVALID
    assert _decode(p, kt=FAKE) == INVALID             # one tail without the other
    assert _decode(p, bts=10) == INVALID              # block table narrower than max pages
    assert _decode(p, scale=float("nan")) == INVALID
    assert _decode(p, out=ctypes.c_void_p(0x10002)) == INVALID
    assert _decode(p, wsb=16) == WS
    need = K.decode_workspace_bytes(p, 2, 64, 8, 16384)
    assert _decode(p, wsb=need - 1) == WS


def _noalloc(p, **kw):
    a = dict(q=FAKE, B=2, hq=64, hkv=8, kp=FAKE, vp=FAKE, npages=100, bt=FAKE, bts=200, sl=FAKE,
             mx=16384, kt=None, vt=None, scale=0.088, out=FAKE)
    a.update(kw)
    return K.lib.kvarn_decode_attention_noalloc(ctypes.byref(p), a["q"], a["B"], a["hq"], a["hkv"],
                                                a["kp"], a["vp"], a["npages"], a["bt"], a["bts"],
                                                a["sl"], a["mx"], a["kt"], a["vt"], a["scale"],
                                                a["out"], None)


def test_decode_noalloc_validation():
    """The entry point that allocates nothing: the checks of kvarn_decode_attention, and
    KVARN_ERR_WORKSPACE for a shape whose workspace exceeds the fixed 32 MiB scratch (all
    rejected on the host, before any HIP call)."""
    p = K.params_from_dtype()
    cap = K.decode_noalloc_max_workspace_bytes()
    assert cap == 32 << 20
    assert _noalloc(p, B=0) == OK
    assert _noalloc(p, hq=63) == INVALID
    assert _noalloc(p, hq=128) == UNSUP
    assert _noalloc(p, B=70000) == UNSUP
    assert _noalloc(p, q=None) == INVALID
    assert _noalloc(p, out=None) == INVALID
    assert _noalloc(p, kt=FAKE) == INVALID
    assert _noalloc(p, bts=10) == INVALID
    assert _noalloc(p, scale=float("nan")) == INVALID
    assert _noalloc(p, out=ctypes.c_void_p(0x10002)) == INVALID
    assert _noalloc(p, kp=None) == INVALID
    # 1024 sequences of 4096 tokens need ~78 MB of partials: more than the scratch holds
    big = K.decode_workspace_bytes(p, 1024, 64, 8, 4096)
    assert big > cap
    assert _noalloc(p, B=1024, bts=64, mx=4096) == WS
    # the decode workloads' shapes fit
    for B, mx in ((1, 16384), (32, 32784), (1, 131136), (64, 16384)):
        assert K.decode_workspace_bytes(p, B, 64, 8, mx) <= cap, (B, mx)


def _chunk(p, **kw):
    a = dict(q=FAKE, tq=16, cu=FAKE, B=2, hq=64, hkv=8, kp=FAKE, vp=FAKE, npages=100, bt=FAKE,
             bts=200, sl=FAKE, mx=16384, kt=None, vt=None, scale=0.088, ws=FAKE, wsb=1 << 30,
             out=FAKE)
    a.update(kw)
    return K.lib.kvarn_chunk_attention(ctypes.byref(p), a["q"], a["tq"], a["cu"], a["B"], a["hq"],
                                       a["hkv"], a["kp"], a["vp"], a["npages"], a["bt"], a["bts"],
                                       a["sl"], a["mx"], a["kt"], a["vt"], a["scale"], a["ws"],
                                       a["wsb"], a["out"], None)


def test_chunk_attention_validation():
    p = K.params_from_dtype()
    assert _chunk(p, tq=0) == OK
    assert _chunk(p, B=0) == INVALID                  # rows without a sequence
    assert _chunk(p, tq=-1) == INVALID
    assert _chunk(p, tq=70000) == UNSUP
    assert _chunk(p, tq=40000, hq=65535, hkv=65535) == UNSUP   # rows * Hkv above INT32_MAX
    assert _chunk(p, cu=None) == INVALID
    assert _chunk(p, hq=63) == INVALID
    assert _chunk(p, hq=128) == UNSUP
    assert _chunk(p, kt=FAKE) == INVALID
    assert _chunk(p, bts=10) == INVALID
    assert _chunk(p, scale=float("inf")) == INVALID
    assert _chunk(p, q=ctypes.c_void_p(0x10002)) == INVALID
    need = K.chunk_workspace_bytes(p, 16, 64, 8, 16384)
    assert need >= 16 * 64 * (K.decode_num_splits(p, 16, 8, 16384) + 1) * 132 * 4   # split layout
    assert _chunk(p, wsb=need - 1) == WS


def test_chunk_workspace_formula():
    """Either read layout fits: the workspace holds max(decode splits, multi-query splits) + 1
    partials per (row, query head)."""
    p = K.params_from_dtype()
    for tq, hq, hkv, mx in ((1024, 64, 8, 16512), (16, 64, 8, 16384), (3, 8, 8, 100),
                            (200, 8, 1, 131072), (65535, 8, 8, 1024)):
        b = K.chunk_workspace_bytes(p, tq, hq, hkv, mx)
        d = tq * hq * (K.decode_num_splits(p, tq, hkv, mx) + 1) * 132 * 4   # split layout
        assert b >= d and b % (tq * hq * 132 * 4) == 0
        ns = b // (tq * hq * 132 * 4) - 1
        assert 1 <= ns <= max(1, mx // 128)
    assert K.chunk_workspace_bytes(p, 0, 64, 8, 1024) == 0
    assert K.chunk_workspace_bytes(p, 70000, 64, 8, 1024) == 0
    assert K.chunk_workspace_bytes(p, 16, 128, 8, 1024) == 0


def _balanced_bytes(B, hq, hkv, mx):
    """Workspace of the balanced decode layout (2..1024 sequences): one partial slot per (page
    wave, segment) index sum i + (b Hkv + g) with i < 4 x page workgroups (at most 512, one
    round of 2 waves per SIMD on 256 CUs), G query heads each; one tail partial per (b, query
    head); then B + 1 int32 page prefix sums."""
    work = B * hkv * (mx // 128)
    if B < 2 or B > 1024 or mx < 128 or work >= 2 ** 31:
        return 0
    wg = min((work + 3) // 4, 512)
    return (((4 * wg + B * hkv) * (hq // hkv) + B * hq) * 132 + B + 1) * 4


def test_decode_workspace_formula():
    p = K.params_from_dtype()
    for B, hq, hkv, mx in ((1, 64, 8, 16384), (32, 64, 8, 32768), (1, 64, 8, 131072),
                           (64, 64, 8, 16384), (3, 8, 8, 100), (4, 16, 2, 1400),
                           (1024, 64, 8, 4096), (1025, 64, 8, 4096)):
        ns = K.decode_num_splits(p, B, hkv, mx)
        assert ns >= 1
        split = B * hq * (ns + 1) * 132 * 4
        want = max(split, _balanced_bytes(B, hq, hkv, mx))
        assert K.decode_workspace_bytes(p, B, hq, hkv, mx) == want
    assert K.decode_workspace_bytes(p, 1, 64, 8, -1) == 0
    assert K.decode_workspace_bytes(p, 1, 128, 8, 1024) == 0
