"""C-ABI checks that need no GPU: exported symbols and the validation paths.

Every call here fails validation (or is a pure host query), so nothing is ever
enqueued and no device is touched.  Pointers are fake, aligned addresses.
"""
import ctypes
import os
import re

import pytest

from bit_flashattention_hifa4_amd import binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bit_flashattention_hifa4_amd")


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    return re.findall(r"^HIFA4\w*_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


@pytest.mark.parametrize("header,lib", [("hifa4.h", "libhifa4.so"),
                                        ("hifa4_probes.h", "libhifa4_probes.so")])
def test_library_exports_every_declared_symbol(header, lib):
    names = _declared(header)
    assert len(names) >= 6
    so = ctypes.CDLL(os.path.join(PKG, lib))
    for n in names:
        assert hasattr(so, n), "%s does not export %s" % (lib, n)


@pytest.fixture(scope="module")
def lib():
    return hb.load_library()


A = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)


def _mx(base):
    return hb.MxTensorC(base, base + 0x1000000)


def _quant(lib, **kw):
    args = dict(q=A, k=A + 0x4000000, v=A + 0x8000000, dt=hb.HIFA4_BF16, B=1, Hq=4, Hkv=2, Sq=64,
                Sk=64, stride=0, d=128, smooth=None, qo=_mx(0x20000000), ko=_mx(0x40000000),
                vo=_mx(0x60000000))
    args.update(kw)
    return lib.hifa4_quantize_qkv(args["q"], args["k"], args["v"], args["dt"], args["B"],
                                  args["Hq"], args["Hkv"], args["Sq"], args["Sk"], args["stride"],
                                  args["d"], args["smooth"], args["qo"], args["ko"], args["vo"],
                                  None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=96), hb.HIFA4_ERR_UNSUPPORTED, "head dim"),
    (dict(Hq=3), hb.HIFA4_ERR_INVALID_ARGUMENT, "Hq % Hkv"),
    (dict(B=-1), hb.HIFA4_ERR_INVALID_ARGUMENT, "negative"),
    (dict(dt=7), hb.HIFA4_ERR_INVALID_ARGUMENT, "in_dtype"),
    (dict(stride=32), hb.HIFA4_ERR_INVALID_ARGUMENT, "kv_stride"),
    (dict(q=A + 8), hb.HIFA4_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(qo=hb.MxTensorC(None, 0x20000000)), hb.HIFA4_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(q=None, k=None, v=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "all NULL"),
    (dict(ko=_mx(A + 0x100)), hb.HIFA4_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(vo=hb.MxTensorC(0x20000000, 0x61000000)), hb.HIFA4_ERR_INVALID_ARGUMENT, "overlap"),
])
def test_quantize_rejects_bad_arguments(lib, kw, status, msg):
    assert _quant(lib, **kw) == status
    assert msg in hb.hifa4_last_error()


def _params(**kw):
    p = dict(B=2, Hq=8, Hkv=2, Sq=128, Sk=128, d=128, causal=True, sm_scale=None, kv_stride=0,
             kv_lens=None, decode_chunk=0, normaliser=0)
    p.update(kw)
    lens = p.pop("kv_lens")
    params = hb.make_params(**{k: p[k] for k in ("B", "Hq", "Hkv", "Sq", "Sk", "d")},
                            causal=p["causal"], sm_scale=p["sm_scale"], kv_stride=p["kv_stride"],
                            decode_chunk=p["decode_chunk"], normaliser=p["normaliser"])
    if lens is not None:
        params.kv_lens = lens
    return params


def _attn(lib, params, ws=None, ws_bytes=0, out=0x70000000):
    return lib.hifa4_attn_fwd(ctypes.byref(params), _mx(0x10000000), _mx(0x20000000),
                              _mx(0x30000000), out, hb.HIFA4_BF16, None, ws, ws_bytes, None)


def test_schedule_and_workspace_are_host_queries(lib):
    p = _params()
    bn, ch = hb.hifa4_attn_schedule(p)
    assert bn == 64 and ch == 0
    assert hb.hifa4_attn_workspace_size(p) == 0
    assert hb.hifa4_attn_decode_piece_tiles(p, 100) == 0      # prefill: no decode schedule
    # balanced decode: one partial row of G = 4 heads x (m, l, 2 unused, acc[128]) per
    # (piece, pair) run, at row piece + pair: W + pairs - 1 rows for a W-wave grid
    d = _params(Sq=1, Sk=5000, kv_stride=8192)
    bn, ch = hb.hifa4_attn_schedule(d)
    assert ch == 0
    row_bytes = 4 * (128 + 4) * 4
    need = hb.hifa4_attn_workspace_size(d)
    assert need % row_bytes == 0
    waves = need // row_bytes - 4 + 1                         # B * Hkv = 4 pairs
    assert waves >= 256
    for total in (0, 1, waves - 1, waves, waves + 1, 3 * waves, 79 * 4):
        pt = hb.hifa4_attn_decode_piece_tiles(d, total)
        assert pt == max(1, -(-total // waves))
        assert -(-total // pt) <= waves                       # never more pieces than waves
    # a caller's piece length: pieces of decode_chunk / 64 tiles over at most
    # B * Hkv * ceil(Sk / 64) = 4 * 79 tiles
    d2 = _params(Sq=1, Sk=5000, decode_chunk=bn * 3)
    assert hb.hifa4_attn_schedule(d2)[1] == bn * 3
    assert hb.hifa4_attn_decode_piece_tiles(d2, 1000) == 3
    assert hb.hifa4_attn_workspace_size(d2) == (-(-(4 * 79) // 3) + 4 - 1) * row_bytes
    assert hb.hifa4_attn_workspace_size(_params(Sq=1, Sk=0)) == 0   # no keys
    assert hb.hifa4_attn_workspace_size(_params(d=100)) == 0   # invalid -> 0
    assert hb.hifa4_attn_decode_piece_tiles(_params(Sq=1, d=100), 10) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=32), hb.HIFA4_ERR_UNSUPPORTED, "head dim"),
    (dict(Hkv=3), hb.HIFA4_ERR_INVALID_ARGUMENT, "Hq % Hkv"),
    (dict(kv_lens=0x5000000), hb.HIFA4_ERR_UNSUPPORTED, "kv_lens"),
    (dict(decode_chunk=64), hb.HIFA4_ERR_INVALID_ARGUMENT, "decode_chunk"),
    (dict(Sq=1, decode_chunk=100), hb.HIFA4_ERR_INVALID_ARGUMENT, "decode_chunk"),
    (dict(Sq=1, decode_chunk=-64), hb.HIFA4_ERR_INVALID_ARGUMENT, "decode_chunk"),
    (dict(Sq=1, B=1 << 20, Hq=64, Hkv=64, Sk=1 << 20), hb.HIFA4_ERR_UNSUPPORTED, "too large"),
    (dict(kv_stride=64), hb.HIFA4_ERR_INVALID_ARGUMENT, "kv_stride"),
    (dict(sm_scale=float("nan")), hb.HIFA4_ERR_INVALID_ARGUMENT, "sm_scale"),
    (dict(normaliser=2), hb.HIFA4_ERR_INVALID_ARGUMENT, "normaliser"),
])
def test_attn_rejects_bad_params(lib, kw, status, msg):
    assert _attn(lib, _params(**kw)) == status
    assert msg in hb.hifa4_last_error()


def test_attn_workspace_and_pointer_checks(lib):
    d = _params(Sq=1, Sk=3000)
    assert _attn(lib, d, ws=0x7F000000, ws_bytes=16) == hb.HIFA4_ERR_WORKSPACE_TOO_SMALL
    assert _attn(lib, _params(), out=None) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert _attn(lib, _params(), out=0x70000008) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert _attn(lib, _params(), out=0x10000000) == hb.HIFA4_ERR_INVALID_ARGUMENT   # aliases q
    assert "overlaps" in hb.hifa4_last_error()
    assert lib.hifa4_attn_fwd(None, _mx(0x10000000), _mx(0x20000000), _mx(0x30000000), 0x70000000,
                              hb.HIFA4_BF16, None, None, 0, None) == hb.HIFA4_ERR_INVALID_ARGUMENT


def test_attn_qraw_validation(lib):
    def call(params, q=0x10000000, q_dtype=hb.HIFA4_BF16, smooth=None):
        return lib.hifa4_attn_fwd_qraw(ctypes.byref(params), q, q_dtype, smooth, _mx(0x20000000),
                                       _mx(0x30000000), 0x70000000, hb.HIFA4_BF16, None, None, 0,
                                       None)
    assert call(_params(), q=None) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "q is NULL" in hb.hifa4_last_error()
    assert call(_params(Sq=1)) == hb.HIFA4_ERR_UNSUPPORTED
    assert "prefill" in hb.hifa4_last_error()
    assert call(_params(), q_dtype=7) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert call(_params(), q=0x10000004) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "not 16-byte aligned" in hb.hifa4_last_error()
    assert call(_params(), smooth=0x40000004) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "smooth" in hb.hifa4_last_error()
    assert call(_params(d=32)) == hb.HIFA4_ERR_UNSUPPORTED


def test_bf16_path_rejects_bad_arguments(lib):
    p = _params()
    assert lib.bf16_attn_fwd(ctypes.byref(p), A, A + 0x1000000, A + 0x2000000, A + 0x10, None, None,
                             0, None) == hb.HIFA4_ERR_INVALID_ARGUMENT
    p = _params(kv_lens=0x5000000, Sq=1)
    assert lib.bf16_attn_fwd(ctypes.byref(p), A, A + 0x1000000, A + 0x2000000, A + 0x3000000, None,
                             None, 0, None) == hb.HIFA4_ERR_UNSUPPORTED
    p = _params(d=48)
    assert lib.bf16_attn_fwd(ctypes.byref(p), A, A + 0x1000000, A + 0x2000000, A + 0x3000000, None,
                             None, 0, None) == hb.HIFA4_ERR_UNSUPPORTED
    p = _params(normaliser=1)
    assert lib.bf16_attn_fwd(ctypes.byref(p), A, A + 0x1000000, A + 0x2000000, A + 0x3000000, None,
                             None, 0, None) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "normaliser" in hb.hifa4_last_error()


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert hb.hifa4_status_string(s)
    assert hb.hifa4_status_string(5) == "unknown status"
