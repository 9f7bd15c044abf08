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
    (dict(ko=hb.MxTensorC(0x40000000, 0x41000000, 2)), hb.HIFA4_ERR_INVALID_ARGUMENT,
     "scale_rule"),
    (dict(qo=hb.MxTensorC(0x20000000, 0x21000000, -1)), hb.HIFA4_ERR_INVALID_ARGUMENT,
     "scale_rule"),
])
def test_quantize_rejects_bad_arguments(lib, kw, status, msg):
    assert _quant(lib, **kw) == status
    assert msg in hb.hifa4_last_error()


def _quant_rope(lib, rope, **kw):
    args = dict(q=A, k=A + 0x4000000, v=A + 0x8000000, dt=hb.HIFA4_BF16, B=1, Hq=4, Hkv=2, Sq=64,
                Sk=64, stride=0, d=128, smooth=None, qo=_mx(0x20000000), ko=_mx(0x40000000),
                vo=_mx(0x60000000))
    args.update(kw)
    return lib.hifa4_quantize_qkv_rope(args["q"], args["k"], args["v"], args["dt"], args["B"],
                                       args["Hq"], args["Hkv"], args["Sq"], args["Sk"],
                                       args["stride"], args["d"], args["smooth"],
                                       ctypes.byref(rope) if rope is not None else None,
                                       args["qo"], args["ko"], args["vo"], None)


T = 0x7000000  # fake table address, clear of every buffer above


def _rope(**kw):
    r = dict(cos=T, sin=T + 0x100000, n_pos=128, q_pos0=0, k_pos0=0)
    r.update(kw)
    return hb.RopeC(r["cos"], r["sin"], r["n_pos"], r["q_pos0"], r["k_pos0"])


@pytest.mark.parametrize("rope,kw,status,msg", [
    (None, {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "rope is NULL"),
    (dict(sin=None), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "table is NULL"),
    (dict(cos=T + 4), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(n_pos=-1), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "negative"),
    (dict(q_pos0=-2), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "negative"),
    (dict(q_pos0=65), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "query positions"),
    (dict(k_pos0=100), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "key positions"),
    (dict(n_pos=63), dict(k=None, v=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "query positions"),
    (dict(cos=0x20000000), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "overlaps input rope.cos"),
    (dict(d_bad=True), dict(d=96), hb.HIFA4_ERR_UNSUPPORTED, "head dim"),
])
def test_quantize_rope_rejects_bad_arguments(lib, rope, kw, status, msg):
    if rope is not None:
        rope.pop("d_bad", None)
    assert _quant_rope(lib, _rope(**rope) if rope is not None else None, **kw) == status
    assert msg in hb.hifa4_last_error()


def test_quantize_rope_positions_only_checked_for_given_tensors(lib):
    # Key positions past the table are an error only when K is given.  Each call still
    # fails validation (q_out overlaps q), so nothing is enqueued.
    r = _rope(k_pos0=1000)
    assert _quant_rope(lib, r, k=None, v=None, qo=_mx(A)) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "overlaps input q" in hb.hifa4_last_error()
    assert _quant_rope(lib, r, qo=_mx(A)) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "key positions" in hb.hifa4_last_error()


def _append(lib, rope=None, **kw):
    args = dict(q=A, k=A + 0x4000000, v=A + 0x8000000, dt=hb.HIFA4_BF16, B=2, Hq=4, Hkv=2, n=1,
                cap=256, d=128, lens=0x9000000, lens_out=0x9001000, smooth=None,
                tail=0x9100000, qo=_mx(0x20000000), kc=_mx(0x40000000), vc=_mx(0x60000000))
    args.update(kw)
    return lib.hifa4_kv_append(args["q"], args["k"], args["v"], args["dt"], args["B"], args["Hq"],
                               args["Hkv"], args["n"], args["cap"], args["d"], args["lens"],
                               args["lens_out"], args["smooth"],
                               ctypes.byref(rope) if rope is not None else None, args["tail"],
                               args["qo"], args["kc"], args["vc"], None)


@pytest.mark.parametrize("rope,kw,status,msg", [
    (None, dict(d=96), hb.HIFA4_ERR_UNSUPPORTED, "head dim"),
    (None, dict(cap=0), hb.HIFA4_ERR_INVALID_ARGUMENT, "capacity"),
    (None, dict(n=-1), hb.HIFA4_ERR_INVALID_ARGUMENT, "negative"),
    (None, dict(Hq=5), hb.HIFA4_ERR_INVALID_ARGUMENT, "Hq % Hkv"),
    (None, dict(lens=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "kv_lens is NULL"),
    (None, dict(tail=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "v_tail is NULL"),
    (None, dict(k=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "k is NULL"),
    (None, dict(qo=hb.MxTensorC(None, 0x20000000)), hb.HIFA4_ERR_INVALID_ARGUMENT, "q_out.codes"),
    (None, dict(lens_out=0x9000004), hb.HIFA4_ERR_INVALID_ARGUMENT, "aligned"),
    (None, dict(lens_out=0x9000000), hb.HIFA4_ERR_INVALID_ARGUMENT, "kv_lens_out overlaps input kv_lens"),
    (None, dict(tail=0x40000100), hb.HIFA4_ERR_INVALID_ARGUMENT, "overlap"),
    (None, dict(kc=_mx(A + 0x40)), hb.HIFA4_ERR_INVALID_ARGUMENT, "overlaps input q"),
    (None, dict(vc=hb.MxTensorC(0x60000000, 0x61000000, 3)), hb.HIFA4_ERR_INVALID_ARGUMENT,
     "scale_rule"),
    (dict(n_pos=0), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "n_pos >= 1"),
    (dict(cos=None), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "table is NULL"),
    (dict(q_pos0=0x7FFFFF00), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "overflow"),
    (dict(sin=0x9100000), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "v_tail overlaps input rope.sin"),
])
def test_kv_append_rejects_bad_arguments(lib, rope, kw, status, msg):
    assert _append(lib, _rope(**rope) if rope is not None else None, **kw) == status
    assert msg in hb.hifa4_last_error()


def test_kv_append_allows_null_kv_only_when_empty(lib):
    # n = 0: k and v may be NULL; the call still validates the rest (here: an overlap)
    assert _append(lib, k=None, v=None, n=0, tail=0x40000100) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "overlap" in hb.hifa4_last_error()
    assert _append(lib, k=None, n=1) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "k is NULL" in hb.hifa4_last_error()


def _calib(lib, rope=None, **kw):
    args = dict(q=A, k=A + 0x4000000, dt=hb.HIFA4_BF16, B=1, Hq=4, Hkv=2, S=64, d=128, alpha=0.5,
                out=0x20000000, ws=0x30000000, ws_bytes=2 * 2 * 128 * 4)
    args.update(kw)
    return lib.hifa4_smooth_calibrate(args["q"], args["k"], args["dt"], args["B"], args["Hq"],
                                      args["Hkv"], args["S"], args["d"],
                                      ctypes.byref(rope) if rope is not None else None,
                                      args["alpha"], args["out"], args["ws"], args["ws_bytes"],
                                      None)


@pytest.mark.parametrize("rope,kw,status,msg", [
    (None, dict(d=96), hb.HIFA4_ERR_UNSUPPORTED, "head dim"),
    (None, dict(Hq=3), hb.HIFA4_ERR_INVALID_ARGUMENT, "Hq % Hkv"),
    (None, dict(S=-1), hb.HIFA4_ERR_INVALID_ARGUMENT, "negative"),
    (None, dict(dt=5), hb.HIFA4_ERR_INVALID_ARGUMENT, "in_dtype"),
    (None, dict(alpha=float("nan")), hb.HIFA4_ERR_INVALID_ARGUMENT, "alpha"),
    (None, dict(alpha=float("inf")), hb.HIFA4_ERR_INVALID_ARGUMENT, "alpha"),
    (None, dict(k=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "NULL"),
    (None, dict(q=A + 2), hb.HIFA4_ERR_INVALID_ARGUMENT, "aligned"),
    (None, dict(out=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "smooth_out"),
    (None, dict(ws=None), hb.HIFA4_ERR_INVALID_ARGUMENT, "workspace"),
    (None, dict(ws_bytes=2047), hb.HIFA4_ERR_WORKSPACE_TOO_SMALL, "need 2048"),
    (None, dict(out=A + 0x100), hb.HIFA4_ERR_INVALID_ARGUMENT, "overlaps input q"),
    (None, dict(ws=0x20000200), hb.HIFA4_ERR_INVALID_ARGUMENT, "overlap"),
    (dict(k_pos0=70), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "key positions"),
    (dict(sin=0x30000000), {}, hb.HIFA4_ERR_INVALID_ARGUMENT, "workspace overlaps input rope.sin"),
])
def test_calibrate_rejects_bad_arguments(lib, rope, kw, status, msg):
    assert _calib(lib, _rope(**rope) if rope is not None else None, **kw) == status
    assert msg in hb.hifa4_last_error()


def test_calibrate_workspace_size(lib):
    assert lib.hifa4_smooth_calibrate_workspace_size(8, 128) == 2 * 8 * 128 * 4
    assert lib.hifa4_smooth_calibrate_workspace_size(1, 64) == 512
    assert lib.hifa4_smooth_calibrate_workspace_size(0, 128) == 0
    assert lib.hifa4_smooth_calibrate_workspace_size(2, 96) == 0


def _params(**kw):
    p = dict(B=2, Hq=8, Hkv=2, Sq=128, Sk=128, d=128, causal=True, sm_scale=None, kv_stride=0,
             kv_lens=None, decode_chunk=0, normaliser=0, scale_rule=0, rescale_threshold=0.0)
    p.update(kw)
    lens = p.pop("kv_lens")
    params = hb.make_params(**{k: p[k] for k in ("B", "Hq", "Hkv", "Sq", "Sk", "d")},
                            causal=p["causal"], sm_scale=p["sm_scale"], kv_stride=p["kv_stride"],
                            decode_chunk=p["decode_chunk"], normaliser=p["normaliser"],
                            scale_rule=p["scale_rule"],
                            rescale_threshold=p["rescale_threshold"])
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
    (dict(scale_rule=2), hb.HIFA4_ERR_INVALID_ARGUMENT, "scale_rule"),
    (dict(Sq=1, scale_rule=-1), hb.HIFA4_ERR_INVALID_ARGUMENT, "scale_rule"),
    # P reaches 2^threshold: past 64 the fp32 accumulators could overflow
    (dict(rescale_threshold=64.5), hb.HIFA4_ERR_INVALID_ARGUMENT, "rescale_threshold"),
    (dict(rescale_threshold=-1.0), hb.HIFA4_ERR_INVALID_ARGUMENT, "rescale_threshold"),
    # a head's codes are addressed with 32-bit offsets: Sk * d / 2 must stay below 2^31
    (dict(Sk=1 << 24, d=256), hb.HIFA4_ERR_UNSUPPORTED, "2^31 bytes"),
    (dict(Sq=1, Sk=(1 << 24) - 16, d=256), hb.HIFA4_ERR_UNSUPPORTED, "2^31 bytes"),
])
def test_attn_rejects_bad_params(lib, kw, status, msg):
    assert _attn(lib, _params(**kw)) == status
    assert msg in hb.hifa4_last_error()


def test_attn_limits_accept_their_bounds(lib):
    # validation only (no launch): the largest threshold and head size still accepted
    assert hb.hifa4_attn_schedule(_params(rescale_threshold=64.0))[0] == 64
    assert hb.hifa4_attn_schedule(_params(Sk=(1 << 24) - 32, Sq=1 << 23, d=256))[0] == 64


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
    # bf16 keys of one head past 2^31 bytes (a capacity the 4-bit path still takes)
    p = _params(Sk=1 << 22, d=256)
    assert lib.bf16_attn_fwd(ctypes.byref(p), A, A + 0x1000000, A + 0x2000000, A + 0x3000000, None,
                             None, 0, None) == hb.HIFA4_ERR_UNSUPPORTED
    assert "2^31 bytes" in hb.hifa4_last_error()
    p = _params(scale_rule=1)
    assert lib.bf16_attn_fwd(ctypes.byref(p), A, A + 0x1000000, A + 0x2000000, A + 0x3000000, None,
                             None, 0, None) == hb.HIFA4_ERR_INVALID_ARGUMENT
    assert "scale_rule" in hb.hifa4_last_error()


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert hb.hifa4_status_string(s)
    assert hb.hifa4_status_string(5) == "unknown status"


def test_noalloc_refuses_partials_beyond_its_scratch(lib):
    """hifa4_attn_fwd_noalloc: decode partials larger than its device scratch are refused
    before any HIP call (64 sequences x 8 KV heads x 32 query heads each at d = 256)."""
    B, Hkv, G, d, cap = 64, 8, 32, 256, 32768
    p = hb.make_params(B, Hkv * G, Hkv, 1, cap, d, causal=True, kv_stride=cap)
    assert hb.hifa4_attn_workspace_size(p) > hb.NOALLOC_SCRATCH_BYTES
    st = lib.hifa4_attn_fwd_noalloc(ctypes.byref(p), _mx(0x10000000), _mx(0x30000000),
                                    _mx(0x50000000), 0x70000000, hb.HIFA4_BF16, None, None)
    assert st == hb.HIFA4_ERR_UNSUPPORTED
    assert "scratch" in hb.hifa4_last_error()
    # parameters are validated first, as in hifa4_attn_fwd
    st = lib.hifa4_attn_fwd_noalloc(ctypes.byref(_params(d=32)), _mx(0x10000000),
                                    _mx(0x30000000), _mx(0x50000000), 0x70000000, hb.HIFA4_BF16,
                                    None, None)
    assert st == hb.HIFA4_ERR_UNSUPPORTED and "head dim" in hb.hifa4_last_error()
    assert lib.hifa4_attn_fwd_noalloc(None, _mx(0x10000000), _mx(0x30000000), _mx(0x50000000),
                                      0x70000000, hb.HIFA4_BF16, None, None) \
        == hb.HIFA4_ERR_INVALID_ARGUMENT
