"""gfx950 instruction facts the attention kernels depend on (GPU).

Each probe runs one instruction per wave on random operands and compares the
result with a host computation of the hypothesised semantics:
  * scaled FP4 MFMA 32x32x64 / 16x16x128: lane l of A holds row l % M and the
    32-element K block l // M (byte i low nibble = element 2i), its E8M0 scale
    in byte 0 of the scale register; the accumulator holds D[m][n] with
    n = l % N and m as documented in device_common.hpp;
  * bf16 MFMA 32x32x16: lane l holds row / column l % 32, K elements
    8 * (l // 32) .. + 7;
  * v_cvt_scalef32_pk_fp4_f32 rounds x / scale to nearest-even E2M1 with
    saturation, like the oracle's encoder, and writes the selected byte.
  * a memory -> LDS buffer load of `size` bytes per lane writes lane i's
    bytes at M0 + size * i for 4 and 16 bytes; the 1- and 2-byte forms write
    a zero-extended dword at M0 + 4 * i (the prefill kernel stages K / V
    tiles with the 16-, 4- and 2-byte forms).
Also measures the v_exp_f32 and FP4 MFMA issue rates (printed, loosely bounded).
Set HIFA4_PROBE_DUMP=<dir> to save raw operands / results for offline study.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = os.path.join(ROOT, "bit_flashattention_hifa4_amd", "libhifa4_probes.so")
MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
CODE_VAL = np.array([MAG[c & 7] * (-1 if c & 8 else 1) for c in range(16)])


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(PROBES):
        pytest.fail("libhifa4_probes.so is not built")
    l = ctypes.CDLL(PROBES)
    for name in ("probe_mfma_fp4_32x32x64", "probe_mfma_fp4_16x16x128"):
        getattr(l, name).argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_int,
                                                             ctypes.c_void_p]
    l.probe_mfma_bf16_32x32x16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
    l.probe_cvt_pk_fp4.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int,
                                                           ctypes.c_void_p]
    l.probe_half_swap.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    l.probe_exp2_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    l.probe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    l.probe_mfma16_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    l.probe_coexec.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_void_p]
    l.probe_valu_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    l.probe_lds_read_tr16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    l.probe_lds_dma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    l.probe_buffer_range.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    l.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    return l


def _dump(name, **arrays):
    d = os.environ.get("HIFA4_PROBE_DUMP")
    if d:
        os.makedirs(d, exist_ok=True)
        np.savez(os.path.join(d, name + ".npz"), **arrays)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _nibbles(words: np.ndarray) -> np.ndarray:
    """[..., 4] uint32 -> [..., 32] codes, element i = nibble i (little-endian)."""
    b = words.astype("<u4").view(np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def _expected_fp4(a, b, sa, sb, M, N, sel):
    """Host D = A @ B for one wave under the hypothesised lane layout."""
    kb = 64 // M          # K blocks per lane group: 2 for 32x32x64, 4 for 16x16x128
    K = 32 * kb
    A = np.zeros((M, K))
    Bm = np.zeros((K, N))
    ca, cb = _nibbles(a), _nibbles(b)
    sca = ((sa >> (8 * sel)) & 0xFF).astype(np.int64)
    scb = ((sb >> (8 * sel)) & 0xFF).astype(np.int64)
    for l in range(64):
        blk = l // M
        A[l % M, 32 * blk:32 * blk + 32] = CODE_VAL[ca[l]] * 2.0 ** (sca[l] - 127)
        Bm[32 * blk:32 * blk + 32, l % N] = CODE_VAL[cb[l]] * 2.0 ** (scb[l] - 127)
    return A @ Bm


def _acc_index(M, l, r):
    if M == 32:
        return 8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32
    return 4 * (l // 16) + r, l % 16


def _run_fp4(lib, M, opsel, n_waves=64, seed=0, scale_byte=None):
    rng = np.random.default_rng(seed)
    R = 16 if M == 32 else 4
    a = rng.integers(0, 2**32, size=(n_waves, 64, 4), dtype=np.uint64).astype(np.uint32)
    b = rng.integers(0, 2**32, size=(n_waves, 64, 4), dtype=np.uint64).astype(np.uint32)
    sa = rng.integers(0, 2**32, size=(n_waves, 64), dtype=np.uint64).astype(np.uint32)
    sb = rng.integers(0, 2**32, size=(n_waves, 64), dtype=np.uint64).astype(np.uint32)
    sel = 0 if scale_byte is None else scale_byte
    # the scale that matters lives in byte `sel`, in [117, 137]; other bytes are random
    mask = np.uint32(0xFF << (8 * sel))
    sa = (sa & ~mask) | (rng.integers(117, 138, size=sa.shape).astype(np.uint32) << (8 * sel))
    sb = (sb & ~mask) | (rng.integers(117, 138, size=sb.shape).astype(np.uint32) << (8 * sel))
    dev = lambda x: torch.from_numpy(x.view(np.int32)).cuda()
    ta, tb, tsa, tsb = dev(a), dev(b), dev(sa), dev(sb)
    d = torch.zeros((n_waves, 64, R), dtype=torch.float32, device="cuda")
    fn = lib.probe_mfma_fp4_32x32x64 if M == 32 else lib.probe_mfma_fp4_16x16x128
    assert fn(ta.data_ptr(), tb.data_ptr(), tsa.data_ptr(), tsb.data_ptr(), d.data_ptr(), n_waves,
              opsel, _stream()) == 0
    torch.cuda.synchronize()
    return a, b, sa, sb, d.cpu().numpy()


def _compare_fp4(a, b, sa, sb, d, M, sel):
    R = d.shape[-1]
    worst = 0.0
    for w in range(a.shape[0]):
        ref = _expected_fp4(a[w], b[w], sa[w], sb[w], M, M, sel)
        got = np.zeros_like(ref)
        for l in range(64):
            for r in range(R):
                m, n = _acc_index(M, l, r)
                got[m, n] = d[w, l, r]
        err = np.abs(got - ref) / (np.abs(ref).max() + 1e-300)
        worst = max(worst, err.max())
    return worst


@pytest.mark.parametrize("M", [32, 16])
def test_scaled_fp4_mfma_layout(lib, M):
    a, b, sa, sb, d = _run_fp4(lib, M, opsel=0, seed=M)
    _dump("mfma_fp4_%d" % M, a=a, b=b, sa=sa, sb=sb, d=d)
    worst = _compare_fp4(a, b, sa, sb, d, M, 0)
    print("fp4 %dx%d MFMA layout: worst relative error %.3g" % (M, M, worst))
    assert worst < 1e-5


@pytest.mark.parametrize("opsel", [1, 2, 3])
def test_scaled_fp4_mfma_opsel_report(lib, opsel):
    """Which scale byte does a non-zero opsel pick?  Reported; only byte 0 is relied on."""
    a, b, sa, sb, d = _run_fp4(lib, 32, opsel=opsel, seed=100 + opsel, n_waves=8,
                               scale_byte=opsel)
    e_sel = _compare_fp4(a, b, sa, sb, d, 32, opsel)
    e_b0 = _compare_fp4(a, b, sa, sb, d, 32, 0)
    print("opsel=%d: error if byte %d used %.3g, if byte 0 used %.3g" % (opsel, opsel, e_sel, e_b0))
    assert min(e_sel, e_b0) < 1e-5


def test_bf16_mfma_layout(lib):
    rng = np.random.default_rng(5)
    n_waves = 16
    a = torch.randn(n_waves, 64, 8).to(torch.bfloat16)
    b = torch.randn(n_waves, 64, 8).to(torch.bfloat16)
    d = torch.zeros((n_waves, 64, 16), dtype=torch.float32, device="cuda")
    ta, tb = a.cuda(), b.cuda()
    assert lib.probe_mfma_bf16_32x32x16(ta.data_ptr(), tb.data_ptr(), d.data_ptr(), n_waves,
                                        _stream()) == 0
    torch.cuda.synchronize()
    af, bf, dd = a.double().numpy(), b.double().numpy(), d.cpu().numpy()
    for w in range(n_waves):
        A = np.zeros((32, 16))
        Bm = np.zeros((16, 32))
        for l in range(64):
            A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = af[w, l]
            Bm[8 * (l // 32):8 * (l // 32) + 8, l % 32] = bf[w, l]
        ref = A @ Bm
        got = np.zeros_like(ref)
        for l in range(64):
            for r in range(16):
                m, n = _acc_index(32, l, r)
                got[m, n] = dd[w, l, r]
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    del rng


def test_permlane32_swap_exchanges_wave_halves(lib):
    """The kernels take max(r0, r1) of v_permlane32_swap(x, x) as max(x[l], x[l ^ 32])."""
    n_waves = 8
    x = torch.randn(n_waves * 64)
    out = torch.zeros(n_waves * 64 * 2, device="cuda")
    xd = x.cuda()
    assert lib.probe_half_swap(xd.data_ptr(), out.data_ptr(), n_waves, _stream()) == 0
    torch.cuda.synchronize()
    r = out.cpu().numpy().reshape(n_waves, 64, 2)
    xv = x.numpy().reshape(n_waves, 64)
    partner = xv[:, np.arange(64) ^ 32]
    # each lane sees its own value and its partner's, one in each result
    got = np.sort(r, axis=-1)
    want = np.sort(np.stack([xv, partner], axis=-1), axis=-1)
    np.testing.assert_array_equal(got, want)


def _cvt_inputs():
    rng = np.random.default_rng(17)
    pts = [0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0]
    bits = []
    for p in pts:
        c = int(np.array([p], dtype=np.float32).view(np.uint32)[0])
        bits.append(np.arange(c - 2048, c + 2048, dtype=np.int64).astype(np.uint32))
    bits.append(rng.integers(0, 0x41000000, size=1 << 16, dtype=np.uint32))
    bits.append(np.array([0, 0x41000000, 0x42000000], dtype=np.uint32))   # 0, 8, 32
    y = np.concatenate(bits).view(np.float32)
    y = np.concatenate([y, -y])
    if y.size % 2:
        y = y[:-1]
    return y


@pytest.mark.parametrize("sel", [0, 1, 2, 3])
def test_cvt_pk_fp4_rounding_matches_oracle(lib, sel):
    y = _cvt_inputs()                      # values already divided by the scale
    n = y.size // 2
    rng = np.random.default_rng(sel)
    k = rng.integers(-100, 101, size=n)    # normal power-of-two scales
    scale = np.exp2(k).astype(np.float32)
    x = (y.reshape(n, 2).astype(np.float64) * scale[:, None]).astype(np.float32)
    tx, ts = torch.from_numpy(x).cuda(), torch.from_numpy(scale).cuda()
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    assert lib.probe_cvt_pk_fp4(tx.data_ptr(), ts.data_ptr(), out.data_ptr(), n, sel,
                                _stream()) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32)
    byte = (o >> (8 * sel)) & 0xFF
    got = np.stack([byte & 0xF, byte >> 4], axis=1).astype(np.uint8)
    # exact quotient x / scale (power-of-two scale) rounded by the oracle's encoder
    want = oracle.e2m1_encode_array(x.astype(np.float64) / scale[:, None].astype(np.float64))
    other = o & ~np.uint32(0xFF << (8 * sel))
    bad = np.nonzero((got != want).any(axis=1))[0]
    _dump("cvt_fp4_sel%d" % sel, x=x, scale=scale, out=o)
    assert bad.size == 0, [(x[i], scale[i], got[i], want[i]) for i in bad[:8]]
    assert not other.any(), "bytes other than the selected one were written"


def test_cvt_pk_fp4_small_scales_report(lib):
    """Scales 2^-127 (denormal) .. 2^-120: reported, the kernel's P path avoids relying on them."""
    e = np.arange(-127, -119)
    scale = np.exp2(e.astype(np.float64)).astype(np.float32)
    x = np.stack([scale * 4.0, scale * 1.0], axis=1).astype(np.float32)
    tx, ts = torch.from_numpy(x).cuda(), torch.from_numpy(scale).cuda()
    out = torch.zeros(e.size, dtype=torch.int32, device="cuda")
    assert lib.probe_cvt_pk_fp4(tx.data_ptr(), ts.data_ptr(), out.data_ptr(), e.size, 0,
                                _stream()) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32) & 0xFF
    print("small-scale converts (want 0x26):", [hex(v) for v in o])


def _time(fn, reps=3):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps * 1e-3


def test_issue_rates_report(lib):
    n_blocks, iters = 256 * 8, 2000
    out = torch.zeros(n_blocks * 256, device="cuda")
    t = _time(lambda: lib.probe_exp2_rate(out.data_ptr(), n_blocks, iters, _stream()))
    exps = n_blocks * 256 * iters * 8
    per_cu_clk = exps / t / 256 / 2.4e9
    print("v_exp_f32: %.3g /s = %.1f lanes per CU per clock at 2.4 GHz" % (exps / t, per_cu_clk))
    n_blocks, iters = 256 * 2, 200
    t = _time(lambda: lib.probe_mfma_rate(out.data_ptr(), n_blocks, iters, _stream()))
    mfmas = n_blocks * 4 * iters * 4
    flops = mfmas * 2 * 32 * 32 * 64
    print("fp4 32x32x64 MFMA: %.3g TFLOP/s (%.1f%% of 10.066 PFLOP/s), %.1f cycles per MFMA per SIMD"
          % (flops / t / 1e12, flops / t / 10.066e15 * 100, t * 2.4e9 * 1024 / mfmas))
    assert per_cu_clk > 4 and flops / t > 1e15
    t16 = _time(lambda: lib.probe_mfma16_rate(out.data_ptr(), n_blocks, iters, _stream()))
    mfmas16 = n_blocks * 4 * iters * 8
    flops16 = mfmas16 * 2 * 16 * 16 * 128
    print("fp4 16x16x128 MFMA: %.3g TFLOP/s (%.1f%% of 10.066 PFLOP/s), %.1f cycles per MFMA per "
          "SIMD" % (flops16 / t16 / 1e12, flops16 / t16 / 10.066e15 * 100,
                    t16 * 2.4e9 * 1024 / mfmas16))
    assert flops16 / t16 > 1e15


@pytest.mark.parametrize("pattern", ["contiguous", "rows", "bf16_v_operand"])
def test_lds_transpose_read_layout(lib, pattern):
    """ds_read_b64_tr_b16, as the bf16 kernel's V operand read uses it: each group of
    16 lanes reads the 16 x 4 matrix M[j] = the 4 elements at lane j's address and lane
    L of the group receives M[4i + L // 4][L % 4] for i = 0..3."""
    lanes = np.arange(64)
    if pattern == "contiguous":
        addr = 4 * lanes
    elif pattern == "rows":
        addr = 64 * lanes
    else:
        # the kernel's pattern for one channel tile: lane (group gq, 4 i + a) points at
        # key 8 (gq // 2) + i, channels 16 (gq % 2) + 4 a of 64-channel rows
        gq, jl = lanes // 16, lanes % 16
        addr = 64 * (8 * (gq // 2) + jl // 4) + 16 * (gq % 2) + 4 * (jl % 4)
    a = torch.tensor(addr, dtype=torch.int32, device="cuda")
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    assert lib.probe_lds_read_tr16(a.data_ptr(), out.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(64, 4)
    want = np.zeros((64, 4), np.int64)
    for lane in range(64):
        g0, L = 16 * (lane // 16), lane % 16
        for i in range(4):
            want[lane, i] = addr[g0 + 4 * i + L // 4] + L % 4
    assert np.array_equal(got.astype(np.int64), want), pattern
    if pattern == "bf16_v_operand":
        # lane (n, h) = lane 32 h + n gets channel n of keys 8h .. 8h + 3
        for lane in range(64):
            n, h = lane % 32, lane // 32
            assert [v % 64 for v in got[lane]] == [n] * 4
            assert [v // 64 for v in got[lane]] == [8 * h + i for i in range(4)]


def test_mfma_and_vector_co_execution_report(lib):
    """How much FP4 MFMA work and exp2 / fma work overlap on a SIMD: alone, interleaved
    inside each of two waves, and split over two waves of one kind each.  Cycles per
    SIMD per iteration (16 MFMAs and 32 exp2(fma) pairs per wave-iteration)."""
    n_blocks, iters = 256, 2000
    out = torch.zeros(n_blocks * 512, device="cuda")
    cyc = {}
    for mode, name in ((0, "mfma only"), (1, "vector only"), (2, "both, every wave"),
                       (3, "one wave of each kind")):
        t = _time(lambda: lib.probe_coexec(out.data_ptr(), mode, n_blocks, iters, _stream()))
        # two waves per SIMD; modes 0-2 give each SIMD two waves' worth of the work
        cyc[mode] = t * 2.4e9 / iters
        print("co-execution, %s: %.0f cycles per SIMD per iteration" % (name, cyc[mode]))
    assert lib.probe_coexec(out.data_ptr(), 4, n_blocks, iters, _stream()) == -1
    # in mode 3 each SIMD does half of mode 2's work: one wave's MFMAs beside one wave's
    # vector work; that overlap is near perfect when the pair costs no more than the
    # slower kind alone (half of modes 0 / 1) plus a quarter of the faster one
    one = max(cyc[0], cyc[1]) / 2 + min(cyc[0], cyc[1]) / 8
    print("one of each kind: %.0f cycles against %.0f for the slower kind alone"
          % (cyc[3], max(cyc[0], cyc[1]) / 2))
    assert cyc[3] < one * 1.2


def test_vector_issue_cost_report(lib):
    """SIMD cycles per wave64 instruction of the softmax step's vector work (two waves
    per SIMD, 8 independent chains each).  The exponential and the FP4 convert take
    several fma slots, and pairing an exponential with an fma costs their sum whether
    both are in each wave or one wave issues each kind: the transcendental does not run
    beside the other vector work."""
    n_blocks, iters = 256, 4000
    out = torch.zeros(n_blocks * 512, device="cuda")
    names = {0: "fma", 1: "v_exp_f32", 2: "exp / fma alternating", 3: "FP4 convert / fma alternating",
             4: "v_maximum3_f32", 5: "FP4 convert / exp alternating",
             6: "exp-only wave beside fma-only wave"}
    cyc = {}
    for mode, name in names.items():
        t = _time(lambda: lib.probe_valu_rate(out.data_ptr(), mode, n_blocks, iters, _stream()))
        # 1024 SIMDs, two waves each, 32 instructions per wave and iteration
        cyc[mode] = t * 2.4e9 / iters / 64
        print("vector issue cost, %s: %.2f SIMD cycles per instruction" % (name, cyc[mode]))
    assert lib.probe_valu_rate(out.data_ptr(), 7, n_blocks, iters, _stream()) == -1
    cvt = 2 * cyc[3] - cyc[0]
    print("derived: FP4 convert %.2f, exp / fma ratio %.2f" % (cvt, cyc[1] / cyc[0]))
    assert cyc[1] > 2 * cyc[0] and cvt > 2 * cyc[0]
    # no overlap of the exponential with fma: the pair costs about the sum
    assert cyc[2] > 0.85 * (cyc[0] + cyc[1]) / 2 and cyc[6] > 0.85 * (cyc[0] + cyc[1]) / 2


@pytest.mark.parametrize("size", [1, 2, 4, 16])
def test_lds_dma_lane_placement(lib, size):
    """4- and 16-byte forms: lane i's bytes land at M0 + size*i.  The 1- and
    2-byte forms write a whole dword per lane, at M0 + 4*i, zero-extended."""
    src = torch.tensor((np.arange(1024) * 7 + 3) % 251, dtype=torch.uint8, device="cuda")
    out = torch.empty(64 + 16 * 64, dtype=torch.uint8, device="cuda")
    assert lib.probe_lds_dma(src.data_ptr(), out.data_ptr(), size, _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    s = src.cpu().numpy()
    _dump("lds_dma_%d" % size, src=s, window=got)
    exp = np.full_like(got, 0xEE)
    stride = max(size, 4)
    for i in range(64):
        slot = np.zeros(stride, np.uint8)
        slot[:size] = s[size * i: size * (i + 1)]
        exp[64 + stride * i: 64 + stride * (i + 1)] = slot
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, "placement differs at window bytes %s" % bad[:16]


@pytest.mark.parametrize("soffset,num_records", [(0, 128), (64, 128), (64, 1024), (256, 300)])
def test_buffer_range_check_with_sgpr_offset(lib, soffset, num_records):
    """The raw-buffer range check counts the SGPR offset: lane i is in range
    iff soffset + 4i + 4 <= num_records (register and memory -> LDS forms).
    The prefill kernel relies on it: one descriptor per (batch, kv head) over
    the valid keys, the tile offset in soffset."""
    src = torch.arange(1, 1 + 512, dtype=torch.int32, device="cuda")
    out = torch.zeros(128, dtype=torch.int32, device="cuda")
    assert lib.probe_buffer_range(src.data_ptr(), out.data_ptr(), soffset, num_records,
                                  _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64)
    lanes = np.arange(64)
    data = soffset // 4 + lanes + 1
    with_so = np.where(4 * lanes + soffset + 4 <= num_records, data, 0)
    without_so = np.where(4 * lanes + 4 <= num_records, data, 0)
    for name, part in (("register", got[:64]), ("lds", got[64:])):
        print("%s soffset=%d num_records=%d: counts soffset %s, ignores it %s" % (
            name, soffset, num_records, (part == with_so).all(), (part == without_so).all()))
        assert (part == with_so).all()


def test_stream_read_covers_every_word_once(lib):
    """Each thread's xor covers exactly the words i, i + stride, ... below the end
    (a ragged tail past the unrolled part included), checked on the host."""
    rng = np.random.default_rng(8)
    n_blocks = 3
    n16 = 3 * 256 * 4 * 2 + 3 * 256 + 37        # two unrolled rounds, a tail, a ragged end
    words = rng.integers(0, 2**32, size=n16 * 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.empty(n_blocks * 256, dtype=torch.int32, device="cuda")
    assert lib.probe_stream_read(src.data_ptr(), n16 * 16, out.data_ptr(), n_blocks, _stream()) == 0
    torch.cuda.synchronize()
    w4 = np.bitwise_xor.reduce(words.reshape(n16, 4), axis=1)
    stride = n_blocks * 256
    exp = np.array([np.bitwise_xor.reduce(w4[t::stride]) if t < n16 else 0
                    for t in range(stride)], dtype=np.uint32)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), exp)
    assert lib.probe_stream_read(src.data_ptr(), 8, out.data_ptr(), n_blocks, _stream()) == -1
