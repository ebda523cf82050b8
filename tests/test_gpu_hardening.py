"""Exhaustive and boundary GPU parity of the producers and the GEMM.

Every comparison is against the oracle on inputs chosen to reach the edges of
the contract that random tensors miss:
  * the SR decision at its exact threshold, for every bf16 magnitude under
    every block exponent, in both the fast and the exact form of the encoder
    (a test-only kernel feeds the library's encoder chosen draws);
  * every bf16 pattern under every block exponent through fp4_quantize_rows
    (RTN and SR), so the hardware E2M1 converter and the SR path see all of
    them;
  * every finite bf16 value of the gate pre-activation a through the SwiGLU
    backward and the fused backward producer (the exp, the reciprocal and the
    bf16 packing on all of them);
  * GEMM scale bytes at both ends of E8M0, with products in the fp32
    subnormal range;
  * column H32 on bf16 subnormals and on the largest inputs the H32 bound
    admits;
  * sentinel-filled outputs of every kernel (every byte must be written);
  * operand checks of the SwiGLU bindings, which must refuse before any launch.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import synthetic
from oracle import formats as F
from oracle import gemm as G
from oracle import philox as P
from oracle import quant as Q
from oracle import swiglu as S

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host16(t):
    return host(t).view(np.uint16)


def assert_same(got, want, what):
    got = host(got) if isinstance(got, torch.Tensor) else got
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: "
                             f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")


def max_bits_for_exponent(e):
    """bf16 pattern of the block maximum whose upward exponent is e: 6 * 2^e
    (1.5 * 2^(e+2)); for e = 126 the largest finite value."""
    return 0x7F7F if e == 126 else (((e + 2 + 127) << 7) | 0x40)


# ----------------------------------------------------------------- SR threshold
def _probe():
    from precision_mxfp4_producers_amd.build import probe_path
    path = probe_path("sr_probe")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.sr_probe.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_void_p]
    lib.sr_probe.restype = ctypes.c_int
    return lib


def _thresholds(y):
    """T = ceil(frac * 2^32) for each y (0 on the grid): the draws T - 1 and T
    straddle the rounding decision.  Used only to pick draws; the expected
    nibbles come from oracle.formats.sr_code."""
    grid = F.E2M1_GRID
    lo = np.clip(np.searchsorted(grid, y, side="right") - 1, 0, 7)
    hi = np.clip(lo + 1, 0, 7)
    on = grid[lo] == y
    frac = np.where(on, 0.0, (y - grid[lo]) / np.where(on, 1.0, grid[hi] - grid[lo]))
    return np.ceil(frac * 2.0 ** 32).astype(np.uint64)


def _lanes(mags, signs, draws, e, wave_pad):
    """Pack elements into lanes of eight (same exponent), padded with zeros to
    a whole number of 64-lane waves when wave_pad."""
    n = len(mags)
    per = 512 if wave_pad else 8
    m = -(-n // per) * per
    bits = np.zeros(m, dtype=np.uint16)
    bits[:n] = mags | (signs.astype(np.uint16) << 15)
    u = np.zeros(m, dtype=np.uint32)
    u[:n] = draws
    return bits, u, np.full(m // 8, e, dtype=np.int32), n


def _sr_threshold_cases(rng):
    """Host side of the threshold test: per block exponent, lanes of the
    elements the fast form takes and, apart, of those that need the exact
    form (the encoder's own criterion: 1 <= mag < max(e + 111, 1) << 7, or
    e >= 126)."""
    mags_all = np.arange(0, 0x7F80, dtype=np.uint16)
    vals_all = F.bf16_bits_to_f64(mags_all)
    parts_fast, parts_exact = [], []
    for e in range(-127, 127):
        y = vals_all * 2.0 ** -e
        keep = y <= 6.0
        m, yk = mags_all[keep], y[keep]
        t = _thresholds(yk)
        u_lo = np.where(t == 0, 0, t - 1)
        u_hi = np.where(t == 0, 2 ** 32 - 1, np.minimum(t, 2 ** 32 - 1))
        mm = np.concatenate([m, m])
        uu = np.concatenate([u_lo, u_hi]).astype(np.uint32)
        ss = rng.integers(0, 2, size=len(mm)).astype(np.uint16)
        lim = max(e + 111, 1) << 7
        exact = (mm >= 1) & (mm < lim)
        # the fast form is exact wherever the criterion lets it run: y = 0 or y >= 2^-16
        ym = np.concatenate([yk, yk])
        assert np.all((ym[~exact] == 0) | (ym[~exact] >= 2.0 ** -16))
        for sel, parts in ((~exact, parts_fast), (exact, parts_exact)):
            if sel.any():
                parts.append(_lanes(mm[sel], ss[sel], uu[sel], e, True))
    return parts_fast, parts_exact


def test_sr_encoder_at_every_threshold(gpu_lib):
    """Every finite bf16 magnitude m with y = m 2^-e <= 6 under every block
    exponent e in [-127, 126], each at the draws T - 1 and T around its
    threshold (or 0 and 2^32 - 1 on the grid), with random signs.  Elements
    that need the exact form (y in (0, 2^-16), or a subnormal input under
    e <= -111) are kept in waves of their own, so that every other wave with
    e < 126 takes the fast form; the fast-form elements are then run once
    more behind one exact-form element per wave, which sends every wave to
    the exact form."""
    lib = _probe()
    parts_fast, parts_tiny = _sr_threshold_cases(np.random.default_rng(101))

    def run(parts, force_exact):
        bits = np.concatenate([p[0] for p in parts])
        u = np.concatenate([p[1] for p in parts])
        ex = np.concatenate([p[2] for p in parts])
        if force_exact:
            # lane 0 of every wave holds one value of 2^-133 (y = 2^-133 under e = 0)
            bits = bits.reshape(-1, 512).copy()
            u = u.reshape(-1, 512).copy()
            ex = ex.reshape(-1, 64).copy()
            bits[:, :8] = 0
            bits[:, 0] = 0x0001
            ex[:, 0] = 0
            u[:, :8] = 0
            bits, u, ex = bits.reshape(-1), u.reshape(-1), ex.reshape(-1)
        n = len(ex)
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        took = torch.empty(n, dtype=torch.int32, device="cuda")
        wd, ud, ed = dev16(bits), torch.from_numpy(u.view(np.int32)).cuda(), torch.from_numpy(ex).cuda()
        st = lib.sr_probe(wd.data_ptr(), ed.data_ptr(), ud.data_ptr(), out.data_ptr(), took.data_ptr(), n,
                          torch.cuda.current_stream().cuda_stream)
        assert st == 0
        got = host(out).view(np.uint32)
        # expected nibbles from the oracle
        e_el = np.repeat(ex.astype(np.int64), 8)
        x64 = F.bf16_bits_to_f64(bits)
        y = F.scaled_magnitude(x64, e_el)
        code = F.sign_nibble(x64, F.sr_code(y, u))
        want = F.pack_nibbles(code.reshape(-1, 8)).view(np.uint32).reshape(-1)
        assert_same(got, want, f"SR nibbles (force_exact={force_exact})")
        return host(took)

    took = run(parts_fast, False)
    # every fast-eligible wave with e < 126 took the fast form; e >= 126 always the exact one
    ex = np.concatenate([p[2] for p in parts_fast])
    assert np.all(took[ex < 126] == 0) and np.all(took[ex >= 126] == 1)
    took = run(parts_tiny, False)
    assert np.all(took == 1)
    took = run(parts_fast, True)
    assert np.all(took == 1)


# ----------------------------------------------------------------- every pattern, every exponent
def _all_patterns_tensor(rng):
    """Rows of 4096 values in blocks of 32: each block starts with +-6 * 2^e
    (fixing the block exponent e) and holds 31 bf16 patterns of magnitude at
    most that maximum, random signs; over all blocks, every pattern appears
    under every exponent e in [-127, 126] that admits it."""
    blocks = []
    for e in range(-127, 127):
        mx = max_bits_for_exponent(e)
        mags = np.arange(0, mx + 1, dtype=np.uint16)
        nb = -(-len(mags) // 31)
        fill = np.zeros(nb * 31, dtype=np.uint16)
        fill[:len(mags)] = mags
        blk = np.empty((nb, 32), dtype=np.uint16)
        blk[:, 0] = mx
        blk[:, 1:] = fill.reshape(nb, 31)
        blocks.append(blk)
    b = np.concatenate(blocks)
    b |= (rng.integers(0, 2, size=b.shape, dtype=np.uint16) << 15)
    nb = -(-len(b) // 128) * 128
    out = np.zeros((nb, 32), dtype=np.uint16)
    out[:len(b)] = b
    return out.reshape(-1, 4096)


@pytest.mark.parametrize("mode", [Q.RTN, Q.SR])
def test_rows_every_pattern_every_exponent(gpu_lib, mode):
    x = _all_patterns_tensor(np.random.default_rng(7))
    codes, scales = gpu_lib.fp4_quantize_rows(dev16(x), mode, 12345, 6)
    gc, gs = host(codes), host(scales)
    for r0 in range(0, x.shape[0], 128):
        rows = np.arange(r0, min(r0 + 128, x.shape[0]))
        want = Q.quantize_rows(x[rows], mode, 12345, 6, row_ids=rows)
        assert_same(gc[rows], want[0], f"codes rows {r0}+ mode {mode}")
        assert_same(gs[rows], want[1], f"scales rows {r0}+ mode {mode}")


# ----------------------------------------------------------------- every a through the SwiGLU backward
def test_swiglu_backward_every_finite_a(gpu_lib):
    """All 65,280 finite bf16 patterns of a (padded to 256 x 256 with zeros)
    through fp4_swiglu_backward and the fused backward producer: dA, dB
    bit-exact, and the producer's four MXFP4 views equal the oracle's
    quantization of the oracle's dA, dB."""
    mx = gpu_lib
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = pats[(pats & 0x7F80) != 0x7F80]
    a = np.zeros(1 << 16, dtype=np.uint16)
    a[:len(finite)] = finite
    a = a.reshape(256, 256)
    b = synthetic.tensor((256, 256), std=1.3, seed=61)
    rng = np.random.default_rng(62)
    dh = (rng.standard_normal((256, 256)) * 1e-3).astype(np.float32)
    dhd, ad, bd = torch.from_numpy(dh).cuda(), dev16(a), dev16(b)
    da, db = mx.fp4_swiglu_backward(dhd, ad, bd)
    want_da, want_db = S.swiglu_backward(dh, a, b)
    assert np.all(np.isfinite(F.bf16_bits_to_f64(want_da))) and np.all(np.isfinite(F.bf16_bits_to_f64(want_db)))
    assert_same(host16(da), want_da, "dA")
    assert_same(host16(db), want_db, "dB")
    seed, oa, ob, mask = 77, 3, 4, P.sign_mask_from_seed(9)
    got = mx.fp4_swiglu_backward_producer(dhd, ad, bd, seed, oa, ob, mask)
    want = (Q.quantize_rows(want_da, Q.SR, seed, oa), Q.quantize_rows(want_db, Q.SR, seed, ob),
            Q.quantize_cols(want_da, 32, mask), Q.quantize_cols(want_db, 32, mask))
    for g, w, nm in zip(got, want, ("dA rows", "dB rows", "dA cols", "dB cols")):
        assert_same(g[0], w[0], nm + " codes")
        assert_same(g[1], w[1], nm + " scales")


# ----------------------------------------------------------------- GEMM scale extremes
@pytest.mark.parametrize("k", [512, 288])                 # fast and generic main loops
def test_gemm_e8m0_extremes(gpu_lib, k):
    """Scale bytes over the whole E8M0 range the producers write (0 = 2^-127
    up to 253), paired so that every product stays finite: A's bytes span
    [0, 40] and [200, 253] and B's [0, 40], so the products' scales span
    2^-254 ... 2^39: exact products far below the fp32 range (whose sums
    must come out as zero), and normal values.  Rows 0-31 of A against
    rows 0-39 of B have every product in the fp32 subnormal range (scales
    2^-136 ... 2^-132): a scaled MFMA that flushed subnormal products or
    results would return zero there.  Bound: |C - C_ref| <= 1e-5 * sum |ab|
    + K * 2^-150 (the fp32 subnormal spacing, half an ulp per accumulated
    term) with C_ref the fp64 sum rounded once to fp32."""
    m, n = 96, 160
    rng = np.random.default_rng(71)
    ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    asc = np.where(rng.random((m, k // 32)) < 0.5, rng.integers(0, 41, size=(m, k // 32)),
                   rng.integers(200, 254, size=(m, k // 32))).astype(np.uint8)
    bsc = rng.integers(0, 41, size=(n, k // 32)).astype(np.uint8)
    # rows 0-31 of A x rows 0-39 of B: products entirely in the fp32
    # subnormal range (scales 2^(a+b-254), a + b in [118, 122]: |products| <=
    # 36 * 2^-132 < 2^-126), sums up to about 2^-122
    asc[:32] = rng.integers(78, 83, size=(32, k // 32)).astype(np.uint8)
    bsc[:40] = 40
    t = [torch.from_numpy(v).cuda() for v in (ac, asc, bc, bsc)]
    c = gpu_lib.fp4_gemm(*t)
    ref, e = G.gemm_ref(ac, asc, bc, bsc)
    ref32 = ref.astype(np.float32).astype(np.float64)
    got = host(c).astype(np.float64)
    ok = G.within_bound(got, ref32, e, k=k)
    assert ok.all(), (f"{(~ok).sum()} elements outside the bound; first {np.argwhere(~ok)[0].tolist()}: "
                      f"got {got[~ok][0]!r} want {ref32[~ok][0]!r}")
    sub = np.abs(ref32[:32, :40])
    assert ((sub > 0) & (sub < 2.0 ** -126)).mean() > 0.3      # the case really reaches the subnormals


# ----------------------------------------------------------------- H32 on subnormals and near the bound
@pytest.mark.parametrize("had", [0, 32])
def test_cols_subnormal_and_large_inputs(gpu_lib, had):
    rng = np.random.default_rng(81)
    x = rng.integers(0, 0x80, size=(256, 192), dtype=np.uint16)          # bf16 subnormals and zeros
    x[:, 64:96] |= 0x0080 * rng.integers(0, 3, size=(256, 32)).astype(np.uint16)   # next to the smallest normals
    x[:, 96:128] = rng.integers(0x7C00, 0x7C80, size=(256, 32), dtype=np.uint16)   # |x| in [2^121, 2^122)
    x[:, 128:160] = rng.integers(0x7C00, 0x7C80, size=(256, 32), dtype=np.uint16)
    x[:, 128:160][::5] = rng.integers(0, 0x80, size=x[:, 128:160][::5].shape, dtype=np.uint16)   # mixed
    x |= (rng.integers(0, 2, size=x.shape, dtype=np.uint16) << 15)
    x[:, 96:112] &= 0x7FFF                                              # one sign: largest H32 sums
    mask = P.sign_mask_from_seed(3)
    codes, scales = gpu_lib.fp4_quantize_cols(dev16(x), had, mask)
    want = Q.quantize_cols(x, had, mask)
    assert_same(codes, want[0], "col codes")
    assert_same(scales, want[1], "col scales")
    dual = gpu_lib.fp4_quantize_dual(dev16(x), gpu_lib.FP4_SR, 5, 1, had, mask)
    for g, w, nm in zip(dual, Q.quantize_rows(x, Q.SR, 5, 1) + want, ("row codes", "row scales", "col codes",
                                                                       "col scales")):
        assert_same(g, w, "dual " + nm)


# ----------------------------------------------------------------- sentinels
def _sentinel(shape, dtype, val):
    return torch.full(shape, val, dtype=dtype, device="cuda")


def test_every_kernel_writes_every_output_byte(gpu_lib):
    """Outputs pre-filled with sentinel bytes (0xAB codes, 0xFF scales, NaN
    fp32, 0x7FFF bf16), shapes with ragged tails: after each call every
    element equals the oracle's, so none was skipped."""
    mask = P.sign_mask_from_seed(4)
    # 2D32 and the single-read producer
    w = synthetic.tensor((160, 352), std=0.02, seed=91)
    outs = [_sentinel(s, torch.uint8, v) for s, v in (((160, 176), 0xAB), ((160, 11), 0xFF), ((352, 80), 0xAB),
                                                       ((352, 5), 0xFF))]
    gpu_lib.fp4_quantize_w2d32(dev16(w), 0.87, *outs)
    for g, wv, nm in zip(outs, Q.quantize_w2d32(w, 0.87), ("row codes", "row scales", "col codes", "col scales")):
        assert_same(g, wv, "2D32 " + nm)
    x = synthetic.tensor((160, 352), std=1.0, seed=92)
    for mode in (Q.RTN, Q.SR):
        outs = [_sentinel(s, torch.uint8, v) for s, v in (((160, 176), 0xAB), ((160, 11), 0xFF), ((352, 80), 0xAB),
                                                           ((352, 5), 0xFF))]
        gpu_lib.fp4_quantize_dual(dev16(x), mode, 8, 2, 32, mask, *outs)
        for g, wv, nm in zip(outs, Q.quantize_rows(x, mode, 8, 2) + Q.quantize_cols(x, 32, mask),
                             ("row codes", "row scales", "col codes", "col scales")):
            assert_same(g, wv, f"dual mode {mode} " + nm)
    # GEMM, plain (fast and generic) and paired
    for (m, n, k) in ((288, 352, 512), (96, 160, 288)):
        a = gpu_lib.fp4_quantize_rows(dev16(synthetic.tensor((m, k), std=1.0, seed=93)))
        b = gpu_lib.fp4_quantize_rows(dev16(synthetic.tensor((n, k), std=1.0, seed=94)))
        c = _sentinel((m, n), torch.float32, float("nan"))
        gpu_lib.fp4_gemm(a[0], a[1], b[0], b[1], c=c)
        ref, e = G.gemm_ref(host(a[0]), host(a[1]), host(b[0]), host(b[1]))
        assert G.within_bound(host(c), ref, e).all(), f"gemm {m}x{n}x{k}"
        c = _sentinel((m, n), torch.float32, float("nan"))
        gpu_lib.fp4_gemm_pair(a[0], a[1], b[0], b[1], a[0], a[1], b[0], b[1], c=c)
        assert G.within_bound(host(c), 2 * ref, 2 * e).all(), f"gemm pair {m}x{n}x{k}"
    # SwiGLU producer, normal path (fast and generic main loops)
    for (t, f, d) in ((288, 160, 512), (96, 96, 288)):
        xr = gpu_lib.fp4_quantize_rows(dev16(synthetic.tensor((t, d), std=1.0, seed=95)))
        wq = gpu_lib.fp4_quantize_w2d32(dev16(synthetic.tensor((2 * f, d), std=0.02, seed=96)), 0.87)
        outs = [_sentinel(s, dt, v) for s, dt, v in (((t, f), torch.int16, 0x7FFF), ((t, f), torch.int16, 0x7FFF),
                                                    ((t, f // 2), torch.uint8, 0xAB), ((t, f // 32), torch.uint8, 0xFF),
                                                    ((f, t // 2), torch.uint8, 0xAB), ((f, t // 32), torch.uint8, 0xFF))]
        gpu_lib.fp4_swiglu_producer(xr[0], xr[1], wq[0], wq[1], mask, True, *outs)
        av, bv = host16(outs[0]), host16(outs[1])
        assert not np.any(av == 0x7FFF) and not np.any(bv == 0x7FFF)
        ref, e = G.gemm_ref(host(xr[0]), host(xr[1]), host(wq[0]), host(wq[1]))
        tol = G.GEMM_REL_TOL * e
        for got, r, tl in ((av, ref[:, :f], tol[:, :f]), (bv, ref[:, f:], tol[:, f:])):
            lo = F.bf16_bits_to_f64(S.f32_to_bf16_rne((r - tl).astype(np.float32)))
            hi = F.bf16_bits_to_f64(S.f32_to_bf16_rne((r + tl).astype(np.float32)))
            g = F.bf16_bits_to_f64(got)
            assert np.all((g >= lo) & (g <= hi))
        h = S.swiglu_h(av, bv)
        for g, wv, nm in zip(outs[2:], Q.quantize_rows(h) + Q.quantize_cols(h, 32, mask),
                             ("h row codes", "h row scales", "h col codes", "h col scales")):
            assert_same(g, wv, f"swiglu {t}x{f}x{d} " + nm)
    # fused backward producer
    t, f = 288, 160
    a = synthetic.tensor((t, f), std=1.3, seed=97)
    b = synthetic.tensor((t, f), std=1.3, seed=98)
    dh = (np.random.default_rng(99).standard_normal((t, f)) * 1e-3).astype(np.float32)
    outs = [_sentinel(s, torch.uint8, v) for s, v in (((t, f // 2), 0xAB), ((t, f // 32), 0xFF), ((t, f // 2), 0xAB),
                                                       ((t, f // 32), 0xFF), ((f, t // 2), 0xAB), ((f, t // 32), 0xFF),
                                                       ((f, t // 2), 0xAB), ((f, t // 32), 0xFF))]
    gpu_lib.fp4_swiglu_backward_producer(torch.from_numpy(dh).cuda(), dev16(a), dev16(b), 5, 1, 2, mask, outs)
    da, db = S.swiglu_backward(dh, a, b)
    want = (Q.quantize_rows(da, Q.SR, 5, 1) + Q.quantize_rows(db, Q.SR, 5, 2) + Q.quantize_cols(da, 32, mask)
            + Q.quantize_cols(db, 32, mask))
    for g, wv, i in zip(outs, want, range(8)):
        assert_same(g, wv, f"backward producer output {i}")


# ----------------------------------------------------------------- binding checks
def test_swiglu_bindings_refuse_bad_operands(gpu_lib):
    """Mismatched d, an odd W1|W3 row count, wrong scale shapes, a wrong dtype
    and strided operands are refused with Fp4Error before any launch."""
    t, f, d = 64, 96, 256
    xr = gpu_lib.fp4_quantize_rows(dev16(synthetic.tensor((t, d), std=1.0, seed=1)))
    wq = gpu_lib.fp4_quantize_w2d32(dev16(synthetic.tensor((2 * f, d), std=0.02, seed=2)), 0.87)
    mask = P.sign_mask_from_seed(0)
    xs = gpu_lib.fp4_quantize_rows(dev16(synthetic.tensor((t, d // 2), std=1.0, seed=1)))   # d / 2 values per row
    bad = [
        (xs[0], xs[1], wq[0], wq[1]),                                        # d of x differs from w13's
        (xr[0], xr[1], wq[0][: 2 * f - 1], wq[1][: 2 * f - 1]),              # odd W1|W3 row count
        (xr[0], xr[1][:, :4].contiguous(), wq[0], wq[1]),                    # x scales shape
        (xr[0], xr[1], wq[0], wq[1][:, :4].contiguous()),                    # w13 scales shape
        (xr[0].to(torch.int16), xr[1], wq[0], wq[1]),                        # dtype
        (torch.cat([xr[0], xr[0]], 1)[:, : d // 2], xr[1], wq[0], wq[1]),    # strided view
    ]
    for args in bad:
        with pytest.raises(gpu_lib.Fp4Error):
            gpu_lib.fp4_swiglu_producer(*args, mask)
    a = synthetic.tensor((t, f), std=1.0, seed=3)
    dh = torch.zeros((t, f), dtype=torch.float32, device="cuda")
    for aa, bb in ((dev16(a), dev16(a)[:, :32]), (dev16(a).float(), dev16(a)),
                   (dev16(a), torch.cat([dev16(a), dev16(a)], 1)[:, :f])):
        with pytest.raises(gpu_lib.Fp4Error):
            gpu_lib.fp4_swiglu_backward(dh, aa, bb)
    torch.cuda.synchronize()


def test_sr_rule_on_fp32_magnitudes_at_the_threshold(gpu_lib):
    """The adjacent-bin rule as the CTA-local NVFP4 producers apply it, on fp32
    magnitudes with full 24-bit significands (y = RN(|x| r) is any fp32 in
    [0, 6]): random values over [2^-40, 6], every grid point and its fp32
    neighbours, and subnormals; each at the draws T - 1 and T around its
    threshold T = ceil(frac 2^32) (exact in float64: every spacing is a power
    of two), compared with the oracle's rule."""
    lib = _probe()
    lib.sr_y_probe.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_void_p]
    lib.sr_y_probe.restype = ctypes.c_int
    rng = np.random.default_rng(102)
    grid = F.E2M1_GRID.astype(np.float32)
    ys = [rng.uniform(0, 6, 40000).astype(np.float32),
          np.exp2(rng.uniform(-40, np.log2(6), 40000)).astype(np.float32),
          grid, np.nextafter(grid, np.float32(7)), np.nextafter(grid, np.float32(-1)),
          np.float32([1e-45, 3e-42, 1.17e-38, 2.0 ** -33, 2.0 ** -32, 3 * 2.0 ** -34])]
    y = np.concatenate(ys)
    y = y[(y >= 0) & (y <= 6)].astype(np.float32)
    y64 = y.astype(np.float64)
    lo = np.clip(np.searchsorted(F.E2M1_GRID, y64, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    step = np.where(hi > lo, F.E2M1_GRID[hi] - F.E2M1_GRID[lo], 1.0)
    T = np.ceil((y64 - F.E2M1_GRID[lo]) / step * 2.0 ** 32)           # exact: power-of-two step
    cases_y, cases_u = [], []
    for du in (-1, 0):
        u = T + du
        ok = (u >= 0) & (u <= 2.0 ** 32 - 1)
        cases_y.append(y[ok])
        cases_u.append(u[ok].astype(np.uint64).astype(np.uint32))
    cases_y.append(y)                                               # and the extreme draws
    cases_u.append(np.zeros(len(y), dtype=np.uint32))
    cases_y.append(y)
    cases_u.append(np.full(len(y), 0xFFFFFFFF, dtype=np.uint32))
    yy, uu = np.concatenate(cases_y), np.concatenate(cases_u)
    n = len(yy)
    yd = torch.from_numpy(yy).cuda()
    ud = torch.from_numpy(uu.view(np.int32)).cuda()
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    assert lib.sr_y_probe(yd.data_ptr(), ud.data_ptr(), out.data_ptr(), n, torch.cuda.current_stream().cuda_stream) == 0
    got = host(out).view(np.uint32)
    want = F.sr_code(yy.astype(np.float64), uu).astype(np.uint32)
    assert_same(got, want, "SR codes on fp32 magnitudes")


def test_bf16_rounding_of_arithmetic_results(gpu_lib):
    """The bf16 rounding the SwiGLU producer and the backward producers apply to
    their fp32 results (hardware RNE after a maxNum against the canonical quiet
    NaN), on every quiet NaN pattern of both signs, on NaNs that GPU arithmetic
    produces (inf - inf, 0 * inf, NaN inputs carried through a product), and on
    finite values around every bf16 rounding boundary, subnormals, the overflow
    threshold and the infinities: equal to the oracle's RNE with NaN -> 0x7FC0."""
    from precision_mxfp4_producers_amd.build import probe_path
    path = probe_path("bf16_probe")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.bf16_pack_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.bf16_pack_probe.restype = ctypes.c_int
    rng = np.random.default_rng(103)
    qnan = (np.arange(1 << 22, dtype=np.uint32) | np.uint32(0x7FC00000))          # every quiet NaN, + sign
    hi16 = np.arange(1 << 16, dtype=np.uint32) << 16                                  # every bf16 pattern ...
    lows = np.uint32([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF])                          # ... with the tie cases
    fin = (hi16[:, None] | lows[None, :]).reshape(-1)
    fin = fin[(fin & 0x7FFFFFFF) <= 0x7F800000]                                       # finite and infinities
    rnd = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    rnd = rnd[(rnd & 0x7FFFFFFF) <= 0x7F800000]
    bits = np.concatenate([qnan, qnan | np.uint32(0x80000000), fin, rnd])
    if len(bits) % 2:
        bits = np.append(bits, np.uint32(0))
    x = torch.from_numpy(bits.view(np.float32)).cuda()
    # NaNs made by arithmetic on the GPU: inf - inf, 0 * inf, and payload NaNs through a product
    inf = torch.full((4096,), float("inf"), device="cuda")
    made = torch.cat([inf - inf, torch.zeros_like(inf) * inf, x[: 1 << 20] * 1.5, -x[: 1 << 20]])
    x = torch.cat([x, made])
    n = x.numel() // 2
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    assert lib.bf16_pack_probe(x.data_ptr(), out.data_ptr(), n, torch.cuda.current_stream().cuda_stream) == 0
    got = host(out).view(np.uint32)
    xs = host(x)
    want16 = S.f32_to_bf16_rne(xs).astype(np.uint32)
    want = want16[0::2] | (want16[1::2] << 16)
    assert_same(got, want, "bf16 rounding with NaN -> 0x7FC0")
