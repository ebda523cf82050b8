"""GPU parity of every hot-path call against the oracle, at sizes the oracle
finishes in seconds that still span several workgroup tiles plus a ragged tail.

Bar: codes, scales, SR outputs, SwiGLU h/dA/dB bit-exact; GEMM outputs within
|C - C_ref| <= 1e-5 * sum_k |a_k b_k| per element.
"""

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


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host16(t):
    return host(t).view(np.uint16)


def assert_same(got, want, what):
    got = host(got)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: "
                             f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")


def check_gemm(c_gpu, a, b, c_prev=None, what="gemm"):
    ref, e = G.gemm_ref(host(a[0]), host(a[1]), host(b[0]), host(b[1]))
    ok = G.within_bound(host(c_gpu), ref, e, c_prev=c_prev)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements outside bound; first {i}: "
                             f"got {host(c_gpu)[i]} ref {ref[i]} E {e[i]}")


ROW_SHAPES = [(256, 512), (320, 544), (96, 4128), (32, 32)]


@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_rows_rtn(gpu_lib, shape):
    x = synthetic.tensor(shape, std=1.0, seed=11, outlier_rate=0.001, outlier_scale=20.0)
    x[0, :32] = 0
    x[-1, 3] = 0x8000
    codes, scales = gpu_lib.fp4_quantize_rows(dev16(x))
    want = Q.quantize_rows(x)
    assert_same(codes, want[0], "codes")
    assert_same(scales, want[1], "scales")


@pytest.mark.parametrize("shape", ROW_SHAPES)
@pytest.mark.parametrize("seed,offset", [(0, 0), (12345, 7), (2 ** 40 + 3, 2 ** 33 + 1)])
def test_rows_sr(gpu_lib, shape, seed, offset):
    dy = synthetic.tensor(shape, std=1e-3, seed=12, outlier_rate=0.01, outlier_scale=50.0)
    codes, scales = gpu_lib.fp4_quantize_rows(dev16(dy), gpu_lib.FP4_SR, seed, offset)
    want = Q.quantize_rows(dy, Q.SR, seed, offset)
    assert_same(codes, want[0], "SR codes")
    assert_same(scales, want[1], "SR scales")


def test_rows_strided_input(gpu_lib):
    full = synthetic.tensor((64, 640), std=1.0, seed=13)
    xd = dev16(full)[:, 64:576]                          # ldx = 640, cols = 512
    codes, scales = gpu_lib.fp4_quantize_rows(xd)
    want = Q.quantize_rows(np.ascontiguousarray(full[:, 64:576]))
    assert_same(codes, want[0], "codes")
    assert_same(scales, want[1], "scales")


def test_cols_dual_w2d32_strided_input(gpu_lib):
    """The column, single-read and 2D32 producers on a row-strided view
    (ldx = 640, cols = 512, starting 64 values into each row)."""
    full = synthetic.tensor((96, 640), std=1.0, seed=21, outlier_rate=0.01, outlier_scale=30.0)
    x = np.ascontiguousarray(full[:, 64:576])
    xd = dev16(full)[:, 64:576]
    mask = P.sign_mask_from_seed(7)
    codes_t, scales_t = gpu_lib.fp4_quantize_cols(xd, 32, mask)
    want_c = Q.quantize_cols(x, 32, mask)
    assert_same(codes_t, want_c[0], "col codes")
    assert_same(scales_t, want_c[1], "col scales")
    got = gpu_lib.fp4_quantize_dual(xd, 1, 11, 2, 32, mask)
    want_r = Q.quantize_rows(x, Q.SR, 11, 2)
    for g, w, nm in zip(got, want_r + want_c, ("row codes", "row scales", "col codes", "col scales")):
        assert_same(g, w, "dual " + nm)
    got = gpu_lib.fp4_quantize_w2d32(xd, 0.87)
    for g, w, nm in zip(got, Q.quantize_w2d32(x, 0.87), ("row codes", "row scales", "col codes", "col scales")):
        assert_same(g, w, "2D32 " + nm)


def test_rows_extreme_values(gpu_lib):
    # subnormals, huge values and tiny-next-to-huge blocks (SR threshold at 1)
    rng = np.random.default_rng(3)
    x = rng.integers(0, 0x7F80, size=(64, 256), dtype=np.uint16)
    x |= (rng.integers(0, 2, size=x.shape, dtype=np.uint16) << 15)
    x[5, :32] = np.arange(1, 33, dtype=np.uint16)       # bf16 subnormals
    x[6, 0] = 0x7F7F                                    # largest finite
    x[6, 1:32] = 0x0001
    for mode in (Q.RTN, Q.SR):
        codes, scales = gpu_lib.fp4_quantize_rows(dev16(x), mode, 99, 5)
        want = Q.quantize_rows(x, mode, 99, 5)
        assert_same(codes, want[0], f"codes mode {mode}")
        assert_same(scales, want[1], f"scales mode {mode}")


@pytest.mark.parametrize("shape", [(256, 512), (320, 544), (4128, 96), (32, 32)])
@pytest.mark.parametrize("had", [0, 32])
def test_cols(gpu_lib, shape, had):
    x = synthetic.tensor(shape, std=1.0, seed=14, outlier_rate=0.01, outlier_scale=30.0)
    mask = P.sign_mask_from_seed(0)
    codes, scales = gpu_lib.fp4_quantize_cols(dev16(x), had, mask)
    want = Q.quantize_cols(x, had, mask)
    assert_same(codes, want[0], "col codes")
    assert_same(scales, want[1], "col scales")


@pytest.mark.parametrize("shape", [(256, 512), (320, 544), (4128, 96), (32, 32), (160, 288)])
@pytest.mark.parametrize("mode,had", [(1, 32), (0, 0), (1, 0), (0, 32)])
def test_dual(gpu_lib, shape, mode, had):
    """One read, both views: the oracle's row and column codes, and the same
    bytes as the two separate producers."""
    x = synthetic.tensor(shape, std=1e-3, seed=19, outlier_rate=0.01, outlier_scale=50.0)
    mask = P.sign_mask_from_seed(4)
    seed, offset = 2 ** 35 + 9, 3
    got = gpu_lib.fp4_quantize_dual(dev16(x), mode, seed, offset, had, mask)
    rows = Q.quantize_rows(x, Q.SR if mode == 1 else Q.RTN, seed, offset)
    cols = Q.quantize_cols(x, had, mask)
    for g, w, nm in zip(got, rows + cols, ("row codes", "row scales", "col codes", "col scales")):
        assert_same(g, w, nm)
    xd = dev16(x)
    sep = gpu_lib.fp4_quantize_rows(xd, mode, seed, offset) + gpu_lib.fp4_quantize_cols(xd, had, mask)
    for g, w in zip(got, sep):
        assert torch.equal(g, w)


@pytest.mark.parametrize("shape", [(512, 512), (352, 416), (32, 64), (4096, 160),
                                   (1024, 256)])   # 2 x 8 workgroups: the XCD-aware block order
@pytest.mark.parametrize("ratio", [0.87, 0.0])
def test_w2d32(gpu_lib, shape, ratio):
    w = synthetic.tensor(shape, std=0.02, seed=15)
    got = gpu_lib.fp4_quantize_w2d32(dev16(w), ratio)
    want = Q.quantize_w2d32(w, ratio)
    for g, wv, nm in zip(got, want, ("row_codes", "row_scales", "col_codes", "col_scales")):
        assert_same(g, wv, nm)


def test_w2d32_orientation_invariant_on_gpu(gpu_lib):
    w = synthetic.tensor((384, 640), std=0.02, seed=16)
    rc, rs, cc, cs = gpu_lib.fp4_quantize_w2d32(dev16(w), 0.87)
    assert np.array_equal(F.decode(host(rc), host(rs)), F.decode(host(cc), host(cs)).T)


@pytest.mark.parametrize("mnk", [(256, 512, 512), (288, 352, 544), (512, 256, 1024), (32, 32, 32), (96, 544, 288)])
def test_gemm(gpu_lib, mnk):
    m, n, k = mnk
    x = synthetic.tensor((m, k), std=1.0, seed=17, outlier_rate=0.001, outlier_scale=20.0)
    w = synthetic.tensor((n, k), std=0.02, seed=18)
    a = gpu_lib.fp4_quantize_rows(dev16(x))
    b = gpu_lib.fp4_quantize_rows(dev16(w))
    c = gpu_lib.fp4_gemm(a[0], a[1], b[0], b[1])
    check_gemm(c, a, b)
    prev = host(c).copy()
    c2 = gpu_lib.fp4_gemm(a[0], a[1], b[0], b[1], c=c, accumulate=True)
    check_gemm(c2, a, b, c_prev=prev, what="accumulate")


@pytest.mark.parametrize("mnk", [(288, 352, 512), (256, 512, 1024), (96, 544, 256), (64, 96, 288), (32, 32, 32)])
def test_gemm_pair(gpu_lib, mnk):
    """C = A1 B1^T + A2 B2^T within the bound of the summed products; with K a
    multiple of 256 it is one accumulation, byte-equal to fp4_gemm over the
    operands concatenated along K."""
    m, n, k = mnk
    q = []
    for i, (rows, std) in enumerate(((m, 1.0), (n, 0.02), (m, 1e-3), (n, 0.02))):
        t = synthetic.tensor((rows, k), std=std, seed=40 + i, outlier_rate=0.001, outlier_scale=20.0)
        q.append(gpu_lib.fp4_quantize_rows(dev16(t)))
    a1, b1, a2, b2 = q
    c = gpu_lib.fp4_gemm_pair(*a1, *b1, *a2, *b2)
    r1, e1 = G.gemm_ref(host(a1[0]), host(a1[1]), host(b1[0]), host(b1[1]))
    r2, e2 = G.gemm_ref(host(a2[0]), host(a2[1]), host(b2[0]), host(b2[1]))
    ok = G.within_bound(host(c), r1 + r2, e1 + e2)
    assert ok.all(), f"{(~ok).sum()} elements outside the bound"
    prev = host(c).copy()
    c2 = gpu_lib.fp4_gemm_pair(*a1, *b1, *a2, *b2, c=c, accumulate=True)
    ok = G.within_bound(host(c2), r1 + r2, e1 + e2, c_prev=prev)
    assert ok.all(), f"accumulate: {(~ok).sum()} elements outside the bound"
    if k % 256 == 0:
        cat = [torch.cat((x, y), dim=1).contiguous() for x, y in zip(a1 + b1, a2 + b2)]
        whole = gpu_lib.fp4_gemm(*cat)
        assert np.array_equal(host(gpu_lib.fp4_gemm_pair(*a1, *b1, *a2, *b2)).view(np.uint32),
                              host(whole).view(np.uint32))


@pytest.mark.parametrize("k", [768, 1024])
def test_gemm_more_tiles_than_cus(gpu_lib, k):
    """17 x 17 tiles (ragged in both dimensions): more tiles than CUs, so each
    workgroup of the launch computes one or two tiles in turn; plain,
    accumulating and paired forms."""
    m, n = 4160, 4128
    x = synthetic.tensor((m, k), std=1.0, seed=51, outlier_rate=0.001, outlier_scale=20.0)
    w = synthetic.tensor((n, k), std=0.02, seed=52)
    a = gpu_lib.fp4_quantize_rows(dev16(x))
    b = gpu_lib.fp4_quantize_rows(dev16(w))
    c = gpu_lib.fp4_gemm(a[0], a[1], b[0], b[1])
    check_gemm(c, a, b)
    prev = host(c).copy()
    c2 = gpu_lib.fp4_gemm(a[0], a[1], b[0], b[1], c=c, accumulate=True)
    check_gemm(c2, a, b, c_prev=prev, what="accumulate")
    x2 = synthetic.tensor((m, k), std=1e-3, seed=53)
    a2 = gpu_lib.fp4_quantize_rows(dev16(x2))
    cp = gpu_lib.fp4_gemm_pair(a[0], a[1], b[0], b[1], a2[0], a2[1], b[0], b[1])
    r1, e1 = G.gemm_ref(host(a[0]), host(a[1]), host(b[0]), host(b[1]))
    r2, e2 = G.gemm_ref(host(a2[0]), host(a2[1]), host(b[0]), host(b[1]))
    assert G.within_bound(host(cp), r1 + r2, e1 + e2).all()


def test_gemm_layout_one_hot(gpu_lib):
    # one non-zero product per output element pins the MFMA register layout
    m, n, k = 64, 96, 256
    ac = np.zeros((m, k // 2), dtype=np.uint8)
    bc = np.zeros((n, k // 2), dtype=np.uint8)
    for i in range(m):
        kk = (7 * i) % k
        ac[i, kk // 2] |= (2 if kk % 2 == 0 else 0x20)           # value 1.0
    rng = np.random.default_rng(5)
    bc[:] = rng.integers(0, 256, size=bc.shape, dtype=np.uint8)
    as_ = np.full((m, k // 32), 127, dtype=np.uint8)
    bs = rng.integers(120, 135, size=(n, k // 32), dtype=np.uint8)
    t = [torch.from_numpy(v).cuda() for v in (ac, as_, bc, bs)]
    c = gpu_lib.fp4_gemm(*t)
    ref, _ = G.gemm_ref(ac, as_, bc, bs)
    assert np.array_equal(host(c).astype(np.float64), ref)


def test_linear_fprop_dgrad_wgrad(gpu_lib):
    """Eq. 4-6 with the producers feeding the GEMMs: Fprop Q_r(X)Q_r(W)^T,
    Dgrad Q_r(dY, SR)Q_c(W) with the 2D32 column layout, Wgrad Q_c(dY)^T Q_c(X)
    with paired H32."""
    T, D, N = 320, 288, 224
    x = synthetic.tensor((T, D), std=1.0, seed=19)
    w = synthetic.tensor((N, D), std=0.02, seed=20)
    dy = synthetic.tensor((T, N), std=1e-3, seed=21)
    mask = P.sign_mask_from_seed(0)
    xr = gpu_lib.fp4_quantize_rows(dev16(x))
    wq = gpu_lib.fp4_quantize_w2d32(dev16(w), 0.87)
    dyr = gpu_lib.fp4_quantize_rows(dev16(dy), gpu_lib.FP4_SR, 0, 1)
    dyc = gpu_lib.fp4_quantize_cols(dev16(dy), 32, mask)
    xc = gpu_lib.fp4_quantize_cols(dev16(x), 32, mask)
    check_gemm(gpu_lib.fp4_gemm(xr[0], xr[1], wq[0], wq[1]), xr, wq[:2], what="Fprop")
    check_gemm(gpu_lib.fp4_gemm(dyr[0], dyr[1], wq[2], wq[3]), dyr, wq[2:], what="Dgrad")
    check_gemm(gpu_lib.fp4_gemm(dyc[0], dyc[1], xc[0], xc[1]), dyc, xc, what="Wgrad")


@pytest.mark.parametrize("tfd", [(256, 128, 512), (288, 160, 320), (512, 384, 256), (32, 32, 32)])
@pytest.mark.parametrize("emit_cols", [True, False])
def test_swiglu_producer(gpu_lib, tfd, emit_cols):
    t, f, d = tfd
    x = synthetic.tensor((t, d), std=1.0, seed=22)
    w13 = synthetic.tensor((2 * f, d), std=0.02, seed=23)
    mask = P.sign_mask_from_seed(0)
    xr = gpu_lib.fp4_quantize_rows(dev16(x))
    wq = gpu_lib.fp4_quantize_w2d32(dev16(w13), 0.87)
    a, b, hc, hs, htc, hts = gpu_lib.fp4_swiglu_producer(xr[0], xr[1], wq[0], wq[1], mask, emit_cols)
    # a, b: bf16 of an fp32 value within the GEMM bound of the reference
    ref, e = G.gemm_ref(host(xr[0]), host(xr[1]), host(wq[0]), host(wq[1]))
    tol = G.GEMM_REL_TOL * e
    for got, lo_hi in ((host16(a), (ref[:, :f] - tol[:, :f], ref[:, :f] + tol[:, :f])),
                       (host16(b), (ref[:, f:] - tol[:, f:], ref[:, f:] + tol[:, f:]))):
        lo = F.bf16_bits_to_f64(S.f32_to_bf16_rne(lo_hi[0].astype(np.float32)))
        hi = F.bf16_bits_to_f64(S.f32_to_bf16_rne(lo_hi[1].astype(np.float32)))
        g = F.bf16_bits_to_f64(got)
        assert np.all((g >= lo) & (g <= hi))
    h = S.swiglu_h(host16(a), host16(b))
    want_r = Q.quantize_rows(h)
    assert_same(hc, want_r[0], "h row codes")
    assert_same(hs, want_r[1], "h row scales")
    if emit_cols:
        want_c = Q.quantize_cols(h, 32, mask)
        assert_same(htc, want_c[0], "h col codes")
        assert_same(hts, want_c[1], "h col scales")


@pytest.mark.parametrize("tfd", [(256, 128, 512), (288, 160, 256)])
def test_swiglu_producer_wide_range(gpu_lib, tfd):
    """Pre-activations spread over about +-300, so many waves hold some
    a < -87.3 (1 + exp(-a) > 2^126, where the batch divides instead of using
    the Newton reciprocal) and others none: h codes still bit-exact."""
    t, f, d = tfd
    x = synthetic.tensor((t, d), std=1.0, seed=27)
    w13 = synthetic.tensor((2 * f, d), std=4.0, seed=28)
    mask = P.sign_mask_from_seed(2)
    xr = gpu_lib.fp4_quantize_rows(dev16(x))
    wq = gpu_lib.fp4_quantize_w2d32(dev16(w13), 0.87)
    a, b, hc, hs, htc, hts = gpu_lib.fp4_swiglu_producer(xr[0], xr[1], wq[0], wq[1], mask, True)
    av = F.bf16_bits_to_f64(host16(a))
    assert (av < -87.4).any() and (av > -87.0).any()
    h = S.swiglu_h(host16(a), host16(b))
    for got, want, nm in zip((hc, hs, htc, hts), Q.quantize_rows(h) + Q.quantize_cols(h, 32, mask),
                             ("h row codes", "h row scales", "h col codes", "h col scales")):
        assert_same(got, want, nm)


@pytest.mark.parametrize("tf", [(64, 288), (256, 512), (32, 32)])
def test_swiglu_backward(gpu_lib, tf):
    t, f = tf
    a = synthetic.tensor((t, f), std=1.3, seed=24)
    b = synthetic.tensor((t, f), std=1.3, seed=25)
    a[0, :8] = np.array([0x0000, 0x8000, 0x4300, 0xC300, 0x42C8, 0xC2C8, 0x7F7F, 0xFF7F], dtype=np.uint16)
    # non-finite inputs: NaNs with payloads and either sign, infinities; every NaN result is 0x7FC0
    a[1, :8] = np.array([0x7FC1, 0xFFC0, 0x7F81, 0x7F80, 0xFF80, 0x3F80, 0xBF80, 0x0000], dtype=np.uint16)
    b[1, 4:8] = np.array([0x7F80, 0xFFA0, 0x0000, 0x7FFF], dtype=np.uint16)
    rng = np.random.default_rng(26)
    dh = (rng.standard_normal((t, f)) * 1e-3).astype(np.float32)
    dh[1, 8:12] = np.array([np.inf, -np.inf, np.nan, 0.0], dtype=np.float32)
    dh[1, 12:16] = np.uint32([0x7FC00001, 0xFFC00000, 0x7FA00000, 0x7F800001]).view(np.float32)
    b[1, 8:16] = np.array([0x0000, 0x3F80, 0x3F80, 0x7F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80], dtype=np.uint16)
    da, db = gpu_lib.fp4_swiglu_backward(torch.from_numpy(dh).cuda(), dev16(a), dev16(b))
    want_da, want_db = S.swiglu_backward(dh, a, b)
    assert np.array_equal(host16(da), want_da)
    assert np.array_equal(host16(db), want_db)


@pytest.mark.parametrize("tf", [(256, 256), (288, 160), (64, 96), (32, 32), (320, 416), (512, 128),
                                (512, 1024)])   # 8 x 2 workgroups: the XCD-aware block order
def test_swiglu_backward_producer(gpu_lib, tf):
    """Fused backward producer == SwiGLU backward, then SR rows and H32 cols
    of dA and dB (oracle composition and the unfused GPU calls)."""
    t, f = tf
    a = synthetic.tensor((t, f), std=1.3, seed=40)
    b = synthetic.tensor((t, f), std=1.3, seed=41)
    a[0, :8] = np.array([0x0000, 0x8000, 0x4300, 0xC300, 0x42C8, 0xC2C8, 0x7F7F, 0xFF7F], dtype=np.uint16)
    rng = np.random.default_rng(42)
    dh = (rng.standard_normal((t, f)) * 1e-3).astype(np.float32)
    dh[1, :32] = 0.0
    seed, oa, ob, mask = 2 ** 35 + 11, 5, 2 ** 33 + 9, P.sign_mask_from_seed(7)
    dhd, ad, bd = torch.from_numpy(dh).cuda(), dev16(a), dev16(b)
    (dar, dbr, dac, dbc) = gpu_lib.fp4_swiglu_backward_producer(dhd, ad, bd, seed, oa, ob, mask)
    da, db = S.swiglu_backward(dh, a, b)
    for got, want, nm in ((dar, Q.quantize_rows(da, Q.SR, seed, oa), "dA rows"),
                          (dbr, Q.quantize_rows(db, Q.SR, seed, ob), "dB rows"),
                          (dac, Q.quantize_cols(da, 32, mask), "dA cols"),
                          (dbc, Q.quantize_cols(db, 32, mask), "dB cols")):
        assert_same(got[0], want[0], nm + " codes")
        assert_same(got[1], want[1], nm + " scales")
    # same bytes as the unfused calls
    dag, dbg = gpu_lib.fp4_swiglu_backward(dhd, ad, bd)
    ref = (gpu_lib.fp4_quantize_rows(dag, gpu_lib.FP4_SR, seed, oa), gpu_lib.fp4_quantize_rows(dbg, gpu_lib.FP4_SR, seed, ob),
           gpu_lib.fp4_quantize_cols(dag, 32, mask), gpu_lib.fp4_quantize_cols(dbg, 32, mask))
    for got, want in zip((dar, dbr, dac, dbc), ref):
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])


def test_swiglu_backward_producer_nonfinite(gpu_lib):
    """NaN payloads of both signs and infinities in dH, a and b: the fused
    producer gives the bytes of the unfused calls (whose bf16 dA, dB carry the
    canonical NaN 0x7FC0), so a wave that meets a NaN takes the canonical
    packing.  Quantizer codes of non-finite blocks are outside the contract;
    only the fused/unfused agreement is checked there."""
    t, f = 128, 256
    a = synthetic.tensor((t, f), std=1.3, seed=46)
    b = synthetic.tensor((t, f), std=1.3, seed=47)
    rng = np.random.default_rng(48)
    dh = (rng.standard_normal((t, f)) * 1e-3).astype(np.float32)
    bits = dh.view(np.uint32)
    bits[3, 5] = 0x7FC00001
    bits[3, 6] = 0xFFA00000
    bits[70, 40] = 0x7F800001
    dh[9, 100] = np.inf
    dh[9, 101] = -np.inf
    a[20, 7] = 0x7F80                                    # +inf
    a[20, 8] = 0xFF80                                    # -inf
    a[90, 200] = 0x7FC3                                  # NaN with payload
    b[33, 64] = 0xFFC1
    b[33, 65] = 0x7F80
    dhd, ad, bd = torch.from_numpy(dh).cuda(), dev16(a), dev16(b)
    seed, oa, ob, mask = 5, 1, 2, P.sign_mask_from_seed(2)
    fused = gpu_lib.fp4_swiglu_backward_producer(dhd, ad, bd, seed, oa, ob, mask)
    dag, dbg = gpu_lib.fp4_swiglu_backward(dhd, ad, bd)
    want_da, want_db = S.swiglu_backward(dh, a, b)
    assert np.array_equal(host16(dag), want_da) and np.array_equal(host16(dbg), want_db)
    assert (want_da == 0x7FC0).sum() > 0 and (want_db == 0x7FC0).sum() > 0
    ref = (gpu_lib.fp4_quantize_rows(dag, gpu_lib.FP4_SR, seed, oa), gpu_lib.fp4_quantize_rows(dbg, gpu_lib.FP4_SR, seed, ob),
           gpu_lib.fp4_quantize_cols(dag, 32, mask), gpu_lib.fp4_quantize_cols(dbg, 32, mask))
    for got, want, nm in zip(fused, ref, ("dA rows", "dB rows", "dA cols", "dB cols")):
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), nm


@pytest.mark.parametrize("tfp", [(352, 160, 96), (96, 288, 8)])
def test_swiglu_backward_producer_strided_dh(gpu_lib, tfp):
    """dH read with a row pitch beyond f (a column slice of a wider buffer),
    and tiles whose last 64-token chunk holds only 32 tokens."""
    t, f, pad = tfp
    a = synthetic.tensor((t, f), std=1.3, seed=43)
    b = synthetic.tensor((t, f), std=1.3, seed=44)
    rng = np.random.default_rng(45)
    wide = (rng.standard_normal((t, f + pad)) * 1e-3).astype(np.float32)
    dh = np.ascontiguousarray(wide[:, :f])
    seed, oa, ob, mask = 3, 1, 2, P.sign_mask_from_seed(0)
    dhd = torch.from_numpy(wide).cuda()[:, :f]
    assert dhd.stride(0) == f + pad
    got = gpu_lib.fp4_swiglu_backward_producer(dhd, dev16(a), dev16(b), seed, oa, ob, mask)
    da, db = S.swiglu_backward(dh, a, b)
    want = (Q.quantize_rows(da, Q.SR, seed, oa), Q.quantize_rows(db, Q.SR, seed, ob),
            Q.quantize_cols(da, 32, mask), Q.quantize_cols(db, 32, mask))
    for g, w, nm in zip(got, want, ("dA rows", "dB rows", "dA cols", "dB cols")):
        assert_same(g[0], w[0], nm + " codes")
        assert_same(g[1], w[1], nm + " scales")


@pytest.mark.parametrize("tfd", [(256, 256, 256), (288, 160, 512), (512, 384, 256), (32, 32, 256), (96, 416, 768),
                                 (320, 288, 512)])
def test_gemm_swiglu_backward_producer(gpu_lib, tfd):
    """W2 Dgrad with the SwiGLU backward producer in its epilogue, ragged
    tiles included: every output byte equals fp4_gemm followed by
    fp4_swiglu_backward_producer, and the oracle's SwiGLU backward and
    quantizers on the GPU's dH (itself within the GEMM bound) give the same
    bytes.  Outputs start as sentinels, so every byte is written."""
    t, f, d = tfd
    dy = synthetic.tensor((t, d), std=1e-3, seed=50)
    w2 = synthetic.tensor((d, f), std=0.02, seed=51)
    a = synthetic.tensor((t, f), std=1.3, seed=52)
    b = synthetic.tensor((t, f), std=1.3, seed=53)
    seed, oa, ob, mask = 2 ** 33 + 5, 1, 2, P.sign_mask_from_seed(6)
    dyr = gpu_lib.fp4_quantize_rows(dev16(dy), gpu_lib.FP4_SR, seed, 0)
    w2q = gpu_lib.fp4_quantize_w2d32(dev16(w2), 0.87)
    ad, bd = dev16(a), dev16(b)
    shapes = [(t, f // 2), (t, f // 32), (t, f // 2), (t, f // 32), (f, t // 2), (f, t // 32), (f, t // 2),
              (f, t // 32)]
    outs = [torch.full(shp, 0xAB if i % 2 == 0 else 0xFF, dtype=torch.uint8, device="cuda")
            for i, shp in enumerate(shapes)]
    got = gpu_lib.fp4_gemm_swiglu_backward_producer(dyr[0], dyr[1], w2q[2], w2q[3], ad, bd, seed, oa, ob, mask, outs)
    dh = gpu_lib.fp4_gemm(dyr[0], dyr[1], w2q[2], w2q[3])
    check_gemm(dh, dyr, w2q[2:], what="W2 Dgrad dH")
    ref = gpu_lib.fp4_swiglu_backward_producer(dh, ad, bd, seed, oa, ob, mask)
    for g, r, nm in zip(got, ref, ("dA rows", "dB rows", "dA cols", "dB cols")):
        assert torch.equal(g[0], r[0]) and torch.equal(g[1], r[1]), nm
    da, db = S.swiglu_backward(host(dh), a, b)
    want = (Q.quantize_rows(da, Q.SR, seed, oa), Q.quantize_rows(db, Q.SR, seed, ob),
            Q.quantize_cols(da, 32, mask), Q.quantize_cols(db, 32, mask))
    for g, w, nm in zip(got, want, ("dA rows", "dB rows", "dA cols", "dB cols")):
        assert_same(g[0], w[0], nm + " codes")
        assert_same(g[1], w[1], nm + " scales")


def test_gemm_swiglu_backward_producer_rejects_short_k(gpu_lib):
    """The fused kernel runs the fast main loop only: d not a multiple of 256
    is refused before any launch."""
    t, f, d = 64, 64, 288
    dyr = gpu_lib.fp4_quantize_rows(dev16(synthetic.tensor((t, d), std=1e-3, seed=54)), gpu_lib.FP4_SR, 0, 0)
    w2q = gpu_lib.fp4_quantize_w2d32(dev16(synthetic.tensor((d, f), std=0.02, seed=55)), 0.87)
    ab = dev16(synthetic.tensor((t, f), std=1.0, seed=56))
    with pytest.raises(gpu_lib.Fp4Error):
        gpu_lib.fp4_gemm_swiglu_backward_producer(dyr[0], dyr[1], w2q[2], w2q[3], ab, ab, 0, 1, 2, 0)
    torch.cuda.synchronize()


def test_empty_tensors(gpu_lib):
    """Empty inputs give empty outputs (no launch)."""
    x = torch.empty((0, 64), dtype=torch.int16, device="cuda")
    codes, scales = gpu_lib.fp4_quantize_rows(x, gpu_lib.FP4_SR, 1, 2)
    assert tuple(codes.shape) == (0, 32) and tuple(scales.shape) == (0, 2)
    ct, st = gpu_lib.fp4_quantize_cols(torch.empty((0, 64), dtype=torch.int16, device="cuda"), 32, 5)
    assert tuple(ct.shape) == (64, 0) and tuple(st.shape) == (64, 0)
    a = torch.empty((0, 32), dtype=torch.uint8, device="cuda")
    sa = torch.empty((0, 2), dtype=torch.uint8, device="cuda")
    c = gpu_lib.fp4_gemm(a, sa, a, sa)
    assert tuple(c.shape) == (0, 0)
    torch.cuda.synchronize()


def test_gemm_k0_is_an_empty_sum(gpu_lib):
    """K = 0: every element of C is the empty sum 0; accumulating leaves C."""
    m, n = 96, 160
    a = torch.empty((m, 0), dtype=torch.uint8, device="cuda")
    sa = torch.empty((m, 0), dtype=torch.uint8, device="cuda")
    b = torch.empty((n, 0), dtype=torch.uint8, device="cuda")
    sb = torch.empty((n, 0), dtype=torch.uint8, device="cuda")
    c = torch.full((m, n), 7.5, dtype=torch.float32, device="cuda")
    gpu_lib.fp4_gemm(a, sa, b, sb, c=c, accumulate=True)
    assert torch.all(c == 7.5)
    gpu_lib.fp4_gemm(a, sa, b, sb, c=c)
    ref, e = G.gemm_ref(np.zeros((m, 0), np.uint8), np.zeros((m, 0), np.uint8),
                        np.zeros((n, 0), np.uint8), np.zeros((n, 0), np.uint8))
    assert np.array_equal(host(c).astype(np.float64), ref) and not np.any(e)


def test_swiglu_producer_d0(gpu_lib):
    """d = 0: a = b = 0, h = SiLU(0) * 0 = 0, quantized as all-zero blocks."""
    t, f = 64, 96
    x = torch.empty((t, 0), dtype=torch.uint8, device="cuda")
    xs = torch.empty((t, 0), dtype=torch.uint8, device="cuda")
    w = torch.empty((2 * f, 0), dtype=torch.uint8, device="cuda")
    ws = torch.empty((2 * f, 0), dtype=torch.uint8, device="cuda")
    outs = [torch.full(shp, 0x55, dtype=dt, device="cuda") for shp, dt in
            (((t, f), torch.int16), ((t, f), torch.int16), ((t, f // 2), torch.uint8), ((t, f // 32), torch.uint8),
             ((f, t // 2), torch.uint8), ((f, t // 32), torch.uint8))]
    gpu_lib.fp4_swiglu_producer(x, xs, w, ws, P.sign_mask_from_seed(0), True, *outs)
    zero = np.zeros((t, f), dtype=np.uint16)
    h = S.swiglu_h(zero, zero)
    want = Q.quantize_rows(h) + Q.quantize_cols(h, 32, P.sign_mask_from_seed(0))
    assert np.array_equal(host16(outs[0]), zero) and np.array_equal(host16(outs[1]), zero)
    for got, wv in zip(outs[2:], want):
        assert_same(got, wv, "d=0 output")


def test_run_twice_bitwise_deterministic(gpu_lib):
    x = synthetic.tensor((512, 1024), std=1.0, seed=27)
    w = synthetic.tensor((768, 1024), std=0.02, seed=28)
    xd, wd = dev16(x), dev16(w)
    outs = []
    for _ in range(2):
        xr = gpu_lib.fp4_quantize_rows(xd, gpu_lib.FP4_SR, 3, 4)
        wq = gpu_lib.fp4_quantize_w2d32(wd)
        outs.append([host(t) for t in xr + wq + (gpu_lib.fp4_gemm(xr[0], xr[1], wq[0], wq[1]),)])
    for u, v in zip(*outs):
        assert np.array_equal(u, v)


def test_outputs_fully_written(gpu_lib):
    # sentinel-filled outputs: every byte must be overwritten
    x = synthetic.tensor((160, 352), std=1.0, seed=29)
    codes = torch.full((160, 176), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((160, 11), 0xFF, dtype=torch.uint8, device="cuda")
    gpu_lib.fp4_quantize_rows(dev16(x), codes=codes, scales=scales)
    want = Q.quantize_rows(x)
    assert_same(codes, want[0], "codes")
    assert_same(scales, want[1], "scales")
    ct = torch.full((352, 80), 0xAB, dtype=torch.uint8, device="cuda")
    st = torch.full((352, 5), 0xFF, dtype=torch.uint8, device="cuda")
    gpu_lib.fp4_quantize_cols(dev16(x), 32, 0x1234, codes_t=ct, scales_t=st)
    want = Q.quantize_cols(x, 32, 0x1234)
    assert_same(ct, want[0], "col codes")
    assert_same(st, want[1], "col scales")
