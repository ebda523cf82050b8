"""GPU parity of the CTA-local NVFP4 calls against oracle/nvfp4.py.

Bar: codes, E4M3 scale bytes, panel maxima and factors bit-exact (RTN and SR);
the contraction within |C - C_ref| <= 1e-5 * E + k * 2^-150 per element, E the
factored magnitude sum (the MX GEMM's bound: the inner products are exact in
bf16 and the sum is fp32, as there).
"""

import numpy as np
import pytest
import torch

import synthetic
from oracle import formats as F
from oracle import gemm as G
from oracle import nvfp4 as N

pytestmark = pytest.mark.gpu


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_same(got, want, what):
    got = host(got)
    want = np.asarray(want)
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        want = np.asarray(want, dtype=np.float32).view(np.uint32)
    if got.shape != want.shape or not np.array_equal(got, want):
        bad = np.argwhere(got != want) if got.shape == want.shape else np.zeros((1, got.ndim), dtype=int)
        raise AssertionError(f"{what}: shape {got.shape} vs {want.shape}, {len(bad)} mismatches, first at "
                             f"{bad[:5].tolist()}")


def scaled(bits, f):
    """bf16 patterns of the values times a power of two (exact)."""
    return synthetic.bf16_bits((F.bf16_bits_to_f64(bits) * f).astype(np.float32))


def check_rows(lib, x, mode=N.RTN, seed=0, offset=0):
    got = lib.fp4_nv_quantize_rows(dev16(x), mode, seed, offset)
    want = N.quantize_rows(x, mode, seed, offset)
    for g, w, nm in zip(got, want, ("codes", "scales", "factors", "panel maxima")):
        assert_same(g, w, nm)
    return got


ROW_SHAPES = [(256, 512), (320, 544), (96, 4128), (32, 32), (600, 96)]


@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_nv_rows_rtn(gpu_lib, shape):
    x = synthetic.tensor(shape, std=1.0, seed=31, outlier_rate=0.002, outlier_scale=40.0)
    x[0, :16] = 0
    x[-1, 5] = 0x8000                                          # -0
    check_rows(gpu_lib, x)


@pytest.mark.parametrize("shape", ROW_SHAPES)
@pytest.mark.parametrize("seed,offset", [(0, 0), (12345, 7), (2 ** 40 + 3, 2 ** 33 + 1)])
def test_nv_rows_sr(gpu_lib, shape, seed, offset):
    dy = synthetic.tensor(shape, std=1e-3, seed=32, outlier_rate=0.01, outlier_scale=50.0)
    check_rows(gpu_lib, dy, N.SR, seed, offset)


def test_nv_rows_panels_of_different_ranges(gpu_lib):
    """Each 256-row panel owns its factor: panels whose ranges differ by 2^40,
    an all-zero panel (S = 1) and a panel holding one non-zero value."""
    x = synthetic.tensor((1024 + 64, 160), std=1.0, seed=33)
    xv = x.view(np.uint16)
    xv[256:512] = scaled(xv[256:512], 2.0 ** -40)
    xv[512:768] = 0
    xv[768:1024] = 0
    xv[900, 17] = synthetic.bf16_bits(np.array([-3.0e5], dtype=np.float32))[0]
    for mode in (N.RTN, N.SR):
        check_rows(gpu_lib, x, mode, 5, 9)


def test_nv_rows_vanishing_blocks_and_extremes(gpu_lib):
    """Blocks far below the panel maximum vanish (E4M3 scale 0); values up to
    the largest finite bf16; panel maxima down to 2^-100."""
    x = np.zeros((512, 64), dtype=np.uint16)
    big = synthetic.bf16_bits(np.array([3.3e38, -1.0e-30, 7.0, 1.0e-6], dtype=np.float32))
    x[0, 0] = big[0]
    x[1, 16:32] = big[1]
    x[2, 32:48] = big[2]
    x[3, 48:64] = big[3]
    tiny = synthetic.tensor((256, 64), std=1.0, seed=34).view(np.uint16)
    x[256:] = scaled(tiny, 2.0 ** -100)
    for mode in (N.RTN, N.SR):
        check_rows(gpu_lib, x, mode, 1, 2)


def test_nv_rows_strided_input(gpu_lib):
    full = synthetic.tensor((288, 640), std=1.0, seed=35)
    xd = dev16(full)[:, 64:576]
    got = gpu_lib.fp4_nv_quantize_rows(xd, N.SR, 3, 4)
    want = N.quantize_rows(np.ascontiguousarray(full[:, 64:576]), N.SR, 3, 4)
    for g, w, nm in zip(got, want, ("codes", "scales", "factors", "panel maxima")):
        assert_same(g, w, nm)


W_SHAPES = [(512, 512), (352, 416), (32, 64), (4096, 160), (96, 160), (160, 4128)]


@pytest.mark.parametrize("shape", W_SHAPES)
def test_nv_w2d16(gpu_lib, shape):
    w = synthetic.tensor(shape, std=0.02, seed=36, outlier_rate=0.001, outlier_scale=30.0)
    w[:16, :16] = 0                                              # an all-zero tile
    got = gpu_lib.fp4_nv_quantize_w2d16(dev16(w))
    rc, rs, cc, cs, S, amax = N.quantize_w2d16(w)
    for g, want, nm in zip(got, (rc, rs, cc, cs, [S], [amax]),
                           ("row_codes", "row_scales", "col_codes", "col_scales", "factor", "amax")):
        assert_same(g, want, nm)


def test_nv_w2d16_strided_and_zero(gpu_lib):
    full = synthetic.tensor((128, 320), std=0.5, seed=37)
    got = gpu_lib.fp4_nv_quantize_w2d16(dev16(full)[:, 32:288])
    want = N.quantize_w2d16(np.ascontiguousarray(full[:, 32:288]))
    for g, w, nm in zip(got, (*want[:4], [want[4]], [want[5]]), ("rc", "rs", "cc", "cs", "S", "amax")):
        assert_same(g, w, nm)
    z = np.zeros((64, 96), dtype=np.uint16)
    got = gpu_lib.fp4_nv_quantize_w2d16(dev16(z))
    assert host(got[4])[0] == 1.0 and host(got[5])[0] == 0.0
    assert not host(got[0]).any() and not host(got[1]).any() and not host(got[2]).any()


def panel_factors(f, rows):
    """A one-element factor vector (shared by all rows) as one factor per panel."""
    f = np.asarray(f, dtype=np.float32).reshape(-1)
    return np.repeat(f, (rows + N.PANEL - 1) // N.PANEL) if f.size == 1 else f


def check_nv_gemm(c, a, b, k, c_prev=None, what="nv gemm"):
    fa, fb = panel_factors(host(a[2]), a[0].shape[0]), panel_factors(host(b[2]), b[0].shape[0])
    ref, e = N.gemm_ref(host(a[0]), host(a[1]), fa, host(b[0]), host(b[1]), fb)
    ok = G.within_bound(host(c), ref, e, c_prev=c_prev, k=k)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements outside bound; first {i}: got {host(c)[i]} "
                             f"ref {ref[i]} E {e[i]}")


MNK = [(256, 512, 512), (288, 352, 576), (512, 256, 1024), (32, 32, 64), (96, 544, 320), (544, 96, 192)]


@pytest.mark.parametrize("mnk", MNK)
def test_nv_gemm_rows_by_rows(gpu_lib, mnk):
    """Both operands with per-panel factors (row factor x column factor)."""
    m, n, k = mnk
    x = synthetic.tensor((m, k), std=1.0, seed=38, outlier_rate=0.002, outlier_scale=20.0)
    w = synthetic.tensor((n, k), std=0.05, seed=39)
    if n > 256:
        w[256:] = scaled(w[256:], 64.0)                              # the second B panel has another factor
    a = gpu_lib.fp4_nv_quantize_rows(dev16(x))[:3]
    b = gpu_lib.fp4_nv_quantize_rows(dev16(w))[:3]
    c = gpu_lib.fp4_nv_gemm(*a, *b)
    check_nv_gemm(c, a, b, k)
    prev = host(c).copy()
    gpu_lib.fp4_nv_gemm(*a, *b, c=c, accumulate=True)
    check_nv_gemm(c, a, b, k, c_prev=prev, what="nv gemm accumulate")


@pytest.mark.parametrize("mnk", [(288, 352, 512), (512, 512, 256), (64, 160, 128)])
def test_nv_gemm_dgrad_route(gpu_lib, mnk):
    """The CTA-local Dgrad: dX = Q_r^SR(dY) W with the weight's 2D16 column
    view and its one common factor (stride 0)."""
    t, d, f = mnk
    dy = synthetic.tensor((t, f), std=1e-3, seed=40, outlier_rate=0.01, outlier_scale=30.0)
    w = synthetic.tensor((f, d), std=0.02, seed=41)                     # W [f][d]: Y = X W^T
    a = gpu_lib.fp4_nv_quantize_rows(dev16(dy), N.SR, 11, 13)[:3]
    rc, rs, cc, cs, S, _ = gpu_lib.fp4_nv_quantize_w2d16(dev16(w))
    c = gpu_lib.fp4_nv_gemm(*a, cc, cs, S)
    check_nv_gemm(c, a, (cc, cs, S), f)
    # the same product from the oracle's own operands, end to end
    ac, asc, af, _ = N.quantize_rows(dy, N.SR, 11, 13)
    _, _, occ, ocs, oS, _ = N.quantize_w2d16(w)
    ref, e = N.gemm_ref(ac, asc, af, occ, ocs, panel_factors(oS, d))
    assert G.within_bound(host(c), ref, e, k=f).all()


def test_nv_gemm_zero_factors_and_empty_sums(gpu_lib):
    m, n = 64, 96
    c = torch.full((m, n), 5.0, device="cuda")
    gpu_lib.fp4_nv_gemm(torch.empty((m, 0), dtype=torch.uint8, device="cuda"),
                        torch.empty((m, 0), dtype=torch.uint8, device="cuda"), torch.ones(1, device="cuda"),
                        torch.empty((n, 0), dtype=torch.uint8, device="cuda"),
                        torch.empty((n, 0), dtype=torch.uint8, device="cuda"), torch.ones(1, device="cuda"), c=c)
    assert not host(c).any()
    z = np.zeros((m, 128), dtype=np.uint16)
    a = gpu_lib.fp4_nv_quantize_rows(dev16(z))[:3]
    b = gpu_lib.fp4_nv_quantize_rows(dev16(synthetic.tensor((n, 128), std=1.0, seed=42)))[:3]
    c = gpu_lib.fp4_nv_gemm(*a, *b)
    assert not host(c).any()


def test_nv_binding_refusals(gpu_lib):
    x = dev16(synthetic.tensor((64, 64), std=1.0, seed=43))
    a = gpu_lib.fp4_nv_quantize_rows(x)[:3]
    with pytest.raises(gpu_lib.Fp4Error):
        a16, s2 = a[0][:, :16].contiguous(), a[1][:, :2].contiguous()
        gpu_lib.fp4_nv_gemm(a16, s2, a[2], a16, s2, a[2])                # k = 32: not a multiple of 64
    with pytest.raises(gpu_lib.Fp4Error):
        gpu_lib.fp4_nv_gemm(*a, a[0], a[1], torch.ones(3, device="cuda"))
    with pytest.raises(gpu_lib.Fp4Error):
        gpu_lib.fp4_nv_quantize_rows(dev16(synthetic.tensor((64, 48), std=1.0, seed=44)))


def test_nv_outputs_fully_written(gpu_lib):
    """Sentinel-filled outputs: every byte and factor is overwritten."""
    x = synthetic.tensor((320, 544), std=1.0, seed=45)
    outs = [torch.full((320, 272), 0xAB, dtype=torch.uint8, device="cuda"),
            torch.full((320, 34), 0xAB, dtype=torch.uint8, device="cuda"),
            torch.full((2,), float("nan"), device="cuda"), torch.full((2,), float("nan"), device="cuda")]
    got = gpu_lib.fp4_nv_quantize_rows(dev16(x), N.SR, 1, 1, out=outs)
    want = N.quantize_rows(x, N.SR, 1, 1)
    for g, w, nm in zip(got, want, ("codes", "scales", "factors", "amax")):
        assert_same(g, w, nm)
    w = synthetic.tensor((96, 160), std=0.1, seed=46)
    outs = [torch.full(s, 0xAB, dtype=torch.uint8, device="cuda") for s in ((96, 80), (96, 10), (160, 48), (160, 6))]
    outs += [torch.full((1,), float("nan"), device="cuda"), torch.full((1,), float("nan"), device="cuda")]
    got = gpu_lib.fp4_nv_quantize_w2d16(dev16(w), out=outs)
    want = N.quantize_w2d16(w)
    for g, ww, nm in zip(got, (*want[:4], [want[4]], [want[5]]), ("rc", "rs", "cc", "cs", "S", "amax")):
        assert_same(g, ww, nm)
    a = gpu_lib.fp4_nv_quantize_rows(dev16(x[:, :512]))[:3]
    b = gpu_lib.fp4_nv_quantize_rows(dev16(synthetic.tensor((96, 512), std=1.0, seed=47)))[:3]
    c = torch.full((320, 96), float("nan"), device="cuda")
    gpu_lib.fp4_nv_gemm(*a, *b, c=c)
    check_nv_gemm(c, a, b, 512)


def pick(n, k, rng, step=1):
    groups = n // step
    idx = rng.choice(groups, size=min(k, groups), replace=False)
    return (np.unique(np.concatenate([idx, [0, groups - 1]])) * step).astype(np.int64)


def test_nv_dgrad_route_full_size(gpu_lib):
    """The CTA-local Dgrad of the FFN step at full size (T 8192, D 4096,
    F 14336), with the calls and shapes `bench.py --nvfp4-dgrad` times:
    row SR of dY and of a dA-shaped gradient, 2D16 of W2 and W1, dH = dY W2
    (K 4096) and dX = dA W1 (K 14336).  Whole sampled panels (row producer)
    and 32-row strips (2D16, with the tensor's factor) bit-exact; sampled
    outputs of both contractions within the GEMM bound."""
    h = synthetic.workload("ffn_step_8192x4096x14336")
    rng = np.random.default_rng(7)
    seed = 0
    dY, W2, W1 = h["dY"], h["W2"], h["W1"]
    T, D = dY.shape
    F_ = W1.shape[0]
    dA = synthetic.tensor((T, F_), std=1e-3, seed=48, outlier_rate=0.001, outlier_scale=20.0)
    # row producer: three whole panels (first, last, one between) per tensor
    q_dy = gpu_lib.fp4_nv_quantize_rows(dev16(dY), N.SR, seed, 0)
    q_da = gpu_lib.fp4_nv_quantize_rows(dev16(dA), N.SR, seed, 1)
    for x, q, off in ((dY, q_dy, 0), (dA, q_da, 1)):
        panels = x.shape[0] // N.PANEL
        for p in sorted({0, panels - 1, int(rng.integers(1, panels - 1))}):
            r0 = p * N.PANEL
            want = N.quantize_rows(x[r0:r0 + N.PANEL], N.SR, seed, off, row0=r0)
            assert_same(q[0][r0:r0 + N.PANEL], want[0], f"codes panel {p}")
            assert_same(q[1][r0:r0 + N.PANEL], want[1], f"scales panel {p}")
            assert_same(q[2][p:p + 1], want[2], f"factor panel {p}")
            assert_same(q[3][p:p + 1], want[3], f"panel max {p}")
    # 2D16 weights: the whole-tensor maximum and factor, then sampled strips
    q_w2 = gpu_lib.fp4_nv_quantize_w2d16(dev16(W2))
    q_w1 = gpu_lib.fp4_nv_quantize_w2d16(dev16(W1))
    for w, q in ((W2, q_w2), (W1, q_w1)):
        amax = np.float32(np.abs(F.bf16_bits_to_f64(w)).max())
        assert host(q[5])[0] == amax
        S = N.outer_factor(amax)
        assert host(q[4])[0] == S
        for n0 in pick(w.shape[0], 3, rng, step=32):
            want = N.quantize_w2d16(w[n0:n0 + 32], factor=S)
            assert_same(q[0][n0:n0 + 32], want[0], f"row codes strip {n0}")
            assert_same(q[1][n0:n0 + 32], want[1], f"row scales strip {n0}")
            assert_same(q[2][:, n0 // 2:n0 // 2 + 16], want[2], f"col codes strip {n0}")
            assert_same(q[3][:, n0 // 16:n0 // 16 + 2], want[3], f"col scales strip {n0}")
    # contractions, sampled outputs against the exact reference on the GPU's codes
    for a, b, k in ((q_dy, q_w2, D), (q_da, q_w1, F_)):
        c = gpu_lib.fp4_nv_gemm(a[0], a[1], a[2], b[2], b[3], b[4])
        m, n = c.shape
        rows, cols = pick(m, 96, rng), pick(n, 1024, rng)
        fb = panel_factors(host(b[4]), n)
        ref, e = N.gemm_ref(host(a[0]), host(a[1]), host(a[2]), host(b[2]), host(b[3]), fb, rows=rows, cols=cols)
        got = host(c)[np.ix_(rows, cols)]
        ok = G.within_bound(got, ref, e, k=k)
        assert ok.all(), f"k={k}: {np.count_nonzero(~ok)} sampled outputs outside the bound"
        del c
        torch.cuda.empty_cache()


def test_nv_long_k_and_tall_tensor(gpu_lib):
    """Size extremes: a contraction over K = 65536 (1024 steps; the bound
    holds over the long fp32 sum) and a row producer over 131072 x 32 (the
    grid's rows loop and the largest maxima batches), checked on panels."""
    k = 65536
    a_bits = synthetic.tensor((32, k), std=1.0, seed=49, outlier_rate=0.001, outlier_scale=30.0)
    b_bits = synthetic.tensor((96, k), std=0.02, seed=50)
    a = gpu_lib.fp4_nv_quantize_rows(dev16(a_bits), N.SR, 2, 3)[:3]
    b = gpu_lib.fp4_nv_quantize_rows(dev16(b_bits))[:3]
    want_a = N.quantize_rows(a_bits, N.SR, 2, 3)
    assert_same(a[0], want_a[0], "long-k codes")
    assert_same(a[1], want_a[1], "long-k scales")
    c = gpu_lib.fp4_nv_gemm(*a, *b)
    check_nv_gemm(c, a, b, k, what="nv gemm k 65536")
    rows = 131072
    x = synthetic.tensor((rows, 32), std=1.0, seed=51)
    x[rows // 2: rows // 2 + 256] = 0                              # one all-zero panel in the middle
    q = gpu_lib.fp4_nv_quantize_rows(dev16(x), N.SR, 4, 5)
    for p in (0, 255, 256, 511):
        r0 = p * N.PANEL
        want = N.quantize_rows(x[r0:r0 + N.PANEL], N.SR, 4, 5, row0=r0)
        for g, w, nm in zip(q, want, ("codes", "scales", "factor", "max")):
            got = g[r0:r0 + N.PANEL] if nm in ("codes", "scales") else g[p:p + 1]
            assert_same(got, w, f"tall tensor {nm} panel {p}")


def test_nv_gemm_strided_c(gpu_lib):
    """C as a column slice of a wider fp32 tensor (ldc > n): the columns
    outside the slice keep their values, with and without accumulation."""
    m, n, k = 288, 160, 192
    a = gpu_lib.fp4_nv_quantize_rows(dev16(synthetic.tensor((m, k), std=1.0, seed=52)))[:3]
    b = gpu_lib.fp4_nv_quantize_rows(dev16(synthetic.tensor((n, k), std=0.1, seed=53)))[:3]
    wide = torch.full((m, n + 96), 7.0, device="cuda")
    view = wide[:, 32:32 + n]
    gpu_lib.fp4_nv_gemm(*a, *b, c=view)
    check_nv_gemm(view, a, b, k)
    prev = host(view).copy()
    gpu_lib.fp4_nv_gemm(*a, *b, c=view, accumulate=True)
    check_nv_gemm(view, a, b, k, c_prev=prev, what="strided accumulate")
    w = host(wide)
    assert np.all(w[:, :32] == 7.0) and np.all(w[:, 32 + n:] == 7.0)
