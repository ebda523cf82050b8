"""Seeded sweep of random shapes through every hot-path call: all
dimensions random multiples of 32 (ragged tiles on every side), strided
inputs and outputs where the call takes a pitch, both rounding modes, both
Hadamard settings.  Each case is checked against the oracle to the same bar
as the fixed-shape parity tests: codes and scales bit-exact, GEMM outputs
within |C - C_ref| <= 1e-5 * sum_k |a_k b_k|.  Each case prints its name
before it runs."""

import numpy as np
import pytest
import torch

import synthetic
from oracle import gemm as G
from oracle import philox as P
from oracle import quant as Q
from oracle import swiglu as S
from oracle import formats as F

pytestmark = pytest.mark.gpu

CASES = 16


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host16(t):
    return host(t).view(np.uint16)


def same(got, want, what):
    got = host(got)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}")


def case(name):
    print(f"[sweep] {name}", flush=True)


def dims(rng, hi, n=2):
    return [32 * int(v) for v in rng.integers(1, hi + 1, size=n)]


def strided(x, rng):
    """x as a device view with a row pitch up to 96 values beyond its width."""
    pad = 32 * int(rng.integers(0, 4))
    if pad == 0:
        return dev16(x)
    wide = np.zeros((x.shape[0], x.shape[1] + pad), dtype=np.uint16)
    lead = 32 * int(rng.integers(0, pad // 32 + 1))
    wide[:, lead:lead + x.shape[1]] = x
    return dev16(wide)[:, lead:lead + x.shape[1]]


def test_sweep_quantizers(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(2024)
    for i in range(CASES):
        r, c = dims(rng, 40)
        seed, off = int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40))
        mask = P.sign_mask_from_seed(i)
        x = synthetic.tensor((r, c), std=float(10.0 ** rng.uniform(-4, 1)), seed=100 + i, outlier_rate=0.01,
                             outlier_scale=30.0)
        xd = strided(x, rng)
        case(f"quantizers {r}x{c} pitch {xd.stride(0)}")
        for mode in (Q.RTN, Q.SR):
            got = mx.fp4_quantize_rows(xd, mode, seed, off)
            want = Q.quantize_rows(x, mode, seed, off)
            same(got[0], want[0], f"rows mode {mode} codes")
            same(got[1], want[1], f"rows mode {mode} scales")
        for had in (0, 32):
            got = mx.fp4_quantize_cols(xd, had, mask)
            want = Q.quantize_cols(x, had, mask)
            same(got[0], want[0], f"cols H{had} codes")
            same(got[1], want[1], f"cols H{had} scales")
        mode, had = int(rng.integers(0, 2)), 32 * int(rng.integers(0, 2))
        got = mx.fp4_quantize_dual(xd, mode, seed, off, had, mask)
        want = Q.quantize_rows(x, Q.SR if mode else Q.RTN, seed, off) + Q.quantize_cols(x, had, mask)
        for g, w, nm in zip(got, want, ("row codes", "row scales", "col codes", "col scales")):
            same(g, w, f"dual mode {mode} H{had} {nm}")
        ratio = 0.87 if i % 2 == 0 else 0.0
        got = mx.fp4_quantize_w2d32(xd, ratio)
        for g, w, nm in zip(got, Q.quantize_w2d32(x, ratio), ("row codes", "row scales", "col codes", "col scales")):
            same(g, w, f"2D32 ratio {ratio} {nm}")


def quantized(mx, rows, k, std, seed):
    x = synthetic.tensor((rows, k), std=std, seed=seed, outlier_rate=0.001, outlier_scale=20.0)
    return mx.fp4_quantize_rows(dev16(x))


def within(c, pairs, c_prev=None):
    ref = e = 0
    for a, b in pairs:
        r, ee = G.gemm_ref(host(a[0]), host(a[1]), host(b[0]), host(b[1]))
        ref, e = ref + r, e + ee
    ok = G.within_bound(host(c), ref, e, c_prev=c_prev)
    return ok.all(), int((~ok).sum())


def test_sweep_gemm(gpu_lib):
    """Plain, accumulating and pair-form products with C as a column slice of
    a wider tensor; K drawn so that both the K % 256 == 0 kernel and the
    generic one are reached."""
    mx = gpu_lib
    rng = np.random.default_rng(2025)
    for i in range(2 * CASES):
        m, n = dims(rng, 30)
        k = 256 * int(rng.integers(1, 5)) if i % 2 == 0 else 32 * int(rng.integers(1, 49))
        pad = 32 * int(rng.integers(0, 3))
        case(f"gemm {m}x{n}x{k} ldc {n + pad}")
        a, b = quantized(mx, m, k, 1.0, 200 + 4 * i), quantized(mx, n, k, 0.02, 201 + 4 * i)
        a2, b2 = quantized(mx, m, k, 1e-3, 202 + 4 * i), quantized(mx, n, k, 0.5, 203 + 4 * i)
        wide = torch.full((m, n + pad), float("nan"), device="cuda")
        c = mx.fp4_gemm(a[0], a[1], b[0], b[1], c=wide[:, :n])
        ok, nbad = within(c, [(a, b)])
        assert ok, f"plain: {nbad} outside the bound"
        if pad:
            assert torch.isnan(wide[:, n:]).all(), "wrote past the C slice"
        prev = host(c).copy()
        mx.fp4_gemm_pair(*a, *b, *a2, *b2, c=c, accumulate=True)
        ok, nbad = within(c, [(a, b), (a2, b2)], c_prev=prev)
        assert ok, f"pair accumulate: {nbad} outside the bound"


def test_sweep_grouped_gemm(gpu_lib):
    """Groups of two to four random products (mixed K, plain and pair form):
    each C has the bytes of the same product run alone."""
    mx = gpu_lib
    rng = np.random.default_rng(2026)
    for g in range(8):
        probs, alone = [], []
        count = int(rng.integers(2, 5))
        names = []
        for q in range(count):
            m, n = dims(rng, 24)
            k = 256 * int(rng.integers(1, 4)) if rng.integers(0, 3) else 32 * int(rng.integers(1, 33))
            a, b = quantized(mx, m, k, 1.0, 300 + 10 * g + q), quantized(mx, n, k, 0.02, 400 + 10 * g + q)
            pr = dict(a_codes=a[0], a_scales=a[1], b_codes=b[0], b_scales=b[1])
            if rng.integers(0, 2):
                a2, b2 = quantized(mx, m, k, 0.1, 500 + 10 * g + q), quantized(mx, n, k, 0.02, 600 + 10 * g + q)
                pr.update(a2_codes=a2[0], a2_scales=a2[1], b2_codes=b2[0], b2_scales=b2[1])
                alone.append(mx.fp4_gemm_pair(*a, *b, *a2, *b2))
            else:
                alone.append(mx.fp4_gemm(*a, *b))
            probs.append(pr)
            names.append(f"{m}x{n}x{k}{'p' if 'a2_codes' in pr else ''}")
        case(f"grouped {' '.join(names)}")
        outs = mx.fp4_gemm_grouped(probs)
        for q, (x, y) in enumerate(zip(outs, alone)):
            assert np.array_equal(host(x).view(np.uint32), host(y).view(np.uint32)), f"problem {q}"


def test_sweep_swiglu_producer(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(2027)
    for i in range(CASES):
        t, f = dims(rng, 12)
        d = 256 * int(rng.integers(1, 4)) if i % 2 == 0 else 32 * int(rng.integers(1, 25))
        case(f"swiglu producer t {t} f {f} d {d}")
        x = synthetic.tensor((t, d), std=1.0, seed=700 + i)
        w13 = synthetic.tensor((2 * f, d), std=0.05, seed=800 + i)
        mask = P.sign_mask_from_seed(i)
        xr = mx.fp4_quantize_rows(dev16(x))
        wq = mx.fp4_quantize_w2d32(dev16(w13), 0.87)
        a, b, hc, hs, htc, hts = mx.fp4_swiglu_producer(xr[0], xr[1], wq[0], wq[1], mask, True)
        ref, e = G.gemm_ref(host(xr[0]), host(xr[1]), host(wq[0]), host(wq[1]))
        tol = G.GEMM_REL_TOL * e
        for got, sl in ((host16(a), slice(0, f)), (host16(b), slice(f, 2 * f))):
            lo = F.bf16_bits_to_f64(S.f32_to_bf16_rne((ref[:, sl] - tol[:, sl]).astype(np.float32)))
            hi = F.bf16_bits_to_f64(S.f32_to_bf16_rne((ref[:, sl] + tol[:, sl]).astype(np.float32)))
            gv = F.bf16_bits_to_f64(got)
            assert np.all((gv >= lo) & (gv <= hi)), "a or b outside the GEMM bound"
        h = S.swiglu_h(host16(a), host16(b))
        want_r, want_c = Q.quantize_rows(h), Q.quantize_cols(h, 32, mask)
        same(hc, want_r[0], "h row codes")
        same(hs, want_r[1], "h row scales")
        same(htc, want_c[0], "h col codes")
        same(hts, want_c[1], "h col scales")


def test_sweep_swiglu_backward_producer(gpu_lib):
    mx = gpu_lib
    rng = np.random.default_rng(2028)
    for i in range(CASES):
        t, f = dims(rng, 20)
        case(f"backward producer t {t} f {f}")
        a = synthetic.tensor((t, f), std=1.3, seed=900 + i)
        b = synthetic.tensor((t, f), std=1.3, seed=950 + i)
        dh = (rng.standard_normal((t, f)) * 10.0 ** rng.uniform(-5, 0)).astype(np.float32)
        seed, oa, ob = int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40)), int(rng.integers(0, 2 ** 40))
        mask = P.sign_mask_from_seed(i + 3)
        got = mx.fp4_swiglu_backward_producer(torch.from_numpy(dh).cuda(), dev16(a), dev16(b), seed, oa, ob, mask)
        da, db = S.swiglu_backward(dh, a, b)
        want = (Q.quantize_rows(da, Q.SR, seed, oa), Q.quantize_rows(db, Q.SR, seed, ob),
                Q.quantize_cols(da, 32, mask), Q.quantize_cols(db, 32, mask))
        for g, w, nm in zip(got, want, ("dA rows", "dB rows", "dA cols", "dB cols")):
            same(g[0], w[0], nm + " codes")
            same(g[1], w[1], nm + " scales")


def test_sweep_nvfp4(gpu_lib):
    """CTA-local NVFP4: rows (RTN and SR, strided input) and 2D16 weights
    bit-exact against the oracle, and the contraction over rows x rows and
    rows x 2D16 columns (one common factor) within the GEMM bound."""
    from oracle import nvfp4 as N
    mx = gpu_lib

    def same_f32(got, want, what):
        same(got.view(torch.int32), np.asarray(want, dtype=np.float32).view(np.int32), what)

    def factors(f, rows):
        f = np.asarray(f, dtype=np.float32).reshape(-1)
        return np.repeat(f, (rows + N.PANEL - 1) // N.PANEL) if f.size == 1 else f

    rng = np.random.default_rng(2029)
    for i in range(CASES):
        m, n = dims(rng, 20)
        k = 64 * int(rng.integers(1, 17))
        seed, off = int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40))
        case(f"nvfp4 {m}x{n}x{k}")
        x = synthetic.tensor((m, k), std=float(10.0 ** rng.uniform(-4, 0)), seed=1000 + i, outlier_rate=0.005,
                             outlier_scale=30.0)
        w = synthetic.tensor((n, k), std=0.02, seed=1100 + i)
        mode = N.SR if i % 2 else N.RTN
        a = mx.fp4_nv_quantize_rows(strided(x, rng), mode, seed, off)
        for g, wv, nm in zip(a, N.quantize_rows(x, mode, seed, off), ("codes", "scales", "factors", "maxima")):
            if nm in ("factors", "maxima"):
                same_f32(g, wv, f"rows {nm}")
            else:
                same(g, wv, f"rows {nm}")
        b = mx.fp4_nv_quantize_rows(dev16(w))
        c = mx.fp4_nv_gemm(*a[:3], *b[:3])
        ref, e = N.gemm_ref(host(a[0]), host(a[1]), factors(host(a[2]), m), host(b[0]), host(b[1]),
                            factors(host(b[2]), n))
        assert G.within_bound(host(c), ref, e, k=k).all(), "rows x rows outside the bound"
        # the Dgrad route: W [k][n] in 2D16, its column view [n][k] with one factor
        wt = synthetic.tensor((k, n), std=0.02, seed=1200 + i)
        got = mx.fp4_nv_quantize_w2d16(strided(wt, rng))
        want = N.quantize_w2d16(wt)
        for g, wv, nm in zip(got[:4], want[:4], ("row codes", "row scales", "col codes", "col scales")):
            same(g, wv, f"2D16 {nm}")
        same_f32(got[4], [want[4]], "2D16 factor")
        c = mx.fp4_nv_gemm(*a[:3], got[2], got[3], got[4])
        ref, e = N.gemm_ref(host(a[0]), host(a[1]), factors(host(a[2]), m), host(got[2]), host(got[3]),
                            factors(host(got[4]), n))
        assert G.within_bound(host(c), ref, e, k=k).all(), "rows x 2D16 columns outside the bound"
