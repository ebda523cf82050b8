"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (same calls, same shapes, same buffers layout).

The oracle cannot redo 10^11-element GEMMs or 10^9-element quantizers in
seconds, so it checks sampled outputs that it computes one by one:
  * quantizers: whole sampled rows (row-facing, SR with the rows' global
    element indices), whole sampled columns over all tokens (column-facing,
    H32), whole 32-row tile strips (2D32, both layouts) -- bit-exact;
  * GEMMs: sampled rows x sampled columns of C against the exact reference on
    the same operand codes, |C - C_ref| <= 1e-5 * sum_k |a_k b_k|;
  * SwiGLU: a, b within the GEMM bound (before bf16 rounding) at sampled
    outputs; h codes and dA / dB bit-exact from the saved a, b and the W2
    Dgrad output on sampled rows and columns.
Where a value has several correct results (the fp32 order of a GEMM sum), the
next stage is checked from the GPU's value, itself checked above.
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

N_ROWS = 128         # sampled rows / columns per quantizer check
N_TILES = 6          # sampled 32-row strips per 2D32 check
N_GEMM_M, N_GEMM_N = 96, 1024


def pick(n, k, rng, step=1):
    """k sampled indices in [0, n) (multiples of `step`), always with the first
    and the last."""
    groups = n // step
    idx = rng.choice(groups, size=min(k, groups), replace=False)
    idx = np.unique(np.concatenate([idx, [0, groups - 1]])) * step
    return idx.astype(np.int64)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host16(t):
    return host(t).view(np.uint16)


def rows_of(t, idx):
    return t[torch.from_numpy(idx).cuda()]


def cols_of(t, idx):
    return t[:, torch.from_numpy(idx).cuda()]


def same(got, want, what):
    got = host(got) if isinstance(got, torch.Tensor) else got
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:4].tolist()}")


def check_rows(q, x_rows, ridx, what, mode=Q.RTN, seed=0, offset=0):
    want = Q.quantize_rows(x_rows, mode, seed, offset, row_ids=ridx)
    same(rows_of(q[0], ridx), want[0], what + " codes")
    same(rows_of(q[1], ridx), want[1], what + " scales")


def check_cols(q, x_cols, cidx, mask, what):
    want = Q.quantize_cols(x_cols, 32, mask)
    same(rows_of(q[0], cidx), want[0], what + " codes")
    same(rows_of(q[1], cidx), want[1], what + " scales")


def check_w2d32(q, w_host, rng, what, ratio=0.87):
    for r0 in pick(w_host.shape[0], N_TILES, rng, 32):
        g = r0 // 32
        rc, rs, cc, cs = Q.quantize_w2d32(w_host[r0:r0 + 32], ratio)
        same(q[0][r0:r0 + 32], rc, what + " row codes")
        same(q[1][r0:r0 + 32], rs, what + " row scales")
        same(q[2][:, 16 * g:16 * g + 16], cc, what + " col codes")
        same(q[3][:, g:g + 1], cs, what + " col scales")


def check_gemm(c, a, b, rng, what, c_prev=None):
    ms = pick(a[0].shape[0], N_GEMM_M, rng)
    ns = pick(b[0].shape[0], N_GEMM_N, rng)
    ref, e = G.gemm_ref(host(rows_of(a[0], ms)), host(rows_of(a[1], ms)),
                        host(rows_of(b[0], ns)), host(rows_of(b[1], ns)))
    got = host(cols_of(rows_of(c, ms), ns))
    prev = None if c_prev is None else c_prev(ms, ns)
    ok = G.within_bound(got, ref, e, c_prev=prev)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} sampled elements outside the bound; "
                             f"first ({ms[i[0]]}, {ns[i[1]]}): got {got[i]} ref {ref[i]} E {e[i]}")


def check_gemm_pair(c, a1, b1, a2, b2, rng, what):
    ms = pick(a1[0].shape[0], N_GEMM_M, rng)
    ns = pick(b1[0].shape[0], N_GEMM_N, rng)
    r1, e1 = G.gemm_ref(host(rows_of(a1[0], ms)), host(rows_of(a1[1], ms)),
                        host(rows_of(b1[0], ns)), host(rows_of(b1[1], ns)))
    r2, e2 = G.gemm_ref(host(rows_of(a2[0], ms)), host(rows_of(a2[1], ms)),
                        host(rows_of(b2[0], ns)), host(rows_of(b2[1], ns)))
    got = host(cols_of(rows_of(c, ms), ns))
    ok = G.within_bound(got, r1 + r2, e1 + e2)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} sampled elements outside the bound; "
                             f"first ({ms[i[0]]}, {ns[i[1]]}): got {got[i]} ref {(r1 + r2)[i]}")


def test_fprop_256x512x512_full(gpu_lib):
    """Single Fprop linear, 1x32 blocks for both operands: the whole output."""
    h = synthetic.workload("fprop_256x512x512")
    xr = gpu_lib.fp4_quantize_rows(dev(h["X"]))
    wr = gpu_lib.fp4_quantize_rows(dev(h["W"]))
    for q, x, nm in ((xr, h["X"], "X"), (wr, h["W"], "W")):
        want = Q.quantize_rows(x)
        same(q[0], want[0], nm + " codes")
        same(q[1], want[1], nm + " scales")
    c = gpu_lib.fp4_gemm(xr[0], xr[1], wr[0], wr[1])
    ref, e = G.gemm_ref(*(host(t) for t in (xr[0], xr[1], wr[0], wr[1])))
    assert G.within_bound(host(c), ref, e).all()


def test_attn_proj_8192x4096x4096(gpu_lib):
    """Attention-projection Fprop + Dgrad: outlier X, 2D32 W, SR dY."""
    name = "attn_proj_8192x4096x4096"
    h = synthetic.workload(name)
    seed = synthetic.WORKLOADS[name]["seed"]
    rng = np.random.default_rng(101)
    X, W, dY = dev(h["X"]), dev(h["W"]), dev(h["dY"])
    xr = gpu_lib.fp4_quantize_rows(X)
    wq = gpu_lib.fp4_quantize_w2d32(W, 0.87)
    dyr = gpu_lib.fp4_quantize_rows(dY, gpu_lib.FP4_SR, seed, 0)
    y = gpu_lib.fp4_gemm(xr[0], xr[1], wq[0], wq[1])
    dx = gpu_lib.fp4_gemm(dyr[0], dyr[1], wq[2], wq[3])
    r = pick(8192, N_ROWS, rng)
    check_rows(xr, h["X"][r], r, "rows(X)")
    check_rows(dyr, h["dY"][r], r, "rows(dY,SR)", Q.SR, seed, 0)
    check_w2d32(wq, h["W"], rng, "w2d32(W)")
    check_gemm(y, xr, wq[:2], rng, "Fprop")
    check_gemm(dx, dyr, wq[2:], rng, "Dgrad")


def test_wgrad_h32_8192x14336x4096(gpu_lib):
    """Wgrad with the paired fixed-sign H32 along the 8192-token axis."""
    name = "wgrad_h32_8192x14336x4096"
    h = synthetic.workload(name)
    mask = P.sign_mask_from_seed(synthetic.WORKLOADS[name]["seed"])
    assert gpu_lib.fp4_sign_mask_from_seed(synthetic.WORKLOADS[name]["seed"]) == mask
    rng = np.random.default_rng(102)
    dyc = gpu_lib.fp4_quantize_cols(dev(h["dY"]), 32, mask)
    xc = gpu_lib.fp4_quantize_cols(dev(h["X"]), 32, mask)
    dw = gpu_lib.fp4_gemm(dyc[0], dyc[1], xc[0], xc[1])
    for x, q, nm in ((h["dY"], dyc, "cols(dY,H32)"), (h["X"], xc, "cols(X,H32)")):
        c = pick(x.shape[1], N_ROWS, rng)
        check_cols(q, np.ascontiguousarray(x[:, c]), c, mask, nm)
    check_gemm(dw, dyc, xc, rng, "Wgrad")


def test_gemm_streamed_c_ragged(gpu_lib):
    """A C larger than 192 MB is written with non-temporal stores; here with M
    and N that are not multiples of the 256 x 256 tile, plain and accumulating."""
    m, n, k = 7200, 7232, 512
    assert m * n * 4 > (192 << 20)
    rng = np.random.default_rng(104)
    x = synthetic.tensor((m, k), std=1.0, seed=61, outlier_rate=0.001, outlier_scale=20.0)
    w = synthetic.tensor((n, k), std=0.02, seed=62)
    a = gpu_lib.fp4_quantize_rows(dev(x))
    b = gpu_lib.fp4_quantize_rows(dev(w))
    c = gpu_lib.fp4_gemm(a[0], a[1], b[0], b[1])
    check_gemm(c, a, b, rng, "streamed C")
    c_first = c.clone()
    gpu_lib.fp4_gemm(a[0], a[1], b[0], b[1], c=c, accumulate=True)
    check_gemm(c, a, b, rng, "streamed C (+=)",
               c_prev=lambda ms_, ns_: host(cols_of(rows_of(c_first, ms_), ns_)))
    a2 = gpu_lib.fp4_quantize_rows(dev(synthetic.tensor((m, k), std=1e-3, seed=63)))
    cp = gpu_lib.fp4_gemm_pair(a[0], a[1], b[0], b[1], a2[0], a2[1], b[0], b[1])
    check_gemm_pair(cp, a, b, a2, b, rng, "streamed C, paired")


@pytest.mark.parametrize("name", ["ffn_step_8192x4096x14336", "ffn_large_32768x8192x28672"])
def test_ffn_step(gpu_lib, name):
    """The whole SwiGLU FFN step, forward and backward, as the benchmark runs it."""
    h = synthetic.workload(name)
    seed = synthetic.WORKLOADS[name]["seed"]
    mask = P.sign_mask_from_seed(seed)
    rng = np.random.default_rng(103)
    X, W1, W3, W2, dY = (dev(h[k]) for k in ("X", "W1", "W3", "W2", "dY"))
    T, D = X.shape
    Fw = W1.shape[0]
    u8 = dict(dtype=torch.uint8, device="cuda")

    # forward
    xr = gpu_lib.fp4_quantize_rows(X)
    w13_rc, w13_rs = torch.empty((2 * Fw, D // 2), **u8), torch.empty((2 * Fw, D // 32), **u8)
    w1 = gpu_lib.fp4_quantize_w2d32(W1, 0.87, w13_rc[:Fw], w13_rs[:Fw])
    w3 = gpu_lib.fp4_quantize_w2d32(W3, 0.87, w13_rc[Fw:], w13_rs[Fw:])
    w2 = gpu_lib.fp4_quantize_w2d32(W2, 0.87)
    a, b, hrc, hrs, hcc, hcs = gpu_lib.fp4_swiglu_producer(xr[0], xr[1], w13_rc, w13_rs, mask, True)
    y = gpu_lib.fp4_gemm(hrc, hrs, w2[0], w2[1])
    # backward
    dyr = gpu_lib.fp4_quantize_rows(dY, gpu_lib.FP4_SR, seed, 0)
    dyc = gpu_lib.fp4_quantize_cols(dY, 32, mask)
    dh = gpu_lib.fp4_gemm(dyr[0], dyr[1], w2[2], w2[3])
    dw2 = gpu_lib.fp4_gemm(dyc[0], dyc[1], hcc, hcs)
    da, db = gpu_lib.fp4_swiglu_backward(dh, a, b)
    dar = gpu_lib.fp4_quantize_rows(da, gpu_lib.FP4_SR, seed, 1)
    dbr = gpu_lib.fp4_quantize_rows(db, gpu_lib.FP4_SR, seed, 2)
    dac = gpu_lib.fp4_quantize_cols(da, 32, mask)
    dbc = gpu_lib.fp4_quantize_cols(db, 32, mask)
    xc = gpu_lib.fp4_quantize_cols(X, 32, mask)
    dx = gpu_lib.fp4_gemm(dar[0], dar[1], w1[2], w1[3])
    dx_first = dx.clone()
    gpu_lib.fp4_gemm(dbr[0], dbr[1], w3[2], w3[3], c=dx, accumulate=True)
    dx_pair = gpu_lib.fp4_gemm_pair(dar[0], dar[1], w1[2], w1[3], dbr[0], dbr[1], w3[2], w3[3])
    dw1 = gpu_lib.fp4_gemm(dac[0], dac[1], xc[0], xc[1])
    dw3 = gpu_lib.fp4_gemm(dbc[0], dbc[1], xc[0], xc[1])
    torch.cuda.synchronize()

    # producers of the inputs
    r = pick(T, N_ROWS, rng)
    check_rows(xr, h["X"][r], r, "rows(X)")
    check_rows(dyr, h["dY"][r], r, "rows(dY,SR)", Q.SR, seed, 0)
    for w, q, nm in ((h["W1"], w1, "W1"), (h["W3"], w3, "W3"), (h["W2"], w2, "W2")):
        check_w2d32(q, w, rng, "w2d32(" + nm + ")")
    c = pick(D, N_ROWS, rng)
    check_cols(dyc, np.ascontiguousarray(h["dY"][:, c]), c, mask, "cols(dY,H32)")
    check_cols(xc, np.ascontiguousarray(h["X"][:, c]), c, mask, "cols(X,H32)")

    # SwiGLU producer: a, b within the GEMM bound at sampled outputs
    ms, ns = pick(T, N_GEMM_M, rng), pick(Fw, N_GEMM_N, rng)
    ref, e = G.gemm_ref(host(rows_of(xr[0], ms)), host(rows_of(xr[1], ms)),
                        host(rows_of(w13_rc, np.concatenate([ns, Fw + ns]))),
                        host(rows_of(w13_rs, np.concatenate([ns, Fw + ns]))))
    tol = G.GEMM_REL_TOL * e
    lo = F.bf16_bits_to_f64(S.f32_to_bf16_rne((ref - tol).astype(np.float32)))
    hi = F.bf16_bits_to_f64(S.f32_to_bf16_rne((ref + tol).astype(np.float32)))
    ab = np.concatenate([host16(cols_of(rows_of(a, ms), ns)), host16(cols_of(rows_of(b, ms), ns))], axis=1)
    g = F.bf16_bits_to_f64(ab)
    assert np.all((g >= lo) & (g <= hi)), "swiglu a/b outside the GEMM bound"
    # h codes from the saved a, b: whole sampled rows and whole sampled columns
    hrow = S.swiglu_h(host16(rows_of(a, r)), host16(rows_of(b, r)))
    check_rows((hrc, hrs), hrow, r, "h rows")
    fc = pick(Fw, N_ROWS, rng)
    hcol = S.swiglu_h(host16(cols_of(a, fc)), host16(cols_of(b, fc)))
    check_cols((hcc, hcs), np.ascontiguousarray(hcol), fc, mask, "h cols(H32)")

    # SwiGLU backward and the gradient producers fed by it
    want_da, want_db = S.swiglu_backward(host(rows_of(dh, r)), host16(rows_of(a, r)), host16(rows_of(b, r)))
    same(host16(rows_of(da, r)), want_da, "dA rows")
    same(host16(rows_of(db, r)), want_db, "dB rows")
    check_rows(dar, host16(rows_of(da, r)), r, "rows(dA,SR)", Q.SR, seed, 1)
    check_rows(dbr, host16(rows_of(db, r)), r, "rows(dB,SR)", Q.SR, seed, 2)
    check_cols(dac, np.ascontiguousarray(host16(cols_of(da, fc))), fc, mask, "cols(dA,H32)")
    check_cols(dbc, np.ascontiguousarray(host16(cols_of(db, fc))), fc, mask, "cols(dB,H32)")

    # single-read dY producer: the same bytes as the two separate calls, everywhere
    dual = gpu_lib.fp4_quantize_dual(dY, gpu_lib.FP4_SR, seed, 0, 32, mask)
    for got, want, nm in zip(dual, dyr + dyc, ("dY row codes", "dY row scales", "dY col codes", "dY col scales")):
        assert torch.equal(got, want), "dual " + nm
    del dual

    # fused backward producer: the same bytes as the unfused calls, everywhere
    fused = gpu_lib.fp4_swiglu_backward_producer(dh, a, b, seed, 1, 2, mask)
    for got, want, nm in zip(fused, (dar, dbr, dac, dbc), ("dA rows", "dB rows", "dA cols", "dB cols")):
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), "fused " + nm
    del fused
    # W2 Dgrad with the backward producer in its epilogue: the same bytes again
    fused = gpu_lib.fp4_gemm_swiglu_backward_producer(dyr[0], dyr[1], w2[2], w2[3], a, b, seed, 1, 2, mask)
    for got, want, nm in zip(fused, (dar, dbr, dac, dbc), ("dA rows", "dB rows", "dA cols", "dB cols")):
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), "Dgrad epilogue " + nm
    del fused

    # the seven contractions
    check_gemm(y, (hrc, hrs), w2[:2], rng, "W2 Fprop")
    check_gemm(dh, dyr, w2[2:], rng, "W2 Dgrad")
    check_gemm(dw2, dyc, (hcc, hcs), rng, "W2 Wgrad")
    check_gemm(dx_first, dar, w1[2:], rng, "W1 Dgrad")
    check_gemm(dx, dbr, w3[2:], rng, "W3 Dgrad (+=)",
               c_prev=lambda ms_, ns_: host(cols_of(rows_of(dx_first, ms_), ns_)))
    check_gemm_pair(dx_pair, dar, w1[2:], dbr, w3[2:], rng, "W1+W3 Dgrad (one accumulation)")
    check_gemm(dw1, dac, xc, rng, "W1 Wgrad")
    check_gemm(dw3, dbc, xc, rng, "W3 Wgrad")
    # the two Wgrads stacked into one contraction (M = 2F) give the same bytes
    stacked = gpu_lib.fp4_gemm(torch.cat([dac[0], dbc[0]]), torch.cat([dac[1], dbc[1]]), xc[0], xc[1])
    assert torch.equal(stacked[:Fw], dw1) and torch.equal(stacked[Fw:], dw3), "stacked Wgrad"
