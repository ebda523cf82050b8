"""Tensors of more than 2^34 elements: the SR producers' counters then need
their second word (the element index shifted by two passes 2^32), so these
calls run the kernels' 64-bit counter forms, which smaller tensors never
reach.  131136 x 131072 values (2^34 + 2^23); sampled rows on both sides of
index 2^34 and the last token blocks are checked against the oracle bit for
bit.  Each test needs 40-170 GB of device memory and skips where that is not
free."""

import numpy as np
import pytest
import torch

from oracle import nvfp4 as N
from oracle import philox as P
from oracle import quant as Q
from oracle import swiglu as S

pytestmark = pytest.mark.gpu

R, C = 131072 + 64, 131072                      # R * C = 2^34 + 2^23
ROWS = [0, 1, 65536, 131071, 131072, 131100, 131135]     # row 131072 starts at index 2^34
GIB = 1 << 30


@pytest.fixture(autouse=True)
def release_memory():
    """Hand the cached blocks back after each test, so that the next one's
    free-memory check sees them."""
    yield
    torch.cuda.empty_cache()


def need(gib):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < gib * GIB:
        pytest.skip(f"needs {gib} GiB of free device memory, {free / GIB:.0f} free")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def fill_bf16(rows, cols, seed, lo=0x3000, hi=0x4000):
    """Finite bf16 patterns (magnitudes 2^-31 .. 2, random sign), generated
    on the device in slabs."""
    x = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(seed)
    for r0 in range(0, rows, 8192):
        r1 = min(rows, r0 + 8192)
        mag = torch.randint(lo, hi, (r1 - r0, cols), dtype=torch.int16, device="cuda", generator=g)
        sgn = torch.randint(0, 2, (r1 - r0, cols), dtype=torch.int16, device="cuda", generator=g)
        x[r0:r1] = mag | (sgn << 15)
        del mag, sgn
    return x


def rows_of(t, rows):
    return np.stack([host(t[r]) for r in rows])


def test_huge_rows_and_dual_sr(gpu_lib):
    mx = gpu_lib
    need(60)
    seed, off, mask = 2 ** 40 + 5, 7, P.sign_mask_from_seed(3)
    x = fill_bf16(R, C, 1)
    print(f"[huge] rows SR {R}x{C}", flush=True)
    codes, scales = mx.fp4_quantize_rows(x, mx.FP4_SR, seed, off)
    xs = rows_of(x, ROWS).view(np.uint16)
    want = Q.quantize_rows(xs, Q.SR, seed, off, row_ids=ROWS)
    assert np.array_equal(rows_of(codes, ROWS), want[0]), "rows SR codes"
    assert np.array_equal(rows_of(scales, ROWS), want[1]), "rows SR scales"
    del codes, scales
    torch.cuda.empty_cache()
    print(f"[huge] dual SR + H32 {R}x{C}", flush=True)
    rc, rs, cc, cs = mx.fp4_quantize_dual(x, mx.FP4_SR, seed, off, 32, mask)
    assert np.array_equal(rows_of(rc, ROWS), want[0]), "dual row codes"
    assert np.array_equal(rows_of(rs, ROWS), want[1]), "dual row scales"
    tb = R // 32 - 1                                                 # the last token block
    blk = host(x[32 * tb:32 * tb + 32]).view(np.uint16)
    wc = Q.quantize_cols(blk, 32, mask)
    assert np.array_equal(host(cc[:, 16 * tb:16 * tb + 16]), wc[0]), "dual column codes"
    assert np.array_equal(host(cs[:, tb:tb + 1]), wc[1]), "dual column scales"
    del rc, rs, cc, cs
    torch.cuda.empty_cache()
    print(f"[huge] dual SR, plain columns {R}x{C}", flush=True)
    rc, rs, cc, cs = mx.fp4_quantize_dual(x, mx.FP4_SR, seed, off, 0, 0)
    assert np.array_equal(rows_of(rc, ROWS), want[0]), "dual (no H32) row codes"
    wc = Q.quantize_cols(blk, 0, 0)
    assert np.array_equal(host(cc[:, 16 * tb:16 * tb + 16]), wc[0]), "dual (no H32) column codes"
    assert np.array_equal(host(cs[:, tb:tb + 1]), wc[1]), "dual (no H32) column scales"


def test_huge_nv_rows_sr(gpu_lib):
    mx = gpu_lib
    need(50)
    seed, off = 9, 2 ** 33 + 1
    x = fill_bf16(R, C, 2)
    print(f"[huge] CTA-local NVFP4 rows SR {R}x{C}", flush=True)
    codes, scales, factors, amax = mx.fp4_nv_quantize_rows(x, mx.FP4_SR, seed, off)
    r0 = (R // N.PANEL) * N.PANEL                                    # the last, partial panel
    xs = host(x[r0:]).view(np.uint16)
    wc, ws, wf, wa = N.quantize_rows(xs, N.SR, seed, off, row0=r0)
    p = r0 // N.PANEL
    assert np.array_equal(host(codes[r0:]), wc), "codes"
    assert np.array_equal(host(scales[r0:]), ws), "scales"
    assert host(factors[p:p + 1]).view(np.uint32)[0] == np.float32(wf[0]).view(np.uint32), "factor"
    assert host(amax[p:p + 1]).view(np.uint32)[0] == np.float32(wa[0]).view(np.uint32), "panel maximum"


def test_huge_swiglu_backward_producer(gpu_lib):
    mx = gpu_lib
    need(175)
    seed, oa, ob, mask = 2 ** 36 + 1, 3, 2 ** 34 + 5, P.sign_mask_from_seed(4)
    a = fill_bf16(R, C, 3, 0x3C00, 0x4100)
    b = fill_bf16(R, C, 4, 0x3C00, 0x4100)
    dh = torch.empty((R, C), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    for r0 in range(0, R, 8192):
        dh[r0:r0 + 8192].normal_(0.0, 1e-3, generator=g)
    print(f"[huge] backward producer {R}x{C}", flush=True)
    (dar, dbr, dac, dbc) = mx.fp4_swiglu_backward_producer(dh, a, b, seed, oa, ob, mask)
    sa, sb = rows_of(a, ROWS).view(np.uint16), rows_of(b, ROWS).view(np.uint16)
    da, db = S.swiglu_backward(rows_of(dh, ROWS), sa, sb)
    for got, d, off, nm in ((dar, da, oa, "dA"), (dbr, db, ob, "dB")):
        want = Q.quantize_rows(d, Q.SR, seed, off, row_ids=ROWS)
        assert np.array_equal(rows_of(got[0], ROWS), want[0]), nm + " row codes"
        assert np.array_equal(rows_of(got[1], ROWS), want[1]), nm + " row scales"
    tb = R // 32 - 1
    sl = slice(32 * tb, 32 * tb + 32)
    da, db = S.swiglu_backward(host(dh[sl]), host(a[sl]).view(np.uint16), host(b[sl]).view(np.uint16))
    for got, d, nm in ((dac, da, "dA"), (dbc, db, "dB")):
        want = Q.quantize_cols(d, 32, mask)
        assert np.array_equal(host(got[0][:, 16 * tb:16 * tb + 16]), want[0]), nm + " column codes"
        assert np.array_equal(host(got[1][:, tb:tb + 1]), want[1]), nm + " column scales"
