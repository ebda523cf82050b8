"""The call sequence of one linear layer's Fprop, Dgrad and Wgrad, as the
README shows it: each product within the oracle's bound of its quantized
operands, and each the right contraction of the bf16 inputs (relative L2 error
of MXFP4 size against the fp32 product, where a transposed or mismatched
operand gives an error near 1.4)."""

import numpy as np
import pytest
import torch

from oracle import gemm as G

pytestmark = pytest.mark.gpu


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_linear_layer_usage(gpu_lib):
    mx = gpu_lib
    T, D, N = 512, 256, 384
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn(T, D, device="cuda", generator=g).bfloat16()
    w = (0.02 * torch.randn(N, D, device="cuda", generator=g)).bfloat16()
    dy = (1e-3 * torch.randn(T, N, device="cuda", generator=g)).bfloat16()
    mask = mx.fp4_sign_mask_from_seed(0)

    xr, xrs, xc, xcs = mx.fp4_quantize_dual(x, mx.FP4_RTN, 0, 0, 32, mask)
    wr, wrs, wc, wcs = mx.fp4_quantize_w2d32(w, 0.87)
    dyr, dyrs, dyc, dycs = mx.fp4_quantize_dual(dy, mx.FP4_SR, 1234, 0, 32, mask)

    y = mx.fp4_gemm(xr, xrs, wr, wrs)
    dx = mx.fp4_gemm(dyr, dyrs, wc, wcs)
    dw = mx.fp4_gemm(dyc, dycs, xc, xcs)
    for c, a, b in ((y, (xr, xrs), (wr, wrs)), (dx, (dyr, dyrs), (wc, wcs)), (dw, (dyc, dycs), (xc, xcs))):
        ref, e = G.gemm_ref(host(a[0]), host(a[1]), host(b[0]), host(b[1]))
        assert G.within_bound(host(c), ref, e).all()

    xf, wf, dyf = x.float(), w.float(), dy.float()
    for nm, got, want, shape in (("Y = X W^T", y, xf @ wf.T, (T, N)), ("dX = dY W", dx, dyf @ wf, (T, D)),
                                 ("dW = dY^T X", dw, dyf.T @ xf, (N, D))):
        assert tuple(got.shape) == shape, nm
        rel = float((got - want).norm() / want.norm())
        assert rel < 0.3, f"{nm}: relative L2 error {rel:.3f}"
