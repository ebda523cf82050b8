"""fp4_gemm_grouped: independent products in one launch give the bytes of the
same products run as separate fp4_gemm / fp4_gemm_pair calls, and each lies
within the oracle's bound of the exact sum (§2.3 Eq. 4-6 of "Format-Aware
Fusion for Fast FP4 Pretraining")."""

import numpy as np
import pytest
import torch

import synthetic
from oracle import gemm as G

pytestmark = pytest.mark.gpu


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantized(mx, rows, k, std, seed):
    return mx.fp4_quantize_rows(dev16(synthetic.tensor((rows, k), std=std, seed=seed, outlier_rate=0.001,
                                                       outlier_scale=20.0)))


def filled(shape, word, ld=None):
    """fp32 output pre-set to one bit pattern (a sentinel no result equals)."""
    t = torch.empty((shape[0], ld or shape[1]), dtype=torch.float32, device="cuda")
    t.view(torch.int32).fill_(word)
    return t[:, :shape[1]]


def same_bytes(x, y):
    torch.cuda.synchronize()
    return torch.equal(x.contiguous().view(torch.int32), y.contiguous().view(torch.int32))


def within_oracle(c, pairs, c_prev=None):
    ref = e = 0
    for a, b in pairs:
        r, ee = G.gemm_ref(host(a[0]), host(a[1]), host(b[0]), host(b[1]))
        ref, e = ref + r, e + ee
    return G.within_bound(host(c), ref, e, c_prev=c_prev).all()


def run_both(mx, probs):
    """The group in one call (outputs pre-set to one sentinel) and each problem
    on its own (outputs pre-set to another): returns both lists of C."""
    grouped, separate = [], []
    for pr in probs:
        m, n = pr["a_codes"].shape[0], pr["b_codes"].shape[0]
        ld = pr.get("ldc")
        cg, cs = filled((m, n), 0x7FBFFFFF, ld), filled((m, n), -1, ld)
        if "prev" in pr:
            cg.copy_(pr["prev"])
            cs.copy_(pr["prev"])
        grouped.append(cg)
        separate.append(cs)
    mx.fp4_gemm_grouped([dict({k: v for k, v in pr.items() if k not in ("prev", "ldc")}, c=cg)
                         for pr, cg in zip(probs, grouped)])
    for pr, cs in zip(probs, separate):
        acc = pr.get("accumulate", False)
        if "a2_codes" in pr:
            mx.fp4_gemm_pair(pr["a_codes"], pr["a_scales"], pr["b_codes"], pr["b_scales"], pr["a2_codes"],
                             pr["a2_scales"], pr["b2_codes"], pr["b2_scales"], c=cs, accumulate=acc)
        else:
            mx.fp4_gemm(pr["a_codes"], pr["a_scales"], pr["b_codes"], pr["b_scales"], c=cs, accumulate=acc)
    return grouped, separate


def prob(a, b, a2=None, b2=None, **kw):
    d = dict(a_codes=a[0], a_scales=a[1], b_codes=b[0], b_scales=b[1], **kw)
    if a2 is not None:
        d.update(a2_codes=a2[0], a2_scales=a2[1], b2_codes=b2[0], b2_scales=b2[1])
    return d


def test_grouped_plain_pair_accumulate_strided(gpu_lib):
    """Four problems of different K in one launch: ragged plain, pair form,
    accumulating into a prefilled C, and C as a column slice of a wider tensor."""
    mx = gpu_lib
    a0, b0 = quantized(mx, 544, 512, 1.0, 1), quantized(mx, 800, 512, 0.02, 2)
    a1, b1 = quantized(mx, 288, 768, 1.0, 3), quantized(mx, 352, 768, 0.02, 4)
    a1b, b1b = quantized(mx, 288, 768, 1e-3, 5), quantized(mx, 352, 768, 0.02, 6)
    a2, b2 = quantized(mx, 1024, 256, 1.0, 7), quantized(mx, 256, 256, 0.02, 8)
    a3, b3 = quantized(mx, 256, 1024, 1.0, 9), quantized(mx, 288, 1024, 0.02, 10)
    prev_bits = synthetic.tensor((1024, 256), std=1.0, seed=11).astype(np.uint32) << 16
    prev = torch.from_numpy(prev_bits.view(np.float32)).cuda()
    probs = [prob(a0, b0), prob(a1, b1, a1b, b1b), prob(a2, b2, accumulate=True, prev=prev),
             prob(a3, b3, ldc=352)]
    grouped, separate = run_both(mx, probs)
    for q, (cg, cs) in enumerate(zip(grouped, separate)):
        assert same_bytes(cg, cs), f"problem {q}"
    assert within_oracle(grouped[0], [(a0, b0)])
    assert within_oracle(grouped[1], [(a1, b1), (a1b, b1b)])
    assert within_oracle(grouped[2], [(a2, b2)], c_prev=host(prev))
    assert within_oracle(grouped[3], [(a3, b3)])


def test_grouped_fills_a_part_empty_round(gpu_lib):
    """A long-K problem with 384 tiles (one and a half rounds on 256 CUs)
    followed by a short-K problem with 512 tiles, as the W2 Wgrad and W2 Dgrad
    of the FFN backward: the grouped launch gives the separate calls' bytes."""
    mx = gpu_lib
    aw, bw = quantized(mx, 4096, 2048, 1.0, 21), quantized(mx, 6144, 2048, 0.5, 22)     # 16 x 24 tiles
    ad, bd = quantized(mx, 4096, 512, 1.0, 23), quantized(mx, 8192, 512, 0.02, 24)      # 16 x 32 tiles
    grouped, separate = run_both(mx, [prob(ad, bd), prob(aw, bw)])
    assert same_bytes(grouped[0], separate[0]) and same_bytes(grouped[1], separate[1])
    rows = np.array([0, 1, 255, 256, 2047, 4095])
    cw = host(grouped[1])[rows]
    ref, e = G.gemm_ref(host(aw[0])[rows], host(aw[1])[rows], host(bw[0]), host(bw[1]))
    assert G.within_bound(cw, ref, e).all()


def test_grouped_with_generic_and_empty_problems(gpu_lib):
    """K % 256 != 0 (plain and pair form, the pair accumulating) and K = 0
    problems run as calls of their own beside the shared launch; an empty C
    is a no-op."""
    mx = gpu_lib
    a0, b0 = quantized(mx, 256, 256, 1.0, 31), quantized(mx, 512, 256, 0.02, 32)
    a1, b1 = quantized(mx, 96, 288, 1.0, 33), quantized(mx, 160, 288, 0.02, 34)
    z = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    zs = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    zb = torch.zeros((96, 0), dtype=torch.uint8, device="cuda")
    e = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    es = torch.zeros((0, 8), dtype=torch.uint8, device="cuda")
    a2, b2 = quantized(mx, 96, 288, 1e-3, 36), quantized(mx, 160, 288, 0.02, 37)
    probs = [prob(a1, b1), prob((z, zs), (zb, zb)), prob(a0, b0), prob(a1, b1, a2, b2, accumulate=True,
                                                                       prev=torch.ones((96, 160), device="cuda"))]
    grouped, separate = run_both(mx, probs)
    for q, (cg, cs) in enumerate(zip(grouped, separate)):
        assert same_bytes(cg, cs), f"problem {q}"
    assert not host(grouped[1]).any()                      # empty sums
    assert within_oracle(grouped[0], [(a1, b1)])
    assert within_oracle(grouped[3], [(a1, b1), (a2, b2)], c_prev=np.ones((96, 160), dtype=np.float32))
    bd = quantized(mx, 64, 256, 1.0, 35)
    out = mx.fp4_gemm_grouped([prob((e, es), bd), prob(a0, b0)])
    assert out[0].shape == (0, 64) and within_oracle(out[1], [(a0, b0)])


def test_grouped_binding_refusals(gpu_lib):
    mx = gpu_lib
    a, b = quantized(mx, 64, 256, 1.0, 41), quantized(mx, 64, 256, 1.0, 42)
    with pytest.raises(mx.Fp4Error):
        mx.fp4_gemm_grouped([prob(a, b)] * 5)
    with pytest.raises(mx.Fp4Error):
        mx.fp4_gemm_grouped([prob(a, (b[0][:, :64].contiguous(), b[1]))])
    with pytest.raises(mx.Fp4Error):
        mx.fp4_gemm_grouped([prob(a, b, accumulate=True)])


def test_grouped_ffn_backward_w2_full_size(gpu_lib):
    """The FFN backward's W2 Dgrad (8192 x 14336 x 4096, 1792 tiles) and W2
    Wgrad (4096 x 14336 x 8192, 896 tiles) at full size in one launch, on
    random codes and scales: byte-equal to the two separate calls, every
    element written (distinct sentinels), sampled rows within the oracle's
    bound."""
    mx = gpu_lib
    g = torch.Generator(device="cuda").manual_seed(7)

    def rnd(rows, k):
        codes = torch.randint(0, 256, (rows, k // 2), dtype=torch.uint8, device="cuda", generator=g)
        scales = torch.randint(118, 130, (rows, k // 32), dtype=torch.uint8, device="cuda", generator=g)
        return codes, scales

    dy, w2c = rnd(8192, 4096), rnd(14336, 4096)
    dyc, hc = rnd(4096, 8192), rnd(14336, 8192)
    grouped, separate = run_both(mx, [prob(dy, w2c), prob(dyc, hc)])
    assert same_bytes(grouped[0], separate[0]) and same_bytes(grouped[1], separate[1])
    for (a, b), c in (((dy, w2c), grouped[0]), ((dyc, hc), grouped[1])):
        rows = np.array([0, 255, 256, 4095])
        ref, e = G.gemm_ref(host(a[0])[rows], host(a[1])[rows], host(b[0]), host(b[1]))
        assert G.within_bound(host(c)[rows], ref, e).all()
