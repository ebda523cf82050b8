"""A whole FFN step (every hot-path call) captured in one HIP graph: each of
several replays, with eager work and synchronisations between them, gives the
same bytes as the eager step (the kernels are deterministic)."""

import numpy as np
import pytest
import torch

import synthetic
from oracle import philox as P

pytestmark = pytest.mark.gpu


def build_step(mx, t=256, d=512, f=384, seed=3):
    h = synthetic.workload("ffn_step_8192x4096x14336", seed=seed,
                           shapes={"X": (t, d), "W1": (f, d), "W3": (f, d), "W2": (d, f), "dY": (t, d)})
    dv = {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in h.items()}
    mask = P.sign_mask_from_seed(seed)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    o = {"xr": (u8(t, d // 2), u8(t, d // 32)), "w13": (u8(2 * f, d // 2), u8(2 * f, d // 32)),
         "w1c": (u8(d, f // 2), u8(d, f // 32)), "w3c": (u8(d, f // 2), u8(d, f // 32)),
         "w2": (u8(d, f // 2), u8(d, f // 32), u8(f, d // 2), u8(f, d // 32)),
         "a": torch.empty((t, f), dtype=torch.int16, device="cuda"), "b": torch.empty((t, f), dtype=torch.int16, device="cuda"),
         "hr": (u8(t, f // 2), u8(t, f // 32)), "hc": (u8(f, t // 2), u8(f, t // 32)),
         "y": torch.empty((t, d), dtype=torch.float32, device="cuda"),
         "dyr": (u8(t, d // 2), u8(t, d // 32)), "dyc": (u8(d, t // 2), u8(d, t // 32)),
         "dh": torch.empty((t, f), dtype=torch.float32, device="cuda"),
         "dw2": torch.empty((d, f), dtype=torch.float32, device="cuda"),
         "bwd": [u8(t, f // 2), u8(t, f // 32), u8(t, f // 2), u8(t, f // 32),
                 u8(f, t // 2), u8(f, t // 32), u8(f, t // 2), u8(f, t // 32)],
         "xc": (u8(d, t // 2), u8(d, t // 32)),
         "dx": torch.empty((t, d), dtype=torch.float32, device="cuda"),
         "dx2": torch.empty((t, d), dtype=torch.float32, device="cuda"),
         "dyd": [u8(t, d // 2), u8(t, d // 32), u8(d, t // 2), u8(d, t // 32)],
         "dw1": torch.empty((f, d), dtype=torch.float32, device="cuda"),
         "dw3": torch.empty((f, d), dtype=torch.float32, device="cuda"),
         # the CTA-local NVFP4 Dgrad: fill kernels (not memsets) clear its maxima
         "nvdy": [u8(t, d // 2), u8(t, d // 16), torch.empty(1, device="cuda"), torch.empty(1, device="cuda")],
         "nvw2": [u8(d, f // 2), u8(d, f // 16), u8(f, d // 2), u8(f, d // 16), torch.empty(1, device="cuda"),
                  torch.empty(1, device="cuda")],
         "nvdh": torch.empty((t, f), dtype=torch.float32, device="cuda"),
         # the backward contractions again, as one grouped launch
         "dhg": torch.empty((t, f), dtype=torch.float32, device="cuda"),
         "dw2g": torch.empty((d, f), dtype=torch.float32, device="cuda"),
         "dxg": torch.empty((t, d), dtype=torch.float32, device="cuda")}

    def run():
        mx.fp4_quantize_rows(dv["X"], codes=o["xr"][0], scales=o["xr"][1])
        mx.fp4_quantize_w2d32(dv["W1"], 0.87, o["w13"][0][:f], o["w13"][1][:f], *o["w1c"])
        mx.fp4_quantize_w2d32(dv["W3"], 0.87, o["w13"][0][f:], o["w13"][1][f:], *o["w3c"])
        mx.fp4_quantize_w2d32(dv["W2"], 0.87, *o["w2"])
        mx.fp4_swiglu_producer(o["xr"][0], o["xr"][1], o["w13"][0], o["w13"][1], mask, True, o["a"], o["b"],
                               o["hr"][0], o["hr"][1], o["hc"][0], o["hc"][1])
        mx.fp4_gemm(o["hr"][0], o["hr"][1], o["w2"][0], o["w2"][1], c=o["y"])
        mx.fp4_quantize_rows(dv["dY"], mx.FP4_SR, seed, 0, codes=o["dyr"][0], scales=o["dyr"][1])
        mx.fp4_quantize_cols(dv["dY"], 32, mask, codes_t=o["dyc"][0], scales_t=o["dyc"][1])
        mx.fp4_gemm(o["dyr"][0], o["dyr"][1], o["w2"][2], o["w2"][3], c=o["dh"])
        mx.fp4_gemm(o["dyc"][0], o["dyc"][1], o["hc"][0], o["hc"][1], c=o["dw2"])
        mx.fp4_swiglu_backward_producer(o["dh"], o["a"], o["b"], seed, 1, 2, mask, o["bwd"])
        mx.fp4_quantize_cols(dv["X"], 32, mask, codes_t=o["xc"][0], scales_t=o["xc"][1])
        mx.fp4_gemm(o["bwd"][0], o["bwd"][1], o["w1c"][0], o["w1c"][1], c=o["dx"])
        mx.fp4_gemm(o["bwd"][2], o["bwd"][3], o["w3c"][0], o["w3c"][1], c=o["dx"], accumulate=True)
        mx.fp4_gemm_pair(o["bwd"][0], o["bwd"][1], o["w1c"][0], o["w1c"][1], o["bwd"][2], o["bwd"][3], o["w3c"][0],
                         o["w3c"][1], c=o["dx2"])
        mx.fp4_quantize_dual(dv["dY"], mx.FP4_SR, seed, 0, 32, mask, *o["dyd"])
        mx.fp4_gemm(o["bwd"][4], o["bwd"][5], o["xc"][0], o["xc"][1], c=o["dw1"])
        mx.fp4_gemm(o["bwd"][6], o["bwd"][7], o["xc"][0], o["xc"][1], c=o["dw3"])
        mx.fp4_nv_quantize_rows(dv["dY"], mx.FP4_SR, seed, 0, out=o["nvdy"])
        mx.fp4_nv_quantize_w2d16(dv["W2"], out=o["nvw2"])
        mx.fp4_nv_gemm(o["nvdy"][0], o["nvdy"][1], o["nvdy"][2], o["nvw2"][2], o["nvw2"][3], o["nvw2"][4],
                       c=o["nvdh"])
        mx.fp4_gemm_grouped([
            dict(a_codes=o["dyc"][0], a_scales=o["dyc"][1], b_codes=o["hc"][0], b_scales=o["hc"][1], c=o["dw2g"]),
            dict(a_codes=o["dyr"][0], a_scales=o["dyr"][1], b_codes=o["w2"][2], b_scales=o["w2"][3], c=o["dhg"]),
            dict(a_codes=o["bwd"][0], a_scales=o["bwd"][1], b_codes=o["w1c"][0], b_scales=o["w1c"][1],
                 a2_codes=o["bwd"][2], a2_scales=o["bwd"][3], b2_codes=o["w3c"][0], b2_scales=o["w3c"][1],
                 c=o["dxg"])])

    def snapshot():
        torch.cuda.synchronize()
        flat = []
        for v in o.values():
            for x in (v if isinstance(v, (list, tuple)) else [v]):
                flat.append(x.clone())
        return flat

    return run, snapshot, o


@pytest.mark.parametrize("f", [384, 512])          # generic (K % 256 != 0) and fast kernels
def test_captured_step_replays_match_eager(gpu_lib, f):
    run, snapshot, o = build_step(gpu_lib, f=f)
    run()
    eager = snapshot()
    for grouped, alone in (("dhg", "dh"), ("dw2g", "dw2"), ("dxg", "dx2")):
        assert torch.equal(o[grouped], o[alone]), f"grouped {grouped} differs from its separate call"
    # poison every output, then capture
    for v in o.values():
        for x in (v if isinstance(v, (list, tuple)) else [v]):
            x.fill_(0x55 if x.dtype == torch.uint8 else 7)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for v in o.values():                               # eager work between replays
            for x in (v if isinstance(v, (list, tuple)) else [v]):
                x.fill_(0x33 if x.dtype == torch.uint8 else -1)
        junk.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for i, (g, e) in enumerate(zip(got, eager)):
            assert torch.equal(g, e), f"replay {rep}: output {i} differs from the eager step"
