"""Benchmark of the MXFP4 producer + block-scaled E2M1 GEMM hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--eager] [--unfused-backward] [--quality] [--copy-calibration]
                    [--quantizer-sweep] [--nvfp4-dgrad]

A step is one pass of the whole hot path over one batch of synthetic input.
The default workload is the full Llama-3-8B SwiGLU FFN step (T 8192, D 4096,
F 14336), in launch order: forward (row-RTN and column-H32 X from one read,
2D32 W1/W3, fused SwiGLU producer emitting h row- and column-facing, 2D32 W2,
W2 Fprop) and backward (row-SR and column-H32 dY from one read, W2 Dgrad and
Wgrad, the fused SwiGLU backward producer emitting dA/dB row-SR and column-H32,
W1/W3 Wgrad stacked into one launch, W1/W3 Dgrad as one accumulation over
K = 2F): nine contractions, 8.66 TFLOP, timed as one captured HIP graph
(per-call times come from eager steps with events around every call).

Prints one JSON line.  `value` = GEMM FLOPs of the step / step time (the
"quantize+GEMM TFLOP/s": producer time is inside the step).  Timing uses HIP
events on the stream the kernels run on; inputs are resident in HBM before the
timed region.  The roofline object covers the dominant kernel (the GEMM);
cpu_baseline times the CPU oracle on a bounded sample of the same step.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MXFP4_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA, published
PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E, published
METRIC = "MXFP4 quantize+GEMM TFLOP/s (Fprop/Dgrad/Wgrad) and quantizer GB/s, % of peak"

# Algorithmic bytes per element (what the producer must move):
B_SINGLE = 2 + 0.5 + 1 / 32          # bf16 in, one orientation of codes + scales
B_2D32 = 2 + 2 * (0.5 + 1 / 32)      # bf16 in, two layouts
B_DUAL = 2 + 2 * (0.5 + 1 / 32)      # bf16 in once, row and column codes + scales
B_SWIGLU_BWD = 4 + 2 + 2 + 2 + 2     # dH fp32, a, b in; dA, dB out
B_BWD_PRODUCER = 4 + 2 + 2 + 4 * (0.5 + 1 / 32)   # dH, a, b in; dA, dB as row SR + column H32 MXFP4


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="ffn_step_8192x4096x14336")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--unfused-backward", action="store_true",
                   help="FFN step: separate producer calls (SR rows and H32 cols of dY as two calls; SwiGLU backward, "
                        "SR rows and H32 cols of dA/dB as five)")
    p.add_argument("--dgrad-epilogue", action="store_true",
                   help="FFN step: W2 Dgrad with the SwiGLU backward producer in its epilogue (one launch; dH never "
                        "in memory) instead of W2 Dgrad followed by the backward producer")
    p.add_argument("--separate-gemms", action="store_true",
                   help="FFN step: W2 Dgrad and W2 Wgrad as two launches instead of one fp4_gemm_grouped")
    p.add_argument("--eager", action="store_true",
                   help="time the step as eager launches instead of one captured HIP graph")
    p.add_argument("--quality", action="store_true",
                   help="numerical quality of the MXFP4 contractions against fp32 on the bf16 inputs, with ablations")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of known size (for scaling HBM byte counters)")
    p.add_argument("--quantizer-sweep", action="store_true",
                   help="each producer alone at the FFN step's shapes after a read-only cache flush, beside a plain "
                        "streaming kernel with the same bytes read and written per element")
    p.add_argument("--hybrid-dgrad", action="store_true",
                   help="FFN step as the operand-wise hybrid: MXFP4 forward and Wgrads, CTA-local NVFP4 Dgrads")
    p.add_argument("--nvfp4-dgrad", action="store_true",
                   help="the CTA-local NVFP4 Dgrad of the FFN workload (producers, bf16-MFMA contraction) call by "
                        "call")
    return p.parse_args()


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_fast_kernel_ffn_step_8192x4096x14336_traffic.md")
# the sources gemm_fast_kernel is built from (its epilogue, main loop and helpers)
GEMM_SOURCES = [os.path.join(ROOT, "precision_mxfp4_producers_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_core.h", "mx_device.h")]


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, launches):
    """HBM bytes per gemm_fast_kernel launch from the committed counter summary,
    if it was taken on this workload, with the same launches per step and the
    current kernel source; else None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    fields = {}
    for line in open(TRAFFIC_SUMMARY):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if (fields.get("gemm kernel sources sha256 (first 16 hex)") != gemm_source_hash() or fields.get("workload") != workload
            or fields.get("gemm launches per step") != str(launches)):
        return None
    try:
        return float(fields["hbm bytes per launch (calibrated)"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of 1 GiB, three times: its FETCH_SIZE / WRITE_SIZE
    counters calibrate the byte counters against a known transfer."""
    import torch
    n = 1 << 28                                            # 2^28 fp32 = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                      "launches": 3}), flush=True)


def quantizer_sweep(mx, torch, reps=9):
    """Each producer alone, after a read-only pass over 1 GiB (evicts the
    256 MB Infinity Cache without leaving dirty lines), timed with HIP events;
    beside it a hand-written streaming kernel with the traffic of a
    one-orientation producer (2 B read with 16-byte loads, 0.5 B of nibbles
    written as whole lines and 1/32 B of side bytes per element, no rounding
    work: libmxfp4_bench.so), which shows what plain streaming reaches at that
    size on this part."""
    import ctypes
    import synthetic
    from precision_mxfp4_producers_amd.build import BENCH_LIB
    blib = ctypes.CDLL(BENCH_LIB)
    blib.mxfp4_stream_reference.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]
    blib.mxfp4_stream_reference.restype = ctypes.c_int
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    dev = torch.device("cuda:0")

    def timed(fn):
        ts = []
        for r in range(reps + 2):
            flush.max()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if r >= 2:
                ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    mask = mx.fp4_sign_mask_from_seed(0)
    rows = []
    for (R, C) in ((8192, 4096), (14336, 4096), (8192, 14336)):
        x = torch.from_numpy(synthetic.tensor((R, C), std=1.0, seed=5).view(np.int16)).to(dev)
        n = R * C
        rc, rs = torch.empty((R, C // 2), dtype=torch.uint8, device=dev), torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
        cc, cs = torch.empty((C, R // 2), dtype=torch.uint8, device=dev), torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
        def stream_ref():
            st = blib.mxfp4_stream_reference(x.data_ptr(), n, rc.data_ptr(), rs.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"streaming reference launch failed ({st})")
        ref_ms = timed(stream_ref)
        ref_gbps = n * B_SINGLE / (ref_ms * 1e-3) / 1e9
        calls = [
            ("rows RTN", B_SINGLE, lambda: mx.fp4_quantize_rows(x, 0, 0, 0, codes=rc, scales=rs)),
            ("rows SR", B_SINGLE, lambda: mx.fp4_quantize_rows(x, 1, 0, 0, codes=rc, scales=rs)),
            ("cols H32", B_SINGLE, lambda: mx.fp4_quantize_cols(x, 32, mask, codes_t=cc, scales_t=cs)),
            ("dual RTN rows + H32 cols", B_DUAL, lambda: mx.fp4_quantize_dual(x, 0, 0, 0, 32, mask, rc, rs, cc, cs)),
            ("dual SR rows + H32 cols", B_DUAL, lambda: mx.fp4_quantize_dual(x, 1, 0, 0, 32, mask, rc, rs, cc, cs)),
            ("2D32", B_2D32, lambda: mx.fp4_quantize_w2d32(x, 0.87, rc, rs, cc, cs)),
        ]
        for label, bpe, fn in calls:
            ms = timed(fn)
            gbps = n * bpe / (ms * 1e-3) / 1e9
            rows.append({"shape": f"{R}x{C}", "call": label, "us": round(ms * 1e3, 1), "gbps": round(gbps, 1),
                         "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                         "frac_streaming_reference": round(gbps / ref_gbps, 4)})
        rows.append({"shape": f"{R}x{C}", "call": "streaming reference (2 B in, 0.53125 B out)",
                     "us": round(ref_ms * 1e3, 1), "gbps": round(ref_gbps, 1),
                     "frac_hbm_peak": round(ref_gbps / PEAK_HBM_GBPS, 4), "frac_streaming_reference": 1.0})
    return rows


W2_GROUP = "W2 Wgrad | W2 Dgrad"          # label of the FFN backward's grouped launch


class Step:
    """Holds device inputs/outputs and enqueues one step as a list of named calls."""

    def __init__(self, name, seed, mx, torch, fused_backward=True, dgrad_epilogue=False, nvfp4_dgrad=False,
                 grouped=True):
        self.grouped = grouped
        self.fused_backward = fused_backward
        self.dgrad_epilogue = dgrad_epilogue and fused_backward
        self.nvfp4_dgrad = nvfp4_dgrad
        import synthetic
        self.mx, self.torch = mx, torch
        self.name = name
        self.host = synthetic.workload(name, seed=seed)
        self.seed = synthetic.WORKLOADS[name]["seed"] if seed is None else seed
        self.mask = mx.fp4_sign_mask_from_seed(self.seed)
        dev = torch.device("cuda:0")
        self.d = {k: torch.from_numpy(v.view(np.int16)).to(dev) for k, v in self.host.items()}
        self.o = {}
        self.calls = []          # (label, kind, units, fn, algorithmic bytes of a GEMM)
        self.charge = {}         # contraction label -> producer calls charged to it (each charged once)
        kind = name.split("_")[0]
        getattr(self, "_build_ffn_hybrid" if (kind == "ffn" and nvfp4_dgrad) else "_build_" + kind)()
        charged = sorted(q for v in self.charge.values() for q in v)
        producers = sorted(c[0] for c in self.calls if c[1] == "quant")
        assert charged == producers, f"every producer call is charged to exactly one contraction: {charged} {producers}"

    def e(self, shape, dtype):
        key = len(self.o)
        t = self.torch.empty(shape, dtype=dtype, device="cuda:0")
        self.o[key] = t
        return t

    def u8(self, *shape):
        return self.e(shape, self.torch.uint8)

    def q_rows(self, label, x, mode=0, offset=0):
        mx, (R, C) = self.mx, x.shape
        out = (self.u8(R, C // 2), self.u8(R, C // 32))
        self.calls.append((label, "quant", R * C * B_SINGLE,
                           lambda: mx.fp4_quantize_rows(x, mode, self.seed, offset, codes=out[0], scales=out[1]), 0))
        return out

    def q_cols(self, label, x, out=None):
        mx, (R, C) = self.mx, x.shape
        out = out if out is not None else (self.u8(C, R // 2), self.u8(C, R // 32))
        self.calls.append((label, "quant", R * C * B_SINGLE,
                           lambda: mx.fp4_quantize_cols(x, 32, self.mask, codes_t=out[0], scales_t=out[1]), 0))
        return out

    def q_dual(self, label, x, mode=1, offset=0):
        """Row-facing (SR or RTN) and column-facing H32 of x from one read."""
        mx, (R, C) = self.mx, x.shape
        out = (self.u8(R, C // 2), self.u8(R, C // 32), self.u8(C, R // 2), self.u8(C, R // 32))
        self.calls.append((label, "quant", R * C * B_DUAL,
                           lambda: mx.fp4_quantize_dual(x, mode, self.seed, offset, 32, self.mask, *out), 0))
        return out[:2], out[2:]

    def q_w(self, label, w, row_codes=None, row_scales=None):
        mx, (N, K) = self.mx, w.shape
        rc = row_codes if row_codes is not None else self.u8(N, K // 2)
        rs = row_scales if row_scales is not None else self.u8(N, K // 32)
        out = (rc, rs, self.u8(K, N // 2), self.u8(K, N // 32))
        self.calls.append((label, "quant", N * K * B_2D32,
                           lambda: mx.fp4_quantize_w2d32(w, 0.87, *out), 0))
        return out

    def gemm(self, label, a, b, c=None, accumulate=False):
        mx = self.mx
        m, n, k = a[0].shape[0], b[0].shape[0], 2 * a[0].shape[1]
        if c is None:
            c = self.e((m, n), self.torch.float32)
        alg_bytes = (m + n) * k * (0.5 + 1 / 32) + 4 * m * n * (2 if accumulate else 1)
        self.calls.append((label, "gemm", 2.0 * m * n * k,
                           lambda: mx.fp4_gemm(a[0], a[1], b[0], b[1], c=c, accumulate=accumulate), alg_bytes))
        return c

    def gemm_pair(self, label, a1, b1, a2, b2):
        mx = self.mx
        m, n, k = a1[0].shape[0], b1[0].shape[0], 2 * a1[0].shape[1]
        c = self.e((m, n), self.torch.float32)
        alg_bytes = 2 * (m + n) * k * (0.5 + 1 / 32) + 4 * m * n
        self.calls.append((label, "gemm", 2.0 * m * n * 2 * k,
                           lambda: mx.fp4_gemm_pair(a1[0], a1[1], b1[0], b1[1], a2[0], a2[1], b2[0], b2[1], c=c),
                           alg_bytes))
        return c

    def gemm_group(self, label, probs):
        """Independent contractions in one launch (fp4_gemm_grouped).  probs:
        (a, b, a2, b2, c) with a2 = b2 = None for the plain form."""
        mx, torch = self.mx, self.torch
        flops = alg_bytes = 0
        args = []
        for a, b, a2, b2, c in probs:
            m, n, k = a[0].shape[0], b[0].shape[0], 2 * a[0].shape[1]
            npair = 1 if a2 is None else 2
            flops += 2.0 * m * n * k * npair
            alg_bytes += npair * (m + n) * k * (0.5 + 1 / 32) + 4 * m * n
            d = dict(a_codes=a[0], a_scales=a[1], b_codes=b[0], b_scales=b[1], c=c)
            if a2 is not None:
                d.update(a2_codes=a2[0], a2_scales=a2[1], b2_codes=b2[0], b2_scales=b2[1])
            args.append(d)
        self.calls.append((label, "gemm", flops, lambda: mx.fp4_gemm_grouped(args), alg_bytes))

    # CTA-local NVFP4 calls (the operand-wise hybrid's Dgrads)
    def nv_rows(self, label, x, offset):
        mx, torch, (R, C) = self.mx, self.torch, x.shape
        p = (R + 255) // 256
        out = [self.u8(R, C // 2), self.u8(R, C // 16), self.e((p,), torch.float32), self.e((p,), torch.float32)]
        self.calls.append((label, "quant", R * C * B_NV_ROWS,
                           lambda: mx.fp4_nv_quantize_rows(x, 1, self.seed, offset, out=out), 0))
        return out

    def nv_w(self, label, w):
        mx, torch, (N, K) = self.mx, self.torch, w.shape
        out = [self.u8(N, K // 2), self.u8(N, K // 16), self.u8(K, N // 2), self.u8(K, N // 16),
               self.e((1,), torch.float32), self.e((1,), torch.float32)]
        self.calls.append((label, "quant", N * K * B_NV_W2D16, lambda: mx.fp4_nv_quantize_w2d16(w, out=out), 0))
        return out

    def nv_gemm(self, label, a, b, c=None, accumulate=False):
        mx = self.mx
        m, n, k = a[0].shape[0], b[0].shape[0], 2 * a[0].shape[1]
        if c is None:
            c = self.e((m, n), self.torch.float32)
        self.calls.append((label, "nvgemm", 2.0 * m * n * k,
                           lambda: mx.fp4_nv_gemm(a[0], a[1], a[2], b[0], b[1], b[2], c=c, accumulate=accumulate), 0))
        return c

    # -------------------------------------------------------------- workloads
    def _build_fprop(self):                      # fprop_256x512x512: 1x32 blocks for X and W
        xr = self.q_rows("rows(X)", self.d["X"])
        wr = self.q_rows("rows(W)", self.d["W"])
        self.gemm("Fprop", xr, wr)
        self.charge = {"Fprop": ["rows(X)", "rows(W)"]}

    def _build_attn(self):                       # attn_proj: Fprop + Dgrad
        xr = self.q_rows("rows(X)", self.d["X"])
        wq = self.q_w("w2d32(W)", self.d["W"])
        dyr = self.q_rows("rows(dY,SR)", self.d["dY"], 1, 0)
        self.gemm("Fprop", xr, wq[:2])
        self.gemm("Dgrad", dyr, wq[2:])
        self.charge = {"Fprop": ["rows(X)", "w2d32(W)"], "Dgrad": ["rows(dY,SR)"]}

    def _build_wgrad(self):                      # wgrad_h32: paired H32 Wgrad
        dyc = self.q_cols("cols(dY,H32)", self.d["dY"])
        xc = self.q_cols("cols(X,H32)", self.d["X"])
        self.gemm("Wgrad", dyc, xc)
        self.charge = {"Wgrad": ["cols(dY,H32)", "cols(X,H32)"]}

    def _build_ffn(self):                        # full SwiGLU FFN step
        torch, mx = self.torch, self.mx
        X, W1, W3, W2, dY = (self.d[k] for k in ("X", "W1", "W3", "W2", "dY"))
        T, D = X.shape
        F = W1.shape[0]
        if self.fused_backward:
            # X row RTN (forward) and column H32 (W1/W3 Wgrad) from one read
            xr, xc_dual = self.q_dual("dual(X: RTN rows, H32 cols)", X, 0)
        else:
            xr = self.q_rows("rows(X)", X)
        w13_rc, w13_rs = self.u8(2 * F, D // 2), self.u8(2 * F, D // 32)
        w1 = self.q_w("w2d32(W1)", W1, w13_rc[:F], w13_rs[:F])
        w3 = self.q_w("w2d32(W3)", W3, w13_rc[F:], w13_rs[F:])
        a, b = self.e((T, F), torch.int16), self.e((T, F), torch.int16)
        hr = (self.u8(T, F // 2), self.u8(T, F // 32))
        hc = (self.u8(F, T // 2), self.u8(F, T // 32))
        self.calls.append(("swiglu_producer", "producer", 2.0 * T * 2 * F * D,
                           lambda: mx.fp4_swiglu_producer(xr[0], xr[1], w13_rc, w13_rs, self.mask, True,
                                                          a, b, hr[0], hr[1], hc[0], hc[1]), 0))
        # W2's producer runs right before the contraction that reads it, so its
        # codes are still in the Infinity Cache (launch orders measured on one
        # MI355X: this and the Wgrad-before-Dgrad order below save about 1%)
        w2 = self.q_w("w2d32(W2)", W2)
        self.gemm("W2 Fprop", hr, w2[:2])
        if self.fused_backward:
            dyr, dyc = self.q_dual("dual(dY: SR rows, H32 cols)", dY, 1, 0)
        else:
            dyr = self.q_rows("rows(dY,SR)", dY, 1, 0)
            dyc = self.q_cols("cols(dY,H32)", dY)
        if self.dgrad_epilogue:
            # dH = dY W2 with the SwiGLU backward producer in the epilogue
            shapes = [(T, F // 2), (T, F // 32)] * 2
            outs = [self.u8(*shp) for shp in shapes] + [None] * 4
            label = "W2 Dgrad + swiglu_bwd_producer"
            self.calls.append((label, "producer", 2.0 * T * F * D,
                               lambda: mx.fp4_gemm_swiglu_backward_producer(dyr[0], dyr[1], w2[2], w2[3], a, b,
                                                                            self.seed, 1, 2, self.mask, outs), 0))
            self.gemm("W2 Wgrad", dyc, hc)
        elif self.grouped:
            # W2 Wgrad has 896 tiles of 32 K steps (3.5 rounds of 256 CUs): in
            # one launch with W2 Dgrad's 1792 shorter tiles, those fill the CUs
            # that its last round leaves idle
            dh = self.e((T, F), torch.float32)
            dw2 = self.e((D, F), torch.float32)
            self.gemm_group(W2_GROUP, [(dyc, hc, None, None, dw2), (dyr, w2[2:], None, None, dh)])
        else:
            dh = self.gemm("W2 Dgrad", dyr, w2[2:])
            self.gemm("W2 Wgrad", dyc, hc)
        # column-facing dA and dB land in one stacked [2F][T/2] buffer, so that
        # the W1 and W3 Wgrads (same B operand, X column-facing) run as one
        # contraction with M = 2F: 2x896 256x256 tiles (3.5 rounds of 256 CUs
        # each) become 1792 (7 full rounds)
        dabc = (self.u8(2 * F, T // 2), self.u8(2 * F, T // 32))
        dac, dbc = (dabc[0][:F], dabc[1][:F]), (dabc[0][F:], dabc[1][F:])
        if self.dgrad_epilogue:
            outs[4:] = [dac[0], dac[1], dbc[0], dbc[1]]
            dar, dbr = (outs[0], outs[1]), (outs[2], outs[3])
        elif self.fused_backward:
            shapes = [(T, F // 2), (T, F // 32)] * 2
            outs = [self.u8(*shp) for shp in shapes] + [dac[0], dac[1], dbc[0], dbc[1]]
            dar, dbr = (outs[0], outs[1]), (outs[2], outs[3])
            self.calls.append(("swiglu_bwd_producer", "quant", T * F * B_BWD_PRODUCER,
                               lambda: mx.fp4_swiglu_backward_producer(dh, a, b, self.seed, 1, 2, self.mask, outs), 0))
        else:
            da, db = self.e((T, F), torch.int16), self.e((T, F), torch.int16)
            self.calls.append(("swiglu_backward", "quant", T * F * B_SWIGLU_BWD,
                               lambda: mx.fp4_swiglu_backward(dh, a, b, da, db), 0))
            dar = self.q_rows("rows(dA,SR)", da, 1, 1)
            dbr = self.q_rows("rows(dB,SR)", db, 1, 2)
            self.q_cols("cols(dA,H32)", da, out=dac)
            self.q_cols("cols(dB,H32)", db, out=dbc)
        xc = xc_dual if self.fused_backward else self.q_cols("cols(X,H32)", X)
        # the stacked Wgrad reads the column-facing dA, dB just written; then
        # dX = dA W1 + dB W3 as one contraction over K = 2F (no fp32 read-back of dX)
        # (these two stay separate launches: grouped, with the longer Dgrad tiles
        # first, they saved about 3 us themselves but the next step's SwiGLU
        # producer ran about 22 us slower after them, on four alternating runs)
        self.gemm("W1|W3 Wgrad", dabc, xc)
        self.gemm_pair("W1+W3 Dgrad", dar, w1[2:], dbr, w3[2:])
        # each producer is charged to the first contraction that reads it
        self.charge = {"swiglu_producer": ["w2d32(W1)", "w2d32(W3)"], "W2 Fprop": ["w2d32(W2)"]}
        w2dg = "W2 Dgrad + swiglu_bwd_producer" if self.dgrad_epilogue else W2_GROUP if self.grouped else "W2 Dgrad"
        w2wg = W2_GROUP if self.grouped and not self.dgrad_epilogue else "W2 Wgrad"
        w13wg, w13dg = "W1|W3 Wgrad", "W1+W3 Dgrad"
        if self.fused_backward:
            self.charge["swiglu_producer"].append("dual(X: RTN rows, H32 cols)")
            self.charge[w2dg] = ["dual(dY: SR rows, H32 cols)"]
        else:
            self.charge["swiglu_producer"].append("rows(X)")
            self.charge[w2dg] = ["rows(dY,SR)"]
            self.charge.setdefault(w2wg, []).append("cols(dY,H32)")
            self.charge.setdefault(w13wg, []).append("cols(X,H32)")
        if self.dgrad_epilogue:
            pass
        elif self.fused_backward:
            self.charge.setdefault(w13dg, []).append("swiglu_bwd_producer")
        else:
            self.charge.setdefault(w13dg, []).extend(["swiglu_backward", "rows(dA,SR)", "rows(dB,SR)"])
            self.charge[w13wg] += ["cols(dA,H32)", "cols(dB,H32)"]

    def _build_ffn_hybrid(self):
        """The operand-wise hybrid (FAF §3.3): the forward and both Wgrads in
        MXFP4 as in the default step, both Dgrads in CTA-local NVFP4 (row SR of
        dY, dA and dB with panel factors; 2D16 column views of W2, W1 and W3;
        the contraction on the f16 matrix cores).  dY and dA/dB are quantized
        twice (NVFP4 rows for Dgrad, MXFP4 H32 columns for Wgrad)."""
        torch, mx = self.torch, self.mx
        X, W1, W3, W2, dY = (self.d[k] for k in ("X", "W1", "W3", "W2", "dY"))
        T, D = X.shape
        F = W1.shape[0]
        xr, xc = self.q_dual("dual(X: RTN rows, H32 cols)", X, 0)
        w13_rc, w13_rs = self.u8(2 * F, D // 2), self.u8(2 * F, D // 32)
        self.q_w("w2d32(W1)", W1, w13_rc[:F], w13_rs[:F])
        self.q_w("w2d32(W3)", W3, w13_rc[F:], w13_rs[F:])
        a, b = self.e((T, F), torch.int16), self.e((T, F), torch.int16)
        hr = (self.u8(T, F // 2), self.u8(T, F // 32))
        hc = (self.u8(F, T // 2), self.u8(F, T // 32))
        self.calls.append(("swiglu_producer", "producer", 2.0 * T * 2 * F * D,
                           lambda: mx.fp4_swiglu_producer(xr[0], xr[1], w13_rc, w13_rs, self.mask, True,
                                                          a, b, hr[0], hr[1], hc[0], hc[1]), 0))
        w2 = self.q_w("w2d32(W2)", W2)
        self.gemm("W2 Fprop", hr, w2[:2])
        dyc = self.q_cols("cols(dY,H32)", dY)
        dyn = self.nv_rows("nv rows(dY,SR)", dY, 0)
        w2n = self.nv_w("nv 2D16(W2)", W2)
        dh = self.nv_gemm("W2 Dgrad (NVFP4)", dyn[:3], w2n[2:5])
        self.gemm("W2 Wgrad", dyc, hc)
        da, db = self.e((T, F), torch.int16), self.e((T, F), torch.int16)
        self.calls.append(("swiglu_backward", "quant", T * F * B_SWIGLU_BWD,
                           lambda: mx.fp4_swiglu_backward(dh, a, b, da, db), 0))
        dabc = (self.u8(2 * F, T // 2), self.u8(2 * F, T // 32))
        self.q_cols("cols(dA,H32)", da, out=(dabc[0][:F], dabc[1][:F]))
        self.q_cols("cols(dB,H32)", db, out=(dabc[0][F:], dabc[1][F:]))
        self.gemm("W1|W3 Wgrad", dabc, xc)
        dan = self.nv_rows("nv rows(dA,SR)", da, 1)
        dbn = self.nv_rows("nv rows(dB,SR)", db, 2)
        w1n = self.nv_w("nv 2D16(W1)", W1)
        w3n = self.nv_w("nv 2D16(W3)", W3)
        dx = self.nv_gemm("W1 Dgrad (NVFP4)", dan[:3], w1n[2:5])
        self.nv_gemm("W3 Dgrad (NVFP4)", dbn[:3], w3n[2:5], c=dx, accumulate=True)
        self.charge = {"swiglu_producer": ["w2d32(W1)", "w2d32(W3)", "dual(X: RTN rows, H32 cols)"],
                       "W2 Fprop": ["w2d32(W2)"],
                       "W2 Dgrad (NVFP4)": ["nv rows(dY,SR)", "nv 2D16(W2)"],
                       "W2 Wgrad": ["cols(dY,H32)"],
                       "W1|W3 Wgrad": ["swiglu_backward", "cols(dA,H32)", "cols(dB,H32)"],
                       "W1 Dgrad (NVFP4)": ["nv rows(dA,SR)", "nv 2D16(W1)"],
                       "W3 Dgrad (NVFP4)": ["nv rows(dB,SR)", "nv 2D16(W3)"]}

    def run(self, events=None):
        for i, (_, _, _, fn, _) in enumerate(self.calls):
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()

    def gemm_flops(self):
        return sum(c[2] for c in self.calls if c[1] in ("gemm", "producer", "nvgemm"))


CPU_SAMPLE_SHAPES = {
    # reduced instances of each workload: same laws, fewer rows
    "ffn": dict(T=256, F=6144),
    "attn": dict(T=64),
    "wgrad": dict(T=64),
    "fprop": dict(),
}


def oracle_step(name, h, seed, mask):
    """The CPU oracle's version of one step on host tensors; returns GEMM FLOPs."""
    from oracle import gemm as G
    from oracle import quant as Q
    from oracle import swiglu as S

    def mm(a, b):
        return G.gemm_ref(a[0], a[1], b[0], b[1])[0], 2.0 * a[0].shape[0] * b[0].shape[0] * a[0].shape[1] * 2

    kind = name.split("_")[0]
    flops = 0.0
    if kind == "fprop":
        _, f = mm(Q.quantize_rows(h["X"]), Q.quantize_rows(h["W"]))
        return f
    if kind == "attn":
        xr, w = Q.quantize_rows(h["X"]), Q.quantize_w2d32(h["W"])
        dyr = Q.quantize_rows(h["dY"], Q.SR, seed, 0)
        for a, b in ((xr, w[:2]), (dyr, w[2:])):
            flops += mm(a, b)[1]
        return flops
    if kind == "wgrad":
        return mm(Q.quantize_cols(h["dY"], 32, mask), Q.quantize_cols(h["X"], 32, mask))[1]
    X, W1, W3, W2, dY = (h[k] for k in ("X", "W1", "W3", "W2", "dY"))
    F = W1.shape[0]
    xr = Q.quantize_rows(X)
    w1, w3, w2 = Q.quantize_w2d32(W1), Q.quantize_w2d32(W3), Q.quantize_w2d32(W2)
    ab, f = mm(xr, (np.concatenate([w1[0], w3[0]]), np.concatenate([w1[1], w3[1]])))
    flops += f
    a = S.f32_to_bf16_rne(ab[:, :F].astype(np.float32))
    b = S.f32_to_bf16_rne(ab[:, F:].astype(np.float32))
    hb = S.swiglu_h(a, b)
    hr, hc = Q.quantize_rows(hb), Q.quantize_cols(hb, 32, mask)
    flops += mm(hr, w2[:2])[1]
    dyr, dyc = Q.quantize_rows(dY, Q.SR, seed, 0), Q.quantize_cols(dY, 32, mask)
    dh, f = mm(dyr, w2[2:])
    flops += f + mm(dyc, hc)[1]
    da, db = S.swiglu_backward(dh.astype(np.float32), a, b)
    dar, dbr = Q.quantize_rows(da, Q.SR, seed, 1), Q.quantize_rows(db, Q.SR, seed, 2)
    dac, dbc, xc = Q.quantize_cols(da, 32, mask), Q.quantize_cols(db, 32, mask), Q.quantize_cols(X, 32, mask)
    for a_, b_ in ((dar, w1[2:]), (dbr, w3[2:]), (dac, xc), (dbc, xc)):
        flops += mm(a_, b_)[1]
    return flops


def cpu_baseline(step):
    """Time the CPU oracle on a bounded sample: the same step on a reduced
    instance of the workload (same laws and model width, fewer tokens / FFN
    columns), reported as GEMM FLOPs of that instance per second."""
    import threadpoolctl
    import synthetic
    kind = step.name.split("_")[0]
    spec = synthetic.WORKLOADS[step.name]["tensors"]
    red = CPU_SAMPLE_SHAPES[kind]
    shapes = {}
    for nm, (R, C, *_rest) in spec.items():
        if kind == "ffn":
            T, F = red["T"], red["F"]
            shapes[nm] = {"X": (T, C), "dY": (T, C), "W1": (F, C), "W3": (F, C), "W2": (R, F)}[nm]
        elif nm in ("X", "dY") and "T" in red:
            shapes[nm] = (red["T"], C)
    h = synthetic.workload(step.name, seed=step.seed, shapes=shapes)
    t0 = time.perf_counter()
    flops = oracle_step(step.name, h, step.seed, step.mask)
    dt = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    desc = ", ".join(f"{k} {v[0]}x{v[1]}" for k, v in (shapes or {k: v[:2] for k, v in spec.items()}).items())
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"whole step on a reduced instance ({desc}), {flops / 1e9:.2f} GFLOP in {dt:.1f} s",
            "host_cpus": os.cpu_count()}



QUALITY_CASES = {
    # attention-projection laws at full size: X with 0.1% x20 outliers
    "attn_proj_8192x4096x4096": None,
    # heavy-tailed laws of the large FFN workload (Student-t3 X, W ~ N(0,0.015),
    # dY ~ N(0,1e-4) with 1% x50 outliers) on one 8192 x 4096 x 4096 layer
    "ffn_large_32768x8192x28672": {"X": (8192, 4096), "W1": (4096, 4096), "dY": (8192, 4096)},
}


SR_DRAWS = 8


def quality_metrics(c, ref):
    """Error of an MXFP4 contraction c against its fp32 reference ref (both
    converted to float64): relative L2 error ||c - ref|| / ||ref||, the SNR
    -20 log10 of it in dB, the cosine <c, ref> / (||c|| ||ref||), and the
    bias mean(c - ref) / rms(ref).  Accepts numpy arrays or torch tensors."""
    c = np.asarray(c.double().cpu().numpy() if hasattr(c, "double") else c, dtype=np.float64).ravel()
    ref = np.asarray(ref.double().cpu().numpy() if hasattr(ref, "double") else ref, dtype=np.float64).ravel()
    d = c - ref
    rl2 = float(np.linalg.norm(d) / np.linalg.norm(ref))
    return {"rel_l2": round(rl2, 6),
            "snr_db": round(-20 * math.log10(rl2), 2) if rl2 > 0 else float("inf"),
            "cosine": round(float(c @ ref / (np.linalg.norm(c) * np.linalg.norm(ref))), 7),
            "bias": round(float(d.mean() / np.sqrt(np.mean(ref * ref))), 7)}


def quality_report(mx, torch):
    """Relative L2 error, cosine and bias of each MXFP4 contraction against the
    fp32 contraction of the same bf16 tensors, with the method's ablations:
    2D32 weights vs 1x32 blocks, finer 2D32 scale on/off, SR vs RTN for Dgrad,
    H32 vs none for Wgrad."""
    import synthetic
    out = []
    for name, shapes in QUALITY_CASES.items():
        h = synthetic.workload(name, shapes=shapes)
        seed = synthetic.WORKLOADS[name]["seed"]
        mask = mx.fp4_sign_mask_from_seed(seed)
        dev = lambda k: torch.from_numpy(h[k].view(np.int16)).cuda()
        X, dY = dev("X"), dev("dY")
        W = dev("W" if "W" in h else "W1")
        f32 = lambda t: t.view(torch.bfloat16).float()
        refs = {"Fprop": f32(X) @ f32(W).T, "Dgrad": f32(dY) @ f32(W), "Wgrad": f32(dY).T.contiguous() @ f32(X)}

        def score(kind, variant, c):
            out.append({"workload": name, "contraction": kind, "variant": variant,
                        **quality_metrics(c, refs[kind])})

        xr = mx.fp4_quantize_rows(X)
        for ratio, tag in ((0.87, "2D32, finer rule 0.87"), (0.0, "2D32, finer rule off")):
            wq = mx.fp4_quantize_w2d32(W, ratio)
            score("Fprop", tag, mx.fp4_gemm(xr[0], xr[1], wq[0], wq[1]))
            if ratio:
                for mode, mtag in ((mx.FP4_SR, "SR"), (mx.FP4_RTN, "RTN")):
                    dyr = mx.fp4_quantize_rows(dY, mode, seed, 0)
                    score("Dgrad", f"dY {mtag}, W 2D32 columns", mx.fp4_gemm(dyr[0], dyr[1], wq[2], wq[3]))
                # SR's point is an unbiased estimate across steps: the mean of
                # independent draws (offsets 0..7) approaches the exact product
                # while RTN's error stays
                acc = None
                for off in range(SR_DRAWS):
                    dyr = mx.fp4_quantize_rows(dY, mx.FP4_SR, seed, off)
                    c = mx.fp4_gemm(dyr[0], dyr[1], wq[2], wq[3])
                    acc = c if acc is None else acc.add_(c)
                score("Dgrad", f"dY SR, mean of {SR_DRAWS} draws, W 2D32 columns", acc.div_(SR_DRAWS))
        # CTA-local NVFP4 Dgrad (E4M3 16-value scales, 256-row panel factors,
        # 2D16 weight with one factor) beside the MXFP4 Dgrad on the same
        # tensors and draws; the error energy is the squared L2 error
        wq = mx.fp4_quantize_w2d32(W, 0.87)
        wn = mx.fp4_nv_quantize_w2d16(W)
        for mode, mtag in ((mx.FP4_SR, "SR"), (mx.FP4_RTN, "RTN")):
            dyr = mx.fp4_quantize_rows(dY, mode, seed, 0)
            c_mx = mx.fp4_gemm(dyr[0], dyr[1], wq[2], wq[3])
            dyn = mx.fp4_nv_quantize_rows(dY, mode, seed, 0)
            c_nv = mx.fp4_nv_gemm(dyn[0], dyn[1], dyn[2], wn[2], wn[3], wn[4])
            score("Dgrad", f"CTA-local NVFP4: dY {mtag}, W 2D16 columns", c_nv)
            e_mx = float(((c_mx.double() - refs["Dgrad"].double()) ** 2).sum())
            e_nv = float(((c_nv.double() - refs["Dgrad"].double()) ** 2).sum())
            out.append({"workload": name, "contraction": "Dgrad", "variant": f"error energy ratio E_MX / E_NV, dY {mtag}",
                        "e_mx": e_mx, "e_nv": e_nv, "ratio": round(e_mx / e_nv, 4)})
            del c_mx, c_nv
        wr = mx.fp4_quantize_rows(W)
        score("Fprop", "1x32 weight blocks", mx.fp4_gemm(xr[0], xr[1], wr[0], wr[1]))
        for had, tag in ((32, "paired fixed-sign H32"), (0, "no Hadamard")):
            dyc = mx.fp4_quantize_cols(dY, had, mask)
            xc = mx.fp4_quantize_cols(X, had, mask)
            score("Wgrad", tag, mx.fp4_gemm(dyc[0], dyc[1], xc[0], xc[1]))
        del refs
        torch.cuda.empty_cache()
    return out

PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 / f16 MFMA, published
B_NV_ROWS = 2 + 0.5 + 1 / 16     # bf16 in, codes and E4M3 scales out
B_NV_W2D16 = 2 + 2 * (0.5 + 1 / 16)


def nvfp4_dgrad(mx, torch, name, reps=7):
    """The CTA-local NVFP4 Dgrad of the gated FFN at full size, call by call
    (eager, HIP events, median of `reps` after two untimed passes): row SR of
    dY and 2D16 of W2, dH = dY W2, the SwiGLU backward to bf16 dA and dB, their
    row SR, 2D16 of W1 and W3, dX = dA W1 + dB W3 (second product accumulating).
    a, b come from the MXFP4 forward producer.  GEMMs against the dense 16-bit
    MFMA peak (the contraction runs on the f16 matrix cores), producers
    against HBM."""
    import synthetic
    h = synthetic.workload(name)
    seed = synthetic.WORKLOADS[name]["seed"]
    dev = lambda k: torch.from_numpy(h[k].view(np.int16)).cuda()
    X, W1, W3, W2, dY = (dev(k) for k in ("X", "W1", "W3", "W2", "dY"))
    T, D = X.shape
    F = W1.shape[0]
    xr = mx.fp4_quantize_rows(X)
    w13 = torch.cat([W1, W3])
    wq = mx.fp4_quantize_w2d32(w13)
    a, b = mx.fp4_swiglu_producer(xr[0], xr[1], wq[0], wq[1], mx.fp4_sign_mask_from_seed(seed), emit_cols=False)[:2]
    del wq, w13
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device="cuda")
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    o = {}
    o["dy"] = [u8(T, D // 2), u8(T, D // 16), f32((T + 255) // 256), f32((T + 255) // 256)]
    for nm, (n_, k_) in (("w2", (D, F)), ("w1", (F, D)), ("w3", (F, D))):
        o[nm] = [u8(n_, k_ // 2), u8(n_, k_ // 16), u8(k_, n_ // 2), u8(k_, n_ // 16), f32(1), f32(1)]
    for nm in ("da", "db"):
        o[nm] = [u8(T, F // 2), u8(T, F // 16), f32((T + 255) // 256), f32((T + 255) // 256)]
    dh, dx = f32(T, F), f32(T, D)
    da, db = torch.empty((T, F), dtype=torch.int16, device="cuda"), torch.empty((T, F), dtype=torch.int16, device="cuda")
    calls = [
        ("nv rows SR (dY)", "producer", T * D * B_NV_ROWS, lambda: mx.fp4_nv_quantize_rows(dY, 1, seed, 0, out=o["dy"])),
        ("nv 2D16 (W2)", "producer", D * F * B_NV_W2D16, lambda: mx.fp4_nv_quantize_w2d16(W2, out=o["w2"])),
        ("nv GEMM dH = dY W2", "gemm", 2.0 * T * F * D,
         lambda: mx.fp4_nv_gemm(o["dy"][0], o["dy"][1], o["dy"][2], o["w2"][2], o["w2"][3], o["w2"][4], c=dh)),
        ("SwiGLU backward (bf16 dA, dB)", "other", T * F * 12, lambda: mx.fp4_swiglu_backward(dh, a, b, da, db)),
        ("nv rows SR (dA)", "producer", T * F * B_NV_ROWS, lambda: mx.fp4_nv_quantize_rows(da, 1, seed, 1, out=o["da"])),
        ("nv rows SR (dB)", "producer", T * F * B_NV_ROWS, lambda: mx.fp4_nv_quantize_rows(db, 1, seed, 2, out=o["db"])),
        ("nv 2D16 (W1)", "producer", F * D * B_NV_W2D16, lambda: mx.fp4_nv_quantize_w2d16(W1, out=o["w1"])),
        ("nv 2D16 (W3)", "producer", F * D * B_NV_W2D16, lambda: mx.fp4_nv_quantize_w2d16(W3, out=o["w3"])),
        ("nv GEMM dX = dA W1", "gemm", 2.0 * T * D * F,
         lambda: mx.fp4_nv_gemm(o["da"][0], o["da"][1], o["da"][2], o["w1"][2], o["w1"][3], o["w1"][4], c=dx)),
        ("nv GEMM dX += dB W3", "gemm", 2.0 * T * D * F,
         lambda: mx.fp4_nv_gemm(o["db"][0], o["db"][1], o["db"][2], o["w3"][2], o["w3"][3], o["w3"][4], c=dx,
                                accumulate=True)),
    ]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(reps + 2)]
    for r in range(reps + 2):
        for i, (_, _, _, fn) in enumerate(calls):
            ev[r][i][0].record()
            fn()
            ev[r][i][1].record()
        print(f"[bench] nvfp4 dgrad pass {r + 1}/{reps + 2}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    rows, total = [], 0.0
    for i, (label, kind, units, _) in enumerate(calls):
        ms = float(np.median([ev[r][i][0].elapsed_time(ev[r][i][1]) for r in range(2, reps + 2)]))
        total += ms
        e = {"call": label, "us": round(ms * 1e3, 1)}
        if kind == "gemm":
            e["tflops"] = round(units / ms / 1e9, 1)
            e["frac_16bit_mfma_peak"] = round(units / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
        else:
            e["gbps"] = round(units / ms / 1e6, 1)
            e["frac_hbm_peak"] = round(units / ms / 1e6 / PEAK_HBM_GBPS, 4)
        rows.append(e)
    flops = sum(c[2] for c in calls if c[1] == "gemm")
    return {"workload": name, "calls": rows, "total_us": round(total * 1e3, 1),
            "dgrad_tflop": round(flops / 1e12, 4), "quantize_gemm_tflops": round(flops / (total * 1e-3) / 1e12, 1)}


def cpu_baseline_nv(name, seed=None):
    """Time the CPU oracle's CTA-local NVFP4 Dgrad route (the calls of
    nvfp4_dgrad) on a reduced instance of the FFN workload (T 256, F 6144,
    same laws); a, b come from the oracle's MXFP4 forward outside the timed
    region.  Reported as contraction FLOPs per second."""
    import threadpoolctl
    import synthetic
    from oracle import gemm as G
    from oracle import nvfp4 as NV
    from oracle import quant as Q
    from oracle import swiglu as S
    red = CPU_SAMPLE_SHAPES["ffn"]
    T, F = red["T"], red["F"]
    spec = synthetic.WORKLOADS[name]["tensors"]
    D = spec["X"][1]
    shapes = {"X": (T, D), "dY": (T, D), "W1": (F, D), "W3": (F, D), "W2": (D, F)}
    seed = synthetic.WORKLOADS[name]["seed"] if seed is None else seed
    h = synthetic.workload(name, seed=seed, shapes=shapes)
    xr = Q.quantize_rows(h["X"])
    w1, w3 = Q.quantize_w2d32(h["W1"]), Q.quantize_w2d32(h["W3"])
    ab = G.gemm_ref(xr[0], xr[1], np.concatenate([w1[0], w3[0]]), np.concatenate([w1[1], w3[1]]))[0]
    a = S.f32_to_bf16_rne(ab[:, :F].astype(np.float32))
    b = S.f32_to_bf16_rne(ab[:, F:].astype(np.float32))

    def one(w):                                          # a weight's 2D16 column view with its factor
        q = NV.quantize_w2d16(w)
        return q[2], q[3], np.repeat(np.float32(q[4]), (q[2].shape[0] + NV.PANEL - 1) // NV.PANEL)

    t0 = time.perf_counter()
    dyq = NV.quantize_rows(h["dY"], NV.SR, seed, 0)
    w2c = one(h["W2"])
    dh = NV.gemm_ref(dyq[0], dyq[1], dyq[2], *w2c)[0]
    da, db = S.swiglu_backward(dh.astype(np.float32), a, b)
    daq, dbq = NV.quantize_rows(da, NV.SR, seed, 1), NV.quantize_rows(db, NV.SR, seed, 2)
    w1c, w3c = one(h["W1"]), one(h["W3"])
    dx = NV.gemm_ref(daq[0], daq[1], daq[2], *w1c)[0] + NV.gemm_ref(dbq[0], dbq[1], dbq[2], *w3c)[0]
    dt = time.perf_counter() - t0
    del dx
    flops = 3 * 2.0 * T * F * D
    info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"the NVFP4 Dgrad route on a reduced FFN instance (T {T}, D {D}, F {F}), "
                      f"{flops / 1e9:.2f} GFLOP in {dt:.1f} s", "host_cpus": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU's share of the step; --gpus must be 1",
                          "gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    import precision_mxfp4_producers_amd as mx
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_calibration:
        copy_calibration()
        return
    mx.load()
    torch.cuda.set_device(0)
    if args.quality:
        print(json.dumps({"quality": quality_report(mx, torch)}), flush=True)
        return
    if args.quantizer_sweep:
        print(json.dumps({"quantizer_sweep": quantizer_sweep(mx, torch)}), flush=True)
        return
    if args.nvfp4_dgrad:
        res = nvfp4_dgrad(mx, torch, args.workload)
        if not args.no_cpu_baseline:
            print("[bench] timing the CPU oracle's NVFP4 route on a sample", file=sys.stderr, flush=True)
            res["cpu_baseline"] = cpu_baseline_nv(args.workload)
        print(json.dumps({"nvfp4_dgrad": res}), flush=True)
        return
    print(f"[bench] building inputs for {args.workload}", file=sys.stderr, flush=True)
    step = Step(args.workload, args.seed, mx, torch, fused_backward=not args.unfused_backward,
                dgrad_epilogue=args.dgrad_epilogue, nvfp4_dgrad=args.hybrid_dgrad,
                grouped=not args.separate_gemms)
    ncalls = len(step.calls)
    print(f"[bench] warmup {args.warmup} steps, {ncalls} calls per step", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # per-call times: eager steps with HIP events around every call
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(ncalls)]
          for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step.run(ev[s])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    print(f"[bench] {args.steps} eager steps in {total_ms:.2f} ms", file=sys.stderr, flush=True)
    mode = "eager"
    if not args.eager:
        # the step as one captured HIP graph (every call writes preallocated
        # buffers; no memsets): removes the launch gaps between the calls
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step.run()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            graph.replay()
        stop.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(stop)
        mode = "hip graph"
        print(f"[bench] {args.steps} graph replays in {total_ms:.2f} ms", file=sys.stderr, flush=True)
    ms_per_step = total_ms / args.steps

    per = []
    for i, (label, kind, units, _, _) in enumerate(step.calls):
        ms = float(np.median([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
        entry = {"call": label, "ms": round(ms, 4)}
        if kind in ("gemm", "producer"):
            entry["tflops"] = round(units / ms / 1e9, 1)
            entry["frac_mfma_peak"] = round(units / ms / 1e9 / PEAK_MXFP4_TFLOPS, 4)
        elif kind == "nvgemm":
            entry["tflops"] = round(units / ms / 1e9, 1)
            entry["frac_16bit_mfma_peak"] = round(units / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
        else:
            entry["gbps"] = round(units / ms / 1e6, 1)
            entry["frac_hbm_peak"] = round(units / ms / 1e6 / PEAK_HBM_GBPS, 4)
        per.append(entry)

    # quantize+GEMM TFLOP/s per contraction: 2MNK over the contraction's time
    # plus that of the producer calls charged to it
    ms_of = {e["call"]: e["ms"] for e in per}
    contractions = []
    for label, kind, units, _, _ in step.calls:
        if kind not in ("gemm", "producer", "nvgemm"):
            continue
        prod_ms = sum(ms_of[p] for p in step.charge.get(label, []))
        contractions.append({"contraction": label, "tflop": round(units / 1e12, 4), "gemm_ms": ms_of[label],
                             "producers": step.charge.get(label, []), "producer_ms": round(prod_ms, 4),
                             "quantize_gemm_tflops": round(units / ((ms_of[label] + prod_ms) * 1e-3) / 1e12, 1)})
    flops = step.gemm_flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_ms = sum(e["ms"] for e, c in zip(per, step.calls) if c[1] == "gemm")
    gemm_flops = sum(c[2] for c in step.calls if c[1] == "gemm")
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else 0.0
    n_gemm = sum(1 for c in step.calls if c[1] == "gemm")
    gemm_alg_bytes = sum(c[4] for c in step.calls if c[1] == "gemm")
    q_bytes = sum(c[2] for c in step.calls if c[1] == "quant")
    q_ms = sum(e["ms"] for e, c in zip(per, step.calls) if c[1] == "quant")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1/e8m0 operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": args.workload, "gemm_tflop_per_step": round(flops / 1e12, 3),
                   "swiglu_backward": ("unfused" if (args.unfused_backward or step.nvfp4_dgrad) else
                                       "in the W2 Dgrad epilogue" if step.dgrad_epilogue else "fused producer"),
                   "dgrad": "CTA-local NVFP4 (operand-wise hybrid)" if step.nvfp4_dgrad else "MXFP4",
                   "launch": mode,
                   "quantizer_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1) if q_ms > 0 else None,
                   "quantizer_frac_hbm_peak": round(q_bytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4) if q_ms > 0 else None},
        "roofline": {"bound": "mfma", "kernel": "gemm_fast_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_MXFP4_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MXFP4_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload, n_gemm),
                     "algorithmic_bytes_per_launch": round(gemm_alg_bytes / max(1, n_gemm)),
                     "launches_per_step": n_gemm},
        "breakdown": per,
        "contractions": contractions,
    }
    if step.nvfp4_dgrad:
        out["cpu_baseline"] = None                         # the oracle step is the MXFP4 one: see --nvfp4-dgrad
    elif not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(step)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
