"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module holds no arithmetic of the method: it draws float32 samples with
numpy's PCG64 and rounds them to bf16 bit patterns.  Each workload has one
SeedSequence; every tensor is drawn from its own spawned child stream in a fixed
order, so a tensor's values do not depend on which other tensors are drawn, and
each tensor is drawn in row chunks from further spawned streams.

Workloads stand in for the Llama-3-8B training tensors of "Format-Aware Fusion
for Fast FP4 Pretraining" (§4.1: hidden 4096, FFN 14336, 8192-token sequences),
whose data are not available.  "N(0, s)" reads s as the standard deviation.
Outliers: a Bernoulli mask of the stated rate, drawn after the values from the
same child stream, multiplies the selected entries by the stated factor.
"""

import os

import numpy as np

__all__ = ["bf16_bits", "draw", "WORKLOADS", "workload", "tensor"]


def bf16_bits(x):
    """float32 -> bf16 bit patterns (round to nearest even) as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


CHUNK_ROWS = 512


def _draw_chunk(ss, rows, C, law, std, outlier_rate, outlier_scale):
    rng = np.random.Generator(np.random.PCG64(ss))
    if law == "normal":
        v = rng.standard_normal((rows, C), dtype=np.float32)
    elif law == "student_t3":
        v = (rng.standard_t(3.0, size=(rows, C)) / np.sqrt(3.0)).astype(np.float32)
    else:
        raise ValueError(law)
    v *= np.float32(std)
    if outlier_rate > 0.0:
        v[rng.random((rows, C)) < outlier_rate] *= np.float32(outlier_scale)
    return bf16_bits(v)


def draw(ss, shape, law, std, outlier_rate=0.0, outlier_scale=1.0):
    """Draw a bf16 tensor [R][C] from `law` ('normal' or 'student_t3') with the
    given standard deviation and optional Bernoulli outliers.

    The rows are cut into chunks of CHUNK_ROWS; chunk j draws from the j-th
    child of `ss` (values first, then the outlier mask), so chunks are drawn in
    parallel and any chunk can be regenerated alone."""
    from concurrent.futures import ThreadPoolExecutor
    R, C = shape
    out = np.empty((R, C), dtype=np.uint16)
    starts = list(range(0, R, CHUNK_ROWS))
    children = ss.spawn(len(starts))

    def one(j):
        r0 = starts[j]
        r1 = min(R, r0 + CHUNK_ROWS)
        out[r0:r1] = _draw_chunk(children[j], r1 - r0, C, law, std, outlier_rate, outlier_scale)

    workers = max(1, min(16, os.cpu_count() or 1, len(starts)))
    if workers == 1:
        for j in range(len(starts)):
            one(j)
    else:
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(one, range(len(starts))))
    return out


# Tensor recipes per workload, in generation order:
# name -> (rows, cols, law, std, outlier_rate, outlier_scale)
def _recipes(T, D, F, law_x="normal", std_w=0.02, std_dy=1e-3, dy_out=(0.0, 1.0), x_out=(0.0, 1.0)):
    return {
        "X": (T, D, law_x, 1.0) + x_out,
        "W1": (F, D, "normal", std_w, 0.0, 1.0),
        "W3": (F, D, "normal", std_w, 0.0, 1.0),
        "W2": (D, F, "normal", std_w, 0.0, 1.0),
        "dY": (T, D, "normal", std_dy) + dy_out,
    }


WORKLOADS = {
    # Single Fprop linear: X 256x512 ~N(0,1), W 512x512 ~N(0,0.02), RTN, 1x32 blocks.
    "fprop_256x512x512": dict(seed=0, tensors={
        "X": (256, 512, "normal", 1.0, 0.0, 1.0),
        "W": (512, 512, "normal", 0.02, 0.0, 1.0)}),
    # Llama-3-8B attention projection, Fprop + Dgrad.
    "attn_proj_8192x4096x4096": dict(seed=0, tensors={
        "X": (8192, 4096, "normal", 1.0, 0.001, 20.0),
        "W": (4096, 4096, "normal", 0.02, 0.0, 1.0),
        "dY": (8192, 4096, "normal", 1e-3, 0.0, 1.0)}),
    # Wgrad with paired H32 along the 8192-token axis.
    "wgrad_h32_8192x14336x4096": dict(seed=0, tensors={
        "dY": (8192, 14336, "normal", 1e-3, 0.0, 1.0),
        "X": (8192, 4096, "normal", 1.0, 0.0, 1.0)}),
    # Full Llama-3-8B SwiGLU FFN step: T 8192, D 4096, F 14336.
    "ffn_step_8192x4096x14336": dict(seed=0, tensors=_recipes(8192, 4096, 14336)),
    # Large heavy-tailed FFN: T 32768, D 8192, F 28672.
    "ffn_large_32768x8192x28672": dict(seed=0, tensors=_recipes(
        32768, 8192, 28672, law_x="student_t3", std_w=0.015, std_dy=1e-4, dy_out=(0.01, 50.0))),
}


def workload(name, seed=None, shapes=None):
    """Return {tensor name: bf16 bits} for a workload.

    `shapes` may override (rows, cols) per tensor to draw a smaller instance of
    the same laws (used by parity tests); `seed` overrides the workload seed.
    """
    spec = WORKLOADS[name]
    seed = spec["seed"] if seed is None else seed
    names = list(spec["tensors"])
    children = np.random.SeedSequence(seed).spawn(len(names))
    out = {}
    for nm, ss in zip(names, children):
        R, C, law, std, rate, scale = spec["tensors"][nm]
        if shapes and nm in shapes:
            R, C = shapes[nm]
        out[nm] = draw(ss, (R, C), law, std, rate, scale)
    return out


def tensor(shape, law="normal", std=1.0, seed=0, outlier_rate=0.0, outlier_scale=1.0):
    """One standalone bf16 tensor (for tests of single calls)."""
    return draw(np.random.SeedSequence(seed), shape, law, std, outlier_rate, outlier_scale)
