"""Pin of the oracle's Philox4x32-10 (and its counter layout) against an
independent implementation of the same published generator: rocRAND's
host-callable engine, compiled here from its open-source header.

The pages fix only that stochastic rounding draws from a seed and a counter
offset ("Format-Aware Fusion for Fast FP4 Pretraining", App. A.1); the
generator is Philox4x32-10 of Salmon et al. (SC'11), with the element's
row-major index addressing the counter and the SR offset selecting a disjoint
counter range.  rocRAND's engine seeded with (seed, subsequence, offset) yields
exactly that word when subsequence is the SR offset and offset the element
index, so every draw, and the H32 sign mask (word 0 at counter 0), is checked
against it on seeds, offsets and indices chosen to carry across the 32-bit
halves of the key and counter.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox as P

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_ref", "rocrand_philox_draws.cpp")
HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


@pytest.fixture(scope="module")
def rocrand_draws(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not (os.path.exists(hipcc) and os.path.exists(HEADER)):
        pytest.skip("rocRAND header or hipcc not installed")
    exe = str(tmp_path_factory.mktemp("philox_ref") / "rocrand_philox_draws")
    subprocess.run([hipcc, "-O1", "-o", exe, SRC], check=True, capture_output=True)

    def run(triples):
        text = "".join(f"{s} {q} {o}\n" for s, q, o in triples)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [int(v) for v in out.split()]
    return run


def _triples():
    rng = np.random.default_rng(2026)
    seeds = [0, 1, 7, 0xFFFFFFFF, 1 << 32, 2 ** 35 + 11, 2 ** 64 - 1] + \
        [int(v) for v in rng.integers(0, 2 ** 63, size=5, dtype=np.int64)]
    subs = [0, 1, 2, 5, 0xFFFFFFFF, 1 << 32, 2 ** 33 + 9, 2 ** 64 - 1] + \
        [int(v) for v in rng.integers(0, 2 ** 63, size=3, dtype=np.int64)]
    idx = list(range(9)) + [4 * 0xFFFFFFFF + 3, 4 * (1 << 32), 4 * (1 << 32) + 2, 8192 * 14336 - 1,
                            32768 * 28672 - 5] + [int(v) for v in rng.integers(0, 2 ** 62, size=4, dtype=np.int64)]
    out = []
    for s in seeds:
        for q in subs:
            for i in (idx if (s, q) in ((0, 0), (2 ** 35 + 11, 5)) else idx[::3]):
                out.append((s, q, i))
    return out


def test_draws_match_rocrand_philox(rocrand_draws):
    triples = _triples()
    want = rocrand_draws(triples)
    got = [int(P.draws(s, q, np.array([i], dtype=np.uint64))[0]) for s, q, i in triples]
    bad = [(t, g, w) for t, g, w in zip(triples, got, want) if g != w]
    assert not bad, f"{len(bad)} of {len(triples)} draws differ, first: {bad[:3]}"
    assert len(triples) > 500


def test_sign_mask_matches_rocrand_word0(rocrand_draws):
    seeds = [0, 1, 3, 7, 12345, 2 ** 32 + 1, 2 ** 63 + 5]
    want = rocrand_draws([(s, 0, 0) for s in seeds])
    assert [P.sign_mask_from_seed(s) for s in seeds] == [w & 0xFFFF for w in want]
