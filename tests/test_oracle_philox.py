"""Pins of the oracle's Philox4x32-10 and noise maps against published vectors, an
independent library implementation (rocRAND, run here) and distributional facts."""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat():
    out = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            out.append((w[:4], w[4:6], w[6:10]))
    return out


def test_known_answer_vectors():
    for ctr, key, expect in _kat():
        got = philox.philox4x32_10(*ctr, *key)
        assert [int(g) for g in got] == expect


def test_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(5)
    words = rng.integers(0, 2 ** 32, size=(50, 6), dtype=np.uint64)
    vec = philox.philox4x32_10(*[words[:, i] for i in range(6)])
    for j in range(50):
        one = philox.philox4x32_10(*[int(words[j, i]) for i in range(6)])
        assert [int(x) for x in one] == [int(v[j]) for v in vec]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_against_rocrand(tmp_path):
    """rocRAND's open-source philox4x32_10 engine, compiled and run on chosen inputs."""
    exe = tmp_path / "rr"
    src = os.path.join(HERE, "golden", "rocrand_philox_ref.cpp")
    subprocess.run(["hipcc", "-O1", "-x", "hip", "--offload-arch=gfx950", "-o", str(exe), src],
                   check=True, capture_output=True, timeout=300)
    rng = np.random.default_rng(11)
    inp = rng.integers(0, 2 ** 32, size=(200, 6), dtype=np.uint64)
    # include the stream layouts actually used by the sampler
    inp[0] = [7, 3, 2, philox.TAG_GUMBEL, 0x1234, 0]
    inp[1] = [0, 255, 9, philox.TAG_RENOISE, 0xFFFFFFFF, 0xFFFFFFFF]
    inp[2] = [0, 16383, 0, philox.TAG_QSAMPLE, 0, 0]
    text = "\n".join(" ".join("%x" % int(v) for v in row) for row in inp) + "\n"
    res = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True)
    ref = np.array([[int(x, 16) for x in line.split()] for line in res.stdout.strip().splitlines()],
                   dtype=np.uint64)
    got = np.stack(philox.philox4x32_10(*[inp[:, i] for i in range(6)]), axis=1).astype(np.uint64)
    assert np.array_equal(ref, got)


def test_uniform_map_bounds_and_exactness():
    x = np.array([0, 511, 512, 2 ** 32 - 1], dtype=np.uint64).astype(np.uint32)
    u = philox.uniform01(x)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[2] == 1.5 * 2.0 ** -23
    assert u[3] == 1.0 - 2.0 ** -24
    # every value is representable in fp32
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_gumbel_noise_distribution():
    """g = -ln(-ln u) is standard Gumbel: KS test, mean = Euler-Mascheroni, var = pi^2/6."""
    g = np.concatenate([philox.gumbel_noise(r, 4096, seed=3, step=1) for r in range(64)])
    assert g.size == 64 * 4096
    ks = stats.kstest(g, stats.gumbel_r.cdf)
    assert ks.pvalue > 1e-4
    se = math.sqrt(math.pi ** 2 / 6 / g.size)
    assert abs(g.mean() - 0.5772156649015329) < 5 * se
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05
    # support of the 23-bit uniform map
    assert g.min() >= -math.log(-math.log(2.0 ** -24)) - 1e-12
    assert g.max() <= -math.log(-math.log(1 - 2.0 ** -24)) + 1e-9


def test_gumbel_words_layout():
    """word v of a row is word (v & 3) of the block with counter (v >> 2, row, step, tag)."""
    w = philox.gumbel_words(row=5, V=10, seed=0x0000000200000001, step=3)
    for v in range(10):
        blk = philox.philox4x32_10(v >> 2, 5, 3, philox.TAG_GUMBEL, 1, 2)
        assert int(w[v]) == int(blk[v & 3])


def test_uniform_token_power_of_two_is_exact_and_uniform():
    rng = np.random.default_rng(2)
    x = rng.integers(0, 2 ** 32, size=100000, dtype=np.uint64).astype(np.uint32)
    t = philox.uniform_token(x, 2 ** 18)
    assert np.array_equal(t, (x >> np.uint32(14)).astype(np.int64))
    rows = np.arange(200000)
    tok = philox.renoise_tokens(rows, 16, seed=9, step=0)
    counts = np.bincount(tok, minlength=16)
    assert stats.chisquare(counts).pvalue > 1e-4
    tok = philox.renoise_tokens(rows, 50257, seed=9, step=4)
    assert tok.min() >= 0 and tok.max() < 50257
    assert stats.chisquare(np.bincount(tok % 97, minlength=97)).pvalue > 1e-4
