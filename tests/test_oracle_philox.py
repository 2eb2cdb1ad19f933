"""Pins of the oracle's Philox4x32-10 and the draws derived from it.

The oracle's generator is checked against rocRAND's Philox4x32-10 engine (an
independent implementation of the same published algorithm, built here from
its header with g++), plus statistical and closed-form properties of the
derived uniforms, Gumbel draws and uniform ids."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.philox import (philox4x32_10, uniform24, gumbel_from_word,
                           uniform_id, gumbel_row, canvas_id, renoise_id)

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    cxx = shutil.which("g++")
    if cxx is None or not os.path.exists(hdr):
        pytest.skip("g++ or rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("ph") / "ph_ref")
    subprocess.run([cxx, "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp"),
                    "-o", exe], check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(123)
    n = 20000
    c0 = rng.integers(0, 2**32, n, dtype=np.uint64)
    c1 = rng.integers(0, 2**30, n, dtype=np.uint64)
    c2 = rng.integers(0, 2**32, n, dtype=np.uint64)
    c3 = rng.integers(0, 2**32, n, dtype=np.uint64)
    seed = rng.integers(0, 2**63, n, dtype=np.uint64)
    # edge counters and keys
    c0[:4] = [0, 0xFFFFFFFF, 0, 1]
    c1[:4] = [0, 2**30 - 1, 0, 0]
    c2[:4] = [0, 0xFFFFFFFF, 0, 0]
    c3[:4] = [0, 0xFFFFFFFF, (2 << 24) | 3, 0]
    seed[:4] = [0, 2**63 - 1, 0, 0xFFFFFFFF]
    lines = "\n".join(f"{a} {b} {c} {d} {s}" for a, b, c, d, s in
                      zip(c0, c1, c2, c3, seed)) + "\n"
    out = subprocess.run([rocrand_ref], input=lines, capture_output=True,
                         text=True, check=True).stdout.split()
    ref = np.array(out, dtype=np.uint64).reshape(n, 4)
    for i in range(n):
        got = philox4x32_10(c0[i], c1[i], c2[i], c3[i], int(seed[i]))
        assert tuple(int(x) for x in got) == tuple(int(x) for x in ref[i]), i
        if i > 2000:
            break
    # the vectorized path on the whole batch must agree too (same seed only)
    s0 = int(seed[10])
    got = np.stack(philox4x32_10(c0, c1, c2, c3, s0), axis=1)
    lines = "\n".join(f"{a} {b} {c} {d} {s0}" for a, b, c, d in
                      zip(c0, c1, c2, c3)) + "\n"
    out = subprocess.run([rocrand_ref], input=lines, capture_output=True,
                         text=True, check=True).stdout.split()
    ref = np.array(out, dtype=np.uint64).reshape(n, 4)
    assert np.array_equal(got.astype(np.uint64), ref)


def test_philox_uniformity():
    words = np.stack(philox4x32_10(np.arange(1 << 16), 7, 3, 0, 42)).reshape(-1)
    counts = np.bincount((words >> 24).astype(np.int64), minlength=256)
    expect = words.size / 256
    chi2 = ((counts - expect) ** 2 / expect).sum()
    # 255 dof: mean 255, sd ~22.6; 6 sd bound
    assert chi2 < 255 + 6 * 22.6
    bits = np.unpackbits(words.view(np.uint8))
    assert abs(bits.mean() - 0.5) < 0.002


def test_uniform24_exact_and_bounds():
    w = np.array([0, 255, 256, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u = uniform24(w)
    assert np.all(u > 0) and np.all(u < 1)
    # exact: u * 2^24 - 0.5 is the integer w >> 8
    assert np.array_equal(u * 2.0**24 - 0.5, (w >> np.uint64(8)).astype(np.float64))
    # u has up to 25 significant bits: float32 holds u exactly below 1/2 and
    # 1 - u exactly above it (what a float32 implementation must use)
    lo = u < 0.5
    assert np.array_equal(u[lo].astype(np.float32).astype(np.float64), u[lo])
    one_minus = 1.0 - u[~lo]
    assert np.array_equal(one_minus.astype(np.float32).astype(np.float64), one_minus)
    g = gumbel_from_word(np.array([0, 0xFFFFFFFF], dtype=np.uint64))
    assert abs(g[0] - (-2.8523629)) < 1e-6
    assert abs(g[1] - 17.3286795) < 1e-6


def test_gumbel_distribution():
    g = gumbel_row(seed=9, pos=3, step=1, row=0, V=1 << 18)
    # standard Gumbel: mean = Euler-Mascheroni, variance = pi^2 / 6
    assert abs(g.mean() - 0.5772157) < 0.01
    assert abs(g.var() - np.pi**2 / 6) < 0.03
    assert g.min() >= -2.853 and g.max() <= 17.329


def test_uniform_id_closed_form():
    rng = np.random.default_rng(1)
    w = rng.integers(0, 2**32, 10000, dtype=np.uint64)
    for V in (512, 262144, 2):
        sh = 32 - int(np.log2(V))
        assert np.array_equal(uniform_id(w, V), (w >> np.uint64(sh)).astype(np.int64))
    ids = uniform_id(w, 1000)          # non power of two: floor(w * V / 2^32)
    assert np.array_equal(ids, np.array([(int(x) * 1000) >> 32 for x in w]))
    assert ids.min() >= 0 and ids.max() < 1000


def test_streams_are_distinct():
    a = canvas_id(0, 5, 0, 512)
    b = renoise_id(0, 5, 0, 0, 512)
    words_c = philox4x32_10(0, 5, 0, (2 << 24), 0)[0]
    words_r = philox4x32_10(0, 5, 0, (1 << 24), 0)[0]
    assert a == int((int(words_c) * 512) >> 32)
    assert b == int((int(words_r) * 512) >> 32)
    assert int(words_c) != int(words_r)
