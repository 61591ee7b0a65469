"""Pins of the oracle's noise generator (CPU only).

The pages say only that the noise is standard Gaussian, independent per token and per draw
(Dust explainer, cnblogs.com/32bin/p/23212811, "Credit assignment"). The generator is this
library's definition: Philox4x32-10 words (SC'11) -> Box-Muller. Pins:
  * Philox words equal those of rocRAND's open-source, host-callable Philox4x32-10 engine, an
    implementation the oracle shares nothing with (compiled here from its header, test-only);
  * the words are balanced and uniform; the normals have N(0, 1) moments and distribution, and
    are uncorrelated across channels, tokens, draws, tags and seeds.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
XCHECK_SRC = os.path.join(HERE, "rocrand_philox_xcheck.cpp")


@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc or the rocRAND header is not available")
    exe = str(tmp_path_factory.mktemp("xcheck") / "xcheck")
    subprocess.check_call([hipcc, "-O1", "-o", exe, XCHECK_SRC])

    def run(cases):
        # rocRAND counter = (offset/4 lo, offset/4 hi, subsequence lo, subsequence hi)
        lines = ["%d %d %d" % (seed, draw | (tag << 32), 4 * (q | (token << 32)))
                 for seed, tag, draw, token, q in cases]
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                             check=True).stdout.split("\n")
        return np.array([[int(v) for v in ln.split()] for ln in out if ln.strip()], dtype=np.uint64)

    return run


def _cases(n, seed=11):
    g = np.random.default_rng(seed)
    m32 = 0xFFFFFFFF
    # rocRAND's 64-bit offset is 4x the (q, token) counter pair, so tokens stay below 2^30 here
    t30 = (1 << 30) - 1
    fixed = [(0, 0, 0, 0, 0), (m32 | (m32 << 32), m32, m32, t30, m32), (1, 0, 0, 0, 0),
             (0, 1, 0, 0, 0), (0, 0, 1, 0, 0), (0, 0, 0, 1, 0), (0, 0, 0, 0, 1),
             (0x0D057002, 1, 63, 16383, 511), (1 << 32, 0x100, 16383, 16383, 127)]
    rnd = [(int(g.integers(0, 2**63)) * 2 + int(g.integers(0, 2)), int(g.integers(0, 2**32)),
            int(g.integers(0, 2**32)), int(g.integers(0, 2**30)), int(g.integers(0, 2**32)))
           for _ in range(n)]
    return fixed + rnd


def test_philox_words_match_rocrand(rocrand_words):
    cases = _cases(3000)
    ref = rocrand_words(cases)
    got = np.array([oracle.noise_words(*c) for c in cases], dtype=np.uint64)
    assert got.shape == ref.shape
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, "first mismatch at case %s: %s vs %s" % (cases[bad[0]], got[bad[0]], ref[bad[0]])


def test_counter_layout_is_q_token_draw_tag():
    # counter (q, token, draw, tag), key (seed lo, seed hi)
    seed, tag, draw, token, q = 0x1234567890ABCDEF, 7, 11, 13, 17
    w = oracle.noise_words(seed, tag, draw, token, q)
    direct = oracle.philox4x32_10([q, token, draw, tag], [seed & 0xFFFFFFFF, seed >> 32])
    assert (w == direct).all()


def test_words_are_balanced_and_uniform():
    words = np.array([oracle.noise_words(99, 1, i, t, q) for i in range(2) for t in range(32)
                      for q in range(64)], dtype=np.uint64).ravel()
    assert words.size == 2 * 32 * 64 * 4
    bits = ((words[:, None] >> np.arange(32, dtype=np.uint64)) & 1).mean(axis=0)
    sd = 0.5 / np.sqrt(words.size)
    assert np.all(np.abs(bits - 0.5) < 5 * sd), bits
    hist = np.bincount((words >> np.uint64(24)).astype(np.int64), minlength=256)
    chi2 = ((hist - words.size / 256) ** 2 / (words.size / 256)).sum()
    assert stats.chi2.sf(chi2, 255) > 1e-4


def test_uniform_map_is_exact_and_inside_unit_interval():
    assert oracle.uniform(0) == 2.0 ** -24
    assert oracle.uniform(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert oracle.uniform(511) == 2.0 ** -24          # same 23-bit bin as 0
    assert oracle.uniform(512) == 3 * 2.0 ** -24
    # representable exactly in fp32
    for w in (0, 12345678, 0xFFFFFFFF, 0x80000000):
        u = oracle.uniform(w)
        assert float(np.float32(u)) == u


def test_angle_map_is_exact_left_bin_edge():
    assert oracle.angle(0) == 0.0
    assert oracle.angle(511) == 0.0                    # same 23-bit bin as 0
    assert oracle.angle(512) == 2.0 ** -23
    assert oracle.angle(0xFFFFFFFF) == 1.0 - 2.0 ** -23
    for w in (0, 12345678, 0xFFFFFFFF, 0x80000000):
        v = oracle.angle(w)
        assert float(np.float32(v)) == v and 0.0 <= v < 1.0


def test_box_muller_at_special_angles():
    """Angles 0, 1/4, 1/2 and 3/4 turn put the pair on the axes: one normal of the pair is
    exactly 0 (angle 0) or |.| <= 1e-15 rho, the other is +-rho; rho^2 + 0 = the pair's squared
    norm, the same for every angle."""
    wa = 0x5A5A5A5A
    quarter = 1 << 30             # top 23 bits = 2^21 -> v = 1/4
    rho_c = oracle.box_muller(wa, 0, False)
    assert rho_c > 0 and oracle.box_muller(wa, 0, True) == 0.0
    assert abs(oracle.box_muller(wa, quarter, False)) <= 1e-15 * rho_c
    assert oracle.box_muller(wa, quarter, True) == pytest.approx(rho_c, rel=1e-15)
    assert oracle.box_muller(wa, 2 * quarter, False) == pytest.approx(-rho_c, rel=1e-15)
    assert oracle.box_muller(wa, 3 * quarter, True) == pytest.approx(-rho_c, rel=1e-15)
    for wb in (1 << 9, 12345 << 9, 0xFFFFFFFF):
        c, s = oracle.box_muller(wa, wb, False), oracle.box_muller(wa, wb, True)
        assert c * c + s * s == pytest.approx(rho_c * rho_c, rel=1e-14)


@pytest.fixture(scope="module")
def big_normals():
    return oracle.normals(0xBEEF, 1, 0, 0, 0, 8, 1024, 512)   # 4.2M normals [K, T, d]


def test_normal_moments(big_normals):
    n = big_normals.ravel()
    N = n.size
    assert abs(n.mean()) < 5 / np.sqrt(N)
    assert abs(n.var() - 1) < 5 * np.sqrt(2 / N)
    assert abs(stats.skew(n)) < 5 * np.sqrt(6 / N)
    assert abs(stats.kurtosis(n)) < 5 * np.sqrt(24 / N)
    # tails are truncated at sqrt(-2 ln 2^-24)
    assert np.abs(n).max() <= np.sqrt(-2 * np.log(2.0 ** -24)) + 1e-12


def test_normal_distribution_ks(big_normals):
    sample = big_normals.ravel()[::7][:500000]
    assert stats.kstest(sample, "norm").pvalue > 1e-4


def test_normals_uncorrelated_across_indices(big_normals):
    n = big_normals
    N = n[:, :, 0::2].size
    lim = 5 / np.sqrt(N)
    pairs = {
        "channel pair (Box-Muller cos/sin)": (n[:, :, 0::2], n[:, :, 1::2]),
        "adjacent channel groups": (n[:, :, 0:256], n[:, :, 256:512]),
        "adjacent tokens": (n[:, 0::2, :], n[:, 1::2, :]),
        "adjacent draws": (n[0::2], n[1::2]),
    }
    for name, (a, b) in pairs.items():
        r = np.corrcoef(a.ravel(), b.ravel())[0, 1]
        assert abs(r) < 5 / np.sqrt(a.size), (name, r, lim)
    # squared values too (Box-Muller pairs share a radius, which must not correlate |n|
    # beyond what independence allows)
    a, b = n[:, :, 0::2].ravel(), n[:, :, 1::2].ravel()
    r2 = np.corrcoef(a * a, b * b)[0, 1]
    assert abs(r2) < 5 / np.sqrt(a.size)


def test_tag_and_seed_give_independent_streams():
    a = oracle.normals(1, 1, 0, 0, 0, 4, 256, 256).ravel()
    b = oracle.normals(1, 2, 0, 0, 0, 4, 256, 256).ravel()
    c = oracle.normals(2, 1, 0, 0, 0, 4, 256, 256).ravel()
    lim = 5 / np.sqrt(a.size)
    assert abs(np.corrcoef(a, b)[0, 1]) < lim
    assert abs(np.corrcoef(a, c)[0, 1]) < lim


def test_global_indices_make_noise_split_invariant():
    full = oracle.normals(77, 5, 0, 0, 0, 6, 20, 40)
    part = oracle.normals(77, 5, 2, 3, 8, 3, 10, 20)   # draws 2..4, tokens 3..12, channels 8..27
    assert np.array_equal(part, full[2:5, 3:13, 8:28])


def test_golden_fixture_unchanged():
    """Regression pin: the oracle still produces the words and normals stored by
    tests/golden/make_golden.py."""
    path = os.path.join(HERE, "golden", "oracle_noise.txt")
    for line in open(path):
        if line.startswith("#"):
            continue
        head, words, norms = line.split("|")
        seed, tag, draw, token, q = (int(v) for v in head.split())
        assert [int(v) for v in words.split()] == list(oracle.noise_words(seed, tag, draw, token, q))
        ref = [float(v) for v in norms.split()]
        got = [oracle.normal(seed, tag, draw, token, 4 * q + e) for e in range(4)]
        assert np.allclose(got, ref, rtol=1e-15, atol=1e-15)
