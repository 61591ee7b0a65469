"""Pins of the oracle's sampled and rounding helpers (CPU only).

The full-size GPU parity tests take their expected values from three helpers that sample or
round what the pinned oracle steps compute: `normals_at` (normals at chosen draw/token/channel
triples), `head_ce_at` (the perturbed chunk cross-entropy at chosen draw/token pairs) and
`round_bf16` (nearest bfloat16, ties to even). Each is pinned here to something other than
itself:
  - round_bf16: torch's float32 -> bfloat16 conversion (round to nearest even) on fp32 values,
    and an exhaustive nearest-value search over every bfloat16 bit pattern (the format's
    definition: 1 sign, 8 exponent, 7 fraction bits) on fp64 values, with exact ties,
    subnormals and the overflow edge constructed explicitly;
  - normals_at: element-for-element equal to slices of the bulk `normals` (pinned by the
    generator tests) under non-zero draw, token and channel offsets, channels beyond 2^32;
  - head_ce_at: torch.nn.functional.cross_entropy (fp64) of explicitly perturbed logits
    (explainer, "The real work", third measure: only the chunk's logits move, the loss is over
    the whole vocabulary), with targets inside, at the edges of and outside the chunk.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

# ------------------------------------------------------------------------------ round_bf16


def _bf16_positive_table():
    """Every finite non-negative bfloat16 value, indexed by its bit pattern 0x0000..0x7F7F."""
    bits = np.arange(0x7F80, dtype=np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


_BF16 = _bf16_positive_table()
_TWO128 = Fraction(2) ** 128           # the value pattern 0x7F80 (infinity) would take


def _nearest_even_exhaustive(x: float) -> float:
    """Nearest bfloat16 of x by search over the bit patterns, ties to the even pattern; a
    magnitude that rounds to pattern 0x7F80 is infinite."""
    if x == 0.0 or np.isnan(x) or np.isinf(x):
        return x
    ax = Fraction(abs(x))
    i = int(np.searchsorted(_BF16, abs(x), side="right")) - 1      # _BF16[i] <= |x|
    lo = Fraction(float(_BF16[i]))
    hi = Fraction(float(_BF16[i + 1])) if i + 1 < len(_BF16) else _TWO128
    dlo, dhi = ax - lo, hi - ax
    if dlo < dhi or (dlo == dhi and i % 2 == 0):
        pick = i
    else:
        pick = i + 1
    v = np.inf if pick == len(_BF16) else float(_BF16[pick])
    return -v if x < 0 else v


def _ties_and_edges() -> np.ndarray:
    g = np.random.default_rng(71)
    pats = np.concatenate([np.arange(0, 0x90), g.integers(0x80, 0x7F7F, 400),
                           np.arange(0x7F70, 0x7F7F)])
    vals = []
    for p in pats:
        a = float(_BF16[p])
        b = float(_BF16[p + 1]) if p + 1 < len(_BF16) else 2.0 ** 128
        mid = (a + b) / 2                            # exact in fp64 (8-bit significands)
        vals += [a, mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf),
                 a + (b - a) * 0.25, a + (b - a) * 0.75]
    vals += [2.0 ** -134, np.nextafter(2.0 ** -134, 1.0), np.nextafter(2.0 ** -134, 0.0),
             2.0 ** -140, 2.0 ** -126, np.nextafter(2.0 ** -126, 0.0), 5e-324,
             float(_BF16[-1]), (float(_BF16[-1]) + 2.0 ** 128) / 2, 2.0 ** 128, 1e300]
    vals = np.array(vals, dtype=np.float64)
    return np.concatenate([vals, -vals])


def test_round_bf16_equals_exhaustive_nearest_even_on_ties_subnormals_and_overflow():
    x = _ties_and_edges()
    got = oracle.round_bf16(x)
    ref = np.array([_nearest_even_exhaustive(v) for v in x])
    np.testing.assert_array_equal(got, ref)
    # the constructed ties went both ways (to the even neighbour, up and down)
    assert np.sum(np.abs(got) > np.abs(x)) > 50 and np.sum(np.abs(got) < np.abs(x)) > 50


def test_round_bf16_equals_exhaustive_search_on_random_fp64():
    g = np.random.default_rng(72)
    x = g.standard_normal(3000) * np.exp2(g.integers(-140, 128, 3000).astype(np.float64))
    got = oracle.round_bf16(x)
    ref = np.array([_nearest_even_exhaustive(v) for v in x])
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_equals_torch_on_fp32_values():
    g = np.random.default_rng(73)
    bits = np.concatenate([g.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32),
                           # exact ties: low 16 bits 0x8000, both parities of bit 16
                           (g.integers(0, 2**16, 2000).astype(np.uint32) << 16) | 0x8000,
                           np.arange(0, 0x20000, 7, dtype=np.uint32)])     # subnormals
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(f.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------------------------ normals_at


@pytest.mark.parametrize("draw0,tok0,chan0", [(0, 0, 0), (5, 1000, 16), (3, 7, 2**32 + 8),
                                              (2**31 + 1, 2**31 - 3, 2**33 - 64)])
def test_normals_at_equals_slices_of_bulk_normals(draw0, tok0, chan0):
    K, T, d = 3, 5, 40
    bulk = oracle.normals(0xA11CE, 9, draw0, tok0, chan0, K, T, d)
    k, t, j = np.meshgrid(np.arange(K), np.arange(T), np.arange(d), indexing="ij")
    got = oracle.normals_at(0xA11CE, 9, k.ravel(), t.ravel(), j.ravel(), draw0=draw0,
                            tok0=tok0, chan0=chan0)
    np.testing.assert_array_equal(got, bulk.ravel())
    # a sampled, unordered subset gives the same values
    g = np.random.default_rng(74)
    pick = g.choice(K * T * d, 50, replace=False)
    got2 = oracle.normals_at(0xA11CE, 9, k.ravel()[pick], t.ravel()[pick], j.ravel()[pick],
                             draw0=draw0, tok0=tok0, chan0=chan0)
    np.testing.assert_array_equal(got2, bulk.ravel()[pick])


# ------------------------------------------------------------------------------ head_ce_at


@pytest.mark.parametrize("V,v0,C", [(64, 12, 20), (97, 88, 9), (40, 0, 40)])
def test_head_ce_at_equals_torch_cross_entropy_of_perturbed_logits(V, v0, C):
    g = np.random.default_rng(75)
    T, K, sigma, draw0, tok0 = 6, 4, 0.3, 9, 17
    z = g.standard_normal((T, V)) * np.sqrt(2)
    tgt = g.integers(0, V, T).astype(np.int32)
    tgt[0] = v0                         # first id of the chunk
    tgt[1] = v0 + C - 1                 # last id of the chunk
    tgt[2] = (v0 + C) % V               # just past it (or wrapped to 0)
    tgt[3] = (v0 - 1) % V               # just before it
    k, t = np.meshgrid(np.arange(K), np.arange(T), indexing="ij")
    got = oracle.head_ce_at(z, tgt, v0, C, k.ravel(), t.ravel(), sigma, seed=6, tag=2,
                            draw0=draw0, tok0=tok0).reshape(K, T)
    a = oracle.normals(6, 2, draw0, tok0, v0, K, T, C)
    zp = np.repeat(z[None], K, axis=0)
    zp[:, :, v0:v0 + C] += sigma * a
    ref = torch.nn.functional.cross_entropy(torch.tensor(zp.reshape(K * T, V)),
                                            torch.tensor(np.tile(tgt, K)).long(),
                                            reduction="none").numpy().reshape(K, T)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    lp, _ = oracle.head_ce_chunk(z, tgt, v0, C, K, sigma, seed=6, tag=2, draw0=draw0, tok0=tok0)
    np.testing.assert_allclose(got, lp, rtol=0, atol=1e-12)
