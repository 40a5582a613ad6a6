"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (the codec's accuracy contract):
  - packed codes bit-exact, except coordinates whose oracle z (double, in
    N(0,1) units) lies within 1e-6 of a decision threshold; there a code may
    differ by exactly 1.  The fraction of such coordinates is reported.
  - norms and decoded values within 1e-3 relative; decoded values are
    compared on identical packed input, against
    1e-3 * max(|ref|, norm/sqrt(d)) so that a coordinate near zero is
    measured against the vector's scale, or one binary16 ulp of the exact
    value where that is coarser (subnormal outputs), and an infinity of the
    right sign where the exact value is past the binary16 range;
  - attention outputs within 2e-3 absolute of the oracle rounded to binary16,
    or within one binary16 ulp where that ulp itself exceeds 2e-3 (|o| >= 4).
"""
from __future__ import annotations

import sys

import numpy as np

D = 128
BAND = 1e-6
NORM_RTOL = 1e-3
DEC_RTOL = 1e-3
ATTN_ATOL = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """LSB-first bitstream -> codes [..., d] (numpy, independent of the oracle)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    d = p.shape[-1] * 8 // bits
    b = np.unpackbits(p, axis=-1, bitorder="little")
    b = b.reshape(p.shape[:-1] + (d, bits)).astype(np.int16)
    return (b << np.arange(bits, dtype=np.int16)).sum(-1)


def compare_codes(gpu_packed, ref_packed, z, thresholds, bits, what=""):
    """Returns (band_fraction, mismatch_fraction); asserts the parity rule."""
    g = unpack_codes(gpu_packed, bits)
    r = unpack_codes(ref_packed, bits)
    t = np.asarray(thresholds, np.float64)
    zz = np.asarray(z, np.float64)
    # distance to the nearest threshold (sorted thresholds, searchsorted)
    idx = np.searchsorted(t, zz)
    lo = np.abs(zz - t[np.clip(idx - 1, 0, len(t) - 1)])
    hi = np.abs(zz - t[np.clip(idx, 0, len(t) - 1)])
    inband = np.minimum(lo, hi) <= BAND
    mism = g != r
    n = g.size
    band_frac = inband.sum() / n
    mism_frac = mism.sum() / n
    log("%s codes: %d coords, in-band %d (%.2e), mismatched %d (%.2e)"
        % (what, n, inband.sum(), band_frac, mism.sum(), mism_frac))
    bad = mism & ~inband
    assert not bad.any(), "%d code mismatches outside the 1e-6 band (first at %s)" % (
        bad.sum(), np.argwhere(bad)[:3].tolist())
    assert np.all(np.abs(g[mism] - r[mism]) == 1), "in-band mismatches must be +-1 code"
    return band_frac, mism_frac


def compare_norms(gpu, ref, what=""):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(g - r)
    tol = NORM_RTOL * np.abs(r)
    rel = np.max(err / np.maximum(np.abs(r), 1e-30)) if r.size else 0.0
    log("%s norms: max rel err %.2e" % (what, rel))
    assert np.all(err <= tol), "norm mismatch beyond 1e-3 relative"


FP16_MAX = 65504.0


def compare_decoded(gpu_f16, ref_f64, norms, what=""):
    """Values past the binary16 range round to +-inf (IEEE overflow); there the
    GPU must give the infinity of the same sign, or a finite value within the
    tolerance when the exact value sits just above 65504."""
    g = np.asarray(gpu_f16).astype(np.float64)
    r = np.asarray(ref_f64, np.float64)
    d = r.shape[-1]
    scale = np.maximum(np.abs(r), np.asarray(norms, np.float64)[..., None] / np.sqrt(d))
    fin = np.isfinite(g)
    err = np.where(fin, np.abs(g - r), 0.0)
    # the output is binary16: one ulp of it is the finest agreement possible
    # (it only matters for subnormal outputs, where an ulp exceeds 1e-3 relative)
    ulp16 = np.spacing(np.minimum(np.abs(r), FP16_MAX).astype(np.float16)).astype(np.float64)
    ok = fin & (err <= np.maximum(DEC_RTOL * scale, ulp16))
    over = ~fin & (np.abs(r) >= FP16_MAX) & (np.sign(g) == np.sign(r))
    worst = float(np.max(err / np.maximum(scale, 1e-30))) if r.size else 0.0
    log("%s decode: max err / max(|ref|, n/sqrt(d)) = %.2e, %d overflowed to inf"
        % (what, worst, int(over.sum())))
    assert np.all(ok | over), "decoded values beyond 1e-3 relative"


def compare_attn(gpu_f16, ref_f64, what=""):
    g = np.asarray(gpu_f16).astype(np.float64)
    r16 = np.asarray(ref_f64, np.float64).astype(np.float16).astype(np.float64)
    err = np.abs(g - r16)
    ulp = np.spacing(np.abs(r16).astype(np.float16)).astype(np.float64)
    big = ulp > ATTN_ATOL
    ok = (err <= ATTN_ATOL) | (big & (err <= ulp))
    log("%s attention: %d outputs, max |err| %.2e, %d outputs with |o| >= 4"
        % (what, g.size, float(err.max()) if g.size else 0.0, int(big.sum())))
    assert ok.all(), "attention outputs beyond 2e-3 (first at %s, err %s)" % (
        np.argwhere(~ok)[:3].tolist(), err[~ok][:3])
