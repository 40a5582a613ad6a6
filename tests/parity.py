"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (the codec's accuracy contract):
  - packed codes bit-exact, except coordinates whose oracle z (double, in
    N(0,1) units) lies within 1e-6 of a decision threshold; there a code may
    differ by exactly 1.  The fraction of such coordinates is reported per
    case, and pooled over the random-data cases of a run it must stay at or
    below 1e-5 (``pooled_band_fraction``).
  - norms within 1e-3 relative.
  - decoded values, compared on identical packed input, are the binary16
    round-to-nearest-even (RNE) of a value within delta of the exact decode:
    the GPU's binary16 g must satisfy RNE(ref - delta) <= g <= RNE(ref + delta),
    where delta bounds the kernel's f32 arithmetic (``decode_delta``).  Away
    from a rounding midpoint that is bit equality with the oracle's RNE
    binary16; a round-toward-zero or other wrong rounding fails.  On top of
    that the values must lie within 1e-3 * max(|ref|, norm/sqrt(d)), or one
    binary16 ulp of ref where that is coarser (subnormal outputs), or be the
    infinity of ref's sign past the binary16 range.
  - attention outputs within 2e-3 absolute of the oracle rounded to binary16,
    or within one binary16 ulp where that ulp itself exceeds 2e-3 (|o| >= 4).
    Where the caller can bound the kernel's f32 error (a context of one token,
    whose softmax weight is exactly 1), the same RNE rule as for decode is
    applied on top (``single_token_delta``).
"""
from __future__ import annotations

import sys

import numpy as np

D = 128
BAND = 1e-6
BAND_POOLED_MAX = 1e-5
NORM_RTOL = 1e-3
DEC_RTOL = 1e-3
ATTN_ATOL = 2e-3
U32 = 2.0 ** -24            # unit roundoff of f32 (round to nearest)

# in-band and total coordinates of the random-data codec cases of this run
_POOL = {"inband": 0, "coords": 0, "cases": 0}


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


def in_band(z, thresholds) -> np.ndarray:
    """Coordinates whose z lies within BAND of a decision threshold."""
    t = np.asarray(thresholds, np.float64)
    zz = np.asarray(z, np.float64)
    idx = np.searchsorted(t, zz)
    lo = np.abs(zz - t[np.clip(idx - 1, 0, len(t) - 1)])
    hi = np.abs(zz - t[np.clip(idx, 0, len(t) - 1)])
    return np.minimum(lo, hi) <= BAND


def compare_codes(gpu_packed, ref_packed, z, thresholds, bits, what="", pooled=True):
    """Returns (band_fraction, mismatch_fraction); asserts the parity rule.
    ``pooled`` adds the case to the run's pooled band count (random data; the
    hand-built special vectors sit on thresholds on purpose and are left out)."""
    g = unpack_codes(gpu_packed, bits)
    r = unpack_codes(ref_packed, bits)
    inband = in_band(z, thresholds)
    mism = g != r
    n = g.size
    band_frac = inband.sum() / n if n else 0.0
    mism_frac = mism.sum() / n if n else 0.0
    log("%s codes: %d coords, in-band %d (%.2e), mismatched %d (%.2e)"
        % (what, n, inband.sum(), band_frac, mism.sum(), mism_frac))
    bad = mism & ~inband
    assert not bad.any(), "%d code mismatches outside the 1e-6 band (first at %s)" % (
        bad.sum(), np.argwhere(bad)[:3].tolist())
    assert np.all(np.abs(g[mism] - r[mism]) == 1), "in-band mismatches must be +-1 code"
    if pooled:
        _POOL["inband"] += int(inband.sum())
        _POOL["coords"] += int(n)
        _POOL["cases"] += 1
    return band_frac, mism_frac


def pooled_band_fraction():
    """(in-band coordinates, coordinates, cases) pooled over this run."""
    return _POOL["inband"], _POOL["coords"], _POOL["cases"]


def reset_pool():
    _POOL.update(inband=0, coords=0, cases=0)


def compare_norms(gpu, ref, what=""):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(g - r)
    tol = NORM_RTOL * np.abs(r)
    rel = np.max(err / np.maximum(np.abs(r), 1e-30)) if r.size else 0.0
    log("%s norms: max rel err %.2e" % (what, rel))
    assert np.all(err <= tol), "norm mismatch beyond 1e-3 relative"


FP16_MAX = 65504.0


def rne16(x) -> np.ndarray:
    """binary16 round-to-nearest-even of float64 values (numpy converts
    double to half with one correct rounding; past 65520 it gives inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float64).astype(np.float16)


def decode_delta(packed, norms, levels, bits, d) -> np.ndarray:
    """Bound on |decode kernel's f32 value - exact decode| per vector [n, 1].

    The kernel sums +-c[code_i] through log2(d) butterfly stages in f32 (the
    first one or two inside its lookup table), multiplies by n/d inside the
    last stage (one extra rounding) and uses f32 levels (one rounding of the
    level).  Every partial sum is bounded by sum_i |c_i|, so each of these
    roundings adds at most 2^-24 * (n/d) * sum_i |c[code_i]|; the bound takes
    log2(d) + 4 of them."""
    codes = unpack_codes(packed, bits)
    c = np.asarray(levels, np.float64)
    s1 = np.abs(c[codes]).sum(-1)
    n = np.asarray(norms, np.float64)
    k = np.log2(d) + 4
    return (k * U32 * n * s1 / d)[..., None]


def single_token_delta(v_packed_rows, v_norms_rows, levels, bits, d) -> np.ndarray:
    """Bound on |attention kernel's f32 output - exact output| when the context
    is one token (weight exactly 1, so the output is that token's value).

    The value weight n*2^k is split into a truncated binary16 high part and a
    rounded low part (residual <= 2^-21 relative), the level 16c into two
    rounded binary16 parts (<= 2^-22), the low*low product is dropped
    (<= 2^-21); the matrix product adds 2 roundings, the f32 level 1 and the
    inverse transform log2(d) more.  2.5 * 2^-21 + (log2(d) + 3) * 2^-24 is
    below 2^-18 for d <= 256, which is the factor used (per row [n, 1])."""
    codes = unpack_codes(v_packed_rows, bits)
    c = np.asarray(levels, np.float64)
    s1 = np.abs(c[codes]).sum(-1)
    n = np.asarray(v_norms_rows, np.float64)
    return (2.0 ** -18 * n * s1 / d)[..., None]


def rounding_check(g16, ref, delta):
    """Boolean array: g16 is the RNE binary16 of some value within delta of ref.
    RNE is monotone, so that is RNE(ref - delta) <= g <= RNE(ref + delta)."""
    g = np.asarray(g16, np.float16).astype(np.float64)
    r = np.asarray(ref, np.float64)
    dl = np.broadcast_to(np.asarray(delta, np.float64), r.shape)
    lo = rne16(r - dl).astype(np.float64)
    hi = rne16(r + dl).astype(np.float64)
    return (lo <= g) & (g <= hi)


def compare_decoded(gpu_f16, ref_f64, norms, what="", packed=None, levels=None, bits=None):
    """Decode parity.  With (packed, levels, bits) the RNE rule applies: the GPU
    value must be the RNE binary16 of a value within decode_delta of ref.
    Values past the binary16 range round to +-inf (IEEE overflow)."""
    g16 = np.asarray(gpu_f16, np.float16)
    g = g16.astype(np.float64)
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
    msg = "%s decode: max err / max(|ref|, n/sqrt(d)) = %.2e, %d overflowed to inf" % (
        what, worst, int(over.sum()))
    rne_ok = np.ones(r.shape, bool)
    if packed is not None:
        delta = decode_delta(packed, norms, levels, bits, d)
        rne_ok = rounding_check(g16, r, delta)
        differ = (g != rne16(r).astype(np.float64))
        msg += ", %d of %d differ from RNE(oracle) (all inside the f32 bound)" % (
            int(differ.sum()), r.size) if rne_ok.all() else ""
    log(msg)
    assert np.all(ok | over), "decoded values beyond 1e-3 relative"
    assert rne_ok.all(), "decoded values not the RNE binary16 of the kernel's bounded f32 " \
        "value (first at %s: gpu %s, exact %s)" % (
            np.argwhere(~rne_ok)[:3].tolist(), g[~rne_ok][:3], r[~rne_ok][:3])


def compare_attn(gpu_f16, ref_f64, what="", delta=None):
    """Attention parity: 2e-3 absolute against RNE(oracle), or one binary16
    ulp where that ulp exceeds 2e-3; with ``delta`` (a bound on the kernel's
    f32 error) the RNE rule of compare_decoded applies as well."""
    g16 = np.asarray(gpu_f16, np.float16)
    g = g16.astype(np.float64)
    r = np.asarray(ref_f64, np.float64)
    r16 = rne16(r).astype(np.float64)
    err = np.abs(g - r16)
    ulp = np.spacing(np.abs(r16).astype(np.float16)).astype(np.float64)
    big = ulp > ATTN_ATOL
    ok = (err <= ATTN_ATOL) | (big & (err <= ulp))
    differ = int((g != r16).sum())
    log("%s attention: %d outputs, max |err| %.2e, %d outputs with |o| >= 4, %d differ "
        "from RNE(oracle)" % (what, g.size, float(err.max()) if g.size else 0.0,
                              int(big.sum()), differ))
    assert ok.all(), "attention outputs beyond 2e-3 (first at %s, err %s)" % (
        np.argwhere(~ok)[:3].tolist(), err[~ok][:3])
    if delta is not None:
        rne_ok = rounding_check(g16, r, delta)
        assert rne_ok.all(), "attention outputs not the RNE binary16 of the kernel's bounded " \
            "f32 value (first at %s: gpu %s, exact %s)" % (
                np.argwhere(~rne_ok)[:3].tolist(), g[~rne_ok][:3], r[~rne_ok][:3])
