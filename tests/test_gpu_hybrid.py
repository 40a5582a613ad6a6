"""GPU parity of the hybrid modes tq35 / tq25 (tq_hybrid_encode /
tq_hybrid_decode) against the oracle.

Encode: each group's codes bit-exact outside the 1e-6 band of its oracle z
(in-band differences +-1), group norms within 1e-3; on vectors whose codes all
match, rho within 1e-3 and the sign bits of the sketch bit-exact except where
the oracle's projection t lies within the kernel's f32 error bound of 0.
Decode, on the oracle's own rows: the binary16 nearest-even of a value within
the kernel's f32 error bound of the oracle's exact decode."""
import math

import numpy as np
import pytest
import torch

import oracle
import parity as P
from kv_cache_vector_amd import _lib
from kv_cache_vector_amd import workloads as W
from kv_cache_vector_amd.turboquant import HybridTurboQuant

pytestmark = pytest.mark.gpu
D, H = 128, 64
U = 2.0 ** -24
BITS = {"tq35": (3, 2), "tq25": (2, 1)}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an AMD Instinct GPU"
    _lib.load()
    return torch.device("cuda:0")


def _fields(rows, mode):
    """Split packed rows: codes A, codes B [n, 64] each, sign bits [n, 128],
    norms [n, 3] (norm A, norm B, rho)."""
    ba, bb = BITS[mode]
    pa, pb = H * ba // 8, H * bb // 8
    ca = P.unpack_codes(rows[:, :pa], ba)
    cb = P.unpack_codes(rows[:, pa:pa + pb], bb)
    sb = np.unpackbits(rows[:, pa + pb:pa + pb + 16], axis=-1, bitorder="little")
    nv = np.ascontiguousarray(rows[:, pa + pb + 16:]).view(np.float32)
    return ca, cb, sb, nv


def _group_sums(ca, cb, mode):
    """sum_i |c[code_i]| per group [n], with the oracle's levels."""
    ba, bb = BITS[mode]
    la, _ = oracle.codebook(ba)
    lb, _ = oracle.codebook(bb)
    return np.abs(la[ca]).sum(1), np.abs(lb[cb]).sum(1)


def run_hybrid(dev, x_np, mode, seed, perm, what):
    n = x_np.shape[0]
    P.log("[hybrid] %s: n=%d mode=%s seed=%d" % (what, n, mode, seed))
    ba, bb = BITS[mode]
    h = HybridTurboQuant(D, mode, seed, dev)
    h._perm = np.asarray(perm, np.int32).copy()
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(dev)
    gp = h.encode(x)
    torch.cuda.synchronize()
    gp = gp.cpu().numpy()
    rp = check_rows(gp, x_np, mode, seed, perm, what)
    # decode, on the oracle's rows
    gd = h.decode(torch.from_numpy(rp).to(dev))
    torch.cuda.synchronize()
    check_decode(gd.cpu().numpy(), rp, mode, seed, perm, what)
    return gp


def check_rows(gp, x_np, mode, seed, perm, what):
    """The encode-side rules on GPU rows gp of the vectors x_np; returns the
    oracle's rows."""
    n = x_np.shape[0]
    ba, bb = BITS[mode]
    rp, z, t = oracle.hybrid_encode(x_np, mode, seed, perm, want_z=True, want_t=True)
    gca, gcb, gsb, gnv = _fields(gp, mode)
    rca, rcb, rsb, rnv = _fields(rp, mode)
    # group codes and norms
    _, ta = oracle.codebook(ba)
    _, tb = oracle.codebook(bb)
    pa, pb = H * ba // 8, H * bb // 8
    P.compare_codes(gp[:, :pa], rp[:, :pa], z[:, :H], ta, ba, what + " group A", pooled=False)
    P.compare_codes(gp[:, pa:pa + pb], rp[:, pa:pa + pb], z[:, H:], tb, bb, what + " group B",
                    pooled=False)
    P.compare_norms(gnv[:, :2], rnv[:, :2], what + " group norms")
    same = np.all(gca == rca, axis=1) & np.all(gcb == rcb, axis=1)
    P.log("%s: %d of %d vectors with identical group codes" % (what, int(same.sum()), n))
    # in-band code differences (allowed above) change the residual, so those
    # vectors' sketches are not compared; they must stay rare
    assert same.sum() >= n - max(2, n // 20)
    # rho and the sketch, on those vectors
    P.compare_norms(gnv[same, 2], rnv[same, 2], what + " rho")
    xd = x_np.astype(np.float64)
    ym = _mse_only(rp, mode, seed, perm)[:, perm]             # group order
    r = xd[:, perm] - ym
    sa, sb_ = _group_sums(rca, rcb, mode)
    na, nb = rnv[:, 0].astype(np.float64), rnv[:, 1].astype(np.float64)
    dr = np.concatenate([np.repeat((10 * U * na * sa / H)[:, None], H, 1),
                         np.repeat((10 * U * nb * sb_ / H)[:, None], H, 1)], 1)
    dr = dr + 2.0 ** -20 * np.abs(ym) + U * np.abs(r)
    dt = dr.sum(1) + 8 * U * np.abs(r).sum(1)                 # bound on |t_gpu - t| per vector
    near = np.abs(t) <= dt[:, None]
    bad = (gsb != rsb) & same[:, None] & ~near
    P.log("%s sketch: %d of %d sign bits within the bound of 0, %d differ"
          % (what, int((near & same[:, None]).sum()), int(same.sum()) * D,
             int(((gsb != rsb) & same[:, None]).sum())))
    assert not bad.any(), "sketch sign bits differ outside the f32 bound (%d)" % bad.sum()
    return rp


def check_decode(g16, rows, mode, seed, perm, what):
    """GPU decode g16 of `rows` against the oracle's exact decode: the binary16
    nearest-even of a value within the kernel's f32 error bound (per group:
    10 roundings of (n/64) sum|c|; the sketch: 10 of sqrt(pi/2) rho; the sum:
    2 of |xhat|)."""
    n = rows.shape[0]
    _, xh = oracle.hybrid_decode(rows, D, mode, seed, perm, want_f64=True)
    ca, cb, _, nv = _fields(rows, mode)
    sa, sb_ = _group_sums(ca, cb, mode)
    na, nb, rho = (nv[:, i].astype(np.float64) for i in range(3))
    dg = np.empty((n, D))
    dg[:, perm[:H]] = (10 * U * na * sa / H)[:, None]
    dg[:, perm[H:]] = (10 * U * nb * sb_ / H)[:, None]
    delta = dg + (10 * U * math.sqrt(math.pi / 2) * rho)[:, None] + 2 * U * np.abs(xh)
    ok = P.rounding_check(g16, xh, delta)
    differ = int((g16.astype(np.float64) != P.rne16(xh).astype(np.float64)).sum())
    P.log("%s decode: %d of %d differ from RNE(oracle), all inside the f32 bound: %s"
          % (what, differ, xh.size, bool(ok.all())))
    assert ok.all(), "hybrid decode not the RNE binary16 of the bounded f32 value (first at %s)" % (
        np.argwhere(~ok)[:3].tolist())


def _mse_only(rows, mode, seed, perm):
    p0 = rows.copy()
    p0[:, -4:] = 0
    return oracle.hybrid_decode(p0, D, mode, seed, perm, want_f64=True)[1]


@pytest.mark.parametrize("mode", ["tq35", "tq25"])
def test_outlier_workload_identity_split(dev, mode):
    run_hybrid(dev, W.outlier_channels_fixed(), mode, 0, np.arange(D), "outliers " + mode)


@pytest.mark.parametrize("mode", ["tq35", "tq25"])
def test_calibrated_split(dev, mode):
    """Group A = the calibrated outlier channels of an 8B-shaped layer slice."""
    x = W.llama8b_layer(4, tokens=256)
    h = HybridTurboQuant(D, mode, 7, dev)
    h.calibrate(torch.from_numpy(x[:4096]).to(dev))
    perm = h.perm
    assert sorted(perm.tolist()) == list(range(D))
    run_hybrid(dev, x, mode, 7, perm, "calibrated " + mode)


@pytest.mark.parametrize("mode", ["tq35", "tq25"])
def test_random_split_and_ragged_counts(dev, mode):
    """Random channel permutations and the identity (which takes the kernels'
    direct-load path); counts that leave partial quads, waves and blocks;
    nothing past the n rows is written."""
    rng = np.random.default_rng(11)
    row = HybridTurboQuant.packed_dim_for_mode(D, mode)
    s = torch.cuda.current_stream().cuda_stream
    for n, perm in [(n, p) for n in (1, 3, 17, 63, 64, 65, 1000)
                    for p in (rng.permutation(D).astype(np.int32), np.arange(D, dtype=np.int32))]:
        x_np = W.gaussian(n, seed=n)
        run_hybrid(dev, x_np, mode, 5, perm, "n=%d %s %s" % (n, mode, "identity" if np.array_equal(perm, np.arange(D)) else "random"))
        x = torch.from_numpy(x_np).to(dev)
        buf = torch.full((n * row + 256,), 0xA5, dtype=torch.uint8, device=dev)
        assert _lib.tq_hybrid_encode(x.data_ptr(), n, D, HybridTurboQuant.MODES[mode], 5,
                                     perm.ctypes.data, buf.data_ptr(), s) == 0
        out = torch.full((n * D + 512,), 1234.0, dtype=torch.float16, device=dev)
        assert _lib.tq_hybrid_decode(buf.data_ptr(), n, D, HybridTurboQuant.MODES[mode], 5,
                                     perm.ctypes.data, out.data_ptr(), s) == 0
        torch.cuda.synchronize()
        assert np.all(buf.cpu().numpy()[n * row:] == 0xA5)
        assert np.all(out.cpu().numpy()[n * D:] == 1234.0)


@pytest.mark.parametrize("mode", ["tq35", "tq25"])
def test_special_vectors(dev, mode):
    """Zero vector, a vector with one empty group, huge and tiny magnitudes."""
    rng = np.random.default_rng(3)
    rows = [np.zeros(D), np.r_[np.ones(H), np.zeros(H)], np.r_[np.zeros(H), -np.ones(H)],
            np.full(D, 60000.0), np.full(D, 2.0 ** -20)]
    for _ in range(11):
        rows.append(rng.standard_normal(D) * 10.0 ** rng.uniform(-3, 3))
    x = np.array(rows).astype(np.float16)
    gp = run_hybrid(dev, x, mode, 1, np.arange(D), "special " + mode)
    assert np.all(gp[0, -12:] == 0)                    # zero vector: zero norms


@pytest.mark.parametrize("mode", ["tq35", "tq25"])
def test_large_launch_sampled(dev, mode):
    """One 8B-shaped layer (524,288 vectors) in one launch, compared on 4096
    sampled rows plus the first and last."""
    x_np = W.llama8b_layer(9)
    n = x_np.shape[0]
    h = HybridTurboQuant(D, mode, 9, dev)
    h.calibrate_uniform(8)
    P.log("[hybrid] large n=%d %s" % (n, mode))
    x = torch.from_numpy(x_np).to(dev)
    gp = h.encode(x)
    out = h.decode(gp)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(9).choice(n, 4096, replace=False),
                                     [0, n - 1]]))
    ridx = torch.from_numpy(rows).to(dev)
    perm = np.arange(D, dtype=np.int32)
    got = gp[ridx].cpu().numpy()
    check_rows(got, x_np[rows], mode, 9, perm, "large " + mode)
    # the decode of the GPU's own rows against the oracle's decode of them
    check_decode(out[ridx].cpu().numpy(), got, mode, 9, perm, "large " + mode)


def test_inner_products_unbiased_on_gpu(dev):
    """HybridTurboQuant.validate: over many vectors <x, xhat> averages to
    ||x||^2 (the sketch removes the TurboQuant part's shrinkage, 7% at tq35
    and 23% at tq25), and the round-trip MSE sits near its expected value."""
    for mode, mse_lo, mse_hi in (("tq35", 0.035, 0.05), ("tq25", 0.11, 0.16)):
        r = HybridTurboQuant(D, mode, 3, dev).validate(200000)
        P.log("[hybrid] validate %s: %s" % (mode, r))
        assert mse_lo < r["mse"] < mse_hi
        assert abs(r["inner_product_bias"]) < 3e-3
