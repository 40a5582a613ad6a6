"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each ``check_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a closed form, a library routine, a published
value or brute force.  The regular tests run them on the committed oracle; the
mutation test runs them on copies of the oracle with a planted mistake and
requires that every planted mistake trips at least one of them.
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.integrate as si
import scipy.linalg as sl
from scipy.stats import norm as _norm

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
D = 128


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ---------------------------------------------------------------------------
# binary16 conversions: numpy's float16 is IEEE binary16 with RNE
# ---------------------------------------------------------------------------

def check_half_to_double(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = o.half_to_double(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def check_double_to_half(o, n=20000, seed=3):
    rng = np.random.default_rng(seed)
    # values spread over the whole binary16 range, plus exact ties
    mags = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), n))
    x = mags * rng.choice([-1.0, 1.0], n)
    h = np.arange(0, 0x7bff, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = (lo + hi) / 2.0           # exactly half-way: must round to even
    edge = np.array([65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                     3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -26, -0.0, 0.0])
    xs = np.concatenate([x, ties, -ties, edge])
    ref = xs.astype(np.float16).view(np.uint16)
    got = o.double_to_half(xs)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# SplitMix64 and the sign vector
# ---------------------------------------------------------------------------

def check_splitmix64(o):
    for row in _read_rows("splitmix64_vectors.txt"):
        seed, idx, hexv = row.split()
        seq = o.splitmix64(int(seed), int(idx) + 1)
        assert int(seq[int(idx)]) == int(hexv, 16), (seed, idx)


def check_signs(o):
    # sigma_i = -1 exactly when the top bit of the i-th output is set
    for seed in (0, 1, 42, 2 ** 63 + 5):
        seq = o.splitmix64(seed, D)
        s = o.signs(seed, D)
        assert np.array_equal(s, np.where(seq >> np.uint64(63), -1, 1).astype(np.int8))
    # seed 0 from the published outputs: 0xe2.. and 0x6e.. and 0x06..
    s0 = o.signs(0, D)
    assert list(s0[:3]) == [-1, 1, 1]
    assert "".join("-" if v < 0 else "+" for v in s0[:16]) == "-++-+++-+-+-----"
    assert int((s0 < 0).sum()) == 63


# ---------------------------------------------------------------------------
# Hadamard matrix and rotation
# ---------------------------------------------------------------------------

def check_hadamard(o):
    for d in (2, 4, 32, 64, 128, 256):
        H = o.hadamard(d).astype(np.int64)
        assert np.array_equal(H, sl.hadamard(d))            # Sylvester construction
        assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))


def check_rotation_unit_vectors(o, bits=4, seed=7, d=D):
    """x = sigma_k e_k has D x = e_k, so z = H e_k = column k of H: every z is
    +-1 exactly and the codes are those of +-1."""
    s = o.signs(seed, d)
    H = sl.hadamard(d)
    c, t = o.codebook(bits)
    code_p = int(np.sum(t < 1.0))
    code_m = int(np.sum(t < -1.0))
    for k in (0, 1, 5, d // 2, d - 1):
        x = np.zeros((1, d), dtype=np.float16)
        x[0, k] = s[k]
        packed, norms, z = o.encode(x, bits, seed, want_z=True)
        assert norms[0] == 1.0
        assert np.array_equal(z[0], H[:, k].astype(np.float64))
        codes = o.unpack(packed[0], d, bits)
        assert np.array_equal(codes, np.where(H[:, k] > 0, code_p, code_m))


def check_rotation_norm(o, seed=11, d=D):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, d)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float16)
    _, norms, z = o.encode(x, 4, 3, want_z=True)
    ref = np.sqrt((x.astype(np.float64) ** 2).sum(1))
    assert np.array_equal(norms, ref.astype(np.float32))    # double norm, nearest f32
    # ||z||^2 = d: H D / sqrt(d) is orthogonal
    assert np.allclose((z ** 2).sum(1), d, rtol=0, atol=1e-10)
    # z = H D x / ||x|| (library Hadamard, signs from the generator)
    s = o.signs(3, d).astype(np.float64)
    zr = (sl.hadamard(d) @ (s[:, None] * (x.astype(np.float64) / ref[:, None]).T)).T
    assert np.allclose(z, zr, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook
# ---------------------------------------------------------------------------

def _cell_integrals(lo, hi):
    mass = si.quad(_norm.pdf, lo, hi, epsabs=1e-14, epsrel=1e-13, limit=200)[0]
    first = si.quad(lambda v: v * _norm.pdf(v), lo, hi, epsabs=1e-14, epsrel=1e-13,
                    limit=200)[0]
    return mass, first


def check_codebook_closed_form_b1(o):
    c, t = o.codebook(1)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-14 and c[0] == -c[1] and t[0] == 0.0
    assert abs(o.codebook_distortion(1) - (1 - 2 / math.pi)) < 1e-14


def check_codebook_structure(o):
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        L = 1 << b
        assert np.all(np.diff(c) > 0)
        assert np.array_equal(c, -c[::-1])                  # exactly symmetric
        assert t[L // 2 - 1] == 0.0                        # middle threshold exactly 0
        assert np.allclose(t, (c[:-1] + c[1:]) / 2, rtol=0, atol=1e-15)


def check_codebook_centroids(o):
    """Every level is the N(0,1) mean of its cell, by numerical integration."""
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        for k in range(len(c)):
            mass, first = _cell_integrals(edges[k], edges[k + 1])
            assert abs(first / mass - c[k]) < 1e-9, (b, k)


def check_codebook_distortion(o):
    """Distortion by numerical integration of (x - q(x))^2 against N(0,1)."""
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        tot = 0.0
        for k in range(len(c)):
            tot += si.quad(lambda v, ck=c[k]: (v - ck) ** 2 * _norm.pdf(v), edges[k],
                           edges[k + 1], epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        assert abs(tot - o.codebook_distortion(b)) < 1e-10, b


def check_codebook_textbook(o):
    """Max (1960), Table I."""
    for row in _read_rows("lloyd_max_gaussian.txt"):
        f = row.split()
        L, kind, vals = int(f[0]), f[1], [float(v) for v in f[2:]]
        b = L.bit_length() - 1
        c, t = o.codebook(b)
        if kind == "level":
            assert np.allclose(c[L // 2:], vals, rtol=0, atol=6e-4), (L, c[L // 2:])
        elif kind == "threshold":
            assert np.allclose(t[L // 2:], vals, rtol=0, atol=6e-4), (L, t[L // 2:])
        else:
            assert abs(o.codebook_distortion(b) / vals[0] - 1) < 5e-4, (L, kind)


def check_codebook_is_local_minimum(o):
    """Moving any one level or threshold raises the (integrated) distortion."""
    b = 3
    c, t = o.codebook(b)

    def dist(cc, tt):
        edges = np.concatenate([[-np.inf], tt, [np.inf]])
        return sum(si.quad(lambda v, ck=cc[k]: (v - ck) ** 2 * _norm.pdf(v), edges[k],
                           edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
                   for k in range(len(cc)))

    base = dist(c, t)
    for k in range(len(c)):
        for eps in (1e-3, -1e-3):
            cc = c.copy()
            cc[k] += eps
            assert dist(cc, t) > base
    for k in range(len(t)):
        for eps in (1e-3, -1e-3):
            tt = t.copy()
            tt[k] += eps
            assert dist(c, tt) > base


# ---------------------------------------------------------------------------
# scalar quantizer
# ---------------------------------------------------------------------------

def check_quantizer_bruteforce(o, seed=5):
    rng = np.random.default_rng(seed)
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        z = np.concatenate([np.linspace(-4, 4, 4001), rng.standard_normal(3000) * 2])
        got = o.quantize_many(z, b)
        # nearest level, first one on a tie (brute force over all levels)
        ref = np.argmin(np.abs(z[:, None] - c[None, :]), axis=1)
        assert np.array_equal(got, ref), b


def check_quantizer_special_points(o):
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        L = 1 << b
        assert np.array_equal(o.quantize_many(c, b), np.arange(L))        # z = c_k -> k
        assert np.array_equal(o.quantize_many(t, b), np.arange(L - 1))    # tie -> lower
        assert np.array_equal(o.quantize_many(np.nextafter(t, np.inf), b), np.arange(1, L))
        assert list(o.quantize_many([0.0, -0.0], b)) == [L // 2 - 1] * 2
        assert list(o.quantize_many([-1e9, 1e9], b)) == [0, L - 1]


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------

def check_pack_vectors(o):
    for row in _read_rows("pack_vectors.txt"):
        bits_s, codes_s, bytes_s = [p.strip() for p in row.split(";")]
        bits = int(bits_s)
        codes = np.array([int(v) for v in codes_s.split()], dtype=np.uint8)
        want = np.array([int(v, 16) for v in bytes_s.split()], dtype=np.uint8)
        assert np.array_equal(o.pack(codes, bits), want), row
        assert np.array_equal(o.unpack(want, len(codes), bits), codes), row


def check_pack_roundtrip(o, seed=9):
    rng = np.random.default_rng(seed)
    for b in (2, 3, 4):
        P = D * b // 8
        for _ in range(20):
            codes = rng.integers(0, 1 << b, D).astype(np.uint8)
            p = o.pack(codes, b)
            assert p.shape == (P,)
            assert np.array_equal(o.unpack(p, D, b), codes)
            raw = rng.integers(0, 256, P).astype(np.uint8)     # every byte string is valid
            assert np.array_equal(o.pack(o.unpack(raw, D, b), b), raw)


def check_sizes(o):
    for b, P in ((2, 32), (3, 48), (4, 64)):
        assert o.packed_bytes(D, b) == P
    # 256 B of fp16 against P + 4 B (codes + f32 norm): 3.76x at 4 bits, 7.11x at 2 bits
    assert round(256 / (64 + 4), 2) == 3.76 and round(256 / (32 + 4), 1) == 7.1


# ---------------------------------------------------------------------------
# round-trip MSE against the exact value for d = 128
# ---------------------------------------------------------------------------

def exact_mse_d(b: int, c, t, d: int = D) -> float:
    """E[(z - q(z))^2] where z = sqrt(d) * (coordinate of a uniform unit vector):
    density proportional to (1 - z^2/d)^((d-3)/2) on [-sqrt(d), sqrt(d)]."""
    r = math.sqrt(d)
    logc = math.lgamma(d / 2) - math.lgamma((d - 1) / 2) - 0.5 * math.log(math.pi * d)
    pdf = lambda z: math.exp(logc + (d - 3) / 2 * math.log1p(-(z * z) / d))
    edges = np.concatenate([[-r], t, [r]])
    return sum(si.quad(lambda z, ck=c[k]: (z - ck) ** 2 * pdf(z), edges[k], edges[k + 1],
                       epsabs=1e-15, epsrel=1e-12, limit=200)[0] for k in range(len(c)))


GAUSS_D = {2: 0.1175, 3: 0.03455, 4: 0.009497}   # Max (1960) distortions


def check_mse(o, n=50000, seed=21):
    """Round trip on N(0,1) vectors: the per-coordinate MSE ||x - xhat||^2/||x||^2
    equals the exact d=128 value (within Monte-Carlo error), is within 2% of the
    Gaussian Lloyd-Max distortion, and within 2.7x of the 4^-b lower bound."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)).astype(np.float16)
    xd = x.astype(np.float64)
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        packed, norms = o.encode(x, b, 1)
        _, xh = o.decode(packed, norms, D, b, 1, want_f64=True)
        mse = float(np.mean(((xd - xh) ** 2).sum(1) / (xd ** 2).sum(1)))
        ex = exact_mse_d(b, c, t)
        assert abs(mse / ex - 1) < 3e-3, (b, mse, ex)
        assert abs(mse / GAUSS_D[b] - 1) < 0.02, (b, mse)
        assert mse < 2.7 * 4.0 ** -b


def check_z_distribution(o, seed=23):
    """After the rotation, coordinates look N(0,1) (the pages' 'each coordinate
    ~N(0, 1/d)', in units of the unit vector times sqrt(d)), and outlier
    channels are spread over all coordinates."""
    rng = np.random.default_rng(seed)
    # iid Laplace input (far from Gaussian per channel): rotated coordinates
    # have exactly unit mean square and Gaussian-like quantiles
    x = rng.laplace(size=(4000, D))
    _, _, z = o.encode(x.astype(np.float16), 4, 0, want_z=True)
    zz = z.ravel()
    assert abs(zz.mean()) < 0.01 and abs(np.mean(zz ** 2) - 1) < 1e-12
    q = np.quantile(zz, [0.025, 0.5, 0.975])
    assert np.allclose(q, [-1.96, 0.0, 1.96], atol=0.05)
    # two x20 outlier channels: before rotation they reach ~6-11 in these
    # units; after it no coordinate carries much more than its share
    x = rng.standard_normal((4000, D))
    x[:, [7, 93]] *= 20
    xf = x.astype(np.float16).astype(np.float64)
    u = np.sqrt(D) * xf / np.linalg.norm(xf, axis=1, keepdims=True)
    _, _, z = o.encode(x.astype(np.float16), 4, 0, want_z=True)
    assert np.abs(u).max() > 9 and np.abs(z).max() < 4.5


# ---------------------------------------------------------------------------
# invariants of encode
# ---------------------------------------------------------------------------

def check_scale_invariance(o, seed=31):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((256, D))
    x = np.where(np.abs(x) < 0.05, np.copysign(0.05, x), x)   # keep 2^-3 x normal in fp16
    x = x.astype(np.float16)
    for b in (2, 3, 4):
        p0, n0 = o.encode(x, b, 5)
        for k in (-3, -1, 2, 4):
            xs = (x.astype(np.float64) * 2.0 ** k).astype(np.float16)
            assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** k)
            p, n = o.encode(xs, b, 5)
            assert np.array_equal(p, p0)
            assert np.array_equal(n, (n0.astype(np.float64) * 2.0 ** k).astype(np.float32))


def check_negation(o, seed=37):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((256, D)).astype(np.float16)
    for b in (2, 3, 4):
        L = 1 << b
        _, t = o.codebook(b)
        p0, _, z = o.encode(x, b, 5, want_z=True)
        p1, _ = o.encode(-x, b, 5)
        on_thr = np.isin(z, t) | np.isin(-z, t)
        for v in range(x.shape[0]):
            c0 = o.unpack(p0[v], D, b).astype(int)
            c1 = o.unpack(p1[v], D, b).astype(int)
            ok = (c1 == L - 1 - c0) | on_thr[v]
            assert ok.all()


def check_zero_vector(o):
    x = np.zeros((3, D), dtype=np.float16)
    x[1] = -0.0
    for b in (2, 3, 4):
        L = 1 << b
        p, n = o.encode(x, b, 9)
        assert np.all(n == 0)
        for v in range(3):
            assert np.all(o.unpack(p[v], D, b) == L // 2 - 1)
        y = o.decode(p, n, D, b, 9)
        assert np.all(y.astype(np.float64) == 0)


def check_reencode_fixed_point(o, seed=41, d=D):
    """Build x = fp16(D H c[code] / d) from codes drawn with the Gaussian cell
    probabilities; re-encoding it returns the same codes."""
    rng = np.random.default_rng(seed)
    H = sl.hadamard(d).astype(np.float64)
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        s = o.signs(13, d).astype(np.float64)
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        prob = np.diff(_norm.cdf(edges))
        done = 0
        while done < 20:
            code = rng.choice(len(c), size=d, p=prob)
            if not (0.85 <= np.mean(c[code] ** 2) <= 1.2):
                continue
            x = (s * (H @ c[code]) / d).astype(np.float16)[None, :]
            p, _ = o.encode(x, b, 13)
            assert np.array_equal(o.unpack(p[0], d, b), code.astype(np.uint8)), b
            done += 1


def check_decode_definition(o, seed=43, d=D):
    """Decode of hand-made codes: xhat = n * D * H * c[code] / d, with the
    library Hadamard; the fp16 output is that value rounded to nearest-even."""
    rng = np.random.default_rng(seed)
    H = sl.hadamard(d).astype(np.float64)
    for b in (2, 3, 4):
        c, _ = o.codebook(b)
        s = o.signs(17, d).astype(np.float64)
        codes = rng.integers(0, 1 << b, (8, d)).astype(np.uint8)
        packed = np.stack([o.pack(cc, b) for cc in codes])
        norms = rng.uniform(0.5, 50, 8).astype(np.float32)
        y, yf = o.decode(packed, norms, d, b, 17, want_f64=True)
        ref = norms[:, None].astype(np.float64) * s[None, :] * (c[codes] @ H.T) / d
        assert np.allclose(yf, ref, rtol=1e-13, atol=1e-12)
        assert np.array_equal(y, yf.astype(np.float16))


# ---------------------------------------------------------------------------
# paged decode attention
# ---------------------------------------------------------------------------

def small_attn_case(o, B=2, Hq=8, Hkv=2, T=37, bs=16, bits=4, seed=51, ragged=True, d=D):
    from kv_cache_vector_amd import workloads as w
    wl = w.attn_workload(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, context=T,
                         block_size=bs, seed=seed, perm_seed=seed + 1, ragged=ragged,
                         extra_blocks=3, head_dim=d)
    kp, kn = o.encode(wl["k"], bits, 0)
    vp, vn = o.encode(wl["v"], bits, 0)
    wl.update(kp=kp, kn=kn, vp=vp, vn=vn, bits=bits)
    return wl


def _attn(o, wl, q=None, cl=None, bt=None, kp=None, kn=None, vp=None, vn=None, scale=None):
    q = wl["q"] if q is None else q
    return o.attn_decode(q, wl["kp"] if kp is None else kp, wl["kn"] if kn is None else kn,
                         wl["vp"] if vp is None else vp, wl["vn"] if vn is None else vn,
                         wl["block_tables"] if bt is None else bt,
                         wl["context_lens"] if cl is None else cl, wl["num_kv_heads"],
                         wl["bits"], 0, 1 / math.sqrt(q.shape[-1]) if scale is None else scale,
                         want_f64=True)


def _dequant_rows(o, wl, which, b, g):
    """Decoded (double) rows of sequence b, kv head g, in token order."""
    bs = wl["block_size"]
    T = int(wl["context_lens"][b])
    d = wl["q"].shape[-1]
    P = d * wl["bits"] // 8
    pk = wl["kp" if which == "k" else "vp"]
    nm = wl["kn" if which == "k" else "vn"]
    rows_p = np.zeros((T, P), np.uint8)
    rows_n = np.zeros(T, np.float32)
    for j in range(T):
        blk = wl["block_tables"][b, j // bs]
        rows_p[j] = pk[blk, j % bs, g]
        rows_n[j] = nm[blk, j % bs, g]
    _, xh = o.decode(rows_p, rows_n, d, wl["bits"], 0, want_f64=True)
    return xh


def check_attn_rotated_domain_identity(o, d=D, bits_list=(4, 3, 2)):
    """Score and accumulate in the rotated domain (q rotated once, K and V
    used as codebook values, one inverse rotation at the end) -- the fused
    path the pages describe -- equals the plain definition."""
    D = d
    H = sl.hadamard(D).astype(np.float64)
    for bits in bits_list:
        wl = small_attn_case(o, bits=bits, d=D)
        _, of = _attn(o, wl)
        c, _ = o.codebook(bits)
        s = o.signs(0, D).astype(np.float64)
        B, Hq, _ = wl["q"].shape
        grp = Hq // wl["num_kv_heads"]
        bs = wl["block_size"]
        for b in range(B):
            T = int(wl["context_lens"][b])
            for h in range(Hq):
                g = h // grp
                qt = H @ (s * wl["q"][b, h].astype(np.float64))         # rotate q once
                sc = np.zeros(T)
                vacc = np.zeros((T, D))
                for j in range(T):
                    blk = wl["block_tables"][b, j // bs]
                    kc = c[o.unpack(wl["kp"][blk, j % bs, g], D, bits)]
                    vc = c[o.unpack(wl["vp"][blk, j % bs, g], D, bits)]
                    sc[j] = (1 / math.sqrt(D)) * float(wl["kn"][blk, j % bs, g]) / D * (qt @ kc)
                    vacc[j] = float(wl["vn"][blk, j % bs, g]) * vc
                p = np.exp(sc - sc.max())
                acc = (p[:, None] * vacc).sum(0) / p.sum()
                ref = s * (H @ acc) / D                                   # rotate back once
                assert np.allclose(of[b, h], ref, rtol=0, atol=1e-10), (bits, b, h)


def check_attn_special_cases(o, d=D):
    wl = small_attn_case(o, B=4, T=40, d=d)
    B, Hq, _ = wl["q"].shape
    grp = Hq // wl["num_kv_heads"]
    # context_len = 1: the output is the decoded first value row
    cl1 = np.ones(B, np.int32)
    wl1 = dict(wl, context_lens=cl1)
    y, yf = _attn(o, wl1, cl=cl1)
    for b in range(B):
        for h in range(Hq):
            v0 = _dequant_rows(o, wl1, "v", b, h // grp)[0]
            assert np.allclose(yf[b, h], v0, rtol=0, atol=1e-12)
            assert np.array_equal(y[b, h], v0.astype(np.float16))
    # q = 0: uniform softmax, the output is the mean of the decoded values
    _, yf = _attn(o, wl, q=np.zeros_like(wl["q"]))
    for b in range(B):
        for h in range(Hq):
            vm = _dequant_rows(o, wl, "v", b, h // grp).mean(0)
            assert np.allclose(yf[b, h], vm, rtol=0, atol=1e-12)
    # all keys equal (every K row encodes the same vector): mean of V again
    kp = np.broadcast_to(wl["kp"][0, 0, 0], wl["kp"].shape).copy()
    kn = np.full_like(wl["kn"], wl["kn"][0, 0, 0])
    _, yf = _attn(o, wl, kp=kp, kn=kn)
    for b in range(B):
        for h in range(Hq):
            vm = _dequant_rows(o, wl, "v", b, h // grp).mean(0)
            assert np.allclose(yf[b, h], vm, rtol=0, atol=1e-12)
    # context_len = 0: zeros
    cl0 = np.zeros(B, np.int32)
    y, yf = _attn(o, wl, cl=cl0)
    assert np.all(yf == 0) and np.all(y.astype(np.float64) == 0)


def check_attn_paging_invariance(o, seed=61):
    """Moving physical blocks (and the block table with them) and changing
    cache rows beyond context_len leave the output unchanged."""
    rng = np.random.default_rng(seed)
    wl = small_attn_case(o, B=3, T=45)
    y0, _ = _attn(o, wl)
    nblk = wl["kp"].shape[0]
    perm = rng.permutation(nblk)            # new physical position of every block
    inv = np.argsort(perm)
    kp, kn, vp, vn = (a[inv] for a in (wl["kp"], wl["kn"], wl["vp"], wl["vn"]))
    bt = perm[wl["block_tables"]].astype(np.int32)
    y1, _ = _attn(o, wl, bt=bt, kp=kp, kn=kn, vp=vp, vn=vn)
    assert np.array_equal(y0, y1)
    # garbage after the last valid token of every sequence
    kp2, vp2, kn2 = wl["kp"].copy(), wl["vp"].copy(), wl["kn"].copy()
    bs = wl["block_size"]
    for b in range(3):
        T = int(wl["context_lens"][b])
        for j in range(T, wl["block_tables"].shape[1] * bs):
            blk = wl["block_tables"][b, j // bs]
            kp2[blk, j % bs] = rng.integers(0, 256, kp2.shape[2:])
            vp2[blk, j % bs] = rng.integers(0, 256, vp2.shape[2:])
            kn2[blk, j % bs] = 1e3
    y2, _ = _attn(o, wl, kp=kp2, kn=kn2, vp=vp2)
    assert np.array_equal(y0, y2)


def check_attn_bruteforce_tiny(o):
    """B=1, T=3, one kv head: softmax written out by hand on decoded rows."""
    wl = small_attn_case(o, B=1, Hq=2, Hkv=1, T=3, ragged=False)
    _, yf = _attn(o, wl)
    K = _dequant_rows(o, wl, "k", 0, 0)
    V = _dequant_rows(o, wl, "v", 0, 0)
    for h in range(2):
        q = wl["q"][0, h].astype(np.float64)
        s0, s1, s2 = (float(q @ K[j]) / math.sqrt(D) for j in range(3))
        m = max(s0, s1, s2)
        e0, e1, e2 = math.exp(s0 - m), math.exp(s1 - m), math.exp(s2 - m)
        ref = (e0 * V[0] + e1 * V[1] + e2 * V[2]) / (e0 + e1 + e2)
        assert np.allclose(yf[0, h], ref, rtol=0, atol=1e-12)


def check_attn_gqa_grouping(o):
    """Query heads h and h' of the same kv group with the same query give
    the same output; the group of head h is h // (Hq/Hkv)."""
    wl = small_attn_case(o, B=1, Hq=8, Hkv=2, T=30, ragged=False)
    q = wl["q"].copy()
    q[0, 1] = q[0, 0]
    q[0, 4] = q[0, 0]
    y, _ = _attn(o, wl, q=q)
    assert np.array_equal(y[0, 0], y[0, 1])
    assert not np.array_equal(y[0, 0], y[0, 4])     # head 4 belongs to kv head 1
    # swapping the two kv heads' cache content swaps the groups' outputs
    sw = lambda a: a[:, :, ::-1].copy()
    q2 = q.copy()
    q2[0, 4:] = q[0, :4]
    q2[0, :4] = q[0, 4:]
    y2, _ = _attn(o, wl, q=q2, kp=sw(wl["kp"]), kn=sw(wl["kn"]), vp=sw(wl["vp"]),
                  vn=sw(wl["vn"]))
    assert np.array_equal(y2[0, 4:], y[0, :4]) and np.array_equal(y2[0, :4], y[0, 4:])


def check_attn_mixed_widths(o):
    """Keys at one width and values at another (4-bit keys with 2-bit values,
    as on the KVarN repository page, "What it does", and the other pairs):
    a softmax written out by hand over keys decoded at the key width and
    values decoded at the value width; context_len = 1 gives the first value
    row at the value width; equal widths reproduce the single-width call."""
    from kv_cache_vector_amd import workloads as w
    wl = w.attn_workload(batch=1, num_q_heads=2, num_kv_heads=1, context=3, block_size=16,
                         seed=71, perm_seed=72, ragged=False, extra_blocks=1)
    blk = int(wl["block_tables"][0, 0])
    sc = 1 / math.sqrt(D)
    for kb, vb in ((4, 2), (2, 4), (3, 4), (4, 3), (2, 3), (3, 2)):
        kp, kn = o.encode(wl["k"], kb, 0)
        vp, vn = o.encode(wl["v"], vb, 0)
        args = (wl["q"], kp, kn, vp, vn, wl["block_tables"])
        _, yf = o.attn_decode(*args, wl["context_lens"], 1, kb, 0, sc, want_f64=True, v_bits=vb)
        _, K = o.decode(kp[blk, :3, 0], kn[blk, :3, 0], D, kb, 0, want_f64=True)
        _, V = o.decode(vp[blk, :3, 0], vn[blk, :3, 0], D, vb, 0, want_f64=True)
        for h in range(2):
            q = wl["q"][0, h].astype(np.float64)
            s = [float(q @ K[j]) * sc for j in range(3)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            ref = (e[0] * V[0] + e[1] * V[1] + e[2] * V[2]) / sum(e)
            assert np.allclose(yf[0, h], ref, rtol=0, atol=1e-12), (kb, vb, h)
        y1, _ = o.attn_decode(*args, np.ones(1, np.int32), 1, kb, 0, sc, want_f64=True,
                              v_bits=vb)
        assert np.array_equal(y1[0, 0], V[0].astype(np.float16)), (kb, vb)
    for b in (2, 3, 4):
        kp, kn = o.encode(wl["k"], b, 0)
        vp, vn = o.encode(wl["v"], b, 0)
        args = (wl["q"], kp, kn, vp, vn, wl["block_tables"], wl["context_lens"], 1, b, 0, sc)
        assert np.array_equal(o.attn_decode(*args), o.attn_decode(*args, v_bits=b))


def check_mse_head_dim(o, d, n, seed=25):
    """Round-trip MSE on N(0,1) vectors of dimension d against the exact value
    for that d (the rotated coordinate is sqrt(d) times a coordinate of a
    uniform unit vector, whose law depends on d), within five standard errors
    of the sample mean, and under the 2.7 x 4^-b bound."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float16)
    xd = x.astype(np.float64)
    for b in (2, 3, 4):
        c, t = o.codebook(b)
        packed, norms = o.encode(x, b, 2)
        _, xh = o.decode(packed, norms, d, b, 2, want_f64=True)
        r = ((xd - xh) ** 2).sum(1) / (xd ** 2).sum(1)
        mse = float(np.mean(r))
        se = float(np.std(r) / np.sqrt(n))
        ex = exact_mse_d(b, c, t, d)
        assert se < 2e-3 * ex, (d, b, se)                 # the sample resolves 1%
        assert abs(mse - ex) < 5 * se, (d, b, mse, ex, se)
        assert mse < 2.7 * 4.0 ** -b


def check_head_dims(o):
    """The codec at head_dim 64 and 256 against the same closed forms and
    definitions as at 128: unit vectors rotate onto Hadamard columns, the
    rotation is H D / ||x|| with ||z||^2 = d, decode is n D H c / d, decoded
    codes re-encode to themselves, and the round-trip MSE is the exact value
    for d."""
    for d in (64, 256):
        check_rotation_unit_vectors(o, d=d)
        check_rotation_norm(o, d=d)
        check_decode_definition(o, d=d)
        check_reencode_fixed_point(o, d=d)
        assert [o.packed_bytes(d, b) for b in (2, 3, 4)] == [d // 4, 3 * d // 8, d // 2]
    check_mse_head_dim(o, 64, 40000)
    check_mse_head_dim(o, 256, 12000)


def check_attn_head_dims(o):
    """Attention at head_dim 64 and 256: the rotated-domain computation
    (with the d-point Hadamard matrix and the first d signs) equals the plain
    definition, and the special cases (context 1, q = 0, equal keys, context
    0) hold."""
    for d in (64, 256):
        check_attn_rotated_domain_identity(o, d=d, bits_list=(4, 3))
        check_attn_special_cases(o, d=d)


# ---------------------------------------------------------------------------
# hybrid modes tq35 / tq25 (split groups + QJL residual)
# ---------------------------------------------------------------------------

SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
HYBRID_BITS = {"tq35": (3, 2), "tq25": (2, 1)}


def _stream_seed(seed: int, skip: int) -> int:
    """The seed whose SplitMix64 stream starts at output `skip` of seed's
    stream (the state advances by the fixed increment per output)."""
    return (seed + skip * SPLITMIX_GAMMA) % (1 << 64)


def _hybrid_mse_only(o, packed, d, mode, seed, perm):
    """Decode with rho set to 0: the two groups' TurboQuant part alone."""
    p0 = np.array(packed, copy=True)
    p0[..., -4:] = 0
    return o.hybrid_decode(p0, d, mode, seed, perm, want_f64=True)[1]


def check_hybrid_sizes(o):
    """Row bytes: codes of the two halves at (3, 2) or (2, 1) bits, d sign bits
    and three f32 norms (68 / 52 bytes at d = 128, 3.76x / 4.92x against 256
    bytes of binary16); unsupported modes and sizes give 0."""
    for d in (64, 128, 256):
        for mode, (ba, bb) in HYBRID_BITS.items():
            assert o.hybrid_packed_bytes(d, mode) == d // 2 * ba // 8 + d // 2 * bb // 8 + d // 8 + 12
    assert o.hybrid_packed_bytes(128, "tq35") == 68 and o.hybrid_packed_bytes(128, "tq25") == 52
    assert abs(256 / 68 - 3.7647) < 1e-4 and abs(256 / 52 - 4.9231) < 1e-4
    assert o.L.tqo_hybrid_packed_bytes(128, 30) == 0 and o.L.tqo_hybrid_packed_bytes(96, 35) == 0


def check_hybrid_groups_are_turboquant(o, seed=17):
    """Each channel group is a TurboQuant vector of dimension d/2: group A's
    codes and norm equal the (pinned) codec's encode of x[perm[:h]] with the
    seed, group B's those of x[perm[h:]] with the seed whose stream starts at
    output h; with rho zeroed, decode is the codec's decode of each group put
    back through perm."""
    rng = np.random.default_rng(seed)
    for d in (64, 128, 256):
        h = d // 2
        x = (rng.standard_normal((300, d)) * rng.uniform(0.2, 5, (1, d))).astype(np.float16)
        perm = rng.permutation(d).astype(np.int32)
        for mode, (ba, bb) in HYBRID_BITS.items():
            pk = o.hybrid_encode(x, mode, seed, perm)
            PA, PB = h * ba // 8, h * bb // 8
            nv = pk[:, PA + PB + d // 8:].copy().view(np.float32)
            ra, na = o.encode(x[:, perm[:h]], ba, seed)
            rb, nb = o.encode(x[:, perm[h:]], bb, _stream_seed(seed, h))
            assert np.array_equal(pk[:, :PA], ra) and np.array_equal(nv[:, 0], na)
            assert np.array_equal(pk[:, PA:PA + PB], rb) and np.array_equal(nv[:, 1], nb)
            _, xa = o.decode(ra, na, h, ba, seed, want_f64=True)
            _, xb = o.decode(rb, nb, h, bb, _stream_seed(seed, h), want_f64=True)
            want = np.zeros((300, d))
            want[:, perm[:h]] = xa
            want[:, perm[h:]] = xb
            got = _hybrid_mse_only(o, pk, d, mode, seed, perm)
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def check_hybrid_qjl_sketch(o, seed=19):
    """The sign sketch: t = H_d D_Q r (scipy's Hadamard matrix, D_Q the signs
    of the stream from output d, r = x[perm] minus the groups' decode) has the
    stored signs (bit set iff t < 0) and ||r|| is the stored f32 rho; the
    decoded correction has norm exactly sqrt(pi/2) rho (D_Q H_d s has norm d)
    and inner product sqrt(pi/2)/d rho ||t||_1 with r."""
    rng = np.random.default_rng(seed)
    for d in (64, 128, 256):
        H = sl.hadamard(d).astype(np.float64)
        sq = o.signs(_stream_seed(seed, d), d).astype(np.float64)
        x = rng.standard_normal((200, d)).astype(np.float16)
        perm = rng.permutation(d).astype(np.int32)
        for mode, (ba, bb) in HYBRID_BITS.items():
            pk, t = o.hybrid_encode(x, mode, seed, perm, want_t=True)
            off = d // 2 * ba // 8 + d // 2 * bb // 8
            bits = np.unpackbits(pk[:, off:off + d // 8], axis=-1, bitorder="little")
            rho = pk[:, off + d // 8 + 8:].copy().view(np.float32)[:, 0].astype(np.float64)
            ym = _hybrid_mse_only(o, pk, d, mode, seed, perm)[:, perm]   # group order
            r = x.astype(np.float64)[:, perm] - ym
            tt = (r * sq) @ H.T
            assert np.allclose(t, tt, rtol=1e-9, atol=1e-9 * np.abs(tt).max())
            assert np.array_equal(bits, (t < 0).astype(np.uint8))
            assert np.array_equal(rho.astype(np.float32),
                                  np.sqrt((r ** 2).sum(1)).astype(np.float32))
            _, xh = o.hybrid_decode(pk, d, mode, seed, perm, want_f64=True)
            corr = xh[:, perm] - ym
            cn = np.sqrt((corr ** 2).sum(1))
            assert np.allclose(cn, math.sqrt(math.pi / 2) * rho, rtol=1e-10, atol=1e-12)
            ip = (corr * r).sum(1)
            assert np.allclose(ip, math.sqrt(math.pi / 2) / d * rho * np.abs(t).sum(1),
                               rtol=1e-9, atol=1e-12)


def check_hybrid_inner_products_unbiased(o, nseeds=3000):
    """QJL's purpose: the correction is an unbiased estimate of the residual
    in every direction, so over the seeds the hybrid decode's inner product
    with x matches <x, r>-corrected truth: the pooled ratio
    sum <x, correction> / sum <x, r> is 1 within 1.5% (the TurboQuant part
    alone is biased low by the whole <x, r>, 7% of ||x||^2 at tq35 and 23% at
    tq25), and <y, xhat> for independent y has no bias beyond 0.5% of
    ||x|| ||y||."""
    d = D
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, d)).astype(np.float16)
    xd = x.astype(np.float64)
    y = rng.standard_normal((6, d))
    perm = np.arange(d, dtype=np.int32)
    for mode in HYBRID_BITS:
        qx = np.zeros((6, nseeds))
        rx = np.zeros((6, nseeds))
        ey = np.zeros((6, nseeds))
        for s in range(nseeds):
            pk = o.hybrid_encode(x, mode, s, perm)
            _, xh = o.hybrid_decode(pk, d, mode, s, perm, want_f64=True)
            xm = _hybrid_mse_only(o, pk, d, mode, s, perm)
            qx[:, s] = (xd * (xh - xm)).sum(1)
            rx[:, s] = (xd * (xd - xm)).sum(1)
            ey[:, s] = (y * xh).sum(1)
        ratio = qx.sum() / rx.sum()
        assert abs(ratio - 1) < 0.015, (mode, ratio)
        assert rx.mean() > 0.05 * (xd ** 2).sum(1).mean()      # the bias QJL removes is real
        bias_y = np.abs(ey.mean(1) - (y * xd).sum(1)) / (np.linalg.norm(xd, axis=1) *
                                                         np.linalg.norm(y, axis=1))
        assert bias_y.max() < 5e-3, (mode, bias_y)


def check_hybrid_mse(o, n=20000, seed=27):
    """Round trip on N(0,1) vectors: ||x - xhat||^2 / ||x||^2 lies within 5% of
    (pi/2 - 1) times the mean of the two groups' exact TurboQuant values at
    dimension d/2 (the residual keeps (pi/2 - 1) of its energy when its
    projection is Gaussian), and the sign sketch lowers it below the groups'
    value alone."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)).astype(np.float16)
    xd = x.astype(np.float64)
    perm = np.arange(D, dtype=np.int32)
    for mode, (ba, bb) in HYBRID_BITS.items():
        pk = o.hybrid_encode(x, mode, 3, perm)
        _, xh = o.hybrid_decode(pk, D, mode, 3, perm, want_f64=True)
        mse = float(np.mean(((xd - xh) ** 2).sum(1) / (xd ** 2).sum(1)))
        groups = 0.5 * sum(exact_mse_d(b, *o.codebook(b), d=D // 2) for b in (ba, bb))
        assert abs(mse / ((math.pi / 2 - 1) * groups) - 1) < 0.05, (mode, mse, groups)
        xm = _hybrid_mse_only(o, pk, D, mode, 3, perm)
        assert mse < float(np.mean(((xd - xm) ** 2).sum(1) / (xd ** 2).sum(1)))


def check_hybrid_special_cases(o):
    """The zero vector stores zero norms and no sign bits and decodes to zeros;
    encoding x with channel permutation perm equals encoding x[perm] with the
    identity; decode puts group position k back on channel perm[k]."""
    d = D
    z = np.zeros((1, d), np.float16)
    ident = np.arange(d, dtype=np.int32)
    for mode in HYBRID_BITS:
        pk = o.hybrid_encode(z, mode, 1, ident)
        assert np.all(pk[:, -12:] == 0)
        _, xh = o.hybrid_decode(pk, d, mode, 1, ident, want_f64=True)
        assert np.all(xh == 0.0)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, d)).astype(np.float16)
    perm = rng.permutation(d).astype(np.int32)
    for mode in HYBRID_BITS:
        a = o.hybrid_encode(x, mode, 9, perm)
        b = o.hybrid_encode(x[:, perm], mode, 9, ident)
        assert np.array_equal(a, b)
        _, xa = o.hybrid_decode(a, d, mode, 9, perm, want_f64=True)
        _, xb = o.hybrid_decode(b, d, mode, 9, ident, want_f64=True)
        assert np.array_equal(xa[:, perm], xb)


ALL_CHECKS = [
    check_half_to_double, check_double_to_half, check_splitmix64, check_signs,
    check_hadamard, check_rotation_unit_vectors, check_rotation_norm,
    check_codebook_closed_form_b1, check_codebook_structure, check_codebook_centroids,
    check_codebook_distortion, check_codebook_textbook, check_codebook_is_local_minimum,
    check_quantizer_bruteforce, check_quantizer_special_points, check_pack_vectors,
    check_pack_roundtrip, check_sizes, check_mse, check_z_distribution,
    check_scale_invariance, check_negation, check_zero_vector, check_reencode_fixed_point,
    check_decode_definition, check_attn_rotated_domain_identity, check_attn_special_cases,
    check_attn_paging_invariance, check_attn_bruteforce_tiny, check_attn_gqa_grouping,
    check_attn_mixed_widths, check_head_dims, check_attn_head_dims,
    check_hybrid_sizes, check_hybrid_groups_are_turboquant, check_hybrid_qjl_sketch,
    check_hybrid_special_cases, check_hybrid_mse, check_hybrid_inner_products_unbiased,
]
