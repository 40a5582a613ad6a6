/*
 * TurboQuant KV-cache codec -- CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, double-precision
 * definition of what the codec computes.  It is used by the test-suite, by the
 * smoke check and by the CPU-baseline leg of the benchmark, and by nothing else:
 * the product library never links, loads or calls it, and it shares no code,
 * header, table or constant generator with the GPU path.
 *
 * Sources (web pages describing the method):
 *   [PyPI]    pypi.org/project/aither-kvcache -- project page "aither-kvcache";
 *             sections "Algorithm", "API Reference", "Paged KV cache",
 *             "Zero-buffer fused attention", "Benchmarks".
 *   [Crucible] aitherium.github.io/aitherkvcache -- "aitherkvcache -- the
 *             crucible"; hero code sample and "Three engines".
 *   [QBC]     qbc.network/blog/turboquant-efficient-inference; sections
 *             "What TurboQuant is" and "What we shipped, in three layers".
 *
 * Readings where the pages leave a step open (each one is listed in the
 * design notes of the repository):
 *   - sign flip: sigma_i = -1 iff bit 63 of the i-th SplitMix64 output is set
 *     (SplitMix64 as published by Steele, Lea and Flood, 2014);
 *   - rotation R = H * D / sqrt(d), H the Sylvester-ordered Hadamard matrix
 *     H[i][j] = (-1)^popcount(i & j); the codebook is applied to
 *     z = H * D * x / ||x|| = sqrt(d) * R * u, whose coordinates are ~N(0,1);
 *   - codebook: Lloyd-Max quantizer of N(0,1) with 2^b levels, thresholds at
 *     the midpoints, the positive half solved and mirrored;
 *   - a coordinate exactly on a threshold takes the lower level;
 *   - packing: one LSB-first bitstream per vector (code i occupies stream bits
 *     [b*i, b*i+b); stream bit k is bit k%8 of byte k/8);
 *   - zero vector: norm 0, every code L/2-1, decodes to exact zeros;
 *   - attention: plain softmax(scale * q.k) v over [0, context_len), with
 *     GQA kv head = h / (Hq/Hkv) and scale supplied by the caller.
 *
 * Parity status: every function below is pinned by a CPU test against a
 * closed form, a library routine, a published value or brute force
 * (tests/test_oracle_*.py).  No function here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TQO_OK 0
#define TQO_EINVAL 1

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> double                                                  */
/* ------------------------------------------------------------------------ */

/* Exact value of a binary16 bit pattern (every binary16 is a double). */
double tqo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1.m) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a double to binary16, round-to-nearest-even, overflow to +-inf. */
uint16_t tqo_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00; /* 65504 + half an ulp rounds up (odd mantissa) */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24; rint() rounds half to even */
        double q = rint(a * 16777216.0);
        return sign | (uint16_t)q; /* q == 1024 is exactly the smallest normal */
    }
    int E;
    frexp(a, &E);          /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;         /* a in [2^e, 2^(e+1)) */
    double s = ldexp(a, 10 - e); /* exact, in [1024, 2048) */
    double r = rint(s);
    if (r == 2048.0) { r = 1024.0; e += 1; }
    if (e > 15) return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)r - 1024));
}

/* ------------------------------------------------------------------------ */
/* SplitMix64 and the sign vector                                            */
/* ------------------------------------------------------------------------ */

/* One SplitMix64 step: advance the state by the golden-ratio increment, then
 * apply the published finaliser (Steele, Lea, Flood, OOPSLA 2014). */
static uint64_t splitmix64_next(uint64_t *state)
{
    uint64_t z = (*state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* The first n outputs of SplitMix64 started from `seed`. */
void tqo_splitmix64_seq(uint64_t seed, int n, uint64_t *out)
{
    uint64_t s = seed;
    for (int i = 0; i < n; ++i) out[i] = splitmix64_next(&s);
}

/* The fixed random sign flip D = diag(sigma) of the rotation
 * ([PyPI] "Algorithm", step 2: a fixed, data-oblivious random orthogonal
 * matrix; `seed` is the constructor argument of the "API Reference"). */
int tqo_signs(uint64_t seed, int d, int8_t *sigma)
{
    if (d <= 0 || !sigma) return TQO_EINVAL;
    uint64_t s = seed;
    for (int i = 0; i < d; ++i) {
        uint64_t r = splitmix64_next(&s);
        sigma[i] = (r >> 63) ? -1 : 1;
    }
    return TQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Hadamard matrix (plain definition)                                        */
/* ------------------------------------------------------------------------ */

static int popcount_u32(unsigned v)
{
    int c = 0;
    while (v) { c += v & 1u; v >>= 1; }
    return c;
}

/* H[i][j] = (-1)^popcount(i & j), d a power of two (Sylvester order). */
int tqo_hadamard(int d, int8_t *H)
{
    if (d <= 0 || (d & (d - 1)) || !H) return TQO_EINVAL;
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j)
            H[(size_t)i * d + j] = (popcount_u32((unsigned)(i & j)) & 1) ? -1 : 1;
    return TQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max codebook for N(0,1)                                             */
/* ------------------------------------------------------------------------ */

static double std_pdf(double t)
{
    if (isinf(t)) return 0.0;
    return exp(-0.5 * t * t) / sqrt(2.0 * M_PI);
}

/* P(a < X <= b) for X ~ N(0,1), 0 <= a < b <= inf, written with erfc so the
 * tail cells keep their relative precision. */
static double std_mass_pos(double a, double b)
{
    double ua = 0.5 * erfc(a / sqrt(2.0));
    double ub = isinf(b) ? 0.0 : 0.5 * erfc(b / sqrt(2.0));
    return ua - ub;
}

/*
 * Lloyd-Max quantizer for the standard normal with L = 2^bits levels
 * ([PyPI] "Algorithm", step 3: a precomputed Lloyd-Max codebook;
 * [QBC] "What TurboQuant is": the known best levels for a bell curve).
 *
 * Lloyd's conditions: every threshold is the midpoint of its two levels, and
 * every level is the conditional mean of N(0,1) over its cell,
 *   c = (pdf(lo) - pdf(hi)) / (P(hi) - P(lo)).
 * The density is symmetric, so the optimal quantizer is symmetric: only the
 * L/2 positive levels are iterated (their first cell starts at 0) and the
 * negative half is their mirror image, which makes the middle threshold
 * exactly 0 and the codebook exactly symmetric.
 *
 * levels[L] ascending, thresholds[L-1] ascending (thresholds[k] separates
 * levels k and k+1).  Returns the number of iterations used, or -1.
 */
int tqo_codebook(int bits, double *levels, double *thresholds)
{
    if (bits < 1 || bits > 8 || !levels || !thresholds) return -1;
    const int L = 1 << bits;
    const int h = L / 2;
    double p[128], bnd[129];
    /* start: levels spread evenly over (0, 3] */
    for (int j = 0; j < h; ++j) p[j] = 3.0 * (j + 0.5) / h;
    int it;
    for (it = 1; it <= 200000; ++it) {
        bnd[0] = 0.0;
        for (int j = 1; j < h; ++j) bnd[j] = 0.5 * (p[j - 1] + p[j]);
        bnd[h] = INFINITY;
        double change = 0.0;
        for (int j = 0; j < h; ++j) {
            double num = std_pdf(bnd[j]) - std_pdf(bnd[j + 1]);
            double den = std_mass_pos(bnd[j], bnd[j + 1]);
            double c = num / den;
            double dlt = fabs(c - p[j]);
            if (dlt > change) change = dlt;
            p[j] = c;
        }
        if (change <= 2e-15) break; /* a few ulp of the largest level */
    }
    for (int j = 1; j < h; ++j) bnd[j] = 0.5 * (p[j - 1] + p[j]);
    for (int j = 0; j < h; ++j) {
        levels[h + j] = p[j];
        levels[h - 1 - j] = -p[j];
    }
    thresholds[h - 1] = 0.0;
    for (int j = 1; j < h; ++j) {
        thresholds[h - 1 + j] = bnd[j];
        thresholds[h - 1 - j] = -bnd[j];
    }
    return it;
}

/* Mean squared error of the scalar quantizer on N(0,1):
 * E[(X - q(X))^2] = 1 - sum_k c_k^2 P(cell k), valid because every level is
 * its cell's centroid. */
double tqo_codebook_distortion(int bits)
{
    double c[256], t[255];
    if (tqo_codebook(bits, c, t) < 0) return NAN;
    const int L = 1 << bits;
    double acc = 0.0;
    for (int k = L / 2; k < L; ++k) {
        double lo = (k == L / 2) ? 0.0 : t[k - 1];
        double hi = (k == L - 1) ? INFINITY : t[k];
        acc += 2.0 * c[k] * c[k] * std_mass_pos(lo, hi);
    }
    return 1.0 - acc;
}

/* Scalar quantizer ([PyPI] "Algorithm", step 3): the index of the cell that
 * holds z, i.e. the number of thresholds strictly below z.  A value exactly
 * on a threshold therefore takes the lower level. */
int tqo_quantize(double z, const double *thresholds, int L)
{
    int code = 0;
    for (int k = 0; k < L - 1; ++k)
        if (thresholds[k] < z) ++code;
    return code;
}

/* ------------------------------------------------------------------------ */
/* Bit packing ([PyPI] "Algorithm", step 4; [Crucible] hero sample shows     */
/* [...,128] fp16 -> [...,64] uint8 at 4 bits)                               */
/* ------------------------------------------------------------------------ */

/* LSB-first bitstream: code i occupies stream bits [b*i, b*i + b); stream
 * bit k is bit (k % 8) of byte k / 8. */
void tqo_pack(const uint8_t *codes, int d, int bits, uint8_t *out)
{
    int nbytes = d * bits / 8;
    memset(out, 0, (size_t)nbytes);
    for (int i = 0; i < d; ++i)
        for (int q = 0; q < bits; ++q) {
            int k = bits * i + q;
            if ((codes[i] >> q) & 1) out[k / 8] |= (uint8_t)(1u << (k % 8));
        }
}

void tqo_unpack(const uint8_t *in, int d, int bits, uint8_t *codes)
{
    for (int i = 0; i < d; ++i) {
        unsigned c = 0;
        for (int q = 0; q < bits; ++q) {
            int k = bits * i + q;
            c |= (unsigned)((in[k / 8] >> (k % 8)) & 1) << q;
        }
        codes[i] = (uint8_t)c;
    }
}

/* ------------------------------------------------------------------------ */
/* Encode / decode                                                           */
/* ------------------------------------------------------------------------ */

static int valid_shape(int d, int bits)
{
    return d > 0 && d <= 1024 && (d & (d - 1)) == 0 && bits >= 1 && bits <= 8 &&
           (d * bits) % 8 == 0;
}

/* Everything fixed by (d, bits, seed): codebook, signs and the matrix H. */
typedef struct {
    int d, bits, L, P;
    double c[256], t[255];
    int8_t *sg; /* [d] */
    int8_t *H;  /* [d, d] */
} codec_t;

static int codec_init(codec_t *k, int d, int bits, uint64_t seed)
{
    k->d = d; k->bits = bits; k->L = 1 << bits; k->P = d * bits / 8;
    k->sg = malloc((size_t)d);
    k->H = malloc((size_t)d * d);
    if (!k->sg || !k->H) { free(k->sg); free(k->H); return TQO_EINVAL; }
    tqo_codebook(bits, k->c, k->t);
    tqo_signs(seed, d, k->sg);
    tqo_hadamard(d, k->H);
    return TQO_OK;
}

static void codec_free(codec_t *k) { free(k->sg); free(k->H); }

/* One vector: steps 1-5 of encode (see tqo_encode). */
static void encode_one(const codec_t *k, const uint16_t *xv, uint8_t *pv, float *nv_out, double *z)
{
    const int d = k->d;
    double u[1024];
    uint8_t codes[1024];
    double ss = 0.0;
    for (int i = 0; i < d; ++i) {
        double xi = tqo_half_to_double(xv[i]);
        u[i] = xi;
        ss += xi * xi;
    }
    double nv = sqrt(ss);
    *nv_out = (float)nv;
    for (int i = 0; i < d; ++i) u[i] = (nv > 0.0) ? u[i] / nv : 0.0;
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += (double)k->H[(size_t)i * d + j] * k->sg[j] * u[j];
        z[i] = acc;
    }
    for (int i = 0; i < d; ++i) codes[i] = (uint8_t)tqo_quantize(z[i], k->t, k->L);
    tqo_pack(codes, d, k->bits, pv);
}

/* One vector: decode to double (see tqo_decode). */
static void decode_one(const codec_t *k, const uint8_t *pv, float norm, double *xhat)
{
    const int d = k->d;
    uint8_t codes[1024];
    double cv[1024];
    tqo_unpack(pv, d, k->bits, codes);
    for (int j = 0; j < d; ++j) cv[j] = k->c[codes[j]];
    double nv = (double)norm;
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += (double)k->H[(size_t)i * d + j] * cv[j];
        xhat[i] = nv * k->sg[i] * acc / d;
    }
}

/*
 * Encode n vectors of dimension d ([PyPI] "Algorithm", steps 1-5):
 *   1. n_v = ||x||_2 (in double), stored as the f32 nearest to it;
 *   2. u = x / n_v (u = 0 when n_v = 0);
 *   3. z = H * D * u   (so z = sqrt(d) * R * u, R = H D / sqrt(d) orthogonal);
 *   4. code_i = number of thresholds strictly below z_i;
 *   5. codes packed LSB-first, d*bits/8 bytes per vector.
 * x is row-major [n, d] binary16; packed [n, d*bits/8]; norms [n].
 * z_out (optional, [n, d]) receives the double z of step 3.
 */
int tqo_encode(const uint16_t *x, int64_t n, int d, int bits, uint64_t seed,
               uint8_t *packed, float *norms, double *z_out)
{
    if (!valid_shape(d, bits) || n < 0) return TQO_EINVAL;
    if (n == 0) return TQO_OK;
    if (!x || !packed || !norms) return TQO_EINVAL;
    codec_t k;
    if (codec_init(&k, d, bits, seed)) return TQO_EINVAL;
    double z[1024];
    for (int64_t v = 0; v < n; ++v) {
        encode_one(&k, x + v * d, packed + v * k.P, norms + v, z);
        if (z_out) memcpy(z_out + v * d, z, sizeof(double) * d);
    }
    codec_free(&k);
    return TQO_OK;
}

/*
 * Decode ([PyPI] "Algorithm": decoding runs the encode steps backwards):
 *   unpack the codes, look each one up in the codebook, undo the rotation
 *   (R^T = D H / sqrt(d), applied to c/sqrt(d)), multiply by the norm:
 *     xhat = n_v * D * H * c[code] / d.
 * out (optional) receives xhat rounded to binary16 (nearest-even);
 * xhat_out (optional, [n, d]) receives the unrounded double values.
 */
int tqo_decode(const uint8_t *packed, const float *norms, int64_t n, int d, int bits,
               uint64_t seed, uint16_t *out, double *xhat_out)
{
    if (!valid_shape(d, bits) || n < 0) return TQO_EINVAL;
    if (n == 0) return TQO_OK;
    if (!packed || !norms || (!out && !xhat_out)) return TQO_EINVAL;
    codec_t k;
    if (codec_init(&k, d, bits, seed)) return TQO_EINVAL;
    double xh[1024];
    for (int64_t v = 0; v < n; ++v) {
        decode_one(&k, packed + v * k.P, norms[v], xh);
        for (int i = 0; i < d; ++i) {
            if (out) out[v * d + i] = tqo_double_to_half(xh[i]);
            if (xhat_out) xhat_out[v * d + i] = xh[i];
        }
    }
    codec_free(&k);
    return TQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Paged decode attention (plain definition)                                 */
/* ------------------------------------------------------------------------ */

/*
 * Single-token decode attention over a paged, packed K/V cache
 * ([PyPI] "Zero-buffer fused attention" and "Paged KV cache"; argument list of
 * TQPagedAttention.forward in "API Reference").
 *
 * Layout: k_packed/v_packed [num_blocks, block_size, Hkv, P] u8,
 *         k_norms/v_norms   [num_blocks, block_size, Hkv] f32,
 *         block_tables [B, max_blocks] int32, context_lens [B] int32,
 *         q [B, Hq, d] binary16, out [B, Hq, d] binary16.
 * For batch b and query head h (kv head g = h / (Hq/Hkv)), token j < T_b sits
 * in physical block block_tables[b][j / block_size] at row j % block_size.
 * Keys and values are the double-precision decoded rows (never rounded to
 * binary16).  This is the plain definition -- no rotated-domain shortcut --
 * so a fused kernel that works in the rotated domain is checked against the
 * straightforward result:
 *   s_j = scale * <q, k_j>,  p = softmax(s),  o = sum_j p_j v_j.
 * T_b = 0 gives o = 0.  out receives o rounded to binary16 (nearest-even);
 * out_f64 (optional, [B, Hq, d]) receives o unrounded.
 * Only the (b, h) pairs with sel[b * Hq + h] != 0 are computed when sel is
 * non-NULL (the others are left untouched); NULL computes all of them.
 * Keys are decoded with the k_bits codebook and values with the v_bits one
 * (keys and values at different widths, e.g. 4-bit keys with 2-bit values as
 * on the KVarN repository page, "What it does"); both share the seed's
 * rotation.
 */
int tqo_attn_decode_kv(const uint16_t *q, const uint8_t *k_packed, const float *k_norms,
                       const uint8_t *v_packed, const float *v_norms,
                       const int32_t *block_tables, const int32_t *context_lens,
                       int B, int Hq, int Hkv, int d, int k_bits, int v_bits, uint64_t seed,
                       int block_size, int max_blocks, int64_t num_blocks, double scale,
                       const uint8_t *sel, uint16_t *out, double *out_f64)
{
    if (!valid_shape(d, k_bits) || !valid_shape(d, v_bits) || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv ||
        block_size <= 0 || max_blocks < 0 || num_blocks < 0)
        return TQO_EINVAL;
    for (int b = 0; b < B; ++b)
        if (context_lens[b] < 0 || context_lens[b] > max_blocks * block_size) return TQO_EINVAL;
    codec_t k, v;
    if (codec_init(&k, d, k_bits, seed)) return TQO_EINVAL;
    if (codec_init(&v, d, v_bits, seed)) { codec_free(&k); return TQO_EINVAL; }
    const int PK = k.P, PV = v.P;
    const int grp = Hq / Hkv;
    int rc = TQO_OK;
    double qd[1024];
    for (int b = 0; b < B && rc == TQO_OK; ++b) {
        const int T = context_lens[b];
        for (int g = 0; g < Hkv && rc == TQO_OK; ++g) {
            int any = 0;
            for (int hh = 0; hh < grp; ++hh)
                if (!sel || sel[(size_t)b * Hq + g * grp + hh]) any = 1;
            if (!any) continue;
            /* decoded K and V rows of this (sequence, kv head), in token order */
            size_t rows = T > 0 ? (size_t)T : 1;
            double *K = malloc(sizeof(double) * d * rows);
            double *V = malloc(sizeof(double) * d * rows);
            double *s = malloc(sizeof(double) * rows);
            for (int j = 0; j < T; ++j) {
                int32_t blk = block_tables[(size_t)b * max_blocks + j / block_size];
                if (blk < 0 || blk >= num_blocks) { rc = TQO_EINVAL; break; }
                int64_t row = ((int64_t)blk * block_size + j % block_size) * Hkv + g;
                decode_one(&k, k_packed + row * PK, k_norms[row], K + (size_t)j * d);
                decode_one(&v, v_packed + row * PV, v_norms[row], V + (size_t)j * d);
            }
            for (int hh = 0; hh < grp && rc == TQO_OK; ++hh) {
                const int h = g * grp + hh;
                if (sel && !sel[(size_t)b * Hq + h]) continue;
                const size_t ob = ((size_t)b * Hq + h) * d;
                for (int i = 0; i < d; ++i) qd[i] = tqo_half_to_double(q[ob + i]);
                double m = -INFINITY;
                for (int j = 0; j < T; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += qd[i] * K[(size_t)j * d + i];
                    s[j] = scale * acc;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int j = 0; j < T; ++j) { s[j] = exp(s[j] - m); l += s[j]; }
                for (int i = 0; i < d; ++i) {
                    double o = 0.0;
                    for (int j = 0; j < T; ++j) o += s[j] * V[(size_t)j * d + i];
                    o = (T > 0) ? o / l : 0.0;
                    if (out) out[ob + i] = tqo_double_to_half(o);
                    if (out_f64) out_f64[ob + i] = o;
                }
            }
            free(s); free(K); free(V);
        }
    }
    codec_free(&k);
    codec_free(&v);
    return rc;
}

/* The same with one bit width for K and V. */
int tqo_attn_decode(const uint16_t *q, const uint8_t *k_packed, const float *k_norms,
                    const uint8_t *v_packed, const float *v_norms,
                    const int32_t *block_tables, const int32_t *context_lens,
                    int B, int Hq, int Hkv, int d, int bits, uint64_t seed,
                    int block_size, int max_blocks, int64_t num_blocks, double scale,
                    const uint8_t *sel, uint16_t *out, double *out_f64)
{
    return tqo_attn_decode_kv(q, k_packed, k_norms, v_packed, v_norms, block_tables,
                              context_lens, B, Hq, Hkv, d, bits, bits, seed, block_size,
                              max_blocks, num_blocks, scale, sel, out, out_f64);
}

/* Bytes of packed codes per vector. */
int tqo_packed_bytes(int d, int bits)
{
    return valid_shape(d, bits) ? d * bits / 8 : 0;
}

/* ------------------------------------------------------------------------ */
/* Hybrid modes tq35 / tq25 ([PyPI] "Hybrid modes (tq35/tq25)": split-group  */
/* quantization with a QJL residual; "API Reference": HybridTurboQuant with  */
/* calibrate, encode returning the packed bytes only (norms embedded),       */
/* decode, packed_dim_for_mode)                                              */
/* ------------------------------------------------------------------------ */

/*
 * The pages give the mode names, the two-part description and the API; the
 * construction below is this repository's reading of them (listed in the
 * design notes):
 *   - a mode's number is the bits per coordinate of its codes: tq35 = 3.5,
 *     tq25 = 2.5, of which 1 bit is the QJL sign sketch, so the two channel
 *     groups carry (3, 2) bits (tq35) or (2, 1) bits (tq25), 2.5 or 1.5 on
 *     average;
 *   - split groups: a permutation perm of the d channels (chosen by
 *     calibration) puts channels perm[0..d/2) in group A (the more bits) and
 *     perm[d/2..d) in group B; y = x[perm] is the vector in group order;
 *   - each group is a TurboQuant vector of dimension h = d/2 on its own:
 *     norm, sign flip, h-point Walsh-Hadamard transform, Lloyd-Max N(0,1)
 *     code per coordinate, with sign vectors sigma_A = SplitMix64 outputs
 *     [0, h) and sigma_B = outputs [h, d) of the seed;
 *   - QJL residual: r = y - yhat_mse (yhat_mse decoded from the codes and
 *     the stored f32 norms), t = H_d D_Q r with sigma_Q = SplitMix64 outputs
 *     [d, 2d); the sketch keeps the sign bits of t (bit i set iff t_i < 0)
 *     and rho = ||r||.  Decode adds sqrt(pi/2)/d * rho * D_Q H_d s, s_i = +-1
 *     the stored signs: the QJL estimate with the structured random projection
 *     S = H_d D_Q (QJL's projection is Gaussian; this one is the codec's own
 *     kind of random rotation, scaled to the same expected norm);
 *   - row layout (bytes): codes A (h*bA/8) | codes B (h*bB/8) | sign bits
 *     (d/8) | f32 norm_A | f32 norm_B | f32 rho.
 */

static int hybrid_bits(int mode, int *ba, int *bb)
{
    if (mode == 35) { *ba = 3; *bb = 2; return 1; }
    if (mode == 25) { *ba = 2; *bb = 1; return 1; }
    return 0;
}

/* Bytes of one packed row, norms included; 0 for an unsupported shape. */
int tqo_hybrid_packed_bytes(int d, int mode)
{
    int ba, bb;
    if (!hybrid_bits(mode, &ba, &bb) || d < 16 || d > 1024 || (d & (d - 1))) return 0;
    const int h = d / 2;
    return h * ba / 8 + h * bb / 8 + d / 8 + 12;
}

typedef struct {
    int d, h, ba, bb, PA, PB, PQ, row;
    double ca[16], ta[15], cb[16], tb[15];
    int8_t sa[512], sb[512], sq[1024];
    int8_t *Hh, *Hd;
} hybrid_t;

static int hybrid_init(hybrid_t *k, int d, int mode, uint64_t seed)
{
    if (!tqo_hybrid_packed_bytes(d, mode)) return TQO_EINVAL;
    hybrid_bits(mode, &k->ba, &k->bb);
    k->d = d;
    k->h = d / 2;
    k->PA = k->h * k->ba / 8;
    k->PB = k->h * k->bb / 8;
    k->PQ = d / 8;
    k->row = tqo_hybrid_packed_bytes(d, mode);
    tqo_codebook(k->ba, k->ca, k->ta);
    tqo_codebook(k->bb, k->cb, k->tb);
    int8_t s[2048];
    tqo_signs(seed, 2 * d, s);                 /* one stream: A, B, then Q */
    memcpy(k->sa, s, (size_t)k->h);
    memcpy(k->sb, s + k->h, (size_t)k->h);
    memcpy(k->sq, s + d, (size_t)d);
    k->Hh = malloc((size_t)k->h * k->h);
    k->Hd = malloc((size_t)d * d);
    if (!k->Hh || !k->Hd) { free(k->Hh); free(k->Hd); return TQO_EINVAL; }
    tqo_hadamard(k->h, k->Hh);
    tqo_hadamard(d, k->Hd);
    return TQO_OK;
}

static void hybrid_free(hybrid_t *k) { free(k->Hh); free(k->Hd); }

/* TurboQuant of one group of h coordinates (steps 1-5 of the codec at
 * dimension h): returns the f32 norm, writes codes and (optional) z. */
static float group_encode(const hybrid_t *k, const double *y, const int8_t *sg, const double *t,
                          int bits, uint8_t *codes, double *z)
{
    const int h = k->h;
    double ss = 0.0;
    for (int i = 0; i < h; ++i) ss += y[i] * y[i];
    const double n = sqrt(ss);
    for (int i = 0; i < h; ++i) {
        double acc = 0.0;
        for (int j = 0; j < h; ++j)
            acc += (double)k->Hh[(size_t)i * h + j] * sg[j] * ((n > 0.0) ? y[j] / n : 0.0);
        z[i] = acc;
        codes[i] = (uint8_t)tqo_quantize(acc, t, 1 << bits);
    }
    return (float)n;
}

/* yhat of one group: n * D * H_h * c[code] / h. */
static void group_decode(const hybrid_t *k, const uint8_t *codes, const double *c,
                         const int8_t *sg, float norm, double *yh)
{
    const int h = k->h;
    for (int i = 0; i < h; ++i) {
        double acc = 0.0;
        for (int j = 0; j < h; ++j) acc += (double)k->Hh[(size_t)i * h + j] * c[codes[j]];
        yh[i] = (double)norm * sg[i] * acc / h;
    }
}

static void put_f32(uint8_t *p, float v) { memcpy(p, &v, 4); }

/* perm must hold every channel 0..d-1 exactly once. */
static int valid_perm(const int32_t *perm, int d)
{
    uint8_t seen[1024] = {0};
    for (int i = 0; i < d; ++i) {
        if (perm[i] < 0 || perm[i] >= d || seen[perm[i]]) return 0;
        seen[perm[i]] = 1;
    }
    return 1;
}
static float get_f32(const uint8_t *p) { float v; memcpy(&v, p, 4); return v; }

/* The MSE part of a row (both groups) in group order, double. */
static void hybrid_mse(const hybrid_t *k, const uint8_t *pv, double *yh)
{
    uint8_t ca[512], cb[512];
    tqo_unpack(pv, k->h, k->ba, ca);
    tqo_unpack(pv + k->PA, k->h, k->bb, cb);
    const uint8_t *nv = pv + k->PA + k->PB + k->PQ;
    group_decode(k, ca, k->ca, k->sa, get_f32(nv), yh);
    group_decode(k, cb, k->cb, k->sb, get_f32(nv + 4), yh + k->h);
}

/*
 * Encode n vectors (x [n, d] binary16) with the channel permutation perm
 * ([d], perm[k] = the channel at group-order position k) into packed rows
 * [n, tqo_hybrid_packed_bytes(d, mode)].  Optional outputs, [n, d] doubles:
 * z_out (the two groups' rotated coordinates, group A then B) and t_out (the
 * QJL projection H_d D_Q r whose signs are stored).
 */
int tqo_hybrid_encode(const uint16_t *x, int64_t n, int d, int mode, uint64_t seed,
                      const int32_t *perm, uint8_t *packed, double *z_out, double *t_out)
{
    if (n < 0 || !tqo_hybrid_packed_bytes(d, mode)) return TQO_EINVAL;
    if (n == 0) return TQO_OK;
    if (!x || !perm || !packed || !valid_perm(perm, d)) return TQO_EINVAL;
    hybrid_t k;
    if (hybrid_init(&k, d, mode, seed)) return TQO_EINVAL;
    for (int64_t v = 0; v < n; ++v) {
        const uint16_t *xv = x + v * d;
        uint8_t *pv = packed + v * k.row;
        double y[1024], z[1024], yh[1024], r[1024], t[1024];
        uint8_t ca[512], cb[512], bits[1024];
        for (int i = 0; i < d; ++i) y[i] = tqo_half_to_double(xv[perm[i]]);
        memset(pv, 0, (size_t)k.row);
        const float na = group_encode(&k, y, k.sa, k.ta, k.ba, ca, z);
        const float nb = group_encode(&k, y + k.h, k.sb, k.tb, k.bb, cb, z + k.h);
        tqo_pack(ca, k.h, k.ba, pv);
        tqo_pack(cb, k.h, k.bb, pv + k.PA);
        uint8_t *nv = pv + k.PA + k.PB + k.PQ;
        put_f32(nv, na);
        put_f32(nv + 4, nb);
        /* residual of what decode reconstructs from the codes and f32 norms */
        hybrid_mse(&k, pv, yh);
        double rr = 0.0;
        for (int i = 0; i < d; ++i) {
            r[i] = y[i] - yh[i];
            rr += r[i] * r[i];
        }
        put_f32(nv + 8, (float)sqrt(rr));
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j) acc += (double)k.Hd[(size_t)i * d + j] * k.sq[j] * r[j];
            t[i] = acc;
            bits[i] = (acc < 0.0) ? 1 : 0;
        }
        tqo_pack(bits, d, 1, pv + k.PA + k.PB);
        if (z_out) memcpy(z_out + v * d, z, sizeof(double) * d);
        if (t_out) memcpy(t_out + v * d, t, sizeof(double) * d);
    }
    hybrid_free(&k);
    return TQO_OK;
}

/*
 * Decode packed rows: yhat = yhat_mse + sqrt(pi/2)/d * rho * D_Q H_d s
 * (s_i = -1 where sign bit i is set, else +1), then x[perm[k]] = yhat[k].
 * out (optional) binary16 nearest-even; xhat_out (optional) doubles; both
 * [n, d] in channel order.
 */
int tqo_hybrid_decode(const uint8_t *packed, int64_t n, int d, int mode, uint64_t seed,
                      const int32_t *perm, uint16_t *out, double *xhat_out)
{
    if (n < 0 || !tqo_hybrid_packed_bytes(d, mode)) return TQO_EINVAL;
    if (n == 0) return TQO_OK;
    if (!packed || !perm || (!out && !xhat_out) || !valid_perm(perm, d)) return TQO_EINVAL;
    hybrid_t k;
    if (hybrid_init(&k, d, mode, seed)) return TQO_EINVAL;
    const double qscale = sqrt(M_PI / 2.0) / d;
    for (int64_t v = 0; v < n; ++v) {
        const uint8_t *pv = packed + v * k.row;
        double yh[1024];
        uint8_t bits[1024];
        hybrid_mse(&k, pv, yh);
        tqo_unpack(pv + k.PA + k.PB, d, 1, bits);
        const double rho = (double)get_f32(pv + k.PA + k.PB + k.PQ + 8);
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j) acc += (double)k.Hd[(size_t)i * d + j] * (bits[j] ? -1.0 : 1.0);
            yh[i] += qscale * rho * k.sq[i] * acc;
        }
        for (int i = 0; i < d; ++i) {
            const int c = perm[i];
            if (out) out[v * d + c] = tqo_double_to_half(yh[i]);
            if (xhat_out) xhat_out[v * d + c] = yh[i];
        }
    }
    hybrid_free(&k);
    return TQO_OK;
}
