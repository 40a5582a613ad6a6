"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
at least one pin catches each of them.  This is how the pins are shown to be
sensitive: a dropped term, a wrong sign or index, a transposed operand or a
different tie rule must not survive them."""
import os

import pytest

import oracle
import oracle_pins as pins

# (name, text in tq_oracle.c, replacement)
MUTATIONS = [
    ("sign_polarity", "sigma[i] = (r >> 63) ? -1 : 1;", "sigma[i] = (r >> 63) ? 1 : -1;"),
    ("sign_low_bit", "sigma[i] = (r >> 63) ? -1 : 1;", "sigma[i] = (r & 1) ? -1 : 1;"),
    ("splitmix_shift", "z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;",
     "z = (z ^ (z >> 28)) * 0x94d049bb133111ebULL;"),
    ("hadamard_or", "(popcount_u32((unsigned)(i & j)) & 1)", "(popcount_u32((unsigned)(i | j)) & 1)"),
    ("tie_upper", "if (thresholds[k] < z) ++code;", "if (thresholds[k] <= z) ++code;"),
    ("pack_msb_first", "if ((codes[i] >> q) & 1) out[k / 8] |= (uint8_t)(1u << (k % 8));",
     "if ((codes[i] >> q) & 1) out[k / 8] |= (uint8_t)(1u << (7 - k % 8));"),
    ("unpack_msb_first", "c |= (unsigned)((in[k / 8] >> (k % 8)) & 1) << q;",
     "c |= (unsigned)((in[k / 8] >> (7 - k % 8)) & 1) << q;"),
    ("threshold_not_midpoint", "for (int j = 1; j < h; ++j) bnd[j] = 0.5 * (p[j - 1] + p[j]);\n        bnd[h]",
     "for (int j = 1; j < h; ++j) bnd[j] = 0.45 * (p[j - 1] + p[j]);\n        bnd[h]"),
    ("centroid_no_pdf_diff", "double num = std_pdf(bnd[j]) - std_pdf(bnd[j + 1]);",
     "double num = std_pdf(bnd[j]);"),
    ("no_normalise", "u[i] = (nv > 0.0) ? u[i] / nv : 0.0;", "u[i] = u[i];"),
    ("sign_after_hadamard_in_encode",
     "acc += (double)k->H[(size_t)i * d + j] * k->sg[j] * u[j];",
     "acc += (double)k->H[(size_t)i * d + j] * k->sg[i] * u[j];"),
    ("decode_missing_sign", "xhat[i] = nv * k->sg[i] * acc / d;", "xhat[i] = nv * acc / d;"),
    ("decode_sqrt_d", "xhat[i] = nv * k->sg[i] * acc / d;", "xhat[i] = nv * k->sg[i] * acc / sqrt(d);"),
    ("decode_fixed_128", "xhat[i] = nv * k->sg[i] * acc / d;", "xhat[i] = nv * k->sg[i] * acc / 128;"),
    ("decode_transposed_H", "acc += (double)k->H[(size_t)i * d + j] * cv[j];",
     "acc += (double)k->H[(size_t)j * d + (i ^ 1)] * cv[j];"),
    ("norm_f32_truncated", "*nv_out = (float)nv;", "*nv_out = nextafterf((float)nv, 0.0f);"),
    ("half_round_away", "double r = rint(s);", "double r = floor(s + 0.5);"),
    ("attn_no_scale", "s[j] = scale * acc;", "s[j] = acc;"),
    ("attn_values_with_key_codebook",
     "decode_one(&v, v_packed + row * PV, v_norms[row], V + (size_t)j * d);",
     "decode_one(&k, v_packed + row * PV, v_norms[row], V + (size_t)j * d);"),
    ("attn_no_max_sub", "s[j] = exp(s[j] - m);", "s[j] = exp(s[j] - m + 1e-3 * j);"),
    ("attn_gqa_mod", "int64_t row = ((int64_t)blk * block_size + j % block_size) * Hkv + g;",
     "int64_t row = ((int64_t)blk * block_size + j % block_size) * Hkv + (g + 1) % Hkv;"),
    ("attn_page_row", "int64_t row = ((int64_t)blk * block_size + j % block_size) * Hkv + g;",
     "int64_t row = ((int64_t)blk * block_size + (j + 1) % block_size) * Hkv + g;"),
    ("attn_off_by_one_len", "for (int j = 0; j < T; ++j) { s[j] = exp(s[j] - m); l += s[j]; }",
     "for (int j = 0; j < T; ++j) { s[j] = exp(s[j] - m); l += s[j]; }\n                if (T > 1) s[T - 1] = 0.0;"),
    # hybrid modes (split groups + QJL residual)
    ("hybrid_group_bits_swapped", "if (mode == 35) { *ba = 3; *bb = 2; return 1; }",
     "if (mode == 35) { *ba = 2; *bb = 3; return 1; }"),
    ("hybrid_qjl_scale", "const double qscale = sqrt(M_PI / 2.0) / d;",
     "const double qscale = 1.05 * sqrt(M_PI / 2.0) / d;"),
    ("hybrid_qjl_transposed_in_decode",
     "acc += (double)k.Hd[(size_t)i * d + j] * (bits[j] ? -1.0 : 1.0);\n            yh[i] += qscale * rho * k.sq[i] * acc;",
     "acc += (double)k.Hd[(size_t)i * d + j] * k.sq[j] * (bits[j] ? -1.0 : 1.0);\n            yh[i] += qscale * rho * acc;"),
    ("hybrid_qjl_signs_overlap_group_b", "memcpy(k->sq, s + d, (size_t)d);",
     "memcpy(k->sq, s + k->h, (size_t)d);"),
    ("hybrid_sign_bit_polarity", "bits[i] = (acc < 0.0) ? 1 : 0;", "bits[i] = (acc > 0.0) ? 1 : 0;"),
    ("hybrid_rho_squared", "put_f32(nv + 8, (float)sqrt(rr));", "put_f32(nv + 8, (float)rr);"),
    ("hybrid_no_unpermute", "const int c = perm[i];", "const int c = i;"),
    ("hybrid_residual_before_rounding_norms", "hybrid_mse(&k, pv, yh);\n        double rr = 0.0;",
     "hybrid_mse(&k, pv, yh);\n        for (int i = 0; i < d; ++i) yh[i] *= 1.0 + 1e-3;\n        double rr = 0.0;"),
]

# cheap checks first; the Monte-Carlo MSE and the other head dims last
ORDER = sorted(pins.ALL_CHECKS,
               key=lambda f: (f is pins.check_mse) + 2 * (f is pins.check_head_dims))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation anchor must occur exactly once: " + name
    mutant = oracle.build_variant(src.replace(old, new), os.path.join(tmp_path, name + ".so"))
    caught = []
    for check in ORDER:
        try:
            check(mutant)
        except (AssertionError, ValueError) as e:
            caught.append(check.__name__)
            break
    assert caught, "no pin caught the planted mistake " + name
