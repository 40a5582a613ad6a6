// libtq: the C ABI declared in include/tq.h.
//
// Host side only: argument checks, the Lloyd-Max codebook and the sign mask
// (both computed here, on the host, and handed to the kernels by value), and
// the kernel launches.  The library allocates no device memory.
#include "tq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "tq_attn_internal.h"

namespace {

using tq::CodecConsts;


// ---------------------------------------------------------------------------
// Lloyd-Max quantizer of the standard normal (aither-kvcache PyPI page,
// "Algorithm" step 3: a precomputed Lloyd-Max codebook; qbc.network blog,
// "What TurboQuant is": the best fixed levels for a bell curve).
//
// The optimum is symmetric, so only the positive half is solved: interior
// decision points 0 = b_0 < b_1 < ... < b_{h-1} < b_h = inf, levels
// p_j = E[X | b_j < X <= b_{h}] cell means.  This solver iterates on the
// decision points in extended precision: each sweep computes the cell means
// of the current points, then moves every interior point to the midpoint of
// its two neighbouring means, until the points stop moving.
// ---------------------------------------------------------------------------
struct Codebook {
    float level[16];
    float thr[15];
};

long double upper_tail(long double t) {   // P(X > t)
    return 0.5L * std::erfc(t / std::sqrt(2.0L));
}

long double density(long double t) {
    return std::exp(-0.5L * t * t) / std::sqrt(2.0L * 3.141592653589793238462643383279502884L);
}

Codebook solve_codebook(int bits) {
    const int L = 1 << bits, h = L / 2;
    long double b[9], p[8];
    b[0] = 0.0L;
    for (int j = 1; j < h; ++j) b[j] = 4.0L * j / h;   // spread over (0, 4)
    for (int it = 0; it < 1000000; ++it) {
        for (int j = 0; j < h; ++j) {
            const long double lo = b[j];
            const long double dens_hi = (j + 1 < h) ? density(b[j + 1]) : 0.0L;
            const long double mass_hi = (j + 1 < h) ? upper_tail(b[j + 1]) : 0.0L;
            p[j] = (density(lo) - dens_hi) / (upper_tail(lo) - mass_hi);
        }
        long double moved = 0.0L;
        for (int j = 1; j < h; ++j) {
            const long double nb = 0.5L * (p[j - 1] + p[j]);
            const long double dl = std::fabs(nb - b[j]);
            if (dl > moved) moved = dl;
            b[j] = nb;
        }
        if (moved < 1e-17L) break;
    }
    Codebook cb{};
    for (int j = 0; j < h; ++j) {
        cb.level[h + j] = (float)(double)p[j];
        cb.level[h - 1 - j] = -(float)(double)p[j];
    }
    cb.thr[h - 1] = 0.0f;
    for (int j = 1; j < h; ++j) {
        const long double mid = 0.5L * (p[j - 1] + p[j]);
        cb.thr[h - 1 + j] = (float)(double)mid;
        cb.thr[h - 1 - j] = -(float)(double)mid;
    }
    return cb;
}

const Codebook &codebook(int bits) {
    static Codebook cbs[5];
    static std::once_flag once;
    std::call_once(once, [] {
        for (int b = 1; b <= 4; ++b) cbs[b] = solve_codebook(b);   // 1 bit: hybrid tq25
    });
    return cbs[bits];
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): sigma_i = -1 iff the top bit of
// the i-th output is set (i < d; d / 32 mask words).
void sign_mask(uint64_t seed, int d, uint32_t *mask) {
    uint64_t state = seed;
    for (int w = 0; w < d / 32; ++w) mask[w] = 0;
    for (int i = 0; i < d; ++i) {
        state += 0x9e3779b97f4a7c15ULL;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
        z ^= z >> 31;
        if (z >> 63) mask[i >> 5] |= 1u << (i & 31);
    }
}

CodecConsts make_consts(int head_dim, int bits, uint64_t seed) {
    CodecConsts k{};
    sign_mask(seed, head_dim, k.sign);
    const Codebook &cb = codebook(bits);
    const int L = 1 << bits;
    for (int i = 0; i < L; ++i) k.level[i] = cb.level[i];
    return k;
}

// Cells of y = 8 z: cell i > 0 is [i, i+1), i < 0 is (i-1, i], i = 0 is
// (-1, 1).  The narrowest gap between two thresholds at 4 bits is 0.258, i.e.
// 2.07 in y units, so no cell holds more than one threshold.
tq::EncTable make_enc_table(int bits) {
    tq::EncTable t{};
    const Codebook &cb = codebook(bits);
    const int L = 1 << bits;
    for (int c = 0; c < 2 * tq::kEncCells + 1; ++c) {
        const int i = c - tq::kEncCells;
        const float lo = (i > 0) ? float(i) : float(i - 1);
        const float hi = (i < 0) ? float(i) : float(i + 1);
        uint32_t base = 0;
        float thr = INFINITY;
        for (int j = 0; j < L - 1; ++j) {
            const float T = 8.0f * cb.thr[j];
            if (T < lo) ++base;
            else if (T <= hi) thr = T;
        }
        // 4 bits: the four bytes hold base, base + 1, and both shifted into
        // the high nibble, for the kernel's byte-select packing; 2 bits:
        // base and base + 1 in bytes 0 and 1; 3 bits: the plain base code
        uint32_t bb = (bits == 4)   ? (base | (base + 1) << 8 | (base << 4) << 16 |
                                       ((base + 1) << 4) << 24)
                      : (bits == 2) ? (base | (base + 1) << 8)
                                    : base;
        float bf;
        std::memcpy(&bf, &bb, 4);
        t.cell[c] = make_float2(thr, bf);
    }
    return t;
}

const tq::EncTable &enc_table(int bits) {
    static tq::EncTable tabs[5];
    static std::once_flag once;
    std::call_once(once, [] {
        for (int b = 2; b <= 4; ++b) tabs[b] = make_enc_table(b);
    });
    return tabs[bits];
}

// Hybrid modes: the group widths of a mode (35: 3 and 2 bits; 25: 2 and 1).
bool hybrid_widths(int mode, int *ba, int *bb) {
    if (mode == 35) { *ba = 3; *bb = 2; return true; }
    if (mode == 25) { *ba = 2; *bb = 1; return true; }
    return false;
}

// Everything the hybrid kernels take by value.  The seed's SplitMix64 stream
// gives the signs of group-order positions 0..127 (group A then B) and then
// those of the sketch's projection; perm (host, head_dim entries, NULL for
// the identity) becomes the per-lane channel table of the kernels' layout
// (register r of lane q holds group-order position 32 (r / 8) + 8 q + r % 8).
tq::HybridConsts make_hybrid_consts(int mode, uint64_t seed, const int32_t *perm) {
    tq::HybridConsts k{};
    int ba = 0, bb = 0;
    hybrid_widths(mode, &ba, &bb);
    uint32_t words[8];
    sign_mask(seed, 256, words);
    for (int w = 0; w < 4; ++w) {
        k.sign[w] = words[w];
        k.qsign[w] = words[4 + w];
    }
    const Codebook &ca = codebook(ba), &cb = codebook(bb);
    for (int i = 0; i < (1 << ba); ++i) k.lev_a[i] = ca.level[i];
    for (int i = 0; i + 1 < (1 << ba); ++i) k.thr_a[i] = 8.0f * ca.thr[i];
    for (int i = 0; i < (1 << bb); ++i) k.lev_b[i] = cb.level[i];
    for (int i = 0; i + 1 < (1 << bb); ++i) k.thr_b[i] = 8.0f * cb.thr[i];
    uint8_t *g = reinterpret_cast<uint8_t *>(k.gidx);
    for (int q = 0; q < 4; ++q)
        for (int r = 0; r < 32; ++r) {
            const int pos = 32 * (r / 8) + 8 * q + r % 8;
            g[32 * q + r] = (uint8_t)(perm ? perm[pos] : pos);
        }
    return k;
}

// perm holds every channel 0..d-1 exactly once (NULL: the identity)
bool valid_perm(const int32_t *perm, int d) {
    if (!perm) return true;
    bool seen[256] = {};
    for (int i = 0; i < d; ++i) {
        if (perm[i] < 0 || perm[i] >= d || seen[perm[i]]) return false;
        seen[perm[i]] = true;
    }
    return true;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [a, a + na) and [b, b + nb) overlap (sizes in bytes)
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

bool codec_head_dim(int d) { return d == 64 || d == 128 || d == 256; }

// Every entry point takes head_dim 64, 128 or 256 and bits 2, 3 or 4.
tq_status check_shape(int head_dim, int bits) {
    if (head_dim <= 0 || bits <= 0) return TQ_ERR_INVALID_ARG;
    if (!codec_head_dim(head_dim) || bits < 2 || bits > 4) return TQ_ERR_UNSUPPORTED;
    return TQ_OK;
}

tq_status from_hip(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

// Launch extents of the attention kernels: at most 65535 sequences (grid y),
// batch * num_q_heads combine workgroups, and contexts whose token count
// fits an int.
bool attn_extents_ok(int batch, int num_q_heads, int max_blocks_per_seq) {
    return batch <= tq::kAttnMaxBatch && max_blocks_per_seq <= tq::kAttnMaxBlocks &&
           (int64_t)batch * num_q_heads <= 0x7fffffff;
}

}  // namespace

extern "C" {

const char *tq_status_string(tq_status s) {
    switch (s) {
        case TQ_OK: return "TQ_OK";
        case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
        case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
        case TQ_ERR_MISALIGNED: return "TQ_ERR_MISALIGNED";
        case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
        case TQ_ERR_HIP: return "TQ_ERR_HIP";
    }
    return "TQ_ERR_UNKNOWN";
}

int tq_abi_version(void) { return TQ_ABI_VERSION; }

size_t tq_packed_bytes(int head_dim, int bits) {
    if (check_shape(head_dim, bits) != TQ_OK) return 0;
    return (size_t)head_dim * bits / 8;
}

tq_status tq_codebook(int bits, float *levels, float *thresholds) {
    if (bits < 2 || bits > 4) return TQ_ERR_UNSUPPORTED;
    if (!levels || !thresholds) return TQ_ERR_INVALID_ARG;
    const Codebook &cb = codebook(bits);
    const int L = 1 << bits;
    std::memcpy(levels, cb.level, sizeof(float) * L);
    std::memcpy(thresholds, cb.thr, sizeof(float) * (L - 1));
    return TQ_OK;
}

tq_status tq_signs(uint64_t seed, int head_dim, uint32_t *mask) {
    if (!mask || head_dim <= 0) return TQ_ERR_INVALID_ARG;
    if (!codec_head_dim(head_dim)) return TQ_ERR_UNSUPPORTED;
    sign_mask(seed, head_dim, mask);
    return TQ_OK;
}

tq_status tq_encode(const void *x_f16, int64_t n, int head_dim, int bits, uint64_t seed,
                    uint8_t *packed, float *norms, void *stream) {
    tq_status st = check_shape(head_dim, bits);
    if (st != TQ_OK) return st;
    if (n < 0) return TQ_ERR_INVALID_ARG;
    if (n == 0) return TQ_OK;
    if (!x_f16 || !packed || !norms) return TQ_ERR_INVALID_ARG;
    if (!aligned(x_f16, 16) || !aligned(packed, 16) || !aligned(norms, 4))
        return TQ_ERR_MISALIGNED;
    const size_t P = tq_packed_bytes(head_dim, bits);
    const size_t nx = (size_t)n * head_dim * 2, np = (size_t)n * P, nn = (size_t)n * 4;
    if (overlap(x_f16, nx, packed, np) || overlap(x_f16, nx, norms, nn) ||
        overlap(packed, np, norms, nn))
        return TQ_ERR_INVALID_ARG;
    const CodecConsts k = make_consts(head_dim, bits, seed);
    return from_hip(tq::launch_encode(head_dim, bits, x_f16, n, nullptr, 0, k, enc_table(bits),
                                      packed, norms, (hipStream_t)stream));
}

tq_status tq_encode_paged(const void *x_f16, const int64_t *slots, int64_t n, int head_dim,
                          int bits, uint64_t seed, uint8_t *cache_packed, float *cache_norms,
                          int64_t num_slots, void *stream) {
    tq_status st = check_shape(head_dim, bits);
    if (st != TQ_OK) return st;
    if (n < 0 || num_slots < 0) return TQ_ERR_INVALID_ARG;
    if (n == 0) return TQ_OK;
    if (!x_f16 || !slots || !cache_packed || !cache_norms) return TQ_ERR_INVALID_ARG;
    if (!aligned(x_f16, 16) || !aligned(cache_packed, 16) || !aligned(cache_norms, 4) ||
        !aligned(slots, 8))
        return TQ_ERR_MISALIGNED;
    const size_t P = tq_packed_bytes(head_dim, bits);
    const size_t nx = (size_t)n * head_dim * 2, ns = (size_t)n * 8;
    const size_t np = (size_t)num_slots * P, nn = (size_t)num_slots * 4;
    if (overlap(x_f16, nx, cache_packed, np) || overlap(x_f16, nx, cache_norms, nn) ||
        overlap(slots, ns, cache_packed, np) || overlap(slots, ns, cache_norms, nn) ||
        overlap(cache_packed, np, cache_norms, nn))
        return TQ_ERR_INVALID_ARG;
    const CodecConsts k = make_consts(head_dim, bits, seed);
    return from_hip(tq::launch_encode(head_dim, bits, x_f16, n, slots, num_slots, k,
                                      enc_table(bits), cache_packed, cache_norms,
                                      (hipStream_t)stream));
}

tq_status tq_decode(const uint8_t *packed, const float *norms, int64_t n, int head_dim,
                    int bits, uint64_t seed, void *out_f16, void *stream) {
    tq_status st = check_shape(head_dim, bits);
    if (st != TQ_OK) return st;
    if (n < 0) return TQ_ERR_INVALID_ARG;
    if (n == 0) return TQ_OK;
    if (!packed || !norms || !out_f16) return TQ_ERR_INVALID_ARG;
    if (!aligned(out_f16, 16) || !aligned(packed, 16) || !aligned(norms, 4))
        return TQ_ERR_MISALIGNED;
    const size_t P = tq_packed_bytes(head_dim, bits);
    const size_t no = (size_t)n * head_dim * 2, np = (size_t)n * P, nn = (size_t)n * 4;
    if (overlap(out_f16, no, packed, np) || overlap(out_f16, no, norms, nn))
        return TQ_ERR_INVALID_ARG;
    const CodecConsts k = make_consts(head_dim, bits, seed);
    return from_hip(tq::launch_decode(head_dim, bits, packed, norms, n, k, out_f16,
                                      (hipStream_t)stream));
}

size_t tq_hybrid_packed_bytes(int head_dim, int mode) {
    int ba, bb;
    if (head_dim != tq::kHybridHeadDim || !hybrid_widths(mode, &ba, &bb)) return 0;
    return (size_t)tq::hybrid_row_bytes(mode);
}

tq_status tq_hybrid_encode(const void *x_f16, int64_t n, int head_dim, int mode, uint64_t seed,
                           const int32_t *perm, uint8_t *packed, void *stream) {
    const size_t row = tq_hybrid_packed_bytes(head_dim, mode);
    if (head_dim <= 0) return TQ_ERR_INVALID_ARG;
    if (row == 0) return TQ_ERR_UNSUPPORTED;
    if (n < 0 || !valid_perm(perm, head_dim)) return TQ_ERR_INVALID_ARG;
    if (n == 0) return TQ_OK;
    if (!x_f16 || !packed) return TQ_ERR_INVALID_ARG;
    if (!aligned(x_f16, 16) || !aligned(packed, 4)) return TQ_ERR_MISALIGNED;
    if (overlap(x_f16, (size_t)n * head_dim * 2, packed, (size_t)n * row))
        return TQ_ERR_INVALID_ARG;
    return from_hip(tq::launch_hybrid_encode(mode, x_f16, n, make_hybrid_consts(mode, seed, perm),
                                             packed, (hipStream_t)stream));
}

tq_status tq_hybrid_decode(const uint8_t *packed, int64_t n, int head_dim, int mode,
                           uint64_t seed, const int32_t *perm, void *out_f16, void *stream) {
    const size_t row = tq_hybrid_packed_bytes(head_dim, mode);
    if (head_dim <= 0) return TQ_ERR_INVALID_ARG;
    if (row == 0) return TQ_ERR_UNSUPPORTED;
    if (n < 0 || !valid_perm(perm, head_dim)) return TQ_ERR_INVALID_ARG;
    if (n == 0) return TQ_OK;
    if (!packed || !out_f16) return TQ_ERR_INVALID_ARG;
    if (!aligned(out_f16, 16) || !aligned(packed, 4)) return TQ_ERR_MISALIGNED;
    if (overlap(out_f16, (size_t)n * head_dim * 2, packed, (size_t)n * row))
        return TQ_ERR_INVALID_ARG;
    return from_hip(tq::launch_hybrid_decode(mode, packed, n, make_hybrid_consts(mode, seed, perm),
                                             out_f16, (hipStream_t)stream));
}

size_t tq_attn_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || !codec_head_dim(head_dim) ||
        block_size != tq::kAttnBlockSize || max_blocks_per_seq < 0 ||
        num_q_heads % num_kv_heads || !attn_extents_ok(batch, num_q_heads, max_blocks_per_seq))
        return 0;
    tq::AttnShape s{batch, num_q_heads, num_kv_heads, head_dim, 4, 4, max_blocks_per_seq, 0};
    if (!tq::attn_supported(s)) return 0;   // group size beyond what the kernels take
    return tq::attn_workspace_bytes(s);
}

}  // extern "C"

namespace {

// Shared by the attention entry points.  With `own_ws` the workspace is the
// library's static per-device array (the caller passes none), checked
// against its fixed size instead of a caller's buffer.
tq_status attn_decode(const void *q_f16, const uint8_t *k_packed, const float *k_norms,
                      const uint8_t *v_packed, const float *v_norms,
                      const int32_t *block_tables, const int32_t *context_lens, int batch,
                      int num_q_heads, int num_kv_heads, int head_dim, int k_bits, int v_bits,
                      uint64_t seed, int block_size, int max_blocks_per_seq, int64_t num_blocks,
                      float scale, void *out_f16, void *workspace, size_t workspace_bytes,
                      bool own_ws, void *stream) {
    tq_status st = check_shape(head_dim, k_bits);
    if (st != TQ_OK) return st;
    st = check_shape(head_dim, v_bits);
    if (st != TQ_OK) return st;
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 ||
        num_blocks < 0 || !std::isfinite(scale))
        return TQ_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads) return TQ_ERR_INVALID_ARG;
    if (num_q_heads / num_kv_heads > tq::kAttnMaxGroup || block_size != tq::kAttnBlockSize ||
        !attn_extents_ok(batch, num_q_heads, max_blocks_per_seq))
        return TQ_ERR_UNSUPPORTED;
    if (batch == 0) return TQ_OK;
    if (!q_f16 || !out_f16 || !context_lens || (max_blocks_per_seq > 0 && !block_tables))
        return TQ_ERR_INVALID_ARG;
    if (num_blocks > 0 && (!k_packed || !k_norms || !v_packed || !v_norms))
        return TQ_ERR_INVALID_ARG;
    if (!aligned(q_f16, 16) || !aligned(out_f16, 16) || !aligned(k_packed, 16) ||
        !aligned(v_packed, 16) || !aligned(k_norms, 4) || !aligned(v_norms, 4) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
        (!own_ws && !aligned(workspace, 16)))
        return TQ_ERR_MISALIGNED;
    tq::AttnShape s{batch, num_q_heads, num_kv_heads, head_dim, k_bits, v_bits,
                    max_blocks_per_seq, num_blocks};
    if (!tq::attn_supported(s)) return TQ_ERR_UNSUPPORTED;
    const size_t need = tq::attn_workspace_bytes(s);
    if (own_ws) {
        if (need > tq::kAttnStaticWorkspaceBytes) return TQ_ERR_WORKSPACE;
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return TQ_ERR_WORKSPACE;
    }
    // the written arrays (output and a caller's workspace) against each other
    // and against every input
    const size_t nout = (size_t)batch * num_q_heads * head_dim * 2;
    const size_t rows = (size_t)num_blocks * tq::kAttnBlockSize * num_kv_heads;
    const struct { const void *p; size_t n; } in[] = {
        {q_f16, nout},
        {k_packed, rows * tq_packed_bytes(head_dim, k_bits)},
        {k_norms, rows * 4},
        {v_packed, rows * tq_packed_bytes(head_dim, v_bits)},
        {v_norms, rows * 4},
        {block_tables, (size_t)batch * max_blocks_per_seq * 4},
        {context_lens, (size_t)batch * 4},
    };
    const size_t nws = own_ws ? 0 : need;
    if (overlap(out_f16, nout, workspace, nws)) return TQ_ERR_INVALID_ARG;
    for (const auto &a : in)
        if (overlap(out_f16, nout, a.p, a.n) || overlap(workspace, nws, a.p, a.n))
            return TQ_ERR_INVALID_ARG;
    if (own_ws) {
        // the library's array on the current device (looked up on the first
        // call there); no allocation
        if (tq::attn_static_workspace(&workspace) != hipSuccess) return TQ_ERR_HIP;
    }
    const CodecConsts kc = make_consts(head_dim, k_bits, seed);
    const CodecConsts vc = make_consts(head_dim, v_bits, seed);
    return from_hip(tq::launch_attn(s, kc, vc, q_f16, k_packed, k_norms, v_packed, v_norms,
                                    block_tables, context_lens, scale, out_f16, workspace,
                                    (hipStream_t)stream));
}

}  // namespace

extern "C" {

tq_status tq_attn_decode_kv(const void *q_f16, const uint8_t *k_packed, const float *k_norms,
                            const uint8_t *v_packed, const float *v_norms,
                            const int32_t *block_tables, const int32_t *context_lens, int batch,
                            int num_q_heads, int num_kv_heads, int head_dim, int k_bits,
                            int v_bits, uint64_t seed, int block_size, int max_blocks_per_seq,
                            int64_t num_blocks, float scale, void *out_f16, void *workspace,
                            size_t workspace_bytes, void *stream) {
    return attn_decode(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, k_bits, v_bits, seed,
                       block_size, max_blocks_per_seq, num_blocks, scale, out_f16, workspace,
                       workspace_bytes, false, stream);
}

tq_status tq_attn_decode_kv_noalloc(const void *q_f16, const uint8_t *k_packed,
                                    const float *k_norms, const uint8_t *v_packed,
                                    const float *v_norms, const int32_t *block_tables,
                                    const int32_t *context_lens, int batch, int num_q_heads,
                                    int num_kv_heads, int head_dim, int k_bits, int v_bits,
                                    uint64_t seed, int block_size, int max_blocks_per_seq,
                                    int64_t num_blocks, float scale, void *out_f16,
                                    void *stream) {
    return attn_decode(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables, context_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, k_bits, v_bits, seed,
                       block_size, max_blocks_per_seq, num_blocks, scale, out_f16, nullptr, 0,
                       true, stream);
}

tq_status tq_attn_decode(const void *q_f16, const uint8_t *k_packed, const float *k_norms,
                         const uint8_t *v_packed, const float *v_norms,
                         const int32_t *block_tables, const int32_t *context_lens, int batch,
                         int num_q_heads, int num_kv_heads, int head_dim, int bits,
                         uint64_t seed, int block_size, int max_blocks_per_seq,
                         int64_t num_blocks, float scale, void *out_f16, void *workspace,
                         size_t workspace_bytes, void *stream) {
    return tq_attn_decode_kv(q_f16, k_packed, k_norms, v_packed, v_norms, block_tables,
                             context_lens, batch, num_q_heads, num_kv_heads, head_dim, bits,
                             bits, seed, block_size, max_blocks_per_seq, num_blocks, scale,
                             out_f16, workspace, workspace_bytes, stream);
}

}  // extern "C"
