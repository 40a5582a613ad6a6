// Fused single-token decode attention over the packed, paged TurboQuant cache,
// for gfx950.
//
// Method: aither-kvcache PyPI page, "Zero-buffer fused attention" (rotate the
// query forward once, score against codebook values in the rotated domain,
// accumulate the weighted values in the rotated domain, rotate back once) and
// "Paged KV cache" (16-token blocks, [16, heads, P] uint8 + [16, heads] f32
// per block); qbc.network blog, "What we shipped" item 2.  Keys and values may
// use different widths (4-bit keys with 2-bit values: KVarN repository page,
// "What it does").
//
// With R = H D / sqrt(d) and a cached row decoding to n * R^T c[code] / sqrt(d):
//   <q, k_j>      = (n_j / d) * <H D q, c[k_j]>
//   sum_j p_j v_j = D H (sum_j p_j n_j c[v_j]) / d
// so the query is transformed once per (sequence, query head), every cached
// row is used as plain codebook values, and one inverse transform finishes.
//
// Two kernels, flash-decoding style:
//   split   8 waves per workgroup, one per (kv head, context split) of a
//           sequence: a workgroup takes the kv heads of one split, or, for
//           caches with fewer kv heads, all of them for several splits.  Per 16-token page the scores and the value
//           accumulation run as 16x16x32 f16 MFMA tiles:
//             scores  S^T[16 tokens][16 heads] = C_k[16 tokens][K] Q[K][16 heads]
//             values  O[16 heads][16 dims]    += W[16 heads][K] C_v[K][16 dims]
//           with the group's query heads (up to 16) padded to 16.  With at most
//           8 heads per kv head the padding carries the operands' low halves
//           (see below).  One partial state per (sequence, query head, split)
//           goes to the workspace.
//   combine grid (sequence * query head), one wave: log-sum-exp merge of the
//           splits, the inverse transform D H / d, binary16 rounding.
//
// binary16 carries 11 significant bits, too few for the 2e-3 output bound
// under peaked softmaxes, so every operand is split as x = x_hi + x_lo (both
// binary16) and the products x_hi y_hi + x_lo y_hi + x_hi y_lo are formed.
// The split costs no repacking: a code is looked up as the binary16 pair
// (c_hi, c_lo), which fills two adjacent K slots; the other operand holds
// (q_hi, q_hi) in those slots for one product and (q_lo, 0) for a second.
// With at most 8 query heads per kv head both products fit one tile: score
// columns 8-15 and value rows 8-15 hold the low halves of heads 0-7.
//
// Scale factors keep every binary16 operand in range and its low part
// normal: levels are stored times 16, the rotated query times a per-head
// power of two, and the value weights times 2^6 / vlim (vlim a power of two
// above the value norms); all are powers of two and removed exactly before
// the partial state is written.
//
// Lane layouts (l = lane, m = l % 16, r = l / 16), verified on gfx950:
//   A[m][8r .. 8r+7], B[8r .. 8r+7][m], C[4r .. 4r+3][m].
// Scores (head_dim d, G = d / 4): lane (token m, r) holds the codes of dims
// G r .. G r + G - 1 of its token; chunk j covers dims G r + 4j .. +3 of every
// r.  The query operand of lane (head m, r) covers the same dims.  The score
// tile leaves lane (head m, r) with tokens 4r .. 4r+3 -- exactly the K slots
// the value product wants in its A operand, so the weights never move
// between lanes.  Values (N = d / 16 dims per lane column): lane (column m,
// r) reads dims N m .. N m + N - 1 of tokens 4r .. 4r+3; chunk jj
// accumulates dim N m + jj.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tq_attn_internal.h"

namespace tq {
namespace {

// workspace entry per (sequence, query head, split): m, l, acc[head_dim]
constexpr int partial_floats(int head_dim) { return 2 + head_dim; }
constexpr float kLazy = 8.0f;               // rescale when a score passes m + 8 (base 2)
constexpr int kMaxSplitTokens = 4096;       // block-table entries of a split staged in LDS
constexpr int kMWaves = 8;                  // waves per workgroup
constexpr int kMThreads = 64 * kMWaves;
// split-kernel waves aimed for: one full round on MI355X, whose 256 CUs x 4
// SIMDs hold 2 waves each of this kernel with its 8-wave workgroups (170-210
// VGPRs at head_dim 128); measured, 1.5 or 2-3 rounds are slower, half a
// round much slower, and 12-wave workgroups at 168 VGPRs (3 waves per SIMD,
// 3072 waves) slower too
constexpr int kMTargetWaves = 2048;
// Share of a split (in 64ths) that each even split takes from the odd split
// after it when the two share a SIMD (see split_bounds).
constexpr int kSkew64 = 8;
constexpr float kLevelScale = 16.0f;        // binary16 levels are 16 c
constexpr float kWShift = 6.0f;             // value weights carry 2^6
constexpr int kLutRow = 256;                // bytes per table row (64 banks of 4 bytes)
constexpr int kQuadPrev = 0x90;             // quad_perm [0,0,1,2]: lane q <- lane q-1 (0 <- 0)
constexpr int kRowRor8 = 0x128;             // row_ror:8: lane m of a 16-lane row <- lane m ^ 8

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

struct AttnParams {
    const uint16_t *q;
    const uint8_t *kp;
    const float *kn;
    const uint8_t *vp;
    const float *vn;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *ws;
    uint16_t *out;
    int batch, hq, hkv, max_blocks, split_tokens, num_splits;
    int spw;             // splits per workgroup of the split kernel
    int skew;            // tokens moved from each odd split to the even split before it
    int64_t num_blocks;
    float qscale;        // scale * log2(e) / head_dim
    CodecConsts k;       // key codebook and the sign mask (shared by keys and values)
    CodecConsts v;       // value codebook
};

// Token range [t0, t1) of a context split (t1 clipped to the context T).
// Splits are split_tokens long, except that each even split takes `skew`
// more tokens and the odd split after it `skew` fewer: the two run as
// waves w and w + 4 of one workgroup, which share a SIMD, and the SIMD's
// issue arbiter favours the older wave.
__device__ __forceinline__ void split_bounds(const AttnParams &p, int split, int T, int &t0, int &t1) {
    const int odd = split & 1;
    t0 = split * p.split_tokens + (odd ? p.skew : 0);
    const int e = (split + 1) * p.split_tokens + (odd ? 0 : p.skew);
    t1 = e < T ? e : T;
}

// The value of lane l ^ S of a wave (S a power of two below 64).  For S = 16
// and 32 it comes from gfx950's v_permlane16_swap / v_permlane32_swap with
// both operands v: a VALU exchange, where a shuffle through ds_bpermute
// would take an LDS round trip.  permlane16_swap(a, b) trades the odd 16-lane
// rows of a with the even rows of b, so the first result holds row r ^ 1 in
// the odd rows and the second in the even rows; permlane32_swap trades rows
// 2-3 of a with rows 0-1 of b in the same way.
// Within a 16-lane row the exchange is a DPP move: quad permutations for 1
// and 2, the row shifted by 4 lanes one way or the other for 4 (row_shl
// reads lane l + 4, row_shr lane l - 4), the row rotated by 8 for 8.
template <int S>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "power of two below 64");
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const bool hi = (threadIdx.x & S) != 0;
    if constexpr (S == 1) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, u, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    } else if constexpr (S == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, u, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    } else if constexpr (S == 4) {
        const uint32_t up = __builtin_amdgcn_update_dpp(0u, u, 0x104, 0xF, 0xF, false);   // row_shl:4
        const uint32_t dn = __builtin_amdgcn_update_dpp(0u, u, 0x114, 0xF, 0xF, false);   // row_shr:4
        return __builtin_bit_cast(float, hi ? dn : up);
    } else if constexpr (S == 8) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, u, 0x128, 0xF, 0xF, false));  // row_ror:8
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __builtin_bit_cast(float, hi ? r[0] : r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __builtin_bit_cast(float, hi ? r[0] : r[1]);
    }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ int sign_of(const CodecConsts &k, int i) {
    return (k.sign[i >> 5] >> (i & 31)) & 1;
}

// Buffer resource over `bytes` bytes at `base` (wave-uniform).  Loads through
// it take a scalar base and a 32-bit per-lane offset, and read 0 outside the
// range instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t pack_half2(_Float16 a, _Float16 b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// (c_hi, c_lo) of 16 * level[code] as a binary16 pair.
__device__ __forceinline__ uint32_t level_pair(const CodecConsts &k, int code) {
    const float c = k.level[code] * kLevelScale;
    const _Float16 hi = (_Float16)c;
    const _Float16 lo = (_Float16)(c - (float)hi);
    return pack_half2(hi, lo);
}

// Lane m ^ 8 of this lane's 16-lane row.  The value is taken by value:
// clang's __builtin_bit_cast applied directly to an element of an
// ext_vector_type value reads element 0 whatever the element named.
__device__ __forceinline__ float row_ror8(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kRowRor8,
                                                              0xF, 0xF, true));
}

__device__ __forceinline__ f4 mfma(const u32x4 &a, const u32x4 &b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c,
                                                  0, 0, 0);
}

// Code lookup tables.  One table entry turns a group of codes into their
// (c_hi, c_lo) pairs: a byte of two 4-bit codes (8 bytes), a byte of four
// 2-bit codes (16 bytes) or a 6-bit field of two 3-bit codes (8 bytes).
// Entry e of a table fills row e (256 bytes), repeated once per lane of a
// group of 256 / entry-bytes lanes.  gfx950's LDS serves a 64-bit read 32
// lanes at a time (a 128-bit read 16 lanes) over its 64 four-byte banks, so
// the lanes served together always cover every bank once: no bank conflicts,
// whatever the codes.  Keys and values of one width share a codebook and so
// one table; with different widths the value table follows the key table
// (a byte-indexed table sits at a multiple of 64 KB, a 3-bit table at a
// multiple of 16 KB, so the index bits and the table base never overlap).
// For a byte index one v_perm forms the address (byte << 8 | lane offset,
// table base from the lane offset's bits 16-23).
template <int B>
struct Side {
    static constexpr int EB = (B == 2) ? 16 : 8;           // bytes per table entry
    static constexpr int NE = (B == 3) ? 64 : 256;         // table entries
    static constexpr int COPIES = kLutRow / EB;            // lane copies per row
    static constexpr int BYTES = NE * kLutRow;
};

// LDS placement of the key and value tables for widths KB, VB.
template <int KB, int VB>
struct Tables {
    static constexpr bool SHARED = KB == VB;
    // a byte-indexed table first, at 0; the other one at 64 KB
    static constexpr int KOFF = SHARED ? 0 : (KB == 3 ? 65536 : 0);
    static constexpr int VOFF = SHARED ? 0 : (KB == 3 ? 0 : 65536);
    static constexpr int BYTES = SHARED ? Side<KB>::BYTES
                                        : 65536 + (KB == 3 ? Side<KB>::BYTES : Side<VB>::BYTES);
};

// Thread t = 64 w + l writes 16-byte piece l % 16 of entries e = 32 i + 4 w + r
// (r = l / 16, i < NE / 32).  Every code index is then either wave-uniform,
// read as a scalar, or a uniform base plus r, one of four scalars: the table
// needs no per-lane load, so it is built without waiting on the vector loads
// the kernel has in flight.
template <int B>
__device__ __forceinline__ void fill_table(char *tab, const CodecConsts &k) {
    using S = Side<B>;
    constexpr int IT = S::NE * (kLutRow / 16) / kMThreads;
    static_assert(IT * kMThreads == S::NE * (kLutRow / 16), "whole rounds of the workgroup");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = (threadIdx.x >> 4) & 3, c = threadIdx.x & 15;
    auto lvl = [&](int code) -> uint32_t {        // code wave-uniform
        return level_pair(k, __builtin_amdgcn_readfirstlane(code));
    };
    auto lane_lvl = [&](int base) -> uint32_t {   // code base + r
        const uint32_t a0 = lvl(base), a1 = lvl(base + 1), a2 = lvl(base + 2), a3 = lvl(base + 3);
        return r == 0 ? a0 : (r == 1 ? a1 : (r == 2 ? a2 : a3));
    };
    // 4 bits: codes e % 16 = 4 (w % 4) + r and e / 16 = 2 i + w / 4; 3 bits:
    // e % 8 = 4 (w % 2) + r and e / 8 = 4 i + w / 2; 2 bits: e % 4 = r,
    // (e / 4) % 4 = w % 4, (e / 16) % 4 = (2 i + w / 4) % 4, e / 64 = i / 2
    const uint32_t a = (B == 4) ? lane_lvl(4 * (w & 3)) : (B == 3 ? lane_lvl(4 * (w & 1)) : lane_lvl(0));
    const uint32_t b2 = (B == 2) ? lvl(w & 3) : 0u;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = 32 * i + 4 * w + r;
        u32x4 v;
        if constexpr (B == 2) {
            v = u32x4{a, b2, lvl((2 * i + (w >> 2)) & 3), lvl(i >> 1)};
        } else {
            const uint32_t hi = (B == 4) ? lvl(2 * i + (w >> 2)) : lvl(4 * i + (w >> 1));
            v = u32x4{a, hi, a, hi};
        }
        *reinterpret_cast<u32x4 *>(tab + e * kLutRow + 16 * c) = v;
    }
}

template <int K>
__device__ __forceinline__ uint32_t byte_addr(uint32_t word, uint32_t laneoff) {
    return __builtin_amdgcn_perm(word, laneoff, 0x0C020000u | ((4u + K) << 8));
}

// Pairs of the codes in byte K of `word` (4-bit codes: 2 pairs).
template <int K>
__device__ __forceinline__ u32x2 lut8(const char *tab, uint32_t word, uint32_t laneoff) {
    return *reinterpret_cast<const u32x2 *>(tab + byte_addr<K>(word, laneoff));
}
// Pairs of the codes in byte K of `word` (2-bit codes: 4 pairs).
template <int K>
__device__ __forceinline__ u32x4 lut16(const char *tab, uint32_t word, uint32_t laneoff) {
    return *reinterpret_cast<const u32x4 *>(tab + byte_addr<K>(word, laneoff));
}
// Pairs of the two 3-bit codes in a 6-bit field.
__device__ __forceinline__ u32x2 lut8f(const char *tab, uint32_t field, uint32_t laneoff) {
    return *reinterpret_cast<const u32x2 *>(tab + ((field << 8) | laneoff));
}

// Bits [b, b + 6) of the little-endian bit string w[0], w[1], ...
template <int b, int N>
__device__ __forceinline__ uint32_t field6(const uint32_t (&w)[N]) {
    constexpr int wi = b >> 5, sh = b & 31;
    if constexpr (sh <= 26) return (w[wi] >> sh) & 63u;
    else return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & 63u;
}

// A operand of score chunk J: dims 4J .. 4J+3 of the lane's slice of its
// token, as (c_hi, c_lo) pairs, from the lane's packed key words kc.
template <int J, int KB, int N>
__device__ __forceinline__ u32x4 key_chunk(const char *tab, const uint32_t (&kc)[N], uint32_t laneoff) {
    if constexpr (KB == 4) {             // bytes 2J, 2J+1
        const u32x2 a0 = lut8<(2 * J) & 3>(tab, kc[J >> 1], laneoff);
        const u32x2 a1 = lut8<(2 * J + 1) & 3>(tab, kc[J >> 1], laneoff);
        return u32x4{a0.x, a0.y, a1.x, a1.y};
    } else if constexpr (KB == 2) {      // byte J
        return lut16<J & 3>(tab, kc[J >> 2], laneoff);
    } else {                             // bits 12J .. 12J+11
        const u32x2 a0 = lut8f(tab, field6<12 * J>(kc), laneoff);
        const u32x2 a1 = lut8f(tab, field6<12 * J + 6>(kc), laneoff);
        return u32x4{a0.x, a0.y, a1.x, a1.y};
    }
}

// One score chain over NJ chunks: columns 0-7 carry (q_hi, q_hi) of heads
// 0-7 and columns 8-15 carry (q_lo, 0) of the same heads (at most 8 query
// heads per kv head).
template <int J, int NJ, int KB, int N>
__device__ __forceinline__ void score_chunks_paired(const char *tab, const uint32_t (&kc)[N],
                                                    uint32_t laneoff, const u32x4 (&bq)[NJ],
                                                    f4 &S) {
    S = mfma(key_chunk<J, KB>(tab, kc, laneoff), bq[J], S);
    if constexpr (J + 1 < NJ) score_chunks_paired<J + 1, NJ, KB>(tab, kc, laneoff, bq, S);
}

template <int J, int NJ, int KB, int N>
__device__ __forceinline__ void score_chunks(const char *tab, const uint32_t (&kc)[N], uint32_t laneoff,
                                             const u32x4 (&bq1)[NJ], const u32x4 (&bq2)[NJ],
                                             f4 &S0, f4 &S1) {
    const u32x4 A = key_chunk<J, KB>(tab, kc, laneoff);
    S0 = mfma(A, bq1[J], S0);
    S1 = mfma(A, bq2[J], S1);
    if constexpr (J + 1 < NJ) score_chunks<J + 1, NJ, KB>(tab, kc, laneoff, bq1, bq2, S0, S1);
}

// Value operand builders: Bv[jj] holds value dim jj of the lane's slice for
// tokens 4r .. 4r+3, as (c_hi, c_lo) pairs; vc[i] is the lane's packed value
// bits for token 4r + i.
// 4-bit values: the index bytes pair two tokens' codes of one dim, so one
// lookup (the same byte -> two-code table as the keys') returns the (c_hi,
// c_lo) pairs of both tokens, already in the order of the operand's K slots.
// x[p] byte k: dim 2k of tokens 2p (low nibble) and 2p + 1 (high nibble);
// y[p] byte k: dim 2k + 1.
template <int K, int NJJ>
__device__ __forceinline__ void value_pairs4(const char *tab, const uint32_t (&x)[2],
                                             const uint32_t (&y)[2], uint32_t laneoff,
                                             u32x4 (&Bv)[NJJ]) {
    const u32x2 e0 = lut8<K>(tab, x[0], laneoff), e1 = lut8<K>(tab, x[1], laneoff);
    const u32x2 o0 = lut8<K>(tab, y[0], laneoff), o1 = lut8<K>(tab, y[1], laneoff);
    Bv[2 * K] = u32x4{e0.x, e0.y, e1.x, e1.y};
    Bv[2 * K + 1] = u32x4{o0.x, o0.y, o1.x, o1.y};
}

template <int K, int K0, int NJJ>
__device__ __forceinline__ void value_bytes2(const char *tab, const uint32_t (&vc)[4],
                                             uint32_t laneoff, u32x4 (&Bv)[NJJ]) {
    u32x4 L[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) L[i] = lut16<K>(tab, vc[i], laneoff);
#pragma unroll
    for (int t = 0; t < 4; ++t) Bv[4 * (K - K0) + t] = u32x4{L[0][t], L[1][t], L[2][t], L[3][t]};
}

// 3-bit values: v[i] holds the lane's fields (NJJ / 2 fields of two codes)
// from bit 0 up.
template <int NJJ>
__device__ __forceinline__ void value_fields3(const char *tab, const uint32_t (&v)[4],
                                              uint32_t laneoff, u32x4 (&Bv)[NJJ]) {
#pragma unroll
    for (int s = 0; s < NJJ / 2; ++s) {  // field s: dims 2s, 2s+1
        u32x2 L[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) L[i] = lut8f(tab, (v[i] >> (6 * s)) & 63u, laneoff);
        Bv[2 * s] = u32x4{L[0].x, L[1].x, L[2].x, L[3].x};
        Bv[2 * s + 1] = u32x4{L[0].y, L[1].y, L[2].y, L[3].y};
    }
}

// The value operands of the page for a slice of NT dims per lane column
// (4-bit NT / 2 bytes, 2-bit NT / 4 bytes, 3-bit 3 NT / 8 bytes), built NB =
// min(NT, 8) dims at a time: Bv[jj] is dim 8 H + jj of the slice.  vc holds
// VW words per token as loaded (see the value loads in the split kernel);
// vsh is the 3-bit field's bit offset within them.
template <int NT, int VB, int VW, int H = 0>
__device__ __forceinline__ void value_operands(const char *tab, const uint32_t (&vc)[4][VW],
                                               uint32_t laneoff, int q4, uint32_t vsh,
                                               u32x4 (&Bv)[NT > 8 ? 8 : NT]) {
    constexpr int NB = NT > 8 ? 8 : NT;
    if constexpr (VB == 4) {             // word H: dims 8H .. 8H+7
        uint32_t x[2], y[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t a = vc[2 * p][H], b = vc[2 * p + 1][H];
            x[p] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
            y[p] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
        }
        value_pairs4<0>(tab, x, y, laneoff, Bv);
        value_pairs4<1>(tab, x, y, laneoff, Bv);
        if constexpr (NB == 8) {
            value_pairs4<2>(tab, x, y, laneoff, Bv);
            value_pairs4<3>(tab, x, y, laneoff, Bv);
        }
    } else if constexpr (VB == 2) {      // bytes 2H, 2H+1
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = vc[i][0];
        value_bytes2<2 * H, 2 * H>(tab, w, laneoff, Bv);
        if constexpr (NB == 8) value_bytes2<2 * H + 1, 2 * H>(tab, w, laneoff, Bv);
    } else if constexpr (NT == 8) {
        // 24 bits at bit 24m of the slice.  Lanes m = 4a .. 4a+3 of a quad
        // loaded dwords 3a, 3a+1, 3a+2, 3a+2; lane q's field starts in the
        // dword of lane q-1 (lane 0: its own) at bit 24q mod 32.
        const uint32_t sh = (24u * (uint32_t)q4) & 31u;
        uint32_t v24[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t prev = (uint32_t)__builtin_amdgcn_mov_dpp((int)vc[i][0], kQuadPrev, 0xF, 0xF, true);
            const uint32_t lo = q4 == 0 ? vc[i][0] : prev;
            v24[i] = __builtin_amdgcn_alignbit(vc[i][0], lo, sh);
        }
        value_fields3<NB>(tab, v24, laneoff, Bv);
    } else {
        // 3 NT bits at bit 3 NT m of the slice (12 at NT = 4, 48 at NT = 16),
        // inside the two dwords the lane loaded from the dword that holds its
        // first bit; half H takes bits 24H .. 24H+23
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = __builtin_amdgcn_alignbit(vc[i][VW - 1], vc[i][0], vsh);
            if constexpr (H == 0) v[i] = lo;
            else v[i] = __builtin_amdgcn_alignbit(vc[i][VW - 1] >> vsh, lo, 24);
        }
        value_fields3<NB>(tab, v, laneoff, Bv);
    }
}

// PAIRED (at most 8 query heads per kv head): the low halves of the split
// operands ride in the otherwise padded half of each tile -- score columns
// and value rows 8-15 belong to heads 0-7 -- so each page takes 8 + 8 matrix
// products instead of 16 + 16.  Otherwise (9-16 heads) the low halves take a
// second product per tile.
// Shape of the split kernel's per-lane slices for head dimension D.
template <int D, int KB, int VB>
struct Slices {
    static constexpr int DG = D / 4;                  // score dims per lane row group r
    static constexpr int NJ = DG / 4;                 // score chunks (4 dims each)
    static constexpr int KBY = DG * KB / 8;           // key bytes per lane and token
    // key words per lane: the slice, or at D = 64 and 3 bits (6 bytes at a
    // 2-byte offset) the two dwords around it
    static constexpr int KW = (KBY % 4) ? 2 : KBY / 4;
    static constexpr int NJJ = D / 16;                // value dims per lane column
    // value words per lane and token: one; two for 4 bits at D = 256 (8
    // bytes), and for 3 bits at D = 64 and 256 (12 or 48 bits at bit 3 NJJ m,
    // not dword-aligned: the two dwords from the one holding the first bit)
    static constexpr int VW = ((VB == 3 && NJJ != 8) || (VB == 4 && NJJ == 16)) ? 2 : 1;
    static constexpr int NB = NJJ > 8 ? 8 : NJJ;      // value operands built at a time
    static constexpr int PK = D * KB / 8;             // packed bytes per key row
    static constexpr int PV = D * VB / 8;
};

// Loads of the lane's packed key words for one token (n bytes at `off`; at
// D = 64 and 3 bits the 8 bytes from the dword holding the slice's start).
template <int KBY, int KW>
__device__ __forceinline__ void load_key(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t (&kc)[KW]) {
    if constexpr (KBY == 4) {
        kc[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
    } else if constexpr (KBY == 8 || KBY == 6) {
        const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
        kc[0] = t.x;
        kc[1] = t.y;
    } else if constexpr (KBY == 12) {
        const u32x3 t = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0));
        kc[0] = t.x;
        kc[1] = t.y;
        kc[2] = t.z;
    } else {
        static_assert(KBY % 16 == 0 || KBY == 24, "key slice size");
#pragma unroll
        for (int c = 0; c < KBY / 16; ++c) {
            const u32x4 t = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * c, 0, 0));
            kc[4 * c] = t.x;
            kc[4 * c + 1] = t.y;
            kc[4 * c + 2] = t.z;
            kc[4 * c + 3] = t.w;
        }
        if constexpr (KBY % 16) {
            const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 16u * (KBY / 16), 0, 0));
            kc[KW - 2] = t.x;
            kc[KW - 1] = t.y;
        }
    }
}

// PAIRED (at most 8 query heads per kv head): the low halves of the split
// operands ride in the otherwise padded half of each tile -- score columns
// and value rows 8-15 belong to heads 0-7 -- so each page takes NJ + NJJ
// matrix products instead of twice that.  Otherwise (9-16 heads) the low
// halves take a second product per tile.
//
// Head dimension D: lane row group r holds score dims D/4 r .. D/4 r + D/4 - 1,
// and lane column m accumulates value dims D/16 m .. D/16 m + D/16 - 1.  At
// D = 256 the value operands are built and multiplied 8 dims at a time.
//
// KVW kv heads per wave (KVW = 2: at most 4 query heads per kv head, head_dim
// up to 128).  The 8 head slots of the paired tile then hold the query heads
// of two kv heads, g (slots 0-3) and g + 1 (slots 4-7), so no column is
// padding: each kv head's keys form their own score chain against the
// shared query operand and a lane keeps the chain of its column's kv head;
// the value products run once per kv head, with the other kv head's weight
// rows zero.  Per kv head the matrix products are those of KVW = 1, the
// softmax arithmetic is halved, and each wave reads whole 128-byte lines.
template <int D, int KB, int VB, bool PAIRED, int KVW>
__global__ __launch_bounds__(kMThreads) void attn_split_kernel(AttnParams p) {
    static_assert(KVW == 1 || (KVW == 2 && PAIRED && D <= 128), "two kv heads per wave: paired, d <= 128");
    using SK = Side<KB>;
    using SV = Side<VB>;
    using SL = Slices<D, KB, VB>;
    constexpr int DG = SL::DG, NJ = SL::NJ, NJJ = SL::NJJ, NB = SL::NB;
    constexpr int partial = 2 + D;
    using TB = Tables<KB, VB>;
    __shared__ __attribute__((aligned(256))) char tab[TB::BYTES];
    __shared__ int32_t bt_all[kMWaves][kMaxSplitTokens / kAttnBlockSize];

    // The workgroup's waves form p.spw slots of kMWaves / p.spw units of
    // KVW kv heads; slot s works on split blockIdx.x * p.spw + s (several
    // splits per workgroup when the cache has fewer kv-head units than waves).
    const int b = blockIdx.y;
    int T = p.context_lens[b];
    T = T < 0 ? 0 : T;
    const int tmax = p.max_blocks * kAttnBlockSize;
    T = T > tmax ? tmax : T;
    if (p.num_blocks <= 0) T = 0;
    const int hps = kMWaves / p.spw;                          // kv-head units per slot
    const int first = blockIdx.x * p.spw;
    if (first * p.split_tokens >= T) return;                 // the whole workgroup is past the context

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = wave;                                    // kv-head unit
    const int slot = unit / hps;
    const int g = (blockIdx.z * hps + unit % hps) * KVW;      // (first) kv head
    const int split = first + slot;
    int t0, t1;
    split_bounds(p, split, T, t0, t1);
    const bool live = g < p.hkv && t0 < T;                    // wave-uniform
    const int npages = live ? (t1 - t0 + kAttnBlockSize - 1) / kAttnBlockSize : 0;
    const int32_t *bt_lds = bt_all[slot];
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, r = lane >> 4;
    const int grp = p.hq / p.hkv;
    const int hcol = PAIRED ? (m & 7) : m;                    // head slot of this lane's column
    const bool lo_col = PAIRED && m >= 8;                     // a column of low halves
    const int kvs = KVW == 2 ? (hcol >> 2) : 0;               // the column's kv head: g + kvs
    const int hh = KVW == 2 ? (hcol & 3) : hcol;              // its query head within the kv head's group
    const bool hv = hh < grp;                                 // a real query head column
    const uint32_t lok = TB::KOFF + (uint32_t)(lane & (SK::COPIES - 1)) * SK::EB;
    const uint32_t lov = TB::VOFF + (uint32_t)(lane & (SV::COPIES - 1)) * SV::EB;

    // per-lane byte offsets inside one page of this kv head
    const uint32_t rowk = (uint32_t)p.hkv * SL::PK;           // one token of all kv heads
    const uint32_t rowv = (uint32_t)p.hkv * SL::PV;
    const uint32_t kslice = (uint32_t)SL::KBY * r;            // the slice's byte offset in the row
    const uint32_t offk = (uint32_t)m * rowk + (uint32_t)g * SL::PK + (kslice & ~3u);
    const uint32_t ksh = (kslice & 3u) * 8u;                  // 3 bits at D = 64: 0 or 16
    const int q4 = m & 3;
    const uint32_t vsh = (3u * NJJ * (uint32_t)m) & 31u;      // 3 bits at D = 64, 256
    uint32_t offv[4], offn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t row = (uint32_t)(4 * r + i) * rowv + (uint32_t)g * SL::PV;
        if (VB == 4) offv[i] = row + (uint32_t)(NJJ / 2) * m;
        else if (VB == 2) offv[i] = row + (uint32_t)(NJJ / 4) * m;
        else if (NJJ == 8) offv[i] = row + 4u * (3u * (uint32_t)(m >> 2) + (uint32_t)(q4 < 2 ? q4 : 2));
        else offv[i] = row + 4u * ((3u * NJJ * (uint32_t)m) >> 5);
        offn[i] = ((uint32_t)(4 * r + i) * p.hkv + g + kvs) * 4u;   // the column's kv head
    }
    const uint32_t pagek = kAttnBlockSize * rowk;
    const uint32_t pagev = kAttnBlockSize * rowv;
    const uint32_t pagen = kAttnBlockSize * p.hkv * 4u;

    // Ring of two page slots: even pages in slot 0, odd pages in slot 1.  The
    // pages are taken two at a time: the scores of both, one softmax update
    // for both, then the value products of each.  A slot's key words are
    // refilled (with the page two further on) as soon as its scores are
    // formed, its value words and norms once its value products are issued,
    // so each load has about one pair of pages of work in which to arrive.
    // The loads are unconditional (a page past the split re-reads the split's
    // last page, an L2 hit): straight-line loads let every wait for a page
    // leave the later pages' loads in flight.  (At D = 256 the kernel fills
    // the 256 VGPRs that keep 2 waves per SIMD; with 4-bit keys and 3-bit
    // values two values are spilled.)
    constexpr int KW = SL::KW, VW = SL::VW;
    uint32_t rk[2][KVW][KW];
    uint32_t rv[2][KVW][4][VW];
    float rkn[2][4], rvn[2][4];
    bool rok[2];
    auto fetch_keys = [&](int32_t blk, int slot) {     // blk wave-uniform
        blk = (blk >= 0 && blk < p.num_blocks) ? blk : 0;
        const __amdgpu_buffer_rsrc_t rsk = page_rsrc(p.kp + (size_t)blk * pagek, pagek);
#pragma unroll
        for (int kv = 0; kv < KVW; ++kv)     // kv head g + kv: SL::PK bytes further in the row
            load_key<SL::KBY, KW>(rsk, offk + kv * SL::PK, rk[slot][kv]);
    };
    auto fetch_values = [&](int pg, int32_t blk, int slot) {   // blk wave-uniform
        rok[slot] = pg < npages && blk >= 0 && blk < p.num_blocks;
        blk = (blk >= 0 && blk < p.num_blocks) ? blk : 0;
        const __amdgpu_buffer_rsrc_t rsv = page_rsrc(p.vp + (size_t)blk * pagev, pagev);
        const __amdgpu_buffer_rsrc_t rkn_ = page_rsrc(p.kn + (size_t)blk * kAttnBlockSize * p.hkv, pagen);
        const __amdgpu_buffer_rsrc_t rvn_ = page_rsrc(p.vn + (size_t)blk * kAttnBlockSize * p.hkv, pagen);
#pragma unroll
        for (int kv = 0; kv < KVW; ++kv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t ov = offv[i] + kv * SL::PV;
                if constexpr (VW == 2) {
                    const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsv, ov, 0, 0));
                    rv[slot][kv][i][0] = t.x;
                    rv[slot][kv][i][VW - 1] = t.y;
                } else if constexpr (VB == 2 && NJJ == 4) {
                    rv[slot][kv][i][0] = __builtin_amdgcn_raw_buffer_load_b8(rsv, ov, 0, 0);
                } else if constexpr ((VB == 2 && NJJ == 8) || (VB == 4 && NJJ == 4)) {
                    rv[slot][kv][i][0] = __builtin_amdgcn_raw_buffer_load_b16(rsv, ov, 0, 0);
                } else {
                    rv[slot][kv][i][0] = __builtin_amdgcn_raw_buffer_load_b32(rsv, ov, 0, 0);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rkn[slot][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkn_, offn[i], 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rvn[slot][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvn_, offn[i], 0, 0));
    };
    auto bt_at = [&](int pg) -> int32_t {
        return __builtin_amdgcn_readfirstlane(bt_lds[pg < npages ? pg : npages - 1]);
    };

    // Vector loads count down in issue order, so a load the prologue uses must
    // be issued before the first pages' loads, or using it would wait for
    // them too: first the lane's query slice and the block-table entries of
    // the wave's slot (copied to LDS by the slot's waves), then the first two
    // pages, whose block ids are read straight from the block table, so that
    // they arrive while the tables are built and the query is rotated.
    // Every one of these loads is issued unconditionally, at a valid address
    // (a wave without work reads the first query, the start of the block
    // table and block 0), so that no path merge makes the compiler wait for
    // all loads at once.
    constexpr int QV = DG / 8;                                // 16-byte pieces of the query slice
    u32x4 qraw[QV];
    {
        // padding columns read head 0, then drop it
        const uint16_t *qp = live ? p.q + ((size_t)b * p.hq + (size_t)(g + kvs) * grp + (hv ? hh : 0)) * D + DG * r
                                  : p.q;
#pragma unroll
        for (int j = 0; j < QV; ++j) qraw[j] = reinterpret_cast<const u32x4 *>(qp)[j];
    }
    int s0, s1;
    split_bounds(p, first + slot, T, s0, s1);
    const int np_slot = s0 < T ? (s1 - s0 + kAttnBlockSize - 1) / kAttnBlockSize : 0;
    const int32_t *bts = p.block_tables + (size_t)b * p.max_blocks + (np_slot > 0 ? s0 / kAttnBlockSize : 0);
    constexpr int kCopy = kMaxSplitTokens / kAttnBlockSize / 64;   // entries per lane at one wave per slot
    const int cbase = (unit % hps) * 64 + lane, cstride = hps * 64;
    int32_t bv[kCopy];
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
        const int i = cbase + k * cstride;
        bv[k] = bts[i < np_slot ? i : 0];
    }
    {
        const int32_t *btg = p.block_tables + (size_t)b * p.max_blocks + (live ? t0 / kAttnBlockSize : 0);
        const int32_t b0 = __builtin_amdgcn_readfirstlane(btg[0]);
        const int32_t b1 = __builtin_amdgcn_readfirstlane(btg[npages > 1 ? 1 : 0]);
        fetch_keys(b0, 0);
        fetch_values(0, b0, 0);
        fetch_keys(b1, 1);
        fetch_values(1, b1, 1);
    }

    fill_table<KB>(tab + TB::KOFF, p.k);
    if constexpr (!TB::SHARED) fill_table<VB>(tab + TB::VOFF, p.v);
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
        const int i = cbase + k * cstride;
        if (i < np_slot) bt_all[slot][i] = bv[k];
    }
    // the barrier orders the LDS writes only: the page loads stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    if (!live) {                                              // no barrier follows
        __builtin_amdgcn_s_waitcnt(0);                        // its loads end before the wave
        return;
    }

    // ---- rotated query, one head per lane column, dims DG r .. DG r + DG - 1 ----
    u32x4 bq1[NJ], bq2[PAIRED ? 1 : NJ];
    float qsl;
    {
        float qv[DG];
        // the sign words of dims DG r .. DG r + DG - 1, selected from scalar reads
        constexpr int NW = DG >= 32 ? DG / 32 : 1;
        uint32_t sw[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const int widx = (DG * r) / 32 + j;
            // (readfirstlane keeps each word a scalar value: a select of the
            // words themselves would become one per-lane load)
            uint32_t v = __builtin_amdgcn_readfirstlane(p.k.sign[0]);
#pragma unroll
            for (int q = 1; q < D / 32; ++q) v = (widx == q) ? __builtin_amdgcn_readfirstlane(p.k.sign[q]) : v;
            sw[j] = v;
        }
#pragma unroll
        for (int e = 0; e < DG; ++e) {
            const uint32_t wq = qraw[e >> 3][(e >> 1) & 3];
            const float v = hv ? half_bits_to_float((e & 1) ? (wq >> 16) : (wq & 0xFFFFu)) : 0.0f;
            const int i = DG * r + e;
            qv[e] = ((sw[DG >= 32 ? (e >> 5) : 0] >> (i & 31)) & 1u) ? -v : v;
        }
#pragma unroll
        for (int s = 1; s < DG; s <<= 1)
#pragma unroll
            for (int e = 0; e < DG; ++e) {
                if (e & s) continue;
                const float a = qv[e], c = qv[e + s];
                qv[e] = a + c;
                qv[e + s] = a - c;
            }
#pragma unroll
        for (int s = 16; s < 64; s <<= 1)
#pragma unroll
            for (int e = 0; e < DG; ++e) {
                const float o = __shfl_xor(qv[e], s);
                qv[e] = (lane & s) ? (o - qv[e]) : (qv[e] + o);
            }
        // per-head power of two bringing max |q~| to [2^13, 2^14)
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < DG; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(qv[e]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
        int ex = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 14;   // amax in [2^(ex-1), 2^ex)
        ex = ex < -100 ? -100 : ex;
        const float sc = __builtin_bit_cast(float, (uint32_t)(127 + 14 - ex) << 23);   // 2^(14 - ex)
        qsl = p.qscale / (sc * kLevelScale);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            uint32_t w1[4], w2[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float v = qv[4 * j + t] * sc;
                const _Float16 hi = (_Float16)v;
                const _Float16 lo = (_Float16)(v - (float)hi);
                w1[t] = pack_half2(hi, hi);
                w2[t] = pack_half2(lo, (_Float16)0.0f);
            }
            if constexpr (PAIRED) {
                bq1[j] = lo_col ? u32x4{w2[0], w2[1], w2[2], w2[3]} : u32x4{w1[0], w1[1], w1[2], w1[3]};
            } else {
                bq1[j] = u32x4{w1[0], w1[1], w1[2], w1[3]};
                bq2[j] = u32x4{w2[0], w2[1], w2[2], w2[3]};
            }
        }
    }

    f4 acc[NJJ];
#pragma unroll
    for (int jj = 0; jj < NJJ; ++jj) acc[jj] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float M = -__builtin_inff();          // base-2 reference of head m (uniform over r)
    float lsum = 0.0f;                    // sum of exp2(s - M) over this lane's tokens
    float vlim = 0.0f;                    // power of two above every value norm seen (wave-uniform)
    float vscale = 0.0f;                  // 2^6 / vlim

    // scores of the page in slot d: tokens 4r .. 4r+3 for head column hcol
    auto scores = [&](int d) -> f4 {
        // the lane's key slice of kv head g + kv, from bit 0 (3 bits at D = 64:
        // shifted into place)
        auto key_slice = [&](int kv, uint32_t (&kc)[KW]) {
            if constexpr (SL::KBY % 4) {
                kc[0] = __builtin_amdgcn_alignbit(rk[d][kv][1], rk[d][kv][0], ksh);
                kc[KW - 1] = rk[d][kv][1] >> ksh;
            } else {
#pragma unroll
                for (int w = 0; w < KW; ++w) kc[w] = rk[d][kv][w];
            }
        };
        uint32_t kc[KW];
        key_slice(0, kc);
        f4 S;
        if constexpr (PAIRED) {
            f4 S0 = f4{0.0f, 0.0f, 0.0f, 0.0f};
            score_chunks_paired<0, NJ, KB>(tab, kc, lok, bq1, S0);
            if constexpr (KVW == 2) {   // kv head g + 1's chain; each column keeps its own kv head's
                uint32_t kc1[KW];
                key_slice(1, kc1);
                f4 S1 = f4{0.0f, 0.0f, 0.0f, 0.0f};
                score_chunks_paired<0, NJ, KB>(tab, kc1, lok, bq1, S1);
#pragma unroll
                for (int i = 0; i < 4; ++i) S0[i] = kvs ? S1[i] : S0[i];
            }
            // column m + (q_lo column m ^ 8): row_ror:8 pairs lanes m and m ^ 8
            // of each 16-lane row, so both columns end with the full score
#pragma unroll
            for (int i = 0; i < 4; ++i) S[i] = S0[i] + row_ror8(S0[i]);
        } else {
            f4 S0 = f4{0.0f, 0.0f, 0.0f, 0.0f}, S1 = S0;   // two independent chains
            score_chunks<0, NJ, KB>(tab, kc, lok, bq1, bq2, S0, S1);
            S = S0 + S1;
        }
        return S;
    };

    // Online softmax in base 2 over the NP pages of slots ds[] (pages pgs[]).
    // Two lazily raised references: M per head (rescale when a score passes
    // M + 8) and a power of two vlim per wave bounding the value norms
    // (rescale when a norm passes it); the weights w = 2^(s - M) * n_v * 2^6 /
    // vlim then stay below 2^14, inside binary16.  Leaves t = s - M and the
    // value norms of the pages' tokens.
    auto softmax = [&](auto np, const f4 *S, const int *pgs, const int *ds, float *t, float *vn) {
        constexpr int NP = decltype(np)::value;
        // exponents against the current reference: t = s - Mc (one fma per token)
        const float Mc0 = (M == -__builtin_inff()) ? 0.0f : M;
#pragma unroll
        for (int q = 0; q < NP; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t[4 * q + i] = __builtin_fmaf(S[q][i], rkn[ds[q]][i] * qsl, -Mc0);
                vn[4 * q + i] = rvn[ds[q]][i];
            }
        bool full = true;                                             // wave-uniform
#pragma unroll
        for (int q = 0; q < NP; ++q)
            full = full & rok[ds[q]] & (t0 + (pgs[q] + 1) * kAttnBlockSize <= t1);
        if (!full) {                                                  // one join for all pages
#pragma unroll
            for (int q = 0; q < NP; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = rok[ds[q]] & (t0 + pgs[q] * kAttnBlockSize + 4 * r + i < t1);
                    t[4 * q + i] = ok ? t[4 * q + i] : -__builtin_inff();
                    vn[4 * q + i] = ok ? vn[4 * q + i] : 0.0f;
                }
        }
        float smax = t[0], vmax = vn[0];
#pragma unroll
        for (int e = 1; e < 4 * NP; ++e) {
            smax = __builtin_fmaxf(smax, t[e]);
            vmax = __builtin_fmaxf(vmax, vn[e]);
        }
        smax = hv ? smax : -__builtin_inff();
        const float lim = (M == -__builtin_inff()) ? -__builtin_inff() : kLazy;
        if (__builtin_amdgcn_ballot_w64(smax > lim || vmax > vlim)) {
            // new score reference of every head whose scores passed it by 2^8
            float mx = __builtin_fmaxf(smax, __shfl_xor(smax, 16));
            mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
            const float Mn = (mx > lim) ? Mc0 + mx : M;
            const float f = (Mn == M) ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
            lsum *= f;
            const float sh = (Mn == M) ? 0.0f : Mn - Mc0;   // the pages against the new reference
#pragma unroll
            for (int e = 0; e < 4 * NP; ++e) t[e] -= sh;
            M = Mn;
            // new norm bound: the power of two above the wave's largest norm
            float vw = vmax;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) vw = __builtin_fmaxf(vw, __shfl_xor(vw, o));
            float fv = 1.0f;
            if (vw > vlim) {                              // wave-uniform
                int e = __builtin_amdgcn_frexp_expf(vw);         // vw in [2^(e-1), 2^e)
                e = e > 126 ? 126 : (e < -120 ? -120 : e);         // keeps 2^e, 2^-e, 2^(6-e) normal
                fv = vlim * __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);   // exact: powers of two (or 0)
                vlim = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);
                vscale = __builtin_bit_cast(float, (uint32_t)(127 + (int)kWShift - e) << 23);   // 2^6 / vlim
            }
            // accumulator rows are heads 4r + i (PAIRED: row h holds head h % 8)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float fi = __shfl(f, PAIRED ? ((4 * r + i) & 7) : (4 * r + i)) * fv;
#pragma unroll
                for (int jj = 0; jj < NJJ; ++jj) acc[jj][i] *= fi;
            }
        }
    };

    // Value products of the page in slot d with exponents t and norms vn of
    // its 4 tokens per lane; Bv holds the value operands of kv head g.
    auto values = [&](int d, const float *t, const float *vn, u32x4 (&Bv)[NB]) {
        uint32_t w1[4], w2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(t[i]);
            lsum += pr;
            const float w = pr * (vn[i] * vscale);
            // w = hi + lo; hi is w truncated to binary16, lo the remainder
            const uint32_t hh = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w, w));
            const float hf = (float)__builtin_bit_cast(_Float16, (uint16_t)(hh & 0xFFFFu));
            w1[i] = hh;
            w2[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(w - hf));
        }
        // values: dims NJJ m + jj, tokens 4r .. 4r+3
        if constexpr (PAIRED && KVW == 2) {
            // rows 0-7: (w_hi, w_hi) of head slots 0-7; rows 8-15: (w_lo, 0);
            // the rows of the other kv head are zero in each product
            const u32x4 A = lo_col ? u32x4{w2[0], w2[1], w2[2], w2[3]} : u32x4{w1[0], w1[1], w1[2], w1[3]};
            const u32x4 z = u32x4{0u, 0u, 0u, 0u};
            const u32x4 A0 = kvs ? z : A, A1 = kvs ? A : z;
#pragma unroll
            for (int jj = 0; jj < NJJ; ++jj) acc[jj] = mfma(A0, Bv[jj], acc[jj]);
            value_operands<NJJ, VB, VW>(tab, rv[d][1], lov, q4, vsh, Bv);
#pragma unroll
            for (int jj = 0; jj < NJJ; ++jj) acc[jj] = mfma(A1, Bv[jj], acc[jj]);
        } else if constexpr (PAIRED) {
            // rows 0-7: (w_hi, w_hi) of heads 0-7; rows 8-15: (w_lo, 0)
            const u32x4 A = lo_col ? u32x4{w2[0], w2[1], w2[2], w2[3]} : u32x4{w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) acc[jj] = mfma(A, Bv[jj], acc[jj]);
            if constexpr (NJJ > NB) {        // the second 8 value dims of each lane column
                value_operands<NJJ, VB, VW, 1>(tab, rv[d][0], lov, q4, vsh, Bv);
#pragma unroll
                for (int jj = 0; jj < NB; ++jj) acc[NB + jj] = mfma(A, Bv[jj], acc[NB + jj]);
            }
        } else {
            const u32x4 A1 = u32x4{w1[0], w1[1], w1[2], w1[3]};
            const u32x4 A2 = u32x4{w2[0], w2[1], w2[2], w2[3]};
#pragma unroll
            for (int jj = 0; jj < NJJ; ++jj) {
                acc[jj] = mfma(A1, Bv[jj], acc[jj]);
                acc[jj] = mfma(A2, Bv[jj], acc[jj]);
            }
        }
    };

    int pg0 = 0;
    for (; pg0 + 2 <= npages; pg0 += 2) {     // wave-uniform
        const int32_t bA = bt_at(pg0 + 2), bB = bt_at(pg0 + 3);
        f4 S[2];
        S[0] = scores(0);
        fetch_keys(bA, 0);
        S[1] = scores(1);
        fetch_keys(bB, 1);
        u32x4 Bv[NB];    // value codes of kv head g (KVW = 2: g + 1's follow in values())
        value_operands<NJJ, VB, VW>(tab, rv[0][0], lov, q4, vsh, Bv);
        const int pgs[2] = {pg0, pg0 + 1}, ds[2] = {0, 1};
        float t[8], vn[8];
        softmax(std::integral_constant<int, 2>{}, S, pgs, ds, t, vn);
        values(0, t, vn, Bv);
        fetch_values(pg0 + 2, bA, 0);
        value_operands<NJJ, VB, VW>(tab, rv[1][0], lov, q4, vsh, Bv);
        values(1, t + 4, vn + 4, Bv);
        fetch_values(pg0 + 3, bB, 1);
    }
    if (pg0 < npages) {                       // the last page of an odd count, in slot 0
        f4 S[1];
        S[0] = scores(0);
        u32x4 Bv[NB];
        value_operands<NJJ, VB, VW>(tab, rv[0][0], lov, q4, vsh, Bv);
        const int pgs[1] = {pg0}, ds[1] = {0};
        float t[4], vn[4];
        softmax(std::integral_constant<int, 1>{}, S, pgs, ds, t, vn);
        values(0, t, vn, Bv);
    }

    lsum += lane_xor<16>(lsum);
    lsum += lane_xor<32>(lsum);
    if constexpr (PAIRED) {
        // rows 4r + i and 4r + i + 8 (lanes l and l ^ 32) are one head's
        // high and low parts
#pragma unroll
        for (int jj = 0; jj < NJJ; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[jj][i] += lane_xor<32>(acc[jj][i]);
    }
    // partial state of head g*grp + h: m and l from the lane of h's column,
    // accumulators from lanes (column c, row s / 4) at register s % 4 (s: the
    // head slot of h) -> dims NJJ c .. NJJ c + NJJ - 1.  KVW = 2: slot s
    // holds head (s / 4) grp + s % 4.
    const float unscale = vlim / (kLevelScale * 64.0f);     // undo 16 c and 2^6 / vlim
    float *base = p.ws + (((size_t)b * p.hq + (size_t)g * grp) * p.num_splits + split) * partial;
    const size_t hstride = (size_t)p.num_splits * partial;
    if (r == 0 && hv && !lo_col) {
        float *dst = base + (size_t)(KVW == 2 ? kvs * grp + hh : m) * hstride;
        dst[0] = M;
        dst[1] = lsum;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int h = 4 * r + i;
        if constexpr (KVW == 2) {
            if (r >= 2 || i >= grp) break;
            h = r * grp + i;
        } else {
            if (h >= grp || (PAIRED && r >= 2)) break;
        }
        float2 *dst = reinterpret_cast<float2 *>(base + (size_t)h * hstride + 2 + NJJ * m);   // 8-byte aligned
#pragma unroll
        for (int jj = 0; jj < NJJ; jj += 2) dst[jj >> 1] = float2(acc[jj][i] * unscale, acc[jj + 1][i] * unscale);
    }
}

// One wave per (sequence, query head): merge the splits, undo the rotation.
// Lane l holds coordinates E l .. E l + E - 1 (E = D / 64).
template <int D>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnParams p) {
    constexpr int E = D / 64;
    constexpr int partial = 2 + D;
    const int bh = blockIdx.x;
    const int b = bh / p.hq;
    const int lane = threadIdx.x;
    int T = p.context_lens[b];
    T = T < 0 ? 0 : T;
    const int tmax = p.max_blocks * kAttnBlockSize;
    T = T > tmax ? tmax : T;
    if (p.num_blocks <= 0) T = 0;
    int ns = (T + p.split_tokens - 1) / p.split_tokens;
    // the last of these splits is empty when it is odd and the even split
    // before it (skew tokens longer) reaches T; it wrote no partial
    if (ns > 0 && ((ns - 1) & 1) && (ns - 1) * p.split_tokens + p.skew >= T) --ns;
    const float *src = p.ws + (size_t)bh * p.num_splits * partial;

    // The partials of the first G splits and the (m, l) pairs of the first 64
    // (lane s: split s) are loaded together, before the maximum is formed:
    // one round of loads for up to G splits instead of three in a row.
    constexpr int G = E <= 2 ? 32 : 16;
    auto load_batch = [&](float (&ev)[G][E], int s0, int j0, int cnt) {
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int j = (j0 + u < cnt) ? j0 + u : j0;          // in range; weight 0 below
            const float *q = src + (size_t)(s0 + j) * partial + 2 + E * lane;
            if constexpr (E == 1) {
                ev[u][0] = *q;
            } else {
                // entries are 4 (2 + D) bytes, so only 8-byte alignment holds
#pragma unroll
                for (int e = 0; e < E; e += 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(q + e);
                    ev[u][e] = v.x;
                    ev[u][e + 1] = v.y;
                }
            }
        }
    };
    float a[E];
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = 0.0f;
    auto accumulate = [&](const float (&ev)[G][E], int j0, int cnt, float w) {
#pragma unroll
        for (int u = 0; u < G; ++u) {
            float wj = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (j0 + u) & 63));
            wj = (j0 + u < cnt) ? wj : 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) a[e] = __builtin_fmaf(wj, ev[u][e], a[e]);
        }
    };
    const int cnt0 = ns < 64 ? ns : 64;
    float m0 = -__builtin_inff(), l0 = 0.0f;
    if (lane < cnt0) {
        m0 = src[(size_t)lane * partial];
        l0 = src[(size_t)lane * partial + 1];
    }
    float ev0[G][E];
    load_batch(ev0, 0, 0, cnt0);          // in range even for no split (never accumulated then)

    // the largest running maximum over the splits (lane s holds split s)
    float mx = m0;
    for (int s0 = 64; s0 < ns; s0 += 64) {
        const int s = s0 + lane;
        if (s < ns) {
            const float ms = src[(size_t)s * partial];
            mx = ms > mx ? ms : mx;
        }
    }
    mx = __builtin_fmaxf(mx, lane_xor<32>(mx));
    mx = __builtin_fmaxf(mx, lane_xor<16>(mx));
    mx = __builtin_fmaxf(mx, lane_xor<8>(mx));
    mx = __builtin_fmaxf(mx, lane_xor<4>(mx));
    mx = __builtin_fmaxf(mx, lane_xor<2>(mx));
    mx = __builtin_fmaxf(mx, lane_xor<1>(mx));
    // split weights, then this lane's coordinates, G splits per round of loads
    float lsum = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int s = s0 + lane;
        float w = 0.0f;
        if (s0 == 0) {
            if (lane < cnt0) {
                w = (l0 > 0.0f) ? __builtin_amdgcn_exp2f(m0 - mx) : 0.0f;
                lsum += w * l0;
            }
        } else if (s < ns) {
            const float ls = src[(size_t)s * partial + 1];
            w = (ls > 0.0f) ? __builtin_amdgcn_exp2f(src[(size_t)s * partial] - mx) : 0.0f;
            lsum += w * ls;
        }
        const int cnt = (ns - s0 < 64) ? ns - s0 : 64;
        int j0 = 0;
        if (s0 == 0) {
            accumulate(ev0, 0, cnt, w);
            j0 = G;
        }
        for (; j0 < cnt; j0 += G) {
            float ev[G][E];
            load_batch(ev, s0, j0, cnt);
            accumulate(ev, j0, cnt, w);
        }
    }
    lsum += lane_xor<32>(lsum);
    lsum += lane_xor<16>(lsum);
    lsum += lane_xor<8>(lsum);
    lsum += lane_xor<4>(lsum);
    lsum += lane_xor<2>(lsum);
    lsum += lane_xor<1>(lsum);
    const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
    // inverse transform: x = D H acc / D -- the low log2(E) coordinate bits
    // in registers, the next 6 across lanes
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = a[e] * inv;
#pragma unroll
    for (int st = 1; st < E; st <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (e & st) continue;
            const float u = x[e], v = x[e + st];
            x[e] = u + v;
            x[e + st] = u - v;
        }
    auto cross = [&](auto sc) {          // the stage across lanes l and l ^ S
        constexpr int S = decltype(sc)::value;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float o = lane_xor<S>(x[e]);
            x[e] = (lane & S) ? (o - x[e]) : (x[e] + o);
        }
    };
    cross(std::integral_constant<int, 1>{});
    cross(std::integral_constant<int, 2>{});
    cross(std::integral_constant<int, 4>{});
    cross(std::integral_constant<int, 8>{});
    cross(std::integral_constant<int, 16>{});
    cross(std::integral_constant<int, 32>{});
    uint16_t hv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        float v = x[e] * (1.0f / D);
        if (sign_of(p.k, E * lane + e)) v = -v;
        hv[e] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
    uint16_t *o = p.out + (size_t)bh * D + E * lane;
    if constexpr (E == 1) {
        o[0] = hv[0];
    } else {
#pragma unroll
        for (int e = 0; e < E; e += 2)
            reinterpret_cast<uint32_t *>(o)[e >> 1] = (uint32_t)hv[e] | ((uint32_t)hv[e + 1] << 16);
    }
}

bool bits_ok(int b) { return b == 2 || b == 3 || b == 4; }

// The split kernel for (D, KB, VB); head_dim 256 has the paired form only
// (attn_supported keeps its group size at 8 or below).
template <int D, int KB, int VB>
void launch_split(bool paired, int kvw, dim3 grid, dim3 block, hipStream_t stream, const AttnParams &p) {
    if constexpr (D <= 128) {
        if (kvw == 2) hipLaunchKernelGGL((attn_split_kernel<D, KB, VB, true, 2>), grid, block, 0, stream, p);
        else if (paired) hipLaunchKernelGGL((attn_split_kernel<D, KB, VB, true, 1>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_split_kernel<D, KB, VB, false, 1>), grid, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((attn_split_kernel<D, KB, VB, true, 1>), grid, block, 0, stream, p);
    }
}

}  // namespace

// Library-owned workspace for callers that cannot allocate: one fixed array
// per GPU (each device holds its own copy at its own address, from the first
// call on that device until the process ends).  The array's name is a host
// stand-in; kernels get the device address that hipGetSymbolAddress returns.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kAttnStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t attn_static_workspace(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

bool attn_supported(const AttnShape &s) {
    if (s.num_kv_heads <= 0 || s.num_q_heads % s.num_kv_heads) return false;
    if (s.head_dim != 64 && s.head_dim != 128 && s.head_dim != 256) return false;
    const int grp = s.num_q_heads / s.num_kv_heads;
    // head_dim 256 runs the paired form only (its two-product form spills)
    const int gmax = s.head_dim > 128 ? kAttnMaxGroupD256 : kAttnMaxGroup;
    return grp >= 1 && grp <= gmax && bits_ok(s.k_bits) && bits_ok(s.v_bits);
}

// kv heads per wave of the split kernel: two where at most 4 query heads
// share a kv head (head_dim up to 128, an even number of kv heads), else one
int attn_kv_per_wave(const AttnShape &s) {
    const int grp = s.num_q_heads / s.num_kv_heads;
    return (s.head_dim <= 128 && grp <= 4 && s.num_kv_heads % 2 == 0) ? 2 : 1;
}

int attn_split_tokens(const AttnShape &s) {
    // one wave per (sequence, unit of attn_kv_per_wave kv heads) and split;
    // about kMTargetWaves waves
    const int ctx = s.max_blocks * kAttnBlockSize;
    const int units = s.batch * s.num_kv_heads / attn_kv_per_wave(s);
    const int per_seq = units > 0 ? (kMTargetWaves + units - 1) / units : 1;
    int st = (ctx + per_seq - 1) / per_seq;
    st = (st + kAttnBlockSize - 1) / kAttnBlockSize * kAttnBlockSize;
    st = st < 256 ? 256 : st;
    return st > kMaxSplitTokens ? kMaxSplitTokens : st;
}

int attn_num_splits(const AttnShape &s) {
    const int ctx = s.max_blocks * kAttnBlockSize;
    const int st = attn_split_tokens(s);
    const int ns = (ctx + st - 1) / st;
    return ns < 1 ? 1 : ns;
}

size_t attn_workspace_bytes(const AttnShape &s) {
    return (size_t)s.batch * s.num_q_heads * attn_num_splits(s) * partial_floats(s.head_dim) *
           sizeof(float);
}

hipError_t launch_attn(const AttnShape &s, const CodecConsts &kc, const CodecConsts &vc,
                       const void *q, const uint8_t *k_packed, const float *k_norms,
                       const uint8_t *v_packed, const float *v_norms,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       void *out, void *workspace, hipStream_t stream) {
    if (!attn_supported(s)) return hipErrorInvalidValue;
    AttnParams p;
    p.q = static_cast<const uint16_t *>(q);
    p.kp = k_packed;
    p.kn = k_norms;
    p.vp = v_packed;
    p.vn = v_norms;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.ws = static_cast<float *>(workspace);
    p.out = static_cast<uint16_t *>(out);
    p.batch = s.batch;
    p.hq = s.num_q_heads;
    p.hkv = s.num_kv_heads;
    p.max_blocks = s.max_blocks;
    p.split_tokens = attn_split_tokens(s);
    p.num_splits = attn_num_splits(s);
    p.num_blocks = s.num_blocks;
    p.qscale = scale * 1.4426950408889634f / s.head_dim;
    p.k = kc;
    p.v = vc;
    // units of kvw kv heads; fewer units per split than a workgroup's: the
    // spare waves take further splits
    const int kvw = attn_kv_per_wave(s);
    const int units = s.num_kv_heads / kvw;                   // per split
    const int upw = kMWaves;                                  // units per workgroup
    p.spw = (units < upw && upw % units == 0) ? upw / units : 1;
    p.skew = 0;
    if (p.spw == 2) {            // slots 0 and 1: even and odd splits, waves w and w + 4
        int sk = p.split_tokens * kSkew64 / 64 / kAttnBlockSize * kAttnBlockSize;
        if (p.split_tokens + sk > kMaxSplitTokens) sk = kMaxSplitTokens - p.split_tokens;
        p.skew = sk;
    }
    const int ups = upw / p.spw;
    const dim3 grid((p.num_splits + p.spw - 1) / p.spw, s.batch, (units + ups - 1) / ups);
    const dim3 block(kMThreads);
    const bool paired = s.num_q_heads / s.num_kv_heads <= 8;
#define TQ_WIDTHS(D)                                                                                 \
    switch (s.k_bits * 10 + s.v_bits) {                                                              \
        case 44: launch_split<D, 4, 4>(paired, kvw, grid, block, stream, p); break;                       \
        case 43: launch_split<D, 4, 3>(paired, kvw, grid, block, stream, p); break;                       \
        case 42: launch_split<D, 4, 2>(paired, kvw, grid, block, stream, p); break;                       \
        case 34: launch_split<D, 3, 4>(paired, kvw, grid, block, stream, p); break;                       \
        case 33: launch_split<D, 3, 3>(paired, kvw, grid, block, stream, p); break;                       \
        case 32: launch_split<D, 3, 2>(paired, kvw, grid, block, stream, p); break;                       \
        case 24: launch_split<D, 2, 4>(paired, kvw, grid, block, stream, p); break;                       \
        case 23: launch_split<D, 2, 3>(paired, kvw, grid, block, stream, p); break;                       \
        case 22: launch_split<D, 2, 2>(paired, kvw, grid, block, stream, p); break;                       \
        default: return hipErrorInvalidValue;                                                        \
    }
    switch (s.head_dim) {
        case 64: TQ_WIDTHS(64) break;
        case 128: TQ_WIDTHS(128) break;
        case 256: TQ_WIDTHS(256) break;
        default: return hipErrorInvalidValue;
    }
#undef TQ_WIDTHS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 cgrid(s.batch * s.num_q_heads);
    switch (s.head_dim) {
        case 64: hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, dim3(64), 0, stream, p); break;
        case 128: hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, dim3(64), 0, stream, p); break;
        default: hipLaunchKernelGGL(attn_combine_kernel<256>, cgrid, dim3(64), 0, stream, p); break;
    }
    return hipGetLastError();
}

}  // namespace tq
