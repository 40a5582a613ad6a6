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
//           sequence (two per kv head at head_dim 256, each accumulating
//           half of the value dims): a workgroup takes the kv heads of one
//           split, or, for caches with fewer kv heads, all of them for
//           several splits.  Per 16-token page the scores and the value
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
// between lanes.  Values (N = min(d, 128) / 16 dims per lane column): lane
// (column m, r) reads dims N m .. N m + N - 1 of tokens 4r .. 4r+3 (of the
// wave's half at d = 256); chunk jj accumulates dim N m + jj.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_attn_internal.h"

namespace tq {
namespace {

// workspace entry per (sequence, query head, split): m, l, acc[head_dim]
constexpr int partial_floats(int head_dim) { return 2 + head_dim; }
// waves per kv head of the split kernel (two at head_dim 256)
constexpr int waves_per_head(int head_dim) { return head_dim > 128 ? 2 : 1; }
constexpr float kLazy = 8.0f;               // rescale when a score passes m + 8 (base 2)
constexpr int kMaxSplitTokens = 4096;       // block-table entries of a split staged in LDS
constexpr int kMWaves = 8;                  // waves per workgroup
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMPrefetch = 1;               // extra ring slots: pages of loads in flight ahead of use
// split-kernel waves aimed for: one full round on MI355X, whose 256 CUs x 4
// SIMDs hold 2 waves each of this kernel (its 210-220 VGPRs allow no more);
// measured, 1.5 or 2-3 rounds are slower and half a round much slower
constexpr int kMTargetWaves = 2048;
constexpr float kLevelScale = 16.0f;        // binary16 levels are 16 c
constexpr float kWShift = 6.0f;             // value weights carry 2^6
constexpr int kLutRow = 256;                // bytes per table row: keys' half, values' half
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
    int64_t num_blocks;
    float qscale;        // scale * log2(e) / head_dim
    CodecConsts k;       // key codebook and the sign mask (shared by keys and values)
    CodecConsts v;       // value codebook
};

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
// Entry e of a side lives in row e of the LDS table (256 bytes: keys in the
// first half, values in the second), repeated once per lane of a group of
// 128 / entry-bytes lanes, so that lanes of a group never share a bank.  For
// a byte index one v_perm forms the address (byte << 8 | lane offset).
template <int B>
struct Side {
    static constexpr int EB = (B == 2) ? 16 : 8;           // bytes per table entry
    static constexpr int NE = (B == 3) ? 64 : 256;         // table entries
    static constexpr int COPIES = 128 / EB;                // lane copies per half row
};

template <int B>
__device__ __forceinline__ void fill_side(char *tab, const CodecConsts &k, int half) {
    using S = Side<B>;
    for (int t = threadIdx.x; t < S::NE * 32; t += kMThreads) {
        const int e = t >> 5, w = t & 31;                  // entry, dword of the half row
        const int dw = w % (S::EB / 4);                    // code group within the entry
        int code;
        if (B == 4) code = dw == 0 ? (e & 15) : (e >> 4);
        else if (B == 3) code = dw == 0 ? (e & 7) : (e >> 3);
        else code = (e >> (2 * dw)) & 3;
        *reinterpret_cast<uint32_t *>(tab + e * kLutRow + half + 4 * w) = level_pair(k, code);
    }
}

template <int K>
__device__ __forceinline__ uint32_t byte_addr(uint32_t word, uint32_t laneoff) {
    return __builtin_amdgcn_perm(word, laneoff, 0x0C0C0000u | ((4u + K) << 8));
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
template <int K, int NJJ>
__device__ __forceinline__ void value_bytes4(const char *tab, const uint32_t (&vc)[4],
                                             uint32_t laneoff, u32x4 (&Bv)[NJJ]) {
    u32x2 L[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) L[i] = lut8<K>(tab, vc[i], laneoff);
    Bv[2 * K] = u32x4{L[0].x, L[1].x, L[2].x, L[3].x};
    Bv[2 * K + 1] = u32x4{L[0].y, L[1].y, L[2].y, L[3].y};
}

template <int K, int NJJ>
__device__ __forceinline__ void value_bytes2(const char *tab, const uint32_t (&vc)[4],
                                             uint32_t laneoff, u32x4 (&Bv)[NJJ]) {
    u32x4 L[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) L[i] = lut16<K>(tab, vc[i], laneoff);
#pragma unroll
    for (int t = 0; t < 4; ++t) Bv[4 * K + t] = u32x4{L[0][t], L[1][t], L[2][t], L[3][t]};
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

// The value operands of the page for a slice of NJJ dims per lane column:
// 4-bit NJJ / 2 bytes, 2-bit NJJ / 4 bytes, 3-bit 3 NJJ / 8 bytes.  vc holds
// VW words per token as loaded (see the value loads in the split kernel);
// vsh is the 3-bit field's bit offset within them.
template <int NJJ, int VB, int VW>
__device__ __forceinline__ void value_operands(const char *tab, const uint32_t (&vc)[4][VW],
                                               uint32_t laneoff, int q4, uint32_t vsh,
                                               u32x4 (&Bv)[NJJ]) {
    if constexpr (VB == 4) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = vc[i][0];
        value_bytes4<0>(tab, w, laneoff, Bv);
        value_bytes4<1>(tab, w, laneoff, Bv);
        if constexpr (NJJ == 8) {
            value_bytes4<2>(tab, w, laneoff, Bv);
            value_bytes4<3>(tab, w, laneoff, Bv);
        }
    } else if constexpr (VB == 2) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = vc[i][0];
        value_bytes2<0>(tab, w, laneoff, Bv);
        if constexpr (NJJ == 8) value_bytes2<1>(tab, w, laneoff, Bv);
    } else if constexpr (NJJ == 8) {
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
        value_fields3<NJJ>(tab, v24, laneoff, Bv);
    } else {
        // 12 bits at bit 12m of the slice, inside the two dwords the lane
        // loaded from the dword that holds its first bit
        uint32_t v12[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v12[i] = __builtin_amdgcn_alignbit(vc[i][VW - 1], vc[i][0], vsh);
        value_fields3<NJJ>(tab, v12, laneoff, Bv);
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
    static constexpr int VH = D < 128 ? D : 128;      // value dims per wave
    static constexpr int WPH = D / VH;                // waves per kv head
    static constexpr int NJJ = VH / 16;               // value dims per lane column
    // value words per lane and token: one, or at D = 64 and 3 bits (12 bits
    // at bit 12m) the two dwords around the field
    static constexpr int VW = (VB == 3 && NJJ == 4) ? 2 : 1;
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
// Head dimension D: lane row group r holds score dims D/4 r .. D/4 r + D/4 - 1.
// Each wave accumulates VH = min(D, 128) value dims; at D = 256 a kv head
// takes two waves, which both form the full scores and accumulate one half
// of the value dims each.
template <int D, int KB, int VB, bool PAIRED>
__global__ __launch_bounds__(kMThreads) void attn_split_kernel(AttnParams p) {
    using SK = Side<KB>;
    using SV = Side<VB>;
    using SL = Slices<D, KB, VB>;
    constexpr int DG = SL::DG, NJ = SL::NJ, NJJ = SL::NJJ, WPH = SL::WPH;
    constexpr int partial = 2 + D;
    __shared__ __attribute__((aligned(16))) char tab[256 * kLutRow];
    __shared__ int32_t bt_all[kMWaves][kMaxSplitTokens / kAttnBlockSize];

    // The workgroup's waves form p.spw slots of kMWaves / (WPH p.spw) kv
    // heads; slot s works on split blockIdx.x * p.spw + s (several splits per
    // workgroup when the cache has fewer kv heads than waves).
    const int b = blockIdx.y;
    int T = p.context_lens[b];
    T = T < 0 ? 0 : T;
    const int tmax = p.max_blocks * kAttnBlockSize;
    T = T > tmax ? tmax : T;
    if (p.num_blocks <= 0) T = 0;
    const int hps = kMWaves / WPH / p.spw;                    // kv heads per slot
    const int first = blockIdx.x * p.spw;
    if (first * p.split_tokens >= T) return;                 // the whole workgroup is past the context

    fill_side<KB>(tab, p.k, 0);
    fill_side<VB>(tab, p.v, kLutRow / 2);
    for (int sl = 0; sl < p.spw; ++sl) {                      // block-table entries of every slot
        const int u0 = (first + sl) * p.split_tokens;
        if (u0 >= T) break;
        const int u1 = (u0 + p.split_tokens < T) ? u0 + p.split_tokens : T;
        const int np = (u1 - u0 + kAttnBlockSize - 1) / kAttnBlockSize;
        const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks + u0 / kAttnBlockSize;
        for (int i = threadIdx.x; i < np; i += kMThreads) bt_all[sl][i] = bt[i];
    }
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = wave / WPH, half = wave % WPH;           // kv-head unit, value half
    const int slot = unit / hps;
    const int g = blockIdx.z * hps + unit % hps;              // kv head
    const int split = first + slot;
    const int t0 = split * p.split_tokens;
    if (g >= p.hkv || t0 >= T) return;                        // no barrier follows
    const int t1 = (t0 + p.split_tokens < T) ? t0 + p.split_tokens : T;
    const int npages = (t1 - t0 + kAttnBlockSize - 1) / kAttnBlockSize;
    const int32_t *bt_lds = bt_all[slot];
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, r = lane >> 4;
    const int grp = p.hq / p.hkv;
    const int hcol = PAIRED ? (m & 7) : m;                    // head of this lane's column
    const bool lo_col = PAIRED && m >= 8;                     // a column of low halves
    const bool hv = hcol < grp;                               // a real query head column
    const uint32_t lok = (uint32_t)(lane & (SK::COPIES - 1)) * SK::EB;
    const uint32_t lov = kLutRow / 2 + (uint32_t)(lane & (SV::COPIES - 1)) * SV::EB;

    // ---- rotated query, one head per lane column, dims DG r .. DG r + DG - 1 ----
    u32x4 bq1[NJ], bq2[PAIRED ? 1 : NJ];
    float qsl;
    {
        float qv[DG];
        const int mq = hv ? hcol : 0;                         // padding columns read head 0, then drop it
        const uint16_t *qp = p.q + ((size_t)b * p.hq + (size_t)g * grp + mq) * D + DG * r;
#pragma unroll
        for (int e = 0; e < DG; ++e) {
            const float v = hv ? half_bits_to_float(qp[e]) : 0.0f;
            qv[e] = sign_of(p.k, DG * r + e) ? -v : v;
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

    // per-lane byte offsets inside one page of this kv head
    const uint32_t rowk = (uint32_t)p.hkv * SL::PK;           // one token of all kv heads
    const uint32_t rowv = (uint32_t)p.hkv * SL::PV;
    const uint32_t kslice = (uint32_t)SL::KBY * r;            // the slice's byte offset in the row
    const uint32_t offk = (uint32_t)m * rowk + (uint32_t)g * SL::PK + (kslice & ~3u);
    const uint32_t ksh = (kslice & 3u) * 8u;                  // 3 bits at D = 64: 0 or 16
    const int q4 = m & 3;
    const uint32_t vhalf = (uint32_t)half * (SL::VH * VB / 8);
    const uint32_t vsh = (12u * (uint32_t)m) & 31u;           // 3 bits at D = 64
    uint32_t offv[4], offn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t row = (uint32_t)(4 * r + i) * rowv + (uint32_t)g * SL::PV + vhalf;
        if (VB == 4) offv[i] = row + (uint32_t)(NJJ / 2) * m;
        else if (VB == 2) offv[i] = row + (uint32_t)(NJJ / 4) * m;
        else if (NJJ == 8) offv[i] = row + 4u * (3u * (uint32_t)(m >> 2) + (uint32_t)(q4 < 2 ? q4 : 2));
        else offv[i] = row + 4u * ((12u * (uint32_t)m) >> 5);
        offn[i] = ((uint32_t)(4 * r + i) * p.hkv + g) * 4u;
    }
    const uint32_t pagek = kAttnBlockSize * rowk;
    const uint32_t pagev = kAttnBlockSize * rowv;
    const uint32_t pagen = kAttnBlockSize * p.hkv * 4u;

    // Loads of page pg sit in ring slot pg % R.  The refill for page pg + R
    // is issued at the end of step pg, once the slot has been consumed; its
    // block number was read from LDS one step earlier.  (At D = 256 with
    // 4-bit keys the two slots cost a few spilled registers; measured, that
    // is still faster than a one-slot ring.)
    constexpr int R = kMPrefetch + 1;
    constexpr int KW = SL::KW, VW = SL::VW;
    uint32_t rk[R][KW];
    uint32_t rv[R][4][VW];
    float rkn[R][4], rvn[R][4];
    bool rok[R];
    // The loads are unconditional (a page past the split re-reads the split's
    // last page, an L2 hit): straight-line loads let every wait for a page
    // leave the later pages' loads in flight.
    auto fetch = [&](int pg, int32_t blk, int slot) {
        blk = __builtin_amdgcn_readfirstlane(blk);
        const bool bok = pg < npages && blk >= 0 && blk < p.num_blocks;
        rok[slot] = bok;
        blk = (blk >= 0 && blk < p.num_blocks) ? blk : 0;
        const __amdgpu_buffer_rsrc_t rsk = page_rsrc(p.kp + (size_t)blk * pagek, pagek);
        const __amdgpu_buffer_rsrc_t rsv = page_rsrc(p.vp + (size_t)blk * pagev, pagev);
        const __amdgpu_buffer_rsrc_t rkn_ = page_rsrc(p.kn + (size_t)blk * kAttnBlockSize * p.hkv, pagen);
        const __amdgpu_buffer_rsrc_t rvn_ = page_rsrc(p.vn + (size_t)blk * kAttnBlockSize * p.hkv, pagen);
        load_key<SL::KBY, KW>(rsk, offk, rk[slot]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (VW == 2) {
                const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsv, offv[i], 0, 0));
                rv[slot][i][0] = t.x;
                rv[slot][i][VW - 1] = t.y;
            } else if constexpr (VB == 2 && NJJ == 4) {
                rv[slot][i][0] = __builtin_amdgcn_raw_buffer_load_b8(rsv, offv[i], 0, 0);
            } else if constexpr ((VB == 2 && NJJ == 8) || (VB == 4 && NJJ == 4)) {
                rv[slot][i][0] = __builtin_amdgcn_raw_buffer_load_b16(rsv, offv[i], 0, 0);
            } else {
                rv[slot][i][0] = __builtin_amdgcn_raw_buffer_load_b32(rsv, offv[i], 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rkn[slot][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkn_, offn[i], 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rvn[slot][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvn_, offn[i], 0, 0));
    };
    auto bt_at = [&](int pg) -> int32_t { return bt_lds[pg < npages ? pg : npages - 1]; };
#pragma unroll
    for (int d = 0; d < R; ++d) fetch(d, bt_at(d), d);
    int32_t blk_next = bt_at(R);

    // one page: score tiles, value operands, softmax, value tiles, refill
    auto step = [&](const int pg, const int d) {
        // the lane's key slice, from bit 0 (3 bits at D = 64: shifted into place)
        uint32_t kc[KW];
        if constexpr (SL::KBY % 4) {
            kc[0] = __builtin_amdgcn_alignbit(rk[d][1], rk[d][0], ksh);
            kc[KW - 1] = rk[d][1] >> ksh;
        } else {
#pragma unroll
            for (int w = 0; w < KW; ++w) kc[w] = rk[d][w];
        }
        // scores of tokens 4r .. 4r+3 for head hcol
        f4 S;
        if constexpr (PAIRED) {
            f4 S0 = f4{0.0f, 0.0f, 0.0f, 0.0f};
            score_chunks_paired<0, NJ, KB>(tab, kc, lok, bq1, S0);
            // column m + (q_lo column m ^ 8): row_ror:8 pairs lanes m and m ^ 8
            // of each 16-lane row, so both columns end with the full score
#pragma unroll
            for (int i = 0; i < 4; ++i) S[i] = S0[i] + row_ror8(S0[i]);
        } else {
            f4 S0 = f4{0.0f, 0.0f, 0.0f, 0.0f}, S1 = S0;   // two independent chains
            score_chunks<0, NJ, KB>(tab, kc, lok, bq1, bq2, S0, S1);
            S = S0 + S1;
        }
        // value codes of the page
        u32x4 Bv[NJJ];
        value_operands<NJJ, VB, VW>(tab, rv[d], lov, q4, vsh, Bv);

        // online softmax in base 2.  Two lazily raised references: M per head
        // (rescale when a score passes M + 8) and a power of two vlim per wave
        // bounding the value norms (rescale when a norm passes it); the
        // weights w = 2^(s - M) * n_v * 2^6 / vlim then stay below 2^14,
        // inside binary16.
        const int tbase = t0 + pg * kAttnBlockSize + 4 * r;
        const bool full = rok[d] && (t0 + pg * kAttnBlockSize + kAttnBlockSize <= t1);
        float s2[4], vn[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s2[i] = S[i] * (rkn[d][i] * qsl);
            vn[i] = rvn[d][i];
        }
        if (!full) {                                    // wave-uniform
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = rok[d] && (tbase + i < t1);
                s2[i] = ok ? s2[i] : -__builtin_inff();
                vn[i] = ok ? vn[i] : 0.0f;
            }
        }
        float smax = __builtin_fmaxf(__builtin_fmaxf(s2[0], s2[1]), __builtin_fmaxf(s2[2], s2[3]));
        smax = hv ? smax : -__builtin_inff();
        const float vmax = __builtin_fmaxf(__builtin_fmaxf(vn[0], vn[1]), __builtin_fmaxf(vn[2], vn[3]));
        if (__builtin_amdgcn_ballot_w64(smax > M + kLazy || vmax > vlim)) {
            // new score reference of every head whose scores passed it by 2^8
            float mx = __builtin_fmaxf(smax, __shfl_xor(smax, 16));
            mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
            const float Mn = (mx > M + kLazy) ? mx : M;
            const float f = (Mn == M) ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
            lsum *= f;
            M = Mn;
            // new norm bound: the power of two above the wave's largest norm
            float vw = vmax;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) vw = __builtin_fmaxf(vw, __shfl_xor(vw, o));
            float fv = 1.0f;
            if (vw > vlim) {                              // wave-uniform
                const int e = __builtin_amdgcn_frexp_expf(vw);   // vw in [2^(e-1), 2^e)
                const float vn_lim = __builtin_bit_cast(float, (uint32_t)(127 + (e > 127 ? 127 : e)) << 23);
                fv = vlim / vn_lim;                         // exact: both powers of two (or 0)
                vlim = vn_lim;
                vscale = (float)(1 << (int)kWShift) / vlim;
            }
            // accumulator rows are heads 4r + i (PAIRED: row h holds head h % 8)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float fi = __shfl(f, PAIRED ? ((4 * r + i) & 7) : (4 * r + i)) * fv;
#pragma unroll
                for (int jj = 0; jj < NJJ; ++jj) acc[jj][i] *= fi;
            }
        }
        // before any valid token M is -inf; masked tokens must still give 0
        const float Mc = (M == -__builtin_inff()) ? 0.0f : M;
        uint32_t w1[4], w2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(s2[i] - Mc);
            lsum += pr;
            const float w = pr * (vn[i] * vscale);
            // w = hi + lo; hi is w truncated to binary16, lo the remainder
            const uint32_t hh = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w, w));
            const float hf = (float)__builtin_bit_cast(_Float16, (uint16_t)(hh & 0xFFFFu));
            w1[i] = hh;
            w2[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(w - hf));
        }
        // values: dims NJJ m + jj of the wave's half, tokens 4r .. 4r+3
        if constexpr (PAIRED) {
            // rows 0-7: (w_hi, w_hi) of heads 0-7; rows 8-15: (w_lo, 0)
            const u32x4 A = lo_col ? u32x4{w2[0], w2[1], w2[2], w2[3]} : u32x4{w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
            for (int jj = 0; jj < NJJ; ++jj) acc[jj] = mfma(A, Bv[jj], acc[jj]);
        } else {
            const u32x4 A1 = u32x4{w1[0], w1[1], w1[2], w1[3]};
            const u32x4 A2 = u32x4{w2[0], w2[1], w2[2], w2[3]};
#pragma unroll
            for (int jj = 0; jj < NJJ; ++jj) {
                acc[jj] = mfma(A1, Bv[jj], acc[jj]);
                acc[jj] = mfma(A2, Bv[jj], acc[jj]);
            }
        }

        fetch(pg + R, blk_next, d);
        blk_next = bt_at(pg + R + 1);
    };
    // Whole rounds of R pages, then the remainder after the loop, so that the
    // loop head sees the R slots refilled in the same order on every path.
    int pg0 = 0;
    for (; pg0 + R <= npages; pg0 += R) {      // wave-uniform
#pragma unroll
        for (int d = 0; d < R; ++d) step(pg0 + d, d);
    }
#pragma unroll
    for (int d = 0; d < R - 1; ++d)
        if (pg0 + d < npages) step(pg0 + d, d);

    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if constexpr (PAIRED) {
        // rows 4r + i and 4r + i + 8 (lanes l and l ^ 32) are one head's
        // high and low parts
#pragma unroll
        for (int jj = 0; jj < NJJ; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[jj][i] += __shfl_xor(acc[jj][i], 32);
    }
    // partial state of head g*grp + h: m and l from lane h, accumulators from
    // lanes (column c, row h / 4) at register h % 4 -> dims NJJ c .. NJJ c + NJJ - 1
    // of the wave's value half
    const float unscale = vlim / (kLevelScale * 64.0f);     // undo 16 c and 2^6 / vlim
    float *base = p.ws + (((size_t)b * p.hq + (size_t)g * grp) * p.num_splits + split) * partial;
    const size_t hstride = (size_t)p.num_splits * partial;
    if (r == 0 && hv && !lo_col && half == 0) {
        float *dst = base + (size_t)m * hstride;
        dst[0] = M;
        dst[1] = lsum;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * r + i;
        if (h >= grp || (PAIRED && r >= 2)) break;
        float2 *dst = reinterpret_cast<float2 *>(base + (size_t)h * hstride + 2 + SL::VH * half + NJJ * m);   // 8-byte aligned
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
    const int ns = (T + p.split_tokens - 1) / p.split_tokens;
    const float *src = p.ws + (size_t)bh * p.num_splits * partial;

    // the largest running maximum over the splits (lane s reads split s)
    float mx = -__builtin_inff();
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int s = s0 + lane;
        if (s < ns) {
            const float ms = src[(size_t)s * partial];
            mx = ms > mx ? ms : mx;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float other = __shfl_xor(mx, o);
        mx = other > mx ? other : mx;
    }
    // split weights, then this lane's coordinates; the partials of 8 splits
    // are loaded before any of them is accumulated
    float lsum = 0.0f;
    float a[E];
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int s = s0 + lane;
        float w = 0.0f;
        if (s < ns) {
            const float ls = src[(size_t)s * partial + 1];
            w = (ls > 0.0f) ? __builtin_amdgcn_exp2f(src[(size_t)s * partial] - mx) : 0.0f;
            lsum += w * ls;
        }
        const int cnt = (ns - s0 < 64) ? ns - s0 : 64;
        for (int j0 = 0; j0 < cnt; j0 += 8) {
            float ev[8][E];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
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
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float wj = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (j0 + u) & 63));
                wj = (j0 + u < cnt) ? wj : 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) a[e] = __builtin_fmaf(wj, ev[u][e], a[e]);
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
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
#pragma unroll
    for (int s = 1; s < 64; s <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float o = __shfl_xor(x[e], s);
            x[e] = (lane & s) ? (o - x[e]) : (x[e] + o);
        }
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
void launch_split(bool paired, dim3 grid, dim3 block, hipStream_t stream, const AttnParams &p) {
    if constexpr (D <= 128) {
        if (paired) hipLaunchKernelGGL((attn_split_kernel<D, KB, VB, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_split_kernel<D, KB, VB, false>), grid, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((attn_split_kernel<D, KB, VB, true>), grid, block, 0, stream, p);
    }
}

}  // namespace

bool attn_supported(const AttnShape &s) {
    if (s.num_kv_heads <= 0 || s.num_q_heads % s.num_kv_heads) return false;
    if (s.head_dim != 64 && s.head_dim != 128 && s.head_dim != 256) return false;
    const int grp = s.num_q_heads / s.num_kv_heads;
    // head_dim 256 runs the paired form only (its two-product form spills)
    const int gmax = s.head_dim > 128 ? kAttnMaxGroupD256 : kAttnMaxGroup;
    return grp >= 1 && grp <= gmax && bits_ok(s.k_bits) && bits_ok(s.v_bits);
}

int attn_split_tokens(const AttnShape &s) {
    // waves_per_head waves per (sequence, kv head) and split; about
    // kMTargetWaves waves
    const int ctx = s.max_blocks * kAttnBlockSize;
    const int units = s.batch * s.num_kv_heads * waves_per_head(s.head_dim);
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
    // fewer kv heads than kv-head units: the spare waves take further splits
    const int hpw = kMWaves / waves_per_head(s.head_dim);     // kv heads per workgroup
    p.spw = (s.num_kv_heads < hpw && hpw % s.num_kv_heads == 0) ? hpw / s.num_kv_heads : 1;
    const int hps = hpw / p.spw;
    const dim3 grid((p.num_splits + p.spw - 1) / p.spw, s.batch, (s.num_kv_heads + hps - 1) / hps);
    const dim3 block(kMThreads);
    const bool paired = s.num_q_heads / s.num_kv_heads <= 8;
#define TQ_WIDTHS(D)                                                                                 \
    switch (s.k_bits * 10 + s.v_bits) {                                                              \
        case 44: launch_split<D, 4, 4>(paired, grid, block, stream, p); break;                       \
        case 43: launch_split<D, 4, 3>(paired, grid, block, stream, p); break;                       \
        case 42: launch_split<D, 4, 2>(paired, grid, block, stream, p); break;                       \
        case 34: launch_split<D, 3, 4>(paired, grid, block, stream, p); break;                       \
        case 33: launch_split<D, 3, 3>(paired, grid, block, stream, p); break;                       \
        case 32: launch_split<D, 3, 2>(paired, grid, block, stream, p); break;                       \
        case 24: launch_split<D, 2, 4>(paired, grid, block, stream, p); break;                       \
        case 23: launch_split<D, 2, 3>(paired, grid, block, stream, p); break;                       \
        case 22: launch_split<D, 2, 2>(paired, grid, block, stream, p); break;                       \
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
