// Fused single-token decode attention over the packed, paged TurboQuant cache,
// for gfx950.
//
// Method: aither-kvcache PyPI page, "Zero-buffer fused attention" (rotate the
// query forward once, score against codebook values in the rotated domain,
// accumulate the weighted values in the rotated domain, rotate back once) and
// "Paged KV cache" (16-token blocks, [16, heads, 64] uint8 + [16, heads] f32
// per block at 4 bits); qbc.network blog, "What we shipped" item 2.
//
// With R = H D / sqrt(d) and a cached row decoding to n * R^T c[code] / sqrt(d):
//   <q, k_j>      = (n_j / d) * <H D q, c[k_j]>
//   sum_j p_j v_j = D H (sum_j p_j n_j c[v_j]) / d
// so the query is transformed once per (sequence, query head), every cached
// row is used as plain codebook values, and one inverse transform finishes.
//
// Two kernels, flash-decoding style:
//   split   grid (context split, sequence, kv-head chunk), 4 waves.  Eight
//           lanes own one (token, kv head) pair, 16 coordinates each; a wave
//           covers 8 such pairs per step -- one token of all 8 kv heads of a
//           Llama-style GQA cache, whose 8 rows of codes are 512 contiguous
//           bytes.  Each lane keeps the rotated query (16 coordinates per query
//           head of its group) and the running softmax state in registers.
//           The softmax is online in base 2 with a lazily raised reference:
//           the accumulators are rescaled only when a score exceeds the
//           reference by more than 2^8, which after the first token is rare.
//           The four waves merge through LDS; one partial state per
//           (sequence, query head, split) goes to the workspace.
//   combine grid (sequence * query head), one wave: log-sum-exp merge of the
//           splits, the inverse transform D H / d, binary16 rounding.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPartial = 2 + kHeadDim;      // m, l, acc[128] per workspace entry
constexpr float kLazy = 8.0f;               // rescale when a score passes m + 8 (base 2)
constexpr int kTargetGroups = 512;          // split-kernel workgroups aimed for
constexpr int kMaxSplitTokens = 4096;       // block-table entries of a split staged in LDS
constexpr int kPrefetch = 4;                // wave steps of K/V loads kept in flight

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i within each 8
constexpr int kRowMirror = 0x140;      // lane i <- lane 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Value of lane h of this lane's quad (quad_perm [h,h,h,h]).
__device__ __forceinline__ float quad_bcast(float v, int h) {
    const int x = __builtin_bit_cast(int, v);
    switch (h & 3) {
        case 0: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x00, 0xF, 0xF, true));
        case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x55, 0xF, 0xF, true));
        case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xAA, 0xF, 0xF, true));
        default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xFF, 0xF, 0xF, true));
    }
}

// Sum over the LPU lanes of a unit (LPU = 8 or 16, aligned groups).
template <int LPU>
__device__ __forceinline__ float unit_sum(float v) {
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kRowHalfMirror>(v);
    if (LPU == 16) v += dpp<kRowMirror>(v);
    return v;
}

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
    int64_t num_blocks;
    float qscale;        // scale * log2(e) / 128, folded into the rotated query
    CodecConsts k;
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

// This lane's E codes (E * BITS / 8 bytes at byte offset `off`).
template <int BITS, int E>
__device__ __forceinline__ void load_codes_buf(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               uint32_t (&c)[2]) {
    constexpr int BYTES = E * BITS / 8;
    if constexpr (BYTES == 8) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 u = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        c[0] = u.x;
        c[1] = u.y;
    } else if constexpr (BYTES == 4) {
        c[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        c[1] = 0;
    } else if constexpr (BYTES == 6) {   // b = 3, E = 16: 2-byte aligned
        const uint32_t h0 = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        const uint32_t h1 = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2, 0, 0);
        const uint32_t h2 = __builtin_amdgcn_raw_buffer_load_b16(r, off + 4, 0, 0);
        c[0] = h0 | (h1 << 16);
        c[1] = h2;
    } else if constexpr (BYTES == 2) {   // b = 2, E = 8
        c[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        c[1] = 0;
    } else {                             // b = 3, E = 8: 3 bytes, byte aligned
        const uint32_t b0 = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
        const uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b8(r, off + 1, 0, 0);
        const uint32_t b2 = __builtin_amdgcn_raw_buffer_load_b8(r, off + 2, 0, 0);
        c[0] = b0 | (b1 << 8) | (b2 << 16);
        c[1] = 0;
    }
}

// LDS lookup table: pairs of codes (b = 3, 4) or bytes of four codes (b = 2).
template <int BITS>
struct LevelTable {
    static constexpr int G = (BITS == 2) ? 4 : 2;
    static constexpr int NENT = 1 << (G * BITS);
};

template <int BITS, int E>
__device__ __forceinline__ void expand(const float *tab, const uint32_t (&c)[2], float (&val)[E]) {
    constexpr int G = LevelTable<BITS>::G;
    constexpr int IB = G * BITS;   // index bits per lookup
#pragma unroll
    for (int gi = 0; gi < E / G; ++gi) {
        const int bit = gi * IB;
        uint32_t idx;
        if ((bit & 31) + IB <= 32)
            idx = (c[bit >> 5] >> (bit & 31)) & ((1u << IB) - 1);
        else
            idx = __builtin_amdgcn_alignbit(c[(bit >> 5) + 1], c[bit >> 5], bit & 31) &
                  ((1u << IB) - 1);
        if (G == 2) {
            const float2 e = reinterpret_cast<const float2 *>(tab)[idx];
            val[2 * gi] = e.x;
            val[2 * gi + 1] = e.y;
        } else {
            const float4 e = reinterpret_cast<const float4 *>(tab)[idx];
            val[4 * gi] = e.x;
            val[4 * gi + 1] = e.y;
            val[4 * gi + 2] = e.z;
            val[4 * gi + 3] = e.w;
        }
    }
}

template <int BITS, int GRP, int E>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(AttnParams p) {
    constexpr int LPU = kHeadDim / E;     // lanes per (token, kv head) unit
    constexpr int UPW = 64 / LPU;         // units per wave step
    constexpr int P = kHeadDim * BITS / 8;
    constexpr int L = 1 << BITS;
    constexpr int G = LevelTable<BITS>::G;
    constexpr int NENT = LevelTable<BITS>::NENT;
    __shared__ float tab[NENT * G];
    __shared__ float xchg[2][64 * (GRP * E + 2 * GRP)];

    const int b = blockIdx.y;
    const int split = blockIdx.x;
    int T = p.context_lens[b];
    T = T < 0 ? 0 : T;
    const int tmax = p.max_blocks * kAttnBlockSize;
    T = T > tmax ? tmax : T;
    if (p.num_blocks <= 0) T = 0;
    const int t0 = split * p.split_tokens;
    if (t0 >= T) return;                 // nothing here; combine skips this split
    const int t1 = (t0 + p.split_tokens < T) ? t0 + p.split_tokens : T;

    for (int t = threadIdx.x; t < NENT; t += kThreads) {
#pragma unroll
        for (int j = 0; j < G; ++j) tab[G * t + j] = p.k.level[(t >> (BITS * j)) & (L - 1)];
    }
    // block-table entries of this split's pages (read before the token loop so
    // the code loads of a token do not wait on a dependent global load)
    __shared__ int32_t bt_lds[kMaxSplitTokens / kAttnBlockSize];
    {
        const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks + t0 / kAttnBlockSize;
        const int npages = (t1 - t0 + kAttnBlockSize - 1) / kAttnBlockSize;
        for (int i = threadIdx.x; i < npages; i += kThreads) bt_lds[i] = bt[i];
    }

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int lane = threadIdx.x & 63;
    const int gam = lane / LPU;          // unit slot in the wave
    const int sub = lane % LPU;          // coordinate slice [sub*E, sub*E + E)
    const bool wide = p.hkv >= UPW;
    const int g = wide ? blockIdx.z * UPW + gam : gam % p.hkv;
    const int tau = wide ? 0 : gam / p.hkv;
    const int tpi = wide ? 1 : UPW / p.hkv;   // tokens per wave step
    const bool live = wide || (gam < tpi * p.hkv);

    // rotated, pre-scaled query of the GRP heads of kv head g: q~ = H D q
    float qt[GRP][E];
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
        const int h = g * GRP + hh;
        const uint16_t *qp = p.q + ((size_t)b * p.hq + h) * kHeadDim + sub * E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float v = half_bits_to_float(live ? qp[e] : 0);
            qt[hh][e] = sign_of(p.k, sub * E + e) ? -v : v;
        }
#pragma unroll
        for (int s = 1; s < E; s <<= 1)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (e & s) continue;
                const float a = qt[hh][e], c = qt[hh][e + s];
                qt[hh][e] = a + c;
                qt[hh][e + s] = a - c;
            }
#pragma unroll
        for (int s = 1; s < LPU; s <<= 1)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float o = __shfl_xor(qt[hh][e], s, LPU);
                qt[hh][e] = (sub & s) ? (o - qt[hh][e]) : (qt[hh][e] + o);
            }
#pragma unroll
        for (int e = 0; e < E; ++e) qt[hh][e] *= p.qscale;
    }
    __syncthreads();

    float acc[GRP][E];
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = 0.0f;
    // Softmax state.  With at most 4 query heads per kv head, lane q of each
    // quad of a unit owns head q % GRP: it alone runs the online softmax of
    // that head, and the value weights reach the other lanes by DPP
    // broadcast within the quad.  With 8 query heads every lane runs all of
    // them.
    constexpr bool SPLIT = GRP <= 4;
    constexpr int NS = SPLIT ? 1 : GRP;          // softmax states per lane
    const int hown = sub % GRP;
    float m[NS], l[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        m[i] = -__builtin_inff();
        l[i] = 0.0f;
    }

    const int step = kWaves * tpi;
    const int tfirst = t0 + wave * tpi + tau;    // this lane group's first token
    // tokens tb = t0 + wave*tpi + i*step (i < nsteps) are this wave's steps
    const int nsteps = (t1 - (t0 + wave * tpi) + step - 1) / step;

    // K/V codes and norms of step i, loaded kPrefetch steps ahead of use into
    // a ring of kPrefetch + 1 slots (the slot refilled is the one used by the
    // previous step, so nothing is copied).
    //
    // All lanes of a wave step read the same 16-token page (a step covers tpi
    // tokens, tpi divides 16, and steps start on multiples of tpi), so the
    // page's block number and the step's row inside the page are
    // wave-uniform: they form a scalar base address, and every lane adds the
    // same per-lane byte offset each step.
    constexpr int R = kPrefetch + 1;
    const uint32_t lane_row = (uint32_t)(tau * p.hkv + g);          // row within a token's rows
    const uint32_t lane_code = lane_row * P + (uint32_t)(sub * (E * BITS / 8));
    const uint32_t lane_norm = lane_row * 4u;
    const uint64_t page_rows = (uint64_t)kAttnBlockSize * p.hkv;    // rows per block
    const uint32_t step_rows = (uint32_t)(tpi * p.hkv);             // rows read per step
    uint32_t rk[R][2], rv[R][2];
    float rkn[R], rvn[R];
    bool rok[R];
    auto fetch = [&](int i, int slot) {
        const int tb = t0 + wave * tpi + i * step;                    // wave-uniform
        int32_t blk = (tb < t1) ? bt_lds[(tb - t0) / kAttnBlockSize] : 0;
        blk = __builtin_amdgcn_readfirstlane(blk);
        const bool bok = blk >= 0 && blk < p.num_blocks;
        blk = bok ? blk : 0;
        rok[slot] = bok && live && (tb + tau < t1);
        // first row of this step: block * rows-per-block + token-in-page * hkv;
        // the step's rows are [row0, row0 + step_rows)
        const uint64_t row0 = (uint64_t)blk * page_rows + (uint64_t)((tb % kAttnBlockSize) * p.hkv);
        // unconditional loads: a step past the end reads block 0, which exists
        // whenever any token does; its score is masked below
        load_codes_buf<BITS, E>(page_rsrc(p.kp + row0 * P, step_rows * P), lane_code, rk[slot]);
        load_codes_buf<BITS, E>(page_rsrc(p.vp + row0 * P, step_rows * P), lane_code, rv[slot]);
        rkn[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  page_rsrc(p.kn + row0, step_rows * 4), lane_norm, 0, 0));
        rvn[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  page_rsrc(p.vn + row0, step_rows * 4), lane_norm, 0, 0));
    };
#pragma unroll
    for (int d = 0; d < kPrefetch; ++d) fetch(d, d);

    for (int i0 = 0; i0 < nsteps; i0 += R) {     // wave-uniform
#pragma unroll
        for (int d = 0; d < R; ++d) {
            if (i0 + d >= nsteps) break;
            fetch(i0 + d + kPrefetch, (d + kPrefetch) % R);
            const bool ok = rok[d];
            float val[E];
            expand<BITS, E>(tab, rk[d], val);
            float s[GRP];
#pragma unroll
            for (int hh = 0; hh < GRP; ++hh) {
                float dd = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) dd = __builtin_fmaf(qt[hh][e], val[e], dd);
                s[hh] = unit_sum<LPU>(dd) * rkn[d];
            }
            if constexpr (!SPLIT) {
#pragma unroll
                for (int hh = 0; hh < GRP; ++hh) s[hh] = ok ? s[hh] : -__builtin_inff();
            }
            float w[GRP];
            if constexpr (SPLIT) {
                float so = s[0];
#pragma unroll
                for (int hh = 1; hh < GRP; ++hh) so = (hown == hh) ? s[hh] : so;
                so = ok ? so : -__builtin_inff();
                // lazily raised reference: rescale only when a score passes m + 8
                if (__builtin_amdgcn_ballot_w64(so > m[0] + kLazy)) {
                    const float mn = (so > m[0] + kLazy) ? so : m[0];
                    const float a = (mn == m[0]) ? 1.0f : __builtin_amdgcn_exp2f(m[0] - mn);
                    l[0] *= a;
                    m[0] = mn;
#pragma unroll
                    for (int hh = 0; hh < GRP; ++hh) {
                        const float ah = quad_bcast(a, hh);
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[hh][e] *= ah;
                    }
                }
                const float pr = ok ? __builtin_amdgcn_exp2f(so - m[0]) : 0.0f;
                l[0] += pr;
                const float wo = pr * rvn[d];
#pragma unroll
                for (int hh = 0; hh < GRP; ++hh) w[hh] = quad_bcast(wo, hh);
            } else {
                bool need = false;
#pragma unroll
                for (int hh = 0; hh < GRP; ++hh) need |= s[hh] > m[hh % NS] + kLazy;
                if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
                    for (int hh = 0; hh < GRP; ++hh) {
                        const int i = hh % NS;
                        const float mn = (s[hh] > m[i] + kLazy) ? s[hh] : m[i];
                        const float a = (mn == m[i]) ? 1.0f : __builtin_amdgcn_exp2f(m[i] - mn);
                        l[i] *= a;
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[hh][e] *= a;
                        m[i] = mn;
                    }
                }
#pragma unroll
                for (int hh = 0; hh < GRP; ++hh) {
                    const int i = hh % NS;
                    const float pr = ok ? __builtin_amdgcn_exp2f(s[hh] - m[i]) : 0.0f;
                    l[i] += pr;
                    w[hh] = pr * rvn[d];
                }
            }
            expand<BITS, E>(tab, rv[d], val);
#pragma unroll
            for (int hh = 0; hh < GRP; ++hh)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[hh][e] = __builtin_fmaf(w[hh], val[e], acc[hh][e]);
        }
    }

    // every lane gets the softmax state of all its heads for the merges
    float mh[GRP], lh[GRP];
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
        mh[hh] = SPLIT ? quad_bcast(m[0], hh) : m[hh % NS];
        lh[hh] = SPLIT ? quad_bcast(l[0], hh) : l[hh % NS];
    }

    // merge the TPI units of the same kv head inside the wave (narrow caches)
    for (int off = p.hkv * LPU; off < tpi * p.hkv * LPU; off <<= 1) {
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh) {
            const float mo = __shfl_xor(mh[hh], off);
            const float lo = __shfl_xor(lh[hh], off);
            const float mn = mh[hh] > mo ? mh[hh] : mo;
            const float a = (mh[hh] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mh[hh] - mn);
            const float ao = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
            lh[hh] = lh[hh] * a + lo * ao;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float o = __shfl_xor(acc[hh][e], off);
                acc[hh][e] = acc[hh][e] * a + o * ao;
            }
            mh[hh] = mn;
        }
    }

    // merge the four waves through LDS: 2,3 -> 0,1, then 1 -> 0
    auto put = [&](float *buf) {
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh) {
#pragma unroll
            for (int e = 0; e < E; ++e) buf[(hh * E + e) * 64 + lane] = acc[hh][e];
            buf[(GRP * E + 2 * hh) * 64 + lane] = mh[hh];
            buf[(GRP * E + 2 * hh + 1) * 64 + lane] = lh[hh];
        }
    };
    auto take = [&](const float *buf) {
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh) {
            const float mo = buf[(GRP * E + 2 * hh) * 64 + lane];
            const float lo = buf[(GRP * E + 2 * hh + 1) * 64 + lane];
            const float mn = mh[hh] > mo ? mh[hh] : mo;
            const float a = (mh[hh] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mh[hh] - mn);
            const float ao = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
            lh[hh] = lh[hh] * a + lo * ao;
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[hh][e] = acc[hh][e] * a + buf[(hh * E + e) * 64 + lane] * ao;
            mh[hh] = mn;
        }
    };
    if (wave >= 2) put(xchg[wave - 2]);
    __syncthreads();
    if (wave < 2) take(xchg[wave]);
    __syncthreads();
    if (wave == 1) put(xchg[0]);
    __syncthreads();
    if (wave != 0 || !live || tau != 0) return;
    take(xchg[0]);

#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
        const int h = g * GRP + hh;
        float *dst = p.ws + (((size_t)b * p.hq + h) * p.num_splits + split) * kPartial;
        if (sub == 0) {
            dst[0] = mh[hh];
            dst[1] = lh[hh];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) dst[2 + sub * E + e] = acc[hh][e];
    }
}

// ---------------------------------------------------------------------------
// Matrix-core split kernel (4-bit codes).
//
// Per (sequence, kv head, split) one wave walks the split's pages; per page it
// runs the scores and the value accumulation as 16x16x32 f16 MFMA tiles:
//   scores  S^T[16 tokens][16 heads] = C_k[16 tokens][K] * Q[K][16 heads]
//   values  O[16 heads][16 dims]    += W[16 heads][K]   * C_v[K][16 dims]
// with the group's query heads padded to 16 columns / rows.
//
// binary16 carries 11 significant bits, too few for the 2e-3 output bound
// under peaked softmaxes, so every operand is split as x = x_hi + x_lo (both
// binary16) and the products x_hi y_hi + x_lo y_hi + x_hi y_lo are formed.
// The split costs no repacking: a code is looked up as the binary16 pair
// (c_hi, c_lo), which fills two adjacent K slots; the other operand holds
// (q_hi, q_hi) in those slots for one product and (q_lo, 0) for a second.
//
// Scale factors keep every binary16 operand in range and its low part
// normal: levels are stored times 16, the rotated query times a per-head
// power of two, and the value weights times 2^6 / vlim (vlim a power of two
// above the value norms); all are powers of two and removed exactly before
// the partial state is written.
//
// Lane layouts (l = lane, m = l % 16, r = l / 16), verified on gfx950:
//   A[m][8r .. 8r+7], B[8r .. 8r+7][m], C[4r .. 4r+3][m].
// Scores: lane (token m, r) holds codes of dims 32r .. 32r+31 of its token
// (one 16-byte load); chunk j covers dims 32r + 4j .. +3 of every r.  The
// query operand of lane (head m, r) covers the same dims.  The score tile
// leaves lane (head m, r) with tokens 4r .. 4r+3 -- exactly the K slots the
// value product wants in its A operand, so the weights never move between
// lanes.  Values: lane (column m, r) reads dword m (dims 8m .. 8m+7) of
// tokens 4r .. 4r+3; chunk jj accumulates dim 8m + jj.
constexpr int kMWaves = 4;                 // kv heads (waves) per workgroup
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMPrefetch = 1;              // extra ring slots: pages of loads in flight ahead of use
constexpr float kLevelScale = 16.0f;       // binary16 levels are 16 c
constexpr float kWShift = 6.0f;            // value weights carry 2^6
constexpr int kLutStride = 256;            // bytes per table entry row (32 lane copies of 8 B)
constexpr int kMTargetWaves = 4096;        // split-kernel waves aimed for

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Pairs of codes byte `k` of `word` decodes to.  The table holds, for each
// byte value, (pair of the low nibble, pair of the high nibble) in 32 copies
// 8 bytes apart -- one per lane of a 32-lane half wave -- filling a 256-byte
// row per byte value: lane s of a half wave always hits banks 2s, 2s+1,
// whatever the byte, so a table read never has a bank conflict.  One v_perm
// forms the address (byte << 8 | 8 s).
template <int K>
__device__ __forceinline__ u32x2 lut_pair(const char *tab, uint32_t word, uint32_t laneoff) {
    const uint32_t addr = __builtin_amdgcn_perm(word, laneoff, 0x0C0C0000u | ((4u + K) << 8));
    return *reinterpret_cast<const u32x2 *>(tab + addr);
}
__device__ __forceinline__ u32x2 lut_pair_rt(const char *tab, uint32_t word, int k, uint32_t laneoff) {
    switch (k & 3) {
        case 0: return lut_pair<0>(tab, word, laneoff);
        case 1: return lut_pair<1>(tab, word, laneoff);
        case 2: return lut_pair<2>(tab, word, laneoff);
        default: return lut_pair<3>(tab, word, laneoff);
    }
}

__device__ __forceinline__ f4 mfma(const u32x4 &a, const u32x4 &b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c,
                                                  0, 0, 0);
}

__global__ __launch_bounds__(kMThreads) void attn_mfma_kernel(AttnParams p) {
    constexpr int P = 64;                                    // packed bytes per row (4 bits)
    __shared__ __attribute__((aligned(16))) char tab[256 * kLutStride];
    __shared__ int32_t bt_lds[kMaxSplitTokens / kAttnBlockSize];

    const int b = blockIdx.y;
    const int split = blockIdx.x;
    int T = p.context_lens[b];
    T = T < 0 ? 0 : T;
    const int tmax = p.max_blocks * kAttnBlockSize;
    T = T > tmax ? tmax : T;
    if (p.num_blocks <= 0) T = 0;
    const int t0 = split * p.split_tokens;
    if (t0 >= T) return;                 // nothing here; combine skips this split
    const int t1 = (t0 + p.split_tokens < T) ? t0 + p.split_tokens : T;
    const int npages = (t1 - t0 + kAttnBlockSize - 1) / kAttnBlockSize;

    for (int i = threadIdx.x; i < 256 * 32; i += kMThreads) {
        const int e = i >> 5, c = i & 31;
        u32x2 v;
        v.x = level_pair(p.k, e & 15);
        v.y = level_pair(p.k, e >> 4);
        *reinterpret_cast<u32x2 *>(tab + e * kLutStride + 8 * c) = v;
    }
    {
        const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks + t0 / kAttnBlockSize;
        for (int i = threadIdx.x; i < npages; i += kMThreads) bt_lds[i] = bt[i];
    }
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.z * kMWaves + wave;                // kv head
    if (g >= p.hkv) return;                                   // no barrier follows
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, r = lane >> 4;
    const int grp = p.hq / p.hkv;
    const bool hv = m < grp;                                  // a real query head column
    const uint32_t laneoff = 8u * (uint32_t)(lane & 31);

    // ---- rotated query, one head per lane column, dims 32r .. 32r+31 ----
    u32x4 bq1[8], bq2[8];
    float qsl;
    {
        float qv[32];
        const int mq = hv ? m : 0;                            // padding columns read head 0, then drop it
        const uint16_t *qp = p.q + ((size_t)b * p.hq + (size_t)g * grp + mq) * kHeadDim + 32 * r;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const float v = hv ? half_bits_to_float(qp[e]) : 0.0f;
            qv[e] = sign_of(p.k, 32 * r + e) ? -v : v;
        }
#pragma unroll
        for (int s = 1; s < 32; s <<= 1)
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                if (e & s) continue;
                const float a = qv[e], c = qv[e + s];
                qv[e] = a + c;
                qv[e + s] = a - c;
            }
#pragma unroll
        for (int s = 16; s < 64; s <<= 1)
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const float o = __shfl_xor(qv[e], s);
                qv[e] = (lane & s) ? (o - qv[e]) : (qv[e] + o);
            }
        // per-head power of two bringing max |q~| to [2^13, 2^14)
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(qv[e]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
        int ex = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 14;   // amax in [2^(ex-1), 2^ex)
        ex = ex < -100 ? -100 : ex;
        const float sc = __builtin_bit_cast(float, (uint32_t)(127 + 14 - ex) << 23);   // 2^(14 - ex)
        qsl = p.qscale / (sc * kLevelScale);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t w1[4], w2[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float v = qv[4 * j + t] * sc;
                const _Float16 hi = (_Float16)v;
                const _Float16 lo = (_Float16)(v - (float)hi);
                w1[t] = pack_half2(hi, hi);
                w2[t] = pack_half2(lo, (_Float16)0.0f);
            }
            bq1[j] = u32x4{w1[0], w1[1], w1[2], w1[3]};
            bq2[j] = u32x4{w2[0], w2[1], w2[2], w2[3]};
        }
    }

    f4 acc[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[jj] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float M = -__builtin_inff();          // base-2 reference of head m (uniform over r)
    float lsum = 0.0f;                    // sum of exp2(s - M) over this lane's tokens
    float vlim = 0.0f;                    // power of two above every value norm seen (wave-uniform)
    float vscale = 0.0f;                  // 2^6 / vlim

    // per-lane byte offsets inside one page of this kv head
    const uint32_t row_bytes = (uint32_t)p.hkv * P;           // one token of all kv heads
    const uint32_t offk = (uint32_t)m * row_bytes + (uint32_t)g * P + 16u * r;
    uint32_t offv[4], offn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        offv[i] = (uint32_t)(4 * r + i) * row_bytes + (uint32_t)g * P + 4u * m;
        offn[i] = ((uint32_t)(4 * r + i) * p.hkv + g) * 4u;
    }
    const uint32_t page_bytes = kAttnBlockSize * row_bytes;
    const uint32_t page_nbytes = kAttnBlockSize * p.hkv * 4u;

    // Loads of page pg sit in ring slot pg % R.  The refill for page pg + R
    // is issued at the end of step pg, once the slot has been consumed; its
    // block number was read from LDS one step earlier.
    constexpr int R = kMPrefetch + 1;
    u32x4 rk[R];
    uint32_t rv[R][4];
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
        const __amdgpu_buffer_rsrc_t rsk = page_rsrc(p.kp + (size_t)blk * page_bytes, page_bytes);
        const __amdgpu_buffer_rsrc_t rsv = page_rsrc(p.vp + (size_t)blk * page_bytes, page_bytes);
        const __amdgpu_buffer_rsrc_t rkn_ = page_rsrc(p.kn + (size_t)blk * kAttnBlockSize * p.hkv, page_nbytes);
        const __amdgpu_buffer_rsrc_t rvn_ = page_rsrc(p.vn + (size_t)blk * kAttnBlockSize * p.hkv, page_nbytes);
        rk[slot] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsk, offk, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[slot][i] = __builtin_amdgcn_raw_buffer_load_b32(rsv, offv[i], 0, 0);
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

    // one page: table reads, score tiles, softmax, value tiles, refill
    auto step = [&](const int pg, const int d) {
            // scores of tokens 4r .. 4r+3 for head m, over two independent chains
            u32x2 ka[16];
#pragma unroll
            for (int kb = 0; kb < 16; ++kb) ka[kb] = lut_pair_rt(tab, rk[d][kb >> 2], kb & 3, laneoff);
            f4 S0 = f4{0.0f, 0.0f, 0.0f, 0.0f}, S1 = S0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const u32x4 A = u32x4{ka[2 * j].x, ka[2 * j].y, ka[2 * j + 1].x, ka[2 * j + 1].y};
                S0 = mfma(A, bq1[j], S0);
                S1 = mfma(A, bq2[j], S1);
            }
            // value codes of the page, read while the score tiles finish
            u32x2 va[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) va[i][k2] = lut_pair_rt(tab, rv[d][i], k2, laneoff);
            const f4 S = S0 + S1;

            // online softmax in base 2.  Two lazily raised references: M per
            // head (rescale when a score passes M + 8) and a power of two vlim
            // per wave bounding the value norms (rescale when a norm passes
            // it); the weights w = 2^(s - M) * n_v * 2^6 / vlim then stay
            // below 2^14, inside binary16.
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
                // accumulator rows are heads 4r + i
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float fi = __shfl(f, 4 * r + i) * fv;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) acc[jj][i] *= fi;
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
            const u32x4 A1 = u32x4{w1[0], w1[1], w1[2], w1[3]};
            const u32x4 A2 = u32x4{w2[0], w2[1], w2[2], w2[3]};

            // values: dims 8m + jj of tokens 4r .. 4r+3
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                const u32x4 B0 = u32x4{va[0][k2].x, va[1][k2].x, va[2][k2].x, va[3][k2].x};
                const u32x4 B1 = u32x4{va[0][k2].y, va[1][k2].y, va[2][k2].y, va[3][k2].y};
                acc[2 * k2] = mfma(A1, B0, acc[2 * k2]);
                acc[2 * k2 + 1] = mfma(A1, B1, acc[2 * k2 + 1]);
                acc[2 * k2] = mfma(A2, B0, acc[2 * k2]);
                acc[2 * k2 + 1] = mfma(A2, B1, acc[2 * k2 + 1]);
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
    // partial state of head g*grp + h: m and l from lane h, accumulators from
    // lanes (column c, row h / 4) at register h % 4 -> dims 8c .. 8c+7
    const float unscale = vlim / (kLevelScale * 64.0f);     // undo 16 c and 2^6 / vlim
    float *base = p.ws + (((size_t)b * p.hq + (size_t)g * grp) * p.num_splits + split) * kPartial;
    const size_t hstride = (size_t)p.num_splits * kPartial;
    if (r == 0 && hv) {
        float *dst = base + (size_t)m * hstride;
        dst[0] = M;
        dst[1] = lsum;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * r + i;
        if (h >= grp) break;
        float2 *dst = reinterpret_cast<float2 *>(base + (size_t)h * hstride + 2 + 8 * m);   // 8-byte aligned
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) dst[jj >> 1] = float2(acc[jj][i] * unscale, acc[jj + 1][i] * unscale);
    }
}

// One wave per (sequence, query head): merge the splits, undo the rotation.
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnParams p) {
    const int bh = blockIdx.x;
    const int b = bh / p.hq;
    const int lane = threadIdx.x;
    int T = p.context_lens[b];
    T = T < 0 ? 0 : T;
    const int tmax = p.max_blocks * kAttnBlockSize;
    T = T > tmax ? tmax : T;
    if (p.num_blocks <= 0) T = 0;
    const int ns = (T + p.split_tokens - 1) / p.split_tokens;
    const float *src = p.ws + (size_t)bh * p.num_splits * kPartial;

    // the largest running maximum over the splits (lane s reads split s)
    float mx = -__builtin_inff();
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int s = s0 + lane;
        if (s < ns) {
            const float ms = src[(size_t)s * kPartial];
            mx = ms > mx ? ms : mx;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float other = __shfl_xor(mx, o);
        mx = other > mx ? other : mx;
    }
    // split weights, then this lane's coordinates 2*lane, 2*lane+1
    float lsum = 0.0f, a0 = 0.0f, a1 = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int s = s0 + lane;
        float w = 0.0f;
        if (s < ns) {
            const float ls = src[(size_t)s * kPartial + 1];
            w = (ls > 0.0f) ? __builtin_amdgcn_exp2f(src[(size_t)s * kPartial] - mx) : 0.0f;
            lsum += w * ls;
        }
        const int cnt = (ns - s0 < 64) ? ns - s0 : 64;
#pragma unroll 8
        for (int j = 0; j < cnt; ++j) {
            const float wj = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
            const float2 e =
                *reinterpret_cast<const float2 *>(src + (size_t)(s0 + j) * kPartial + 2 + 2 * lane);
            a0 = __builtin_fmaf(wj, e.x, a0);
            a1 = __builtin_fmaf(wj, e.y, a1);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
    // inverse transform: x = D H acc / 128 -- coordinate bit 0 in registers,
    // bits 1..6 across lanes
    float x0 = (a0 + a1) * inv, x1 = (a0 - a1) * inv;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const float o0 = __shfl_xor(x0, s), o1 = __shfl_xor(x1, s);
        x0 = (lane & s) ? (o0 - x0) : (x0 + o0);
        x1 = (lane & s) ? (o1 - x1) : (x1 + o1);
    }
    const int i0 = 2 * lane, i1 = 2 * lane + 1;
    x0 *= (1.0f / kHeadDim);
    x1 *= (1.0f / kHeadDim);
    if (sign_of(p.k, i0)) x0 = -x0;
    if (sign_of(p.k, i1)) x1 = -x1;
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    uint16_t *o = p.out + (size_t)bh * kHeadDim;
    const uint32_t packed2 = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    reinterpret_cast<uint32_t *>(o)[lane] = packed2;
}

int wave_units(int grp) { return grp <= 4 ? 8 : 4; }   // units per wave: E = 16 or 8

// The matrix-core kernel serves 4-bit caches with up to 16 query heads per
// kv head; the vector kernel serves the rest.
bool mfma_path(const AttnShape &s) {
    const int grp = s.num_q_heads / s.num_kv_heads;
    return s.bits == 4 && grp >= 1 && grp <= 16;
}

}  // namespace

bool attn_supported(const AttnShape &s) {
    if (mfma_path(s)) return true;
    const int grp = s.num_q_heads / s.num_kv_heads;
    if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return false;
    const int upw = wave_units(grp);
    return s.num_kv_heads % upw == 0 || upw % s.num_kv_heads == 0;
}

namespace {

int valu_split_tokens(const AttnShape &s) {
    const int ctx = s.max_blocks * kAttnBlockSize;
    const int grp = s.num_q_heads / s.num_kv_heads;
    const int upw = wave_units(grp);
    const int zch = s.num_kv_heads >= upw ? s.num_kv_heads / upw : 1;
    const int per_seq = s.batch * zch > 0 ? (kTargetGroups + s.batch * zch - 1) / (s.batch * zch) : 1;
    int st = (ctx + per_seq - 1) / per_seq;
    st = (st + 63) / 64 * 64;
    st = st < 256 ? 256 : st;
    return st > kMaxSplitTokens ? kMaxSplitTokens : st;
}

int mfma_split_tokens(const AttnShape &s) {
    const int ctx = s.max_blocks * kAttnBlockSize;
    const int units = s.batch * s.num_kv_heads;           // one wave each per split
    const int per_seq = units > 0 ? (kMTargetWaves + units - 1) / units : 1;
    int st = (ctx + per_seq - 1) / per_seq;
    st = (st + kAttnBlockSize - 1) / kAttnBlockSize * kAttnBlockSize;
    st = st < 256 ? 256 : st;
    return st > kMaxSplitTokens ? kMaxSplitTokens : st;
}

int splits_for(const AttnShape &s, int st) {
    const int ctx = s.max_blocks * kAttnBlockSize;
    const int ns = (ctx + st - 1) / st;
    return ns < 1 ? 1 : ns;
}

}  // namespace

int attn_split_tokens(const AttnShape &s) {
    return mfma_path(s) ? mfma_split_tokens(s) : valu_split_tokens(s);
}

int attn_num_splits(const AttnShape &s) { return splits_for(s, attn_split_tokens(s)); }

size_t attn_workspace_bytes(const AttnShape &s) {
    // enough for either kernel, so that the size does not depend on the bit width
    AttnShape s4 = s;
    s4.bits = 4;
    const int ns = std::max(splits_for(s, valu_split_tokens(s)),
                            mfma_path(s4) ? splits_for(s, mfma_split_tokens(s4)) : 1);
    return (size_t)s.batch * s.num_q_heads * ns * kPartial * sizeof(float);
}

hipError_t launch_attn(const AttnShape &s, const CodecConsts &k, const void *q,
                       const uint8_t *k_packed, const float *k_norms, const uint8_t *v_packed,
                       const float *v_norms, const int32_t *block_tables,
                       const int32_t *context_lens, float scale, void *out, void *workspace,
                       hipStream_t stream) {
    const int grp = s.num_q_heads / s.num_kv_heads;
    const int upw = wave_units(grp);
    const bool mf = mfma_path(s);
    if (!mf && !(s.num_kv_heads % upw == 0 || upw % s.num_kv_heads == 0)) return hipErrorInvalidValue;
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
    p.qscale = scale * 1.4426950408889634f / kHeadDim;
    p.k = k;
    if (mf) {
        const dim3 grid(p.num_splits, s.batch, (s.num_kv_heads + kMWaves - 1) / kMWaves);
        hipLaunchKernelGGL(attn_mfma_kernel, grid, dim3(kMThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_combine_kernel, dim3(s.batch * s.num_q_heads), dim3(64), 0, stream, p);
        return hipGetLastError();
    }
    const int zch = s.num_kv_heads >= upw ? s.num_kv_heads / upw : 1;
    const dim3 grid(p.num_splits, s.batch, zch), block(kThreads);
#define TQ_SPLIT(B, GR, E) \
    hipLaunchKernelGGL((attn_split_kernel<B, GR, E>), grid, block, 0, stream, p)
#define TQ_BITS(GR, E)                           \
    switch (s.bits) {                            \
        case 2: TQ_SPLIT(2, GR, E); break;       \
        case 3: TQ_SPLIT(3, GR, E); break;       \
        case 4: TQ_SPLIT(4, GR, E); break;       \
        default: return hipErrorInvalidValue;   \
    }
    switch (grp) {
        case 1: TQ_BITS(1, 16) break;
        case 2: TQ_BITS(2, 16) break;
        case 4: TQ_BITS(4, 16) break;
        case 8: TQ_BITS(8, 8) break;
        default: return hipErrorInvalidValue;
    }
#undef TQ_BITS
#undef TQ_SPLIT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(s.batch * s.num_q_heads), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
