// TurboQuant encode / decode kernels for gfx950 (CDNA4, wave64).
//
// Method: aither-kvcache PyPI page, "Algorithm" (normalise, rotate by a fixed
// random orthogonal matrix, quantize each coordinate with a Lloyd-Max
// codebook, pack, store the f32 norm; decode reverses it).  The rotation is a
// seeded sign flip followed by a Walsh-Hadamard transform (qbc.network blog,
// "What TurboQuant is": a multiplier-free Walsh-Hadamard rotation).
//
// Work mapping.  Four lanes (a DPP quad) own one vector of D = 64, 128 or
// 256 coordinates; K = D / 32.  Lane q of the quad owns coordinates
// 32k + 8q + j (k < K, j < 8), held in register r = 8k + j.  Each fp16 access
// instruction therefore moves 64 contiguous bytes per quad (16 B per lane),
// and a wave of 16 quads touches 16 whole 64-byte segments.  Coordinate bits
// 0-2 and 5 up are register bits, bits 3-4 are the lane's place in the quad:
// the D-point fast Walsh-Hadamard transform is log2(D) - 2 register butterfly
// stages plus 2 cross-lane stages done with DPP quad permutations -- no LDS
// traffic for the transform.
//
// The codes of one lane and group k are 8 consecutive codes, i.e. a
// contiguous 8*bits-bit field of the packed row.  At 4 bits each field is a
// dword; at 2 and 3 bits neighbouring lanes splice their fields into whole
// dwords with one DPP move, so packed rows are read and written as dwords.
//
// Cross-lane stages use one DPP-fused multiply-add per value,
// v += partner * m, m = +1 on the lower lane and -1 on the upper one.  The
// upper lane then holds the negated difference; that sign is tracked per lane
// (eps) and folded into the per-vector scale, which is multiplied in during
// the last register stage anyway.
//
// Quantizer.  y = 8 z is formed as w * (8 eps / ||x||).  The integer part of
// y indexes a 257-entry LDS table whose cells are narrower than the smallest
// gap between two thresholds, so each cell holds at most one threshold:
// code = base[cell] + (y > thr[cell]).  A coordinate exactly on a threshold
// takes the lower code, as in the definition.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kCells = kEncCells;     // quantizer cells cover y in (-129, 129)
constexpr int kThreads = 256;         // 4 waves: one vector per quad per pass, 64 per pass
constexpr int kVecPerBlock = kThreads / 4;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// DPP quad permutations
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]: partner q^1
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]: partner q^2
constexpr int kQuadNext = 0xF9;   // quad_perm [1,2,3,3]: lane q reads lane q+1
// DPP row rotations
constexpr int kRowRor4 = 0x124;   // row_ror:4: lane m of a 16-lane row <- lane (m - 4) mod 16
constexpr int kRowRor12 = 0x12C;  // row_ror:12: lane m <- lane (m + 4) mod 16

template <int CTRL>
__device__ __forceinline__ uint32_t quad_move(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float quad_move(float v) {
    return __builtin_bit_cast(float, quad_move<CTRL>(__builtin_bit_cast(uint32_t, v)));
}

// The two cross-lane butterfly stages (coordinate bits 3 and 4):
//   f[r] += f[r] of lane q^1 * ma,  then  f[r] += f[r] of lane q^2 * mb.
// One v_fmac_f32 with a DPP source per value, 16 or 32 values per asm block.
// The leading s_nop 1 provides the two wait states a DPP read of a VGPR needs
// after a VALU write; inside a block no instruction reads a register written
// by the one before it.
#define TQ_FMAC2(A, B, CTRL, M)                                                                  \
    "v_fmac_f32_dpp %" #A ", %" #A ", %" #M " " CTRL "\n\t"                                     \
    "v_fmac_f32_dpp %" #B ", %" #B ", %" #M " " CTRL "\n\t"
#define TQ_FMAC16(CTRL, M)                                                                       \
    TQ_FMAC2(0, 1, CTRL, M) TQ_FMAC2(2, 3, CTRL, M) TQ_FMAC2(4, 5, CTRL, M)                     \
    TQ_FMAC2(6, 7, CTRL, M) TQ_FMAC2(8, 9, CTRL, M) TQ_FMAC2(10, 11, CTRL, M)                   \
    TQ_FMAC2(12, 13, CTRL, M) TQ_FMAC2(14, 15, CTRL, M)
#define TQ_FMAC32(CTRL, M)                                                                       \
    TQ_FMAC16(CTRL, M) TQ_FMAC2(16, 17, CTRL, M) TQ_FMAC2(18, 19, CTRL, M)                      \
    TQ_FMAC2(20, 21, CTRL, M) TQ_FMAC2(22, 23, CTRL, M) TQ_FMAC2(24, 25, CTRL, M)               \
    TQ_FMAC2(26, 27, CTRL, M) TQ_FMAC2(28, 29, CTRL, M) TQ_FMAC2(30, 31, CTRL, M)
#define TQ_OPS16(O)                                                                              \
    "+v"(f[O + 0]), "+v"(f[O + 1]), "+v"(f[O + 2]), "+v"(f[O + 3]), "+v"(f[O + 4]),            \
        "+v"(f[O + 5]), "+v"(f[O + 6]), "+v"(f[O + 7]), "+v"(f[O + 8]), "+v"(f[O + 9]),        \
        "+v"(f[O + 10]), "+v"(f[O + 11]), "+v"(f[O + 12]), "+v"(f[O + 13]), "+v"(f[O + 14]),   \
        "+v"(f[O + 15])
#define TQ_XOR1 "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
#define TQ_XOR2 "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"

template <int R>
__device__ __forceinline__ void fwht_quad(float (&f)[R], float ma, float mb) {
    static_assert(R == 16 || R % 32 == 0, "16, 32 or 64 registers");
    if constexpr (R == 16) {
        asm volatile("s_nop 1\n\t" TQ_FMAC16(TQ_XOR1, 16) : TQ_OPS16(0) : "v"(ma));
        asm volatile("s_nop 1\n\t" TQ_FMAC16(TQ_XOR2, 16) : TQ_OPS16(0) : "v"(mb));
    } else {
#pragma unroll
        for (int c = 0; c < R; c += 32)
            asm volatile("s_nop 1\n\t" TQ_FMAC32(TQ_XOR1, 32)
                         : TQ_OPS16(c), TQ_OPS16(c + 16) : "v"(ma));
#pragma unroll
        for (int c = 0; c < R; c += 32)
            asm volatile("s_nop 1\n\t" TQ_FMAC32(TQ_XOR2, 32)
                         : TQ_OPS16(c), TQ_OPS16(c + 16) : "v"(mb));
    }
}
#undef TQ_XOR2
#undef TQ_XOR1
#undef TQ_OPS16
#undef TQ_FMAC32
#undef TQ_FMAC16
#undef TQ_FMAC2

// Register butterfly stages with strides FIRST..R/4 (register bits), then the
// stride-R/2 stage fused with the per-vector scale s:
//   (a, b) -> ((a + b) s, (a - b) s) = (fma(a, s, b s), fma(a, s, -b s)).
template <int FIRST, int R>
__device__ __forceinline__ void fwht_registers_scaled(float (&f)[R], float s) {
    constexpr int H = R / 2;
#pragma unroll
    for (int st = FIRST; st < H; st <<= 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r & st) continue;
            const float a = f[r], b = f[r + st];
            f[r] = a + b;
            f[r + st] = a - b;
        }
    }
#pragma unroll
    for (int r = 0; r < H; ++r) {
        const float a = f[r], bs = f[r + H] * s;
        f[r] = __builtin_fmaf(a, s, bs);
        f[r + H] = __builtin_fmaf(a, s, -bs);
    }
}

// Buffer resource over `bytes` bytes at `base` (wave-uniform).  Accesses
// through it take a scalar base and a 32-bit per-lane offset; reads outside
// the range return 0 and writes outside it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Signs of register pair (2i, 2i+1) of lane q, i.e. of coordinates
// 32(i/4) + 8q + 2(i%4) + {0, 1}: XOR masks of the binary16 sign bits, or
// (ONES) the binary16 pair (sigma_a, sigma_b) itself.  Thread t < 16K writes
// word i = t % 4K of lane q = t / 4K to LDS once per block; every lane then
// reads its 4K words with K broadcast 16-byte LDS reads.
template <int K, bool ONES>
__device__ __forceinline__ void store_sign_mask(const CodecConsts &k, int t, uint32_t *smask) {
    const int q = t / (4 * K), i = t % (4 * K);
    const uint32_t w = k.sign[i >> 2] >> (8 * q + 2 * (i & 3));
    const uint32_t m = ((w & 1u) << 15) | (((w >> 1) & 1u) << 31);
    smask[t] = ONES ? (m | 0x3C003C00u) : m;   // 0x3C00: binary16 1.0
}

// The mask word store_sign_mask writes for thread t, from K sign words that
// are selected as scalars: a private copy of the words indexed per lane would
// live in scratch memory.
template <int K, bool ONES>
__device__ __forceinline__ uint32_t sign_mask_word(const uint32_t *sign, int t) {
    const int q = t / (4 * K), i = t % (4 * K);
    uint32_t sw = __builtin_amdgcn_readfirstlane(sign[0]);
#pragma unroll
    for (int j = 1; j < K; ++j) sw = (i >> 2) == j ? __builtin_amdgcn_readfirstlane(sign[j]) : sw;
    const uint32_t w = sw >> (8 * q + 2 * (i & 3));
    const uint32_t m = ((w & 1u) << 15) | (((w >> 1) & 1u) << 31);
    return ONES ? (m | 0x3C003C00u) : m;   // 0x3C00: binary16 1.0
}

// sigma_a a + sigma_b b and sigma_a a - sigma_b b for binary16 pairs
// x = (a, b), s = (sigma_a, sigma_b): v_dot2_f32_f16 with a zero addend (the
// three-operand form, which needs no zeroed destination), the second with
// the high half of s negated.  The products are exact.
__device__ __forceinline__ float dot2_sum(uint32_t x, uint32_t s) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(s));
    return r;
}
__device__ __forceinline__ float dot2_diff(uint32_t x, uint32_t s) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(s));
    return r;
}

template <int K>
__device__ __forceinline__ void load_sign_masks(const u32x4 *smask, int q,
                                                uint32_t (&xm)[4 * K]) {
#pragma unroll
    for (int m = 0; m < K; ++m) {
        const u32x4 u = smask[K * q + m];
        xm[4 * m] = u.x;
        xm[4 * m + 1] = u.y;
        xm[4 * m + 2] = u.z;
        xm[4 * m + 3] = u.w;
    }
}

// 4-bit packing of one code into byte DB of `acc`: the cell's code word W
// holds base / base + 1 in bytes S0 / S1 (pre-shifted by 0 or 4); a compare
// against the cell's threshold picks one of them and an SDWA v_cndmask writes
// it into the byte, leaving the other bytes untouched.
// The first byte written into a dword (byte 0) zero-pads the rest.
#define TQ_PUT_CODE(DB, S0, S1)                                                                \
    asm volatile("v_cmp_gt_f32 vcc, %1, %2\n\t"                                                 \
                 "v_cndmask_b32_sdwa %0, %3, %3, vcc dst_sel:BYTE_" #DB                         \
                 " dst_unused:UNUSED_PRESERVE src0_sel:BYTE_" #S0 " src1_sel:BYTE_" #S1          \
                 : "+v"(acc)                                                                    \
                 : "v"(y), "v"(thr), "v"(W)                                                     \
                 : "vcc")
#define TQ_PUT_FIRST(S0, S1)                                                                   \
    asm volatile("v_cmp_gt_f32 vcc, %1, %2\n\t"                                                 \
                 "v_cndmask_b32_sdwa %0, %3, %3, vcc dst_sel:BYTE_0"                            \
                 " dst_unused:UNUSED_PAD src0_sel:BYTE_" #S0 " src1_sel:BYTE_" #S1               \
                 : "=v"(acc)                                                                    \
                 : "v"(y), "v"(thr), "v"(W)                                                     \
                 : "vcc")

template <int R>
__device__ __forceinline__ void put_code4(uint32_t &acc, float y, float thr, uint32_t W) {
    constexpr int j = R & 7;
    if (j == 0) TQ_PUT_FIRST(0, 1);
    if (j == 1) TQ_PUT_FIRST(2, 3);
    if (j == 2) TQ_PUT_CODE(1, 0, 1);
    if (j == 3) TQ_PUT_CODE(1, 2, 3);
    if (j == 4) TQ_PUT_CODE(2, 0, 1);
    if (j == 5) TQ_PUT_CODE(2, 2, 3);
    if (j == 6) TQ_PUT_CODE(3, 0, 1);
    if (j == 7) TQ_PUT_CODE(3, 2, 3);
}

// 2-bit packing: the code word holds base / base + 1 in bytes 0 / 1, and the
// selected code goes, unshifted, into byte DB of one of four accumulators (one
// per code position within a byte); FIRST marks an accumulator's first write,
// which is always byte 0.
template <int DB, bool FIRST>
__device__ __forceinline__ void put_code2(uint32_t &acc, float y, float thr, uint32_t W) {
    if constexpr (FIRST) TQ_PUT_FIRST(0, 1);
    else if constexpr (DB == 1) TQ_PUT_CODE(1, 0, 1);
    else if constexpr (DB == 2) TQ_PUT_CODE(2, 0, 1);
    else TQ_PUT_CODE(3, 0, 1);
}
#undef TQ_PUT_CODE
#undef TQ_PUT_FIRST

// LDS writes of a wave made visible to its other lanes: LDS instructions of
// one wave execute in order, so only the compiler has to be kept from moving
// the accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Store QW consecutive dwords (a quarter of a packed row) at byte offset off.
template <int QW>
__device__ __forceinline__ void store_quarter(const uint32_t (&v)[QW], __amdgpu_buffer_rsrc_t rp,
                                              uint32_t off) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    if constexpr (QW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < QW; i += 4)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{v[i], v[i + 1], v[i + 2], v[i + 3]}, rp,
                                                   off + 4u * i, 0, 0);
    } else if constexpr (QW == 3) {
        __builtin_amdgcn_raw_buffer_store_b96(u32x3{v[0], v[1], v[2]}, rp, off, 0, 0);
    } else if constexpr (QW == 6) {
        __builtin_amdgcn_raw_buffer_store_b96(u32x3{v[0], v[1], v[2]}, rp, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b96(u32x3{v[3], v[4], v[5]}, rp, off + 12u, 0, 0);
    } else if constexpr (QW == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{v[0], v[1]}, rp, off, 0, 0);
    } else {
        static_assert(QW == 1, "quarter size");
        __builtin_amdgcn_raw_buffer_store_b32(v[0], rp, off, 0, 0);
    }
}

// 2-bit codes of f[R..]: code r = 8k + j of the lane's stream sits at bit
// 16 (k & 1) + 2j of stream dword k / 2, i.e. in byte 2 (k & 1) + j / 4 at
// position j % 4; a[p][m] collects position p of stream dword m.
template <int R, int N>
__device__ __forceinline__ void quantize2(const float (&f)[N], const float2 *qtab,
                                          uint32_t (&a)[4][N / 16]) {
    if constexpr (R < N) {
        constexpr int k = R >> 3, j = R & 7;
        constexpr int byte = 2 * (k & 1) + (j >> 2);
        const float y = f[R];
        const float2 e = qtab[(int)y + kCells];
        put_code2<byte, byte == 0>(a[j & 3][k >> 1], y, e.x, __builtin_bit_cast(uint32_t, e.y));
        quantize2<R + 1, N>(f, qtab, a);
    }
}

template <int R, int N>
__device__ __forceinline__ void quantize4(const float (&f)[N], const float2 *qtab,
                                          uint32_t (&lo)[N / 8], uint32_t (&hi)[N / 8]) {
    if constexpr (R < N) {
        const float y = f[R];
        const float2 e = qtab[(int)y + kCells];
        const uint32_t W = __builtin_bit_cast(uint32_t, e.y);
        if (R & 1) put_code4<R>(hi[R >> 3], y, e.x, W);
        else put_code4<R>(lo[R >> 3], y, e.x, W);
        quantize4<R + 1, N>(f, qtab, lo, hi);
    }
}

// Encode: vectors per quad, chosen by timing 1, 2 and 4 on MI355X over a 4 GiB
// cache.  At head_dim 64 a vector is only 128 bytes, and four per quad (all
// loads issued first) run 9-12% faster than one; at 128 and 256 one is
// fastest.
constexpr int enc_vpq(int d) { return d == 64 ? 4 : 1; }

template <int D, int BITS, bool PAGED>
__global__ __launch_bounds__(kThreads) void encode_kernel(const u32x4 *__restrict__ x, int64_t n,
                                                          const int64_t *__restrict__ slots,
                                                          int64_t num_slots,
                                                          uint32_t *__restrict__ packed,
                                                          float *__restrict__ norms,
                                                          CodecConsts k, EncTable tb) {
    constexpr int K = D / 32;                   // register groups per lane
    constexpr int R = 8 * K;                    // coordinates per lane
    constexpr int PW = D * BITS / 32;           // packed dwords per vector
    constexpr uint32_t VB = 2 * D;              // fp16 bytes per vector
    constexpr int NPK = (K * BITS + 3) / 4;     // dwords of the lane's field stream (4, 2 bits)
    __shared__ float2 qtab[2 * kCells + 1];
    __shared__ u32x4 smask[4 * K];
    // one staging row per quad for the packed output: PW dwords, padded to a
    // multiple of 4 dwords (16-byte reads) whose quarter is odd, so that the
    // quads of a wave spread over the LDS banks
    // (rows of a whole number of dwords per lane only: not 3 bits at head_dim 64)
    constexpr bool kStage = !PAGED && PW % 4 == 0;
    constexpr int kStageRow = ((PW / 4) % 2 == 0) ? PW + 4 : PW;
    __shared__ __attribute__((aligned(16))) uint32_t stage[kStage ? kVecPerBlock * kStageRow : 1];
    for (int t = threadIdx.x; t < 2 * kCells + 1; t += blockDim.x) qtab[t] = tb.cell[t];
    if (threadIdx.x < 16 * K)
        store_sign_mask<K, true>(k, threadIdx.x, reinterpret_cast<uint32_t *>(smask));
    __syncthreads();

    const int q = threadIdx.x & 3;
    uint32_t sg[4 * K];   // binary16 sign pairs (sigma_a, sigma_b)
    load_sign_masks<K>(smask, q, sg);
    const float ma = (q & 1) ? -1.0f : 1.0f;
    const float mb = (q & 2) ? -1.0f : 1.0f;
    const float eps8 = 8.0f * ma * mb;
    // 2-bit: byte selectors splicing this lane's and the partner's 16-bit fields
    const uint32_t sel2 = (q & 1) ? 0x03020706u : 0x05040100u;

    // this block's vectors [v0, v0 + nb): scalar base, per-lane offsets.  Quad
    // qi takes vectors v0 + 64 vi + qi (vi < VPQ), so that every access
    // instruction of a wave covers 16 consecutive vectors; all their loads
    // are issued before the first one is transformed.
    constexpr int VPQ = enc_vpq(D);
    constexpr int VPB = kVecPerBlock * VPQ;
    const int64_t v0 = (int64_t)blockIdx.x * VPB;
    const uint32_t nb = (uint32_t)((n - v0 < VPB) ? n - v0 : VPB);
    const uint32_t qi = threadIdx.x >> 2;
    if (v0 + qi >= n) return;   // uniform over the quad; no barrier follows
    const __amdgpu_buffer_rsrc_t rx = span_rsrc(x + v0 * (D / 8), nb * VB);
    uint32_t wv[VPQ][4 * K];   // lanes past the end read zeros (bounds check)
#pragma unroll
    for (int vi = 0; vi < VPQ; ++vi) {
        const uint32_t xo = (vi * kVecPerBlock + qi) * VB + 16u * q;
#pragma unroll
        for (int g = 0; g < K; ++g) {
            const u32x4 u = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 64u * g, 0, 0));
            wv[vi][4 * g + 0] = u.x;
            wv[vi][4 * g + 1] = u.y;
            wv[vi][4 * g + 2] = u.z;
            wv[vi][4 * g + 3] = u.w;
        }
    }
#pragma unroll
    for (int vi = 0; vi < VPQ; ++vi) {
        const uint32_t qv = vi * kVecPerBlock + qi;   // vector within the block
        const int64_t v = v0 + qv;
        if (v >= n) break;   // uniform over the quad
        const uint32_t (&w)[4 * K] = wv[vi];
        // ||x||^2 from the fp16 pairs (products exact in f32, f32 accumulate)
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 4 * K; ++j) {
            const half2_t h = __builtin_bit_cast(half2_t, w[j]);
            ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        }
        // sign flip, widening to f32 and the first butterfly stage in one
        // v_dot2_f32_f16 per output: sigma_a a + sigma_b b and sigma_a a - sigma_b b
        float f[R];
#pragma unroll
        for (int j = 0; j < 4 * K; ++j) {
            f[2 * j] = dot2_sum(w[j], sg[j]);
            f[2 * j + 1] = dot2_diff(w[j], sg[j]);
        }
        ss += quad_move<kQuadXor1>(ss);
        ss += quad_move<kQuadXor2>(ss);
        const float nrm = __builtin_sqrtf(ss);
        // 8 eps / nrm: hardware reciprocal refined by one Newton step
        float rc = __builtin_amdgcn_rcpf(nrm);
        rc = __builtin_fmaf(rc, __builtin_fmaf(-nrm, rc, 1.0f), rc);
        const float kk = (nrm > 0.0f) ? eps8 * rc : 0.0f;

        fwht_quad<R>(f, ma, mb);
        fwht_registers_scaled<2>(f, kk);   // f[r] = 8 z of coordinate r

        uint32_t pk[NPK];   // the lane's field stream (4 and 2 bits)
        uint32_t G3[K];     // 3 bits: group k's 24-bit field, code j at bit 3j
#pragma unroll
        for (int i = 0; i < NPK; ++i) pk[i] = 0;
        if constexpr (BITS == 4) {
            uint32_t lo[K], hi[K];
            quantize4<0>(f, qtab, lo, hi);
#pragma unroll
            for (int g = 0; g < K; ++g) pk[g] = lo[g] | hi[g];
        } else if constexpr (BITS == 2) {
            uint32_t a[4][NPK];
            quantize2<0>(f, qtab, a);
#pragma unroll
            for (int m = 0; m < NPK; ++m)
                pk[m] = (a[3][m] << 6) | (a[2][m] << 4) | (a[1][m] << 2) | a[0][m];
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float y = f[r];
                const float2 e = qtab[(int)y + kCells];
                const uint32_t code = __builtin_bit_cast(uint32_t, e.y) + (y > e.x ? 1u : 0u);
                if ((r & 7) == 0) G3[r >> 3] = code;
                else G3[r >> 3] |= code << (3 * (r & 7));
            }
        }

        // the dwords this lane stores and their indices within the packed row
        constexpr int NS = (BITS == 2) ? K / 2 : K;
        uint32_t sv[NS];
        int si[NS];
        if constexpr (BITS == 4) {
            // group k of lane q is dword 4k + q
#pragma unroll
            for (int g = 0; g < K; ++g) {
                sv[g] = pk[g];
                si[g] = 4 * g + q;
            }
        } else if constexpr (BITS == 2) {
            // group k of lane q is half (q & 1) of dword 2k + (q >> 1); lanes
            // q and q^1 splice their halves (dword m of the stream holds
            // groups 2m, 2m + 1), each lane stores K / 2 dwords
            const int base = 2 * (q & 1) + (q >> 1);
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                const uint32_t p = quad_move<kQuadXor1>(pk[m]);
                sv[m] = __builtin_amdgcn_perm(p, pk[m], sel2);
                si[m] = base + 4 * m;
            }
        } else {
            // group k of lane q is the 24-bit field at bit 96k + 24q; lane q < 3
            // stores dword 3k + q, made of its field and lane q+1's
            const uint32_t (&G)[K] = G3;
            const uint32_t sh = 8 * q + 8;
#pragma unroll
            for (int g = 0; g < K; ++g) {
                const uint32_t nbv = quad_move<kQuadNext>(G[g]);
                sv[g] = __builtin_amdgcn_alignbit(nbv, G[g] << 8, sh);
                si[g] = 3 * g + q;   // stored only by lanes q < 3
            }
        }
        if (PAGED) {
            const int64_t row = slots[v];
            if (row < 0 || row >= num_slots) continue;   // uniform over the quad
            uint32_t *dst = packed + row * PW;
#pragma unroll
            for (int i = 0; i < NS; ++i)
                if (BITS != 3 || q < 3) dst[si[i]] = sv[i];
            if (q == 0) norms[row] = nrm;
        } else if constexpr (!kStage) {
            const __amdgpu_buffer_rsrc_t rp = span_rsrc(packed + v0 * PW, nb * (PW * 4u));
#pragma unroll
            for (int i = 0; i < NS; ++i)
                if (BITS != 3 || q < 3)
                    __builtin_amdgcn_raw_buffer_store_b32(sv[i], rp, qv * (PW * 4u) + 4u * si[i], 0, 0);
            if (q == 0)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, nrm),
                                                      span_rsrc(norms + v0, nb * 4u), qv * 4u, 0, 0);
        } else {
            // Whole rows per store instruction: the quad's dwords go through
            // its own LDS row (wave-local, so LDS order within the wave is
            // the only synchronisation needed), then lane q stores the
            // contiguous quarter q of the row.  A wave's store then covers
            // its 16 consecutive rows without gaps.
            uint32_t *srow = stage + (threadIdx.x >> 2) * kStageRow;
#pragma unroll
            for (int i = 0; i < NS; ++i)
                if (BITS != 3 || q < 3) srow[si[i]] = sv[i];
            wave_lds_sync();
            constexpr int QW = PW / 4;                  // dwords per lane
            uint32_t ov[QW];
#pragma unroll
            for (int i = 0; i < QW; ++i) ov[i] = srow[QW * q + i];
            wave_lds_sync();
            const __amdgpu_buffer_rsrc_t rp = span_rsrc(packed + v0 * PW, nb * (PW * 4u));
            const uint32_t off = qv * (PW * 4u) + 4u * QW * q;
            store_quarter<QW>(ov, rp, off);
            if (q == 0)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, nrm),
                                                      span_rsrc(norms + v0, nb * 4u), qv * 4u, 0, 0);
        }
    }
}

// Decode launch shape per (head_dim, bits), chosen by timing 1 or 2 vectors
// per quad, each with and without paired stores, on MI355X over a 4 GiB cache:
// - vectors per quad: all their loads are issued before the first one is
//   transformed; one at 4 bits from head_dim 128 up, two otherwise;
// - paired stores: neighbouring quads trade chunks so that every store
//   instruction writes whole 128-byte lines; 3-10% faster than per-quad
//   64-byte pieces in the write-heavy mix, except at head_dim 128 and 2 bits
//   (3% slower there).
constexpr int dec_vpq(int d, int bits) { return (bits == 4 && d >= 128) ? 1 : 2; }
constexpr bool dec_pair(int d, int bits) { return !(d == 128 && bits == 2); }

template <int D, int BITS>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint32_t *__restrict__ packed,
                                                          const float *__restrict__ norms,
                                                          int64_t n, u32x4 *__restrict__ out,
                                                          CodecConsts k) {
    constexpr int L = 1 << BITS;
    constexpr int K = D / 32;
    constexpr int R = 8 * K;
    constexpr int PW = D * BITS / 32;
    constexpr int VPQ = dec_vpq(D, BITS);
    // One lookup returns G already-transformed values: the first butterfly
    // stage (b = 3, 4: pairs of codes) or the first two (b = 2: a byte holds
    // four codes) is folded into the table.
    constexpr int G = (BITS == 2) ? 4 : 2;
    constexpr int NENT = 1 << (G * BITS);
    __shared__ float tab[NENT * G];
    for (int t = threadIdx.x; t < NENT; t += blockDim.x) {
        if (G == 2) {
            const float a = k.level[t & (L - 1)], b = k.level[(t >> BITS) & (L - 1)];
            tab[2 * t] = a + b;
            tab[2 * t + 1] = a - b;
        } else {
            const float c0 = k.level[t & 3], c1 = k.level[(t >> 2) & 3];
            const float c2 = k.level[(t >> 4) & 3], c3 = k.level[(t >> 6) & 3];
            const float a0 = c0 + c1, a1 = c0 - c1, a2 = c2 + c3, a3 = c2 - c3;
            tab[4 * t + 0] = a0 + a2;
            tab[4 * t + 1] = a1 + a3;
            tab[4 * t + 2] = a0 - a2;
            tab[4 * t + 3] = a1 - a3;
        }
    }
    __shared__ u32x4 smask[4 * K];
    if (threadIdx.x < 16 * K)
        store_sign_mask<K, false>(k, threadIdx.x, reinterpret_cast<uint32_t *>(smask));
    __syncthreads();

    const int q = threadIdx.x & 3;
    uint32_t xm[4 * K];
    load_sign_masks<K>(smask, q, xm);
    const float ma = (q & 1) ? -1.0f : 1.0f;
    const float mb = (q & 2) ? -1.0f : 1.0f;
    const float eps_d = (ma * mb) * (1.0f / D);
    const uint32_t sel2 = (q & 1) ? 0x07060302u : 0x05040100u;   // halves (q & 1) of two dwords
    const int w3a = (3 * q) >> 2;                                 // 3-bit: first dword of the field
    const int w3b = (w3a + 1 < 3) ? w3a + 1 : 2;
    const uint32_t s3 = (24u * q) & 31u;

    // VPQ vectors per quad, 64 apart, so that every access instruction of
    // a wave covers 16 consecutive vectors; all their loads are issued before
    // the first vector is transformed.
    constexpr int NW = (BITS == 3) ? 2 * K : K;   // packed dwords this lane reads per vector
    const int64_t vb = (int64_t)blockIdx.x * (kVecPerBlock * VPQ) + (threadIdx.x >> 2);
    uint32_t raw[VPQ][NW];
    float nrm[VPQ];
#pragma unroll
    for (int i = 0; i < VPQ; ++i) {
        const int64_t v = vb + (int64_t)i * kVecPerBlock;
        if (v >= n) break;   // uniform over the quad
        const uint32_t *src = packed + v * PW;
        nrm[i] = norms[v];
#pragma unroll
        for (int g = 0; g < K; ++g) {
            if constexpr (BITS == 4) {
                raw[i][g] = src[4 * g + q];
            } else if constexpr (BITS == 2) {
                raw[i][g] = src[2 * g + (q >> 1)];
            } else {
                raw[i][2 * g] = src[3 * g + w3a];
                raw[i][2 * g + 1] = src[3 * g + w3b];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < VPQ; ++i) {
        const int64_t v = vb + (int64_t)i * kVecPerBlock;
        if (v >= n) break;
        float f[R];
        if constexpr (BITS == 4) {
#pragma unroll
            for (int j = 0; j < 4 * K; ++j) {
                const uint32_t idx = (raw[i][j >> 2] >> (8 * (j & 3))) & 0xFFu;
                const float2 e = reinterpret_cast<const float2 *>(tab)[idx];
                f[2 * j] = e.x;
                f[2 * j + 1] = e.y;
            }
        } else if constexpr (BITS == 2) {
            // c[m]: this lane's halves of groups 2m and 2m + 1
            uint32_t c[K / 2];
#pragma unroll
            for (int m = 0; m < K / 2; ++m)
                c[m] = __builtin_amdgcn_perm(raw[i][2 * m + 1], raw[i][2 * m], sel2);
#pragma unroll
            for (int j = 0; j < 2 * K; ++j) {
                const uint32_t idx = (c[j >> 2] >> (8 * (j & 3))) & 0xFFu;
                const float4 e = reinterpret_cast<const float4 *>(tab)[idx];
                f[4 * j] = e.x;
                f[4 * j + 1] = e.y;
                f[4 * j + 2] = e.z;
                f[4 * j + 3] = e.w;
            }
        } else {
#pragma unroll
            for (int g = 0; g < K; ++g) {
                const uint32_t fld = __builtin_amdgcn_alignbit(raw[i][2 * g + 1], raw[i][2 * g], s3);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t idx = (fld >> (6 * p)) & 63u;
                    const float2 e = reinterpret_cast<const float2 *>(tab)[idx];
                    f[8 * g + 2 * p] = e.x;
                    f[8 * g + 2 * p + 1] = e.y;
                }
            }
        }
        fwht_quad<R>(f, ma, mb);
        fwht_registers_scaled<(BITS == 2) ? 4 : 2>(f, nrm[i] * eps_d);

        uint32_t o[4 * K];
#pragma unroll
        for (int j = 0; j < 4 * K; ++j) {
            half2_t h;
            h.x = (_Float16)f[2 * j];
            h.y = (_Float16)f[2 * j + 1];
            o[j] = __builtin_bit_cast(uint32_t, h) ^ xm[j];
        }
        // Paired stores: quads 2p and 2p + 1 of a wave hold consecutive
        // vectors a, a + 1.  When all 16 vectors of the wave exist, the two
        // quads trade one 16-byte chunk per 128-byte line, so that each store
        // instruction writes whole lines: line L of a vector is groups 2L
        // (lanes of the even quad) and 2L + 1 (odd quad).  The ragged last
        // wave keeps the per-quad pattern.
        const int64_t wave_first = vb - (threadIdx.x & 63) / 4 + (int64_t)i * kVecPerBlock;
        if (dec_pair(D, BITS) && __builtin_amdgcn_readfirstlane((int)(wave_first + 15 < n))) {
            const int odd = (threadIdx.x >> 2) & 1;
            u32x4 *dst = out + (v - odd) * (D / 8) + 4 * odd + q;
#pragma unroll
            for (int L = 0; L < K / 2; ++L) {
                uint32_t xv[4], yv[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t lo = o[8 * L + t], hi = o[8 * L + 4 + t];
                    // odd lanes take the even quad's group 2L + 1 (four lanes
                    // down: row_ror:4, banks 1 and 3); even lanes take the odd
                    // quad's group 2L (four lanes up: row_ror:12, banks 0 and 2)
                    xv[t] = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)hi, kRowRor4, 0xF, 0xA, false);
                    yv[t] = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)lo, kRowRor12, 0xF, 0x5, false);
                }
                dst[8 * L] = u32x4{xv[0], xv[1], xv[2], xv[3]};
                dst[8 * L + D / 8] = u32x4{yv[0], yv[1], yv[2], yv[3]};
            }
        } else {
            u32x4 *dst = out + v * (D / 8) + q;
#pragma unroll
            for (int g = 0; g < K; ++g) {
                const u32x4 val = {o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]};
                dst[4 * g] = val;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Hybrid modes tq35 / tq25 at head_dim 128 (aither-kvcache PyPI page, "Hybrid
// modes (tq35/tq25)": split-group quantization with a QJL residual; "API
// Reference": HybridTurboQuant, norms embedded in the packed bytes).
//
// A vector is taken in group order y = x[perm] (perm from calibration): the
// halves y[0..64) and y[64..128) are two TurboQuant vectors of dimension 64
// at (3, 2) bits (tq35) or (2, 1) bits (tq25); the residual r = y - yhat of
// their decode is sketched by the signs of H_128 D_Q r and its norm rho, and
// decode adds sqrt(pi/2)/128 * rho * D_Q H_128 s.  Row: codes A | codes B |
// 128 sign bits | f32 norm A, norm B, rho (68 or 52 bytes).
//
// Work mapping: one quad per vector; lane q holds group-order positions
// 32K + 8q + j in register 8K + j, i.e. the head_dim-128 layout, whose
// registers 0-15 are the head_dim-64 layout of group A and 16-31 that of
// group B.  So both 64-point transforms, the 128-point transform of the
// sketch, the codes and the sign bits all stay in registers; only the
// channel permutation goes through LDS (a gather on encode, a scatter on
// decode, through a staged row per quad).
// ---------------------------------------------------------------------------

// Staged binary16 rows of the hybrid kernels: 128 channels padded to 136
// (272 bytes), so that the 16 rows a wave touches start 16 bytes apart in
// the 64 LDS banks: the channel gather / scatter, where every quad reads or
// writes the same channel of its own row, then hits 16 different banks
// instead of one, and the 16-byte row accesses stay aligned.
constexpr int kHybridRowPad = 136;

template <int MODE>
struct HybridBits {
    static constexpr int A = (MODE == 35) ? 3 : 2;
    static constexpr int B = (MODE == 35) ? 2 : 1;
    static constexpr int PA = 64 * A / 32;                 // dwords of group-A codes
    static constexpr int PB = 64 * B / 32;                 // dwords of group-B codes
    static constexpr int RW = PA + PB + 4 + 3;             // dwords per row
};

// The same count from the positive half of a codebook symmetric about 0
// (thresholds thr[2^(B-1) + k] = -thr[2^(B-1) - 2 - k], thr[2^(B-1) - 1] = 0):
// 2^(B-1) + #(t < |y|) for y > 0, 2^(B-1) - 1 - #(t < |y|) otherwise, over
// the 2^(B-1) - 1 positive thresholds t.  It differs from count_below only
// where |y| equals a threshold exactly.
template <int B>
__device__ __forceinline__ uint32_t count_below_sym(float y, const float *thr) {
    constexpr int H = 1 << (B - 1);
    const float a = __builtin_fabsf(y);
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < H - 1; ++k) c += (thr[H + k] < a) ? 1u : 0u;
    return y > 0.0f ? H + c : H - 1 - c;
}

// code = number of the 2^B - 1 (scaled) thresholds strictly below y
template <int B>
__device__ __forceinline__ uint32_t count_below(float y, const float *thr) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < (1 << B) - 1; ++k) c += (thr[k] < y) ? 1u : 0u;
    return c;
}

// v with its sign bit XORed by bit 31 of m (the binary16 sign-pair masks hold
// the signs of registers 2i and 2i + 1 in bits 15 and 31 of word i)
__device__ __forceinline__ float flip(float v, uint32_t m) {
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) ^ m);
}

// First butterfly stage (stride 1) on register pairs.
template <int N>
__device__ __forceinline__ void stage1(float (&f)[N]) {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
        const float a = f[i], b = f[i + 1];
        f[i] = a + b;
        f[i + 1] = a - b;
    }
}

// Pack group codes of a half: N = 16 codes per lane (two runs of 8) at BITS
// bits; returns the dwords this lane stores and their indices within the
// group's section (count in *ns; lanes with nothing to store get 0).
template <int BITS>
__device__ __forceinline__ int pack_half(const uint32_t (&c)[16], int q, uint32_t (&sv)[2],
                                         int (&si)[2]) {
    if constexpr (BITS == 3) {
        // run K: 24-bit field at bit 96K + 24q; lane q < 3 stores dword 3K + q
        const uint32_t sh = 8 * q + 8;
#pragma unroll
        for (int K = 0; K < 2; ++K) {
            uint32_t G = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) G |= c[8 * K + j] << (3 * j);
            const uint32_t nbv = quad_move<kQuadNext>(G);
            sv[K] = __builtin_amdgcn_alignbit(nbv, G << 8, sh);
            si[K] = 3 * K + q;
        }
        return q < 3 ? 2 : 0;
    } else if constexpr (BITS == 2) {
        // run K: 16-bit field at bit 64K + 16q, i.e. half (q & 1) of dword
        // 2K + (q >> 1); lanes q and q ^ 1 splice their halves
        uint32_t pk = 0;
#pragma unroll
        for (int K = 0; K < 2; ++K)
#pragma unroll
            for (int j = 0; j < 8; ++j) pk |= c[8 * K + j] << (16 * K + 2 * j);
        const uint32_t sel2 = (q & 1) ? 0x03020706u : 0x05040100u;
        const uint32_t p = quad_move<kQuadXor1>(pk);
        sv[0] = __builtin_amdgcn_perm(p, pk, sel2);
        si[0] = 2 * (q & 1) + (q >> 1);
        return 1;
    } else {
        // run K: byte 4K + q (code j at bit j); the quad ORs its bytes
#pragma unroll
        for (int K = 0; K < 2; ++K) {
            uint32_t b = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) b |= c[8 * K + j] << j;
            uint32_t w = b << (8 * q);
            w |= quad_move<kQuadXor1>(w);
            w |= quad_move<kQuadXor2>(w);
            sv[K] = w;
            si[K] = K;
        }
        return q < 2 ? 1 : 0;   // lane q < 2 stores dword q (both lanes hold both)
    }
}

// The codes of lane q's 16 positions of a half from that half's section
// (row dwords `sec`), the inverse of pack_half.
template <int BITS>
__device__ __forceinline__ void unpack_half(const uint32_t *sec, int q, uint32_t (&c)[16]) {
    if constexpr (BITS == 3) {
        const int wa = (3 * q) >> 2;
        const int wb = (wa + 1 < 3) ? wa + 1 : 2;
        const uint32_t s3 = (24u * q) & 31u;
#pragma unroll
        for (int K = 0; K < 2; ++K) {
            const uint32_t fld = __builtin_amdgcn_alignbit(sec[3 * K + wb], sec[3 * K + wa], s3);
#pragma unroll
            for (int j = 0; j < 8; ++j) c[8 * K + j] = (fld >> (3 * j)) & 7u;
        }
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int K = 0; K < 2; ++K) {
            const uint32_t w = sec[2 * K + (q >> 1)] >> (16 * (q & 1));
#pragma unroll
            for (int j = 0; j < 8; ++j) c[8 * K + j] = (w >> (2 * j)) & 3u;
        }
    } else {
#pragma unroll
        for (int K = 0; K < 2; ++K) {
            const uint32_t b = sec[K] >> (8 * q);
#pragma unroll
            for (int j = 0; j < 8; ++j) c[8 * K + j] = (b >> j) & 1u;
        }
    }
}

// TurboQuant decode of a half in registers: levels -> n D H_64 c / 64, with
// the lane sign eps of the cross-lane stages folded into the scale.
__device__ __forceinline__ void half_decode(float (&f)[16], float scale, const uint32_t (&xm)[8]) {
    stage1(f);
    fwht_quad<16>(f, (threadIdx.x & 1) ? -1.0f : 1.0f, (threadIdx.x & 2) ? -1.0f : 1.0f);
    fwht_registers_scaled<2>(f, scale);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = flip(f[2 * i], (xm[i] << 16) & 0x80000000u);
        f[2 * i + 1] = flip(f[2 * i + 1], xm[i] & 0x80000000u);
    }
}

// IDENT: the channel permutation is the identity (the data-free split), so
// the group-order registers are the channel-order loads themselves and the
// LDS staging and gather (scatter on decode) are skipped.
template <int MODE, bool IDENT>
__global__ __launch_bounds__(kThreads) void hybrid_encode_kernel(const u32x4 *__restrict__ x,
                                                                 int64_t n,
                                                                 uint32_t *__restrict__ packed,
                                                                 HybridConsts k) {
    using HB = HybridBits<MODE>;
    constexpr int RW = HB::RW;
    __shared__ __attribute__((aligned(16))) uint16_t xs[kVecPerBlock][kHybridRowPad];
    __shared__ __attribute__((aligned(16))) uint32_t rows[kVecPerBlock * RW];
    __shared__ u32x4 gidx[8];
    __shared__ u32x4 smask[16], qmask[16];
    __shared__ float lev[12];
    if (threadIdx.x < 8) gidx[threadIdx.x] = u32x4{k.gidx[4 * threadIdx.x], k.gidx[4 * threadIdx.x + 1],
                                                   k.gidx[4 * threadIdx.x + 2], k.gidx[4 * threadIdx.x + 3]};
    if (threadIdx.x < 12) lev[threadIdx.x] = threadIdx.x < 8 ? k.lev_a[threadIdx.x] : k.lev_b[threadIdx.x - 8];
    if (threadIdx.x < 64)
        reinterpret_cast<uint32_t *>(smask)[threadIdx.x] = sign_mask_word<4, true>(k.sign, threadIdx.x);
    else if (threadIdx.x < 128)
        reinterpret_cast<uint32_t *>(qmask)[threadIdx.x - 64] = sign_mask_word<4, false>(k.qsign, threadIdx.x - 64);
    __syncthreads();

    const int q = threadIdx.x & 3;
    const uint32_t qi = threadIdx.x >> 2;
    const int64_t v0 = (int64_t)blockIdx.x * kVecPerBlock;
    const uint32_t nb = (uint32_t)((n - v0 < kVecPerBlock) ? n - v0 : kVecPerBlock);
    // Quads past the end stay (their loads read zeros and their rows are not
    // stored): every lane of a wave takes part in the wave's row stores.
    if (16 * (threadIdx.x >> 6) >= nb) return;   // the whole wave is past the end
    const __amdgpu_buffer_rsrc_t rx = span_rsrc(x + v0 * 16, nb * 256u);
    uint32_t w[16];   // binary16 pairs of positions (2i, 2i + 1) in group order
    if constexpr (IDENT) {
        // position 32 K + 8 q + j is channel 32 K + 8 q + j: w[4 K .. 4 K + 3]
        // are the 16 bytes at 64 K + 16 q of the lane's row
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x4 u = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, qi * 256u + 16u * q + 64u * g, 0, 0));
            w[4 * g] = u.x;
            w[4 * g + 1] = u.y;
            w[4 * g + 2] = u.z;
            w[4 * g + 3] = u.w;
        }
    } else {
        // the row, staged per quad for the channel gather
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x4 u = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, qi * 256u + 16u * q + 64u * g, 0, 0));
            *reinterpret_cast<u32x4 *>(&xs[qi][8 * q + 32 * g]) = u;
        }
        wave_lds_sync();
        const u32x4 ga = gidx[2 * q], gb = gidx[2 * q + 1];
        const uint32_t gw[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t ch0 = (gw[i >> 1] >> (16 * (i & 1))) & 0xFFu;
            const uint32_t ch1 = (gw[i >> 1] >> (16 * (i & 1) + 8)) & 0xFFu;
            w[i] = (uint32_t)xs[qi][ch0] | ((uint32_t)xs[qi][ch1] << 16);
        }
    }
    uint32_t sg[16], sq[16];
    load_sign_masks<4>(smask, q, sg);
    load_sign_masks<4>(qmask, q, sq);
    const float ma = (q & 1) ? -1.0f : 1.0f;
    const float mb = (q & 2) ? -1.0f : 1.0f;
    const float eps = ma * mb;

    // norms of the two halves
    float ssa = 0.0f, ssb = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const half2_t ha = __builtin_bit_cast(half2_t, w[i]);
        const half2_t hb = __builtin_bit_cast(half2_t, w[8 + i]);
        ssa = __builtin_amdgcn_fdot2(ha, ha, ssa, false);
        ssb = __builtin_amdgcn_fdot2(hb, hb, ssb, false);
    }
    ssa += quad_move<kQuadXor1>(ssa);
    ssa += quad_move<kQuadXor2>(ssa);
    ssb += quad_move<kQuadXor1>(ssb);
    ssb += quad_move<kQuadXor2>(ssb);
    const float na = __builtin_sqrtf(ssa), nbn = __builtin_sqrtf(ssb);

    // forward transforms of the halves: sign flip and stride-1 stage in one
    // dot2 per output, then the 64-point transform scaled to 8 z
    float fa[16], fb[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        fa[2 * i] = dot2_sum(w[i], sg[i]);
        fa[2 * i + 1] = dot2_diff(w[i], sg[i]);
        fb[2 * i] = dot2_sum(w[8 + i], sg[8 + i]);
        fb[2 * i + 1] = dot2_diff(w[8 + i], sg[8 + i]);
    }
    auto inv = [](float nv) {
        float rc = __builtin_amdgcn_rcpf(nv);
        rc = __builtin_fmaf(rc, __builtin_fmaf(-nv, rc, 1.0f), rc);
        return (nv > 0.0f) ? rc : 0.0f;
    };
    fwht_quad<16>(fa, ma, mb);
    fwht_registers_scaled<2>(fa, 8.0f * eps * inv(na));
    fwht_quad<16>(fb, ma, mb);
    fwht_registers_scaled<2>(fb, 8.0f * eps * inv(nbn));
    uint32_t ca[16], cb[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ca[r] = count_below_sym<HB::A>(fa[r], k.thr_a);
        cb[r] = count_below_sym<HB::B>(fb[r], k.thr_b);
    }
    // decode of the halves and the residual, in group order
    float ra[16], rb[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ra[r] = lev[ca[r]];
        rb[r] = lev[8 + cb[r]];
    }
    uint32_t xa[8], xb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        xa[i] = sg[i];
        xb[i] = sg[8 + i];
    }
    half_decode(ra, na * eps * (1.0f / 64), xa);
    half_decode(rb, nbn * eps * (1.0f / 64), xb);
    float t[32];
    float rr = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const half2_t ha = __builtin_bit_cast(half2_t, w[i]);
        const half2_t hb = __builtin_bit_cast(half2_t, w[8 + i]);
        t[2 * i] = (float)ha.x - ra[2 * i];
        t[2 * i + 1] = (float)ha.y - ra[2 * i + 1];
        t[16 + 2 * i] = (float)hb.x - rb[2 * i];
        t[16 + 2 * i + 1] = (float)hb.y - rb[2 * i + 1];
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) rr = __builtin_fmaf(t[r], t[r], rr);
    rr += quad_move<kQuadXor1>(rr);
    rr += quad_move<kQuadXor2>(rr);
    const float rho = __builtin_sqrtf(rr);
    // the sketch: signs of H_128 D_Q r (lane sign eps folded into the last stage)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        t[2 * i] = flip(t[2 * i], (sq[i] << 16) & 0x80000000u);
        t[2 * i + 1] = flip(t[2 * i + 1], sq[i] & 0x80000000u);
    }
    stage1(t);
    fwht_quad<32>(t, ma, mb);
    fwht_registers_scaled<2>(t, eps);

    // the row, assembled in LDS: codes A, codes B, sign bits, norms
    uint32_t *row = rows + qi * RW;
    {
        uint32_t sv[2];
        int si[2];
        int c = pack_half<HB::A>(ca, q, sv, si);
        for (int i = 0; i < c; ++i) row[si[i]] = sv[i];
        c = pack_half<HB::B>(cb, q, sv, si);
        if (HB::B == 1) {
            if (c) row[HB::PA + q] = sv[q];
        } else {
            for (int i = 0; i < c; ++i) row[HB::PA + si[i]] = sv[i];
        }
        // sign bits: byte 4K + q holds the signs of positions 32K + 8q + j
        uint32_t sb[4];
#pragma unroll
        for (int K = 0; K < 4; ++K) {
            uint32_t b = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) b |= (t[8 * K + j] < 0.0f ? 1u : 0u) << j;
            uint32_t wv = b << (8 * q);
            wv |= quad_move<kQuadXor1>(wv);
            wv |= quad_move<kQuadXor2>(wv);
            sb[K] = wv;
        }
        row[HB::PA + HB::PB + q] = sb[q];
        if (q < 3)
            row[HB::PA + HB::PB + 4 + q] = __builtin_bit_cast(uint32_t, q == 0 ? na : (q == 1 ? nbn : rho));
    }
    wave_lds_sync();
    // the wave's rows go out as one contiguous span of dwords
    // wave-uniform (readfirstlane): the buffer resources built from it stay scalar
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const uint32_t wrow0 = 16 * wave;                         // first row of the wave in the block
    const uint32_t wrows = (nb > wrow0) ? ((nb - wrow0 < 16) ? nb - wrow0 : 16) : 0;
    const __amdgpu_buffer_rsrc_t rp = span_rsrc(packed + (v0 + wrow0) * RW, wrows * RW * 4u);
#pragma unroll
    for (uint32_t i = lane; i < 16 * RW; i += 64)
        __builtin_amdgcn_raw_buffer_store_b32(rows[wrow0 * RW + i], rp, 4u * i, 0, 0);
}

template <int MODE, bool IDENT>
__global__ __launch_bounds__(kThreads) void hybrid_decode_kernel(const uint32_t *__restrict__ packed,
                                                                 int64_t n,
                                                                 u32x4 *__restrict__ out,
                                                                 HybridConsts k) {
    using HB = HybridBits<MODE>;
    constexpr int RW = HB::RW;
    __shared__ __attribute__((aligned(16))) uint16_t xs[kVecPerBlock][kHybridRowPad];
    __shared__ __attribute__((aligned(16))) uint32_t rows[kVecPerBlock * RW + 64];   // + a spare slot per lane
    __shared__ u32x4 gidx[8];
    __shared__ u32x4 smask[16], qmask[16];
    __shared__ float lev[12];
    // the kernel-argument words this thread puts into LDS, read first (their
    // wait then leaves the row loads in flight)
    u32x4 gv{};
    if (threadIdx.x < 8) gv = u32x4{k.gidx[4 * threadIdx.x], k.gidx[4 * threadIdx.x + 1],
                                    k.gidx[4 * threadIdx.x + 2], k.gidx[4 * threadIdx.x + 3]};
    const float lv = threadIdx.x < 8 ? k.lev_a[threadIdx.x] : (threadIdx.x < 12 ? k.lev_b[threadIdx.x - 8] : 0.0f);

    const int q = threadIdx.x & 3;
    const uint32_t qi = threadIdx.x >> 2;
    const int64_t v0 = (int64_t)blockIdx.x * kVecPerBlock;
    const uint32_t nb = (uint32_t)((n - v0 < kVecPerBlock) ? n - v0 : kVecPerBlock);
    // wave-uniform (readfirstlane): the buffer resources built from it stay scalar
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const uint32_t wrow0 = 16 * wave;
    const uint32_t wrows = (wrow0 >= nb) ? 0 : ((nb - wrow0 < 16) ? nb - wrow0 : 16);
    // the wave's rows, one contiguous span of dwords: every load is issued
    // before the tables are built and the barrier taken
    constexpr int NL = (16 * RW + 63) / 64;              // loads per lane
    uint32_t rv[NL];
    {
        const __amdgpu_buffer_rsrc_t rp = span_rsrc(packed + (v0 + wrow0) * RW, wrows * RW * 4u);
#pragma unroll
        for (int j = 0; j < NL; ++j)
            rv[j] = __builtin_amdgcn_raw_buffer_load_b32(rp, 4u * (lane + 64u * j), 0, 0);
    }
    if (threadIdx.x < 8) gidx[threadIdx.x] = gv;
    if (threadIdx.x < 12) lev[threadIdx.x] = lv;
    if (threadIdx.x < 64)
        reinterpret_cast<uint32_t *>(smask)[threadIdx.x] = sign_mask_word<4, false>(k.sign, threadIdx.x);
    else if (threadIdx.x < 128)
        reinterpret_cast<uint32_t *>(qmask)[threadIdx.x - 64] = sign_mask_word<4, false>(k.qsign, threadIdx.x - 64);
    __syncthreads();
    if (wrows == 0) return;    // the whole wave is past the end; no barrier follows
    // into LDS; lanes past the wave's 16 rows write their (zero) word to a
    // spare slot: an unconditional write keeps the last load with the others
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const uint32_t i = lane + 64u * j;
        rows[i < 16u * RW ? wrow0 * RW + i : kVecPerBlock * RW + lane] = rv[j];
    }
    wave_lds_sync();
    if (qi >= nb) return;      // uniform over the quad; only wave-local LDS follows
    const uint32_t *row = rows + qi * RW;
    uint32_t ca[16], cb[16];
    unpack_half<HB::A>(row, q, ca);
    unpack_half<HB::B>(row + HB::PA, q, cb);
    const uint32_t *sbits = row + HB::PA + HB::PB;
    const float na = __builtin_bit_cast(float, row[HB::PA + HB::PB + 4]);
    const float nbn = __builtin_bit_cast(float, row[HB::PA + HB::PB + 5]);
    const float rho = __builtin_bit_cast(float, row[HB::PA + HB::PB + 6]);
    uint32_t sg[16], sq[16];
    load_sign_masks<4>(smask, q, sg);
    load_sign_masks<4>(qmask, q, sq);
    const float eps = ((q & 1) ? -1.0f : 1.0f) * ((q & 2) ? -1.0f : 1.0f);

    float ra[16], rb[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ra[r] = lev[ca[r]];
        rb[r] = lev[8 + cb[r]];
    }
    uint32_t xa[8], xb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        xa[i] = sg[i];
        xb[i] = sg[8 + i];
    }
    half_decode(ra, na * eps * (1.0f / 64), xa);
    half_decode(rb, nbn * eps * (1.0f / 64), xb);
    // the sketch's correction sqrt(pi/2)/128 rho D_Q H_128 s
    float t[32];
#pragma unroll
    for (int K = 0; K < 4; ++K) {
        const uint32_t b = sbits[K] >> (8 * q);
#pragma unroll
        for (int j = 0; j < 8; ++j) t[8 * K + j] = ((b >> j) & 1u) ? -1.0f : 1.0f;
    }
    stage1(t);
    fwht_quad<32>(t, (q & 1) ? -1.0f : 1.0f, (q & 2) ? -1.0f : 1.0f);
    fwht_registers_scaled<2>(t, rho * eps * (1.2533141373155003f / 128));
    uint16_t hv[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float c0 = flip(t[2 * i], (sq[i] << 16) & 0x80000000u);
        const float c1 = flip(t[2 * i + 1], sq[i] & 0x80000000u);
        const float y0 = (i < 8 ? ra[2 * i] : rb[2 * i - 16]) + c0;
        const float y1 = (i < 8 ? ra[2 * i + 1] : rb[2 * i - 15]) + c1;
        hv[2 * i] = __builtin_bit_cast(uint16_t, (_Float16)y0);
        hv[2 * i + 1] = __builtin_bit_cast(uint16_t, (_Float16)y1);
    }
    u32x4 *dst = out + (v0 + qi) * 16 + q;
    if constexpr (IDENT) {
        // register 8 K + j is channel 32 K + 8 q + j: 16 bytes at 64 K + 16 q
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t d[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) d[m] = (uint32_t)hv[8 * g + 2 * m] | ((uint32_t)hv[8 * g + 2 * m + 1] << 16);
            dst[4 * g] = u32x4{d[0], d[1], d[2], d[3]};
        }
    } else {
        // back to channel order through the quad's staged row
        {
            const u32x4 ga = gidx[2 * q], gb = gidx[2 * q + 1];
            const uint32_t gw[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
            for (int r = 0; r < 32; ++r) xs[qi][(gw[r >> 2] >> (8 * (r & 3))) & 0xFFu] = hv[r];
        }
        wave_lds_sync();
#pragma unroll
        for (int g = 0; g < 4; ++g) dst[4 * g] = *reinterpret_cast<const u32x4 *>(&xs[qi][8 * q + 32 * g]);
    }
}

// One block per 64 enc_vpq(d) (encode) or 64 dec_vpq(d, bits) (decode)
// vectors: a full grid, so the hardware keeps every CU fed without a tail of
// long-running blocks (a grid-stride loop measured 10-30% slower).
dim3 grid_for(int64_t n, int vectors_per_block) {
    const int64_t b = (n + vectors_per_block - 1) / vectors_per_block;
    return dim3((unsigned)b);
}

}  // namespace

int device_cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}

hipError_t launch_encode(int head_dim, int bits, const void *x, int64_t n, const int64_t *slots,
                         int64_t num_slots, const CodecConsts &k, const EncTable &tb,
                         uint8_t *packed, float *norms, hipStream_t stream) {
    const int vpb = kVecPerBlock * enc_vpq(head_dim);
    if (n > (int64_t)vpb * 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid = grid_for(n, vpb), block(kThreads);
    const u32x4 *xs = static_cast<const u32x4 *>(x);
    uint32_t *pk = reinterpret_cast<uint32_t *>(packed);
#define TQ_ENC(D, B)                                                                            \
    if (slots)                                                                                  \
        hipLaunchKernelGGL((encode_kernel<D, B, true>), grid, block, 0, stream, xs, n, slots,   \
                           num_slots, pk, norms, k, tb);                                        \
    else                                                                                        \
        hipLaunchKernelGGL((encode_kernel<D, B, false>), grid, block, 0, stream, xs, n, slots,  \
                           num_slots, pk, norms, k, tb);
    switch (head_dim * 10 + bits) {
        case 642: TQ_ENC(64, 2) break;
        case 643: TQ_ENC(64, 3) break;
        case 644: TQ_ENC(64, 4) break;
        case 1282: TQ_ENC(128, 2) break;
        case 1283: TQ_ENC(128, 3) break;
        case 1284: TQ_ENC(128, 4) break;
        case 2562: TQ_ENC(256, 2) break;
        case 2563: TQ_ENC(256, 3) break;
        case 2564: TQ_ENC(256, 4) break;
        default: return hipErrorInvalidValue;
    }
#undef TQ_ENC
    return hipGetLastError();
}

hipError_t launch_decode(int head_dim, int bits, const uint8_t *packed, const float *norms,
                         int64_t n, const CodecConsts &k, void *out, hipStream_t stream) {
    const int vpb = kVecPerBlock * dec_vpq(head_dim, bits);
    if (n > (int64_t)vpb * 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid = grid_for(n, vpb), block(kThreads);
    u32x4 *o = static_cast<u32x4 *>(out);
    const uint32_t *pk = reinterpret_cast<const uint32_t *>(packed);
#define TQ_DEC(D, B) hipLaunchKernelGGL((decode_kernel<D, B>), grid, block, 0, stream, pk, norms, n, o, k)
    switch (head_dim * 10 + bits) {
        case 642: TQ_DEC(64, 2); break;
        case 643: TQ_DEC(64, 3); break;
        case 644: TQ_DEC(64, 4); break;
        case 1282: TQ_DEC(128, 2); break;
        case 1283: TQ_DEC(128, 3); break;
        case 1284: TQ_DEC(128, 4); break;
        case 2562: TQ_DEC(256, 2); break;
        case 2563: TQ_DEC(256, 3); break;
        case 2564: TQ_DEC(256, 4); break;
        default: return hipErrorInvalidValue;
    }
#undef TQ_DEC
    return hipGetLastError();
}

int hybrid_row_bytes(int mode) {
    return mode == 35 ? 4 * HybridBits<35>::RW : (mode == 25 ? 4 * HybridBits<25>::RW : 0);
}

// Whether the channel table is the identity (register r of lane q holds
// channel 32 (r / 8) + 8 q + r % 8).
bool hybrid_identity(const HybridConsts &k) {
    const uint8_t *g = reinterpret_cast<const uint8_t *>(k.gidx);
    for (int q = 0; q < 4; ++q)
        for (int r = 0; r < 32; ++r)
            if (g[32 * q + r] != 32 * (r / 8) + 8 * q + r % 8) return false;
    return true;
}

hipError_t launch_hybrid_encode(int mode, const void *x, int64_t n, const HybridConsts &k,
                                uint8_t *packed, hipStream_t stream) {
    if (n > (int64_t)kVecPerBlock * 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid = grid_for(n, kVecPerBlock), block(kThreads);
    const u32x4 *xs = static_cast<const u32x4 *>(x);
    uint32_t *pk = reinterpret_cast<uint32_t *>(packed);
    const bool id = hybrid_identity(k);
    if (mode == 35 && id) hipLaunchKernelGGL((hybrid_encode_kernel<35, true>), grid, block, 0, stream, xs, n, pk, k);
    else if (mode == 35) hipLaunchKernelGGL((hybrid_encode_kernel<35, false>), grid, block, 0, stream, xs, n, pk, k);
    else if (mode == 25 && id) hipLaunchKernelGGL((hybrid_encode_kernel<25, true>), grid, block, 0, stream, xs, n, pk, k);
    else if (mode == 25) hipLaunchKernelGGL((hybrid_encode_kernel<25, false>), grid, block, 0, stream, xs, n, pk, k);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_hybrid_decode(int mode, const uint8_t *packed, int64_t n,
                                const HybridConsts &k, void *out, hipStream_t stream) {
    if (n > (int64_t)kVecPerBlock * 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid = grid_for(n, kVecPerBlock), block(kThreads);
    const uint32_t *pk = reinterpret_cast<const uint32_t *>(packed);
    u32x4 *o = static_cast<u32x4 *>(out);
    const bool id = hybrid_identity(k);
    if (mode == 35 && id) hipLaunchKernelGGL((hybrid_decode_kernel<35, true>), grid, block, 0, stream, pk, n, o, k);
    else if (mode == 35) hipLaunchKernelGGL((hybrid_decode_kernel<35, false>), grid, block, 0, stream, pk, n, o, k);
    else if (mode == 25 && id) hipLaunchKernelGGL((hybrid_decode_kernel<25, true>), grid, block, 0, stream, pk, n, o, k);
    else if (mode == 25) hipLaunchKernelGGL((hybrid_decode_kernel<25, false>), grid, block, 0, stream, pk, n, o, k);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tq
