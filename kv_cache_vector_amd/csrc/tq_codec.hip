// TurboQuant encode / decode kernels for gfx950 (CDNA4, wave64).
//
// Method: aither-kvcache PyPI page, "Algorithm" (normalise, rotate by a fixed
// random orthogonal matrix, quantize each coordinate with a Lloyd-Max
// codebook, pack, store the f32 norm; decode reverses it).  The rotation is a
// seeded sign flip followed by a Walsh-Hadamard transform (qbc.network blog,
// "What TurboQuant is": a multiplier-free Walsh-Hadamard rotation).
//
// Work mapping.  Four lanes (a DPP quad) own one 128-dim vector.  Lane q of
// the quad owns coordinates 32k + 8q + j (k = 0..3, j = 0..7), held in
// register r = 8k + j.  Each fp16 access instruction therefore moves 64
// contiguous bytes per quad (16 B per lane), and a wave of 16 quads touches
// 16 whole 64-byte segments.  Coordinate bits 0-2 and 5-6 are register bits,
// bits 3-4 are the lane's place in the quad: the 128-point fast
// Walsh-Hadamard transform is 5 register butterfly stages plus 2 cross-lane
// stages done with DPP quad permutations -- no LDS traffic for the transform.
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
// y indexes a 193-entry LDS table whose cells are narrower than the smallest
// gap between two thresholds, so each cell holds at most one threshold:
// code = base[cell] + (y > thr[cell]).  A coordinate exactly on a threshold
// takes the lower code, as in the definition.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kCells = kEncCells;     // quantizer cells cover y in (-97, 97)
constexpr int kThreads = 256;         // 4 waves, 64 vectors per block iteration
constexpr int kVecPerBlock = kThreads / 4;
constexpr int kDecVpq = 4;            // decode: vectors per quad

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// DPP quad permutations
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]: partner q^1
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]: partner q^2
constexpr int kQuadNext = 0xF9;   // quad_perm [1,2,3,3]: lane q reads lane q+1

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
// One v_fmac_f32 with a DPP source per value.  The leading s_nop 1 provides
// the two wait states a DPP read of a VGPR needs after a VALU write; inside
// the block no instruction reads a register written by the one before it.
__device__ __forceinline__ void fwht_quad(float (&f)[32], float ma, float mb) {
#define TQ_STAGE(CTRL, M)                                                                        \
    asm volatile(                                                                                \
        "s_nop 1\n\t"                                                                            \
        "v_fmac_f32_dpp %0, %0, %32 " CTRL "\n\tv_fmac_f32_dpp %1, %1, %32 " CTRL "\n\t"         \
        "v_fmac_f32_dpp %2, %2, %32 " CTRL "\n\tv_fmac_f32_dpp %3, %3, %32 " CTRL "\n\t"         \
        "v_fmac_f32_dpp %4, %4, %32 " CTRL "\n\tv_fmac_f32_dpp %5, %5, %32 " CTRL "\n\t"         \
        "v_fmac_f32_dpp %6, %6, %32 " CTRL "\n\tv_fmac_f32_dpp %7, %7, %32 " CTRL "\n\t"         \
        "v_fmac_f32_dpp %8, %8, %32 " CTRL "\n\tv_fmac_f32_dpp %9, %9, %32 " CTRL "\n\t"         \
        "v_fmac_f32_dpp %10, %10, %32 " CTRL "\n\tv_fmac_f32_dpp %11, %11, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %12, %12, %32 " CTRL "\n\tv_fmac_f32_dpp %13, %13, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %14, %14, %32 " CTRL "\n\tv_fmac_f32_dpp %15, %15, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %16, %16, %32 " CTRL "\n\tv_fmac_f32_dpp %17, %17, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %18, %18, %32 " CTRL "\n\tv_fmac_f32_dpp %19, %19, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %20, %20, %32 " CTRL "\n\tv_fmac_f32_dpp %21, %21, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %22, %22, %32 " CTRL "\n\tv_fmac_f32_dpp %23, %23, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %24, %24, %32 " CTRL "\n\tv_fmac_f32_dpp %25, %25, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %26, %26, %32 " CTRL "\n\tv_fmac_f32_dpp %27, %27, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %28, %28, %32 " CTRL "\n\tv_fmac_f32_dpp %29, %29, %32 " CTRL "\n\t"     \
        "v_fmac_f32_dpp %30, %30, %32 " CTRL "\n\tv_fmac_f32_dpp %31, %31, %32 " CTRL            \
        : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]), "+v"(f[6]),   \
          "+v"(f[7]), "+v"(f[8]), "+v"(f[9]), "+v"(f[10]), "+v"(f[11]), "+v"(f[12]),            \
          "+v"(f[13]), "+v"(f[14]), "+v"(f[15]), "+v"(f[16]), "+v"(f[17]), "+v"(f[18]),         \
          "+v"(f[19]), "+v"(f[20]), "+v"(f[21]), "+v"(f[22]), "+v"(f[23]), "+v"(f[24]),         \
          "+v"(f[25]), "+v"(f[26]), "+v"(f[27]), "+v"(f[28]), "+v"(f[29]), "+v"(f[30]),         \
          "+v"(f[31])                                                                            \
        : "v"(M))
    TQ_STAGE("quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf", ma);
    TQ_STAGE("quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf", mb);
#undef TQ_STAGE
}

// Register butterfly stages with strides FIRST..8 (register bits), then the
// stride-16 stage fused with the per-vector scale s:
//   (a, b) -> ((a + b) s, (a - b) s) = (fma(a, s, b s), fma(a, s, -b s)).
template <int FIRST>
__device__ __forceinline__ void fwht_registers_scaled(float (&f)[32], float s) {
#pragma unroll
    for (int st = FIRST; st < 16; st <<= 1) {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            if (r & st) continue;
            const float a = f[r], b = f[r + st];
            f[r] = a + b;
            f[r + st] = a - b;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float a = f[r], bs = f[r + 16] * s;
        f[r] = __builtin_fmaf(a, s, bs);
        f[r + 16] = __builtin_fmaf(a, s, -bs);
    }
}

// Buffer resource over `bytes` bytes at `base` (wave-uniform).  Accesses
// through it take a scalar base and a 32-bit per-lane offset; reads outside
// the range return 0 and writes outside it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// XOR masks flipping the binary16 sign bits of register pair (2i, 2i+1) of
// lane q, i.e. of coordinates 32(i/4) + 8q + 2(i%4) + {0, 1}.  Thread t < 64
// writes mask i = t % 16 of lane q = t / 16 to LDS once per block; every lane
// then reads its 16 masks with four broadcast 16-byte LDS reads.
__device__ __forceinline__ void store_sign_mask(const CodecConsts &k, int t, uint32_t *smask) {
    const int q = t >> 4, i = t & 15;
    const uint32_t w = k.sign[i >> 2] >> (8 * q + 2 * (i & 3));
    smask[t] = ((w & 1u) << 15) | (((w >> 1) & 1u) << 31);
}

__device__ __forceinline__ void load_sign_masks(const u32x4 *smask, int q, uint32_t (&xm)[16]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const u32x4 u = smask[4 * q + m];
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
#undef TQ_PUT_CODE
#undef TQ_PUT_FIRST

template <int R>
__device__ __forceinline__ void quantize4(const float (&f)[32], const float2 *qtab,
                                          uint32_t (&lo)[4], uint32_t (&hi)[4]) {
    if constexpr (R < 32) {
        const float y = f[R];
        const float2 e = qtab[(int)y + kCells];
        const uint32_t W = __builtin_bit_cast(uint32_t, e.y);
        if (R & 1) put_code4<R>(hi[R >> 3], y, e.x, W);
        else put_code4<R>(lo[R >> 3], y, e.x, W);
        quantize4<R + 1>(f, qtab, lo, hi);
    }
}

template <int BITS, bool PAGED>
__global__ __launch_bounds__(kThreads) void encode_kernel(const u32x4 *__restrict__ x, int64_t n,
                                                          const int64_t *__restrict__ slots,
                                                          int64_t num_slots,
                                                          uint32_t *__restrict__ packed,
                                                          float *__restrict__ norms,
                                                          CodecConsts k, EncTable tb) {
    constexpr int PW = kHeadDim * BITS / 32;    // packed dwords per vector
    __shared__ float2 qtab[2 * kCells + 1];
    __shared__ u32x4 smask[16];
    for (int t = threadIdx.x; t < 2 * kCells + 1; t += blockDim.x) qtab[t] = tb.cell[t];
    if (threadIdx.x < 64) store_sign_mask(k, threadIdx.x, reinterpret_cast<uint32_t *>(smask));
    __syncthreads();

    const int q = threadIdx.x & 3;
    uint32_t xm[16];
    load_sign_masks(smask, q, xm);
    const float ma = (q & 1) ? -1.0f : 1.0f;
    const float mb = (q & 2) ? -1.0f : 1.0f;
    const float eps8 = 8.0f * ma * mb;
    const float one = k.one;
    // 2-bit: byte selectors splicing this lane's and the partner's 16-bit fields
    const uint32_t sel2 = (q & 1) ? 0x03020706u : 0x05040100u;

    {
        // this block's vectors [v0, v0 + nb): scalar base, per-lane offsets
        const int64_t v0 = (int64_t)blockIdx.x * kVecPerBlock;
        const uint32_t nb = (uint32_t)((n - v0 < kVecPerBlock) ? n - v0 : kVecPerBlock);
        const uint32_t qi = threadIdx.x >> 2;
        const int64_t v = v0 + qi;
        if (v >= n) return;   // uniform over the quad; no barrier follows
        const __amdgpu_buffer_rsrc_t rx = span_rsrc(x + v0 * 16, nb * 256u);
        const uint32_t xo = qi * 256u + 16u * q;
        uint32_t w[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x4 u = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 64u * g, 0, 0));
            w[4 * g + 0] = u.x;
            w[4 * g + 1] = u.y;
            w[4 * g + 2] = u.z;
            w[4 * g + 3] = u.w;
        }
        // ||x||^2 from the fp16 pairs (products exact in f32, f32 accumulate)
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const half2_t h = __builtin_bit_cast(half2_t, w[j]);
            ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        }
        // sign flip on the fp16 bits; widening to f32 fused with the first
        // butterfly stage (v_fma_mix: the multiplier `one` is a kernel
        // argument, so the compiler cannot fold these into plain adds)
        float f[32];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const half2_t h = __builtin_bit_cast(half2_t, w[j] ^ xm[j]);
            const float lo = (float)h.x, hi = (float)h.y;
            f[2 * j] = __builtin_fmaf(hi, one, lo);
            f[2 * j + 1] = __builtin_fmaf(hi, -one, lo);
        }
        ss += quad_move<kQuadXor1>(ss);
        ss += quad_move<kQuadXor2>(ss);
        const float nrm = __builtin_sqrtf(ss);
        // 8 eps / nrm: hardware reciprocal refined by one Newton step
        float rc = __builtin_amdgcn_rcpf(nrm);
        rc = __builtin_fmaf(rc, __builtin_fmaf(-nrm, rc, 1.0f), rc);
        const float kk = (nrm > 0.0f) ? eps8 * rc : 0.0f;

        fwht_quad(f, ma, mb);
        fwht_registers_scaled<2>(f, kk);   // f[r] = 8 z of coordinate r

        uint32_t pk[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) pk[i] = 0;
        if (BITS == 4) {
            uint32_t lo[4], hi[4];
            quantize4<0>(f, qtab, lo, hi);
#pragma unroll
            for (int g = 0; g < 4; ++g) pk[g % BITS] = lo[g] | hi[g];
        } else {
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                const float y = f[r];
                const float2 e = qtab[(int)y + kCells];
                const uint32_t code = __builtin_bit_cast(uint32_t, e.y) + (y > e.x ? 1u : 0u);
                const int bit = r * BITS;   // lane-local field stream: group k at bits 8*BITS*k
                pk[bit >> 5] |= code << (bit & 31);
                if ((bit & 31) + BITS > 32) pk[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
            }
        }

        // the dwords this lane stores and their indices within the packed row
        uint32_t sv[4];
        int si[4];
        int ns = 0;
        if (BITS == 4) {
            // group k of lane q is dword 4k + q
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                sv[g] = pk[g % BITS];
                si[g] = 4 * g + q;
            }
            ns = 4;
        } else if (BITS == 2) {
            // group k of lane q is half (q & 1) of dword 2k + (q >> 1); lanes
            // q and q^1 splice their halves, each lane stores two dwords
            const uint32_t p0 = quad_move<kQuadXor1>(pk[0]);
            const uint32_t p1 = quad_move<kQuadXor1>(pk[1 % BITS]);
            const int base = 2 * (q & 1) + (q >> 1);
            sv[0] = __builtin_amdgcn_perm(p0, pk[0], sel2);
            si[0] = base;
            sv[1] = __builtin_amdgcn_perm(p1, pk[1 % BITS], sel2);
            si[1] = base + 4;
            ns = 2;
        } else {
            // group k of lane q is the 24-bit field at bit 96k + 24q; lane q < 3
            // stores dword 3k + q, made of its field and lane q+1's
            uint32_t G[4];
            G[0] = pk[0] & 0xFFFFFFu;
            G[1] = __builtin_amdgcn_alignbit(pk[1 % BITS], pk[0], 24) & 0xFFFFFFu;
            G[2] = __builtin_amdgcn_alignbit(pk[2 % BITS], pk[1 % BITS], 16) & 0xFFFFFFu;
            G[3] = pk[2 % BITS] >> 8;
            const uint32_t sh = 8 * q + 8;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t nbv = quad_move<kQuadNext>(G[g]);
                sv[g] = __builtin_amdgcn_alignbit(nbv, G[g] << 8, sh);
                si[g] = 3 * g + q;   // stored only by lanes q < 3
            }
            ns = 4;
        }
        if (PAGED) {
            const int64_t row = slots[v];
            if (row < 0 || row >= num_slots) return;     // uniform over the quad
            uint32_t *dst = packed + row * PW;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < ns && (BITS != 3 || q < 3)) dst[si[i]] = sv[i];
            if (q == 0) norms[row] = nrm;
        } else {
            const __amdgpu_buffer_rsrc_t rp = span_rsrc(packed + v0 * PW, nb * (PW * 4u));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < ns && (BITS != 3 || q < 3))
                    __builtin_amdgcn_raw_buffer_store_b32(sv[i], rp, qi * (PW * 4u) + 4u * si[i], 0, 0);
            if (q == 0)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, nrm),
                                                      span_rsrc(norms + v0, nb * 4u), qi * 4u, 0, 0);
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint32_t *__restrict__ packed,
                                                          const float *__restrict__ norms,
                                                          int64_t n, u32x4 *__restrict__ out,
                                                          CodecConsts k) {
    constexpr int L = 1 << BITS;
    constexpr int PW = kHeadDim * BITS / 32;
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
    __shared__ u32x4 smask[16];
    if (threadIdx.x < 64) store_sign_mask(k, threadIdx.x, reinterpret_cast<uint32_t *>(smask));
    __syncthreads();

    const int q = threadIdx.x & 3;
    uint32_t xm[16];
    load_sign_masks(smask, q, xm);
    const float ma = (q & 1) ? -1.0f : 1.0f;
    const float mb = (q & 2) ? -1.0f : 1.0f;
    const float eps_d = (ma * mb) * (1.0f / kHeadDim);
    const uint32_t sel2 = (q & 1) ? 0x07060302u : 0x05040100u;   // halves (q & 1) of two dwords
    const int w3a = (3 * q) >> 2;                                 // 3-bit: first dword of the field
    const int w3b = (w3a + 1 < 3) ? w3a + 1 : 2;
    const uint32_t s3 = (24u * q) & 31u;

    // kDecVpq vectors per quad, 64 apart, so that every access instruction of
    // a wave covers 16 consecutive vectors; all their loads are issued before
    // the first vector is transformed.
    constexpr int NW = (BITS == 3) ? 8 : 4;   // packed dwords this lane reads per vector
    const int64_t vb = (int64_t)blockIdx.x * (kVecPerBlock * kDecVpq) + (threadIdx.x >> 2);
    uint32_t raw[kDecVpq][NW];
    float nrm[kDecVpq];
#pragma unroll
    for (int i = 0; i < kDecVpq; ++i) {
        const int64_t v = vb + (int64_t)i * kVecPerBlock;
        if (v >= n) break;   // uniform over the quad
        const uint32_t *src = packed + v * PW;
        nrm[i] = norms[v];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (BITS == 4) {
                raw[i][g] = src[4 * g + q];
            } else if (BITS == 2) {
                raw[i][g] = src[2 * g + (q >> 1)];
            } else {
                raw[i][2 * g] = src[3 * g + w3a];
                raw[i][2 * g + 1 % NW] = src[3 * g + w3b];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kDecVpq; ++i) {
        const int64_t v = vb + (int64_t)i * kVecPerBlock;
        if (v >= n) break;
        float f[32];
        if (BITS == 4) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t idx = (raw[i][j >> 2] >> (8 * (j & 3))) & 0xFFu;
                const float2 e = reinterpret_cast<const float2 *>(tab)[idx];
                f[2 * j] = e.x;
                f[2 * j + 1] = e.y;
            }
        } else if (BITS == 2) {
            const uint32_t c0 = __builtin_amdgcn_perm(raw[i][1], raw[i][0], sel2);   // groups 0, 1
            const uint32_t c1 = __builtin_amdgcn_perm(raw[i][3], raw[i][2], sel2);   // groups 2, 3
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t idx = ((j < 4 ? c0 : c1) >> (8 * (j & 3))) & 0xFFu;
                const float4 e = reinterpret_cast<const float4 *>(tab)[idx];
                f[4 * j] = e.x;
                f[4 * j + 1] = e.y;
                f[4 * j + 2] = e.z;
                f[4 * j + 3] = e.w;
            }
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t fld =
                    __builtin_amdgcn_alignbit(raw[i][(2 * g + 1) % NW], raw[i][2 * g], s3);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t idx = (fld >> (6 * p)) & 63u;
                    const float2 e = reinterpret_cast<const float2 *>(tab)[idx];
                    f[8 * g + 2 * p] = e.x;
                    f[8 * g + 2 * p + 1] = e.y;
                }
            }
        }
        fwht_quad(f, ma, mb);
        fwht_registers_scaled<(BITS == 2) ? 4 : 2>(f, nrm[i] * eps_d);

        uint32_t o[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            half2_t h;
            h.x = (_Float16)f[2 * j];
            h.y = (_Float16)f[2 * j + 1];
            o[j] = __builtin_bit_cast(uint32_t, h) ^ xm[j];
        }
        u32x4 *dst = out + v * 16 + q;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x4 val = {o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]};
            dst[4 * g] = val;
        }
    }
}

// One block per 64 (encode) or 64 * kDecVpq (decode) vectors: a full grid, so
// the hardware keeps every CU fed without a tail of long-running blocks.
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

hipError_t launch_encode(int bits, const void *x, int64_t n, const int64_t *slots,
                         int64_t num_slots, const CodecConsts &k, const EncTable &tb,
                         uint8_t *packed, float *norms, hipStream_t stream) {
    if (n > (int64_t)kVecPerBlock * 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid = grid_for(n, kVecPerBlock), block(kThreads);
    const u32x4 *xs = static_cast<const u32x4 *>(x);
    uint32_t *pk = reinterpret_cast<uint32_t *>(packed);
#define TQ_ENC(B)                                                                               \
    if (slots)                                                                                  \
        hipLaunchKernelGGL((encode_kernel<B, true>), grid, block, 0, stream, xs, n, slots,      \
                           num_slots, pk, norms, k, tb);                                        \
    else                                                                                        \
        hipLaunchKernelGGL((encode_kernel<B, false>), grid, block, 0, stream, xs, n, slots,     \
                           num_slots, pk, norms, k, tb);
    switch (bits) {
        case 2: TQ_ENC(2) break;
        case 3: TQ_ENC(3) break;
        case 4: TQ_ENC(4) break;
        default: return hipErrorInvalidValue;
    }
#undef TQ_ENC
    return hipGetLastError();
}

hipError_t launch_decode(int bits, const uint8_t *packed, const float *norms, int64_t n,
                         const CodecConsts &k, void *out, hipStream_t stream) {
    if (n > (int64_t)kVecPerBlock * kDecVpq * 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid = grid_for(n, kVecPerBlock * kDecVpq), block(kThreads);
    u32x4 *o = static_cast<u32x4 *>(out);
    const uint32_t *pk = reinterpret_cast<const uint32_t *>(packed);
    switch (bits) {
        case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, pk, norms, n, o, k); break;
        case 3: hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, stream, pk, norms, n, o, k); break;
        case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, stream, pk, norms, n, o, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
