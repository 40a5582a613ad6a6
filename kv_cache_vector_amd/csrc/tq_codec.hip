// TurboQuant encode / decode kernels for gfx950 (CDNA4, wave64).
//
// Method: aither-kvcache PyPI page, "Algorithm" (normalise, rotate by a fixed
// random orthogonal matrix, quantize each coordinate with a Lloyd-Max
// codebook, pack, store the f32 norm; decode reverses it).  The rotation is a
// seeded sign flip followed by a Walsh-Hadamard transform (qbc.network blog,
// "What TurboQuant is": a multiplier-free Walsh-Hadamard rotation).
//
// Work mapping.  Four lanes (a DPP quad) own one 128-dim vector; lane q of the
// quad owns coordinates [32q, 32q + 32), i.e. 64 contiguous bytes of fp16
// input, 4*bits contiguous bytes of packed output.  Coordinate index bits 0..4
// live in registers, bits 5..6 in the lane's position in the quad, so the
// 128-point fast Walsh-Hadamard transform is 5 register butterfly stages and
// 2 DPP quad-permute stages -- no LDS traffic for the transform.  A wave
// handles 16 vectors per iteration; every global access of a quad is a
// contiguous run (64 B per fp16 load instruction, 64/48/32 B of codes).
//
// Cross-lane stages use one fused multiply-add per value: v += partner * m,
// with m = +1 on the lower lane and -1 on the upper one.  The upper lane thus
// holds the negated difference; the sign is tracked per lane (eps) and folded
// into the per-vector scale, which is multiplied in anyway.
//
// Quantizer.  y = 8 * z is formed as w * (8 * eps / ||x||).  The integer part
// of y indexes a 193-entry LDS table whose cells are narrower than the
// smallest gap between two thresholds, so each cell holds at most one
// threshold: code = base[cell] + (y > thr[cell]).  A coordinate exactly on a
// threshold takes the lower code, as in the definition.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kCells = 96;            // quantizer cells cover y in (-97, 97)
constexpr int kThreads = 256;         // 4 waves, 64 vectors per block iteration
constexpr int kVecPerBlock = kThreads / 4;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// DPP quad permutations: partner lane q^1 and q^2.
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t sign_word(const CodecConsts &k, int q) {
    return q == 0 ? k.sign[0] : q == 1 ? k.sign[1] : q == 2 ? k.sign[2] : k.sign[3];
}

// XOR masks that flip the binary16 sign bits of the coordinate pairs
// (2j, 2j+1) owned by this lane, for j = 0..15.
__device__ __forceinline__ void pair_sign_masks(uint32_t sw, uint32_t (&xm)[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
        xm[j] = (((sw >> (2 * j)) & 1u) << 15) | (((sw >> (2 * j + 1)) & 1u) << 31);
}

// In-register butterfly stages on coordinate bits [first, 5).
template <int FIRST_STRIDE>
__device__ __forceinline__ void fwht_registers(float (&f)[32]) {
#pragma unroll
    for (int s = FIRST_STRIDE; s < 32; s <<= 1) {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            if (r & s) continue;
            const float a = f[r], b = f[r + s];
            f[r] = a + b;
            f[r + s] = a - b;
        }
    }
}

// The two cross-lane stages (coordinate bits 5 and 6).  Afterwards the lane
// holds eps * (true value), eps = m5 * m6.
__device__ __forceinline__ void fwht_quad(float (&f)[32], float m5, float m6) {
#pragma unroll
    for (int r = 0; r < 32; ++r) f[r] = __builtin_fmaf(quad_swap<kQuadXor1>(f[r]), m5, f[r]);
#pragma unroll
    for (int r = 0; r < 32; ++r) f[r] = __builtin_fmaf(quad_swap<kQuadXor2>(f[r]), m6, f[r]);
}

template <int BITS, bool PAGED>
__global__ __launch_bounds__(kThreads) void encode_kernel(const u32x4 *__restrict__ x, int64_t n,
                                                          const int64_t *__restrict__ slots,
                                                          int64_t num_slots,
                                                          uint8_t *__restrict__ packed,
                                                          float *__restrict__ norms,
                                                          CodecConsts k) {
    constexpr int L = 1 << BITS;
    constexpr int P = kHeadDim * BITS / 8;      // packed bytes per vector
    constexpr int LANE_BYTES = 4 * BITS;        // packed bytes per lane
    __shared__ float2 qtab[2 * kCells + 1];

    // Cell i: i > 0 -> [i, i+1), i < 0 -> (i-1, i], i = 0 -> (-1, 1): the
    // values whose conversion to int (toward zero) gives i.
    for (int t = threadIdx.x; t < 2 * kCells + 1; t += blockDim.x) {
        const int i = t - kCells;
        const float lo = (i > 0) ? float(i) : float(i - 1);
        const float hi = (i < 0) ? float(i) : float(i + 1);
        uint32_t base = 0;
        float thr = __builtin_inff();
#pragma unroll
        for (int j = 0; j < L - 1; ++j) {
            const float T = k.thr8[j];
            if (T < lo) ++base;
            else if (T <= hi) thr = T;
        }
        qtab[t] = make_float2(thr, __builtin_bit_cast(float, base));
    }
    __syncthreads();

    const int lq = threadIdx.x & 3;
    uint32_t xm[16];
    pair_sign_masks(sign_word(k, lq), xm);
    const float m5 = (lq & 1) ? -1.0f : 1.0f;
    const float m6 = (lq & 2) ? -1.0f : 1.0f;
    const float eps = m5 * m6;

    const int64_t stride = (int64_t)gridDim.x * kVecPerBlock;
    for (int64_t v = (int64_t)blockIdx.x * kVecPerBlock + (threadIdx.x >> 2); v < n; v += stride) {
        const u32x4 *src = x + v * 16 + lq * 4;
        uint32_t w[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const u32x4 u = __builtin_nontemporal_load(src + m);
            w[4 * m + 0] = u.x;
            w[4 * m + 1] = u.y;
            w[4 * m + 2] = u.z;
            w[4 * m + 3] = u.w;
        }
        // ||x||^2 from the fp16 pairs (products exact in f32, f32 accumulate)
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const half2_t h = __builtin_bit_cast(half2_t, w[j]);
            ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        }
        // sign flip on the fp16 bits, then the first butterfly stage while
        // widening to f32
        float f[32];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const half2_t h = __builtin_bit_cast(half2_t, w[j] ^ xm[j]);
            const float lo = (float)h.x, hi = (float)h.y;
            f[2 * j] = lo + hi;
            f[2 * j + 1] = lo - hi;
        }
        fwht_registers<2>(f);
        fwht_quad(f, m5, m6);

        ss += quad_swap<kQuadXor1>(ss);
        ss += quad_swap<kQuadXor2>(ss);
        const float nrm = __builtin_sqrtf(ss);
        const float kk = (nrm > 0.0f) ? (8.0f * eps) / nrm : 0.0f;

        uint32_t pk[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) pk[i] = 0;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const float y = f[r] * kk;
            const float2 e = qtab[(int)y + kCells];
            const uint32_t code = __builtin_bit_cast(uint32_t, e.y) + (y > e.x ? 1u : 0u);
            const int bit = r * BITS;
            pk[bit >> 5] |= code << (bit & 31);
            if ((bit & 31) + BITS > 32) pk[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
        }

        int64_t row = v;
        if (PAGED) {
            row = slots[v];
            if (row < 0 || row >= num_slots) continue;   // uniform over the quad
        }
        uint8_t *dst = packed + row * P + lq * LANE_BYTES;
        if (BITS == 4) {
            const u32x4 val = {pk[0], pk[1], pk[2], pk[3 % BITS]};
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(dst));
        } else if (BITS == 2) {
            const u32x2 val = {pk[0], pk[1 % BITS]};
            __builtin_nontemporal_store(val, reinterpret_cast<u32x2 *>(dst));
        } else {
            uint32_t *d32 = reinterpret_cast<uint32_t *>(dst);
#pragma unroll
            for (int i = 0; i < BITS; ++i) __builtin_nontemporal_store(pk[i], d32 + i);
        }
        if (lq == 0) norms[row] = nrm;
    }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint8_t *__restrict__ packed,
                                                          const float *__restrict__ norms,
                                                          int64_t n, u32x4 *__restrict__ out,
                                                          CodecConsts k) {
    constexpr int L = 1 << BITS;
    constexpr int P = kHeadDim * BITS / 8;
    constexpr int LANE_BYTES = 4 * BITS;
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
    __syncthreads();

    const int lq = threadIdx.x & 3;
    uint32_t xm[16];
    pair_sign_masks(sign_word(k, lq), xm);
    const float m5 = (lq & 1) ? -1.0f : 1.0f;
    const float m6 = (lq & 2) ? -1.0f : 1.0f;
    const float eps_d = (m5 * m6) * (1.0f / kHeadDim);

    const int64_t stride = (int64_t)gridDim.x * kVecPerBlock;
    for (int64_t v = (int64_t)blockIdx.x * kVecPerBlock + (threadIdx.x >> 2); v < n; v += stride) {
        const uint8_t *src = packed + v * P + lq * LANE_BYTES;
        uint32_t c[BITS];
        if (BITS == 4) {
            const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
            c[0] = u.x; c[1] = u.y; c[2] = u.z; c[3 % BITS] = u.w;
        } else if (BITS == 2) {
            const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(src));
            c[0] = u.x; c[1 % BITS] = u.y;
        } else {
#pragma unroll
            for (int i = 0; i < BITS; ++i)
                c[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(src) + i);
        }
        const float nrm = norms[v];

        float f[32];
        if (BITS == 4) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t idx = (c[j >> 2] >> (8 * (j & 3))) & 0xFFu;
                const float2 e = reinterpret_cast<const float2 *>(tab)[idx];
                f[2 * j] = e.x;
                f[2 * j + 1] = e.y;
            }
            fwht_registers<2>(f);
        } else if (BITS == 2) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t idx = (c[j >> 2] >> (8 * (j & 3))) & 0xFFu;
                const float4 e = reinterpret_cast<const float4 *>(tab)[idx];
                f[4 * j] = e.x;
                f[4 * j + 1] = e.y;
                f[4 * j + 2] = e.z;
                f[4 * j + 3] = e.w;
            }
            fwht_registers<4>(f);
        } else {
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const int bit = 6 * g;
                uint32_t idx;
                if ((bit & 31) + 6 <= 32)
                    idx = (c[bit >> 5] >> (bit & 31)) & 63u;
                else
                    idx = __builtin_amdgcn_alignbit(c[(bit >> 5) + 1], c[bit >> 5], bit & 31) & 63u;
                const float2 e = reinterpret_cast<const float2 *>(tab)[idx];
                f[2 * g] = e.x;
                f[2 * g + 1] = e.y;
            }
            fwht_registers<2>(f);
        }
        fwht_quad(f, m5, m6);

        const float sc = nrm * eps_d;
        uint32_t o[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            half2_t h;
            h.x = (_Float16)(f[2 * j] * sc);
            h.y = (_Float16)(f[2 * j + 1] * sc);
            o[j] = __builtin_bit_cast(uint32_t, h) ^ xm[j];
        }
        u32x4 *dst = out + v * 16 + lq * 4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const u32x4 val = {o[4 * m], o[4 * m + 1], o[4 * m + 2], o[4 * m + 3]};
            __builtin_nontemporal_store(val, dst + m);
        }
    }
}

int grid_for(int64_t n) {
    const int64_t need = (n + kVecPerBlock - 1) / kVecPerBlock;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    return (int)(need < cap ? need : cap);
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
                         int64_t num_slots, const CodecConsts &k, uint8_t *packed, float *norms,
                         hipStream_t stream) {
    const dim3 grid(grid_for(n)), block(kThreads);
    const u32x4 *xs = static_cast<const u32x4 *>(x);
#define TQ_ENC(B)                                                                               \
    if (slots)                                                                                  \
        hipLaunchKernelGGL((encode_kernel<B, true>), grid, block, 0, stream, xs, n, slots,      \
                           num_slots, packed, norms, k);                                        \
    else                                                                                        \
        hipLaunchKernelGGL((encode_kernel<B, false>), grid, block, 0, stream, xs, n, slots,     \
                           num_slots, packed, norms, k);
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
    const dim3 grid(grid_for(n)), block(kThreads);
    u32x4 *o = static_cast<u32x4 *>(out);
    switch (bits) {
        case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, packed, norms, n, o, k); break;
        case 3: hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, stream, packed, norms, n, o, k); break;
        case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, stream, packed, norms, n, o, k); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
