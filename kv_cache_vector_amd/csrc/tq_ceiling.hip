// Streaming ceilings for the codec's byte mix on gfx950: kernels with no codec
// arithmetic that move exactly the bytes encode and decode move, in the same
// grid (one 256-thread block per 64 vectors, full grid), each wave's accesses
// contiguous, so that the codec kernels can be rated against what this byte
// mix achieves on the same chip.  Measurement support only; not part of the
// codec.
//
//   encode mix: read [n, 256] bytes (binary16 head_dim-128 rows), write
//               [n, P] packed bytes and [n] 4-byte norms
//   decode mix: read [n, P] bytes and [n] 4-byte norms, write [n, 256] bytes
// P = 32, 48 or 64 (2, 3 or 4 bits at head_dim 128).  The values written are
// an XOR fold of the values read, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_ceiling.h"

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;            // 64 vectors (quads) per block
constexpr int kVecPerBlock = kThreads / 4;
constexpr uint32_t kRow = 256;           // bytes of one binary16 row

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// QW consecutive dwords (a quarter of a packed row) at byte offset off.
template <int QW>
__device__ __forceinline__ void store_q(const uint32_t (&v)[QW], __amdgpu_buffer_rsrc_t r,
                                        uint32_t off) {
    if constexpr (QW == 4) __builtin_amdgcn_raw_buffer_store_b128(u32x4{v[0], v[1], v[2], v[3]}, r, off, 0, 0);
    else if constexpr (QW == 3) __builtin_amdgcn_raw_buffer_store_b96(u32x3{v[0], v[1], v[2]}, r, off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b64(u32x2{v[0], v[1]}, r, off, 0, 0);
}

template <int QW>
__device__ __forceinline__ void load_q(uint32_t (&v)[QW], __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (QW == 4) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if constexpr (QW == 3) {
        const u32x3 t = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
        v[0] = t.x; v[1] = t.y; v[2] = t.z;
    } else {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        v[0] = t.x; v[1] = t.y;
    }
}

// Both mixes move a wave's 16 vectors as contiguous spans: every load and
// store instruction of a wave covers one contiguous run of 16-byte (or 12-,
// 8-byte) pieces, the best access pattern for the mix.  Lane l of a wave
// reads/writes bytes 16 l + 1024 g of the wave's 4 KiB of binary16 rows and
// bytes P l / 4 of its 16 P bytes of packed rows; lanes 0-15 move the norms.

// Encode mix: read 16 x 256 bytes, write 16 x P + 16 x 4 bytes per wave.
template <int QW>
__global__ __launch_bounds__(kThreads) void encode_mix(const uint8_t *__restrict__ x, int64_t n,
                                                       uint8_t *__restrict__ packed,
                                                       uint32_t *__restrict__ norms) {
    constexpr uint32_t P = 16 * QW;
    const int64_t v0 = (int64_t)blockIdx.x * kVecPerBlock + 16 * (threadIdx.x >> 6);
    if (v0 >= n) return;                                  // uniform over the wave
    const uint32_t nw = (uint32_t)((n - v0 < 16) ? n - v0 : 16);
    const uint32_t l = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rx = rsrc(x + v0 * kRow, nw * kRow);
    uint32_t f[4] = {0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rx, 16u * l + 1024u * g, 0, 0);
        f[0] ^= t.x; f[1] ^= t.y; f[2] ^= t.z; f[3] ^= t.w;
    }
    uint32_t o[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i) o[i] = f[i & 3] ^ (uint32_t)i;
    store_q<QW>(o, rsrc(packed + v0 * P, nw * P), 4u * QW * l);
    if (l < 16)
        __builtin_amdgcn_raw_buffer_store_b32(f[0] ^ f[1] ^ f[2] ^ f[3], rsrc(norms + v0, nw * 4u),
                                              4u * l, 0, 0);
}

// Decode mix: read 16 x P + 16 x 4 bytes, write 16 x 256 bytes per wave.
template <int QW>
__global__ __launch_bounds__(kThreads) void decode_mix(const uint8_t *__restrict__ packed,
                                                       const uint32_t *__restrict__ norms,
                                                       int64_t n, uint8_t *__restrict__ out) {
    constexpr uint32_t P = 16 * QW;
    const int64_t v0 = (int64_t)blockIdx.x * kVecPerBlock + 16 * (threadIdx.x >> 6);
    if (v0 >= n) return;                                  // uniform over the wave
    const uint32_t nw = (uint32_t)((n - v0 < 16) ? n - v0 : 16);
    const uint32_t l = threadIdx.x & 63;
    uint32_t c[QW];
    load_q<QW>(c, rsrc(packed + v0 * P, nw * P), 4u * QW * l);
    uint32_t f = __builtin_amdgcn_raw_buffer_load_b32(rsrc(norms + v0, nw * 4u), 4u * (l & 15), 0, 0);
#pragma unroll
    for (int i = 0; i < QW; ++i) f ^= c[i];
    const __amdgpu_buffer_rsrc_t ro = rsrc(out + v0 * kRow, nw * kRow);
#pragma unroll
    for (int g = 0; g < 4; ++g)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{f, f ^ 1u, f ^ 2u, f ^ (uint32_t)g}, ro,
                                               16u * l + 1024u * g, 0, 0);
}

}  // namespace

extern "C" int tq_ceiling_stream(int mode, int packed_bytes, const void *in0, const void *in1,
                                 int64_t n, void *out0, void *out1, void *stream) {
    if (mode != 0 && mode != 1) return 1;
    if (packed_bytes != 32 && packed_bytes != 48 && packed_bytes != 64) return 1;
    if (n < 0) return 1;
    if (n == 0) return 0;
    if (!in0 || !out0 || (mode == 0 ? !out1 : !in1)) return 1;
    if (n > (int64_t)kVecPerBlock * 0x7fffffff) return 1;
    const dim3 grid((unsigned)((n + kVecPerBlock - 1) / kVecPerBlock)), block(kThreads);
    hipStream_t s = (hipStream_t)stream;
    const uint8_t *i0 = static_cast<const uint8_t *>(in0);
    uint8_t *o0 = static_cast<uint8_t *>(out0);
#define TQ_MIX(QW)                                                                                \
    if (mode == 0)                                                                                \
        hipLaunchKernelGGL(encode_mix<QW>, grid, block, 0, s, i0, n, o0,                          \
                           static_cast<uint32_t *>(out1));                                        \
    else                                                                                          \
        hipLaunchKernelGGL(decode_mix<QW>, grid, block, 0, s, i0,                                 \
                           static_cast<const uint32_t *>(in1), n, o0);
    switch (packed_bytes) {
        case 64: TQ_MIX(4) break;
        case 48: TQ_MIX(3) break;
        default: TQ_MIX(2) break;
    }
#undef TQ_MIX
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
