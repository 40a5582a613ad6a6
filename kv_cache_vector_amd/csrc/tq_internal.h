// Internal interface between the C-ABI host code (tq_abi.cpp) and the codec
// kernels (tq_codec.hip); the attention kernels' part is tq_attn_internal.h.
// Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kMaxHeadDim = 256;   // the kernels take head_dim 64, 128 and 256

// Everything the kernels need that is fixed by (bits, seed).  Passed by value
// as a kernel argument, so the library needs no device allocation.
struct CodecConsts {
    uint32_t sign[kMaxHeadDim / 32];   // bit i of sign[i / 32] set  <=>  sigma_i = -1
    float level[16];    // Lloyd-Max levels, ascending (2^bits used)
};

// Decision table of the encode kernel: cell i (index i + kEncCells) covers
// the values y = 8 z whose conversion to int (toward zero) is i; it holds the
// one threshold inside the cell (+inf if none) and the number of thresholds
// below the cell.  Built on the host from the f32 thresholds.  |y| is at most
// 8 sqrt(head_dim) (all of the unit vector's mass on one rotated coordinate),
// 128 at head_dim 256.
constexpr int kEncCells = 128;
struct EncTable {
    // (threshold * 8, code word): at 4 bits the bytes {base, base + 1,
    // base << 4, (base + 1) << 4}, at 2 bits {base, base + 1, 0, 0}, at 3
    // bits the base code
    float2 cell[2 * kEncCells + 1];
};

// Encode `n` vectors of head_dim (64, 128 or 256) binary16 values.  With
// `slots` non-null, vector v is written to row slots[v] of (packed, norms)
// and skipped when that row is outside [0, num_slots); otherwise to row v.
hipError_t launch_encode(int head_dim, int bits, const void *x, int64_t n, const int64_t *slots,
                         int64_t num_slots, const CodecConsts &k, const EncTable &t,
                         uint8_t *packed, float *norms, hipStream_t stream);

hipError_t launch_decode(int head_dim, int bits, const uint8_t *packed, const float *norms,
                         int64_t n, const CodecConsts &k, void *out, hipStream_t stream);

// Hybrid modes (tq35 / tq25) at head_dim 128: two channel groups of 64 coded
// as TurboQuant vectors at (3, 2) or (2, 1) bits, plus the sign sketch of the
// residual.  Everything fixed by (mode, seed, channel permutation).
struct HybridConsts {
    uint32_t sign[4];   // sigma of group-order positions 0..127 (A: 0..63, B: 64..127)
    uint32_t qsign[4];  // sigma_Q of the sketch
    float thr_a[7];     // 8 x the group-A thresholds (2^bA - 1 used), ascending
    float thr_b[3];     // 8 x the group-B thresholds
    float lev_a[8];     // group-A levels
    float lev_b[4];     // group-B levels
    uint32_t gidx[32];  // byte 32 q + r: the channel held in register r of lane q
};

constexpr int kHybridHeadDim = 128;

// Row bytes of a hybrid mode (35 or 25) at head_dim 128: 68 or 52.
int hybrid_row_bytes(int mode);

hipError_t launch_hybrid_encode(int mode, const void *x, int64_t n, const HybridConsts &k,
                                uint8_t *packed, hipStream_t stream);
hipError_t launch_hybrid_decode(int mode, const uint8_t *packed, int64_t n,
                                const HybridConsts &k, void *out, hipStream_t stream);

int device_cu_count();

}  // namespace tq
