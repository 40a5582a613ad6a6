// Internal interface between the C-ABI host code (tq_abi.cpp) and the HIP
// kernels (tq_codec.hip, tq_attn.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kMaxHeadDim = 256;   // the kernels take head_dim 64, 128 and 256

// Everything the kernels need that is fixed by (bits, seed).  Passed by value
// as a kernel argument, so the library needs no device allocation.
struct CodecConsts {
    uint32_t sign[kMaxHeadDim / 32];   // bit i of sign[i / 32] set  <=>  sigma_i = -1
    float thr8[15];     // decision thresholds times 8, ascending (2^bits - 1 used)
    float level[16];    // Lloyd-Max levels, ascending (2^bits used)
    float one;          // 1.0f, kept opaque to the compiler (see the encode kernel)
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

// ---------------------------------------------------------------------------
// decode attention
// ---------------------------------------------------------------------------

constexpr int kAttnBlockSize = 16;   // tokens per cache page
constexpr int kAttnMaxGroup = 16;    // query heads per kv head
constexpr int kAttnMaxGroupD256 = 8; // the same at head_dim 256
constexpr int kAttnMaxBatch = 65535;               // sequences: the split grid's y extent
constexpr int kAttnMaxBlocks = 0x7fffffff / 16;    // pages per sequence: tokens fit an int

struct AttnShape {
    int batch, num_q_heads, num_kv_heads, head_dim, k_bits, v_bits, max_blocks;
    int64_t num_blocks;
};

// Whether the split kernel serves this shape (head_dim 64, 128 or 256, 1..16
// query heads per kv head, 2..4-bit keys and values).
bool attn_supported(const AttnShape &s);

// Tokens handled by one wave of the split kernel, and the number of splits of
// the longest possible context (neither depends on the bit widths).
int attn_split_tokens(const AttnShape &s);
int attn_num_splits(const AttnShape &s);
size_t attn_workspace_bytes(const AttnShape &s);

hipError_t launch_attn(const AttnShape &s, const CodecConsts &kc, const CodecConsts &vc,
                       const void *q, const uint8_t *k_packed, const float *k_norms,
                       const uint8_t *v_packed, const float *v_norms,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       void *out, void *workspace, hipStream_t stream);

int device_cu_count();

}  // namespace tq
