// Internal interface between the C-ABI host code (tq_abi.cpp) and the decode
// attention kernels (tq_attn.hip).  Not installed; not part of the ABI.
#pragma once

#include "tq.h"
#include "tq_internal.h"

namespace tq {

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

// Size of the library-owned attention workspace (per GPU) used by the
// entry point that allocates nothing.
constexpr size_t kAttnStaticWorkspaceBytes = TQ_ATTN_NOALLOC_WORKSPACE_BYTES;

// Device address of that workspace on the current device, looked up once per
// device (hipGetSymbolAddress) and cached.
hipError_t attn_static_workspace(void **ptr);

hipError_t launch_attn(const AttnShape &s, const CodecConsts &kc, const CodecConsts &vc,
                       const void *q, const uint8_t *k_packed, const float *k_norms,
                       const uint8_t *v_packed, const float *v_norms,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       void *out, void *workspace, hipStream_t stream);

}  // namespace tq
