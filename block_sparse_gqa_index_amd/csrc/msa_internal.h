// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

constexpr int kSeg = 128;   // query positions per work item of the key-block-outer kernels

// Validated problem sizes (see msa.h for their meaning).
struct LaunchDims {
    int B, N, Hkv, G, D, Di, k, nb, dtype;   // dtype: 0 = bf16, 1 = fp32
    int Hq() const { return Hkv * G; }
};

// Byte offsets (from the workspace base) of the selection-inversion buffers.
struct ListLayout {
    size_t n_keys, max_entries, max_items;
    size_t counts, offsets, item_offsets, cursor, total, items, list, end;
    bool has_nonlocal;   // some row keeps a block other than its local one
};

struct AttnWorkspace {
    ListLayout lists;
    size_t vt, po, plse, bytes;
};

struct KlWorkspace {
    ListLayout lists;
    size_t part, red, bytes;
    int red_blocks;
};

ListLayout list_layout(const LaunchDims& d, size_t base);
void launch_build_lists(const LaunchDims& d, const int32_t* block_idx, unsigned char* ws, const ListLayout& L,
                        hipStream_t st);

AttnWorkspace attn_workspace_layout(const LaunchDims& d);
KlWorkspace kl_workspace_layout(const LaunchDims& d);

hipError_t launch_index_topk(const LaunchDims& d, const void* q_idx, const void* k_idx,
                             int32_t* block_idx, hipStream_t st);

hipError_t launch_sparse_attn(const LaunchDims& d, const void* q, const void* k, const void* v,
                              const int32_t* block_idx, float scale, void* o, float* lse, void* ws,
                              hipStream_t st);

hipError_t launch_kl_align(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                           const void* k_idx, const int32_t* block_idx, const float* lse, float scale,
                           float index_scale, float* kl_rows, float* kl_sum, void* ws, hipStream_t st);

}  // namespace msa
