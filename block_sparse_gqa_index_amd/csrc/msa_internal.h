// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

constexpr int kSeg = 128;        // query positions per work item of the key-block-outer kernels
constexpr int kWindow = 65536;   // query positions per window of the inverted selection

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
int windows(const LaunchDims& d);   // kWindow-position windows of the sequence

// Work item handled by work-group x of a key-block-outer launch (grid a
// multiple of 64): the 8 XCDs take turns on runs of 8 consecutive items, so all
// XCDs move through the item list (and its windows) together while each XCD's
// consecutive items usually share a key block in its L2.
__device__ __forceinline__ int item_of_workgroup(int x) { return (x & ~63) + ((x & 7) << 3) + ((x >> 3) & 7); }
// Lists for the query positions [p_lo, p_hi) of every (batch, group).
void launch_build_lists(const LaunchDims& d, int p_lo, int p_hi, const int32_t* block_idx, unsigned char* ws,
                        const ListLayout& L, hipStream_t st);
// Upper bound on the work items launch_build_lists produces for that range.
size_t list_items_bound(const LaunchDims& d, int p_lo, int p_hi, const ListLayout& L);

// Number of rows of block_idx that break the selection layout -> *bad.
hipError_t launch_check_block_idx(const LaunchDims& d, const int32_t* block_idx, int32_t* bad, hipStream_t st);

AttnWorkspace attn_workspace_layout(const LaunchDims& d);
KlWorkspace kl_workspace_layout(const LaunchDims& d);

// Selection for the query blocks [qb_lo, qb_hi).
hipError_t launch_index_topk(const LaunchDims& d, int qb_lo, int qb_hi, const void* q_idx, const void* k_idx,
                             int32_t* block_idx, hipStream_t st);

// V^T copy into the attention workspace (needed once per forward).
hipError_t launch_transpose_v(const LaunchDims& d, const void* v, void* ws, hipStream_t st);

// Attention for the query blocks [qb_lo, qb_hi); the V^T copy must be in ws.
// `stages`: bit 0 builds the query lists, bit 1 runs the non-local blocks,
// bit 2 the local blocks and the merge (the MSA_STAGE_* values).
hipError_t launch_sparse_attn(const LaunchDims& d, int qb_lo, int qb_hi, const void* q, const void* k,
                              const int32_t* block_idx, float scale, void* o, float* lse, void* ws, int stages,
                              hipStream_t st);

hipError_t launch_kl_align(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                           const void* k_idx, const int32_t* block_idx, const float* lse, float scale,
                           float index_scale, float* kl_rows, float* kl_sum, void* ws, hipStream_t st);

}  // namespace msa
