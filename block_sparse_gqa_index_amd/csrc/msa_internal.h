// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

constexpr int kSeg = 128;        // query positions per work item of the key-block-outer forward kernels
constexpr int kSegBwd = 1024;    // query positions per work item of the backward kernel
constexpr int kWindow = 65536;   // query positions per window of the inverted selection

// Validated problem sizes (see msa.h for their meaning).
struct LaunchDims {
    int B, N, Hkv, G, D, Di, k, nb, dtype;   // dtype: 0 = bf16, 1 = fp32 (2 = fp8, 3 = fp4: selection only)
    int Bk = 128;   // block size of the selection (nb counts 128-token blocks whatever Bk is)
    int Hq() const { return Hkv * G; }
};

// A selection at block size 64 or 256 rewritten over 128-token blocks (entries,
// per-entry half masks for Bk = 64, per-row counts and local-block flag) for
// the attention and KL kernels; nothing for Bk = 128 (end == base).
struct ExpandLayout {
    size_t ids, hmask, info, end;
};

// Byte offsets (from the workspace base) of the selection-inversion buffers.
struct ListLayout {
    size_t n_keys, max_entries, max_items;
    size_t bits, counts, offsets, item_offsets, cursor, total, items, list, end;
    int seg;             // list entries per work item
    bool sorted;         // lists in ascending position order (built through per-key bitmaps)
    bool has_nonlocal;   // some row keeps a block other than its local one
};

struct AttnWorkspace {
    ExpandLayout ex;   // Bk != 128 only
    ListLayout lists;
    size_t vt, po, plse, bytes;
};


struct KlWorkspace {
    ExpandLayout ex;   // Bk != 128 only
    ListLayout lists;
    size_t part, red, bytes;
    int red_blocks;
};

ListLayout list_layout(const LaunchDims& d, size_t base, int seg = kSeg, bool sorted = false);

int expanded_topk(const LaunchDims& d);    // entries per row after the rewrite
LaunchDims as_128(const LaunchDims& d);    // the same problem over 128-token blocks, expanded_topk entries
ExpandLayout expand_layout(const LaunchDims& d, size_t base);
void launch_expand(const LaunchDims& d, const int32_t* block_idx, unsigned char* ws, const ExpandLayout& E,
                   hipStream_t st);
int windows(const LaunchDims& d);   // kWindow-position windows of the sequence

// Work item handled by work-group x of a key-block-outer launch (grid a
// multiple of 64): the 8 XCDs take turns on runs of 8 consecutive items, so all
// XCDs move through the item list (and its windows) together while each XCD's
// consecutive items usually share a key block in its L2.
__device__ __forceinline__ int item_of_workgroup(int x) { return (x & ~63) + ((x & 7) << 3) + ((x >> 3) & 7); }
// Lists for the query positions [p_lo, p_hi) of every (batch, group) (sorted
// layouts: the whole sequence only).
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
// The same per-block transposed copy of any [B, N, Hkv, D] tensor into dst
// [B, Hkv, nb, D, 128] (keys permuted within groups of 16, zeros past N).
hipError_t launch_transpose_kv(const LaunchDims& d, const void* src, void* dst, hipStream_t st);

// Attention for the query blocks [qb_lo, qb_hi); the V^T copy must be in ws.
// `stages`: bit 0 builds the query lists, bit 1 runs the non-local blocks,
// bit 2 the local blocks and the merge (the MSA_STAGE_* values).
hipError_t launch_sparse_attn(const LaunchDims& d, int qb_lo, int qb_hi, const void* q, const void* k,
                              const int32_t* block_idx, float scale, void* o, float* lse, void* ws, int stages,
                              hipStream_t st);


// KL forward; index_lse (nullable) receives the student's natural-log LSE per row.
hipError_t launch_kl_align(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                           const void* k_idx, const int32_t* block_idx, const float* lse, float scale,
                           float index_scale, float* kl_rows, float* kl_sum, float* index_lse, void* ws,
                           hipStream_t st);

// Dl = <dO, O> per (b, h, i) row in fp32 ([B, Hq, N]).
void launch_bwd_delta(const LaunchDims& d, const void* o, const void* dout, float* dl, hipStream_t st);

// Backward over the cached block ids (bf16), query window by query window of
// kWindow positions: dq, dk, dv of the main branch for <dO, O> and/or dq_idx,
// dk_idx of the KL term for sum_rows w_row KL_row (both from one pass in which
// the main-branch probabilities are computed once). BwdParts: the parts one
// call computes (the pointers of a part not computed are unused).
struct BwdParts {
    bool main, kl;
};
struct FusedBwdArgs {
    const void *q, *k, *v, *q_idx, *k_idx, *o, *dout;
    const int32_t* block_idx;
    const float *lse, *index_lse, *dkl_rows;
    float scale, iscale, kl_weight;
    void *dq, *dk, *dv, *dq_idx, *dk_idx;
    BwdParts parts;
};
struct FusedBwdWorkspace {
    ListLayout lists;   // position-sorted, kSegBwd entries per item, for the whole sequence
    size_t kt, kit, dl, teacher, dq_part, dqi_part, dkv_part, dki_part, acc_dkv, acc_dki, bytes;
    int bound;          // non-local work-item slots per (b, g) and window
    size_t items;       // partial slots of one window: non-local, then local
};
FusedBwdWorkspace fused_bwd_workspace_layout(const LaunchDims& d, BwdParts parts);
hipError_t launch_fused_bwd(const LaunchDims& d, const FusedBwdArgs& a, void* ws, hipStream_t st);

// Window of the fused backward: query positions [p0, p0 + len) of every
// (b, g) and the work-item slots of their lists. Non-local slot x of (b, g)
// (work-group (b * Hkv + g) * bound + x) is the x-th item of the keys
// (b, g, w, 0 .. nb-1), which the position-sorted lists keep contiguous; the
// local items of the window's query blocks follow all non-local slots.
struct FusedWindow {
    int w, p0, len, qb0;   // window index, first position, positions, first query block
    int bound;             // non-local work-item slots per (b, g)
};

// Dense causal attention (every visible key kept): V^T copy into ws, then the
// query-block-outer kernel. ws holds dense_workspace_bytes(d).
size_t dense_workspace_bytes(const LaunchDims& d);
hipError_t launch_dense_attn(const LaunchDims& d, const void* q, const void* k, const void* v, float scale, void* o,
                             float* lse, void* ws, hipStream_t st);

// Dense KL (every visible token; lse from the dense attention): kl_rows, the
// fixed-order kl_sum, optional index_lse. ws holds dense_kl_workspace_bytes(d).
size_t dense_kl_workspace_bytes(const LaunchDims& d);
hipError_t launch_dense_kl_align(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                                 const void* k_idx, const float* lse, float scale, float index_scale, float* kl_rows,
                                 float* kl_sum, float* index_lse, void* ws, hipStream_t st);

}  // namespace msa
