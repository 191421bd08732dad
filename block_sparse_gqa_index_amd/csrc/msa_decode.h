// Host-side launch interface of the decode kernels (one new query per
// sequence against a cache of C tokens per sequence).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Validated decode sizes: B sequences, cache capacity C tokens, dtype 0 = bf16, 1 = fp32, 2 = fp8 e4m3
// (the selection only).
struct DecodeDims {
    int B, C, Hkv, G, D, Di, k, dtype;
    int R;   // new queries per sequence (positions n_b - R .. n_b - 1)
    int nbs() const { return (C + 127) / 128; }   // blocks of a full cache
};

// Byte offsets from the workspace base. The selection's block scores and the
// attention's partials are never live at the same time, so both start at 0.
struct DecodeWorkspace {
    size_t scores, index_bytes;   // block scores [B, R * Hkv, nbs] fp32
    size_t po, plse, attn_bytes;  // partial outputs [B, R, Hkv, k, G, D] fp32 and LSEs [B, R, Hkv, k, G] fp32
};

DecodeWorkspace decode_workspace_layout(const DecodeDims& d);

// Block scores then top-k -> block_idx [B, Hkv, k]. `pages` (nullable): block
// table [B, ceil(C/128)] into a pool of num_pages 128-token pages holding k_idx.
hipError_t launch_decode_index(const DecodeDims& d, const void* q_idx, const void* k_idx, const int32_t* seqlens,
                               const int32_t* pages, int num_pages, int32_t* block_idx, void* ws, hipStream_t st);

// Per-block partials then their merge -> o [B, Hq, D], lse [B, Hq]; `pages` as above for K and V.
hipError_t launch_decode_attn(const DecodeDims& d, const void* q, const void* k, const void* v,
                              const int32_t* seqlens, const int32_t* block_idx, const int32_t* pages, int num_pages,
                              float scale, void* o, float* lse, void* ws, hipStream_t st);

}  // namespace msa
