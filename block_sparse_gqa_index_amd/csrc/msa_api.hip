// C ABI of the MSA forward path and of the main branch's backward: argument
// validation, workspace sizing and dispatch to the kernels. Every check here
// runs on the host before any HIP call, so a rejected call enqueues nothing
// and writes nothing.
#include "../../include/msa.h"

#include <limits.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "msa_decode.h"
#include "msa_internal.h"

namespace {

using msa::LaunchDims;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_upto32(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32; }

constexpr int kOpLayout = -1;   // the block_idx layout check: neither heads nor index dims

// Shape checks shared by all entry points; fills `out` on success. The index
// selection does not look at group_size/head_dim and the attention does not
// look at index_dim, so those are only checked for the ops that use them.
int check_dims(const msa_dims* d, int op, LaunchDims* out) {
    if (!d) return MSA_ERR_NULL;
    // MSA_OP_FORWARD and MSA_OP_DECODE: both
    const bool uses_heads = op != MSA_OP_INDEX && op != kOpLayout && op != MSA_OP_DECODE_INDEX;
    const bool uses_index = op != MSA_OP_ATTN && op != MSA_OP_ATTN_BWD && op != kOpLayout &&
                            op != MSA_OP_DECODE_ATTN && op != MSA_OP_DENSE_ATTN;
    const bool uses_topk = op != MSA_OP_DENSE_ATTN && op != MSA_OP_DENSE_KL;
    if (d->batch < 0 || d->seqlen < 0 || d->kv_heads < 1 || d->block_size < 1 || (uses_topk && d->topk < 1) ||
        (uses_heads && (d->group_size < 1 || d->head_dim < 1)) || (uses_index && d->index_dim < 1))
        return MSA_ERR_SHAPE;
    // fp8 index inputs: selection only; fp4 (two values per byte): the forward selection only
    const bool fp8_ok = op == MSA_OP_INDEX || op == kOpLayout || op == MSA_OP_DECODE_INDEX;
    const bool fp4_ok = op == MSA_OP_INDEX || op == kOpLayout;
    // Block sizes: 128 everywhere; 64 and 256 for the selection (bf16, fp32)
    // and for the attention and KL forward, which take a 256-token block as two
    // 128-token ones (so at most 16 of them fit the 32 slots).
    const bool bk_ok = d->block_size == 128 ||
                       ((d->block_size == 64 || d->block_size == 256) && (d->dtype == MSA_BF16 || d->dtype == MSA_F32) &&
                        (op == MSA_OP_INDEX || op == kOpLayout || op == MSA_OP_ATTN || op == MSA_OP_KL ||
                         op == MSA_OP_FORWARD) &&
                        (d->block_size == 64 || op == MSA_OP_INDEX || op == kOpLayout || d->topk <= 16));
    if (!bk_ok || (uses_topk && d->topk > 32) ||
        (d->dtype != MSA_BF16 && d->dtype != MSA_F32 && !(fp8_ok && d->dtype == MSA_FP8_E4M3) &&
         !(fp4_ok && d->dtype == MSA_FP4_E2M1)) ||
        ((op == MSA_OP_ATTN_BWD || op == MSA_OP_KL_BWD || op == MSA_OP_FUSED_BWD) && d->dtype != MSA_BF16) ||
        d->causal != 1 || (uses_heads && (!pow2_upto32(d->group_size) || (d->head_dim != 64 && d->head_dim != 128))) ||
        (uses_index && d->index_dim != 64 && d->index_dim != 128))
        return MSA_ERR_UNSUPPORTED;
    // Positions are packed into 26 bits of a list entry; row counts and list
    // offsets are 32-bit.
    if (d->seqlen >= (int64_t(1) << 26)) return MSA_ERR_SHAPE;
    if (d->kv_heads > 4096) return MSA_ERR_SHAPE;
    const bool decode = op == MSA_OP_DECODE_INDEX || op == MSA_OP_DECODE_ATTN || op == MSA_OP_DECODE;
    // Decode grids: sequences x group chunks of 32 on one grid axis.
    if (decode && (d->batch > 65535 || d->batch * ((d->kv_heads + 31) / 32) > 65535)) return MSA_ERR_SHAPE;
    // (Decode kernels index the caches with 64-bit offsets; only their grids are bounded.)
    const int64_t rows = d->batch * d->seqlen * d->kv_heads;
    if (!decode && (d->batch > INT_MAX || rows > INT_MAX || rows * (int64_t)(uses_topk ? d->topk : 1) > INT_MAX))
        return MSA_ERR_SHAPE;
    // Work items of the inverted selection carry a 32-bit key per (batch,
    // group, query window, key block).
    const int64_t nb64 = (d->seqlen + 127) / 128, nwin64 = (d->seqlen + msa::kWindow - 1) / msa::kWindow;
    if (!decode && d->batch * d->kv_heads * nwin64 * nb64 > INT_MAX) return MSA_ERR_SHAPE;
    out->B = (int)d->batch;
    out->N = (int)d->seqlen;
    out->Hkv = d->kv_heads;
    out->G = uses_heads ? d->group_size : 1;
    out->D = uses_heads ? d->head_dim : 0;
    out->Di = uses_index ? d->index_dim : 0;
    out->k = uses_topk ? d->topk : 1;
    out->nb = (int)((d->seqlen + 127) / 128);
    out->dtype = d->dtype;
    out->Bk = d->block_size;
    return MSA_OK;
}

bool empty(const LaunchDims& L) { return L.B == 0 || L.N == 0; }

msa::DecodeDims decode_dims(const LaunchDims& L, int R = 1) {
    return msa::DecodeDims{L.B, L.N, L.Hkv, L.G, L.D, L.Di, L.k, L.dtype, R};
}

size_t decode_ws(const LaunchDims& L, int op, int R) {
    const msa::DecodeWorkspace W = msa::decode_workspace_layout(decode_dims(L, R));
    if (op == MSA_OP_DECODE_INDEX) return W.index_bytes;
    if (op == MSA_OP_DECODE_ATTN) return W.attn_bytes;
    return W.index_bytes > W.attn_bytes ? W.index_bytes : W.attn_bytes;
}

// Decode calls share their argument checks: sizes, the per-op pointers, and
// the workspace of `op`.
int check_decode(const msa_dims* dims, int R, int op, LaunchDims* L, std::initializer_list<const void*> ptrs,
                 const void* ws, size_t ws_bytes, bool check_ws = true) {
    int st = check_dims(dims, op, L);
    if (st != MSA_OK) return st;
    // R new queries per sequence; the grids put sequences x queries (x group chunks of 32) on one axis.
    if (R < 1 || R > 65535 || (int64_t)L->B * R > 65535 ||
        (int64_t)L->B * (((int64_t)R * L->Hkv + 31) / 32) > 65535)
        return MSA_ERR_SHAPE;
    if (dims->dtype != MSA_BF16 && dims->dtype != MSA_F32 &&
        !(op == MSA_OP_DECODE_INDEX && dims->dtype == MSA_FP8_E4M3))
        return MSA_ERR_UNSUPPORTED;
    if (empty(*L)) return MSA_OK;
    for (const void* p : ptrs)
        if (!p) return MSA_ERR_NULL;
    for (const void* p : ptrs)
        if (!aligned16(p)) return MSA_ERR_ALIGN;
    const size_t need = decode_ws(*L, op, R);
    if (check_ws && need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MSA_ERR_WORKSPACE;
    return MSA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

}  // namespace

// ------------------------------------------------- no-allocation decoding --
// The scratch memory of msa_decode_noalloc: a file-scope device array, one copy
// per GPU, in place of a caller-provided workspace (the decode's block scores,
// then its per-block partial outputs and LSEs). Every call on a GPU uses that
// GPU's copy, so calls that overlap on one GPU race on it. Host code never
// passes the array's name to a kernel or a copy (on the host it is only a
// stand-in): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept.
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array (MSA_ERR_HIP if HIP
// cannot name the device or the symbol; nothing is enqueued either way).
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_HIP;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_HIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MSA_OK;
}

}  // namespace

extern "C" {

int msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_strerror(int status) {
    switch (status) {
        case MSA_OK: return "ok";
        case MSA_ERR_NULL: return "a required pointer is NULL";
        case MSA_ERR_SHAPE: return "invalid or too large problem sizes";
        case MSA_ERR_UNSUPPORTED: return "unsupported sizes or dtype (block_size 128, or 64/256 for the selection, "
                                         "attention and KL forward (256: topk <= 16 there), topk 1..32, group_size "
                                         "power of two <= 32, head/index dim 64 or 128, bf16/fp32 (fp8 e4m3 "
                                         "and fp4 e2m1 for the selection only, bf16 for the backward), causal)";
        case MSA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case MSA_ERR_WORKSPACE: return "workspace missing or smaller than msa_workspace_bytes";
        case MSA_ERR_HIP: return "HIP kernel launch failed";
        case MSA_ERR_SCRATCH: return "the problem needs more than the no-allocation entry point's scratch memory "
                                     "(MSA_NOALLOC_SCRATCH_BYTES = 64 MiB)";
        default: return "unknown status";
    }
}

size_t msa_workspace_bytes(const msa_dims* dims, int op) {
    LaunchDims L;
    if (op < MSA_OP_INDEX || op > MSA_OP_FUSED_BWD) return 0;
    if (check_dims(dims, op, &L) != MSA_OK || empty(L)) return 0;
    switch (op) {
        case MSA_OP_INDEX: return 0;
        case MSA_OP_ATTN:
        case MSA_OP_FORWARD: return msa::attn_workspace_layout(L).bytes;
        case MSA_OP_ATTN_BWD: return msa::fused_bwd_workspace_layout(L, msa::BwdParts{true, false}).bytes;
        case MSA_OP_KL: return msa::kl_workspace_layout(L).bytes;
        case MSA_OP_KL_BWD: return msa::fused_bwd_workspace_layout(L, msa::BwdParts{false, true}).bytes;
        case MSA_OP_DECODE_INDEX:
        case MSA_OP_DECODE_ATTN: return decode_ws(L, op, 1);
        case MSA_OP_DENSE_ATTN: return msa::dense_workspace_bytes(L);
        case MSA_OP_DENSE_KL: return msa::dense_kl_workspace_bytes(L);
        case MSA_OP_DECODE: return decode_ws(L, op, 1);
        case MSA_OP_FUSED_BWD: return msa::fused_bwd_workspace_layout(L, msa::BwdParts{true, true}).bytes;
        default: return 0;
    }
}

int msa_index_topk(const msa_dims* dims, const void* q_idx, const void* k_idx, int32_t* block_idx,
                   void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_INDEX, &L);
    if (st != MSA_OK) return st;
    if (empty(L)) return MSA_OK;
    if (!q_idx || !k_idx || !block_idx) return MSA_ERR_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(block_idx)) return MSA_ERR_ALIGN;
    return hip_status(msa::launch_index_topk(L, 0, L.nb, q_idx, k_idx, block_idx, static_cast<hipStream_t>(stream)));
}

int msa_check_block_idx(const msa_dims* dims, const int32_t* block_idx, int32_t* bad_rows, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, kOpLayout, &L);
    if (st != MSA_OK) return st;
    if (!bad_rows || (!empty(L) && !block_idx)) return MSA_ERR_NULL;
    if (!aligned16(block_idx) || (reinterpret_cast<uintptr_t>(bad_rows) & 3u)) return MSA_ERR_ALIGN;
    return hip_status(msa::launch_check_block_idx(L, block_idx, bad_rows, static_cast<hipStream_t>(stream)));
}

int msa_sparse_attn_fwd_stages(const msa_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, float softmax_scale, void* o, float* lse, void* ws,
                               size_t ws_bytes, int stages, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_ATTN, &L);
    if (st != MSA_OK) return st;
    if (stages <= 0 || (stages & ~MSA_STAGE_ALL)) return MSA_ERR_UNSUPPORTED;
    if (empty(L)) return MSA_OK;
    if (!q || !k || !v || !block_idx || !o || !lse) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) || !aligned16(o) ||
        !aligned16(lse))
        return MSA_ERR_ALIGN;
    const size_t need = msa::attn_workspace_layout(L).bytes;
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((stages & MSA_STAGE_PREPARE) && msa::launch_transpose_v(L, v, ws, s) != hipSuccess) return MSA_ERR_HIP;
    return hip_status(msa::launch_sparse_attn(L, 0, L.nb, q, k, block_idx, scale, o, lse, ws, stages, s));
}

int msa_sparse_attn_fwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* block_idx, float softmax_scale, void* o, float* lse, void* ws,
                        size_t ws_bytes, void* stream) {
    return msa_sparse_attn_fwd_stages(dims, q, k, v, block_idx, softmax_scale, o, lse, ws, ws_bytes,
                                      MSA_STAGE_ALL, stream);
}

int msa_forward(const msa_dims* dims, const void* q_idx, const void* k_idx, const void* q, const void* k,
                const void* v, float softmax_scale, int32_t* block_idx, void* o, float* lse, void* ws,
                size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_FORWARD, &L);
    if (st != MSA_OK) return st;
    if (empty(L)) return MSA_OK;
    if (!q_idx || !k_idx || !q || !k || !v || !block_idx || !o || !lse) return MSA_ERR_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
        !aligned16(block_idx) || !aligned16(o) || !aligned16(lse))
        return MSA_ERR_ALIGN;
    const size_t need = msa::attn_workspace_layout(L).bytes;
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (msa::launch_index_topk(L, 0, L.nb, q_idx, k_idx, block_idx, s) != hipSuccess) return MSA_ERR_HIP;
    if (msa::launch_transpose_v(L, v, ws, s) != hipSuccess) return MSA_ERR_HIP;
    return hip_status(msa::launch_sparse_attn(L, 0, L.nb, q, k, block_idx, scale, o, lse, ws, MSA_STAGE_ALL, s));
}

int msa_sparse_attn_bwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* block_idx, const void* o, const float* lse, const void* dout,
                        float softmax_scale, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_ATTN_BWD, &L);
    if (st != MSA_OK) return st;
    if (empty(L)) return MSA_OK;
    if (!q || !k || !v || !block_idx || !o || !lse || !dout || !dq || !dk || !dv) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) || !aligned16(o) ||
        !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return MSA_ERR_ALIGN;
    const size_t need = msa::fused_bwd_workspace_layout(L, msa::BwdParts{true, false}).bytes;
    if (!ws || ws_bytes < need || !aligned16(ws)) return MSA_ERR_WORKSPACE;
    msa::FusedBwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.block_idx = block_idx;
    a.lse = lse;
    a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.parts = msa::BwdParts{true, false};
    return hip_status(msa::launch_fused_bwd(L, a, ws, static_cast<hipStream_t>(stream)));
}

int msa_kl_align_fwd(const msa_dims* dims, const void* q, const void* k, const void* q_idx,
                     const void* k_idx, const int32_t* block_idx, const float* lse, float softmax_scale,
                     float index_scale, float* kl_rows, float* kl_sum, float* index_lse, void* ws,
                     size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_KL, &L);
    if (st != MSA_OK) return st;
    if (!kl_sum) return MSA_ERR_NULL;
    if (!q || !k || !q_idx || !k_idx || !block_idx || !lse || !kl_rows) {
        if (!empty(L)) return MSA_ERR_NULL;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx) || !aligned16(block_idx) ||
        !aligned16(lse) || !aligned16(kl_rows) || (reinterpret_cast<uintptr_t>(index_lse) & 3u))
        return MSA_ERR_ALIGN;
    const size_t need = msa::kl_workspace_layout(L).bytes;
    if (!empty(L) && need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    const float iscale = index_scale > 0.f ? index_scale : 1.0f / sqrtf((float)L.Di);
    // kl_sum is written even for an empty problem (the sum of nothing is 0).
    return hip_status(msa::launch_kl_align(L, q, k, q_idx, k_idx, block_idx, lse, scale, iscale, kl_rows,
                                           kl_sum, index_lse, ws, static_cast<hipStream_t>(stream)));
}

int msa_kl_align_bwd(const msa_dims* dims, const void* q, const void* k, const void* q_idx, const void* k_idx,
                     const int32_t* block_idx, const float* lse, const float* index_lse, float softmax_scale,
                     float index_scale, const float* dkl_rows, float kl_weight, void* dq_idx, void* dk_idx,
                     void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_KL_BWD, &L);
    if (st != MSA_OK) return st;
    if (empty(L)) return MSA_OK;
    if (!q || !k || !q_idx || !k_idx || !block_idx || !lse || !index_lse || !dq_idx || !dk_idx) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx) || !aligned16(block_idx) ||
        !aligned16(lse) || !aligned16(index_lse) || !aligned16(dkl_rows) || !aligned16(dq_idx) ||
        !aligned16(dk_idx))
        return MSA_ERR_ALIGN;
    const size_t need = msa::fused_bwd_workspace_layout(L, msa::BwdParts{false, true}).bytes;
    if (!ws || ws_bytes < need || !aligned16(ws)) return MSA_ERR_WORKSPACE;
    msa::FusedBwdArgs a{};
    a.q = q;
    a.k = k;
    a.q_idx = q_idx;
    a.k_idx = k_idx;
    a.block_idx = block_idx;
    a.lse = lse;
    a.index_lse = index_lse;
    a.dkl_rows = dkl_rows;
    a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    a.iscale = index_scale > 0.f ? index_scale : 1.0f / sqrtf((float)L.Di);
    a.kl_weight = kl_weight;
    a.dq_idx = dq_idx;
    a.dk_idx = dk_idx;
    a.parts = msa::BwdParts{false, true};
    return hip_status(msa::launch_fused_bwd(L, a, ws, static_cast<hipStream_t>(stream)));
}

int msa_fused_bwd(const msa_dims* dims, const void* q, const void* k, const void* v, const void* q_idx,
                  const void* k_idx, const int32_t* block_idx, const void* o, const float* lse, const float* index_lse,
                  const void* dout, float softmax_scale, float index_scale, const float* dkl_rows, float kl_weight,
                  void* dq, void* dk, void* dv, void* dq_idx, void* dk_idx, void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_FUSED_BWD, &L);
    if (st != MSA_OK) return st;
    if (empty(L)) return MSA_OK;
    if (!q || !k || !v || !q_idx || !k_idx || !block_idx || !o || !lse || !index_lse || !dout || !dq || !dk || !dv ||
        !dq_idx || !dk_idx)
        return MSA_ERR_NULL;
    for (const void* p : {q, k, v, q_idx, k_idx, (const void*)block_idx, o, (const void*)lse, (const void*)index_lse,
                          dout, (const void*)dkl_rows, (const void*)dq, (const void*)dk, (const void*)dv,
                          (const void*)dq_idx, (const void*)dk_idx})
        if (!aligned16(p)) return MSA_ERR_ALIGN;
    const size_t need = msa::fused_bwd_workspace_layout(L, msa::BwdParts{true, true}).bytes;
    if (!ws || ws_bytes < need || !aligned16(ws)) return MSA_ERR_WORKSPACE;
    msa::FusedBwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.q_idx = q_idx;
    a.k_idx = k_idx;
    a.o = o;
    a.dout = dout;
    a.block_idx = block_idx;
    a.lse = lse;
    a.index_lse = index_lse;
    a.dkl_rows = dkl_rows;
    a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    a.iscale = index_scale > 0.f ? index_scale : 1.0f / sqrtf((float)L.Di);
    a.kl_weight = kl_weight;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dq_idx = dq_idx;
    a.dk_idx = dk_idx;
    a.parts = msa::BwdParts{true, true};
    return hip_status(msa::launch_fused_bwd(L, a, ws, static_cast<hipStream_t>(stream)));
}

int msa_dense_attn_fwd(const msa_dims* dims, const void* q, const void* k, const void* v, float softmax_scale,
                       void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_DENSE_ATTN, &L);
    if (st != MSA_OK) return st;
    if (empty(L)) return MSA_OK;
    if (!q || !k || !v || !o || !lse) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return MSA_ERR_ALIGN;
    const size_t need = msa::dense_workspace_bytes(L);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    return hip_status(msa::launch_dense_attn(L, q, k, v, scale, o, lse, ws, static_cast<hipStream_t>(stream)));
}

size_t msa_decode_workspace_bytes(const msa_dims* dims, int op, int32_t num_queries) {
    LaunchDims L;
    if (op != MSA_OP_DECODE_INDEX && op != MSA_OP_DECODE_ATTN && op != MSA_OP_DECODE) return 0;
    if (num_queries < 1 || check_dims(dims, op, &L) != MSA_OK || empty(L)) return 0;
    return decode_ws(L, op, num_queries);
}

int msa_dense_kl_align_fwd(const msa_dims* dims, const void* q, const void* k, const void* q_idx, const void* k_idx,
                           const float* lse, float softmax_scale, float index_scale, float* kl_rows, float* kl_sum,
                           float* index_lse, void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_dims(dims, MSA_OP_DENSE_KL, &L);
    if (st != MSA_OK) return st;
    if (!kl_sum) return MSA_ERR_NULL;
    if (!empty(L) && (!q || !k || !q_idx || !k_idx || !lse || !kl_rows)) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx) || !aligned16(lse) ||
        !aligned16(kl_rows) || (reinterpret_cast<uintptr_t>(index_lse) & 3u))
        return MSA_ERR_ALIGN;
    const size_t need = msa::dense_kl_workspace_bytes(L);
    if (!empty(L) && (!ws || ws_bytes < need || !aligned16(ws))) return MSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    const float iscale = index_scale > 0.f ? index_scale : 1.0f / sqrtf((float)L.Di);
    // kl_sum is written even for an empty problem (the sum of nothing is 0).
    return hip_status(msa::launch_dense_kl_align(L, q, k, q_idx, k_idx, lse, scale, iscale, kl_rows, kl_sum,
                                                 index_lse, ws, static_cast<hipStream_t>(stream)));
}

int msa_decode_index_topk(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx, const int32_t* seqlens,
                          int32_t* block_idx, void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_decode(dims, num_queries, MSA_OP_DECODE_INDEX, &L, {q_idx, k_idx, seqlens, block_idx}, ws, ws_bytes);
    if (st != MSA_OK || empty(L)) return st;
    return hip_status(msa::launch_decode_index(decode_dims(L, num_queries), q_idx, k_idx, seqlens, nullptr, 0, block_idx, ws,
                                               static_cast<hipStream_t>(stream)));
}

int msa_decode_attn(const msa_dims* dims, int32_t num_queries, const void* q, const void* k, const void* v, const int32_t* seqlens,
                    const int32_t* block_idx, float softmax_scale, void* o, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
    LaunchDims L;
    int st = check_decode(dims, num_queries, MSA_OP_DECODE_ATTN, &L, {q, k, v, seqlens, block_idx, o, lse}, ws, ws_bytes);
    if (st != MSA_OK || empty(L)) return st;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    return hip_status(msa::launch_decode_attn(decode_dims(L, num_queries), q, k, v, seqlens, block_idx, nullptr, 0, scale, o, lse, ws,
                                              static_cast<hipStream_t>(stream)));
}

int msa_decode(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx, const void* q, const void* k,
               const void* v, const int32_t* seqlens, float softmax_scale, int32_t* block_idx, void* o, float* lse,
               void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    int st = check_decode(dims, num_queries, MSA_OP_DECODE, &L, {q_idx, k_idx, q, k, v, seqlens, block_idx, o, lse}, ws,
                          ws_bytes);
    if (st != MSA_OK || empty(L)) return st;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const msa::DecodeDims d = decode_dims(L, num_queries);
    if (msa::launch_decode_index(d, q_idx, k_idx, seqlens, nullptr, 0, block_idx, ws, s) != hipSuccess)
        return MSA_ERR_HIP;
    return hip_status(msa::launch_decode_attn(d, q, k, v, seqlens, block_idx, nullptr, 0, scale, o, lse, ws, s));
}

int msa_decode_paged_index_topk(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx_pages,
                                const int32_t* block_table, int32_t num_pages, const int32_t* seqlens,
                                int32_t* block_idx, void* ws, size_t ws_bytes, void* stream) {
    LaunchDims L;
    if (num_pages < 0) return MSA_ERR_SHAPE;
    int st = check_decode(dims, num_queries, MSA_OP_DECODE_INDEX, &L, {q_idx, k_idx_pages, block_table, seqlens, block_idx}, ws,
                          ws_bytes);
    if (st != MSA_OK || empty(L)) return st;
    return hip_status(msa::launch_decode_index(decode_dims(L, num_queries), q_idx, k_idx_pages, seqlens, block_table, num_pages,
                                               block_idx, ws, static_cast<hipStream_t>(stream)));
}

int msa_decode_paged_attn(const msa_dims* dims, int32_t num_queries, const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, int32_t num_pages, const int32_t* seqlens,
                          const int32_t* block_idx, float softmax_scale, void* o, float* lse, void* ws,
                          size_t ws_bytes, void* stream) {
    LaunchDims L;
    if (num_pages < 0) return MSA_ERR_SHAPE;
    int st = check_decode(dims, num_queries, MSA_OP_DECODE_ATTN, &L, {q, k_pages, v_pages, block_table, seqlens, block_idx, o, lse},
                          ws, ws_bytes);
    if (st != MSA_OK || empty(L)) return st;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    return hip_status(msa::launch_decode_attn(decode_dims(L, num_queries), q, k_pages, v_pages, seqlens, block_idx, block_table,
                                              num_pages, scale, o, lse, ws, static_cast<hipStream_t>(stream)));
}

int msa_decode_paged(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx_pages, const void* q,
                     const void* k_pages, const void* v_pages, const int32_t* block_table, int32_t num_pages,
                     const int32_t* seqlens, float softmax_scale, int32_t* block_idx, void* o, float* lse, void* ws,
                     size_t ws_bytes, void* stream) {
    LaunchDims L;
    if (num_pages < 0) return MSA_ERR_SHAPE;
    int st = check_decode(dims, num_queries, MSA_OP_DECODE, &L,
                          {q_idx, k_idx_pages, q, k_pages, v_pages, block_table, seqlens, block_idx, o, lse}, ws,
                          ws_bytes);
    if (st != MSA_OK || empty(L)) return st;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const msa::DecodeDims d = decode_dims(L, num_queries);
    if (msa::launch_decode_index(d, q_idx, k_idx_pages, seqlens, block_table, num_pages, block_idx, ws, s) !=
        hipSuccess)
        return MSA_ERR_HIP;
    return hip_status(msa::launch_decode_attn(d, q, k_pages, v_pages, seqlens, block_idx, block_table, num_pages,
                                              scale, o, lse, ws, s));
}

}  // extern "C"

extern "C" int msa_decode_noalloc(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx,
                                  const void* q, const void* k, const void* v, const int32_t* seqlens,
                                  float softmax_scale, int32_t* block_idx, void* o, float* lse, void* stream) {
    LaunchDims L;
    int st = check_decode(dims, num_queries, MSA_OP_DECODE, &L, {q_idx, k_idx, q, k, v, seqlens, block_idx, o, lse},
                          nullptr, 0, /*check_ws=*/false);
    if (st != MSA_OK || empty(L)) return st;
    if (decode_ws(L, MSA_OP_DECODE, num_queries) > MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != MSA_OK) return st;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)L.D);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const msa::DecodeDims d = decode_dims(L, num_queries);
    if (msa::launch_decode_index(d, q_idx, k_idx, seqlens, nullptr, 0, block_idx, ws, s) != hipSuccess)
        return MSA_ERR_HIP;
    return hip_status(msa::launch_decode_attn(d, q, k, v, seqlens, block_idx, nullptr, 0, scale, o, lse, ws, s));
}
