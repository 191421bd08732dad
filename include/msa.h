/*
 * msa.h - C ABI of the MSA (MiniMax Sparse Attention) forward hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (MiniMax Sparse Attention (MSA) article on 7minutos.es, sections
 * "¿Qué es MSA?" and "Cómo funcionan las dos ramas"): an index branch scores
 * every causally visible key token with one index-query head per GQA group
 * against one shared index-key head, max-pools the scores over blocks of Bk
 * tokens, and keeps for every (query, group) the k best blocks, the block that
 * holds the query always among them; the main branch then runs exact softmax
 * GQA attention over the causally visible tokens of the kept blocks only. The
 * KL alignment loss (same article, section "Cómo se entrena MSA") compares the
 * group-mean main distribution with the index distribution over those tokens.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, densely
 *    packed (row-major, last dimension contiguous) and 16-byte aligned.
 *  - Batch B, tokens N (queries = keys), groups Hkv (= KV heads = index-query
 *    heads), G query heads per group (Hq = Hkv*G), head dim D, index dim Di,
 *    block size Bk, blocks kept k. Query head h belongs to group h / G.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    on it and outputs are valid once it has completed; the calls never
 *    synchronise and never allocate or free device memory.
 *  - Every status other than MSA_OK and MSA_ERR_HIP is returned before any
 *    device work is enqueued, with no output written. MSA_ERR_HIP reports a
 *    failed launch (the outputs are then unspecified).
 *  - Calls are thread-safe; calls that share a workspace must not overlap.
 *  - Results are deterministic: the same inputs give bitwise the same block
 *    indices, O, LSE, kl_rows (kl_sum too: it is reduced in a fixed order)
 *    and gradients.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 6

#if defined(__GNUC__)
#define MSA_API __attribute__((visibility("default")))
#else
#define MSA_API
#endif

/* Element type of the tensors. MSA_FP8_E4M3 (OCP fp8 e4m3, the variant with no
 * infinities, |x| <= 448) is accepted by msa_index_topk, msa_decode_index_topk
 * and msa_check_block_idx only: q_idx and k_idx in fp8 on the fp8 matrix cores, scores accumulated in
 * fp32 (exact, and the selection bit-exact, for integer-valued inputs).
 * MSA_FP4_E2M1 (OCP fp4 e2m1: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}) is accepted by
 * msa_index_topk and msa_check_block_idx only: q_idx and k_idx hold two values
 * per byte (element 2c in bits 0-3 of byte c, element 2c+1 in bits 4-7), so a
 * row of Di values is Di/2 bytes; the fp4 matrix cores multiply them exactly
 * and accumulate in fp32, which is exact for any such inputs (every product
 * is a multiple of 1/4 below 37, every score below 2^13 in magnitude), so the
 * selection is exact for every fp4 input. The MSA article (7minutos.es, "El
 * codiseño del kernel") names FP4 among the precisions of the open kernel. */
enum msa_dtype { MSA_BF16 = 0, MSA_F32 = 1, MSA_FP8_E4M3 = 2, MSA_FP4_E2M1 = 3 };

/* Selector for msa_workspace_bytes. */
enum msa_op {
    MSA_OP_INDEX = 0, MSA_OP_ATTN = 1, MSA_OP_KL = 2, MSA_OP_FORWARD = 3, MSA_OP_ATTN_BWD = 4, MSA_OP_KL_BWD = 5,
    MSA_OP_DECODE_INDEX = 6, MSA_OP_DECODE_ATTN = 7, MSA_OP_DECODE = 8, MSA_OP_DENSE_ATTN = 9, MSA_OP_DENSE_KL = 10,
    MSA_OP_FUSED_BWD = 11
};

enum msa_status {
    MSA_OK = 0,
    MSA_ERR_NULL = 1,        /* a required pointer is NULL                        */
    MSA_ERR_SHAPE = 2,       /* negative sizes, or a size that overflows indexing */
    MSA_ERR_UNSUPPORTED = 3, /* a size or dtype this build has no kernel for      */
    MSA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned           */
    MSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than msa_workspace_bytes */
    MSA_ERR_HIP = 6,         /* a HIP launch failed                               */
    MSA_ERR_SCRATCH = 7      /* msa_decode_noalloc: more than its scratch memory   */
};

/*
 * Problem sizes. Supported: batch >= 0, seqlen >= 0 (any value; the last block
 * may be partial), kv_heads >= 1, group_size in {1,2,4,8,16,32}, head_dim and
 * index_dim in {64,128}, block_size 128 (also 64 and 256 for the selection,
 * msa_check_block_idx, the attention and KL forward and msa_forward, in bf16
 * or fp32, with topk <= 16 at 256 outside the selection: a 256-token block
 * takes two of the 128-token slots those kernels work in), topk in [1,32],
 * dtype MSA_BF16 or MSA_F32 (MSA_FP8_E4M3 and MSA_FP4_E2M1 for the selection
 * only), causal == 1. batch == 0 or seqlen == 0 is a valid empty problem.
 * The MSA article (7minutos.es, "¿Qué es MSA?") gives 128 as the default block
 * size, not the only one.
 */
typedef struct msa_dims {
    int64_t batch;
    int64_t seqlen;
    int32_t kv_heads;
    int32_t group_size;
    int32_t head_dim;
    int32_t index_dim;
    int32_t block_size;
    int32_t topk;
    int32_t dtype;
    int32_t causal;
} msa_dims;

/*
 * Index branch: block selection.
 * Defined by the MSA article (7minutos.es), "Cómo funcionan las dos ramas"
 * (scores of visible keys, max-pool per block, top-k per query and group, local
 * block always kept) and "El codiseño del kernel" (exp-free top-k on the raw
 * scores); the Flash-MSA article (tech.kuratif.com) sets the local block's
 * score to +inf so the window stays open.
 *
 *   Uses batch, seqlen, kv_heads, index_dim, block_size, topk, dtype and
 *   causal of `dims` (group_size and head_dim are not read).
 *   q_idx     [B, N, Hkv, Di]  index queries, dtype (bf16, fp32, fp8 e4m3, or
 *                              fp4 e2m1 packed as [B, N, Hkv, Di/2] bytes)
 *   k_idx     [B, N, Di]       shared index keys, dtype (fp4: [B, N, Di/2] bytes)
 *   block_idx [B, Hkv, N, k]   int32 OUTPUT. For query i (local block L = i/Bk)
 *             and group g: the block ids j < L with the k-1 largest
 *             m_j = max_{t in block j} <q_idx[b,i,g], k_idx[b,t]> (ties: lower
 *             id first; all of them if fewer than k-1), plus L; written in
 *             ascending order (so L is the last valid entry), padded with -1 to
 *             length k. Scores accumulate in fp32; selection is exact when the
 *             scores are (e.g. integer-valued inputs with |score| < 2^24).
 *   ws        not used (may be NULL; msa_workspace_bytes(.., MSA_OP_INDEX) = 0)
 */
MSA_API int msa_index_topk(const msa_dims* dims, const void* q_idx, const void* k_idx,
                   int32_t* block_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Checks block_idx against the layout msa_index_topk writes, which is the
 * precondition of msa_sparse_attn_fwd(_stages) and msa_kl_align_fwd: for the
 * row of query i (local block L = i/Bk), the first min(k, L+1) entries are
 * strictly ascending block ids in [0, L] with L last, and the other entries
 * are -1. For callers that bring their own selection.
 *
 *   Uses batch, seqlen, kv_heads, block_size, topk, dtype and causal of `dims`.
 *   block_idx [B, Hkv, N, k]  int32
 *   bad_rows  [1] int32 OUTPUT on the device (overwritten): the number of rows
 *             that break the layout (0 for an empty problem).
 */
MSA_API int msa_check_block_idx(const msa_dims* dims, const int32_t* block_idx, int32_t* bad_rows, void* stream);

/*
 * Main branch: block-sparse GQA attention forward.
 * Defined by the MSA article (7minutos.es), "Cómo funcionan las dos ramas":
 * exact scaled-dot-product softmax over the causally visible tokens of the
 * group's kept blocks, each query head with its own query; the Flash-MSA
 * article keeps the LSE of every row for the backward.
 *
 *   Uses every field of `dims` except index_dim.
 *   q         [B, N, Hq, D]   dtype
 *   k, v      [B, N, Hkv, D]  dtype
 *   block_idx [B, Hkv, N, k]  int32, as written by msa_index_topk (per row:
 *             ascending distinct ids <= L, L last, -1 padding; see
 *             msa_check_block_idx). Other contents give unspecified outputs
 *             (the kernels never access memory outside the given buffers).
 *   softmax_scale  sigma in z = sigma * <q, k_t>; <= 0 selects 1/sqrt(D).
 *   o         [B, N, Hq, D]   OUTPUT, dtype: sum_t exp(z_t - LSE) v_t
 *   lse       [B, Hq, N]      OUTPUT, fp32 natural-log log-sum-exp of z_t
 *   ws        device workspace of at least msa_workspace_bytes(dims,
 *             MSA_OP_ATTN) bytes (partial results of the non-local blocks).
 */
MSA_API int msa_sparse_attn_fwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* block_idx, float softmax_scale, void* o, float* lse,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * The attention of msa_sparse_attn_fwd in separately enqueued stages, for
 * callers that time or interleave them. Same arguments and results as
 * msa_sparse_attn_fwd; `stages` is a bitwise OR of
 *   MSA_STAGE_PREPARE   V^T copy and the inversion of block_idx into per-key-
 *                       block query lists (workspace only)
 *   MSA_STAGE_NONLOCAL  every non-local kept block: per-(row, slot) partial
 *                       outputs and LSEs (workspace only)
 *   MSA_STAGE_COMBINE   the local block of every row and the merge of its
 *                       partials: writes o and lse
 * A stage reads what the earlier stages left in `ws`, so for one result the
 * three must run in this order on the same workspace, with unchanged inputs
 * (separate calls are fine). MSA_STAGE_ALL is msa_sparse_attn_fwd. `stages`
 * == 0 or with other bits set is MSA_ERR_UNSUPPORTED.
 */
enum { MSA_STAGE_PREPARE = 1, MSA_STAGE_NONLOCAL = 2, MSA_STAGE_COMBINE = 4, MSA_STAGE_ALL = 7 };
MSA_API int msa_sparse_attn_fwd_stages(const msa_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* block_idx, float softmax_scale, void* o, float* lse,
                        void* ws, size_t ws_bytes, int stages, void* stream);

/*
 * The whole forward hot path in one call: msa_index_topk followed by
 * msa_sparse_attn_fwd on `stream`, with the same arguments and results
 * (block_idx, o and lse are outputs; every field of `dims` is used).
 *   ws        at least msa_workspace_bytes(dims, MSA_OP_FORWARD) bytes.
 */
MSA_API int msa_forward(const msa_dims* dims, const void* q_idx, const void* k_idx, const void* q,
                        const void* k, const void* v, float softmax_scale, int32_t* block_idx,
                        void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Main branch: backward of msa_sparse_attn_fwd over the cached block indices.
 * Defined by the Flash-MSA article (tech.kuratif.com), paragraph on the
 * backward: with the block indices kept from the forward, the backward visits
 * only the selected blocks (linear in N) and uses the forward's LSE; the
 * function differentiated is the forward above (MSA article, "Cómo funcionan
 * las dos ramas"). For the loss <dO, O>, with z_t = sigma <q, k_t> and
 * P_t = exp(z_t - LSE) over the row's selected tokens T:
 *   dV_t = sum over the rows that see t of P_t dO,
 *   dS_t = P_t (<dO, v_t> - <dO, O>),
 *   dQ = sigma sum_t dS_t k_t,  dK_t = sigma sum over those rows of dS_t q.
 *
 *   Uses every field of `dims` except index_dim; dtype MSA_BF16 only (others:
 *   MSA_ERR_UNSUPPORTED).
 *   q, k, v, block_idx, softmax_scale  as for msa_sparse_attn_fwd
 *   o         [B, N, Hq, D]   bf16, the forward output of the same inputs
 *   lse       [B, Hq, N]      fp32, the forward LSE of the same inputs
 *   dout      [B, N, Hq, D]   bf16, gradient of the loss w.r.t. o
 *   dq        [B, N, Hq, D]   OUTPUT bf16
 *   dk, dv    [B, N, Hkv, D]  OUTPUT bf16 (every key is written; keys no row
 *             selects get 0)
 *   ws        at least msa_workspace_bytes(dims, MSA_OP_ATTN_BWD) bytes
 *             (the query rows are processed 65,536 positions at a time: the
 *             window's per-(row, slot) dQ partials and per-work-item dK/dV
 *             partials, fp32 running sums across windows; about 21 GB for
 *             N = 128K, Hkv = 8, G = 8, D = 128, k = 16, 24 GB at N = 1M, Hkv 4).
 * Deterministic: every sum runs in a fixed order. This is msa_fused_bwd's
 * pass without the KL term.
 */
MSA_API int msa_sparse_attn_bwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                                const int32_t* block_idx, const void* o, const float* lse, const void* dout,
                                float softmax_scale, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * KL alignment loss forward.
 * Defined by the MSA article (7minutos.es), "Cómo se entrena MSA": the teacher
 * is the main-branch distribution averaged over the group's heads over the
 * selected tokens, the student the index branch's distribution over the same
 * tokens; the Flash-MSA article computes the loss without materialising the
 * distributions.
 *
 *   q, k, q_idx, k_idx, block_idx  as above
 *   lse       [B, Hq, N] fp32, the main-branch LSE of the same inputs (as
 *             written by msa_sparse_attn_fwd)
 *   softmax_scale  as above; index_scale: student logits are
 *             index_scale * <q_idx, k_idx_t>; <= 0 selects 1/sqrt(Di).
 *   kl_rows   [B, Hkv, N] OUTPUT fp32: sum_t p_t (ln p_t - ln s_t) with
 *             p_t = mean_h exp(z_{h,t} - LSE_h), s_t the student softmax.
 *   kl_sum    [1] OUTPUT fp32 (overwritten): sum of kl_rows, fixed order.
 *   index_lse [B, Hkv, N] optional OUTPUT fp32 (NULL: not written): the
 *             student's natural-log LSE_u = ln sum_t exp(index_scale u_t) per
 *             row, which msa_kl_align_bwd takes.
 *   ws        at least msa_workspace_bytes(dims, MSA_OP_KL) bytes.
 */
MSA_API int msa_kl_align_fwd(const msa_dims* dims, const void* q, const void* k, const void* q_idx,
                     const void* k_idx, const int32_t* block_idx, const float* lse,
                     float softmax_scale, float index_scale, float* kl_rows, float* kl_sum,
                     float* index_lse, void* ws, size_t ws_bytes, void* stream);

/*
 * KL alignment loss backward: gradients of L = sum over rows of
 * w_row * KL_row, w_row = kl_weight * (dkl_rows ? dkl_rows[row] : 1), with
 * respect to q_idx and k_idx.
 * Defined by the MSA article (7minutos.es), "Cómo se entrena MSA": the KL loss
 * trains the index branch toward the main branch's attention pattern and the
 * gradient is stopped at the index branch's input, so the teacher is held
 * fixed and nothing flows into q, k; the Flash-MSA article computes the proxy
 * gradient from the cached block indices. With u_t = <q_idx, k_idx_t>,
 * s the student softmax and p the teacher of msa_kl_align_fwd:
 *   dU_t = w_row index_scale (s_t - p_t),
 *   dq_idx[b,i,g] = sum_t dU_t k_idx_t,  dk_idx[b,t] = sum over the rows of
 *   every group that see t of dU_t q_idx[b,i,g].
 *
 *   Uses every field of `dims`; dtype MSA_BF16 only (others:
 *   MSA_ERR_UNSUPPORTED).
 *   q, k, q_idx, k_idx, block_idx, lse, softmax_scale, index_scale  as for
 *             msa_kl_align_fwd (the same values)
 *   index_lse [B, Hkv, N] fp32, as written by msa_kl_align_fwd
 *   dkl_rows  [B, Hkv, N] fp32 row weights, or NULL for all ones
 *   dq_idx    [B, N, Hkv, Di] OUTPUT bf16
 *   dk_idx    [B, N, Di]      OUTPUT bf16 (every key written; 0 if unseen)
 *   ws        at least msa_workspace_bytes(dims, MSA_OP_KL_BWD) bytes (65,536
 *             query positions at a time: the teacher p per (row, slot, key),
 *             dq_idx and dk_idx partials; about 8 GB at N = 128K, Hkv = 8,
 *             11 GB at N = 1M, Hkv = 4).
 * Deterministic: every sum runs in a fixed order. This is msa_fused_bwd's
 * pass without the main-branch gradients (S and P only, for the teacher).
 */
MSA_API int msa_kl_align_bwd(const msa_dims* dims, const void* q, const void* k, const void* q_idx,
                             const void* k_idx, const int32_t* block_idx, const float* lse,
                             const float* index_lse, float softmax_scale, float index_scale,
                             const float* dkl_rows, float kl_weight, void* dq_idx, void* dk_idx, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Fused backward of both branches: msa_sparse_attn_bwd's dq, dk, dv (main
 * branch, loss <dO, O>) and msa_kl_align_bwd's dq_idx, dk_idx (KL term, loss
 * sum_rows w_row KL_row, teacher held fixed) from one pass over the selected
 * blocks, in which the main-branch scores and probabilities are computed once
 * and serve both the main gradient and the teacher.
 * Defined by the Flash-MSA article (tech.kuratif.com), paragraph on the
 * backward (proxy and main attention gradients fused, over the cached block
 * indices, linear in N) and "Accelerating Million-Token Training with Sparse
 * Attention Kernels" (DeepHorus: the fused backward is what makes training at
 * a million tokens possible); the functions differentiated are those of
 * msa_sparse_attn_fwd and msa_kl_align_fwd (MSA article, 7minutos.es).
 *
 *   Uses every field of `dims`; dtype MSA_BF16 and block_size 128 only.
 *   q, k, v, q_idx, k_idx, block_idx, softmax_scale, index_scale as for the
 *             forward calls; o, lse: msa_sparse_attn_fwd's outputs; index_lse:
 *             msa_kl_align_fwd's; dout [B, N, Hq, D] bf16; dkl_rows, kl_weight
 *             as for msa_kl_align_bwd (row weights w_row = kl_weight *
 *             (dkl_rows ? dkl_rows[row] : 1)).
 *   dq [B, N, Hq, D], dk, dv [B, N, Hkv, D], dq_idx [B, N, Hkv, Di],
 *   dk_idx [B, N, Di]  OUTPUTS bf16 (every element written; keys no row
 *             selects get 0).
 *   ws        at least msa_workspace_bytes(dims, MSA_OP_FUSED_BWD) bytes. The
 *             query rows are processed 65,536 positions at a time, so the
 *             per-(row, slot) partials never exceed one such window: about
 *             30 GB for N = 1,048,576, Hkv = 4, G = 8, D = Di = 128, k = 16.
 * Deterministic: every sum runs in a fixed order.
 */
MSA_API int msa_fused_bwd(const msa_dims* dims, const void* q, const void* k, const void* v, const void* q_idx,
                          const void* k_idx, const int32_t* block_idx, const void* o, const float* lse,
                          const float* index_lse, const void* dout, float softmax_scale, float index_scale,
                          const float* dkl_rows, float kl_weight, void* dq, void* dk, void* dv, void* dq_idx,
                          void* dk_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Dense causal GQA attention forward: the main branch with every causally
 * visible key kept.
 * Defined by the MSA article (7minutos.es), "Cómo se entrena MSA": during the
 * indexer warm-up both branches attend to everything; this is the main
 * branch's output then, i.e. msa_sparse_attn_fwd's result when every row keeps
 * all of its visible blocks (which that entry point cannot be given once the
 * blocks outnumber topk <= 32).
 *
 *   Uses batch, seqlen, kv_heads, group_size, head_dim, block_size, dtype and
 *   causal of `dims` (topk and index_dim are not read).
 *   q [B, N, Hq, D], k, v [B, N, Hkv, D], softmax_scale, o [B, N, Hq, D] and
 *   lse [B, Hq, N] as for msa_sparse_attn_fwd, with T_i = {0 .. i}.
 *   ws        at least msa_workspace_bytes(dims, MSA_OP_DENSE_ATTN) bytes (a
 *             per-block transposed copy of V, the size of v).
 */
MSA_API int msa_dense_attn_fwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                               float softmax_scale, void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * KL alignment loss forward over every causally visible token: the index
 * branch's side of the warm-up (MSA article, "Cómo se entrena MSA": during
 * the first iterations both branches attend to everything and the indexer
 * learns from the KL loss before it routes). msa_kl_align_fwd's loss with
 * T_i = {0 .. i} for every row.
 *
 *   Uses every field of `dims` except topk.
 *   q, k, q_idx, k_idx, softmax_scale, index_scale, kl_rows, kl_sum and
 *   index_lse as for msa_kl_align_fwd;
 *   lse       [B, Hq, N] fp32, the dense main-branch LSE of the same inputs (as
 *             written by msa_dense_attn_fwd).
 *   ws        at least msa_workspace_bytes(dims, MSA_OP_DENSE_KL) bytes (the
 *             fixed-order reduction's partial sums).
 */
MSA_API int msa_dense_kl_align_fwd(const msa_dims* dims, const void* q, const void* k, const void* q_idx,
                                   const void* k_idx, const float* lse, float softmax_scale, float index_scale,
                                   float* kl_rows, float* kl_sum, float* index_lse, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * Decoding: R >= 1 new queries per sequence against a cache (one decode step,
 * or several tokens appended at once, e.g. speculative drafts).
 * Defined by the same passages as msa_index_topk and msa_sparse_attn_fwd (MSA
 * article on 7minutos.es, "Cómo funcionan las dos ramas" and "El codiseño del
 * kernel"): sequence b holds n_b = seqlens[b] cached tokens, positions
 * 0 .. n_b - 1 with the new tokens last, and its r-th new query is position
 * i = n_b - R + r, so the selection and the attention are exactly those of the
 * forward's row i; the per-layer state a sparse layer keeps is the block ids
 * (Flash-MSA article on tech.kuratif.com, block-wise sparsity).
 *
 * `dims`: batch = B sequences, seqlen = C, the cache capacity in tokens per
 * sequence; other fields as above (dtype MSA_BF16 or MSA_F32; the selection
 * calls also take MSA_FP8_E4M3 for an fp8 index cache, scores accumulated in
 * fp32 as in msa_index_topk). num_queries = R >= 1, with B * R <= 65535 and
 * B * ceil(R * Hkv / 32) <= 65535 (MSA_ERR_SHAPE otherwise). Cache slots at or
 * past n_b are never read.
 *   seqlens   [B] int32 on the DEVICE (read by the kernels, so a step can be
 *             enqueued without a host round trip). A sequence whose length is
 *             outside [1, C], and a query whose position is negative, is not
 *             an error: its block ids are -1, O = 0 and LSE = -inf.
 * Tensor layouts (for R = 1 they are the same bytes as [B, Hkv, Di], [B, Hq, D],
 * [B, Hkv, k] and [B, Hq]):
 *   q_idx     [B, R, Hkv, Di]  the new tokens' index queries
 *   k_idx     [B, C, Di]       index-key cache
 *   q         [B, R, Hq, D]    the new tokens' queries
 *   k, v      [B, C, Hkv, D]   key and value caches
 *   block_idx [B, Hkv, R, k]   int32, the layout of msa_index_topk's rows
 *             (ascending kept ids, local block i / Bk last, -1 padding),
 *             bit-identical to the forward's rows; an OUTPUT of the selection
 *             calls, an input of the attention call (ids < 0 or past the
 *             query's block are skipped without any read; other layouts give
 *             unspecified outputs but never an access outside the buffers).
 *   o         [B, R, Hq, D]    OUTPUT, dtype
 *   lse       [B, Hq, R]       OUTPUT fp32, natural log
 *   ws        at least msa_decode_workspace_bytes(dims, op, R) bytes (op
 *             MSA_OP_DECODE_INDEX: block scores; MSA_OP_DECODE_ATTN: one fp32
 *             partial output and LSE per kept block and head; MSA_OP_DECODE:
 *             the larger of the two, as the stages run one after the other).
 */
MSA_API int msa_decode_index_topk(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx,
                                  const int32_t* seqlens, int32_t* block_idx, void* ws, size_t ws_bytes,
                                  void* stream);
MSA_API int msa_decode_attn(const msa_dims* dims, int32_t num_queries, const void* q, const void* k, const void* v,
                            const int32_t* seqlens, const int32_t* block_idx, float softmax_scale, void* o,
                            float* lse, void* ws, size_t ws_bytes, void* stream);
/* msa_decode_index_topk then msa_decode_attn on `stream`. */
MSA_API int msa_decode(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx,
                       const void* q, const void* k, const void* v, const int32_t* seqlens, float softmax_scale,
                       int32_t* block_idx, void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Decoding against a paged cache: the same computation as the three calls
 * above, with each cache held as a pool of 128-token pages and a block table
 * naming the page of every block of every sequence (the MSA block, the unit the
 * index branch selects, is the page: Flash-MSA article, block-wise sparsity).
 *   k_idx_pages [P, 128, Di], k_pages and v_pages [P, 128, Hkv, D]: pools of
 *             P = num_pages pages (dtype as for the contiguous calls).
 *   block_table [B, ceil(C / 128)] int32 on the DEVICE: page of block j of
 *             sequence b (C = dims.seqlen, the capacity). Entries of blocks
 *             at or past ceil(n_b / 128) are not read. An entry outside
 *             [0, num_pages) is not an error: that block is never read, it
 *             scores -inf in the selection and contributes no tokens.
 *   num_pages < 0 is MSA_ERR_SHAPE. Other arguments, outputs and workspaces
 *   as for the contiguous calls.
 */
MSA_API int msa_decode_paged_index_topk(const msa_dims* dims, int32_t num_queries, const void* q_idx,
                                        const void* k_idx_pages, const int32_t* block_table, int32_t num_pages,
                                        const int32_t* seqlens, int32_t* block_idx, void* ws, size_t ws_bytes,
                                        void* stream);
MSA_API int msa_decode_paged_attn(const msa_dims* dims, int32_t num_queries, const void* q, const void* k_pages,
                                  const void* v_pages, const int32_t* block_table, int32_t num_pages,
                                  const int32_t* seqlens, const int32_t* block_idx, float softmax_scale, void* o,
                                  float* lse, void* ws, size_t ws_bytes, void* stream);
MSA_API int msa_decode_paged(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx_pages,
                             const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                             int32_t num_pages, const int32_t* seqlens, float softmax_scale, int32_t* block_idx,
                             void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Decoding without any allocation: msa_decode with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Arguments, results
 * and errors are those of msa_decode (every output bitwise the same); the
 * scratch memory msa_decode takes from `ws` is instead a fixed array of
 * MSA_NOALLOC_SCRATCH_BYTES bytes in the library's device memory, one per GPU,
 * held until the process ends. A problem whose decode workspace
 * (msa_decode_workspace_bytes(dims, MSA_OP_DECODE, num_queries)) is larger is
 * refused with MSA_ERR_SCRATCH before any launch (64 MiB holds, e.g., 120
 * sequences at k = 16, Hkv = 8, G = 8, D = 128). The call allocates and frees
 * nothing. Every call on a GPU uses that GPU's one array: calls that overlap
 * on one GPU (other streams, other threads) race and give unspecified
 * results. The first call on each device (the calling thread's current
 * device, which must be the stream's) looks the array's device address up
 * once; MSA_ERR_HIP if that fails.
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
MSA_API int msa_decode_noalloc(const msa_dims* dims, int32_t num_queries, const void* q_idx, const void* k_idx,
                               const void* q, const void* k, const void* v, const int32_t* seqlens,
                               float softmax_scale, int32_t* block_idx, void* o, float* lse, void* stream);

/* Workspace bytes of a decode call with num_queries new queries per sequence
 * (op MSA_OP_DECODE_INDEX, MSA_OP_DECODE_ATTN or MSA_OP_DECODE); 0 if the sizes
 * are invalid. msa_workspace_bytes gives the same for num_queries = 1. */
MSA_API size_t msa_decode_workspace_bytes(const msa_dims* dims, int op, int32_t num_queries);

/* Workspace bytes the given entry point needs for these sizes; 0 if the sizes
 * are invalid or the op needs none. Pure host arithmetic. */
MSA_API size_t msa_workspace_bytes(const msa_dims* dims, int op);

/* Static description of a status code (never NULL). */
MSA_API const char* msa_strerror(int status);

/* MSA_ABI_VERSION of the library. */
MSA_API int msa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
