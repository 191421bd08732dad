// Main branch of MSA: exact softmax GQA attention over the causally visible
// tokens of each group's kept blocks, writing O and the per-row LSE (gfx950).
//
// Method: MiniMax Sparse Attention (MSA) article on 7minutos.es, section "Cómo
// funcionan las dos ramas" (gather the causally visible tokens of the selected
// blocks; scaled-dot-product softmax restricted to them; every query head of a
// group shares the group's block set); the Flash-MSA article (tech.kuratif.com)
// keeps the LSE for the backward pass.
//
// Data flow on the GPU (one stream, no host round trip):
//   1. invert the selection: for every (batch, group, key block j) the list of
//      query rows that kept j as a NON-local block (count -> scan -> scatter,
//      then fixed-size work items);
//   2. attn_nonlocal: one work-group per work item stages K_j and V_j^T in LDS
//      once and streams the item's query rows through them in 32-row tiles
//      (32/G positions x G heads). It writes, per (row, slot), the block's
//      normalised partial output and its LSE. Iterating over key blocks instead
//      of queries is what gives the K/V loads reuse (the MSA article's kernel
//      section makes the same argument about arithmetic intensity);
//   3. attn_local_combine: one work-group per (batch, query block, group) does
//      the causal local block for all 128*G rows from LDS-resident K/V, then
//      merges the row's partials in slot order into O and LSE.
// Every row's result is computed independently of the other rows in its tile,
// so the (atomic, unordered) list order does not change any output bit.
//
// Matrix-core layout: S^T = K Q^T (A = keys from LDS, B = query rows from
// VGPRs) puts one query row in each lane, so the row max/sum need one
// half-wave swap. P^T then feeds O^T = V^T P^T directly as the B operand: the
// lane's 8 probabilities of a 16-key slice are keys {4h..4h+3, 8+4h..8+4h+3}
// (h = lane/32), and the A operand reads V^T with the same key assignment.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"

namespace msa {

// ------------------------------------------------------- non-local blocks --

// Partial layout, per (row (b,g,i), slot s < k-1): po[.][G][D] with each 32-wide
// slice of D stored lane-major (slot dt*32 + 16*h + r holds
// d = dt*32 + 8*(r/4) + 4*h + r%4), plse[.][G] natural-log LSE.
template <typename T, int D, int G>
__global__ __launch_bounds__(256, 1) void attn_nonlocal_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ list, const int4* __restrict__ items, const int32_t* __restrict__ total_items,
    T* __restrict__ po, float* __restrict__ plse, int N, int Hkv, int nb, int KP, float scale_log2) {
    using KV = KVTile<T, D>;
    constexpr int PPT = 32 / G;   // positions per 32-row tile
    __shared__ __align__(16) unsigned char lds[KV::BYTES];

    // Items of one XCD are contiguous (blocks are dealt to the 8 XCDs round-robin).
    const int total = total_items[0];
    const int per_xcd = (total + 7) / 8;
    const int slot_in_xcd = blockIdx.x / 8;
    if (slot_in_xcd >= per_xcd) return;
    const int item_id = (blockIdx.x % 8) * per_xcd + slot_in_xcd;
    if (item_id >= total) return;
    const int4 it = items[item_id];
    const int key = it.x, start = it.y, count = it.z;
    const int j = key % nb;
    const int g = (key / nb) % Hkv;
    const int b = key / (nb * Hkv);
    const int Hq = Hkv * G;

    const size_t kv_row = (size_t)Hkv * D;
    const size_t kv_off = ((size_t)b * N + (size_t)j * kBlock) * kv_row + (size_t)g * D;
    KV::stage(lds, k + kv_off, v + kv_off, kv_row, kBlock);
    __syncthreads();

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int hh = col % G;
    for (int base = w * PPT; base < count; base += 4 * PPT) {
        const int e = base + col / G;
        const bool valid = e < count;
        const int packed = list[start + (valid ? e : 0)];
        const int i = packed >> 5, slot = packed & 31;
        Op8<T> bq[D / 16];
        load_q_op<T, D>(bq, q + ((size_t)b * N + i) * Hq * D + (size_t)(g * G + hh) * D, valid, half);

        floatx16 s[4];
        tile_scores<T, D>(s, bq, lds, col, half);
        float mz, l;
        tile_softmax(s, scale_log2, mz, l);
        floatx16 o[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
        tile_pv<T, D>(o, s, lds, col, half);

        if (valid) {
            const float inv = 1.f / l;
            const size_t pidx = (((size_t)b * Hkv + g) * N + i) * KP + slot;
            T* dst = po + (pidx * G + hh) * D + 16 * half;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                if constexpr (sizeof(T) == 2) {
                    uint32_t wv[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        wv[r] = (uint32_t)f32_to_bf16(o[dt][2 * r] * inv) |
                                ((uint32_t)f32_to_bf16(o[dt][2 * r + 1] * inv) << 16);
                    uint4* d4 = reinterpret_cast<uint4*>(dst + dt * 32);
                    d4[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                    d4[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
                } else {
                    float4* d4 = reinterpret_cast<float4*>(dst + dt * 32);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        d4[r] = make_float4(o[dt][4 * r] * inv, o[dt][4 * r + 1] * inv,
                                            o[dt][4 * r + 2] * inv, o[dt][4 * r + 3] * inv);
                }
            }
            if (half == 0) plse[pidx * G + hh] = (mz + __log2f(l)) * 0.69314718055994531f;
        }
    }
}

// ------------------------------------------------ local block + combination --

template <typename T, int D, int G>
__global__ __launch_bounds__(256, 1) void attn_local_combine_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ po, const float* __restrict__ plse, T* __restrict__ o, float* __restrict__ lse,
    int B, int N, int Hkv, int nb, int topk, int KP, float scale_log2) {
    using KV = KVTile<T, D>;
    __shared__ __align__(16) unsigned char lds[KV::BYTES];
    const int g = blockIdx.x % Hkv;
    const int b = (blockIdx.x / Hkv) % B;
    const int qb = blockIdx.x / (Hkv * B);
    const int Hq = Hkv * G;
    const int q0 = qb * kBlock;
    const int valid_keys = min(kBlock, N - q0);

    const size_t kv_row = (size_t)Hkv * D;
    const size_t kv_off = ((size_t)b * N + (size_t)q0) * kv_row + (size_t)g * D;
    KV::stage(lds, k + kv_off, v + kv_off, kv_row, valid_keys);
    __syncthreads();

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int hh = col % G;
    const int h = g * G + hh;
    const int nnl = min(topk - 1, qb);         // non-local slots of every row here
    constexpr float kLog2e = 1.4426950408889634f;

    for (int tile = w; tile < kBlock * G / 32; tile += 4) {
        const int p = (tile * 32 + col) / G;   // position within the block
        const int i = q0 + p;
        const bool valid = i < N;
        Op8<T> bq[D / 16];
        load_q_op<T, D>(bq, q + ((size_t)b * N + (valid ? i : q0)) * Hq * D + (size_t)h * D, valid, half);

        floatx16 s[4];
        tile_scores<T, D>(s, bq, lds, col, half);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                if (key > p) s[kt][r] = -__builtin_inff();
            }
        }
        float mz, l;
        tile_softmax(s, scale_log2, mz, l);
        floatx16 acc[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
        tile_pv<T, D>(acc, s, lds, col, half);

        // Merge with the non-local partials (log2 domain), slot order.
        const float lse_loc = mz + __log2f(l);
        const size_t prow = (((size_t)b * Hkv + g) * N + (valid ? i : q0)) * KP;
        float mx = lse_loc;
        for (int sl = 0; sl < nnl; ++sl) mx = fmaxf(mx, plse[(prow + sl) * G + hh] * kLog2e);
        float tot = exp2f(lse_loc - mx);
        for (int sl = 0; sl < nnl; ++sl) tot += exp2f(plse[(prow + sl) * G + hh] * kLog2e - mx);
        const float lse_all = mx + __log2f(tot);
        const float wl = exp2f(lse_loc - lse_all) / l;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= wl;
        }
        for (int sl = 0; sl < nnl; ++sl) {
            const float ws = exp2f(plse[(prow + sl) * G + hh] * kLog2e - lse_all);
            const T* src = po + ((prow + sl) * G + hh) * D + 16 * half;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                if constexpr (sizeof(T) == 2) {
                    const uint4* s4 = reinterpret_cast<const uint4*>(src + dt * 32);
                    const uint4 x0 = s4[0], x1 = s4[1];
                    const uint32_t wv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        acc[dt][2 * r] += ws * bf16_to_f32((bf16_t)(wv[r] & 0xffffu));
                        acc[dt][2 * r + 1] += ws * bf16_to_f32((bf16_t)(wv[r] >> 16));
                    }
                } else {
                    const float4* s4 = reinterpret_cast<const float4*>(src + dt * 32);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float4 x = s4[r];
                        acc[dt][4 * r] += ws * x.x;
                        acc[dt][4 * r + 1] += ws * x.y;
                        acc[dt][4 * r + 2] += ws * x.z;
                        acc[dt][4 * r + 3] += ws * x.w;
                    }
                }
            }
        }
        if (valid) {
            T* dst = o + ((size_t)b * N + i) * Hq * D + (size_t)h * D;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    T* d4 = dst + dt * 32 + 8 * rq + 4 * half;
                    if constexpr (sizeof(T) == 2) {
                        const uint32_t a0 = (uint32_t)f32_to_bf16(acc[dt][4 * rq]) |
                                            ((uint32_t)f32_to_bf16(acc[dt][4 * rq + 1]) << 16);
                        const uint32_t a1 = (uint32_t)f32_to_bf16(acc[dt][4 * rq + 2]) |
                                            ((uint32_t)f32_to_bf16(acc[dt][4 * rq + 3]) << 16);
                        *reinterpret_cast<uint2*>(d4) = make_uint2(a0, a1);
                    } else {
                        *reinterpret_cast<float4*>(d4) = make_float4(acc[dt][4 * rq], acc[dt][4 * rq + 1],
                                                                      acc[dt][4 * rq + 2], acc[dt][4 * rq + 3]);
                    }
                }
            }
            if (half == 0) lse[((size_t)b * Hq + h) * N + i] = lse_all * 0.69314718055994531f;
        }
    }
}

// -------------------------------------------------------------------- host --

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

AttnWorkspace attn_workspace_layout(const LaunchDims& d) {
    AttnWorkspace w{};
    w.lists = list_layout(d, 0);
    const size_t es = d.dtype == 0 ? 2 : 4;
    size_t off = w.lists.end;
    w.po = off;    off = align_up(off + w.lists.max_entries * d.G * d.D * es);
    w.plse = off;  off = align_up(off + w.lists.max_entries * d.G * 4);
    w.bytes = w.lists.has_nonlocal ? off : 0;
    return w;
}

template <typename T, int D, int G>
static hipError_t launch_attn_t(const LaunchDims& d, const void* q, const void* k, const void* v,
                                const int32_t* block_idx, float scale, void* o, float* lse,
                                unsigned char* ws, hipStream_t st) {
    const AttnWorkspace L = attn_workspace_layout(d);
    const float scale_log2 = scale * 1.4426950408889634f;
    const int KP = d.k > 1 ? d.k - 1 : 1;
    const T* tq = static_cast<const T*>(q);
    const T* tk = static_cast<const T*>(k);
    const T* tv = static_cast<const T*>(v);
    T* po = nullptr;
    float* plse = nullptr;
    if (L.lists.has_nonlocal) {
        launch_build_lists(d, block_idx, ws, L.lists, st);
        const int4* items = reinterpret_cast<const int4*>(ws + L.lists.items);
        const int32_t* list = reinterpret_cast<const int32_t*>(ws + L.lists.list);
        const int32_t* total = reinterpret_cast<const int32_t*>(ws + L.lists.total);
        po = reinterpret_cast<T*>(ws + L.po);
        plse = reinterpret_cast<float*>(ws + L.plse);
        const size_t grid = (L.lists.max_items + 7) / 8 * 8;
        hipLaunchKernelGGL((attn_nonlocal_kernel<T, D, G>), dim3((unsigned)grid), dim3(256), 0, st, tq, tk, tv,
                           list, items, total, po, plse, d.N, d.Hkv, d.nb, KP, scale_log2);
    }
    hipLaunchKernelGGL((attn_local_combine_kernel<T, D, G>), dim3((unsigned)(d.nb * d.B * d.Hkv)), dim3(256), 0, st,
                       tq, tk, tv, po, plse, static_cast<T*>(o), lse, d.B, d.N, d.Hkv, d.nb,
                       L.lists.has_nonlocal ? d.k : 1, KP, scale_log2);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_d(const LaunchDims& d, const void* q, const void* k, const void* v,
                                const int32_t* bi, float scale, void* o, float* lse, unsigned char* ws,
                                hipStream_t st) {
    switch (d.G) {
        case 1: return launch_attn_t<T, D, 1>(d, q, k, v, bi, scale, o, lse, ws, st);
        case 2: return launch_attn_t<T, D, 2>(d, q, k, v, bi, scale, o, lse, ws, st);
        case 4: return launch_attn_t<T, D, 4>(d, q, k, v, bi, scale, o, lse, ws, st);
        case 8: return launch_attn_t<T, D, 8>(d, q, k, v, bi, scale, o, lse, ws, st);
        case 16: return launch_attn_t<T, D, 16>(d, q, k, v, bi, scale, o, lse, ws, st);
        default: return launch_attn_t<T, D, 32>(d, q, k, v, bi, scale, o, lse, ws, st);
    }
}

hipError_t launch_sparse_attn(const LaunchDims& d, const void* q, const void* k, const void* v,
                              const int32_t* block_idx, float scale, void* o, float* lse, void* ws,
                              hipStream_t st) {
    if (d.B == 0 || d.N == 0) return hipSuccess;
    unsigned char* w = static_cast<unsigned char*>(ws);
    if (d.dtype == 0)
        return d.D == 128 ? launch_attn_d<bf16_t, 128>(d, q, k, v, block_idx, scale, o, lse, w, st)
                          : launch_attn_d<bf16_t, 64>(d, q, k, v, block_idx, scale, o, lse, w, st);
    return d.D == 128 ? launch_attn_d<float, 128>(d, q, k, v, block_idx, scale, o, lse, w, st)
                      : launch_attn_d<float, 64>(d, q, k, v, block_idx, scale, o, lse, w, st);
}

}  // namespace msa
