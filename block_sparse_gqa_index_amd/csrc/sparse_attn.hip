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

// ------------------------------------------------------------- V^T copy --

// V [B, N, Hkv, D] -> V^T [B, Hkv, nb, D, 128]: one key block of one group per
// work-group. Within every group of 16 keys the positions are permuted so that
// position 8h + e holds key 8*(e/4) + 4h + e%4 (h = 0, 1; e = 0..7): the keys a
// lane of half-wave h feeds to the P V product for that 16-key slice (the
// accumulator layout of the scores) then sit in one contiguous 16-byte chunk.
// A thread transposes one 16-key x (16 bytes of dims) tile in registers. Keys
// past N are written as zeros.
template <typename T, int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T* __restrict__ v, T* __restrict__ vt, int N, int Hkv,
                                                          int nb) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr int KG = kBlock / 16, DC = D / EPC;
    const int j = blockIdx.x % nb;
    const int bg = blockIdx.x / nb;
    const int g = bg % Hkv, b = bg / Hkv;
    T* dst = vt + (size_t)blockIdx.x * D * kBlock;
    for (int item = threadIdx.x; item < KG * DC; item += blockDim.x) {
        const int dc = item % DC, kg = item / DC;
        u32x4 x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = j * kBlock + kg * 16 + e;
            x[e] = u32x4{0u, 0u, 0u, 0u};
            if (key < N)
                x[e] = *reinterpret_cast<const u32x4*>(v + (((size_t)b * N + key) * Hkv + g) * D + dc * EPC);
        }
#pragma unroll
        for (int dd = 0; dd < EPC; ++dd) {
            T* row = dst + (size_t)(dc * EPC + dd) * kBlock + kg * 16;
            if constexpr (EPC == 8) {   // bf16: chunk h holds keys 4h..4h+3, 8+4h..8+4h+3
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    u32x4 y;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const int k0 = 8 * (w / 2) + 4 * h + 2 * (w % 2);
                        const uint32_t lo = (x[k0][dd / 2] >> (16 * (dd % 2))) & 0xffffu;
                        const uint32_t hi = (x[k0 + 1][dd / 2] >> (16 * (dd % 2))) & 0xffffu;
                        y[w] = lo | (hi << 16);
                    }
                    *reinterpret_cast<u32x4*>(row + 8 * h) = y;
                }
            } else {                    // fp32: 4-key chunk q holds keys 8*(q%2) + 4*(q/2) + 0..3
#pragma unroll
                for (int qc = 0; qc < 4; ++qc) {
                    u32x4 y;
                    const int k0 = 8 * (qc % 2) + 4 * (qc / 2);
#pragma unroll
                    for (int w = 0; w < 4; ++w) y[w] = x[k0 + w][dd];
                    *reinterpret_cast<u32x4*>(row + 4 * qc) = y;
                }
            }
        }
    }
}

// ------------------------------------------------------- non-local blocks --

// Partial layout, per (row (b,g,i), slot s < k-1): po[.][G][D] with each 32-wide
// slice of D stored lane-major (slot dt*32 + 16*h + r holds
// d = dt*32 + 8*(r/4) + 4*h + r%4), plse[.][G] natural-log LSE.
// Partial O of one (row, slot): G heads x D values, stored as 16-byte pieces
// interleaved across the 2G lanes (head hh, half h) that hold them in the
// matrix-core output layout: piece q of lane (hh, h) sits at byte
// 16 * (q * 2G + 2 * hh + h). One store (or load) instruction then covers 2G
// consecutive pieces per position, i.e. whole cache lines, instead of 16
// bytes in each of 2G different head rows. The pieces are stored
// non-temporally: they are read back only by the merge kernel, and written
// through the caches they would evict the query rows that the other items of
// the same window gather again. Piece q of a lane holds its values
// 8q..8q+7 (bf16) or 4q..4q+3 (fp32) in accumulator order: for each 32-wide
// slice dt of D, values r = 0..15 are d = dt*32 + 8*(r/4) + 4*h + r%4.
template <typename T, int D, int G>
__device__ __forceinline__ u32x4* partial_piece(T* region, int q, int hh, int half) {
    return reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(region) + 16 * (q * 2 * G + 2 * hh + half));
}

template <typename T, int D, int G>
__device__ __forceinline__ void store_partial(T* __restrict__ po, float* __restrict__ plse, size_t pidx, int hh,
                                              int half, const floatx16 (&o)[D / 32], float mz, float l) {
    const float inv = 1.f / l;
    T* region = po + pidx * G * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        if constexpr (sizeof(T) == 2) {
            u32x4 w0, w1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                w0[r] = pack_bf16x2(o[dt][2 * r] * inv, o[dt][2 * r + 1] * inv);
                w1[r] = pack_bf16x2(o[dt][8 + 2 * r] * inv, o[dt][8 + 2 * r + 1] * inv);
            }
            __builtin_nontemporal_store(w0, partial_piece<T, D, G>(region, 2 * dt, hh, half));
            __builtin_nontemporal_store(w1, partial_piece<T, D, G>(region, 2 * dt + 1, hh, half));
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = __float_as_uint(o[dt][4 * r + e] * inv);
                __builtin_nontemporal_store(x, partial_piece<T, D, G>(region, 4 * dt + r, hh, half));
            }
        }
    }
    if (half == 0) plse[pidx * G + hh] = (mz + __log2f(l)) * 0.69314718055994531f;
}

// Keys of the 128-key block a row keeps when its selection was made with
// 64-token blocks: bit 0 of the entry's mask keeps keys 0-63 (key tiles 0-1),
// bit 1 keys 64-127 (tiles 2-3).
__device__ __forceinline__ void mask_halves(floatx16 (&s)[4], int m) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        const bool keep = (m >> (kt >> 1)) & 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = keep ? s[kt][r] : -__builtin_inff();
    }
}

// One 32-row tile of a non-local work item: the lane's row is list entry `e`
// (position << 5 | slot); scores against the staged block, softmax, P V and
// the partial store (to the spare partial for the padding rows past the
// item's end). HM: the entry keeps only the halves its mask byte names
// (64-token selections).
template <typename T, int D, int G, bool HM>
__device__ __forceinline__ void nonlocal_tile(const Op8<T> (&qop)[D / 16], int e, bool valid,
                                              const unsigned char* lds, T* __restrict__ po,
                                              float* __restrict__ plse, int b, int g, int N, int Hkv, int KP,
                                              const uint8_t* __restrict__ hmask, float scale_log2, int hh, int col,
                                              int half, size_t spare) {
    floatx16 s[4];
    tile_scores<T, D>(s, qop, lds, col, half);
    if constexpr (HM) mask_halves(s, hmask[(((size_t)b * Hkv + g) * N + (e >> 5)) * (KP + 1) + (e & 31)]);
    float mz, l;
    tile_softmax(s, scale_log2, mz, l);
    floatx16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
    tile_pv<T, D>(o, s, lds, col, half);
    // Padding rows store to the spare partial so the store is unconditional
    // (the next tile's waits then count it in order with the loads).
    const size_t pidx = valid ? (((size_t)b * Hkv + g) * N + (e >> 5)) * KP + (e & 31) : spare;
    store_partial<T, D, G>(po, plse, pidx, hh, half, o, mz, l);
}

// Pipelined form of a bf16 tile. A tile reads its A operands from the
// LDS-resident block in one fixed order: the K operands of S^T (D/16 slices x
// 4 key tiles), then the V^T operands of O^T (D/32 dim tiles x 8 key slices).
// Every tile of a work item repeats that order, so the operands go through an
// 8-register ring loaded 6 products ahead, across the softmax and across tiles.
template <int D>
struct TileOps {
    static constexpr int NS = (D / 16) * 4, NP = 8 * (D / 32), N = NS + NP;
    static constexpr int RING = 8, PF = 6;
    static_assert(N % RING == 0, "the ring must tile the operand sequence");
};

template <int D>
__device__ __forceinline__ void tile_op(Op8<bf16_t>& a, const unsigned char* lds, int n, int col, int half) {
    using O = TileOps<D>;
    using KS = SwzTile<bf16_t, D>;
    if (n < O::NS) {
        KS::load8(a, lds, (n % 4) * 32 + col, 16 * (n / 4) + 8 * half);
    } else {
        const int m = n - O::NS;
        load_vt_op<bf16_t>(a, lds + kBlock * KS::ROWB, (m / 8) * 32 + col, m % 8, half);
    }
}

// One 32-row bf16 tile: S^T, softmax, then O^T one 32-dim tile at a time over
// the 8 key slices (the probabilities packed once as the B operands), each dim
// tile's normalised partial stored while the next one is on the matrix cores.
// Rows past the item's end store to the spare partial, so every tile issues the
// same stores; both half-waves hold the row's LSE and write it (same value).
template <int D, int G, bool HM>
__device__ __forceinline__ void nonlocal_tile_pipe(Op8<bf16_t> (&ring)[TileOps<D>::RING],
                                                   const Op8<bf16_t> (&qop)[D / 16], int e, bool valid,
                                                   const unsigned char* lds, bf16_t* __restrict__ po,
                                                   float* __restrict__ plse, int b, int g, int N, int Hkv, int KP,
                                                   const uint8_t* __restrict__ hmask, float scale_log2, int hh,
                                                   int col, int half, size_t spare) {
    using O = TileOps<D>;
    floatx16 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s[kt] = zero16();
#pragma unroll
    for (int n = 0; n < O::NS; ++n) {
        tile_op<D>(ring[(n + O::PF) % O::RING], lds, (n + O::PF) % O::N, col, half);
        mma16(s[n % 4], ring[n % O::RING], qop[n / 4]);
        __builtin_amdgcn_sched_barrier(0);   // keep each load PF products ahead, no further
    }
    if constexpr (HM) mask_halves(s, hmask[(((size_t)b * Hkv + g) * N + (e >> 5)) * (KP + 1) + (e & 31)]);
    float mz, l;
    tile_softmax(s, scale_log2, mz, l);
    Op8<bf16_t> bp[8];   // key slice c: the lane's 8 probabilities of keys 16c ..
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float pe[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) pe[x] = s[c / 2][8 * (c % 2) + x];
        PType<bf16_t>::pack(bp[c], pe);
    }
    const size_t pidx = valid ? (((size_t)b * Hkv + g) * N + (e >> 5)) * KP + (e & 31) : spare;
    bf16_t* region = po + pidx * G * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        floatx16 o = zero16();
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int n = O::NS + 8 * dt + c;
            tile_op<D>(ring[(n + O::PF) % O::RING], lds, (n + O::PF) % O::N, col, half);
            mma16(o, ring[n % O::RING], bp[c]);
            __builtin_amdgcn_sched_barrier(0);
        }
        u32x4 w0, w1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w0[r] = pack_bf16x2(o[2 * r] * inv, o[2 * r + 1] * inv);
            w1[r] = pack_bf16x2(o[8 + 2 * r] * inv, o[8 + 2 * r + 1] * inv);
        }
        __builtin_nontemporal_store(w0, partial_piece<bf16_t, D, G>(region, 2 * dt, hh, half));
        __builtin_nontemporal_store(w1, partial_piece<bf16_t, D, G>(region, 2 * dt + 1, hh, half));
    }
    // Streamed past the caches like the pieces: the 32-byte LSE records of one
    // tile land in different lines, which no later store of this kernel fills.
    __builtin_nontemporal_store((mz + __log2f(l)) * 0.69314718055994531f, plse + pidx * G + hh);
}

// One work-group per work item (batch, group, key block j, <= kSeg query
// positions that kept j). K_j and V_j^T are staged in LDS once; each wave
// streams 32-row tiles through them, loading the next tile's query rows while
// the current tile is on the matrix cores.
template <typename T, int D, int G, bool HM>
__global__ __launch_bounds__(256, 2) void attn_nonlocal_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ list, const int4* __restrict__ items, const int32_t* __restrict__ total_items,
    const T* __restrict__ vt, T* __restrict__ po, float* __restrict__ plse, const uint8_t* __restrict__ hmask, int N,
    int Hkv, int nb, int nwin, int KP, float scale_log2, size_t spare) {
    using KV = KVTile<T, D>;
    constexpr int PPT = 32 / G;   // positions per 32-row tile
    __shared__ __align__(16) unsigned char lds[KV::BYTES];

    const int total = total_items[0];
    const int item_id = item_of_workgroup(blockIdx.x);
    if (item_id >= total) return;
    const int4 it = items[item_id];
    const int key = it.x, start = it.y, count = it.z;
    const int j = key % nb;
    const int bg = key / (nb * nwin);   // key = ((b * Hkv + g) * nwin + window) * nb + j
    const int g = bg % Hkv;
    const int b = bg / Hkv;
    const int Hq = Hkv * G;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int hh = col % G, pp = col / G;
    const int stride = 4 * PPT;
    const T* qbase = q + (size_t)b * N * Hq * D + (size_t)(g * G + hh) * D;

    // First tile's list entry and query rows are requested before the K/V staging.
    int base = w * PPT;
    int e_cur = list[start + min(base + pp, count - 1)];
    Op8<T> q_cur[D / 16];
    load_q_op<T, D>(q_cur, qbase + (size_t)(e_cur >> 5) * Hq * D, true, half);
    int e_nxt = list[start + min(base + stride + pp, count - 1)];

    const size_t kv_row = (size_t)Hkv * D;
    const size_t kv_off = ((size_t)b * N + (size_t)j * kBlock) * kv_row + (size_t)g * D;
    KV::stage(lds, k + kv_off, kv_row, vt + (((size_t)b * Hkv + g) * nb + j) * D * kBlock, kBlock);
    __syncthreads();

    // Two query-operand buffers in turn (the loop body is written out twice so
    // neither is copied into the other): the tile at `base` runs from one while
    // the next tile's rows load into the other.
    Op8<T> q_nxt[D / 16];
    if constexpr (sizeof(T) == 2) {
        using O = TileOps<D>;
        Op8<bf16_t> ring[O::RING];
#pragma unroll
        for (int n = 0; n < O::PF; ++n) tile_op<D>(ring[n], lds, n, col, half);
        for (; base < count; base += 2 * stride) {
            load_q_op<T, D>(q_nxt, qbase + (size_t)(e_nxt >> 5) * Hq * D, true, half);
            const int e_2 = list[start + min(base + 2 * stride + pp, count - 1)];
            nonlocal_tile_pipe<D, G, HM>(ring, q_cur, e_cur, base + pp < count, lds, po, plse, b, g, N, Hkv, KP,
                                         hmask, scale_log2, hh, col, half, spare);
            if (base + stride >= count) break;
            load_q_op<T, D>(q_cur, qbase + (size_t)(e_2 >> 5) * Hq * D, true, half);
            const int e_3 = list[start + min(base + 3 * stride + pp, count - 1)];
            nonlocal_tile_pipe<D, G, HM>(ring, q_nxt, e_nxt, base + stride + pp < count, lds, po, plse, b, g, N,
                                         Hkv, KP, hmask, scale_log2, hh, col, half, spare);
            e_cur = e_2;
            e_nxt = e_3;
        }
        return;
    }
    for (; base < count; base += 2 * stride) {
        load_q_op<T, D>(q_nxt, qbase + (size_t)(e_nxt >> 5) * Hq * D, true, half);
        const int e_2 = list[start + min(base + 2 * stride + pp, count - 1)];
        nonlocal_tile<T, D, G, HM>(q_cur, e_cur, base + pp < count, lds, po, plse, b, g, N, Hkv, KP, hmask,
                                   scale_log2, hh, col, half, spare);
        if (base + stride >= count) break;
        load_q_op<T, D>(q_cur, qbase + (size_t)(e_2 >> 5) * Hq * D, true, half);
        const int e_3 = list[start + min(base + 3 * stride + pp, count - 1)];
        nonlocal_tile<T, D, G, HM>(q_nxt, e_nxt, base + stride + pp < count, lds, po, plse, b, g, N, Hkv, KP,
                                   hmask, scale_log2, hh, col, half, spare);
        e_cur = e_2;
        e_nxt = e_3;
    }
}

// ------------------------------------------------ local block + combination --

// Adds w * (partial O of one slot) to the lane's output accumulators; `x`
// holds the lane's 16 values per 32-wide slice of D in the stored order.
template <typename T, int D>
struct PartialRow {
    static constexpr int NV = sizeof(T) == 2 ? D / 16 : D / 8;   // 16-byte pieces per lane
    u32x4 x[NV];
    // `region`: the G x D partial of one (row, slot), in the interleaved order
    // written by store_partial; read once, so non-temporally.
    template <int G>
    __device__ __forceinline__ void fetch(const T* region, int hh, int half) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
            x[v] = __builtin_nontemporal_load(partial_piece<T, D, G>(const_cast<T*>(region), v, hh, half));
    }
    __device__ __forceinline__ void axpy(floatx16 (&acc)[D / 32], float w) const {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const uint32_t wv = x[2 * dt + r / 4][r % 4];
                    acc[dt][2 * r] += w * __uint_as_float(wv << 16);
                    acc[dt][2 * r + 1] += w * __uint_as_float(wv & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] += w * __uint_as_float(x[4 * dt + r / 4][r % 4]);
            }
        }
    }
};

// One work-group per (batch, query block, group): the causal local block for
// all 128*G rows from LDS-resident K/V, then the merge with the rows'
// non-local partials (log2 domain, slot order). The partial LSEs of all SL
// possible slots are requested before the local block's math and kept in
// registers (the loops over slots are unrolled, predicated on the row's slot
// count); the partial outputs are fetched two slots at a time.
// XP: the selection was made with another block size and rewritten over
// 128-token blocks; info (per row) gives the row's number of non-local
// entries and whether the first half of its own 128-key block is kept.
template <typename T, int D, int G, int SL, bool XP>
__global__ __launch_bounds__(256, 2) void attn_local_combine_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt, const T* __restrict__ po,
    const float* __restrict__ plse, const uint8_t* __restrict__ info, T* __restrict__ o, float* __restrict__ lse,
    int B, int N, int Hkv, int nb, int qb_lo, int topk, int KP, float scale_log2) {
    using KV = KVTile<T, D>;
    constexpr int BATCH = 2;
    __shared__ __align__(16) unsigned char lds[KV::BYTES];
    const int g = blockIdx.x % Hkv;
    const int b = (blockIdx.x / Hkv) % B;
    const int qb = qb_lo + blockIdx.x / (Hkv * B);
    const int Hq = Hkv * G;
    const int q0 = qb * kBlock;
    const int valid_keys = min(kBlock, N - q0);

    const size_t kv_row = (size_t)Hkv * D;
    const size_t kv_off = ((size_t)b * N + (size_t)q0) * kv_row + (size_t)g * D;
    KV::stage(lds, k + kv_off, kv_row, vt + (((size_t)b * Hkv + g) * nb + qb) * D * kBlock, valid_keys);
    __syncthreads();

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int hh = col % G;
    const int h = g * G + hh;
    const int nnl_all = min(topk - 1, qb);     // non-local slots of every row here (Bk = 128)
    constexpr float kLog2e = 1.4426950408889634f;

    for (int tile = w; tile < kBlock * G / 32; tile += 4) {
        const int p = (tile * 32 + col) / G;   // position within the block
        const int i = q0 + p;
        const bool valid = i < N;
        const int ii = valid ? i : q0;
        int nnl = nnl_all, klo = 0;
        if constexpr (XP) {
            const int x = info[((size_t)b * Hkv + g) * N + ii];
            nnl = min(x & 63, topk - 1);
            klo = (x & 64) ? 0 : 64;
        }
        Op8<T> bq[D / 16];
        load_q_op<T, D>(bq, q + ((size_t)b * N + ii) * Hq * D + (size_t)h * D, valid, half);
        const size_t prow = (((size_t)b * Hkv + g) * N + ii) * KP;
        const float* pl = plse + prow * G + hh;
        float pls[SL];   // log2-domain LSE of each non-local slot (-inf past the row's count)
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) pls[sl] = sl < nnl ? pl[sl * G] * kLog2e : -__builtin_inff();

        floatx16 s[4];
        tile_scores<T, D, false>(s, bq, lds, col, half);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                if (key > p || key < klo) s[kt][r] = -__builtin_inff();
            }
        }
        float mz, l;
        tile_softmax(s, scale_log2, mz, l);
        floatx16 acc[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();
        tile_pv<T, D>(acc, s, lds, col, half);

        // LSE over the local block and every non-local slot (log2 domain).
        const float lse_loc = mz + __log2f(l);
        float mx = lse_loc;
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) mx = fmaxf(mx, pls[sl]);
        float tot = exp2_hw(lse_loc - mx);
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) tot += exp2_hw(pls[sl] - mx);   // 0 for absent slots
        const float lse_all = mx + __log2f(tot);
        const float wl = exp2_hw(lse_loc - lse_all) / l;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= wl;
        }
        const T* pbase = po + prow * G * D;
#pragma unroll
        for (int sl0 = 0; sl0 < SL; sl0 += BATCH) {
            if (sl0 < nnl) {
                PartialRow<T, D> pr[BATCH];
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (sl0 + u < SL && sl0 + u < nnl) pr[u].template fetch<G>(pbase + (size_t)(sl0 + u) * G * D, hh, half);
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (sl0 + u < SL && sl0 + u < nnl) pr[u].axpy(acc, exp2_hw(pls[sl0 + u] - lse_all));
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
                        const uint32_t a0 = pack_bf16x2(acc[dt][4 * rq], acc[dt][4 * rq + 1]);
                        const uint32_t a1 = pack_bf16x2(acc[dt][4 * rq + 2], acc[dt][4 * rq + 3]);
                        *reinterpret_cast<uint2*>(d4) = make_uint2(a0, a1);
                    } else {
                        floatx4 x;
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = acc[dt][4 * rq + e];
                        *reinterpret_cast<floatx4*>(d4) = x;
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
    const size_t es = d.dtype == 0 ? 2 : 4;
    w.ex = expand_layout(d, 0);   // other block sizes: the selection over 128-token blocks first
    const LaunchDims e = as_128(d);
    size_t off = w.ex.end;
    w.vt = off;    off = align_up(off + (size_t)e.B * e.Hkv * e.nb * e.D * kBlock * es);
    w.lists = list_layout(e, off);
    if (w.lists.has_nonlocal) {
        off = w.lists.end;
        // One spare (row, slot) past the last: the padding rows' partials.
        w.po = off;    off = align_up(off + (w.lists.max_entries + 1) * e.G * e.D * es);
        w.plse = off;  off = align_up(off + (w.lists.max_entries + 1) * e.G * 4);
    }
    w.bytes = off;
    return w;
}

template <typename T, int D, int G>
static hipError_t launch_attn_t(const LaunchDims& d0, int qb_lo, int qb_hi, const void* q, const void* k,
                                const int32_t* block_idx0, float scale, void* o, float* lse, unsigned char* ws,
                                int stages, hipStream_t st) {
    const AttnWorkspace L = attn_workspace_layout(d0);
    // Other block sizes: the rows' selections over 128-token blocks (rewritten
    // by the first stage), with the half masks of 64-token selections.
    const bool xp = d0.Bk != 128, hm = d0.Bk == 64;
    const LaunchDims d = as_128(d0);
    const int32_t* block_idx = xp ? reinterpret_cast<const int32_t*>(ws + L.ex.ids) : block_idx0;
    const uint8_t* hmask = reinterpret_cast<const uint8_t*>(ws + L.ex.hmask);
    const uint8_t* info = reinterpret_cast<const uint8_t*>(ws + L.ex.info);
    if (xp && (stages & 1)) launch_expand(d0, block_idx0, ws, L.ex, st);
    const float scale_log2 = scale * 1.4426950408889634f;
    const int KP = d.k > 1 ? d.k - 1 : 1;
    const T* tq = static_cast<const T*>(q);
    const T* tk = static_cast<const T*>(k);
    const T* vt = reinterpret_cast<const T*>(ws + L.vt);
    T* po = nullptr;
    float* plse = nullptr;
    // Rows of query block 0 keep no non-local block.
    const bool nonlocal = L.lists.has_nonlocal && qb_hi > 1;
    if (nonlocal) {
        const int p_lo = qb_lo * kBlock, p_hi = min(d.N, qb_hi * kBlock);
        if (stages & 1) launch_build_lists(d, p_lo, p_hi, block_idx, ws, L.lists, st);
        const int4* items = reinterpret_cast<const int4*>(ws + L.lists.items);
        const int32_t* list = reinterpret_cast<const int32_t*>(ws + L.lists.list);
        const int32_t* total = reinterpret_cast<const int32_t*>(ws + L.lists.total);
        po = reinterpret_cast<T*>(ws + L.po);
        plse = reinterpret_cast<float*>(ws + L.plse);
        const size_t grid = (list_items_bound(d, p_lo, p_hi, L.lists) + 63) / 64 * 64;
        if ((stages & 2) && hm)
            hipLaunchKernelGGL((attn_nonlocal_kernel<T, D, G, true>), dim3((unsigned)grid), dim3(256), 0, st, tq, tk,
                               list, items, total, vt, po, plse, hmask, d.N, d.Hkv, d.nb, windows(d), KP, scale_log2,
                               L.lists.max_entries);
        else if (stages & 2)
            hipLaunchKernelGGL((attn_nonlocal_kernel<T, D, G, false>), dim3((unsigned)grid), dim3(256), 0, st, tq, tk,
                               list, items, total, vt, po, plse, hmask, d.N, d.Hkv, d.nb, windows(d), KP, scale_log2,
                               L.lists.max_entries);
    }
    if (stages & 4) {
        const dim3 grid((unsigned)((qb_hi - qb_lo) * d.B * d.Hkv));
        const int kk = nonlocal ? d.k : 1;
        T* to = static_cast<T*>(o);
        if (xp) {
            if (kk <= 8)
                hipLaunchKernelGGL((attn_local_combine_kernel<T, D, G, 7, true>), grid, dim3(256), 0, st, tq, tk, vt,
                                   po, plse, info, to, lse, d.B, d.N, d.Hkv, d.nb, qb_lo, kk, KP, scale_log2);
            else if (kk <= 16)
                hipLaunchKernelGGL((attn_local_combine_kernel<T, D, G, 15, true>), grid, dim3(256), 0, st, tq, tk, vt,
                                   po, plse, info, to, lse, d.B, d.N, d.Hkv, d.nb, qb_lo, kk, KP, scale_log2);
            else
                hipLaunchKernelGGL((attn_local_combine_kernel<T, D, G, 31, true>), grid, dim3(256), 0, st, tq, tk, vt,
                                   po, plse, info, to, lse, d.B, d.N, d.Hkv, d.nb, qb_lo, kk, KP, scale_log2);
        } else if (kk <= 8)
            hipLaunchKernelGGL((attn_local_combine_kernel<T, D, G, 7, false>), grid, dim3(256), 0, st, tq, tk, vt, po,
                               plse, info, to, lse, d.B, d.N, d.Hkv, d.nb, qb_lo, kk, KP, scale_log2);
        else if (kk <= 16)
            hipLaunchKernelGGL((attn_local_combine_kernel<T, D, G, 15, false>), grid, dim3(256), 0, st, tq, tk, vt, po,
                               plse, info, to, lse, d.B, d.N, d.Hkv, d.nb, qb_lo, kk, KP, scale_log2);
        else
            hipLaunchKernelGGL((attn_local_combine_kernel<T, D, G, 31, false>), grid, dim3(256), 0, st, tq, tk, vt, po,
                               plse, info, to, lse, d.B, d.N, d.Hkv, d.nb, qb_lo, kk, KP, scale_log2);
    }
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_d(const LaunchDims& d, int lo, int hi, const void* q, const void* k,
                                const int32_t* bi, float scale, void* o, float* lse, unsigned char* ws, int sg,
                                hipStream_t st) {
    switch (d.G) {
        case 1: return launch_attn_t<T, D, 1>(d, lo, hi, q, k, bi, scale, o, lse, ws, sg, st);
        case 2: return launch_attn_t<T, D, 2>(d, lo, hi, q, k, bi, scale, o, lse, ws, sg, st);
        case 4: return launch_attn_t<T, D, 4>(d, lo, hi, q, k, bi, scale, o, lse, ws, sg, st);
        case 8: return launch_attn_t<T, D, 8>(d, lo, hi, q, k, bi, scale, o, lse, ws, sg, st);
        case 16: return launch_attn_t<T, D, 16>(d, lo, hi, q, k, bi, scale, o, lse, ws, sg, st);
        default: return launch_attn_t<T, D, 32>(d, lo, hi, q, k, bi, scale, o, lse, ws, sg, st);
    }
}

hipError_t launch_sparse_attn(const LaunchDims& d, int qb_lo, int qb_hi, const void* q, const void* k,
                              const int32_t* block_idx, float scale, void* o, float* lse, void* ws, int stages,
                              hipStream_t st) {
    if (d.B == 0 || d.N == 0 || qb_hi <= qb_lo) return hipSuccess;
    unsigned char* w = static_cast<unsigned char*>(ws);
    if (d.dtype == 0)
        return d.D == 128 ? launch_attn_d<bf16_t, 128>(d, qb_lo, qb_hi, q, k, block_idx, scale, o, lse, w, stages, st)
                          : launch_attn_d<bf16_t, 64>(d, qb_lo, qb_hi, q, k, block_idx, scale, o, lse, w, stages, st);
    return d.D == 128 ? launch_attn_d<float, 128>(d, qb_lo, qb_hi, q, k, block_idx, scale, o, lse, w, stages, st)
                      : launch_attn_d<float, 64>(d, qb_lo, qb_hi, q, k, block_idx, scale, o, lse, w, stages, st);
}

template <typename T, int D>
static void transpose_t(const LaunchDims& d, const void* src, void* dst, hipStream_t st) {
    hipLaunchKernelGGL((transpose_v_kernel<T, D>), dim3((unsigned)(d.B * d.Hkv * d.nb)), dim3(256), 0, st,
                       static_cast<const T*>(src), static_cast<T*>(dst), d.N, d.Hkv, d.nb);
}

hipError_t launch_transpose_kv(const LaunchDims& d, const void* src, void* dst, hipStream_t st) {
    if (d.B == 0 || d.N == 0) return hipSuccess;
    if (d.dtype == 0) {
        if (d.D == 128) transpose_t<bf16_t, 128>(d, src, dst, st);
        else transpose_t<bf16_t, 64>(d, src, dst, st);
    } else {
        if (d.D == 128) transpose_t<float, 128>(d, src, dst, st);
        else transpose_t<float, 64>(d, src, dst, st);
    }
    return hipGetLastError();
}

hipError_t launch_transpose_v(const LaunchDims& d, const void* v, void* ws, hipStream_t st) {
    return launch_transpose_kv(d, v, static_cast<unsigned char*>(ws) + attn_workspace_layout(d).vt, st);
}

}  // namespace msa
