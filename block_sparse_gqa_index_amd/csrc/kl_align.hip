// KL alignment loss forward of MSA (gfx950).
//
// Method: MiniMax Sparse Attention (MSA) article on 7minutos.es, section "Cómo
// se entrena MSA": the index branch is trained with a KL loss whose teacher is
// the main-branch distribution averaged over the group's heads, restricted to
// the selected tokens; the Flash-MSA article (tech.kuratif.com) computes it
// without materialising either distribution.
//
// For a row (b, g, i) with selected tokens T_i:
//   p_t = (1/G) sum_h exp(z_{h,t} - LSE_h)          (teacher; LSE_h from the main pass)
//   u_t = index_scale * <q_idx[b,i,g], k_idx[b,t]>    (student logits)
//   KL  = sum_t p_t (ln p_t - u_t + LSE_u),  LSE_u = ln sum_t exp(u_t)
// Every term is a sum over tokens, so each kept block contributes five
// numbers (sum p ln p, sum p u, sum p, max u, sum exp(u - max u)) that merge
// exactly. Non-local blocks are processed key-block-outer from the same
// inverted selection as the attention; the local block and the merge run per
// (batch, query block, group); kl_sum is a fixed-order two-stage reduction.
// dense_kl_kernel computes the same loss over every visible token (warm-up).
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"

namespace msa {

constexpr int kKlPart = 8;          // floats per (row, slot) partial record
constexpr int kRedThreads = 256;

struct KlAcc {
    float A, Bs, P, mu, lu;
};

// Value of the partner lane whose hh differs from this lane's in bit BIT and
// agrees in every higher bit (lower bits may differ): DPP quad permutes for
// bits 0 and 1, the 8- and 16-lane mirrors for bits 2 and 3 (lane i <-> 7-i,
// 15-i), an LDS permute only for bit 4.
template <int BIT>
__device__ __forceinline__ float lane_pair(float x) {
    const int v = __float_as_int(x);
    if constexpr (BIT == 0) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
    else if constexpr (BIT == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
    else if constexpr (BIT == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));
    else if constexpr (BIT == 3) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));
    else return __shfl_xor(x, 1 << BIT);
}

// One reduce-scatter step over bit BIT of the head index (see tile_kl): keeps
// the upper or lower half of the first N tokens, adding the partner's half.
// The u values (equal in all lanes of the group) are narrowed with a bitwise
// select under a lane mask rather than a select of floats: selects of plain
// copies of accumulator elements are folded by the compiler, across the
// unrolled steps, into one lane-dependent element index that it expands as a
// compare chain per value; the integer form stays one instruction per value.
template <int BIT, int N>
__device__ __forceinline__ void scatter_step(float (&v)[64], float (&uv)[64], int hh, int& base) {
    const bool hi = (hh >> BIT) & 1;
    const uint32_t msk = hi ? 0xffffffffu : 0u;
#pragma unroll
    for (int t = 0; t < N / 2; ++t) {
        const float send = hi ? v[t] : v[t + N / 2];
        const float keep = hi ? v[t + N / 2] : v[t];
        v[t] = keep + lane_pair<BIT>(send);
        uv[t] = __uint_as_float((__float_as_uint(uv[t + N / 2]) & msk) | (__float_as_uint(uv[t]) & ~msk));
    }
    base += hi ? N / 2 : 0;
}

// Merges another (max, sum of exp(x - max)) pair into (mu, lu); -inf maxima
// stand for empty sets.
__device__ __forceinline__ void merge_lse(float& mu, float& lu, float omu, float olu) {
    const float m = fmaxf(mu, omu);
    lu = (mu == -__builtin_inff() ? 0.f : lu * exp2_hw((mu - m) * 1.4426950408889634f)) +
         (omu == -__builtin_inff() ? 0.f : olu * exp2_hw((omu - m) * 1.4426950408889634f));
    mu = m;
}

// All-reduce step of the five sums over bit BIT of the head index (no-op when
// the group has no such bit).
template <int BIT, int G>
__device__ __forceinline__ void combine_bit(KlAcc& a) {
    if constexpr ((1 << BIT) < G) {
        a.A += lane_pair<BIT>(a.A);
        a.Bs += lane_pair<BIT>(a.Bs);
        a.P += lane_pair<BIT>(a.P);
        merge_lse(a.mu, a.lu, lane_pair<BIT>(a.mu), lane_pair<BIT>(a.lu));
    }
}

// Partial sums of one 32-row tile (32/G positions x G heads) over one 128-key
// block. With MASK, keys past `p_limit` (the query's offset in its block) are
// not visible. The teacher probability of a token is the mean over the G head
// lanes of a position, so the per-token terms are the same in those G lanes:
// a reduce-scatter over them (log2 G exchange steps, halving the values kept
// per lane each time) leaves every lane with the head-sum of 64/G of the 64
// tokens it holds, and the logarithms and exponentials below run once per
// token instead of G times. The index scores u are equal in the G lanes (same
// index query) and are only narrowed the same way.
// MASK: only keys k_lo .. p_limit of the block are among the row's tokens
// (the causal limit of the local block; the kept half of a 64-token selection).
template <int G, bool MASK>
__device__ __forceinline__ KlAcc tile_kl(const floatx16 (&s)[4], const floatx16 (&u)[4], float scale_log2, float lse2,
                                         float iscale, int p_limit, int half, int hh, int k_lo = 0) {
    constexpr float kLn2 = 0.69314718055994531f;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr int NV = 64 / G;   // tokens per lane after the reduce-scatter
    // Per-token values as plain scalars (token t = kt * 16 + r of the lane's
    // accumulator layout): selecting between two elements of one vector
    // register tuple with a lane-dependent condition is compiled as a dynamic
    // element index (a compare chain per element), between scalars as one
    // v_cndmask.
    float v[64], uv[64];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
            const bool vis = !MASK || (key <= p_limit && key >= k_lo);
            v[kt * 16 + r] = vis ? exp2_hw(fmaf(s[kt][r], scale_log2, -lse2)) : 0.f;
            uv[kt * 16 + r] = u[kt][r];
        }
    }
    // Highest head bit first: the mirror pairings flip the lower bits too,
    // which is harmless while those bits are still to be reduced.
    int base = 0;   // first token index the lane keeps
    if constexpr (G >= 32) scatter_step<4, 64>(v, uv, hh, base);
    if constexpr (G >= 16) scatter_step<3, 64 * 16 / G>(v, uv, hh, base);
    if constexpr (G >= 8) scatter_step<2, 64 * 8 / G>(v, uv, hh, base);
    if constexpr (G >= 4) scatter_step<1, 64 * 4 / G>(v, uv, hh, base);
    if constexpr (G >= 2) scatter_step<0, 64 * 2 / G>(v, uv, hh, base);
    KlAcc a{0.f, 0.f, 0.f, -__builtin_inff(), 0.f};
    float uk[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
        const int t = base + e, kt = t >> 4, r = t & 15;
        const int key = kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const bool vis = !MASK || (key <= p_limit && key >= k_lo);
        const float p = v[e] * (1.0f / G);
        const float uu = uv[e] * iscale;
        uk[e] = vis ? uu : -__builtin_inff();
        if (vis) {
            if (p > 0.f) a.A += p * (__log2f(p) * kLn2);
            a.Bs += p * uu;
            a.P += p;
            a.mu = fmaxf(a.mu, uu);
        }
    }
#pragma unroll
    for (int e = 0; e < NV; ++e) a.lu += exp2_hw((uk[e] - a.mu) * kLog2e);   // 0 for masked tokens
    if (a.mu == -__builtin_inff()) a.lu = 0.f;
    // Combine the G lanes of the position, then the two half-waves.
    combine_bit<0, G>(a);
    combine_bit<1, G>(a);
    combine_bit<2, G>(a);
    combine_bit<3, G>(a);
    combine_bit<4, G>(a);
    a.A += swap_halves(a.A);
    a.Bs += swap_halves(a.Bs);
    a.P += swap_halves(a.P);
    merge_lse(a.mu, a.lu, swap_halves(a.mu), swap_halves(a.lu));
    return a;
}

// HM: each entry keeps only the halves of the block its mask byte names (a
// selection made with 64-token blocks: bit 0 keys 0-63, bit 1 keys 64-127).
template <typename T, int D, int DI, int G, bool HM>
__global__ __launch_bounds__(256, 2) void kl_nonlocal_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ q_idx, const T* __restrict__ k_idx,
    const float* __restrict__ lse, const int32_t* __restrict__ list, const int4* __restrict__ items,
    const int32_t* __restrict__ total_items, float* __restrict__ part, const uint8_t* __restrict__ hmask, int N,
    int Hkv, int nb, int nwin, int KP, float scale_log2, float iscale, size_t spare) {
    constexpr int PPT = 32 / G;
    __shared__ __align__(16) unsigned char lds[SwzTile<T, D>::BYTES + SwzTile<T, DI>::BYTES];
    unsigned char* lds_i = lds + SwzTile<T, D>::BYTES;

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
    constexpr float kLog2e = 1.4426950408889634f;
    auto entry = [&](int at) { return list[start + min(at + pp, count - 1)]; };
    auto qrow = [&](int e) { return q + ((size_t)b * N + (e >> 5)) * Hq * D + (size_t)(g * G + hh) * D; };
    auto qirow = [&](int e) { return q_idx + (((size_t)b * N + (e >> 5)) * Hkv + g) * DI; };

    // The first tile's rows are requested before the K staging; afterwards each
    // tile's query operands are refilled with the next tile's rows as soon as
    // its scores are on the matrix cores.
    int base = w * PPT;
    int e_cur = entry(base);
    Op8<T> bq[D / 16];
    Op8<T> bi[DI / 16];
    load_q_op<T, D>(bq, qrow(e_cur), sizeof(T) == 2 || base + pp < count, half);
    load_q_op<T, DI>(bi, qirow(e_cur), sizeof(T) == 2 || base + pp < count, half);

    stage_rows<T, D>(lds, k + ((size_t)b * N + (size_t)j * kBlock) * Hkv * D + (size_t)g * D, (size_t)Hkv * D,
                     kBlock);
    stage_rows<T, DI>(lds_i, k_idx + ((size_t)b * N + (size_t)j * kBlock) * DI, DI, kBlock);
    __syncthreads();

    if constexpr (sizeof(T) == 2) {
        // bf16: the A operands of a tile (the K slices of S^T, then the K_idx
        // slices of U^T) repeat every tile, so they go through an 8-register ring
        // loaded 6 products ahead across tiles; the rows' loads (clamped to the
        // item's last entry) and the partial stores (the other lanes and the
        // padding rows to the spare record) are unconditional, so each tile's
        // wait covers only the next rows' loads.
        constexpr int NS = (D / 16) * 4, N_OPS = NS + (DI / 16) * 4, RING = 8, PF = 6;
        static_assert(N_OPS % RING == 0, "the ring must tile the operand sequence");
        auto op = [&](Op8<bf16_t>& a, int n) {
            if (n < NS) SwzTile<bf16_t, D>::load8(a, lds, (n % 4) * 32 + col, 16 * (n / 4) + 8 * half);
            else SwzTile<bf16_t, DI>::load8(a, lds_i, ((n - NS) % 4) * 32 + col, 16 * ((n - NS) / 4) + 8 * half);
        };
        Op8<bf16_t> ring[RING];
#pragma unroll
        for (int n = 0; n < PF; ++n) op(ring[n], n);
        for (; base < count; base += stride) {
            const bool valid = base + pp < count;
            const int i = e_cur >> 5, slot = e_cur & 31;
            const float lse_row = lse[((size_t)b * Hq + g * G + hh) * N + i];
            const int e_nxt = entry(base + stride);
            floatx16 s[4], u[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) s[kt] = u[kt] = zero16();
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                op(ring[(n + PF) % RING], (n + PF) % N_OPS);
                mma16(s[n % 4], ring[n % RING], bq[n / 4]);
                __builtin_amdgcn_sched_barrier(0);
            }
            load_q_op<T, D>(bq, qrow(e_nxt), true, half);
#pragma unroll
            for (int n = NS; n < N_OPS; ++n) {
                op(ring[(n + PF) % RING], (n + PF) % N_OPS);
                mma16(u[(n - NS) % 4], ring[n % RING], bi[(n - NS) / 4]);
                __builtin_amdgcn_sched_barrier(0);
            }
            load_q_op<T, DI>(bi, qirow(e_nxt), true, half);
            const float lse2 = valid ? lse_row * kLog2e : 0.f;
            KlAcc a;
            if constexpr (HM) {
                const int m = hmask[(((size_t)b * Hkv + g) * N + i) * (KP + 1) + slot];
                a = tile_kl<G, true>(s, u, scale_log2, lse2, iscale, (m & 2) ? 127 : 63, half, hh, (m & 1) ? 0 : 64);
            } else {
                a = tile_kl<G, false>(s, u, scale_log2, lse2, iscale, 0, half, hh);
            }
            const size_t rec = valid && hh == 0 && half == 0 ? (((size_t)b * Hkv + g) * N + i) * KP + slot : spare;
            float* dst = part + rec * kKlPart;
            *reinterpret_cast<float4*>(dst) = make_float4(a.A, a.Bs, a.P, a.mu);
            dst[4] = a.lu;
            e_cur = e_nxt;
        }
        return;
    }

    for (; base < count; base += stride) {
        const bool valid = base + pp < count;
        const int i = e_cur >> 5, slot = e_cur & 31;
        const float lse2 = valid ? lse[((size_t)b * Hq + g * G + hh) * N + i] * kLog2e : 0.f;
        const int e_nxt = entry(base + stride);
        const bool nvalid = base + stride + pp < count;
        floatx16 s[4], u[4];
        tile_scores<T, D>(s, bq, lds, col, half);
        load_q_op<T, D>(bq, qrow(e_nxt), nvalid, half);
        tile_scores<T, DI>(u, bi, lds_i, col, half);
        load_q_op<T, DI>(bi, qirow(e_nxt), nvalid, half);
        KlAcc a;
        if constexpr (HM) {
            const int m = hmask[(((size_t)b * Hkv + g) * N + i) * (KP + 1) + slot];
            a = tile_kl<G, true>(s, u, scale_log2, lse2, iscale, (m & 2) ? 127 : 63, half, hh, (m & 1) ? 0 : 64);
        } else {
            a = tile_kl<G, false>(s, u, scale_log2, lse2, iscale, 0, half, hh);
        }
        if (valid && hh == 0 && half == 0) {
            float* dst = part + ((((size_t)b * Hkv + g) * N + i) * KP + slot) * kKlPart;
            *reinterpret_cast<float4*>(dst) = make_float4(a.A, a.Bs, a.P, a.mu);
            dst[4] = a.lu;
        }
        e_cur = e_nxt;
    }
}

// XP: the selection was made with another block size and rewritten over
// 128-token blocks; info (per row) gives the row's number of non-local
// entries and whether the first half of its own 128-key block is kept.
template <typename T, int D, int DI, int G, bool XP>
__global__ __launch_bounds__(256, 2) void kl_local_combine_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ q_idx, const T* __restrict__ k_idx,
    const float* __restrict__ lse, const float* __restrict__ part, const uint8_t* __restrict__ info,
    float* __restrict__ kl_rows, float* __restrict__ index_lse, int B, int N, int Hkv, int nb, int topk, int KP,
    float scale_log2, float iscale) {
    __shared__ __align__(16) unsigned char lds[SwzTile<T, D>::BYTES + SwzTile<T, DI>::BYTES];
    unsigned char* lds_i = lds + SwzTile<T, D>::BYTES;
    const int g = blockIdx.x % Hkv;
    const int b = (blockIdx.x / Hkv) % B;
    const int qb = blockIdx.x / (Hkv * B);
    const int Hq = Hkv * G;
    const int q0 = qb * kBlock;
    const int valid_keys = min(kBlock, N - q0);

    stage_rows<T, D>(lds, k + ((size_t)b * N + q0) * Hkv * D + (size_t)g * D, (size_t)Hkv * D, valid_keys);
    stage_rows<T, DI>(lds_i, k_idx + ((size_t)b * N + q0) * DI, DI, valid_keys);
    __syncthreads();

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int hh = col % G;
    const int nnl_all = min(topk - 1, qb);
    constexpr float kLog2e = 1.4426950408889634f;
    for (int tile = w; tile < kBlock * G / 32; tile += 4) {
        const int p = (tile * 32 + col) / G;
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
        load_q_op<T, D>(bq, q + ((size_t)b * N + ii) * Hq * D + (size_t)(g * G + hh) * D, valid, half);
        Op8<T> bi[DI / 16];
        load_q_op<T, DI>(bi, q_idx + (((size_t)b * N + ii) * Hkv + g) * DI, valid, half);
        floatx16 s[4], u[4];
        tile_scores<T, D>(s, bq, lds, col, half);
        tile_scores<T, DI>(u, bi, lds_i, col, half);
        const float lse2 = valid ? lse[((size_t)b * Hq + g * G + hh) * N + i] * kLog2e : 0.f;
        KlAcc a = tile_kl<G, true>(s, u, scale_log2, lse2, iscale, p, half, hh, klo);

        const float* src = part + (((size_t)b * Hkv + g) * N + ii) * KP * kKlPart;
        for (int sl = 0; sl < nnl; ++sl) {
            const float4 x = *reinterpret_cast<const float4*>(src + sl * kKlPart);
            const float xl = src[sl * kKlPart + 4];
            a.A += x.x;
            a.Bs += x.y;
            a.P += x.z;
            merge_lse(a.mu, a.lu, x.w, xl);
        }
        const float lse_u = a.mu + __logf(a.lu);
        if (valid && hh == 0 && half == 0) {
            kl_rows[((size_t)b * Hkv + g) * N + i] = a.A - a.Bs + lse_u * a.P;
            if (index_lse) index_lse[((size_t)b * Hkv + g) * N + i] = lse_u;
        }
    }
}

// ------------------------------------------------------------- dense KL --
//
// The warm-up's KL (MSA article, "Cómo se entrena MSA": during the first
// iterations both branches attend to every visible token): the same per-row
// KL with T_i = {0 .. i}, the teacher normalised by the dense attention's LSE.
// Query-block outer like the dense attention: one 8-wave work-group per
// (batch, query block, group, 256-row part), each wave one resident 32-row
// tile (main and index query operands, the five running sums; two waves per
// SIMD, so one wave's KL-tile vector work can run beside the other's matrix
// products); K_j and K_idx_j stream through two LDS buffers (bf16: the next
// block's rows copied global -> LDS directly, which keeps the wave within 256
// registers; fp32: through registers).

constexpr int kDenseKlWaves = 8;

// Rows [128][W] of T moved global -> registers -> LDS (SwzTile<T, W>) by NT
// threads; rows at or past valid_rows are zero-filled.
template <typename T, int W, int NT>
struct RowPrefetch {
    using S = SwzTile<T, W>;
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CH = kBlock * S::CPR;
    static constexpr int PER = CH / NT;
    static_assert(CH % NT == 0, "chunk split");
    u32x4 r[PER];
    __device__ __forceinline__ void load(const T* src, size_t row_stride, int valid_rows) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int ch = threadIdx.x + u * NT;
            const int row = ch / S::CPR, cc = ch % S::CPR;
            r[u] = row < valid_rows ? *reinterpret_cast<const u32x4*>(src + row * row_stride + cc * EPC)
                                    : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void commit(unsigned char* lds) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int ch = threadIdx.x + u * NT;
            const int row = ch / S::CPR, cc = ch % S::CPR;
            *reinterpret_cast<u32x4*>(lds + S::offset(row, cc * 16)) = r[u];
        }
    }
};

template <typename T, int D, int DI, int G, int NBUF>
__global__ __launch_bounds__(kDenseKlWaves * kWave) void dense_kl_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ q_idx, const T* __restrict__ k_idx,
    const float* __restrict__ lse, float* __restrict__ kl_rows, float* __restrict__ index_lse, int B, int N,
    int Hkv, int nb, int parts, float scale_log2, float iscale) {
    constexpr int NT = kDenseKlWaves * kWave;
    constexpr int KB = SwzTile<T, D>::BYTES, BUF = KB + SwzTile<T, DI>::BYTES;
    __shared__ __align__(16) unsigned char lds[NBUF * BUF];
    // Runs of 8 * parts work-groups give each XCD one whole (batch, query
    // block, group) unit, so the unit's parts share that XCD's L2 for the K and
    // K_idx blocks they all stream; latest (heaviest) query blocks first.
    const int x = blockIdx.x;
    const int unit = (x / (8 * parts)) * 8 + x % 8;
    if (unit >= nb * B * Hkv) return;   // padding of the last run
    const int pt = (x / 8) % parts;
    const int g = unit % Hkv;
    const int b = (unit / Hkv) % B;
    const int qb = nb - 1 - unit / (Hkv * B);
    const int Hq = Hkv * G;
    const int q0 = qb * kBlock;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int tile = pt * kDenseKlWaves + w;
    const bool tile_ok = tile < kBlock * G / 32;   // wave-uniform
    const int p = (tile * 32 + col) / G;
    const int hh = col % G;
    const int i = q0 + p;
    const bool valid = tile_ok && i < N;
    const int ii = valid ? i : 0;
    Op8<T> bq[D / 16];
    load_q_op<T, D>(bq, q + ((size_t)b * N + ii) * Hq * D + (size_t)(g * G + hh) * D, valid, half);
    Op8<T> bi[DI / 16];
    load_q_op<T, DI>(bi, q_idx + (((size_t)b * N + ii) * Hkv + g) * DI, valid, half);
    constexpr float kLog2e = 1.4426950408889634f;
    const float lse2 = valid ? lse[((size_t)b * Hq + g * G + hh) * N + i] * kLog2e : 0.f;

    const size_t krow = (size_t)Hkv * D;
    const T* kbase = k + (size_t)b * N * krow + (size_t)g * D;
    const T* kibase = k_idx + (size_t)b * N * DI;
    RowPrefetch<T, D, NT> pk;
    RowPrefetch<T, DI, NT> pi;
    // bf16 with two buffers: K_{j+1} and K_idx_{j+1} are copied global -> LDS
    // directly (no registers) into the other buffer at the start of block j;
    // the barrier that ends block j waits for them. Rows past the sequence
    // repeat its last key (masked for every stored row; a row past the
    // sequence has zero queries).
    constexpr bool kDma = sizeof(T) == 2 && NBUF == 2;
    auto dma_keys = [&](unsigned char* buf, int jb) {
        if constexpr (kDma) {
            constexpr int KR = 64 / SwzTile<T, D>::CPR, IR = 64 / SwzTile<T, DI>::CPR;
            const int last = min(kBlock, N - jb * kBlock) - 1;
            for (int r0 = w * KR; r0 < kBlock; r0 += kDenseKlWaves * KR)
                dma_rows<D>(buf, reinterpret_cast<const bf16_t*>(kbase) + (size_t)jb * kBlock * krow, krow, r0, last,
                            lane);
            for (int r0 = w * IR; r0 < kBlock; r0 += kDenseKlWaves * IR)
                dma_rows<DI>(buf + KB, reinterpret_cast<const bf16_t*>(kibase) + (size_t)jb * kBlock * DI, DI, r0,
                             last, lane);
        }
    };
    if constexpr (kDma) {
        dma_keys(lds, 0);
    } else {
        pk.load(kbase, krow, min(kBlock, N));
        pi.load(kibase, DI, min(kBlock, N));
        pk.commit(lds);
        pi.commit(lds + KB);
    }
    __syncthreads();

    KlAcc acc{0.f, 0.f, 0.f, -__builtin_inff(), 0.f};
    for (int j = 0; j <= qb; ++j) {
        const unsigned char* cur = lds + (NBUF == 2 ? (j & 1) * BUF : 0);
        unsigned char* nxt = lds + (NBUF == 2 ? ((j + 1) & 1) * BUF : 0);
        const bool more = j < qb;
        const int nvalid = more ? min(kBlock, N - (j + 1) * kBlock) : 0;
        if constexpr (kDma) {
            if (more) dma_keys(nxt, j + 1);
        } else {
            if (more) pk.load(kbase + (size_t)(j + 1) * kBlock * krow, krow, nvalid);
        }
        if (tile_ok) {
            floatx16 s[4], u[4];
            tile_scores<T, D>(s, bq, cur, col, half);
            tile_scores<T, DI>(u, bi, cur + KB, col, half);
            if constexpr (NBUF == 2 && !kDma) {
                if (more) {
                    pi.load(kibase + (size_t)(j + 1) * kBlock * DI, DI, nvalid);
                    pk.commit(nxt);
                }
            }
            // Every key of a block before the query's own is visible.
            const KlAcc a = tile_kl<G, true>(s, u, scale_log2, lse2, iscale, j == qb ? p : kBlock - 1, half, hh);
            acc.A += a.A;
            acc.Bs += a.Bs;
            acc.P += a.P;
            merge_lse(acc.mu, acc.lu, a.mu, a.lu);
        } else if constexpr (NBUF == 2 && !kDma) {
            if (more) {
                pi.load(kibase + (size_t)(j + 1) * kBlock * DI, DI, nvalid);
                pk.commit(nxt);
            }
        }
        if (more) {
            if constexpr (kDma) {
            } else if constexpr (NBUF == 2) {
                pi.commit(nxt + KB);
            } else {
                pi.load(kibase + (size_t)(j + 1) * kBlock * DI, DI, nvalid);
                __syncthreads();   // everyone is done reading the single buffer
                pk.commit(nxt);
                pi.commit(nxt + KB);
            }
        }
        __syncthreads();
    }
    if (valid && hh == 0 && half == 0) {
        const float lse_u = acc.mu + __logf(acc.lu);
        kl_rows[((size_t)b * Hkv + g) * N + i] = acc.A - acc.Bs + lse_u * acc.P;
        if (index_lse) index_lse[((size_t)b * Hkv + g) * N + i] = lse_u;
    }
}

// Fixed-order two-stage sum of kl_rows (deterministic for a given size).
__global__ __launch_bounds__(kRedThreads) void kl_reduce_partial(const float* __restrict__ x, size_t n,
                                                                 double* __restrict__ partial) {
    __shared__ double s[kRedThreads];
    const size_t per = (n + gridDim.x - 1) / gridDim.x;
    const size_t lo = min(n, blockIdx.x * per), hi = min(n, lo + per);
    double acc = 0.0;
    for (size_t t = lo + threadIdx.x; t < hi; t += kRedThreads) acc += (double)x[t];
    s[threadIdx.x] = acc;
    __syncthreads();
    for (int off = kRedThreads / 2; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) s[threadIdx.x] += s[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = s[0];
}

__global__ __launch_bounds__(kRedThreads) void kl_reduce_final(const double* __restrict__ partial, int n,
                                                               float* __restrict__ out) {
    __shared__ double s[kRedThreads];
    double acc = 0.0;
    for (int t = threadIdx.x; t < n; t += kRedThreads) acc += partial[t];
    s[threadIdx.x] = acc;
    __syncthreads();
    for (int off = kRedThreads / 2; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) s[threadIdx.x] += s[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = (float)s[0];
}

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

static int red_blocks_for(size_t rows) {
    const size_t want = (rows + 16383) / 16384;
    return (int)(want < 1 ? 1 : (want > 1024 ? 1024 : want));
}

KlWorkspace kl_workspace_layout(const LaunchDims& d0) {
    KlWorkspace w{};
    w.ex = expand_layout(d0, 0);   // other block sizes: the selection over 128-token blocks first
    const LaunchDims d = as_128(d0);
    w.lists = list_layout(d, w.ex.end);
    const size_t rows = (size_t)d.B * d.Hkv * d.N;
    w.red_blocks = red_blocks_for(rows);
    size_t off = w.lists.has_nonlocal ? w.lists.end : w.ex.end;
    // one spare record past the last (row, slot): the stores of padding rows and non-writer lanes
    w.part = off;  off = align_up(off + (w.lists.has_nonlocal ? (w.lists.max_entries + 1) * kKlPart * 4 : 0));
    w.red = off;   off = align_up(off + (size_t)w.red_blocks * 8);
    w.bytes = off;
    return w;
}

template <typename T, int D, int DI, int G>
static hipError_t launch_kl_t(const LaunchDims& d0, const void* q, const void* k, const void* q_idx,
                              const void* k_idx, const int32_t* block_idx0, const float* lse, float scale,
                              float iscale, float* kl_rows, float* kl_sum, float* index_lse, unsigned char* ws,
                              hipStream_t st) {
    const KlWorkspace L = kl_workspace_layout(d0);
    // Other block sizes: the rows' selections over 128-token blocks, with the
    // half masks of 64-token selections.
    const bool xp = d0.Bk != 128, hm = d0.Bk == 64;
    const LaunchDims d = as_128(d0);
    if (xp) launch_expand(d0, block_idx0, ws, L.ex, st);
    const int32_t* block_idx = xp ? reinterpret_cast<const int32_t*>(ws + L.ex.ids) : block_idx0;
    const uint8_t* hmask = reinterpret_cast<const uint8_t*>(ws + L.ex.hmask);
    const uint8_t* info = reinterpret_cast<const uint8_t*>(ws + L.ex.info);
    const float scale_log2 = scale * 1.4426950408889634f;
    const int KP = d.k > 1 ? d.k - 1 : 1;
    const T* tq = static_cast<const T*>(q);
    const T* tk = static_cast<const T*>(k);
    const T* tqi = static_cast<const T*>(q_idx);
    const T* tki = static_cast<const T*>(k_idx);
    float* part = nullptr;
    if (L.lists.has_nonlocal) {
        launch_build_lists(d, 0, d.N, block_idx, ws, L.lists, st);
        part = reinterpret_cast<float*>(ws + L.part);
        const size_t grid = (L.lists.max_items + 63) / 64 * 64;
        const int32_t* list = reinterpret_cast<const int32_t*>(ws + L.lists.list);
        const int4* items = reinterpret_cast<const int4*>(ws + L.lists.items);
        const int32_t* total = reinterpret_cast<const int32_t*>(ws + L.lists.total);
        if (hm)
            hipLaunchKernelGGL((kl_nonlocal_kernel<T, D, DI, G, true>), dim3((unsigned)grid), dim3(256), 0, st, tq, tk,
                               tqi, tki, lse, list, items, total, part, hmask, d.N, d.Hkv, d.nb, windows(d), KP,
                               scale_log2, iscale, L.lists.max_entries);
        else
            hipLaunchKernelGGL((kl_nonlocal_kernel<T, D, DI, G, false>), dim3((unsigned)grid), dim3(256), 0, st, tq,
                               tk, tqi, tki, lse, list, items, total, part, hmask, d.N, d.Hkv, d.nb, windows(d), KP,
                               scale_log2, iscale, L.lists.max_entries);
    }
    const dim3 cgrid((unsigned)(d.nb * d.B * d.Hkv));
    const int kk = L.lists.has_nonlocal ? d.k : 1;
    if (xp)
        hipLaunchKernelGGL((kl_local_combine_kernel<T, D, DI, G, true>), cgrid, dim3(256), 0, st, tq, tk, tqi, tki, lse,
                           part, info, kl_rows, index_lse, d.B, d.N, d.Hkv, d.nb, kk, KP, scale_log2, iscale);
    else
        hipLaunchKernelGGL((kl_local_combine_kernel<T, D, DI, G, false>), cgrid, dim3(256), 0, st, tq, tk, tqi, tki,
                           lse, part, info, kl_rows, index_lse, d.B, d.N, d.Hkv, d.nb, kk, KP, scale_log2, iscale);
    double* red = reinterpret_cast<double*>(ws + L.red);
    const size_t rows = (size_t)d.B * d.Hkv * d.N;
    hipLaunchKernelGGL(kl_reduce_partial, dim3(L.red_blocks), dim3(kRedThreads), 0, st, kl_rows, rows, red);
    hipLaunchKernelGGL(kl_reduce_final, dim3(1), dim3(kRedThreads), 0, st, red, L.red_blocks, kl_sum);
    return hipGetLastError();
}

template <typename T, int D, int DI>
static hipError_t launch_kl_g(const LaunchDims& d, const void* q, const void* k, const void* qi, const void* ki,
                              const int32_t* bi, const float* lse, float sc, float isc, float* rows, float* sum,
                              float* ilse, unsigned char* ws, hipStream_t st) {
    switch (d.G) {
        case 1: return launch_kl_t<T, D, DI, 1>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
        case 2: return launch_kl_t<T, D, DI, 2>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
        case 4: return launch_kl_t<T, D, DI, 4>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
        case 8: return launch_kl_t<T, D, DI, 8>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
        case 16: return launch_kl_t<T, D, DI, 16>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
        default: return launch_kl_t<T, D, DI, 32>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
    }
}

template <typename T>
static hipError_t launch_kl_dt(const LaunchDims& d, const void* q, const void* k, const void* qi, const void* ki,
                               const int32_t* bi, const float* lse, float sc, float isc, float* rows, float* sum,
                               float* ilse, unsigned char* ws, hipStream_t st) {
    if (d.D == 128 && d.Di == 128)
        return launch_kl_g<T, 128, 128>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
    if (d.D == 128) return launch_kl_g<T, 128, 64>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
    if (d.Di == 128) return launch_kl_g<T, 64, 128>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
    return launch_kl_g<T, 64, 64>(d, q, k, qi, ki, bi, lse, sc, isc, rows, sum, ilse, ws, st);
}

size_t dense_kl_workspace_bytes(const LaunchDims& d) {
    return align_up((size_t)red_blocks_for((size_t)d.B * d.Hkv * d.N) * 8);
}

template <typename T, int D, int DI, int G>
static void launch_dense_kl_t(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                              const void* k_idx, const float* lse, float scale_log2, float iscale, float* kl_rows,
                              float* index_lse, hipStream_t st) {
    constexpr int kTiles = kBlock * G / 32;
    const int parts = (kTiles + kDenseKlWaves - 1) / kDenseKlWaves;
    constexpr int BUF = SwzTile<T, D>::BYTES + SwzTile<T, DI>::BYTES;
    constexpr int NBUF = 2 * BUF <= 160 * 1024 ? 2 : 1;
    const size_t units = (size_t)d.nb * d.B * d.Hkv;
    const size_t grid = (units + 7) / 8 * 8 * parts;
    hipLaunchKernelGGL((dense_kl_kernel<T, D, DI, G, NBUF>), dim3((unsigned)grid), dim3(kDenseKlWaves * kWave), 0,
                       st, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(q_idx),
                       static_cast<const T*>(k_idx), lse, kl_rows, index_lse, d.B, d.N, d.Hkv, d.nb, parts,
                       scale_log2, iscale);
}

template <typename T, int D, int DI>
static void launch_dense_kl_g(const LaunchDims& d, const void* q, const void* k, const void* qi, const void* ki,
                              const float* lse, float sl2, float isc, float* rows, float* ilse, hipStream_t st) {
    switch (d.G) {
        case 1: launch_dense_kl_t<T, D, DI, 1>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st); break;
        case 2: launch_dense_kl_t<T, D, DI, 2>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st); break;
        case 4: launch_dense_kl_t<T, D, DI, 4>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st); break;
        case 8: launch_dense_kl_t<T, D, DI, 8>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st); break;
        case 16: launch_dense_kl_t<T, D, DI, 16>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st); break;
        default: launch_dense_kl_t<T, D, DI, 32>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st); break;
    }
}

template <typename T>
static void launch_dense_kl_dt(const LaunchDims& d, const void* q, const void* k, const void* qi, const void* ki,
                               const float* lse, float sl2, float isc, float* rows, float* ilse, hipStream_t st) {
    if (d.D == 128 && d.Di == 128) launch_dense_kl_g<T, 128, 128>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st);
    else if (d.D == 128) launch_dense_kl_g<T, 128, 64>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st);
    else if (d.Di == 128) launch_dense_kl_g<T, 64, 128>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st);
    else launch_dense_kl_g<T, 64, 64>(d, q, k, qi, ki, lse, sl2, isc, rows, ilse, st);
}

hipError_t launch_dense_kl_align(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                                 const void* k_idx, const float* lse, float scale, float index_scale, float* kl_rows,
                                 float* kl_sum, float* index_lse, void* ws, hipStream_t st) {
    if (d.B == 0 || d.N == 0) {
        hipLaunchKernelGGL(kl_reduce_final, dim3(1), dim3(kRedThreads), 0, st, (const double*)nullptr, 0, kl_sum);
        return hipGetLastError();
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    if (d.dtype == 0)
        launch_dense_kl_dt<bf16_t>(d, q, k, q_idx, k_idx, lse, scale_log2, index_scale, kl_rows, index_lse, st);
    else
        launch_dense_kl_dt<float>(d, q, k, q_idx, k_idx, lse, scale_log2, index_scale, kl_rows, index_lse, st);
    const size_t rows = (size_t)d.B * d.Hkv * d.N;
    const int red_blocks = red_blocks_for(rows);
    double* red = static_cast<double*>(ws);
    hipLaunchKernelGGL(kl_reduce_partial, dim3(red_blocks), dim3(kRedThreads), 0, st, kl_rows, rows, red);
    hipLaunchKernelGGL(kl_reduce_final, dim3(1), dim3(kRedThreads), 0, st, red, red_blocks, kl_sum);
    return hipGetLastError();
}

hipError_t launch_kl_align(const LaunchDims& d, const void* q, const void* k, const void* q_idx, const void* k_idx,
                           const int32_t* block_idx, const float* lse, float scale, float index_scale,
                           float* kl_rows, float* kl_sum, float* index_lse, void* ws, hipStream_t st) {
    if (d.B == 0 || d.N == 0) {
        hipLaunchKernelGGL(kl_reduce_final, dim3(1), dim3(kRedThreads), 0, st, (const double*)nullptr, 0, kl_sum);
        return hipGetLastError();
    }
    unsigned char* w = static_cast<unsigned char*>(ws);
    if (d.dtype == 0)
        return launch_kl_dt<bf16_t>(d, q, k, q_idx, k_idx, block_idx, lse, scale, index_scale, kl_rows, kl_sum,
                                    index_lse, w, st);
    return launch_kl_dt<float>(d, q, k, q_idx, k_idx, block_idx, lse, scale, index_scale, kl_rows, kl_sum, index_lse,
                               w, st);
}

}  // namespace msa
