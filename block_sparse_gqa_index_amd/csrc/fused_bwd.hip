// Fused backward of both branches over the cached block indices (bf16 inputs,
// fp32 accumulation), gfx950: the main branch's dQ, dK, dV for the loss
// <dO, O> and the KL term's dq_idx, dk_idx for the loss sum_rows w_row KL_row,
// from one pass over the selected blocks in which the main-branch scores S
// (and so P) are computed once and serve both the main gradient and the
// teacher of the KL term.
//
// Method: the Flash-MSA article (tech.kuratif.com), paragraph on the backward:
// the proxy (index) and main attention gradients are fused, over the block
// indices cached by the forward, linear in N; "Accelerating Million-Token
// Training with Sparse Attention Kernels" (DeepHorus) describes the same fused
// backward as what makes million-token training possible. The MSA article on
// 7minutos.es ("Cómo funcionan las dos ramas", "Cómo se entrena MSA") defines
// the forward that is differentiated and the KL loss, whose gradient is stopped
// at the index branch's input (the teacher is a constant). Per row with
// selected tokens T, z = sigma q.k, u = q_idx.k_idx:
//   P = exp(z - LSE),  dV_t = sum P dO,  dS = P (dO.v_t - <dO, O>),
//   dQ = sigma sum_t dS k_t,  dK_t = sigma sum dS q,
//   p_t = mean over the group's heads of P,  s_t = exp(c u_t - LSE_u),
//   dU_t = w c (s_t - p_t),  dq_idx = sum_t dU_t k_idx_t,  dk_idx_t = sum dU_t q_idx.
//
// Work is key-block-outer over the position-sorted lists, one 64K-position
// window of query rows at a time, so the per-(row, slot) dQ and dq_idx partials
// only ever hold one window (the workspace stays bounded at a million tokens):
//   per window: fused_bwd_kernel on the window's non-local items, then on the
//   causal local blocks of its query blocks; fused_dkv_reduce and
//   fused_dki_reduce add the window's per-item partials, in item order, to fp32
//   running sums per key block (written as bf16 after the last window);
//   dq_combine_kernel sums the window's rows' slot partials.
// Every sum runs in a fixed order, so the gradients are deterministic.
//
// Matrix-core orientation as in the separate backward kernels: S = Q K^T,
// dP = dO V^T and U = Q_idx K_idx^T with A = tile rows (LDS) and B = the wave's
// 32 keys (VGPRs) leave one key per lane and 16 rows in its accumulators; P, dS
// and dU in that layout are the B operands of dV^T = dO^T P, dK^T = Q^T dS and
// dk_idx^T = Q_idx^T (dU / G) against transposed tiles staged with the matching
// row permutation; dQ and dq_idx contract over keys, so dS and dU go through
// LDS and the A operands are the per-block K^T and K_idx^T copies.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"
#include "msa_bwd_tiles.h"

#include <algorithm>

namespace msa {

// v_mfma_f32_16x16x32_bf16: A (16 x 32) lane l supplies row l % 16 and
// contraction elements 8*(l/16) .. +7, B (32 x 16) column l % 16 and the same
// elements, C (16 x 16) lane l holds column l % 16, rows 4*(l/16) + r, r < 4.
__device__ __forceinline__ void mma1632(floatx4& c, const Op8<bf16_t>& a, const Op8<bf16_t>& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// Row order of the transposed tiles (the contraction over a tile's 32 rows):
// lane group q = l / 16 holds rows 4q .. 4q+3 (first row half) and 16 + 4q ..
// 16 + 4q + 3 (second) in its accumulators, so chunk q of a transposed row
// (8 positions, 16 bytes) holds exactly those rows: row m sits at position
// 8 * ((m % 16) / 4) + 4 * (m / 16) + m % 4.
__device__ __forceinline__ int fused_tpos(int m) { return 8 * ((m & 15) >> 2) + 4 * (m >> 4) + (m & 3); }

// One staged 32-row tile: query, output-gradient and index-query rows, natural
// and transposed (chunk-major, in the row order above), and the rows' scalars.
template <int D, int DI>
struct FusedTile {
    using QT = SwzTile<bf16_t, D>;    // [32 rows][D]
    using IT = SwzTile<bf16_t, DI>;   // [32 rows][DI]
    using QCT = ColTile<D>;           // [D][32 rows, permuted]
    using ICT = ColTile<DI>;          // [DI][32 rows, permuted]
    unsigned char q[32 * QT::ROWB], dout[32 * QT::ROWB], qi[32 * IT::ROWB];
    unsigned char qt[QCT::BYTES], dot[QCT::BYTES], qit[ICT::BYTES];
    float lse2[32], dl[32], lseu2[32], wkl[32];
    int pos[32], slot[32];
};

// LDS of one work-group: two tile buffers (tile t is computed from one while
// tile t + 1 is written into the other), the dS and dU tiles, the key block's
// K_idx^T (A operand of dq_idx; K^T, that of dQ, stays in registers), the
// item's list entries.
template <int D, int DI>
struct FusedLds {
    using DsT = SwzTile<bf16_t, kBlock>;   // [rows][128 keys, permuted]: dS, dU, K_idx^T
    FusedTile<D, DI> tile[2];
    unsigned char ds[32 * DsT::ROWB], du[32 * DsT::ROWB];
    unsigned char kit[DI * DsT::ROWB];
    int entries[kSegBwd];
};

// Staging of one tile in quarter units: 4 rows x 16 bytes (dims 8*dc .. +7) of
// one tensor (Q, dO, Q_idx, in that order), every quarter stored natural and
// transposed.
template <int D, int DI>
struct FusedUnits {
    static constexpr int NQ = 8 * (D / 8), NI = 8 * (DI / 8), N = 2 * NQ + NI;
};
struct FusedQuarter {
    u32x4 x[4];
};

template <int D, int DI, int G, bool LOCAL>
__device__ __forceinline__ void fused_stage_load(FusedQuarter& su, const BwdItem<LOCAL>& it, int t, int u,
                                                 const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
                                                 const bf16_t* __restrict__ q_idx, int N, int Hkv) {
    constexpr int NQ = FusedUnits<D, DI>::NQ, PPT = 32 / G;
    const int tensor = u < NQ ? 0 : (u < 2 * NQ ? 1 : 2);
    const int v = u - tensor * NQ;
    const int rq = v & 7, dc = v >> 3;   // the row quarter varies fastest across lanes
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * rq + e;
        const int pe = t * PPT + m / G;
        su.x[e] = u32x4{0u, 0u, 0u, 0u};
        if (pe < it.count) {
            int i, s;
            it.entry(pe, i, s);
            const bf16_t* src = tensor == 2 ? q_idx + (((size_t)it.b * N + i) * Hkv + it.g) * DI + dc * 8
                                            : (tensor ? dout : q) + (((size_t)it.b * N + i) * Hkv * G + it.g * G + m % G) * D +
                                                  dc * 8;
            su.x[e] = *reinterpret_cast<const u32x4*>(src);
        }
    }
}

template <int D, int DI>
__device__ __forceinline__ void fused_stage_store(const FusedQuarter& su, FusedTile<D, DI>& sh, int u) {
    constexpr int NQ = FusedUnits<D, DI>::NQ;
    using F = FusedTile<D, DI>;
    const int tensor = u < NQ ? 0 : (u < 2 * NQ ? 1 : 2);
    const int v = u - tensor * NQ;
    const int rq = v & 7, dc = v >> 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * rq + e;
        unsigned char* dst = tensor == 2 ? sh.qi + F::IT::offset(m, dc * 16)
                                         : (tensor ? sh.dout : sh.q) + F::QT::offset(m, dc * 16);
        *reinterpret_cast<u32x4*>(dst) = su.x[e];
    }
    // rows 4rq .. 4rq+3 are 4 consecutive positions of chunk rq % 4 (first or second half of it)
    const int chunk = rq & 3, sub = (rq >> 2) * 8;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        uint2 y;
        const uint32_t sel = dd % 2 ? 0x07060302u : 0x05040100u;   // the 16-bit element dd of two rows
        y.x = __builtin_amdgcn_perm(su.x[1][dd / 2], su.x[0][dd / 2], sel);
        y.y = __builtin_amdgcn_perm(su.x[3][dd / 2], su.x[2][dd / 2], sel);
        unsigned char* dst = tensor == 2 ? sh.qit + F::ICT::offset(dc * 8 + dd, chunk)
                                         : (tensor ? sh.dot : sh.qt) + F::QCT::offset(dc * 8 + dd, chunk);
        *reinterpret_cast<uint2*>(dst + sub) = y;
    }
}

// Teacher of each of the lane's 8 rows (rh*4 + r: row 16*rh + 4*(l/16) + r):
// the mean of P over the G rows of the row's position (G consecutive rows).
template <int G>
__device__ __forceinline__ void head_mean8(float (&p)[8]) {
    if constexpr (G == 1) return;
    float a[2][4];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
        if constexpr (G == 2) {
            a[rh][0] = a[rh][1] = p[4 * rh] + p[4 * rh + 1];
            a[rh][2] = a[rh][3] = p[4 * rh + 2] + p[4 * rh + 3];
        } else {
            float s = p[4 * rh] + p[4 * rh + 1] + p[4 * rh + 2] + p[4 * rh + 3];
            if constexpr (G >= 8) s += __shfl_xor(s, 16);
            if constexpr (G >= 16) s += __shfl_xor(s, 32);
#pragma unroll
            for (int r = 0; r < 4; ++r) a[rh][r] = s;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float lo = a[0][r], hi = a[1][r];
        if constexpr (G == 32) lo = hi = lo + hi;
        p[r] = lo * (1.f / G);
        p[4 + r] = hi * (1.f / G);
    }
}

// Window of the fused backward: query positions [p0, p0 + len) and the slots
// of its work items (see fused_bwd_workspace_layout).
struct FusedWindow {
    int w, p0, len, qb0;   // window index, first position, positions, first query block
    int bound;             // work-item slots per (b, g)
};

constexpr int kFusedWaves = 8;

// One 8-wave work-group (two waves per SIMD) per work item: the window's
// non-local rows of key block j (LOCAL = false), or the rows of query block j
// against their own block under the causal mask (LOCAL = true). Wave w owns
// keys 16w .. 16w+15 of the block for S, dP, U and the dK, dV, dk_idx sums,
// and dims 16w .. 16w+15 of the dQ and dq_idx tiles.
template <int D, int DI, int G, bool LOCAL>
__global__ __launch_bounds__(64 * kFusedWaves, 1) void fused_bwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ q_idx, const bf16_t* __restrict__ k_idx, const bf16_t* __restrict__ kt,
    const bf16_t* __restrict__ kit, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dl, const float* __restrict__ index_lse, const float* __restrict__ dkl_rows,
    float kl_weight, const int32_t* __restrict__ list, const int4* __restrict__ items,
    const int32_t* __restrict__ item_offsets, const int32_t* __restrict__ total_items, int n_keys,
    bf16_t* __restrict__ dq_part, bf16_t* __restrict__ dqi_part, float* __restrict__ dkv_part,
    float* __restrict__ dki_part, int B, int N, int Hkv, int nb, int nwin, int topk, FusedWindow win,
    float scale_log2, float scale, float iscale) {
    constexpr int PPT = 32 / G, DT = D / 16, DIT = DI / 16, KS = D / 32, KSI = DI / 32;
    constexpr int NST = FusedUnits<D, DI>::N;
    constexpr int NTHR = 64 * kFusedWaves;
    static_assert(NST <= NTHR - 32, "staging threads and the 32 row-scalar threads share the work-group");
    static_assert(DT <= kFusedWaves && DIT <= kFusedWaves, "a wave per 16 dims of dQ and dq_idx");
    __shared__ __align__(16) FusedLds<D, DI> sh;
    using F = FusedTile<D, DI>;
    using L = FusedLds<D, DI>;
    const int Hq = Hkv * G;

    BwdItem<LOCAL> it;
    size_t pidx;   // the item's dK/dV and dk_idx partial slot in this window
    if constexpr (LOCAL) {
        const int nqb = (win.len + kBlock - 1) / kBlock;
        const int x = blockIdx.x;
        it.g = x % Hkv;
        it.b = (x / Hkv) % B;
        it.j = win.qb0 + x / (Hkv * B);
        it.q0 = it.j * kBlock;
        it.count = min(kBlock, N - it.q0);
        it.lslot = min(topk, it.j + 1) - 1;
        it.start = 0;
        it.entries = nullptr;
        pidx = (size_t)B * Hkv * win.bound + ((size_t)it.b * Hkv + it.g) * nqb + (it.j - win.qb0);
    } else {
        // slot x of (b, g): the x-th item of the keys (b, g, window, 0 .. nb-1),
        // which the position-sorted lists keep contiguous
        const int bgi = blockIdx.x / win.bound, x = blockIdx.x % win.bound;
        const int kf = (bgi * nwin + win.w) * nb;
        const int first = item_offsets[kf];
        const int end = kf + nb < n_keys ? item_offsets[kf + nb] : total_items[0];
        if (first + x >= end) return;
        const int4 e = items[first + x];
        it.j = e.x % nb;
        it.g = bgi % Hkv;
        it.b = bgi / Hkv;
        it.start = e.y;
        it.count = e.z;
        it.q0 = 0;
        it.lslot = 0;
        it.entries = sh.entries;
        pidx = blockIdx.x;
        for (int y = threadIdx.x; y < it.count; y += blockDim.x) sh.entries[y] = list[it.start + y];
        __syncthreads();
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ql = lane >> 4, cl = lane & 15;   // lane group (row quarter / contraction octet), column
    const int ntiles = (it.count + PPT - 1) / PPT;

    // The wave's 16 keys as B operands (S, dP, U) and its 16 dims of K^T as the A operand of dQ.
    const int key = 16 * w + cl;
    const int kabs = it.j * kBlock + key;
    Op8<bf16_t> kop[KS], vop[KS], kiop[KSI], ktop[4];
    {
        const size_t roff = (((size_t)it.b * N + kabs) * Hkv + it.g) * D + 8 * ql;
        const size_t ioff = ((size_t)it.b * N + kabs) * DI + 8 * ql;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (kabs < N) {
                kop[s].load(k + roff + 32 * s);
                vop[s].load(v + roff + 32 * s);
            } else {
                kop[s].zero();
                vop[s].zero();
            }
        }
#pragma unroll
        for (int s = 0; s < KSI; ++s) {
            if (kabs < N) kiop[s].load(k_idx + ioff + 32 * s);
            else kiop[s].zero();
        }
        if (w < DT) {
            const bf16_t* src = kt + ((((size_t)it.b * Hkv + it.g) * nb + it.j) * D + 16 * w + cl) * kBlock + 8 * ql;
#pragma unroll
            for (int c = 0; c < 4; ++c) ktop[c].load(src + 32 * c);
        }
    }
    // The block's K_idx^T rows (dims) into LDS, 16 bytes per thread per step.
    {
        using KT = typename L::DsT;
        const bf16_t* srci = kit + ((size_t)it.b * nb + it.j) * DI * kBlock;
        for (int ch = threadIdx.x; ch < DI * KT::CPR; ch += blockDim.x)
            *reinterpret_cast<u32x4*>(sh.kit + KT::offset(ch / KT::CPR, (ch % KT::CPR) * 16)) =
                *reinterpret_cast<const u32x4*>(srci + (size_t)ch * 8);
    }

    floatx4 dkt[DT], dvt[DT], dkit[DIT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dkt[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        dvt[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt) dkit[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    constexpr float kLog2e = 1.4426950408889634f;
    const float iscale_log2 = iscale * kLog2e;
    // Threads 0 .. NST-1 stage one quarter of every tile: tile t + 2 is
    // requested when tile t + 1 is stored, while tile t is on the matrix cores;
    // the last 32 threads load the per-row scalars.
    FusedQuarter su;
    const int u = threadIdx.x;
    const int m_row = (int)threadIdx.x - (NTHR - 32);
    float r_lse = 0.f, r_dl = 0.f, r_lseu = 0.f, r_w = 0.f;
    int r_pos = -1, r_slot = 0;
    auto row_load = [&](int t) {
        if (m_row >= 0) {
            const int m = m_row;
            const int pe = t * PPT + m / G;
            r_pos = -1;
            r_lse = __builtin_inff();
            r_lseu = __builtin_inff();
            r_dl = 0.f;
            r_w = 0.f;
            if (pe < it.count) {
                int i, s;
                it.entry(pe, i, s);
                const size_t hr = ((size_t)it.b * Hq + it.g * G + m % G) * N + i;
                const size_t rr = ((size_t)it.b * Hkv + it.g) * N + i;
                r_pos = i;
                r_slot = s;
                r_lse = lse[hr];   // scaled when stored: no use right after the load
                r_dl = dl[hr];
                r_lseu = index_lse[rr];
                r_w = dkl_rows ? dkl_rows[rr] : 1.f;
            }
        }
    };
    auto store_tile = [&](int t) {
        F& tb = sh.tile[t & 1];
        if (u < NST) fused_stage_store<D, DI>(su, tb, u);
        if (m_row >= 0) {
            tb.lse2[m_row] = r_lse * kLog2e;
            tb.dl[m_row] = r_dl;
            tb.lseu2[m_row] = r_lseu * kLog2e;
            tb.wkl[m_row] = r_w * kl_weight * iscale;
            tb.pos[m_row] = r_pos;
            tb.slot[m_row] = r_slot;
        }
    };
    auto load_tile = [&](int t) {
        if (u < NST) fused_stage_load<D, DI, G, LOCAL>(su, it, t, u, q, dout, q_idx, N, Hkv);
        row_load(t);
    };
    if (ntiles > 0) load_tile(0);
    // Every load issued so far (the key block's operands, tile 0) completes here,
    // so the loop below only ever waits for its own prefetches.
    __builtin_amdgcn_s_waitcnt(0);
    if (ntiles > 0) {
        store_tile(0);
        if (ntiles > 1) load_tile(1);
    }

    for (int t = 0; t < ntiles; ++t) {
        // Tile t is complete in its buffer; the other buffer's readers (tile
        // t - 1) and the dS / dU readers are done.
        __syncthreads();
        if (t + 1 < ntiles) {   // overlaps tile t's math
            store_tile(t + 1);
            if (t + 2 < ntiles) load_tile(t + 2);
        }
        const F& sh_t = sh.tile[t & 1];

        // S = Q K_w^T, dP = dO V_w^T, U = Q_idx K_idx,w^T for both 16-row halves:
        // lane = key 16w + l % 16, accumulators = rows 16 rh + 4 (l / 16) + r.
        floatx4 s[2], dp[2], uu[2];
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
            s[rh] = dp[rh] = uu[rh] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Op8<bf16_t> a, b;
                a.load(sh_t.q + F::QT::offset(16 * rh + cl, (32 * ks + 8 * ql) * 2));
                b.load(sh_t.dout + F::QT::offset(16 * rh + cl, (32 * ks + 8 * ql) * 2));
                mma1632(s[rh], a, kop[ks]);
                mma1632(dp[rh], b, vop[ks]);
            }
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) {
                Op8<bf16_t> a;
                a.load(sh_t.qi + F::IT::offset(16 * rh + cl, (32 * ks + 8 * ql) * 2));
                mma1632(uu[rh], a, kiop[ks]);
            }
        }
        float p[8], ds[8], du[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 16 * (e >> 2) + 4 * ql + (e & 3);
            float pr = exp2_hw(fmaf(s[e >> 2][e & 3], scale_log2, -sh_t.lse2[m]));
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) pr = 0.f;   // also the rows past the item (pos = -1)
            }
            p[e] = pr;
            ds[e] = pr * (dp[e >> 2][e & 3] - sh_t.dl[m]);
            du[e] = pr;
        }
        head_mean8<G>(du);   // the teacher of each row's position
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 16 * (e >> 2) + 4 * ql + (e & 3);
            float st = exp2_hw(fmaf(uu[e >> 2][e & 3], iscale_log2, -sh_t.lseu2[m]));
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) st = 0.f;
            }
            du[e] = sh_t.wkl[m] * (st - du[e]);
        }
        // dV^T += dO^T P, dK^T += Q^T dS and dk_idx^T += Q_idx^T (dU / G) (every
        // position's G replicated rows count once): the lane's 8 values are the
        // contraction elements of its key column, in the transposed tiles' row order.
        {
            Op8<bf16_t> bp, bds, bdu;
            PType<bf16_t>::pack(bp, p);
            PType<bf16_t>::pack(bds, ds);
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = du[e] * (1.f / G);
            PType<bf16_t>::pack(bdu, x);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                Op8<bf16_t> a, b;
                a.load(sh_t.dot + F::QCT::offset(16 * dt + cl, ql));
                b.load(sh_t.qt + F::QCT::offset(16 * dt + cl, ql));
                mma1632(dvt[dt], a, bp);
                mma1632(dkt[dt], b, bds);
            }
#pragma unroll
            for (int dt = 0; dt < DIT; ++dt) {
                Op8<bf16_t> a;
                a.load(sh_t.qit + F::ICT::offset(16 * dt + cl, ql));
                mma1632(dkit[dt], a, bdu);
            }
        }
        // dS and dU -> LDS as [row][permuted key] for the dQ and dq_idx products.
        {
            uint16_t* dsl = reinterpret_cast<uint16_t*>(sh.ds);
            uint16_t* dul = reinterpret_cast<uint16_t*>(sh.du);
            const int pk = perm16(key);
#pragma unroll
            for (int e = 0; e < 8; e += 2) {   // rows m and m + 1: one conversion, two 16-bit stores
                const int m = 16 * (e >> 2) + 4 * ql + (e & 3);
                const uint32_t a2 = pack_bf16x2(ds[e], ds[e + 1]);
                const uint32_t b2 = pack_bf16x2(du[e], du[e + 1]);
                dsl[L::DsT::offset(m, pk * 2) / 2] = (uint16_t)(a2 & 0xffffu);
                dsl[L::DsT::offset(m + 1, pk * 2) / 2] = (uint16_t)(a2 >> 16);
                dul[L::DsT::offset(m, pk * 2) / 2] = (uint16_t)(b2 & 0xffffu);
                dul[L::DsT::offset(m + 1, pk * 2) / 2] = (uint16_t)(b2 >> 16);
            }
        }
        __syncthreads();
        // dQ^T (dims 16w.., rows) = K^T dS^T and dq_idx^T = K_idx^T dU^T over the
        // block's 128 keys: lane = row 16 rh + l % 16, accumulators = dims 16w + 4 (l / 16) + r.
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
            const int row = 16 * rh + cl;
            const int i = sh_t.pos[row];
            const size_t prow =
                i >= 0 ? (((size_t)it.b * Hkv + it.g) * win.len + (i - win.p0)) * topk + sh_t.slot[row] : 0;
            if (w < DT) {
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    Op8<bf16_t> b;
                    b.load(sh.ds + L::DsT::offset(row, (32 * c + 8 * ql) * 2));
                    mma1632(acc, ktop[c], b);
                }
                if (i >= 0) {
                    // partial of (row, slot), head row % G: [G][D] bf16 in natural dim order
                    bf16_t* dst = dq_part + prow * G * D + (size_t)(row % G) * D + 16 * w + 4 * ql;
                    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0] * scale, acc[1] * scale),
                                                                pack_bf16x2(acc[2] * scale, acc[3] * scale));
                }
            }
            if (w < DIT) {
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    Op8<bf16_t> a, b;
                    a.load(sh.kit + L::DsT::offset(16 * w + cl, (32 * c + 8 * ql) * 2));
                    b.load(sh.du + L::DsT::offset(row, (32 * c + 8 * ql) * 2));
                    mma1632(acc, a, b);
                }
                if (i >= 0 && row % G == 0) {   // the position's first head row writes it
                    bf16_t* dst = dqi_part + prow * DI + 16 * w + 4 * ql;
                    *reinterpret_cast<uint2*>(dst) =
                        make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
                }
            }
        }
    }

    // The item's partials: dK, dV [2][128 keys][D] fp32 (dK scaled by sigma), dk_idx [128 keys][DI] fp32.
    float* pk = dkv_part + pidx * 2 * kBlock * D + (size_t)key * D;
    float* pv = pk + (size_t)kBlock * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        floatx4 xk;
#pragma unroll
        for (int e = 0; e < 4; ++e) xk[e] = dkt[dt][e] * scale;
        *reinterpret_cast<floatx4*>(pk + 16 * dt + 4 * ql) = xk;
        *reinterpret_cast<floatx4*>(pv + 16 * dt + 4 * ql) = dvt[dt];
    }
    float* pki = dki_part + pidx * kBlock * DI + (size_t)key * DI;
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt) *reinterpret_cast<floatx4*>(pki + 16 * dt + 4 * ql) = dkit[dt];
}

// One work-group per (b, g, key block j < the window's last query block): the
// window's partials of key block j (its local item if its query block is in
// the window, then its non-local items in list order) added to the running
// fp32 sums; the first window that reaches j (the one holding its query block)
// starts the sums, the last window writes dK and dV in bf16.
template <int D>
__global__ __launch_bounds__(256) void fused_dkv_reduce_kernel(
    const float* __restrict__ dkv_part, const int32_t* __restrict__ counts, const int32_t* __restrict__ item_offsets,
    float* __restrict__ acc_dkv, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int B, int N, int Hkv, int nb,
    int nwin, int seg, FusedWindow win, int nbw, int last, int has_lists) {
    constexpr int PER = 2 * kBlock * D / 4 / 256;   // float4 per thread (dK and dV)
    const int j = blockIdx.x % nbw;
    const int bg = blockIdx.x / nbw;
    const int g = bg % Hkv, b = bg / Hkv;
    const int nqb = (win.len + kBlock - 1) / kBlock;
    const bool starts = j >= win.qb0;   // the block's query block is in this window
    const size_t key = ((size_t)bg * nwin + win.w) * nb + j;
    const int kf = (bg * nwin + win.w) * nb;
    const int n = has_lists ? (counts[key] + seg - 1) / seg : 0;
    if (n == 0 && !starts && !last) return;   // nothing new for this block: its running sum stays as it is
    floatx4 sum[PER];
    float* accp = acc_dkv + (((size_t)bg * nb + j) * 2 * kBlock * D);
    auto add = [&](const float* p) {
#pragma unroll
        for (int x = 0; x < PER; ++x)
            sum[x] += __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p) + threadIdx.x + 256 * x);
    };
#pragma unroll
    for (int x = 0; x < PER; ++x) sum[x] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (!starts) add(accp);
    else add(dkv_part + ((size_t)B * Hkv * win.bound + (size_t)bg * nqb + (j - win.qb0)) * 2 * kBlock * D);
    if (n > 0) {
        const int first = item_offsets[key] - item_offsets[kf];   // the item's slot in this window's partials
        for (int y = 0; y < n; ++y) add(dkv_part + ((size_t)bg * win.bound + first + y) * 2 * kBlock * D);
    }
    if (!last) {
#pragma unroll
        for (int x = 0; x < PER; ++x) reinterpret_cast<floatx4*>(accp)[threadIdx.x + 256 * x] = sum[x];
        return;
    }
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int f = (threadIdx.x + 256 * x) * 4;   // element of [2][128][D]
        const int which = f / (kBlock * D);
        const int kk = (f / D) % kBlock, d = f % D;
        const int t = j * kBlock + kk;
        if (t < N) {
            bf16_t* dst = (which ? dv : dk) + (((size_t)b * N + t) * Hkv + g) * D + d;
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(sum[x][0], sum[x][1]),
                                                        pack_bf16x2(sum[x][2], sum[x][3]));
        }
    }
}

// One work-group per (b, key block j < the window's last query block): dk_idx
// of the block's keys, the same running sum over the groups in order (each
// group's local item, then its items of this window).
template <int DI>
__global__ __launch_bounds__(256) void fused_dki_reduce_kernel(
    const float* __restrict__ dki_part, const int32_t* __restrict__ counts, const int32_t* __restrict__ item_offsets,
    float* __restrict__ acc_dki, bf16_t* __restrict__ dk_idx, int B, int N, int Hkv, int nb, int nwin, int seg,
    FusedWindow win, int nbw, int last, int has_lists) {
    constexpr int PER = kBlock * DI / 4 / 256;
    const int j = blockIdx.x % nbw;
    const int b = blockIdx.x / nbw;
    const int nqb = (win.len + kBlock - 1) / kBlock;
    const bool starts = j >= win.qb0;
    floatx4 sum[PER];
    float* accp = acc_dki + ((size_t)b * nb + j) * kBlock * DI;
    auto add = [&](const float* p) {
#pragma unroll
        for (int x = 0; x < PER; ++x)
            sum[x] += __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p) + threadIdx.x + 256 * x);
    };
#pragma unroll
    for (int x = 0; x < PER; ++x) sum[x] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (!starts) add(accp);
    for (int g = 0; g < Hkv; ++g) {
        const int bg = b * Hkv + g;
        if (starts) add(dki_part + ((size_t)B * Hkv * win.bound + (size_t)bg * nqb + (j - win.qb0)) * kBlock * DI);
        if (!has_lists) continue;
        const size_t key = ((size_t)bg * nwin + win.w) * nb + j;
        const int kf = (bg * nwin + win.w) * nb;
        const int n = (counts[key] + seg - 1) / seg;
        const int first = item_offsets[key] - item_offsets[kf];
        for (int y = 0; y < n; ++y) add(dki_part + ((size_t)bg * win.bound + first + y) * kBlock * DI);
    }
    if (!last) {
#pragma unroll
        for (int x = 0; x < PER; ++x) reinterpret_cast<floatx4*>(accp)[threadIdx.x + 256 * x] = sum[x];
        return;
    }
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int f = (threadIdx.x + 256 * x) * 4;
        const int kk = f / DI, d = f % DI;
        const int t = j * kBlock + kk;
        if (t < N)
            *reinterpret_cast<uint2*>(dk_idx + ((size_t)b * N + t) * DI + d) =
                make_uint2(pack_bf16x2(sum[x][0], sum[x][1]), pack_bf16x2(sum[x][2], sum[x][3]));
    }
}

// -------------------------------------------------------------------- host --

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Work-item slots per (b, g) in one window: every key's items (a list entry per
// kept non-local block of the window's rows, cut every kSegBwd) fit in
// ceil(W (k-1) / kSegBwd) + nb.
static int fused_bound(const LaunchDims& d) {
    const size_t W = (size_t)std::min(d.N, kWindow);
    const size_t kp = d.k > 1 ? (size_t)(d.k - 1) : 0;
    return (int)((W * kp + kSegBwd - 1) / kSegBwd + (size_t)d.nb);
}

FusedBwdWorkspace fused_bwd_workspace_layout(const LaunchDims& d) {
    FusedBwdWorkspace w{};
    const size_t W = (size_t)std::min(d.N, kWindow);
    const size_t bg = (size_t)d.B * d.Hkv;
    size_t off = 0;
    w.kt = off;    off = align_up(off + bg * d.nb * d.D * kBlock * 2);
    w.kit = off;   off = align_up(off + (size_t)d.B * d.nb * d.Di * kBlock * 2);
    w.dl = off;    off = align_up(off + (size_t)d.B * d.Hq() * d.N * 4);
    w.lists = list_layout(d, off, kSegBwd, true);
    off = w.lists.end;
    w.bound = w.lists.has_nonlocal ? fused_bound(d) : 0;
    w.items = bg * w.bound + bg * ((W + kBlock - 1) / kBlock);   // non-local slots, then local ones
    w.dq_part = off;   off = align_up(off + bg * W * d.k * d.G * d.D * 2);
    w.dqi_part = off;  off = align_up(off + bg * W * d.k * d.Di * 2);
    w.dkv_part = off;  off = align_up(off + w.items * 2 * kBlock * d.D * 4);
    w.dki_part = off;  off = align_up(off + w.items * kBlock * d.Di * 4);
    const bool multi = windows(d) > 1;   // running sums across windows
    w.acc_dkv = off;   off = align_up(off + (multi ? bg * d.nb * 2 * kBlock * d.D * 4 : 0));
    w.acc_dki = off;   off = align_up(off + (multi ? (size_t)d.B * d.nb * kBlock * d.Di * 4 : 0));
    w.bytes = off;
    return w;
}

template <int D, int DI, int G>
static hipError_t launch_fused_t(const LaunchDims& d, const FusedBwdArgs& a, unsigned char* ws, hipStream_t st) {
    const FusedBwdWorkspace L = fused_bwd_workspace_layout(d);
    const bf16_t* tq = static_cast<const bf16_t*>(a.q);
    const bf16_t* tk = static_cast<const bf16_t*>(a.k);
    const bf16_t* tv = static_cast<const bf16_t*>(a.v);
    const bf16_t* tqi = static_cast<const bf16_t*>(a.q_idx);
    const bf16_t* tki = static_cast<const bf16_t*>(a.k_idx);
    const bf16_t* tdo = static_cast<const bf16_t*>(a.dout);
    bf16_t* kt = reinterpret_cast<bf16_t*>(ws + L.kt);
    bf16_t* kit = reinterpret_cast<bf16_t*>(ws + L.kit);
    float* dl = reinterpret_cast<float*>(ws + L.dl);
    bf16_t* dq_part = reinterpret_cast<bf16_t*>(ws + L.dq_part);
    bf16_t* dqi_part = reinterpret_cast<bf16_t*>(ws + L.dqi_part);
    float* dkv_part = reinterpret_cast<float*>(ws + L.dkv_part);
    float* dki_part = reinterpret_cast<float*>(ws + L.dki_part);
    float* acc_dkv = reinterpret_cast<float*>(ws + L.acc_dkv);
    float* acc_dki = reinterpret_cast<float*>(ws + L.acc_dki);
    const float scale_log2 = a.scale * 1.4426950408889634f;
    const int nwin = windows(d);

    hipError_t e = launch_transpose_kv(d, a.k, kt, st);
    if (e != hipSuccess) return e;
    LaunchDims di = d;   // k_idx as a one-head [B, N, 1, Di] tensor
    di.Hkv = 1;
    di.G = 1;
    di.D = d.Di;
    e = launch_transpose_kv(di, a.k_idx, kit, st);
    if (e != hipSuccess) return e;
    launch_bwd_delta(d, a.o, a.dout, dl, st);
    const bool nonlocal = L.lists.has_nonlocal;
    if (nonlocal) launch_build_lists(d, 0, d.N, a.block_idx, ws, L.lists, st);
    const int32_t* list = reinterpret_cast<const int32_t*>(ws + L.lists.list);
    const int4* items = reinterpret_cast<const int4*>(ws + L.lists.items);
    const int32_t* counts = reinterpret_cast<const int32_t*>(ws + L.lists.counts);
    const int32_t* item_offsets = reinterpret_cast<const int32_t*>(ws + L.lists.item_offsets);
    const int32_t* total = reinterpret_cast<const int32_t*>(ws + L.lists.total);
    const int bg = d.B * d.Hkv;
    for (int w = 0; w < nwin; ++w) {
        FusedWindow win;
        win.w = w;
        win.p0 = w * kWindow;
        win.len = std::min(d.N - win.p0, kWindow);
        win.qb0 = win.p0 / kBlock;
        win.bound = L.bound;
        const int nqb = (win.len + kBlock - 1) / kBlock;
        const int nbw = win.qb0 + nqb;   // key blocks the window's rows can keep
        const int last = w == nwin - 1;
        if (nonlocal)
            hipLaunchKernelGGL((fused_bwd_kernel<D, DI, G, false>), dim3((unsigned)(bg * L.bound)),
                               dim3(64 * kFusedWaves), 0, st,
                               tq, tk, tv, tqi, tki, kt, kit, tdo, a.lse, dl, a.index_lse, a.dkl_rows, a.kl_weight,
                               list, items, item_offsets, total, (int)L.lists.n_keys, dq_part, dqi_part, dkv_part,
                               dki_part, d.B, d.N, d.Hkv, d.nb, nwin, d.k, win, scale_log2, a.scale, a.iscale);
        hipLaunchKernelGGL((fused_bwd_kernel<D, DI, G, true>), dim3((unsigned)(bg * nqb)), dim3(64 * kFusedWaves), 0,
                           st, tq, tk,
                           tv, tqi, tki, kt, kit, tdo, a.lse, dl, a.index_lse, a.dkl_rows, a.kl_weight, nullptr,
                           nullptr, nullptr, nullptr, 0, dq_part, dqi_part, dkv_part, dki_part, d.B, d.N, d.Hkv, d.nb,
                           nwin, d.k, win, scale_log2, a.scale, a.iscale);
        hipLaunchKernelGGL((fused_dkv_reduce_kernel<D>), dim3((unsigned)(bg * nbw)), dim3(256), 0, st, dkv_part,
                           counts, item_offsets, acc_dkv, static_cast<bf16_t*>(a.dk), static_cast<bf16_t*>(a.dv), d.B,
                           d.N, d.Hkv, d.nb, nwin, kSegBwd, win, nbw, last, nonlocal ? 1 : 0);
        hipLaunchKernelGGL((fused_dki_reduce_kernel<DI>), dim3((unsigned)(d.B * nbw)), dim3(256), 0, st, dki_part,
                           counts, item_offsets, acc_dki, static_cast<bf16_t*>(a.dk_idx), d.B, d.N, d.Hkv, d.nb, nwin,
                           kSegBwd, win, nbw, last, nonlocal ? 1 : 0);
        const int64_t units = (int64_t)bg * win.len * G * (D / 16);
        hipLaunchKernelGGL((dq_combine_kernel<D, G, true>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st,
                           dq_part,
                           static_cast<bf16_t*>(a.dq), units, d.N, d.Hkv, d.k, win.p0, win.len, win.len);
        const int64_t iunits = (int64_t)bg * win.len * (DI / 16);
        hipLaunchKernelGGL((dq_combine_kernel<DI, 1, true>), dim3((unsigned)((iunits + 255) / 256)), dim3(256), 0, st,
                           dqi_part, static_cast<bf16_t*>(a.dq_idx), iunits, d.N, d.Hkv, d.k, win.p0, win.len,
                           win.len);
    }
    return hipGetLastError();
}

template <int D, int DI>
static hipError_t launch_fused_g(const LaunchDims& d, const FusedBwdArgs& a, unsigned char* ws, hipStream_t st) {
    switch (d.G) {
        case 1: return launch_fused_t<D, DI, 1>(d, a, ws, st);
        case 2: return launch_fused_t<D, DI, 2>(d, a, ws, st);
        case 4: return launch_fused_t<D, DI, 4>(d, a, ws, st);
        case 8: return launch_fused_t<D, DI, 8>(d, a, ws, st);
        case 16: return launch_fused_t<D, DI, 16>(d, a, ws, st);
        default: return launch_fused_t<D, DI, 32>(d, a, ws, st);
    }
}

hipError_t launch_fused_bwd(const LaunchDims& d, const FusedBwdArgs& a, void* ws, hipStream_t st) {
    if (d.B == 0 || d.N == 0) return hipSuccess;
    unsigned char* w = static_cast<unsigned char*>(ws);
    if (d.D == 128 && d.Di == 128) return launch_fused_g<128, 128>(d, a, w, st);
    if (d.D == 128) return launch_fused_g<128, 64>(d, a, w, st);
    if (d.Di == 128) return launch_fused_g<64, 128>(d, a, w, st);
    return launch_fused_g<64, 64>(d, a, w, st);
}

}  // namespace msa
