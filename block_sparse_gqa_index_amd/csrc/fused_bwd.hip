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

// One staged 32-row tile: query, output-gradient and index-query rows, each
// natural and transposed, and the rows' scalars.
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

// LDS of one work-group: the staged tile, the dS and dU tiles, the key
// block's K^T and K_idx^T (A operands of dQ and dq_idx, read from here rather
// than held in registers, which the other operands and the dK, dV, dk_idx sums
// already fill), the item's list entries.
template <int D, int DI>
struct FusedLds {
    using DsT = SwzTile<bf16_t, kBlock>;   // [rows][128 keys, permuted]: dS, dU, K^T, K_idx^T
    FusedTile<D, DI> tile;
    unsigned char ds[32 * DsT::ROWB], du[32 * DsT::ROWB];
    unsigned char kt[D * DsT::ROWB], kit[DI * DsT::ROWB];
    int entries[kSegBwd];
};

struct FusedUnit {
    u32x4 x[8];
};

// Staging units of one tile: 4*(D/8) units of Q rows, 4*(D/8) of dO rows, then
// 4*(DI/8) of index-query rows (the position's one index query on each of its
// G rows). Unit v of a tensor: row group v % 4 (rows 16c + {4h..4h+3,
// 8+4h..8+4h+3}), dims 8*(v/4) .. +7; every unit is stored natural and
// transposed.
template <int D, int DI>
struct FusedUnits {
    static constexpr int NQ = 4 * (D / 8), NI = 4 * (DI / 8), N = 2 * NQ + NI;
};

template <int D, int DI, int G, bool LOCAL>
__device__ __forceinline__ void fused_stage_load(FusedUnit& su, const BwdItem<LOCAL>& it, int t, int u,
                                                 const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
                                                 const bf16_t* __restrict__ q_idx, int N, int Hkv) {
    constexpr int NQ = FusedUnits<D, DI>::NQ, PPT = 32 / G;
    const int tensor = u < NQ ? 0 : (u < 2 * NQ ? 1 : 2);
    const int v = u - tensor * NQ;
    const int grp = v & 3, dc = v >> 2;   // the row group varies fastest across lanes
    const int c = grp >> 1, h = grp & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int m = 16 * c + 8 * (e / 4) + 4 * h + e % 4;
        const int pe = t * PPT + m / G;
        su.x[e] = u32x4{0u, 0u, 0u, 0u};
        if (pe < it.count) {
            int i, s;
            it.entry(pe, i, s);
            const size_t hrow = ((size_t)it.b * N + i) * Hkv * G + it.g * G + m % G;
            const bf16_t* src = tensor == 2 ? q_idx + (((size_t)it.b * N + i) * Hkv + it.g) * DI + dc * 8
                                            : (tensor ? dout : q) + hrow * D + dc * 8;
            su.x[e] = *reinterpret_cast<const u32x4*>(src);
        }
    }
}

template <int D, int DI>
__device__ __forceinline__ void fused_stage_store(const FusedUnit& su, FusedTile<D, DI>& sh, int u) {
    constexpr int NQ = FusedUnits<D, DI>::NQ;
    using F = FusedTile<D, DI>;
    const int tensor = u < NQ ? 0 : (u < 2 * NQ ? 1 : 2);
    const int v = u - tensor * NQ;
    const int grp = v & 3, dc = v >> 2;
    const int c = grp >> 1, h = grp & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int m = 16 * c + 8 * (e / 4) + 4 * h + e % 4;
        unsigned char* dst = tensor == 2 ? sh.qi + F::IT::offset(m, dc * 16)
                                         : (tensor ? sh.dout : sh.q) + F::QT::offset(m, dc * 16);
        *reinterpret_cast<u32x4*>(dst) = su.x[e];
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        u32x4 y;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // the 16-bit element dd of rows 2w and 2w + 1 (low and high half of the word)
            y[w] = __builtin_amdgcn_perm(su.x[2 * w + 1][dd / 2], su.x[2 * w][dd / 2],
                                         dd % 2 ? 0x07060302u : 0x05040100u);
        }
        unsigned char* dst = tensor == 2 ? sh.qit + F::ICT::offset(dc * 8 + dd, 2 * c + h)
                                         : (tensor ? sh.dot : sh.qt) + F::QCT::offset(dc * 8 + dd, 2 * c + h);
        *reinterpret_cast<u32x4*>(dst) = y;
    }
}

// Window of the fused backward: query positions [p0, p0 + len) and the slots
// of its work items (see fused_bwd_workspace_layout).
struct FusedWindow {
    int w, p0, len, qb0;   // window index, first position, positions, first query block
    int bound;             // work-item slots per (b, g)
};

// One work-group (4 waves) per work item: the window's non-local rows of key
// block j (LOCAL = false), or the rows of query block j against their own
// block under the causal mask (LOCAL = true). Wave w owns keys 32w .. 32w+31
// of the block for S, dP, U and the dK, dV, dk_idx sums, and dims 32w ..
// 32w+31 of the dQ and dq_idx tiles.
template <int D, int DI, int G, bool LOCAL>
__global__ __launch_bounds__(256, 1) void fused_bwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ q_idx, const bf16_t* __restrict__ k_idx, const bf16_t* __restrict__ kt,
    const bf16_t* __restrict__ kit, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dl, const float* __restrict__ index_lse, const float* __restrict__ dkl_rows,
    float kl_weight, const int32_t* __restrict__ list, const int4* __restrict__ items,
    const int32_t* __restrict__ item_offsets, const int32_t* __restrict__ total_items, int n_keys,
    bf16_t* __restrict__ dq_part, bf16_t* __restrict__ dqi_part, float* __restrict__ dkv_part,
    float* __restrict__ dki_part, int B, int N, int Hkv, int nb, int nwin, int topk, FusedWindow win,
    float scale_log2, float scale, float iscale) {
    constexpr int PPT = 32 / G, DT = D / 32, DIT = DI / 32, KS = D / 16, KSI = DI / 16;
    constexpr int NST = FusedUnits<D, DI>::N;
    static_assert(NST <= 224, "staging threads and the 32 row-scalar threads share the work-group");
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
    const int half = lane >> 5, col = lane & 31;
    const int ntiles = (it.count + PPT - 1) / PPT;

    // The wave's keys as B operands (S, dP, U), its dims of K^T and K_idx^T as A operands (dQ, dq_idx).
    const int key = 32 * w + col;
    const int kabs = it.j * kBlock + key;
    Op8<bf16_t> kop[KS], vop[KS], kiop[KSI];
    {
        const size_t roff = (((size_t)it.b * N + kabs) * Hkv + it.g) * D + 8 * half;
        const size_t ioff = ((size_t)it.b * N + kabs) * DI + 8 * half;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (kabs < N) {
                kop[s].load(k + roff + 16 * s);
                vop[s].load(v + roff + 16 * s);
            } else {
                kop[s].zero();
                vop[s].zero();
            }
        }
#pragma unroll
        for (int s = 0; s < KSI; ++s) {
            if (kabs < N) kiop[s].load(k_idx + ioff + 16 * s);
            else kiop[s].zero();
        }
    }
    // The block's K^T and K_idx^T rows (dims) into LDS, 16 bytes per thread per step.
    {
        using KT = typename L::DsT;
        const bf16_t* src = kt + (((size_t)it.b * Hkv + it.g) * nb + it.j) * D * kBlock;
        for (int ch = threadIdx.x; ch < D * KT::CPR; ch += blockDim.x)
            *reinterpret_cast<u32x4*>(sh.kt + KT::offset(ch / KT::CPR, (ch % KT::CPR) * 16)) =
                *reinterpret_cast<const u32x4*>(src + (size_t)ch * 8);
        const bf16_t* srci = kit + ((size_t)it.b * nb + it.j) * DI * kBlock;
        for (int ch = threadIdx.x; ch < DI * KT::CPR; ch += blockDim.x)
            *reinterpret_cast<u32x4*>(sh.kit + KT::offset(ch / KT::CPR, (ch % KT::CPR) * 16)) =
                *reinterpret_cast<const u32x4*>(srci + (size_t)ch * 8);
    }

    floatx16 dkt[DT], dvt[DT], dkit[DIT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dkt[dt] = zero16();
        dvt[dt] = zero16();
    }
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt) dkit[dt] = zero16();

    constexpr float kLog2e = 1.4426950408889634f;
    const float iscale_log2 = iscale * kLog2e;
    // Threads 0 .. NST-1 stage one unit of every tile (tile t + 1 requested when
    // tile t is stored, so its loads are in flight while tile t is on the
    // matrix cores); threads 224 .. 255 load the per-row scalars.
    FusedUnit su;
    const int u = threadIdx.x;
    const int m_row = (int)threadIdx.x - 224;
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
    auto store_tile = [&]() {
        F& tb = sh.tile;
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

    for (int t = 0; t < ntiles; ++t) {
        // The readers of tile t - 1 and of the dS / dU tiles are done.
        __syncthreads();
        store_tile();
        if (t + 1 < ntiles) load_tile(t + 1);   // in flight during tile t's math
        __syncthreads();
        const F& sh_t = sh.tile;

        // S = Q K_w^T, dP = dO V_w^T, U = Q_idx K_idx,w^T: lane = key, accumulators = rows.
        floatx16 s = zero16(), dp = zero16(), uu = zero16();
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
            Op8<bf16_t> a, b;
            a.load(sh_t.q + F::QT::offset(col, (16 * sl + 8 * half) * 2));
            b.load(sh_t.dout + F::QT::offset(col, (16 * sl + 8 * half) * 2));
            mma16(s, a, kop[sl]);
            mma16(dp, b, vop[sl]);
        }
#pragma unroll
        for (int sl = 0; sl < KSI; ++sl) {
            Op8<bf16_t> a;
            a.load(sh_t.qi + F::IT::offset(col, (16 * sl + 8 * half) * 2));
            mma16(uu, a, kiop[sl]);
        }
        float p[16], ds[16], du[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * half + r % 4;
            float pr = exp2_hw(fmaf(s[r], scale_log2, -sh_t.lse2[m]));
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) pr = 0.f;   // also the rows past the item (pos = -1)
            }
            p[r] = pr;
            ds[r] = pr * (dp[r] - sh_t.dl[m]);
            du[r] = pr;
        }
        head_mean<G>(du);   // the teacher of each row's position
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * half + r % 4;
            float st = exp2_hw(fmaf(uu[r], iscale_log2, -sh_t.lseu2[m]));
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) st = 0.f;
            }
            du[r] = sh_t.wkl[m] * (st - du[r]);
        }
        // dV^T += dO^T P, dK^T += Q^T dS and dk_idx^T += Q_idx^T (dU / G) (every
        // position's G replicated rows count once) over the tile's two 16-row slices.
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            Op8<bf16_t> bp, bds, bdu;
            PType<bf16_t>::pack(bp, p + 8 * sl);
            PType<bf16_t>::pack(bds, ds + 8 * sl);
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = du[8 * sl + e] * (1.f / G);
            PType<bf16_t>::pack(bdu, x);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                Op8<bf16_t> a, b;
                a.load(sh_t.dot + F::QCT::offset(32 * dt + col, 2 * sl + half));
                b.load(sh_t.qt + F::QCT::offset(32 * dt + col, 2 * sl + half));
                mma16(dvt[dt], a, bp);
                mma16(dkt[dt], b, bds);
            }
#pragma unroll
            for (int dt = 0; dt < DIT; ++dt) {
                Op8<bf16_t> a;
                a.load(sh_t.qit + F::ICT::offset(32 * dt + col, 2 * sl + half));
                mma16(dkit[dt], a, bdu);
            }
        }
        // dS and dU -> LDS as [row][permuted key] for the dQ and dq_idx products.
        {
            uint16_t* dsl = reinterpret_cast<uint16_t*>(sh.ds);
            uint16_t* dul = reinterpret_cast<uint16_t*>(sh.du);
            const int pk = perm16(key);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {   // rows m and m + 1: one conversion, two 16-bit stores
                const int m = 8 * (r / 4) + 4 * half + r % 4;
                const uint32_t a2 = pack_bf16x2(ds[r], ds[r + 1]);
                const uint32_t b2 = pack_bf16x2(du[r], du[r + 1]);
                dsl[L::DsT::offset(m, pk * 2) / 2] = (uint16_t)(a2 & 0xffffu);
                dsl[L::DsT::offset(m + 1, pk * 2) / 2] = (uint16_t)(a2 >> 16);
                dul[L::DsT::offset(m, pk * 2) / 2] = (uint16_t)(b2 & 0xffffu);
                dul[L::DsT::offset(m + 1, pk * 2) / 2] = (uint16_t)(b2 >> 16);
            }
        }
        __syncthreads();
        // dQ^T (dims 32w.., rows) = K^T dS^T and dq_idx^T = K_idx^T dU^T over the block's 128 keys.
        const int i = sh_t.pos[col];
        const size_t prow = i >= 0 ? (((size_t)it.b * Hkv + it.g) * win.len + (i - win.p0)) * topk + sh_t.slot[col]
                                   : 0;
        if (w < DT) {
            floatx16 acc = zero16();
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                Op8<bf16_t> a, b;
                a.load(sh.kt + L::DsT::offset(32 * w + col, (16 * c + 8 * half) * 2));
                b.load(sh.ds + L::DsT::offset(col, (16 * c + 8 * half) * 2));
                mma16(acc, a, b);
            }
            if (i >= 0) {
                // partial of (row, slot), head col % G: [G][D] bf16, each 32-dim slice lane-major
                bf16_t* dst = dq_part + prow * G * D + (size_t)(col % G) * D + 32 * w + 16 * half;
                u32x4 w0, w1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w0[e] = pack_bf16x2(acc[2 * e] * scale, acc[2 * e + 1] * scale);
                    w1[e] = pack_bf16x2(acc[8 + 2 * e] * scale, acc[8 + 2 * e + 1] * scale);
                }
                *reinterpret_cast<u32x4*>(dst) = w0;
                *reinterpret_cast<u32x4*>(dst + 8) = w1;
            }
        }
        if (w < DIT) {
            floatx16 acc = zero16();
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                Op8<bf16_t> a, b;
                a.load(sh.kit + L::DsT::offset(32 * w + col, (16 * c + 8 * half) * 2));
                b.load(sh.du + L::DsT::offset(col, (16 * c + 8 * half) * 2));
                mma16(acc, a, b);
            }
            if (i >= 0 && col % G == 0) {   // the position's first head row writes it
                bf16_t* dst = dqi_part + prow * DI + 32 * w + 16 * half;
                u32x4 w0, w1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w0[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
                    w1[e] = pack_bf16x2(acc[8 + 2 * e], acc[8 + 2 * e + 1]);
                }
                *reinterpret_cast<u32x4*>(dst) = w0;
                *reinterpret_cast<u32x4*>(dst + 8) = w1;
            }
        }
    }

    // The item's partials: dK, dV [2][128 keys][D] fp32 (dK scaled by sigma), dk_idx [128 keys][DI] fp32.
    float* pk = dkv_part + pidx * 2 * kBlock * D + (size_t)key * D;
    float* pv = pk + (size_t)kBlock * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            floatx4 xk, xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xk[e] = dkt[dt][4 * rq + e] * scale;
                xv[e] = dvt[dt][4 * rq + e];
            }
            const int d0 = 32 * dt + 8 * rq + 4 * half;
            *reinterpret_cast<floatx4*>(pk + d0) = xk;
            *reinterpret_cast<floatx4*>(pv + d0) = xv;
        }
    }
    float* pki = dki_part + pidx * kBlock * DI + (size_t)key * DI;
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            floatx4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = dkit[dt][4 * rq + e];
            *reinterpret_cast<floatx4*>(pki + 32 * dt + 8 * rq + 4 * half) = x;
        }
    }
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
            hipLaunchKernelGGL((fused_bwd_kernel<D, DI, G, false>), dim3((unsigned)(bg * L.bound)), dim3(256), 0, st,
                               tq, tk, tv, tqi, tki, kt, kit, tdo, a.lse, dl, a.index_lse, a.dkl_rows, a.kl_weight,
                               list, items, item_offsets, total, (int)L.lists.n_keys, dq_part, dqi_part, dkv_part,
                               dki_part, d.B, d.N, d.Hkv, d.nb, nwin, d.k, win, scale_log2, a.scale, a.iscale);
        hipLaunchKernelGGL((fused_bwd_kernel<D, DI, G, true>), dim3((unsigned)(bg * nqb)), dim3(256), 0, st, tq, tk,
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
        hipLaunchKernelGGL((dq_combine_kernel<D, G>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, dq_part,
                           static_cast<bf16_t*>(a.dq), units, d.N, d.Hkv, d.k, win.p0, win.len, win.len);
        const int64_t iunits = (int64_t)bg * win.len * (DI / 16);
        hipLaunchKernelGGL((dq_combine_kernel<DI, 1>), dim3((unsigned)((iunits + 255) / 256)), dim3(256), 0, st,
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
