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
// window of query rows at a time, so the per-(row, slot) partials only ever
// hold one window (the workspace stays bounded at a million tokens). Per
// window:
//   main8_bwd_kernel: the main branch over the window's non-local items, then
//     the causal local blocks of its query blocks (eight waves, two per SIMD):
//     S and P once per (row, kept block), dQ partials per (row, slot), dK/dV
//     partials per item, and the teacher p (head mean of P) per (row, slot,
//     key) for the index branch;
//   fused_index_kernel: the index branch over the same items, one row per
//     position, from the teacher: dq_idx partials, dk_idx partials per item;
//   fused_dkv_reduce / fused_dki_reduce: the window's per-item partials, in
//     item order, added to fp32 running sums per key block (bf16 after the
//     last window); dq_combine_kernel: each row's slot partials in slot order.
// Every sum runs in a fixed order, so the gradients are deterministic. The
// teacher goes through memory (512 bytes per (row, slot)) because the index
// branch has one row per position and the main branch G: inside one tile its
// products would be repeated G times and its operands would take registers
// the main branch needs.
//
// Matrix-core orientation: products with A = tile rows (LDS) and B = the
// wave's keys (VGPRs) leave one key per lane and the rows in its accumulators;
// P, dS and dU in that layout are the B operands of dV^T = dO^T P,
// dK^T = Q^T dS and dk_idx^T = Q_idx^T dU against transposed tiles staged with
// the matching row order; dQ and dq_idx contract over keys, so dS and dU go
// through LDS and the A operands are the per-block K^T and K_idx^T copies.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"
#include "msa_bwd_tiles.h"

#include <algorithm>
#include <type_traits>

namespace msa {

// ------------------------------------------------------------- row deltas --

// Dl[b, h, i] = <dO[b, i, h], O[b, i, h]> in fp32; D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
                                                        float* __restrict__ dl, int64_t rows, int N, int Hq) {
    constexpr int LPR = D / 8;
    const int64_t row = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + c * 8);
        const u32x4 x = *reinterpret_cast<const u32x4*>(dout + row * D + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(x[e] << 16), acc);
            acc = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(x[e] & 0xffff0000u), acc);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) {
        const int h = (int)(row % Hq);
        const int64_t bi = row / Hq;   // b * N + i
        const int64_t b = bi / N, i = bi % N;
        dl[(b * Hq + h) * N + i] = acc;
    }
}

// ----------------------------------------------- main branch, two waves/SIMD --

// v_mfma_f32_16x16x32_bf16: A (16 x 32) lane l supplies row l % 16 and
// contraction elements 8*(l/16) .. +7, B (32 x 16) column l % 16 and the same
// elements, C (16 x 16) lane l holds column l % 16, rows 4*(l/16) + r, r < 4.
__device__ __forceinline__ void mma1632(floatx4& c, const Op8<bf16_t>& a, const Op8<bf16_t>& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// One staged 32-row tile of the eight-wave main-branch kernel: Q and dO rows,
// natural and transposed, and the rows' scalars. In the transposed copies the
// contraction over the tile's rows follows the 16 x 16 accumulator layout:
// lane group q = l / 16 holds rows 4q .. 4q+3 and 16 + 4q .. 16 + 4q + 3, so
// chunk q of a transposed row (8 positions) holds exactly those rows, row m at
// position 4 * (m / 16) + m % 4.
// Position (within the tile) and head of tile row m. The 16 x 16 accumulator
// rows of lane group q are m = 16 h4 + 4 q + r (h4 < 2, r < 4): for G = 8 they
// hold position q, head 4 h4 + r, so each lane group has all G rows of one
// position and the KL teacher (the mean over them) stays in the lane; for the
// other G, G consecutive rows per position.
template <int G>
__device__ __forceinline__ int tile_pos(int m) { return G == 8 ? (m >> 2) & 3 : m / G; }
template <int G>
__device__ __forceinline__ int tile_head(int m) { return G == 8 ? ((m >> 4) << 2) | (m & 3) : m % G; }

template <int D>
struct Main8Tile {
    using QT = SwzTile<bf16_t, D>;   // [32 rows][D]
    using QCT = ColTile<D>;          // [D][32 rows, permuted]
    unsigned char q[32 * QT::ROWB], dout[32 * QT::ROWB];
    unsigned char qt[QCT::BYTES], dot[QCT::BYTES];
    float lse2[32], dl[32];
    int pos[32], slot[32];
};

template <int D>
struct Main8Lds {
    using DsT = SwzTile<bf16_t, kBlock>;   // [32 rows][128 keys, permuted]
    Main8Tile<D> tile[2];
    unsigned char ds[32 * DsT::ROWB];
    int entries[kSegBwd];
};

// Staging in quarter units: 4 rows x 16 bytes (dims 8*dc .. +7) of Q (units
// 0 .. D-1) or dO (units D .. 2D-1); rows past the item read its last entry
// (their P is zero).
struct Main8Quarter {
    u32x4 x[4];
};

// Row quarter rq and 16-byte chunk dc of unit v of a tensor. Eight consecutive
// lanes read eight consecutive chunks of a row (whole 128-byte lines); the next
// lane bit picks the row quarter 4 apart (the other half of the same transposed
// chunk), so that the natural rows (16 lanes: 16 different swizzled chunks) and
// the transposed 8-byte writes (16 lanes: both halves of 8 chunk slots) of one
// store instruction fall in different banks.
template <int D>
__device__ __forceinline__ void main8_unit(int v, int& rq, int& dc) {
    if constexpr (D == 128) {
        dc = (v & 7) | (((v >> 4) & 1) << 3);
        rq = (((v >> 3) & 1) << 2) | ((v >> 5) & 3);
    } else {
        dc = v & 7;
        rq = (((v >> 3) & 1) << 2) | ((v >> 4) & 3);
    }
}

template <int D, int G, bool LOCAL, bool MAIN>
__device__ __forceinline__ void main8_stage_load(Main8Quarter& su, const BwdItem<LOCAL>& it, int t, int u,
                                                 const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
                                                 int N, int Hq) {
    constexpr int PPT = 32 / G;
    const int tensor = u >= D, v = tensor ? u - D : u;
    int rq, dc;
    main8_unit<D>(v, rq, dc);
    const bf16_t* src = tensor ? dout : q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * rq + e;
        int i, s;
        it.entry(min(t * PPT + tile_pos<G>(m), it.count - 1), i, s);
        su.x[e] = *reinterpret_cast<const u32x4*>(src + (((size_t)it.b * N + i) * Hq + it.g * G + tile_head<G>(m)) * D +
                                                  dc * 8);
    }
}

template <int D, bool MAIN>
__device__ __forceinline__ void main8_stage_store(const Main8Quarter& su, Main8Tile<D>& tb, int u) {
    using T = Main8Tile<D>;
    const int tensor = u >= D, v = tensor ? u - D : u;
    int rq, dc;
    main8_unit<D>(v, rq, dc);
    unsigned char* nat = tensor ? tb.dout : tb.q;
    unsigned char* tr = tensor ? tb.dot : tb.qt;
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4*>(nat + T::QT::offset(4 * rq + e, dc * 16)) = su.x[e];
    if constexpr (!MAIN) return;   // the transposed copies only feed dV and dK
    // rows 4rq .. 4rq+3 are four consecutive positions of chunk rq % 4
    const int chunk = rq & 3, sub = (rq >> 2) * 8;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        const uint32_t sel = dd % 2 ? 0x07060302u : 0x05040100u;   // the 16-bit element dd of two rows
        *reinterpret_cast<uint2*>(tr + T::QCT::offset(dc * 8 + dd, chunk) + sub) =
            make_uint2(__builtin_amdgcn_perm(su.x[1][dd / 2], su.x[0][dd / 2], sel),
                       __builtin_amdgcn_perm(su.x[3][dd / 2], su.x[2][dd / 2], sel));
    }
}

// Teacher of each of the lane's 8 rows (rh*4 + r: row 16*rh + 4*(l/16) + r):
// the mean of P over the G rows of the row's position (tile_pos, tile_head).
template <int G>
__device__ __forceinline__ void head_mean8(float (&p)[8]) {
    if constexpr (G == 1) return;
    if constexpr (G == 8) {   // the lane's 8 rows are the 8 heads of one position
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += p[e];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = s * (1.f / G);
        return;
    }
    float a[2][4];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
        if constexpr (G == 2) {
            a[rh][0] = a[rh][1] = p[4 * rh] + p[4 * rh + 1];
            a[rh][2] = a[rh][3] = p[4 * rh + 2] + p[4 * rh + 3];
        } else {
            float s = p[4 * rh] + p[4 * rh + 1] + p[4 * rh + 2] + p[4 * rh + 3];
            if constexpr (G >= 16) {
                s += __shfl_xor(s, 16);
                s += __shfl_xor(s, 32);
            }
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

constexpr int kMain8Waves = 8;

// What one pass of the main-branch kernel produces: dQ, dK, dV and the KL
// term's teacher (the fused backward), the gradients only (the main-branch
// backward alone), or the teacher only (the KL term's backward alone: S and P,
// no dP and no gradient products).
enum Main8Mode { kMainAndTeacher = 0, kMainOnly = 1, kTeacherOnly = 2 };

// The main branch of the backward with two waves per SIMD: one 8-wave
// work-group per work item of a window, wave w owning keys 16w .. 16w+15 of
// the block for S, dP, dK, dV (K and V as B operands in VGPRs) and dims
// 16w .. 16w+15 of the dQ tile (its K^T rows as A operands); 16 x 16 x 32
// products throughout. Writes the dQ partials in
// natural dim order, the dK/dV partial of the item and/or the teacher (MODE).
// With MODE = kTeacherOnly, v, kt, dout, dl, dq_part and dkv_part are unused.
template <int D, int G, bool LOCAL, int MODE>
__global__ __launch_bounds__(64 * kMain8Waves, 1) void main8_bwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ kt, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dl, const int32_t* __restrict__ list, const int4* __restrict__ items,
    const int32_t* __restrict__ item_offsets, const int32_t* __restrict__ total_items, int n_keys,
    bf16_t* __restrict__ dq_part, float* __restrict__ dkv_part, float* __restrict__ teacher, int B, int N, int Hkv,
    int nb, int nwin, int topk, FusedWindow win, float scale_log2, float scale) {
    constexpr int PPT = 32 / G, DT = D / 16, KS = D / 32;
    constexpr int NTHR = 64 * kMain8Waves;
    constexpr bool MAIN = MODE != kTeacherOnly, TEACH = MODE != kMainOnly;
    constexpr int NST = MAIN ? 2 * D : D;   // staging units: Q and dO, or Q only
    static_assert(2 * D <= NTHR - 32, "staging threads and the 32 row-scalar threads share the work-group");
    __shared__ __align__(16) Main8Lds<D> sh;
    using T = Main8Tile<D>;
    using L = Main8Lds<D>;
    const int Hq = Hkv * G;

    BwdItem<LOCAL> it;
    size_t pidx;
    if (!fused_item<LOCAL>(it, pidx, sh.entries, list, items, item_offsets, total_items, n_keys, B, N, Hkv, nb, nwin,
                           topk, win))
        return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ql = lane >> 4, cl = lane & 15;
    const int ntiles = (it.count + PPT - 1) / PPT;
    const size_t rbase = ((size_t)it.b * Hkv + it.g) * win.len - win.p0;   // window row of position i: rbase + i
    const size_t spare = (size_t)B * Hkv * win.len * topk;                 // (row, slot) of rows past the item

    const int key = 16 * w + cl;
    const int kabs = it.j * kBlock + key;
    Op8<bf16_t> kop[KS], vop[KS], ktop[4];
    {
        const size_t roff = (((size_t)it.b * N + kabs) * Hkv + it.g) * D + 8 * ql;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (kabs < N) kop[s].load(k + roff + 32 * s);
            else kop[s].zero();
            if constexpr (MAIN) {
                if (kabs < N) vop[s].load(v + roff + 32 * s);
                else vop[s].zero();
            }
        }
        if (MAIN && w < DT) {
            const bf16_t* src = kt + ((((size_t)it.b * Hkv + it.g) * nb + it.j) * D + 16 * w + cl) * kBlock + 8 * ql;
#pragma unroll
            for (int c = 0; c < 4; ++c) ktop[c].load(src + 32 * c);
        }
    }
    floatx4 dkt[DT], dvt[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dkt[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        dvt[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    constexpr float kLog2e = 1.4426950408889634f;
    // Threads 0 .. 2D-1 stage a quarter of every tile, the last 32 threads the
    // rows' scalars: tile t + 1 is written to LDS and tile t + 2 requested while
    // tile t is on the matrix cores.
    Main8Quarter su;
    const int u = threadIdx.x;
    const int m_row = (int)threadIdx.x - (NTHR - 32);
    float r_lse = 0.f, r_dl = 0.f;
    int r_pos = -1, r_slot = 0;
    auto load_tile = [&](int t) {
        if (u < NST) main8_stage_load<D, G, LOCAL, MAIN>(su, it, t, u, q, dout, N, Hq);
        if (m_row >= 0) {
            const int pe = t * PPT + tile_pos<G>(m_row);
            int i, s;
            it.entry(min(pe, it.count - 1), i, s);
            const size_t r = ((size_t)it.b * Hq + it.g * G + tile_head<G>(m_row)) * N + i;
            r_pos = pe < it.count ? i : -1;
            r_slot = s;
            r_lse = lse[r];
            if constexpr (MAIN) r_dl = dl[r];
        }
    };
    auto store_tile = [&](int t) {
        T& tb = sh.tile[t & 1];
        if (u < NST) main8_stage_store<D, MAIN>(su, tb, u);
        if (m_row >= 0) {
            const bool ok = r_pos >= 0;
            tb.lse2[m_row] = ok ? r_lse * kLog2e : __builtin_inff();
            tb.dl[m_row] = ok ? r_dl : 0.f;
            tb.pos[m_row] = r_pos;
            tb.slot[m_row] = r_slot;
        }
    };
    load_tile(0);
    __builtin_amdgcn_s_waitcnt(0);
    store_tile(0);
    if (ntiles > 1) load_tile(1);

    for (int t = 0; t < ntiles; ++t) {
        // Tile t is complete in its buffer; the other buffer's readers (tile
        // t - 1) and the dS readers are done.
        __syncthreads();
        const T& sh_t = sh.tile[t & 1];

        // S = Q K_w^T and dP = dO V_w^T for both 16-row halves: lane = key
        // 16w + l % 16, accumulators = rows 16 rh + 4 (l / 16) + r.
        floatx4 s[2], dp[2];
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
            s[rh] = dp[rh] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Op8<bf16_t> a;
                a.load(sh_t.q + T::QT::offset(16 * rh + cl, (32 * ks + 8 * ql) * 2));
                mma1632(s[rh], a, kop[ks]);
                if constexpr (MAIN) {
                    Op8<bf16_t> b;
                    b.load(sh_t.dout + T::QT::offset(16 * rh + cl, (32 * ks + 8 * ql) * 2));
                    mma1632(dp[rh], b, vop[ks]);
                }
            }
        }
        // Staging of tile t + 1 and request of tile t + 2. It waits for every memory
        // operation before it, so it comes after S and dP (the previous tile's dQ
        // stores have landed by then) and before this tile's stores.
        if (t + 1 < ntiles) {
            store_tile(t + 1);
            if (t + 2 < ntiles) load_tile(t + 2);
        }
        float p[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 16 * (e >> 2) + 4 * ql + (e & 3);
            float pr = exp2_hw(fmaf(s[e >> 2][e & 3], scale_log2, -sh_t.lse2[m]));
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) pr = 0.f;   // also the rows past the item (pos = -1)
            }
            p[e] = pr;
            if constexpr (MAIN) ds[e] = pr * (dp[e >> 2][e & 3] - sh_t.dl[m]);
        }
        if constexpr (TEACH) {
            // The KL term's teacher of (position, key): the mean of P over the position's
            // G head rows. The lanes holding a position's first row write it (G = 8: one
            // store per lane; G >= 16: also the other lane groups of the position, which
            // hold the same mean); rows past the item write the spare row, so every tile
            // issues the same stores.
            {
                float tp[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) tp[e] = p[e];
                head_mean8<G>(tp);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (G == 8 ? e == 0 : (e & 3) % (G < 4 ? G : 4) == 0) {
                        const int m = 16 * (e >> 2) + 4 * ql + (e & 3);
                        const int i = sh_t.pos[m];
                        const size_t row = i >= 0 ? (rbase + i) * topk + sh_t.slot[m] : spare;
                        teacher[row * kBlock + key] = tp[e];
                    }
                }
            }
        }
        if constexpr (MAIN) {
            // dV^T += dO^T P and dK^T += Q^T dS: the lane's 8 values are the contraction
            // elements of its key column, in the transposed tiles' row order.
            {
                Op8<bf16_t> bp, bds;
                PType<bf16_t>::pack(bp, p);
                PType<bf16_t>::pack(bds, ds);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    Op8<bf16_t> a, b;
                    a.load(sh_t.dot + T::QCT::offset(16 * dt + cl, ql));
                    b.load(sh_t.qt + T::QCT::offset(16 * dt + cl, ql));
                    mma1632(dvt[dt], a, bp);
                    mma1632(dkt[dt], b, bds);
                }
            }
            // dS -> LDS as [row][permuted key] for the dQ product.
            {
                uint16_t* dsl = reinterpret_cast<uint16_t*>(sh.ds);
                const int pk = perm16(key);
#pragma unroll
                for (int e = 0; e < 8; e += 2) {   // rows m and m + 1: one conversion, two 16-bit stores
                    const int m = 16 * (e >> 2) + 4 * ql + (e & 3);
                    const uint32_t a2 = pack_bf16x2(ds[e], ds[e + 1]);
                    dsl[L::DsT::offset(m, pk * 2) / 2] = (uint16_t)(a2 & 0xffffu);
                    dsl[L::DsT::offset(m + 1, pk * 2) / 2] = (uint16_t)(a2 >> 16);
                }
            }
            __syncthreads();
            // dQ^T (dims 16w.., rows) = K^T dS^T over the block's 128 keys: lane = row
            // 16 rh + l % 16, accumulators = dims 16w + 4 (l / 16) + r.
            if (w < DT) {
#pragma unroll
                for (int rh = 0; rh < 2; ++rh) {
                    const int row = 16 * rh + cl;
                    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        Op8<bf16_t> b;
                        b.load(sh.ds + L::DsT::offset(row, (32 * c + 8 * ql) * 2));
                        mma1632(acc, ktop[c], b);
                    }
                    const int i = sh_t.pos[row];
                    const size_t prow = i >= 0 ? (rbase + i) * topk + sh_t.slot[row] : spare;
                    // partial of (window row, slot), the row's head: [G][D] bf16 in natural dim order
                    bf16_t* dst = dq_part + prow * G * D + (size_t)tile_head<G>(row) * D + 16 * w + 4 * ql;
                    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0] * scale, acc[1] * scale),
                                                                pack_bf16x2(acc[2] * scale, acc[3] * scale));
                }
            }
        }
    }

    if constexpr (MAIN) {
        // The item's dK, dV partial: [2][128 keys][D] fp32 (dK scaled by sigma).
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
    }
}

// ------------------------------------------------------------ index branch --

// One staged tile of the index branch: the index-query rows of 32 (position,
// slot) entries, natural and transposed, and their scalars.
template <int DI>
struct IdxBwdTile {
    using IT = SwzTile<bf16_t, DI>;   // [32 rows][DI]
    using ICT = ColTile<DI>;          // [DI][32 rows, permuted]
    unsigned char qi[32 * IT::ROWB], qit[ICT::BYTES];
    float lseu2[32], w[32];
    int pos[32], slot[32];
};

// Two tile buffers, the dU tile, the item's entries.
template <int DI>
struct IdxBwdLds {
    using DuT = SwzTile<bf16_t, kBlock>;   // [32 rows][128 keys, permuted]; also K_idx^T [DI][128 keys]
    IdxBwdTile<DI> tile[2];
    unsigned char du[32 * DuT::ROWB];
    unsigned char kit[DI * DuT::ROWB];
    int entries[kSegBwd];
};

// One 4-row x 16-byte unit of the staging: rows 4rq .. 4rq+3 at dims 8*dc .. +7.
// Rows 4rq .. 4rq+3 are four consecutive positions of one transposed chunk.
struct IdxUnit {
    u32x4 x[4];
};

// Row quarter rq and 16-byte chunk dc of unit u (of the 8 * (DI/8) units of a
// tile): eight consecutive lanes read eight consecutive chunks of a row (whole
// 128-byte lines), and the lane bits above are spread over the row quarters so
// that the natural and the transposed writes of one store instruction fall in
// different banks.
template <int DI>
__device__ __forceinline__ void idx_unit(int u, int& rq, int& dc) {
    if constexpr (DI == 128) {
        dc = (u & 7) | (((u >> 4) & 1) << 3);
        rq = ((u >> 5) & 1) | (((u >> 3) & 1) << 1) | (((u >> 6) & 1) << 2);
    } else {
        dc = u & 7;
        rq = ((u >> 4) & 1) | (((u >> 3) & 1) << 1) | (((u >> 5) & 1) << 2);
    }
}

template <int DI, bool LOCAL>
__device__ __forceinline__ void idx_stage_load(IdxUnit& su, const BwdItem<LOCAL>& it, int t, int u,
                                               const bf16_t* __restrict__ q_idx, int N, int Hkv) {
    int rq, dc;
    idx_unit<DI>(u, rq, dc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // rows past the item read its last entry (their dU is zero), so every
        // load is issued unconditionally
        int i, s;
        it.entry(min(32 * t + 4 * rq + e, it.count - 1), i, s);
        su.x[e] = *reinterpret_cast<const u32x4*>(q_idx + (((size_t)it.b * N + i) * Hkv + it.g) * DI + dc * 8);
    }
}

template <int DI>
__device__ __forceinline__ void idx_stage_store(const IdxUnit& su, IdxBwdTile<DI>& tb, int u) {
    using T = IdxBwdTile<DI>;
    int rq, dc;
    idx_unit<DI>(u, rq, dc);
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4*>(tb.qi + T::IT::offset(4 * rq + e, dc * 16)) = su.x[e];
    // row m sits in chunk 2 * (m / 16) + (m / 4) % 2 at position 4 * ((m / 8) % 2) + m % 4
    const int chunk = 2 * (rq >> 2) + (rq & 1), sub = 8 * ((rq >> 1) & 1);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        // the 16-bit element dd of rows 2w and 2w + 1 (low and high half of the word)
        const uint32_t sel = dd % 2 ? 0x07060302u : 0x05040100u;
        *reinterpret_cast<uint2*>(tb.qit + T::ICT::offset(dc * 8 + dd, chunk) + sub) =
            make_uint2(__builtin_amdgcn_perm(su.x[1][dd / 2], su.x[0][dd / 2], sel),
                       __builtin_amdgcn_perm(su.x[3][dd / 2], su.x[2][dd / 2], sel));
    }
}

// Index branch of one window, given the teacher the main-branch kernel wrote
// for every (row, slot, key) of the window: one work-group (4 waves) per work
// item, the same items as the main branch (non-local: the window's entries of
// key block j; LOCAL: query block j against its own block). Rows are (position,
// slot) entries, one per position (the index query has no heads), 32 per tile.
// Wave w owns keys 32w .. 32w+31 for U and dk_idx, dims 32w .. 32w+31 of dq_idx.
//   U = Q_idx K_idx^T,  s = exp(c U - LSE_u),  dU = w c (s - teacher),
//   dk_idx^T += Q_idx^T dU (over the item),  dq_idx^T = K_idx^T dU^T (per tile).
template <int DI, bool LOCAL>
__global__ __launch_bounds__(256, 2) void fused_index_kernel(
    const bf16_t* __restrict__ q_idx, const bf16_t* __restrict__ k_idx, const bf16_t* __restrict__ kit,
    const float* __restrict__ index_lse, const float* __restrict__ dkl_rows, float kl_weight,
    const float* __restrict__ teacher, const int32_t* __restrict__ list, const int4* __restrict__ items,
    const int32_t* __restrict__ item_offsets, const int32_t* __restrict__ total_items, int n_keys,
    bf16_t* __restrict__ dqi_part, float* __restrict__ dki_part, int B, int N, int Hkv, int nb, int nwin, int topk,
    FusedWindow win, float iscale) {
    constexpr int DIT = DI / 32, NST = 8 * (DI / 8);
    __shared__ __align__(16) IdxBwdLds<DI> sh;
    using L = IdxBwdLds<DI>;
    using T = IdxBwdTile<DI>;

    BwdItem<LOCAL> it;
    size_t pidx;
    if (!fused_item<LOCAL>(it, pidx, sh.entries, list, items, item_offsets, total_items, n_keys, B, N, Hkv, nb, nwin,
                           topk, win))
        return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int ntiles = (it.count + 31) / 32;
    const size_t rbase = ((size_t)it.b * Hkv + it.g) * win.len - win.p0;   // window row of position i: rbase + i
    const size_t spare = (size_t)B * Hkv * win.len * topk;                 // (row, slot) of rows past the item

    const int key = 32 * w + col;
    const int kabs = it.j * kBlock + key;
    Op8<bf16_t> kiop[DI / 16];
#pragma unroll
    for (int s = 0; s < DI / 16; ++s) {
        if (kabs < N) kiop[s].load(k_idx + ((size_t)it.b * N + kabs) * DI + 8 * half + 16 * s);
        else kiop[s].zero();
    }
    // The block's K_idx^T (A operand of dq_idx) into LDS, 16 bytes per thread and step.
    {
        const bf16_t* src = kit + ((size_t)it.b * nb + it.j) * DI * kBlock;
        for (int ch = threadIdx.x; ch < DI * L::DuT::CPR; ch += blockDim.x)
            *reinterpret_cast<u32x4*>(sh.kit + L::DuT::offset(ch / L::DuT::CPR, (ch % L::DuT::CPR) * 16)) =
                *reinterpret_cast<const u32x4*>(src + (size_t)ch * 8);
    }
    floatx16 dkit[DIT];
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt) dkit[dt] = zero16();

    // The teacher of the lane's 16 rows (rows 8*(r/4) + 4*half + r%4) at its key, one tile ahead;
    // rows past the item read its last entry's (finite; their weight is zero).
    float tn[16];
    auto teacher_load = [&](int t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int i, s;
            it.entry(min(32 * t + 8 * (r / 4) + 4 * half + r % 4, it.count - 1), i, s);
            tn[r] = teacher[((rbase + i) * topk + s) * kBlock + key];
        }
    };

    constexpr float kLog2e = 1.4426950408889634f;
    const float iscale_log2 = iscale * kLog2e;
    IdxUnit su;
    const int par = threadIdx.x >> 7;
    const int u = threadIdx.x & 127;
    if (u < NST && par < ntiles) idx_stage_load<DI, LOCAL>(su, it, par, u, q_idx, N, Hkv);
    float r_lseu = 0.f, r_w = 0.f;
    int r_pos = -1, r_slot = 0;
    auto row_load = [&](int t) {
        const int m = 127 - u;   // thread 127 - m of each half loads the scalars of row m
        if (m < 32) {
            const int pe = 32 * t + m;
            r_pos = -1;
            r_lseu = __builtin_inff();
            r_w = 0.f;
            if (pe < it.count) {
                int i, s;
                it.entry(pe, i, s);
                const size_t rr = ((size_t)it.b * Hkv + it.g) * N + i;
                r_pos = i;
                r_slot = s;
                r_lseu = index_lse[rr];
                r_w = dkl_rows ? dkl_rows[rr] : 1.f;
            }
        }
    };
    if (par < ntiles) row_load(par);
    if (ntiles > 0) teacher_load(0);
    // Every load issued so far completes here, so the loop below only ever
    // waits for its own prefetches.
    __builtin_amdgcn_s_waitcnt(0);
    // Staging of tile t into buffer t % 2 by the threads of its parity, who
    // then request tile t + 2.
    auto commit = [&](int t) {
        T& tb = sh.tile[t & 1];
        if (u < NST) idx_stage_store<DI>(su, tb, u);
        const int m = 127 - u;
        if (m < 32) {
            tb.lseu2[m] = r_lseu * kLog2e;
            tb.w[m] = r_w * kl_weight * iscale;
            tb.pos[m] = r_pos;
            tb.slot[m] = r_slot;
        }
        if (t + 2 < ntiles) {
            if (u < NST) idx_stage_load<DI, LOCAL>(su, it, t + 2, u, q_idx, N, Hkv);
            row_load(t + 2);
        }
    };
    if (par == 0 && ntiles > 0) commit(0);

    for (int t = 0; t < ntiles; ++t) {
        // Tile t is complete in its buffer; the other buffer's readers (tile
        // t - 1) and the dU readers are done.
        __syncthreads();
        const T& sh_t = sh.tile[t & 1];
        floatx16 uu = zero16();
#pragma unroll
        for (int sl = 0; sl < DI / 16; ++sl) {
            Op8<bf16_t> a;
            a.load(sh_t.qi + T::IT::offset(col, (16 * sl + 8 * half) * 2));
            mma16(uu, a, kiop[sl]);
        }
        // Staging of tile t + 1 (overlaps tile t's math) and the teacher of tile
        // t + 1. The staging waits for every memory operation before it, so it
        // comes after U (the previous tile's stores and this tile's teacher have
        // landed by then) and before this tile's stores and the next teacher loads.
        if (t + 1 < ntiles && ((t + 1) & 1) == par) commit(t + 1);
        float tc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) tc[r] = tn[r];
        if (t + 1 < ntiles) teacher_load(t + 1);
        float du[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * half + r % 4;
            float st = exp2_hw(fmaf(uu[r], iscale_log2, -sh_t.lseu2[m]));   // 0 for the rows past the item
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) st = 0.f;
            }
            du[r] = sh_t.w[m] * (st - tc[r]);
        }
        // dk_idx^T += Q_idx^T dU over the tile's two 16-row slices.
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            Op8<bf16_t> b;
            PType<bf16_t>::pack(b, du + 8 * sl);
#pragma unroll
            for (int dt = 0; dt < DIT; ++dt) {
                Op8<bf16_t> a;
                a.load(sh_t.qit + T::ICT::offset(32 * dt + col, 2 * sl + half));
                mma16(dkit[dt], a, b);
            }
        }
        {
            uint16_t* dul = reinterpret_cast<uint16_t*>(sh.du);
            const int pk = perm16(key);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {   // rows m and m + 1: one conversion, two 16-bit stores
                const int m = 8 * (r / 4) + 4 * half + r % 4;
                const uint32_t v2 = pack_bf16x2(du[r], du[r + 1]);
                dul[L::DuT::offset(m, pk * 2) / 2] = (uint16_t)(v2 & 0xffffu);
                dul[L::DuT::offset(m + 1, pk * 2) / 2] = (uint16_t)(v2 >> 16);
            }
        }
        __syncthreads();
        // dq_idx^T (dims 32w.., rows) = K_idx^T dU^T over the block's 128 keys.
        if (w < DIT) {
            floatx16 acc = zero16();
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                Op8<bf16_t> b;
                b.load(sh.du + L::DuT::offset(col, (16 * c + 8 * half) * 2));
                Op8<bf16_t> a;
                a.load(sh.kit + L::DuT::offset(32 * w + col, (16 * c + 8 * half) * 2));
                mma16(acc, a, b);
            }
            // partial of (window row, slot): [DI] bf16, each 32-dim slice lane-major; rows
            // past the item write the spare row, so every tile issues the same stores
            const int i = sh_t.pos[col];
            const size_t prow = i >= 0 ? (rbase + i) * topk + sh_t.slot[col] : spare;
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

    // The item's dk_idx partial: [128 keys][DI] fp32.
    float* pk = dki_part + pidx * kBlock * DI + (size_t)key * DI;
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            floatx4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = dkit[dt][4 * rq + e];
            *reinterpret_cast<floatx4*>(pk + 32 * dt + 8 * rq + 4 * half) = x;
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

void launch_bwd_delta(const LaunchDims& d, const void* o, const void* dout, float* dl, hipStream_t st) {
    const int64_t rows = (int64_t)d.B * d.N * d.Hq();
    if (d.D == 128)
        hipLaunchKernelGGL((bwd_delta_kernel<128>), dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st,
                           static_cast<const bf16_t*>(o), static_cast<const bf16_t*>(dout), dl, rows, d.N, d.Hq());
    else
        hipLaunchKernelGGL((bwd_delta_kernel<64>), dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0, st,
                           static_cast<const bf16_t*>(o), static_cast<const bf16_t*>(dout), dl, rows, d.N, d.Hq());
}

// Work-item slots per (b, g) in one window: every key's items (a list entry per
// kept non-local block of the window's rows, cut every kSegBwd) fit in
// ceil(W (k-1) / kSegBwd) + nb.
static int fused_bound(const LaunchDims& d) {
    const size_t W = (size_t)std::min(d.N, kWindow);
    const size_t kp = d.k > 1 ? (size_t)(d.k - 1) : 0;
    return (int)((W * kp + kSegBwd - 1) / kSegBwd + (size_t)d.nb);
}

FusedBwdWorkspace fused_bwd_workspace_layout(const LaunchDims& d, BwdParts parts) {
    FusedBwdWorkspace w{};
    const size_t W = (size_t)std::min(d.N, kWindow);
    const size_t bg = (size_t)d.B * d.Hkv;
    const bool mn = parts.main, kl = parts.kl;
    const bool multi = windows(d) > 1;   // running sums across windows
    size_t off = 0;
    w.kt = off;    off = align_up(off + (mn ? bg * d.nb * d.D * kBlock * 2 : 0));
    w.kit = off;   off = align_up(off + (kl ? (size_t)d.B * d.nb * d.Di * kBlock * 2 : 0));
    w.dl = off;    off = align_up(off + (mn ? (size_t)d.B * d.Hq() * d.N * 4 : 0));
    w.lists = list_layout(d, off, kSegBwd, true);
    off = w.lists.end;
    w.bound = w.lists.has_nonlocal ? fused_bound(d) : 0;
    w.items = bg * w.bound + bg * ((W + kBlock - 1) / kBlock);   // non-local slots, then local ones
    w.teacher = off;   off = align_up(off + (kl ? (bg * W * d.k + 1) * kBlock * 4 : 0));   // + spare row
    w.dq_part = off;   off = align_up(off + (mn ? (bg * W * d.k + 1) * d.G * d.D * 2 : 0));   // + spare
    w.dqi_part = off;  off = align_up(off + (kl ? (bg * W * d.k + 1) * d.Di * 2 : 0));   // + spare
    w.dkv_part = off;  off = align_up(off + (mn ? w.items * 2 * kBlock * d.D * 4 : 0));
    w.dki_part = off;  off = align_up(off + (kl ? w.items * kBlock * d.Di * 4 : 0));
    w.acc_dkv = off;   off = align_up(off + (mn && multi ? bg * d.nb * 2 * kBlock * d.D * 4 : 0));
    w.acc_dki = off;   off = align_up(off + (kl && multi ? (size_t)d.B * d.nb * kBlock * d.Di * 4 : 0));
    w.bytes = off;
    return w;
}

template <int D, int DI, int G>
static hipError_t launch_fused_t(const LaunchDims& d, const FusedBwdArgs& a, unsigned char* ws, hipStream_t st) {
    const FusedBwdWorkspace L = fused_bwd_workspace_layout(d, a.parts);
    const bool mn = a.parts.main, kl = a.parts.kl;
    const bf16_t* tq = static_cast<const bf16_t*>(a.q);
    const bf16_t* tk = static_cast<const bf16_t*>(a.k);
    const bf16_t* tv = static_cast<const bf16_t*>(a.v);
    const bf16_t* tdo = static_cast<const bf16_t*>(a.dout);
    const float scale_log2 = a.scale * 1.4426950408889634f;
    const bf16_t* tqi = static_cast<const bf16_t*>(a.q_idx);
    const bf16_t* tki = static_cast<const bf16_t*>(a.k_idx);
    bf16_t* kt = reinterpret_cast<bf16_t*>(ws + L.kt);
    bf16_t* kit = reinterpret_cast<bf16_t*>(ws + L.kit);
    float* dl = reinterpret_cast<float*>(ws + L.dl);
    bf16_t* dq_part = reinterpret_cast<bf16_t*>(ws + L.dq_part);
    bf16_t* dqi_part = reinterpret_cast<bf16_t*>(ws + L.dqi_part);
    float* dkv_part = reinterpret_cast<float*>(ws + L.dkv_part);
    float* dki_part = reinterpret_cast<float*>(ws + L.dki_part);
    float* acc_dkv = reinterpret_cast<float*>(ws + L.acc_dkv);
    float* acc_dki = reinterpret_cast<float*>(ws + L.acc_dki);
    const int nwin = windows(d);

    hipError_t e = hipSuccess;
    if (mn) {
        e = launch_transpose_kv(d, a.k, kt, st);
        if (e != hipSuccess) return e;
        launch_bwd_delta(d, a.o, a.dout, dl, st);
    }
    if (kl) {
        LaunchDims di = d;   // k_idx as a one-head [B, N, 1, Di] tensor
        di.Hkv = 1;
        di.G = 1;
        di.D = d.Di;
        e = launch_transpose_kv(di, a.k_idx, kit, st);
        if (e != hipSuccess) return e;
    }
    const bool nonlocal = L.lists.has_nonlocal;
    if (nonlocal) launch_build_lists(d, 0, d.N, a.block_idx, ws, L.lists, st);
    const int32_t* list = reinterpret_cast<const int32_t*>(ws + L.lists.list);
    const int4* items = reinterpret_cast<const int4*>(ws + L.lists.items);
    const int32_t* counts = reinterpret_cast<const int32_t*>(ws + L.lists.counts);
    const int32_t* item_offsets = reinterpret_cast<const int32_t*>(ws + L.lists.item_offsets);
    const int32_t* total = reinterpret_cast<const int32_t*>(ws + L.lists.total);
    float* teacher = reinterpret_cast<float*>(ws + L.teacher);
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
        // the main-branch kernel of the parts asked for
        auto main_pass = [&](auto mode) {
            constexpr int M = decltype(mode)::value;
            if (nonlocal)
                hipLaunchKernelGGL((main8_bwd_kernel<D, G, false, M>), dim3((unsigned)(bg * L.bound)),
                                   dim3(64 * kMain8Waves), 0, st, tq, tk, tv, kt, tdo, a.lse, dl, list, items,
                                   item_offsets, total, (int)L.lists.n_keys, dq_part, dkv_part, teacher, d.B, d.N,
                                   d.Hkv, d.nb, nwin, d.k, win, scale_log2, a.scale);
            hipLaunchKernelGGL((main8_bwd_kernel<D, G, true, M>), dim3((unsigned)(bg * nqb)), dim3(64 * kMain8Waves),
                               0, st, tq, tk, tv, kt, tdo, a.lse, dl, nullptr, nullptr, nullptr, nullptr, 0, dq_part,
                               dkv_part, teacher, d.B, d.N, d.Hkv, d.nb, nwin, d.k, win, scale_log2, a.scale);
        };
        if (mn && kl) main_pass(std::integral_constant<int, kMainAndTeacher>{});
        else if (mn) main_pass(std::integral_constant<int, kMainOnly>{});
        else main_pass(std::integral_constant<int, kTeacherOnly>{});
        if (kl) {
            if (nonlocal)
                hipLaunchKernelGGL((fused_index_kernel<DI, false>), dim3((unsigned)(bg * L.bound)), dim3(256), 0, st,
                                   tqi, tki, kit, a.index_lse, a.dkl_rows, a.kl_weight, teacher, list, items,
                                   item_offsets, total, (int)L.lists.n_keys, dqi_part, dki_part, d.B, d.N, d.Hkv, d.nb,
                                   nwin, d.k, win, a.iscale);
            hipLaunchKernelGGL((fused_index_kernel<DI, true>), dim3((unsigned)(bg * nqb)), dim3(256), 0, st, tqi, tki,
                               kit, a.index_lse, a.dkl_rows, a.kl_weight, teacher, nullptr, nullptr, nullptr, nullptr,
                               0, dqi_part, dki_part, d.B, d.N, d.Hkv, d.nb, nwin, d.k, win, a.iscale);
        }
        if (mn) {
            hipLaunchKernelGGL((fused_dkv_reduce_kernel<D>), dim3((unsigned)(bg * nbw)), dim3(256), 0, st, dkv_part,
                               counts, item_offsets, acc_dkv, static_cast<bf16_t*>(a.dk), static_cast<bf16_t*>(a.dv),
                               d.B, d.N, d.Hkv, d.nb, nwin, kSegBwd, win, nbw, last, nonlocal ? 1 : 0);
            const int64_t units = (int64_t)bg * win.len * G * (D / 16);
            hipLaunchKernelGGL((dq_combine_kernel<D, G, true>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                               st, dq_part, static_cast<bf16_t*>(a.dq), units, d.N, d.Hkv, d.k, win.p0, win.len,
                               win.len);
        }
        if (kl) {
            hipLaunchKernelGGL((fused_dki_reduce_kernel<DI>), dim3((unsigned)(d.B * nbw)), dim3(256), 0, st, dki_part,
                               counts, item_offsets, acc_dki, static_cast<bf16_t*>(a.dk_idx), d.B, d.N, d.Hkv, d.nb,
                               nwin, kSegBwd, win, nbw, last, nonlocal ? 1 : 0);
            const int64_t iunits = (int64_t)bg * win.len * (DI / 16);
            hipLaunchKernelGGL((dq_combine_kernel<DI, 1>), dim3((unsigned)((iunits + 255) / 256)), dim3(256), 0, st,
                               dqi_part, static_cast<bf16_t*>(a.dq_idx), iunits, d.N, d.Hkv, d.k, win.p0, win.len,
                               win.len);
        }
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
