// Backward of the main branch over the cached block indices: dQ, dK and dV of
// exact softmax GQA attention restricted to each row's selected tokens (bf16
// inputs, fp32 accumulation), gfx950.
//
// Method: the Flash-MSA article (tech.kuratif.com), paragraph on the backward:
// with the block indices cached by the forward the backward only visits the
// selected blocks, so it is linear in N; it uses the LSE the forward kept. The
// MSA article on 7minutos.es ("Cómo funcionan las dos ramas") defines the
// forward that is differentiated. For the loss <dO, O>:
//   P = exp(sigma q.k - LSE),  dV_t = sum P dO,  dP = dO.v_t,
//   Dl = <dO, O> (= sum_t P dP),  dS = P (dP - Dl),
//   dQ = sigma sum_t dS k_t,  dK_t = sigma sum dS q.
//
// Data flow (one stream):
//   1. K^T copy (same permuted layout as the forward's V^T) and Dl per row;
//   2. position-sorted inversion of the selection into per-(b, g, window, j)
//      lists, cut into work items of up to 1024 positions;
//   3. attn_bwd_kernel, one work-group per item (non-local blocks), then one
//      per (b, g, query block) for the causal local block: the key block stays
//      in VGPRs (K and V as matrix-core operands), the item's rows stream
//      through in 32-row tiles staged in LDS (natural and transposed); dK and
//      dV accumulate in registers over the item and are written once as an
//      fp32 partial; dQ of every (row, slot) is written as a bf16 partial;
//   4. dkv_reduce: per key block, the partials of its items (and of its local
//      item) summed in item order -> dK, dV;
//   5. dq_combine: per row, its slots' partials summed in slot order -> dQ.
// Every sum runs in a fixed order over sorted lists, so the results are
// deterministic.
//
// Matrix-core orientation: S = Q K^T with A = query rows (LDS), B = the wave's
// 32 keys (VGPRs) leaves one key per lane and 16 rows in its accumulators
// (rows 8*(r/4) + 4*h + r%4, h = lane/32). P and dS in that layout are the B
// operands of dV^T = dO^T P and dK^T = Q^T dS (contraction over rows): a
// 16-row slice of the lane's accumulators is rows {4h..4h+3, 8+4h..8+4h+3},
// and the transposed tiles dO^T and Q^T are staged with that row permutation
// so the A operand is one 16-byte read. dQ (contraction over keys) needs the
// other orientation: dS goes through LDS, and the A operand is the K^T copy.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"
#include "msa_bwd_tiles.h"

namespace msa {


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

// One staged 32-row tile: Q and dO natural and transposed, per-row scalars.
template <int D>
struct BwdTile {
    using RowT = SwzTile<bf16_t, D>;        // [32 rows][D]
    using ColT = ColTile<D>;                // [D][32 rows, permuted]
    static constexpr int ROWB = 32 * RowT::ROWB, COLB = ColT::BYTES;
    unsigned char q[ROWB], dout[ROWB], qt[COLB], dot[COLB];
    float lse2[32], dl[32];
    int pos[32], slot[32];
};

// LDS of one work-group: two tile buffers (tile t is computed from one while
// tile t + 1 is written into the other), the dS tile, the item's entries.
template <int D>
struct BwdLds {
    using RowT = SwzTile<bf16_t, D>;
    using ColT = ColTile<D>;
    using DsT = SwzTile<bf16_t, kBlock>;    // [32 rows][128 keys, permuted]
    static constexpr int DSB = 32 * DsT::ROWB;
    BwdTile<D> tile[2];
    unsigned char ds[DSB];
    int entries[kSegBwd];   // the item's list entries (non-local items)
};

// One 8-row x 16-byte unit of the tile staging: rows 16c + {4h..4h+3, 8+4h..8+4h+3}
// (the rows of one transposed 16-byte chunk) at dims 8*dc .. 8*dc+7.
struct StageUnit {
    u32x4 x[8];
};

// Global loads of one staging unit for tile `t` (thread u of the 2*4*(D/8)
// staging threads: tensor u / (4*(D/8)) is Q or dO).
template <int D, int G, bool LOCAL>
__device__ __forceinline__ void stage_load(StageUnit& su, const BwdItem<LOCAL>& it, int t, int u,
                                           const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout, int N,
                                           int Hq) {
    constexpr int DC = D / 8, PPT = 32 / G;
    const int tensor = u / (4 * DC), v = u % (4 * DC);
    const int grp = v & 3, dc = v >> 2;   // the row group varies fastest across lanes
    const int c = grp >> 1, h = grp & 1;
    const bf16_t* src = tensor ? dout : q;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int m = 16 * c + 8 * (e / 4) + 4 * h + e % 4;
        const int pe = t * PPT + m / G;
        su.x[e] = u32x4{0u, 0u, 0u, 0u};
        if (pe < it.count) {
            int i, s;
            it.entry(pe, i, s);
            su.x[e] = *reinterpret_cast<const u32x4*>(src + (((size_t)it.b * N + i) * Hq + it.g * G + m % G) * D +
                                                      dc * 8);
        }
    }
}

// LDS writes of a staged unit: 8 natural 16-byte rows and 8 transposed
// 16-byte chunks (one per dim).
template <int D>
__device__ __forceinline__ void stage_store(const StageUnit& su, BwdTile<D>& sh, int u) {
    constexpr int DC = D / 8;
    const int tensor = u / (4 * DC), v = u % (4 * DC);
    const int grp = v & 3, dc = v >> 2;   // the row group varies fastest across lanes
    const int c = grp >> 1, h = grp & 1;
    unsigned char* nat = tensor ? sh.dout : sh.q;
    unsigned char* tr = tensor ? sh.dot : sh.qt;
    using RowT = typename BwdTile<D>::RowT;
    using ColT = typename BwdTile<D>::ColT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int m = 16 * c + 8 * (e / 4) + 4 * h + e % 4;
        *reinterpret_cast<u32x4*>(nat + RowT::offset(m, dc * 16)) = su.x[e];
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
        *reinterpret_cast<u32x4*>(tr + ColT::offset(dc * 8 + dd, 2 * c + h)) = y;
    }
}

// One work-group (4 waves) per work item: the non-local rows of key block j
// (LOCAL = false), or the rows of query block j against their own block
// under the causal mask (LOCAL = true). Wave w owns keys 32w .. 32w+31 of the
// block for S, dP, dK, dV, and dims 32w .. 32w+31 of the dQ tile.
template <int D, int G, bool LOCAL>
__global__ __launch_bounds__(256, 1) void attn_bwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ kt, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dl, const int32_t* __restrict__ list, const int4* __restrict__ items,
    const int32_t* __restrict__ total_items, bf16_t* __restrict__ dq_part, float* __restrict__ dkv_part, int B, int N,
    int Hkv, int nb, int nwin, int topk, size_t local_base, float scale_log2, float scale) {
    constexpr int PPT = 32 / G, DT = D / 32, KS = D / 16;
    constexpr int NSTAGE = 2 * 4 * (D / 8);   // staging threads
    __shared__ __align__(16) BwdLds<D> sh;
    const int Hq = Hkv * G;

    BwdItem<LOCAL> it;
    size_t pidx;
    if constexpr (LOCAL) {
        const int x = blockIdx.x;
        it.g = x % Hkv;
        it.b = (x / Hkv) % B;
        it.j = x / (Hkv * B);
        it.q0 = it.j * kBlock;
        it.count = min(kBlock, N - it.q0);
        it.lslot = min(topk, it.j + 1) - 1;
        it.start = 0;
        it.entries = nullptr;
        pidx = local_base + ((size_t)it.b * Hkv + it.g) * nb + it.j;
    } else {
        const int item_id = item_of_workgroup(blockIdx.x);
        if (item_id >= total_items[0]) return;
        const int4 e = items[item_id];
        it.j = e.x % nb;
        const int bg = e.x / (nb * nwin);
        it.g = bg % Hkv;
        it.b = bg / Hkv;
        it.start = e.y;
        it.count = e.z;
        it.q0 = 0;
        it.lslot = 0;
        it.entries = sh.entries;
        pidx = item_id;
        for (int x = threadIdx.x; x < it.count; x += blockDim.x) sh.entries[x] = list[it.start + x];
        __syncthreads();
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int ntiles = (it.count + PPT - 1) / PPT;

    // The wave's keys as B operands (S and dP), its dims of K^T as A operands (dQ).
    const int key = 32 * w + col;
    const int kabs = it.j * kBlock + key;
    Op8<bf16_t> kop[KS], vop[KS];
    {
        const size_t roff = (((size_t)it.b * N + kabs) * Hkv + it.g) * D + 8 * half;
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
    }
    Op8<bf16_t> ktop[8];
    if (w < DT) {
        const bf16_t* src = kt + ((((size_t)it.b * Hkv + it.g) * nb + it.j) * D + 32 * w + col) * kBlock + 8 * half;
#pragma unroll
        for (int c = 0; c < 8; ++c) ktop[c].load(src + 16 * c);
    }

    floatx16 dkt[DT], dvt[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dkt[dt] = zero16();
        dvt[dt] = zero16();
    }

    constexpr float kLog2e = 1.4426950408889634f;
    // Spare (row, slot) of the dQ partials, for rows past the item.
    const size_t spare = (size_t)B * Hkv * N * topk;
    // Tiles are staged two ahead: the threads of half `par` (threadIdx.x / 128)
    // stage the tiles t with t % 2 == par, the global loads of tile t + 2
    // being issued while tiles t and t + 1 are on the matrix cores.
    StageUnit su;
    const int par = threadIdx.x >> 7;
    const int u = threadIdx.x & 127;
    if (u < NSTAGE && par < ntiles) stage_load<D, G, LOCAL>(su, it, par, u, q, dout, N, Hq);
    float r_lse = 0.f, r_dl = 0.f;
    int r_pos = -1, r_slot = 0;
    auto row_load = [&](int t) {
        // thread 127 - m of each half loads the scalars of row m (rows past the item: P = 0)
        const int m = 127 - u;
        if (m < 32) {
            const int pe = t * PPT + m / G;
            r_pos = -1;
            r_lse = __builtin_inff();
            r_dl = 0.f;
            if (pe < it.count) {
                int i, s;
                it.entry(pe, i, s);
                const size_t r = ((size_t)it.b * Hq + it.g * G + m % G) * N + i;
                r_pos = i;
                r_slot = s;
                r_lse = lse[r];   // scaled when stored: no use right after the load
                r_dl = dl[r];
            }
        }
    };
    if (par < ntiles) row_load(par);
    // Every load issued so far (the key block's operands, the first two tiles)
    // completes here, so the loop below only ever waits for its own prefetches.
    __builtin_amdgcn_s_waitcnt(0);
    // Staging of tile t into buffer t % 2 by the threads of its parity, who
    // then request tile t + 2.
    auto commit = [&](int t) {
        BwdTile<D>& tb = sh.tile[t & 1];
        if (u < NSTAGE) stage_store<D>(su, tb, u);
        const int m = 127 - u;
        if (m < 32) {
            tb.lse2[m] = r_lse * kLog2e;
            tb.dl[m] = r_dl;
            tb.pos[m] = r_pos;
            tb.slot[m] = r_slot;
        }
        if (t + 2 < ntiles) {
            if (u < NSTAGE) stage_load<D, G, LOCAL>(su, it, t + 2, u, q, dout, N, Hq);
            row_load(t + 2);
        }
    };
    if (par == 0 && ntiles > 0) commit(0);

    for (int t = 0; t < ntiles; ++t) {
        // Tile t is complete in its buffer; the other buffer's readers (tile
        // t - 1) and the dS readers are done.
        __syncthreads();
        const BwdTile<D>& sh_t = sh.tile[t & 1];

        // S = Q K_w^T and dP = dO V_w^T: lane = key, accumulators = rows. The
        // phase's LDS operands are all requested before its first product.
        floatx16 s = zero16(), dp = zero16();
        {
            Op8<bf16_t> a[KS], b[KS];
#pragma unroll
            for (int sl = 0; sl < KS; ++sl) {
                a[sl].load(sh_t.q + BwdLds<D>::RowT::offset(col, (16 * sl + 8 * half) * 2));
                b[sl].load(sh_t.dout + BwdLds<D>::RowT::offset(col, (16 * sl + 8 * half) * 2));
            }
#pragma unroll
            for (int sl = 0; sl < KS; ++sl) {
                mma16(s, a[sl], kop[sl]);
                mma16(dp, b[sl], vop[sl]);
            }
        }
        float rl[16], rd[16];
        int rp[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * half + r % 4;
            rl[r] = sh_t.lse2[m];
            rd[r] = sh_t.dl[m];
            if constexpr (LOCAL) rp[r] = sh_t.pos[m];
        }
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float pr = exp2_hw(fmaf(s[r], scale_log2, -rl[r]));
            if constexpr (LOCAL) {
                if (it.q0 + key > rp[r]) pr = 0.f;   // also the rows past the item (pos = -1)
            }
            p[r] = pr;
            ds[r] = pr * (dp[r] - rd[r]);
        }
        // Staging of tile t + 1 (overlaps tile t's math). It waits for every memory
        // operation before it, so it comes after S and dP (the previous tile's dQ
        // stores have landed by then) and before this tile's stores.
        if (t + 1 < ntiles && ((t + 1) & 1) == par) commit(t + 1);
        // dV^T += dO^T P and dK^T += Q^T dS over the tile's two 16-row slices.
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            Op8<bf16_t> bp, bds;
            PType<bf16_t>::pack(bp, p + 8 * sl);
            PType<bf16_t>::pack(bds, ds + 8 * sl);
            Op8<bf16_t> a[DT], b[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                a[dt].load(sh_t.dot + BwdLds<D>::ColT::offset(32 * dt + col, 2 * sl + half));
                b[dt].load(sh_t.qt + BwdLds<D>::ColT::offset(32 * dt + col, 2 * sl + half));
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                mma16(dvt[dt], a[dt], bp);
                mma16(dkt[dt], b[dt], bds);
            }
        }
        // dS -> LDS as [row][permuted key] for the dQ product.
        {
            uint16_t* dsl = reinterpret_cast<uint16_t*>(sh.ds);
            const int pk = perm16(key);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {   // rows m and m + 1: one conversion, two 16-bit stores
                const int m = 8 * (r / 4) + 4 * half + r % 4;
                const uint32_t v2 = pack_bf16x2(ds[r], ds[r + 1]);
                dsl[BwdLds<D>::DsT::offset(m, pk * 2) / 2] = (uint16_t)(v2 & 0xffffu);
                dsl[BwdLds<D>::DsT::offset(m + 1, pk * 2) / 2] = (uint16_t)(v2 >> 16);
            }
        }
        __syncthreads();
        // dQ^T (dims 32w.., rows) = K^T dS^T over the block's 128 keys.
        if (w < DT) {
            // two accumulation chains (even and odd 16-key slices)
            floatx16 acc = zero16(), acc2 = zero16();
            Op8<bf16_t> b[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) b[c].load(sh.ds + BwdLds<D>::DsT::offset(col, (16 * c + 8 * half) * 2));
#pragma unroll
            for (int c = 0; c < 8; c += 2) {
                mma16(acc, ktop[c], b[c]);
                mma16(acc2, ktop[c + 1], b[c + 1]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] += acc2[r];
            const int i = sh_t.pos[col];
            // partial of (row (b, g, i), slot), head col % G: [G][D] bf16, each 32-dim slice lane-major
            // (element 32w + 16h + r holds dim 32w + 8*(r/4) + 4h + r%4); rows past the item write
            // the spare partial, so the stores are issued on every tile
            const size_t prow = i >= 0 ? (((size_t)it.b * Hkv + it.g) * N + i) * topk + sh_t.slot[col] : spare;
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

    // The item's dK, dV partial: [2][128 keys][D] fp32 (dK scaled by sigma).
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
}

// One work-group per (b, g, key block j): dK_j, dV_j = the local item's
// partial plus the partials of the items of keys (b, g, window, j), windows
// and items in order.
template <int D>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(const float* __restrict__ dkv_part,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ item_offsets, bf16_t* __restrict__ dk,
                                                         bf16_t* __restrict__ dv, int B, int N, int Hkv, int nb, int nwin,
                                                         int seg, size_t local_base, int has_lists) {
    constexpr int PER = 2 * kBlock * D / 4 / 256;   // float4 per thread (dK and dV)
    const int j = blockIdx.x % nb;
    const int bg = blockIdx.x / nb;
    const int g = bg % Hkv, b = bg / Hkv;
    floatx4 acc[PER];
    auto add = [&](size_t p, bool first) {
        const floatx4* src = reinterpret_cast<const floatx4*>(dkv_part + p * 2 * kBlock * D);
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const floatx4 y = __builtin_nontemporal_load(src + threadIdx.x + 256 * x);
            acc[x] = first ? y : acc[x] + y;
        }
    };
    add(local_base + (size_t)bg * nb + j, true);
    if (has_lists) {
        for (int win = 0; win < nwin; ++win) {
            const size_t key = ((size_t)bg * nwin + win) * nb + j;
            const int n = (counts[key] + seg - 1) / seg;
            const int first = item_offsets[key];
            for (int u = 0; u < n; ++u) add((size_t)first + u, false);
        }
    }
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int f = (threadIdx.x + 256 * x) * 4;   // element of [2][128][D]
        const int which = f / (kBlock * D);
        const int key = (f / D) % kBlock, d = f % D;
        const int t = j * kBlock + key;
        if (t < N) {
            bf16_t* dst = (which ? dv : dk) + (((size_t)b * N + t) * Hkv + g) * D + d;
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[x][0], acc[x][1]),
                                                        pack_bf16x2(acc[x][2], acc[x][3]));
        }
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

BwdWorkspace bwd_workspace_layout(const LaunchDims& d) {
    BwdWorkspace w{};
    size_t off = 0;
    w.kt = off;   off = align_up(off + (size_t)d.B * d.Hkv * d.nb * d.D * kBlock * 2);
    w.dl = off;   off = align_up(off + (size_t)d.B * d.Hq() * d.N * 4);
    w.lists = list_layout(d, off, kSegBwd, true);
    off = w.lists.end;
    w.dq_part = off;   off = align_up(off + ((size_t)d.B * d.Hkv * d.N * d.k + 1) * d.G * d.D * 2);   // + spare
    w.local_items = (size_t)d.B * d.Hkv * d.nb;
    w.dkv_items = w.local_items + (w.lists.has_nonlocal ? w.lists.max_items : 0);
    w.dkv_part = off;  off = align_up(off + w.dkv_items * 2 * kBlock * d.D * 4);
    w.bytes = off;
    return w;
}

template <int D, int G>
static hipError_t launch_bwd_t(const LaunchDims& d, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, const void* o, const float* lse, const void* dout,
                               float scale, void* dq, void* dk, void* dv, unsigned char* ws, hipStream_t st) {
    const BwdWorkspace L = bwd_workspace_layout(d);
    const bf16_t* tq = static_cast<const bf16_t*>(q);
    const bf16_t* tk = static_cast<const bf16_t*>(k);
    const bf16_t* tv = static_cast<const bf16_t*>(v);
    const bf16_t* tdo = static_cast<const bf16_t*>(dout);
    bf16_t* kt = reinterpret_cast<bf16_t*>(ws + L.kt);
    float* dl = reinterpret_cast<float*>(ws + L.dl);
    bf16_t* dq_part = reinterpret_cast<bf16_t*>(ws + L.dq_part);
    float* dkv_part = reinterpret_cast<float*>(ws + L.dkv_part);
    const float scale_log2 = scale * 1.4426950408889634f;
    const int nwin = windows(d);

    hipError_t e = launch_transpose_kv(d, k, kt, st);
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)d.B * d.N * d.Hq();
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, st,
                       static_cast<const bf16_t*>(o), tdo, dl, rows, d.N, d.Hq());
    const size_t local_base = L.dkv_items - L.local_items;
    const bool nonlocal = L.lists.has_nonlocal;
    const int32_t* counts = reinterpret_cast<const int32_t*>(ws + L.lists.counts);
    const int32_t* item_offsets = reinterpret_cast<const int32_t*>(ws + L.lists.item_offsets);
    if (nonlocal) {
        launch_build_lists(d, 0, d.N, block_idx, ws, L.lists, st);
        const size_t grid = (list_items_bound(d, 0, d.N, L.lists) + 63) / 64 * 64;
        hipLaunchKernelGGL((attn_bwd_kernel<D, G, false>), dim3((unsigned)grid), dim3(256), 0, st, tq, tk, tv, kt,
                           tdo, lse, dl, reinterpret_cast<const int32_t*>(ws + L.lists.list),
                           reinterpret_cast<const int4*>(ws + L.lists.items),
                           reinterpret_cast<const int32_t*>(ws + L.lists.total), dq_part, dkv_part, d.B, d.N, d.Hkv,
                           d.nb, nwin, d.k, local_base, scale_log2, scale);
    }
    hipLaunchKernelGGL((attn_bwd_kernel<D, G, true>), dim3((unsigned)(d.B * d.Hkv * d.nb)), dim3(256), 0, st,
                       tq, tk, tv, kt, tdo, lse, dl, nullptr, nullptr, nullptr, dq_part, dkv_part, d.B, d.N, d.Hkv,
                       d.nb, nwin, d.k, local_base, scale_log2, scale);
    hipLaunchKernelGGL((dkv_reduce_kernel<D>), dim3((unsigned)(d.B * d.Hkv * d.nb)), dim3(256), 0, st, dkv_part,
                       counts, item_offsets, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), d.B, d.N, d.Hkv, d.nb,
                       nwin, kSegBwd, local_base, nonlocal ? 1 : 0);
    const int64_t units = (int64_t)d.B * d.Hkv * d.N * G * (D / 16);
    hipLaunchKernelGGL((dq_combine_kernel<D, G>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, dq_part,
                       static_cast<bf16_t*>(dq), units, d.N, d.Hkv, d.k, 0, d.N, d.N);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const LaunchDims& d, const void* q, const void* k, const void* v, const int32_t* bi,
                               const void* o, const float* lse, const void* dout, float scale, void* dq, void* dk,
                               void* dv, unsigned char* ws, hipStream_t st) {
    switch (d.G) {
        case 1: return launch_bwd_t<D, 1>(d, q, k, v, bi, o, lse, dout, scale, dq, dk, dv, ws, st);
        case 2: return launch_bwd_t<D, 2>(d, q, k, v, bi, o, lse, dout, scale, dq, dk, dv, ws, st);
        case 4: return launch_bwd_t<D, 4>(d, q, k, v, bi, o, lse, dout, scale, dq, dk, dv, ws, st);
        case 8: return launch_bwd_t<D, 8>(d, q, k, v, bi, o, lse, dout, scale, dq, dk, dv, ws, st);
        case 16: return launch_bwd_t<D, 16>(d, q, k, v, bi, o, lse, dout, scale, dq, dk, dv, ws, st);
        default: return launch_bwd_t<D, 32>(d, q, k, v, bi, o, lse, dout, scale, dq, dk, dv, ws, st);
    }
}

hipError_t launch_sparse_attn_bwd(const LaunchDims& d, const void* q, const void* k, const void* v,
                                  const int32_t* block_idx, const void* o, const float* lse, const void* dout,
                                  float scale, void* dq, void* dk, void* dv, void* ws, hipStream_t st) {
    if (d.B == 0 || d.N == 0) return hipSuccess;
    unsigned char* w = static_cast<unsigned char*>(ws);
    return d.D == 128 ? launch_bwd_d<128>(d, q, k, v, block_idx, o, lse, dout, scale, dq, dk, dv, w, st)
                      : launch_bwd_d<64>(d, q, k, v, block_idx, o, lse, dout, scale, dq, dk, dv, w, st);
}

}  // namespace msa
