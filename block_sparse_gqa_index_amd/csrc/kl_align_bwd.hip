// Backward of the KL alignment term (index branch), gfx950, bf16 inputs.
//
// Method: MiniMax Sparse Attention (MSA) article on 7minutos.es, section "Cómo
// se entrena MSA": the KL loss pulls the index branch toward the main branch's
// attention pattern, and the gradient is stopped at the index branch's input,
// so the loss only trains the index projections: the teacher (group-mean
// main-branch probabilities) is a constant here. The Flash-MSA article
// (tech.kuratif.com), paragraph on the backward: the proxy gradient is computed
// from the cached block indices over the selected blocks only.
//
// For a row (b, g, i) with selected tokens T, weight w (dL/dKL_row):
//   p_t = (1/G) sum_h exp(z_{h,t} - LSE_h)      teacher, z = sigma <q_h, k_t>
//   s_t = exp(c u_t - LSE_u),  u_t = <q_idx, k_idx_t>, c = index_scale
//   dU_t = w c (s_t - p_t)                      (the teacher sums to 1 over T)
//   dq_idx[b,i,g] = sum_t dU_t k_idx_t,  dk_idx[b,t] += dU_t q_idx[b,i,g]
// k_idx is shared by the groups, so dk_idx sums over every group's rows.
//
// Same organisation as the main-branch backward: key-block-outer over the
// position-sorted lists (and the causal local blocks), the wave's 32 keys of K
// and k_idx as B operands in VGPRs, 32-row tiles (32/G positions x G heads)
// staged two ahead. The index query of a position is replicated on its G
// rows, so U = Q_idx K_idx^T comes out in the layout of the teacher's scores;
// the head mean is an in-lane sum (plus one half-wave swap for G >= 8). dk_idx
// accumulates over the item as dk_idx^T += Q_idx^T (dU / G) (each position
// counted once); dq_idx goes through LDS as for dQ and is written by the first
// head row of each position. Fixed-order partial sums: deterministic.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"
#include "msa_bwd_tiles.h"

namespace msa {

// One staged 32-row tile: query rows, index-query rows (natural and
// transposed), per-row scalars.
template <int D, int DI>
struct KlTile {
    using QT = SwzTile<bf16_t, D>;        // [32 rows][D]
    using IT = SwzTile<bf16_t, DI>;       // [32 rows][DI]
    using ICT = ColTile<DI>;              // [DI][32 rows, permuted]
    unsigned char q[32 * QT::ROWB], qi[32 * IT::ROWB], qit[ICT::BYTES];
    float lse2[32], lseu2[32], w[32];
    int pos[32], slot[32];
};

// Two tile buffers (tile t computed from one while tile t + 1 is written into
// the other), the dU tile, the item's entries.
template <int D, int DI>
struct KlBwdLds {
    using QT = SwzTile<bf16_t, D>;
    using IT = SwzTile<bf16_t, DI>;
    using ICT = ColTile<DI>;
    using DuT = SwzTile<bf16_t, kBlock>;  // [32 rows][128 keys, permuted]
    KlTile<D, DI> tile[2];
    unsigned char du[32 * DuT::ROWB];
    int entries[kSegBwd];
};

struct KlUnit {
    u32x4 x[8];
};

// Staging units of one tile: NQ = 4*(D/8) units of query rows (natural layout
// only), then NI = 4*(DI/8) units of index-query rows (natural and transposed).
// Unit v of a tensor: row group v % 4 (rows 16c + {4h..4h+3, 8+4h..8+4h+3}),
// dims 8*(v/4) .. +7.
template <int D, int DI, int G, bool LOCAL>
__device__ __forceinline__ void kl_stage_load(KlUnit& su, const BwdItem<LOCAL>& it, int t, int u,
                                              const bf16_t* __restrict__ q, const bf16_t* __restrict__ q_idx, int N,
                                              int Hkv) {
    constexpr int NQ = 4 * (D / 8), PPT = 32 / G;
    const bool isq = u < NQ;
    const int v = isq ? u : u - NQ;
    const int grp = v & 3, dc = v >> 2;
    const int c = grp >> 1, h = grp & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int m = 16 * c + 8 * (e / 4) + 4 * h + e % 4;
        const int pe = t * PPT + m / G;
        su.x[e] = u32x4{0u, 0u, 0u, 0u};
        if (pe < it.count) {
            int i, s;
            it.entry(pe, i, s);
            const bf16_t* src = isq ? q + (((size_t)it.b * N + i) * Hkv * G + it.g * G + m % G) * D + dc * 8
                                    : q_idx + (((size_t)it.b * N + i) * Hkv + it.g) * DI + dc * 8;
            su.x[e] = *reinterpret_cast<const u32x4*>(src);
        }
    }
}

template <int D, int DI>
__device__ __forceinline__ void kl_stage_store(const KlUnit& su, KlTile<D, DI>& sh, int u) {
    constexpr int NQ = 4 * (D / 8);
    using L = KlTile<D, DI>;
    const bool isq = u < NQ;
    const int v = isq ? u : u - NQ;
    const int grp = v & 3, dc = v >> 2;
    const int c = grp >> 1, h = grp & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int m = 16 * c + 8 * (e / 4) + 4 * h + e % 4;
        if (isq) *reinterpret_cast<u32x4*>(sh.q + L::QT::offset(m, dc * 16)) = su.x[e];
        else *reinterpret_cast<u32x4*>(sh.qi + L::IT::offset(m, dc * 16)) = su.x[e];
    }
    if (!isq) {
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            u32x4 y;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // the 16-bit element dd of rows 2w and 2w + 1 (low and high half of the word)
                y[w] = __builtin_amdgcn_perm(su.x[2 * w + 1][dd / 2], su.x[2 * w][dd / 2],
                                         dd % 2 ? 0x07060302u : 0x05040100u);
            }
            *reinterpret_cast<u32x4*>(sh.qit + L::ICT::offset(dc * 8 + dd, 2 * c + h)) = y;
        }
    }
}


template <int D, int DI, int G, bool LOCAL>
__global__ __launch_bounds__(256, 1) void kl_bwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ q_idx,
    const bf16_t* __restrict__ k_idx, const bf16_t* __restrict__ kit, const float* __restrict__ lse,
    const float* __restrict__ index_lse, const float* __restrict__ dkl_rows, float kl_weight,
    const int32_t* __restrict__ list, const int4* __restrict__ items, const int32_t* __restrict__ total_items,
    bf16_t* __restrict__ dqi_part, float* __restrict__ dki_part, int B, int N, int Hkv, int nb, int nwin, int topk,
    size_t local_base, float scale_log2, float iscale) {
    constexpr int PPT = 32 / G, DIT = DI / 32;
    constexpr int NST = 4 * (D / 8) + 4 * (DI / 8);
    __shared__ __align__(16) KlBwdLds<D, DI> sh;
    using L = KlBwdLds<D, DI>;
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

    const int key = 32 * w + col;
    const int kabs = it.j * kBlock + key;
    Op8<bf16_t> kop[D / 16], kiop[DI / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        if (kabs < N) kop[s].load(k + (((size_t)it.b * N + kabs) * Hkv + it.g) * D + 8 * half + 16 * s);
        else kop[s].zero();
    }
#pragma unroll
    for (int s = 0; s < DI / 16; ++s) {
        if (kabs < N) kiop[s].load(k_idx + ((size_t)it.b * N + kabs) * DI + 8 * half + 16 * s);
        else kiop[s].zero();
    }
    Op8<bf16_t> kitop[8];
    if (w < DIT) {
        const bf16_t* src = kit + (((size_t)it.b * nb + it.j) * DI + 32 * w + col) * kBlock + 8 * half;
#pragma unroll
        for (int c = 0; c < 8; ++c) kitop[c].load(src + 16 * c);
    }
    floatx16 dkit[DIT];
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt) dkit[dt] = zero16();

    constexpr float kLog2e = 1.4426950408889634f;
    const float iscale_log2 = iscale * kLog2e;
    KlUnit su;
    const int par = threadIdx.x >> 7;
    const int u = threadIdx.x & 127;
    if (u < NST && par < ntiles) kl_stage_load<D, DI, G, LOCAL>(su, it, par, u, q, q_idx, N, Hkv);
    float r_lse = 0.f, r_lseu = 0.f, r_w = 0.f;
    int r_pos = -1, r_slot = 0;
    auto row_load = [&](int t) {
        const int m = 127 - u;
        if (m < 32) {
            const int pe = t * PPT + m / G;
            r_pos = -1;
            r_lse = __builtin_inff();
            r_lseu = __builtin_inff();
            r_w = 0.f;
            if (pe < it.count) {
                int i, s;
                it.entry(pe, i, s);
                const size_t rr = ((size_t)it.b * Hkv + it.g) * N + i;
                r_pos = i;
                r_slot = s;
                r_lse = lse[((size_t)it.b * Hq + it.g * G + m % G) * N + i];
                r_lseu = index_lse[rr];
                r_w = dkl_rows ? dkl_rows[rr] : 1.f;
            }
        }
    };
    if (par < ntiles) row_load(par);
    __builtin_amdgcn_s_waitcnt(0);
    // Staging of tile t into buffer t % 2 by the threads of its parity, who
    // then request tile t + 2.
    auto commit = [&](int t) {
        KlTile<D, DI>& tb = sh.tile[t & 1];
        if (u < NST) kl_stage_store<D, DI>(su, tb, u);
        const int m = 127 - u;
        if (m < 32) {
            tb.lse2[m] = r_lse * kLog2e;
            tb.lseu2[m] = r_lseu * kLog2e;
            tb.w[m] = r_w * kl_weight * iscale;
            tb.pos[m] = r_pos;
            tb.slot[m] = r_slot;
        }
        if (t + 2 < ntiles) {
            if (u < NST) kl_stage_load<D, DI, G, LOCAL>(su, it, t + 2, u, q, q_idx, N, Hkv);
            row_load(t + 2);
        }
    };
    if (par == 0 && ntiles > 0) commit(0);

    for (int t = 0; t < ntiles; ++t) {
        // Tile t is complete in its buffer; the other buffer's readers (tile
        // t - 1) and the dU readers are done.
        __syncthreads();
        if (t + 1 < ntiles && ((t + 1) & 1) == par) commit(t + 1);   // overlaps tile t's math
        const KlTile<D, DI>& sh_t = sh.tile[t & 1];

        // S = Q K_w^T (teacher scores) and U = Q_idx K_idx,w^T (student logits / c).
        floatx16 s = zero16(), uu = zero16();
#pragma unroll
        for (int sl = 0; sl < D / 16; ++sl) {
            Op8<bf16_t> a;
            a.load(sh_t.q + L::QT::offset(col, (16 * sl + 8 * half) * 2));
            mma16(s, a, kop[sl]);
        }
#pragma unroll
        for (int sl = 0; sl < DI / 16; ++sl) {
            Op8<bf16_t> a;
            a.load(sh_t.qi + L::IT::offset(col, (16 * sl + 8 * half) * 2));
            mma16(uu, a, kiop[sl]);
        }
        float p[16], du[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * half + r % 4;
            float pr = exp2_hw(fmaf(s[r], scale_log2, -sh_t.lse2[m]));
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) pr = 0.f;
            }
            p[r] = pr;
        }
        head_mean<G>(p);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r / 4) + 4 * half + r % 4;
            float st = exp2_hw(fmaf(uu[r], iscale_log2, -sh_t.lseu2[m]));
            if constexpr (LOCAL) {
                if (it.q0 + key > sh_t.pos[m]) st = 0.f;
            }
            du[r] = sh_t.w[m] * (st - p[r]);
        }
        // dk_idx^T += Q_idx^T (dU / G): every position's G replicated rows count once.
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = du[8 * sl + e] * (1.f / G);
            Op8<bf16_t> b;
            PType<bf16_t>::pack(b, x);
#pragma unroll
            for (int dt = 0; dt < DIT; ++dt) {
                Op8<bf16_t> a;
                a.load(sh_t.qit + L::ICT::offset(32 * dt + col, 2 * sl + half));
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
        // dq_idx^T (dims 32w.., rows) = K_idx^T dU^T over the block's 128 keys;
        // the first head row of each position writes it.
        if (w < DIT) {
            floatx16 acc = zero16();
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                Op8<bf16_t> b;
                b.load(sh.du + L::DuT::offset(col, (16 * c + 8 * half) * 2));
                mma16(acc, kitop[c], b);
            }
            const int i = sh_t.pos[col];
            if (i >= 0 && col % G == 0) {
                bf16_t* dst = dqi_part + ((((size_t)it.b * Hkv + it.g) * N + i) * topk + sh_t.slot[col]) * DI +
                              32 * w + 16 * half;
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

// One work-group per (b, key block j): dk_idx of the block's keys = for each
// group in order, its local item's partial, then the partials of the items of
// (b, g, window, j), windows and items in order.
template <int DI>
__global__ __launch_bounds__(256) void dki_reduce_kernel(const float* __restrict__ dki_part,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ item_offsets,
                                                         bf16_t* __restrict__ dk_idx, int N, int Hkv, int nb, int nwin,
                                                         int seg, size_t local_base, int has_lists) {
    constexpr int PER = kBlock * DI / 4 / 256;
    const int j = blockIdx.x % nb;
    const int b = blockIdx.x / nb;
    floatx4 acc[PER];
#pragma unroll
    for (int x = 0; x < PER; ++x) acc[x] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto add = [&](size_t p) {
        const floatx4* src = reinterpret_cast<const floatx4*>(dki_part + p * kBlock * DI);
#pragma unroll
        for (int x = 0; x < PER; ++x) acc[x] += __builtin_nontemporal_load(src + threadIdx.x + 256 * x);
    };
    for (int g = 0; g < Hkv; ++g) {
        const int bg = b * Hkv + g;
        add(local_base + (size_t)bg * nb + j);
        if (has_lists) {
            for (int win = 0; win < nwin; ++win) {
                const size_t key = ((size_t)bg * nwin + win) * nb + j;
                const int n = (counts[key] + seg - 1) / seg;
                const int first = item_offsets[key];
                for (int v = 0; v < n; ++v) add((size_t)first + v);
            }
        }
    }
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int f = (threadIdx.x + 256 * x) * 4;
        const int kk = f / DI, d = f % DI;
        const int t = j * kBlock + kk;
        if (t < N)
            *reinterpret_cast<uint2*>(dk_idx + ((size_t)b * N + t) * DI + d) =
                make_uint2(pack_bf16x2(acc[x][0], acc[x][1]), pack_bf16x2(acc[x][2], acc[x][3]));
    }
}

// -------------------------------------------------------------------- host --

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

KlBwdWorkspace kl_bwd_workspace_layout(const LaunchDims& d) {
    KlBwdWorkspace w{};
    size_t off = 0;
    w.kit = off;  off = align_up(off + (size_t)d.B * d.nb * d.Di * kBlock * 2);
    w.lists = list_layout(d, off, kSegBwd, true);
    off = w.lists.end;
    w.dqi_part = off;  off = align_up(off + (size_t)d.B * d.Hkv * d.N * d.k * d.Di * 2);
    w.local_items = (size_t)d.B * d.Hkv * d.nb;
    w.dki_items = w.local_items + (w.lists.has_nonlocal ? w.lists.max_items : 0);
    w.dki_part = off;  off = align_up(off + w.dki_items * kBlock * d.Di * 4);
    w.bytes = off;
    return w;
}

template <int D, int DI, int G>
static hipError_t launch_kl_bwd_t(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                                  const void* k_idx, const int32_t* block_idx, const float* lse,
                                  const float* index_lse, float scale, float iscale, const float* dkl_rows,
                                  float kl_weight, void* dq_idx, void* dk_idx, unsigned char* ws, hipStream_t st) {
    const KlBwdWorkspace L = kl_bwd_workspace_layout(d);
    const bf16_t* tq = static_cast<const bf16_t*>(q);
    const bf16_t* tk = static_cast<const bf16_t*>(k);
    const bf16_t* tqi = static_cast<const bf16_t*>(q_idx);
    const bf16_t* tki = static_cast<const bf16_t*>(k_idx);
    bf16_t* kit = reinterpret_cast<bf16_t*>(ws + L.kit);
    bf16_t* dqi_part = reinterpret_cast<bf16_t*>(ws + L.dqi_part);
    float* dki_part = reinterpret_cast<float*>(ws + L.dki_part);
    const float scale_log2 = scale * 1.4426950408889634f;
    const int nwin = windows(d);

    LaunchDims di = d;   // k_idx as a one-head [B, N, 1, Di] tensor
    di.Hkv = 1;
    di.G = 1;
    di.D = d.Di;
    hipError_t e = launch_transpose_kv(di, k_idx, kit, st);
    if (e != hipSuccess) return e;
    const size_t local_base = L.dki_items - L.local_items;
    const bool nonlocal = L.lists.has_nonlocal;
    if (nonlocal) {
        launch_build_lists(d, 0, d.N, block_idx, ws, L.lists, st);
        const size_t grid = (list_items_bound(d, 0, d.N, L.lists) + 63) / 64 * 64;
        hipLaunchKernelGGL((kl_bwd_kernel<D, DI, G, false>), dim3((unsigned)grid), dim3(256), 0, st, tq, tk, tqi, tki,
                           kit, lse, index_lse, dkl_rows, kl_weight,
                           reinterpret_cast<const int32_t*>(ws + L.lists.list),
                           reinterpret_cast<const int4*>(ws + L.lists.items),
                           reinterpret_cast<const int32_t*>(ws + L.lists.total), dqi_part, dki_part, d.B, d.N, d.Hkv,
                           d.nb, nwin, d.k, local_base, scale_log2, iscale);
    }
    hipLaunchKernelGGL((kl_bwd_kernel<D, DI, G, true>), dim3((unsigned)(d.B * d.Hkv * d.nb)), dim3(256), 0, st, tq,
                       tk, tqi, tki, kit, lse, index_lse, dkl_rows, kl_weight, nullptr, nullptr, nullptr, dqi_part,
                       dki_part, d.B, d.N, d.Hkv, d.nb, nwin, d.k, local_base, scale_log2, iscale);
    hipLaunchKernelGGL((dki_reduce_kernel<DI>), dim3((unsigned)(d.B * d.nb)), dim3(256), 0, st, dki_part,
                       reinterpret_cast<const int32_t*>(ws + L.lists.counts),
                       reinterpret_cast<const int32_t*>(ws + L.lists.item_offsets), static_cast<bf16_t*>(dk_idx), d.N,
                       d.Hkv, d.nb, nwin, kSegBwd, local_base, nonlocal ? 1 : 0);
    const int64_t units = (int64_t)d.B * d.Hkv * d.N * (DI / 16);
    hipLaunchKernelGGL((dq_combine_kernel<DI, 1>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, dqi_part,
                       static_cast<bf16_t*>(dq_idx), units, d.N, d.Hkv, d.k, 0, d.N, d.N);
    return hipGetLastError();
}

template <int D, int DI>
static hipError_t launch_kl_bwd_g(const LaunchDims& d, const void* q, const void* k, const void* qi, const void* ki,
                                  const int32_t* bi, const float* lse, const float* ilse, float sc, float isc,
                                  const float* dkl, float kw, void* dqi, void* dki, unsigned char* ws, hipStream_t st) {
    switch (d.G) {
        case 1: return launch_kl_bwd_t<D, DI, 1>(d, q, k, qi, ki, bi, lse, ilse, sc, isc, dkl, kw, dqi, dki, ws, st);
        case 2: return launch_kl_bwd_t<D, DI, 2>(d, q, k, qi, ki, bi, lse, ilse, sc, isc, dkl, kw, dqi, dki, ws, st);
        case 4: return launch_kl_bwd_t<D, DI, 4>(d, q, k, qi, ki, bi, lse, ilse, sc, isc, dkl, kw, dqi, dki, ws, st);
        case 8: return launch_kl_bwd_t<D, DI, 8>(d, q, k, qi, ki, bi, lse, ilse, sc, isc, dkl, kw, dqi, dki, ws, st);
        case 16: return launch_kl_bwd_t<D, DI, 16>(d, q, k, qi, ki, bi, lse, ilse, sc, isc, dkl, kw, dqi, dki, ws, st);
        default: return launch_kl_bwd_t<D, DI, 32>(d, q, k, qi, ki, bi, lse, ilse, sc, isc, dkl, kw, dqi, dki, ws, st);
    }
}

hipError_t launch_kl_align_bwd(const LaunchDims& d, const void* q, const void* k, const void* q_idx,
                               const void* k_idx, const int32_t* block_idx, const float* lse,
                               const float* index_lse, float scale, float index_scale, const float* dkl_rows,
                               float kl_weight, void* dq_idx, void* dk_idx, void* ws, hipStream_t st) {
    if (d.B == 0 || d.N == 0) return hipSuccess;
    unsigned char* w = static_cast<unsigned char*>(ws);
    if (d.D == 128 && d.Di == 128)
        return launch_kl_bwd_g<128, 128>(d, q, k, q_idx, k_idx, block_idx, lse, index_lse, scale, index_scale,
                                         dkl_rows, kl_weight, dq_idx, dk_idx, w, st);
    if (d.D == 128)
        return launch_kl_bwd_g<128, 64>(d, q, k, q_idx, k_idx, block_idx, lse, index_lse, scale, index_scale,
                                        dkl_rows, kl_weight, dq_idx, dk_idx, w, st);
    if (d.Di == 128)
        return launch_kl_bwd_g<64, 128>(d, q, k, q_idx, k_idx, block_idx, lse, index_lse, scale, index_scale,
                                        dkl_rows, kl_weight, dq_idx, dk_idx, w, st);
    return launch_kl_bwd_g<64, 64>(d, q, k, q_idx, k_idx, block_idx, lse, index_lse, scale, index_scale, dkl_rows,
                                   kl_weight, dq_idx, dk_idx, w, st);
}

}  // namespace msa
