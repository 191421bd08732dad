// Dense causal GQA attention forward: the main branch with every causally
// visible key kept, as the indexer warm-up runs it (MiniMax Sparse Attention
// article on 7minutos.es, "Cómo se entrena MSA": during the first iterations
// both branches attend to everything). It is the limit k >= (visible blocks)
// of the block-sparse attention, computed without the selection and without
// per-block partial outputs, which at that k would need Θ(N^2) workspace.
//
// Query-block outer (flash-attention order): one work-group per (batch, query
// block, group, part) of 256 rows (32-row tiles of 32/G positions x G heads of
// the block's 128*G rows; 8 waves x 1 tile, two waves per SIMD), held for the
// whole sweep over key blocks 0 .. qb. K_j and V_j^T (from the per-block
// transposed copy of V) sit in LDS in the swizzled layout of the sparse
// kernels, in two buffers: the next block's K/V are copied into the other
// buffer while the current block is computed (bf16: global -> LDS directly;
// fp32: through registers, stored after the block's math), so one barrier per
// key block separates the two.
// Per block and tile: S^T = K Q^T, online softmax (log2 domain, running max
// and sum per row, accumulator rescaled), O^T += V^T P^T. The local block
// (j = qb) is masked causally; heavy (late) query blocks are launched first.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"

namespace msa {

namespace {

// K block [128][D] (PART 0) or V^T block [D][128] (PART 1) moved global ->
// registers -> LDS in the KVTile layout by NT threads: thread t owns chunks
// t, t + NT, ... The two halves are separate so that only one is held in
// registers at a time.
template <typename T, int D, int PART, int NT>
struct KVPrefetch {
    using KS = SwzTile<T, D>;
    using VS = SwzTile<T, kBlock>;
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = PART == 0 ? KS::CPR : VS::CPR;
    static constexpr int CH = PART == 0 ? kBlock * KS::CPR : D * VS::CPR;
    static constexpr int PER = CH / NT;
    static_assert(CH % NT == 0, "chunk split");
    u32x4 r[PER];

    // PART 0: src = first key row (rows row_stride elements apart, zero past
    // valid_keys); PART 1: src = the block's V^T [D][128].
    __device__ __forceinline__ void load(const T* src, size_t row_stride, int valid_keys) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int ch = threadIdx.x + u * NT;
            const int row = ch / CPR, cc = ch % CPR;
            if constexpr (PART == 0)
                r[u] = row < valid_keys ? *reinterpret_cast<const u32x4*>(src + row * row_stride + cc * EPC)
                                        : u32x4{0u, 0u, 0u, 0u};
            else
                r[u] = *reinterpret_cast<const u32x4*>(src + (size_t)row * kBlock + cc * EPC);
        }
    }
    __device__ __forceinline__ void commit(unsigned char* lds) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int ch = threadIdx.x + u * NT;
            const int row = ch / CPR, cc = ch % CPR;
            if constexpr (PART == 0)
                *reinterpret_cast<u32x4*>(lds + KS::offset(row, cc * 16)) = r[u];
            else
                *reinterpret_cast<u32x4*>(lds + kBlock * KS::ROWB + VS::offset(row, cc * 16)) = r[u];
        }
    }
};

// NW waves per work-group, TPW 32-row tiles per wave: every K or V^T operand
// read from LDS feeds TPW matrix-core ops (one per tile), which halves the LDS
// traffic per op at TPW = 2 (one wave per SIMD then, with the two tiles'
// independent chains interleaved in it).
template <typename T, int D, int G, int NBUF, int NW, int TPW>
__global__ __launch_bounds__(NW * kWave) void dense_attn_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                const T* __restrict__ vt, T* __restrict__ o,
                                                                float* __restrict__ lse, int B, int N, int Hkv,
                                                                int nb, int parts, float scale_log2) {
    using KV = KVTile<T, D>;
    using KS = SwzTile<T, D>;
    constexpr int NT = NW * kWave;
    __shared__ __align__(16) unsigned char lds[NBUF * KV::BYTES];
    // The parts of one (batch, query block, group) unit read the same K/V
    // blocks at about the same time: runs of 8 * parts work-groups give each of
    // the 8 XCDs (work-group x runs on XCD x % 8) one whole unit, so its parts
    // share that XCD's L2. Units are numbered latest (heaviest) query block first.
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
    const int tile0 = (pt * NW + w) * TPW;
    const bool wave_ok = tile0 < kBlock * G / 32;   // tiles past the block's rows compute nothing
    const int hh = col % G;
    const int h = g * G + hh;
    int p[TPW];
    bool valid[TPW];
    Op8<T> bq[TPW][D / 16];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        p[t] = ((tile0 + t) * 32 + col) / G;   // position within the query block
        valid[t] = tile0 + t < kBlock * G / 32 && q0 + p[t] < N;
        load_q_op<T, D>(bq[t], q + ((size_t)b * N + (valid[t] ? q0 + p[t] : 0)) * Hq * D + (size_t)h * D, valid[t],
                        half);
    }

    const size_t kv_row = (size_t)Hkv * D;
    const T* kbase = k + (size_t)b * N * kv_row + (size_t)g * D;
    const T* vtbase = vt + ((size_t)b * Hkv + g) * nb * D * kBlock;
    KVPrefetch<T, D, 0, NT> pk;
    KVPrefetch<T, D, 1, NT> pv;
    // bf16 with two buffers: K_{j+1} and V_{j+1} are copied global -> LDS
    // directly (no registers) into the other buffer at the start of block j;
    // the barrier that ends block j waits for them. Rows of K past the
    // sequence repeat its last key (masked for every stored row).
    constexpr bool kDma = sizeof(T) == 2 && NBUF == 2;
    auto dma_kv = [&](unsigned char* buf, int jb) {
        if constexpr (kDma) {
            constexpr int KROWS = 64 / KS::CPR, VROWS = 64 / SwzTile<T, kBlock>::CPR;
            const int last = min(kBlock, N - jb * kBlock) - 1;
            for (int r0 = w * KROWS; r0 < kBlock; r0 += NW * KROWS)
                dma_rows<D>(buf, reinterpret_cast<const bf16_t*>(kbase) + (size_t)jb * kBlock * kv_row, kv_row, r0,
                            last, lane);
            for (int r0 = w * VROWS; r0 < D; r0 += NW * VROWS)
                dma_rows<kBlock>(buf + kBlock * KS::ROWB,
                                 reinterpret_cast<const bf16_t*>(vtbase) + (size_t)jb * D * kBlock, kBlock, r0, D - 1,
                                 lane);
        }
    };
    if constexpr (kDma) {
        dma_kv(lds, 0);
    } else {
        pk.load(kbase, kv_row, min(kBlock, N));
        pv.load(vtbase, 0, 0);
        pk.commit(lds);
        pv.commit(lds);
    }
    __syncthreads();

    float m_run[TPW], l_run[TPW];
    floatx16 acc[TPW][D / 32];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        m_run[t] = -__builtin_inff();
        l_run[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[t][dt] = zero16();
    }

    for (int j = 0; j <= qb; ++j) {
        const unsigned char* cur = lds + (NBUF == 2 ? (j & 1) * KV::BYTES : 0);
        unsigned char* nxt = lds + (NBUF == 2 ? ((j + 1) & 1) * KV::BYTES : 0);
        const bool more = j < qb;
        // Double-buffered: K_{j+1} is requested before block j's scores and
        // stored after them, V^T_{j+1} requested after the softmax and stored
        // after the P V product. Single-buffered: both are stored after a
        // barrier that ends block j.
        if constexpr (kDma) {
            if (more) dma_kv(nxt, j + 1);
        } else {
            if (more) pk.load(kbase + (size_t)(j + 1) * kBlock * kv_row, kv_row, min(kBlock, N - (j + 1) * kBlock));
        }
        if (wave_ok) {
            floatx16 s[TPW][4];
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) s[t][kt] = zero16();
            // Slice outer, key tile inner: four independent accumulation chains.
#pragma unroll
            for (int sl = 0; sl < D / 16; ++sl) {
                Op8<T> a[4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) KS::load8(a[kt], cur, kt * 32 + col, 16 * sl + 8 * half);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int t = 0; t < TPW; ++t) mma16(s[t][kt], a[kt], bq[t][sl]);
            }
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                if (j == qb) {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                            if (key > p[t]) s[t][kt][r] = -__builtin_inff();
                        }
                    }
                }
                float m = -__builtin_inff();
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) m = vmax(m, max16(s[t][kt]));
                m = vmax(m, swap_halves(m));
                const float m_new = fmaxf(m_run[t], m * scale_log2);   // finite: every block has a visible key
                const float alpha = exp2_hw(m_run[t] - m_new);
                float l = 0.f;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = exp2_hw(fmaf(s[t][kt][r], scale_log2, -m_new));
                        s[t][kt][r] = e;
                        l += e;
                    }
                }
                l += swap_halves(l);
                l_run[t] = fmaf(l_run[t], alpha, l);
                m_run[t] = m_new;
                // Most blocks raise no row's maximum (alpha == 1 everywhere):
                // the wave then skips the rescale of its accumulators.
                if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[t][dt][r] *= alpha;
                    }
                }
            }
            if constexpr (NBUF == 2 && !kDma) {
                if (more) {
                    pv.load(vtbase + (size_t)(j + 1) * D * kBlock, 0, 0);
                    pk.commit(nxt);
                }
            }
            // O^T += V^T P^T, 16-key slice c: P from the score accumulators.
            const unsigned char* vtl = cur + kBlock * KS::ROWB;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                Op8<T> bp[TPW];
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    float pe[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pe[e] = s[t][c / 2][8 * (c % 2) + e];
                    PType<T>::pack(bp[t], pe);
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    Op8<T> a;
                    load_vt_op<T>(a, vtl, dt * 32 + col, c, half);
#pragma unroll
                    for (int t = 0; t < TPW; ++t) mma16(acc[t][dt], a, bp[t]);
                }
            }
        } else if constexpr (NBUF == 2 && !kDma) {
            if (more) {
                pv.load(vtbase + (size_t)(j + 1) * D * kBlock, 0, 0);
                pk.commit(nxt);
            }
        }
        if (more) {
            if constexpr (kDma) {
            } else if constexpr (NBUF == 2) {
                pv.commit(nxt);
            } else {
                pv.load(vtbase + (size_t)(j + 1) * D * kBlock, 0, 0);
                __syncthreads();   // everyone is done reading the single buffer
                pk.commit(nxt);
                pv.commit(nxt);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        if (!valid[t]) continue;
        const int i = q0 + p[t];
        const float inv = 1.0f / l_run[t];
        T* dst = o + ((size_t)b * N + i) * Hq * D + (size_t)h * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                T* d4 = dst + dt * 32 + 8 * rq + 4 * half;
                if constexpr (sizeof(T) == 2) {
                    const uint32_t a0 = pack_bf16x2(acc[t][dt][4 * rq] * inv, acc[t][dt][4 * rq + 1] * inv);
                    const uint32_t a1 = pack_bf16x2(acc[t][dt][4 * rq + 2] * inv, acc[t][dt][4 * rq + 3] * inv);
                    *reinterpret_cast<uint2*>(d4) = make_uint2(a0, a1);
                } else {
                    floatx4 y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = acc[t][dt][4 * rq + e] * inv;
                    *reinterpret_cast<floatx4*>(d4) = y;
                }
            }
        }
        if (half == 0) lse[((size_t)b * Hq + h) * N + i] = (m_run[t] + log2f(l_run[t])) * 0.69314718055994531f;
    }
}

template <typename T, int D, int G>
void launch_dense_t(const LaunchDims& d, const void* q, const void* k, const void* vt, void* o, float* lse,
                    float scale_log2, hipStream_t st) {
    // 8 waves x 1 tile: two waves per SIMD. (Two tiles per wave, one wave per
    // SIMD, would halve the LDS operand traffic but needs more than the 512
    // registers a wave can hold, and the kernel's limit is the softmax's VALU
    // work, not LDS.)
    constexpr int NW = 8;
    constexpr int TPW = 1;
    constexpr int kTiles = kBlock * G / 32;
    const int parts = (kTiles + NW * TPW - 1) / (NW * TPW);
    constexpr int NBUF = 2 * KVTile<T, D>::BYTES <= 160 * 1024 ? 2 : 1;
    const size_t units = (size_t)d.nb * d.B * d.Hkv;
    const size_t grid = (units + 7) / 8 * 8 * parts;
    hipLaunchKernelGGL((dense_attn_kernel<T, D, G, NBUF, NW, TPW>), dim3((unsigned)grid), dim3(NW * kWave), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(vt),
                       static_cast<T*>(o), lse, d.B, d.N, d.Hkv, d.nb, parts, scale_log2);
}

template <typename T, int D>
void launch_dense_g(const LaunchDims& d, const void* q, const void* k, const void* vt, void* o, float* lse,
                    float scale_log2, hipStream_t st) {
    switch (d.G) {
        case 1: launch_dense_t<T, D, 1>(d, q, k, vt, o, lse, scale_log2, st); break;
        case 2: launch_dense_t<T, D, 2>(d, q, k, vt, o, lse, scale_log2, st); break;
        case 4: launch_dense_t<T, D, 4>(d, q, k, vt, o, lse, scale_log2, st); break;
        case 8: launch_dense_t<T, D, 8>(d, q, k, vt, o, lse, scale_log2, st); break;
        case 16: launch_dense_t<T, D, 16>(d, q, k, vt, o, lse, scale_log2, st); break;
        default: launch_dense_t<T, D, 32>(d, q, k, vt, o, lse, scale_log2, st); break;
    }
}

}  // namespace

size_t dense_workspace_bytes(const LaunchDims& d) {
    const size_t es = d.dtype == 0 ? 2 : 4;
    return ((size_t)d.B * d.Hkv * d.nb * d.D * kBlock * es + 255) & ~(size_t)255;
}

hipError_t launch_dense_attn(const LaunchDims& d, const void* q, const void* k, const void* v, float scale, void* o,
                             float* lse, void* ws, hipStream_t st) {
    if (launch_transpose_kv(d, v, ws, st) != hipSuccess) return hipGetLastError();
    const float scale_log2 = scale * 1.4426950408889634f;
    if (d.dtype == 0) {
        if (d.D == 128) launch_dense_g<bf16_t, 128>(d, q, k, ws, o, lse, scale_log2, st);
        else launch_dense_g<bf16_t, 64>(d, q, k, ws, o, lse, scale_log2, st);
    } else {
        if (d.D == 128) launch_dense_g<float, 128>(d, q, k, ws, o, lse, scale_log2, st);
        else launch_dense_g<float, 64>(d, q, k, ws, o, lse, scale_log2, st);
    }
    return hipGetLastError();
}

}  // namespace msa
