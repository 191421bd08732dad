// Dense causal GQA attention forward: the main branch with every causally
// visible key kept, as the indexer warm-up runs it (MiniMax Sparse Attention
// article on 7minutos.es, "Cómo se entrena MSA": during the first iterations
// both branches attend to everything). It is the limit k >= (visible blocks)
// of the block-sparse attention, computed without the selection and without
// per-block partial outputs, which at that k would need Θ(N^2) workspace.
//
// Query-block outer (flash-attention order): one work-group of 8 waves per
// (batch, query block, group, part), each wave one 32-row tile (32/G positions
// x G heads of the block's 128*G rows) held for the whole sweep over key
// blocks 0 .. qb. K_j and V_j^T (from the per-block transposed copy of V) sit
// in LDS in the swizzled layout of the sparse kernels; the next block's K/V are
// requested into registers before the current block's math and written to the
// other LDS buffer after it, so one barrier per key block separates the two.
// Per block and tile: S^T = K Q^T, online softmax (log2 domain, running max
// and sum per row, accumulator rescaled), O^T += V^T P^T. The local block
// (j = qb) is masked causally; heavy (late) query blocks are launched first.
#include "msa_common.h"
#include "msa_internal.h"
#include "msa_tiles.h"

namespace msa {

namespace {

constexpr int kDenseWaves = 8;
constexpr int kDenseThreads = kDenseWaves * kWave;

// K block [128][D] (PART 0) or V^T block [D][128] (PART 1) moved global ->
// registers -> LDS in the KVTile layout: thread t owns chunks t, t + NT, ...
// The two halves are separate so that only one is held in registers at a time.
template <typename T, int D, int PART>
struct KVPrefetch {
    using KS = SwzTile<T, D>;
    using VS = SwzTile<T, kBlock>;
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = PART == 0 ? KS::CPR : VS::CPR;
    static constexpr int CH = PART == 0 ? kBlock * KS::CPR : D * VS::CPR;
    static constexpr int PER = CH / kDenseThreads;
    static_assert(CH % kDenseThreads == 0, "chunk split");
    u32x4 r[PER];

    // PART 0: src = first key row (rows row_stride elements apart, zero past
    // valid_keys); PART 1: src = the block's V^T [D][128].
    __device__ __forceinline__ void load(const T* src, size_t row_stride, int valid_keys) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int ch = threadIdx.x + u * kDenseThreads;
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
            const int ch = threadIdx.x + u * kDenseThreads;
            const int row = ch / CPR, cc = ch % CPR;
            if constexpr (PART == 0)
                *reinterpret_cast<u32x4*>(lds + KS::offset(row, cc * 16)) = r[u];
            else
                *reinterpret_cast<u32x4*>(lds + kBlock * KS::ROWB + VS::offset(row, cc * 16)) = r[u];
        }
    }
};

template <typename T, int D, int G, int NBUF>
__global__ __launch_bounds__(kDenseThreads) void dense_attn_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                   const T* __restrict__ vt, T* __restrict__ o,
                                                                   float* __restrict__ lse, int B, int N, int Hkv,
                                                                   int nb, int parts, float scale_log2) {
    using KV = KVTile<T, D>;
    __shared__ __align__(16) unsigned char lds[NBUF * KV::BYTES];
    const int x = blockIdx.x;
    const int pt = x % parts;
    const int g = (x / parts) % Hkv;
    const int b = (x / (parts * Hkv)) % B;
    const int qb = nb - 1 - x / (parts * Hkv * B);   // latest (heaviest) query blocks first
    const int Hq = Hkv * G;
    const int q0 = qb * kBlock;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int tile = pt * kDenseWaves + w;
    const bool tile_ok = tile < kBlock * G / 32;
    const int p = (tile * 32 + col) / G;   // position within the query block
    const int hh = col % G;
    const int h = g * G + hh;
    const int i = q0 + p;
    const bool valid = tile_ok && i < N;
    Op8<T> bq[D / 16];
    load_q_op<T, D>(bq, q + ((size_t)b * N + (valid ? i : 0)) * Hq * D + (size_t)h * D, valid, half);

    const size_t kv_row = (size_t)Hkv * D;
    const T* kbase = k + (size_t)b * N * kv_row + (size_t)g * D;
    const T* vtbase = vt + ((size_t)b * Hkv + g) * nb * D * kBlock;
    KVPrefetch<T, D, 0> pk;
    KVPrefetch<T, D, 1> pv;
    pk.load(kbase, kv_row, min(kBlock, N));
    pv.load(vtbase, 0, 0);
    pk.commit(lds);
    pv.commit(lds);
    __syncthreads();

    float m_run = -__builtin_inff(), l_run = 0.f;
    floatx16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();

    for (int j = 0; j <= qb; ++j) {
        const unsigned char* cur = lds + (NBUF == 2 ? (j & 1) * KV::BYTES : 0);
        unsigned char* nxt = lds + (NBUF == 2 ? ((j + 1) & 1) * KV::BYTES : 0);
        const bool more = j < qb;
        // Double-buffered: K_{j+1} is requested before block j's scores and
        // stored after them, V^T_{j+1} requested after the softmax and stored
        // after the P V product. Single-buffered: both are stored after a
        // barrier that ends block j.
        if (more) pk.load(kbase + (size_t)(j + 1) * kBlock * kv_row, kv_row, min(kBlock, N - (j + 1) * kBlock));
        if (tile_ok) {
            floatx16 s[4];
            tile_scores<T, D, false>(s, bq, cur, col, half);
            if (j == qb) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                        if (key > p) s[kt][r] = -__builtin_inff();
                    }
                }
            }
            float m = -__builtin_inff();
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) m = vmax(m, max16(s[kt]));
            m = vmax(m, swap_halves(m));
            const float m_new = fmaxf(m_run, m * scale_log2);   // finite: every block has a visible key
            const float alpha = exp2_hw(m_run - m_new);
            float l = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = exp2_hw(fmaf(s[kt][r], scale_log2, -m_new));
                    s[kt][r] = e;
                    l += e;
                }
            }
            l += swap_halves(l);
            l_run = fmaf(l_run, alpha, l);
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
            }
            if constexpr (NBUF == 2) {
                if (more) {
                    pv.load(vtbase + (size_t)(j + 1) * D * kBlock, 0, 0);
                    pk.commit(nxt);
                }
            }
            tile_pv<T, D>(acc, s, cur, col, half);
        } else if constexpr (NBUF == 2) {
            if (more) {
                pv.load(vtbase + (size_t)(j + 1) * D * kBlock, 0, 0);
                pk.commit(nxt);
            }
        }
        if (more) {
            if constexpr (NBUF == 2) {
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

    if (valid) {
        const float inv = 1.0f / l_run;
        T* dst = o + ((size_t)b * N + i) * Hq * D + (size_t)h * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                T* d4 = dst + dt * 32 + 8 * rq + 4 * half;
                if constexpr (sizeof(T) == 2) {
                    const uint32_t a0 = pack_bf16x2(acc[dt][4 * rq] * inv, acc[dt][4 * rq + 1] * inv);
                    const uint32_t a1 = pack_bf16x2(acc[dt][4 * rq + 2] * inv, acc[dt][4 * rq + 3] * inv);
                    *reinterpret_cast<uint2*>(d4) = make_uint2(a0, a1);
                } else {
                    floatx4 y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = acc[dt][4 * rq + e] * inv;
                    *reinterpret_cast<floatx4*>(d4) = y;
                }
            }
        }
        if (half == 0) lse[((size_t)b * Hq + h) * N + i] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    }
}

template <typename T, int D, int G>
void launch_dense_t(const LaunchDims& d, const void* q, const void* k, const void* vt, void* o, float* lse,
                    float scale_log2, hipStream_t st) {
    constexpr int kTiles = kBlock * G / 32;
    const int parts = (kTiles + kDenseWaves - 1) / kDenseWaves;
    constexpr int NBUF = 2 * KVTile<T, D>::BYTES <= 160 * 1024 ? 2 : 1;
    const size_t grid = (size_t)d.nb * d.B * d.Hkv * parts;
    hipLaunchKernelGGL((dense_attn_kernel<T, D, G, NBUF>), dim3((unsigned)grid), dim3(kDenseThreads), 0, st,
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
