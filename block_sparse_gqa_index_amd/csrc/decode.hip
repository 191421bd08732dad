// Decoding: R new queries per sequence against a cache of keys.
//
// Sequence b holds n_b cached tokens (positions 0 .. n_b - 1, the new ones
// last); its r-th new query is position i = n_b - R + r, so selection and
// attention are those of the forward's row i (MiniMax Sparse Attention article on
// 7minutos.es, "Cómo funcionan las dos ramas": index scores of the visible
// keys, block max-pool, top-k per query and group with the local block forced
// in, then exact softmax attention over the kept blocks' causally visible
// tokens; "El codiseño del kernel": the ranking runs on the raw scores). Only
// the block indices need caching per layer (Flash-MSA article on
// tech.kuratif.com, block-wise sparsity).
//
// Per decode step the work is a stream over the index-key cache (every
// competing block of every sequence: Di values per token) plus a gather of the
// kept blocks' K and V (k * 128 tokens per (sequence, group)); both are bound
// by HBM bandwidth, so the kernels aim at full-line, many-in-flight loads and
// use the matrix cores only to keep the VALU off the critical path:
//   decode_scores_kernel  one wave per (sequence, competing block, 32 columns
//                         of (new query, group) pairs; one or two sets of 16
//                         when there are at most 32, bf16 or fp8): S^T = K_idx Q_idx^T on
//                         the matrix cores straight from global memory (no
//                         LDS; the index keys are read once for all R queries),
//                         block max in-lane plus one half-wave swap -> block
//                         scores [B, R * Hkv, nb] fp32; an fp8 e4m3 index cache
//                         halves the bytes streamed
//   decode_topk_kernel    one wave per (sequence, new query, group): a
//                         lane-local sorted list over a strided share of the
//                         block scores, then k-1 wave-wide maxima (DPP within
//                         rows, lane reads across them) of packed (score, -id)
//                         keys; ids sorted ascending, the local block appended
//   decode_attn_kernel    one work-group per (sequence, new query, group, kept
//                         block): S^T = K Q^T per wave (32 keys each; the K
//                         block loaded as whole rows and staged in LDS, in the
//                         rows V takes afterwards), block softmax across the four waves through
//                         LDS, O^T = V^T P^T with V staged in LDS (P as a bf16
//                         hi + lo pair: two products, exact to ~2^-17 of P);
//                         a normalised fp32 partial output and its LSE per head
//   decode_combine_kernel one work-group per (sequence, new query, group): the
//                         kept blocks' partials merged in slot order -> O, LSE.
// Every sum runs in a fixed order: results are bitwise reproducible.
//
// The caches are either contiguous per sequence ([B, C, ...]) or paged: a pool
// of 128-token pages ([P, 128, ...]) and a block table [B, ceil(C/128)] naming
// the page of every block of every sequence (the block ids MSA selects are then
// page-table entries: one lookup per block, no other change).
#include "msa_decode.h"
#include "msa_tiles.h"

namespace msa {

namespace {

constexpr int kGroupCols = 32;   // groups (index scores) or heads (attention) per matrix-core column set

__device__ __forceinline__ bool length_ok(int n, int C) { return n >= 1 && n <= C; }

// ------------------------------------------------------------ block scores --

// Matrix-core step of the index scores per element type: a 32 x 32 S^T tile
// accumulates KD-deep slices; lane l supplies row/column l % 32 and the KD/2
// consecutive contraction elements starting at (KD/2) * (l / 32).
template <typename T> struct DecMma;
template <> struct DecMma<bf16_t> {   // v_mfma_f32_32x32x16_bf16
    using Op = Op8<bf16_t>;
    static constexpr int KD = 16;
    static __device__ __forceinline__ void mma(floatx16& acc, const Op& a, const Op& b) { mma16(acc, a, b); }
};
template <> struct DecMma<float> {    // eight v_mfma_f32_32x32x2_f32 per 16-deep slice
    using Op = Op8<float>;
    static constexpr int KD = 16;
    static __device__ __forceinline__ void mma(floatx16& acc, const Op& a, const Op& b) { mma16(acc, a, b); }
};
template <> struct DecMma<fp8_t> {    // v_mfma_scale_f32_32x32x64_f8f6f4: e4m3 x e4m3, unit scales
    struct Op {
        i32x8 v;
        __device__ __forceinline__ void load(const void* p) {
            const uint4 lo = reinterpret_cast<const uint4*>(p)[0], hi = reinterpret_cast<const uint4*>(p)[1];
            v = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        __device__ __forceinline__ void zero() { v = i32x8{0, 0, 0, 0, 0, 0, 0, 0}; }
    };
    static constexpr int KD = 64;
    static __device__ __forceinline__ void mma(floatx16& acc, const Op& a, const Op& b) {
        // format code 0 (fp8 e4m3) for both operands; scale exponents 127 (= 2^0)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, acc, 0, 0, 0, 127, 0, 127);
    }
};

// COLS columns per wave: 32 (32 x 32 tiles, any element type) or 16 x NCS
// (bf16: v_mfma_f32_16x16x32_bf16 on 16-key tiles, lane l supplying row l % 16
// and the 8 contraction elements at 8 * (l / 16) of each 32-deep slice, so one
// load instruction covers 64 contiguous bytes of each of 16 key rows; each key
// operand feeds the NCS column sets).
template <typename T, int DI, int COLS, int NCS = 1>
__global__ __launch_bounds__(256) void decode_scores_kernel(const T* __restrict__ q_idx,
                                                            const T* __restrict__ k_idx,
                                                            const int32_t* __restrict__ seqlens,
                                                            const int32_t* __restrict__ pages, int num_pages,
                                                            float* __restrict__ scores, int C, int Hkv,
                                                            int R, int nbs, int gchunks) {
    static_assert(COLS == 16 || NCS == 1, "32-column waves take one column set");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane % COLS, half = lane >> 5;
    const int b = blockIdx.y / gchunks, gc = blockIdx.y % gchunks;
    const int j = blockIdx.x * 4 + wave;
    const int n = seqlens[b];
    if (!length_ok(n, C)) return;
    const int L = (n - 1) / kBlock;   // competing blocks of the last new query: 0 .. L-1
    if (j >= L) return;
    // Columns are the (new query r, group g) pairs of the sequence, c = r * Hkv + g;
    // an earlier query reads only the blocks it sees.
    const int RH = R * Hkv;
    const int c = gc * COLS + col;
    const bool writer = lane < COLS;   // one lane per column stores its block score
    // Block j of the sequence: contiguous in the cache, or the page the block table names.
    const T* kb = k_idx + ((size_t)b * C + (size_t)j * kBlock) * DI;
    if (pages) {
        const int pg = pages[(size_t)b * nbs + j];
        if (pg < 0 || pg >= num_pages) {   // not a page of the pool: the block scores -inf, nothing is read
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs)
                if (writer && c + 16 * cs < RH) scores[((size_t)b * RH + c + 16 * cs) * nbs + j] = -__builtin_inff();
            return;
        }
        kb = k_idx + (size_t)pg * kBlock * DI;
    }

    if constexpr (COLS == 16 && sizeof(T) == 1) {
        static_assert(DI == 128, "16-column fp8 tiles take one 128-deep product");
        // v_mfma_scale_f32_16x16x128_f8f6f4: lane l supplies row l % 16 and 32
        // contraction bytes, here the 16-byte chunks grp and grp + 4 of the
        // row (the same for keys and queries), so one load instruction covers
        // 64 contiguous bytes of each of 16 key rows.
        const int grp = lane >> 4;
        auto ld = [&](const T* row) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(row + 16 * grp);
            const u32x4 y = *reinterpret_cast<const u32x4*>(row + 64 + 16 * grp);
            return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        };
        i32x8 bq[NCS];
        float m[NCS];
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
            const int cc = c + 16 * cs;
            bq[cs] = cc < RH ? ld(q_idx + ((size_t)b * RH + cc) * DI) : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            m[cs] = -__builtin_inff();
        }
        i32x8 a[8];   // eight 16-key tiles, all in flight
#pragma unroll
        for (int t = 0; t < 8; ++t) a[t] = ld(kb + (size_t)(t * 16 + col) * DI);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) {
                // format code 0 (fp8 e4m3) for both operands; scale exponents 127 (= 2^0)
                const floatx4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a[t], bq[cs], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                m[cs] = vmax(m[cs], vmax(vmax(acc[0], acc[1]), vmax(acc[2], acc[3])));
            }
        }
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
            float x = vmax(m[cs], __shfl_xor(m[cs], 16));
            x = vmax(x, __shfl_xor(x, 32));
            if (writer && c + 16 * cs < RH) scores[((size_t)b * RH + c + 16 * cs) * nbs + j] = x;
        }
        return;
    } else if constexpr (COLS == 16) {
        static_assert(sizeof(T) == 2, "16-column tiles are bf16 or fp8");
        constexpr int NS = DI / 32;   // 32-deep contraction slices
        const int grp = lane >> 4;    // contraction group of the lane
        Op8<T> bq[NCS][NS];
        float m[NCS];
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
            const int cc = c + 16 * cs;
            const T* qrow = q_idx + ((size_t)b * RH + (cc < RH ? cc : 0)) * DI;   // q_idx [B, R, Hkv, Di]
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                if (cc < RH) bq[cs][sl].load(qrow + 32 * sl + 8 * grp);
                else bq[cs][sl].zero();
            }
            m[cs] = -__builtin_inff();
        }
        // Eight 16-key tiles, four tiles' operands in flight.
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
            Op8<T> a[4][NS];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const T* row = kb + (size_t)((t0 + t) * 16 + col) * DI;
#pragma unroll
                for (int sl = 0; sl < NS; ++sl) a[t][sl].load(row + 32 * sl + 8 * grp);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs) {
                    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int sl = 0; sl < NS; ++sl)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t][sl].v, bq[cs][sl].v, acc, 0, 0, 0);
                    m[cs] = vmax(m[cs], vmax(vmax(acc[0], acc[1]), vmax(acc[2], acc[3])));
                }
            }
        }
        // Lanes l, l + 16, l + 32, l + 48 hold the four row quarters of column l % 16.
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
            float x = vmax(m[cs], __shfl_xor(m[cs], 16));
            x = vmax(x, __shfl_xor(x, 32));
            if (writer && c + 16 * cs < RH) scores[((size_t)b * RH + c + 16 * cs) * nbs + j] = x;
        }
        return;
    }

    using MM = DecMma<T>;
    constexpr int NS = DI / MM::KD;   // contraction slices
    constexpr int KH = MM::KD / 2;    // elements per lane and slice
    typename MM::Op bq[NS];
    const T* qrow = q_idx + ((size_t)b * RH + (c < RH ? c : 0)) * DI;   // q_idx [B, R, Hkv, Di]
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
        if (c < RH) bq[sl].load(qrow + MM::KD * sl + KH * half);
        else bq[sl].zero();
    }

    // Tiles of 32 keys; bf16 and fp8 keep all four tiles' operands in flight, fp32 two.
    constexpr int TF = sizeof(T) == 4 ? 2 : 4;
    float m = -__builtin_inff();
#pragma unroll
    for (int t0 = 0; t0 < 4; t0 += TF) {
        typename MM::Op a[TF][NS];
#pragma unroll
        for (int t = 0; t < TF; ++t) {
            const T* row = kb + (size_t)((t0 + t) * 32 + col) * DI;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) a[t][sl].load(row + MM::KD * sl + KH * half);
        }
#pragma unroll
        for (int t = 0; t < TF; ++t) {
            floatx16 acc = zero16();
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) MM::mma(acc, a[t][sl], bq[sl]);
            m = vmax(m, max16(acc));
        }
    }
    m = vmax(m, swap_halves(m));
    if (writer && c < RH) scores[((size_t)b * RH + c) * nbs + j] = m;
}

// ------------------------------------------------------------------- top-k --

// Orderable 64-bit key: score bits mapped to an unsigned order (larger score
// -> larger key) in the high word, ~id in the low word (lower id -> larger key
// among equal scores). 0 is below every key of a real score.
__device__ __forceinline__ uint64_t rank_key(float s, int id) {
    uint32_t u = __float_as_uint(s + 0.0f);   // -0 -> +0: equal scores compare equal
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)id);
}

// Key of a partner lane by DPP: CTRL 0xB1 / 0x4E are the quad permutes
// [1,0,3,2] / [2,3,0,1], 0x141 / 0x140 the 8- and 16-lane mirrors.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Largest key of the wave (the same value in every lane): in-row maxima by
// DPP (each 16-lane row ends uniform), then the four rows' values read out.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = max_u64(x, dpp_u64<0xB1>(x));
    x = max_u64(x, dpp_u64<0x4E>(x));
    x = max_u64(x, dpp_u64<0x141>(x));
    x = max_u64(x, dpp_u64<0x140>(x));
    return max_u64(max_u64(readlane_u64(x, 0), readlane_u64(x, 16)), max_u64(readlane_u64(x, 32), readlane_u64(x, 48)));
}

template <int K1MAX>
__global__ __launch_bounds__(256) void decode_topk_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ seqlens,
                                                          int32_t* __restrict__ block_idx, int B, int C, int Hkv,
                                                          int R, int nbs, int k) {
    const int lane = threadIdx.x & 63;
    const int rr = blockIdx.x * 4 + (threadIdx.x >> 6);   // (sequence, new query, group) row of this wave
    const int RH = R * Hkv;
    if (rr >= B * RH) return;
    const int b = rr / RH, qr = (rr % RH) / Hkv, g = rr % Hkv;
    const int n = seqlens[b];
    const int i = n - R + qr;   // the query's position
    int32_t* out = block_idx + (((size_t)b * Hkv + g) * R + qr) * k;   // [B, Hkv, R, k]
    if (!length_ok(n, C) || i < 0) {
        if (lane < k) out[lane] = -1;
        return;
    }
    const int L = i / kBlock;
    const int k1 = min(k - 1, L);
    const float* row = scores + (size_t)rr * nbs;

    // Lane-local best K1MAX keys, descending (0 = empty).
    uint64_t best[K1MAX];
#pragma unroll
    for (int e = 0; e < K1MAX; ++e) best[e] = 0;
    // Chunks of 16 scores per lane, all requested before the first insert.
    constexpr int kPer = 16;
    for (int j0 = 0; j0 < L; j0 += kPer * kWave) {
        float v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int j = j0 + u * kWave + lane;
            v[u] = j < L ? row[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int j = j0 + u * kWave + lane;
            uint64_t key = j < L ? rank_key(v[u], j) : 0;
            if (key > best[K1MAX - 1]) {
#pragma unroll
                for (int e = 0; e < K1MAX; ++e) {
                    const uint64_t hi = key > best[e] ? key : best[e];
                    key = key > best[e] ? best[e] : key;
                    best[e] = hi;
                }
            }
        }
    }
    // k1 rounds: the wave-wide largest head is taken and its lane pops it.
    int mine = 0;   // lane q keeps the id chosen in round q
    for (int q = 0; q < k1; ++q) {
        const uint64_t mx = wave_max_u64(best[0]);
        if (best[0] == mx) {
#pragma unroll
            for (int e = 0; e + 1 < K1MAX; ++e) best[e] = best[e + 1];
            best[K1MAX - 1] = 0;
        }
        if (lane == q) mine = (int)(~(uint32_t)mx);
    }
    // Ascending order: lane q's rank among the k1 chosen ids.
    int rank = 0;
    for (int q = 0; q < k1; ++q) rank += __builtin_amdgcn_readlane(mine, q) < mine ? 1 : 0;
    if (lane < k1) out[rank] = mine;
    else if (lane == k1) out[k1] = L;
    else if (lane < k) out[lane] = -1;
}

// --------------------------------------------------------------- attention --

template <typename T, int D>
struct DecodeLds {
    static constexpr int ES = sizeof(T);
    static constexpr int VROW = D * ES + 16;            // padded V row: the two half-waves hit other banks
    static constexpr int V_BYTES = kBlock * VROW;
    // [wave][slice][lane] P operands; bf16 keeps P = hi + lo as two operands
    // (hi = bf16(p), lo = bf16(p - hi)), so P V is exact to ~2^-17 of p.
    static constexpr int P_HALF = 4 * 2 * kWave * 8 * ES;
    static constexpr int P_BYTES = (ES == 2 ? 2 : 1) * P_HALF;
    static constexpr int RED_BYTES = 2 * 4 * kGroupCols * 4;
    static constexpr int BYTES = V_BYTES + P_BYTES + RED_BYTES;
};

template <typename T>
__device__ __forceinline__ T lds_elem(const unsigned char* p) { return *reinterpret_cast<const T*>(p); }

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_attn_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                                                          const T* __restrict__ vc,
                                                          const int32_t* __restrict__ seqlens,
                                                          const int32_t* __restrict__ block_idx,
                                                          const int32_t* __restrict__ pages, int num_pages,
                                                          float* __restrict__ po, float* __restrict__ plse, int C,
                                                          int Hkv, int G, int R, int k, float scale_log2) {
    using LD = DecodeLds<T, D>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LD::BYTES];
    unsigned char* vs = lds;
    unsigned char* pl = lds + LD::V_BYTES;
    float* red_m = reinterpret_cast<float*>(lds + LD::V_BYTES + LD::P_BYTES);
    float* red_l = red_m + 4 * kGroupCols;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z / R, qr = blockIdx.z % R;
    const size_t item = ((size_t)blockIdx.z * Hkv + g) * k + slot;   // (sequence, new query, group, slot)
    const int n = seqlens[b];
    const int i = n - R + qr;   // the query's position
    const int j = i >= 0 ? block_idx[(((size_t)b * Hkv + g) * R + qr) * k + slot] : -1;
    // Empty slot (padding, a block past the query, or an invalid length): no
    // tokens, LSE -inf, and the merge skips the slot.
    const int nbs = (C + kBlock - 1) / kBlock;
    const int pg = (pages && j >= 0 && j < nbs) ? pages[(size_t)b * nbs + j] : 0;
    if (!length_ok(n, C) || j < 0 || (int64_t)j * kBlock > i || (pages && (pg < 0 || pg >= num_pages))) {
        if (threadIdx.x < G) plse[item * G + threadIdx.x] = -__builtin_inff();
        return;
    }
    const int t0 = j * kBlock;
    const int t_last = min(t0 + kBlock - 1, i);
    const size_t kv_row = (size_t)Hkv * D;   // elements between consecutive tokens of one head
    // First token of the block (contiguous cache, or the named page); token
    // t0 + r is r rows further.
    const size_t first = pages ? (size_t)pg * kBlock : (size_t)b * C + t0;
    const T* kbase = kc + (first * Hkv + g) * D;
    const T* vbase = vc + (first * Hkv + g) * D;

    // Requests in flight together: the query operands, then the K and V blocks
    // as whole rows (each load instruction covers 4 rows of the block; rows past
    // the last visible token zero-filled). K goes to LDS first and is read back
    // as this wave's operands; V then takes the same LDS rows.
    Op8<T> bq[D / 16];
    const int Hq = Hkv * G;
    load_q_op<T, D>(bq, q + ((size_t)blockIdx.z * Hq + (size_t)g * G + (col < G ? col : 0)) * D, col < G, half);
    constexpr int EPC = 16 / LD::ES;
    constexpr int CPR = D / EPC;
    constexpr int VPER = kBlock * CPR / 256;
    static_assert(kBlock * CPR % 256 == 0, "K/V chunk split");
    u32x4 kr[VPER], vr[VPER];
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
        const int ch = threadIdx.x + u * 256, row = ch / CPR, cc = ch % CPR;
        kr[u] = t0 + row <= t_last ? *reinterpret_cast<const u32x4*>(kbase + (size_t)row * kv_row + cc * EPC)
                                   : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
        const int ch = threadIdx.x + u * 256, row = ch / CPR, cc = ch % CPR;
        vr[u] = t0 + row <= t_last ? *reinterpret_cast<const u32x4*>(vbase + (size_t)row * kv_row + cc * EPC)
                                   : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
        const int ch = threadIdx.x + u * 256, row = ch / CPR, cc = ch % CPR;
        *reinterpret_cast<u32x4*>(vs + row * LD::VROW + cc * 16) = kr[u];
    }
    __syncthreads();
    floatx16 s = zero16();
    {
        const unsigned char* krow = vs + (wave * 32 + col) * LD::VROW;
#pragma unroll
        for (int sl = 0; sl < D / 16; ++sl) {
            Op8<T> a;
            a.load(krow + (16 * sl + 8 * half) * LD::ES);
            mma16(s, a, bq[sl]);
        }
    }
    __syncthreads();   // every wave has read its key operands: V takes the rows
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
        const int ch = threadIdx.x + u * 256, row = ch / CPR, cc = ch % CPR;
        *reinterpret_cast<u32x4*>(vs + row * LD::VROW + cc * 16) = vr[u];
    }
    // Lane holds head `col`, keys t0 + 32*wave + 8*(r/4) + 4*half + r%4.
    float m = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int t = t0 + wave * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        s[r] = t <= t_last ? s[r] * scale_log2 : -__builtin_inff();
        m = vmax(m, s[r]);
    }
    m = vmax(m, swap_halves(m));
    if (half == 0) red_m[wave * kGroupCols + col] = m;
    __syncthreads();
    const float M = max3f(red_m[col], red_m[kGroupCols + col],
                          vmax(red_m[2 * kGroupCols + col], red_m[3 * kGroupCols + col]));
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        s[r] = exp2_hw(s[r] - M);
        l += s[r];
    }
    l += swap_halves(l);
    if (half == 0) red_l[wave * kGroupCols + col] = l;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = s[8 * s2 + e];
        Op8<T> bp;
        PType<T>::pack(bp, pe);
        *reinterpret_cast<Op8<T>*>(pl + ((wave * 2 + s2) * kWave + lane) * 8 * LD::ES) = bp;
        if constexpr (LD::ES == 2) {
            const u32x4 hw = __builtin_bit_cast(u32x4, bp.v);
            float lo[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[2 * e] = pe[2 * e] - __uint_as_float(hw[e] << 16);
                lo[2 * e + 1] = pe[2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u);
            }
            Op8<T> bl;
            PType<T>::pack(bl, lo);
            *reinterpret_cast<Op8<T>*>(pl + LD::P_HALF + ((wave * 2 + s2) * kWave + lane) * 8 * LD::ES) = bl;
        }
    }
    __syncthreads();
    const float lsum = red_l[col] + red_l[kGroupCols + col] + red_l[2 * kGroupCols + col] + red_l[3 * kGroupCols + col];

    // O^T (32 dims of tile `wave`) = V^T P^T over the 128 keys: slice (w2, s2)
    // pairs element e of both operands with key
    // 32*w2 + 16*s2 + 8*(e/4) + 4*half + e%4.
    if (wave < D / 32) {
        const int d = wave * 32 + col;
        floatx16 o = zero16();
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const Op8<T> bp = *reinterpret_cast<const Op8<T>*>(pl + ((w2 * 2 + s2) * kWave + lane) * 8 * LD::ES);
                Op8<T> a;
                if constexpr (LD::ES == 2) {
                    uint16_t u[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int kk = 32 * w2 + 16 * s2 + 8 * (e >> 2) + 4 * half + (e & 3);
                        u[e] = lds_elem<uint16_t>(vs + kk * LD::VROW + d * 2);
                    }
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)u[2 * e] | ((uint32_t)u[2 * e + 1] << 16);
                    a.v = __builtin_bit_cast(bf16x8, w);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int kk = 32 * w2 + 16 * s2 + 8 * (e >> 2) + 4 * half + (e & 3);
                        a.v[e] = lds_elem<float>(vs + kk * LD::VROW + d * 4);
                    }
                }
                mma16(o, a, bp);
                if constexpr (LD::ES == 2) {
                    const Op8<T> bl =
                        *reinterpret_cast<const Op8<T>*>(pl + LD::P_HALF + ((w2 * 2 + s2) * kWave + lane) * 8 * LD::ES);
                    mma16(o, a, bl);
                }
            }
        }
        // Lane holds head `col`, dims wave*32 + 8*(r/4) + 4*half + r%4.
        if (col < G) {
            const float inv = 1.0f / lsum;
            float* dst = po + (item * G + col) * D + wave * 32 + 4 * half;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 x = make_float4(o[4 * q4] * inv, o[4 * q4 + 1] * inv, o[4 * q4 + 2] * inv,
                                             o[4 * q4 + 3] * inv);
                *reinterpret_cast<float4*>(dst + 8 * q4) = x;
            }
        }
    }
    if (wave == 0 && half == 0 && col < G) plse[item * G + col] = (M + log2f(lsum)) * 0.69314718055994531f;
}

// ------------------------------------------------------------------- merge --

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t* p, float x) { *p = f32_to_bf16(x); }
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }

template <typename T>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ po,
                                                             const float* __restrict__ plse, T* __restrict__ o,
                                                             float* __restrict__ lse, int Hkv, int G, int D,
                                                             int R, int k) {
    __shared__ float sl[32 * 32];    // slot LSEs [slot][head], then merge weights
    __shared__ float tot[32];        // merged LSE per head
    const int g = blockIdx.x, z = blockIdx.y;   // z = (sequence, new query)
    const size_t item0 = ((size_t)z * Hkv + g) * k;
    const int Hq = Hkv * G;
    // The row's k * G slot LSEs are contiguous: one load per thread.
    for (int t = threadIdx.x; t < k * G; t += blockDim.x) sl[t] = plse[item0 * G + t];
    __syncthreads();
    if ((int)threadIdx.x < G) {
        const int h = threadIdx.x;
        float mx = -__builtin_inff();
        for (int s = 0; s < k; ++s) mx = fmaxf(mx, sl[s * G + h]);
        float total = -__builtin_inff();
        if (mx > -__builtin_inff()) {
            float sum = 0.f;
            for (int s = 0; s < k; ++s) {
                const float x = sl[s * G + h];
                if (x > -__builtin_inff()) sum += __expf(x - mx);
            }
            total = mx + __logf(sum);
        }
        tot[h] = total;
        lse[((size_t)(z / R) * Hq + (size_t)g * G + h) * R + z % R] = total;   // [B, Hq, R]
    }
    __syncthreads();
    for (int t = threadIdx.x; t < k * G; t += blockDim.x) {
        const float x = sl[t];
        sl[t] = x > -__builtin_inff() ? __expf(x - tot[t % G]) : 0.f;
    }
    __syncthreads();
    // Each thread: 4 consecutive dims of one head; the slots' partials are
    // requested four slots at a time, summed in slot order.
    for (int e = threadIdx.x * 4; e < G * D; e += blockDim.x * 4) {
        const int h = e / D, d = e % D;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < k; s0 += 4) {
            float4 x[4];
            float wv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = s0 + u;
                wv[u] = s < k ? sl[s * G + h] : 0.f;
                x[u] = wv[u] != 0.f ? *reinterpret_cast<const float4*>(po + ((item0 + s) * G + h) * D + d)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc.x = fmaf(wv[u], x[u].x, acc.x);
                acc.y = fmaf(wv[u], x[u].y, acc.y);
                acc.z = fmaf(wv[u], x[u].z, acc.z);
                acc.w = fmaf(wv[u], x[u].w, acc.w);
            }
        }
        T* dst = o + ((size_t)z * Hq + (size_t)g * G + h) * D + d;   // [B, R, Hq, D]
        store_out<T>(dst, acc.x);
        store_out<T>(dst + 1, acc.y);
        store_out<T>(dst + 2, acc.z);
        store_out<T>(dst + 3, acc.w);
    }
}

template <int K1MAX>
void launch_topk(const float* scores, const int32_t* seqlens, int32_t* block_idx, int B, int C, int Hkv, int R,
                 int nbs, int k, hipStream_t st) {
    const int rows = B * R * Hkv;
    hipLaunchKernelGGL(decode_topk_kernel<K1MAX>, dim3((rows + 3) / 4), dim3(256), 0, st, scores, seqlens,
                       block_idx, B, C, Hkv, R, nbs, k);
}

template <typename T, int DI>
void launch_scores(const DecodeDims& d, const void* q_idx, const void* k_idx, const int32_t* seqlens,
                   const int32_t* pages, int num_pages, float* scores, hipStream_t st) {
    const int lmax = (d.C - 1) / kBlock;   // competing blocks of a full cache
    if (lmax == 0) return;
    const int RH = d.R * d.Hkv;
    // bf16 (or fp8 with Di = 128) with at most 32 columns: one wave takes one
    // or two 16-column sets, each key block read once per sequence. More
    // columns take 32-column sets, one wave each.
    if constexpr (sizeof(T) == 2 || (sizeof(T) == 1 && DI == 128)) {
        if (RH <= 16) {
            hipLaunchKernelGGL((decode_scores_kernel<T, DI, 16, 1>), dim3((lmax + 3) / 4, d.B), dim3(256), 0, st,
                               static_cast<const T*>(q_idx), static_cast<const T*>(k_idx), seqlens, pages, num_pages,
                               scores, d.C, d.Hkv, d.R, d.nbs(), 1);
            return;
        }
        if (RH <= 32) {
            hipLaunchKernelGGL((decode_scores_kernel<T, DI, 16, 2>), dim3((lmax + 3) / 4, d.B), dim3(256), 0, st,
                               static_cast<const T*>(q_idx), static_cast<const T*>(k_idx), seqlens, pages, num_pages,
                               scores, d.C, d.Hkv, d.R, d.nbs(), 1);
            return;
        }
    }
    const int g32 = (RH + kGroupCols - 1) / kGroupCols;
    hipLaunchKernelGGL((decode_scores_kernel<T, DI, 32>), dim3((lmax + 3) / 4, d.B * g32), dim3(256), 0, st,
                       static_cast<const T*>(q_idx), static_cast<const T*>(k_idx), seqlens, pages, num_pages, scores,
                       d.C, d.Hkv, d.R, d.nbs(), g32);
}

template <typename T, int D>
void launch_attn(const DecodeDims& d, const void* q, const void* k, const void* v, const int32_t* seqlens,
                 const int32_t* block_idx, const int32_t* pages, int num_pages, float scale, void* o, float* lse,
                 const DecodeWorkspace& W, unsigned char* ws, hipStream_t st) {
    float* po = reinterpret_cast<float*>(ws + W.po);
    float* pl = reinterpret_cast<float*>(ws + W.plse);
    hipLaunchKernelGGL((decode_attn_kernel<T, D>), dim3(d.k, d.Hkv, d.B * d.R), dim3(256), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), seqlens,
                       block_idx, pages, num_pages, po, pl, d.C, d.Hkv, d.G, d.R, d.k, scale * 1.4426950408889634f);
    hipLaunchKernelGGL((decode_combine_kernel<T>), dim3(d.Hkv, d.B * d.R), dim3(256), 0, st, po, pl,
                       static_cast<T*>(o), lse, d.Hkv, d.G, D, d.R, d.k);
}

}  // namespace

DecodeWorkspace decode_workspace_layout(const DecodeDims& d) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    DecodeWorkspace W;
    W.scores = 0;
    W.index_bytes = up((size_t)d.B * d.R * d.Hkv * d.nbs() * sizeof(float));
    W.po = 0;
    W.plse = up((size_t)d.B * d.R * d.Hkv * d.k * d.G * d.D * sizeof(float));
    W.attn_bytes = W.plse + up((size_t)d.B * d.R * d.Hkv * d.k * d.G * sizeof(float));
    return W;
}

hipError_t launch_decode_index(const DecodeDims& d, const void* q_idx, const void* k_idx, const int32_t* seqlens,
                               const int32_t* pages, int num_pages, int32_t* block_idx, void* ws, hipStream_t st) {
    float* scores = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + decode_workspace_layout(d).scores);
    if (d.dtype == 0) {
        if (d.Di == 128) launch_scores<bf16_t, 128>(d, q_idx, k_idx, seqlens, pages, num_pages, scores, st);
        else launch_scores<bf16_t, 64>(d, q_idx, k_idx, seqlens, pages, num_pages, scores, st);
    } else if (d.dtype == 2) {
        if (d.Di == 128) launch_scores<fp8_t, 128>(d, q_idx, k_idx, seqlens, pages, num_pages, scores, st);
        else launch_scores<fp8_t, 64>(d, q_idx, k_idx, seqlens, pages, num_pages, scores, st);
    } else {
        if (d.Di == 128) launch_scores<float, 128>(d, q_idx, k_idx, seqlens, pages, num_pages, scores, st);
        else launch_scores<float, 64>(d, q_idx, k_idx, seqlens, pages, num_pages, scores, st);
    }
    const int k1 = d.k - 1;
    if (k1 <= 3) launch_topk<3>(scores, seqlens, block_idx, d.B, d.C, d.Hkv, d.R, d.nbs(), d.k, st);
    else if (k1 <= 7) launch_topk<7>(scores, seqlens, block_idx, d.B, d.C, d.Hkv, d.R, d.nbs(), d.k, st);
    else if (k1 <= 15) launch_topk<15>(scores, seqlens, block_idx, d.B, d.C, d.Hkv, d.R, d.nbs(), d.k, st);
    else launch_topk<31>(scores, seqlens, block_idx, d.B, d.C, d.Hkv, d.R, d.nbs(), d.k, st);
    return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeDims& d, const void* q, const void* k, const void* v,
                              const int32_t* seqlens, const int32_t* block_idx, const int32_t* pages, int num_pages,
                              float scale, void* o, float* lse, void* ws, hipStream_t st) {
    const DecodeWorkspace W = decode_workspace_layout(d);
    unsigned char* base = static_cast<unsigned char*>(ws);
    if (d.dtype == 0) {
        if (d.D == 128) launch_attn<bf16_t, 128>(d, q, k, v, seqlens, block_idx, pages, num_pages, scale, o, lse, W, base, st);
        else launch_attn<bf16_t, 64>(d, q, k, v, seqlens, block_idx, pages, num_pages, scale, o, lse, W, base, st);
    } else {
        if (d.D == 128) launch_attn<float, 128>(d, q, k, v, seqlens, block_idx, pages, num_pages, scale, o, lse, W, base, st);
        else launch_attn<float, 64>(d, q, k, v, seqlens, block_idx, pages, num_pages, scale, o, lse, W, base, st);
    }
    return hipGetLastError();
}

}  // namespace msa
