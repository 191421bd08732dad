// Index branch of MSA: causal index scores -> block max-pool -> forced-local,
// exp-free top-k, fused in one kernel (gfx950).
//
// Method: MiniMax Sparse Attention (MSA) article on 7minutos.es, section "Cómo
// funcionan las dos ramas" (one index-query head per group against one shared
// index-key head, block max-pooling, top-k per query and group with the local
// block always kept) and section "El codiseño del kernel" (softmax keeps the
// order, so the ranking runs on raw scores: no max/exp/sum before selection).
// The Flash-MSA article (tech.kuratif.com) describes the proxy pass as a
// stream over keys that keeps running top-k candidates and accumulates no
// output; these kernels do the same with a CDNA4 layout:
//
//  * A work-group owns 32*NT*WAVES (query, group) rows of one query block
//    (64 rows per wave, two waves per SIMD for bf16). Rows of a query block
//    share one candidate range (blocks j < L), so no causal mask is needed
//    anywhere: the local block is forced in and never scored.
//  * The rows' index queries stay in VGPRs as the B operand of
//    v_mfma_f32_32x32x16_bf16 for the whole kernel; each key block of k_idx
//    (128 keys x Di) is staged once per work-group in LDS (16-byte padded
//    rows) and read as the A operand, so the product is S^T: every lane's 16
//    accumulators belong to ONE query row. The 128-key block max is then
//    4 x 16 in-lane maxima plus one half-wave exchange (v_permlane32_swap).
//  * Each lane keeps the running top-(k-1) of its rows in registers, sorted by
//    score; blocks arrive in ascending id order, so "strictly greater" is the
//    whole tie-break (an equal score never displaces a lower id).
//  * Work-groups are numbered heaviest query block first (longest-processing-
//    time order over the triangular load).
//
// index_topk_pipe_kernel (bf16, fp8, fp4 when 512 rows tile a query block) is
// the software-pipelined form with one 8-wave work-group per CU (bf16: four LDS
// stages filled by direct global -> LDS copies; fp8/fp4: three stages staged
// through registers); index_topk_kernel (2- or 4-wave work-groups, two LDS
// stages) serves the other shapes and fp32.
#include "msa_common.h"
#include <type_traits>
#include "msa_internal.h"

namespace msa {

// Matrix-core contraction step of the index scores per element type: one
// 32 x 32 S^T tile accumulates KD-deep slices; an operand holds the KD/2
// consecutive contraction elements of one row (A) or column (B) that a lane
// supplies (lane l: row/column l % 32, elements (KD/2)*(l/32) .. + KD/2 - 1).
template <typename T> struct IdxMma;
template <> struct IdxMma<bf16_t> {   // v_mfma_f32_32x32x16_bf16
    using Op = Op8<bf16_t>;
    static constexpr int KD = 16;
    static __device__ __forceinline__ void mma(floatx16& acc, const Op& a, const Op& b) { mma16(acc, a, b); }
};
template <> struct IdxMma<float> {    // 8 x v_mfma_f32_32x32x2_f32 over the same 16-deep slice
    using Op = Op8<float>;
    static constexpr int KD = 16;
    static __device__ __forceinline__ void mma(floatx16& acc, const Op& a, const Op& b) { mma16(acc, a, b); }
};
template <> struct IdxMma<fp8_t> {    // v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3, unit scales
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
        // format codes 0 (fp8 e4m3) for both operands; scale exponents 127 = 2^0
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, acc, 0, 0, 0, 127, 0, 127);
    }
};

template <> struct IdxMma<fp4x2_t> {  // v_mfma_scale_f32_32x32x64_f8f6f4, e2m1 x e2m1, unit scales
    struct Op {
        i32x8 v;   // 32 values = 16 bytes; the fp4 form of the instruction reads the first four registers
        __device__ __forceinline__ void load(const void* p) {
            const uint4 x = *reinterpret_cast<const uint4*>(p);
            v = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        }
        __device__ __forceinline__ void zero() { v = i32x8{0, 0, 0, 0, 0, 0, 0, 0}; }
    };
    static constexpr int KD = 64;
    static __device__ __forceinline__ void mma(floatx16& acc, const Op& a, const Op& b) {
        // format codes 4 (fp4 e2m1) for both operands; scale exponents 127 = 2^0
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, acc, 4, 4, 0, 127, 0, 127);
    }
};

// Bits per element of an index input, and the byte offset of element e of a row.
template <typename T> struct IdxBits { static constexpr int v = 8 * (int)sizeof(T); };
template <> struct IdxBits<fp4x2_t> { static constexpr int v = 4; };
template <typename T> __device__ __host__ constexpr int elem_bytes(int e) { return e * IdxBits<T>::v / 8; }

// Inserts (x, j) into the descending list; a no-op when x does not beat the
// last entry, so it runs without a branch and can be scheduled under the
// matrix-core work of the next key block. Every slot is computed from the old
// list and x alone (no chain through the slots): slot s takes the entry above
// it when x beats that entry, x when x beats only its own entry, else keeps
// its entry; the score is then the median of (entry above, x, own entry),
// which is the same value in all three cases. "Beats" is strictly greater, so
// an equal score never displaces a lower id.
template <int SLOTS>
__device__ __forceinline__ void topk_insert(float (&sc)[SLOTS], int (&id)[SLOTS], float x, int j) {
    bool gt[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) gt[s] = x > sc[s];
#pragma unroll
    for (int s = SLOTS - 1; s > 0; --s) {   // bottom up: slot s still reads the old slot s - 1
        id[s] = gt[s - 1] ? id[s - 1] : (gt[s] ? j : id[s]);
        sc[s] = __builtin_amdgcn_fmed3f(sc[s - 1], x, sc[s]);
    }
    id[0] = gt[0] ? j : id[0];
    sc[0] = gt[0] ? x : sc[0];
}

template <int SLOTS>
__device__ __forceinline__ void sort_ascending(int (&v)[SLOTS]) {
#pragma unroll
    for (int p = 0; p < SLOTS; ++p) {
#pragma unroll
        for (int i = (p & 1); i + 1 < SLOTS; i += 2) {
            const int a = v[i], b = v[i + 1];
            v[i] = min(a, b);
            v[i + 1] = max(a, b);
        }
    }
}

// Rows, candidate blocks and staging shared by both index kernels for a block
// size BK of 64, 128 or 256 keys. The kernels always scan 128-key blocks (one
// LDS stage); a 256-key block's score is the larger of its two halves', and a
// 128-key block holds two 64-key blocks (the max over its key tiles 0-1 and
// 2-3). For BK = 64 the query block's own 128-key block is scanned too: its
// first half competes for the rows in the second half of the query block.
template <int BK>
struct BlockPlan {
    static_assert(BK == 64 || BK == 128 || BK == 256, "block size");
    // 128-key blocks scanned for query block qb (whole pairs for BK = 256)
    static __device__ __forceinline__ int scanned(int qb) { return BK == 128 ? qb : BK == 256 ? (qb & ~1) : qb + 1; }
    // competing BK-blocks of the row at position p of query block qb (= its local block id)
    static __device__ __forceinline__ int local(int qb, int p) {
        return BK == 128 ? qb : BK == 256 ? qb / 2 : 2 * qb + (p >= 64 ? 1 : 0);
    }
};

template <typename T, int DI, int NT, int WAVES, int SLOTS, int BPB, int BK>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void index_topk_kernel(
    const T* __restrict__ q_idx, const T* __restrict__ k_idx, int32_t* __restrict__ block_idx,
    int B, int N, int Hkv, int k, int qb_lo, int qb_cnt, int chunks) {
    constexpr int NTHR = 64 * WAVES;
    constexpr int RB = elem_bytes<T>(DI);     // bytes of one index row
    constexpr int ROWB = RB + 16;             // padded LDS row, bytes
    using MM = IdxMma<T>;
    constexpr int KD = MM::KD;
    constexpr int KS = DI / KD;               // KD-deep slices of the contraction
    constexpr int CPR = RB / 16;              // 16-byte chunks per key row
    constexpr int CPT = kBlock * CPR / NTHR;  // chunks per thread per key block
    constexpr int NO = NT >= 2 ? NT / 2 : 1;  // rows each lane keeps a top-k list for
    static_assert(CPT * NTHR == kBlock * CPR, "staging must tile the block");
    // Two stages of BPB key blocks: one barrier per BPB blocks.
    __shared__ __align__(16) unsigned char lds[2][BPB][kBlock * ROWB];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int per_qb = B * chunks;
    const int qb = qb_lo + qb_cnt - 1 - (int)(blockIdx.x / per_qb);   // heaviest first
    const int b = (int)(blockIdx.x % per_qb) / chunks;
    const int c = (int)(blockIdx.x % chunks);
    const int r0 = c * (32 * NT * WAVES) + w * (32 * NT);
    const size_t qrow0 = ((size_t)b * N + (size_t)qb * kBlock) * Hkv;

    // Index queries of this wave's rows: B operand, resident for the whole kernel.
    typename MM::Op bq[NT][KS];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int R = r0 + 32 * t + col;
        const bool valid = qb * kBlock + R / Hkv < N;
        const unsigned char* src =
            reinterpret_cast<const unsigned char*>(q_idx) + (qrow0 + R) * RB + elem_bytes<T>((KD / 2) * half);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (valid) bq[t][s].load(src + elem_bytes<T>(KD * s));
            else bq[t][s].zero();
        }
    }

    float sc[NO][SLOTS];
    int id[NO][SLOTS];
    const int nslots = k - 1;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const bool dummy = s < SLOTS - nslots;   // unused slots sit above every score
            sc[o][s] = dummy ? __builtin_inff() : -__builtin_inff();
            id[o][s] = dummy ? -2 : -1;
        }
    }

    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(k_idx) + (size_t)b * N * RB;
    const int nj = BlockPlan<BK>::scanned(qb);
    int lrow[NO];   // per owned row: its competing blocks (= its local block id)
#pragma unroll
    for (int o = 0; o < NO; ++o) lrow[o] = BlockPlan<BK>::local(qb, (r0 + 32 * (NT >= 2 ? 2 * o + half : 0) + col) / Hkv);
    // 16-byte chunk ch of scanned block j (the query's own block, scanned for
    // BK = 64, may end past N: its rows there repeat row N - 1, never used)
    auto chunk_src = [&](int j, int ch) {
        const int key = BK == 64 ? min(j * kBlock + ch / CPR, N - 1) : j * kBlock + ch / CPR;
        return reinterpret_cast<const u32x4*>(kbase + (size_t)key * RB + (ch % CPR) * 16);
    };
    if (nj > 0) {   // a row of query block 0 has no candidate block at BK >= 128
        u32x4 stage[BPB][CPT];
#pragma unroll
        for (int bb = 0; bb < BPB; ++bb) {
#pragma unroll
            for (int u = 0; u < CPT; ++u) stage[bb][u] = *chunk_src(min(bb, nj - 1), tid + NTHR * u);
        }
        {
#pragma unroll
            for (int bb = 0; bb < BPB; ++bb) {
#pragma unroll
                for (int u = 0; u < CPT; ++u) {
                    const int ch = tid + NTHR * u;
                    *reinterpret_cast<u32x4*>(&lds[0][bb][(ch / CPR) * ROWB + (ch % CPR) * 16]) = stage[bb][u];
                }
            }
        }
    }
    __syncthreads();

    // Block j's candidate (per owned row) is inserted while block j+1 is on the
    // matrix cores; each key tile's max overlaps the next tile's MFMAs.
    float x_prev[NO], stash[NO];   // pending candidate; BK = 256: the first half's max
    int id_prev = -1;
#pragma unroll
    for (int o = 0; o < NO; ++o) x_prev[o] = stash[o] = -__builtin_inff();
    for (int jp = 0; jp < nj; jp += BPB) {
        const int cur = (jp / BPB) & 1;
        // Next BPB key blocks: global -> VGPRs now, VGPRs -> LDS after this stage's math.
        u32x4 stage[BPB][CPT];
#pragma unroll
        for (int bb = 0; bb < BPB; ++bb) {
#pragma unroll
            for (int u = 0; u < CPT; ++u) stage[bb][u] = *chunk_src(min(jp + BPB + bb, nj - 1), tid + NTHR * u);
        }
#pragma unroll
        for (int bb = 0; bb < BPB; ++bb) {
            const int j = jp + bb;
            if (j < nj) {
                float bm[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) bm[t] = -__builtin_inff();
                floatx16 acc[2][NT];
#pragma unroll
                for (int kt = 0; kt < kBlock / 32; ++kt) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) acc[kt & 1][t] = zero16();
                    const unsigned char* arow = &lds[cur][bb][(kt * 32 + col) * ROWB + elem_bytes<T>((KD / 2) * half)];
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        typename MM::Op a;
                        a.load(arow + elem_bytes<T>(KD * s));
#pragma unroll
                        for (int t = 0; t < NT; ++t) MM::mma(acc[kt & 1][t], a, bq[t][s]);
                    }
                    if (kt == 0) {
                        if (j > 0) {
#pragma unroll
                            for (int o = 0; o < NO; ++o) topk_insert<SLOTS>(sc[o], id[o], x_prev[o], id_prev);
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < NT; ++t) bm[t] = fmaxf(bm[t], max16(acc[(kt - 1) & 1][t]));
                        if (BK == 64 && kt == 2) {
                            // key tiles 0-1 done: the first 64-key block of j (for the
                            // query's own block only the rows of the second half see it)
#pragma unroll
                            for (int t = 0; t < NT; ++t) bm[t] = fmaxf(bm[t], swap_halves(bm[t]));
#pragma unroll
                            for (int o = 0; o < NO; ++o) {
                                const float x = NT >= 2 ? (half ? bm[2 * o + 1] : bm[2 * o]) : bm[0];
                                topk_insert<SLOTS>(sc[o], id[o], 2 * j < lrow[o] ? x : -__builtin_inff(), 2 * j);
                            }
#pragma unroll
                            for (int t = 0; t < NT; ++t) bm[t] = -__builtin_inff();
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    bm[t] = fmaxf(bm[t], max16(acc[(kBlock / 32 - 1) & 1][t]));
                    bm[t] = fmaxf(bm[t], swap_halves(bm[t]));
                }
#pragma unroll
                for (int o = 0; o < NO; ++o) {
                    const float x = NT >= 2 ? (half ? bm[2 * o + 1] : bm[2 * o]) : bm[0];
                    if (BK == 128) {
                        x_prev[o] = x;
                    } else if (BK == 64) {   // the second 64-key block of j (never a candidate in the query's block)
                        x_prev[o] = 2 * j + 1 < lrow[o] ? x : -__builtin_inff();
                    } else if (j & 1) {      // BK = 256: both halves seen
                        x_prev[o] = fmaxf(stash[o], x);
                    } else {
                        stash[o] = x;
                        x_prev[o] = -__builtin_inff();
                    }
                }
                id_prev = BK == 128 ? j : BK == 64 ? 2 * j + 1 : j / 2;
            }
        }
        // Unconditional (the last iteration writes a copy of the last block that
        // nobody reads): a store under a branch lets the compiler sink the
        // global loads above into that branch, after the math, where their
        // latency is no longer hidden. The buffer written was last read before
        // the previous barrier.
#pragma unroll
        for (int bb = 0; bb < BPB; ++bb) {
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int ch = tid + NTHR * u;
                *reinterpret_cast<u32x4*>(&lds[cur ^ 1][bb][(ch / CPR) * ROWB + (ch % CPR) * 16]) = stage[bb][u];
            }
        }
        __syncthreads();
    }
    if (nj > 0) {
#pragma unroll
        for (int o = 0; o < NO; ++o) topk_insert<SLOTS>(sc[o], id[o], x_prev[o], id_prev);
    }

#pragma unroll
    for (int o = 0; o < NO; ++o) {
        const int t = NT >= 2 ? 2 * o + half : 0;
        const int R = r0 + 32 * t + col;
        const int pos = qb * kBlock + R / Hkv;
        const int g = R % Hkv;
        const bool writer = pos < N && (NT >= 2 || half == 0);
        const int nvalid = min(nslots, lrow[o]);
        int v[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) v[s] = id[o][s] < 0 ? 0x7fffffff : id[o][s];
        sort_ascending<SLOTS>(v);
        if (writer) {
            int32_t* dst = block_idx + (((size_t)b * Hkv + g) * N + pos) * k;
#pragma unroll
            for (int s = 0; s <= SLOTS; ++s) {
                if (s < k) dst[s] = s < nvalid ? v[s < SLOTS ? s : SLOTS - 1] : (s == nvalid ? lrow[o] : -1);
            }
        }
    }
}

// Software-pipelined variant for 8-wave work-groups (one per CU, two waves
// per SIMD): several LDS stages so that the first operands of key block j+1
// can be requested while block j is still on the matrix cores (fp8/fp4: three
// stages, block j+2 written to the third one meanwhile and block j+3 in flight
// in VGPRs; bf16: four stages, block j+3 copied straight into the stage block
// j-1 freed; one barrier per block either way), and the A operands of a block
// are requested PF ahead of the MFMA that uses them, across block boundaries. The last key tile's max of
// block j is taken under block j+1's first MFMAs, and its candidate inserted
// right after.
template <typename T, int DI, int NT, int WAVES, int SLOTS, int BK>
__global__ __launch_bounds__(64 * WAVES, 1) void index_topk_pipe_kernel(
    const T* __restrict__ q_idx, const T* __restrict__ k_idx, int32_t* __restrict__ block_idx,
    int B, int N, int Hkv, int k, int qb_lo, int qb_cnt, int chunks) {
    constexpr int NTHR = 64 * WAVES;
    constexpr int RB = elem_bytes<T>(DI);     // bytes of one index row
    constexpr int ROWB = RB + 16;             // padded LDS row, bytes
    constexpr int BUF = kBlock * ROWB;        // one stage
    using MM = IdxMma<T>;
    constexpr int KD = MM::KD;
    constexpr int KS = DI / KD;               // KD-deep slices of the contraction
    constexpr int CPR = RB / 16;              // 16-byte chunks per key row
    constexpr int CPT = kBlock * CPR / NTHR;  // chunks per thread per key block
    constexpr int NO = NT >= 2 ? NT / 2 : 1;  // rows each lane keeps a top-k list for
    constexpr int NOPS = (kBlock / 32) * KS;  // A operands per key block
    constexpr int RING = NOPS < 8 ? NOPS : 8, PF = RING - 2;   // operand registers; requests ahead of use
    static_assert(CPT * NTHR == kBlock * CPR, "staging must tile the block");
    static_assert(NOPS % RING == 0 && PF < RING, "operand ring must tile the block");
    static_assert(NT % 2 == 0, "lanes of both half-waves own rows");
    // bf16 blocks are copied global -> LDS directly (no registers), through
    // four stages. Each 64-lane copy fills 1 KiB of consecutive LDS, i.e. 64 chunks
    // of the padded rows (a row's pad chunk takes a copy of its first chunk),
    // so a stage is exactly DMA_N copies; every wave issues DMA_W of them per
    // block (the ones past DMA_N into a scratch area), so that the wait at the
    // end of a block can leave exactly the next block's copies in flight. The
    // 8-bit and 4-bit inputs keep the register-staged three-stage form: their
    // blocks take a quarter or an eighth of the matrix-core time, too little to
    // hide the copies (fp8 7.6 ms with them against 6.2-6.5, fp4 5.5 against 4.6).
    constexpr bool kDma = std::is_same<T, bf16_t>::value;
    constexpr int DMA_N = kBlock * (CPR + 1) / 64, DMA_W = (DMA_N + WAVES - 1) / WAVES;
    constexpr int DMA_X = DMA_W * WAVES - DMA_N;   // scratch copies
    static_assert(!kDma || (ROWB == 16 * (CPR + 1) && DMA_W <= 15), "copies fill padded rows; vmcnt field");
    __shared__ __align__(16) unsigned char lds[kDma ? 4 * BUF + 1024 * (DMA_X > 0 ? DMA_X : 1) : 3 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int per_qb = B * chunks;
    const int qb = qb_lo + qb_cnt - 1 - (int)(blockIdx.x / per_qb);   // heaviest first
    const int b = (int)(blockIdx.x % per_qb) / chunks;
    const int c = (int)(blockIdx.x % chunks);
    const int r0 = c * (32 * NT * WAVES) + w * (32 * NT);
    const size_t qrow0 = ((size_t)b * N + (size_t)qb * kBlock) * Hkv;

    typename MM::Op bq[NT][KS];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int R = r0 + 32 * t + col;
        const bool valid = qb * kBlock + R / Hkv < N;
        const unsigned char* src =
            reinterpret_cast<const unsigned char*>(q_idx) + (qrow0 + R) * RB + elem_bytes<T>((KD / 2) * half);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (valid) bq[t][s].load(src + elem_bytes<T>(KD * s));
            else bq[t][s].zero();
        }
    }

    float sc[NO][SLOTS];
    int id[NO][SLOTS];
    const int nslots = k - 1;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const bool dummy = s < SLOTS - nslots;   // unused slots sit above every score
            sc[o][s] = dummy ? __builtin_inff() : -__builtin_inff();
            id[o][s] = dummy ? -2 : -1;
        }
    }

    // Stage offsets of this thread's chunks (global: linear; LDS: padded rows).
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(k_idx) + (size_t)b * N * RB;
    const unsigned char* opbase = lds + col * ROWB + elem_bytes<T>((KD / 2) * half);   // + stage + operand offset
    const int nj = BlockPlan<BK>::scanned(qb);
    int lrow[NO];   // per owned row (t = 2o + half): its competing blocks (= its local block id)
#pragma unroll
    for (int o = 0; o < NO; ++o) lrow[o] = BlockPlan<BK>::local(qb, (r0 + 32 * (2 * o + half) + col) / Hkv);
    // 16-byte chunk ch of scanned block j (the query's own block, scanned for
    // BK = 64, may end past N: its rows there repeat row N - 1, never used)
    auto chunk_src = [&](int j, int ch) {
        const int key = BK == 64 ? min(j * kBlock + ch / CPR, N - 1) : j * kBlock + ch / CPR;
        return reinterpret_cast<const u32x4*>(kbase + (size_t)key * RB + (ch % CPR) * 16);
    };
    int dch[kDma ? DMA_W : 1];   // source chunk (row * CPR + column) of each of this wave's copies
#pragma unroll
    for (int u = 0; u < (kDma ? DMA_W : 1); ++u) {
        const int c = 64 * (w + WAVES * u) + lane;
        const int row = c / (CPR + 1), cc = c % (CPR + 1);
        dch[u] = c < 64 * DMA_N ? row * CPR + (cc < CPR ? cc : 0) : 0;
    }
    auto dma_block = [&](int jb, int st) {
#pragma unroll
        for (int u = 0; u < DMA_W; ++u) {
            const int i = w + WAVES * u;
            unsigned char* dst = i < DMA_N ? lds + st * BUF + 1024 * i : lds + 4 * BUF + 1024 * (i - DMA_N);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)chunk_src(jb, dch[u]),
                                             (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };
    // End of a block on the copy path: this wave's copies of the block after
    // next have landed (only the DMA_W copies requested since may be in flight)
    // and its LDS reads are done; then the barrier. The wavefront-scope fences
    // emit no wait of their own but keep the compiler from moving LDS accesses
    // across the barrier.
    auto dma_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0x70 | DMA_W);   // vmcnt(DMA_W) lgkmcnt(0)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    u32x4 stage[kDma ? 1 : CPT];
    typename MM::Op a[RING];
    if (kDma) {
        if (nj > 0) {
            dma_block(0, 0);
            dma_block(min(1, nj - 1), 1);
            dma_block(min(2, nj - 1), 2);
            dma_barrier();   // blocks 0 and 1 in LDS
        }
    } else if (nj > 0) {   // a row of query block 0 has no candidate block at BK >= 128
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
            for (int u = 0; u < CPT; ++u) stage[u] = *chunk_src(min(bb, nj - 1), tid + NTHR * u);
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int ch = tid + NTHR * u;
                *reinterpret_cast<u32x4*>(lds + bb * BUF + (ch / CPR) * ROWB + (ch % CPR) * 16) = stage[u];
            }
        }
#pragma unroll
        for (int u = 0; u < CPT; ++u) stage[u] = *chunk_src(min(2, nj - 1), tid + NTHR * u);
    }
    if constexpr (!kDma) __syncthreads();
    if (nj > 0) {
#pragma unroll
        for (int m = 0; m < PF; ++m) a[m].load(opbase + ((m / KS) * 32) * ROWB + elem_bytes<T>(KD * (m % KS)));
    }

    float bm[NT], bm_prev[NT];
    float stash[NO];   // BK = 256: the max of the pair's first block
    floatx16 acc[2][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        bm_prev[t] = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[1][t][r] = -__builtin_inff();
    }
#pragma unroll
    for (int o = 0; o < NO; ++o) stash[o] = -__builtin_inff();
    // Candidate of a finished block j (BK = 128: its max; 64: the max of its
    // second half, never a candidate in the query's own block; 256: the pair's
    // max once both halves are in).
    auto finish_block = [&](int jb, float x, int o) {
        if (BK == 128) {
            if (__builtin_amdgcn_ballot_w64(x > sc[o][SLOTS - 1])) topk_insert<SLOTS>(sc[o], id[o], x, jb);
        } else if (BK == 64) {
            if (2 * jb + 1 < lrow[o]) topk_insert<SLOTS>(sc[o], id[o], x, 2 * jb + 1);
        } else if (jb & 1) {
            topk_insert<SLOTS>(sc[o], id[o], fmaxf(stash[o], x), jb / 2);
        } else {
            stash[o] = x;
        }
    };
    int sb = 0;   // stage of block j
    for (int j = 0; j < nj; ++j) {
        // stages of blocks j+1 and j+2 (three stages: that of block j-1; four: block j+3 goes there)
        const int nb1 = kDma ? (sb + 1) & 3 : (sb == 2 ? 0 : sb + 1);
        const int wb = kDma ? (sb + 2) & 3 : (nb1 == 2 ? 0 : nb1 + 1);
        if constexpr (kDma) dma_block(min(j + 3, nj - 1), (sb + 3) & 3);
#pragma unroll
        for (int n = 0; n < NOPS; ++n) {
            const int kt = n / KS, s = n % KS;
            const int m = n + PF;
            if (m < NOPS) a[m % RING].load(opbase + sb * BUF + ((m / KS) * 32) * ROWB + elem_bytes<T>(KD * (m % KS)));
            else a[m % RING].load(opbase + nb1 * BUF + (((m - NOPS) / KS) * 32) * ROWB +
                                  elem_bytes<T>(KD * ((m - NOPS) % KS)));
            if (s == 0) {
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[kt & 1][t] = zero16();
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) MM::mma(acc[kt & 1][t], a[n % RING], bq[t][s]);
            if (s == KS - 1) {
                if (kt == 0) {
                    // block j-1: last tile's max, then its candidate (at BK = 128 the
                    // insert is skipped by the whole wave when no row's candidate beats
                    // its current last entry, rare for late blocks of long rows)
                    if (j > 0) {
#pragma unroll
                        for (int o = 0; o < NO; ++o)
                            finish_block(j - 1,
                                         pair_max_own(fmaxf(bm_prev[2 * o], max16(acc[1][2 * o])),
                                                      fmaxf(bm_prev[2 * o + 1], max16(acc[1][2 * o + 1]))),
                                         o);
                    }
                } else if (BK == 64 && kt == 3) {
                    // the second half starts at key tile 2
#pragma unroll
                    for (int t = 0; t < NT; ++t) bm[t] = max16(acc[0][t]);
                } else {
#pragma unroll
                    for (int t = 0; t < NT; ++t) bm[t] = kt == 1 ? max16(acc[0][t]) : fmaxf(bm[t], max16(acc[(kt - 1) & 1][t]));
                    if (BK == 64 && kt == 2) {
                        // key tiles 0-1 done: the first 64-key block of j (for the
                        // query's own block only the rows of the second half see it)
#pragma unroll
                        for (int o = 0; o < NO; ++o) {
                            const float x = pair_max_own(bm[2 * o], bm[2 * o + 1]);
                            if (2 * j < lrow[o]) topk_insert<SLOTS>(sc[o], id[o], x, 2 * j);
                        }
                    }
                }
            }
            // bf16: each step stays where it is written; left free, the scheduler moves
            // a key tile's max up to right behind the tile's last product, where it
            // waits for that product's result with the matrix core idle (10.6 against
            // 10.8 ms at 128K). The fp8/fp4 forms, with a quarter of the products per
            // step, run faster without the constraint (6.03 against 6.25 ms, 4.26
            // against 4.49 ms).
            if constexpr (kDma) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) bm_prev[t] = bm[t];
        if constexpr (kDma) {
            dma_barrier();
        } else {
            // Block j+2 into the stage block j-1 used; block j+3 into VGPRs.
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int ch = tid + NTHR * u;
                *reinterpret_cast<u32x4*>(lds + wb * BUF + (ch / CPR) * ROWB + (ch % CPR) * 16) = stage[u];
            }
#pragma unroll
            for (int u = 0; u < CPT; ++u) stage[u] = *chunk_src(min(j + 3, nj - 1), tid + NTHR * u);
            __syncthreads();
        }
        sb = nb1;
    }
    // no copy may still be writing this work-group's LDS when its waves end
    if constexpr (kDma) __builtin_amdgcn_s_waitcnt(0);
    if (nj > 0) {
#pragma unroll
        for (int o = 0; o < NO; ++o)
            finish_block(nj - 1,
                         pair_max_own(fmaxf(bm_prev[2 * o], max16(acc[1][2 * o])),
                                      fmaxf(bm_prev[2 * o + 1], max16(acc[1][2 * o + 1]))),
                         o);
    }

#pragma unroll
    for (int o = 0; o < NO; ++o) {
        const int t = NT >= 2 ? 2 * o + half : 0;
        const int R = r0 + 32 * t + col;
        const int pos = qb * kBlock + R / Hkv;
        const int g = R % Hkv;
        const bool writer = pos < N && (NT >= 2 || half == 0);
        const int nvalid = min(nslots, lrow[o]);
        int v[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) v[s] = id[o][s] < 0 ? 0x7fffffff : id[o][s];
        sort_ascending<SLOTS>(v);
        if (writer) {
            int32_t* dst = block_idx + (((size_t)b * Hkv + g) * N + pos) * k;
#pragma unroll
            for (int s = 0; s <= SLOTS; ++s) {
                if (s < k) dst[s] = s < nvalid ? v[s < SLOTS ? s : SLOTS - 1] : (s == nvalid ? lrow[o] : -1);
            }
        }
    }
}

template <typename T, int DI, int NT, int WAVES, int BK>
static hipError_t launch_cfg(const LaunchDims& d, int qb_lo, int qb_cnt, const void* q_idx, const void* k_idx,
                             int32_t* out, hipStream_t st) {
    // One key block per barrier: two such work-groups share a CU (two LDS
    // stages each), which measured faster than fewer, larger stages.
    constexpr int BPB = 1;
    const int chunks = (kBlock * d.Hkv) / (32 * NT * WAVES);
    const dim3 grid((unsigned)(qb_cnt * d.B * chunks)), block(64 * WAVES);
    const T* q = static_cast<const T*>(q_idx);
    const T* kk = static_cast<const T*>(k_idx);
    if (d.k <= 8)
        hipLaunchKernelGGL((index_topk_kernel<T, DI, NT, WAVES, 7, BPB, BK>), grid, block, 0, st, q, kk, out, d.B, d.N,
                           d.Hkv, d.k, qb_lo, qb_cnt, chunks);
    else if (d.k <= 16)
        hipLaunchKernelGGL((index_topk_kernel<T, DI, NT, WAVES, 15, BPB, BK>), grid, block, 0, st, q, kk, out, d.B, d.N,
                           d.Hkv, d.k, qb_lo, qb_cnt, chunks);
    else
        hipLaunchKernelGGL((index_topk_kernel<T, DI, NT, WAVES, 31, BPB, BK>), grid, block, 0, st, q, kk, out, d.B, d.N,
                           d.Hkv, d.k, qb_lo, qb_cnt, chunks);
    return hipGetLastError();
}

// Shapes: the pipelined 8-wave kernel when 512 rows tile a query block (128*Hkv
// rows) in bf16; else 4-wave work-groups (one wave per SIMD, 64 rows per wave
// for bf16, two work-groups per CU) when 256 rows do, else 2-wave ones.
template <typename T, int DI, int BK>
static hipError_t launch_pipe(const LaunchDims& d, int qb_lo, int qb_cnt, const void* q_idx, const void* k_idx,
                              int32_t* out, hipStream_t st) {
    constexpr int NT = 2, WAVES = 8;
    const int chunks = (kBlock * d.Hkv) / (32 * NT * WAVES);
    const dim3 grid((unsigned)(qb_cnt * d.B * chunks)), block(64 * WAVES);
    const T* q = static_cast<const T*>(q_idx);
    const T* kk = static_cast<const T*>(k_idx);
    if (d.k <= 8)
        hipLaunchKernelGGL((index_topk_pipe_kernel<T, DI, NT, WAVES, 7, BK>), grid, block, 0, st, q, kk, out, d.B, d.N,
                           d.Hkv, d.k, qb_lo, qb_cnt, chunks);
    else if (d.k <= 16)
        hipLaunchKernelGGL((index_topk_pipe_kernel<T, DI, NT, WAVES, 15, BK>), grid, block, 0, st, q, kk, out, d.B, d.N,
                           d.Hkv, d.k, qb_lo, qb_cnt, chunks);
    else
        hipLaunchKernelGGL((index_topk_pipe_kernel<T, DI, NT, WAVES, 31, BK>), grid, block, 0, st, q, kk, out, d.B, d.N,
                           d.Hkv, d.k, qb_lo, qb_cnt, chunks);
    return hipGetLastError();
}

template <typename T, int DI, int BK>
static hipError_t launch_bk(const LaunchDims& d, int qb_lo, int qb_cnt, const void* q_idx, const void* k_idx,
                            int32_t* out, hipStream_t st) {
    constexpr int NT = sizeof(T) <= 2 ? 2 : 1;   // fp32 operands take twice the VGPRs
    const int rows = kBlock * d.Hkv;
    // the pipelined kernel stages a key block with one 16-byte chunk per thread
    if constexpr (sizeof(T) <= 2 && kBlock * elem_bytes<T>(DI) / 16 >= 512) {
        if (rows % (32 * 2 * 8) == 0) return launch_pipe<T, DI, BK>(d, qb_lo, qb_cnt, q_idx, k_idx, out, st);
    }
    if (rows % (32 * NT * 4) == 0) return launch_cfg<T, DI, NT, 4, BK>(d, qb_lo, qb_cnt, q_idx, k_idx, out, st);
    return launch_cfg<T, DI, NT, 2, BK>(d, qb_lo, qb_cnt, q_idx, k_idx, out, st);
}

// Block sizes 64 and 256 for bf16 and fp32 index inputs; fp8 and fp4 at 128.
template <typename T, int DI>
static hipError_t launch_di(const LaunchDims& d, int qb_lo, int qb_cnt, const void* q_idx, const void* k_idx,
                            int32_t* out, hipStream_t st) {
    if constexpr (sizeof(T) == 2 || sizeof(T) == 4) {
        if (d.Bk == 64) return launch_bk<T, DI, 64>(d, qb_lo, qb_cnt, q_idx, k_idx, out, st);
        if (d.Bk == 256) return launch_bk<T, DI, 256>(d, qb_lo, qb_cnt, q_idx, k_idx, out, st);
    }
    return launch_bk<T, DI, 128>(d, qb_lo, qb_cnt, q_idx, k_idx, out, st);
}

hipError_t launch_index_topk(const LaunchDims& d, int qb_lo, int qb_hi, const void* q_idx, const void* k_idx,
                             int32_t* block_idx, hipStream_t st) {
    if (d.B == 0 || d.N == 0 || qb_hi <= qb_lo) return hipSuccess;
    const int cnt = qb_hi - qb_lo;
    if (d.dtype == 0) {
        return d.Di == 128 ? launch_di<bf16_t, 128>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st)
                           : launch_di<bf16_t, 64>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st);
    }
    if (d.dtype == 2) {
        return d.Di == 128 ? launch_di<fp8_t, 128>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st)
                           : launch_di<fp8_t, 64>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st);
    }
    if (d.dtype == 3) {
        return d.Di == 128 ? launch_di<fp4x2_t, 128>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st)
                           : launch_di<fp4x2_t, 64>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st);
    }
    return d.Di == 128 ? launch_di<float, 128>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st)
                       : launch_di<float, 64>(d, qb_lo, cnt, q_idx, k_idx, block_idx, st);
}

}  // namespace msa
