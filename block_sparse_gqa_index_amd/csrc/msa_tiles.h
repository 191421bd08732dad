// Tile-level building blocks shared by the attention and KL kernels: one
// 32-row tile of query rows against one LDS-resident block of 128 keys.
//
// S^T = K Q^T on the matrix cores (A = keys from LDS, B = query rows held in
// VGPRs) leaves one query row per lane: lane l holds row l % 32 and keys
// 8*(r/4) + 4*(l/32) + r%4 (+32 per key tile) in accumulator r. P^T = the
// probabilities in that layout feed O^T = V^T P^T as the B operand, with V^T
// read from LDS under the same key assignment.
#pragma once

#include "msa_common.h"

namespace msa {

// LDS tile of rows of W elements of T, unpadded, with the 16-byte chunks of
// every row XOR-swizzled by the row index (physical chunk = c ^ (row % SW)).
// Both access patterns used here then hit distinct banks: 16 lanes reading
// the same logical chunk of 16 consecutive rows, and 16 lanes writing the 16
// chunks of one row.
template <typename T, int W>
struct SwzTile {
    static constexpr int ES = sizeof(T);
    static constexpr int ROWB = W * ES;
    static constexpr int CPR = ROWB / 16;
    static constexpr int SW = CPR < 16 ? CPR : 16;
    static constexpr int BYTES = kBlock * ROWB;   // for a 128-row tile
    __device__ static __forceinline__ int offset(int row, int byte) {
        return row * ROWB + (((byte >> 4) ^ (row & (SW - 1))) << 4) + (byte & 15);
    }
    // Eight consecutive elements starting at element `e` of `row`.
    __device__ static __forceinline__ void load8(Op8<T>& a, const unsigned char* base, int row, int e) {
        if constexpr (ES == 2) {
            a.load(base + offset(row, e * ES));
        } else {
            const float4 x = *reinterpret_cast<const float4*>(base + offset(row, e * ES));
            const float4 y = *reinterpret_cast<const float4*>(base + offset(row, e * ES + 16));
            a.v[0] = x.x; a.v[1] = x.y; a.v[2] = x.z; a.v[3] = x.w;
            a.v[4] = y.x; a.v[5] = y.y; a.v[6] = y.z; a.v[7] = y.w;
        }
    }
};

// Direct global -> LDS copy (no registers) of rows [r0, r0 + 64 / CPR) of a
// swizzled bf16 tile [rows][W] (SwzTile layout): the wave's 64 lanes fill 64
// consecutive 16-byte LDS chunks, lane i physical chunk i % CPR of row
// r0 + i / CPR, so it reads logical chunk (i % CPR) ^ (row % SW) of that row.
// Source rows past max_row repeat row max_row.
template <int W>
__device__ __forceinline__ void dma_rows(unsigned char* tile, const bf16_t* src, size_t stride, int r0, int max_row,
                                         int lane) {
    using S = SwzTile<bf16_t, W>;
    const int row = r0 + lane / S::CPR, pc = lane % S::CPR;
    const int lc = pc ^ (row & (S::SW - 1));
    const bf16_t* g = src + (size_t)min(row, max_row) * stride + lc * (16 / sizeof(bf16_t));
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)(tile + r0 * S::ROWB), 16, 0, 0);
}

// A [128][W] tile from global rows `row_stride` elements apart; rows at or
// beyond `valid_rows` are zero-filled.
template <typename T, int W>
__device__ void stage_rows(unsigned char* lds, const T* src, size_t row_stride, int valid_rows) {
    using S = SwzTile<T, W>;
    constexpr int EPC = 16 / sizeof(T);
    for (int ch = threadIdx.x; ch < kBlock * S::CPR; ch += blockDim.x) {
        const int row = ch / S::CPR, cc = ch % S::CPR;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < valid_rows) x = *reinterpret_cast<const u32x4*>(src + row * row_stride + cc * EPC);
        *reinterpret_cast<u32x4*>(lds + S::offset(row, cc * 16)) = x;
    }
}

// K block [128 keys][D] (the A operand of S^T = K Q^T) followed by the V^T
// block [D][128 keys] (the A operand of O^T = V^T P^T), copied from the
// pre-transposed V^T (zero past the last key). Keys at or beyond `valid_keys`
// are zero-filled in K.
template <typename T, int D>
struct KVTile {
    using KS = SwzTile<T, D>;
    using VS = SwzTile<T, kBlock>;
    static constexpr int BYTES = kBlock * KS::ROWB + D * VS::ROWB;

    __device__ static void stage(unsigned char* lds, const T* kb, size_t row_stride, const T* vtb,
                                 int valid_keys) {
        stage_rows<T, D>(lds, kb, row_stride, valid_keys);
        constexpr int EPC = 16 / sizeof(T);
        unsigned char* vt = lds + kBlock * KS::ROWB;
        for (int ch = threadIdx.x; ch < D * VS::CPR; ch += blockDim.x) {
            const int d = ch / VS::CPR, vc = ch % VS::CPR;
            *reinterpret_cast<u32x4*>(vt + VS::offset(d, vc * 16)) =
                *reinterpret_cast<const u32x4*>(vtb + (size_t)d * kBlock + vc * EPC);
        }
    }
};

template <typename T> struct PType;
template <> struct PType<bf16_t> {
    static __device__ __forceinline__ void pack(Op8<bf16_t>& o, const float* p) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
        o.v = __builtin_bit_cast(bf16x8, w);
    }
};
template <> struct PType<float> {
    static __device__ __forceinline__ void pack(Op8<float>& o, const float* p) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = p[e];
    }
};

// V^T operand for 16-key slice c: keys 16c + {4h..4h+3} and 16c + 8 + {4h..4h+3}
// of V^T row `d`, which the V^T copy stores contiguously at positions
// 16c + 8h .. 16c + 8h + 7.
template <typename T>
__device__ __forceinline__ void load_vt_op(Op8<T>& a, const unsigned char* vt, int d, int c, int half) {
    using VS = SwzTile<T, kBlock>;
    constexpr int ES = sizeof(T);
    if constexpr (ES == 2) {
        a.load(vt + VS::offset(d, (16 * c + 8 * half) * ES));
    } else {
        const float4 x = *reinterpret_cast<const float4*>(vt + VS::offset(d, (16 * c + 8 * half) * ES));
        const float4 y = *reinterpret_cast<const float4*>(vt + VS::offset(d, (16 * c + 8 * half + 4) * ES));
        a.v[0] = x.x; a.v[1] = x.y; a.v[2] = x.z; a.v[3] = x.w;
        a.v[4] = y.x; a.v[5] = y.y; a.v[6] = y.z; a.v[7] = y.w;
    }
}

// One 32-row tile against one LDS-resident 128-key block:
// s[kt] = S^T tile kt (32 keys x 32 rows), scores only.
// WIDE: k-slice outer, key tile inner (four independent accumulation chains
// per slice, the slice's four key operands live at a time); otherwise key tile
// outer (one chain at a time, one operand live: fewer VGPRs).
template <typename T, int D, bool WIDE = true>
__device__ __forceinline__ void tile_scores(floatx16 (&s)[4], const Op8<T> (&bq)[D / 16],
                                            const unsigned char* lds, int col, int half) {
    using KS = SwzTile<T, D>;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s[kt] = zero16();
    if constexpr (!WIDE) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int sl = 0; sl < D / 16; ++sl) {
                Op8<T> a;
                KS::load8(a, lds, kt * 32 + col, 16 * sl + 8 * half);
                mma16(s[kt], a, bq[sl]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl) {
        Op8<T> a[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) KS::load8(a[kt], lds, kt * 32 + col, 16 * sl + 8 * half);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mma16(s[kt], a[kt], bq[sl]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// o[dt] += V^T(dt) * P^T with P taken from the score accumulators.
template <typename T, int D>
__device__ __forceinline__ void tile_pv(floatx16 (&o)[D / 32], const floatx16 (&p)[4],
                                        const unsigned char* lds, int col, int half) {
    const unsigned char* vt = lds + kBlock * SwzTile<T, D>::ROWB;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = p[c / 2][8 * (c % 2) + e];
        Op8<T> bp;
        PType<T>::pack(bp, pe);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            Op8<T> a;
            load_vt_op<T>(a, vt, dt * 32 + col, c, half);
            mma16(o[dt], a, bp);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <typename T, int D>
__device__ __forceinline__ void load_q_op(Op8<T> (&bq)[D / 16], const T* row, bool valid, int half) {
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl) {
        if (valid) bq[sl].load(row + 16 * sl + 8 * half);
        else bq[sl].zero();
    }
}

// Row softmax over the lane's 64 scores + the other half's 64 (log2 domain):
// returns the row max of z = s * scale_log2 and the row sum of 2^(z - max),
// and overwrites the scores with those probabilities.
__device__ __forceinline__ void tile_softmax(floatx16 (&s)[4], float scale_log2, float& mx, float& sum) {
    float m = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) m = vmax(m, max16(s[kt]));
    m = vmax(m, swap_halves(m));
    const float mz = m * scale_log2;
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = exp2_hw(fmaf(s[kt][r], scale_log2, -mz));
            s[kt][r] = p;
            l += p;
        }
    }
    l += swap_halves(l);
    mx = mz;
    sum = l;
}

}  // namespace msa
