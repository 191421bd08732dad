// Pieces shared by the two backward kernels (main branch and KL term): both
// visit the rows of one key block in 32-row tiles, key-block-outer, over the
// position-sorted selection lists.
#pragma once

#include "msa_common.h"

namespace msa {

// Position of key `kk` of a 16-key group in the permuted K^T / V^T copies and
// of row `m` in the transposed tiles: bits 2 and 3 swapped.
__device__ __forceinline__ int perm16(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// Transposed 32-row tile [D][32 rows, permuted], stored chunk-major: the
// 16-byte chunk q (rows 8q .. 8q+7 of the permuted order) of dim d sits at
// q * (16 D + 16) + 16 d. The 16 lanes of a read phase (consecutive d, one q)
// then cover all banks once; the 16-byte pad between chunk columns spreads the
// staging writes of different q.
template <int D>
struct ColTile {
    static constexpr int QSTRIDE = 16 * D + 16;
    static constexpr int BYTES = 4 * QSTRIDE;
    __device__ static __forceinline__ int offset(int d, int q) { return q * QSTRIDE + 16 * d; }
};

// Work item of a backward kernel: the rows of one (b, g, key block j) item of
// the sorted lists (LOCAL = false), or the rows of query block j against their
// own block (LOCAL = true).
template <bool LOCAL>
struct BwdItem {
    int b, g, j, count, start, q0, lslot;
    const int* entries;   // LDS copy of the item's list entries
    // (position, slot) of entry e < count.
    __device__ __forceinline__ void entry(int e, int& i, int& s) const {
        if constexpr (LOCAL) {
            i = q0 + e;
            s = lslot;
        } else {
            const int v = entries[e];
            i = v >> 5;
            s = v & 31;
        }
    }
};

// Per row: the sum of its slots' bf16 partials in slot order (dQ, with G heads
// of D dims per row; the KL term's dq_idx, with G = 1 and D = Di). One thread
// per (row, head, 16 stored elements = one (32-dim slice, half) of the
// lane-major order).
template <int D, int G>
__global__ __launch_bounds__(256) void dq_combine_kernel(const bf16_t* __restrict__ dq_part, bf16_t* __restrict__ dq,
                                                         int64_t units, int N, int Hkv, int topk) {
    constexpr int QPH = D / 16;   // 16-element groups per head
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x >= units) return;
    const int qg = (int)(x % QPH);
    const int hh = (int)((x / QPH) % G);
    const int64_t row = x / (QPH * G);   // (b * Hkv + g) * N + i
    const int i = (int)(row % N);
    const int64_t bg = row / N;
    const int g = (int)(bg % Hkv), b = (int)(bg / Hkv);
    const int nv = min(topk, i / kBlock + 1);
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const bf16_t* src = dq_part + (size_t)row * topk * G * D + (size_t)hh * D + 16 * qg;
    for (int s = 0; s < nv; ++s) {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)s * G * D));
        const u32x4 c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)s * G * D + 8));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(a[e] << 16);
            acc[2 * e + 1] += __uint_as_float(a[e] & 0xffff0000u);
            acc[8 + 2 * e] += __uint_as_float(c[e] << 16);
            acc[8 + 2 * e + 1] += __uint_as_float(c[e] & 0xffff0000u);
        }
    }
    // stored element 16*qg + r of the head: slice dt = qg/2, half h = qg%2,
    // dim 32*dt + 8*(r/4) + 4*h + r%4
    const int dt = qg / 2, h = qg % 2;
    const int Hq = Hkv * G;
    bf16_t* dst = dq + (((size_t)b * N + i) * Hq + g * G + hh) * D + 32 * dt + 4 * h;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<uint2*>(dst + 8 * rq) = make_uint2(pack_bf16x2(acc[4 * rq], acc[4 * rq + 1]),
                                                             pack_bf16x2(acc[4 * rq + 2], acc[4 * rq + 3]));
}

}  // namespace msa
