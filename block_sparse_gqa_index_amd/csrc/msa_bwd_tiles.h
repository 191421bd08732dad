// Pieces shared by the backward kernels (main branch and KL term): both visit
// the rows of one key block in 32-row tiles, key-block-outer, over the
// position-sorted selection lists.
#pragma once

#include "msa_common.h"
#include "msa_internal.h"

namespace msa {

// Position of key `kk` of a 16-key group in the permuted K^T / V^T copies and
// of row `m` in the transposed tiles: bits 2 and 3 swapped.
__device__ __forceinline__ int perm16(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// Transposed 32-row tile [D][32 rows, permuted], stored chunk-major: the
// 16-byte chunk q (rows 8q .. 8q+7 of the permuted order) of dim d sits at
// q * 16 D + 16 (d ^ ((d / 8) % 16)).
// LDS banking on gfx950 (measured with the bank-conflict counter): a 16-byte
// read is served 16 lanes per cycle over 64 four-byte banks, a cycle pairing
// eight lanes of one 16-lane group with eight of another (0-7 with 24-31,
// 8-15 with 16-23, likewise in the upper half); writes go 128 bytes per cycle
// over 32 banks, consecutive lanes together. The readers take 16 consecutive
// d of one or two chunk columns per cycle: with the columns 16 D bytes apart
// (a multiple of the 256-byte bank cycle) those are 16 different slots, where
// any pad between the columns would shift one 8-lane run onto the other. The
// XOR sends the staging writes of one dim offset d % 8 from sixteen 8-dim
// groups to sixteen different slots (without it they all hit the same banks).
template <int D>
struct ColTile {
    static constexpr int QSTRIDE = 16 * D;
    static constexpr int BYTES = 4 * QSTRIDE;
    __device__ static __forceinline__ int offset(int d, int q) { return q * QSTRIDE + 16 * (d ^ ((d >> 3) & 15)); }
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

// Sets up the work item of this work-group in window `win` (LOCAL: the causal
// block of query block qb0 + blockIdx.x / (B * Hkv)) and its partial slot;
// false when the slot is empty (the whole work-group returns). Non-local items
// copy their list entries into `entries` (LDS), then synchronise.
template <bool LOCAL>
__device__ __forceinline__ bool fused_item(BwdItem<LOCAL>& it, size_t& pidx, int* entries,
                                           const int32_t* __restrict__ list, const int4* __restrict__ items,
                                           const int32_t* __restrict__ item_offsets,
                                           const int32_t* __restrict__ total_items, int n_keys, int B, int N, int Hkv,
                                           int nb, int nwin, int topk, const FusedWindow& win) {
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
        return true;
    } else {
        const int bgi = blockIdx.x / win.bound, x = blockIdx.x % win.bound;
        const int kf = (bgi * nwin + win.w) * nb;
        const int first = item_offsets[kf];
        const int end = kf + nb < n_keys ? item_offsets[kf + nb] : total_items[0];
        if (first + x >= end) return false;
        const int4 e = items[first + x];
        it.j = e.x % nb;
        it.g = bgi % Hkv;
        it.b = bgi / Hkv;
        it.start = e.y;
        it.count = e.z;
        it.q0 = 0;
        it.lslot = 0;
        it.entries = entries;
        pidx = blockIdx.x;
        for (int y = threadIdx.x; y < it.count; y += blockDim.x) entries[y] = list[it.start + y];
        __syncthreads();
        return true;
    }
}

// Per row: the sum of its slots' bf16 partials in slot order (dQ, with G heads
// of D dims per row; the KL term's dq_idx, with G = 1 and D = Di). A slot's
// partial is G * D contiguous stored elements; thread t of a row sums the
// 8-element groups t and t + TPR of it, so each of the wave's two load
// instructions per slot reads whole cache lines (64 consecutive 16-byte
// chunks or whole 128-byte halves of rows) and no line is split between them.
// Stored element 16*qg + r of a head is dim 32*(qg/2) + 8*(r/4) + 4*(qg%2) + r%4
// (the lane-major order of the partials), or dim 16*qg + r when NAT is set
// (partials in natural dim order).
// The rows handled are positions p0 .. p0 + len - 1 of every (b, g), whose
// partials sit at row (b * Hkv + g) * wrows + (i - p0) of dq_part (a window of
// wrows positions; p0 = 0 and len = wrows = N for the whole sequence).
template <int D, int G, bool NAT = false>
__global__ __launch_bounds__(256) void dq_combine_kernel(const bf16_t* __restrict__ dq_part, bf16_t* __restrict__ dq,
                                                         int64_t units, int N, int Hkv, int topk, int p0, int len,
                                                         int wrows) {
    constexpr int SPAN = G * D;      // stored elements per (row, slot)
    constexpr int TPR = SPAN / 16;   // threads per row
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x >= units) return;
    const int t = (int)(x % TPR);
    const int64_t wr = x / TPR;   // (b * Hkv + g) * len + (i - p0)
    const int i = p0 + (int)(wr % len);
    const int64_t bg = wr / len;
    const int g = (int)(bg % Hkv), b = (int)(bg / Hkv);
    const int nv = min(topk, i / kBlock + 1);
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const bf16_t* src = dq_part + ((size_t)bg * wrows + (i - p0)) * topk * SPAN;
    for (int s = 0; s < nv; ++s) {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)s * SPAN + 8 * t));
        const u32x4 c =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)s * SPAN + 8 * (t + TPR)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(a[e] << 16);
            acc[2 * e + 1] += __uint_as_float(a[e] & 0xffff0000u);
            acc[8 + 2 * e] += __uint_as_float(c[e] << 16);
            acc[8 + 2 * e + 1] += __uint_as_float(c[e] & 0xffff0000u);
        }
    }
    const int Hq = Hkv * G;
    if constexpr (NAT) {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            const int e0 = 8 * (t + part * TPR);
            const float* v = acc + 8 * part;
            *reinterpret_cast<u32x4*>(dq + (((size_t)b * N + i) * Hq + g * G) * D + e0) =
                u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7])};
        }
        return;
    }
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        const int e0 = 8 * (t + part * TPR);   // first stored element of the group in the slot's partial
        const int hh = e0 / D, se = e0 % D;
        const int qg = se / 16, r0 = se % 16;   // r0 = 0 or 8
        bf16_t* dst = dq + (((size_t)b * N + i) * Hq + g * G + hh) * D + 32 * (qg / 2) + 4 * (qg % 2);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const float* v = acc + 8 * part + 4 * q2;
            *reinterpret_cast<uint2*>(dst + 8 * (r0 / 4 + q2)) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
}

}  // namespace msa
