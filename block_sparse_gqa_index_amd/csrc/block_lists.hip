// Inversion of the block selection: for every (batch, group, window of
// kWindow query positions, key block) the list of query rows of that window
// that kept that block as a non-local block, cut into work items of at most
// kSeg rows. Used by the attention and KL kernels that iterate over key
// blocks. Keys are ordered batch, group, window, block, so walking the items in
// order walks one window's query rows at a time.
#include "msa_common.h"
#include "msa_internal.h"

#include <algorithm>

namespace msa {

// ---------------------------------------------------------------- inversion --

__global__ void fill_i32_kernel(int32_t* p, size_t n, int32_t v) {
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x)
        p[x] = v;
}

// One thread per (b, g, i) row: count the row's non-local blocks.
__global__ void count_kernel(const int32_t* __restrict__ block_idx, int32_t* __restrict__ counts,
                             int64_t rows, int N, int k, int nb, int nwin, int p_lo, int p_len) {
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x >= rows) return;
    const int i = p_lo + (int)(x % p_len);
    const int64_t bg = x / p_len;
    const int64_t r = bg * N + i;
    const int L = i / kBlock;
    const int32_t* row = block_idx + r * k;
    for (int s = 0; s + 1 < k; ++s) {   // a non-local block never sits in the last slot
        const int j = row[s];
        if (j >= 0 && j < L) atomicAdd(&counts[(bg * nwin + i / kWindow) * nb + j], 1);
    }
}

// The same counts from per-work-group LDS histograms: a work-group takes
// kHistPos consecutive positions of one (b, g) and issues one global atomic per
// block its rows touched instead of one per entry.
constexpr int kHistPos = 2048;   // divides kWindow, so a work-group stays inside one window
constexpr int kHistMaxBins = 8192;   // 2 x 32 KB of LDS in the scatter pass

__global__ __launch_bounds__(256) void count_hist_kernel(const int32_t* __restrict__ block_idx,
                                                         int32_t* __restrict__ counts, int N, int k, int nb,
                                                         int nwin, int chunks, int p_lo, int p_hi) {
    extern __shared__ int32_t hist[];
    const int bg = blockIdx.x / chunks, c = blockIdx.x % chunks;
    const int p0 = p_lo + c * kHistPos, p1 = min(p_hi, p0 + kHistPos);
    const int nbins = (p1 - 1) / kBlock;   // every non-local block of these rows is below this
    for (int x = threadIdx.x; x < nbins; x += blockDim.x) hist[x] = 0;
    __syncthreads();
    for (int i = p0 + threadIdx.x; i < p1; i += blockDim.x) {
        const int L = i / kBlock;
        const int32_t* row = block_idx + ((size_t)bg * N + i) * k;
        for (int s = 0; s + 1 < k; ++s) {
            const int j = row[s];
            if (j >= 0 && j < L) atomicAdd(&hist[j], 1);
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < nbins; x += blockDim.x)
        if (hist[x]) atomicAdd(&counts[((size_t)bg * nwin + p0 / kWindow) * nb + x], hist[x]);
}

// Scatter with the same histogram: one global atomic per touched block
// reserves the work-group's range in that block's list, LDS atomics place the
// entries inside it.
__global__ __launch_bounds__(256) void scatter_hist_kernel(const int32_t* __restrict__ block_idx,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ cursor, int32_t* __restrict__ list,
                                                           int N, int k, int nb, int nwin, int chunks, int p_lo,
                                                           int p_hi) {
    extern __shared__ int32_t sh[];
    const int bg = blockIdx.x / chunks, c = blockIdx.x % chunks;
    const int p0 = p_lo + c * kHistPos, p1 = min(p_hi, p0 + kHistPos);
    const int nbins = (p1 - 1) / kBlock;
    int32_t* hist = sh;
    int32_t* base = sh + nbins;
    for (int x = threadIdx.x; x < nbins; x += blockDim.x) hist[x] = 0;
    __syncthreads();
    for (int i = p0 + threadIdx.x; i < p1; i += blockDim.x) {
        const int L = i / kBlock;
        const int32_t* row = block_idx + ((size_t)bg * N + i) * k;
        for (int s = 0; s + 1 < k; ++s) {
            const int j = row[s];
            if (j >= 0 && j < L) atomicAdd(&hist[j], 1);
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < nbins; x += blockDim.x) {
        const int n = hist[x];
        if (n) {
            const size_t key = ((size_t)bg * nwin + p0 / kWindow) * nb + x;
            base[x] = offsets[key] + atomicAdd(&cursor[key], n);
        }
        hist[x] = 0;
    }
    __syncthreads();
    for (int i = p0 + threadIdx.x; i < p1; i += blockDim.x) {
        const int L = i / kBlock;
        const int32_t* row = block_idx + ((size_t)bg * N + i) * k;
        for (int s = 0; s + 1 < k; ++s) {
            const int j = row[s];
            if (j >= 0 && j < L) list[base[j] + atomicAdd(&hist[j], 1)] = (i << 5) | s;
        }
    }
}

// Single work-group exclusive scan over the (b, g, j) keys: list offsets and
// work-item offsets; also clears the scatter cursors.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ item_offsets,
                                                    int32_t* __restrict__ cursor,
                                                    int32_t* __restrict__ total_items, int n_keys, int seg) {
    __shared__ int64_t s_sum[1024];
    __shared__ int64_t s_items[1024];
    const int t = threadIdx.x;
    const int per = (n_keys + 1023) / 1024;
    const int lo = min(n_keys, t * per), hi = min(n_keys, lo + per);
    int64_t a = 0, it = 0;
    for (int x = lo; x < hi; ++x) {
        a += counts[x];
        it += (counts[x] + seg - 1) / seg;
    }
    s_sum[t] = a;
    s_items[t] = it;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive Hillis-Steele scan
        int64_t va = 0, vi = 0;
        if (t >= off) { va = s_sum[t - off]; vi = s_items[t - off]; }
        __syncthreads();
        s_sum[t] += va;
        s_items[t] += vi;
        __syncthreads();
    }
    int64_t run = s_sum[t] - a, run_it = s_items[t] - it;
    for (int x = lo; x < hi; ++x) {
        offsets[x] = (int32_t)run;
        item_offsets[x] = (int32_t)run_it;
        cursor[x] = 0;
        run += counts[x];
        run_it += (counts[x] + seg - 1) / seg;
    }
    if (t == 1023) total_items[0] = (int32_t)s_items[1023];
}

// One thread per row: append (i << 5 | slot) to the list of every non-local block.
__global__ void scatter_kernel(const int32_t* __restrict__ block_idx, const int32_t* __restrict__ offsets,
                               int32_t* __restrict__ cursor, int32_t* __restrict__ list, int64_t rows,
                               int N, int k, int nb, int nwin, int p_lo, int p_len) {
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x >= rows) return;
    const int i = p_lo + (int)(x % p_len);
    const int64_t bg = x / p_len;
    const int64_t r = bg * N + i;
    const int L = i / kBlock;
    const int32_t* row = block_idx + r * k;
    for (int s = 0; s + 1 < k; ++s) {
        const int j = row[s];
        if (j >= 0 && j < L) {
            const int64_t key = (bg * nwin + i / kWindow) * nb + j;
            const int at = offsets[key] + atomicAdd(&cursor[key], 1);
            list[at] = (i << 5) | s;
        }
    }
}

// One thread per key: its work items (key, first list entry, entry count).
__global__ void items_kernel(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                             const int32_t* __restrict__ item_offsets, int4* __restrict__ items, int n_keys,
                             int seg) {
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n_keys) return;
    const int c = counts[x];
    int at = item_offsets[x];
    for (int u = 0; u * seg < c; ++u) items[at++] = make_int4(x, offsets[x] + u * seg, min(seg, c - u * seg), 0);
}

// ------------------------------------------------ position-sorted lists --

// Sorted variant of the inversion, for kernels whose results depend on the
// order in which they visit a key's rows (sums over rows): every (b, g,
// window, j) key owns a bitmap over the window's positions; a row sets its bit
// in the bitmap of each of its non-local blocks (atomic OR: the result does
// not depend on the order), and the lists are read back from the bitmaps in
// ascending position order. The work items, cut every `seg` entries, then hold
// the same rows on every run.
__global__ void mark_kernel(const int32_t* __restrict__ block_idx, uint32_t* __restrict__ bits, int64_t rows,
                            int N, int k, int nb, int nwin, int wpk) {
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x >= rows) return;
    const int i = (int)(x % N);
    const int64_t bg = x / N;
    const int L = i / kBlock;
    const int32_t* row = block_idx + x * k;
    for (int s = 0; s + 1 < k; ++s) {
        const int j = row[s];
        if (j >= 0 && j < L)
            atomicOr(&bits[((bg * nwin + i / kWindow) * nb + j) * wpk + (i % kWindow) / 32], 1u << (i & 31));
    }
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// One wave per key: counts[key] = set bits of its bitmap.
__global__ __launch_bounds__(256) void count_bits_kernel(const uint32_t* __restrict__ bits,
                                                         int32_t* __restrict__ counts, int n_keys, int wpk) {
    const int key = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (key >= n_keys) return;
    const uint32_t* bw = bits + (size_t)key * wpk;
    int c = 0;
    for (int w = lane; w < wpk; w += 64) c += __popc(bw[w]);
    c = wave_sum(c);
    if (lane == 0) counts[key] = c;
}

// One wave per key: the list entries (i << 5 | slot) of its set bits in
// ascending position order, at the key's offset. The slot is where the row
// keeps j (the row holds j: the bit came from it).
__global__ __launch_bounds__(256) void compact_kernel(const uint32_t* __restrict__ bits,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ block_idx,
                                                      int32_t* __restrict__ list, int n_keys, int wpk, int N, int k,
                                                      int nb, int nwin) {
    const int key = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (key >= n_keys || counts[key] == 0) return;
    const int j = key % nb;
    const int win = (key / nb) % nwin;
    const size_t bg = (size_t)key / ((size_t)nb * nwin);
    const uint32_t* bw = bits + (size_t)key * wpk;
    int at = offsets[key];
    for (int w0 = 0; w0 < wpk; w0 += 64) {
        uint32_t word = w0 + lane < wpk ? bw[w0 + lane] : 0u;
        const int pc = __popc(word);
        int incl = pc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        int pos = at + incl - pc;
        while (word) {
            const int bit = __ffs(word) - 1;
            word &= word - 1;
            const int i = win * kWindow + (w0 + lane) * 32 + bit;
            const int32_t* row = block_idx + (bg * N + i) * k;
            // j's slot = the row's entries before it (ascending, -1 padded): read
            // with independent loads (indexes clamped into the row) instead of a
            // scan that waits for each load before the next
            int slot = 0;
            if (k <= 16) {
                int e[15];
#pragma unroll
                for (int s = 0; s < 15; ++s) e[s] = row[min(s, k - 2)];
#pragma unroll
                for (int s = 0; s < 15; ++s) slot += (s < k - 1 && e[s] >= 0 && e[s] < j) ? 1 : 0;
            } else {
                while (slot + 2 < k && row[slot] != j) ++slot;
            }
            list[pos++] = (i << 5) | slot;
        }
        at += __shfl(incl, 63);
    }
}


// ------------------------------------------------------- layout check --

// One thread per (b, g, i) row: does the row follow the selection layout (the
// first min(k, L+1) entries strictly ascending in [0, L] ending with L, then
// -1)? Broken rows are counted into *bad (cleared first by the caller).
__global__ __launch_bounds__(256) void check_rows_kernel(const int32_t* __restrict__ block_idx, int32_t* bad,
                                                         int64_t rows, int N, int k, int Bk) {
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x >= rows) return;
    const int i = (int)(x % N);
    const int L = i / Bk;
    const int nv = min(k, L + 1);
    const int32_t* row = block_idx + x * k;
    bool ok = true;
    int prev = -1;
    for (int s = 0; s < k; ++s) {
        const int j = row[s];
        if (s < nv) {
            ok &= j > prev && j <= L && (s + 1 < nv || j == L);
            prev = j;
        } else {
            ok &= j == -1;
        }
    }
    if (!ok) atomicAdd(bad, 1);
}

hipError_t launch_check_block_idx(const LaunchDims& d, const int32_t* block_idx, int32_t* bad, hipStream_t st) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, bad, (size_t)1, 0);
    const int64_t rows = (int64_t)d.B * d.Hkv * d.N;
    if (rows > 0)
        hipLaunchKernelGGL(check_rows_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, block_idx, bad,
                           rows, d.N, d.k, d.Bk);
    return hipGetLastError();
}

// ------------------------------------------ other block sizes as 128-blocks --

// A selection at block size 64 or 256, rewritten over 128-token blocks for the
// attention and KL kernels (which work on 128-token blocks). Per row (b, g, i)
// with the layout msa_index_topk writes:
//   Bk = 256: each kept non-local block j -> 128-blocks 2j and 2j + 1; the
//     local block -> its first half 2L if that precedes the query's own
//     128-block (fully visible), then the query's 128-block i / 128;
//   Bk = 64: the kept blocks grouped by 128-block j >> 1, with a mask per
//     entry (bit 0: first half kept, bit 1: second half kept); the last entry
//     is the query's 128-block.
// ids: ascending, -1 padded to ke entries; hmask (Bk = 64) per entry; info per
// row: bits 0-5 the number of entries before the query's 128-block, bit 6 set
// unless the first half of the query's 128-block is visible but not kept (a
// query in the second half whose preceding 64-block was not selected). Rows
// that break the layout give unspecified ids, but never more than ke of them.
__global__ __launch_bounds__(256) void expand_blocks_kernel(const int32_t* __restrict__ block_idx,
                                                            int32_t* __restrict__ ids, uint8_t* __restrict__ hmask,
                                                            uint8_t* __restrict__ info, int64_t rows, int N, int k,
                                                            int ke, int Bk) {
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x >= rows) return;
    const int i = (int)(x % N);
    const int L128 = i / kBlock;
    const int32_t* in = block_idx + x * k;
    int32_t* out = ids + x * ke;
    int n = 0;
    int low_kept = 1;
    if (Bk == 256) {
        const int L = i / 256;
        for (int s = 0; s < k; ++s) {
            const int j = in[s];
            if (j >= 0 && j < L && n + 2 <= ke) {
                out[n++] = 2 * j;
                out[n++] = 2 * j + 1;
            }
        }
        if (L128 > 2 * L && n < ke) out[n++] = 2 * L;
        if (n < ke) out[n++] = L128;
    } else {
        uint8_t* hm = hmask + x * ke;
        const int L = i / 64;
        int cur = -1, m = 0;
        for (int s = 0; s < k; ++s) {
            const int j = in[s];
            if (j < 0 || j > L) continue;
            if ((j >> 1) != cur) {
                if (cur >= 0 && n < ke) {
                    out[n] = cur;
                    hm[n++] = (uint8_t)m;
                }
                cur = j >> 1;
                m = 0;
            }
            m |= 1 << (j & 1);
        }
        if (cur >= 0 && n < ke) {
            out[n] = cur;
            hm[n++] = (uint8_t)m;
        }
        low_kept = (L & 1) == 0 || (m & 1);
        for (int s = n; s < ke; ++s) hm[s] = 0;
    }
    for (int s = n; s < ke; ++s) out[s] = -1;
    info[x] = (uint8_t)((n > 0 ? n - 1 : 0) | (low_kept ? 64 : 0));
}

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int expanded_topk(const LaunchDims& d) { return d.Bk == 256 ? 2 * d.k : d.k; }

LaunchDims as_128(const LaunchDims& d) {
    LaunchDims e = d;
    e.k = expanded_topk(d);
    e.Bk = 128;
    return e;
}

ExpandLayout expand_layout(const LaunchDims& d, size_t base) {
    ExpandLayout e{};
    size_t off = align_up(base);
    if (d.Bk == 128) {
        e.end = off;
        return e;
    }
    const size_t rows = (size_t)d.B * d.Hkv * d.N;
    const size_t ke = (size_t)expanded_topk(d);
    e.ids = off;    off = align_up(off + rows * ke * 4);
    e.hmask = off;  off = align_up(off + (d.Bk == 64 ? rows * ke : 0));
    e.info = off;   off = align_up(off + rows);
    e.end = off;
    return e;
}

void launch_expand(const LaunchDims& d, const int32_t* block_idx, unsigned char* ws, const ExpandLayout& E,
                   hipStream_t st) {
    const int64_t rows = (int64_t)d.B * d.Hkv * d.N;
    if (rows == 0) return;
    hipLaunchKernelGGL(expand_blocks_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, block_idx,
                       reinterpret_cast<int32_t*>(ws + E.ids), reinterpret_cast<uint8_t*>(ws + E.hmask),
                       reinterpret_cast<uint8_t*>(ws + E.info), rows, d.N, d.k, expanded_topk(d), d.Bk);
}

int windows(const LaunchDims& d) { return (d.N + kWindow - 1) / kWindow; }

int bitmap_words_per_key(const LaunchDims& d) { return (min(d.N, kWindow) + 31) / 32; }

ListLayout list_layout(const LaunchDims& d, size_t base, int seg, bool sorted) {
    ListLayout w{};
    const size_t n_keys = (size_t)d.B * d.Hkv * windows(d) * d.nb;
    const size_t kp = d.k > 1 ? (size_t)(d.k - 1) : 0;
    w.max_entries = (size_t)d.B * d.Hkv * d.N * kp;
    w.n_keys = n_keys;
    w.seg = seg;
    w.sorted = sorted;
    w.max_items = (w.max_entries + seg - 1) / seg + n_keys;
    size_t off = align_up(base);
    if (sorted) {
        w.bits = off;
        off = align_up(off + n_keys * bitmap_words_per_key(d) * 4);
    }
    w.counts = off;        off = align_up(off + n_keys * 4);
    w.offsets = off;       off = align_up(off + n_keys * 4);
    w.item_offsets = off;  off = align_up(off + n_keys * 4);
    w.cursor = off;        off = align_up(off + n_keys * 4);
    w.total = off;         off = align_up(off + 4);
    w.items = off;         off = align_up(off + w.max_items * 16);
    w.list = off;          off = align_up(off + w.max_entries * 4);
    w.end = off;
    w.has_nonlocal = kp > 0 && d.nb > 1;
    return w;
}

void launch_build_lists(const LaunchDims& d, int p_lo, int p_hi, const int32_t* block_idx, unsigned char* ws,
                        const ListLayout& L, hipStream_t st) {
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* item_offsets = reinterpret_cast<int32_t*>(ws + L.item_offsets);
    int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.cursor);
    int32_t* total = reinterpret_cast<int32_t*>(ws + L.total);
    int4* items = reinterpret_cast<int4*>(ws + L.items);
    int32_t* list = reinterpret_cast<int32_t*>(ws + L.list);
    const int p_len = p_hi - p_lo;
    const int nwin = windows(d);
    const int64_t rows = (int64_t)d.B * d.Hkv * p_len;
    const int nk = (int)L.n_keys;
    if (L.sorted) {   // every position of the sequence (p_lo = 0, p_hi = N)
        uint32_t* bits = reinterpret_cast<uint32_t*>(ws + L.bits);
        const int wpk = bitmap_words_per_key(d);
        const size_t nw = L.n_keys * (size_t)wpk;
        hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)std::min<size_t>((nw + 255) / 256, 65536)), dim3(256), 0, st,
                           reinterpret_cast<int32_t*>(bits), nw, 0);
        hipLaunchKernelGGL(mark_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, block_idx, bits, rows,
                           d.N, d.k, d.nb, nwin, wpk);
        hipLaunchKernelGGL(count_bits_kernel, dim3((nk + 3) / 4), dim3(256), 0, st, bits, counts, nk, wpk);
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, offsets, item_offsets, cursor, total, nk,
                           L.seg);
        hipLaunchKernelGGL(compact_kernel, dim3((nk + 3) / 4), dim3(256), 0, st, bits, counts, offsets, block_idx,
                           list, nk, wpk, d.N, d.k, d.nb, nwin);
        hipLaunchKernelGGL(items_kernel, dim3((nk + 255) / 256), dim3(256), 0, st, counts, offsets, item_offsets,
                           items, nk, L.seg);
        return;
    }
    hipLaunchKernelGGL(fill_i32_kernel, dim3((nk + 255) / 256), dim3(256), 0, st, counts, (size_t)nk, 0);
    const bool hist = d.nb <= kHistMaxBins;
    const int chunks = (p_len + kHistPos - 1) / kHistPos;
    const unsigned hist_grid = (unsigned)((size_t)d.B * d.Hkv * chunks);
    const size_t hist_lds = (size_t)d.nb * 4;
    if (hist)
        hipLaunchKernelGGL(count_hist_kernel, dim3(hist_grid), dim3(256), hist_lds, st, block_idx, counts, d.N, d.k,
                           d.nb, nwin, chunks, p_lo, p_hi);
    else
        hipLaunchKernelGGL(count_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, block_idx, counts,
                           rows, d.N, d.k, d.nb, nwin, p_lo, p_len);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, offsets, item_offsets, cursor, total, nk,
                       L.seg);
    if (hist)
        hipLaunchKernelGGL(scatter_hist_kernel, dim3(hist_grid), dim3(256), 2 * hist_lds, st, block_idx, offsets,
                           cursor, list, d.N, d.k, d.nb, nwin, chunks, p_lo, p_hi);
    else
        hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, block_idx,
                           offsets, cursor, list, rows, d.N, d.k, d.nb, nwin, p_lo, p_len);
    hipLaunchKernelGGL(items_kernel, dim3((nk + 255) / 256), dim3(256), 0, st, counts, offsets, item_offsets, items,
                       nk, L.seg);
}

size_t list_items_bound(const LaunchDims& d, int p_lo, int p_hi, const ListLayout& L) {
    const size_t kp = d.k > 1 ? (size_t)(d.k - 1) : 0;
    const size_t entries = (size_t)d.B * d.Hkv * (size_t)(p_hi - p_lo) * kp;
    return (entries + L.seg - 1) / L.seg + L.n_keys;
}

}  // namespace msa
