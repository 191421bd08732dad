// HBM read-bandwidth probe for gfx950 (not part of the library): streams an
// 8 GiB buffer with 16-byte loads per lane, UNROLL loads in flight per thread,
// grid-stride over the buffer, with plain or non-temporal loads, at several
// grid sizes (the work-groups beyond those resident at once only refill CUs).
// The loop bound keeps every access inside the buffer; the xor of the data
// keeps the loads alive and is written only if it hits an impossible value.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, size_t n, unsigned* __restrict__ out) {
    const size_t tid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    unsigned acc = 0;
    size_t i = tid;
    for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) acc ^= p[i].x;
    if (acc == 0x12345678u) out[blockIdx.x] = acc;
}

template <int U, bool NT>
static float time_ms(const u32x4* p, size_t n, unsigned* out, int grid) {
    hipEvent_t a, b;
    (void)hipEventCreate(&a);
    (void)hipEventCreate(&b);
    read_kernel<U, NT><<<grid, 256>>>(p, n, out);
    (void)hipEventRecord(a);
    for (int r = 0; r < 5; ++r) read_kernel<U, NT><<<grid, 256>>>(p, n, out);
    (void)hipEventRecord(b);
    (void)hipEventSynchronize(b);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, a, b);
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return ms / 5;
}

int main() {
    const size_t bytes = (size_t)8 << 30;
    const size_t n = bytes / 16;
    u32x4* p = nullptr;
    unsigned* out = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess || hipMalloc(&out, 16384 * sizeof(unsigned)) != hipSuccess) {
        printf("allocation failed\n");
        return 1;
    }
    (void)hipMemset(p, 1, bytes);
    (void)hipDeviceSynchronize();
    for (int grid : {1024, 2048, 4096, 8192, 16384}) {
        const float t4 = time_ms<4, false>(p, n, out, grid), t8 = time_ms<8, false>(p, n, out, grid),
                    t8n = time_ms<8, true>(p, n, out, grid);
        printf("grid %5d: 4 loads/thread %.2f TB/s, 8 loads/thread %.2f TB/s, 8 non-temporal loads/thread %.2f TB/s\n",
               grid, bytes / t4 / 1e9, bytes / t8 / 1e9, bytes / t8n / 1e9);
    }
    (void)hipFree(p);
    (void)hipFree(out);
    return 0;
}
