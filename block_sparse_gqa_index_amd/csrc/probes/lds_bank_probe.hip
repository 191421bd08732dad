// LDS bank-conflict probe for gfx950 (not part of the library): each kernel
// instance repeats one LDS access pattern, 2048 times per wave, so that
// rocprofv3's SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE per dispatch give the
// cycles one instruction of that pattern takes. Patterns 0 and 15-25 are
// plain strides and lane groupings (to find how the hardware groups lanes);
// 1-14 are the backward kernels' staging, operand and dS patterns (1: 32-row
// tile read as the A operand of 16x16x32 products; 2-6: the transposed tile
// read with chunk-column strides 16 D + 16, 16 D, +32, +64 and without the
// XOR; 7: natural staging writes; 8-12: transposed staging writes, same
// strides; 13-14: dS writes as 16-bit and as 32-bit pairs). Addresses are
// masked into the 64 KiB array, so every access is in bounds.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDSP(T, off) ((volatile __attribute__((address_space(3))) T*)(lds3 + (off)))

__device__ inline int swz(int row, int byte) { return row * 256 + ((((byte >> 4) ^ (row & 15))) << 4) + (byte & 15); }
__device__ inline int coltile(int d, int q, int qstride, int xr) { return q * qstride + 16 * (xr ? (d ^ ((d >> 3) & 15)) : d); }
__device__ inline int perm16(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// kind 0: b128 read, 1: b64 write, 2: b128 write, 3: b16 write, 4: b32 write
template <int P> struct Pat;
// 0: linear b128 read
template <> struct Pat<0> { static constexpr int K = 1, kind = 0;
  __device__ static int addr(int k, int l, int w) { return 16 * l; } };
// 1: S-load (Q tile as A of 16x16x32): row 16rh+cl, chunk 4ks+ql
template <> struct Pat<1> { static constexpr int K = 4, kind = 0;
  __device__ static int addr(int k, int l, int w) { int ql = l >> 4, cl = l & 15; return swz(cl, (32 * k + 8 * ql) * 2); } };
// 2..6: ColTile read (dim 16dt+cl, chunk ql), dt = k, qstride variants
template <int QS, int XR> struct ColRead { static constexpr int K = 8, kind = 0;
  __device__ static int addr(int k, int l, int w) { int ql = l >> 4, cl = l & 15; return coltile(16 * k + cl, ql, QS, XR); } };
template <> struct Pat<2> : ColRead<2064, 1> {};
template <> struct Pat<3> : ColRead<2048, 1> {};
template <> struct Pat<4> : ColRead<2080, 1> {};
template <> struct Pat<5> : ColRead<2112, 1> {};
template <> struct Pat<6> : ColRead<2048, 0> {};
// 7: natural staging writes (b128), unit map of the kernel (u = 64w + l, v = u % 128)
__device__ inline void unit(int v, int& rq, int& dc) { dc = (v & 7) | (((v >> 4) & 1) << 3); rq = (((v >> 3) & 1) << 2) | ((v >> 5) & 3); }
template <> struct Pat<7> { static constexpr int K = 4, kind = 2;
  __device__ static int addr(int k, int l, int w) { int v = (64 * w + l) & 127, rq, dc; unit(v, rq, dc); return swz(4 * rq + k, dc * 16); } };
// 8..12: transposed staging writes (b64), qstride variants
template <int QS, int XR> struct ColWrite { static constexpr int K = 8, kind = 1;
  __device__ static int addr(int k, int l, int w) { int v = (64 * w + l) & 127, rq, dc; unit(v, rq, dc);
    return coltile(dc * 8 + k, rq & 3, QS, XR) + (rq >> 2) * 8; } };
template <> struct Pat<8> : ColWrite<2064, 1> {};
template <> struct Pat<9> : ColWrite<2048, 1> {};
template <> struct Pat<10> : ColWrite<2080, 1> {};
template <> struct Pat<11> : ColWrite<2112, 1> {};
template <> struct Pat<12> : ColWrite<2048, 0> {};
// 13: dS writes (b16): row m = 16(e>>2) + 4ql + (e&3), key perm16(16w + cl)
template <> struct Pat<13> { static constexpr int K = 8, kind = 3;
  __device__ static int addr(int e, int l, int w) { int ql = l >> 4, cl = l & 15; int m = 16 * (e >> 2) + 4 * ql + (e & 3);
    return swz(m, perm16(16 * w + cl) * 2); } };
// 14: dS writes as b32 pairs: even lanes row m_e keys (k, k+1), odd lanes row m_{e+1} keys (k-1, k)
template <> struct Pat<14> { static constexpr int K = 4, kind = 4;
  __device__ static int addr(int p, int l, int w) { int ql = l >> 4, cl = l & 15; int e = 2 * p + (cl & 1);
    int m = 16 * (e >> 2) + 4 * ql + (e & 3); return swz(m, perm16(16 * w + (cl & ~1)) * 2); } };
// 15: linear b64 write, 16: linear b16 write, 17: linear b128 write
template <> struct Pat<15> { static constexpr int K = 1, kind = 1; __device__ static int addr(int, int l, int) { return 8 * l; } };
template <> struct Pat<16> { static constexpr int K = 1, kind = 3; __device__ static int addr(int, int l, int) { return 2 * l; } };
template <> struct Pat<17> { static constexpr int K = 1, kind = 2; __device__ static int addr(int, int l, int) { return 16 * l; } };
// 18: stride-128B b128 read (lane l: granule 8l)
template <> struct Pat<18> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 128 * l; } };
// 19: stride-256B b128 read
template <> struct Pat<19> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 256 * l; } };
// 20: b128 read, lanes l and l+32 on the same banks (1 KiB apart), each half linear
template <> struct Pat<20> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 16 * (l & 31) + 1024 * (l >> 5); } };
// 21: b128 read, lanes l and l+16 same banks (1 KiB apart), 16-lane groups linear
template <> struct Pat<21> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 16 * (l & 15) + 1024 * (l >> 4); } };
// 22: b128 read, lanes l and l+8 same 128-byte window, different address (8-lane groups)
template <> struct Pat<22> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 16 * (l & 7) + 1024 * (l >> 3); } };
// 23: b128 read, 4-lane groups on the same 64 bytes window
template <> struct Pat<23> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 16 * (l & 3) + 1024 * (l >> 2); } };
// 24: b128 read, granule (l & 15) within a 256 B window, window 1 KiB * (l >> 4) + 16*? : lanes l, l+16 differ by 256 B
template <> struct Pat<24> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 16 * (l & 15) + 256 * (l >> 4); } };
// 25: b128 read, lanes l and l+8 in 128 B windows 128 B apart (so 16 lanes cover 256 B linear) -> same as linear? lane l: 16*(l&7) + 128*((l>>3)&1) + 2048*(l>>4)
template <> struct Pat<25> { static constexpr int K = 1, kind = 0; __device__ static int addr(int, int l, int) { return 16 * (l & 15) + 2048 * (l >> 4); } };

template <int P>
__global__ __launch_bounds__(256) void probe(uint32_t* out, int iters) {
  __shared__ __align__(16) unsigned char lds[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += 256) reinterpret_cast<u32x4*>(lds)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  __attribute__((address_space(3))) unsigned char* lds3 = (__attribute__((address_space(3))) unsigned char*)(lds);
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  using Q = Pat<P>;
  int a[Q::K];
#pragma unroll
  for (int k = 0; k < Q::K; ++k) a[k] = Q::addr(k, l, w) & 0xFFF0 ? (Q::addr(k, l, w) & 0xFFFF) : (Q::addr(k, l, w) & 0xFFFF);
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < Q::K; ++k) {
      if constexpr (Q::kind == 0) { u32x4 x = *LDSP(u32x4, a[k] & 0xFFF0); acc ^= x.x ^ x.w; }
      else if constexpr (Q::kind == 1) { *LDSP(u32x2, a[k] & 0xFFF8) = u32x2{acc, (uint32_t)it}; }
      else if constexpr (Q::kind == 2) { *LDSP(u32x4, a[k] & 0xFFF0) = u32x4{acc, (uint32_t)it, 0u, 1u}; }
      else if constexpr (Q::kind == 3) { *LDSP(uint16_t, a[k] & 0xFFFE) = (uint16_t)(acc + it); }
      else { *LDSP(uint32_t, a[k] & 0xFFFC) = acc + it; }
    }
  }
  __syncthreads();
  out[blockIdx.x * 256 + threadIdx.x] = acc ^ reinterpret_cast<uint32_t*>(lds)[threadIdx.x];
}

template <int P> void run(uint32_t* out, int iters) {
  hipLaunchKernelGGL(probe<P>, dim3(512), dim3(256), 0, 0, out, iters);
  hipError_t e = hipDeviceSynchronize();
  printf("pattern %d: %s\n", P, hipGetErrorString(e));
  fflush(stdout);
}
template <int... Ps> void run_all(uint32_t* out, int iters, std::integer_sequence<int, Ps...>) { (run<Ps>(out, iters), ...); }

int main() {
  uint32_t* out;
  if (hipMalloc(&out, 512 * 256 * 4) != hipSuccess) return 1;
  run_all(out, 2048, std::make_integer_sequence<int, 26>{});
  hipFree(out);
  return 0;
}
