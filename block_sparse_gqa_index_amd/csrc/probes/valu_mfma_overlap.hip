// VALU / matrix-core overlap probe for gfx950 (not part of the library): in a
// 512-thread work-group (two waves per SIMD) waves 0-3 issue back-to-back
// independent 32x32x16 bf16 MFMAs and waves 4-7, on the same SIMDs, run
// independent VALU chains (fma, or exp2 + fma); the kernel time with either
// group alone and with both shows how much of one hides under the other.
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float floatx16;

template <int MODE>   // bit 0: MFMA waves work, bit 1: VALU waves work, bit 2: VALU uses exp
__global__ __launch_bounds__(512, 1) void probe(float* out, int iters) {
  const int w = threadIdx.x >> 6;
  float r = 0.f;
  if (w < 4) {
    if (MODE & 1) {
      bf16x8 a, b;
      for (int e = 0; e < 8; ++e) { a[e] = (__bf16)(0.001f * (threadIdx.x + e)); b[e] = (__bf16)(0.002f * e); }
      floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
      for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
      for (int e = 0; e < 16; ++e) r += c0[e] + c1[e] + c2[e] + c3[e];
    }
  } else {
    if (MODE & 2) {
      float x[8];
      for (int e = 0; e < 8; ++e) x[e] = 0.0001f * (threadIdx.x + e);
      const float y = 0.999f, z = 0.0001f;
      for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int rep = 0; rep < 4; ++rep) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (MODE & 4) x[e] = __builtin_amdgcn_exp2f(x[e] * y - z);
            else x[e] = fmaf(x[e], y, z);
          }
        }
      }
      for (int e = 0; e < 8; ++e) r += x[e];
    }
  }
  out[blockIdx.x * 512 + threadIdx.x] = r;
}

template <int MODE> float run(float* out, int iters, int blocks) {
  hipEvent_t a, b; hipEventCreate(&a); hipEventCreate(&b);
  hipLaunchKernelGGL(probe<MODE>, dim3(blocks), dim3(512), 0, 0, out, iters);
  hipEventRecord(a);
  for (int k = 0; k < 5; ++k) hipLaunchKernelGGL(probe<MODE>, dim3(blocks), dim3(512), 0, 0, out, iters);
  hipEventRecord(b); hipEventSynchronize(b);
  float ms; hipEventElapsedTime(&ms, a, b);
  return ms / 5;
}
int main() {
  float* out; const int blocks = 256 * 4;
  if (hipMalloc(&out, blocks * 512 * 4) != hipSuccess) return 1;
  const int iters = 4096;
  // per MFMA-wave iteration: 4 MFMAs; per VALU-wave iteration: 32 VALU ops (fma) or 32 (exp + fma pairs)
  float m = run<1>(out, iters, blocks), v = run<2>(out, iters, blocks), mv = run<3>(out, iters, blocks);
  float ve = run<6>(out, iters, blocks), mve = run<7>(out, iters, blocks);
  printf("mfma only %.3f ms | valu fma only %.3f | both %.3f | valu exp only %.3f | both(exp) %.3f\n", m, v, mv, ve, mve);
  hipFree(out);
  return 0;
}
