// Test support (not part of libfa.so): one wave computes one matrix-core
// product, C[32][32] = C0 + A * B, so a test can compare the instruction's
// result with the exact sum and check the accumulation model that the FP8
// forward's tolerance rests on.
//   fa_probe_fp8:  v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes, A [32][64],
//                  B given transposed as Bt [32][64] (unit block scales);
//   fa_probe_bf16: v_mfma_f32_32x32x16_bf16, A [32][16], Bt [32][16].
// Operand layout as in the library's kernels: lane (l32, g) supplies items
// 32g..32g+31 (FP8) or 8g..8g+7 (bf16) of row l32 of A and of column l32 of
// B; register r of the result is row 8(r/4) + 4g + r%4, column l32.  Every
// lane reads and writes inside the buffers' fixed sizes (A, Bt: 2048 bytes
// FP8 or 1024 bytes bf16; C0, C: 1024 floats); the host launches one wave.

#include <hip/hip_runtime.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int c_index(int r, int g, int l32) {
  return (8 * (r / 4) + 4 * g + r % 4) * 32 + l32;
}

__global__ void __launch_bounds__(64) probe_fp8_kernel(const int* A, const int* Bt,
                                                       const float* C0, float* C) {
  const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
  i32x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = A[l32 * 16 + 8 * g + e];
    b[e] = Bt[l32 * 16 + 8 * g + e];
  }
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = C0[c_index(r, g, l32)];
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
#pragma unroll
  for (int r = 0; r < 16; ++r) C[c_index(r, g, l32)] = c[r];
}

__global__ void __launch_bounds__(64) probe_bf16_kernel(const __bf16* A, const __bf16* Bt,
                                                        const float* C0, float* C) {
  const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = A[l32 * 16 + 8 * g + e];
    b[e] = Bt[l32 * 16 + 8 * g + e];
  }
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = C0[c_index(r, g, l32)];
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) C[c_index(r, g, l32)] = c[r];
}

extern "C" __attribute__((visibility("default"))) int fa_probe_fp8(const void* A, const void* Bt,
                                                                   const float* C0, float* C) {
  hipLaunchKernelGGL(probe_fp8_kernel, dim3(1), dim3(64), 0, 0, static_cast<const int*>(A),
                     static_cast<const int*>(Bt), C0, C);
  return (int)hipDeviceSynchronize();
}

extern "C" __attribute__((visibility("default"))) int fa_probe_bf16(const void* A,
                                                                    const void* Bt,
                                                                    const float* C0, float* C) {
  hipLaunchKernelGGL(probe_bf16_kernel, dim3(1), dim3(64), 0, 0, static_cast<const __bf16*>(A),
                     static_cast<const __bf16*>(Bt), C0, C);
  return (int)hipDeviceSynchronize();
}
